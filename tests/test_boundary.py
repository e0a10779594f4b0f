"""Host-side tests of the C-ABI library: it loads, exports every entry point
that include/*.h declares, and rejects bad arguments before any HIP call.

No test here launches a kernel, so they run without a GPU.
"""
import ctypes
import glob
import os
import re

import pytest

import conv2d_backward_amd as gi
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gi.library_path):
        from conv2d_backward_amd import build
        build.build()
    return gi.load_library()


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        names += re.findall(r"^CONV2D_GI_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, re.M)
    return names


def test_header_declares_entry_points():
    names = declared_functions()
    assert "conv2d_grad_input" in names and "conv2d_grad_input_bf16" in names
    assert len(names) == len(set(names))


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(gi.exported_names()) <= set(declared_functions())


def test_version(lib):
    assert re.fullmatch(r"\d+\.\d+\.\d+", lib.conv2d_gi_version().decode())


def test_strerror(lib):
    for code in (gi.OK, gi.EINVAL, gi.EUNSUPPORTED, gi.EHIP):
        assert lib.conv2d_gi_strerror(code)
    assert b"unknown" in lib.conv2d_gi_strerror(99)


def test_validate_accepts_workloads(lib):
    for wl in workloads.WORKLOADS:
        s = wl.shape
        assert gi.validate(gi.make_params(*s.as_tuple()[:10])) == gi.OK, wl.name
    for s in workloads.sweep_shapes():
        assert gi.validate(gi.make_params(*s.as_tuple()[:10])) == gi.OK, s


BAD = [
    dict(H=0), dict(W=-1), dict(kH=0), dict(kW=0), dict(stride=0), dict(stride=-2),
    dict(pad_h=-1), dict(pad_w=-1), dict(N=-1), dict(Ci=-1), dict(Co=-1),
    dict(N=0), dict(Ci=0), dict(Co=0),   # zero sizes: the doppler wrappers throw on them
    dict(oH=57), dict(oW=55), dict(oH=0),
    dict(kH=61, pad_h=1, oH=1),   # H + 2*pad < kH: empty forward output
]


@pytest.mark.parametrize("change", BAD, ids=lambda d: ",".join("%s=%s" % kv for kv in d.items()))
def test_validate_rejects(lib, change):
    base = dict(N=2, Ci=3, H=56, W=56, Co=4, kH=3, kW=3, stride=1, pad_h=1, pad_w=1, oH=56, oW=56)
    base.update(change)
    p = gi.Conv2dGiParams(*[base[f] for f in gi._FIELDS])
    assert gi.validate(p) == gi.EINVAL


def test_validate_index_width(lib):
    p = gi.make_params(1, 70000, 200, 200, 1, 1, 1, 1, 0, 0)  # Ci*H*W > 2^31
    assert gi.validate(p) == gi.EUNSUPPORTED
    p = gi.make_params(70000, 1, 200, 200, 1, 1, 1, 1, 0, 0)  # N*H*W > 2^31
    assert gi.validate(p) == gi.EUNSUPPORTED


def test_validate_forward_index_width(lib):
    """N*oH*oW above 2^31 - 1 (the folded output-pixel axis) is refused even
    where N*H*W fits: padding beyond k - 1 makes the output plane larger than
    the input plane."""
    p = gi.make_params(100000, 1, 100, 100, 1, 1, 1, 1, 30, 30)   # oH = oW = 160
    assert 100000 * 100 * 100 < 2 ** 31 and 100000 * p.oH * p.oW >= 2 ** 31
    assert gi.validate(p) == gi.EUNSUPPORTED


def test_params_passed_by_value(lib):
    """The struct travels by value: the argtypes name the struct itself."""
    assert lib.conv2d_grad_input.argtypes[3] is gi.Conv2dGiParams
    assert lib.conv2d_gi_validate.argtypes[0] is gi.Conv2dGiParams


def _call(lib, fn, g, w, d, p):
    return getattr(lib, fn)(ctypes.c_void_p(g), ctypes.c_void_p(w), ctypes.c_void_p(d), p, None)


@pytest.mark.parametrize("fn", ["conv2d_grad_input", "conv2d_grad_input_bf16"])
def test_entry_rejects_before_any_hip_call(lib, fn):
    """Invalid calls return EINVAL without touching the (fake) pointers."""
    good = gi.make_params(2, 3, 8, 8, 4, 3, 3, 1, 1, 1)
    fake = 0x1000
    bad = gi.make_params(2, 3, 8, 8, 4, 3, 3, 1, 1, 1, oH=9)
    assert _call(lib, fn, fake, fake, fake, bad) == gi.EINVAL
    assert _call(lib, fn, 0, fake, fake, good) == gi.EINVAL
    assert _call(lib, fn, fake, 0, fake, good) == gi.EINVAL
    assert _call(lib, fn, fake, fake, 0, good) == gi.EINVAL
    big = gi.make_params(1, 70000, 200, 200, 1, 1, 1, 1, 0, 0)
    assert _call(lib, fn, fake, fake, fake, big) == gi.EUNSUPPORTED


@pytest.mark.parametrize("fn", ["conv2d_grad_input", "conv2d_grad_input_bf16",
                                "conv2d_grad_input_f16", "conv2d_grad_weight",
                                "conv2d_forward"])
def test_zero_sizes_rejected(lib, fn):
    """N, Ci or Co = 0: EINVAL before any HIP call (the fake pointers are
    never touched), as the doppler wrappers throw on zero sizes."""
    fake = 0x1000
    for p in (gi.make_params(0, 3, 8, 8, 4, 3, 3, 1, 1, 1),
              gi.make_params(2, 0, 8, 8, 4, 3, 3, 1, 1, 1),
              gi.make_params(2, 3, 8, 8, 0, 3, 3, 1, 1, 1)):
        assert _call(lib, fn, fake, fake, fake, p) == gi.EINVAL, p


def test_noalloc_rejects_before_any_hip_call(lib):
    """The no-allocation entry point: bad shapes and null pointers return
    EINVAL, and a plan needing more than its fixed scratch EUNSUPPORTED, all
    before any HIP call (no GPU here)."""
    fake = 0x1000
    fn = "conv2d_grad_input_noalloc"
    assert _call(lib, fn, fake, fake, fake, gi.make_params(0, 3, 8, 8, 4, 3, 3, 1, 1, 1)) == gi.EINVAL
    assert _call(lib, fn, 0, fake, fake, gi.make_params(2, 3, 8, 8, 4, 3, 3, 1, 1, 1)) == gi.EINVAL
    big = gi.make_params(1, 1024, 4, 4, 1024, 3, 3, 1, 1, 1)   # ~37.7 MB weight image
    assert _call(lib, fn, fake, fake, fake, big) == gi.EUNSUPPORTED


def test_backward_rejects_before_any_hip_call(lib):
    fake = ctypes.c_void_p(0x1000)
    null = ctypes.c_void_p(0)
    p = gi.make_params(2, 3, 8, 8, 4, 3, 3, 1, 1, 1)
    # dx without the weight, dw without the input, any output without grad_out
    assert lib.conv2d_backward(fake, null, null, fake, null, null, p, None) == gi.EINVAL
    assert lib.conv2d_backward(fake, null, null, null, fake, null, p, None) == gi.EINVAL
    assert lib.conv2d_backward(null, null, null, null, null, fake, p, None) == gi.EINVAL
    assert lib.conv2d_grad_bias(fake, null, p, None) == gi.EINVAL
    # a zero size
    q = gi.make_params(0, 3, 8, 8, 4, 3, 3, 1, 1, 1)
    assert lib.conv2d_backward(fake, fake, fake, fake, fake, fake, q, None) == gi.EINVAL
    # nothing asked: nothing to do
    assert lib.conv2d_backward(null, null, null, null, null, null, p, None) == gi.OK


def test_hooks_are_thread_local(lib):
    """A hook set in one thread leaves another thread's plans alone."""
    import threading
    s = workloads.BY_NAME["resnet_stage_3x3"].shape
    p = gi.make_params(*s.as_tuple()[:10])
    assert "variant=halo" in gi.plan(p)
    seen = {}
    old = gi.set_variant(gi.VARIANT_GENERIC)
    try:
        assert "variant=generic" in gi.plan(p)
        t = threading.Thread(target=lambda: seen.setdefault("plan", gi.plan(p)))
        t.start()
        t.join()
    finally:
        gi.set_variant(old)
    assert "variant=halo" in seen["plan"]


def test_set_variant(lib):
    old = gi.set_variant(gi.VARIANT_GENERIC)
    try:
        assert gi.set_variant(gi.VARIANT_AUTO) == gi.VARIANT_GENERIC
        assert lib.conv2d_gi_set_variant(12345) == -1
    finally:
        gi.set_variant(old)


def test_plan_phases(lib):
    """The planner splits a stride-s problem into s*s residue classes with the
    tap counts of the phase split (e.g. 3x3, stride 2, pad 1: 1x1, 1x2, 2x1, 2x2)."""
    s = workloads.BY_NAME["strided_downsample"].shape
    txt = gi.plan(gi.make_params(*s.as_tuple()[:10]))
    phases = re.findall(r"phase\((\d+),(\d+)\) taps=(\d+)x(\d+) px=(\d+)x(\d+)", txt)
    assert len(phases) == 4
    taps = {(int(a), int(b)): (int(c), int(d)) for a, b, c, d, _, _ in phases}
    # rho = 0: (0 + 1) mod 2 = 1 -> taps kh in {1}; rho = 1: (1 + 1) mod 2 = 0 -> kh in {0, 2}
    assert taps == {(0, 0): (1, 1), (0, 1): (1, 2), (1, 0): (2, 1), (1, 1): (2, 2)}
    assert all((int(e), int(f)) == (28, 28) for *_, e, f in phases)
    # every tap of the kernel is in exactly one phase per dimension
    # (the phase-split stem plan; the planner's own choice for the stem is
    # the column kernel, which has no phases)
    s1 = workloads.BY_NAME["stem_7x7_s2"].shape
    old = gi.set_variant(gi.VARIANT_STEM)
    try:
        txt = gi.plan(gi.make_params(*s1.as_tuple()[:10]))
    finally:
        gi.set_variant(old)
    ph = re.findall(r"phase\((\d+),(\d+)\) taps=(\d+)x(\d+)", txt)
    assert sum(int(c) for a, b, c, d in ph if b == "0") == 7
    # kernel shorter than the stride: some phases get no taps but keep their pixels
    txt = gi.plan(gi.make_params(1, 2, 9, 9, 3, 2, 2, 3, 0, 0))
    ph = re.findall(r"phase\((\d+),(\d+)\) taps=(\d+)x(\d+) px=(\d+)x(\d+)", txt)
    assert len(ph) == 9
    assert sum(1 for p in ph if p[2] == "0" or p[3] == "0") == 5
    assert sum(int(p[4]) * int(p[5]) for p in ph) == 81


def test_binding_rejects_cpu_tensors(lib):
    torch = pytest.importorskip("torch")
    g = torch.zeros(1, 2, 4, 4)
    w = torch.zeros(2, 3, 3, 3)
    with pytest.raises(ValueError):
        gi.grad_input(g, w, stride=1, padding=1, input_hw=(4, 4))


def test_product_path_does_not_import_oracle():
    """The library package and its binding never reach the CPU oracle."""
    for path in glob.glob(os.path.join(ROOT, "conv2d_backward_amd", "**", "*"), recursive=True):
        if os.path.isfile(path) and path.endswith((".py", ".cpp", ".hip", ".h")):
            text = open(path).read()
            assert "oracle" not in text.lower(), path
