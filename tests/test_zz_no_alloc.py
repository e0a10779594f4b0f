"""conv2d_grad_input_noalloc (fp32 grad_input with no allocation) against
conv2d_grad_input, through the C ABI.

Two calls in a row on one stream, the second with a smaller input, each
compared with the allocating entry point on the same inputs: element by
element to the fp32 criterion |a - b| <= 1e-5 * S + 1e-6 (S from the oracle),
and bit for bit (both run the same plan and kernels, whose sums are in a fixed
order).  Each result is also checked against the oracle itself.  Covers a
plan with weight-image scratch (halo), a strided halo plan, the generic plan
and the stem plan (no scratch).
"""
import ctypes

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import conv2d_backward_amd as gi  # noqa: E402

S = workloads.Shape
REL, ABS = 1e-5, 1e-6


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = gi.load_library()
    lib.conv2d_grad_input_noalloc.argtypes = [ctypes.c_void_p] * 3 + [gi.Conv2dGiParams,
                                                                       ctypes.c_void_p]
    lib.conv2d_grad_input_noalloc.restype = ctypes.c_int
    return lib


def both(lib, sh, seed, variant=gi.VARIANT_AUTO):
    """(noalloc result, allocating result, oracle value, oracle S) as float64."""
    dev = torch.device("cuda:0")
    g, w = workloads.make_case(sh, seed, "normal")
    tg, tw = torch.from_numpy(g).to(dev), torch.from_numpy(w).to(dev)
    a = torch.full(sh.dst_shape, float("nan"), device=dev)
    p = gi.make_params(*sh.as_tuple()[:10])
    s = torch.cuda.current_stream()
    old = gi.set_variant(variant)
    try:
        print("noalloc case %s plan %s" % (sh, gi.plan(p)), flush=True)
        rc = lib.conv2d_grad_input_noalloc(ctypes.c_void_p(tg.data_ptr()),
                                           ctypes.c_void_p(tw.data_ptr()),
                                           ctypes.c_void_p(a.data_ptr()), p,
                                           ctypes.c_void_p(s.cuda_stream))
        assert rc == gi.OK, lib.conv2d_gi_strerror(rc)
        b = gi.grad_input(tg, tw, stride=sh.stride, padding=(sh.pad_h, sh.pad_w),
                          input_hw=(sh.H, sh.W))
    finally:
        gi.set_variant(old)
    torch.cuda.synchronize()
    ref, Ssum = oracle.grad_input(g, w, sh.stride, (sh.pad_h, sh.pad_w), (sh.H, sh.W))
    return (a.cpu().numpy().astype(np.float64), b.cpu().numpy().astype(np.float64), ref, Ssum)


def check(x, y, Ssum, what):
    assert not np.isnan(x).any(), "%s: unwritten elements" % what
    bad = np.abs(x - y) > REL * Ssum + ABS
    assert not bad.any(), "%s: %d elements out of tolerance" % (what, int(bad.sum()))


CASES = [
    # (larger, smaller) pairs run back to back: the second call reuses the
    # same device array with a smaller plan.
    ((S(4, 64, 28, 28, 64, 3, 3, 1, 1, 1), gi.VARIANT_AUTO),      # halo, weight image
     (S(2, 20, 12, 12, 24, 3, 3, 2, 1, 1), gi.VARIANT_AUTO)),     # strided halo, smaller image
    ((S(2, 48, 20, 21, 40, 3, 3, 1, 1, 1), gi.VARIANT_GENERIC),   # generic, tap-major weight
     (S(1, 9, 7, 9, 5, 3, 3, 1, 1, 1), gi.VARIANT_GENERIC)),
    ((S(2, 3, 45, 44, 64, 7, 7, 2, 3, 3), gi.VARIANT_AUTO),       # stem: no scratch
     (S(1, 3, 20, 19, 8, 7, 7, 2, 3, 3), gi.VARIANT_AUTO)),
]


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_noalloc_matches_allocating_entry_point(lib, idx):
    for k, (sh, variant) in enumerate(CASES[idx]):
        a, b, ref, Ssum = both(lib, sh, 7100 + 10 * idx + k, variant)
        check(a, b, Ssum, "noalloc vs conv2d_grad_input, call %d %s" % (k, sh))
        check(a, ref, Ssum, "noalloc vs oracle, call %d %s" % (k, sh))
        assert np.array_equal(a, b), "call %d %s: not bit-identical" % (k, sh)


def test_noalloc_rejects_oversized_plan(lib):
    """A plan needing more scratch than the fixed array: EUNSUPPORTED, and
    the output is left as it was."""
    sh = S(1, 1024, 4, 4, 1024, 3, 3, 1, 1, 1)   # weight image ~ 37.7 MB > 16 MiB
    dev = torch.device("cuda:0")
    g = torch.zeros(sh.grad_out_shape, device=dev)
    w = torch.zeros(sh.weight_shape, device=dev)
    d = torch.full(sh.dst_shape, 5.0, device=dev)
    p = gi.make_params(*sh.as_tuple()[:10])
    rc = lib.conv2d_grad_input_noalloc(ctypes.c_void_p(g.data_ptr()), ctypes.c_void_p(w.data_ptr()),
                                       ctypes.c_void_p(d.data_ptr()), p,
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == gi.EUNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(d == 5.0)
