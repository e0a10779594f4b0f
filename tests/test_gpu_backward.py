"""GPU parity of the fused backward call (dx, dw and the bias gradient db in
one library call) and of the bias gradient alone, through the C ABI, against
the CPU oracle.  Criterion as for the single calls: per element
|gpu - oracle| <= 1e-5 * S + 1e-6, with S the sum of the absolute values of
the element's terms (|g*w| for dx, |g*x| for dw, |g| for db).
"""
import sys
import zlib

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import conv2d_backward_amd as gi  # noqa: E402

REL, ABS = 1e-5, 1e-6
S = workloads.Shape


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gi.load_library()
    return torch.device("cuda:0")


def check(got, ref, Ssum, what):
    assert not np.isnan(got).any(), "%s: NaN in the result" % what
    err = np.abs(got - ref)
    bad = err > REL * Ssum + ABS
    if bad.any():
        i = int(np.argmax(err - (REL * Ssum + ABS)))
        raise AssertionError("%s: %d elements out of tolerance; worst flat %d got %r want %r"
                             % (what, int(bad.sum()), i, got.ravel()[i], ref.ravel()[i]))


def inputs(sh, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(sh.dst_shape).astype(np.float32)
    w = rng.standard_normal(sh.weight_shape).astype(np.float32)
    g = rng.standard_normal(sh.grad_out_shape).astype(np.float32)
    return x, w, g


def run_backward(sh, x, w, g, want):
    dev = torch.device("cuda:0")
    tx, tw, tg = (torch.from_numpy(a).to(dev) for a in (x, w, g))
    # Outputs pre-filled with NaN: an unwritten element fails.
    dx = torch.full(sh.dst_shape, float("nan"), device=dev) if "x" in want else None
    dw = torch.full(sh.weight_shape, float("nan"), device=dev) if "w" in want else None
    db = torch.full((sh.Co,), float("nan"), device=dev) if "b" in want else None
    say("backward case %s want=%s gw plan %s" % (sh, want, gi.grad_weight_plan(
        gi.make_params(*sh.as_tuple()[:10]))))
    gi.backward(tg, tx, tw, stride=sh.stride, padding=(sh.pad_h, sh.pad_w),
                kernel_hw=(sh.kH, sh.kW), want_dx="x" in want, want_dw="w" in want,
                want_db="b" in want, dx=dx, dw=dw, db=db)
    torch.cuda.synchronize()
    host = lambda t: None if t is None else t.cpu().numpy().astype(np.float64)
    return host(dx), host(dw), host(db)


def full_check(sh, seed, want):
    x, w, g = inputs(sh, seed)
    dx, dw, db = run_backward(sh, x, w, g, want)
    if "x" in want:
        ref, Ss = oracle.grad_input(g, w, sh.stride, (sh.pad_h, sh.pad_w), (sh.H, sh.W))
        check(dx, ref, Ss, "dx %s" % (sh,))
    if "w" in want:
        ref, Ss = oracle.grad_weight(x, g, sh.stride, (sh.pad_h, sh.pad_w), (sh.kH, sh.kW))
        check(dw, ref, Ss, "dw %s" % (sh,))
    if "b" in want:
        ref, Ss = oracle.grad_bias(g)
        check(db, ref, Ss, "db %s" % (sh,))


SHAPES = [
    S(2, 20, 12, 12, 70, 3, 3, 1, 1, 1),     # 16-byte grad_weight kernel, flat layout
    S(2, 20, 16, 16, 64, 3, 3, 2, 1, 1),     # row-padded layout, stride 2
    S(1, 3, 24, 24, 64, 7, 7, 2, 3, 3),      # flattened column map (stem-like)
    S(2, 16, 7, 7, 70, 7, 7, 1, 3, 3),       # 4-byte grad_weight kernel: separate bias pass
    S(2, 17, 9, 9, 64, 1, 7, 1, 0, 3),       # 1x7, planes not 16-byte aligned
]
WANTS = ["xwb", "wb", "xb", "b", "xw"]


@pytest.mark.parametrize("idx", range(len(SHAPES)))
@pytest.mark.parametrize("want", WANTS)
def test_backward_parity(idx, want):
    full_check(SHAPES[idx], 7000 + idx, want)


@pytest.mark.parametrize("variant", [1, 2])
def test_backward_bias_both_kernels(variant):
    """The bias gradient from the 16-byte kernel's fused sums (2) and from the
    separate per-channel pass beside the 4-byte kernel (1), several groups
    per work-group."""
    gi.set_gw_variant(variant)
    gi.set_gw_tile(0, 0, 2)
    try:
        full_check(S(3, 16, 14, 14, 64, 3, 3, 1, 1, 1), 7100 + variant, "wb")
        full_check(S(2, 16, 12, 16, 64, 3, 3, 2, 1, 1), 7110 + variant, "wb")
    finally:
        gi.set_gw_tile(0, 0, 0)
        gi.set_gw_variant(0)


def test_grad_bias_alone():
    rng = np.random.default_rng(7200)
    for shape in [(1, 1, 1, 1), (3, 5, 7, 9), (64, 130, 14, 14), (2, 3, 200, 150)]:
        g = rng.standard_normal(shape).astype(np.float32)
        out = gi.grad_bias(torch.from_numpy(g).cuda())
        torch.cuda.synchronize()
        ref, Ss = oracle.grad_bias(g)
        check(out.cpu().numpy().astype(np.float64), ref, Ss, "grad_bias %r" % (shape,))


def test_backward_empty_batch_rejected():
    """N = 0 is an invalid shape: the call raises EINVAL and writes nothing."""
    sh = S(1, 5, 6, 6, 7, 3, 3, 1, 1, 1)
    dev = torch.device("cuda:0")
    x = torch.zeros((0, 5, 6, 6), device=dev)
    w = torch.zeros(sh.weight_shape, device=dev)
    g = torch.zeros((0, 7, 6, 6), device=dev)
    dw = torch.full(sh.weight_shape, 3.0, device=dev)
    with pytest.raises(gi.Conv2dGiError) as e:
        gi.backward(g, x, w, stride=1, padding=1, want_db=True, dw=dw)
    assert e.value.code == gi.EINVAL
    torch.cuda.synchronize()
    assert torch.all(dw == 3.0)


def test_backward_null_inputs_rejected():
    sh = S(1, 4, 6, 6, 5, 3, 3, 1, 1, 1)
    p = gi.make_params(*sh.as_tuple()[:10])
    lib = gi.load_library()
    import ctypes
    dev = torch.device("cuda:0")
    g = torch.zeros(sh.grad_out_shape, device=dev)
    d = torch.zeros(sh.dst_shape, device=dev)
    null = ctypes.c_void_p(0)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # dx without the weight, dw without the input, any output without grad_out
    assert lib.conv2d_backward(ptr(g), null, null, ptr(d), null, null, p, s) == 1
    assert lib.conv2d_backward(ptr(g), null, null, null, ptr(d), null, p, s) == 1
    assert lib.conv2d_backward(null, null, null, null, null, ptr(d), p, s) == 1
    assert lib.conv2d_grad_bias(ptr(g), null, p, s) == 1
    # nothing asked: nothing to do
    assert lib.conv2d_backward(null, null, null, null, null, null, p, s) == 0


@pytest.mark.parametrize("name", ["resnet_stage_3x3", "strided_downsample", "stem_7x7_s2",
                                  "asym_1x7", "deep_late_stage"])
def test_backward_workload_sampled(name):
    """Full-size graded shapes: dx and dw at 200 sampled elements, db whole."""
    wl = workloads.BY_NAME[name]
    sh = wl.shape
    g, w = workloads.make_inputs(wl)
    x = workloads.make_forward_input(wl)
    dx, dw, db = run_backward(sh, x, w, g, "xwb")
    rng = np.random.default_rng(zlib.crc32(name.encode()) + 1)
    idx = rng.integers(0, dx.size, size=200)
    ref, Ss = oracle.grad_input_at(g, w, sh.stride, (sh.pad_h, sh.pad_w), (sh.H, sh.W), idx)
    check(dx.ravel()[idx], ref, Ss, "dx " + name)
    idx = rng.integers(0, dw.size, size=200)
    ref, Ss = oracle.grad_weight_at(x, g, sh.stride, (sh.pad_h, sh.pad_w), (sh.kH, sh.kW), idx)
    check(dw.ravel()[idx], ref, Ss, "dw " + name)
    ref, Ss = oracle.grad_bias(g)
    check(db, ref, Ss, "db " + name)
