"""GPU parity of the forward convolution (through the C ABI) against the CPU
oracle's separately written forward, on both paths (stride 1 on the
grad_input kernels with the transposed, reversed weight; the generic forward
kernel for every shape), and a GPU-side adjoint check of the forward against
grad_input.  Criterion: |gpu - oracle| <= 1e-5 * S + 1e-6 per element, S the
sum of |x * w| over the element's terms.
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
    assert not np.isnan(got).any(), "%s: NaN (unwritten) elements" % what
    err = np.abs(got - ref)
    bad = err > REL * Ssum + ABS
    if bad.any():
        i = int(np.argmax(err - (REL * Ssum + ABS)))
        raise AssertionError("%s: %d elements out of tolerance; worst flat %d got %r want %r"
                             % (what, int(bad.sum()), i, got.ravel()[i], ref.ravel()[i]))


def run_fwd(sh, x, w):
    dev = torch.device("cuda:0")
    tx, tw = torch.from_numpy(x).to(dev), torch.from_numpy(w).to(dev)
    out = torch.full(sh.grad_out_shape, float("nan"), device=dev)
    say("forward case %s plan %s" % (sh, gi.forward_plan(gi.make_params(*sh.as_tuple()[:10]))))
    gi.forward(tx, tw, stride=sh.stride, padding=(sh.pad_h, sh.pad_w), out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def full_check(sh, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(sh.dst_shape).astype(np.float32)
    w = rng.standard_normal(sh.weight_shape).astype(np.float32)
    got = run_fwd(sh, x, w)
    ref, Ss = oracle.conv2d_forward_abs(x, w, sh.stride, (sh.pad_h, sh.pad_w))
    check(got, ref, Ss, str(sh))


SHAPES = [
    S(2, 20, 12, 12, 70, 3, 3, 1, 1, 1),     # same-size 3x3; Co past one 64 tile
    S(2, 16, 10, 9, 24, 3, 3, 1, 0, 0),      # no padding
    S(1, 18, 9, 11, 16, 3, 3, 1, 2, 2),      # pad = k - 1 (largest on the grad_input path)
    S(1, 8, 9, 9, 12, 3, 3, 1, 3, 3),        # pad > k - 1: generic kernel
    S(2, 17, 9, 9, 64, 1, 7, 1, 0, 3),       # 1x7
    S(2, 20, 16, 16, 64, 3, 3, 2, 1, 1),     # stride 2
    S(1, 3, 24, 24, 64, 7, 7, 2, 3, 3),      # stem-like, Ci = 3
    S(1, 4, 12, 13, 8, 2, 3, 3, 1, 1),       # stride 3, even kernel height
    S(2, 5, 11, 10, 3, 5, 5, 1, 2, 2),       # Co = 3 (grad_input path: its stem kernel)
    S(3, 33, 7, 6, 130, 3, 2, 2, 1, 0),      # ragged channel tiles, asymmetric pads
    # Generic-kernel paths: channel-block-major K with kH != kW, 16-byte weight
    # loads (Co % 4 == 0) with a partial output-channel tile, the flattened K
    # just below 16 input channels, an odd output width, a partial last
    # channel block.
    S(2, 16, 9, 11, 68, 2, 3, 3, 1, 1),      # Ci = 16: one block; Co = 68: 64 + 4
    S(1, 15, 10, 10, 4, 3, 3, 2, 1, 1),      # Ci = 15: flattened K; Co = 4; oW = 5
    S(2, 40, 9, 9, 36, 3, 3, 2, 0, 0),       # blocks of 16, 16, 8 channels; Co = 36
]


@pytest.mark.parametrize("idx", range(len(SHAPES)))
def test_forward_parity(idx):
    full_check(SHAPES[idx], 8000 + idx)


@pytest.mark.parametrize("idx", range(len(SHAPES)))
def test_forward_parity_generic(idx):
    gi.set_fwd_variant(2)
    try:
        full_check(SHAPES[idx], 8100 + idx)
    finally:
        gi.set_fwd_variant(0)


def test_forward_variant_hook_rejects_strided():
    gi.set_fwd_variant(1)
    try:
        with pytest.raises(gi.Conv2dGiError):
            gi.forward_plan(gi.make_params(1, 4, 8, 8, 4, 3, 3, 2, 1, 1))
    finally:
        gi.set_fwd_variant(0)


def test_forward_empty_batch_rejected():
    dev = torch.device("cuda:0")
    with pytest.raises(gi.Conv2dGiError) as e:
        gi.forward(torch.zeros((0, 4, 6, 6), device=dev), torch.zeros((5, 4, 3, 3), device=dev),
                   stride=1, padding=1)
    assert e.value.code == gi.EINVAL


@pytest.mark.parametrize("idx", [0, 5, 6])
def test_forward_adjoint_on_gpu(idx):
    """<forward(x, w), g> = <x, grad_input(g, w)> with both sides computed by
    the library on the GPU (inner products in float64 on the host)."""
    sh = SHAPES[idx]
    rng = np.random.default_rng(8200 + idx)
    dev = torch.device("cuda:0")
    x = torch.from_numpy(rng.standard_normal(sh.dst_shape).astype(np.float32)).to(dev)
    w = torch.from_numpy(rng.standard_normal(sh.weight_shape).astype(np.float32)).to(dev)
    g = torch.from_numpy(rng.standard_normal(sh.grad_out_shape).astype(np.float32)).to(dev)
    y = gi.forward(x, w, stride=sh.stride, padding=(sh.pad_h, sh.pad_w))
    dx = gi.grad_input(g, w, stride=sh.stride, padding=(sh.pad_h, sh.pad_w),
                       input_hw=(sh.H, sh.W))
    torch.cuda.synchronize()
    yd, gd = y.double().cpu().numpy(), g.double().cpu().numpy()
    xd, dxd = x.double().cpu().numpy(), dx.double().cpu().numpy()
    lhs, rhs = float(np.sum(yd * gd)), float(np.sum(xd * dxd))
    scale = float(np.sum(np.abs(yd * gd))) + float(np.sum(np.abs(xd * dxd)))
    assert abs(lhs - rhs) <= 1e-5 * scale, (lhs, rhs, scale)


@pytest.mark.parametrize("name", ["resnet_stage_3x3", "strided_downsample", "stem_7x7_s2",
                                  "asym_1x7", "deep_late_stage"])
def test_forward_workload_sampled(name):
    """Full-size graded shapes (forward input and weight of the workload):
    200 sampled outputs."""
    wl = workloads.BY_NAME[name]
    sh = wl.shape
    _, w = workloads.make_inputs(wl)
    x = workloads.make_forward_input(wl)
    got = run_fwd(sh, x, w)
    rng = np.random.default_rng(zlib.crc32(name.encode()) + 2)
    idx = rng.integers(0, got.size, size=200)
    ref, Ss = oracle.conv2d_forward_at(x, w, sh.stride, (sh.pad_h, sh.pad_w), idx)
    check(got.ravel()[idx], ref, Ss, name)


def test_forward_threads_one_stream():
    """Forward calls from four host threads on the same stream, each with its
    own weight: the stride-1 path stages the tap-reversed weight in a scratch
    slot shared per stream, so a call must keep the slot until its
    grad_input kernel is enqueued.  Every call writes its own output, and
    every output is checked against the oracle."""
    import threading
    sh = S(2, 16, 10, 10, 24, 3, 3, 1, 1, 1)
    dev = torch.device("cuda:0")
    nthreads, calls = 4, 8
    rng = np.random.default_rng(8300)
    x = rng.standard_normal(sh.dst_shape).astype(np.float32)
    ws = [rng.standard_normal(sh.weight_shape).astype(np.float32) for _ in range(nthreads)]
    tx = torch.from_numpy(x).to(dev)
    tws = [torch.from_numpy(w).to(dev) for w in ws]
    outs = [[torch.full(sh.grad_out_shape, float("nan"), device=dev) for _ in range(calls)]
            for _ in range(nthreads)]
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    errors = []

    def worker(t):
        try:
            for c in range(calls):
                gi.forward(tx, tws[t], stride=1, padding=1, out=outs[t][c], stream=stream)
        except Exception as e:  # reported after the join
            errors.append(e)

    say("forward threads: %d threads x %d calls, shape %s" % (nthreads, calls, sh))
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(nthreads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for t in range(nthreads):
        ref, Ss = oracle.conv2d_forward_abs(x, ws[t], sh.stride, (sh.pad_h, sh.pad_w))
        for c in range(calls):
            check(outs[t][c].double().cpu().numpy(), ref, Ss, "thread %d call %d" % (t, c))
