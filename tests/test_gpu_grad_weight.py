"""GPU parity of grad_weight: the HIP library (through its C ABI) against the
CPU oracle's grad_weight.

Criterion, element by element, S = sum |grad_out * x| over the element's terms:
  |gpu - oracle| <= 1e-5 * S + 1e-6
the same form as grad_input's fp32 criterion: the GPU sums in fp32 over at most
a few thousand terms per slice and adds the slices in order, well inside 1e-5*S.
dw is pre-filled with NaN (an unwritten element fails) and framed by guard
bands that must stay untouched (an out-of-bounds write fails).
"""
import sys

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import conv2d_backward_amd as gi  # noqa: E402

REL, ABS = 1e-5, 1e-6
GUARD = 4096
SENTINEL = 12345.0
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


def run_gw(x_np, g_np, shape):
    """grad_weight on the GPU for numpy inputs: (dw float64, guard bands intact)."""
    dev = torch.device("cuda:0")
    x = torch.from_numpy(np.ascontiguousarray(x_np, dtype=np.float32)).to(dev)
    g = torch.from_numpy(np.ascontiguousarray(g_np, dtype=np.float32)).to(dev)
    n = int(np.prod(shape.weight_shape))
    buf = torch.full((n + 2 * GUARD,), SENTINEL, dtype=torch.float32, device=dev)
    buf[GUARD:GUARD + n] = float("nan")
    out = buf[GUARD:GUARD + n].view(shape.weight_shape)
    gi.grad_weight(g, x, stride=shape.stride, padding=(shape.pad_h, shape.pad_w),
                   kernel_hw=(shape.kH, shape.kW), out=out)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    ok = bool(np.all(host[:GUARD] == SENTINEL) and np.all(host[GUARD + n:] == SENTINEL))
    return host[GUARD:GUARD + n].astype(np.float64).reshape(shape.weight_shape), ok


def check(got, ref, Ssum, what):
    assert not np.isnan(got).any(), "%s: unwritten (NaN) elements" % what
    err = np.abs(got - ref)
    bound = REL * Ssum + ABS
    bad = err > bound
    if bad.any():
        i = int(np.argmax(err - bound))
        raise AssertionError("%s: %d elements out of tolerance; worst flat %d got %r want %r S %r"
                             % (what, int(bad.sum()), i, got.ravel()[i], ref.ravel()[i],
                                Ssum.ravel()[i]))


def full_parity(shape, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape.dst_shape).astype(np.float32)
    g = rng.standard_normal(shape.grad_out_shape).astype(np.float32)
    say("grad_weight case %s seed=%d plan %s" % (shape, seed, gi.grad_weight_plan(
        gi.make_params(*shape.as_tuple()[:10]))))
    got, ok = run_gw(x, g, shape)
    assert ok, "write outside dw"
    ref, Ssum = oracle.grad_weight(x, g, shape.stride, (shape.pad_h, shape.pad_w),
                                   (shape.kH, shape.kW))
    check(got, ref, Ssum, str(shape))


SHAPES = workloads.sweep_shapes() + [
    S(2, 64, 12, 56, 64, 3, 3, 1, 1, 1),     # resnet-stage rows: one row per group
    S(3, 40, 14, 14, 70, 3, 3, 1, 1, 1),     # 14-wide rows, four per group; Co past 64
    S(2, 20, 17, 17, 24, 1, 7, 1, 0, 3),     # 1x7 instance, three rows per group
    S(1, 3, 30, 100, 8, 7, 7, 2, 3, 3),      # stem-like: 2-row tap groups, 64+ pixel rows
    S(2, 18, 9, 130, 5, 3, 3, 1, 1, 1),      # 130-wide rows: three pixel blocks
    S(1, 4, 6, 9, 3, 2, 16, 1, 0, 7),        # kW = 16: one kernel row per tap group
    S(3, 17, 11, 13, 9, 4, 4, 2, 1, 2),      # run-time tap grid, stride 2, pad_h != pad_w
    S(70, 16, 4, 4, 64, 3, 3, 1, 1, 1),      # many small images: one group per slice
]


@pytest.mark.parametrize("idx", range(len(SHAPES)))
def test_grad_weight_parity(idx):
    full_parity(SHAPES[idx], 5000 + idx)


# Shapes for the 16-byte-load kernel's layouts and column maps.
GWD_SHAPES = [
    S(2, 20, 12, 12, 70, 3, 3, 1, 1, 1),     # flat 3x3: ragged Co and Ci blocks
    S(2, 17, 9, 9, 64, 1, 7, 1, 0, 3),       # flat 1x7: planes not 16-byte aligned
    S(3, 16, 14, 14, 64, 3, 3, 1, 1, 1),     # flat 14x14: groups end inside a K block
    S(2, 20, 16, 16, 64, 3, 3, 2, 1, 1),     # row-padded, tap map, stride 2
    S(2, 16, 10, 16, 64, 3, 3, 1, 0, 1),     # row-padded, tap map, stride 1 (oH != H)
    S(1, 16, 8, 40, 64, 3, 3, 2, 1, 1),      # row-padded: two 16-pixel segments per row
    S(1, 3, 24, 24, 64, 7, 7, 2, 3, 3),      # flattened map, stride 2 (stem-like)
    S(1, 5, 16, 16, 20, 5, 5, 1, 2, 2),      # flattened map, any stride (1)
    S(1, 4, 12, 12, 8, 2, 3, 3, 1, 1),       # flattened map, stride 3
    S(2, 24, 8, 8, 130, 3, 3, 1, 1, 1),      # three Co blocks, last one ragged
    S(2, 20, 21, 36, 70, 3, 3, 1, 1, 1),     # flat, 36-pixel rows: unmasked K blocks
    S(1, 16, 18, 18, 64, 3, 3, 1, 1, 1),     # flat, 18-pixel rows: one unmasked column
    S(2, 16, 9, 24, 64, 1, 3, 1, 0, 1),      # flat 1x3 on 24-pixel rows
]


@pytest.mark.parametrize("idx", range(len(GWD_SHAPES)))
def test_grad_weight_parity_16byte_loads(idx):
    sh = GWD_SHAPES[idx]
    gi.set_gw_variant(2)
    try:
        full_parity(sh, 6000 + idx)
    finally:
        gi.set_gw_variant(0)


@pytest.mark.parametrize("idx", range(len(GWD_SHAPES)))
def test_grad_weight_parity_4byte_loads(idx):
    gi.set_gw_variant(1)
    try:
        full_parity(GWD_SHAPES[idx], 6100 + idx)
    finally:
        gi.set_gw_variant(0)


@pytest.mark.parametrize("rows,stages,slices", [(1, 1, 0), (2, 1, 3), (3, 2, 2), (5, 2, 0),
                                               (14, 1, 1), (4, 2, 1)])
def test_grad_weight_forced_tiles(rows, stages, slices):
    """Forced rows per group, LDS stages and slices (several groups per
    work-group through both pipelines) on the 16-byte-load kernel."""
    gi.set_gw_variant(2)
    gi.set_gw_tile(rows, stages, slices)
    try:
        full_parity(S(2, 16, 14, 14, 64, 3, 3, 1, 1, 1), 6200 + rows)
        full_parity(S(2, 16, 12, 16, 64, 3, 3, 2, 1, 1), 6300 + rows)
    finally:
        gi.set_gw_tile(0, 0)
        gi.set_gw_variant(0)


def test_grad_weight_empty_batch_rejected():
    sh = S(0, 5, 6, 6, 7, 3, 3, 1, 1, 1)
    with pytest.raises(gi.Conv2dGiError) as e:
        run_gw(np.zeros(sh.dst_shape, np.float32), np.zeros(sh.grad_out_shape, np.float32), sh)
    assert e.value.code == gi.EINVAL


def test_grad_weight_wide_kernels():
    """kW = 17: past the 4-byte-load kernel's tap limit (it rejects the
    shape); the 16-byte-load kernel's flattened map serves it."""
    sh = S(1, 2, 4, 40, 2, 1, 17, 1, 0, 8)
    gi.set_gw_variant(1)
    try:
        with pytest.raises(gi.Conv2dGiError):
            run_gw(np.zeros(sh.dst_shape, np.float32), np.zeros(sh.grad_out_shape, np.float32),
                   sh)
    finally:
        gi.set_gw_variant(0)
    full_parity(sh, 6400)


GRADED = ["resnet_stage_3x3", "strided_downsample", "stem_7x7_s2", "asym_1x7",
          "deep_late_stage"]


@pytest.mark.parametrize("name", GRADED)
def test_grad_weight_workload_sampled(name):
    """Full-size graded shapes (seeded synthetic inputs): 200 sampled elements."""
    wl = workloads.BY_NAME[name]
    sh = wl.shape
    g, _ = workloads.make_inputs(wl)
    x = workloads.make_forward_input(wl)
    say("grad_weight workload %s plan %s" % (name, gi.grad_weight_plan(
        gi.make_params(*sh.as_tuple()[:10]))))
    got, ok = run_gw(x, g, sh)
    assert ok and not np.isnan(got).any()
    rng = np.random.default_rng(zlib_seed(name))
    idx = rng.integers(0, got.size, size=200)
    ref, Ssum = oracle.grad_weight_at(x, g, sh.stride, (sh.pad_h, sh.pad_w), (sh.kH, sh.kW), idx)
    check(got.ravel()[idx], ref, Ssum, name)


def zlib_seed(name):
    import zlib
    return zlib.crc32(name.encode())
