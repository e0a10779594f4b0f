"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Criteria (element by element, S = sum |grad_out * weight| over the element's terms):
  fp32 inputs:  |gpu - oracle| <= 1e-5 * S + 1e-6
  bf16 inputs:  ||gpu - oracle||_2 <= 1e-2 * ||oracle||_2  and
                |gpu - oracle| <= 1e-2 * S + 1e-6        (oracle on the same bf16 values)
  fp16 inputs:  |gpu - oracle| <= 1e-5 * S + 1e-6        (oracle on the same fp16 values:
                products of two fp16 values are exact in fp32 and the sums are fp32,
                so the fp32 criterion applies)
dst is pre-filled with NaN (an unwritten element fails) and framed by guard
bands that must stay untouched (an out-of-bounds write fails).
"""
import os
import sys
import zlib

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import conv2d_backward_amd as gi  # noqa: E402

F32_REL, F32_ABS = 1e-5, 1e-6
BF16_REL, BF16_ABS = 1e-2, 1e-6
GUARD = 4096
SENTINEL = 12345.0


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gi.load_library()
    return torch.device("cuda:0")


def run_gpu(g_np, w_np, shape, dtype, variant=gi.VARIANT_AUTO, stream=None):
    """Run the library on numpy inputs; returns (dst numpy float64, guard ok)."""
    dev = torch.device("cuda:0")
    if dtype in ("bf16", "f16"):
        t16 = torch.bfloat16 if dtype == "bf16" else torch.float16
        g = torch.from_numpy(g_np.view(np.int16)).to(dev).view(t16)
        w = torch.from_numpy(w_np.view(np.int16)).to(dev).view(t16)
    else:
        g = torch.from_numpy(np.ascontiguousarray(g_np, dtype=np.float32)).to(dev)
        w = torch.from_numpy(np.ascontiguousarray(w_np, dtype=np.float32)).to(dev)
    n_dst = int(np.prod(shape.dst_shape))
    buf = torch.full((n_dst + 2 * GUARD,), SENTINEL, dtype=torch.float32, device=dev)
    buf[GUARD:GUARD + n_dst] = float("nan")
    out = buf[GUARD:GUARD + n_dst].view(shape.dst_shape)
    old = gi.set_variant(variant)
    if stream is not None:
        # The library orders work within the caller's stream only: the fills
        # above are queued on the current stream, so the side stream waits.
        stream.wait_stream(torch.cuda.current_stream())
    try:
        gi.grad_input(g, w, stride=shape.stride, padding=(shape.pad_h, shape.pad_w),
                      input_hw=(shape.H, shape.W), out=out, stream=stream)
        torch.cuda.synchronize()
    finally:
        gi.set_variant(old)
    host = buf.cpu().numpy()
    guard_ok = bool(np.all(host[:GUARD] == SENTINEL) and np.all(host[GUARD + n_dst:] == SENTINEL))
    return host[GUARD:GUARD + n_dst].astype(np.float64).reshape(shape.dst_shape), guard_ok


def oracle_inputs(g_np, w_np, dtype):
    if dtype == "bf16":
        return workloads.bf16_to_f32(g_np), workloads.bf16_to_f32(w_np)
    if dtype == "f16":
        return workloads.f16_to_f32(g_np), workloads.f16_to_f32(w_np)
    return g_np, w_np


def check(got, ref, S, dtype, what):
    assert not np.isnan(got).any(), "%s: unwritten (NaN) elements" % what
    err = np.abs(got - ref)
    if dtype == "bf16":
        bound = BF16_REL * S + BF16_ABS
        nrm = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
        assert nrm <= BF16_REL, "%s: normwise rel err %.3g" % (what, nrm)
    else:
        bound = F32_REL * S + F32_ABS
    bad = err > bound
    if bad.any():
        i = int(np.argmax(err - bound))
        raise AssertionError("%s: %d elements out of tolerance; worst flat %d got %r want %r S %r"
                             % (what, int(bad.sum()), i, got.ravel()[i], ref.ravel()[i],
                                S.ravel()[i]))
    return float(np.max(err / (bound)))


def full_parity(shape, seed, dtype, variant=gi.VARIANT_AUTO, dist="uniform"):
    g, w = workloads.make_case(shape, seed, dist)
    if dtype == "bf16":
        g, w = workloads.bf16_bits(g), workloads.bf16_bits(w)
    elif dtype == "f16":
        g, w = workloads.f16_bits(g), workloads.f16_bits(w)
    say("case %s dtype=%s variant=%d seed=%d" % (shape, dtype, variant, seed))
    got, guard_ok = run_gpu(g, w, shape, dtype, variant)
    assert guard_ok, "write outside dst"
    go, wo = oracle_inputs(g, w, dtype)
    ref, S = oracle.grad_input(go, wo, shape.stride, (shape.pad_h, shape.pad_w),
                               (shape.H, shape.W))
    return check(got, ref, S, dtype, str(shape))


SWEEP = workloads.sweep_shapes()


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("idx", range(len(SWEEP)))
def test_sweep(idx, dtype):
    full_parity(SWEEP[idx], 100 + idx, dtype)


# Mid-size shapes: several tiles in every direction plus ragged tails.
MID = [
    workloads.Shape(2, 130, 20, 21, 96, 3, 3, 1, 1, 1),
    workloads.Shape(3, 64, 17, 17, 80, 1, 7, 1, 0, 3),
    workloads.Shape(2, 100, 23, 22, 72, 3, 3, 2, 1, 1),
    workloads.Shape(2, 3, 45, 44, 64, 7, 7, 2, 3, 3),
    workloads.Shape(1, 200, 9, 9, 300, 3, 3, 1, 1, 1),
    workloads.Shape(2, 48, 30, 30, 40, 5, 5, 3, 2, 2),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("idx", range(len(MID)))
def test_mid(idx, dtype):
    full_parity(MID[idx], 500 + idx, dtype, dist="normal")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_forced_generic(dtype):
    for i, s in enumerate([SWEEP[4], SWEEP[9], MID[0], MID[2]]):
        full_parity(s, 900 + i, dtype, gi.VARIANT_GENERIC)


HALO_SHAPES = [s for s in SWEEP + MID if s.Ci >= 16] + [
    workloads.Shape(2, 16, 9, 9, 5, 3, 3, 1, 1, 1),      # Co below one channel chunk
    workloads.Shape(1, 20, 33, 70, 9, 3, 3, 1, 1, 1),     # wide rows: several column tiles
    workloads.Shape(3, 24, 11, 13, 12, 5, 5, 2, 2, 2),    # stride 2, 5x5
    workloads.Shape(2, 17, 10, 9, 6, 2, 3, 3, 0, 1),      # stride 3: phases with different taps
    workloads.Shape(4, 32, 7, 7, 40, 1, 3, 1, 0, 1),      # 1xk: tile rows fold across images
    workloads.Shape(1, 64, 6, 6, 8, 2, 3, 1, 0, 0),       # even kernel, no padding
]


@pytest.mark.parametrize("idx", range(len(HALO_SHAPES)))
def test_forced_halo(idx):
    s = HALO_SHAPES[idx]
    gi.set_variant(gi.VARIANT_HALO)
    desc = gi.plan(gi.make_params(*s.as_tuple()[:10]), False)
    gi.set_variant(gi.VARIANT_AUTO)
    assert "variant=halo" in desc, desc
    full_parity(s, 1300 + idx, "f32", gi.VARIANT_HALO, dist="normal")


HALO_BF16_SHAPES = [
    MID[0],                                                # ragged Ci tiles, 3 chunks
    MID[4],                                                # Co = 300: partial last chunk
    workloads.Shape(2, 16, 9, 9, 5, 3, 3, 1, 1, 1),       # Co below one chunk
    workloads.Shape(3, 40, 17, 17, 50, 1, 3, 1, 0, 1),    # 1x3
    workloads.Shape(2, 24, 11, 13, 12, 3, 1, 1, 1, 0),    # 3x1
    workloads.Shape(1, 64, 6, 6, 8, 3, 3, 1, 0, 0),       # pad 0
    workloads.Shape(1, 32, 6, 6, 16, 3, 3, 1, 3, 3),      # pad beyond kernel - 1
    workloads.Shape(2, 64, 14, 14, 64, 3, 3, 1, 1, 1),    # the deep-stage tile
    workloads.Shape(1, 70, 31, 40, 33, 3, 3, 1, 1, 1),    # several tiles per image
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("idx", range(len(HALO_BF16_SHAPES)))
def test_forced_halo_bf16(idx, dtype):
    s = HALO_BF16_SHAPES[idx]
    gi.set_variant(gi.VARIANT_HALO)
    desc = gi.plan(gi.make_params(*s.as_tuple()[:10]), 1 if dtype == "bf16" else 2)
    gi.set_variant(gi.VARIANT_AUTO)
    assert "variant=halo" in desc and ("dtype=" + dtype) in desc, desc
    full_parity(s, 1500 + idx, dtype, gi.VARIANT_HALO, dist="normal")


# The whole-image 16-bit kernel (forced with its 13 pixel blocks): ragged
# input-channel tiles, a partial last output-channel chunk, pad 0 and pad 2
# (grad_out planes smaller and larger than the image), short images, an odd
# batch and four 128-channel tiles.
IMAGE_SHAPES = [
    workloads.Shape(2, 64, 14, 14, 64, 3, 3, 1, 1, 1),
    workloads.Shape(3, 130, 14, 14, 70, 3, 3, 1, 1, 1),
    workloads.Shape(2, 40, 8, 14, 33, 3, 3, 1, 0, 0),
    workloads.Shape(1, 24, 12, 14, 16, 3, 3, 1, 2, 2),
    workloads.Shape(2, 512, 14, 14, 40, 3, 3, 1, 1, 1),
    workloads.Shape(5, 128, 14, 14, 96, 3, 3, 1, 1, 1),
    workloads.Shape(2, 16, 2, 14, 8, 3, 3, 1, 1, 1),
    workloads.Shape(2, 64, 14, 14, 128, 3, 3, 1, 1, 1),     # 4 chunks: one past a stage cycle
    workloads.Shape(1, 64, 14, 14, 160, 3, 3, 1, 1, 1),     # 5 chunks
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("idx", range(len(IMAGE_SHAPES)))
def test_forced_image_kernel(idx, dtype):
    s = IMAGE_SHAPES[idx]
    gi.set_halo_tile(13, s.H, s.W, 0)
    try:
        desc = gi.plan(gi.make_params(*s.as_tuple()[:10]), 1 if dtype == "bf16" else 2)
        assert "image kernel" in desc, desc
        full_parity(s, 1600 + idx, dtype, gi.VARIANT_AUTO, dist="normal")
    finally:
        gi.set_halo_tile()


STEM_SHAPES = [
    workloads.Shape(2, 3, 45, 44, 64, 7, 7, 2, 3, 3),      # stem-like, ragged tiles
    workloads.Shape(1, 4, 20, 19, 7, 3, 3, 1, 1, 1),       # Ci = 4, Co not a multiple of 4
    workloads.Shape(3, 1, 17, 33, 9, 4, 4, 1, 1, 2),       # 4x4 stride 1 (16 taps), Ci = 1
    workloads.Shape(1, 2, 12, 18, 5, 2, 4, 1, 0, 1),       # 2x4 (8 taps)
    workloads.Shape(2, 3, 9, 40, 6, 1, 3, 1, 0, 1),        # 1x3
    workloads.Shape(1, 3, 23, 21, 10, 3, 3, 2, 1, 1),      # stride 2, odd sizes
    workloads.Shape(1, 3, 30, 30, 13, 5, 5, 2, 2, 2),      # 5x5 stride 2: 9, 6, 6, 4 taps
    workloads.Shape(2, 2, 11, 10, 3, 2, 2, 3, 0, 0),       # kernel < stride: empty phases
    workloads.Shape(1, 3, 40, 36, 64, 7, 7, 2, 3, 3),      # several tiles per phase
    workloads.Shape(1, 3, 1, 40, 8, 7, 7, 2, 3, 3),        # one image row: one phase group
    workloads.Shape(1, 3, 36, 36, 8, 6, 6, 2, 3, 3),       # phases' halos at different origins
    workloads.Shape(2, 3, 20, 30, 8, 1, 6, 1, 0, 2),       # 1x6: run-time pitch, one group
    workloads.Shape(1, 3, 20, 40, 10, 2, 12, 2, 0, 5),     # 2x12 stride 2: run-time pitch, two groups
    workloads.Shape(70, 3, 34, 34, 8, 7, 7, 2, 3, 3),      # whole tiles, then quarter tiles
    workloads.Shape(65, 3, 20, 20, 5, 3, 3, 1, 1, 1),      # the same with one phase group
]


@pytest.mark.parametrize("idx", range(len(STEM_SHAPES)))
def test_forced_stem(idx):
    s = STEM_SHAPES[idx]
    gi.set_variant(gi.VARIANT_STEM)
    desc = gi.plan(gi.make_params(*s.as_tuple()[:10]), False)
    gi.set_variant(gi.VARIANT_AUTO)
    assert "variant=stem" in desc, desc
    full_parity(s, 1900 + idx, "f32", gi.VARIANT_STEM, dist="normal")


COL2IM_SHAPES = [
    workloads.Shape(2, 3, 45, 44, 64, 7, 7, 2, 3, 3),      # stem-like, ragged tiles
    workloads.Shape(1, 3, 40, 36, 64, 7, 7, 2, 3, 3),      # several tiles per image
    workloads.Shape(2, 3, 23, 19, 50, 7, 7, 2, 3, 3),      # Co not a multiple of 4, W % 4 != 0
    workloads.Shape(1, 4, 17, 30, 64, 3, 3, 1, 1, 1),      # stride 1
    workloads.Shape(1, 10, 9, 13, 60, 3, 4, 1, 0, 2),      # Ci = 10, kH != kW
    workloads.Shape(1, 2, 11, 14, 57, 5, 8, 2, 4, 1),      # pad > k - 1, kW = 4 * stride
    workloads.Shape(1, 1, 7, 7, 64, 2, 2, 2, 2, 2),        # kernel = stride, pad = k
    workloads.Shape(1, 3, 30, 30, 64, 7, 7, 2, 0, 6),      # asymmetric pads
    workloads.Shape(3, 16, 14, 14, 49, 3, 3, 1, 1, 1),     # 144 columns
    workloads.Shape(1, 3, 1, 40, 64, 7, 7, 2, 3, 3),       # one image row
    workloads.Shape(1, 5, 50, 9, 64, 2, 3, 1, 1, 0),       # tall, narrow, even kernel
    workloads.Shape(300, 3, 8, 8, 64, 3, 3, 1, 1, 1),      # more work-groups than CUs
    workloads.Shape(2, 1, 30, 31, 64, 1, 1, 1, 0, 0),      # 1 x 1: one column
    workloads.Shape(1, 6, 19, 21, 64, 5, 5, 2, 2, 2),      # 150 columns: last block partial
    workloads.Shape(1, 3, 224, 224, 64, 7, 7, 2, 3, 3),    # one stem image at full size
    workloads.Shape(2, 1, 33, 29, 64, 7, 7, 2, 3, 3),      # 49 columns: a 1-column tail
    workloads.Shape(1, 2, 26, 31, 52, 7, 7, 2, 3, 3),      # 98 columns: a 2-column tail, Co % 4 = 0
    workloads.Shape(1, 4, 21, 18, 61, 5, 5, 2, 2, 2),      # 100 columns: a 4-column tail, ragged Co
    workloads.Shape(2, 4, 13, 15, 64, 3, 3, 1, 1, 1),      # 36 columns: tail at stride 1
]


@pytest.mark.parametrize("idx", range(len(COL2IM_SHAPES)))
def test_forced_col2im(idx):
    s = COL2IM_SHAPES[idx]
    gi.set_variant(gi.VARIANT_COL2IM)
    desc = gi.plan(gi.make_params(*s.as_tuple()[:10]), False)
    gi.set_variant(gi.VARIANT_AUTO)
    assert "variant=col2im" in desc, desc
    full_parity(s, 2100 + idx, "f32", gi.VARIANT_COL2IM, dist="normal")


# (shape, nb, tile_rows, tile_cols): tiles with ragged row and column tails,
# tiles wider than the image, rows folded across images, strided phases.
FORCED_TILES = [
    (MID[0], 8, 3, 11),
    (MID[0], 13, 6, 29),
    (MID[0], 13, 8, 25),
    (MID[0], 4, 1, 50),
    (workloads.Shape(4, 32, 7, 7, 40, 1, 3, 1, 0, 1), 8, 5, 7),
    (workloads.Shape(4, 32, 7, 7, 40, 1, 3, 1, 0, 1), 13, 9, 3),
    (MID[2], 8, 4, 5),
    (MID[2], 13, 12, 12),
    (MID[5], 13, 6, 7),
    (workloads.Shape(3, 70, 31, 33, 20, 3, 3, 2, 1, 1), 4, 3, 17),
    (workloads.Shape(2, 64, 14, 14, 24, 3, 3, 1, 1, 1), 13, 14, 14),   # the deep-stage tile
    (workloads.Shape(2, 70, 28, 28, 40, 3, 3, 2, 1, 1), 13, 14, 14),   # the downsample tile
]


@pytest.mark.parametrize("idx", range(len(FORCED_TILES)))
def test_forced_halo_tile(idx):
    s, nb, tr, tc = FORCED_TILES[idx]
    gi.set_halo_tile(nb, tr, tc, 0)
    try:
        gi.set_variant(gi.VARIANT_HALO)
        desc = gi.plan(gi.make_params(*s.as_tuple()[:10]), False)
        gi.set_variant(gi.VARIANT_AUTO)
        assert "variant=halo" in desc and ("tile=%dx%d" % (tr, tc)) in desc, desc
        full_parity(s, 1700 + idx, "f32", gi.VARIANT_HALO, dist="normal")
    finally:
        gi.set_halo_tile()


# Every compile-time kernel instance on ragged channel counts (the planner
# choices are pinned by tests/test_planner.py).
from test_planner import FIXED_INSTANCES  # noqa: E402


@pytest.mark.parametrize("idx", range(len(FIXED_INSTANCES)))
def test_fixed_instances(idx):
    shape, bf16, variant, tile, parts = FIXED_INSTANCES[idx]
    if tile:
        gi.set_halo_tile(tile[0], tile[1], tile[2], 0)
        gi.set_halo_split(tile[3])
        gi.set_halo_fusion(tile[4])
    try:
        gi.set_variant(variant)
        desc = gi.plan(gi.make_params(*shape.as_tuple()[:10]), bf16)
        gi.set_variant(gi.VARIANT_AUTO)
        for part in parts:
            assert part in desc, (part, desc)
        full_parity(shape, 2100 + idx, "bf16" if bf16 else "f32", variant, dist="normal")
    finally:
        gi.set_variant(gi.VARIANT_AUTO)
        gi.set_halo_tile()
        gi.set_halo_split()
        gi.set_halo_fusion()


def test_tiny_workload_full():
    wl = workloads.BY_NAME["tiny"]
    s = wl.shape
    g, w = workloads.make_inputs(wl)
    got, ok = run_gpu(g, w, s, "f32")
    assert ok
    ref, S = oracle.grad_input(g, w, s.stride, (s.pad_h, s.pad_w), (s.H, s.W))
    check(got, ref, S, "f32", "tiny")


def sample_indices(shape, rng, count=6000):
    """Random flat indices plus structured ones: every corner/edge pixel of the
    first and last image on the first and last channels, and channel tile edges."""
    N, Ci, H, W = shape.dst_shape
    idx = list(rng.integers(0, N * Ci * H * W, size=count))
    for n in {0, N - 1}:
        for ci in sorted({0, 31, 32, 63, 64, Ci - 1} & set(range(Ci))):
            for ih in {0, 1, H // 2, H - 2, H - 1} & set(range(H)):
                for iw in {0, 1, W // 2, W - 2, W - 1} & set(range(W)):
                    idx.append(((n * Ci + ci) * H + ih) * W + iw)
    return np.array(idx, dtype=np.int64)


@pytest.mark.parametrize("name", [w.name for w in workloads.WORKLOADS if w.name != "tiny"])
def test_workload_sampled(name):
    """Full-size workloads, launched as the benchmark launches them; checked on
    sampled elements against the oracle, and every element for NaN (unwritten)."""
    wl = workloads.BY_NAME[name]
    s = wl.shape
    g, w = workloads.make_inputs(wl)
    say("workload %s" % name)
    got, ok = run_gpu(g, w, s, wl.dtype)
    assert ok, "write outside dst"
    assert not np.isnan(got).any()
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    idx = sample_indices(s, rng)
    go, wo = oracle_inputs(g, w, wl.dtype)
    ref, S = oracle.grad_input_at(go, wo, s.stride, (s.pad_h, s.pad_w), (s.H, s.W), idx)
    check(got.ravel()[idx], ref, S, wl.dtype, name)


def test_deterministic():
    s = MID[0]
    g, w = workloads.make_case(s, 77, "normal")
    a, _ = run_gpu(g, w, s, "f32")
    b, _ = run_gpu(g, w, s, "f32")
    assert np.array_equal(a, b)


def test_zero_output_channels_rejected():
    """Co = 0 is an invalid shape: EINVAL, and dst keeps what it held."""
    s = workloads.Shape(2, 5, 6, 6, 0, 3, 3, 1, 1, 1)
    g = np.zeros(s.grad_out_shape, np.float32)
    w = np.zeros(s.weight_shape, np.float32)
    with pytest.raises(gi.Conv2dGiError) as e:
        run_gpu(g, w, s, "f32")
    assert e.value.code == gi.EINVAL


def test_side_stream():
    s = SWEEP[6]
    g, w = workloads.make_case(s, 5, "uniform")
    side = torch.cuda.Stream()
    got, ok = run_gpu(g, w, s, "f32", stream=side)
    ref, S = oracle.grad_input(g, w, s.stride, (s.pad_h, s.pad_w), (s.H, s.W))
    assert ok
    check(got, ref, S, "f32", "side stream")


def test_invalid_leaves_dst_untouched():
    """H = 9 with pad 1 and a 3x3 kernel gives oH = 9, but grad_out has oH = 8:
    the call fails with EINVAL and launches nothing."""
    dev = torch.device("cuda:0")
    g = torch.randn(1, 4, 8, 8, device=dev)
    w = torch.randn(4, 3, 3, 3, device=dev)
    out = torch.full((1, 3, 9, 8), 7.0, device=dev)
    with pytest.raises(gi.Conv2dGiError) as e:
        gi.grad_input(g, w, stride=1, padding=1, input_hw=(9, 8), out=out)
    assert e.value.code == gi.EINVAL
    with pytest.raises(ValueError):
        gi.grad_input(g, w.to(torch.bfloat16), stride=1, padding=1, input_hw=(8, 8))
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_generic_past_2gib_sampled():
    """dst of exactly 2^31 bytes (N=8, Ci=64, 1024 x 1024): past the halo
    kernels' 32-bit byte offsets, so the planner takes the generic kernel with
    64-bit batch offsets.  Every element is checked for NaN (unwritten) and
    the guard bands for stray writes on the GPU; sampled elements (random,
    plus corners and edges of the first and last image) against the oracle."""
    s = workloads.Shape(8, 64, 1024, 1024, 16, 3, 3, 1, 1, 1)
    n_dst = s.N * s.Ci * s.H * s.W
    assert n_dst * 4 == 2 ** 31
    desc = gi.plan(gi.make_params(*s.as_tuple()[:10]), False)
    assert "variant=generic" in desc, desc
    g, w = workloads.make_case(s, 4711, "normal")
    dev = torch.device("cuda:0")
    tg, tw = torch.from_numpy(g).to(dev), torch.from_numpy(w).to(dev)
    buf = torch.full((n_dst + 2 * GUARD,), SENTINEL, dtype=torch.float32, device=dev)
    buf[GUARD:GUARD + n_dst] = float("nan")
    out = buf[GUARD:GUARD + n_dst].view(s.dst_shape)
    say("case %s (2 GiB dst) plan %s" % (s, desc))
    gi.grad_input(tg, tw, stride=1, padding=1, input_hw=(s.H, s.W), out=out)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(out).any()), "unwritten (NaN) elements"
    assert bool((buf[:GUARD] == SENTINEL).all()) and bool((buf[GUARD + n_dst:] == SENTINEL).all())
    idx = sample_indices(s, np.random.default_rng(4712), count=4000)
    got = out.view(-1)[torch.from_numpy(idx).to(dev)].double().cpu().numpy()
    del buf, out
    ref, S = oracle.grad_input_at(g, w, 1, (1, 1), (s.H, s.W), idx)
    check(got, ref, S, "f32", str(s))
