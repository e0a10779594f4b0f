"""Host-only checks of the planner (no GPU): the graded workloads get the
compile-time kernel instances documented for them, forced tiles reach each
compile-time instance, and forced tiles are validated."""
import re

import pytest

import conv2d_backward_amd as gi
import workloads

S = workloads.Shape


@pytest.fixture(scope="module", autouse=True)
def lib():
    gi.load_library()
    yield
    gi.set_halo_tile()
    gi.set_halo_split()
    gi.set_halo_fusion()
    gi.set_variant(gi.VARIANT_AUTO)


def plan_of(shape, bf16=False):
    return gi.plan(gi.make_params(*shape.as_tuple()[:10]), bf16)


# Workload -> substrings its plan must contain.
WORKLOAD_PLANS = {
    "resnet_stage_3x3": ["variant=halo", "cfg=0", "HP=30"],
    "deep_late_stage": ["variant=halo", "cfg=0", "tile=14x14", "HP=30"],
    "strided_downsample": ["variant=halo", "cfg=11 fused", "HP=15"],
    "asym_1x7": ["variant=halo", "cfg=10 split=2", "fold", "HP=23"],
    "stem_7x7_s2": ["variant=col2im", "ws_bytes=0", "tile=56x56 wgs=256 cols=147",
                    "rows_per_wave=8"],
    "deep_late_stage_bf16": ["variant=halo", "dtype=bf16", "image kernel cfg=0", "nb=13",
                             "wgs=64x4", "pitch=30"],
    "deep_late_stage_f16": ["variant=halo", "dtype=f16", "image kernel cfg=0", "wgs=64x4"],
    "tiny": ["variant=generic"],
}


@pytest.mark.parametrize("name", sorted(WORKLOAD_PLANS))
def test_workload_plans(name):
    wl = workloads.BY_NAME[name]
    desc = plan_of(wl.shape, {"f32": 0, "bf16": 1, "f16": 2}[wl.dtype])
    for part in WORKLOAD_PLANS[name]:
        assert part in desc, (name, part, desc)


# (shape, bf16, variant, forced (nb, rows, cols, split, fusion) or None, plan
# substrings): ragged channel counts on each compile-time instance (split: the
# fp32 output-channel split forced to 1 or 2 thread groups; fusion: the fp32
# stride phases forced phase at a time (1) or fused (2); 0: the planner's
# choice).
FIXED_INSTANCES = [
    (S(3, 40, 28, 28, 20, 3, 3, 1, 1, 1), False, gi.VARIANT_HALO, (13, 14, 14, 0, 0),
     ["cfg=0", "HP=30", "tile=14x14"]),
    (S(3, 40, 28, 28, 20, 3, 3, 1, 1, 1), False, gi.VARIANT_HALO, (13, 7, 28, 0, 0),
     ["cfg=0", "HP=30", "tile=7x28"]),
    (S(2, 70, 28, 28, 20, 3, 3, 2, 1, 1), False, gi.VARIANT_HALO, (13, 14, 14, 0, 1),
     ["cfg=2", "HP=15"]),
    (S(2, 70, 28, 28, 20, 3, 3, 2, 1, 1), False, gi.VARIANT_HALO, (13, 14, 14, 0, 2),
     ["cfg=11 fused", "HP=15"]),
    (S(2, 70, 28, 28, 20, 3, 3, 2, 1, 1), False, gi.VARIANT_HALO, (8, 7, 14, 0, 2),
     ["cfg=12 fused", "HP=15", "tile=7x14"]),
    (S(2, 70, 27, 29, 20, 3, 3, 2, 1, 1), False, gi.VARIANT_HALO, (13, 7, 15, 0, 2),
     ["cfg=13 fused"]),
    # Fused stride 2 with whole-row stores: odd H (one phase's grid a row
    # shorter, the last row tile ragged) and ragged column and row tiles.
    (S(2, 70, 27, 28, 20, 3, 3, 2, 1, 1), False, gi.VARIANT_HALO, (13, 7, 14, 0, 2),
     ["cfg=11 fused", "tile=7x14", "wgs=4x2"]),
    (S(3, 50, 30, 36, 24, 3, 3, 2, 1, 1), False, gi.VARIANT_HALO, (8, 7, 14, 0, 2),
     ["cfg=12 fused", "tile=7x14", "wgs=18x1"]),
    (S(1, 40, 21, 22, 12, 3, 2, 2, 1, 0), False, gi.VARIANT_HALO, (13, 11, 11, 0, 2),
     ["cfg=13 fused"]),
    (S(4, 30, 17, 17, 36, 1, 7, 1, 0, 3), False, gi.VARIANT_HALO, (8, 7, 17, 1, 0),
     ["cfg=4", "HP=33", "fold"]),
    (S(4, 30, 17, 17, 36, 1, 7, 1, 0, 3), False, gi.VARIANT_HALO, (8, 7, 17, 2, 0),
     ["cfg=10 split=2", "HP=23", "fold"]),
    (S(3, 64, 17, 17, 80, 1, 7, 1, 0, 3), False, gi.VARIANT_HALO, (8, 4, 17, 2, 0),
     ["cfg=10 split=2", "HP=23", "fold", "tile=4x17"]),
    (S(3, 72, 14, 14, 40, 3, 3, 1, 1, 1), True, gi.VARIANT_HALO, (7, 14, 14, 0, 0),
     ["cfg=0", "pitch=30"]),
    (S(3, 130, 14, 14, 70, 3, 3, 1, 1, 1), True, gi.VARIANT_HALO, (13, 14, 14, 0, 0),
     ["image kernel cfg=0", "wgs=3x2", "pitch=30"]),
    (S(1, 2, 30, 30, 6, 7, 7, 2, 3, 3), False, gi.VARIANT_STEM, None,
     ["variant=stem"]),
]


@pytest.mark.parametrize("idx", range(len(FIXED_INSTANCES)))
def test_fixed_instance_plans(idx):
    shape, bf16, variant, tile, parts = FIXED_INSTANCES[idx]
    try:
        if tile:
            gi.set_halo_tile(tile[0], tile[1], tile[2], 0)
            gi.set_halo_split(tile[3])
            gi.set_halo_fusion(tile[4])
        gi.set_variant(variant)
        desc = plan_of(shape, bf16)
    finally:
        gi.set_variant(gi.VARIANT_AUTO)
        gi.set_halo_tile()
        gi.set_halo_split()
        gi.set_halo_fusion()
    for part in parts:
        assert part in desc, (part, desc)


def test_forced_tile_validation():
    with pytest.raises(gi.Conv2dGiError):
        gi.set_halo_tile(5, 4, 4, 0)          # no such block count
    with pytest.raises(gi.Conv2dGiError):
        gi.set_halo_tile(7, 15, 15, 0)        # 225 > 2 * 7 * 16 pixels
    with pytest.raises(gi.Conv2dGiError):
        gi.set_halo_tile(13, 14, 14, 1)       # one stage is no pipeline
    gi.set_halo_tile(7, 14, 14, 0)            # a bf16 tile of 196 pixels
    gi.set_halo_tile()


def test_image_kernel_needs_its_instance():
    """The whole-image 16-bit kernel serves 3x3 kernels on images of up to
    14 x 14 with 14 columns (pitch 30) and whole 4-pixel grad_out quads; other
    shapes keep the halo-tile kernel even when its tile is forced."""
    gi.set_halo_tile(13, 14, 14, 0)
    try:
        assert "image kernel" in plan_of(S(2, 64, 10, 14, 64, 3, 3, 1, 1, 1), 1)
        assert "image kernel" not in plan_of(S(2, 64, 14, 13, 64, 3, 3, 1, 1, 1), 1)  # W = 13
        assert "image kernel" not in plan_of(S(2, 64, 16, 14, 64, 3, 3, 1, 1, 1), 1)  # H = 16
        assert "image kernel" not in plan_of(S(2, 64, 7, 14, 64, 3, 3, 1, 1, 1), 1)   # 98 pixels: 24.5 quads
        assert "image kernel" not in plan_of(S(2, 64, 7, 14, 64, 3, 3, 1, 0, 0), 1)   # 60 grad_out pixels, 98 image pixels
        assert "image kernel" not in plan_of(S(2, 64, 14, 14, 64, 3, 3, 1, 1, 1), 0)  # fp32
    finally:
        gi.set_halo_tile()
    # Unforced, it needs a grid of at least one work-group per compute unit.
    assert "image kernel" not in plan_of(S(2, 64, 14, 14, 64, 3, 3, 1, 1, 1), 1)
    assert "image kernel" in plan_of(S(128, 256, 14, 14, 64, 3, 3, 1, 1, 1), 2)


# ----------------------------------------------------------------------------
# Planner invariants over seeded random shapes (host only).
# ----------------------------------------------------------------------------

def planner_shapes(seed, count):
    """Shapes from tiny to production sizes: channel counts up to 640, planes
    up to 120x120, batches up to 64, kernels 1..7, strides 1..4; a quarter
    are network-style layers (channels in multiples of 32, square planes of
    7..56, 3x3 or 1x1 at stride 1 or 2), the shapes the tiled kernels take."""
    import random
    rng = random.Random(seed)
    out = []
    while len(out) < count:
        if rng.random() < 0.25:
            k = rng.choice([1, 3, 3, 3])
            hw = rng.choice([7, 14, 28, 56])
            out.append(S(rng.choice([8, 16, 32, 64]), 32 * rng.randint(1, 16), hw, hw,
                         32 * rng.randint(1, 16), k, k, rng.choice([1, 1, 1, 2]), k // 2, k // 2))
            continue
        k_h, k_w = rng.randint(1, 7), rng.randint(1, 7)
        stride = rng.choice([1, 1, 1, 2, 2, 3, 4])
        H, W = rng.randint(1, 120), rng.randint(1, 120)
        ph, pw = rng.randint(0, k_h), rng.randint(0, k_w)
        if H + 2 * ph < k_h or W + 2 * pw < k_w:
            continue
        out.append(S(rng.choice([1, 2, 4, 8, 16, 32, 64]), rng.randint(1, 640), H, W,
                     rng.randint(1, 640), k_h, k_w, stride, ph, pw))
    return out


def fp32_bytes_over_limit(s):
    oH = (s.H + 2 * s.pad_h - s.kH) // s.stride + 1
    oW = (s.W + 2 * s.pad_w - s.kW) // s.stride + 1
    return max(s.N * s.Ci * s.H * s.W, s.N * s.Co * oH * oW) * 4 > 0x7fff0000


FP32_HALO_TAPS = {0, 1, 2, 3, 4, 6, 7, 9}


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_planner_invariants(seed):
    import re
    for s in planner_shapes(seed, 400):
        p = gi.make_params(*s.as_tuple()[:10])
        if gi.validate(p) != 0:
            continue
        for dt in (0, 1, 2):
            desc = gi.plan(p, dt)
            assert desc == gi.plan(p, dt), "plan is not deterministic"
            variant = re.match(r"variant=(\w+) ", desc).group(1)
            assert variant in ("generic", "halo", "stem", "col2im"), desc
            if variant == "col2im":
                assert dt == 0 and s.Ci * s.kH * s.kW <= 160 and 48 < s.Co <= 64, desc
                assert s.kW <= 4 * s.stride, desc
            assert int(re.search(r"ws_bytes=(\d+)", desc).group(1)) >= 0
            if variant == "stem":
                assert dt == 0, desc
            if "image kernel" in desc:
                assert dt != 0 and s.stride == 1, desc
            lds = re.search(r"\blds=(\d+)", desc)
            if lds:
                assert 0 < int(lds.group(1)) <= 160 * 1024, desc
            wgs = re.search(r"\bwgs=(\d+)x(\d+)", desc)
            if wgs:
                a, b = int(wgs.group(1)), int(wgs.group(2))
                assert a >= 1 and b >= 1 and a * b < 2 ** 31, desc
            phases = re.findall(r"taps=(\d+)x(\d+) px=(\d+)x(\d+)", desc)
            if phases and "fused" not in desc:
                # Every input pixel falls in exactly one phase, and so does
                # every tap when every residue class owns a pixel.
                if s.H >= s.stride and s.W >= s.stride:
                    assert sum(int(a) * int(b) for a, b, _, _ in phases) == s.kH * s.kW, desc
                assert sum(int(c) * int(d) for _, _, c, d in phases) == s.H * s.W, desc
            if fp32_bytes_over_limit(s):
                assert variant == "generic", desc
            if variant == "halo" and dt == 0:
                # The fp32 halo kernel has cases for these tap counts only.
                for a, b, _, _ in phases:
                    assert int(a) * int(b) in FP32_HALO_TAPS, desc


def test_planner_picks_generic_past_buffer_range():
    """Tensors past the 32-bit buffer range go to the generic kernel, whose
    batch offsets are 64-bit, for every element type."""
    for s in [S(8, 64, 1024, 1024, 16, 3, 3, 1, 1, 1), S(1, 16, 64, 64, 512, 3, 3, 1, 1, 1),
              S(600, 512, 40, 40, 64, 1, 1, 1, 0, 0), S(2, 64, 1200, 1200, 64, 7, 7, 2, 3, 3)]:
        p = gi.make_params(*s.as_tuple()[:10])
        assert gi.validate(p) == 0
        for dt in (0, 1, 2):
            desc = gi.plan(p, dt)
            if fp32_bytes_over_limit(s):
                assert desc.startswith("variant=generic"), (s, dt, desc)


@pytest.mark.parametrize("shape", [S(3, 49, 15, 1, 9, 7, 5, 1, 3, 4), S(2, 64, 20, 20, 32, 5, 7, 1, 2, 3),
                                   S(1, 64, 12, 12, 16, 6, 6, 1, 2, 2), S(1, 64, 12, 12, 16, 1, 5, 1, 0, 2),
                                   S(1, 64, 24, 24, 16, 7, 7, 1, 3, 3)])
def test_fp32_halo_rejects_unserved_tap_counts(shape):
    """Tap counts the fp32 halo kernel has no case for (5, 35, 36, 49 ...;
    past 31 a shift-built mask would wrap onto a served count) go to another
    kernel rather than to a halo plan that would leave the pixels at zero."""
    desc = plan_of(shape)
    assert not desc.startswith("variant=halo"), desc


def test_col2im_scope():
    """The column kernel takes fp32 shapes of at most 160 columns, 48 < Co <=
    64 and kW <= 4 * stride; the 7x7 stride-2 stem can still be forced onto
    the 4x4-block kernel."""
    stem = S(16, 3, 224, 224, 64, 7, 7, 2, 3, 3)
    assert plan_of(stem).startswith("variant=col2im")
    assert not plan_of(stem, True).startswith("variant=col2im")
    for s in [S(16, 3, 224, 224, 48, 7, 7, 2, 3, 3), S(16, 3, 224, 224, 65, 7, 7, 2, 3, 3),
              S(4, 4, 32, 32, 64, 7, 7, 2, 3, 3), S(4, 3, 32, 32, 64, 3, 5, 1, 1, 2)]:
        assert not plan_of(s).startswith("variant=col2im"), s
    old = gi.set_variant(gi.VARIANT_STEM)
    try:
        assert plan_of(stem).startswith("variant=stem")
    finally:
        gi.set_variant(old)


def test_col2im_reciprocal_division_exact():
    """The column kernel splits a column index into (ci, kh, kw) as
    (x * ceil(2^16 / d)) >> 16: exact for every x, d below 256 (the error
    x * (ceil(2^16/d) - 2^16/d) / 2^16 < x / 2^16 < 1/256 <= 1/d stays under
    the distance from x/d to the next integer)."""
    import numpy as np
    x = np.arange(256, dtype=np.int64)
    for d in range(1, 256):
        m = (65536 + d - 1) // d
        assert np.array_equal((x * m) >> 16, x // d), d
    # outside that range the shortcut does fail (the bound is needed)
    xs = np.arange(1 << 15, dtype=np.int64)
    assert (((xs * ((65536 + 299) // 300)) >> 16) != xs // 300).any()


def test_col2im_bank_layout():
    """Column-kernel plans: tile pitch = kW and channel plane = kH*kW (mod 32),
    so a column's LDS bank is its index plus a per-lane constant; the staged
    weight's row stride covers every column block and is 8 (stride 2) or
    16 (stride 1) mod 32."""
    import workloads as wl
    seen = 0
    for s in wl.random_shapes(20241203, 160, co_range=(49, 64)) + [S(16, 3, 224, 224, 64, 7, 7, 2, 3, 3)]:
        txt = plan_of(s)
        if not txt.startswith("variant=col2im"):
            continue
        seen += 1
        f = dict(re.findall(r"\b(pitch|plane|stage|cols)=(\d+)", txt))
        lp, plane, ws, ncols = (int(f[k]) for k in ("pitch", "plane", "stage", "cols"))
        assert (lp - s.kW) % 32 == 0 and (plane - s.kH * s.kW) % 32 == 0, txt
        assert ws >= 16 * ((ncols + 15) // 16) and ws % 32 == (8 if s.stride == 2 else 16), txt
    assert seen >= 10


def test_div24_exact():
    """The grad_weight kernel's piece divisions: q = (s * m) >> k with
    2^k >= 2^14 d and m = ceil(2^k / d) equals s // d for every s < 2^14, and
    s * m stays below 2^29 (one 24-bit multiply)."""
    for d in list(range(1, 600)) + [1021, 4093, 16383]:
        k = 14
        while (1 << k) < 16384 * d:
            k += 1
        m = ((1 << k) + d - 1) // d
        assert m < (1 << 15)
        for s in range(0, 16384, 1 if d < 64 else 7):
            assert (s * m) >> k == s // d, (d, s)
            assert s * m < (1 << 29)
