"""Seeded randomized GPU sweep: a few hundred random small shapes (strides
1-4, kernels 1-7 with kH != kW, pads 0..k per dimension, ragged channel
counts) per input type and forced kernel variant, each compared element by
element with the oracle to the criteria of test_gpu_parity.  Each test walks
its shapes in order and stops at the first failure, naming the shape.
A forced variant that does not serve a shape falls back to the planner's
generic kernel, so every shape is still checked.
"""
import pytest

import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import conv2d_backward_amd as gi  # noqa: E402

import test_gpu_parity as gp  # noqa: E402

SHAPES = workloads.random_shapes(20241202, 240)

CASES = [("f32", gi.VARIANT_AUTO), ("f32", gi.VARIANT_GENERIC), ("f32", gi.VARIANT_HALO),
         ("f32", gi.VARIANT_STEM), ("bf16", gi.VARIANT_AUTO), ("bf16", gi.VARIANT_GENERIC),
         ("f16", gi.VARIANT_AUTO)]


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gi.load_library()


@pytest.mark.parametrize("dtype,variant", CASES, ids=["%s-v%d" % c for c in CASES])
def test_random_sweep(dtype, variant):
    for i, s in enumerate(SHAPES):
        gp.full_parity(s, 30000 + i, dtype, variant, dist="normal")


# Output-channel counts the column kernel serves (48 < Co <= 64), the same
# kind of random shapes otherwise; the shapes it does not serve (more than
# 160 columns, kW > 4 * stride) fall back to the generic kernel.
SHAPES_COL2IM = workloads.random_shapes(20241203, 160, co_range=(49, 64))


def test_random_sweep_col2im():
    for i, s in enumerate(SHAPES_COL2IM):
        gp.full_parity(s, 40000 + i, "f32", gi.VARIANT_COL2IM, dist="normal")
