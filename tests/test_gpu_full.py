"""Whole-tensor GPU parity at the graded sizes.

Every graded workload is launched exactly as the benchmark launches it (the
planner's own choice, the caller's stream, no forced variant), and EVERY
element of the result is compared with the CPU oracle on the same seeded
inputs:
  grad_input fp32 / fp16 inputs: |gpu - oracle| <= 1e-5 * S + 1e-6 per element
  grad_input bf16 inputs:        ||gpu - oracle||_2 <= 1e-2 * ||oracle||_2 over the
                                 whole tensor, and |gpu - oracle| <= 1e-2 * S + 1e-6
                                 per element (oracle on the same bf16 values)
  grad_weight, forward, fused dx/dw/db (fp32): the fp32 form with S the sum of
                                 |products| of the element's own terms
S is the oracle's sum of |products| over the element's terms.  Each output is
pre-filled with NaN and framed by guard bands (see the helpers imported below).
The oracle runs on every host thread; the largest case (the deep late stage,
59 GFLOP) takes a few seconds.
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import conv2d_backward_amd as gi  # noqa: E402

import test_gpu_parity as gp  # noqa: E402
import test_gpu_grad_weight as gw  # noqa: E402
import test_gpu_forward as gf  # noqa: E402
import test_gpu_backward as gb  # noqa: E402

GRAD_INPUT_RUNS = [w.name for w in workloads.WORKLOADS if w.name != "tiny"]
FP32_RUNS = [w.name for w in workloads.WORKLOADS if w.name != "tiny" and w.dtype == "f32"]


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gi.load_library()
    return torch.device("cuda:0")


@pytest.mark.parametrize("name", GRAD_INPUT_RUNS)
def test_grad_input_workload_every_element(name):
    wl = workloads.BY_NAME[name]
    s = wl.shape
    g, w = workloads.make_inputs(wl)
    dt = {"f32": 0, "bf16": 1, "f16": 2}[wl.dtype]
    gp.say("grad_input workload %s plan %s" % (name, gi.plan(gi.make_params(*s.as_tuple()[:10]),
                                                            dt)))
    got, ok = gp.run_gpu(g, w, s, wl.dtype)
    assert ok, "write outside dst"
    go, wo = gp.oracle_inputs(g, w, wl.dtype)
    ref, S = oracle.grad_input(go, wo, s.stride, (s.pad_h, s.pad_w), (s.H, s.W))
    worst = gp.check(got, ref, S, wl.dtype, name)
    gp.say("  %d elements, worst |err| / bound = %.3g" % (got.size, worst))


@pytest.mark.parametrize("name", FP32_RUNS)
def test_grad_weight_workload_every_element(name):
    wl = workloads.BY_NAME[name]
    sh = wl.shape
    g, _ = workloads.make_inputs(wl)
    x = workloads.make_forward_input(wl)
    gp.say("grad_weight workload %s plan %s" % (name, gi.grad_weight_plan(
        gi.make_params(*sh.as_tuple()[:10]))))
    got, ok = gw.run_gw(x, g, sh)
    assert ok, "write outside dw"
    ref, Ssum = oracle.grad_weight(x, g, sh.stride, (sh.pad_h, sh.pad_w), (sh.kH, sh.kW))
    gw.check(got, ref, Ssum, name)


@pytest.mark.parametrize("name", FP32_RUNS)
def test_forward_workload_every_element(name):
    wl = workloads.BY_NAME[name]
    sh = wl.shape
    _, w = workloads.make_inputs(wl)
    x = workloads.make_forward_input(wl)
    gp.say("forward workload %s plan %s" % (name, gi.forward_plan(
        gi.make_params(*sh.as_tuple()[:10]))))
    got = gf.run_fwd(sh, x, w)
    ref, Ss = oracle.conv2d_forward_abs(x, w, sh.stride, (sh.pad_h, sh.pad_w))
    gf.check(got, ref, Ss, name)


@pytest.mark.parametrize("name", FP32_RUNS)
def test_backward_workload_every_element(name):
    """The fused call: dx, dw and db, each compared whole."""
    wl = workloads.BY_NAME[name]
    sh = wl.shape
    g, w = workloads.make_inputs(wl)
    x = workloads.make_forward_input(wl)
    gp.say("backward workload %s" % name)
    dx, dw, db = gb.run_backward(sh, x, w, g, "xwb")
    ref, Ss = oracle.grad_input(g, w, sh.stride, (sh.pad_h, sh.pad_w), (sh.H, sh.W))
    gb.check(dx, ref, Ss, "dx " + name)
    ref, Ss = oracle.grad_weight(x, g, sh.stride, (sh.pad_h, sh.pad_w), (sh.kH, sh.kW))
    gb.check(dw, ref, Ss, "dw " + name)
    ref, Ss = oracle.grad_bias(g)
    gb.check(db, ref, Ss, "db " + name)
