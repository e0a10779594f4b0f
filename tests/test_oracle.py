"""Pins for the CPU oracle: it is checked against things other than itself.

* hand-worked examples (tests/golden, each derivation in its header);
* a closed form: with grad_out = 1 and weight = 1 each element is the product
  of per-dimension tap counts, counted here from the forward mapping;
* the adjoint identity <conv2d(x,w), g> = <x, grad_input(g,w)> with the
  separately written forward convolution;
* central finite differences of L(x) = <conv2d(x,w), g>;
* the transpose of the forward operator built column by column;
* torch-CPU float64 library routines (conv_transpose2d, grad.conv2d_input,
  conv2d) on random shapes;
* special cases: a 1x1 kernel is a matmul; kernel == stride with no padding
  is a scatter in closed form;
* the sampled entry point against the full tensor;
* and mutants: copies of oracle.c with one plausible mistake planted (a sign,
  an index, a dropped test) must each fail at least one of the pins above.

Definition followed by the oracle: doppler conv2d_backward_input.wgsl (direct
kernel), equal to the general-stride gather of meganeura
conv2d_grad_input_gemm.wgsl.
"""
import glob
import itertools
import os
import re

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def parse_fixture(path):
    blocks, cur = {}, None
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head = line.split()
            if head[0] in ("shape", "grad_out", "weight", "expected"):
                cur = head[0]
                blocks[cur] = [float(v) for v in head[1:]]
            else:
                blocks[cur].extend(float(v) for v in head)
    N, Ci, H, W, Co, kH, kW, s, ph, pw, oH, oW = (int(v) for v in blocks["shape"])
    g = np.array(blocks["grad_out"]).reshape(N, Co, oH, oW)
    w = np.array(blocks["weight"]).reshape(Co, Ci, kH, kW)
    e = np.array(blocks["expected"]).reshape(N, Ci, H, W)
    return dict(g=g, w=w, e=e, stride=s, pad=(ph, pw), hw=(H, W))


def rand_shape(rng):
    """A random small shape (any stride 1-4, any pads, kH != kW allowed)."""
    while True:
        kH, kW = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        s = int(rng.integers(1, 5))
        ph, pw = int(rng.integers(0, kH + 1)), int(rng.integers(0, kW + 1))
        H, W = int(rng.integers(1, 10)), int(rng.integers(1, 10))
        oH = (H + 2 * ph - kH) // s + 1
        oW = (W + 2 * pw - kW) // s + 1
        if oH >= 1 and oW >= 1:
            return workloads.Shape(int(rng.integers(1, 3)), int(rng.integers(1, 5)), H, W,
                                   int(rng.integers(1, 5)), kH, kW, s, ph, pw)


def rand_inputs(rng, sh):
    return (rng.standard_normal(sh.grad_out_shape), rng.standard_normal(sh.weight_shape))


# ----------------------------------------------------------------------------
# Pins written as functions of an Oracle, so the mutant test can rerun them.
# Each returns None on success and raises AssertionError otherwise.
# ----------------------------------------------------------------------------

def pin_golden(o):
    files = sorted(glob.glob(os.path.join(GOLDEN, "e*.txt")))
    assert len(files) >= 8
    for f in files:
        c = parse_fixture(f)
        out = o.grad_input(c["g"], c["w"], c["stride"], c["pad"], c["hw"], with_abs=False)
        assert np.array_equal(out, c["e"]), (os.path.basename(f), out, c["e"])


def tap_counts(n_in, k, s, pad, n_out):
    """For each input index, how many (output, tap) pairs the forward pass links
    to it: oh*s - pad + kh == ih.  Counted from the forward side."""
    cnt = np.zeros(n_in)
    for oh in range(n_out):
        for kh in range(k):
            ih = oh * s - pad + kh
            if 0 <= ih < n_in:
                cnt[ih] += 1
    return cnt


def pin_ones_closed_form(o):
    rng = np.random.default_rng(7)
    for _ in range(40):
        sh = rand_shape(rng)
        g = np.ones(sh.grad_out_shape)
        w = np.ones(sh.weight_shape)
        out = o.grad_input(g, w, sh.stride, (sh.pad_h, sh.pad_w), (sh.H, sh.W), with_abs=False)
        ch = tap_counts(sh.H, sh.kH, sh.stride, sh.pad_h, sh.oH)
        cw = tap_counts(sh.W, sh.kW, sh.stride, sh.pad_w, sh.oW)
        want = sh.Co * np.outer(ch, cw)
        assert np.array_equal(out, np.broadcast_to(want, out.shape)), sh


def pin_adjoint(o):
    rng = np.random.default_rng(11)
    for _ in range(60):
        sh = rand_shape(rng)
        x = rng.standard_normal(sh.dst_shape)
        g, w = rand_inputs(rng, sh)
        y = o.conv2d_forward(x, w, sh.stride, (sh.pad_h, sh.pad_w))
        gi = o.grad_input(g, w, sh.stride, (sh.pad_h, sh.pad_w), (sh.H, sh.W), with_abs=False)
        lhs = float(np.sum(y * g))
        rhs = float(np.sum(x * gi))
        scale = float(np.sum(np.abs(x) * o.grad_input(np.abs(g), np.abs(w), sh.stride,
                                                      (sh.pad_h, sh.pad_w), (sh.H, sh.W),
                                                      with_abs=False))) + 1e-300
        assert abs(lhs - rhs) <= 1e-13 * scale, (sh, lhs, rhs)


def pin_finite_differences(o):
    """L(x) = <conv2d(x,w), g> is linear in x, so a central difference with h = 1
    is exact up to rounding: dL/dx_j = (L(x+e_j) - L(x-e_j)) / 2."""
    rng = np.random.default_rng(13)
    for _ in range(6):
        sh = rand_shape(rng)
        g, w = rand_inputs(rng, sh)
        x = rng.standard_normal(sh.dst_shape)
        gi = o.grad_input(g, w, sh.stride, (sh.pad_h, sh.pad_w), (sh.H, sh.W), with_abs=False)
        fd = np.empty(x.size)
        for j in range(x.size):
            e = np.zeros(x.size)
            e[j] = 1.0
            e = e.reshape(x.shape)
            lp = np.sum(o.conv2d_forward(x + e, w, sh.stride, (sh.pad_h, sh.pad_w)) * g)
            lm = np.sum(o.conv2d_forward(x - e, w, sh.stride, (sh.pad_h, sh.pad_w)) * g)
            fd[j] = (lp - lm) / 2.0
        tol = 1e-12 * (np.abs(g).sum() * np.abs(w).sum() + np.abs(x).sum() + 1.0)
        assert np.max(np.abs(fd - gi.ravel())) <= tol, sh


def pin_operator_transpose(o):
    """Build the forward operator M (columns = forward of unit inputs); grad_input = M^T g."""
    rng = np.random.default_rng(17)
    for _ in range(6):
        sh = rand_shape(rng)
        g, w = rand_inputs(rng, sh)
        cols = []
        for j in range(int(np.prod(sh.dst_shape))):
            e = np.zeros(int(np.prod(sh.dst_shape)))
            e[j] = 1.0
            cols.append(o.conv2d_forward(e.reshape(sh.dst_shape), w, sh.stride,
                                         (sh.pad_h, sh.pad_w)).ravel())
        M = np.stack(cols, axis=1)
        want = (M.T @ g.ravel()).reshape(sh.dst_shape)
        gi = o.grad_input(g, w, sh.stride, (sh.pad_h, sh.pad_w), (sh.H, sh.W), with_abs=False)
        assert np.max(np.abs(gi - want)) <= 1e-12 * (1 + np.abs(want).max()), sh


def pin_torch_library(o):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    rng = np.random.default_rng(19)
    for _ in range(60):
        sh = rand_shape(rng)
        g, w = rand_inputs(rng, sh)
        gi, S = o.grad_input(g, w, sh.stride, (sh.pad_h, sh.pad_w), (sh.H, sh.W))
        tg = torch.from_numpy(g)
        tw = torch.from_numpy(w)
        ref = torch.nn.grad.conv2d_input(sh.dst_shape, tw, tg, stride=sh.stride,
                                         padding=(sh.pad_h, sh.pad_w)).numpy()
        assert np.max(np.abs(gi - ref)) <= 1e-12 * (1 + np.abs(ref).max()), sh
        oph = sh.H - ((sh.oH - 1) * sh.stride - 2 * sh.pad_h + sh.kH)
        opw = sh.W - ((sh.oW - 1) * sh.stride - 2 * sh.pad_w + sh.kW)
        if oph < sh.stride and opw < sh.stride:
            ref2 = F.conv_transpose2d(tg, tw, stride=sh.stride, padding=(sh.pad_h, sh.pad_w),
                                      output_padding=(oph, opw)).numpy()
            assert np.max(np.abs(gi - ref2)) <= 1e-12 * (1 + np.abs(ref2).max()), sh
        refS = torch.nn.grad.conv2d_input(sh.dst_shape, tw.abs(), tg.abs(), stride=sh.stride,
                                          padding=(sh.pad_h, sh.pad_w)).numpy()
        assert np.max(np.abs(S - refS)) <= 1e-12 * (1 + refS.max()), sh
        x = rng.standard_normal(sh.dst_shape)
        y = o.conv2d_forward(x, w, sh.stride, (sh.pad_h, sh.pad_w))
        yref = F.conv2d(torch.from_numpy(x), tw, stride=sh.stride,
                        padding=(sh.pad_h, sh.pad_w)).numpy()
        assert y.shape == yref.shape and np.max(np.abs(y - yref)) <= 1e-12 * (1 + np.abs(yref).max())


def pin_matmul_1x1(o):
    rng = np.random.default_rng(23)
    N, Ci, Co, H, W = 2, 5, 7, 3, 4
    g = rng.standard_normal((N, Co, H, W))
    w = rng.standard_normal((Co, Ci, 1, 1))
    gi = o.grad_input(g, w, 1, (0, 0), (H, W), with_abs=False)
    Wm = w[:, :, 0, 0]                               # [Co, Ci]
    want = np.stack([(Wm.T @ g[n].reshape(Co, H * W)).reshape(Ci, H, W) for n in range(N)])
    assert np.max(np.abs(gi - want)) <= 1e-12 * (1 + np.abs(want).max())


def pin_scatter_k_eq_s(o):
    """kernel == stride, no padding: each input pixel gets exactly one tap,
    grad_input[n,ci,ih,iw] = sum_co g[n,co,ih//s,iw//s] * w[co,ci,ih%s,iw%s]."""
    rng = np.random.default_rng(29)
    for s in (1, 2, 3):
        N, Ci, Co, oH, oW = 2, 3, 4, 3, 2
        H, W = oH * s, oW * s
        g = rng.standard_normal((N, Co, oH, oW))
        w = rng.standard_normal((Co, Ci, s, s))
        gi = o.grad_input(g, w, s, (0, 0), (H, W), with_abs=False)
        want = np.zeros((N, Ci, H, W))
        for n, ci, ih, iw in itertools.product(range(N), range(Ci), range(H), range(W)):
            want[n, ci, ih, iw] = np.dot(g[n, :, ih // s, iw // s], w[:, ci, ih % s, iw % s])
        assert np.max(np.abs(gi - want)) <= 1e-12 * (1 + np.abs(want).max()), s


def pin_sampled(o):
    rng = np.random.default_rng(31)
    for _ in range(10):
        sh = rand_shape(rng)
        g, w = rand_inputs(rng, sh)
        full, S = o.grad_input(g, w, sh.stride, (sh.pad_h, sh.pad_w), (sh.H, sh.W))
        idx = rng.integers(0, full.size, size=50)
        v, vs = o.grad_input_at(g, w, sh.stride, (sh.pad_h, sh.pad_w), (sh.H, sh.W), idx)
        assert np.array_equal(v, full.ravel()[idx]) and np.array_equal(vs, S.ravel()[idx])
    v, vs = o.grad_input_at(g, w, sh.stride, (sh.pad_h, sh.pad_w), (sh.H, sh.W),
                            [-1, full.size])
    assert np.isnan(v).all() and np.isnan(vs).all()


ALL_PINS = [pin_golden, pin_ones_closed_form, pin_adjoint, pin_finite_differences,
            pin_operator_transpose, pin_torch_library, pin_matmul_1x1,
            pin_scatter_k_eq_s, pin_sampled]


@pytest.fixture(scope="module")
def o():
    oracle.build()
    return oracle.Oracle(oracle.LIB_PATH)


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(o, pin):
    pin(o)


def test_golden_fixtures_parse():
    for f in sorted(glob.glob(os.path.join(GOLDEN, "e*.txt"))):
        c = parse_fixture(f)
        assert c["e"].size == np.prod(c["e"].shape) > 0


def test_abs_sum_bounds_value(o):
    """|grad_input| <= sum |g*w| elementwise, with equality when all terms are >= 0."""
    rng = np.random.default_rng(37)
    sh = workloads.Shape(2, 3, 7, 6, 4, 3, 3, 2, 1, 1)
    g, w = rand_inputs(rng, sh)
    gi, S = o.grad_input(g, w, sh.stride, (sh.pad_h, sh.pad_w), (sh.H, sh.W))
    assert np.all(np.abs(gi) <= S * (1 + 1e-15))
    gi2, S2 = o.grad_input(np.abs(g), np.abs(w), sh.stride, (sh.pad_h, sh.pad_w), (sh.H, sh.W))
    assert np.allclose(gi2, S2, rtol=1e-15, atol=0)


def test_workload_inputs_are_seeded():
    for wl in workloads.WORKLOADS[:2]:
        a1, b1 = workloads.make_inputs(wl)
        a2, b2 = workloads.make_inputs(wl)
        assert np.array_equal(a1, a2) and np.array_equal(b1, b2)
        assert a1.shape == wl.shape.grad_out_shape and b1.shape == wl.shape.weight_shape


def test_bf16_rounding_is_nearest_even():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(41)
    a = (rng.standard_normal(100000) * 10.0 ** rng.integers(-3, 3, 100000)).astype(np.float32)
    # ties: exact halfway patterns
    ties = (np.arange(0, 64, dtype=np.uint32) << 16 | 0x8000).view(np.float32) + 0
    a = np.concatenate([a, ties.astype(np.float32)])
    mine = workloads.bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    assert np.array_equal(workloads.bf16_to_f32(mine),
                          torch.from_numpy(a).to(torch.bfloat16).float().numpy())


# ----------------------------------------------------------------------------
# Mutants: one plausible mistake planted in a copy of oracle.c must fail a pin.
# ----------------------------------------------------------------------------

MUTANTS = {
    # the tap row read mirrored (kh' = kH-1-kh): a rotated-kernel mix-up in one dimension
    "kh_mirrored": ("const int64_t kh = ih + s->pad_h - oh * s->stride;",
                    "const int64_t kh = s->kH - 1 - (ih + s->pad_h - oh * s->stride);"),
    # the first covering output rounded down instead of up (keeps a position
    # whose window ends before the pixel)
    "lo_floor": ("*lo = bottom <= 0 ? 0 : (bottom + stride - 1) / stride;",
                 "*lo = bottom <= 0 ? 0 : bottom / stride;"),
    # the stride dropped when recovering the tap column
    "kw_no_stride": ("const int64_t kw = iw + s->pad_w - ow * s->stride;",
                     "const int64_t kw = iw + s->pad_w - ow;"),
    # weight read as [Ci,Co,...] (transposed operand)
    "weight_transposed": ("weight + (co * s->Ci + ci) * s->kH * s->kW;",
                          "weight + (ci * s->Co + co) * s->kH * s->kW;"),
    # kernel rotated by 180 degrees (the transposed-conv view applied twice)
    "weight_rotated": ("w_taps[kh * s->kW + kw]",
                       "w_taps[(s->kH - 1 - kh) * s->kW + (s->kW - 1 - kw)]"),
    # pad_w used for the row range
    "pad_h_from_w": ("covering_outputs(ih, s->pad_h,", "covering_outputs(ih, s->pad_w,"),
    # off-by-one clip of the last covering output
    "hi_bound": ("if (*hi > out - 1) *hi = out - 1;", "if (*hi > out) *hi = out;"),
    # a dropped channel (loop stops one short)
    "drop_last_co": ("for (int64_t co = 0; co < s->Co; ++co) {\n        const double *g_plane",
                     "for (int64_t co = 0; co < s->Co - 1; ++co) {\n        const double *g_plane"),
    # the abs-sum accumulates signed terms
    "abs_sum_signed": ("w_taps[kh * s->kW + kw];\n                acc += t;\n                acc_abs += fabs(t);",
                       "w_taps[kh * s->kW + kw];\n                acc += t;\n                acc_abs += t;"),
    # the sampled entry point decodes the flat index with H and W swapped
    "at_index_swap": ("int64_t ih = (f / s.W) % s.H;", "int64_t ih = (f / s.H) % s.W;"),
}

# Run a mutant's pins in a child process: a planted mistake may index outside
# an array, and a crash there must fail the mutant, not the test run.
_RUN_PINS = r"""
import sys
sys.path[:0] = [sys.argv[1], sys.argv[2]]
import oracle, test_oracle
m = oracle.Oracle(sys.argv[3])
caught = []
for pin in test_oracle.ALL_PINS + [test_oracle.test_abs_sum_bounds_value]:
    try:
        pin(m)
    except AssertionError:
        caught.append(pin.__name__)
print("CAUGHT " + ",".join(caught))
"""


def mutant_caught_by(lib_path):
    """Names of the pins the library at lib_path fails ("crashed" when the
    child process dies before it can report)."""
    import subprocess
    import sys
    here = os.path.dirname(os.path.abspath(__file__))
    r = subprocess.run([sys.executable, "-c", _RUN_PINS, os.path.dirname(here), here, lib_path],
                       capture_output=True, text=True, timeout=600)
    lines = [l for l in r.stdout.splitlines() if l.startswith("CAUGHT ")]
    if r.returncode != 0 or not lines:
        return ["crashed (exit %d)" % r.returncode]
    return [n for n in lines[-1][len("CAUGHT "):].split(",") if n]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, "mutation anchor not found or not unique: %s" % name
    mutated = src.replace(old, new, 1)
    cpath = tmp_path / ("mut_%s.c" % name)
    cpath.write_text(mutated)
    lib = oracle.compile_library(str(cpath), str(tmp_path / ("libmut_%s.so" % name)))
    caught = mutant_caught_by(lib)
    assert caught, "mutant %s passed every pin" % name
