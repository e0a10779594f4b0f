"""Pins for the oracle's grad_weight: it is checked against things other than
itself.

* the adjoint identity <conv2d(x,w), g> = <w, grad_weight(x,g)> with the
  separately written forward convolution (grad_weight is the derivative of
  that linear function of w);
* the cross identity <x, grad_input(g,w)> = <w, grad_weight(x,g)> with the
  oracle's grad_input, written from the input side;
* a closed form: with x = 1 and grad_out = 1 each element is N times the
  product of per-dimension counts of output positions whose tap lands inside
  the image, counted here from the forward mapping;
* a special case: a 1x1 kernel at stride 1 without padding is a matmul over
  the pixels of every batch item;
* torch-CPU float64 ``torch.nn.grad.conv2d_weight`` on random shapes;
* the sampled entry point against the full tensor;
* and mutants: copies of oracle.c with one plausible mistake planted in the
  grad_weight code must each fail at least one of the pins above.

Definition followed: the computeGradWeight branch of doppler
conv2d_backward.js (a [Co, Ci, kH, kW] result from grad_out and the forward
input); the shader itself is not on the pages, so the oracle takes the
derivative of the forward mapping the doppler direct kernel's comment states.
"""
import numpy as np
import pytest

import oracle
import workloads


def rand_shape(rng):
    """A random small shape (strides 1-4, any pads, kH != kW allowed)."""
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


def gw(o, x, g, sh, with_abs=False):
    return o.grad_weight(x, g, sh.stride, (sh.pad_h, sh.pad_w), (sh.kH, sh.kW), with_abs)


def pin_gw_adjoint_forward(o):
    rng = np.random.default_rng(101)
    for _ in range(30):
        sh = rand_shape(rng)
        x = rng.standard_normal(sh.dst_shape)
        g = rng.standard_normal(sh.grad_out_shape)
        w = rng.standard_normal(sh.weight_shape)
        y = o.conv2d_forward(x, w, sh.stride, (sh.pad_h, sh.pad_w))
        lhs = float(np.sum(y * g))
        rhs = float(np.sum(w * gw(o, x, g, sh)))
        assert abs(lhs - rhs) <= 1e-10 * (1 + abs(lhs)), (sh, lhs, rhs)


def pin_gw_cross_grad_input(o):
    rng = np.random.default_rng(103)
    for _ in range(30):
        sh = rand_shape(rng)
        x = rng.standard_normal(sh.dst_shape)
        g = rng.standard_normal(sh.grad_out_shape)
        w = rng.standard_normal(sh.weight_shape)
        gi = o.grad_input(g, w, sh.stride, (sh.pad_h, sh.pad_w), (sh.H, sh.W), with_abs=False)
        lhs = float(np.sum(x * gi))
        rhs = float(np.sum(w * gw(o, x, g, sh)))
        assert abs(lhs - rhs) <= 1e-10 * (1 + abs(lhs)), (sh, lhs, rhs)


def out_counts(n_in, k, s, pad, n_out):
    """For each tap, how many output positions read an input index inside
    [0, n_in): oh*s - pad + kh in range.  Counted from the forward side."""
    cnt = np.zeros(k)
    for kh in range(k):
        for oh in range(n_out):
            if 0 <= oh * s - pad + kh < n_in:
                cnt[kh] += 1
    return cnt


def pin_gw_ones_closed_form(o):
    rng = np.random.default_rng(107)
    for _ in range(40):
        sh = rand_shape(rng)
        out = gw(o, np.ones(sh.dst_shape), np.ones(sh.grad_out_shape), sh)
        ch = out_counts(sh.H, sh.kH, sh.stride, sh.pad_h, sh.oH)
        cw = out_counts(sh.W, sh.kW, sh.stride, sh.pad_w, sh.oW)
        want = sh.N * np.outer(ch, cw)
        assert np.array_equal(out, np.broadcast_to(want, out.shape)), sh


def pin_gw_matmul_1x1(o):
    rng = np.random.default_rng(109)
    N, Ci, Co, H, W = 3, 5, 7, 3, 4
    sh = workloads.Shape(N, Ci, H, W, Co, 1, 1, 1, 0, 0)
    x = rng.standard_normal(sh.dst_shape)
    g = rng.standard_normal(sh.grad_out_shape)
    out = gw(o, x, g, sh)[:, :, 0, 0]
    want = sum(g[n].reshape(Co, H * W) @ x[n].reshape(Ci, H * W).T for n in range(N))
    assert np.max(np.abs(out - want)) <= 1e-12 * (1 + np.abs(want).max())


def pin_gw_torch_library(o):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(113)
    for _ in range(25):
        sh = rand_shape(rng)
        x = rng.standard_normal(sh.dst_shape)
        g = rng.standard_normal(sh.grad_out_shape)
        out, S = gw(o, x, g, sh, with_abs=True)
        ref = torch.nn.grad.conv2d_weight(torch.from_numpy(x), sh.weight_shape,
                                          torch.from_numpy(g), stride=sh.stride,
                                          padding=(sh.pad_h, sh.pad_w)).numpy()
        assert np.max(np.abs(out - ref)) <= 1e-12 * (1 + np.abs(ref).max()), sh
        refS = torch.nn.grad.conv2d_weight(torch.from_numpy(np.abs(x)), sh.weight_shape,
                                           torch.from_numpy(np.abs(g)), stride=sh.stride,
                                           padding=(sh.pad_h, sh.pad_w)).numpy()
        assert np.max(np.abs(S - refS)) <= 1e-12 * (1 + refS.max()), sh


def pin_gw_sampled(o):
    rng = np.random.default_rng(127)
    for _ in range(10):
        sh = rand_shape(rng)
        x = rng.standard_normal(sh.dst_shape)
        g = rng.standard_normal(sh.grad_out_shape)
        full, S = gw(o, x, g, sh, with_abs=True)
        idx = rng.integers(0, full.size, size=40)
        v, vs = o.grad_weight_at(x, g, sh.stride, (sh.pad_h, sh.pad_w), (sh.kH, sh.kW), idx)
        assert np.array_equal(v, full.ravel()[idx]) and np.array_equal(vs, S.ravel()[idx])
    v, vs = o.grad_weight_at(x, g, sh.stride, (sh.pad_h, sh.pad_w), (sh.kH, sh.kW),
                             [-1, full.size])
    assert np.isnan(v).all() and np.isnan(vs).all()


def pin_gw_abs_bounds(o):
    """|grad_weight| <= sum |g*x| elementwise, with equality for nonnegative inputs."""
    rng = np.random.default_rng(131)
    sh = workloads.Shape(2, 3, 7, 6, 4, 3, 3, 2, 1, 1)
    x = rng.standard_normal(sh.dst_shape)
    g = rng.standard_normal(sh.grad_out_shape)
    v, S = gw(o, x, g, sh, with_abs=True)
    assert np.all(np.abs(v) <= S * (1 + 1e-15))
    v2, S2 = gw(o, np.abs(x), np.abs(g), sh, with_abs=True)
    assert np.allclose(v2, S2, rtol=1e-15, atol=0)


GW_PINS = [pin_gw_adjoint_forward, pin_gw_cross_grad_input, pin_gw_ones_closed_form,
           pin_gw_matmul_1x1, pin_gw_torch_library, pin_gw_sampled, pin_gw_abs_bounds]


@pytest.fixture(scope="module")
def o():
    oracle.build()
    return oracle.Oracle(oracle.LIB_PATH)


@pytest.mark.parametrize("pin", GW_PINS, ids=lambda p: p.__name__)
def test_gw_pin(o, pin):
    pin(o)


GW_MUTANTS = {
    # wrong sign of the tap offset in the row gather
    "kh_sign": ("for (int64_t oh = 0; oh < s->oH; ++oh) {\n            int64_t ih = oh * s->stride - s->pad_h + kh;",
                "for (int64_t oh = 0; oh < s->oH; ++oh) {\n            int64_t ih = oh * s->stride + s->pad_h - kh;"),
    # pad_w used for the rows
    "pad_h_from_w": ("for (int64_t oh = 0; oh < s->oH; ++oh) {\n            int64_t ih = oh * s->stride - s->pad_h + kh;",
                     "for (int64_t oh = 0; oh < s->oH; ++oh) {\n            int64_t ih = oh * s->stride - s->pad_w + kh;"),
    # stride dropped from the column gather
    "no_w_stride": ("for (int64_t ow = 0; ow < s->oW; ++ow) {\n                int64_t iw = ow * s->stride - s->pad_w + kw;",
                    "for (int64_t ow = 0; ow < s->oW; ++ow) {\n                int64_t iw = ow - s->pad_w + kw;"),
    # off-by-one image bound in w
    "iw_bound": ("if (iw < 0 || iw >= s->W) continue;\n                double t = gp[",
                 "if (iw < 0 || iw > s->W) continue;\n                double t = gp["),
    # the last batch item dropped
    "drop_last_n": ("for (int64_t n = 0; n < s->N; ++n) {\n        const double *gp",
                    "for (int64_t n = 0; n < s->N - 1; ++n) {\n        const double *gp"),
    # input read with the channel index of the gradient (operands mixed up)
    "x_channel_co": ("const double *gp = grad_out + (n * s->Co + co) * s->oH * s->oW;\n        const double *xp = x + (n * s->Ci + ci) * s->H * s->W;",
                     "const double *gp = grad_out + (n * s->Co + co) * s->oH * s->oW;\n        const double *xp = x + (n * s->Ci + co % s->Ci) * s->H * s->W;"),
    # the abs-sum accumulates signed terms
    "abs_sum_signed": ("double t = gp[oh * s->oW + ow] * xp[ih * s->W + iw];\n                acc += t;\n                acc_abs += fabs(t);",
                       "double t = gp[oh * s->oW + ow] * xp[ih * s->W + iw];\n                acc += t;\n                acc_abs += t;"),
    # the flat index decoded with kH and kW swapped
    "index_swap": ("int64_t kh = (e / s.kW) % s.kH;", "int64_t kh = (e / s.kH) % s.kW;"),
}


@pytest.mark.parametrize("name", sorted(GW_MUTANTS))
def test_gw_mutant_is_caught(tmp_path, name):
    old, new = GW_MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, "mutation anchor not found or not unique: %s" % name
    mutated = src.replace(old, new, 1)
    cpath = tmp_path / ("mut_%s.c" % name)
    cpath.write_text(mutated)
    lib = oracle.compile_library(str(cpath), str(tmp_path / ("libmut_%s.so" % name)))
    m = oracle.Oracle(lib)
    caught = []
    for pin in GW_PINS:
        try:
            pin(m)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "mutant %s passed every pin" % name
