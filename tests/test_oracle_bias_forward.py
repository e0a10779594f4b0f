"""Pins for the oracle's grad_bias and for its forward convolution with
abs-sums (the forward row's checker): each is checked against things other
than itself.

grad_bias (doppler bias_add_backward.wgsl: the output gradient summed over
every position the bias was added to; for a convolution's per-channel bias,
all (n, oh, ow)):
* closed form: with grad_out = 1 every channel sums to N*oH*oW;
* the adjoint of adding a bias: <y + b, g> - <y, g> = <b, grad_bias(g)>, with
  the broadcast written here in numpy;
* torch-CPU float64 autograd of conv2d with a bias;
* mutants of oracle.c with one planted mistake each.

Forward with abs-sums (the forward mapping stated in the doppler direct
kernel's comment):
* torch-CPU float64 conv2d, and conv2d of |x| and |w| for the abs-sum;
* the adjoint identity <conv(x,w), g> = <x, grad_input(g,w)> with the
  oracle's grad_input, written from the input side;
* the sampled entry point against the full tensor;
* mutants.
"""
import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")


def rand_shape(rng):
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


def pin_bias_ones(o):
    for N, Co, oH, oW in [(1, 1, 1, 1), (3, 4, 5, 6), (2, 7, 1, 9)]:
        v, S = o.grad_bias(np.ones((N, Co, oH, oW)))
        assert np.array_equal(v, np.full(Co, N * oH * oW, dtype=float))
        assert np.array_equal(S, v)


def pin_bias_adjoint(o):
    rng = np.random.default_rng(201)
    for _ in range(20):
        N, Co, oH, oW = (int(x) for x in rng.integers(1, 6, size=4))
        g = rng.standard_normal((N, Co, oH, oW))
        y = rng.standard_normal((N, Co, oH, oW))
        b = rng.standard_normal(Co)
        yb = y + b[None, :, None, None]
        lhs = float(np.sum(yb * g) - np.sum(y * g))
        rhs = float(np.dot(b, o.grad_bias(g, with_abs=False)))
        assert abs(lhs - rhs) <= 1e-10 * (1 + abs(lhs)), (lhs, rhs)


def pin_bias_torch(o):
    rng = np.random.default_rng(203)
    for _ in range(10):
        sh = rand_shape(rng)
        x = torch.from_numpy(rng.standard_normal(sh.dst_shape))
        w = torch.from_numpy(rng.standard_normal(sh.weight_shape))
        b = torch.zeros(sh.Co, dtype=torch.float64, requires_grad=True)
        y = torch.nn.functional.conv2d(x, w, b, stride=sh.stride, padding=(sh.pad_h, sh.pad_w))
        g = torch.from_numpy(rng.standard_normal(tuple(y.shape)))
        y.backward(g)
        v, S = o.grad_bias(g.numpy())
        assert np.max(np.abs(v - b.grad.numpy())) <= 1e-12 * (1 + np.abs(v).max())
        assert np.all(np.abs(v) <= S * (1 + 1e-15))


def pin_fwd_torch(o):
    rng = np.random.default_rng(207)
    for _ in range(25):
        sh = rand_shape(rng)
        x = rng.standard_normal(sh.dst_shape)
        w = rng.standard_normal(sh.weight_shape)
        y, S = o.conv2d_forward_abs(x, w, sh.stride, (sh.pad_h, sh.pad_w))
        ref = torch.nn.functional.conv2d(torch.from_numpy(x), torch.from_numpy(w),
                                         stride=sh.stride, padding=(sh.pad_h, sh.pad_w)).numpy()
        assert np.max(np.abs(y - ref)) <= 1e-12 * (1 + np.abs(ref).max()), sh
        refS = torch.nn.functional.conv2d(torch.from_numpy(np.abs(x)), torch.from_numpy(np.abs(w)),
                                          stride=sh.stride, padding=(sh.pad_h, sh.pad_w)).numpy()
        assert np.max(np.abs(S - refS)) <= 1e-12 * (1 + refS.max()), sh


def pin_fwd_adjoint(o):
    rng = np.random.default_rng(209)
    for _ in range(25):
        sh = rand_shape(rng)
        x = rng.standard_normal(sh.dst_shape)
        w = rng.standard_normal(sh.weight_shape)
        g = rng.standard_normal(sh.grad_out_shape)
        y = o.conv2d_forward_abs(x, w, sh.stride, (sh.pad_h, sh.pad_w), with_abs=False)
        gi = o.grad_input(g, w, sh.stride, (sh.pad_h, sh.pad_w), (sh.H, sh.W), with_abs=False)
        lhs, rhs = float(np.sum(y * g)), float(np.sum(x * gi))
        assert abs(lhs - rhs) <= 1e-10 * (1 + abs(lhs)), (sh, lhs, rhs)


def pin_fwd_sampled(o):
    rng = np.random.default_rng(211)
    for _ in range(10):
        sh = rand_shape(rng)
        x = rng.standard_normal(sh.dst_shape)
        w = rng.standard_normal(sh.weight_shape)
        y, S = o.conv2d_forward_abs(x, w, sh.stride, (sh.pad_h, sh.pad_w))
        idx = rng.integers(0, y.size, size=30)
        v, vs = o.conv2d_forward_at(x, w, sh.stride, (sh.pad_h, sh.pad_w), idx)
        assert np.array_equal(v, y.ravel()[idx]) and np.array_equal(vs, S.ravel()[idx])
    v, vs = o.conv2d_forward_at(x, w, sh.stride, (sh.pad_h, sh.pad_w), [-1, y.size])
    assert np.isnan(v).all() and np.isnan(vs).all()


PINS = [pin_bias_ones, pin_bias_adjoint, pin_bias_torch, pin_fwd_torch, pin_fwd_adjoint,
        pin_fwd_sampled]


@pytest.fixture(scope="module")
def o():
    oracle.build()
    return oracle.Oracle(oracle.LIB_PATH)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(o, pin):
    pin(o)


MUTANTS = {
    # the last batch item dropped from the bias sum
    "bias_drop_n": ("        for (int64_t n = 0; n < N; ++n) {\n            const double *gp = grad_out + (n * Co + co) * plane;",
                    "        for (int64_t n = 0; n < N - 1; ++n) {\n            const double *gp = grad_out + (n * Co + co) * plane;"),
    # channel planes addressed with the batch stride swapped in
    "bias_plane": ("const double *gp = grad_out + (n * Co + co) * plane;",
                   "const double *gp = grad_out + (co * N + n) * plane;"),
    # the bias abs-sum takes signed values
    "bias_abs_signed": ("acc_abs += fabs(gp[p]);", "acc_abs += gp[p];"),
    # forward: tap offset with the wrong sign
    "fwd_kh_sign": ("int64_t ih = oh * s->stride - s->pad_h + kh;\n            if (ih < 0 || ih >= s->H) continue;\n            for (int64_t kw = 0; kw < s->kW; ++kw) {\n                int64_t iw = ow * s->stride - s->pad_w + kw;",
                    "int64_t ih = oh * s->stride + s->pad_h - kh;\n            if (ih < 0 || ih >= s->H) continue;\n            for (int64_t kw = 0; kw < s->kW; ++kw) {\n                int64_t iw = ow * s->stride - s->pad_w + kw;"),
    # forward: stride dropped from the column
    "fwd_no_stride": ("                int64_t iw = ow * s->stride - s->pad_w + kw;\n                if (iw < 0 || iw >= s->W) continue;\n                double t = xp[ih * s->W + iw] * wp[kh * s->kW + kw];",
                      "                int64_t iw = ow - s->pad_w + kw;\n                if (iw < 0 || iw >= s->W) continue;\n                double t = xp[ih * s->W + iw] * wp[kh * s->kW + kw];"),
    # forward: the abs-sum takes signed values
    "fwd_abs_signed": ("                acc += t;\n                acc_abs += fabs(t);\n            }\n        }\n    }\n    *value = acc;\n    *abs_value = acc_abs;\n}\n\n/*\n * Forward cross-correlation with",
                       "                acc += t;\n                acc_abs += t;\n            }\n        }\n    }\n    *value = acc;\n    *abs_value = acc_abs;\n}\n\n/*\n * Forward cross-correlation with"),
    # forward sampled: index decoded with oH and oW swapped
    "fwd_at_decode": ("        int64_t oh = (f / s.oW) % s.oH;\n        int64_t co = (f / (s.oW * s.oH)) % s.Co;",
                      "        int64_t oh = (f / s.oH) % s.oW;\n        int64_t co = (f / (s.oW * s.oH)) % s.Co;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, "mutation anchor not found: %s" % name
    cpath = tmp_path / ("mut_%s.c" % name)
    cpath.write_text(src.replace(old, new, 1))
    m = oracle.Oracle(oracle.compile_library(str(cpath), str(tmp_path / ("libmut_%s.so" % name))))
    caught = []
    for pin in PINS:
        try:
            pin(m)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "mutant %s passed every pin" % name
