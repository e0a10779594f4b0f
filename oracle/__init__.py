"""CPU oracle for conv2d grad_input and grad_weight (fp64 accumulation).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The GPU library never does, and this
package imports nothing from it.

The arithmetic lives in ``oracle.c`` (plain C, OpenMP over output rows); this
module compiles it with gcc and marshals numpy arrays through ctypes.  What each
function computes, and which page passage it follows, is stated in ``oracle.c``:

* ``grad_input``     -- the definition of grad_input (doppler
  ``conv2d_backward_input.wgsl`` direct kernel; meganeura
  ``conv2d_grad_input_gemm.wgsl`` general-stride gather), batched, with
  per-dimension padding.  Also returns sum |g*w| per element.
* ``grad_input_at``  -- the same at chosen flat indices of [N,Ci,H,W].
* ``conv2d_forward`` -- the forward cross-correlation, written separately from
  the output side (forward mapping stated in the doppler direct kernel).
* ``grad_weight``    -- the gradient with respect to the weight (the
  computeGradWeight branch of doppler ``conv2d_backward.js``: [Co,Ci,kH,kW]
  from grad_out and the forward input), the derivative of the forward mapping,
  written from the weight side.  Also returns sum |g*x| per element.
* ``grad_weight_at`` -- the same at chosen flat indices of [Co,Ci,kH,kW].
* ``conv2d_forward_abs`` / ``conv2d_forward_at`` -- the forward result with
  sum |x*w| per output element, full or at chosen flat indices of [N,Co,oH,oW].
* ``grad_bias``      -- the per-output-channel bias gradient: grad_out summed
  over (n, oh, ow) (doppler ``bias_add_backward.wgsl``), with sum |g|.

Every function is pinned by tests against hand-worked examples, closed forms,
the adjoint identity, finite differences and torch-CPU float64 library
routines; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_I = ctypes.c_int
_P = ctypes.c_void_p
_SHAPE_ARGS = [_I] * 12


def compile_library(src: str, out: str) -> str:
    """gcc -O2 with OpenMP and no fast-math; ``out`` is replaced atomically."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-Werror", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build() -> str:
    """Compile oracle.c into liboracle.so next to it (always recompiles)."""
    global _default
    compile_library(SOURCE, LIB_PATH)
    _default = None
    return LIB_PATH


def _f64(a) -> np.ndarray:
    """Widen to contiguous float64.  bf16 values arrive as float32 (exact)."""
    return np.ascontiguousarray(np.asarray(a), dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _shape(grad_out, weight, stride, padding, input_hw):
    N, Co, oH, oW = grad_out.shape
    Co_w, Ci, kH, kW = weight.shape
    if Co_w != Co:
        raise ValueError("weight has %d output channels, grad_out has %d" % (Co_w, Co))
    H, W = input_hw
    ph, pw = padding
    if stride < 1 or ph < 0 or pw < 0:
        raise ValueError("stride must be >= 1 and padding >= 0")
    return (int(N), int(Ci), int(H), int(W), int(Co), int(kH), int(kW),
            int(stride), int(ph), int(pw), int(oH), int(oW))


class Oracle:
    """The oracle's functions bound to one compiled library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_grad_input_f64.argtypes = [_P, _P, _P, _P] + _SHAPE_ARGS
        lib.oracle_grad_input_f64.restype = None
        lib.oracle_grad_input_at_f64.argtypes = [_P, _P, _P, ctypes.c_int64, _P, _P] + _SHAPE_ARGS
        lib.oracle_grad_input_at_f64.restype = None
        lib.oracle_conv2d_fwd_f64.argtypes = [_P, _P, _P] + _SHAPE_ARGS
        lib.oracle_conv2d_fwd_f64.restype = None
        lib.oracle_grad_weight_f64.argtypes = [_P, _P, _P, _P] + _SHAPE_ARGS
        lib.oracle_grad_weight_f64.restype = None
        lib.oracle_grad_weight_at_f64.argtypes = [_P, _P, _P, ctypes.c_int64, _P, _P] + _SHAPE_ARGS
        lib.oracle_grad_weight_at_f64.restype = None
        lib.oracle_conv2d_fwd_abs_f64.argtypes = [_P, _P, _P, _P] + _SHAPE_ARGS
        lib.oracle_conv2d_fwd_abs_f64.restype = None
        lib.oracle_conv2d_fwd_at_f64.argtypes = [_P, _P, _P, ctypes.c_int64, _P, _P] + _SHAPE_ARGS
        lib.oracle_conv2d_fwd_at_f64.restype = None
        lib.oracle_grad_bias_f64.argtypes = [_P, _P, _P, _I, _I, _I, _I]
        lib.oracle_grad_bias_f64.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = _I
        self.lib = lib
        self.path = path

    def num_threads(self) -> int:
        """OpenMP threads the oracle runs on (OMP_NUM_THREADS, else all cores)."""
        return int(self.lib.oracle_num_threads())

    def grad_input(self, grad_out, weight, stride, padding, input_hw, with_abs=True):
        """grad_input [N,Ci,H,W] (float64) and, if asked, sum |g*w| per element.

        grad_out: [N,Co,oH,oW]; weight: [Co,Ci,kH,kW]; padding = (pad_h, pad_w);
        input_hw = (H, W) of the forward input (several H map to one oH when
        stride > 1, so it is given, not derived).
        """
        g = _f64(grad_out)
        w = _f64(weight)
        sh = _shape(g, w, stride, padding, input_hw)
        N, Ci, H, W = sh[0], sh[1], sh[2], sh[3]
        out = np.empty((N, Ci, H, W), dtype=np.float64)
        s = np.empty_like(out) if with_abs else None
        self.lib.oracle_grad_input_f64(_ptr(g), _ptr(w), _ptr(out),
                                       _ptr(s) if s is not None else None, *sh)
        return (out, s) if with_abs else out

    def grad_input_at(self, grad_out, weight, stride, padding, input_hw, flat_idx):
        """grad_input and sum |g*w| at flat indices of the [N,Ci,H,W] result."""
        g = _f64(grad_out)
        w = _f64(weight)
        sh = _shape(g, w, stride, padding, input_hw)
        idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64).ravel())
        out = np.empty(idx.shape[0], dtype=np.float64)
        s = np.empty_like(out)
        self.lib.oracle_grad_input_at_f64(_ptr(g), _ptr(w), _ptr(idx),
                                          ctypes.c_int64(idx.shape[0]), _ptr(out),
                                          _ptr(s), *sh)
        return out, s

    def _gw_shape(self, x, grad_out, stride, padding, kernel_hw):
        N, Ci, H, W = x.shape
        Ng, Co, oH, oW = grad_out.shape
        if Ng != N:
            raise ValueError("x has %d batch items, grad_out has %d" % (N, Ng))
        kH, kW = kernel_hw
        ph, pw = padding
        if stride < 1 or ph < 0 or pw < 0:
            raise ValueError("stride must be >= 1 and padding >= 0")
        if (H + 2 * ph - kH) // stride + 1 != oH or (W + 2 * pw - kW) // stride + 1 != oW:
            raise ValueError("grad_out size does not match the forward geometry")
        return (int(N), int(Ci), int(H), int(W), int(Co), int(kH), int(kW), int(stride),
                int(ph), int(pw), int(oH), int(oW))

    def grad_weight(self, x, grad_out, stride, padding, kernel_hw, with_abs=True):
        """grad_weight [Co,Ci,kH,kW] (float64) and, if asked, sum |g*x| per element.

        x: the forward input [N,Ci,H,W]; grad_out: [N,Co,oH,oW];
        padding = (pad_h, pad_w); kernel_hw = (kH, kW).
        """
        x = _f64(x)
        g = _f64(grad_out)
        sh = self._gw_shape(x, g, stride, padding, kernel_hw)
        Ci, Co, kH, kW = sh[1], sh[4], sh[5], sh[6]
        out = np.empty((Co, Ci, kH, kW), dtype=np.float64)
        s = np.empty_like(out) if with_abs else None
        self.lib.oracle_grad_weight_f64(_ptr(x), _ptr(g), _ptr(out),
                                        _ptr(s) if s is not None else None, *sh)
        return (out, s) if with_abs else out

    def grad_weight_at(self, x, grad_out, stride, padding, kernel_hw, flat_idx):
        """grad_weight and sum |g*x| at flat indices of the [Co,Ci,kH,kW] result."""
        x = _f64(x)
        g = _f64(grad_out)
        sh = self._gw_shape(x, g, stride, padding, kernel_hw)
        idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64).ravel())
        out = np.empty(idx.shape[0], dtype=np.float64)
        s = np.empty_like(out)
        self.lib.oracle_grad_weight_at_f64(_ptr(x), _ptr(g), _ptr(idx),
                                           ctypes.c_int64(idx.shape[0]), _ptr(out), _ptr(s),
                                           *sh)
        return out, s

    def conv2d_forward(self, x, weight, stride, padding):
        """Forward cross-correlation y [N,Co,oH,oW], oH = (H+2ph-kH)//stride + 1."""
        x = _f64(x)
        w = _f64(weight)
        N, Ci, H, W = x.shape
        Co, Ci_w, kH, kW = w.shape
        if Ci_w != Ci:
            raise ValueError("weight has %d input channels, x has %d" % (Ci_w, Ci))
        ph, pw = padding
        oH = (H + 2 * ph - kH) // stride + 1
        oW = (W + 2 * pw - kW) // stride + 1
        if oH < 1 or oW < 1:
            raise ValueError("empty forward output")
        y = np.empty((N, Co, oH, oW), dtype=np.float64)
        self.lib.oracle_conv2d_fwd_f64(_ptr(x), _ptr(w), _ptr(y), N, Ci, H, W, Co,
                                       kH, kW, int(stride), int(ph), int(pw), oH, oW)
        return y


    def _fwd_shape(self, x, w, stride, padding):
        N, Ci, H, W = x.shape
        Co, Ci_w, kH, kW = w.shape
        if Ci_w != Ci:
            raise ValueError("weight has %d input channels, x has %d" % (Ci_w, Ci))
        ph, pw = padding
        if stride < 1 or ph < 0 or pw < 0:
            raise ValueError("stride must be >= 1 and padding >= 0")
        oH = (H + 2 * ph - kH) // stride + 1
        oW = (W + 2 * pw - kW) // stride + 1
        if oH < 1 or oW < 1:
            raise ValueError("empty forward output")
        return (int(N), int(Ci), int(H), int(W), int(Co), int(kH), int(kW), int(stride),
                int(ph), int(pw), int(oH), int(oW))

    def conv2d_forward_abs(self, x, weight, stride, padding, with_abs=True):
        """Forward y [N,Co,oH,oW] and, if asked, sum |x*w| per output element."""
        x = _f64(x)
        w = _f64(weight)
        sh = self._fwd_shape(x, w, stride, padding)
        y = np.empty((sh[0], sh[4], sh[10], sh[11]), dtype=np.float64)
        s = np.empty_like(y) if with_abs else None
        self.lib.oracle_conv2d_fwd_abs_f64(_ptr(x), _ptr(w), _ptr(y),
                                           _ptr(s) if s is not None else None, *sh)
        return (y, s) if with_abs else y

    def conv2d_forward_at(self, x, weight, stride, padding, flat_idx):
        """Forward result and sum |x*w| at flat indices of [N,Co,oH,oW]."""
        x = _f64(x)
        w = _f64(weight)
        sh = self._fwd_shape(x, w, stride, padding)
        idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64).ravel())
        out = np.empty(idx.shape[0], dtype=np.float64)
        s = np.empty_like(out)
        self.lib.oracle_conv2d_fwd_at_f64(_ptr(x), _ptr(w), _ptr(idx),
                                          ctypes.c_int64(idx.shape[0]), _ptr(out), _ptr(s), *sh)
        return out, s

    def grad_bias(self, grad_out, with_abs=True):
        """grad_bias [Co] (float64) and, if asked, sum |g| per channel."""
        g = _f64(grad_out)
        N, Co, oH, oW = g.shape
        out = np.empty(Co, dtype=np.float64)
        s = np.empty_like(out) if with_abs else None
        self.lib.oracle_grad_bias_f64(_ptr(g), _ptr(out), _ptr(s) if s is not None else None,
                                      int(N), int(Co), int(oH), int(oW))
        return (out, s) if with_abs else out


_default = None


def _get() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build()
        _default = Oracle(LIB_PATH)
    return _default


def num_threads() -> int:
    return _get().num_threads()


def grad_input(grad_out, weight, stride, padding, input_hw, with_abs=True):
    return _get().grad_input(grad_out, weight, stride, padding, input_hw, with_abs)


def grad_input_at(grad_out, weight, stride, padding, input_hw, flat_idx):
    return _get().grad_input_at(grad_out, weight, stride, padding, input_hw, flat_idx)


def conv2d_forward(x, weight, stride, padding):
    return _get().conv2d_forward(x, weight, stride, padding)


def grad_weight(x, grad_out, stride, padding, kernel_hw, with_abs=True):
    return _get().grad_weight(x, grad_out, stride, padding, kernel_hw, with_abs)


def grad_weight_at(x, grad_out, stride, padding, kernel_hw, flat_idx):
    return _get().grad_weight_at(x, grad_out, stride, padding, kernel_hw, flat_idx)


def conv2d_forward_abs(x, weight, stride, padding, with_abs=True):
    return _get().conv2d_forward_abs(x, weight, stride, padding, with_abs)


def conv2d_forward_at(x, weight, stride, padding, flat_idx):
    return _get().conv2d_forward_at(x, weight, stride, padding, flat_idx)


def grad_bias(grad_out, with_abs=True):
    return _get().grad_bias(grad_out, with_abs)


grad_input.__doc__ = Oracle.grad_input.__doc__
grad_input_at.__doc__ = Oracle.grad_input_at.__doc__
conv2d_forward.__doc__ = Oracle.conv2d_forward.__doc__
grad_weight.__doc__ = Oracle.grad_weight.__doc__
grad_weight_at.__doc__ = Oracle.grad_weight_at.__doc__
conv2d_forward_abs.__doc__ = Oracle.conv2d_forward_abs.__doc__
conv2d_forward_at.__doc__ = Oracle.conv2d_forward_at.__doc__
grad_bias.__doc__ = Oracle.grad_bias.__doc__
