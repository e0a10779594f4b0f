"""conv2d grad_input for MI355X (gfx950): Python binding of ``libconv2d_gi.so``.

The binding only marshals arguments: every step of the computation runs in the
library's HIP kernels.  PyTorch provides device memory and the current stream.
If the library has not been built, importing works but every call raises
``LibraryNotBuilt`` -- there is no CPU fallback.

    from conv2d_backward_amd import grad_input
    dx = grad_input(dy, w, stride=2, padding=(1, 1), input_hw=(56, 56))

The C entry points mirror these names (include/conv2d_grad_input.h; the test
hooks are in include/conv2d_grad_input_testing.h and are thread-local).
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "grad_input", "grad_input_noalloc", "Conv2dGiParams", "Conv2dGiError", "LibraryNotBuilt", "load_library",
    "make_params", "validate", "plan", "grad_weight", "grad_weight_plan", "grad_bias", "backward", "forward", "forward_plan", "set_fwd_variant", "set_variant", "set_halo_tile", "set_halo_split", "set_halo_fusion", "set_gw_variant", "set_gw_tile", "release_workspaces", "set_profile_events", "mfma_peak", "library_path", "exported_names",
    "OK", "EINVAL", "EUNSUPPORTED", "EHIP", "VARIANT_AUTO", "VARIANT_GENERIC", "VARIANT_HALO", "VARIANT_STEM",
    "VARIANT_COL2IM",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libconv2d_gi.so")

OK, EINVAL, EUNSUPPORTED, EHIP = 0, 1, 2, 3
VARIANT_AUTO, VARIANT_GENERIC, VARIANT_HALO, VARIANT_STEM, VARIANT_COL2IM = 0, 1, 2, 3, 4

_FIELDS = ("N", "Ci", "H", "W", "Co", "kH", "kW", "stride", "pad_h", "pad_w", "oH", "oW")


class Conv2dGiParams(ctypes.Structure):
    """Mirror of ``conv2d_gi_params`` (twelve int32 fields)."""
    _fields_ = [(f, ctypes.c_int32) for f in _FIELDS]

    def __repr__(self):
        return "Conv2dGiParams(%s)" % ", ".join("%s=%d" % (f, getattr(self, f)) for f in _FIELDS)


class Conv2dGiError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("conv2d_grad_input failed (%d): %s" % (code, msg))
        self.code = code


class LibraryNotBuilt(ImportError):
    pass


_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load the in-tree HIP library (built by ``conv2d_backward_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or library_path
    if not os.path.exists(p):
        raise LibraryNotBuilt(
            "%s is missing: build it with `python -m conv2d_backward_amd.build`" % p)
    lib = ctypes.CDLL(p)
    P = ctypes.c_void_p
    PP = Conv2dGiParams  # passed by value
    lib.conv2d_grad_input.argtypes = [P, P, P, PP, P]
    lib.conv2d_grad_input.restype = ctypes.c_int
    lib.conv2d_grad_input_bf16.argtypes = [P, P, P, PP, P]
    lib.conv2d_grad_input_bf16.restype = ctypes.c_int
    lib.conv2d_grad_input_f16.argtypes = [P, P, P, PP, P]
    lib.conv2d_grad_input_noalloc.argtypes = [P, P, P, PP, P]
    lib.conv2d_grad_input_noalloc.restype = ctypes.c_int
    lib.conv2d_grad_input_f16.restype = ctypes.c_int
    lib.conv2d_gi_validate.argtypes = [PP]
    lib.conv2d_gi_validate.restype = ctypes.c_int
    lib.conv2d_gi_strerror.argtypes = [ctypes.c_int]
    lib.conv2d_gi_strerror.restype = ctypes.c_char_p
    lib.conv2d_gi_last_hip_error.argtypes = []
    lib.conv2d_gi_last_hip_error.restype = ctypes.c_char_p
    lib.conv2d_gi_set_variant.argtypes = [ctypes.c_int]
    lib.conv2d_gi_set_variant.restype = ctypes.c_int
    lib.conv2d_gi_plan.argtypes = [PP, ctypes.c_int, ctypes.c_char_p, ctypes.c_size_t]
    lib.conv2d_gi_plan.restype = ctypes.c_int
    lib.conv2d_grad_weight.argtypes = [P, P, P, PP, P]
    lib.conv2d_grad_weight.restype = ctypes.c_int
    lib.conv2d_backward.argtypes = [P, P, P, P, P, P, PP, P]
    lib.conv2d_backward.restype = ctypes.c_int
    lib.conv2d_forward.argtypes = [P, P, P, PP, P]
    lib.conv2d_forward.restype = ctypes.c_int
    lib.conv2d_fwd_plan.argtypes = [PP, ctypes.c_char_p, ctypes.c_size_t]
    lib.conv2d_fwd_plan.restype = ctypes.c_int
    lib.conv2d_fwd_set_variant.argtypes = [ctypes.c_int]
    lib.conv2d_fwd_set_variant.restype = ctypes.c_int
    lib.conv2d_grad_bias.argtypes = [P, P, PP, P]
    lib.conv2d_grad_bias.restype = ctypes.c_int
    lib.conv2d_gw_plan.argtypes = [PP, ctypes.c_char_p, ctypes.c_size_t]
    lib.conv2d_gw_plan.restype = ctypes.c_int
    lib.conv2d_gi_set_halo_tile.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.conv2d_gi_set_halo_tile.restype = ctypes.c_int
    lib.conv2d_gi_set_halo_split.argtypes = [ctypes.c_int]
    lib.conv2d_gi_set_halo_split.restype = ctypes.c_int
    lib.conv2d_gi_set_halo_fusion.argtypes = [ctypes.c_int]
    lib.conv2d_gi_set_halo_fusion.restype = ctypes.c_int
    lib.conv2d_gw_set_variant.argtypes = [ctypes.c_int]
    lib.conv2d_gw_set_variant.restype = ctypes.c_int
    lib.conv2d_gw_set_tile.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.conv2d_gw_set_tile.restype = ctypes.c_int
    lib.conv2d_gi_set_profile_events.argtypes = [P, P]
    lib.conv2d_gi_set_profile_events.restype = None
    lib.conv2d_gi_release_workspaces.argtypes = []
    lib.conv2d_gi_release_workspaces.restype = ctypes.c_int
    lib.conv2d_gi_version.argtypes = []
    lib.conv2d_gi_version.restype = ctypes.c_char_p
    lib.conv2d_gi_mfma_peak_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P,
                                              ctypes.POINTER(ctypes.c_double)]
    lib.conv2d_gi_mfma_peak_probe.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def exported_names():
    """Names of the C entry points the binding wraps."""
    return ["conv2d_grad_input", "conv2d_grad_input_bf16", "conv2d_grad_input_f16",
            "conv2d_grad_input_noalloc",
            "conv2d_grad_weight",
            "conv2d_backward", "conv2d_grad_bias", "conv2d_forward", "conv2d_fwd_plan",
            "conv2d_fwd_set_variant",
            "conv2d_gw_plan", "conv2d_gi_validate",
            "conv2d_gi_strerror", "conv2d_gi_last_hip_error", "conv2d_gi_set_variant",
            "conv2d_gi_plan", "conv2d_gi_set_halo_tile", "conv2d_gi_set_halo_split",
            "conv2d_gi_set_halo_fusion", "conv2d_gw_set_variant", "conv2d_gw_set_tile",
            "conv2d_gi_set_profile_events",
            "conv2d_gi_release_workspaces", "conv2d_gi_version", "conv2d_gi_mfma_peak_probe"]


def make_params(N, Ci, H, W, Co, kH, kW, stride, pad_h, pad_w, oH=None, oW=None):
    """Build a params struct; oH/oW default to the forward-conv formula."""
    if oH is None:
        oH = (H + 2 * pad_h - kH) // stride + 1
    if oW is None:
        oW = (W + 2 * pad_w - kW) // stride + 1
    return Conv2dGiParams(N, Ci, H, W, Co, kH, kW, stride, pad_h, pad_w, oH, oW)


def _check(code: int):
    if code != OK:
        lib = load_library()
        msg = lib.conv2d_gi_strerror(code).decode()
        if code == EHIP:
            msg += ": " + lib.conv2d_gi_last_hip_error().decode()
        raise Conv2dGiError(code, msg)


def validate(p: Conv2dGiParams) -> int:
    """Host-only shape check; returns the status code (no HIP call)."""
    return load_library().conv2d_gi_validate(p)


def plan(p: Conv2dGiParams, bf16=False) -> str:
    """Host-only: the plan the library would run for this shape; bf16: False
    or 0 for fp32 inputs, True or 1 for bf16, 2 for fp16."""
    buf = ctypes.create_string_buffer(8192)
    _check(load_library().conv2d_gi_plan(p, int(bf16), buf, len(buf)))
    return buf.value.decode()


def set_variant(variant: int) -> int:
    """Force a kernel variant (VARIANT_AUTO restores the planner); returns the old one."""
    old = load_library().conv2d_gi_set_variant(int(variant))
    if old < 0:
        raise ValueError("unknown variant %r" % (variant,))
    return old


def set_halo_tile(nb: int = 0, tile_rows: int = 0, tile_cols: int = 0, stages: int = 0):
    """Force the HALO variant's pixel tile (fp32: blocks per work-group, tile
    and pipeline depth; bf16: blocks per wave and tile) for this thread's later calls (test
    hook); set_halo_tile() restores the planner."""
    _check(load_library().conv2d_gi_set_halo_tile(int(nb), int(tile_rows), int(tile_cols),
                                                  int(stages)))


def set_halo_split(groups: int = 0):
    """Force 1 or 2 thread groups splitting the output channels of an fp32
    HALO work-group for this thread's later calls (test hook); set_halo_split() restores the
    planner."""
    _check(load_library().conv2d_gi_set_halo_split(int(groups)))


def set_halo_fusion(mode: int = 0):
    """Force the fp32 HALO variant to run a tile's stride phases one after
    another (1) or all per chunk over one shared halo (2) for this thread's later
    calls (test hook); set_halo_fusion() restores the planner."""
    _check(load_library().conv2d_gi_set_halo_fusion(int(mode)))


def set_gw_variant(mode: int = 0):
    """Force grad_weight onto the 4-byte-load kernel (1) or the 16-byte-load
    kernel (2; shapes it does not cover raise) for this thread's later calls (test hook);
    set_gw_variant() restores the planner."""
    _check(load_library().conv2d_gw_set_variant(int(mode)))


def set_gw_tile(rows: int = 0, stages: int = 0, max_slices: int = 0):
    """Force the 16-byte-load grad_weight kernel's rows per pixel group, LDS
    stages and most slices for this thread's later calls (test hook); set_gw_tile()
    restores the planner."""
    _check(load_library().conv2d_gw_set_tile(int(rows), int(stages), int(max_slices)))


def release_workspaces():
    """Free the library's cached per-stream scratch buffers."""
    _check(load_library().conv2d_gi_release_workspaces())


def mfma_peak(kind: str, seconds: float = 0.05):
    """Sustained matrix-core rate in TFLOP/s ("f32": V_MFMA_F32_16X16X4_F32,
    "bf16": V_MFMA_F32_16X16X32_BF16) on the current device: a probe kernel
    of back-to-back independent MFMAs on varied data, two waves per SIMD of
    every compute unit, timed with events after a warm-up of about the same
    length (so the clock has settled)."""
    import torch

    lib = load_library()
    k = {"f32": 0, "bf16": 1}[kind]
    dev = torch.cuda.current_device()
    # Two work-groups of 4 waves per compute unit: two waves per SIMD.
    wgs = 2 * torch.cuda.get_device_properties(dev).multi_processor_count
    scratch = torch.empty(wgs, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    fl = ctypes.c_double()

    def launch(iters):
        _check(lib.conv2d_gi_mfma_peak_probe(k, wgs, iters, _ptr(scratch),
                                             ctypes.c_void_p(s.cuda_stream), ctypes.byref(fl)))

    launch(1000)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    launch(1000)
    e1.record()
    torch.cuda.synchronize()
    iters = max(1000, int(1000 * seconds / max(e0.elapsed_time(e1) * 1e-3, 1e-6)))
    launch(iters)   # warm-up of about `seconds`
    e0.record()
    launch(iters)
    e1.record()
    torch.cuda.synchronize()
    return fl.value / (e0.elapsed_time(e1) * 1e-3) / 1e12


def set_profile_events(begin, end):
    """Record the hipEvent_t handles ``begin``/``end`` (ints or ctypes pointers)
    around the GEMM launches of later calls from this thread; None switches it off."""
    if begin is None or end is None:
        load_library().conv2d_gi_set_profile_events(None, None)
        return
    load_library().conv2d_gi_set_profile_events(begin, end)


def grad_input(grad_out, weight, *, stride: int, padding, input_hw, out=None, stream=None):
    """grad_input [N, Ci, H, W] (fp32) of a conv2d, computed on the GPU.

    grad_out [N, Co, oH, oW] and weight [Co, Ci, kH, kW]: both float32, both
    bfloat16 or both float16, contiguous, on the same ROCm device.  padding: int or (pad_h, pad_w).
    input_hw: (H, W) of the forward input.  out: optional float32 [N, Ci, H, W]
    tensor to write (every element is overwritten).  stream: a torch stream
    (default: the device's current stream).  The call is asynchronous on that stream.
    """
    import torch

    if isinstance(padding, int):
        padding = (padding, padding)
    pad_h, pad_w = (int(v) for v in padding)
    H, W = (int(v) for v in input_hw)
    if grad_out.dim() != 4 or weight.dim() != 4:
        raise ValueError("grad_out and weight must be 4-D (NCHW and [Co,Ci,kH,kW])")
    if not (grad_out.is_cuda and weight.is_cuda) or grad_out.device != weight.device:
        raise ValueError("grad_out and weight must be on the same GPU device")
    if grad_out.dtype != weight.dtype or grad_out.dtype not in (torch.float32, torch.bfloat16,
                                                                torch.float16):
        raise ValueError("grad_out and weight must both be float32, bfloat16 or float16")
    if not (grad_out.is_contiguous() and weight.is_contiguous()):
        raise ValueError("grad_out and weight must be contiguous")
    N, Co, oH, oW = (int(v) for v in grad_out.shape)
    Co_w, Ci, kH, kW = (int(v) for v in weight.shape)
    if Co_w != Co:
        raise ValueError("weight has %d output channels, grad_out %d" % (Co_w, Co))
    p = Conv2dGiParams(N, Ci, H, W, Co, kH, kW, int(stride), pad_h, pad_w, oH, oW)
    lib = load_library()
    _check(lib.conv2d_gi_validate(p))
    dev = grad_out.device
    if out is None:
        out = torch.empty((N, Ci, H, W), dtype=torch.float32, device=dev)
    else:
        if (out.dtype != torch.float32 or out.device != dev or not out.is_contiguous()
                or tuple(out.shape) != (N, Ci, H, W)):
            raise ValueError("out must be a contiguous float32 [N,Ci,H,W] tensor on %s" % dev)
    with torch.cuda.device(dev):
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        fn = {torch.bfloat16: lib.conv2d_grad_input_bf16, torch.float16: lib.conv2d_grad_input_f16,
              torch.float32: lib.conv2d_grad_input}[grad_out.dtype]
        code = fn(ctypes.c_void_p(grad_out.data_ptr()), ctypes.c_void_p(weight.data_ptr()),
                  ctypes.c_void_p(out.data_ptr()), p,
                  ctypes.c_void_p(s.cuda_stream))
    _check(code)
    return out


def grad_input_noalloc(grad_out, weight, *, stride: int, padding, input_hw, out, stream=None):
    """fp32 grad_input through ``conv2d_grad_input_noalloc``: the library
    allocates nothing (its scratch is a fixed per-GPU array; plans needing more
    raise with EUNSUPPORTED).  ``out`` (float32 [N, Ci, H, W], contiguous) is
    required.  Calls that can overlap on one GPU race on that array."""
    import torch

    if isinstance(padding, int):
        padding = (padding, padding)
    pad_h, pad_w = (int(v) for v in padding)
    H, W = (int(v) for v in input_hw)
    for t in (grad_out, weight, out):
        if t.dim() != 4 or not t.is_cuda or t.device != grad_out.device:
            raise ValueError("grad_out, weight and out must be 4-D tensors on one GPU device")
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("grad_out, weight and out must be contiguous float32")
    N, Co, oH, oW = (int(v) for v in grad_out.shape)
    Co_w, Ci, kH, kW = (int(v) for v in weight.shape)
    if Co_w != Co or tuple(out.shape) != (N, Ci, H, W):
        raise ValueError("inconsistent shapes: weight [Co,Ci,kH,kW], out [N,Ci,H,W]")
    p = Conv2dGiParams(N, Ci, H, W, Co, kH, kW, int(stride), pad_h, pad_w, oH, oW)
    lib = load_library()
    with torch.cuda.device(grad_out.device):
        s = stream if stream is not None else torch.cuda.current_stream(grad_out.device)
        code = lib.conv2d_grad_input_noalloc(_ptr(grad_out), _ptr(weight), _ptr(out), p,
                                             ctypes.c_void_p(s.cuda_stream))
    _check(code)
    return out


def grad_weight_plan(p: Conv2dGiParams) -> str:
    """Description of the launches conv2d_grad_weight would make for shape p."""
    buf = ctypes.create_string_buffer(1024)
    _check(load_library().conv2d_gw_plan(p, buf, len(buf)))
    return buf.value.decode()


def grad_weight(grad_out, x, *, stride: int, padding, kernel_hw, out=None, stream=None):
    """grad_weight [Co, Ci, kH, kW] (fp32) of a conv2d, computed on the GPU.

    grad_out [N, Co, oH, oW] and x [N, Ci, H, W] (the forward input): float32,
    contiguous, on the same ROCm device.  padding: int or (pad_h, pad_w).
    kernel_hw: (kH, kW).  out: optional float32 [Co, Ci, kH, kW] tensor to write
    (every element is overwritten).  stream: a torch stream (default: the
    device's current stream).  The call is asynchronous on that stream.
    """
    import torch

    if isinstance(padding, int):
        padding = (padding, padding)
    pad_h, pad_w = (int(v) for v in padding)
    kH, kW = (int(v) for v in kernel_hw)
    if grad_out.dim() != 4 or x.dim() != 4:
        raise ValueError("grad_out and x must be 4-D NCHW tensors")
    if not (grad_out.is_cuda and x.is_cuda) or grad_out.device != x.device:
        raise ValueError("grad_out and x must be on the same GPU device")
    if grad_out.dtype != torch.float32 or x.dtype != torch.float32:
        raise ValueError("grad_out and x must be float32")
    if not (grad_out.is_contiguous() and x.is_contiguous()):
        raise ValueError("grad_out and x must be contiguous")
    N, Co, oH, oW = (int(v) for v in grad_out.shape)
    Nx, Ci, H, W = (int(v) for v in x.shape)
    if Nx != N:
        raise ValueError("x has %d batch items, grad_out %d" % (Nx, N))
    p = Conv2dGiParams(N, Ci, H, W, Co, kH, kW, int(stride), pad_h, pad_w, oH, oW)
    lib = load_library()
    _check(lib.conv2d_gi_validate(p))
    dev = grad_out.device
    if out is None:
        out = torch.empty((Co, Ci, kH, kW), dtype=torch.float32, device=dev)
    elif (out.dtype != torch.float32 or out.device != dev or not out.is_contiguous()
          or tuple(out.shape) != (Co, Ci, kH, kW)):
        raise ValueError("out must be a contiguous float32 [Co,Ci,kH,kW] tensor on %s" % dev)
    with torch.cuda.device(dev):
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        code = lib.conv2d_grad_weight(ctypes.c_void_p(grad_out.data_ptr()),
                                      ctypes.c_void_p(x.data_ptr()),
                                      ctypes.c_void_p(out.data_ptr()), p,
                                      ctypes.c_void_p(s.cuda_stream))
    _check(code)
    return out


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def backward(grad_out, x=None, weight=None, *, stride: int, padding, kernel_hw=None,
             want_dx=True, want_dw=True, want_db=False, dx=None, dw=None, db=None, stream=None):
    """The backward pass of a conv2d layer in one library call.

    Returns (dx, dw, db), each None when not asked for.  grad_out [N, Co, oH, oW],
    x [N, Ci, H, W] (needed for dw, and for the input size), weight [Co, Ci, kH,
    kW] (needed for dx): float32, contiguous, on one ROCm device.  kernel_hw
    defaults to the weight's.  dx / dw / db: optional output tensors to write.
    Asynchronous on `stream` (default: the device's current stream).
    """
    import torch

    if isinstance(padding, int):
        padding = (padding, padding)
    pad_h, pad_w = (int(v) for v in padding)
    if x is None:
        raise ValueError("x (or a tensor of its shape) gives the input size")
    if kernel_hw is None:
        if weight is None:
            raise ValueError("kernel_hw is needed without the weight")
        kernel_hw = tuple(weight.shape[2:])
    kH, kW = (int(v) for v in kernel_hw)
    tens = [t for t in (grad_out, x, weight) if t is not None]
    dev = grad_out.device
    for t in tens:
        if t.dim() != 4 or not t.is_cuda or t.device != dev:
            raise ValueError("inputs must be 4-D tensors on one GPU device")
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("inputs must be contiguous float32")
    N, Co, oH, oW = (int(v) for v in grad_out.shape)
    Nx, Ci, H, W = (int(v) for v in x.shape)
    if Nx != N:
        raise ValueError("x has %d batch items, grad_out %d" % (Nx, N))
    if want_dx and weight is None:
        raise ValueError("dx needs the weight")
    if weight is not None and tuple(weight.shape) != (Co, Ci, kH, kW):
        raise ValueError("weight must be [Co, Ci, kH, kW] = %r" % ((Co, Ci, kH, kW),))
    p = Conv2dGiParams(N, Ci, H, W, Co, kH, kW, int(stride), pad_h, pad_w, oH, oW)
    lib = load_library()
    _check(lib.conv2d_gi_validate(p))

    def out_tensor(t, want, shape, name):
        if not want:
            return None
        if t is None:
            return torch.empty(shape, dtype=torch.float32, device=dev)
        if (t.dtype != torch.float32 or t.device != dev or not t.is_contiguous()
                or tuple(t.shape) != tuple(shape)):
            raise ValueError("%s must be a contiguous float32 %r tensor on %s" % (name, shape, dev))
        return t

    dx = out_tensor(dx, want_dx, (N, Ci, H, W), "dx")
    dw = out_tensor(dw, want_dw, (Co, Ci, kH, kW), "dw")
    db = out_tensor(db, want_db, (Co,), "db")
    with torch.cuda.device(dev):
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        code = lib.conv2d_backward(_ptr(grad_out), _ptr(x if want_dw else None),
                                   _ptr(weight if want_dx else None), _ptr(dx), _ptr(dw),
                                   _ptr(db), p, ctypes.c_void_p(s.cuda_stream))
    _check(code)
    return dx, dw, db


def grad_bias(grad_out, *, out=None, stream=None):
    """Bias gradient [Co] (fp32): grad_out [N, Co, oH, oW] summed per channel."""
    import torch

    if grad_out.dim() != 4 or not grad_out.is_cuda:
        raise ValueError("grad_out must be a 4-D tensor on a GPU device")
    if grad_out.dtype != torch.float32 or not grad_out.is_contiguous():
        raise ValueError("grad_out must be contiguous float32")
    N, Co, oH, oW = (int(v) for v in grad_out.shape)
    # A 1x1 stride-1 geometry with the same output plane: only N, Co, oH, oW matter.
    p = Conv2dGiParams(N, 1, oH, oW, Co, 1, 1, 1, 0, 0, oH, oW)
    dev = grad_out.device
    if out is None:
        out = torch.empty((Co,), dtype=torch.float32, device=dev)
    elif (out.dtype != torch.float32 or out.device != dev or not out.is_contiguous()
          or tuple(out.shape) != (Co,)):
        raise ValueError("out must be a contiguous float32 [Co] tensor on %s" % dev)
    lib = load_library()
    with torch.cuda.device(dev):
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        code = lib.conv2d_grad_bias(_ptr(grad_out), _ptr(out), p,
                                    ctypes.c_void_p(s.cuda_stream))
    _check(code)
    return out


def forward_plan(p: Conv2dGiParams) -> str:
    """Description of the launches conv2d_forward would make for shape p."""
    buf = ctypes.create_string_buffer(1024)
    _check(load_library().conv2d_fwd_plan(p, buf, len(buf)))
    return buf.value.decode()


def set_fwd_variant(mode: int = 0):
    """Force the forward onto the grad_input kernels (1, stride 1 only) or the
    generic forward kernel (2) for this thread's later calls (test hook); set_fwd_variant()
    restores the planner."""
    _check(load_library().conv2d_fwd_set_variant(int(mode)))


def forward(x, weight, *, stride: int, padding, out=None, stream=None):
    """Forward conv2d y [N, Co, oH, oW] (fp32) on the GPU: x [N, Ci, H, W] and
    weight [Co, Ci, kH, kW], float32, contiguous, on one ROCm device;
    padding: int or (pad_h, pad_w).  Asynchronous on `stream`."""
    import torch

    if isinstance(padding, int):
        padding = (padding, padding)
    pad_h, pad_w = (int(v) for v in padding)
    for t in (x, weight):
        if t.dim() != 4 or not t.is_cuda or t.device != x.device:
            raise ValueError("x and weight must be 4-D tensors on one GPU device")
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("x and weight must be contiguous float32")
    N, Ci, H, W = (int(v) for v in x.shape)
    Co, Ci_w, kH, kW = (int(v) for v in weight.shape)
    if Ci_w != Ci:
        raise ValueError("weight has %d input channels, x has %d" % (Ci_w, Ci))
    p = make_params(N, Ci, H, W, Co, kH, kW, int(stride), pad_h, pad_w)
    lib = load_library()
    _check(lib.conv2d_gi_validate(p))
    dev = x.device
    if out is None:
        out = torch.empty((N, Co, p.oH, p.oW), dtype=torch.float32, device=dev)
    elif (out.dtype != torch.float32 or out.device != dev or not out.is_contiguous()
          or tuple(out.shape) != (N, Co, p.oH, p.oW)):
        raise ValueError("out must be a contiguous float32 %r tensor on %s"
                         % ((N, Co, p.oH, p.oW), dev))
    with torch.cuda.device(dev):
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        code = lib.conv2d_forward(_ptr(x), _ptr(weight), _ptr(out), p,
                                  ctypes.c_void_p(s.cuda_stream))
    _check(code)
    return out
