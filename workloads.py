"""Seeded synthetic inputs for conv2d grad_input: the named workloads and small
sweep shapes.

This module only draws numbers and names shapes.  It holds none of the
operation's arithmetic, so both the CPU oracle's tests and the GPU path's tests
and benchmark may take their inputs from it without sharing any of the method.

Recipe (every workload): numpy ``Generator(PCG64(seed))``, draws in float64,
scaled in float64, cast to float32.  ``seed = 1000*c + 10*sub + t`` where c is
the workload's index, sub is 0 for the first (or only) shape of a workload and
1 for the second, and t is 1 for grad_out, 2 for weight and 3 for the forward
input x (N(0,1); read by grad_weight).  bf16 inputs are
the float32 draws rounded to nearest-even bf16; both sides consume the same
bf16 bit patterns.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Shape:
    N: int
    Ci: int
    H: int
    W: int
    Co: int
    kH: int
    kW: int
    stride: int
    pad_h: int
    pad_w: int

    @property
    def oH(self) -> int:
        return (self.H + 2 * self.pad_h - self.kH) // self.stride + 1

    @property
    def oW(self) -> int:
        return (self.W + 2 * self.pad_w - self.kW) // self.stride + 1

    @property
    def grad_out_shape(self):
        return (self.N, self.Co, self.oH, self.oW)

    @property
    def weight_shape(self):
        return (self.Co, self.Ci, self.kH, self.kW)

    @property
    def dst_shape(self):
        return (self.N, self.Ci, self.H, self.W)

    @property
    def eff_flops(self) -> int:
        """2*N*Co*oH*oW*Ci*kH*kW: the effective work of one grad_input call."""
        return 2 * self.N * self.Co * self.oH * self.oW * self.Ci * self.kH * self.kW

    def algorithmic_bytes(self, in_bytes: int) -> int:
        """Compulsory traffic: grad_out and weight read once, fp32 dst written once."""
        n_g = self.N * self.Co * self.oH * self.oW
        n_w = self.Co * self.Ci * self.kH * self.kW
        n_d = self.N * self.Ci * self.H * self.W
        return in_bytes * (n_g + n_w) + 4 * n_d

    def as_tuple(self):
        return (self.N, self.Ci, self.H, self.W, self.Co, self.kH, self.kW,
                self.stride, self.pad_h, self.pad_w, self.oH, self.oW)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int      # c in the seed formula
    sub: int        # sub in the seed formula
    shape: Shape
    dtype: str      # "f32", "bf16" or "f16" (inputs); dst is always fp32
    dist: str       # "uniform" (both U[-1,1]) or "kaiming" (g ~ N(0,1), w ~ N(0, 2/fan_in))


# The named workloads.  Weight variance 2/(Ci*kH*kW) is the Kaiming-normal
# fan-in variance of a [Co,Ci,kH,kW] kernel.
WORKLOADS = [
    Workload("tiny", 0, 0, Shape(1, 8, 16, 16, 16, 3, 3, 1, 1, 1), "f32", "uniform"),
    Workload("resnet_stage_3x3", 1, 0, Shape(32, 64, 56, 56, 64, 3, 3, 1, 1, 1), "f32", "kaiming"),
    Workload("strided_downsample", 2, 0, Shape(32, 128, 56, 56, 256, 3, 3, 2, 1, 1), "f32", "kaiming"),
    Workload("stem_7x7_s2", 3, 0, Shape(16, 3, 224, 224, 64, 7, 7, 2, 3, 3), "f32", "kaiming"),
    Workload("asym_1x7", 3, 1, Shape(32, 192, 17, 17, 192, 1, 7, 1, 0, 3), "f32", "kaiming"),
    Workload("deep_late_stage", 4, 0, Shape(64, 512, 14, 14, 512, 3, 3, 1, 1, 1), "f32", "kaiming"),
    Workload("deep_late_stage_bf16", 4, 0, Shape(64, 512, 14, 14, 512, 3, 3, 1, 1, 1), "bf16", "kaiming"),
    Workload("deep_late_stage_f16", 4, 0, Shape(64, 512, 14, 14, 512, 3, 3, 1, 1, 1), "f16", "kaiming"),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def seed_of(index: int, sub: int, tensor: int) -> int:
    return 1000 * index + 10 * sub + tensor


def draw(shape_tuple, seed: int, dist: str, std: float = 1.0) -> np.ndarray:
    """float32 array of the given shape: U[-1,1] or N(0, std^2), drawn in float64."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if dist == "uniform":
        a = rng.uniform(-1.0, 1.0, size=shape_tuple)
    elif dist == "normal":
        a = rng.standard_normal(size=shape_tuple) * std
    else:
        raise ValueError(dist)
    return a.astype(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even) and return the uint16 bit patterns.

    Inputs here are finite, so no NaN handling is needed."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def f16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE binary16 (nearest, ties to even; numpy's cast) and
    return the uint16 bit patterns."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen binary16 bit patterns to float32 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_inputs(w: Workload):
    """(grad_out, weight) for a named workload.

    f32: two float32 arrays.  bf16 / f16: two uint16 arrays of bf16 / binary16
    bit patterns (the float32 draws of the same seeds, rounded)."""
    s = w.shape
    if w.dist == "uniform":
        g = draw(s.grad_out_shape, seed_of(w.index, w.sub, 1), "uniform")
        wt = draw(s.weight_shape, seed_of(w.index, w.sub, 2), "uniform")
    else:
        fan_in = s.Ci * s.kH * s.kW
        g = draw(s.grad_out_shape, seed_of(w.index, w.sub, 1), "normal", 1.0)
        wt = draw(s.weight_shape, seed_of(w.index, w.sub, 2), "normal", math.sqrt(2.0 / fan_in))
    if w.dtype == "bf16":
        return bf16_bits(g), bf16_bits(wt)
    if w.dtype == "f16":
        return f16_bits(g), f16_bits(wt)
    return g, wt


def make_forward_input(w: Workload) -> np.ndarray:
    """The forward input x [N, Ci, H, W] of a named workload, float32 N(0,1)
    (grad_weight's second operand)."""
    return draw(w.shape.dst_shape, seed_of(w.index, w.sub, 3), "normal", 1.0)


def make_case(shape: Shape, seed: int, dist: str = "uniform"):
    """(grad_out, weight) float32 for an arbitrary shape (parity sweeps)."""
    g = draw(shape.grad_out_shape, seed * 2 + 1, dist)
    wt = draw(shape.weight_shape, seed * 2 + 2, dist)
    return g, wt


def sweep_shapes():
    """Small shapes that together cover the method's corner cases: ragged channel
    counts, N=1, Ci=1, Co=1, 1x1 kernels, kH != kW, strides 1-4, kernels smaller
    than the stride (phases with no taps), pads that are not "same", pad_h != pad_w,
    H != W, and inputs whose size leaves a remainder under the stride."""
    S = Shape
    return [
        S(1, 1, 1, 1, 1, 1, 1, 1, 0, 0),
        S(1, 1, 5, 5, 1, 3, 3, 1, 1, 1),
        S(2, 3, 7, 9, 5, 3, 3, 1, 0, 0),       # pad 0 (not "same")
        S(1, 5, 8, 8, 3, 2, 2, 1, 0, 0),       # even kernel
        S(2, 7, 6, 11, 9, 3, 5, 1, 2, 1),      # kH != kW, pad > (k-1)/2 on one side
        S(1, 4, 9, 9, 6, 3, 3, 2, 1, 1),       # stride 2, odd H
        S(2, 6, 10, 10, 5, 3, 3, 2, 1, 1),     # stride 2, even H (output_padding 1)
        S(1, 3, 13, 12, 4, 7, 7, 2, 3, 3),     # stem-like
        S(1, 5, 11, 10, 7, 3, 3, 3, 1, 0),     # stride 3
        S(1, 2, 9, 9, 3, 2, 2, 3, 0, 0),       # kernel < stride: phases with no taps
        S(1, 3, 8, 8, 2, 1, 1, 2, 0, 0),       # 1x1 stride 2: three phases are all zero
        S(3, 33, 5, 7, 17, 1, 7, 1, 0, 3),     # asymmetric 1x7
        S(1, 65, 6, 6, 70, 3, 3, 1, 1, 1),     # channels just past a tile edge
        S(2, 40, 12, 12, 48, 1, 1, 1, 0, 0),   # 1x1 (a plain matmul)
        S(1, 3, 16, 16, 64, 7, 7, 2, 3, 3),    # Ci = 3
        S(2, 130, 7, 7, 66, 3, 3, 1, 1, 1),    # Ci past two tiles
        S(1, 9, 17, 15, 11, 5, 3, 4, 2, 1),    # stride 4
        S(1, 8, 4, 4, 8, 5, 5, 1, 4, 4),       # pad > kernel-1: taps land in padding
        S(1, 16, 3, 3, 32, 3, 3, 1, 0, 0),     # oH = 1
    ]


def random_shapes(seed: int, count: int, co_range=(1, 48)):
    """`count` seeded random small shapes for sweeps: strides 1-4, kernels
    1-7 per dimension (kH != kW allowed), pads 0..k per dimension, ragged
    channel counts (a third of them Ci <= 4, a third Ci >= 16; Co drawn from
    co_range, both ends included), H and W 1-24; every shape has oH, oW >= 1."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    while len(out) < count:
        kH, kW = int(rng.integers(1, 8)), int(rng.integers(1, 8))
        s = int(rng.integers(1, 5))
        ph, pw = int(rng.integers(0, kH + 1)), int(rng.integers(0, kW + 1))
        H, W = int(rng.integers(1, 25)), int(rng.integers(1, 25))
        if (H + 2 * ph - kH) // s + 1 < 1 or (W + 2 * pw - kW) // s + 1 < 1:
            continue
        kind = len(out) % 3
        Ci = int(rng.integers(1, 5)) if kind == 0 else (
            int(rng.integers(16, 81)) if kind == 1 else int(rng.integers(5, 16)))
        out.append(Shape(int(rng.integers(1, 4)), Ci, H, W,
                         int(rng.integers(co_range[0], co_range[1] + 1)), kH, kW, s,
                         ph, pw))
    return out
