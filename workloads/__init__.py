"""Seeded synthetic inputs and the workload shape table.

This module is shared by the tests, the benchmark and the smoke check.  It
holds shapes, seeds and value distributions only -- none of the convolution's
arithmetic -- so that the oracle and the HIP path can both be fed the same
inputs without sharing any code.

Random draws use numpy's PCG64 generator, in float32.  bf16 inputs are the
float32 draws rounded to nearest-even (torch's float32 -> bfloat16
conversion); both sides of a comparison are fed the rounded values.
"""
from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import numpy as np
import torch


@dataclass(frozen=True)
class Dist:
    """A value distribution: kind in {uniform, normal, relu_normal, int}."""
    kind: str
    a: float = 0.0   # uniform low / normal std / int low
    b: float = 0.0   # uniform high / int high


def draw(shape, dist: Dist, seed: int) -> torch.Tensor:
    """float32 CPU tensor of ``shape`` drawn from ``dist`` with PCG64(seed)."""
    g = np.random.Generator(np.random.PCG64(seed))
    shape = tuple(int(s) for s in shape)
    if dist.kind == "uniform":
        v = g.uniform(dist.a, dist.b, size=shape).astype(np.float32)
    elif dist.kind == "normal":
        v = (g.standard_normal(size=shape, dtype=np.float32) * np.float32(dist.a)).astype(np.float32)
    elif dist.kind == "relu_normal":
        v = g.standard_normal(size=shape, dtype=np.float32)
        v = np.maximum(v, np.float32(0.0))  # max(0, z): negatives become +0.0
    elif dist.kind == "int":
        v = g.integers(int(dist.a), int(dist.b) + 1, size=shape).astype(np.float32)
    else:
        raise ValueError(dist.kind)
    return torch.from_numpy(np.ascontiguousarray(v))


def as_dtype(t: torch.Tensor, dtype: str) -> torch.Tensor:
    """Cast a float32 tensor to the named input dtype ('f32' or 'bf16', RNE)."""
    if dtype == "f32":
        return t.to(torch.float32)
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    raise ValueError(dtype)


@dataclass(frozen=True)
class ConvShape:
    """Convolution sizes in the pages' notation; P, Q are stated, not derived."""
    N: int
    C: int
    H: int
    W: int
    K: int
    R: int
    S: int
    pad: Tuple[int, int]
    stride: Tuple[int, int]
    P: int
    Q: int

    @property
    def x_shape(self):
        return (self.N, self.C, self.H, self.W)

    @property
    def w_shape(self):
        return (self.K, self.C, self.R, self.S)

    @property
    def y_shape(self):
        return (self.N, self.K, self.P, self.Q)

    def args13(self):
        return (self.N, self.C, self.H, self.W, self.K, self.R, self.S,
                self.pad[0], self.pad[1], self.stride[0], self.stride[1], self.P, self.Q)

    def flops(self) -> int:
        """2*N*K*P*Q*C*R*S, the per-pass count the metric uses."""
        return 2 * self.N * self.K * self.P * self.Q * self.C * self.R * self.S


@dataclass(frozen=True)
class Workload:
    name: str
    shape: ConvShape            # for deconv: the convolution view (K = C_in, C = C_out)
    dtypes: Tuple[str, ...]
    passes: Tuple[str, ...]
    x: Dist
    w: Dist
    dy: Optional[Dist]
    seeds: Tuple[int, int, int]
    deconv: bool = False
    note: str = ""


def _he(fan_in):
    return float(np.sqrt(2.0 / fan_in))


ALL3 = ("fwd", "bwd_data", "bwd_filter")
DECONV3 = ("deconv_fwd", "deconv_bwd_data", "deconv_bwd_filter")

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(
        "tiny", ConvShape(2, 3, 8, 8, 4, 3, 3, (1, 1), (1, 1), 8, 8), ("f32",), ALL3,
        Dist("uniform", -1.0, 1.0), Dist("uniform", -1.0, 1.0), Dist("uniform", -1.0, 1.0),
        (101, 102, 103), note="tiny conv2d, uniform[-1,1]"),
    "resnet3x3": Workload(
        "resnet3x3", ConvShape(64, 64, 56, 56, 64, 3, 3, (1, 1), (1, 1), 56, 56), ("f32", "bf16"),
        ALL3, Dist("relu_normal"), Dist("normal", _he(64 * 9)), Dist("normal", 0.01),
        (201, 202, 203), note="ResNet-style 3x3 layer, x = ReLU(N(0,1))"),
    "proj1x1": Workload(
        "proj1x1", ConvShape(64, 256, 56, 56, 512, 1, 1, (0, 0), (2, 2), 28, 28), ("f32", "bf16"),
        ALL3, Dist("normal", 1.0), Dist("normal", _he(256)), Dist("normal", 0.01),
        (311, 312, 313), note="1x1 stride-2 projection (bf16 run is an extra)"),
    "stem7x7": Workload(
        "stem7x7", ConvShape(32, 3, 224, 224, 64, 7, 7, (3, 3), (2, 2), 112, 112), ("f32",),
        ALL3, Dist("normal", 1.0), Dist("normal", _he(3 * 49)), Dist("normal", 0.01),
        (321, 322, 323), note="7x7 stride-2 stem"),
    # Deconvolution: input (32, 256, 16, 16), weights (in=256, out=128, 4, 4), stride 2,
    # pad 1, output (32, 128, 32, 32).  Convolution view: K = 256 (deconv in), C = 128
    # (deconv out), H = W = 32 (deconv output), P = Q = 16 (deconv input).
    "deconv4x4": Workload(
        "deconv4x4", ConvShape(32, 128, 32, 32, 256, 4, 4, (1, 1), (2, 2), 16, 16), ("f32", "bf16"),
        DECONV3, Dist("uniform", -1.0, 1.0), Dist("normal", float(np.sqrt(1.0 / (256 * 16)))),
        Dist("normal", 0.01), (401, 402, 403), deconv=True,
        note="transposed conv via backward-data; its backward passes via forward / backward-filter"),
    "deep3x3": Workload(
        "deep3x3", ConvShape(256, 512, 14, 14, 512, 3, 3, (1, 1), (1, 1), 14, 14), ("bf16",),
        ALL3, Dist("relu_normal"), Dist("normal", _he(512 * 9)), Dist("normal", 0.01),
        (501, 502, 503), note="large-batch deep 3x3 layer"),
}


def inputs(wl: Workload, dtype: str, shape: Optional[ConvShape] = None, integer: bool = False,
           seed_offset: int = 0):
    """Seeded inputs for a workload (optionally at a reduced ``shape``).

    Returns a dict of CPU tensors in the requested dtype:
      conv:   {'x': [N,C,H,W], 'w': [K,C,R,S], 'dy': [N,K,P,Q]}
      deconv: {'x_in': [N,K,P,Q], 'w': [K,C,R,S], 'dout': [N,C,H,W]}   (K = C_in, C = C_out;
              dout is the gradient of the deconvolution output)
    ``integer=True`` replaces every distribution by small integers in [-4, 4],
    which are exact in bf16 and keep every partial sum exact in fp32.
    """
    sh = shape or wl.shape
    sx, sw, sdy = (s + seed_offset for s in wl.seeds)
    ints = Dist("int", -4, 4)
    if wl.deconv:
        xin = draw(sh.y_shape, ints if integer else wl.x, sx)
        w = draw(sh.w_shape, ints if integer else wl.w, sw)
        dout = draw(sh.x_shape, ints if integer else wl.dy, sdy)
        return {"x_in": as_dtype(xin, dtype), "w": as_dtype(w, dtype), "dout": as_dtype(dout, dtype)}
    x = draw(sh.x_shape, ints if integer else wl.x, sx)
    w = draw(sh.w_shape, ints if integer else wl.w, sw)
    dy = draw(sh.y_shape, ints if integer else wl.dy, sdy)
    return {"x": as_dtype(x, dtype), "w": as_dtype(w, dtype), "dy": as_dtype(dy, dtype)}
