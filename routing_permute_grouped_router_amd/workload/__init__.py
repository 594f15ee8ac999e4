"""Seeded synthetic workloads for the MoE FFN hot path.

This module draws inputs only; it holds no step of the routing / permutation /
expert FFN / combine method.  Both the HIP path (tests, benchmark) and the CPU
oracle's tests take their inputs from here.

Workloads (T tokens, hidden H, per-expert FFN width F, E experts, top-k):

  tiny_f32        T=256   H=128  F=256   E=8   k=2  softmax            fp32
  mixtral_bf16    T=8192  H=4096 F=14336 E=8   k=2  softmax            bf16
  finegrained_bf16 T=16384 H=2048 F=768  E=128 k=8  softmax, renorm    bf16
  skewed_bf16     as finegrained, plus a Zipf(1.2) per-expert logit bias;
                  forward and backward                                  bf16
  deepseek_mxfp8  T=8192  H=7168 F=2048  E=256 k=8  sigmoid, normalised
                  MXFP8 E4M3 (block-32 E8M0 scales) inputs, bf16 output

and, for the narrower MX format, deepseek_mxfp4: the DeepSeek-shaped layer
with MXFP4 storage (E2M1 elements packed two per byte, the same scales).

Value recipe: x ~ N(0, 1); router weight W_r (H x E) ~ N(0, 0.02); gate/up
weights ~ N(0, H^-1/2); down weights ~ N(0, F^-1/2) (N(0, H^-1/2) for the tiny
workload); output gradient dY ~ N(0, 1).  The second argument is the standard
deviation.  Values are drawn in float64 by a counter-based generator
(Philox4x32-10 + Box-Muller, see workload_gen.c) and stored in the workload's
format: float32, or bfloat16 rounded from the float32 value.  MXFP8 workloads
and MXFP4 workloads hand out float32 values, which each side quantises itself.

Router logits = float32( x @ W_r (+ bias) ) computed in float64 on the host from
the stored x (unquantised float32 x for MXFP8): the router GEMM sits outside the
routed path, whose first step consumes float32 logits.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libworkload.so")
SRC_PATH = os.path.join(_HERE, "workload_gen.c")

# tensor ids of the generator streams
TID_X, TID_WR, TID_GATE, TID_UP, TID_DOWN, TID_DY = 0, 1, 2, 3, 4, 5
_KIND = {"f32": 0, "bf16": 1, "f64": 2}
_NP = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}


def build(verbose: bool = False) -> str:
    """Compile the generator with gcc (OpenMP) next to its source."""
    import subprocess

    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", LIB_PATH, SRC_PATH, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        lib.wl_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int64,
                                  ctypes.c_double, ctypes.c_int, ctypes.c_void_p]
        lib.wl_normal.restype = None
        lib.wl_philox4x32_10.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.wl_philox4x32_10.restype = None
        lib.wl_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def philox4x32_10(ctr, key) -> list:
    """Raw Philox4x32-10 block (used by the generator's known-answer test)."""
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    o = (ctypes.c_uint32 * 4)()
    _load().wl_philox4x32_10(c, k, o)
    return list(o)


def normal(seed: int, tensor: int, start: int, n: int, std: float, kind: str = "f32") -> np.ndarray:
    """Elements [start, start+n) of a tensor's N(0, std) stream."""
    out = np.empty(n, dtype=_NP[kind])
    if n:
        _load().wl_normal(seed, tensor, start, n, std, _KIND[kind], out.ctypes.data)
    return out


@dataclasses.dataclass(frozen=True)
class MoEShape:
    name: str
    T: int
    H: int
    F: int
    E: int
    k: int
    score: str = "softmax"        # "softmax" | "sigmoid"
    renorm: bool = False          # normalise the selected weights over k
    dtype: str = "bf16"           # storage of x / weights: "f32" | "bf16" | "mxfp8" | "mxfp4"
    zipf_bias: Optional[float] = None  # Zipf exponent of the per-expert logit bias
    backward: bool = False
    down_std_from_h: bool = False  # down weights ~ N(0, H^-1/2) instead of F^-1/2
    align: int = 1
    seed: int = 0

    @property
    def out_dtype(self) -> str:
        return "f32" if self.dtype == "f32" else "bf16"

    @property
    def R(self) -> int:
        return self.T * self.k

    @property
    def R_cap(self) -> int:
        return self.T * self.k + self.E * (self.align - 1)

    def replace(self, **kw) -> "MoEShape":
        return dataclasses.replace(self, **kw)


# The five workloads; seed = 1000 + position.
WORKLOADS = [
    MoEShape("tiny_f32", 256, 128, 256, 8, 2, "softmax", False, "f32", down_std_from_h=True, seed=1000),
    MoEShape("mixtral_bf16", 8192, 4096, 14336, 8, 2, "softmax", False, "bf16", seed=1001),
    MoEShape("finegrained_bf16", 16384, 2048, 768, 128, 8, "softmax", True, "bf16", seed=1002),
    MoEShape("skewed_bf16", 16384, 2048, 768, 128, 8, "softmax", True, "bf16", zipf_bias=1.2,
             backward=True, seed=1003),
    MoEShape("deepseek_mxfp8", 8192, 7168, 2048, 256, 8, "sigmoid", True, "mxfp8", seed=1004),
]
# The DeepSeek-shaped layer on MXFP4 storage (the MX analogue of the NVFP4
# recipe of the pages; not one of the five).
EXTRA_WORKLOADS = [
    MoEShape("deepseek_mxfp4", 8192, 7168, 2048, 256, 8, "sigmoid", True, "mxfp4", seed=1005),
]
BY_NAME = {w.name: w for w in WORKLOADS + EXTRA_WORKLOADS}


def zipf_bias(E: int, s: float) -> np.ndarray:
    """b_e = 2 ln(w_r), w_r = r^-s / sum_{j=1..E} j^-s, rank r = e + 1 (float64)."""
    r = np.arange(1, E + 1, dtype=np.float64)
    wr = r ** (-s) / np.sum(r ** (-s))
    return 2.0 * np.log(wr)


class Workload:
    """Deterministic inputs of one MoE shape.  Arrays are numpy, in storage
    form: float32, bfloat16 as uint16 bit patterns, or (MXFP8 shapes) the
    float32 values before quantisation."""

    def __init__(self, shape: MoEShape):
        self.s = shape

    # element stores
    @property
    def gen_kind(self) -> str:
        return "bf16" if self.s.dtype == "bf16" else "f32"

    def x(self, t0: int = 0, t1: Optional[int] = None) -> np.ndarray:
        s = self.s
        t1 = s.T if t1 is None else t1
        return normal(s.seed, TID_X, t0 * s.H, (t1 - t0) * s.H, 1.0, self.gen_kind).reshape(t1 - t0, s.H)

    def x_f64(self) -> np.ndarray:
        x = self.x()
        if self.gen_kind == "bf16":
            return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return x.astype(np.float64)

    def router_weight(self) -> np.ndarray:
        s = self.s
        return normal(s.seed, TID_WR, 0, s.H * s.E, 0.02, "f64").reshape(s.H, s.E)

    def logits(self) -> np.ndarray:
        s = self.s
        lg = self.x_f64() @ self.router_weight()
        if s.zipf_bias is not None:
            lg = lg + zipf_bias(s.E, s.zipf_bias)[None, :]
        return lg.astype(np.float32)

    def _std_gate(self) -> float:
        return self.s.H ** -0.5

    def _std_down(self) -> float:
        return self.s.H ** -0.5 if self.s.down_std_from_h else self.s.F ** -0.5

    def w1(self, e0: int = 0, e1: Optional[int] = None) -> np.ndarray:
        """Stored gate/up weights of experts [e0, e1): [n_e, 2F, H]; rows
        [0, F) are the gate columns and [F, 2F) the up columns of the logical
        fc1 (E, H, 2F)."""
        s = self.s
        e1 = s.E if e1 is None else e1
        ne = e1 - e0
        n = ne * s.F * s.H
        g = normal(s.seed, TID_GATE, e0 * s.F * s.H, n, self._std_gate(), self.gen_kind).reshape(ne, s.F, s.H)
        u = normal(s.seed, TID_UP, e0 * s.F * s.H, n, self._std_gate(), self.gen_kind).reshape(ne, s.F, s.H)
        return np.concatenate([g, u], axis=1)

    def w2(self, e0: int = 0, e1: Optional[int] = None) -> np.ndarray:
        """Stored down weights of experts [e0, e1): [n_e, H, F] (the logical
        fc2 (E, F, H) with the contraction dim F contiguous)."""
        s = self.s
        e1 = s.E if e1 is None else e1
        ne = e1 - e0
        return normal(s.seed, TID_DOWN, e0 * s.H * s.F, ne * s.H * s.F, self._std_down(),
                      self.gen_kind).reshape(ne, s.H, s.F)

    def dy(self) -> np.ndarray:
        s = self.s
        kind = "f32" if s.dtype == "f32" else "bf16"
        return normal(s.seed, TID_DY, 0, s.T * s.H, 1.0, kind).reshape(s.T, s.H)


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def mxfp4_shapes() -> list:
    """MXFP4 parity shapes (H and F multiples of 512): several GEMM tiles,
    ragged group tails, skewed routing with empty experts and 16-row groups,
    a plain-softmax top-2 shape with the down GEMM's K = 1024, and 128-row
    groups (most rows of Xp, h and Yp are padding)."""
    return [
        MoEShape("small_mxfp4", 260, 512, 512, 16, 4, "sigmoid", True, "mxfp4", seed=2020),
        MoEShape("small_mxfp4_skew_align", 300, 1024, 512, 16, 4, "softmax", True, "mxfp4", align=16,
                 zipf_bias=1.2, seed=2021),
        MoEShape("small_mxfp4_k1024", 517, 512, 1024, 8, 2, "softmax", False, "mxfp4", seed=2022),
        MoEShape("small_mxfp4_align128", 260, 512, 512, 8, 2, "sigmoid", True, "mxfp4", align=128, seed=2023),
    ]


def small_shapes() -> list:
    """Shapes the oracle finishes in seconds that still span several GEMM tiles
    and ragged group tails (used by the parity tests)."""
    return [
        WORKLOADS[0],
        MoEShape("small_bf16_softmax", 300, 256, 192, 8, 2, "softmax", False, "bf16", seed=2001),
        MoEShape("small_bf16_renorm", 517, 256, 128, 16, 4, "softmax", True, "bf16", seed=2002),
        MoEShape("small_bf16_sigmoid_align", 333, 128, 128, 12, 3, "sigmoid", True, "bf16", align=16, seed=2003),
        MoEShape("small_skewed_bf16", 512, 256, 128, 16, 4, "softmax", True, "bf16", zipf_bias=1.2,
                 backward=True, seed=2004),
        MoEShape("small_mxfp8", 260, 256, 128, 16, 4, "sigmoid", True, "mxfp8", seed=2005),
        # K = 512 in both GEMMs: the scale words of four stages per load
        MoEShape("small_mxfp8_k512", 300, 512, 512, 8, 2, "sigmoid", True, "mxfp8", seed=2006),
        # skewed routing (empty experts) and 16-row groups (zero padding rows)
        MoEShape("small_mxfp8_skew_align", 300, 512, 256, 16, 4, "softmax", True, "mxfp8", align=16,
                 zipf_bias=1.2, seed=2007),
        # 128-row groups (the alignment of the TransformerEngine layout): most
        # rows of Xp, h and Yp are padding
        MoEShape("small_bf16_align128", 300, 256, 128, 8, 2, "softmax", True, "bf16", align=128, seed=2008),
        MoEShape("small_mxfp8_align128", 260, 256, 128, 8, 2, "sigmoid", True, "mxfp8", align=128, seed=2009),
    ]
