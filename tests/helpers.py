"""Shared helpers of the parity tests: moving seeded workload arrays to the GPU,
running the HIP path through the C ABI, and comparing against the oracle."""
from __future__ import annotations

import functools

import numpy as np
import torch

from oracle import oracle as orc
from routing_permute_grouped_router_amd import workload as wl

TOL = {"f32": 1e-5, "bf16": 2e-2, "mxfp8": 6e-2}


def rel_err(a, b) -> float:
    """Normwise relative error max|a-b| / max|b| (b the oracle)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = float(np.max(np.abs(b))) if b.size else 0.0
    num = float(np.max(np.abs(a - b))) if a.size else 0.0
    if den == 0.0:
        return num
    return num / den


# Per-element bounds |a - b| <= rtol |b| + atol max|b| (b the oracle), next to
# the normwise bar.  rtol is one step of the storage format at |b| (bf16 keeps
# 8 significant bits: a step is at most 2^-7 |b|; E4M3 keeps 4: 2^-3 |b|),
# which is what two roundings of values that differ by less than a step can
# give; atol covers elements near 0, where the float32 accumulation error of
# the kernel (relative to the row's magnitude, not the element's) decides.
#   f32acc: float32 outputs of a float32 sum over bf16 operands (the weight
#   gradients): sqrt(n) 2^-24 accumulation error plus bf16 flips in the
#   operands, diluted by the sum, stay far below 2^-10 |b| + 2^-12 max|b|.
#   e4m3_out: bf16 outputs of a product over a requantised MXFP8 h.  Where the
#   kernel's float32 and the oracle's float64 put an h value on opposite sides
#   of an E4M3 rounding boundary, that term of the sum moves by one step,
#   2^-3 of the value; over a sum of F terms of random sign that is about
#   2^-3 / sqrt(F) of the result, 2^-6.5 for the smallest F here (128).
#   e2m1_out: bf16 outputs of a product over a requantised MXFP4 h.  One E2M1
#   step is up to 2^-1 of the value; in one term of a sum of F >= 512 terms of
#   random sign that is about 2^-1 / sqrt(512) = 2^-5.5 of the result.
ELEM_BOUNDS = {"f32": (2.0 ** -16, 2.0 ** -17), "bf16": (2.0 ** -7, 2.0 ** -9),
               "e4m3": (2.0 ** -3, 2.0 ** -9), "e4m3_out": (2.0 ** -5, 2.0 ** -8),
               "e2m1_out": (2.0 ** -4, 2.0 ** -7), "f32acc": (2.0 ** -10, 2.0 ** -12)}
# normwise bars max|a-b| / max|b| of the same kinds (1e-5 fp32, 2e-2 bf16,
# 6e-2 for the MX formats; float32 weight gradients over bf16 operands take
# the bf16 bar)
NORM_TOL = {"f32": 1e-5, "bf16": 2e-2, "e4m3": 6e-2, "e4m3_out": 6e-2, "e2m1_out": 6e-2, "f32acc": 2e-2}
ELEM_FRAC = 0.999  # share of elements that must meet the per-element bound


def elem_stats(a, b, kind: str) -> dict:
    """Share of elements within the per-element bound of `kind`, and the worst
    element (the largest |a-b| / (rtol |b| + atol max|b|))."""
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    rtol, atol = ELEM_BOUNDS[kind]
    if b.size == 0:
        return {"frac": 1.0, "worst": 0.0, "at": -1, "a": 0.0, "b": 0.0, "n": 0}
    lim = rtol * np.abs(b) + atol * float(np.max(np.abs(b)))
    lim = np.where(lim > 0, lim, np.finfo(np.float64).tiny)
    r = np.abs(a - b) / lim
    r = np.where(np.isnan(r), np.inf, r)
    i = int(np.argmax(r))
    return {"frac": float(np.mean(r <= 1.0)), "worst": float(r[i]), "at": i, "a": float(a[i]), "b": float(b[i]),
            "n": int(b.size)}


def close_elementwise(a, b, kind: str, label: str = "", frac: float = ELEM_FRAC) -> bool:
    """At least `frac` of the elements meet the per-element bound of `kind`;
    prints the share and the worst element either way."""
    st = elem_stats(a, b, kind)
    print(f"{label}: {st['frac'] * 100:.4f} % of {st['n']} elements within the {kind} bound; worst "
          f"element {st['at']}: got {st['a']:.6g}, oracle {st['b']:.6g} ({st['worst']:.3g} x the bound)")
    return st["frac"] >= frac


def assert_parity(got, ref, kind: str, label: str = "") -> None:
    """The normwise bar of `kind` and, next to it, the per-element bound."""
    e = rel_err(got, ref)
    assert e < NORM_TOL[kind], f"{label}: normwise relative error {e:.3g} >= {NORM_TOL[kind]}"
    assert close_elementwise(got, ref, kind, label), f"{label}: fewer than {ELEM_FRAC:.1%} of elements in bound"


def to_dev(a: np.ndarray, fmt: str, device="cuda") -> torch.Tensor:
    """Stored numpy array -> torch tensor of the same bytes on the GPU."""
    if fmt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    if fmt == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """GPU tensor -> numpy array of the same bytes (bf16 as uint16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def decode(fmt: str, a, scale=None) -> np.ndarray:
    return orc.decode(fmt, a, scale)


class Inputs:
    """Seeded inputs of one shape in storage form, host and device."""

    def __init__(self, shape: wl.MoEShape, device="cuda", want_dy: bool = False):
        self.s = shape
        w = wl.Workload(shape)
        self.logits = w.logits()
        if shape.dtype in ("mxfp8", "mxfp4"):
            self.x_f32 = w.x()
            self.w1_f32 = w.w1()
            self.w2_f32 = w.w2()
            self.x, self.x_scale = orc.mx_quantize(self.x_f32, shape.dtype)
            self.w1, self.w1_scale = orc.mx_quantize(self.w1_f32, shape.dtype)
            self.w2, self.w2_scale = orc.mx_quantize(self.w2_f32, shape.dtype)
        else:
            self.x = w.x()
            self.w1 = w.w1()
            self.w2 = w.w2()
            self.x_scale = self.w1_scale = self.w2_scale = None
        self.dy = w.dy() if want_dy else None
        self.device = device

    @functools.cached_property
    def dev(self) -> dict:
        f = self.s.dtype
        d = {"logits": to_dev(self.logits, "f32"), "x": to_dev(self.x, f), "w1": to_dev(self.w1, f),
             "w2": to_dev(self.w2, f)}
        if f in ("mxfp8", "mxfp4"):
            d["x_scale"] = to_dev(self.x_scale, "u8")
            d["w1_scale"] = to_dev(self.w1_scale, "u8")
            d["w2_scale"] = to_dev(self.w2_scale, "u8")
        if self.dy is not None:
            d["dy"] = to_dev(self.dy, self.s.out_dtype)
        return d


def cfg_of(shape):
    from routing_permute_grouped_router_amd import MoEConfig
    return MoEConfig.from_shape(shape)


def run_forward(inp: Inputs, training: bool = False, poison: bool = True, bias=None) -> dict:
    """bias: optional float32 [E] host array, the router's selection bias."""
    import routing_permute_grouped_router_amd as moe
    cfg = cfg_of(inp.s)
    buf = moe.alloc_forward(cfg, training=training)
    if poison:  # every float buffer starts as NaN so unwritten reads show up
        for k in ("xp", "h", "yp", "y", "gu_stash"):
            if k in buf and buf[k].dtype.is_floating_point:
                buf[k].fill_(float("nan"))
        for k in ("src_map", "row_map", "idx"):
            buf[k].fill_(-7)
    d = inp.dev
    moe.moe_forward(cfg, d["logits"], d["x"], d["w1"], d["w2"], buf, x_scale=d.get("x_scale"),
                    w1_scale=d.get("w1_scale"), w2_scale=d.get("w2_scale"),
                    bias=None if bias is None else to_dev(np.asarray(bias, np.float32), "f32"))
    torch.cuda.synchronize()
    return buf
