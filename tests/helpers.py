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
        if shape.dtype == "mxfp8":
            self.x_f32 = w.x()
            self.w1_f32 = w.w1()
            self.w2_f32 = w.w2()
            self.x, self.x_scale = orc.mx_quantize(self.x_f32)
            self.w1, self.w1_scale = orc.mx_quantize(self.w1_f32)
            self.w2, self.w2_scale = orc.mx_quantize(self.w2_f32)
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
        if f == "mxfp8":
            d["x_scale"] = to_dev(self.x_scale, "u8")
            d["w1_scale"] = to_dev(self.w1_scale, "u8")
            d["w2_scale"] = to_dev(self.w2_scale, "u8")
        if self.dy is not None:
            d["dy"] = to_dev(self.dy, self.s.out_dtype)
        return d


def cfg_of(shape):
    from routing_permute_grouped_router_amd import MoEConfig
    return MoEConfig.from_shape(shape)


def run_forward(inp: Inputs, training: bool = False, poison: bool = True) -> dict:
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
                    w1_scale=d.get("w1_scale"), w2_scale=d.get("w2_scale"))
    torch.cuda.synchronize()
    return buf
