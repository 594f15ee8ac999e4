"""ctypes binding of libmoe.so (the C ABI in include/moe.h).

Argument marshalling only: every function here checks the torch tensors it is
handed (device, dtype, shape, contiguity), passes their device pointers and the
current HIP stream to the C entry point of the same name, and turns a failing
status into a Python exception.  All computation happens in the HIP kernels.
torch supplies device memory and streams.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_MXFP8, MOE_MXFP4 = 0, 1, 2, 3
MOE_SOFTMAX, MOE_SIGMOID = 0, 1
DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "mxfp8": MOE_MXFP8, "mxfp4": MOE_MXFP4}
MOE_WEIGHT_AT_COMBINE, MOE_WEIGHT_AT_FC1, MOE_WEIGHT_AT_FC2 = 0, 1, 2
WEIGHT_SITES = {"combine": MOE_WEIGHT_AT_COMBINE, "fc1": MOE_WEIGHT_AT_FC1, "fc2": MOE_WEIGHT_AT_FC2}
SCORES = {"softmax": MOE_SOFTMAX, "sigmoid": MOE_SIGMOID}


class MoEError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class MoEInvalidArgument(MoEError, ValueError):
    pass


class MoEUnsupported(MoEError, NotImplementedError):
    pass


class MoEWorkspaceError(MoEError, ValueError):
    pass


class MoEHipError(MoEError):
    pass


_EXC = {MOE_ERR_INVALID_ARG: MoEInvalidArgument, MOE_ERR_UNSUPPORTED: MoEUnsupported,
        MOE_ERR_WORKSPACE: MoEWorkspaceError, MOE_ERR_HIP: MoEHipError}


class moe_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32)
                for n in ("T", "H", "F", "E", "k", "align", "score", "renorm", "dtype", "weight_site")] + [
                    ("swiglu_limit", ctypes.c_float)]


@dataclass(frozen=True)
class MoEConfig:
    T: int
    H: int
    F: int
    E: int
    k: int
    align: int = 1
    score: str = "softmax"
    renorm: bool = False
    dtype: str = "bf16"
    weight_site: str = "combine"  # where moe_forward applies w: "combine", "fc1" or "fc2"
    swiglu_limit: float = 0.0     # SwiGLU clamp: h = silu(min(g, L)) clamp(u, -L, L); 0 = none

    @classmethod
    def from_shape(cls, s) -> "MoEConfig":
        return cls(s.T, s.H, s.F, s.E, s.k, s.align, s.score, bool(s.renorm), s.dtype)

    def c(self) -> moe_config:
        return moe_config(self.T, self.H, self.F, self.E, self.k, self.align, SCORES[self.score],
                          int(self.renorm), DTYPES[self.dtype], WEIGHT_SITES[self.weight_site],
                          float(self.swiglu_limit))

    @property
    def R_cap(self) -> int:
        return self.T * self.k + self.E * (self.align - 1)

    @property
    def store_dtype(self) -> torch.dtype:
        return {"f32": torch.float32, "bf16": torch.bfloat16, "mxfp8": torch.uint8, "mxfp4": torch.uint8}[self.dtype]

    @property
    def is_mx(self) -> bool:
        return self.dtype in ("mxfp8", "mxfp4")

    def cols(self, n: int) -> int:
        """Stored entries of a row of n elements (MXFP4 packs two per byte)."""
        return n // 2 if self.dtype == "mxfp4" else n

    @property
    def out_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


_lib = None
P = ctypes.c_void_p
CFG = ctypes.POINTER(moe_config)
_SIGS = {
    "moe_rows_capacity": (ctypes.c_int64, [CFG]),
    "moe_workspace_size": (ctypes.c_size_t, [CFG]),
    "moe_backward_workspace_size": (ctypes.c_size_t, [CFG]),
    "moe_route": (ctypes.c_int, [CFG, P, P, P, P, P]),
    "moe_permute": (ctypes.c_int, [CFG, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
    "moe_grouped_swiglu_gemm": (ctypes.c_int, [CFG, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
    "moe_grouped_down_gemm": (ctypes.c_int, [CFG, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
    "moe_combine": (ctypes.c_int, [CFG, P, P, P, P, P]),
    "moe_forward": (ctypes.c_int, [CFG] + [P] * 23 + [ctypes.c_size_t, P]),
    "moe_forward_noalloc": (ctypes.c_int, [CFG] + [P] * 22 + [P]),
    "moe_route_bwd": (ctypes.c_int, [CFG, P, P, P, P, P, P, P, P]),
    "moe_grouped_swiglu_gemm_gather": (ctypes.c_int, [CFG, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
    "moe_grouped_swiglu_gemm_weighted": (ctypes.c_int, [CFG, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
    "moe_grouped_down_gemm_weighted": (ctypes.c_int, [CFG, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
    "moe_combine_bwd": (ctypes.c_int, [CFG, P, P, P, P, P, P, P]),
    "moe_grouped_down_bwd": (ctypes.c_int, [CFG, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
    "moe_grouped_swiglu_bwd": (ctypes.c_int, [CFG, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
    "moe_permute_bwd": (ctypes.c_int, [CFG, P, P, P, P]),
    "moe_backward": (ctypes.c_int, [CFG] + [P] * 17 + [ctypes.c_size_t, P]),
    "moe_quantize_mxfp8": (ctypes.c_int, [P, ctypes.c_int64, ctypes.c_int64, P, P, P]),
    "moe_quantize_mxfp4": (ctypes.c_int, [P, ctypes.c_int64, ctypes.c_int64, P, P, P]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_version": (ctypes.c_char_p, []),
}
EXPORTED = tuple(_SIGS)


def load_library(path: Optional[str] = None):
    """Load libmoe.so (fails loudly when it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build the HIP library first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != MOE_OK:
        lib = load_library()
        msg = lib.moe_last_error().decode()
        raise _EXC.get(status, MoEError)(status, f"{lib.moe_status_string(status).decode()}: {msg}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t, name: str, dtype=None, shape=None, optional: bool = False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def rows_capacity(cfg: MoEConfig) -> int:
    c = cfg.c()
    return load_library().moe_rows_capacity(ctypes.byref(c))


def workspace_size(cfg: MoEConfig) -> int:
    c = cfg.c()
    return load_library().moe_workspace_size(ctypes.byref(c))


def backward_workspace_size(cfg: MoEConfig) -> int:
    c = cfg.c()
    return load_library().moe_backward_workspace_size(ctypes.byref(c))


def _ws(ws):
    if ws is None:
        return None, 0
    if not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous GPU tensor")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def _scale_dtype(cfg):
    return torch.uint8


def moe_route(cfg: MoEConfig, logits, idx, w, stream=None, bias=None):
    """bias (optional, float32 [E]): shifts only the selection key."""
    c = cfg.c()
    _check(load_library().moe_route(
        ctypes.byref(c), _ptr(logits, "logits", torch.float32, (cfg.T, cfg.E)),
        _ptr(bias, "bias", torch.float32, (cfg.E,), optional=True),
        _ptr(idx, "idx", torch.int32, (cfg.T, cfg.k)), _ptr(w, "w", torch.float32, (cfg.T, cfg.k)),
        _stream(stream)))


def moe_permute(cfg: MoEConfig, x, idx, xp, counts, offsets, row_map, src_map, ws, x_scale=None, xp_scale=None,
                err=None, stream=None):
    c = cfg.c()
    mx = cfg.is_mx
    wp, wb = _ws(ws)
    _check(load_library().moe_permute(
        ctypes.byref(c), _ptr(x, "x", cfg.store_dtype, (cfg.T, cfg.cols(cfg.H))),
        _ptr(x_scale, "x_scale", torch.uint8, (cfg.T, cfg.H // 32), optional=not mx),
        _ptr(idx, "idx", torch.int32, (cfg.T, cfg.k)),
        _ptr(xp, "xp", cfg.store_dtype, (cfg.R_cap, cfg.cols(cfg.H)), optional=True),
        _ptr(xp_scale, "xp_scale", torch.uint8, (cfg.R_cap, cfg.H // 32), optional=not mx or xp is None),
        _ptr(counts, "counts", torch.int32, (cfg.E,)), _ptr(offsets, "offsets", torch.int32, (cfg.E + 1,)),
        _ptr(row_map, "row_map", torch.int32, (cfg.T, cfg.k)), _ptr(src_map, "src_map", torch.int32, (cfg.R_cap,)),
        _ptr(err, "err", torch.int32, (1,), optional=True), wp, wb, _stream(stream)))


def moe_grouped_swiglu_gemm(cfg: MoEConfig, xp, w1, offsets, h, ws, xp_scale=None, w1_scale=None, h_scale=None,
                            gu_stash=None, stream=None):
    c = cfg.c()
    mx = cfg.is_mx
    wp, wb = _ws(ws)
    _check(load_library().moe_grouped_swiglu_gemm(
        ctypes.byref(c), _ptr(xp, "xp", cfg.store_dtype, (cfg.R_cap, cfg.cols(cfg.H))),
        _ptr(xp_scale, "xp_scale", torch.uint8, (cfg.R_cap, cfg.H // 32), optional=not mx),
        _ptr(w1, "w1", cfg.store_dtype, (cfg.E, 2 * cfg.F, cfg.cols(cfg.H))),
        _ptr(w1_scale, "w1_scale", torch.uint8, (cfg.E, 2 * cfg.F, cfg.H // 32), optional=not mx),
        _ptr(offsets, "offsets", torch.int32, (cfg.E + 1,)), _ptr(h, "h", cfg.store_dtype, (cfg.R_cap, cfg.cols(cfg.F))),
        _ptr(h_scale, "h_scale", torch.uint8, (cfg.R_cap, cfg.F // 32), optional=not mx),
        _ptr(gu_stash, "gu_stash", cfg.out_dtype, (cfg.R_cap, 2 * cfg.F), optional=True), wp, wb,
        _stream(stream)))


def moe_grouped_swiglu_gemm_gather(cfg: MoEConfig, x, src_map, counts, w1, offsets, h, ws, x_scale=None,
                                   w1_scale=None, h_scale=None, stream=None):
    """The gate/up GEMM reading x[src_map[r] / k] for row r (no materialised Xp)."""
    c = cfg.c()
    mx = cfg.is_mx
    wp, wb = _ws(ws)
    _check(load_library().moe_grouped_swiglu_gemm_gather(
        ctypes.byref(c), _ptr(x, "x", cfg.store_dtype, (cfg.T, cfg.cols(cfg.H))),
        _ptr(x_scale, "x_scale", torch.uint8, (cfg.T, cfg.H // 32), optional=not mx),
        _ptr(src_map, "src_map", torch.int32, (cfg.R_cap,)), _ptr(counts, "counts", torch.int32, (cfg.E,)),
        _ptr(w1, "w1", cfg.store_dtype, (cfg.E, 2 * cfg.F, cfg.cols(cfg.H))),
        _ptr(w1_scale, "w1_scale", torch.uint8, (cfg.E, 2 * cfg.F, cfg.H // 32), optional=not mx),
        _ptr(offsets, "offsets", torch.int32, (cfg.E + 1,)), _ptr(h, "h", cfg.store_dtype, (cfg.R_cap, cfg.cols(cfg.F))),
        _ptr(h_scale, "h_scale", torch.uint8, (cfg.R_cap, cfg.F // 32), optional=not mx), wp, wb, _stream(stream)))


def moe_grouped_swiglu_gemm_weighted(cfg: MoEConfig, xp, w1, offsets, src_map, w, h, ws, xp_scale=None,
                                     w1_scale=None, h_scale=None, stream=None):
    """The gate/up GEMM with h scaled by each row's routing weight w[src_map[r]]."""
    c = cfg.c()
    mx = cfg.is_mx
    wp, wb = _ws(ws)
    _check(load_library().moe_grouped_swiglu_gemm_weighted(
        ctypes.byref(c), _ptr(xp, "xp", cfg.store_dtype, (cfg.R_cap, cfg.cols(cfg.H))),
        _ptr(xp_scale, "xp_scale", torch.uint8, (cfg.R_cap, cfg.H // 32), optional=not mx),
        _ptr(w1, "w1", cfg.store_dtype, (cfg.E, 2 * cfg.F, cfg.cols(cfg.H))),
        _ptr(w1_scale, "w1_scale", torch.uint8, (cfg.E, 2 * cfg.F, cfg.H // 32), optional=not mx),
        _ptr(offsets, "offsets", torch.int32, (cfg.E + 1,)), _ptr(src_map, "src_map", torch.int32, (cfg.R_cap,)),
        _ptr(w, "w", torch.float32, (cfg.T, cfg.k)), _ptr(h, "h", cfg.store_dtype, (cfg.R_cap, cfg.cols(cfg.F))),
        _ptr(h_scale, "h_scale", torch.uint8, (cfg.R_cap, cfg.F // 32), optional=not mx), wp, wb, _stream(stream)))


def moe_grouped_down_gemm_weighted(cfg: MoEConfig, h, w2, offsets, src_map, w, yp, ws, h_scale=None, w2_scale=None,
                                   stream=None):
    """The down GEMM with Yp scaled by each row's routing weight w[src_map[r]]."""
    c = cfg.c()
    mx = cfg.is_mx
    wp, wb = _ws(ws)
    _check(load_library().moe_grouped_down_gemm_weighted(
        ctypes.byref(c), _ptr(h, "h", cfg.store_dtype, (cfg.R_cap, cfg.cols(cfg.F))),
        _ptr(h_scale, "h_scale", torch.uint8, (cfg.R_cap, cfg.F // 32), optional=not mx),
        _ptr(w2, "w2", cfg.store_dtype, (cfg.E, cfg.H, cfg.cols(cfg.F))),
        _ptr(w2_scale, "w2_scale", torch.uint8, (cfg.E, cfg.H, cfg.F // 32), optional=not mx),
        _ptr(offsets, "offsets", torch.int32, (cfg.E + 1,)), _ptr(src_map, "src_map", torch.int32, (cfg.R_cap,)),
        _ptr(w, "w", torch.float32, (cfg.T, cfg.k)), _ptr(yp, "yp", cfg.out_dtype, (cfg.R_cap, cfg.H)),
        wp, wb, _stream(stream)))


def moe_grouped_down_gemm(cfg: MoEConfig, h, w2, offsets, yp, ws, h_scale=None, w2_scale=None, stream=None):
    c = cfg.c()
    mx = cfg.is_mx
    wp, wb = _ws(ws)
    _check(load_library().moe_grouped_down_gemm(
        ctypes.byref(c), _ptr(h, "h", cfg.store_dtype, (cfg.R_cap, cfg.cols(cfg.F))),
        _ptr(h_scale, "h_scale", torch.uint8, (cfg.R_cap, cfg.F // 32), optional=not mx),
        _ptr(w2, "w2", cfg.store_dtype, (cfg.E, cfg.H, cfg.cols(cfg.F))),
        _ptr(w2_scale, "w2_scale", torch.uint8, (cfg.E, cfg.H, cfg.F // 32), optional=not mx),
        _ptr(offsets, "offsets", torch.int32, (cfg.E + 1,)), _ptr(yp, "yp", cfg.out_dtype, (cfg.R_cap, cfg.H)),
        wp, wb, _stream(stream)))


def moe_combine(cfg: MoEConfig, yp, row_map, w, y, stream=None):
    """y[t] = sum_j w[t, j] Yp[row_map[t, j]]; w None sums the routes (weights already applied)."""
    c = cfg.c()
    _check(load_library().moe_combine(
        ctypes.byref(c), _ptr(yp, "yp", cfg.out_dtype, (cfg.R_cap, cfg.H)),
        _ptr(row_map, "row_map", torch.int32, (cfg.T, cfg.k)),
        _ptr(w, "w", torch.float32, (cfg.T, cfg.k), optional=True),
        _ptr(y, "y", cfg.out_dtype, (cfg.T, cfg.H)), _stream(stream)))


def moe_forward(cfg: MoEConfig, logits, x, w1, w2, buf: dict, x_scale=None, w1_scale=None, w2_scale=None,
                stream=None, bias=None):
    """buf: the caller's buffers, as made by alloc_forward(); bias as in moe_route."""
    _forward_call(cfg, logits, x, w1, w2, buf, x_scale, w1_scale, w2_scale, stream, bias, noalloc=False)


def moe_forward_noalloc(cfg: MoEConfig, logits, x, w1, w2, buf: dict, x_scale=None, w1_scale=None, w2_scale=None,
                        stream=None, bias=None):
    """moe_forward with the library's static scratch array instead of buf["ws"]
    (which is not used)."""
    _forward_call(cfg, logits, x, w1, w2, buf, x_scale, w1_scale, w2_scale, stream, bias, noalloc=True)


def _forward_call(cfg, logits, x, w1, w2, buf, x_scale, w1_scale, w2_scale, stream, bias, noalloc):
    c = cfg.c()
    mx = cfg.is_mx
    ws_args = () if noalloc else _ws(buf["ws"])
    fn = load_library().moe_forward_noalloc if noalloc else load_library().moe_forward
    R, T, H, F, E, k = cfg.R_cap, cfg.T, cfg.H, cfg.F, cfg.E, cfg.k
    sd, od = cfg.store_dtype, cfg.out_dtype
    _check(fn(
        ctypes.byref(c), _ptr(logits, "logits", torch.float32, (T, E)),
        _ptr(bias, "bias", torch.float32, (E,), optional=True), _ptr(x, "x", sd, (T, cfg.cols(H))),
        _ptr(x_scale, "x_scale", torch.uint8, (T, H // 32), optional=not mx),
        _ptr(w1, "w1", sd, (E, 2 * F, cfg.cols(H))),
        _ptr(w1_scale, "w1_scale", torch.uint8, (E, 2 * F, H // 32), optional=not mx),
        _ptr(w2, "w2", sd, (E, H, cfg.cols(F))), _ptr(w2_scale, "w2_scale", torch.uint8, (E, H, F // 32), optional=not mx),
        _ptr(buf["y"], "y", od, (T, H)), _ptr(buf["idx"], "idx", torch.int32, (T, k)),
        _ptr(buf["w"], "w", torch.float32, (T, k)), _ptr(buf["counts"], "counts", torch.int32, (E,)),
        _ptr(buf["offsets"], "offsets", torch.int32, (E + 1,)), _ptr(buf["row_map"], "row_map", torch.int32, (T, k)),
        _ptr(buf["src_map"], "src_map", torch.int32, (R,)),
        _ptr(buf.get("xp"), "xp", sd, (R, cfg.cols(H)), optional=True),
        _ptr(buf.get("xp_scale"), "xp_scale", torch.uint8, (R, H // 32), optional=not mx or buf.get("xp") is None),
        _ptr(buf["h"], "h", sd, (R, cfg.cols(F))),
        _ptr(buf.get("h_scale"), "h_scale", torch.uint8, (R, F // 32), optional=not mx),
        _ptr(buf["yp"], "yp", od, (R, H)),
        _ptr(buf.get("gu_stash"), "gu_stash", od, (R, 2 * F), optional=True),
        _ptr(buf.get("err"), "err", torch.int32, (1,), optional=True), *ws_args, _stream(stream)))


def moe_route_bwd(cfg: MoEConfig, dy, yp, logits, idx, row_map, dlogits, dw=None, stream=None):
    """Gradients of the top-k weights (dw, optional) and of the router logits."""
    c = cfg.c()
    _check(load_library().moe_route_bwd(
        ctypes.byref(c), _ptr(dy, "dy", cfg.out_dtype, (cfg.T, cfg.H)),
        _ptr(yp, "yp", cfg.out_dtype, (cfg.R_cap, cfg.H)), _ptr(logits, "logits", torch.float32, (cfg.T, cfg.E)),
        _ptr(idx, "idx", torch.int32, (cfg.T, cfg.k)), _ptr(row_map, "row_map", torch.int32, (cfg.T, cfg.k)),
        _ptr(dw, "dw", torch.float32, (cfg.T, cfg.k), optional=True),
        _ptr(dlogits, "dlogits", torch.float32, (cfg.T, cfg.E)), _stream(stream)))


def moe_combine_bwd(cfg: MoEConfig, dy, row_map, src_map, offsets, w, dyp, stream=None):
    c = cfg.c()
    _check(load_library().moe_combine_bwd(
        ctypes.byref(c), _ptr(dy, "dy", cfg.out_dtype, (cfg.T, cfg.H)),
        _ptr(row_map, "row_map", torch.int32, (cfg.T, cfg.k)),
        _ptr(src_map, "src_map", torch.int32, (cfg.R_cap,)), _ptr(offsets, "offsets", torch.int32, (cfg.E + 1,)),
        _ptr(w, "w", torch.float32, (cfg.T, cfg.k)), _ptr(dyp, "dyp", cfg.out_dtype, (cfg.R_cap, cfg.H)),
        _stream(stream)))


def moe_grouped_down_bwd(cfg: MoEConfig, dyp, w2, h, gu_stash, offsets, dgu, dw2, ws, stream=None):
    c = cfg.c()
    wp, wb = _ws(ws)
    _check(load_library().moe_grouped_down_bwd(
        ctypes.byref(c), _ptr(dyp, "dyp", cfg.out_dtype, (cfg.R_cap, cfg.H)),
        _ptr(w2, "w2", cfg.store_dtype, (cfg.E, cfg.H, cfg.cols(cfg.F))), _ptr(h, "h", cfg.store_dtype, (cfg.R_cap, cfg.cols(cfg.F))),
        _ptr(gu_stash, "gu_stash", cfg.out_dtype, (cfg.R_cap, 2 * cfg.F)),
        _ptr(offsets, "offsets", torch.int32, (cfg.E + 1,)), _ptr(dgu, "dgu", cfg.out_dtype, (cfg.R_cap, 2 * cfg.F)),
        _ptr(dw2, "dw2", torch.float32, (cfg.E, cfg.H, cfg.F)), wp, wb, _stream(stream)))


def moe_grouped_swiglu_bwd(cfg: MoEConfig, dgu, w1, xp, offsets, dxp, dw1, ws, stream=None):
    c = cfg.c()
    wp, wb = _ws(ws)
    _check(load_library().moe_grouped_swiglu_bwd(
        ctypes.byref(c), _ptr(dgu, "dgu", cfg.out_dtype, (cfg.R_cap, 2 * cfg.F)),
        _ptr(w1, "w1", cfg.store_dtype, (cfg.E, 2 * cfg.F, cfg.cols(cfg.H))), _ptr(xp, "xp", cfg.store_dtype, (cfg.R_cap, cfg.cols(cfg.H))),
        _ptr(offsets, "offsets", torch.int32, (cfg.E + 1,)), _ptr(dxp, "dxp", cfg.out_dtype, (cfg.R_cap, cfg.H)),
        _ptr(dw1, "dw1", torch.float32, (cfg.E, 2 * cfg.F, cfg.H)), wp, wb, _stream(stream)))


def moe_permute_bwd(cfg: MoEConfig, dxp, row_map, dx, stream=None):
    c = cfg.c()
    _check(load_library().moe_permute_bwd(
        ctypes.byref(c), _ptr(dxp, "dxp", cfg.out_dtype, (cfg.R_cap, cfg.H)),
        _ptr(row_map, "row_map", torch.int32, (cfg.T, cfg.k)), _ptr(dx, "dx", cfg.out_dtype, (cfg.T, cfg.H)),
        _stream(stream)))


def moe_backward(cfg: MoEConfig, dy, w1, w2, fwd: dict, bwd: dict, stream=None):
    """fwd: the forward's buffers (alloc_forward(training=True)); bwd: alloc_backward()."""
    c = cfg.c()
    wp, wb = _ws(bwd["ws"])
    R, T, H, F, E, k = cfg.R_cap, cfg.T, cfg.H, cfg.F, cfg.E, cfg.k
    sd, od = cfg.store_dtype, cfg.out_dtype
    _check(load_library().moe_backward(
        ctypes.byref(c), _ptr(dy, "dy", od, (T, H)), _ptr(fwd["w"], "w", torch.float32, (T, k)),
        _ptr(w1, "w1", sd, (E, 2 * F, H)), _ptr(w2, "w2", sd, (E, H, F)),
        _ptr(fwd["offsets"], "offsets", torch.int32, (E + 1,)), _ptr(fwd["row_map"], "row_map", torch.int32, (T, k)),
        _ptr(fwd["src_map"], "src_map", torch.int32, (R,)), _ptr(fwd["xp"], "xp", sd, (R, H)),
        _ptr(fwd["h"], "h", sd, (R, F)), _ptr(fwd["gu_stash"], "gu_stash", od, (R, 2 * F)),
        _ptr(bwd["dyp"], "dyp", od, (R, H)), _ptr(bwd["dgu"], "dgu", od, (R, 2 * F)),
        _ptr(bwd["dxp"], "dxp", od, (R, H)), _ptr(bwd["dx"], "dx", od, (T, H)),
        _ptr(bwd["dw1"], "dw1", torch.float32, (E, 2 * F, H)), _ptr(bwd["dw2"], "dw2", torch.float32, (E, H, F)),
        wp, wb, _stream(stream)))


def moe_quantize_mxfp8(x, codes, scales, stream=None):
    rows, cols = x.shape[0], x.shape[-1]
    rows = x.numel() // cols if cols else 0
    _check(load_library().moe_quantize_mxfp8(
        _ptr(x, "x", torch.float32), rows, cols, _ptr(codes, "codes", torch.uint8, tuple(x.shape)),
        _ptr(scales, "scales", torch.uint8, tuple(x.shape[:-1]) + (cols // 32,)), _stream(stream)))


def moe_quantize_mxfp4(x, codes, scales, stream=None):
    """x float32 [..., n] -> codes uint8 [..., n/2] (two E2M1 per byte), scales uint8 [..., n/32]."""
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    _check(load_library().moe_quantize_mxfp4(
        _ptr(x, "x", torch.float32), rows, cols, _ptr(codes, "codes", torch.uint8, tuple(x.shape[:-1]) + (cols // 2,)),
        _ptr(scales, "scales", torch.uint8, tuple(x.shape[:-1]) + (cols // 32,)), _stream(stream)))


# ------------------------------------------------------------ buffer helpers
def alloc_forward(cfg: MoEConfig, device="cuda", training: bool = False) -> dict:
    """Caller-side buffers of moe_forward (plain torch allocations)."""
    R, T, H, F, E, k = cfg.R_cap, cfg.T, cfg.H, cfg.F, cfg.E, cfg.k
    sd, od = cfg.store_dtype, cfg.out_dtype
    b = {
        "y": torch.empty(T, H, dtype=od, device=device),
        "idx": torch.empty(T, k, dtype=torch.int32, device=device),
        "w": torch.empty(T, k, dtype=torch.float32, device=device),
        "counts": torch.empty(E, dtype=torch.int32, device=device),
        "offsets": torch.empty(E + 1, dtype=torch.int32, device=device),
        "row_map": torch.empty(T, k, dtype=torch.int32, device=device),
        "src_map": torch.empty(R, dtype=torch.int32, device=device),
        "xp": torch.empty(R, cfg.cols(H), dtype=sd, device=device),
        "h": torch.empty(R, cfg.cols(F), dtype=sd, device=device),
        "yp": torch.empty(R, H, dtype=od, device=device),
        "err": torch.zeros(1, dtype=torch.int32, device=device),
        "ws": torch.empty(max(workspace_size(cfg), 1), dtype=torch.uint8, device=device),
    }
    if cfg.is_mx:
        b["xp_scale"] = torch.empty(R, H // 32, dtype=torch.uint8, device=device)
        b["h_scale"] = torch.empty(R, F // 32, dtype=torch.uint8, device=device)
    if training:
        b["gu_stash"] = torch.empty(R, 2 * F, dtype=od, device=device)
    return b


def alloc_backward(cfg: MoEConfig, device="cuda") -> dict:
    R, T, H, F, E = cfg.R_cap, cfg.T, cfg.H, cfg.F, cfg.E
    od = cfg.out_dtype
    return {
        "dyp": torch.empty(R, H, dtype=od, device=device),
        "dgu": torch.empty(R, 2 * F, dtype=od, device=device),
        "dxp": torch.empty(R, H, dtype=od, device=device),
        "dx": torch.empty(T, H, dtype=od, device=device),
        "dw1": torch.empty(E, 2 * F, H, dtype=torch.float32, device=device),
        "dw2": torch.empty(E, H, F, dtype=torch.float32, device=device),
        "ws": torch.empty(max(backward_workspace_size(cfg), 1), dtype=torch.uint8, device=device),
    }
