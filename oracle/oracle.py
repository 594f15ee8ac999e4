"""Python (ctypes + numpy) front end of the CPU oracle in moe_oracle.c.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code with
the HIP library.

Formats: "f32" (float32), "bf16" (uint16 bit patterns), "mxfp8" (uint8 E4M3
codes plus uint8 E8M0 scales, one per 32 elements along the last axis),
"mxfp4" (E2M1 codes packed two per byte, element 2i in the low 4 bits of byte
i, so a row of n elements is n / 2 bytes; the same E8M0 scales).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "moe_oracle.c")
FMT = {"f32": 0, "bf16": 1, "mxfp8": 2, "mxfp4": 3}
MX = ("mxfp8", "mxfp4")
SCORE = {"softmax": 0, "sigmoid": 1}
_NP = {"f32": np.float32, "bf16": np.uint16, "mxfp8": np.uint8, "mxfp4": np.uint8}


def row_len(fmt: str, n: int) -> int:
    """Stored entries of a row of n elements (MXFP4: n / 2 bytes)."""
    return n // 2 if fmt == "mxfp4" else n


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", "-o", LIB_PATH, SRC_PATH, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return LIB_PATH


_lib = None
P = ctypes.c_void_p
I32 = ctypes.c_int
I64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "or_bf16_from_double": (ctypes.c_uint16, [ctypes.c_double]),
        "or_double_from_bf16": (ctypes.c_double, [ctypes.c_uint16]),
        "or_e4m3_from_double": (ctypes.c_uint8, [ctypes.c_double]),
        "or_double_from_e4m3": (ctypes.c_double, [ctypes.c_uint8]),
        "or_double_from_e8m0": (ctypes.c_double, [ctypes.c_uint8]),
        "or_bf16_from_double_array": (None, [P, P, I64]),
        "or_e4m3_from_double_array": (None, [P, P, I64]),
        "or_double_from_e4m3_array": (None, [P, P, I64]),
        "or_mx_quantize_f32": (I32, [P, I64, I64, P, P]),
        "or_mx_quantize_f32_fmt": (I32, [I32, P, I64, I64, P, P]),
        "or_e2m1_from_double": (ctypes.c_uint8, [ctypes.c_double]),
        "or_double_from_e2m1": (ctypes.c_double, [ctypes.c_uint8]),
        "or_e2m1_from_double_array": (None, [P, P, I64]),
        "or_route": (I32, [I32, I32, I32, I32, I32, P, P, P]),
        "or_route_biased": (I32, [I32, I32, I32, I32, I32, P, P, P, P]),
        "or_group": (I32, [I32, I32, I32, I32, I64, P, P, P, P, P, P]),
        "or_permute": (None, [I32, I32, I64, I64, P, P, P]),
        "or_forward_tokens": (I32, [I32, I32, I32, I32, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, P, P, P, P,
                                    P, P, P]),
        "or_combine": (None, [I32, I32, I32, I32, P, P, P, P]),
        "or_set_swiglu_limit": (None, [ctypes.c_double]),
        "or_backward": (I32, [I32, I32, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, P, I32, P, I32, P, P, P, P,
                              P, P, P]),
        "or_backward_dx_tokens": (I32, [I32, I32, I32, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, P]),
        "or_backward_dw_entries": (I32, [I32, I32, I32, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, I32, P, P,
                                         P, I32, P, P, P]),
        "or_num_threads": (I32, []),
        "or_swiglu_rows": (None, [P, I64, I32, P, P]),
        "or_swiglu_grad_rows": (None, [P, P, I64, I32, P]),
        "or_store_rows": (None, [I32, P, I64, I64, P, P]),
        "or_decode_rows": (None, [I32, P, P, I64, I64, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype=None):
    a = np.ascontiguousarray(a)
    if dtype is not None and a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def num_threads() -> int:
    return _load().or_num_threads()


# ---------------------------------------------------------------- formats
def bf16_from_f64(v) -> np.ndarray:
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    out = np.empty(v.shape, np.uint16)
    _load().or_bf16_from_double_array(v.ctypes.data, out.ctypes.data, v.size)
    return out


def f64_from_bf16(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3_from_f64(v) -> np.ndarray:
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    out = np.empty(v.shape, np.uint8)
    _load().or_e4m3_from_double_array(v.ctypes.data, out.ctypes.data, v.size)
    return out


def f64_from_e4m3(c) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(c, dtype=np.uint8))
    out = np.empty(c.shape, np.float64)
    _load().or_double_from_e4m3_array(c.ctypes.data, out.ctypes.data, c.size)
    return out


def f64_from_e8m0(c) -> np.ndarray:
    c = np.asarray(c, dtype=np.uint8).astype(np.int64)
    out = np.ldexp(1.0, c - 127).astype(np.float64)
    return np.where(c == 255, np.nan, out)


def e2m1_from_f64(v) -> np.ndarray:
    """Round to E2M1 (RNE, saturating at 6): one 4-bit code per uint8."""
    v = _c(np.asarray(v, np.float64), np.float64)
    out = np.empty(v.shape, np.uint8)
    _load().or_e2m1_from_double_array(v.ctypes.data, out.ctypes.data, v.size)
    return out


def f64_from_e2m1(c) -> np.ndarray:
    """E2M1 codes (low 4 bits of each uint8) to float64."""
    lib = _load()
    tab = np.array([lib.or_double_from_e2m1(i) for i in range(16)])
    return tab[np.asarray(c, np.uint8) & 0xF]


def mx_quantize(v, fmt: str = "mxfp8") -> tuple:
    """float32 [..., n] (n % 32 == 0) -> (codes uint8 [..., n] (E4M3) or [..., n/2]
    (packed E2M1), E8M0 scales uint8 [..., n/32])."""
    v = _c(v, np.float32)
    cols = v.shape[-1]
    rows = v.size // cols
    codes = np.empty(v.shape[:-1] + (row_len(fmt, cols),), np.uint8)
    scales = np.empty(v.shape[:-1] + (cols // 32,), np.uint8)
    if _load().or_mx_quantize_f32_fmt(FMT[fmt], v.ctypes.data, rows, cols, codes.ctypes.data, scales.ctypes.data):
        raise ValueError("last dimension must be a multiple of 32")
    return codes, scales


def mx_dequantize(codes, scales, fmt: str = "mxfp8") -> np.ndarray:
    """Codes [..., n] (E4M3) or [..., n/2] (packed E2M1) with E8M0 scales
    [..., n/32] -> float64 values [..., n]."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    n = codes.shape[-1] * (2 if fmt == "mxfp4" else 1)
    rows = codes.size // codes.shape[-1] if codes.shape[-1] else 0
    if scales.shape != codes.shape[:-1] + (n // 32,):
        raise ValueError("scales must hold one code per 32 elements of the last axis")
    out = np.empty(codes.shape[:-1] + (n,), np.float64)
    if codes.size:
        _load().or_decode_rows(FMT[fmt], codes.ctypes.data, scales.ctypes.data, rows, n, out.ctypes.data)
    return out


def decode(fmt: str, data, scale=None) -> np.ndarray:
    """Stored values to float64."""
    if fmt == "f32":
        return np.asarray(data, np.float32).astype(np.float64)
    if fmt == "bf16":
        return f64_from_bf16(data)
    return mx_dequantize(data, scale, fmt)


# ---------------------------------------------------------------- the path
def route(logits, k: int, score: str = "softmax", renorm: bool = False, bias=None):
    """Top-k routing (or_route_biased): bias (optional, float32 [E]) shifts
    only the selection key, key = fl32(logit + bias); the weights use the
    unbiased logits."""
    lg = _c(logits, np.float32)
    T, E = lg.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    b = None if bias is None else _c(np.asarray(bias, np.float32).reshape(E), np.float32)
    if _load().or_route_biased(T, E, k, SCORE[score], int(renorm), lg.ctypes.data, _p(b), idx.ctypes.data,
                               w.ctypes.data):
        raise ValueError("bad routing sizes")
    return idx, w


def route_bwd(logits, idx, row_map, dy, yp, fmt: str, score: str = "softmax", renorm: bool = False,
              tokens=None):
    """Routing backward, float64.

    The forward gives route (t, j) the weight w[t, j] of its expert idx[t, j]
    as or_route computes it: the softmax over all E logits p, either as is or
    renormalised over the k chosen (p / (sum of the chosen p + 1e-20)), or the
    sigmoid of the chosen logits normalised over the k chosen (s / (sum s +
    1e-20)); the combine forms y[t] = sum_j w[t, j] Yp[row_map[t, j]].  For an
    upstream gradient dy of y:
        dw[t, j]      = <dy[t], Yp[row_map[t, j]]>   (0 for a dropped route, row -1)
        dlogits[t, e] = sum_j dw[t, j] * d w[t, j] / d logits[t, e]
    written out by the chain rule through the normalisation above; the top-k
    choice is piecewise constant and contributes nothing.

    dy [T, H] and yp [R, H] are stored arrays of format fmt; tokens (optional)
    selects the rows of the result.  Returns (dw [n, k], dlogits [n, E])."""
    lg = np.asarray(logits, np.float32)
    T, E = lg.shape
    k = idx.shape[1]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    n = len(tok)
    rm = np.asarray(row_map).reshape(T, k)[tok]
    sel = np.asarray(idx)[tok].astype(np.int64)
    dyv = decode(fmt, np.asarray(dy)[tok])
    dw = np.zeros((n, k))
    for j in range(k):
        ok = rm[:, j] >= 0
        if ok.any():
            dw[ok, j] = np.einsum("th,th->t", dyv[ok], decode(fmt, np.asarray(yp)[rm[ok, j]]))
    l = lg[tok].astype(np.float64)
    ok_sel = (sel >= 0) & (sel < E)
    sel_c = np.where(ok_sel, sel, 0)
    dl = np.zeros((n, E))
    rows = np.arange(n)[:, None]
    if score == "softmax":
        m = l.max(axis=1, keepdims=True)
        a = np.exp(l - m)
        p = a / a.sum(axis=1, keepdims=True)
        sc = np.where(ok_sel, p[rows, sel_c], 0.0)          # p of the chosen experts
        if renorm:
            S = sc.sum(axis=1, keepdims=True) + 1e-20
            dsc = dw / S - (dw * sc).sum(axis=1, keepdims=True) / S ** 2
        else:
            dsc = dw
        dsc = np.where(ok_sel, dsc, 0.0)
        # d p_c / d l_e = p_c (delta_ce - p_e)
        np.add.at(dl, (np.broadcast_to(rows, sel_c.shape), sel_c), dsc * sc)
        dl -= p * (dsc * sc).sum(axis=1, keepdims=True)
    else:
        s = np.where(ok_sel, 1.0 / (1.0 + np.exp(-l[rows, sel_c])), 0.0)
        S = s.sum(axis=1, keepdims=True) + 1e-20
        ds = dw / S - (dw * s).sum(axis=1, keepdims=True) / S ** 2
        ds = np.where(ok_sel, ds, 0.0)
        np.add.at(dl, (np.broadcast_to(rows, sel_c.shape), sel_c), ds * s * (1.0 - s))
    return dw, dl


def group(idx, E: int, align: int = 1, R_cap: int | None = None):
    idx = _c(idx, np.int32)
    T, k = idx.shape
    if R_cap is None:
        R_cap = T * k + E * (align - 1)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    row_map = np.empty((T, k), np.int32)
    src_map = np.empty(R_cap, np.int32)
    bad = np.zeros(1, np.int32)
    rc = _load().or_group(T, E, k, align, R_cap, idx.ctypes.data, counts.ctypes.data, offsets.ctypes.data,
                          row_map.ctypes.data, src_map.ctypes.data, bad.ctypes.data)
    if rc:
        raise ValueError(f"or_group failed ({rc})")
    return counts, offsets, row_map, src_map, int(bad[0])


def permute(x, row_map, n_rows: int):
    """Rows of x (any dtype, 2-D) copied to their routes' rows; padding zero."""
    x = np.ascontiguousarray(x)
    row_map = _c(row_map, np.int32)
    T, k = row_map.shape
    row_bytes = x.strides[0]
    xp = np.empty((n_rows,) + x.shape[1:], x.dtype)
    _load().or_permute(T, k, n_rows, row_bytes, x.ctypes.data, row_map.ctypes.data, xp.ctypes.data)
    return xp


SITES = {"combine": 0, "fc1": 1, "fc2": 2}


def forward_tokens(shape, tokens, x, w1, w2, idx, w, x_scale=None, w1_scale=None, w2_scale=None,
                   want_stash: bool = False, site: str = "combine", limit: float = 0.0):
    """Per-token evaluation of the expert FFN and the combine.

    limit: the optional SwiGLU clamp (0 = none): h = silu(min(g, L)) clamp(u, -L, L).
    site: where the routing weight is applied ([CUDNN] Summary: router weight in
    the FC1 or FC2 epilogue): "combine" (default), "fc1" (h scaled before it is
    stored) or "fc2" (Yp scaled before it is stored; the combine then sums).

    x, w1, w2 are stored arrays of format shape.dtype (w1 [E, 2F, H], w2 [E, H, F]).
    Returns dict with h [n, k, F] (+ h_scale for MXFP8), yp [n, k, H], y [n, H]
    and (optionally) stash [n, k, 2F], all in storage form."""
    s = shape
    fmt = s.dtype
    y_fmt = "f32" if fmt == "f32" else "bf16"
    h_fmt = fmt
    s_fmt = "f32" if fmt == "f32" else "bf16"
    tokens = _c(np.asarray(tokens, np.int32), np.int32)
    n = tokens.size
    k = s.k
    h = np.empty((n, k, row_len(h_fmt, s.F)), _NP[h_fmt])
    h_scale = np.empty((n, k, s.F // 32), np.uint8) if h_fmt in MX else None
    yp = np.empty((n, k, s.H), _NP[y_fmt])
    y = np.empty((n, s.H), _NP[y_fmt])
    stash = np.empty((n, k, 2 * s.F), _NP[s_fmt]) if want_stash else None
    x = np.ascontiguousarray(x)
    w1 = np.ascontiguousarray(w1)
    w2 = np.ascontiguousarray(w2)
    idx = _c(idx, np.int32)
    w = _c(w, np.float32)
    xs = None if x_scale is None else np.ascontiguousarray(x_scale)
    w1s = None if w1_scale is None else np.ascontiguousarray(w1_scale)
    w2s = None if w2_scale is None else np.ascontiguousarray(w2_scale)
    _load().or_set_swiglu_limit(float(limit))
    rc = _load().or_forward_tokens(s.H, s.F, k, FMT[fmt], FMT[h_fmt], FMT[y_fmt], FMT[s_fmt], SITES[site], n,
                                   tokens.ctypes.data,
                                   x.ctypes.data, _p(xs), w1.ctypes.data, _p(w1s), w2.ctypes.data, _p(w2s),
                                   idx.ctypes.data, w.ctypes.data, h.ctypes.data, _p(h_scale), yp.ctypes.data,
                                   _p(stash), y.ctypes.data)
    if rc:
        raise ValueError("or_forward_tokens: unsupported sizes")
    out = {"h": h, "yp": yp, "y": y}
    if h_scale is not None:
        out["h_scale"] = h_scale
    if stash is not None:
        out["stash"] = stash
    return out


def combine(yp, row_map, w, y_fmt: str):
    """y[t] = sum_j w[t, j] Yp[row_map[t, j]]; w None sums the routes unweighted."""
    yp = np.ascontiguousarray(yp)
    row_map = _c(row_map, np.int32)
    w = None if w is None else _c(w, np.float32)
    T, k = row_map.shape
    H = yp.shape[1]
    y = np.empty((T, H), _NP[y_fmt])
    _load().or_combine(T, H, k, FMT[y_fmt], yp.ctypes.data, row_map.ctypes.data, _p(w), y.ctypes.data)
    return y


def backward(shape, x, w1, w2, w, row_map, src_map, offsets, h_rows, stash_rows, dy, limit: float = 0.0):
    """Full backward (small shapes).  h_rows [R_cap, F] / stash_rows [R_cap, 2F]
    are the forward's stored h and stash arranged by permuted row."""
    s = shape
    fmt = s.dtype
    g_fmt = "f32" if fmt == "f32" else "bf16"
    R_cap = src_map.shape[0]
    gdt = _NP[g_fmt]
    dyp = np.zeros((R_cap, s.H), gdt)
    dgu = np.zeros((R_cap, 2 * s.F), gdt)
    dxp = np.zeros((R_cap, s.H), gdt)
    dx = np.empty((s.T, s.H), gdt)
    dw1 = np.empty((s.E, 2 * s.F, s.H), np.float32)
    dw2 = np.empty((s.E, s.H, s.F), np.float32)
    args = [np.ascontiguousarray(a) for a in (x, w1, w2)]
    w = _c(w, np.float32)
    row_map = _c(row_map, np.int32)
    src_map = _c(src_map, np.int32)
    offsets = _c(offsets, np.int32)
    h_rows = np.ascontiguousarray(h_rows)
    stash_rows = np.ascontiguousarray(stash_rows)
    dy = np.ascontiguousarray(dy)
    _load().or_set_swiglu_limit(float(limit))
    rc = _load().or_backward(s.T, s.H, s.F, s.E, s.k, FMT[fmt], FMT[g_fmt], args[0].ctypes.data, args[1].ctypes.data,
                             args[2].ctypes.data, w.ctypes.data, row_map.ctypes.data, src_map.ctypes.data,
                             offsets.ctypes.data, h_rows.ctypes.data, FMT[fmt], stash_rows.ctypes.data,
                             FMT[g_fmt], dy.ctypes.data, dyp.ctypes.data, dgu.ctypes.data, dxp.ctypes.data,
                             dx.ctypes.data, dw1.ctypes.data, dw2.ctypes.data)
    if rc:
        raise ValueError("or_backward: unsupported format")
    return {"dyp": dyp, "dgu": dgu, "dxp": dxp, "dx": dx, "dw1": dw1, "dw2": dw2}


def backward_dx_tokens(shape, tokens, x, w1, w2, idx, w, dy, limit: float = 0.0):
    s = shape
    fmt = s.dtype
    g_fmt = "f32" if fmt == "f32" else "bf16"
    tokens = _c(np.asarray(tokens, np.int32), np.int32)
    dx = np.empty((tokens.size, s.H), _NP[g_fmt])
    a = [np.ascontiguousarray(v) for v in (x, w1, w2, dy)]
    _load().or_set_swiglu_limit(float(limit))
    rc = _load().or_backward_dx_tokens(s.H, s.F, s.k, FMT[fmt], FMT[g_fmt], FMT[fmt], FMT[g_fmt], tokens.size,
                                       tokens.ctypes.data, a[0].ctypes.data, a[1].ctypes.data, a[2].ctypes.data,
                                       _c(idx, np.int32).ctypes.data, _c(w, np.float32).ctypes.data,
                                       a[3].ctypes.data, dx.ctypes.data)
    if rc:
        raise ValueError("unsupported")
    return dx


def backward_dw_entries(shape, e, x, w1, w2, w, src_map, offsets, dy, dw2_idx, dw1_idx, limit: float = 0.0):
    """dW2s[e][o, f] for (o, f) in dw2_idx and dW1s[e][n, c] for (n, c) in dw1_idx (float64)."""
    s = shape
    fmt = s.dtype
    g_fmt = "f32" if fmt == "f32" else "bf16"
    dw2_idx = np.asarray(dw2_idx, np.int32).reshape(-1, 2)
    dw1_idx = np.asarray(dw1_idx, np.int32).reshape(-1, 2)
    o2 = np.ascontiguousarray(dw2_idx[:, 0])
    f2 = np.ascontiguousarray(dw2_idx[:, 1])
    n1 = np.ascontiguousarray(dw1_idx[:, 0])
    c1 = np.ascontiguousarray(dw1_idx[:, 1])
    out2 = np.empty(len(o2), np.float64)
    out1 = np.empty(len(n1), np.float64)
    a = [np.ascontiguousarray(v) for v in (x, w1, w2, dy)]
    _load().or_set_swiglu_limit(float(limit))
    rc = _load().or_backward_dw_entries(s.H, s.F, s.k, FMT[fmt], FMT[g_fmt], FMT[fmt], FMT[g_fmt], int(e),
                                        a[0].ctypes.data, a[1].ctypes.data, a[2].ctypes.data,
                                        _c(w, np.float32).ctypes.data, _c(src_map, np.int32).ctypes.data,
                                        _c(offsets, np.int32).ctypes.data, a[3].ctypes.data, len(o2),
                                        o2.ctypes.data, f2.ctypes.data, out2.ctypes.data, len(n1), n1.ctypes.data,
                                        c1.ctypes.data, out1.ctypes.data)
    if rc:
        raise ValueError("unsupported")
    return out2, out1


# ------------------------------------------------ expert-major float64 front end
# The same definitions as forward_tokens / backward (moe_oracle.c), evaluated
# expert by expert so that the sums over H and F are float64 matrix products
# (numpy's BLAS, a library primitive) instead of ascending loops: fast enough
# to compare full-size layers in full or on thousands of tokens.  The
# per-element steps (SwiGLU and its gradient, the clamp, storage rounding and
# MX quantisation) are the C oracle's own functions.  Only the order of the
# float64 additions differs from the loop form; the tests pin this front end
# to it bit for bit on small shapes.
def _store_rows(fmt: str, v: np.ndarray):
    """float64 [rows, n] -> stored rows (MX formats: (codes, scales))."""
    v = np.ascontiguousarray(v, np.float64)
    rows, n = v.shape
    out = np.empty((rows, row_len(fmt, n)), _NP[fmt])
    sc = np.empty((rows, n // 32), np.uint8) if fmt in MX else None
    _load().or_store_rows(FMT[fmt], v.ctypes.data, rows, n, out.ctypes.data, _p(sc))
    return (out, sc) if fmt in MX else out


def _swiglu_rows(gu: np.ndarray, F: int, rw=None) -> np.ndarray:
    gu = np.ascontiguousarray(gu, np.float64)
    h = np.empty((gu.shape[0], F))
    rw = None if rw is None else np.ascontiguousarray(rw, np.float64)
    _load().or_swiglu_rows(gu.ctypes.data, gu.shape[0], F, _p(rw), h.ctypes.data)
    return h


def _swiglu_grad_rows(gu: np.ndarray, dh: np.ndarray, F: int) -> np.ndarray:
    gu = np.ascontiguousarray(gu, np.float64)
    dh = np.ascontiguousarray(dh, np.float64)
    d = np.empty((gu.shape[0], 2 * F))
    _load().or_swiglu_grad_rows(gu.ctypes.data, dh.ctypes.data, gu.shape[0], F, d.ctypes.data)
    return d


def _weights_f64(fmt: str, wt, wscale, e: int) -> np.ndarray:
    return decode(fmt, wt[e], None if wscale is None else wscale[e])


def forward_experts(shape, tokens, x, w1, w2, idx, w, x_scale=None, w1_scale=None, w2_scale=None,
                    want_stash: bool = False, site: str = "combine", limit: float = 0.0, want_h_f64: bool = False):
    """forward_tokens evaluated expert by expert (same arguments and outputs;
    want_h_f64 adds "h_f64" [n, k, F], the float64 h before it is stored).

    For each expert e, the routes (i, j) of the listed tokens with idx = e form
    X_e (their x rows, decoded); GU = X_e W1s[e]^T, h = store_h(SwiGLU(GU)),
    Yp = store_out(h W2s[e]^T), all sums in float64; then the combine
    y[i] = store_out(sum_{j ascending} c(t, j) Yp(i, j)) as in forward_tokens."""
    s = shape
    fmt = s.dtype
    y_fmt = s_fmt = "f32" if fmt == "f32" else "bf16"
    h_fmt = fmt
    tokens = np.asarray(tokens, np.int64)
    n, k = tokens.size, s.k
    idx = np.asarray(idx, np.int32)
    w = np.asarray(w, np.float32)
    sel = idx[tokens]                                   # [n, k]
    h = np.zeros((n, k, row_len(h_fmt, s.F)), _NP[h_fmt])
    h_sc = np.zeros((n, k, s.F // 32), np.uint8) if h_fmt in MX else None
    yp = np.zeros((n, k, s.H), _NP[y_fmt])
    stash = np.zeros((n, k, 2 * s.F), _NP[s_fmt]) if want_stash else None
    h64 = np.zeros((n, k, s.F)) if want_h_f64 else None
    _load().or_set_swiglu_limit(float(limit))
    for e in np.unique(sel[sel >= 0]):
        ii, jj = np.nonzero(sel == e)
        t = tokens[ii]
        xe = decode(fmt, np.asarray(x)[t], None if x_scale is None else np.asarray(x_scale)[t])
        gu = xe @ _weights_f64(fmt, w1, w1_scale, e).T
        rw = w[t, jj].astype(np.float64)
        hv = _swiglu_rows(gu, s.F, rw if site == "fc1" else None)
        if want_h_f64:
            h64[ii, jj] = hv
        if want_stash:
            stash[ii, jj] = _store_rows(s_fmt, gu)
        hs = _store_rows(h_fmt, hv)
        if h_fmt in MX:
            h[ii, jj], h_sc[ii, jj] = hs
            hq = decode(h_fmt, hs[0], hs[1])
        else:
            h[ii, jj] = hs
            hq = decode(h_fmt, hs)
        ye = hq @ _weights_f64(fmt, w2, w2_scale, e).T
        if site == "fc2":
            ye *= rw[:, None]
        yp[ii, jj] = _store_rows(y_fmt, ye)
    acc = np.zeros((n, s.H))
    for j in range(k):
        live = sel[:, j] >= 0
        c = np.ones(n) if site != "combine" else w[tokens, j].astype(np.float64)
        acc[live] += c[live, None] * decode(y_fmt, yp[live, j])
    out = {"h": h, "yp": yp, "y": _store_rows(y_fmt, acc)}
    if h_sc is not None:
        out["h_scale"] = h_sc
    if want_stash:
        out["stash"] = stash
    if want_h_f64:
        out["h_f64"] = h64
    return out


def down_projection(shape, experts, h, h_scale, w2, w2_scale=None, row_w=None):
    """The down projection of given stored h rows: for row r of expert
    experts[r] (-1: a row with no expert, left zero),
        Yp[r] = store_out( (decode(h[r]) W2s[e]^T) * row_w[r] )
    with float64 sums (row_w None: no weight), as in forward_experts.  h
    [rows, F] in shape.dtype's stored form (MX: with h_scale [rows, F/32])."""
    s = shape
    fmt = s.dtype
    y_fmt = "f32" if fmt == "f32" else "bf16"
    experts = np.asarray(experts)
    yp = np.zeros((experts.size, s.H), _NP[y_fmt])
    for e in np.unique(experts[experts >= 0]):
        r = np.flatnonzero(experts == e)
        hq = decode(fmt, np.asarray(h)[r], None if h_scale is None else np.asarray(h_scale)[r])
        ye = hq @ _weights_f64(fmt, w2, w2_scale, int(e)).T
        if row_w is not None:
            ye *= np.asarray(row_w, np.float64)[r, None]
        yp[r] = _store_rows(y_fmt, ye)
    return yp


def backward_expert(shape, e: int, x, w1, w2, w, src_map, offsets, dy, limit: float = 0.0):
    """Backward of one expert's rows, as or_backward defines it, with the
    forward's stored h and stash recomputed from x (forward_experts' steps):
    dYp = store_g(w dY[t]), dH = dYp W2s[e], dGU = store_g(dSwiGLU(stash, dH)),
    dW2s[e] = dYp^T h, dXp = store_g(dGU W1s[e]), dW1s[e] = dGU^T Xp; weight
    gradients float32 (exactly 0 for an expert with no rows).  Sums in float64.
    Returns dict with dw1 [2F, H] f32, dw2 [H, F] f32 and, for the expert's
    real rows (in row order, `rows`), dyp, dgu, dxp in storage form."""
    s = shape
    fmt = s.dtype
    g_fmt = "f32" if fmt == "f32" else "bf16"
    rows = np.arange(int(offsets[e]), int(offsets[e + 1]))
    src = np.asarray(src_map)[rows]
    rows = rows[src >= 0]
    src = src[src >= 0].astype(np.int64)
    t = src // s.k
    if rows.size == 0:
        return {"dw1": np.zeros((2 * s.F, s.H), np.float32), "dw2": np.zeros((s.H, s.F), np.float32),
                "rows": rows}
    _load().or_set_swiglu_limit(float(limit))
    xe = decode(fmt, np.asarray(x)[t])
    w1e = decode(fmt, np.asarray(w1)[e])
    w2e = decode(fmt, np.asarray(w2)[e])
    gu = xe @ w1e.T
    st = decode(g_fmt, _store_rows(g_fmt, gu))                       # the stash as stored
    hq = decode(fmt, _store_rows(fmt, _swiglu_rows(gu, s.F)))         # h as stored
    wr = np.asarray(w, np.float32).ravel()[src].astype(np.float64)
    dyp = _store_rows(g_fmt, wr[:, None] * decode(g_fmt, np.asarray(dy)[t]))
    dypd = decode(g_fmt, dyp)
    dh = dypd @ w2e
    dgu = _store_rows(g_fmt, _swiglu_grad_rows(st, dh, s.F))
    dgud = decode(g_fmt, dgu)
    dxp = _store_rows(g_fmt, dgud @ w1e)
    return {"dw2": (dypd.T @ hq).astype(np.float32), "dw1": (dgud.T @ xe).astype(np.float32),
            "rows": rows, "dyp": dyp, "dgu": dgu, "dxp": dxp}
