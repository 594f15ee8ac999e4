"""GPU parity of the MXFP4 path (OCP E2M1 elements packed two per byte, E8M0
scales per 32; bf16 output), through the C ABI.

The quantiser is compared bit for bit with the oracle's, and so are the
routing tables and the permuted rows.  h (requantised to MXFP4 in the SwiGLU
epilogue) is compared code by code: an E2M1 step is up to half an element, so
a normwise bar would say nothing.  Scales and codes must be equal except where
the kernel's float32 and the oracle's float64 put a value on opposite sides of
an E2M1 rounding boundary.  That flips one code to its neighbour (same sign,
magnitude codes one apart), and it may happen for at most 0.1 % of the codes.
Yp is compared with the oracle's down projection of the GPU's own h, at the
bf16 bars (helpers.assert_parity), which tests the down GEMM exactly.  y is
compared end to end with the oracle's forward (kind "e2m1_out": one E2M1 step
in one term of a sum of F >= 512 terms)."""
import dataclasses

import numpy as np
import pytest
import torch

import routing_permute_grouped_router_amd as moe
from oracle import oracle as orc
from routing_permute_grouped_router_amd import workload as wl

from helpers import assert_parity, cfg_of, decode, rel_err, to_dev, to_host

pytestmark = pytest.mark.gpu
SHAPES = {s.name: s for s in wl.mxfp4_shapes()}


def _gpu_quantize(x_f32: np.ndarray, out=None):
    t = to_dev(x_f32, "f32")
    codes = torch.empty(t.shape[:-1] + (t.shape[-1] // 2,), dtype=torch.uint8, device="cuda")
    scales = torch.empty(t.shape[:-1] + (t.shape[-1] // 32,), dtype=torch.uint8, device="cuda")
    moe.moe_quantize_mxfp4(t, codes, scales)
    return codes, scales


def _codes(packed):
    p = np.asarray(packed, np.uint8)
    return np.stack([p & 0xF, p >> 4], axis=-1).reshape(p.shape[:-1] + (2 * p.shape[-1],))


def check_h(h, hs, h_ref, hs_ref, label="h", max_flip=1e-3):
    """Codes and scales of h against the oracle's: equal, except one-step
    rounding flips in blocks of equal scale (at most max_flip of the codes)
    and blocks whose scale differs (at most 0.5 % of them: the block's amax
    straddles a power of two between the two evaluations)."""
    same = hs == hs_ref
    assert np.mean(same) >= 0.995, f"{label}: {np.mean(~same):.4%} of the scales differ"
    cg, cr = _codes(h), _codes(h_ref)
    blk = np.repeat(same, 32, axis=-1)
    diff = (cg != cr) & blk
    frac = float(np.mean(diff))
    print(f"{label}: {int(diff.sum())} of {diff.size} codes one step apart ({frac:.2e}), "
          f"{int((~same).sum())} of {same.size} scales differ")
    assert frac <= max_flip, f"{label}: {frac:.3%} of the codes differ"
    g, r = cg[diff].astype(np.int32), cr[diff].astype(np.int32)
    assert np.all((g & 8) == (r & 8)) and np.all(np.abs((g & 7) - (r & 7)) == 1), \
        f"{label}: a differing code is not a neighbour of the oracle's"


def test_quantize_matches_oracle_bitwise():
    rng = np.random.default_rng(31)
    rows, cols = 300, 512
    v = rng.standard_normal((rows, cols)) * 2.0 ** rng.integers(-30, 30, (rows, 1))
    v[3] = 0.0                            # all-zero blocks
    v[4, :32] = 6.0 * 2.0 ** -5           # exact block maximum
    v[5, :32] = 7.99                      # saturating element after scaling
    v[6] = rng.standard_normal(cols) * 1e-38   # float32 subnormal range
    v[7, ::2] = -0.0
    v[8] = np.resize([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0], cols) * 2.0 ** 3  # midpoints
    v[8, 0] = 6.0 * 2.0 ** 3
    v[9, :32] = -0.1                      # block maximum 4 (scale 2^0): -0.1 rounds to -0 (code 8)
    v[9, 1] = 4.0
    v = v.astype(np.float32)
    codes, scales = _gpu_quantize(v)
    c_o, s_o = orc.mx_quantize(v, "mxfp4")
    assert np.array_equal(to_host(scales), s_o)
    assert np.array_equal(to_host(codes), c_o)


def _forward(s, x_f32, w1_f32, w2_f32, logits, training=False, gather=False, **cfg_kw):
    cfg = dataclasses.replace(cfg_of(s), **cfg_kw)
    xq, xs = _gpu_quantize(x_f32)
    w1q, w1s = _gpu_quantize(w1_f32)
    w2q, w2s = _gpu_quantize(w2_f32)
    buf = moe.alloc_forward(cfg, training=training)
    buf["y"].fill_(float("nan"))
    buf["h"].fill_(0xEE)
    if gather:
        buf = dict(buf, xp=None, xp_scale=None)
    moe.moe_forward(cfg, to_dev(logits, "f32"), xq, w1q, w2q, buf, x_scale=xs, w1_scale=w1s, w2_scale=w2s)
    torch.cuda.synchronize()
    return buf, (xq, xs, w2q, w2s)


def _experts_of_rows(offsets, rows):
    return np.searchsorted(offsets, rows, side="right") - 1


@pytest.mark.parametrize("name", list(SHAPES))
def test_forward_mxfp4_small_full_parity(name):
    s = SHAPES[name]
    w = wl.Workload(s)
    x, w1, w2, lg = w.x(), w.w1(), w.w2(), w.logits()
    buf, (xq, xs, w2q, w2s) = _forward(s, x, w1, w2, lg, training=True)
    xq_o, xs_o = orc.mx_quantize(x, "mxfp4")
    w1q_o, w1s_o = orc.mx_quantize(w1, "mxfp4")
    w2q_o, w2s_o = orc.mx_quantize(w2, "mxfp4")
    assert np.array_equal(to_host(xq), xq_o) and np.array_equal(to_host(xs), xs_o)
    assert np.array_equal(to_host(w2q), w2q_o) and np.array_equal(to_host(w2s), w2s_o)
    idx, wt = orc.route(lg, s.k, s.score, s.renorm)
    assert np.array_equal(to_host(buf["idx"]), idx)
    counts, offsets, row_map, src_map, _ = orc.group(idx, s.E, s.align)
    assert np.array_equal(to_host(buf["offsets"]), offsets)
    assert np.array_equal(to_host(buf["row_map"]), row_map)
    assert np.array_equal(to_host(buf["src_map"]), src_map)
    n = int(offsets[-1])
    assert np.array_equal(to_host(buf["xp"])[:n], orc.permute(xq_o, row_map, n))
    assert np.array_equal(to_host(buf["xp_scale"])[:n], orc.permute(xs_o, row_map, n))
    ref = orc.forward_tokens(s, np.arange(s.T), xq_o, w1q_o, w2q_o, idx, wt, xs_o, w1s_o, w2s_o, want_stash=True)
    rm = row_map.ravel()
    live = rm >= 0
    rm = rm[live]
    st = decode("bf16", to_host(buf["gu_stash"])[rm])
    assert_parity(st, decode("bf16", ref["stash"].reshape(-1, 2 * s.F)[live]), "bf16", "stash")
    h, hs = to_host(buf["h"])[rm], to_host(buf["h_scale"])[rm]
    check_h(h, hs, ref["h"].reshape(-1, s.F // 2)[live], ref["h_scale"].reshape(-1, s.F // 32)[live])
    # the down GEMM on the GPU's own h: the oracle's projection of those bytes
    yp_ref = orc.down_projection(s, _experts_of_rows(offsets, rm), h, hs, w2q_o, w2s_o)
    assert_parity(decode("bf16", to_host(buf["yp"])[rm]), decode("bf16", yp_ref), "bf16", "Yp")
    # the combine of the GPU's Yp, and y end to end
    y_of_yp = orc.combine(to_host(buf["yp"]), row_map, wt, "bf16")
    assert_parity(decode("bf16", to_host(buf["y"])), decode("bf16", y_of_yp), "bf16", "y (combine)")
    assert_parity(decode("bf16", to_host(buf["y"])), decode("bf16", ref["y"]), "e2m1_out", "y")
    pad = src_map[:n] < 0
    if s.align > 1:
        assert pad.any(), "the alignment should leave padding rows"
        assert not to_host(buf["xp"])[:n][pad].any() and not to_host(buf["xp_scale"])[:n][pad].any()
    if s.zipf_bias:
        assert (counts == 0).any(), "the skewed routing should leave some experts empty"


@pytest.mark.parametrize("name", ["small_mxfp4", "small_mxfp4_skew_align", "small_mxfp4_align128"])
def test_gather_form_equals_materialised(name):
    """moe_forward with xp NULL (the gate/up GEMM reads x through src_map)
    gives the same bytes as the materialised form; padding rows of h are zero
    codes with zero scales."""
    s = SHAPES[name]
    w = wl.Workload(s)
    x, w1, w2, lg = w.x(), w.w1(), w.w2(), w.logits()
    a, _ = _forward(s, x, w1, w2, lg)
    b, _ = _forward(s, x, w1, w2, lg, gather=True)
    n = int(to_host(a["offsets"])[-1])
    for key in ("h", "h_scale", "yp"):
        assert np.array_equal(to_host(a[key])[:n].view(np.uint8), to_host(b[key])[:n].view(np.uint8)), key
    assert np.array_equal(to_host(a["y"]).view(np.uint16), to_host(b["y"]).view(np.uint16))
    pad = to_host(b["src_map"])[:n] < 0
    assert not to_host(b["h"])[:n][pad].any() and not to_host(b["h_scale"])[:n][pad].any()


@pytest.mark.parametrize("site,limit", [("fc1", 0.0), ("fc2", 0.0), ("combine", 0.75)])
def test_weight_sites_and_clamp(site, limit):
    """The routing weight in the FC1 or FC2 epilogue, and the SwiGLU clamp,
    on MXFP4 storage against the oracle's placements."""
    s = SHAPES["small_mxfp4_k1024"]
    w = wl.Workload(s)
    x, w1, w2, lg = w.x(), w.w1(), w.w2(), w.logits()
    buf, _ = _forward(s, x, w1, w2, lg, weight_site=site, swiglu_limit=limit)
    xq_o, xs_o = orc.mx_quantize(x, "mxfp4")
    w1q_o, w1s_o = orc.mx_quantize(w1, "mxfp4")
    w2q_o, w2s_o = orc.mx_quantize(w2, "mxfp4")
    idx, wt = orc.route(lg, s.k, s.score, s.renorm)
    counts, offsets, row_map, src_map, _ = orc.group(idx, s.E, s.align)
    ref = orc.forward_tokens(s, np.arange(s.T), xq_o, w1q_o, w2q_o, idx, wt, xs_o, w1s_o, w2s_o, site=site,
                             limit=limit)
    rm = row_map.ravel()
    h, hs = to_host(buf["h"])[rm], to_host(buf["h_scale"])[rm]
    check_h(h, hs, ref["h"].reshape(-1, s.F // 2), ref["h_scale"].reshape(-1, s.F // 32))
    yp_ref = orc.down_projection(s, _experts_of_rows(offsets, rm), h, hs, w2q_o, w2s_o,
                                 row_w=wt.ravel() if site == "fc2" else None)
    assert_parity(decode("bf16", to_host(buf["yp"])[rm]), decode("bf16", yp_ref), "bf16", "Yp")
    assert_parity(decode("bf16", to_host(buf["y"])), decode("bf16", ref["y"]), "e2m1_out", "y")


def test_forward_mxfp4_full_size():
    """DeepSeek-V3-shaped layer on MXFP4 storage (T=8192, H=7168, F=2048,
    E=256, top-8 sigmoid): weights streamed expert by expert (the GPU
    quantises its copy, the oracle its own: compared byte for byte), integer
    outputs in full, and h, Yp and y of 1024 seeded tokens."""
    s = wl.BY_NAME["deepseek_mxfp4"]
    w = wl.Workload(s)
    cfg = cfg_of(s)
    lg = w.logits()
    x = w.x()
    xq, xs = _gpu_quantize(x)
    xq_o, xs_o = orc.mx_quantize(x, "mxfp4")
    assert np.array_equal(to_host(xq), xq_o) and np.array_equal(to_host(xs), xs_o)
    idx, wt = orc.route(lg, s.k, s.score, s.renorm)
    rng = np.random.default_rng(s.seed + 6)
    toks = np.sort(rng.choice(s.T, 1024, replace=False)).astype(np.int32)
    need = set(np.unique(idx[toks]).tolist())
    dev = torch.device("cuda")
    w1q = torch.empty(s.E, 2 * s.F, s.H // 2, dtype=torch.uint8, device=dev)
    w1s = torch.empty(s.E, 2 * s.F, s.H // 32, dtype=torch.uint8, device=dev)
    w2q = torch.empty(s.E, s.H, s.F // 2, dtype=torch.uint8, device=dev)
    w2s = torch.empty(s.E, s.H, s.F // 32, dtype=torch.uint8, device=dev)
    w1q_o = np.zeros((s.E, 2 * s.F, s.H // 2), np.uint8)
    w1s_o = np.zeros((s.E, 2 * s.F, s.H // 32), np.uint8)
    w2q_o = np.zeros((s.E, s.H, s.F // 2), np.uint8)
    w2s_o = np.zeros((s.E, s.H, s.F // 32), np.uint8)
    step = 16
    for e0 in range(0, s.E, step):
        a1, a2 = w.w1(e0, e0 + step), w.w2(e0, e0 + step)
        t1, t2 = to_dev(a1, "f32"), to_dev(a2, "f32")
        moe.moe_quantize_mxfp4(t1, w1q[e0:e0 + step], w1s[e0:e0 + step])
        moe.moe_quantize_mxfp4(t2, w2q[e0:e0 + step], w2s[e0:e0 + step])
        del t1, t2
        for e in range(e0, e0 + step):
            if e in need or e == e0:
                w1q_o[e], w1s_o[e] = orc.mx_quantize(a1[e - e0], "mxfp4")
                w2q_o[e], w2s_o[e] = orc.mx_quantize(a2[e - e0], "mxfp4")
                if e == e0:
                    assert np.array_equal(to_host(w1q[e]), w1q_o[e]) and np.array_equal(to_host(w1s[e]), w1s_o[e])
                    assert np.array_equal(to_host(w2q[e]), w2q_o[e]) and np.array_equal(to_host(w2s[e]), w2s_o[e])
    buf = moe.alloc_forward(cfg)
    moe.moe_forward(cfg, to_dev(lg, "f32"), xq, w1q, w2q, buf, x_scale=xs, w1_scale=w1s, w2_scale=w2s)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(buf["idx"]), idx)
    assert rel_err(to_host(buf["w"]), wt) < 1e-5
    counts, offsets, row_map, src_map, _ = orc.group(idx, s.E, s.align)
    assert np.array_equal(to_host(buf["offsets"]), offsets)
    assert np.array_equal(to_host(buf["row_map"]), row_map)
    assert np.array_equal(to_host(buf["src_map"]), src_map)
    ref = orc.forward_experts(s, toks, xq_o, w1q_o, w2q_o, idx, wt, xs_o, w1s_o, w2s_o)
    rows_np = row_map[toks].ravel()
    rows = torch.from_numpy(rows_np).long().cuda()
    h, hs = to_host(buf["h"][rows]), to_host(buf["h_scale"][rows])
    check_h(h, hs, ref["h"].reshape(-1, s.F // 2), ref["h_scale"].reshape(-1, s.F // 32))
    yp_ref = orc.down_projection(s, _experts_of_rows(offsets, rows_np), h, hs, w2q_o, w2s_o)
    assert_parity(decode("bf16", to_host(buf["yp"][rows])), decode("bf16", yp_ref), "bf16", "Yp")
    assert_parity(decode("bf16", to_host(buf["y"])[toks]), decode("bf16", ref["y"]), "e2m1_out", "y")


def test_forward_graph_capture_replays():
    """The MXFP4 forward captures into a HIP graph; replays, with eager work
    between them and the outputs overwritten before each, give the eager
    bytes."""
    s = SHAPES["small_mxfp4_skew_align"]
    w = wl.Workload(s)
    cfg = cfg_of(s)
    (xq, xs), (w1q, w1s), (w2q, w2s) = _gpu_quantize(w.x()), _gpu_quantize(w.w1()), _gpu_quantize(w.w2())
    logits = to_dev(w.logits(), "f32")
    sc = dict(x_scale=xs, w1_scale=w1s, w2_scale=w2s)
    buf = moe.alloc_forward(cfg)
    moe.moe_forward(cfg, logits, xq, w1q, w2q, buf, **sc)
    torch.cuda.synchronize()
    keys = [k for k, v in buf.items() if v is not None and k not in ("ws", "err")]
    eager = {k: to_host(buf[k]).copy() for k in keys}
    n = int(eager["offsets"][-1])
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            moe.moe_forward(cfg, logits, xq, w1q, w2q, buf, **sc)
    for rep in range(3):
        buf["y"].fill_(float("nan"))
        buf["yp"].fill_(float("nan"))
        buf["h"].fill_(0x5A)
        buf["xp"].fill_(0xA5)
        g.replay()
        torch.cuda.synchronize()
        _ = (logits * 2).sum().item()  # unrelated eager work between replays
        for k in keys:
            got, v = to_host(buf[k]), eager[k]
            if k in ("xp", "xp_scale", "h", "h_scale", "yp", "src_map"):
                got, v = got[:n], v[:n]
            assert np.array_equal(got.view(np.uint8), v.view(np.uint8)), f"replay {rep}: {k} differs"
