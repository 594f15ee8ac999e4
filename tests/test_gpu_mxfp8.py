"""GPU parity of the MXFP8 path (OCP E4M3 elements, E8M0 scales per 32).

The quantiser is compared bit for bit with the oracle's; the forward (inputs
quantised by the GPU, h requantised in the SwiGLU epilogue, bf16 output) within
the MXFP8 tolerance 6e-2 of the normwise relative error and, element by
element, within one E4M3 step for h (helpers.ELEM_BOUNDS) for 99.9 % of the
elements.  The DeepSeek-shaped layer is compared on 1024 seeded tokens."""
import numpy as np
import pytest
import torch

import routing_permute_grouped_router_amd as moe
from oracle import oracle as orc
from routing_permute_grouped_router_amd import workload as wl

from helpers import TOL, assert_parity, cfg_of, decode, rel_err, to_dev, to_host

pytestmark = pytest.mark.gpu


def _gpu_quantize(x_f32: np.ndarray):
    t = to_dev(x_f32, "f32")
    codes = torch.empty(t.shape, dtype=torch.uint8, device="cuda")
    scales = torch.empty(t.shape[:-1] + (t.shape[-1] // 32,), dtype=torch.uint8, device="cuda")
    moe.moe_quantize_mxfp8(t, codes, scales)
    return codes, scales


def test_quantize_matches_oracle_bitwise():
    rng = np.random.default_rng(21)
    rows, cols = 300, 512
    v = rng.standard_normal((rows, cols)) * 2.0 ** rng.integers(-30, 30, (rows, 1))
    v[3] = 0.0                          # all-zero blocks
    v[4, :32] = 448.0 * 2.0 ** -5       # exact block maximum
    v[5, :32] = 1.99                    # saturating element after scaling
    v[6] = rng.standard_normal(cols) * 1e-38   # float32 subnormal range
    v[7, ::2] = -0.0
    v = v.astype(np.float32)
    codes, scales = _gpu_quantize(v)
    c_o, s_o = orc.mx_quantize(v)
    assert np.array_equal(to_host(scales), s_o)
    assert np.array_equal(to_host(codes), c_o)


def _forward_mx(s, x_f32, w1_f32, w2_f32, logits, training=False):
    cfg = cfg_of(s)
    xq, xs = _gpu_quantize(x_f32)
    w1q, w1s = _gpu_quantize(w1_f32)
    w2q, w2s = _gpu_quantize(w2_f32)
    buf = moe.alloc_forward(cfg, training=training)
    buf["y"].fill_(float("nan"))
    if training:
        buf["gu_stash"].fill_(float("nan"))
    moe.moe_forward(cfg, to_dev(logits, "f32"), xq, w1q, w2q, buf, x_scale=xs, w1_scale=w1s, w2_scale=w2s)
    torch.cuda.synchronize()
    return buf, (xq, xs)


@pytest.mark.parametrize("name", ["small_mxfp8", "small_mxfp8_k512", "small_mxfp8_skew_align", "small_mxfp8_align128"])
def test_forward_mxfp8_small_full_parity(name):
    """Every output of a small MXFP8 layer in full: K = 256 / 128 (one
    scale word per stage), K = 512 (scale words of four stages per load), and
    skewed routing with 16-row groups (empty experts, zero padding rows)."""
    s = [x for x in wl.small_shapes() if x.name == name][0]
    w = wl.Workload(s)
    x, w1, w2, lg = w.x(), w.w1(), w.w2(), w.logits()
    buf, (xq, xs) = _forward_mx(s, x, w1, w2, lg, training=True)
    xq_o, xs_o = orc.mx_quantize(x)
    w1q_o, w1s_o = orc.mx_quantize(w1)
    w2q_o, w2s_o = orc.mx_quantize(w2)
    assert np.array_equal(to_host(xq), xq_o) and np.array_equal(to_host(xs), xs_o)
    idx, wt = orc.route(lg, s.k, s.score, s.renorm)
    assert np.array_equal(to_host(buf["idx"]), idx)
    counts, offsets, row_map, src_map, _ = orc.group(idx, s.E, s.align)
    assert np.array_equal(to_host(buf["row_map"]), row_map)
    n = int(offsets[-1])
    assert np.array_equal(to_host(buf["xp"])[:n], orc.permute(xq_o, row_map, n))
    assert np.array_equal(to_host(buf["xp_scale"])[:n], orc.permute(xs_o, row_map, n))
    ref = orc.forward_tokens(s, np.arange(s.T), xq_o, w1q_o, w2q_o, idx, wt, xs_o, w1s_o, w2s_o, want_stash=True)
    rm = row_map.ravel()
    # the optional bf16 g | u stash of the SwiGLU GEMM
    st = decode("bf16", to_host(buf["gu_stash"])[rm])
    assert_parity(st, decode("bf16", ref["stash"].reshape(-1, 2 * s.F)), "bf16", "stash")
    h = orc.mx_dequantize(to_host(buf["h"])[rm], to_host(buf["h_scale"])[rm])
    h_ref = orc.mx_dequantize(ref["h"].reshape(-1, s.F), ref["h_scale"].reshape(-1, s.F // 32))
    assert_parity(h, h_ref, "e4m3", "h")
    assert_parity(decode("bf16", to_host(buf["yp"])[rm]), decode("bf16", ref["yp"].reshape(-1, s.H)), "e4m3_out", "Yp")
    assert_parity(decode("bf16", to_host(buf["y"])), decode("bf16", ref["y"]), "e4m3_out", "y")
    if s.align > 1:  # padding rows of Xp are zero codes with zero scales
        pad = src_map[:n] < 0
        assert pad.any(), "the alignment should leave padding rows"
        assert not to_host(buf["xp"])[:n][pad].any() and not to_host(buf["xp_scale"])[:n][pad].any()
    if s.zipf_bias:
        assert (counts == 0).any(), "the skewed routing should leave some experts empty"


def test_forward_mxfp8_full_size():
    """DeepSeek-V3-shaped layer (T=8192, H=7168, F=2048, E=256, top-8 sigmoid):
    weights streamed expert by expert (GPU quantises its copy, the oracle its
    own, compared byte for byte), all integer outputs compared in full, and h,
    Yp and y of 1024 seeded tokens against the oracle's expert-major form."""
    s = wl.BY_NAME["deepseek_mxfp8"]
    w = wl.Workload(s)
    cfg = cfg_of(s)
    lg = w.logits()
    x = w.x()
    xq, xs = _gpu_quantize(x)
    xq_o, xs_o = orc.mx_quantize(x)
    assert np.array_equal(to_host(xq), xq_o) and np.array_equal(to_host(xs), xs_o)
    idx, wt = orc.route(lg, s.k, s.score, s.renorm)
    rng = np.random.default_rng(s.seed + 6)
    toks = np.sort(rng.choice(s.T, 1024, replace=False)).astype(np.int32)
    need = set(np.unique(idx[toks]).tolist())
    dev = torch.device("cuda")
    w1q = torch.empty(s.E, 2 * s.F, s.H, dtype=torch.uint8, device=dev)
    w1s = torch.empty(s.E, 2 * s.F, s.H // 32, dtype=torch.uint8, device=dev)
    w2q = torch.empty(s.E, s.H, s.F, dtype=torch.uint8, device=dev)
    w2s = torch.empty(s.E, s.H, s.F // 32, dtype=torch.uint8, device=dev)
    # the oracle keeps its own quantised copy of the experts the sample uses
    w1q_o = np.zeros((s.E, 2 * s.F, s.H), np.uint8)
    w1s_o = np.zeros((s.E, 2 * s.F, s.H // 32), np.uint8)
    w2q_o = np.zeros((s.E, s.H, s.F), np.uint8)
    w2s_o = np.zeros((s.E, s.H, s.F // 32), np.uint8)
    step = 16
    for e0 in range(0, s.E, step):
        a1, a2 = w.w1(e0, e0 + step), w.w2(e0, e0 + step)
        t1, t2 = to_dev(a1, "f32"), to_dev(a2, "f32")
        moe.moe_quantize_mxfp8(t1, w1q[e0:e0 + step], w1s[e0:e0 + step])
        moe.moe_quantize_mxfp8(t2, w2q[e0:e0 + step], w2s[e0:e0 + step])
        del t1, t2
        for e in range(e0, e0 + step):
            if e in need or e == e0:
                w1q_o[e], w1s_o[e] = orc.mx_quantize(a1[e - e0])
                w2q_o[e], w2s_o[e] = orc.mx_quantize(a2[e - e0])
                if e == e0:  # GPU and oracle quantisers agree byte for byte on real weights
                    assert np.array_equal(to_host(w1q[e]), w1q_o[e]) and np.array_equal(to_host(w1s[e]), w1s_o[e])
                    assert np.array_equal(to_host(w2q[e]), w2q_o[e]) and np.array_equal(to_host(w2s[e]), w2s_o[e])
    buf = moe.alloc_forward(cfg)
    moe.moe_forward(cfg, to_dev(lg, "f32"), xq, w1q, w2q, buf, x_scale=xs, w1_scale=w1s, w2_scale=w2s)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(buf["idx"]), idx)
    assert rel_err(to_host(buf["w"]), wt) < 1e-5
    counts, offsets, row_map, src_map, _ = orc.group(idx, s.E, s.align)
    assert np.array_equal(to_host(buf["counts"]), counts)
    assert np.array_equal(to_host(buf["offsets"]), offsets)
    assert np.array_equal(to_host(buf["row_map"]), row_map)
    assert np.array_equal(to_host(buf["src_map"]), src_map)
    ref = orc.forward_experts(s, toks, xq_o, w1q_o, w2q_o, idx, wt, xs_o, w1s_o, w2s_o)
    rows = torch.from_numpy(row_map[toks].ravel()).long().cuda()
    h = orc.mx_dequantize(to_host(buf["h"][rows]), to_host(buf["h_scale"][rows]))
    h_ref = orc.mx_dequantize(ref["h"].reshape(-1, s.F), ref["h_scale"].reshape(-1, s.F // 32))
    assert_parity(h, h_ref, "e4m3", "h")
    assert_parity(decode("bf16", to_host(buf["yp"][rows])), decode("bf16", ref["yp"].reshape(-1, s.H)), "e4m3_out",
                  "Yp")
    assert_parity(decode("bf16", to_host(buf["y"])[toks]), decode("bf16", ref["y"]), "e4m3_out", "y")
