"""Pins of the oracle's expert FFN (gate/up projection, SwiGLU, down
projection), combine and backward.

References: a hand-worked example (tests/golden/tiny_swiglu_moe.json), torch's
F.linear / F.silu in float64 (library routines) evaluated token by token,
torch autograd in float64 for the backward, closed forms (identical experts,
E = 1), and exact power-of-two scaling."""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as tF

from oracle import oracle as orc
from routing_permute_grouped_router_amd.workload import MoEShape

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_swiglu_moe.json")


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _torch_moe(x, w1, w2, idx, w, F):
    """Token-by-token float64 evaluation with torch's linear and silu."""
    x = torch.from_numpy(x)
    y = torch.zeros_like(x)
    T, k = idx.shape
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if e < 0:
                continue
            gu = tF.linear(x[t], torch.from_numpy(w1[e]))
            hh = tF.silu(gu[:F]) * gu[F:]
            y[t] += float(w[t, j]) * tF.linear(hh, torch.from_numpy(w2[e]))
    return y.numpy()


def test_golden_hand_worked_example():
    g = json.load(open(GOLDEN))
    s = MoEShape("golden", g["T"], g["H"], g["F"], g["E"], g["k"], g["score"], g["renorm"], "f32")
    x = np.array(g["x"], np.float32)
    w1 = np.array(g["w1"], np.float32)
    w2 = np.array(g["w2"], np.float32)
    idx, w = orc.route(np.array(g["logits"], np.float32), s.k, s.score, s.renorm)
    ex = g["expected"]
    assert np.array_equal(idx, np.array(ex["idx"], np.int32))
    np.testing.assert_allclose(w, ex["w"], rtol=1e-7)
    out = orc.forward_tokens(s, np.arange(s.T), x, w1, w2, idx, w)
    np.testing.assert_allclose(out["h"], ex["h"], rtol=1e-6)
    np.testing.assert_allclose(out["yp"], ex["yp"], rtol=1e-6)
    np.testing.assert_allclose(out["y"], ex["y"], rtol=1e-6)


def _rand_problem(T, H, F, E, k, seed, fmt="f32", renorm=True, score="softmax", uniform_expert=None):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    w1 = rng.standard_normal((E, 2 * F, H)) / np.sqrt(H)
    w2 = rng.standard_normal((E, H, F)) / np.sqrt(F)
    if uniform_expert is not None:
        w1[:] = w1[uniform_expert]
        w2[:] = w2[uniform_expert]
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if fmt == "f32":
        cast = lambda a: a.astype(np.float32)
    else:
        cast = orc.bf16_from_f64
    s = MoEShape("rand", T, H, F, E, k, score, renorm, fmt)
    return s, cast(x), cast(w1), cast(w2), lg


def test_ffn_matches_torch_token_by_token():
    s, x, w1, w2, lg = _rand_problem(37, 64, 96, 6, 3, 1, renorm=False)
    idx, w = orc.route(lg, s.k, s.score, s.renorm)
    out = orc.forward_tokens(s, np.arange(s.T), x, w1, w2, idx, w)
    ref = _torch_moe(x.astype(np.float64), w1.astype(np.float64), w2.astype(np.float64), idx, w, s.F)
    assert _rel(out["y"], ref) < 1e-6


def test_identical_experts_reduce_to_dense_swiglu_mlp():
    s, x, w1, w2, lg = _rand_problem(40, 64, 32, 8, 4, 2, renorm=True, uniform_expert=3)
    idx, w = orc.route(lg, s.k, s.score, s.renorm)
    out = orc.forward_tokens(s, np.arange(s.T), x, w1, w2, idx, w)
    xt = torch.from_numpy(x.astype(np.float64))
    gu = tF.linear(xt, torch.from_numpy(w1[0].astype(np.float64)))
    dense = tF.linear(tF.silu(gu[:, : s.F]) * gu[:, s.F:], torch.from_numpy(w2[0].astype(np.float64))).numpy()
    assert _rel(out["y"], dense) < 1e-6


def test_single_expert_top1_is_dense_mlp():
    s, x, w1, w2, lg = _rand_problem(20, 32, 64, 1, 1, 3, renorm=False)
    idx, w = orc.route(lg, 1)
    assert np.all(idx == 0) and np.all(w == 1.0)
    out = orc.forward_tokens(s, np.arange(s.T), x, w1, w2, idx, w)
    xt = torch.from_numpy(x.astype(np.float64))
    gu = tF.linear(xt, torch.from_numpy(w1[0].astype(np.float64)))
    dense = tF.linear(tF.silu(gu[:, : s.F]) * gu[:, s.F:], torch.from_numpy(w2[0].astype(np.float64))).numpy()
    assert _rel(out["y"], dense) < 1e-6


def test_power_of_two_scaling_of_down_weights_is_exact():
    s, x, w1, w2, lg = _rand_problem(30, 64, 64, 4, 2, 4, fmt="bf16")
    idx, w = orc.route(lg, s.k, s.score, s.renorm)
    a = orc.forward_tokens(s, np.arange(s.T), x, w1, w2, idx, w)
    w2x4 = orc.bf16_from_f64(4.0 * orc.f64_from_bf16(w2))
    b = orc.forward_tokens(s, np.arange(s.T), x, w1, w2x4, idx, w)
    assert np.array_equal(a["h"], b["h"])
    assert np.array_equal(orc.f64_from_bf16(b["y"]), 4.0 * orc.f64_from_bf16(a["y"]))


def test_bf16_storage_points():
    """h and Yp are rounded to bf16 once, from the float64 sums."""
    s, x, w1, w2, lg = _rand_problem(16, 64, 32, 4, 2, 5, fmt="bf16")
    idx, w = orc.route(lg, s.k, s.score, s.renorm)
    out = orc.forward_tokens(s, np.arange(s.T), x, w1, w2, idx, w, want_stash=True)
    xd, w1d, w2d = (orc.f64_from_bf16(a) for a in (x, w1, w2))
    for t in range(s.T):
        for j in range(s.k):
            e = idx[t, j]
            gu = w1d[e] @ xd[t]
            hh = tF.silu(torch.from_numpy(gu[: s.F])).numpy() * gu[s.F:]
            hb = orc.f64_from_bf16(out["h"][t, j])
            assert _rel(hb, hh) < 2 ** -8 * 1.01
            assert np.max(np.abs(orc.f64_from_bf16(out["stash"][t, j]) - gu) / np.maximum(np.abs(gu), 1e-30)) <= 2 ** -8
            yp = w2d[e] @ hb
            assert _rel(orc.f64_from_bf16(out["yp"][t, j]), yp) < 2 ** -8 * 1.01


def test_mxfp8_forward_within_quantisation_error():
    rng = np.random.default_rng(6)
    T, H, F, E, k = 24, 64, 64, 4, 2
    x = rng.standard_normal((T, H)).astype(np.float32)
    w1 = (rng.standard_normal((E, 2 * F, H)) / 8).astype(np.float32)
    w2 = (rng.standard_normal((E, H, F)) / 8).astype(np.float32)
    xq, xs = orc.mx_quantize(x)
    w1q, w1s = orc.mx_quantize(w1)
    w2q, w2s = orc.mx_quantize(w2)
    s = MoEShape("mx", T, H, F, E, k, "sigmoid", True, "mxfp8")
    idx, w = orc.route(rng.standard_normal((T, E)).astype(np.float32), k, "sigmoid", True)
    out = orc.forward_tokens(s, np.arange(T), xq, w1q, w2q, idx, w, xs, w1s, w2s)
    ref = _torch_moe(orc.mx_dequantize(xq, xs), orc.mx_dequantize(w1q, w1s), orc.mx_dequantize(w2q, w2s), idx, w, F)
    # differs from the unquantised-h reference only by h's MX rounding and bf16 stores
    assert _rel(orc.f64_from_bf16(out["y"]), ref) < 6e-2
    # the stored h decodes to the MX grid: re-quantising is the identity
    hd = orc.mx_dequantize(out["h"], out["h_scale"])
    hq2, hs2 = orc.mx_quantize(hd.astype(np.float32))
    assert np.array_equal(orc.mx_dequantize(hq2, hs2), hd)


def test_dropped_route_contributes_nothing():
    s, x, w1, w2, lg = _rand_problem(10, 32, 32, 4, 2, 7)
    idx, w = orc.route(lg, s.k, s.score, s.renorm)
    idx2 = idx.copy()
    idx2[:, 1] = -1
    a = orc.forward_tokens(s, np.arange(s.T), x, w1, w2, idx2, w)
    s1 = s.replace(k=1)
    b = orc.forward_tokens(s1, np.arange(s.T), x, w1, w2, np.ascontiguousarray(idx[:, :1]),
                           np.ascontiguousarray(w[:, :1]))
    assert np.array_equal(a["y"], b["y"])


# ---------------------------------------------------------------- backward
def _forward_rows(s, x, w1, w2, idx, w, align=1):
    counts, offsets, row_map, src_map, _ = orc.group(idx, s.E, align)
    out = orc.forward_tokens(s, np.arange(s.T), x, w1, w2, idx, w, want_stash=True)
    R_cap = src_map.shape[0]
    h_rows = np.zeros((R_cap, s.F), out["h"].dtype)
    st_rows = np.zeros((R_cap, 2 * s.F), out["stash"].dtype)
    for i, r in enumerate(row_map.ravel()):
        if r >= 0:
            h_rows[r] = out["h"].reshape(-1, s.F)[i]
            st_rows[r] = out["stash"].reshape(-1, 2 * s.F)[i]
    return counts, offsets, row_map, src_map, h_rows, st_rows, out


def test_backward_matches_torch_autograd():
    T, H, F, E, k = 29, 32, 48, 6, 2
    s, x, w1, w2, lg = _rand_problem(T, H, F, E, k, 8)
    lg[:, 5] = -50.0  # expert 5 never selected: its weight gradients must be exactly zero
    idx, w = orc.route(lg, k, s.score, s.renorm)
    counts, offsets, row_map, src_map, h_rows, st_rows, _ = _forward_rows(s, x, w1, w2, idx, w, align=4)
    assert counts[5] == 0
    dy = np.random.default_rng(9).standard_normal((T, H)).astype(np.float32)
    g = orc.backward(s, x, w1, w2, w, row_map, src_map, offsets, h_rows, st_rows, dy)
    xt = torch.from_numpy(x.astype(np.float64)).requires_grad_(True)
    w1t = torch.from_numpy(w1.astype(np.float64)).requires_grad_(True)
    w2t = torch.from_numpy(w2.astype(np.float64)).requires_grad_(True)
    y = torch.zeros(T, H, dtype=torch.float64)
    rows = []
    for t in range(T):
        acc = torch.zeros(H, dtype=torch.float64)
        for j in range(k):
            e = int(idx[t, j])
            gu = tF.linear(xt[t], w1t[e])
            acc = acc + float(w[t, j]) * tF.linear(tF.silu(gu[:F]) * gu[F:], w2t[e])
        rows.append(acc)
    y = torch.stack(rows)
    (y * torch.from_numpy(dy.astype(np.float64))).sum().backward()
    assert _rel(g["dx"], xt.grad.numpy()) < 1e-5
    assert _rel(g["dw1"], w1t.grad.numpy()) < 1e-5
    assert _rel(g["dw2"], w2t.grad.numpy()) < 1e-5
    assert np.all(g["dw1"][5] == 0) and np.all(g["dw2"][5] == 0)


def test_sampled_backward_helpers_agree_with_full_backward():
    T, H, F, E, k = 33, 64, 32, 5, 2
    s, x, w1, w2, lg = _rand_problem(T, H, F, E, k, 10, fmt="bf16")
    idx, w = orc.route(lg, k, s.score, s.renorm)
    counts, offsets, row_map, src_map, h_rows, st_rows, _ = _forward_rows(s, x, w1, w2, idx, w)
    dy = orc.bf16_from_f64(np.random.default_rng(11).standard_normal((T, H)))
    g = orc.backward(s, x, w1, w2, w, row_map, src_map, offsets, h_rows, st_rows, dy)
    toks = np.array([0, 5, 17, 32])
    dx = orc.backward_dx_tokens(s, toks, x, w1, w2, idx, w, dy)
    assert np.array_equal(dx, g["dx"][toks])
    e = int(np.argmax(counts))
    rng = np.random.default_rng(12)
    i2 = np.stack([rng.integers(0, H, 20), rng.integers(0, F, 20)], 1)
    i1 = np.stack([rng.integers(0, 2 * F, 20), rng.integers(0, H, 20)], 1)
    d2, d1 = orc.backward_dw_entries(s, e, x, w1, w2, w, src_map, offsets, dy, i2, i1)
    np.testing.assert_allclose(d2.astype(np.float32), g["dw2"][e][i2[:, 0], i2[:, 1]], rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(d1.astype(np.float32), g["dw1"][e][i1[:, 0], i1[:, 1]], rtol=1e-6, atol=1e-7)


# ---- the expert-major float64 front end (forward_experts, backward_expert)
# It evaluates the same definitions with the sums over H and F as float64
# matrix products; only the order of the float64 additions differs, which
# moves a stored value only when a sum lies within ~1e-16 of a rounding
# boundary of its storage format.  On these shapes every stored byte agrees.
def _small_mx(T, H, F, E, k, seed):
    rng = np.random.default_rng(seed)
    s = MoEShape("rand_mx", T, H, F, E, k, "sigmoid", True, "mxfp8")
    q = lambda a: orc.mx_quantize(a.astype(np.float32))
    x, xs = q(rng.standard_normal((T, H)))
    w1, w1s = q(rng.standard_normal((E, 2 * F, H)) / np.sqrt(H))
    w2, w2s = q(rng.standard_normal((E, H, F)) / np.sqrt(F))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    return s, (x, xs), (w1, w1s), (w2, w2s), lg


@pytest.mark.parametrize("fmt,site,limit", [("f32", "combine", 0.0), ("bf16", "combine", 0.0),
                                            ("bf16", "fc1", 0.0), ("bf16", "fc2", 0.0), ("bf16", "combine", 0.6)])
def test_expert_major_forward_equals_token_loops(fmt, site, limit):
    s, x, w1, w2, lg = _rand_problem(61, 64, 96, 6, 3, 11, fmt=fmt, renorm=True)
    idx, w = orc.route(lg, s.k, s.score, s.renorm)
    idx[::9, 1] = -1  # dropped routes
    toks = np.arange(s.T)
    a = orc.forward_tokens(s, toks, x, w1, w2, idx, w, want_stash=True, site=site, limit=limit)
    b = orc.forward_experts(s, toks, x, w1, w2, idx, w, want_stash=True, site=site, limit=limit)
    live = idx >= 0
    for key in ("h", "yp", "stash"):
        assert np.array_equal(a[key][live].view(np.uint8), b[key][live].view(np.uint8)), key
    assert np.array_equal(a["y"].view(np.uint8), b["y"].view(np.uint8))
    # a sample of tokens gives the sample's rows of the full evaluation
    sub = np.array([3, 17, 40, 60])
    c = orc.forward_experts(s, sub, x, w1, w2, idx, w, site=site, limit=limit)
    assert np.array_equal(c["y"].view(np.uint8), b["y"][sub].view(np.uint8))


def test_expert_major_forward_equals_token_loops_mxfp8():
    s, (x, xs), (w1, w1s), (w2, w2s), lg = _small_mx(45, 64, 96, 5, 2, 12)
    idx, w = orc.route(lg, s.k, s.score, s.renorm)
    toks = np.arange(s.T)
    a = orc.forward_tokens(s, toks, x, w1, w2, idx, w, xs, w1s, w2s, want_stash=True)
    b = orc.forward_experts(s, toks, x, w1, w2, idx, w, xs, w1s, w2s, want_stash=True)
    for key in ("h", "h_scale", "yp", "stash", "y"):
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), key


@pytest.mark.parametrize("limit", [0.0, 0.7])
def test_expert_major_backward_equals_row_loops(limit):
    s, x, w1, w2, lg = _rand_problem(80, 64, 48, 5, 2, 13, fmt="bf16", renorm=True)
    s = MoEShape("rand_bwd", s.T, s.H, s.F, s.E, s.k, s.score, s.renorm, "bf16", align=4)
    lg[:, 4] -= 50.0  # expert 4 gets no rows
    idx, w = orc.route(lg, s.k, s.score, s.renorm)
    counts, offsets, row_map, src_map, _ = orc.group(idx, s.E, s.align)
    assert counts[4] == 0
    dy = orc.bf16_from_f64(np.random.default_rng(14).standard_normal((s.T, s.H)))
    ref = orc.forward_tokens(s, np.arange(s.T), x, w1, w2, idx, w, want_stash=True, limit=limit)
    R = src_map.shape[0]
    h_rows = np.zeros((R, s.F), np.uint16)
    st_rows = np.zeros((R, 2 * s.F), np.uint16)
    h_rows[row_map.ravel()] = ref["h"].reshape(-1, s.F)
    st_rows[row_map.ravel()] = ref["stash"].reshape(-1, 2 * s.F)
    g = orc.backward(s, x, w1, w2, w, row_map, src_map, offsets, h_rows, st_rows, dy, limit=limit)
    for e in range(s.E):
        b = orc.backward_expert(s, e, x, w1, w2, w, src_map, offsets, dy, limit=limit)
        assert np.array_equal(b["dw1"].view(np.uint32), g["dw1"][e].view(np.uint32)), f"dW1 of expert {e}"
        assert np.array_equal(b["dw2"].view(np.uint32), g["dw2"][e].view(np.uint32)), f"dW2 of expert {e}"
        r = b["rows"]
        if r.size:
            for key in ("dyp", "dgu", "dxp"):
                assert np.array_equal(b[key], g[key][r]), f"{key} of expert {e}"


def _rne_bf16(v):
    """float64 -> the nearest bfloat16 value (8 significant bits, ties to even),
    as float64: frexp splits v = m 2^e with 0.5 <= |m| < 1, and numpy's round
    is half-to-even on m 2^8.  Independent of the oracle's bit-level rounding;
    valid in bf16's normal range, which these values stay in."""
    m, e = np.frexp(np.asarray(v, np.float64))
    return np.ldexp(np.round(m * 256.0) / 256.0, e)


def _ulp_diff_bf16(a_bits, b_f64):
    """Difference in bf16 units between stored bf16 bits and a float64 value
    that is itself a bf16 value (same sign assumed for nonzero pairs)."""
    a = (np.asarray(a_bits, np.uint16).astype(np.int32))
    b = (orc.bf16_from_f64(b_f64).astype(np.int32))
    return np.abs(a - b)


def test_bf16_backward_rounding_points():
    """Every bf16 rounding point of the backward, recomputed with torch float64
    products, torch autograd for the SwiGLU derivative and an independent
    round-to-nearest-even: dYp = bf16(w dY), dH = dYp W2 (not rounded),
    dGU = bf16(dH * dSwiGLU(stash)), dXp = bf16(dGU W1), dX = bf16(sum_j dXp),
    dW2 = f32(dYp^T h) with the rounded dYp and the stored h, dW1 = f32(dGU^T Xp)
    with the rounded dGU.  A misplaced rounding point (dW1 from the unrounded
    dGU, dYp unrounded before the products) moves many values by far more than
    the one bf16 unit, or the float32 rounding, that float64 summation order
    can account for."""
    T, H, F, E, k = 40, 64, 48, 5, 2
    s, x, w1, w2, lg = _rand_problem(T, H, F, E, k, 15, fmt="bf16")
    idx, w = orc.route(lg, k, s.score, s.renorm)
    counts, offsets, row_map, src_map, h_rows, st_rows, _ = _forward_rows(s, x, w1, w2, idx, w)
    dy = orc.bf16_from_f64(np.random.default_rng(16).standard_normal((T, H)))
    g = orc.backward(s, x, w1, w2, w, row_map, src_map, offsets, h_rows, st_rows, dy)
    f = lambda a: torch.from_numpy(orc.f64_from_bf16(a))
    xd, w1d, w2d, dyd = f(x), f(w1), f(w2), f(dy)
    n = int(offsets[-1])
    dyp = torch.zeros(n, H, dtype=torch.float64)
    for r in range(n):
        sidx = int(src_map[r])
        dyp[r] = torch.from_numpy(_rne_bf16((float(w.ravel()[sidx]) * dyd[sidx // k]).numpy()))
    assert np.all(_ulp_diff_bf16(g["dyp"][:n], dyp.numpy()) == 0)
    dgu = torch.zeros(n, 2 * F, dtype=torch.float64)
    dxp = torch.zeros(n, H, dtype=torch.float64)
    dw1 = np.zeros((E, 2 * F, H))
    dw2 = np.zeros((E, H, F))
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        dh = dyp[r0:r1] @ w2d[e]                                  # [rows, F], not rounded
        st = f(st_rows[r0:r1])
        gg = st[:, :F].clone().requires_grad_(True)
        uu = st[:, F:].clone().requires_grad_(True)
        (tF.silu(gg) * uu).backward(dh)
        dgu[r0:r1] = torch.from_numpy(_rne_bf16(torch.cat([gg.grad, uu.grad], 1).numpy()))
        dxp[r0:r1] = torch.from_numpy(_rne_bf16((dgu[r0:r1] @ w1d[e]).numpy()))
        xp = xd[torch.from_numpy(src_map[r0:r1] // k).long()]
        dw1[e] = (dgu[r0:r1].T @ xp).numpy()
        dw2[e] = (dyp[r0:r1].T @ f(h_rows[r0:r1])).numpy()
    # float64 summation order may move a value across a rounding boundary:
    # at most one bf16 unit, in a small share of the values
    for key, ref in (("dgu", dgu), ("dxp", dxp)):
        d = _ulp_diff_bf16(g[key][:n], ref.numpy())
        assert d.max() <= 1 and d.mean() < 1e-3, key
    dx = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            dx[t] += dxp[int(row_map[t, j])].numpy()
    d = _ulp_diff_bf16(g["dx"], _rne_bf16(dx))
    assert d.max() <= 1 and d.mean() < 1e-3
    for key, ref in (("dw1", dw1), ("dw2", dw2)):
        got = g[key].astype(np.float64)
        ref32 = ref.astype(np.float32).astype(np.float64)
        ulp = np.spacing(np.abs(ref32).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(got - ref32) <= ulp), key
    # the misplacements named above are caught: dW1 from the unrounded dGU and
    # dW2 from an unrounded dYp differ from the oracle by far more
    e = int(np.argmax(counts))
    r0, r1 = int(offsets[e]), int(offsets[e + 1])
    dyp_raw = torch.stack([float(w.ravel()[int(src_map[r])]) * dyd[int(src_map[r]) // k] for r in range(r0, r1)])
    bad2 = (dyp_raw.T @ f(h_rows[r0:r1])).numpy()
    assert np.max(np.abs(bad2 - g["dw2"][e])) > 100 * np.max(np.abs(dw2[e] - g["dw2"][e]))


def test_bf16_backward_within_rounding_of_torch_autograd():
    """The bf16 layer's gradients against torch float64 autograd of the
    unrounded layer on the same stored inputs: the storage roundings of h, Yp,
    the stash, dYp, dGU, dXp and dX (each at most 2^-8 relative) bound the
    difference; 2^-6 normwise."""
    T, H, F, E, k = 31, 64, 48, 5, 2
    s, x, w1, w2, lg = _rand_problem(T, H, F, E, k, 17, fmt="bf16")
    idx, w = orc.route(lg, k, s.score, s.renorm)
    counts, offsets, row_map, src_map, h_rows, st_rows, _ = _forward_rows(s, x, w1, w2, idx, w)
    dy = orc.bf16_from_f64(np.random.default_rng(18).standard_normal((T, H)))
    g = orc.backward(s, x, w1, w2, w, row_map, src_map, offsets, h_rows, st_rows, dy)
    f = lambda a: torch.from_numpy(orc.f64_from_bf16(a))
    xt, w1t, w2t = (f(a).requires_grad_(True) for a in (x, w1, w2))
    rows = []
    for t in range(T):
        acc = torch.zeros(H, dtype=torch.float64)
        for j in range(k):
            e = int(idx[t, j])
            gu = tF.linear(xt[t], w1t[e])
            acc = acc + float(w[t, j]) * tF.linear(tF.silu(gu[:F]) * gu[F:], w2t[e])
        rows.append(acc)
    (torch.stack(rows) * f(dy)).sum().backward()
    assert _rel(orc.f64_from_bf16(g["dx"]), xt.grad.numpy()) < 2 ** -6
    assert _rel(g["dw1"], w1t.grad.numpy()) < 2 ** -6
    assert _rel(g["dw2"], w2t.grad.numpy()) < 2 ** -6
