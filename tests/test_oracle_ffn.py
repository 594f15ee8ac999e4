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
