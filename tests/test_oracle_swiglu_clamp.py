"""Pins of the oracle's optional SwiGLU clamp ([CUDNN] Summary: local SwiGLU
experts with an optional DeepSeek-style clamp): h = silu(min(g, L)) *
clamp(u, -L, L), the gradient of each clamp passing where its bound is not
exceeded.

References: torch's clamp, silu and linear with autograd in float64 (library
routines) for the forward and the backward, on random problems and on a
crafted one whose gate and up values sit exactly on the bounds; a limit above
every |g| and |u| reduces to the unclamped layer bit for bit."""
import numpy as np
import torch
import torch.nn.functional as tF

from oracle import oracle as orc
from routing_permute_grouped_router_amd.workload import MoEShape
from test_oracle_ffn import _rand_problem, _rel


def _rows(s, x, w1, w2, idx, w, limit, align=1):
    counts, offsets, row_map, src_map, _ = orc.group(idx, s.E, align)
    out = orc.forward_tokens(s, np.arange(s.T), x, w1, w2, idx, w, want_stash=True, limit=limit)
    R_cap = src_map.shape[0]
    h_rows = np.zeros((R_cap, s.F), out["h"].dtype)
    st_rows = np.zeros((R_cap, 2 * s.F), out["stash"].dtype)
    for i, r in enumerate(row_map.ravel()):
        if r >= 0:
            h_rows[r] = out["h"].reshape(-1, s.F)[i]
            st_rows[r] = out["stash"].reshape(-1, 2 * s.F)[i]
    return counts, offsets, row_map, src_map, h_rows, st_rows, out


def _torch_layer(x, w1, w2, idx, w, F, limit, dy):
    xt = torch.from_numpy(x.astype(np.float64)).requires_grad_(True)
    w1t = torch.from_numpy(w1.astype(np.float64)).requires_grad_(True)
    w2t = torch.from_numpy(w2.astype(np.float64)).requires_grad_(True)
    rows = []
    for t in range(idx.shape[0]):
        acc = torch.zeros(x.shape[1], dtype=torch.float64)
        for j in range(idx.shape[1]):
            e = int(idx[t, j])
            gu = tF.linear(xt[t], w1t[e])
            g = torch.clamp(gu[:F], max=limit)
            u = torch.clamp(gu[F:], min=-limit, max=limit)
            acc = acc + float(w[t, j]) * tF.linear(tF.silu(g) * u, w2t[e])
        rows.append(acc)
    y = torch.stack(rows)
    (y * torch.from_numpy(dy.astype(np.float64))).sum().backward()
    return y.detach().numpy(), xt.grad.numpy(), w1t.grad.numpy(), w2t.grad.numpy()


def _check_against_torch(s, x, w1, w2, idx, w, limit, dy, align=1):
    counts, offsets, row_map, src_map, h_rows, st_rows, out = _rows(s, x, w1, w2, idx, w, limit, align)
    g = orc.backward(s, x, w1, w2, w, row_map, src_map, offsets, h_rows, st_rows, dy, limit=limit)
    y, dx, dw1, dw2 = _torch_layer(x, w1, w2, idx, w, s.F, limit, dy)
    assert _rel(out["y"], y) < 1e-5
    assert _rel(g["dx"], dx) < 1e-5
    assert _rel(g["dw1"], dw1) < 1e-5
    assert _rel(g["dw2"], dw2) < 1e-5
    return out


def test_clamp_matches_torch_autograd():
    T, H, F, E, k = 31, 32, 48, 5, 2
    s, x, w1, w2, lg = _rand_problem(T, H, F, E, k, 21)
    idx, w = orc.route(lg, k, s.score, s.renorm)
    dy = np.random.default_rng(22).standard_normal((T, H)).astype(np.float32)
    limit = 0.6
    out = _check_against_torch(s, x, w1, w2, idx, w, limit, dy, align=4)
    st = out["stash"].reshape(-1, 2 * F).astype(np.float64)
    # the limit is active: a good share of gate and up values lie beyond it
    assert np.mean(st[:, :F] > limit) > 0.15 and np.mean(np.abs(st[:, F:]) > limit) > 0.3


def test_values_on_the_bounds_pass_gradient():
    # x one-hot: g and u are exactly the chosen weights, some of them exactly
    # on +-L (float32 storage, so the stored stash keeps them exact)
    T, H, F, E, k, L = 4, 32, 32, 1, 1, 0.5
    x = np.zeros((T, H), np.float32)
    x[np.arange(T), np.arange(T)] = 1.0
    rng = np.random.default_rng(23)
    w1 = (rng.standard_normal((E, 2 * F, H)) * 0.5).astype(np.float32)
    vals = np.array([L, -L, 2 * L, -2 * L, 0.25 * L, 1.5 * L], np.float32)
    for t in range(T):
        w1[0, : len(vals), t] = vals
        w1[0, F: F + len(vals), t] = vals[::-1]
    w2 = (rng.standard_normal((E, H, F)) / np.sqrt(F)).astype(np.float32)
    idx = np.zeros((T, k), np.int32)
    w = np.ones((T, k), np.float32)
    dy = rng.standard_normal((T, H)).astype(np.float32)
    s = MoEShape("bounds", T, H, F, E, k, "softmax", True, "f32")
    _check_against_torch(s, x, w1, w2, idx, w, L, dy)


def test_limit_beyond_every_value_is_no_clamp():
    s, x, w1, w2, lg = _rand_problem(27, 64, 64, 4, 2, 24, fmt="bf16")
    idx, w = orc.route(lg, s.k, s.score, s.renorm)
    a = orc.forward_tokens(s, np.arange(s.T), x, w1, w2, idx, w, want_stash=True)
    b = orc.forward_tokens(s, np.arange(s.T), x, w1, w2, idx, w, want_stash=True, limit=1e6)
    for key in ("h", "yp", "y", "stash"):
        assert np.array_equal(a[key], b[key]), key


def test_sampled_backward_helpers_follow_the_clamp():
    T, H, F, E, k, L = 33, 64, 32, 5, 2, 0.5
    s, x, w1, w2, lg = _rand_problem(T, H, F, E, k, 25, fmt="bf16")
    idx, w = orc.route(lg, k, s.score, s.renorm)
    counts, offsets, row_map, src_map, h_rows, st_rows, _ = _rows(s, x, w1, w2, idx, w, L)
    dy = orc.bf16_from_f64(np.random.default_rng(26).standard_normal((T, H)))
    g = orc.backward(s, x, w1, w2, w, row_map, src_map, offsets, h_rows, st_rows, dy, limit=L)
    g0 = orc.backward(s, x, w1, w2, w, row_map, src_map, offsets, h_rows, st_rows, dy)
    assert not np.array_equal(g["dx"], g0["dx"])
    toks = np.array([0, 5, 17, 32])
    assert np.array_equal(orc.backward_dx_tokens(s, toks, x, w1, w2, idx, w, dy, limit=L), g["dx"][toks])
    e = int(np.argmax(counts))
    rng = np.random.default_rng(27)
    i2 = np.stack([rng.integers(0, H, 20), rng.integers(0, F, 20)], 1)
    i1 = np.stack([rng.integers(0, 2 * F, 20), rng.integers(0, H, 20)], 1)
    d2, d1 = orc.backward_dw_entries(s, e, x, w1, w2, w, src_map, offsets, dy, i2, i1, limit=L)
    np.testing.assert_allclose(d2.astype(np.float32), g["dw2"][e][i2[:, 0], i2[:, 1]], rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(d1.astype(np.float32), g["dw1"][e][i1[:, 0], i1[:, 1]], rtol=1e-6, atol=1e-7)
