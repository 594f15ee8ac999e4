"""Pins of the oracle's routing (score function, top-k, normalisation) and
grouping (counts, aligned offsets, row maps) and of permute/combine.

References used: stable sorting (brute force), scipy's softmax / expit
(library routines), closed forms for equal logits, numpy's bincount / cumsum,
and the permute-then-combine identity."""
import itertools

import numpy as np
import pytest
from scipy.special import expit, softmax

from oracle import oracle as orc


def _brute_topk(lg, k):
    # ascending sort of (-logit, index): largest first, ties to the lower index
    return np.argsort(-lg, axis=1, kind="stable")[:, :k].astype(np.int32)


@pytest.mark.parametrize("E,k", [(8, 2), (16, 4), (128, 8), (256, 8), (5, 5), (64, 1)])
def test_topk_matches_stable_sort(E, k):
    rng = np.random.default_rng(E * 31 + k)
    lg = rng.standard_normal((300, E)).astype(np.float32)
    lg[::7, : E // 2] = 0.5  # plenty of exact ties
    lg[::11] = np.round(lg[::11])
    idx, _ = orc.route(lg, k)
    assert np.array_equal(idx, _brute_topk(lg, k))


def test_topk_exhaustive_ties_with_signed_zeros():
    vals = [-1.0, -0.0, 0.0, 1.0]
    pats = np.array(list(itertools.product(vals, repeat=4)), np.float32)
    for k in range(1, 5):
        idx, _ = orc.route(pats, k)
        for p, got in zip(pats, idx):
            want = sorted(range(4), key=lambda e: (-float(p[e]), e))[:k]  # -0.0 == 0.0 in Python
            assert list(got) == want


@pytest.mark.parametrize("renorm", [False, True])
def test_softmax_weights_match_scipy(renorm):
    rng = np.random.default_rng(5)
    lg = (rng.standard_normal((200, 32)) * 3).astype(np.float32)
    idx, w = orc.route(lg, 4, "softmax", renorm)
    p = softmax(lg.astype(np.float64), axis=1)
    sel = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    if renorm:
        sel = sel / sel.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(w, sel, rtol=1e-7, atol=0)


def test_sigmoid_weights_match_scipy():
    rng = np.random.default_rng(6)
    lg = (rng.standard_normal((200, 64)) * 4).astype(np.float32)
    idx, w = orc.route(lg, 8, "sigmoid", True)
    s = expit(np.take_along_axis(lg.astype(np.float64), idx.astype(np.int64), axis=1))
    np.testing.assert_allclose(w, s / s.sum(axis=1, keepdims=True), rtol=1e-7, atol=0)


def test_equal_logits_closed_forms():
    lg = np.full((10, 16), 0.3, np.float32)
    idx, w = orc.route(lg, 4, "softmax", False)
    assert np.array_equal(idx, np.tile(np.arange(4, dtype=np.int32), (10, 1)))
    np.testing.assert_allclose(w, 1 / 16, rtol=1e-7)
    _, w = orc.route(lg, 4, "softmax", True)
    np.testing.assert_allclose(w, 1 / 4, rtol=1e-7)
    _, w = orc.route(lg, 4, "sigmoid", True)
    np.testing.assert_allclose(w, 1 / 4, rtol=1e-7)


def test_renorm_with_k_equal_E_is_full_softmax():
    rng = np.random.default_rng(8)
    lg = rng.standard_normal((50, 8)).astype(np.float32)
    idx, w = orc.route(lg, 8, "softmax", True)
    p = softmax(lg.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(p, idx.astype(np.int64), axis=1), rtol=1e-7)


def test_sigmoid_underflow_gives_zero_not_nan():
    lg = np.full((3, 8), -1000.0, np.float32)
    _, w = orc.route(lg, 4, "sigmoid", True)
    assert np.all(w == 0.0)


def test_route_rejects_k_above_E():
    with pytest.raises(ValueError):
        orc.route(np.zeros((2, 4), np.float32), 5)


# ---------------------------------------------------------------- grouping
def _check_maps(idx, E, align, counts, offsets, row_map, src_map):
    T, k = idx.shape
    valid = (idx >= 0) & (idx < E)
    assert np.array_equal(counts, np.bincount(idx[valid].ravel(), minlength=E))
    padded = ((counts + align - 1) // align) * align
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(padded)]).astype(np.int32))
    flat = row_map.ravel()
    real = flat[flat >= 0]
    assert len(np.unique(real)) == len(real) == valid.sum()  # injective
    for i, r in enumerate(flat):
        if r >= 0:
            assert src_map[r] == i
            e = idx.ravel()[i]
            assert offsets[e] <= r < offsets[e] + counts[e]
    # rows of one expert hold ascending tokens, pads and tail hold -1
    for e in range(E):
        rows = src_map[offsets[e]:offsets[e] + counts[e]]
        assert np.all(rows >= 0) and np.all(np.diff(rows) > 0)
        assert np.all(src_map[offsets[e] + counts[e]:offsets[e + 1]] == -1)
    assert np.all(src_map[offsets[E]:] == -1)


@pytest.mark.parametrize("E,k,align", [(8, 2, 1), (16, 4, 1), (12, 3, 16), (128, 8, 128), (7, 7, 3)])
def test_group_invariants(E, k, align):
    rng = np.random.default_rng(E + k + align)
    lg = rng.standard_normal((257, E)).astype(np.float32)
    idx, _ = orc.route(lg, k)
    counts, offsets, row_map, src_map, bad = orc.group(idx, E, align)
    assert bad == 0
    assert counts.sum() == idx.size
    _check_maps(idx, E, align, counts, offsets, row_map, src_map)


def test_group_uniform_routing_empties_experts():
    T, E, k = 100, 16, 4
    idx, _ = orc.route(np.zeros((T, E), np.float32), k)
    counts, offsets, *_ = orc.group(idx, E)
    assert list(counts) == [T] * k + [0] * (E - k)


def test_group_dropped_and_bad_ids():
    idx = np.array([[0, -1], [3, 1], [-1, -1], [7, 0], [1, -5]], np.int32)
    counts, offsets, row_map, src_map, bad = orc.group(idx, 4)
    assert bad == 2  # 7 and -5 are outside [-1, 4)
    assert list(counts) == [2, 2, 0, 1]
    assert row_map[0, 1] == -1 and row_map[2, 0] == -1 and row_map[3, 0] == -1
    assert list(row_map[:, 0]) == [0, 4, -1, -1, 3] and row_map[3, 1] == 1 and row_map[1, 1] == 2


def test_permute_then_combine_identity():
    """Permute, identity expert, combine with unit weights = k * x exactly
    (k a power of two, so the scaling is exact in bf16 and f32)."""
    rng = np.random.default_rng(9)
    for k, fmt, align in [(2, "bf16", 1), (4, "f32", 8), (8, "bf16", 4)]:
        T, E, H = 130, 16, 64
        idx, _ = orc.route(rng.standard_normal((T, E)).astype(np.float32), k)
        counts, offsets, row_map, src_map, _ = orc.group(idx, E, align)
        xv = rng.standard_normal((T, H))
        x = orc.bf16_from_f64(xv) if fmt == "bf16" else xv.astype(np.float32)
        xp = orc.permute(x, row_map, src_map.shape[0])
        for i, r in enumerate(row_map.ravel()):
            assert np.array_equal(xp[r], x[i // k])
        pad = src_map == -1
        assert np.all(xp[pad] == 0)
        y = orc.combine(xp, row_map, np.ones((T, k), np.float32), fmt)
        assert np.array_equal(orc.decode(fmt, y), k * orc.decode(fmt, x))


# ---- selection-only expert bias: key = fl32(logit + bias), weights unbiased
def _biased_problem(seed, T=300, E=32, scale=1.0):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[::9, : E // 2] = 0.25  # exact ties
    bias = (rng.standard_normal(E) * scale).astype(np.float32)
    return lg, bias


@pytest.mark.parametrize("score,renorm", [("softmax", False), ("softmax", True), ("sigmoid", True)])
def test_zero_bias_gives_the_unbiased_routing_bytes(score, renorm):
    lg, _ = _biased_problem(41)
    i0, w0 = orc.route(lg, 4, score, renorm)
    for zero in (np.zeros(32, np.float32), np.full(32, -0.0, np.float32)):
        i1, w1 = orc.route(lg, 4, score, renorm, bias=zero)
        assert np.array_equal(i0, i1) and np.array_equal(w0.view(np.uint32), w1.view(np.uint32))


@pytest.mark.parametrize("E,k,scale", [(8, 2, 0.5), (32, 4, 1.0), (128, 8, 3.0), (256, 8, 0.1)])
def test_biased_topk_matches_stable_sort_of_the_float32_key(E, k, scale):
    lg, bias = _biased_problem(E + k, E=E, scale=scale)
    key = lg + bias[None, :]  # numpy float32 + float32: one rounding to nearest even
    assert key.dtype == np.float32
    idx, _ = orc.route(lg, k, "sigmoid", True, bias=bias)
    assert np.array_equal(idx, _brute_topk(key, k))


@pytest.mark.parametrize("score,renorm", [("softmax", False), ("softmax", True), ("sigmoid", True)])
def test_bias_changes_the_choice_not_the_weights(score, renorm):
    """The weights are the unbiased score function of the chosen experts
    (scipy, float64), whatever bias chose them."""
    lg, bias = _biased_problem(43, E=64, scale=2.0)
    idx, w = orc.route(lg, 6, score, renorm, bias=bias)
    i0, _ = orc.route(lg, 6, score, renorm)
    assert not np.array_equal(idx, i0), "the bias should change some choices"
    l64 = lg.astype(np.float64)
    if score == "softmax":
        sel = np.take_along_axis(softmax(l64, axis=1), idx.astype(np.int64), axis=1)
        if renorm:
            sel = sel / sel.sum(axis=1, keepdims=True)
    else:
        sel = expit(np.take_along_axis(l64, idx.astype(np.int64), axis=1))
        sel = sel / sel.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(w, sel, rtol=1e-7, atol=0)


def test_strong_bias_forces_its_experts():
    """A bias far above the logits' spread picks the biased experts, in the
    order of their (biased) keys; the weights are still the unbiased ones."""
    rng = np.random.default_rng(44)
    lg = rng.standard_normal((100, 16)).astype(np.float32)
    bias = np.zeros(16, np.float32)
    bias[[3, 9, 12]] = [100.0, 200.0, 300.0]
    idx, w = orc.route(lg, 3, "sigmoid", True, bias=bias)
    assert np.all(idx == np.array([12, 9, 3], np.int32))
    s = expit(lg[:, [12, 9, 3]].astype(np.float64))
    np.testing.assert_allclose(w, s / s.sum(axis=1, keepdims=True), rtol=1e-7, atol=0)
