"""Pins of the oracle's routing backward (oracle.route_bwd) against things
other than its own formulas:

- central finite differences of L(logits) = sum_t <dy_t, sum_j w_j Yp[row_j]>,
  with the weights w taken from the C oracle's forward routing (or_route) and
  the selection held fixed (logits spaced far wider than the step);
- k = 1 with renormalisation or the normalised sigmoid: the weight is the
  constant 1, so every logit gradient is zero;
- equal logits without renormalisation: p = 1/E gives the closed form
  dl_e = (dw_e - sum_j dw_j / E) / E;
- both softmax forms spread no net gradient: each row of dlogits sums to 0;
- a dropped route (row -1) gets dw = 0."""
import numpy as np
import pytest

from oracle import oracle as orc


def _case(rng, T, E, k, H):
    # logits: a shuffled ladder with gaps of 0.25 plus small noise, so a step
    # of 1e-3 never changes the top-k choice
    lg = np.stack([rng.permutation(E) * 0.25 + rng.uniform(-0.02, 0.02, E) for _ in range(T)]).astype(np.float32)
    lg -= 0.125 * E  # mixed signs for the sigmoid
    dy = rng.standard_normal((T, H)).astype(np.float32)
    R = T * k + 3
    yp = rng.standard_normal((R, H)).astype(np.float32)
    rm = rng.permutation(R)[: T * k].reshape(T, k).astype(np.int32)
    return lg, dy, yp, rm


def _loss(lg, k, score, renorm, dy, yp, rm):
    idx, w = orc.route(lg, k, score, renorm)
    w = w.astype(np.float64)
    y = np.einsum("tj,tjh->th", w, yp.astype(np.float64)[rm])
    return float((dy.astype(np.float64) * y).sum()), idx


@pytest.mark.parametrize("score,renorm", [("softmax", False), ("softmax", True), ("sigmoid", True)])
def test_route_bwd_matches_finite_differences(score, renorm):
    rng = np.random.default_rng(71 + renorm + 2 * (score == "sigmoid"))
    T, E, k, H = 5, 12, 3, 24
    lg, dy, yp, rm = _case(rng, T, E, k, H)
    idx, _ = orc.route(lg, k, score, renorm)
    dw, dl = orc.route_bwd(lg, idx, rm, dy, yp, "f32", score, renorm)
    h = 1e-3
    num = np.zeros_like(dl)
    for t in range(T):
        for e in range(E):
            lp, lm = lg.copy(), lg.copy()
            lp[t, e] += h
            lm[t, e] -= h
            fp, ip = _loss(lp, k, score, renorm, dy, yp, rm)
            fm, im = _loss(lm, k, score, renorm, dy, yp, rm)
            assert np.array_equal(ip, idx) and np.array_equal(im, idx), "the step changed the selection"
            num[t, e] = (fp - fm) / (2 * h)
    err = np.abs(num - dl).max() / np.abs(dl).max()
    assert err < 1e-3, err
    # the weight gradients: dw[t, j] = dL / dw[t, j] for L linear in w
    base, _ = _loss(lg, k, score, renorm, dy, yp, rm)
    y = yp.astype(np.float64)[rm]
    assert np.allclose(dw, np.einsum("th,tjh->tj", dy.astype(np.float64), y))
    if score == "softmax":
        assert np.abs(dl.sum(axis=1)).max() < 1e-12 * np.abs(dl).max() * E


@pytest.mark.parametrize("score,renorm", [("softmax", True), ("sigmoid", True)])
def test_route_bwd_single_choice_has_no_gradient(score, renorm):
    rng = np.random.default_rng(5)
    lg, dy, yp, rm = _case(rng, 4, 8, 1, 16)
    idx, w = orc.route(lg, 1, score, renorm)
    assert np.allclose(w, 1.0)
    _, dl = orc.route_bwd(lg, idx, rm, dy, yp, "f32", score, renorm)
    assert np.abs(dl).max() < 1e-15


def test_route_bwd_equal_logits_closed_form():
    rng = np.random.default_rng(9)
    T, E, k, H = 3, 8, 2, 16
    _, dy, yp, rm = _case(rng, T, E, k, H)
    lg = np.zeros((T, E), np.float32)
    idx, w = orc.route(lg, k, "softmax", False)
    assert np.array_equal(idx, np.tile(np.arange(k), (T, 1)))  # ties go to the lower index
    dw, dl = orc.route_bwd(lg, idx, rm, dy, yp, "f32", "softmax", False)
    exp = np.zeros((T, E))
    exp[:, :k] = dw
    exp = (exp - dw.sum(axis=1, keepdims=True) / E) / E
    assert np.allclose(dl, exp, rtol=1e-12, atol=1e-15)


def test_route_bwd_dropped_route():
    rng = np.random.default_rng(13)
    lg, dy, yp, rm = _case(rng, 4, 8, 3, 16)
    idx, _ = orc.route(lg, 3, "sigmoid", True)
    rm = rm.copy()
    rm[2, 1] = -1
    dw, _ = orc.route_bwd(lg, idx, rm, dy, yp, "f32", "sigmoid", True)
    assert dw[2, 1] == 0.0 and np.all(dw[np.arange(4) != 2] != 0.0)
