"""Pins of the oracle's placement of the routing weight ([CUDNN] Summary:
router weight in the FC1 or FC2 epilogue; [TE-EP] commits: weights applied
early, before the combine).

In exact arithmetic the three placements give the same layer output, so each
is pinned to torch's float64 token-by-token evaluation of the weighted layer
(a library routine). Further pins: the stored rows carry their own route's
weight, unit weights make the placements identical bit for bit, and an
unweighted combine is the plain sum of the rows."""
import numpy as np
import pytest

from oracle import oracle as orc
from routing_permute_grouped_router_amd.workload import MoEShape
from test_oracle_ffn import _rand_problem, _rel, _torch_moe


def _f64(a):
    return np.asarray(a, np.float64)


def test_every_site_matches_torch_weighted_layer():
    # float32 storage: the sites differ from the float64 reference only by
    # float32 roundings of h, Yp and y
    s, x, w1, w2, lg = _rand_problem(41, 64, 96, 6, 3, 11, renorm=False)
    idx, w = orc.route(lg, s.k, s.score, s.renorm)
    ref = _torch_moe(_f64(x), _f64(w1), _f64(w2), idx, w, s.F)
    for site in ("combine", "fc1", "fc2"):
        out = orc.forward_tokens(s, np.arange(s.T), x, w1, w2, idx, w, site=site)
        assert _rel(out["y"], ref) < 2e-6, site


def test_rows_carry_their_own_route_weight():
    s, x, w1, w2, lg = _rand_problem(29, 64, 64, 5, 3, 12, renorm=False)
    idx, w = orc.route(lg, s.k, s.score, s.renorm)
    toks = np.arange(s.T)
    base = orc.forward_tokens(s, toks, x, w1, w2, idx, w)
    fc1 = orc.forward_tokens(s, toks, x, w1, w2, idx, w, site="fc1")
    fc2 = orc.forward_tokens(s, toks, x, w1, w2, idx, w, site="fc2")
    wt = _f64(w)[:, :, None]
    # FC2: h untouched, Yp(t, j) scaled by w[t, j] (distinct weights per slot,
    # so a weight taken from another slot or token fails)
    assert np.array_equal(fc2["h"], base["h"])
    np.testing.assert_allclose(_f64(fc2["yp"]), wt * _f64(base["yp"]), rtol=2e-7, atol=1e-30)
    # FC1: h(t, j) scaled by w[t, j] before it is stored
    np.testing.assert_allclose(_f64(fc1["h"]), wt * _f64(base["h"]), rtol=2e-7, atol=1e-30)
    assert len(np.unique(np.round(_f64(w), 6))) > s.k


def test_unit_weights_make_the_sites_identical():
    # top-1 with the weights renormalised over the chosen expert: w == 1
    # exactly, so every placement stores the same bf16 bytes
    s, x, w1, w2, lg = _rand_problem(33, 128, 64, 4, 1, 13, fmt="bf16", renorm=True)
    idx, w = orc.route(lg, s.k, s.score, s.renorm)
    assert np.all(w == 1.0)
    toks = np.arange(s.T)
    outs = [orc.forward_tokens(s, toks, x, w1, w2, idx, w, site=site) for site in ("combine", "fc1", "fc2")]
    for o in outs[1:]:
        for key in ("h", "yp", "y"):
            assert np.array_equal(o[key], outs[0][key]), key


def test_unweighted_combine_is_the_plain_sum():
    rng = np.random.default_rng(14)
    T, k, H, R = 23, 3, 32, 80
    yp = rng.standard_normal((R, H)).astype(np.float32)
    row_map = np.stack([rng.choice(R, k, replace=False) for _ in range(T)]).astype(np.int32)
    row_map[3, 1] = -1  # a dropped route
    y = orc.combine(yp, row_map, None, "f32")
    ref = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            if row_map[t, j] >= 0:
                ref[t] += yp[row_map[t, j]]
    np.testing.assert_allclose(y, ref, rtol=1e-6, atol=1e-6)
    assert np.array_equal(y, orc.combine(yp, row_map, np.ones((T, k), np.float32), "f32"))


@pytest.mark.parametrize("fmt", ["bf16", "mxfp8"])
def test_power_of_two_weights_make_the_sites_identical(fmt):
    # Scaling by a power of two commutes with bf16 rounding and with MX
    # quantisation (the block's shared exponent moves, the codes stay), so
    # with such weights h (FC1: up to its scales), Yp and y of every
    # placement are the same bytes.  Weights differ between the slots of a
    # token, so a weight from the wrong slot, a missing or a doubled weight
    # changes them.
    T, H, F, E, k = 24, 128, 128, 4, 3
    s0, x, w1, w2, lg = _rand_problem(T, H, F, E, k, 15, renorm=False)
    idx, _ = orc.route(lg, k, "softmax", False)
    w = np.array([[2.0 ** -(1 + (t + j) % 3) for j in range(k)] for t in range(T)], np.float32)
    if fmt == "mxfp8":
        xq, xs = orc.mx_quantize(x)
        w1q, w1s = orc.mx_quantize(w1)
        w2q, w2s = orc.mx_quantize(w2)
        args = (xq, w1q, w2q, idx, w, xs, w1s, w2s)
    else:
        args = (orc.bf16_from_f64(_f64(x)), orc.bf16_from_f64(_f64(w1)), orc.bf16_from_f64(_f64(w2)), idx, w)
    s = MoEShape("p2", T, H, F, E, k, "softmax", False, fmt)
    base, fc1, fc2 = (orc.forward_tokens(s, np.arange(T), *args, site=site) for site in ("combine", "fc1", "fc2"))
    assert np.array_equal(fc1["y"], base["y"]) and np.array_equal(fc2["y"], base["y"])
    wt = _f64(w)[:, :, None]
    dec = lambda a: orc.f64_from_bf16(a)
    assert np.array_equal(dec(fc2["yp"]), wt * dec(base["yp"]))
    assert np.array_equal(dec(fc1["yp"]), dec(fc2["yp"]))
    if fmt == "mxfp8":
        assert np.array_equal(fc1["h"], base["h"])
        assert np.array_equal(orc.mx_dequantize(fc1["h"], fc1["h_scale"]),
                              wt * orc.mx_dequantize(base["h"], base["h_scale"]))
    else:
        assert np.array_equal(dec(fc1["h"]), wt * dec(base["h"]))
