"""GPU parity of the routing backward (moe_route_bwd: gradients of the top-k
weights and of the router logits) against the oracle's float64 routing
backward, through the C ABI.

Small shapes in full (softmax, renormalised softmax, normalised sigmoid;
fp32, bf16 and MXFP8 storage, whose output dtype is bf16); the full-size
skewed layer on a seeded token sample.  Every quantity is float32 arithmetic
on stored bf16 / fp32 values, so the bar is 1e-4 of the normwise relative
error (tighter than the bf16 output tolerance: nothing here is rounded to
bf16)."""
import numpy as np
import pytest
import torch

import routing_permute_grouped_router_amd as moe
from oracle import oracle as orc
from routing_permute_grouped_router_amd import workload as wl

from helpers import Inputs, cfg_of, rel_err, run_forward, to_dev, to_host

pytestmark = pytest.mark.gpu
TOL_RB = 1e-4


def _dy(s, cfg):
    rng = np.random.default_rng(s.seed + 31)
    v = rng.standard_normal((s.T, s.H))
    return to_dev(v.astype(np.float32), "f32") if cfg.out_dtype == torch.float32 else to_dev(orc.bf16_from_f64(v), "bf16")


def _route_bwd(cfg, dy, buf, logits, want_dw=True):
    dl = torch.full((cfg.T, cfg.E), float("nan"), dtype=torch.float32, device="cuda")
    dw = torch.full((cfg.T, cfg.k), float("nan"), dtype=torch.float32, device="cuda") if want_dw else None
    moe.moe_route_bwd(cfg, dy, buf["yp"], logits, buf["idx"], buf["row_map"], dl, dw=dw)
    torch.cuda.synchronize()
    return dl, dw


@pytest.mark.parametrize("name", [s.name for s in wl.small_shapes()])
def test_route_bwd_small_full_parity(name):
    s = [x for x in wl.small_shapes() if x.name == name][0]
    cfg = cfg_of(s)
    if s.dtype == "mxfp8":
        from test_gpu_mxfp8 import _forward_mx
        w = wl.Workload(s)
        buf, _ = _forward_mx(s, w.x(), w.w1(), w.w2(), w.logits())
        logits = w.logits()
    else:
        inp = Inputs(s)
        buf = run_forward(inp)
        logits = inp.logits
    dy = _dy(s, cfg)
    dl, dw = _route_bwd(cfg, dy, buf, to_dev(logits, "f32"))
    fmt = "f32" if s.dtype == "f32" else "bf16"
    dw_o, dl_o = orc.route_bwd(logits, to_host(buf["idx"]), to_host(buf["row_map"]), to_host(dy),
                               to_host(buf["yp"]), fmt, s.score, s.renorm)
    assert np.all(np.isfinite(to_host(dl))) and np.all(np.isfinite(to_host(dw)))
    assert rel_err(to_host(dw), dw_o) < TOL_RB
    assert rel_err(to_host(dl), dl_o) < TOL_RB
    if s.score == "sigmoid" or s.renorm:  # only the selected experts' logits move
        sel = np.zeros((s.T, s.E), bool)
        np.put_along_axis(sel, to_host(buf["idx"]).astype(np.int64), True, axis=1)
        assert np.all(to_host(dl)[~sel] == 0)
    else:  # the softmax spreads no net gradient
        assert np.abs(to_host(dl).sum(axis=1)).max() < 1e-5 * np.abs(dl_o).max() * s.E
    # without the optional dw output the logit gradient is the same
    dl2, _ = _route_bwd(cfg, dy, buf, to_dev(logits, "f32"), want_dw=False)
    assert np.array_equal(to_host(dl2), to_host(dl))


def test_route_bwd_full_size_skewed():
    s = wl.BY_NAME["skewed_bf16"]
    cfg = cfg_of(s)
    inp = Inputs(s)
    buf = run_forward(inp, poison=False)
    dy = _dy(s, cfg)
    dl, dw = _route_bwd(cfg, dy, buf, to_dev(inp.logits, "f32"))
    rng = np.random.default_rng(s.seed + 7)
    toks = np.sort(rng.choice(s.T, 64, replace=False))
    dw_o, dl_o = orc.route_bwd(inp.logits, to_host(buf["idx"]), to_host(buf["row_map"]), to_host(dy),
                               to_host(buf["yp"]), "bf16", s.score, s.renorm, tokens=toks)
    assert rel_err(to_host(dw)[toks], dw_o) < TOL_RB
    assert rel_err(to_host(dl)[toks], dl_o) < TOL_RB
    assert np.all(np.isfinite(to_host(dl)))


def test_route_bwd_sigmoid_underflow():
    """Normalised sigmoid with k > 1 where every chosen sigmoid of some tokens
    underflows to 0 in float32 (chosen logits at or below -100): the forward
    gives those tokens w = 0 through the + 1e-20 of the normaliser, and the
    backward must give finite gradients that match the float64 oracle (which
    keeps the same + 1e-20), not 0/0."""
    T, H, E, k = 96, 128, 16, 4
    rng = np.random.default_rng(4242)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[::3] = -100.0 - 10.0 * rng.random((len(lg[::3]), E)).astype(np.float32)  # all experts underflow
    lg[1::3, :] -= 80.0                                                            # tiny, not zero
    cfg = moe.MoEConfig(T, H, 64, E, k, 1, "sigmoid", True, "bf16")
    idx_o, w_o = orc.route(lg, k, "sigmoid", True)
    assert np.all(w_o[::3] < 1e-20)  # float64 sigmoids ~1e-44 over 1e-20; float32 underflows to 0
    _, _, row_map, _, _ = orc.group(idx_o, E, 1)
    yp = orc.bf16_from_f64(rng.standard_normal((T * k, H)))
    dy = orc.bf16_from_f64(rng.standard_normal((T, H)))
    buf = {"yp": to_dev(yp, "bf16"), "idx": to_dev(idx_o, "i32"), "row_map": to_dev(row_map, "i32")}
    dl, dw = _route_bwd(cfg, to_dev(dy, "bf16"), buf, to_dev(lg, "f32"))
    dw_o, dl_o = orc.route_bwd(lg, idx_o, row_map, dy, yp, "bf16", "sigmoid", True)
    dl_h, dw_h = to_host(dl), to_host(dw)
    assert np.all(np.isfinite(dl_h)) and np.all(np.isfinite(dw_h))
    assert np.all(dl_h[::3] == 0) and np.all(np.abs(dl_o[::3]) < 1e-20)
    assert rel_err(dw_h, dw_o) < TOL_RB
    assert rel_err(dl_h, dl_o) < TOL_RB
