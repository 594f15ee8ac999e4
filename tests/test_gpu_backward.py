"""GPU parity of the FFN backward (combine backward, down-projection backward
fused with the SwiGLU backward, gate/up backward, permute backward) against
the CPU oracle, through the C ABI.

Small shapes (skewed routing; 16-row group alignment): every gradient compared
in full.  Full-size skewed workload
(T=16384, H=2048, F=768, E=128, top-8, Zipf-biased routing): dX on a seeded
token sample, dW1/dW2 on sampled entries of moderately loaded experts, and
dW of every empty expert exactly zero (it starts as NaN)."""
import numpy as np
import pytest
import torch

import routing_permute_grouped_router_amd as moe
from oracle import oracle as orc
from routing_permute_grouped_router_amd import workload as wl

from helpers import Inputs, TOL, cfg_of, decode, rel_err, run_forward, to_host

pytestmark = pytest.mark.gpu


def _run_backward(inp, fwd):
    cfg = cfg_of(inp.s)
    bwd = moe.alloc_backward(cfg)
    for k in ("dyp", "dgu", "dxp", "dx", "dw1", "dw2"):
        bwd[k].fill_(float("nan"))
    d = inp.dev
    moe.moe_backward(cfg, d["dy"], d["w1"], d["w2"], fwd, bwd)
    torch.cuda.synchronize()
    return bwd


@pytest.mark.parametrize("name", ["small_skewed_bf16", "small_bf16_sigmoid_align"])
def test_backward_small_full_parity(name):
    """Skewed routing (empty experts) and a 16-row group alignment (padding
    rows, which the combine backward must zero)."""
    s = [x for x in wl.small_shapes() if x.name == name][0]
    inp = Inputs(s, want_dy=True)
    fwd = run_forward(inp, training=True)
    bwd = _run_backward(inp, fwd)
    idx, w = orc.route(inp.logits, s.k, s.score, s.renorm)
    counts, offsets, row_map, src_map, _ = orc.group(idx, s.E, s.align)
    ref = orc.forward_tokens(s, np.arange(s.T), inp.x, inp.w1, inp.w2, idx, w, want_stash=True)
    R = src_map.shape[0]
    h_rows = np.zeros((R, s.F), np.uint16)
    st_rows = np.zeros((R, 2 * s.F), np.uint16)
    rm = row_map.ravel()
    h_rows[rm] = ref["h"].reshape(-1, s.F)
    st_rows[rm] = ref["stash"].reshape(-1, 2 * s.F)
    g = orc.backward(s, inp.x, inp.w1, inp.w2, w, row_map, src_map, offsets, h_rows, st_rows, inp.dy)
    n = int(offsets[-1])
    for key in ("dyp", "dgu", "dxp"):
        got = decode("bf16", to_host(bwd[key])[:n])
        assert rel_err(got, decode("bf16", g[key][:n])) < TOL["bf16"], key
    assert rel_err(decode("bf16", to_host(bwd["dx"])), decode("bf16", g["dx"])) < TOL["bf16"]
    dw1, dw2 = to_host(bwd["dw1"]), to_host(bwd["dw2"])
    assert np.all(np.isfinite(dw1)) and np.all(np.isfinite(dw2))
    assert rel_err(dw1, g["dw1"]) < TOL["bf16"]
    assert rel_err(dw2, g["dw2"]) < TOL["bf16"]
    if s.align > 1:
        pad = src_map[:n] < 0
        assert pad.any(), "the alignment should leave padding rows"
        assert np.all(to_host(bwd["dyp"])[:n][pad] == 0)
    empty = np.where(counts == 0)[0]
    if name == "small_skewed_bf16":
        assert len(empty) > 0, "the skewed routing should leave some experts empty"
    assert np.all(dw1[empty] == 0) and np.all(dw2[empty] == 0)


def test_backward_full_size_skewed():
    s = wl.BY_NAME["skewed_bf16"]
    inp = Inputs(s, want_dy=True)
    fwd = run_forward(inp, training=True, poison=False)
    bwd = _run_backward(inp, fwd)
    idx, w = orc.route(inp.logits, s.k, s.score, s.renorm)
    counts, offsets, row_map, src_map, _ = orc.group(idx, s.E, s.align)
    assert np.array_equal(to_host(fwd["offsets"]), offsets)
    rng = np.random.default_rng(s.seed + 6)
    toks = np.sort(rng.choice(s.T, 64, replace=False)).astype(np.int32)
    dx_ref = orc.backward_dx_tokens(s, toks, inp.x, inp.w1, inp.w2, idx, w, inp.dy)
    dx = to_host(bwd["dx"])[toks]
    assert rel_err(decode("bf16", dx), decode("bf16", dx_ref)) < TOL["bf16"]
    dw1, dw2 = to_host(bwd["dw1"]), to_host(bwd["dw2"])
    empty = np.where(counts == 0)[0]
    print(f"skewed routing: {len(empty)} empty experts, max count {int(counts.max())}")
    assert np.all(dw1[empty] == 0) and np.all(dw2[empty] == 0)
    assert np.all(np.isfinite(dw1)) and np.all(np.isfinite(dw2))
    # sampled weight-gradient entries of three experts with 1..3000 rows
    cand = np.where((counts > 0) & (counts <= 3000))[0]
    experts = cand[np.linspace(0, len(cand) - 1, 3).astype(int)]
    for e in experts:
        i2 = np.stack([rng.integers(0, s.H, 24), rng.integers(0, s.F, 24)], 1)
        i1 = np.stack([rng.integers(0, 2 * s.F, 24), rng.integers(0, s.H, 24)], 1)
        d2, d1 = orc.backward_dw_entries(s, int(e), inp.x, inp.w1, inp.w2, w, src_map, offsets, inp.dy, i2, i1)
        assert rel_err(dw2[e][i2[:, 0], i2[:, 1]], d2) < TOL["bf16"], f"dW2 of expert {e}"
        assert rel_err(dw1[e][i1[:, 0], i1[:, 1]], d1) < TOL["bf16"], f"dW1 of expert {e}"


def test_backward_graph_capture_replays():
    s = [x for x in wl.small_shapes() if x.name == "small_skewed_bf16"][0]
    inp = Inputs(s, want_dy=True)
    fwd = run_forward(inp, training=True, poison=False)
    cfg = cfg_of(s)
    bwd = moe.alloc_backward(cfg)
    d = inp.dev
    moe.moe_backward(cfg, d["dy"], d["w1"], d["w2"], fwd, bwd)
    torch.cuda.synchronize()
    eager = {k: to_host(bwd[k]).copy() for k in ("dx", "dw1", "dw2")}
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            moe.moe_backward(cfg, d["dy"], d["w1"], d["w2"], fwd, bwd)
    for rep in range(3):
        for k in ("dx", "dw1", "dw2"):
            bwd[k].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for k, v in eager.items():
            assert np.array_equal(to_host(bwd[k]).view(np.uint8), v.view(np.uint8)), f"replay {rep}: {k}"
