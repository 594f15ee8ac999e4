"""GPU parity of the FFN backward (combine backward, down-projection backward
fused with the SwiGLU backward, gate/up backward, permute backward) against
the CPU oracle, through the C ABI.

Small shapes (skewed routing; 16-row group alignment), a shape whose experts
exceed the 4096-row unit of its weight gradients, and the full-size skewed
workload (T=16384, H=2048, F=768, E=128, top-8, Zipf-biased routing): every
gradient compared in full, normwise and element by element, and dW of every
empty expert exactly zero (it starts as NaN)."""
import numpy as np
import pytest
import torch

import routing_permute_grouped_router_amd as moe
from oracle import oracle as orc
from routing_permute_grouped_router_amd import workload as wl

from helpers import Inputs, assert_parity, cfg_of, decode, run_forward, to_host

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
        assert_parity(decode("bf16", to_host(bwd[key])[:n]), decode("bf16", g[key][:n]), "bf16", key)
    assert_parity(decode("bf16", to_host(bwd["dx"])), decode("bf16", g["dx"]), "bf16", "dX")
    dw1, dw2 = to_host(bwd["dw1"]), to_host(bwd["dw2"])
    assert np.all(np.isfinite(dw1)) and np.all(np.isfinite(dw2))
    assert_parity(dw1, g["dw1"], "f32acc", "dW1")
    assert_parity(dw2, g["dw2"], "f32acc", "dW2")
    if s.align > 1:
        pad = src_map[:n] < 0
        assert pad.any(), "the alignment should leave padding rows"
        assert np.all(to_host(bwd["dyp"])[:n][pad] == 0)
    empty = np.where(counts == 0)[0]
    if name == "small_skewed_bf16":
        assert len(empty) > 0, "the skewed routing should leave some experts empty"
    assert np.all(dw1[empty] == 0) and np.all(dw2[empty] == 0)


def test_backward_split_wgrad_full_parity():
    """Experts with more than 4096 rows: the weight gradients contract over
    such an expert in units of at most 4096 rows, write float32 partial sums
    per unit and add them in unit order in a second kernel.  Logit biases send
    every token to expert 0 (12288 rows: 3 full units), 10000 tokens to expert
    1 (3 units, the last one ragged) and the other 2288 to expert 2 (one unit,
    written directly); the rest stay empty.  Every gradient is compared in full."""
    s = wl.MoEShape("split_wgrad_bf16", 12288, 128, 64, 8, 2, "softmax", False, "bf16", backward=True,
                    seed=2011)
    inp = Inputs(s, want_dy=True)
    lg = inp.logits.astype(np.float64)
    lg[:, 0] += 16.0
    lg[:10000, 1] += 8.0
    lg[10000:, 2] += 8.0
    inp.logits = lg.astype(np.float32)
    fwd = run_forward(inp, training=True)
    bwd = _run_backward(inp, fwd)
    idx, w = orc.route(inp.logits, s.k, s.score, s.renorm)
    counts, offsets, row_map, src_map, _ = orc.group(idx, s.E, s.align)
    assert counts.tolist() == [12288, 10000, 2288, 0, 0, 0, 0, 0]
    assert np.array_equal(to_host(fwd["counts"]), counts)
    ref = orc.forward_tokens(s, np.arange(s.T), inp.x, inp.w1, inp.w2, idx, w, want_stash=True)
    R = src_map.shape[0]
    h_rows = np.zeros((R, s.F), np.uint16)
    st_rows = np.zeros((R, 2 * s.F), np.uint16)
    rm = row_map.ravel()
    h_rows[rm] = ref["h"].reshape(-1, s.F)
    st_rows[rm] = ref["stash"].reshape(-1, 2 * s.F)
    g = orc.backward(s, inp.x, inp.w1, inp.w2, w, row_map, src_map, offsets, h_rows, st_rows, inp.dy)
    dw1, dw2 = to_host(bwd["dw1"]), to_host(bwd["dw2"])
    assert np.all(np.isfinite(dw1)) and np.all(np.isfinite(dw2))
    for e in range(3):
        assert_parity(dw1[e], g["dw1"][e], "f32acc", f"dW1 of expert {e}")
        assert_parity(dw2[e], g["dw2"][e], "f32acc", f"dW2 of expert {e}")
    assert np.all(dw1[3:] == 0) and np.all(dw2[3:] == 0)
    assert_parity(decode("bf16", to_host(bwd["dx"])), decode("bf16", g["dx"]), "bf16", "dX")


def _backward_experts(s, inp, w, src_map, offsets, row_map):
    """The oracle's backward of every expert (expert-major float64 form),
    assembled into the layer's gradients."""
    R = src_map.shape[0]
    g = {"dyp": np.zeros((R, s.H), np.uint16), "dgu": np.zeros((R, 2 * s.F), np.uint16),
         "dxp": np.zeros((R, s.H), np.uint16), "dw1": np.zeros((s.E, 2 * s.F, s.H), np.float32),
         "dw2": np.zeros((s.E, s.H, s.F), np.float32)}
    for e in range(s.E):
        b = orc.backward_expert(s, e, inp.x, inp.w1, inp.w2, w, src_map, offsets, inp.dy)
        g["dw1"][e], g["dw2"][e] = b["dw1"], b["dw2"]
        if b["rows"].size:
            for key in ("dyp", "dgu", "dxp"):
                g[key][b["rows"]] = b[key]
    g["dx"] = orc.combine(g["dxp"], row_map, None, "bf16")  # dX[t] = sum_j dXp[row_map[t, j]]
    return g


def test_backward_full_size_skewed():
    """The skewed layer (T=16384, H=2048, F=768, E=128, top-8) in the launch
    configuration the benchmark times, every gradient compared in full with
    the oracle's expert-major form: dYp, dGU, dXp and dX, and dW1 / dW2 of
    every expert, the split hot experts included (the weight-gradient unit is
    max(4096, T k tiles / 512) rows rounded down to 64: 12288 rows for dW1's
    6 x 8 tiles, 6144 for dW2's 8 x 3)."""
    s = wl.BY_NAME["skewed_bf16"]
    inp = Inputs(s, want_dy=True)
    fwd = run_forward(inp, training=True, poison=False)
    bwd = _run_backward(inp, fwd)
    idx, w = orc.route(inp.logits, s.k, s.score, s.renorm)
    counts, offsets, row_map, src_map, _ = orc.group(idx, s.E, s.align)
    assert np.array_equal(to_host(fwd["offsets"]), offsets)
    empty = np.where(counts == 0)[0]
    unit_dw1 = s.T * s.k * 48 // 512 // 64 * 64
    unit_dw2 = s.T * s.k * 24 // 512 // 64 * 64
    assert (unit_dw1, unit_dw2) == (12288, 6144)
    print(f"skewed routing: {len(empty)} empty experts, max count {int(counts.max())}, "
          f"{int((counts > unit_dw1).sum())} / {int((counts > unit_dw2).sum())} experts split for dW1 / dW2")
    assert (counts > unit_dw1).sum() >= 3, "the hot experts should take the split weight-gradient path"
    g = _backward_experts(s, inp, w, src_map, offsets, row_map)
    n = int(offsets[-1])
    for key in ("dyp", "dgu", "dxp"):
        assert_parity(decode("bf16", to_host(bwd[key])[:n]), decode("bf16", g[key][:n]), "bf16", key)
    assert_parity(decode("bf16", to_host(bwd["dx"])), decode("bf16", g["dx"]), "bf16", "dX")
    dw1, dw2 = to_host(bwd["dw1"]), to_host(bwd["dw2"])
    assert np.all(dw1[empty] == 0) and np.all(dw2[empty] == 0)
    assert np.all(np.isfinite(dw1)) and np.all(np.isfinite(dw2))
    hot = np.argsort(-counts, kind="stable")[:3]
    for e in list(hot) + [e for e in range(s.E) if 0 < counts[e] <= unit_dw2][:3]:
        assert_parity(dw1[e], g["dw1"][e], "f32acc", f"dW1 of expert {e} ({counts[e]} rows)")
        assert_parity(dw2[e], g["dw2"][e], "f32acc", f"dW2 of expert {e} ({counts[e]} rows)")
    assert_parity(dw1, g["dw1"], "f32acc", "dW1")
    assert_parity(dw2, g["dw2"], "f32acc", "dW2")
    # The two hottest (split) experts against float64 products of the call's
    # own bf16 operands (torch float64 matmuls on the device): only the float32
    # accumulation and the order in which the units' partial sums are added
    # separate them, so a unit, slot or reduction fault cannot hide in the
    # rounding flips that the oracle comparison has to allow.
    for e in hot[:2]:
        r = slice(int(offsets[e]), int(offsets[e + 1]))
        pairs = (("dW2", bwd["dw2"][e], bwd["dyp"][r], fwd["h"][r]), ("dW1", bwd["dw1"][e], bwd["dgu"][r], fwd["xp"][r]))
        for name, got, a, b in pairs:
            ref = torch.mm(a.to(torch.float64).t().contiguous(), b.to(torch.float64))
            err = float((got.to(torch.float64) - ref).abs().max())
            top = float(ref.abs().max())
            print(f"{name} of expert {e} ({counts[e]} rows) against its own operands: max error {err / top:.2e} of the maximum")
            assert err <= 2.0 ** -14 * top, (name, int(e), err, top)


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
