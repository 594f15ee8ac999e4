"""The optional SwiGLU clamp (moe_config.swiglu_limit: h = silu(min(g, L)) *
clamp(u, -L, L), gradients zero where a bound is exceeded) against the
oracle, through the C ABI.

Forward: every storage format on the small shapes, both forms of the gate/up
GEMM, tiles cut along K (the reduction kernel clamps there), the clamp
together with the routing weight in the FC1 epilogue, and the full-size
DeepSeek-shaped MXFP8 layer on a token sample.  Backward (bf16): the stash
keeps the unclamped g and u, and every gradient matches the oracle's."""
import dataclasses

import numpy as np
import pytest
import torch

import routing_permute_grouped_router_amd as moe
from oracle import oracle as orc
from routing_permute_grouped_router_amd import workload as wl

from helpers import Inputs, TOL, cfg_of, decode, rel_err, to_host
from test_gpu_forward import SPLIT_K
from test_gpu_gather import SPLIT_K_ALIGN, _inputs, _mx_full, _run
from test_gpu_weight_site import _check

pytestmark = pytest.mark.gpu

LIMIT = 0.75  # the gate/up values of these inputs are ~N(0, 1): a third or more are clamped


@pytest.mark.parametrize("gather", [False, True], ids=["xp", "gather"])
@pytest.mark.parametrize("shape", [wl.BY_NAME["tiny_f32"]] + wl.small_shapes() + SPLIT_K + [SPLIT_K_ALIGN],
                         ids=lambda s: s.name)
def test_clamp_forward_small(shape, gather):
    args = _inputs(shape)
    cfg = dataclasses.replace(cfg_of(shape), swiglu_limit=LIMIT)
    _check(shape, "combine", args, _run(cfg, *args, gather=gather), limit=LIMIT)


@pytest.mark.parametrize("name", ["small_bf16_renorm", "small_mxfp8"])
def test_clamp_with_weight_in_fc1(name):
    s = wl.BY_NAME.get(name) or next(x for x in wl.small_shapes() if x.name == name)
    args = _inputs(s)
    cfg = dataclasses.replace(cfg_of(s), swiglu_limit=LIMIT, weight_site="fc1")
    _check(s, "fc1", args, _run(cfg, *args, gather=True), limit=LIMIT)


def test_clamp_forward_full_size_mxfp8():
    s = wl.BY_NAME["deepseek_mxfp8"]
    args = _mx_full(s)
    cfg = dataclasses.replace(cfg_of(s), swiglu_limit=LIMIT)
    buf = _run(cfg, *args, gather=False)
    toks = np.sort(np.random.default_rng(s.seed + 7).choice(s.T, 48, replace=False)).astype(np.int32)
    _check(s, "combine", args, buf, toks, limit=LIMIT)


@pytest.mark.parametrize("name", ["small_skewed_bf16", "small_bf16_sigmoid_align"])
def test_clamp_backward_small(name):
    s = next(x for x in wl.small_shapes() if x.name == name)
    inp = Inputs(s, want_dy=True)
    d = inp.dev
    cfg = dataclasses.replace(cfg_of(s), swiglu_limit=LIMIT)
    fwd = moe.alloc_forward(cfg, training=True)
    moe.moe_forward(cfg, d["logits"], d["x"], d["w1"], d["w2"], fwd)
    bwd = moe.alloc_backward(cfg)
    for k in ("dyp", "dgu", "dxp", "dx", "dw1", "dw2"):
        bwd[k].fill_(float("nan"))
    moe.moe_backward(cfg, d["dy"], d["w1"], d["w2"], fwd, bwd)
    torch.cuda.synchronize()
    idx, w = orc.route(inp.logits, s.k, s.score, s.renorm)
    counts, offsets, row_map, src_map, _ = orc.group(idx, s.E, s.align)
    ref = orc.forward_tokens(s, np.arange(s.T), inp.x, inp.w1, inp.w2, idx, w, want_stash=True, limit=LIMIT)
    rm = row_map.ravel()
    # the stash holds the unclamped g and u; h the clamped activation
    st = ref["stash"].reshape(-1, 2 * s.F)
    assert rel_err(decode("bf16", to_host(fwd["gu_stash"])[rm]), decode("bf16", st)) < TOL["bf16"]
    assert np.mean(np.abs(decode("bf16", st)) > LIMIT) > 0.2
    assert rel_err(decode("bf16", to_host(fwd["h"])[rm]), decode("bf16", ref["h"].reshape(-1, s.F))) < TOL["bf16"]
    R = src_map.shape[0]
    h_rows = np.zeros((R, s.F), np.uint16)
    st_rows = np.zeros((R, 2 * s.F), np.uint16)
    h_rows[rm] = ref["h"].reshape(-1, s.F)
    st_rows[rm] = st
    g = orc.backward(s, inp.x, inp.w1, inp.w2, w, row_map, src_map, offsets, h_rows, st_rows, inp.dy, limit=LIMIT)
    n = int(offsets[-1])
    for key in ("dgu", "dxp"):
        assert rel_err(decode("bf16", to_host(bwd[key])[:n]), decode("bf16", g[key][:n])) < TOL["bf16"], key
    assert rel_err(decode("bf16", to_host(bwd["dx"])), decode("bf16", g["dx"])) < TOL["bf16"]
    assert rel_err(to_host(bwd["dw1"]), g["dw1"]) < TOL["bf16"]
    assert rel_err(to_host(bwd["dw2"]), g["dw2"]) < TOL["bf16"]
    # a clamped gate or up value passes no gradient
    dgu = decode("bf16", to_host(bwd["dgu"])[rm])
    sv = decode("bf16", st)
    assert np.all(dgu[:, : s.F][sv[:, : s.F] > LIMIT] == 0)
    assert np.all(dgu[:, s.F:][np.abs(sv[:, s.F:]) > LIMIT] == 0)


@pytest.mark.parametrize("name", ["small_bf16_sigmoid_align", "small_mxfp8_skew_align"])
def test_variant_forward_graph_capture_replays(name):
    """The gather form with the weight in the FC2 epilogue and the clamp
    (per-row weights written by a kernel into the workspace) captures into a
    HIP graph; replays, with eager work between them, give the eager bytes."""
    s = next(x for x in wl.small_shapes() if x.name == name)
    logits, x, w1, w2, sc = _inputs(s)
    cfg = dataclasses.replace(cfg_of(s), swiglu_limit=LIMIT, weight_site="fc2")
    buf = moe.alloc_forward(cfg)
    buf["xp"] = None
    buf["xp_scale"] = None
    moe.moe_forward(cfg, logits, x, w1, w2, buf, **sc)
    torch.cuda.synchronize()
    keys = [k for k, v in buf.items() if v is not None and k not in ("ws", "err")]
    eager = {k: to_host(buf[k]).copy() for k in keys}
    n = int(eager["offsets"][-1])
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            moe.moe_forward(cfg, logits, x, w1, w2, buf, **sc)
    for rep in range(3):
        buf["y"].fill_(float("nan"))
        buf["yp"].fill_(float("nan"))
        buf["h"].fill_(0x5A if buf["h"].dtype == torch.uint8 else float("nan"))
        buf["ws"].fill_(0x77)  # the per-row weights must be rewritten on every replay
        g.replay()
        torch.cuda.synchronize()
        _ = (logits * 2).sum().item()  # unrelated eager work between replays
        for k in keys:
            got, v = to_host(buf[k]), eager[k]
            if k in ("h", "h_scale", "yp", "src_map"):
                got, v = got[:n], v[:n]
            assert np.array_equal(got.view(np.uint8), v.view(np.uint8)), f"replay {rep}: {k} differs"
