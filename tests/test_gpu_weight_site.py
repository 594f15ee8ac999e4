"""The routing weight applied in the gate/up (FC1) or down (FC2) epilogue
(moe_config.weight_site, the weighted GEMM entry points and the unweighted
combine) against the oracle's placements, through the C ABI.

Small shapes of every storage format, in both forms of the gate/up GEMM
(materialised Xp and gather), and shapes whose tiles are cut along K (the
reduction kernel applies the weight there): h, Yp of every routed row and y
against the oracle, padding rows zero.  The staged calls equal moe_forward
bit for bit.  Full-size fine-grained bf16 and DeepSeek-shaped MXFP8 layers on
seeded token samples."""
import dataclasses

import numpy as np
import pytest
import torch

import routing_permute_grouped_router_amd as moe
from oracle import oracle as orc
from routing_permute_grouped_router_amd import workload as wl

from helpers import TOL, cfg_of, decode, rel_err, to_host
from test_gpu_forward import SPLIT_K
from test_gpu_gather import SPLIT_K_ALIGN, _inputs, _mx_full, _run

pytestmark = pytest.mark.gpu


def _host(t):
    return None if t is None else to_host(t)


def _check(s, site, args, buf, toks=None, limit=0.0):
    logits, x, w1, w2, scales = args
    idx, w = orc.route(to_host(logits), s.k, s.score, s.renorm)
    counts, offsets, row_map, src_map, _ = orc.group(idx, s.E, s.align)
    if toks is None:
        toks = np.arange(s.T)
        hw = {"w1": _host(w1), "w2": _host(w2), "w1_scale": _host(scales.get("w1_scale")),
              "w2_scale": _host(scales.get("w2_scale"))}
    else:
        # host copies of the experts the sample uses only (the rest stay zero pages)
        hw = {}
        for k, t in (("w1", w1), ("w2", w2), ("w1_scale", scales.get("w1_scale")), ("w2_scale", scales.get("w2_scale"))):
            if t is not None:
                hw[k] = np.zeros(tuple(t.shape), to_host(t[:1]).dtype)
                for e in np.unique(idx[toks]):
                    if e >= 0:
                        hw[k][e] = to_host(t[int(e)])
    ref = orc.forward_tokens(s, toks, _host(x), hw["w1"], hw["w2"], idx, w, _host(scales.get("x_scale")),
                             hw.get("w1_scale"), hw.get("w2_scale"), site=site, limit=limit)
    f = s.dtype
    rows = row_map[toks].ravel()
    ok = rows >= 0
    rows = rows[ok]
    ridx = torch.from_numpy(rows).long().cuda()
    h = to_host(buf["h"][ridx])
    h_ref = ref["h"].reshape(-1, s.F)[ok]
    if f == "mxfp8":
        hd = decode(f, h, to_host(buf["h_scale"][ridx]))
        hr = decode(f, h_ref, ref["h_scale"].reshape(-1, s.F // 32)[ok])
    else:
        hd, hr = decode(f, h), decode(f, h_ref)
    if f == "mxfp8" and limit > 0:
        # The clamp caps h's maximum (at silu(L) L, times the row's weight when
        # this epilogue applies it), so a one-step E4M3 rounding flip in the top
        # binade (up to 2^-3 of the element) is no longer diluted by the
        # tensor's outliers.  Such a flip is where the kernel's float32 and the
        # oracle's float64 put a value on opposite sides of a rounding boundary:
        # same sign and scale, codes one apart, and the oracle's unrounded value
        # at the midpoint of the two decoded values (within 1e-4).  Flips are
        # counted apart (under 2 % of the codes); the rest of h keeps the MXFP8
        # bar.
        ex = orc.forward_experts(s, toks, _host(x), hw["w1"], hw["w2"], idx, w, _host(scales.get("x_scale")),
                                 hw.get("w1_scale"), hw.get("w2_scale"), site=site, limit=limit, want_h_f64=True)
        assert np.array_equal(ex["h"].reshape(-1, s.F)[ok], h_ref), "expert-major form"
        h64 = ex["h_f64"].reshape(-1, s.F)[ok]
        cg, cr = h.astype(np.int32), h_ref.astype(np.int32)
        sg = np.repeat(to_host(buf["h_scale"][ridx]), 32, axis=1)
        sr = np.repeat(ref["h_scale"].reshape(-1, s.F // 32)[ok], 32, axis=1)
        step = ((cg ^ cr) < 0x80) & (np.abs((cg & 0x7F) - (cr & 0x7F)) == 1) & (sg == sr)
        mid = (hd + hr) / 2
        at_mid = np.abs(h64 - mid) <= 1e-4 * np.abs(h64)
        flip = (hd != hr) & step & at_mid
        assert rel_err(hd[~flip], hr[~flip]) < TOL[f], "h apart from rounding flips"
        assert np.mean(flip) < 0.02, f"h: {np.mean(flip):.4f} of the codes are rounding flips"
    else:
        assert rel_err(hd, hr) < TOL[f], "h"
    yp = decode(s.out_dtype, to_host(buf["yp"][ridx]))
    assert rel_err(yp, decode(s.out_dtype, ref["yp"].reshape(-1, s.H)[ok])) < TOL[f], "yp"
    y = decode(s.out_dtype, to_host(buf["y"])[toks])
    assert rel_err(y, decode(s.out_dtype, ref["y"])) < TOL[f], "y"
    # padding rows of a group (weight 0) are zero in h and in Yp
    pad = np.nonzero(src_map[: offsets[-1]] < 0)[0]
    if len(pad) and toks.size == s.T:
        assert np.all(to_host(buf["h"])[pad].view(np.uint8) == 0)
        assert np.all(decode(s.out_dtype, to_host(buf["yp"])[pad]) == 0)
    return ref


@pytest.mark.parametrize("gather", [False, True], ids=["xp", "gather"])
@pytest.mark.parametrize("site", ["fc1", "fc2"])
@pytest.mark.parametrize("shape", [wl.BY_NAME["tiny_f32"]] + wl.small_shapes() + SPLIT_K + [SPLIT_K_ALIGN],
                         ids=lambda s: s.name)
def test_weight_site_small(shape, site, gather):
    args = _inputs(shape)
    cfg = dataclasses.replace(cfg_of(shape), weight_site=site)
    buf = _run(cfg, *args, gather=gather)
    _check(shape, site, args, buf)


@pytest.mark.parametrize("site", ["fc1", "fc2"])
@pytest.mark.parametrize("name", ["small_bf16_sigmoid_align", "small_mxfp8_skew_align"])
def test_staged_weighted_calls_equal_forward(name, site):
    s = next(x for x in wl.small_shapes() if x.name == name)
    logits, x, w1, w2, sc = _inputs(s)
    cfg = dataclasses.replace(cfg_of(s), weight_site=site)
    fused = _run(cfg, logits, x, w1, w2, sc, gather=False)
    b = moe.alloc_forward(cfg)
    moe.moe_route(cfg, logits, b["idx"], b["w"])
    moe.moe_permute(cfg, x, b["idx"], b["xp"], b["counts"], b["offsets"], b["row_map"], b["src_map"], b["ws"],
                    x_scale=sc.get("x_scale"), xp_scale=b.get("xp_scale"))
    mx = dict(xp_scale=b.get("xp_scale"), w1_scale=sc.get("w1_scale"), h_scale=b.get("h_scale"))
    if site == "fc1":
        moe.moe_grouped_swiglu_gemm_weighted(cfg, b["xp"], w1, b["offsets"], b["src_map"], b["w"], b["h"], b["ws"],
                                             **mx)
        moe.moe_grouped_down_gemm(cfg, b["h"], w2, b["offsets"], b["yp"], b["ws"], h_scale=b.get("h_scale"),
                                  w2_scale=sc.get("w2_scale"))
    else:
        moe.moe_grouped_swiglu_gemm(cfg, b["xp"], w1, b["offsets"], b["h"], b["ws"], **mx)
        moe.moe_grouped_down_gemm_weighted(cfg, b["h"], w2, b["offsets"], b["src_map"], b["w"], b["yp"], b["ws"],
                                           h_scale=b.get("h_scale"), w2_scale=sc.get("w2_scale"))
    moe.moe_combine(cfg, b["yp"], b["row_map"], None, b["y"])
    torch.cuda.synchronize()
    n = int(to_host(b["offsets"])[-1])
    for k in ("h", "h_scale", "yp"):
        if b.get(k) is not None:
            assert np.array_equal(to_host(b[k])[:n].view(np.uint8), to_host(fused[k])[:n].view(np.uint8)), k
    assert np.array_equal(to_host(b["y"]).view(np.uint8), to_host(fused["y"]).view(np.uint8)), "y"


@pytest.mark.parametrize("name,site", [("finegrained_bf16", "fc2"), ("deepseek_mxfp8", "fc1")])
def test_weight_site_full_size(name, site):
    """Gather form with the weight in an epilogue, the launch configuration
    the benchmark's variants time; floats on a seeded token sample."""
    s = wl.BY_NAME[name]
    args = _mx_full(s) if s.dtype == "mxfp8" else _inputs(s)
    cfg = dataclasses.replace(cfg_of(s), weight_site=site)
    buf = _run(cfg, *args, gather=True)
    rng = np.random.default_rng(s.seed + 6)
    toks = np.sort(rng.choice(s.T, 64, replace=False)).astype(np.int32)
    _check(s, site, args, buf, toks)
