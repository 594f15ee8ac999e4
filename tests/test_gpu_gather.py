"""The gather form of the gate/up GEMM (moe_forward with xp = None: row r of
the grouped operand read as x[src_map[r] / k], no materialised Xp) against the
materialised path, bit for bit: h (+ h_scale), Yp over the used rows
[0, offsets[E]) (padding rows zero in both) and y.  The materialised path is
itself checked against the oracle in test_gpu_forward / test_gpu_mxfp8.

Small shapes of every storage format (ragged groups, 16-row alignment, empty
experts), tiles cut along K with padding rows (their partial sums go through
the reduction kernel, which zeroes padding rows), and the full-size
fine-grained and DeepSeek-shaped layers."""
import numpy as np
import pytest
import torch

import routing_permute_grouped_router_amd as moe
from routing_permute_grouped_router_amd import workload as wl

from helpers import Inputs, cfg_of, to_dev, to_host

pytestmark = pytest.mark.gpu

SPLIT_K_ALIGN = wl.MoEShape("split_k_gateup_align_bf16", 1024, 4096, 128, 8, 2, "softmax", False, "bf16",
                            align=16, seed=2008)


def _inputs(s):
    """(logits, x, w1, w2, scales) on the device."""
    if s.dtype != "mxfp8":
        inp = Inputs(s)
        d = inp.dev
        return d["logits"], d["x"], d["w1"], d["w2"], {}
    from test_gpu_mxfp8 import _gpu_quantize
    w = wl.Workload(s)
    xq, xs = _gpu_quantize(w.x())
    w1q, w1s = _gpu_quantize(w.w1())
    w2q, w2s = _gpu_quantize(w.w2())
    return to_dev(w.logits(), "f32"), xq, w1q, w2q, dict(x_scale=xs, w1_scale=w1s, w2_scale=w2s)


def _mx_full(s):
    """A full-size MXFP8 layer: weights generated and quantised expert by expert."""
    from test_gpu_mxfp8 import _gpu_quantize
    w = wl.Workload(s)
    xq, xs = _gpu_quantize(w.x())
    u8 = dict(dtype=torch.uint8, device="cuda")
    w1q, w1s = torch.empty(s.E, 2 * s.F, s.H, **u8), torch.empty(s.E, 2 * s.F, s.H // 32, **u8)
    w2q, w2s = torch.empty(s.E, s.H, s.F, **u8), torch.empty(s.E, s.H, s.F // 32, **u8)
    step = 16
    for e0 in range(0, s.E, step):
        t1, t2 = to_dev(w.w1(e0, e0 + step), "f32"), to_dev(w.w2(e0, e0 + step), "f32")
        moe.moe_quantize_mxfp8(t1, w1q[e0:e0 + step], w1s[e0:e0 + step])
        moe.moe_quantize_mxfp8(t2, w2q[e0:e0 + step], w2s[e0:e0 + step])
        del t1, t2
    return to_dev(w.logits(), "f32"), xq, w1q, w2q, dict(x_scale=xs, w1_scale=w1s, w2_scale=w2s)


def _run(cfg, logits, x, w1, w2, scales, gather):
    buf = moe.alloc_forward(cfg)
    for k in ("h", "yp", "y"):
        if buf[k].dtype.is_floating_point:
            buf[k].fill_(float("nan"))
        else:
            buf[k].fill_(0x5A)
    if gather:
        buf["xp"] = None
        buf["xp_scale"] = None
    moe.moe_forward(cfg, logits, x, w1, w2, buf, **scales)
    torch.cuda.synchronize()
    return buf


def _same(a, b, n):
    for k in ("h", "h_scale", "yp"):
        if k in a and a[k] is not None:
            assert np.array_equal(to_host(a[k])[:n].view(np.uint8), to_host(b[k])[:n].view(np.uint8)), k
    assert np.array_equal(to_host(a["y"]).view(np.uint8), to_host(b["y"]).view(np.uint8)), "y"


@pytest.mark.parametrize("shape", wl.small_shapes() + [SPLIT_K_ALIGN], ids=lambda s: s.name)
def test_gather_matches_materialised_small(shape):
    cfg = cfg_of(shape)
    args = _inputs(shape)
    a = _run(cfg, *args, gather=False)
    b = _run(cfg, *args, gather=True)
    n = int(to_host(a["offsets"])[-1])
    assert np.array_equal(to_host(a["offsets"]), to_host(b["offsets"]))
    _same(a, b, n)
    if shape.align > 1:  # padding rows of h are zero in the gather form too
        pad = to_host(b["src_map"])[:n] < 0
        assert pad.any() and not to_host(b["h"])[:n][pad].view(np.uint8).any()


def test_gather_split_k_shape_cuts_tiles():
    """The aligned split-K shape above does take the K-split path."""
    from test_gpu_forward import _split_tiles
    s = SPLIT_K_ALIGN
    cfg = cfg_of(s)
    a = _run(cfg, *_inputs(s), gather=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert _split_tiles(to_host(a["offsets"]), s.R_cap, s.E, s.H, s.F, 128, cus) > 0


@pytest.mark.parametrize("name", ["finegrained_bf16", "deepseek_mxfp8"])
def test_gather_matches_materialised_full_size(name):
    s = wl.BY_NAME[name]
    cfg = cfg_of(s)
    args = _mx_full(s) if s.dtype == "mxfp8" else _inputs(s)
    a = _run(cfg, *args, gather=False)
    b = _run(cfg, *args, gather=True)
    _same(a, b, int(to_host(a["offsets"])[-1]))
