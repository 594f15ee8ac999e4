"""moe_forward_noalloc (the forward with the library's static scratch array
instead of a caller workspace) against moe_forward, through the C ABI: every
output byte for byte, on two calls in a row, the second on a smaller input (the
array keeps the first call's contents), for bf16 with the per-row epilogue
weights and the SwiGLU clamp, and for MXFP8 and MXFP4."""
import numpy as np
import pytest
import torch

import routing_permute_grouped_router_amd as moe
from routing_permute_grouped_router_amd import workload as wl

from helpers import Inputs, decode, to_host

pytestmark = pytest.mark.gpu

OUTS = ("y", "idx", "w", "counts", "offsets", "row_map", "src_map", "h", "yp")


def _run(inp, cfg, noalloc):
    buf = moe.alloc_forward(cfg)
    for k in ("xp", "h", "yp", "y"):
        if buf[k].dtype.is_floating_point:
            buf[k].fill_(float("nan"))
    if noalloc:
        buf["ws"].fill_(0)  # not used by the no-allocation form
    d = inp.dev
    fn = moe.moe_forward_noalloc if noalloc else moe.moe_forward
    fn(cfg, d["logits"], d["x"], d["w1"], d["w2"], buf, x_scale=d.get("x_scale"), w1_scale=d.get("w1_scale"),
       w2_scale=d.get("w2_scale"))
    torch.cuda.synchronize()
    n = int(to_host(buf["offsets"])[-1])
    out = {}
    for k in OUTS:
        v = to_host(buf[k])
        out[k] = v[:n] if k in ("h", "yp", "src_map") else v
    return out


def _same(a, b, label):
    for k in OUTS:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), f"{label}: {k} differs"


@pytest.mark.parametrize("first,second,site,limit", [
    ("finegrained_bf16", "small_bf16_renorm", "combine", 0.0),
    ("small_bf16_sigmoid_align", "small_bf16_softmax", "fc2", 7.0),
    ("small_mxfp8", "small_mxfp8_k512", "fc1", 0.0),
    ("small_mxfp4", "small_mxfp4_align128", "combine", 0.0),
])
def test_noalloc_forward_matches_forward_twice(first, second, site, limit):
    shapes = {s.name: s for s in wl.small_shapes() + wl.mxfp4_shapes() + wl.WORKLOADS}
    for name in (first, second):  # the second call is smaller than the first
        s = shapes[name]
        cfg = moe.MoEConfig(s.T, s.H, s.F, s.E, s.k, s.align, s.score, bool(s.renorm), s.dtype, site, limit)
        inp = Inputs(s)
        ref = _run(inp, cfg, noalloc=False)
        got = _run(inp, cfg, noalloc=True)
        _same(got, ref, name)
        assert np.all(np.isfinite(decode("f32" if s.dtype == "f32" else "bf16", got["y"])))
    assert shapes[second].T * shapes[second].k < shapes[first].T * shapes[first].k
