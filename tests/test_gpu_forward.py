"""GPU parity of the forward hot path against the CPU oracle, through the C ABI.

Integers (idx, counts, offsets, row_map, src_map, permuted rows) must match
bit for bit; floats within the normwise tolerance of their storage format
(f32 1e-5, bf16 2e-2) and, element by element, within one storage step plus a
small share of the tensor's maximum (helpers.ELEM_BOUNDS) for 99.9 % of the
elements.  Small shapes are compared in full.  At full size every integer
output is compared in full; the float outputs of the fine-grained and skewed
layers in full, those of the Mixtral-shaped layer on 1024 seeded tokens (a
token's output depends only on its row and the weights)."""
import numpy as np
import pytest
import torch

import routing_permute_grouped_router_amd as moe
from oracle import oracle as orc
from routing_permute_grouped_router_amd import workload as wl

from helpers import Inputs, TOL, assert_parity, cfg_of, decode, rel_err, run_forward, to_dev, to_host

pytestmark = pytest.mark.gpu

SMALL = [s for s in wl.small_shapes() if s.dtype != "mxfp8"]


def _check_routing(inp, buf):
    s = inp.s
    idx_o, w_o = orc.route(inp.logits, s.k, s.score, s.renorm)
    assert np.array_equal(to_host(buf["idx"]), idx_o), "idx differs"
    assert rel_err(to_host(buf["w"]), w_o) < 1e-5
    counts, offsets, row_map, src_map, bad = orc.group(idx_o, s.E, s.align)
    assert np.array_equal(to_host(buf["counts"]), counts)
    assert np.array_equal(to_host(buf["offsets"]), offsets)
    assert np.array_equal(to_host(buf["row_map"]), row_map)
    assert np.array_equal(to_host(buf["src_map"]), src_map)
    return idx_o, w_o, counts, offsets, row_map, src_map


def _check_xp(inp, buf, row_map, offsets):
    xp_o = orc.permute(inp.x, row_map, int(offsets[-1]))
    xp = to_host(buf["xp"])[: offsets[-1]]
    assert np.array_equal(xp.view(np.uint8), xp_o.view(np.uint8)), "permuted rows differ"


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: s.name)
def test_forward_small_full_parity(shape):
    inp = Inputs(shape)
    buf = run_forward(inp, training=True)
    s = shape
    idx, w, counts, offsets, row_map, src_map = _check_routing(inp, buf)
    _check_xp(inp, buf, row_map, offsets)
    ref = orc.forward_tokens(s, np.arange(s.T), inp.x, inp.w1, inp.w2, idx, w, want_stash=True)
    rm = row_map.ravel()
    f = s.dtype
    h = to_host(buf["h"])
    yp = to_host(buf["yp"])
    st = to_host(buf["gu_stash"])
    assert_parity(decode(f, h[rm]), decode(f, ref["h"].reshape(-1, s.F)), f, "h")
    assert_parity(decode(s.out_dtype, yp[rm]), decode(s.out_dtype, ref["yp"].reshape(-1, s.H)), f, "Yp")
    assert_parity(decode(s.out_dtype, st[rm]), decode(s.out_dtype, ref["stash"].reshape(-1, 2 * s.F)), f, "stash")
    y = decode(s.out_dtype, to_host(buf["y"]))
    assert_parity(y, decode(s.out_dtype, ref["y"]), f, "y")
    # padding rows of Xp and h are zero; the tail beyond offsets[E] is untouched (still NaN)
    pad = np.where(src_map[: offsets[-1]] == -1)[0]
    if len(pad):
        assert np.all(decode(f, to_host(buf["xp"])[pad]) == 0)
        assert np.all(decode(f, h[pad]) == 0)
    tail = decode(f, to_host(buf["xp"])[offsets[-1]:])
    assert np.all(np.isnan(tail))
    assert np.all(np.isfinite(y))


FULL = [wl.WORKLOADS[0], wl.WORKLOADS[1], wl.WORKLOADS[2], wl.WORKLOADS[3]]
SAMPLE = {"mixtral_bf16": 1024}  # tokens compared; the others in full


@pytest.mark.parametrize("shape", FULL, ids=lambda s: s.name)
def test_forward_full_size(shape):
    """The full workload in the launch configuration the benchmark times:
    integers in full, floats in full or on 1024 seeded tokens (the oracle's
    expert-major float64 form)."""
    inp = Inputs(shape)
    s = shape
    training = s.backward  # the benchmark's step: with the stash only where it runs the backward
    buf = run_forward(inp, training=training, poison=False)
    idx, w, counts, offsets, row_map, src_map = _check_routing(inp, buf)
    _check_xp(inp, buf, row_map, offsets)
    rng = np.random.default_rng(s.seed + 6)
    n = min(SAMPLE.get(s.name, s.T), s.T)
    toks = np.arange(s.T) if n == s.T else np.sort(rng.choice(s.T, n, replace=False))
    ref = orc.forward_experts(s, toks, inp.x, inp.w1, inp.w2, idx, w, want_stash=training)
    f = s.dtype
    rows = torch.from_numpy(row_map[toks].ravel()).long().cuda()
    assert_parity(decode(f, to_host(buf["h"][rows])), decode(f, ref["h"].reshape(-1, s.F)), f, "h")
    if training:
        assert_parity(decode(s.out_dtype, to_host(buf["gu_stash"][rows])),
                      decode(s.out_dtype, ref["stash"].reshape(-1, 2 * s.F)), f, "stash")
    assert_parity(decode(s.out_dtype, to_host(buf["yp"][rows])), decode(s.out_dtype, ref["yp"].reshape(-1, s.H)),
                  f, "Yp")
    assert_parity(decode(s.out_dtype, to_host(buf["y"])[toks]), decode(s.out_dtype, ref["y"]), f, "y")
    if s.zipf_bias is not None:
        # the skewed routing leaves many experts empty; report the histogram
        print(f"{s.name}: {int((counts == 0).sum())} empty experts, max count {int(counts.max())}")


# Shapes whose contraction (H for the gate/up GEMM, F for the down GEMM) is
# long enough that the GEMMs cut tiles along K: the gate/up GEMM (with the
# g | u stash) in the first, the down GEMM in the second.
SPLIT_K = [
    wl.MoEShape("split_k_gateup_bf16", 1024, 4096, 128, 8, 2, "softmax", False, "bf16", seed=2006),
    wl.MoEShape("split_k_down_bf16", 1024, 256, 4096, 8, 2, "softmax", False, "bf16", seed=2007),
]


def _split_tiles(offsets, rows_cap, E, K, n_out, cols_per_tile, cus):
    """Tiles the grouped bf16 GEMM cuts along K for these group offsets: the
    launch's work-queue layout (8 XCD ranges, the last partial round of each
    split when that shortens it), restated so the test can require that its
    shape takes the split path."""
    n_tiles = -(-n_out // cols_per_tile)
    max_tiles = (rows_cap // 256 + E) * n_tiles
    grid = min(cus // 8 * 8, max(-(-max_tiles // 8) * 8, 8))
    nb, nk = grid // 8, K // 64
    total = sum(-(-int(offsets[e + 1] - offsets[e]) // 256) for e in range(E)) * n_tiles
    split = 0
    for x in range(8):
        n = total * (x + 1) // 8 - total * x // 8
        r = n % nb
        if r == 0:
            continue
        best, best_rounds = 1, 1
        for S in range(2, min(8, nk // 32, 32 // r) + 1):
            rounds = -(-r * S // nb)
            if rounds * best < best_rounds * S:
                best, best_rounds = S, rounds
        split += r if best > 1 else 0
    return split


@pytest.mark.parametrize("shape", SPLIT_K, ids=lambda s: s.name)
def test_forward_split_k_tiles(shape):
    """Tiles cut along K (partial sums added by the reduction kernel, which also
    applies the SwiGLU epilogue and writes the stash) against the oracle, in full."""
    inp = Inputs(shape)
    buf = run_forward(inp, training=True)
    s = shape
    idx, w, counts, offsets, row_map, src_map = _check_routing(inp, buf)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    R = s.T * s.k
    gate_up = _split_tiles(offsets, R, s.E, s.H, s.F, 128, cus)
    down = _split_tiles(offsets, R, s.E, s.F, s.H, 256, cus)
    assert (gate_up if s.H > s.F else down) > 0, "the shape no longer exercises the K-split path"
    ref = orc.forward_tokens(s, np.arange(s.T), inp.x, inp.w1, inp.w2, idx, w, want_stash=True)
    rm = row_map.ravel()
    h, yp, st = to_host(buf["h"]), to_host(buf["yp"]), to_host(buf["gu_stash"])
    assert_parity(decode("bf16", h[rm]), decode("bf16", ref["h"].reshape(-1, s.F)), "bf16", "h")
    assert_parity(decode("bf16", st[rm]), decode("bf16", ref["stash"].reshape(-1, 2 * s.F)), "bf16", "stash")
    assert_parity(decode("bf16", yp[rm]), decode("bf16", ref["yp"].reshape(-1, s.H)), "bf16", "Yp")
    y = decode("bf16", to_host(buf["y"]))
    assert np.all(np.isfinite(y))
    assert_parity(y, decode("bf16", ref["y"]), "bf16", "y")


def test_route_edge_cases():
    # ties, signed zeros and uniform logits (every token picks experts 0..k-1)
    T, E, k = 130, 16, 4
    cfg = moe.MoEConfig(T, 128, 64, E, k, 1, "softmax", True, "bf16")
    lg = np.zeros((T, E), np.float32)
    lg[1::3, 5] = -0.0
    lg[2::3, :] = np.round(np.random.default_rng(1).standard_normal((len(range(2, T, 3)), E)))
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    moe.moe_route(cfg, to_dev(lg, "f32"), idx, w)
    i_o, w_o = orc.route(lg, k, "softmax", True)
    assert np.array_equal(to_host(idx), i_o)
    assert rel_err(to_host(w), w_o) < 1e-5
    # sigmoid underflow: w = 0, not NaN
    cfg2 = moe.MoEConfig(T, 128, 64, E, k, 1, "sigmoid", True, "bf16")
    moe.moe_route(cfg2, to_dev(np.full((T, E), -1000.0, np.float32), "f32"), idx, w)
    assert np.all(to_host(w) == 0)


def test_permute_dropped_and_bad_ids():
    """Caller-supplied routing tables: -1 drops a route; ids outside [-1, E)
    and repeated ids within a token are dropped and counted in err."""
    T, E, k, H = 300, 8, 3, 128
    rng = np.random.default_rng(3)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx[::7, 1] = -1
    idx[::11, 2] = 9
    idx[::13, 0] = -4
    idx[5::17, 2] = idx[5::17, 0]  # repeat within a token
    cfg = moe.MoEConfig(T, H, 64, E, k, 4, "softmax", False, "bf16")
    x = orc.bf16_from_f64(rng.standard_normal((T, H)))
    R = cfg.R_cap
    dev = lambda *shape, dt=torch.int32: torch.full(shape, -7, dtype=dt, device="cuda")
    xp = torch.full((R, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    counts, offsets, row_map, src_map = dev(E), dev(E + 1), dev(T, k), dev(R)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(moe.workspace_size(cfg), dtype=torch.uint8, device="cuda")
    moe.moe_permute(cfg, to_dev(x, "bf16"), to_dev(idx, "i32"), xp, counts, offsets, row_map, src_map, ws, err=err)
    c_o, o_o, r_o, s_o, bad = orc.group(idx, E, 4)
    assert int(to_host(err)[0]) == bad > 0
    assert np.array_equal(to_host(counts), c_o)
    assert np.array_equal(to_host(offsets), o_o)
    assert np.array_equal(to_host(row_map), r_o)
    assert np.array_equal(to_host(src_map), s_o)
    assert np.array_equal(to_host(xp)[: o_o[-1]], orc.permute(x, r_o, int(o_o[-1])))


def test_empty_batch_and_empty_experts():
    s = wl.MoEShape("empty_tokens", 0, 128, 64, 8, 2, "softmax", False, "bf16", seed=5)
    cfg = cfg_of(s)
    buf = moe.alloc_forward(cfg)
    moe.moe_forward(cfg, torch.empty(0, 8, device="cuda"), torch.empty(0, 128, dtype=torch.bfloat16, device="cuda"),
                    torch.zeros(8, 128, 128, dtype=torch.bfloat16, device="cuda"),
                    torch.zeros(8, 128, 64, dtype=torch.bfloat16, device="cuda"), buf)
    torch.cuda.synchronize()
    assert np.all(to_host(buf["counts"]) == 0) and np.all(to_host(buf["offsets"]) == 0)
    # all tokens on the same k experts (uniform logits), the rest empty
    s2 = wl.MoEShape("uniform", 200, 256, 128, 16, 2, "softmax", True, "bf16", seed=6)
    inp = Inputs(s2)
    inp.logits = np.zeros_like(inp.logits)
    inp.__dict__.pop("dev", None)
    buf = run_forward(inp)
    assert list(to_host(buf["counts"])) == [200, 200] + [0] * 14
    idx, w = orc.route(inp.logits, 2, "softmax", True)
    ref = orc.forward_tokens(s2, np.arange(200), inp.x, inp.w1, inp.w2, idx, w)
    assert rel_err(decode("bf16", to_host(buf["y"])), decode("bf16", ref["y"])) < TOL["bf16"]


def test_forward_graph_capture_replays():
    """moe_forward is sync-free: it captures into a HIP graph, and replays
    (with eager work in between) reproduce the eager result exactly."""
    s = wl.small_shapes()[2]
    inp = Inputs(s)
    cfg = cfg_of(s)
    d = inp.dev
    buf = moe.alloc_forward(cfg)
    moe.moe_forward(cfg, d["logits"], d["x"], d["w1"], d["w2"], buf)
    torch.cuda.synchronize()
    eager = {k: to_host(v).copy() for k, v in buf.items() if k not in ("ws", "err")}
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            moe.moe_forward(cfg, d["logits"], d["x"], d["w1"], d["w2"], buf)
    for rep in range(3):
        for k in ("y", "h", "yp", "xp"):
            buf[k].fill_(float("nan"))
        buf["row_map"].fill_(-3)
        g.replay()
        torch.cuda.synchronize()
        _ = (d["x"].float() * 2).sum().item()  # unrelated eager work between replays
        for k, v in eager.items():
            got = to_host(buf[k])
            if k in ("xp", "h", "yp", "src_map"):
                n = int(eager["offsets"][-1])
                got, v = got[:n], v[:n]
            assert np.array_equal(got.view(np.uint8), v.view(np.uint8)), f"replay {rep}: {k} differs"
