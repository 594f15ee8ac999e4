"""Benchmark of the MoE FFN hot path on one MI355X.

One step = one pass of the whole forward hot path (route -> permute -> grouped
gate/up GEMM + SwiGLU -> grouped down GEMM -> top-k combine: the calls whose
kernels moe_forward launches, issued one by one with a HIP event after each)
over one batch of seeded synthetic input already resident in HBM.  Default
workload: the Mixtral-shaped layer (T=8192, H=4096, F=14336, E=8, top-2
softmax, bf16 with fp32 accumulation).  The skewed workload's step also runs
the FFN backward.

Prints one JSON line: tokens/s of the layer over the K timed steps, each
kernel's duration in those steps (mean, median, p10, p90; HIP events on the
launch stream), route / permute / combine again with cold caches (a 512 MiB
read before each of 50 calls), a route sweep over T, the roofline of the
dominant kernel (the grouped gate/up GEMM) and the CPU oracle timed on a
bounded token sample.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 / MXFP8 MFMA
PEAK_FP4_TFLOPS = 10100.0   # MI355X dense fp4 / MXFP4 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    # the clocks settle over the first ~100 steps: fewer warm-up steps
    # measured the fine-grained step ~7 % slower
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--flush-iters", type=int, default=50,
                   help="calls of each bandwidth kernel timed with cold caches (512 MiB read before each)")
    p.add_argument("--workload", default="mixtral_bf16")
    p.add_argument("--no-variants", action="store_true",
                   help="skip the variant timings (gather form, weight placements, clamp): counter passes")
    p.add_argument("--cpu-sample", type=int, default=256, help="tokens of the oracle CPU baseline (0 = skip)")
    p.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                   help="HBM bytes per dispatch measured with rocprofv3 counters (optional)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="also run a plain device copy of this many MiB (reference for counter scaling)")
    p.add_argument("--lds-calibration", type=int, default=0, metavar="MIB",
                   help="also run one 256 x 256 tile of the bf16 down GEMM whose two operands (this many MiB "
                        "together) are each read exactly once through direct-to-LDS loads: the reference for "
                        "scaling the FETCH_SIZE of the grouped GEMMs")
    p.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, WRITE_SIZE) of a "
                        "--copy-calibration run into the traffic file and exit (no GPU needed)")
    p.add_argument("--only", default="", help="comma list of staged kernels to run in the per-kernel loop "
                   "(for profiling one kernel); default all")
    return p.parse_args()


# Sources of the dominant kernel per storage dtype: measured traffic is used
# only while these files are unchanged.
GEMM1_SOURCES = {
    "bf16": ["gemm_bf16_kernel.h", "gemm_bf16.hip", "tiles.h", "moe_internal.h"],
    "mxfp8": ["gemm_mxfp8_kernel.h", "gemm_bf16_kernel.h", "mxfp8.hip", "mxfp8.h", "tiles.h", "moe_internal.h"],
    "mxfp4": ["gemm_mxfp8_kernel.h", "gemm_bf16_kernel.h", "mxfp8.hip", "mxfp8.h", "tiles.h", "moe_internal.h"],
    "f32": ["gemm_f32.hip", "tiles.h", "moe_internal.h"],
}
GEMM1_KERNEL = {"bf16": "grouped_gemm_bf16<true", "mxfp8": "grouped_gemm_mxfp8<true", "mxfp4": "grouped_gemm_mxfp8<true",
                "f32": "grouped_gemm_f32<true"}


def kernel_source_hash(dtype: str) -> str:
    import hashlib

    h = hashlib.sha256()
    for f in GEMM1_SOURCES[dtype]:
        with open(os.path.join(ROOT, "routing_permute_grouped_router_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def lds_calibration(mib: int, dev) -> None:
    """One tile of the bf16 down GEMM (E = 1, 256 rows, H = 256, K = F) whose
    A and B are each read once, as the grouped GEMMs read their operands
    (direct-to-LDS loads): mib MiB of operand bytes in one dispatch."""
    import torch

    import routing_permute_grouped_router_amd as moe

    F = (mib << 20) // (2 * 256 * 2)
    cfg = moe.MoEConfig(256, 256, F, 1, 1)
    h = torch.ones(256, F, dtype=torch.bfloat16, device=dev)
    w2 = torch.ones(1, 256, F, dtype=torch.bfloat16, device=dev)
    offsets = torch.tensor([0, 256], dtype=torch.int32, device=dev)
    yp = torch.empty(256, 256, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(moe.workspace_size(cfg), 1), dtype=torch.uint8, device=dev)
    moe.moe_grouped_down_gemm(cfg, h, w2, offsets, yp, ws)
    torch.cuda.synchronize()
    del h, w2, yp, ws


def pmc_summary(fetch_csv: str, write_csv: str, workload: str, out_path: str, lds_mib: int = 0) -> None:
    """Per-dispatch HBM bytes of the grouped GEMM1 from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by the ratio the same counter shows for a
    dispatch of known bytes in the same run: the largest plain device copy (the
    --copy-calibration copy), and for the GEMM's fetches, when the run had one,
    the --lds-calibration tile (the first bf16 down-GEMM dispatch), whose loads
    are of the GEMMs' own kind."""
    import csv
    import collections

    import numpy as np

    from routing_permute_grouped_router_amd import workload as wl

    s = wl.BY_NAME[workload]
    res = {}
    lds_fetch = None
    for cnt, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        per = collections.defaultdict(list)
        copies = []
        rows = sorted((r for r in csv.DictReader(open(path)) if r["Counter_Name"] == cnt),
                      key=lambda r: int(r["Dispatch_Id"]))
        for r in rows:
            v = float(r["Counter_Value"])
            if "copyBuffer" in r["Kernel_Name"]:
                copies.append(v)
            name_ = r["Kernel_Name"].split("(")[0]
            if cnt == "FETCH_SIZE" and lds_mib and lds_fetch is None and "grouped_gemm_bf16<false" in name_:
                lds_fetch = v  # the first bf16 down-GEMM dispatch: the calibration tile
                continue
            per[name_].append(v)
        kib_copy = max(copies)  # the calibration copy of `cal` MiB is the largest copy
        res[cnt] = (per, kib_copy)
    cal_kib = res["WRITE_SIZE"][1]  # written bytes of a copy are its size (checked below)
    f_scale = cal_kib / res["FETCH_SIZE"][1]
    w_scale = 1.0
    # the GEMM's own loads: scale by the direct-to-LDS calibration tile if the run had one
    g_scale = (lds_mib * 1024) / lds_fetch if lds_fetch else f_scale
    name = [n for n in res["FETCH_SIZE"][0] if GEMM1_KERNEL[s.dtype] in n][0]
    fetch = float(np.mean(res["FETCH_SIZE"][0][name])) * g_scale * 1024
    write = float(np.mean(res["WRITE_SIZE"][0][name])) * w_scale * 1024
    out = {"workload": workload, "kernel": "swiglu_gemm", "kernel_name": name,
           "source_hash": kernel_source_hash(s.dtype), "bytes_per_dispatch": round(fetch + write),
           "fetch_bytes": round(fetch), "write_bytes": round(write), "copy_kib": cal_kib,
           "fetch_scale": round(g_scale, 4), "copy_fetch_scale": round(f_scale, 4), "write_scale": w_scale,
           "lds_calibration_mib": lds_mib if lds_fetch else 0}
    with open(out_path, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out))


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.workload, args.traffic, args.lds_calibration)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU's share of the MoE layer and runs on one GPU only "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import routing_permute_grouped_router_amd as moe
    from routing_permute_grouped_router_amd import workload as wl

    s = wl.BY_NAME[args.workload]
    cfg = moe.MoEConfig.from_shape(s)

    def note(msg):  # progress on stderr; the JSON line stays alone on stdout
        print(f"[bench {s.name}] {msg}", file=sys.stderr, flush=True)
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)

    w = wl.Workload(s)
    t_gen = time.time()

    def up(a, fmt):
        if fmt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    logits = up(w.logits(), "f32")
    gen_fmt = "bf16" if s.dtype == "bf16" else "f32"
    x = up(w.x(), gen_fmt)
    # weights expert by expert (bounded host memory)
    sd = cfg.store_dtype
    w1 = torch.empty(s.E, 2 * s.F, cfg.cols(s.H), dtype=sd, device=dev)
    w2 = torch.empty(s.E, s.H, cfg.cols(s.F), dtype=sd, device=dev)
    scales = {}
    quantize = moe.moe_quantize_mxfp4 if s.dtype == "mxfp4" else moe.moe_quantize_mxfp8
    if cfg.is_mx:
        scales["w1_scale"] = torch.empty(s.E, 2 * s.F, s.H // 32, dtype=torch.uint8, device=dev)
        scales["w2_scale"] = torch.empty(s.E, s.H, s.F // 32, dtype=torch.uint8, device=dev)
        xq = torch.empty(s.T, cfg.cols(s.H), dtype=torch.uint8, device=dev)
        scales["x_scale"] = torch.empty(s.T, s.H // 32, dtype=torch.uint8, device=dev)
        quantize(x, xq, scales["x_scale"])
        x = xq
    step_e = max(1, (1 << 28) // (2 * s.F * s.H))
    for e0 in range(0, s.E, step_e):
        e1 = min(s.E, e0 + step_e)
        a1, a2 = up(w.w1(e0, e1), gen_fmt), up(w.w2(e0, e1), gen_fmt)
        if cfg.is_mx:
            quantize(a1, w1[e0:e1], scales["w1_scale"][e0:e1])
            quantize(a2, w2[e0:e1], scales["w2_scale"][e0:e1])
        else:
            w1[e0:e1].copy_(a1)
            w2[e0:e1].copy_(a2)
        del a1, a2
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen
    note(f"inputs resident ({t_gen:.1f} s)")

    buf = moe.alloc_forward(cfg, training=s.backward)
    bwd = moe.alloc_backward(cfg) if s.backward else None
    dy = up(w.dy(), "bf16" if s.dtype != "f32" else "f32") if s.backward else None
    stream = torch.cuda.current_stream()
    g = {kk: v for kk, v in scales.items()}

    # One step: the calls of the forward (and, for the training workload, of
    # the backward) issued one by one on the launch stream -- the kernels
    # moe_forward / moe_backward launch -- with a HIP event after each call,
    # so every kernel's duration is measured inside the timed region.
    names = ["route", "permute", "swiglu_gemm", "down_gemm", "combine"]
    if s.backward:
        names += ["combine_bwd", "down_bwd", "swiglu_bwd", "permute_bwd"]

    def step(ev=None):
        rec = (lambda i: ev[i].record(stream)) if ev else (lambda i: None)
        rec(0)
        moe.moe_route(cfg, logits, buf["idx"], buf["w"])
        rec(1)
        moe.moe_permute(cfg, x, buf["idx"], buf["xp"], buf["counts"], buf["offsets"], buf["row_map"],
                        buf["src_map"], buf["ws"], x_scale=g.get("x_scale"), xp_scale=buf.get("xp_scale"),
                        err=buf["err"])
        rec(2)
        moe.moe_grouped_swiglu_gemm(cfg, buf["xp"], w1, buf["offsets"], buf["h"], buf["ws"], xp_scale=buf.get("xp_scale"),
                                    w1_scale=g.get("w1_scale"), h_scale=buf.get("h_scale"),
                                    gu_stash=buf.get("gu_stash"))
        rec(3)
        moe.moe_grouped_down_gemm(cfg, buf["h"], w2, buf["offsets"], buf["yp"], buf["ws"], h_scale=buf.get("h_scale"),
                                  w2_scale=g.get("w2_scale"))
        rec(4)
        moe.moe_combine(cfg, buf["yp"], buf["row_map"], buf["w"], buf["y"])
        rec(5)
        if s.backward:
            moe.moe_combine_bwd(cfg, dy, buf["row_map"], buf["src_map"], buf["offsets"], buf["w"], bwd["dyp"])
            rec(6)
            moe.moe_grouped_down_bwd(cfg, bwd["dyp"], w2, buf["h"], buf["gu_stash"], buf["offsets"], bwd["dgu"],
                                     bwd["dw2"], bwd["ws"])
            rec(7)
            moe.moe_grouped_swiglu_bwd(cfg, bwd["dgu"], w1, buf["xp"], buf["offsets"], bwd["dxp"], bwd["dw1"],
                                       bwd["ws"])
            rec(8)
            moe.moe_permute_bwd(cfg, bwd["dxp"], buf["row_map"], bwd["dx"])
            rec(9)

    if args.copy_calibration:
        src = torch.empty(args.copy_calibration << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.lds_calibration:
        lds_calibration(args.lds_calibration, dev)

    for _ in range(args.warmup):
        step()
    note(f"{args.warmup} warm-up steps done")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.time()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t_wall = time.time() - t_wall
    ms = evs[0][0].elapsed_time(evs[-1][-1]) / args.steps
    per_step = sorted(e[0].elapsed_time(e[-1]) for e in evs)
    kern_samples = {n: sorted(e[i].elapsed_time(e[i + 1]) for e in evs) for i, n in enumerate(names)}
    kern_ms = {n: sum(v) / len(v) for n, v in kern_samples.items()}
    note(f"{args.steps} timed steps: {ms:.4f} ms per step")

    def pct(v, q):
        return v[min(len(v) - 1, int(q * len(v)))]

    # Bandwidth kernels with cold caches: a 512 MiB read (outside the event
    # window) evicts L2 and the 256 MiB MALL before each of `flush_iters`
    # calls, so route, permute and combine read their inputs from HBM.  A read
    # leaves clean lines; a write would leave the caches full of dirty ones,
    # whose write-back to HBM would then be charged to the timed kernel.
    flushbuf = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
    flush_words = flushbuf.view(torch.int32)
    bw_calls = {
        "route": lambda: moe.moe_route(cfg, logits, buf["idx"], buf["w"]),
        "permute": lambda: moe.moe_permute(cfg, x, buf["idx"], buf["xp"], buf["counts"], buf["offsets"],
                                           buf["row_map"], buf["src_map"], buf["ws"], x_scale=g.get("x_scale"),
                                           xp_scale=buf.get("xp_scale"), err=buf["err"]),
        "combine": lambda: moe.moe_combine(cfg, buf["yp"], buf["row_map"], buf["w"], buf["y"]),
    }
    cold = {}
    for n, f in bw_calls.items():
        samples = []
        for it in range(args.flush_iters):
            flush_words.sum()
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            f()
            a1.record(stream)
            samples.append((a0, a1))
        torch.cuda.synchronize()
        cold[n] = sorted(a0.elapsed_time(a1) for a0, a1 in samples)
    note("cold-cache bandwidth kernels done")

    # Route at growing T (E and k of this workload; logits N(0,1)): where the
    # kernel leaves the launch-latency regime and what bandwidth it reaches.
    route_sweep = []
    for Ts in (s.T, 65536, 262144, 1048576):
        cs = dataclasses.replace(cfg, T=Ts)
        lg = torch.randn(Ts, s.E, device=dev)
        ix = torch.empty(Ts, s.k, dtype=torch.int32, device=dev)
        wt = torch.empty(Ts, s.k, dtype=torch.float32, device=dev)
        for _ in range(3):
            moe.moe_route(cs, lg, ix, wt)
        samples = []
        for it in range(20):
            flush_words.sum()
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            moe.moe_route(cs, lg, ix, wt)
            a1.record(stream)
            samples.append((a0, a1))
        torch.cuda.synchronize()
        v = sorted(a0.elapsed_time(a1) for a0, a1 in samples)
        nb = Ts * s.E * 4 + Ts * s.k * 8
        route_sweep.append({"T": Ts, "ms": round(pct(v, 0.5), 4), "gbs": round(nb / (pct(v, 0.5) * 1e-3) / 1e9, 1),
                            "frac_hbm": round(nb / (pct(v, 0.5) * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)})
        del lg, ix, wt
    del flushbuf, flush_words
    note("route sweep done")

    if s.backward:
        # the routing backward (gradients of the top-k weights and router
        # logits): timed on its own, outside the step
        dlog = torch.empty(s.T, s.E, dtype=torch.float32, device=dev)
        dwr = torch.empty(s.T, s.k, dtype=torch.float32, device=dev)
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        moe.moe_route_bwd(cfg, dy, buf["yp"], logits, buf["idx"], buf["row_map"], dlog, dw=dwr)
        r0.record(stream)
        for _ in range(args.steps):
            moe.moe_route_bwd(cfg, dy, buf["yp"], logits, buf["idx"], buf["row_map"], dlog, dw=dwr)
        r1.record(stream)
        torch.cuda.synchronize()
        kern_ms["route_bwd"] = r0.elapsed_time(r1) / args.steps
        names.append("route_bwd")

    variants = None
    if not s.backward and not args.no_variants:
        # The gather form of the forward (no materialised Xp: the gate/up GEMM
        # reads x[src_map[r] / k] itself), timed as whole steps and as the
        # gather GEMM alone; reported beside the step, which stays the
        # materialised path.
        bg = dict(buf, xp=None, xp_scale=None)

        def gstep():
            moe.moe_forward(cfg, logits, x, w1, w2, bg, **scales)

        for _ in range(2):
            gstep()
        g0, g1, g2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        torch.cuda.synchronize()
        g0.record(stream)
        for _ in range(args.steps):
            gstep()
        g1.record(stream)
        for _ in range(args.steps):
            moe.moe_grouped_swiglu_gemm_gather(cfg, x, buf["src_map"], buf["counts"], w1, buf["offsets"], buf["h"],
                                               buf["ws"], x_scale=g.get("x_scale"), w1_scale=g.get("w1_scale"),
                                               h_scale=buf.get("h_scale"))
        g2.record(stream)
        torch.cuda.synchronize()
        gms = g0.elapsed_time(g1) / args.steps
        variants = {"gather_forward": {"ms_per_step": round(gms, 4), "tokens_per_s": round(s.T / (gms * 1e-3), 1),
                                       "swiglu_gemm_gather_ms": round(g1.elapsed_time(g2) / args.steps, 4)}}
        # The routing weight applied in the gate/up (FC1) or down (FC2)
        # epilogue instead of the combine, and the SwiGLU clamp (its cost does
        # not depend on the limit), each on the materialised step.
        for vname, change in (("weight_fc1", dict(weight_site="fc1")), ("weight_fc2", dict(weight_site="fc2")),
                              ("swiglu_clamp", dict(swiglu_limit=7.0))):
            cw = dataclasses.replace(cfg, **change)
            for _ in range(2):
                moe.moe_forward(cw, logits, x, w1, w2, buf, **scales)
            torch.cuda.synchronize()
            g0.record(stream)
            for _ in range(args.steps):
                moe.moe_forward(cw, logits, x, w1, w2, buf, **scales)
            g1.record(stream)
            torch.cuda.synchronize()
            wms = g0.elapsed_time(g1) / args.steps
            variants[vname] = {"ms_per_step": round(wms, 4), "tokens_per_s": round(s.T / (wms * 1e-3), 1)}
        note("variants done")

    R, T, H, F, E, k = s.R, s.T, s.H, s.F, s.E, s.k
    esz = {"f32": 4, "bf16": 2, "mxfp8": 1 + 1 / 32, "mxfp4": 0.5 + 1 / 32}[s.dtype]
    osz = 4 if s.dtype == "f32" else 2
    flops = {"swiglu_gemm": 4.0 * R * H * F, "down_gemm": 2.0 * R * H * F}
    # algorithmic bytes (each operand read once, each output written once)
    bytes_ = {
        "route": T * E * 4 + T * k * 8,
        "permute": T * k * 4 + T * H * esz + R * H * esz + T * k * 4 + R * 4,
        "combine": R * H * osz + T * H * osz + T * k * 8,
        "swiglu_gemm": R * H * esz + E * 2 * F * H * esz + R * F * esz,
        "down_gemm": R * F * esz + E * H * F * esz + R * H * osz,
        # backward bandwidth kernels: dY read, dYp rows written (padding rows
        # zeroed too), w and maps; dXp rows read, dX written, map
        "combine_bwd": T * H * osz + s.R_cap * H * osz + T * k * 8 + s.R_cap * 4,
        "permute_bwd": R * H * osz + T * H * osz + T * k * 4,
        # routing backward: dY and the routed Yp rows read, logits read,
        # dlogits and dw written, idx and row_map read
        "route_bwd": T * H * osz + R * H * osz + 2 * T * E * 4 + T * k * 12,
    }
    peak_mm = {"f32": PEAK_FP32_TFLOPS, "bf16": PEAK_BF16_TFLOPS, "mxfp8": PEAK_FP8_TFLOPS,
               "mxfp4": PEAK_FP4_TFLOPS}[s.dtype]
    kern = {}
    for n in names:
        d = {"ms": round(kern_ms[n], 4)}
        if n in kern_samples:  # in-step durations over the K timed steps
            v = kern_samples[n]
            d.update(ms_median=round(pct(v, 0.5), 4), ms_p10=round(pct(v, 0.1), 4), ms_p90=round(pct(v, 0.9), 4))
        if n in flops:
            tf = flops[n] / (kern_ms[n] * 1e-3) / 1e12
            d.update(tflops=round(tf, 1), frac_mfma=round(tf / peak_mm, 4))
        if n in bytes_:
            gbs = bytes_[n] / (kern_ms[n] * 1e-3) / 1e9
            d.update(gbs=round(gbs, 1), frac_hbm=round(gbs / PEAK_HBM_GBS, 4))
        if n in cold:  # caches flushed before each call: inputs from HBM
            v = cold[n]
            gc = bytes_[n] / (pct(v, 0.5) * 1e-3) / 1e9
            d["cold"] = {"iters": len(v), "ms_median": round(pct(v, 0.5), 4), "ms_p10": round(pct(v, 0.1), 4),
                         "ms_p90": round(pct(v, 0.9), 4), "gbs": round(gc, 1), "frac_hbm": round(gc / PEAK_HBM_GBS, 4)}
        kern[n] = d

    traffic = None
    try:
        tr = json.load(open(args.traffic))
        if (tr.get("workload") == s.name and tr.get("kernel") == "swiglu_gemm"
                and tr.get("source_hash") == kernel_source_hash(s.dtype)):
            traffic = tr.get("bytes_per_dispatch")
    except (OSError, ValueError):
        pass
    tf = flops["swiglu_gemm"] / (kern_ms["swiglu_gemm"] * 1e-3) / 1e12
    if cfg.is_mx:
        # MX weights are streamed once at ~433 FLOP/B (MXFP8; ~840 for MXFP4),
        # below the ridge (5000 TFLOP/s / 8 TB/s = 625 FLOP/B for MXFP8,
        # 10100 / 8 = 1262 for MXFP4): the kernel is HBM-bound.
        gbs = bytes_["swiglu_gemm"] / (kern_ms["swiglu_gemm"] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": f"grouped_gemm_{s.dtype}_swiglu", "achieved": round(gbs, 1),
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                    "bytes_per_launch": bytes_["swiglu_gemm"], "tflops": round(tf, 1),
                    "frac_mfma": round(tf / peak_mm, 4)}
    else:
        roofline = {"bound": "mfma", "kernel": "grouped_gemm_swiglu", "achieved": round(tf, 2), "peak": peak_mm,
                    "unit": "TFLOP/s", "frac": round(tf / peak_mm, 4), "traffic": traffic,
                    "flops_per_launch": flops["swiglu_gemm"]}

    cpu = None
    if args.cpu_sample > 0:
        from oracle import oracle as orc

        note("CPU oracle baseline ...")

        lg = w.logits()
        xs = w.x()
        n = min(args.cpu_sample, T)
        rng = np.random.default_rng(s.seed + 6)
        toks = np.sort(rng.choice(T, n, replace=False)).astype(np.int32)
        t0 = time.time()
        idx_o, w_o = orc.route(lg, k, s.score, s.renorm)
        orc.group(idx_o, E, s.align)
        t_route = time.time() - t0
        # host weights of the experts the sample uses (the others stay zero pages)
        need = np.unique(idx_o[toks])
        mx = cfg.is_mx
        wdt = {"f32": np.float32, "bf16": np.uint16, "mxfp8": np.uint8, "mxfp4": np.uint8}[s.dtype]
        w1h = np.zeros((E, 2 * F, cfg.cols(H)), wdt)
        w2h = np.zeros((E, H, cfg.cols(F)), wdt)
        xsc = w1sc = w2sc = None
        if mx:
            xs, xsc = orc.mx_quantize(xs, s.dtype)
            w1sc = np.zeros((E, 2 * F, H // 32), np.uint8)
            w2sc = np.zeros((E, H, F // 32), np.uint8)
        for e in need[need >= 0]:
            a1, a2 = w.w1(int(e), int(e) + 1)[0], w.w2(int(e), int(e) + 1)[0]
            if mx:
                (w1h[e], w1sc[e]), (w2h[e], w2sc[e]) = orc.mx_quantize(a1, s.dtype), orc.mx_quantize(a2, s.dtype)
            else:
                w1h[e], w2h[e] = a1, a2
        t0 = time.time()
        orc.forward_tokens(s, toks, xs, w1h, w2h, idx_o, w_o, xsc, w1sc, w2sc)
        t_ffn = time.time() - t0
        per_tok = t_ffn / n + t_route / T
        cpu = {"value": round(1.0 / per_tok, 3), "unit": "tokens/s", "cores": orc.num_threads(), "kind": "oracle",
               "sample": f"route+group over all {T} tokens ({t_route:.2f} s), expert FFN + combine of {n} "
                         f"seeded tokens ({t_ffn:.2f} s); tokens/s = 1 / (FFN s per token + routing s per token)"}

    out = {
        "metric": "MoE layer tokens/s; grouped-GEMM TFLOP/s as % of MFMA peak; permute GB/s",
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "mxfp8": "mxfp8-e4m3", "mxfp4": "mxfp4-e2m1"}[s.dtype],
        "data": "synthetic",
        "config": {"workload": s.name, "T": T, "H": H, "F": F, "E": E, "k": k, "score": s.score,
                   "renorm": s.renorm, "storage": s.dtype, "accumulate": "f32", "backward": s.backward,
                   "parallelism": "single GPU"},
        "step_ms": {"median": round(pct(per_step, 0.5), 4), "p10": round(pct(per_step, 0.1), 4),
                    "p90": round(pct(per_step, 0.9), 4)},
        "kernels": kern,
        "route_sweep": route_sweep,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "variants": variants,
        "wall_s_timed": round(t_wall, 3),
        "setup_s": round(t_gen, 1),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
