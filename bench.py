#!/usr/bin/env python3
"""Benchmark of the block-quantized matrix-vector path on one MI355X.

Headline (the `value`): Q4_K GEMV at M=1 over the dense 27B-like FFN shapes --
gate and up 17408x5120, down 5120x17408 -- cycling a pool of 128 independent
layer copies (19.25 GB, far above the 256 MB Infinity Cache), reported as
achieved GB/s of algorithmic bytes (weights + activations + outputs). One step
is one pass over the whole pool (384 GEMVs). Also reported: the M = 1..4
speculative-verify curve, the 1024x1024 Q8_0 GEMV latency, the routed-expert
MoE rate (tok-equiv/s over a 48-bank pool), the M=512 prefill GEMM rate, a copy
bandwidth calibration, the roofline of the dominant kernel from per-launch HIP
events, and the CPU oracle timed on the host cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0

# HBM bytes per q4k_gemv_kernel launch at M=1 (mean over gate, up and down) from
# rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE passes (profiles/q4k_gemv_m1_hbm_traffic.md),
# each scaled by what the same counter reads for a 4 GiB device copy in the same
# run (FETCH_SIZE reads half the bytes copied, WRITE_SIZE all of them). The figure
# describes the kernel code hashed here (comments and whitespace excluded) and is
# reported as null once it changes.
GEMV_TRAFFIC = {
    "sources": ("gguf_block_quantized_qmv_amd/csrc/q4k_gemv.hip", "gguf_block_quantized_qmv_amd/csrc/q4k_common.h",
                "gguf_block_quantized_qmv_amd/csrc/qmv_device.h"),
    "sha256": "e2f82a7bfb9b4910f66acc2c9acd9d81a339a99a104cd8ed6f8fa4606edfd976",
    "bytes_per_launch": 50875056,
}


def gemv_sources_sha256():
    """sha256 of the kernel's sources with comments and whitespace removed (code only)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in GEMV_TRAFFIC["sources"]:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def gemv_traffic():
    return GEMV_TRAFFIC["bytes_per_launch"] if gemv_sources_sha256() == GEMV_TRAFFIC["sha256"] else None
BF16_PEAK_TFLOPS = 2500.0
METRIC = "Q4_K GEMV achieved HBM GB/s (% of 8 TB/s peak) at M=1; MoE tok-equiv/s"
SHAPES = (("gate", 17408, 5120), ("up", 17408, 5120), ("down", 5120, 17408))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--copies", type=int, default=128, help="layer copies in the dense weight pool")
    p.add_argument("--moe-banks", type=int, default=48)
    p.add_argument("--iq4-copies", type=int, default=48, help="layer copies in the IQ4_XS, Q5_K, Q6_K and Q4_0 weight pools")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the CPU oracle sample")
    p.add_argument("--skip", default="", help="comma list of sections to skip: verify,q8,moe,prefill,iq4,q5,q6,q40,cpu")
    return p.parse_args()


def current_stream_ptr(torch):
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class Timer:
    """HIP-event timing on the current torch stream."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, fn, reps):
        t = self.torch
        s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        t.cuda.synchronize()
        return s.elapsed_time(e) / 1e3 / reps   # seconds per rep


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on exactly one GPU; the multi-GPU sharding is designed "
                                   "but not built, so only --gpus 1 is measured", "n_gpus": args.gpus}))
        sys.exit(2)
    skip = set(filter(None, args.skip.split(",")))

    import numpy as np
    import torch

    import gguf_block_quantized_qmv_amd as q
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = q.lib
    timer = Timer(torch)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    # ------------------------------------------------------------ dense pool
    log(f"[bench] generating the Q4_K pool: {args.copies} copies x gate/up/down")
    pool = [[synth.torch_q4_k_weights(11, n, k, dev, stream=3 * c + i) for i, (_, n, k) in enumerate(SHAPES)]
            for c in range(args.copies)]
    xs = {k: synth.bf16_normal(12, (4, k)) for _, _, k in SHAPES}
    x_dev = {k: torch.from_numpy(v.view(np.int16)).to(dev) for k, v in xs.items()}
    y_dev = {n: torch.empty((4, n), dtype=torch.float32, device=dev) for _, n, _ in SHAPES}
    torch.cuda.synchronize()
    wbytes = [q.q4_k_bytes(n, k) for _, n, k in SHAPES]
    pool_bytes = args.copies * sum(wbytes)

    def calls(m, stream_ptr=None):
        st = stream_ptr if stream_ptr is not None else sp
        out = []
        for c in range(args.copies):
            for i, (_, n, k) in enumerate(SHAPES):
                out.append((ctypes.c_void_p(pool[c][i].data_ptr()), wbytes[i], ctypes.c_void_p(x_dev[k].data_ptr()),
                            ctypes.c_void_p(y_dev[n].data_ptr()), m, n, k, st))
        return out

    def algo_bytes(m):
        return args.copies * sum(wb + m * k * 2 + m * n * 4 for wb, (_, n, k) in zip(wbytes, SHAPES))

    def make_step(m, stream_ptr=None):
        cl = calls(m, stream_ptr)
        fn = L.qmv_q4_k

        def step():
            for a in cl:
                rc = fn(*a)
                if rc:
                    raise q.QmvError(rc, "qmv_q4_k")
        return step

    def graph_of(m):
        # the launches must name the capture stream that torch.cuda.graph makes current
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            make_step(m, current_stream_ptr(torch))()
        return g

    res = {}
    step1 = make_step(1)
    for _ in range(max(1, args.warmup)):
        step1()
    t_eager = timer.run(step1, args.steps)
    log(f"[bench] M=1 stream launches: {t_eager * 1e3:.3f} ms/step, {algo_bytes(1) / t_eager / 1e9:.1f} GB/s")

    g1 = graph_of(1)
    for _ in range(max(1, args.warmup)):
        g1.replay()
    t_graph = timer.run(g1.replay, args.steps)
    log(f"[bench] M=1 hipGraph replay:   {t_graph * 1e3:.3f} ms/step, {algo_bytes(1) / t_graph / 1e9:.1f} GB/s")

    # the replayed graph must reproduce the stream-launched result bit for bit (outputs cleared in between)
    step1()
    torch.cuda.synchronize()
    y_ref = {n: y_dev[n][:1].clone() for n in y_dev}
    for n in y_dev:
        y_dev[n].fill_(float("nan"))
    torch.cuda.synchronize()
    g1.replay()
    torch.cuda.synchronize()
    for n in y_dev:
        assert torch.equal(y_dev[n][:1], y_ref[n]), "graph replay and stream launch disagree"

    best_t, launch_mode = (t_graph, "hipGraph") if t_graph < t_eager else (t_eager, "stream")
    value = algo_bytes(1) / best_t / 1e9

    # per-launch kernel durations (HIP events around every launch, on the launch stream)
    cl = calls(1)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in cl]
    torch.cuda.synchronize()
    for (s, e), a in zip(evs, cl):
        s.record()
        L.qmv_q4_k(*a)
        e.record()
    torch.cuda.synchronize()
    dur = {name: [] for name, _, _ in SHAPES}
    for i, (s, e) in enumerate(evs):
        dur[SHAPES[i % 3][0]].append(s.elapsed_time(e) / 1e3)
    per_shape = {}
    for i, (name, n, k) in enumerate(SHAPES):
        d = float(np.mean(dur[name]))
        per_shape[name] = {"us": d * 1e6, "GBps": (wbytes[i] + k * 2 + n * 4) / d / 1e9}
    # roofline: the timed region is a pass over the pool made of this kernel only, so its
    # average launch duration is the region's time over the launches in it (HIP events on
    # the launch stream, back-to-back launches); the per-launch bracketing above adds the
    # launch overhead of each isolated call and is reported separately
    launch_bytes = float(np.mean([wb + k * 2 + n * 4 for wb, (_, n, k) in zip(wbytes, SHAPES)]))
    avg_dur = best_t / (args.copies * len(SHAPES))
    achieved = launch_bytes / avg_dur / 1e9
    res["per_shape_m1"] = per_shape
    res["isolated_launch_us_mean"] = float(np.mean([np.mean(v) for v in dur.values()])) * 1e6
    log(f"[bench] per-launch: " + ", ".join(f"{k} {v['us']:.2f} us {v['GBps']:.0f} GB/s" for k, v in per_shape.items()))

    # speculative verify: GB/s vs M
    if "verify" not in skip:
        curve = {}
        for m in (1, 2, 3, 4):
            g = graph_of(m)
            g.replay()
            tm = timer.run(g.replay, max(2, args.steps // 2))
            curve[str(m)] = {"GBps": algo_bytes(m) / tm / 1e9, "ms_per_step": tm * 1e3,
                             "weights_per_s": args.copies * sum(n * k for _, n, k in SHAPES) / tm}
            del g
        res["verify_GBps_vs_M"] = curve
        log("[bench] verify curve: " + ", ".join(f"M={m} {v['GBps']:.0f}" for m, v in curve.items()))

    # copy calibration: device-to-device copy of 4 GiB (read + write bytes)
    buf_a = torch.empty(1 << 32, dtype=torch.uint8, device=dev)
    buf_b = torch.empty_like(buf_a)
    buf_b.copy_(buf_a)
    t_copy = timer.run(lambda: buf_b.copy_(buf_a), 5)
    res["copy_calibration_GBps"] = 2 * buf_a.numel() / t_copy / 1e9
    del buf_a, buf_b
    log(f"[bench] copy calibration {res['copy_calibration_GBps']:.0f} GB/s (read+write)")

    # Q8_0 1024x1024 (cache-resident; latency, not a bandwidth figure)
    if "q8" not in skip:
        w8 = torch.from_numpy(synth.q8_0_weights(13, 1024, 1024)).to(dev)
        x8 = torch.from_numpy(synth.f32_normal(14, (1, 1024))).to(dev)
        y8 = torch.empty((1, 1024), dtype=torch.float32, device=dev)
        a8 = (ctypes.c_void_p(w8.data_ptr()), w8.numel(), ctypes.c_void_p(x8.data_ptr()),
              ctypes.c_void_p(y8.data_ptr()), 1, 1024, 1024, sp)
        L.qmv_q8_0(*a8)
        g8 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g8):
            a8g = a8[:-1] + (current_stream_ptr(torch),)
            for _ in range(100):
                L.qmv_q8_0(*a8g)
        g8.replay()
        t8 = timer.run(g8.replay, 5) / 100
        res["q8_0_1024x1024_us"] = t8 * 1e6
        log(f"[bench] Q8_0 1024x1024: {t8 * 1e6:.2f} us/call (graph)")

    if "moe" not in skip:
        res["moe"] = bench_moe(args, torch, np, q, synth, timer, dev, sp)
    if "prefill" not in skip:
        res["prefill"] = bench_prefill(args, torch, np, q, synth, timer, dev, sp, pool)

    del pool
    torch.cuda.empty_cache()
    if "iq4" not in skip:
        res["iq4_xs_gemv"] = bench_format(args, torch, np, q, synth, timer, dev, sp, "iq4_xs")
        if "moe" not in skip:
            res["moe_iq4_xs"] = bench_moe(args, torch, np, q, synth, timer, dev, sp, fmt="iq4_xs")
        torch.cuda.empty_cache()
    if "q5" not in skip:
        res["q5_k_gemv"] = bench_format(args, torch, np, q, synth, timer, dev, sp, "q5_k")
        torch.cuda.empty_cache()
    if "q6" not in skip:
        res["q6_k_gemv"] = bench_format(args, torch, np, q, synth, timer, dev, sp, "q6_k")
        torch.cuda.empty_cache()
    if "q40" not in skip:
        res["q4_0_gemv"] = bench_format(args, torch, np, q, synth, timer, dev, sp, "q4_0")
        torch.cuda.empty_cache()

    cpu = None
    if "cpu" not in skip:
        cpu = cpu_baseline(args, np, synth)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(best_t * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4_k(exact bf16 q) x bf16 -> fp32",
        "data": "synthetic",
        "config": {
            "workload": "Q4_K GEMV M=1: gate/up 17408x5120 + down 5120x17408, 128-copy pool "
                        f"({pool_bytes / 1e9:.2f} GB), one step = one pass over the pool",
            "pool_bytes": pool_bytes,
            "launch": launch_mode,
            "frac_of_8TBps": round(value / HBM_PEAK_GBPS, 4),
            "stream_launch_GBps": round(algo_bytes(1) / t_eager / 1e9, 1),
            "graph_replay_GBps": round(algo_bytes(1) / t_graph / 1e9, 1),
        },
        "roofline": {
            "kernel": "q4k_gemv_kernel<1>",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": gemv_traffic(),
            "traffic_unit": "HBM bytes per launch",
            "avg_launch_us": round(avg_dur * 1e6, 3),
            "algorithmic_bytes_per_launch": launch_bytes,
        },
        "cpu_baseline": cpu,
        "extra": res,
    }
    print(json.dumps(line), flush=True)


def bench_moe(args, torch, np, q, synth, timer, dev, sp, fmt="q4_k"):
    hidden, ffn, ne, tk = 2048, 768, 128, 8
    L = q.lib
    gen = synth.torch_q4_k_weights if fmt == "q4_k" else synth.torch_iq4_xs_weights
    entry = L.qmv_q4_k_moe if fmt == "q4_k" else L.qmv_iq4_xs_moe
    ws_fn = L.qmv_q4_k_moe_workspace if fmt == "q4_k" else L.qmv_iq4_xs_moe_workspace
    name = f"qmv_{fmt}_moe"
    banks = []
    log(f"[bench] generating the {fmt} MoE pool: {args.moe_banks} banks x {ne} experts")
    for b in range(args.moe_banks):
        banks.append([gen(21, ne * (ffn if i < 2 else hidden), hidden if i < 2 else ffn, dev, stream=3 * b + i)
                      for i in range(3)])
    bank_bytes = banks[0][0].numel()
    out = {}
    for t in (1, 3):
        logits = torch.from_numpy(synth.moe_logits(22, t * args.moe_banks, ne)).to(dev).view(args.moe_banks, t, ne)
        x = torch.from_numpy(synth.bf16_normal(23, (t, hidden)).view(np.int16)).to(dev)
        y = torch.empty((t, hidden), dtype=torch.float32, device=dev)
        need = ws_fn(t, hidden, ffn, ne, tk)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        ids = torch.empty((args.moe_banks, t, tk), dtype=torch.int32, device=dev)
        def make_calls(stream_ptr):
            return [(*(ctypes.c_void_p(banks[b][i].data_ptr()) for i in range(3)), bank_bytes,
                     ctypes.c_void_p(logits[b].data_ptr()), ctypes.c_void_p(x.data_ptr()),
                     ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(ids[b].data_ptr()), None, None,
                     ctypes.c_void_p(ws.data_ptr()), need, t, hidden, ffn, ne, tk, stream_ptr)
                    for b in range(args.moe_banks)]

        def make_step(stream_ptr):
            cl = make_calls(stream_ptr)

            def step():
                for a in cl:
                    rc = entry(*a)
                    if rc:
                        raise q.QmvError(rc, name)
            return step
        step = make_step(sp)
        step()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            make_step(current_stream_ptr(torch))()
        g.replay()
        t_eager = timer.run(step, max(2, args.steps))
        t_graph = timer.run(g.replay, max(2, args.steps))
        tl = min(t_eager, t_graph) / args.moe_banks
        # distinct experts per layer decide the bytes streamed
        idh = ids.cpu().numpy()
        distinct = np.mean([len(np.unique(idh[b])) for b in range(args.moe_banks)])
        expert_bytes = 3 * bank_bytes // ne
        out[f"T{t}"] = {
            "tok_equiv_per_s": t / (args.moe_banks * tl),
            "us_per_layer": tl * 1e6,
            "distinct_experts": float(distinct),
            "GBps_distinct_expert_bytes": distinct * expert_bytes / tl / 1e9,
            "launch": "hipGraph" if t_graph < t_eager else "stream",
        }
        log(f"[bench] {fmt} MoE T={t}: {tl * 1e6:.2f} us/layer, {out[f'T{t}']['tok_equiv_per_s']:.0f} tok-equiv/s, "
            f"{out[f'T{t}']['GBps_distinct_expert_bytes']:.0f} GB/s")
    if fmt == "q4_k":
        # prompt-sized form: 512 tokens per call over 8 of the pool's banks
        t, nb = 512, min(8, args.moe_banks)
        logits = torch.from_numpy(synth.moe_logits(24, t * nb, ne)).to(dev).view(nb, t, ne)
        x = torch.from_numpy(synth.bf16_normal(25, (t, hidden)).view(np.int16)).to(dev)
        y = torch.empty((t, hidden), dtype=torch.float32, device=dev)
        need = L.qmv_q4_k_moe_prefill_workspace(t, hidden, ffn, ne, tk)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        calls = [(*(ctypes.c_void_p(banks[b][i].data_ptr()) for i in range(3)), bank_bytes,
                  ctypes.c_void_p(logits[b].data_ptr()), ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                  None, None, ctypes.c_void_p(ws.data_ptr()), need, t, hidden, ffn, ne, tk, sp) for b in range(nb)]

        def pstep():
            for a in calls:
                rc = L.qmv_q4_k_moe_prefill(*a)
                if rc:
                    raise q.QmvError(rc, "qmv_q4_k_moe_prefill")
        pstep()
        tl = timer.run(pstep, 2) / nb
        # algorithmic work: per (token, rank) pair 2 flop per weight of W_gate, W_up and W_down
        flops = t * tk * 2 * 3 * hidden * ffn
        out["prefill_T512"] = {"us_per_layer": tl * 1e6, "tokens_per_s_per_layer": t / tl,
                               "TFLOPs": flops / tl / 1e12}
        log(f"[bench] {fmt} MoE prefill T={t}: {tl * 1e3:.3f} ms/layer, {t / tl:.0f} tokens/s per layer, "
            f"{flops / tl / 1e12:.0f} TFLOP/s")
    del banks
    return out


def bench_format(args, torch, np, q, synth, timer, dev, sp, fmt):
    """GEMV of another block format (IQ4_XS, Q5_K, Q6_K or Q4_0) over a pool of layer copies
    (the dense FFN shapes), M = 1..4."""
    L = q.lib
    copies = args.iq4_copies
    gen = {"iq4_xs": synth.torch_iq4_xs_weights, "q5_k": synth.torch_q5_k_weights,
           "q6_k": synth.torch_q6_k_weights, "q4_0": synth.torch_q4_0_weights}[fmt]
    entry = {"iq4_xs": L.qmv_iq4_xs, "q5_k": L.qmv_q5_k, "q6_k": L.qmv_q6_k, "q4_0": L.qmv_q4_0}[fmt]
    nbytes = {"iq4_xs": q.iq4_xs_bytes, "q5_k": q.q5_k_bytes, "q6_k": q.q6_k_bytes, "q4_0": q.q4_0_bytes}[fmt]
    log(f"[bench] generating the {fmt} pool: {copies} layer copies")
    pool = [[gen(41, n, k, dev, stream=3 * c + i) for i, (_, n, k) in enumerate(SHAPES)] for c in range(copies)]
    xs = {k: torch.from_numpy(synth.bf16_normal(42, (4, k)).view(np.int16)).to(dev) for _, _, k in SHAPES}
    ys = {n: torch.empty((4, n), dtype=torch.float32, device=dev) for _, n, _ in SHAPES}
    shape_bytes = [nbytes(n, k) for _, n, k in SHAPES]
    out = {}

    def calls_for(m, shapes):
        return [(ctypes.c_void_p(pool[c][i].data_ptr()), pool[c][i].numel(), ctypes.c_void_p(xs[k].data_ptr()),
                 ctypes.c_void_p(ys[n].data_ptr()), m, n, k, sp)
                for c in range(copies) for i, (_, n, k) in enumerate(SHAPES) if i in shapes]

    def stepper(cl):
        def step():
            for a in cl:
                rc = entry(*a)
                if rc:
                    raise q.QmvError(rc, f"qmv_{fmt}")
        return step

    for m in (1, 2, 3, 4):
        step = stepper(calls_for(m, (0, 1, 2)))
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.3:
            step()
        t = timer.run(step, max(2, args.steps // 2))
        out[f"M{m}"] = {"GBps": copies * sum(shape_bytes) / t / 1e9, "us_per_launch": t / (3 * copies) * 1e6}
    for i, (name, n, k) in enumerate(SHAPES):
        t = timer.run(stepper(calls_for(1, (i,))), max(2, args.steps // 2)) / copies
        out[f"M1_{name}"] = {"us_per_launch": t * 1e6, "GBps": shape_bytes[i] / t / 1e9}
    log(f"[bench] {fmt} GEMV: " + ", ".join(f"M={m} {out[f'M{m}']['GBps']:.0f} GB/s" for m in (1, 2, 3, 4)) +
        "; M=1 per launch " + ", ".join(f"{nm} {out[f'M1_{nm}']['us_per_launch']:.2f} us" for nm, _, _ in SHAPES))
    del pool
    return out


def bench_prefill(args, torch, np, q, synth, timer, dev, sp, pool):
    m = 512
    out = {}
    L = q.lib
    for i, (name, n, k) in enumerate(SHAPES[1:], start=1):
        x = torch.from_numpy(synth.bf16_normal(31, (m, k)).view(np.int16)).to(dev)
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        copies = min(20, len(pool))
        need = L.qmm_q4_k_prefill_workspace(m, n, k)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        ws_arg = ctypes.c_void_p(ws.data_ptr()) if need else None
        calls = [(ctypes.c_void_p(pool[c][i].data_ptr()), pool[c][i].numel(), ctypes.c_void_p(x.data_ptr()),
                  ctypes.c_void_p(y.data_ptr()), m, n, k, ws_arg, need, sp) for c in range(copies)]

        def step():
            for a in calls:
                rc = L.qmm_q4_k_prefill(*a)
                if rc:
                    raise q.QmvError(rc, "qmm_q4_k_prefill")
        # matrix-core clocks settle only after sustained work: about 0.3 s of
        # untimed passes before the timed ones
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.3:
            step()
            torch.cuda.synchronize()
        tp = timer.run(step, 5) / copies
        flops = 2.0 * m * n * k
        # dense bf16 torch GEMM of the same shape, as an achievable-rate reference
        a = torch.randn((m, k), device=dev, dtype=torch.bfloat16)
        b = torch.randn((n, k), device=dev, dtype=torch.bfloat16)
        torch.matmul(a, b.t())
        tt = timer.run(lambda: torch.matmul(a, b.t()), 10)
        out[name] = {"us": tp * 1e6, "TFLOPs": flops / tp / 1e12, "frac_of_bf16_peak": flops / tp / 1e12 / BF16_PEAK_TFLOPS,
                     "torch_bf16_dense_TFLOPs": flops / tt / 1e12, "k_split_workspace_bytes": need}
        log(f"[bench] prefill {name} {m}x{n}x{k}: {tp * 1e6:.1f} us, {flops / tp / 1e12:.0f} TFLOP/s "
            f"(torch dense bf16: {flops / tt / 1e12:.0f})")
    return out


def cpu_baseline(args, np, synth):
    """The fp64 oracle on the host cores: layer copies (gate, up, down) at M=1 until the budget is spent."""
    import oracle

    # threads actually used: the dequant is single-threaded numpy, the matvec runs on the BLAS pool
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] + [1])
    except ImportError:
        cores = len(os.sched_getaffinity(0))
    done_bytes, spent, mats = 0, 0.0, 0
    while spent < args.cpu_seconds or mats < 3:
        i = mats % 3
        _, n, k = SHAPES[i]
        raw = synth.q4_k_weights(40 + mats // 3, n, k, stream=i)
        x = synth.bf16_normal(41, (1, k))
        t0 = time.perf_counter()
        oracle.qmv_q4_k(raw, x, n, k)
        spent += time.perf_counter() - t0
        done_bytes += raw.size
        mats += 1
    log(f"[bench] cpu oracle: {mats} matrices, {spent:.1f} s, {done_bytes / spent / 1e9:.3f} GB/s")
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{mats} Q4_K matrices of the dense pool shapes (gate/up 17408x5120, down 5120x17408) at M=1, "
                      f"{done_bytes / 1e9:.2f} GB of blocks: fp64 dequant (numpy, one thread) + fp64 matvec "
                      f"(BLAS, up to `cores` threads); input generation excluded",
            "seconds": round(spent, 2)}


if __name__ == "__main__":
    main()
