#!/usr/bin/env python3
"""Benchmark: 3D-RoPE full spatiotemporal attention forward on one MI355X.

Workload: the 81-frame 832x480 Wan2.1-1.3B-shaped clip, token grid 21 x 30 x 52 = 32,760 tokens,
12 heads, head dim 128, bf16 q/k/v ~ N(0, 1) (seeded, synthetic), RoPE split 44/42/42,
theta 10000, non-causal full attention, batch 1.

One step = the whole hot path on resident inputs, exactly what st_attn3d_fwd enqueues: the
staging step (RoPE angle table, rotated fp16 K tiles) and the attention kernel (RoPE of Q fused
into its load, flash attention on MFMA, V read directly).  The two halves are issued as
st_attn3d_stage + st_attn3d_attend so that HIP events on the launch stream can bracket the
attention kernel alone.  value = 4 N^2 heads d FLOP per step / wall time per step, in TFLOP/s.

Prints one JSON line on stdout (diagnostics go to stderr).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

GRID = (21, 30, 52)
HEADS = 12
D = 128
SPLIT = (44, 42, 42)
THETA = 10000.0
SEED = 2000
BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk/CU
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fast_kernel_wan13b_81f_traffic.txt")
COPY_BYTES = 256 << 20       # device copy timed under the counters to scale FETCH_SIZE/WRITE_SIZE
KERNEL_SOURCES = ["full_spatiotemporal_attention_amd/csrc/attn_bf16.hip",
                  "full_spatiotemporal_attention_amd/csrc/st_internal.h"]


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 counter summary (lines
    ``key: value``), or None when the counters were taken on another version of the kernel."""
    rec = {}
    try:
        with open(TRAFFIC_FILE) as f:
            for line in f:
                key, sep, val = line.partition(":")
                if sep and key.strip() in ("kernel_source_hash", "hbm_bytes_per_launch"):
                    rec[key.strip()] = val.strip()
    except OSError:
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash() or "hbm_bytes_per_launch" not in rec:
        return None
    return int(float(rec["hbm_bytes_per_launch"]))


def cpu_baseline(rows_per_head: int):
    """Time the float64 oracle on a sample of query rows (all keys, every head)."""
    import numpy as np
    import oracle
    from st_inputs import make_qkv, sample_rows
    try:
        import threadpoolctl
    except ImportError:  # pragma: no cover
        threadpoolctl = None
    n = GRID[0] * GRID[1] * GRID[2]
    x = make_qkv(n, HEADS, D, SEED, "bf16")
    rows = sample_rows(n, n, GRID[1] * GRID[2], rows_per_head, SEED + 3)
    np.ones((64, 64)) @ np.ones((64, 64))  # load BLAS so its thread count is visible
    threads = 1
    if threadpoolctl is not None:
        info = threadpoolctl.threadpool_info()
        if info:
            threads = max(int(i.get("num_threads", 1)) for i in info)
    t0 = time.perf_counter()
    oracle.full_attention_ref(x.q, x.k, x.v, GRID, 0, SPLIT, THETA, rows=rows)
    dt = time.perf_counter() - t0
    flop = 4.0 * rows.size * n * D * HEADS
    return {
        "value": round(flop / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{rows.size} query rows x {HEADS} heads against all {n} keys of the same "
                   f"workload, float64 NumPy (BLAS matmuls on {threads} threads, exp on one); "
                   f"{dt:.1f} s for {flop / 1e12:.3f} TFLOP; full step extrapolates to "
                   f"{4.0 * n * n * HEADS * D / (flop / dt):.0f} s"),
    }


ALL_LEGS = ["wan13b_17f", "wan14b_720p", "hunyuan_joint", "factorized", "factorized_hunyuan",
            "rope_apply", "fused_rope", "cross_512", "merge2", "qkv_rope", "window_7x10x13"]


def _timed(fn, stream, reps, warm=2, min_ms=30.0):
    """Average ms per call of fn() over at least `reps` back-to-back calls, and at least `min_ms`
    of work, bracketed by HIP events on the launch stream.  Untimed calls first: `warm` of them,
    then more until about `min_ms` of work has run, so that the clock has settled after the
    previous leg (the chip runs power-limited, and a few milliseconds after a heavy leg a short
    one measured up to 17 % slow)."""
    import math
    import torch
    for _ in range(warm):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    fn()
    e1.record(stream)
    torch.cuda.synchronize()
    one = max(e0.elapsed_time(e1), 1e-3)
    extra = max(0, math.ceil(min_ms / one) - warm - 1)
    for _ in range(extra):
        fn()
    reps = max(reps, math.ceil(min_ms / one))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _mfma_rate(flop, ms):
    tf = flop / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 4), "TFLOPs": round(tf, 2), "frac": round(tf / BF16_PEAK_TFLOPS, 4)}


def _full_config(name, grid, heads, n_text, split, seed, row_scale, stream, dev):
    """Full attention at one of the workload configurations, on its seeded inputs."""
    import numpy as np
    import torch
    import full_spatiotemporal_attention_amd as fa
    from st_inputs import make_qkv
    n = grid[0] * grid[1] * grid[2] + n_text
    t0 = time.perf_counter()
    x = make_qkv(n, heads, D, seed, "bf16", row_scale=row_scale)
    qq, kk, vv = (torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
                  for b in (x.q_bits, x.k_bits, x.v_bits))
    del x
    eprint(f"  {name}: inputs generated in {time.perf_counter() - t0:.1f} s")
    ws = torch.empty(fa.attn3d_workspace_bytes(grid, heads, n_text, D, split), dtype=torch.uint8, device=dev)
    o = torch.empty_like(qq)
    ms = _timed(lambda: fa.attn3d(qq, kk, vv, grid, n_text, split, THETA, out=o, workspace=ws), stream,
                reps=3 if n > 50000 else 10, warm=1 if n > 50000 else 2)
    r = _mfma_rate(4.0 * n * n * heads * D, ms)
    r.update({"grid": list(grid), "heads": heads, "n_text": n_text, "rope_split": list(split),
              "inputs": "N(0,1)" + (" x per-row U(%g,%g)" % row_scale if row_scale else "") +
                        f" bf16, PCG64 seeds {seed}..{seed + 2}", "scope": "stage + attend (st_attn3d_fwd)"})
    del qq, kk, vv, ws, o
    return r


def run_legs(legs, q, k, v, out, full_ms, stream, dev):
    """Timings after the headline: the other workload configurations and the other entry points
    (factorised path, stand-alone RoPE, fused-RoPE variant, cross-attention, merge, QKV projection,
    windows).  Each leg can be run alone (--legs), so a profile can cover exactly one leg."""
    import torch
    import full_spatiotemporal_attention_amd as fa
    from full_spatiotemporal_attention_amd import _lib
    n = GRID[0] * GRID[1] * GRID[2]
    flop = 4.0 * n * n * HEADS * D
    extras = {}
    reps = 10
    for leg in legs:
        if leg not in ALL_LEGS:
            raise SystemExit(f"unknown leg {leg!r}; known: {', '.join(ALL_LEGS)}")
        eprint(f"leg {leg}")
        if leg == "wan13b_17f":
            extras[leg] = _full_config(leg, (5, 30, 52), 12, 0, SPLIT, 1000, None, stream, dev)
        elif leg == "wan14b_720p":
            extras[leg] = _full_config(leg, (21, 45, 80), 40, 0, SPLIT, 3000, (0.5, 2.0), stream, dev)
        elif leg == "hunyuan_joint":
            extras[leg] = _full_config(leg, (33, 45, 80), 24, 256, (16, 56, 56), 4000, None, stream, dev)
        elif leg == "factorized":
            ws = torch.empty(fa.attn_factorized_workspace_bytes(GRID, HEADS, D, SPLIT), dtype=torch.uint8,
                             device=dev)
            fout = torch.empty_like(q)
            ms = _timed(lambda: fa.attn_factorized(q, k, v, GRID, SPLIT, THETA, out=fout, workspace=ws),
                        stream, reps)
            fflop = (4.0 * GRID[0] * (GRID[1] * GRID[2]) ** 2 * HEADS * D
                     + 4.0 * GRID[1] * GRID[2] * GRID[0] ** 2 * HEADS * D)
            # Whole path (staging, spatial stage, temporal stage) against the bf16 peak; the
            # temporal stage is HBM-bound, so this fraction is a blend of two rooflines.
            extras[leg] = dict(_mfma_rate(fflop, ms), flop=fflop,
                               full_over_factorized_time=round(full_ms / ms, 3),
                               full_over_factorized_flop=round(flop / fflop, 3))
        elif leg == "factorized_hunyuan":
            # The factorised path at HunyuanVideo's latent grid (33 x 45 x 80, 24 heads, 16/56/56):
            # T' = 33 takes the two-block temporal kernel.
            hgrid, hheads, hsplit = (33, 45, 80), 24, (16, 56, 56)
            hn = hgrid[0] * hgrid[1] * hgrid[2]
            gh = torch.Generator(device=dev).manual_seed(SEED + 40)
            hq, hk, hv = (torch.randn(hn, hheads, D, device=dev, generator=gh).to(torch.bfloat16)
                          for _ in range(3))
            hws = torch.empty(fa.attn_factorized_workspace_bytes(hgrid, hheads, D, hsplit), dtype=torch.uint8,
                              device=dev)
            hout = torch.empty_like(hq)
            ms = _timed(lambda: fa.attn_factorized(hq, hk, hv, hgrid, hsplit, THETA, out=hout, workspace=hws),
                        stream, 5, warm=1)
            s_ = hgrid[1] * hgrid[2]
            hflop = 4.0 * hgrid[0] * s_ * s_ * hheads * D + 4.0 * s_ * hgrid[0] ** 2 * hheads * D
            extras[leg] = dict(_mfma_rate(hflop, ms), flop=hflop, grid=list(hgrid), heads=hheads,
                               rope_split=list(hsplit), inputs="N(0,1) bf16, torch generator on the GPU")
            del hq, hk, hv, hws, hout
        elif leg == "rope_apply":
            rws = torch.empty(fa.rope3d_table_bytes(GRID, SPLIT), dtype=torch.uint8, device=dev)
            rout = torch.empty_like(q)
            ms = _timed(lambda: fa.rope3d_apply(q, GRID, 0, SPLIT, THETA, out=rout, workspace=rws), stream, reps)
            by = 2.0 * q.numel() * q.element_size()
            extras[leg] = {"ms": round(ms, 4), "GBps": round(by / (ms * 1e-3) / 1e9, 1),
                           "hbm_frac": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        elif leg == "fused_rope":
            fws = torch.empty(fa.rope3d_table_bytes(GRID, SPLIT), dtype=torch.uint8, device=dev)
            fout = torch.empty_like(q)
            ms = _timed(lambda: fa.attn3d_fused(q, k, v, GRID, 0, SPLIT, THETA, out=fout, workspace=fws),
                        stream, reps)
            extras[leg] = _mfma_rate(flop, ms)
        elif leg == "cross_512":
            # Text cross-attention next to the self-attention (Wan: at most 512 text tokens).
            n_txt = 512
            g = torch.Generator(device=dev).manual_seed(SEED + 20)
            kt_ = torch.randn(n_txt, HEADS, D, device=dev, generator=g).to(torch.bfloat16)
            vt_ = torch.randn(n_txt, HEADS, D, device=dev, generator=g).to(torch.bfloat16)
            cws = torch.empty(max(256, _lib.load().st_attn_cross_workspace_bytes(n, n_txt, HEADS, D, _lib.ST_BF16)),
                              dtype=torch.uint8, device=dev)
            cout = torch.empty_like(q)
            ms = _timed(lambda: fa.attn_cross(q, kt_, vt_, out=cout, workspace=cws), stream, reps)
            extras[leg] = _mfma_rate(4.0 * n * n_txt * HEADS * D, ms)
        elif leg == "merge2":
            # Merge of two partial results over the whole grid (HBM-bound: 2 reads + 1 write of O).
            lse_a = torch.zeros(n, HEADS, dtype=torch.float32, device=dev)
            lse_b = torch.zeros(n, HEADS, dtype=torch.float32, device=dev)
            other = torch.empty_like(q).copy_(out)
            mo, ml = torch.empty_like(q), torch.empty_like(lse_a)
            ms = _timed(lambda: fa.attn_merge([(out, lse_a), (other, lse_b)], out=mo, lse_out=ml), stream, reps)
            by = 3.0 * q.numel() * 2 + 3.0 * n * HEADS * 4
            extras[leg] = {"ms": round(ms, 4), "GBps": round(by / (ms * 1e-3) / 1e9, 1),
                           "hbm_frac": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        elif leg == "qkv_rope":
            # QKV projection with the rotation of q and k in its epilogue (Wan2.1-1.3B: C = 1536).
            C = HEADS * D
            gx = torch.Generator(device=dev).manual_seed(SEED + 30)
            xq = torch.randn(n, C, device=dev, generator=gx).to(torch.bfloat16)
            wq = (torch.randn(3 * C, C, device=dev, generator=gx) / C ** 0.5).to(torch.bfloat16)
            bq = (0.1 * torch.randn(3 * C, device=dev, generator=gx)).to(torch.bfloat16)
            qws = torch.empty(max(256, fa.rope3d_table_bytes(GRID, SPLIT)), dtype=torch.uint8, device=dev)
            ms = _timed(lambda: fa.qkv_rope(xq, wq, GRID, bias=bq, rope_split=SPLIT, workspace=qws), stream, reps)
            extras[leg] = _mfma_rate(2.0 * n * C * 3 * C, ms)
            del xq, wq, bq
        elif leg == "window_7x10x13":
            # Local 3D windows of 7 x 10 x 13 = 910 tokens (36 windows over the grid).
            WIN = (7, 10, 13)
            L_win = WIN[0] * WIN[1] * WIN[2]
            wws = torch.empty(max(256, _lib.load().st_attn3d_window_workspace_bytes(
                *GRID, HEADS, D, _lib.split_arg(SPLIT), _lib.split_arg(WIN), _lib.ST_BF16)), dtype=torch.uint8,
                device=dev)
            wout = torch.empty_like(q)
            ms = _timed(lambda: fa.attn_window(q, k, v, GRID, WIN, SPLIT, THETA, out=wout, workspace=wws),
                        stream, reps)
            extras[leg] = _mfma_rate(4.0 * n * L_win * HEADS * D, ms)
        torch.cuda.synchronize()
        eprint(f"  {leg}: {extras[leg]}")
    return extras


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-rows", type=int, default=8192, help="oracle rows per head for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip every leg after the headline")
    ap.add_argument("--legs", default=",".join(ALL_LEGS),
                    help="comma-separated legs timed after the headline (default: all): " + ", ".join(ALL_LEGS))
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 256 MiB device-to-device copy first (scale for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        eprint(f"bench.py --gpus {args.gpus}: this build runs on one GPU only (no sharding, no "
               "collectives); run with --gpus 1.")
        sys.exit(2)

    import numpy as np
    import torch
    import full_spatiotemporal_attention_amd as fa
    from full_spatiotemporal_attention_amd import _lib
    from st_inputs import make_qkv

    if not torch.cuda.is_available():
        eprint("bench.py needs a GPU")
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = _lib.load()
    n = GRID[0] * GRID[1] * GRID[2]
    flop = 4.0 * n * n * HEADS * D

    x = make_qkv(n, HEADS, D, SEED, "bf16")
    q, k, v = (torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
               for b in (x.q_bits, x.k_bits, x.v_bits))
    del x
    out = torch.empty_like(q)
    wsb = fa.attn3d_workspace_bytes(GRID, HEADS, 0, D, SPLIT)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    sp = _lib.split_arg(SPLIT)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    def step(ev_mid=None):
        st = lib.st_attn3d_stage(k.data_ptr(), GRID[0], GRID[1], GRID[2], 0, HEADS, D,
                                 sp, THETA, _lib.ST_BF16, ws.data_ptr(), wsb, sh)
        if st:
            raise _lib.StError("st_attn3d_stage", st)
        if ev_mid is not None:
            ev_mid.record(stream)
        st = lib.st_attn3d_attend(q.data_ptr(), v.data_ptr(), GRID[0], GRID[1], GRID[2], 0, HEADS, D,
                                  sp, _lib.ST_BF16, ws.data_ptr(), wsb, out.data_ptr(), sh)
        if st:
            raise _lib.StError("st_attn3d_attend", st)

    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    mids = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(mids[i])
        ends[i].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / args.steps
    ev_ms = start.elapsed_time(ends[-1]) / args.steps
    kern_ms = [mids[i].elapsed_time(ends[i]) for i in range(args.steps)]
    kern_avg = sum(kern_ms) / len(kern_ms)
    value = flop / (wall_ms * 1e-3) / 1e12
    achieved = flop / (kern_avg * 1e-3) / 1e12
    stage_ms = [start.elapsed_time(mids[0])] + [ends[i - 1].elapsed_time(mids[i]) for i in range(1, args.steps)]
    stage_avg = sum(stage_ms) / len(stage_ms)
    eprint(f"step wall {wall_ms:.3f} ms, events {ev_ms:.3f} ms, attention kernel avg {kern_avg:.3f} ms "
           f"(min {min(kern_ms):.3f}, max {max(kern_ms):.3f}), staging avg {stage_avg:.3f} ms")

    result = {
        "metric": "3D-attn fwd TFLOP/s & % bf16 MFMA peak at 21x30x52 tokens, 12 heads, d=128",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "wan1.3b-shaped 81-frame 832x480 clip: full 3D-RoPE attention forward",
            "grid": list(GRID), "tokens": n, "heads": HEADS, "head_dim": D,
            "rope_split": list(SPLIT), "theta": THETA, "batch": 1,
            "inputs": "N(0,1) bf16, PCG64 seeds 2000/2001/2002",
        },
        "pct_of_bf16_peak": round(100.0 * value / BF16_PEAK_TFLOPS, 2),
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_fast_kernel<false, false>",
            "achieved": round(achieved, 2),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(),
            "launch_ms": round(kern_avg, 4),
            "flop_per_launch": flop,
        },
        "stage_ms": round(stage_avg, 4),
    }

    if not args.no_extras:
        legs = [l for l in args.legs.split(",") if l]
        extras = run_legs(legs, q, k, v, out, ev_ms, stream, dev)
        result["extras"] = extras
        eprint(f"extras: {json.dumps(extras)}")

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_rows)
        eprint(f"cpu_baseline: {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
