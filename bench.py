"""Benchmark of the DSA prefill hot path on one MI355X.

One step = one pass of the whole path over the 4096-token causal prefill
workload (batch 1; indexer 64 heads x 128 fp8; top-k 2048; sparse attention
128 heads over 576-wide bf16 latent KV, 512-wide output): dsa_indexer_logits
-> dsa_topk -> dsa_sparse_attn_fwd on one stream (exactly the launches that
dsa_prefill makes), with inputs resident in HBM before timing starts.

Prints ONE JSON line.  `value` is tokens/s of the whole step.  `roofline`
describes the dominant kernel (sparse attention): algorithmic bf16 flops per
launch over its median duration from HIP events on the launch stream,
against the 2.5 PFLOP/s dense bf16 MFMA peak.  `stages` also gives each
stage timed with L2 and the MALL flushed before every step, the dsa_prefill
entry point warm and flushed, the indexer + top-k without a logits buffer
(dsa_indexer_topk: time, and peak device memory against the unfused way),
the attention backward at the same shapes (bf16 kv), and the full-FP8
attention (dsa_sparse_attn_fwd_fp8: e4m3 q and KV quantised from the same
draws, the same top-k indices; against the 5.0 PFLOP/s fp8 peak).  `cpu_baseline`
times the CPU oracle (indexer -> top-k -> attention), stage by stage, on a
bounded sample of rows.

    python bench.py [--steps 20] [--warmup 5] [--gpus 1] [--no-cpu] [--flush-reps 10]
    python bench.py --copy-calibration     # plain 1 GiB copy, for counter scaling

Warm-up runs W steps and goes on until at least one second has passed.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA prefill tokens/s (indexer+top-k+sparse attn) at seq 4096; % of roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
WARMUP_MIN_S = 1.0          # least warm-up time (clock ramp)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sparse_attn_prefill_4096_traffic.json")
ATTN_SRC = os.path.join(ROOT, "fp8_indexer_amd", "csrc", "sparse_attn.hip")


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def work_counts(wl, ks, ke):
    """Algorithmic work of each stage (valid pairs only)."""
    import numpy as np
    s = np.clip(ks.reshape(-1).astype(np.int64), 0, wl.N)
    e = np.maximum(np.clip(ke.reshape(-1).astype(np.int64), 0, wl.N), s)
    ln = e - s
    p_idx = int(ln.sum())
    p_att = int(np.minimum(ln, wl.K).sum())
    rows = wl.B * wl.M
    idx_flops = 2.0 * wl.H * wl.D * p_idx
    idx_bytes = (rows * wl.H * wl.D + wl.B * wl.N * (wl.D + 4) + 8 * rows * wl.H + 4 * p_idx)
    topk_bytes = 4.0 * ln[ln > wl.K].sum() + 4.0 * wl.K * rows
    att_flops = 2.0 * wl.Hq * (wl.Dqk + wl.Dv) * p_att
    return dict(p_idx=p_idx, p_att=p_att, idx_flops=idx_flops, idx_bytes=float(idx_bytes),
                topk_bytes=float(topk_bytes), att_flops=att_flops)


def attn_src_hash():
    with open(ATTN_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(launches_per_step=1):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary; None if absent or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != attn_src_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, x, budget_s):
    """The oracle (indexer -> top-k -> attention) on a bounded sample of
    rows, evenly spaced over the sequence so that the window lengths span
    the workload's; each stage timed on its own, with its algorithmic work
    over the sampled rows."""
    import numpy as np
    import oracle
    R = wl.B * wl.M

    def run(rows):
        t0 = time.perf_counter()
        lg = oracle.indexer_logits(x["q8"], x["q_scale"], x["k8"], x["k_scale"], x["w"],
                                   x["ks"], x["ke"], rows=rows)
        t1 = time.perf_counter()
        ti = oracle.topk(lg, x["ks"], x["ke"], wl.B, wl.M, wl.N, wl.K, rows=rows)
        t2 = time.perf_counter()
        full = np.full((R, wl.K), -1, np.int32)
        full[rows] = ti
        oracle.sparse_attn(x["q"], x["kv"], x["sink"], full.reshape(wl.B, wl.M, wl.K),
                           wl.sm_scale, wl.Dv, kv_scale=x["kv_scale"], rows=rows)
        t3 = time.perf_counter()
        return t1 - t0, t2 - t1, t3 - t2

    n = 16
    rows = np.linspace(0, R - 1, n).round().astype(np.int64)
    dt = sum(run(rows))
    n2 = int(min(R, max(n, n * (budget_s / max(dt, 1e-3)))))
    if n2 > n:
        rows = np.unique(np.linspace(0, R - 1, n2).round().astype(np.int64))
    t_idx, t_topk, t_att = run(rows)
    s = np.clip(x["ks"].reshape(-1)[rows].astype(np.int64), 0, wl.N)
    e = np.maximum(np.clip(x["ke"].reshape(-1)[rows].astype(np.int64), 0, wl.N), s)
    ln = e - s
    idx_flops = 2.0 * wl.H * wl.D * ln.sum()
    topk_bytes = 4.0 * ln[ln > wl.K].sum() + 4.0 * wl.K * len(rows)
    att_flops = 2.0 * wl.Hq * (wl.Dqk + wl.Dv) * np.minimum(ln, wl.K).sum()
    total = t_idx + t_topk + t_att
    return {"value": len(rows) / total, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{len(rows)} of {R} query rows, evenly spaced over the {wl.name} "
                      f"workload (indexer -> top-k -> attention, fp64 C oracle, OpenMP), "
                      f"{total:.1f} s",
            "stages": {
                "indexer": {"s": t_idx, "gflops": idx_flops / t_idx / 1e9},
                "topk": {"s": t_topk, "gbs": topk_bytes / t_topk / 1e9},
                "attention": {"s": t_att, "gflops": att_flops / t_att / 1e9},
            }}


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--flush-reps", type=int, default=10,
                    help="steps timed with L2/MALL flushed before each (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--fp8-attn-reps", type=int, default=5,
                    help="timed runs of the full-FP8 attention (0: skip)")
    ap.add_argument("--backward-reps", type=int, default=3,
                    help="timed calls of the attention backward (0 = skip)")
    ap.add_argument("--workload", default="prefill_4096",
                    help="workload to time (default: the 4096-token causal prefill)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the work would shard by query rows). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch

    import fp8_indexer_amd as dsa
    import workloads as W

    wl = W.WORKLOADS[args.workload]
    eprint(f"[bench] generating inputs for {wl.name}")
    x = W.make_inputs(wl)
    dev = torch.device("cuda:0")
    g = {k: (torch.from_numpy(v).to(dev) if isinstance(v, np.ndarray) else
             (v.to(dev) if isinstance(v, torch.Tensor) else v)) for k, v in x.items()}
    B, M, N = wl.B, wl.M, wl.N
    logits = torch.empty((B, M, N), dtype=torch.float32, device=dev)
    idx = torch.empty((B, M, wl.K), dtype=torch.int32, device=dev)
    o = torch.empty((B, M, wl.Hq, wl.Dv), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        """One pass of the path.  ev: 2 events (around attention) or 4 (stage
        boundaries)."""
        if ev and len(ev) == 4:
            ev[0].record(stream)
        dsa.indexer_logits(g["q8"], g["q_scale"], g["k8"], g["k_scale"], g["w"], g["ks"],
                           g["ke"], logits=logits)
        if ev and len(ev) == 4:
            ev[1].record(stream)
        dsa.topk(logits, g["ks"], g["ke"], wl.K, out=idx)
        if ev:
            ev[-2].record(stream)
        dsa.sparse_attn_fwd(g["q"], g["kv"], g["sink"], idx, wl.sm_scale, wl.Dv, out=o,
                            kv_scale=g.get("kv_scale"))
        if ev:
            ev[-1].record(stream)

    # W warm-up steps, continued until at least WARMUP_MIN_S has passed: the
    # GPU's clocks take a fraction of a second of load to ramp up
    eprint(f"[bench] warmup {args.warmup} steps, at least {WARMUP_MIN_S} s")
    warm_steps = 0
    tw = time.perf_counter()
    while warm_steps < args.warmup or time.perf_counter() - tw < WARMUP_MIN_S:
        step()
        torch.cuda.synchronize()
        warm_steps += 1
    # timed steps: HIP events only around the dominant kernel (attention)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    eprint(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    ms_att = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    # per-stage times: the same steps with events at every stage boundary
    evs4 = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs4[i])
    torch.cuda.synchronize()
    st = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in evs4])
    ms_idx, ms_topk, ms_att4 = np.median(st, axis=0)

    # the same stages with L2 and the 256 MB MALL flushed before each step
    # (a 512 MB write), so no stage reads its input from the previous one's
    # cache footprint
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    fl = []
    for _ in range(args.flush_reps):
        flush_buf.fill_(1)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        step(ev)
        torch.cuda.synchronize()
        fl.append([ev[j].elapsed_time(ev[j + 1]) for j in range(3)])
    flushed = np.median(np.array(fl), axis=0) if fl else [float("nan")] * 3
    pf = []
    for _ in range(args.flush_reps):
        flush_buf.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dsa.prefill(g["q8"], g["q_scale"], g["k8"], g["k_scale"], g["w"], g["ks"], g["ke"],
                    wl.K, g["q"], g["kv"], g["sink"], sm_scale=wl.sm_scale, dv=wl.Dv,
                    logits=logits, topk_idxs=idx, out=o, kv_scale=g.get("kv_scale"))
        e1.record(stream)
        torch.cuda.synchronize()
        pf.append(e0.elapsed_time(e1))
    ms_prefill_flushed = float(np.median(pf)) if pf else float("nan")
    del flush_buf

    # whole-path entry point, same work, as a cross-check of the step time
    for _ in range(2):
        dsa.prefill(g["q8"], g["q_scale"], g["k8"], g["k_scale"], g["w"], g["ks"], g["ke"],
                    wl.K, g["q"], g["kv"], g["sink"], sm_scale=wl.sm_scale, dv=wl.Dv,
                    logits=logits, topk_idxs=idx, out=o, kv_scale=g.get("kv_scale"))
    torch.cuda.synchronize()
    tp0 = time.perf_counter()
    for _ in range(args.steps):
        dsa.prefill(g["q8"], g["q_scale"], g["k8"], g["k_scale"], g["w"], g["ks"], g["ke"],
                    wl.K, g["q"], g["kv"], g["sink"], sm_scale=wl.sm_scale, dv=wl.Dv,
                    logits=logits, topk_idxs=idx, out=o, kv_scale=g.get("kv_scale"))
    torch.cuda.synchronize()
    ms_prefill = (time.perf_counter() - tp0) * 1e3 / args.steps

    # indexer + top-k without the [B, M, N] logits buffer (dsa_indexer_topk):
    # time, and peak device memory of either way of producing topk_idxs from
    # the inputs (logits buffer, or workspace)
    eprint("[bench] fused indexer + top-k")
    fused_idx = torch.empty_like(idx)

    def fused_step():
        dsa.indexer_topk(g["q8"], g["q_scale"], g["k8"], g["k_scale"], g["w"], g["ks"], g["ke"],
                         wl.K, out=fused_idx)

    for _ in range(2):
        fused_step()
    torch.cuda.synchronize()
    fev = []
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fused_step()
        e1.record(stream)
        fev.append((e0, e1))
    torch.cuda.synchronize()
    ms_fused = float(np.median([a.elapsed_time(b) for a, b in fev]))
    fused_same = bool(torch.equal(fused_idx, idx))

    def peak_bytes(fn):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        fn()
        torch.cuda.synchronize()
        return torch.cuda.max_memory_allocated() - base

    del logits
    torch.cuda.empty_cache()
    peak_unfused = peak_bytes(lambda: dsa.topk(
        dsa.indexer_logits(g["q8"], g["q_scale"], g["k8"], g["k_scale"], g["w"], g["ks"],
                           g["ke"]), g["ks"], g["ke"], wl.K, out=fused_idx))
    peak_fused = peak_bytes(fused_step)

    # backward of the sparse attention at the same shapes (bf16 kv only)
    bwd = None
    if not wl.kv_fp8 and args.backward_reps > 0:
        eprint("[bench] backward")
        gO = torch.randn(o.shape, device=dev).to(torch.bfloat16)
        dq = torch.empty((B, M, wl.Hq, wl.Dqk), dtype=torch.float32, device=dev)
        dkv = torch.empty((B, N, wl.Dqk), dtype=torch.float32, device=dev)
        dsk = torch.empty((wl.Hq,), dtype=torch.float32, device=dev)
        bargs = (g["q"], g["kv"], g["sink"], idx, o, gO, wl.sm_scale, dq, dkv, dsk)
        dsa.sparse_attn_bwd(*bargs)
        torch.cuda.synchronize()
        bt = []
        for _ in range(args.backward_reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dsa.sparse_attn_bwd(*bargs)
            e1.record(stream)
            torch.cuda.synchronize()
            bt.append(e0.elapsed_time(e1))
        ms_bwd = float(np.median(bt))
        # S and dP (recomputed), dQ, dK and dV products per valid index
        bwd_flops = 2.0 * wl.Hq * (3 * wl.Dqk + 2 * wl.Dv) * work_counts(wl, x["ks"],
                                                                          x["ke"])["p_att"]
        bwd = {"ms": ms_bwd, "tflops": bwd_flops / (ms_bwd * 1e-3) / 1e12,
               "frac_bf16_peak": bwd_flops / (ms_bwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
               "algorithmic_tflop": bwd_flops / 1e12, "reps": args.backward_reps}
        del dq, dkv, gO

    # full-FP8 attention (e4m3 q and KV, fp8 MFMA for both products) on the
    # same top-k indices, with q and kv quantised from the same draws
    f8 = None
    if dsa.attn_fp8_supported(wl.Hq, wl.Dqk, wl.Dv) and args.fp8_attn_reps > 0:
        eprint("[bench] full-FP8 attention")
        wl8 = wl.with_(name=wl.name + "_fp8attn", q_fp8=True, kv_fp8=True)
        x8 = W.make_inputs(wl8, parts=("attn",))
        g8 = {k: x8[k].to(dev) for k in ("q", "qa_scale", "kv", "kv_scale")}
        del x8
        o8 = torch.empty_like(o)
        f8args = (g8["q"], g8["qa_scale"], g8["kv"], g8["kv_scale"], g["sink"], idx, wl.sm_scale,
                  wl.Dv)
        t_end = time.time() + 0.3  # warm, like the other stages
        while time.time() < t_end:
            dsa.sparse_attn_fwd_fp8(*f8args, out=o8)
            torch.cuda.synchronize()
        ft = []
        for _ in range(args.fp8_attn_reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dsa.sparse_attn_fwd_fp8(*f8args, out=o8)
            e1.record(stream)
            torch.cuda.synchronize()
            ft.append(e0.elapsed_time(e1))
        ms_f8 = float(np.median(ft))
        f8_flops = work_counts(wl, x["ks"], x["ke"])["att_flops"]
        f8 = {"workload": wl8.name, "ms": ms_f8, "tflops": f8_flops / (ms_f8 * 1e-3) / 1e12,
              "frac_fp8_peak": f8_flops / (ms_f8 * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
              "speedup_vs_bf16_attention": ms_att / ms_f8, "reps": args.fp8_attn_reps}
        del g8, o8

    wc = work_counts(wl, x["ks"], x["ke"])
    tokens = B * M
    att_tflops = wc["att_flops"] / (ms_att * 1e-3) / 1e12
    idx_tflops = wc["idx_flops"] / (ms_idx * 1e-3) / 1e12
    topk_gbs = wc["topk_bytes"] / (ms_topk * 1e-3) / 1e9
    roof_s = (wc["idx_flops"] / (PEAK_FP8_TFLOPS * 1e12) + wc["topk_bytes"] / (PEAK_HBM_GBS * 1e9)
              + wc["att_flops"] / (PEAK_BF16_TFLOPS * 1e12))
    traffic = load_traffic() if wl.name == "prefill_4096" else None
    res = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_steps,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8+bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "seq_len": M, "index_heads": wl.H,
                   "index_dim": wl.D, "topk": wl.K, "heads": wl.Hq, "dqk": wl.Dqk, "dv": wl.Dv,
                   "kv": "fp8_e4m3fn" if wl.kv_fp8 else "bf16", "windows": wl.windows},
        "roofline": {"bound": "mfma", "kernel": "sparse_attn_kernel",
                     "achieved": att_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": att_tflops / PEAK_BF16_TFLOPS, "traffic": traffic},
        "stages": {
            "indexer": {"ms": ms_idx, "tflops": idx_tflops,
                        "frac_fp8_peak": idx_tflops / PEAK_FP8_TFLOPS},
            "topk": {"ms": ms_topk, "gbs": topk_gbs, "frac_hbm": topk_gbs / PEAK_HBM_GBS,
                     "rows_per_s": tokens / (ms_topk * 1e-3)},
            "attention": {"ms": ms_att, "tflops": att_tflops,
                          "frac_bf16_peak": att_tflops / PEAK_BF16_TFLOPS},
            "prefill_entry_ms": ms_prefill,
            "prefill_entry_flushed_ms": ms_prefill_flushed,
            "flushed_ms": {"indexer": float(flushed[0]), "topk": float(flushed[1]),
                           "attention": float(flushed[2]), "reps": args.flush_reps},
            "attention_ms_stage_events": float(ms_att4),
            "timing": ("value: wall clock of the timed steps (events only around attention); "
                       "attention ms: median of those events; indexer and top-k ms: median of "
                       "a second run of as many steps with events at every stage boundary"),
            "e2e_roofline_ms": roof_s * 1e3,
            "e2e_frac_of_roofline": roof_s * 1e3 / ms_step,
            "indexer_topk_fused": {
                "ms": ms_fused, "same_topk_as_unfused": fused_same,
                "peak_bytes": peak_fused, "unfused_peak_bytes": peak_unfused,
                "logits_buffer_bytes": B * M * N * 4},
            "backward": bwd,
            "attention_full_fp8": f8,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        eprint("[bench] cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(wl, x, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
