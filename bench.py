"""Benchmark of the CSA / HCA decode hot path on one MI355X.

Workload (default): Pro-shape decode at 1M context. B = 4 independent sequences, each
with n = 2^20 cached tokens, issue one query at t = n. One step is one CSA layer plus
one HCA layer of that decode:
  CSA: csa_compress (the block [n-4, n) completes: new KV entry and new index-key entry)
       -> csa_index_scores over all 262,144 entries (64 heads x 128, bf16 per-head keys)
       -> csa_topk (k = 1,024) -> csa_sparse_attn (128 heads x 512, 1,024 + 128 SWA rows)
  HCA: csa_compress (ratio 128: summary 8,191 completes) -> hca_attn over 8,192 summaries
       + 128 SWA rows.
Inputs are seeded synthetic tensors resident in HBM before the timed region.

Prints one JSON line: decode queries/s (value), the index-scan kernel's achieved HBM
bandwidth against MI355X's 8 TB/s (roofline), and the CPU oracle's rate on a bounded
sample of the same step (cpu_baseline).
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

METRIC = "decode queries/s + indexer GB/s (% HBM roofline), Pro shape, 1M ctx, 1 GPU"
HBM_PEAK_GBS = 8000.0
PMC_FILE = os.path.join(ROOT, "profiles", "index_scan_pro_decode_1m_pmc.json")
SCAN_SRC = os.path.join(ROOT, "long_context_compressed_amd", "csrc", "indexer.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-entries", type=int, default=16384,
                    help="index entries per query in the oracle's bounded sample")
    ap.add_argument("--workload", default="pro_decode_1m",
                    choices=["pro_decode_1m", "flash_decode_128k", "pro_decode_1m_shared_keys", "pro_decode_1m_mxfp4",
                             "pro_decode_1m_kv8",
                             "pro_prefill_chunk",
                             "hca_prefill_4k", "pro_prefill_q_norm_rope", "pro_prefill_projections"],
                    help="pro_decode_1m is the benchmark line; the others print the same record for "
                         "the other configurations' shapes (profiling aid)")
    ap.add_argument("--profile-copy", action="store_true",
                    help="before the timed region, run a plain 1 GiB device copy three times (a kernel of "
                         "known traffic that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    return ap.parse_args()


def scan_source_hash() -> str:
    return hashlib.sha256(open(SCAN_SRC, "rb").read()).hexdigest()[:16]


def traffic_from_profile(alg_bytes):
    """HBM bytes per index-scan launch from the committed rocprofv3 counter summary,
    or None when it is missing or was taken on a different kernel source."""
    try:
        d = json.load(open(PMC_FILE))
    except (OSError, ValueError):
        return None
    if d.get("indexer_hip_sha256_16") != scan_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {a.gpus}); "
              "the multi-GPU sharding is a design, not a measured path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import long_context_compressed_amd as csa
    from long_context_compressed_amd import pipeline
    import workloads as W

    dev = "cuda"
    torch.cuda.set_device(0)
    csa.lib()
    if a.workload in ("pro_prefill_chunk", "hca_prefill_4k"):
        return prefill_main(a)
    if a.workload == "pro_prefill_q_norm_rope":
        return rownorm_main(a)
    if a.workload == "pro_prefill_projections":
        return projections_main(a)
    cfg = W.FLASH if a.workload == "flash_decode_128k" else W.PRO
    shared = a.workload == "pro_decode_1m_shared_keys"
    fp4 = a.workload == "pro_decode_1m_mxfp4"
    kv8 = a.workload == "pro_decode_1m_kv8"  # compressed KV and summaries in the FP8 storage format
    B, T, n, N, D, H, k = cfg.B, cfg.T, cfg.n, cfg.N, cfg.c, cfg.H, cfg.k
    NH = cfg.n // 128  # HCA summaries (8,192 at 2^20 tokens)

    # ---- inputs (HBM-resident) and the step's buffers -----------------------------------
    inp = W.decode_step_inputs(cfg, dev, shared_keys=shared, mxfp4=fp4, kv8=kv8)
    step = pipeline.DecodeStep(inp, k, cfg.window, cfg.rope_dim, cfg.scale)
    torch.cuda.synchronize()

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    if a.profile_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # the events sit on the stream the library launches on (torch's current stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    scan_ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    scan_avg_s = float(np.mean(scan_ms)) / 1e3

    # ---- per-stage times (separate, untimed-for-value pass) ---------------------------
    def timed(fn, reps=50):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    # the same small stages in the step's own conditions: right after an index scan, which
    # has streamed gigabytes of keys past every cache (the events are enqueued while the scan
    # runs, so no host gap is timed); the median of 5
    def in_step(fn, reps=5):
        ts = []
        for _ in range(reps):
            step.index()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    stages_in_step = {
        "compress_kv_index_key_summary": in_step(step.compress),
        **({} if step.fused else {"topk": in_step(step.select)}),
        "sparse_attn": in_step(step.attend),
        "hca_attn": in_step(step.hca),
    }
    stages = {
        "compress_kv_index_key_summary": timed(step.compress),
        **({"quantize_q_mxfp4": timed(step.index_prep)} if fp4 else {}),
        **({"index_topk_fused": timed(step.index, reps=10)} if step.fused else
           {"index_scores": timed(step.index, reps=10), "topk": timed(step.select)}),
        "sparse_attn": timed(step.attend),
        "hca_attn": timed(step.hca),
    }
    kv, k_I, summ, sink_h, scores, idx = inp["kv"], inp["k_I"], inp["summ"], inp["sink_h"], step.scores, step.idx

    # algorithmic bytes of one index-scan launch: every visible key block once
    # (64 x 128 bf16 = 16 KiB per entry per sequence) + q_I + w + the fp32 scores
    # (MXFP4: 64 x 64 bytes of codes + 64 x 4 E8M0 scales = 4,352 B per entry, same for q_I)
    if fp4:  # (fused with the top-k: no score array, the k winners of each 4,096-entry chunk)
        alg_bytes = B * N * 4352 + T * 4352 + T * 64 * 4 + T * ((N + 4095) // 4096) * k * 8
    else:
        alg_bytes = B * N * (1 if shared else 64) * 128 * 2 + T * 64 * 128 * 2 + T * 64 * 4 + T * N * 4
    achieved = alg_bytes / scan_avg_s / 1e9
    traffic = None if shared or a.workload != "pro_decode_1m" else traffic_from_profile(alg_bytes)

    res = {
        "metric": METRIC,
        "value": round(B * a.steps / elapsed, 2),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(elapsed / a.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), bf16)",
        "config": {
            "workload": (f"{a.workload}: one CSA layer + one HCA layer decode step, B={B} sequences x 1 query at "
                         f"t={n}; {N:,} entries x {'1 shared' if shared else '64 per-head'} x 128 "
                         f"{'MXFP4 (Hadamard-rotated)' if fp4 else 'bf16'} index keys "
                         f"per sequence, top-k {k:,}, "
                         f"{H} heads x {D} shared KV{' (FP8 rows, 592 B)' if kv8 else ''}, SWA {cfg.window}, "
                         f"{NH:,} HCA summaries"),
            "batch": B, "context": n, "index_entries": N, "topk": k, "heads": H, "head_dim": D,
        },
        "roofline": {
            "kernel": ("index_shared_kernel (csa_index_scores, bf16 keys shared by the 64 heads)" if shared
                       else "index_mxfp4_topk_kernel + the selection over its chunk winners (csa_index_topk: "
                            "MXFP4 per-head keys, scan fused with the top-k; the time covers both)" if fp4
                       else "index_scan_kernel (csa_index_scores, bf16 per-head keys)"),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": alg_bytes,
            "avg_launch_ms": round(scan_avg_s * 1e3, 4),
            "median_launch_ms": round(float(np.median(scan_ms)), 4),
            "min_launch_ms": round(float(np.min(scan_ms)), 4),
        },
        "stages_ms": {kk: round(v, 4) for kk, v in stages.items()},
        "stages_in_step_ms": {kk: round(v, 4) for kk, v in stages_in_step.items()},
    }
    if a.workload != "pro_decode_1m":
        res["metric"] = f"decode queries/s + indexer GB/s, {a.workload} (profiling line, not the benchmark)"
    if not a.no_cpu and a.workload == "pro_decode_1m":
        res["cpu_baseline"] = cpu_baseline(a, inp, kv, k_I, summ, sink_h, scores, idx, cfg, NH)
    res["host"] = host_info()
    print(json.dumps(res), flush=True)


def prefill_main(a):
    """Prefill chunks (profiling aid): the whole CSA or HCA prefill path of one chunk.

    pro_prefill_chunk: 8,192 new tokens after a 65,536-token context. csa_compress of the
      chunk (+ the carry of block 16,383) writes KV rows 16,384..18,431; csa_index_scores
      with MXFP4 operands (8,192 queries x 18,432 entries, causal); csa_topk (k = 1,024);
      csa_sparse_attn (128 heads x 512, 1,024 + 128 rows per query).
    hca_prefill_4k: the last 4,096 tokens of a 2^20 context. csa_compress (ratio 128) writes
      summaries 8,160..8,191; hca_attn (4,096 queries, every visible summary + 128 SWA rows).
    Dominant kernel for the roofline line: the attention (bf16 MFMA, FLOP-bound).
    """
    import numpy as np
    import torch

    from long_context_compressed_amd import pipeline
    import workloads as W

    dev = "cuda"
    inp = W.prefill_inputs(a.workload, dev)
    cfg, T, D, H = inp["cfg"], inp["T"], inp["D"], inp["H"]
    if a.workload == "pro_prefill_chunk":
        chunk = pipeline.ProPrefillChunk(inp, inp["k"], cfg.window, cfg.rope_dim, cfg.scale)
        rows = inp["k"] + cfg.window
        flops = 4.0 * T * H * rows * D
        dominant = "sparse_attn"
    else:
        chunk = pipeline.HcaPrefillChunk(inp, cfg.window, cfg.rope_dim, cfg.scale)
        pos = inp["q_pos"].cpu().numpy()
        rows = float(np.sum(np.minimum(inp["NH"], pos // 128) + cfg.window))
        flops = 4.0 * H * rows * D
        dominant = "hca_attn"
    stages = chunk.stages()
    torch.cuda.synchronize()

    def step():
        for f in stages.values():
            f()

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    dom_ms = []
    t0 = time.perf_counter()
    for _ in range(a.steps):
        for nm, f in stages.items():
            if nm == dominant:
                ev[0].record()
                f()
                ev[1].record()
                ev[1].synchronize()
                dom_ms.append(ev[0].elapsed_time(ev[1]))
            else:
                f()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    stage_ms = {}
    for nm, f in stages.items():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            f()
        e1.record()
        torch.cuda.synchronize()
        stage_ms[nm] = round(e0.elapsed_time(e1) / 3, 4)
    dom_s = float(np.mean(dom_ms)) / 1e3
    achieved = flops / dom_s / 1e12
    res = {
        "metric": f"prefill tokens/s, {a.workload} (profiling line, not the benchmark)",
        "value": round(T * a.steps / elapsed, 1), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(elapsed / a.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": a.workload, "queries": T, "heads": H, "head_dim": D},
        "roofline": {"kernel": dominant, "bound": "mfma", "achieved": round(achieved, 2), "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": round(achieved / 2500.0, 4), "traffic": None,
                     "algorithmic_flops_per_launch": flops, "avg_launch_ms": round(dom_s * 1e3, 4),
                     "median_launch_ms": round(float(np.median(dom_ms)), 4),
                     "min_launch_ms": round(float(np.min(dom_ms)), 4)},
        "stages_ms": stage_ms,
    }
    res["host"] = host_info()
    print(json.dumps(res), flush=True)


def rownorm_main(a):
    """RMSNorm + partial RoPE of the Pro prefill chunk's queries (profiling aid):
    csa_rmsnorm_rope over 8,192 tokens x 128 heads rows of 512 bf16 dims, gains U(0.5, 1.5),
    eps 1e-6, the last 64 dims rotated at each token's position (one angle row per 128 head
    rows), into a separate bf16 output. An HBM stream: 2 x 1,024 bytes per row plus the
    256-byte angle row of each token."""
    import numpy as np
    import torch

    import long_context_compressed_amd as csa
    import workloads as W

    cfg = W.PRO_PREFILL
    T, H, D, R, s = cfg.T, cfg.H, cfg.c, cfg.rope_dim, cfg.seed
    q = W.normal((T, H, D), s, "q", dtype=torch.bfloat16, device="cuda")
    g = W.uniform((D,), s, "q_norm_gain", lo=0.5, hi=1.5, device="cuda")
    cs = W.rope_table(torch.arange(cfg.n, cfg.n + T, dtype=torch.int64), R).to("cuda")
    out = torch.empty_like(q)
    st = torch.cuda.current_stream()
    alg = T * H * D * 2 * 2 + T * R * 4 + D * 4
    for _ in range(a.warmup):
        csa.rmsnorm_rope(q, g, 1e-6, rope_cs=cs, rope_group=H, out=out, stream=st)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(st)
        csa.rmsnorm_rope(q, g, 1e-6, rope_cs=cs, rope_group=H, out=out, stream=st)
        e1.record(st)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    avg = float(np.mean(ms)) / 1e3
    gbs = alg / avg / 1e9
    # context: torch's device copy of the same rows (the same read + write bytes)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out.copy_(q)
    c0.record(st)
    for _ in range(20):
        out.copy_(q)
    c1.record(st)
    torch.cuda.synchronize()
    copy_ms = c0.elapsed_time(c1) / 20
    res = {
        "metric": "query rows/s, RMSNorm + RoPE of the Pro prefill chunk's q (profiling line, not the benchmark)",
        "value": round(T * H * a.steps / elapsed, 1), "unit": "rows/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(elapsed / a.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": a.workload, "rows": T * H, "dim": D, "rope_dim": R},
        "roofline": {"kernel": "rmsnorm_rope_kernel", "bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0,
                     "unit": "GB/s", "frac": round(gbs / 8000.0, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": alg, "avg_launch_ms": round(avg * 1e3, 4),
                     "median_launch_ms": round(float(np.median(ms)), 4), "min_launch_ms": round(float(np.min(ms)), 4),
                     "torch_copy_same_rows_ms": round(copy_ms, 4)},
    }
    res["host"] = host_info()
    print(json.dumps(res), flush=True)


def projections_main(a):
    """The projections around the Pro prefill chunk's attention (profiling aid), both bf16
    matrix-core GEMMs with fp32 sums:
      compress_hidden: the KV compressor fed from the chunk's hidden rows, 8,192 tokens x
        7,168 (the Pro hidden width) through four 7,168 -> 512 projections, pooled 4:1 in
        the epilogue: 2 x 8,192 x 7,168 x 2,048 = 240.5 GFLOP;
      out_proj: 8,192 tokens x 128 heads x 512 -> 16 groups of 1,024 -> 7,168 (group count
        and width are synthetic choices; the pages give neither): 2 x 8,192 x 65,536 x
        1,024 + 2 x 8,192 x 16,384 x 7,168 = 3.024 TFLOP.
    Weights 0.05 N(0, 1), activations N(0, 1), bf16."""
    import numpy as np
    import torch

    import long_context_compressed_amd as csa
    import workloads as W

    dev = "cuda"
    n, d, c = 8192, 7168, 512
    T, H, D, G, dg, dm = 8192, 128, 512, 16, 1024, 7168
    s = 1004
    hid = W.normal((1, n, d), s, "proj_hidden", dtype=torch.bfloat16, device=dev)
    Wc = W.normal((4, c, d), s, "proj_Wc", scale=0.05, dtype=torch.bfloat16, device=dev)
    cH = W.normal((1, 4, d), s, "proj_carry", dtype=torch.bfloat16, device=dev)
    kvo = torch.empty((1, n // 4, c), dtype=torch.bfloat16, device=dev)
    o = W.normal((T, H, D), s, "proj_o", dtype=torch.bfloat16, device=dev)
    Wa = W.normal((G, dg, (H // G) * D), s, "proj_Wa", scale=0.05, dtype=torch.bfloat16, device=dev)
    Wb = W.normal((dm, G * dg), s, "proj_Wb", scale=0.05, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(csa.out_proj_workspace_bytes(T, G, dg), dtype=torch.uint8, device=dev)
    y = torch.empty((T, dm), dtype=torch.bfloat16, device=dev)
    st = torch.cuda.current_stream()
    stages = {"compress_hidden": (lambda: csa.compress_hidden(hid, Wc, cH, out=kvo, stream=st), 2.0 * n * d * 4 * c),
              "out_proj": (lambda: csa.out_proj(o, Wa, Wb, out=y, workspace=ws, stream=st),
                           2.0 * T * H * D * dg + 2.0 * T * G * dg * dm)}
    for _ in range(a.warmup):
        for f, _fl in stages.values():
            f()
    torch.cuda.synchronize()
    ms = {k: [] for k in stages}
    t0 = time.perf_counter()
    for _ in range(a.steps):
        for k, (f, _fl) in stages.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            f()
            e1.record(st)
            ms[k].append((e0, e1))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    avg = {k: float(np.mean([e0.elapsed_time(e1) for e0, e1 in v])) for k, v in ms.items()}
    lines = {k: {"avg_launch_ms": round(avg[k], 4), "tflops": round(fl / avg[k] / 1e9, 1),
                 "frac_of_bf16_peak": round(fl / avg[k] / 1e9 / 2500.0, 4), "algorithmic_flops": fl}
             for k, (_f, fl) in stages.items()}
    fl_tot = sum(fl for _f, fl in stages.values())
    ach = fl_tot / (sum(avg.values()) / 1e3) / 1e12
    res = {
        "metric": "prefill projection TFLOP/s, pro_prefill_projections (profiling line, not the benchmark)",
        "value": round(T * a.steps / elapsed, 1), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(elapsed / a.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": a.workload, "tokens": T, "hidden": d, "kv_dim": c, "heads": H, "head_dim": D,
                   "groups": G, "group_width": dg},
        "roofline": {"kernel": "gemm_bf16_kernel / compress_hidden_kernel", "bound": "mfma",
                     "achieved": round(ach, 1), "peak": 2500.0, "unit": "TFLOP/s", "frac": round(ach / 2500.0, 4),
                     "traffic": None, "algorithmic_flops_per_step": fl_tot},
        "stages": lines,
    }
    res["host"] = host_info()
    print(json.dumps(res), flush=True)


def cpu_baseline(a, inp, kv, k_I, summ, sink_h, scores, idx, cfg, NH):
    """The fp64 oracle on a bounded sample of the same decode step, scaled to queries/s.

    Sample: the index scores of all B queries over `cpu_entries` randomly chosen entries
    (scaled by N / cpu_entries), top-k over the full 262,144 scores of every query, the
    sparse attention of every query (1,152 rows x 128 heads), and the HCA attention of
    one query (8,320 rows x 128 heads, scaled by B). Only the oracle's own calls are
    timed, not the widening of the inputs to fp64.
    """
    import numpy as np
    import torch

    import oracle
    import workloads as W

    oracle.lib()
    B, T, N = cfg.B, cfg.T, cfg.N
    S = min(a.cpu_entries, N)
    f64 = lambda x: x.detach().to("cpu", torch.float64).numpy()
    npy = lambda x: x.detach().cpu().numpy()
    ids = np.sort(W.distinct_sample(S, N, cfg.seed, "cpu_sample"))
    k_s = f64(k_I.index_select(1, torch.from_numpy(ids).to(k_I.device)))
    qI, w, qs, qp = f64(inp["q_I"]), f64(inp["w"]), npy(inp["q_seq"]), npy(inp["q_pos"])
    q, sink, swa, p0, cs = f64(inp["q"]), f64(inp["sink"]), f64(inp["swa"]), npy(inp["swa_pos0"]), f64(inp["rope_cs"])
    # the rows each query's sparse attention reads, gathered (query t reads sequence t)
    idx_h = npy(idx).astype(np.int64)
    kv_c = np.stack([f64(kv[t].index_select(0, torch.from_numpy(np.maximum(idx_h[t], 0)).to(kv.device)))
                     for t in range(T)])
    idx_c = np.where(idx_h >= 0, np.arange(cfg.k)[None, :], -1).astype(np.int32)
    summ1, sinkh = f64(summ[:1]), f64(sink_h)
    sc = scores.double().cpu().numpy()

    t_idx = _time_call(lambda: oracle.index_scores(qI, w, k_s, qs, qp, entry_ids=ids)) * (N / S)
    t_topk = _time_call(lambda: oracle.topk(sc, cfg.k))
    t_attn = _time_call(lambda: oracle.sparse_attn(q, kv_c, sink, idx_c, cfg.scale, swa, p0, cfg.window, qs, qp,
                                                   cs, cfg.rope_dim))
    t_hca = _time_call(lambda: oracle.hca_attn(q[:1], summ1, sinkh, 128, cfg.scale, swa[:1], p0[:1], cfg.window,
                                               np.zeros(1, np.int32), qp[:1], cs[:1], cfg.rope_dim)) * B
    total = t_idx + t_topk + t_attn + t_hca
    return {
        "value": round(B / total, 6),
        "unit": "queries/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": f"index scores of {B} queries over {S} of {N} entries (x{N / S:.0f}), full top-k, full sparse "
                  f"attention, HCA attention of 1 of {B} queries (x{B}); oracle seconds (scaled): index "
                  f"{t_idx:.2f}, topk {t_topk:.2f}, attn {t_attn:.2f}, hca {t_hca:.2f}; 'cores' is the OpenMP "
                  f"thread count (attention steps use at most one thread per query)",
    }


def host_info():
    """CPU model, host threads, ROCm / torch versions and the GPU's name, for the record."""
    import platform

    import torch

    cpu = platform.processor() or ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    rocm = None
    try:
        rocm = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        pass
    return {"cpu_model": cpu, "host_threads": len(os.sched_getaffinity(0)), "rocm": rocm,
            "torch": torch.__version__, "gpu": torch.cuda.get_device_name(0)}


def _time_call(fn):
    """Wall seconds of one oracle call (inputs already widened to fp64 on the host)."""
    t0 = time.perf_counter()
    fn()
    return time.perf_counter() - t0


if __name__ == "__main__":
    main()
