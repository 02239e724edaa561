"""Benchmark of one DSA layer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config decode_v32] [--latent fp8]

A step is one call of dsa_layer_step over the whole batch: index scores over every
cached key of every sequence, top-k, sparse attention over the selected latent rows.
Inputs are seeded synthetic tensors of the configuration's shapes, resident in HBM
before the timed region; several independent input sets are cycled so that the
256 MB Infinity Cache cannot serve a step from the previous one.

Prints one JSON line: layer-steps/s (value), keys scored/s, the roofline of the
dominant kernel from HIP events recorded by the library during a second pass of the
same steps, the HBM traffic measured by rocprofv3 counters (from profiles/, when they
match the current kernel source), and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, published
METRIC = "DSA decode layer-steps/s and indexer keys scored/s; % of HBM/MFMA roofline"
ATTN_SOURCE = os.path.join(ROOT, "deepseek_dsa_indexer_amd", "csrc", "sparse_attn.hip")
INDEX_SOURCE = os.path.join(ROOT, "deepseek_dsa_indexer_amd", "csrc", "index_scores.hip")
PREFILL_SOURCE = os.path.join(ROOT, "deepseek_dsa_indexer_amd", "csrc", "sparse_mha_prefill.hip")


def _sha(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def algorithmic_costs(cfg, lens, latent_form="bf16"):
    """Bytes and flops the method must move / execute per step, per phase.

    Indexer: every sequence's K-cache once, 132 B (128 FP8 + 4 B scale) per cached key,
    plus each row's q (H_I*d_I B), weights and q scales (8*H_I B); 2*H_I*d_I flops per
    visible (row, key).  Latent attention: 1152 B (576 bf16) per selected latent row, or
    656 B in the FP8 row form, shared by all heads, 2*H*(576+512) flops per (head,
    selected row), plus the row's q (H*576*2 B) and output (H*512*2 B).  MHA attention: the chunk's K and V once
    (H*(Dqk+Dv)*2 B per key), q and output, and 2*H*(Dqk+Dv) flops per (head,
    selected row)."""
    import dsa_synth as S
    T = cfg.T
    keys = S.visible_keys(cfg, lens)
    rows = cfg.B * T
    sel = 0
    for L in lens:
        for t in range(T):
            sel += min(cfg.k, int(L) - T + t + 1)
    cached = int(sum(min(int(L), cfg.Lmax) for L in lens))
    idx_bytes = cached * (cfg.D_I + 4) + rows * (cfg.H_I * cfg.D_I + 8 * cfg.H_I)
    idx_flops = keys * 2 * cfg.H_I * cfg.D_I
    if cfg.form == "latent":
        row_bytes = S.FP8_LATENT_ROW_BYTES if latent_form == "fp8" else cfg.Dq * 2
        att_bytes = sel * row_bytes + rows * (cfg.H * cfg.Dq * 2 + cfg.H * cfg.Dv * 2)
        att_flops = sel * 2 * cfg.H * (cfg.Dq + cfg.Dv)
    else:
        att_bytes = rows * cfg.H * (cfg.Dqk + cfg.Dv) * 2 + rows * cfg.H * (cfg.Dqk + cfg.Dv) * 2
        att_flops = sel * 2 * cfg.H * (cfg.Dqk + cfg.Dv)
    return dict(keys=keys, selected=sel, index_bytes=idx_bytes, index_flops=idx_flops,
                attention_bytes=att_bytes, attention_flops=att_flops)


def read_traffic(kernel: str, workload: str, source: str):
    """Per-launch HBM bytes measured with rocprofv3 --pmc (FETCH_SIZE, WRITE_SIZE),
    calibrated against a copy kernel, from profiles/traffic_<kernel>_<workload>.txt;
    None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != _sha(source):
        return None
    try:
        return float(vals["fetch_bytes"]) + float(vals["write_bytes"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(cfg, n_seqs: int, min_seconds: float = 10.0, latent_form: str = "bf16"):
    """The oracle, untuned, on a bounded sample of the same workload, scaled to a step.

    Decode: the whole layer step for the first ``n_seqs`` sequences.  Chunked prefill
    (one sequence, either form): ``4 * n_seqs`` query rows spread evenly over the chunk,
    each scored against its causal keys, selected and attended; the step is T rows.  The sample is
    repeated until ``min_seconds`` of wall time have accumulated."""
    import numpy as np

    import dsa_synth as S
    import oracle as orc
    orc.build(force=False)
    if cfg.form == "latent" and cfg.T == 1:
        seqs = list(range(min(n_seqs, cfg.B)))
        c = S.make_case(cfg, seqs=seqs, latent_form=latent_form)

        def once():
            orc.layer_step_latent(c["q_i"], c["q_scale"], c["w"], c["k_i"], c["k_scale"],
                                  c["lens"], cfg.sm_scale_i, cfg.k, c["q"], c["latent"], cfg.Dv,
                                  cfg.sm_scale)
        frac = len(seqs) / cfg.B
        keys = float(np.sum(c["lens"]))
        threads = min(orc.max_threads(), len(seqs) * cfg.T)
        sample = (f"{len(seqs)} of {cfg.B} sequences of the same workload (full index scan, "
                  f"top-k and attention per sequence), scaled by {cfg.B}/{len(seqs)}")
    else:
        c = S.make_case(cfg)
        n_rows = min(4 * n_seqs, cfg.T)
        rows = [int(t) for t in np.linspace(0, cfg.T - 1, n_rows)]
        idx = np.full((cfg.B, cfg.T, cfg.k), -1, np.int32)

        def once():
            for t in rows:
                sc = orc.index_scores(c["q_i"][:, t:t + 1], c["q_scale"][:, t:t + 1],
                                      c["w"][:, t:t + 1], c["k_i"], c["k_scale"],
                                      np.array([t + 1], np.int32), cfg.sm_scale_i)
                idx[:, t] = orc.topk(sc, np.array([t + 1], np.int32), cfg.k)[:, 0]
                if cfg.form == "latent":
                    orc.sparse_mla_decode(c["q"][:, t:t + 1], c["latent"], idx[:, t:t + 1],
                                          np.array([t + 1], np.int32), cfg.Dv, cfg.sm_scale)
            if cfg.form != "latent":
                orc.sparse_mha_prefill_rows(c["q"], c["k"], c["v"], idx, cfg.sm_scale,
                                            [(0, t) for t in rows])
        frac = n_rows / cfg.T
        keys = float(sum(t + 1 for t in rows))
        threads = orc.max_threads()
        sample = (f"{n_rows} of {cfg.T} query rows spread evenly over the chunk (index "
                  f"scores, top-k and attention per row), scaled by {cfg.T}/{n_rows}")
    reps = 0
    t0 = time.perf_counter()
    while True:
        once()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    keys *= reps
    sample += f"; {reps} repetitions in {dt:.1f} s wall"
    return {"value": reps * frac / dt, "unit": "layer-steps/s", "cores": threads, "kind": "oracle",
            "sample": sample + f"; threads available {orc.max_threads()}",
            "keys_scored_per_s": keys / dt}


def measure_prep(D, S, cfg, n: int):
    """The indexer preparation of the workload's new tokens (B*T of them: rope, rotation,
    FP8 quantisation, key-cache append), timed alone: n launches captured in one HIP
    graph and replayed under HIP events, so the host's launch rate does not enter (a
    decode-sized launch is shorter than a launch from Python).  Not part of the layer
    step; reported beside it.  Algorithmic bytes: the q and k rows and their rope angles
    read, the codes and scales written."""
    import torch
    c = S.make_prep_case(cfg)
    d = S.to_device(c, "cuda")
    R = cfg.rope_i
    tokens = cfg.B * cfg.T
    in_b = 2 if cfg.attn_dtype == "bf16" else 4
    nbytes = tokens * ((cfg.H_I + 1) * cfg.D_I * (in_b + 1) + (cfg.H_I + 1) * 4 + R * 4)
    run = lambda: D.indexer_prep(d["q"], d["k"], d["cos"], d["sin"], d["start"], R, d["k_cache"],
                                 d["k_scale"])
    q_fp8, q_scale = run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            D.indexer_prep(d["q"], d["k"], d["cos"], d["sin"], d["start"], R, d["k_cache"],
                           d["k_scale"], q_fp8, q_scale)
    g.replay()                                       # warm
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    g.replay()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / n
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"tokens": tokens, "avg_launch_ms": round(ms, 5), "algorithmic_bytes_per_launch": nbytes,
            "achieved_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="decode_v32")
    ap.add_argument("--sets", type=int, default=4, help="independent input sets cycled")
    ap.add_argument("--latent", choices=["bf16", "fp8"], default="bf16",
                    help="latent cache rows: bf16 (1152 B) or the FP8 storage form (656 B: "
                         "512 e4m3fn codes, four fp32 block scales, 64 bf16 rope values)")
    ap.add_argument("--graph", action="store_true", help="replay each step from a HIP graph")
    ap.add_argument("--cpu-seqs", type=int, default=32,
                    help="sequences (decode) or rows / 4 (prefill) in the CPU-oracle sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="the CPU-oracle sample repeats until this much wall time has passed")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (10 times) and exit: the "
                         "reference point for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": 4 * n}))
        return

    import deepseek_dsa_indexer_amd as D
    import dsa_synth as S

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    D.load()
    cfg = S.CONFIGS[args.config]
    fp8_lat = args.latent == "fp8"
    if fp8_lat and cfg.form != "latent":
        print("--latent fp8 applies to the latent (decode) workloads only", file=sys.stderr)
        sys.exit(2)
    lens = S.lengths(cfg)
    costs = algorithmic_costs(cfg, lens, args.latent)

    steps = []
    t_gen = time.perf_counter()
    for i in range(args.sets):
        c = S.make_case(dataclasses.replace(cfg, seed=cfg.seed + 1000 * i) if i else cfg,
                        latent_form=args.latent)
        d = S.to_device(c, "cuda")
        del c
        if cfg.form == "latent":
            step = D.LayerStep(d["q_i"], d["q_scale"], d["w"], d["k_i"], d["k_scale"], d["lens"],
                               cfg.sm_scale_i, cfg.k, d["q"], cfg.sm_scale, latent=d["latent"],
                               Dv=cfg.Dv)
        else:
            step = D.LayerStep(d["q_i"], d["q_scale"], d["w"], d["k_i"], d["k_scale"], d["lens"],
                               cfg.sm_scale_i, cfg.k, d["q"], cfg.sm_scale, k=d["k"], v=d["v"])
        steps.append(step)
    torch.cuda.synchronize()
    print(f"[bench] {cfg.name}: {args.sets} input sets on the GPU in "
          f"{time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    run = [s for s in steps]
    if args.graph:
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for s in steps:
                s()                                   # warm the launch path before capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for s in steps:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                s()
            graphs.append(g)
        run = [g.replay for g in graphs]

    for i in range(args.warmup):
        run[i % len(run)]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run[i % len(run)]()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_per_step = 1e3 * dt / args.steps
    value = args.steps / dt

    # per-step distribution: HIP events around every step (the library enqueues on the
    # current stream, which is where torch records its events)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record()
        run[i % len(run)]()
        evs[i][1].record()
    torch.cuda.synchronize()
    step_ms = sorted(a.elapsed_time(b) for a, b in evs)
    pct = lambda q: step_ms[min(len(step_ms) - 1, int(q * len(step_ms)))]

    # next pass of the same steps with the library's per-phase HIP events
    D.profile_begin(args.steps)
    for i in range(args.steps):
        steps[i % len(steps)]()
    prof = D.profile_end()
    torch.cuda.synchronize()
    phase_ms = {k: (v[0] / v[1] if v[1] else None) for k, v in prof.items()}
    print(f"[bench] phases (avg ms): {phase_ms}", file=sys.stderr, flush=True)

    prep = measure_prep(D, S, cfg, args.steps)
    print(f"[bench] indexer prep: {prep}", file=sys.stderr, flush=True)

    att_ms = phase_ms["attention"]
    idx_ms = phase_ms["index_scores"]
    att_gbs = costs["attention_bytes"] / (att_ms * 1e-3) / 1e9
    att_tfs = costs["attention_flops"] / (att_ms * 1e-3) / 1e12
    idx_gbs = costs["index_bytes"] / (idx_ms * 1e-3) / 1e9
    idx_tfs = costs["index_flops"] / (idx_ms * 1e-3) / 1e12
    if cfg.form == "latent":
        kernel, tkey, src = "mla_decode_mfma_kernel", "sparse_mla_decode", ATTN_SOURCE
    else:
        kernel, tkey, src = "mha_prefill_mfma_kernel", "sparse_mha_prefill", PREFILL_SOURCE
    traffic = read_traffic(tkey, cfg.name + ("-fp8" if fp8_lat else ""), src)
    # the attention kernel's bound: whichever of its bytes or its flops takes longer at peak
    mfma_bound = costs["attention_flops"] / (BF16_PEAK_TFLOPS * 1e12) > \
        costs["attention_bytes"] / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        roofline = {"bound": "mfma", "achieved": round(att_tfs, 1), "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(att_tfs / BF16_PEAK_TFLOPS, 4),
                    "algorithmic_flops_per_launch": costs["attention_flops"],
                    "hbm_frac": round(att_gbs / HBM_PEAK_GBS, 4)}
    else:
        roofline = {"bound": "hbm", "achieved": round(att_gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(att_gbs / HBM_PEAK_GBS, 4),
                    "algorithmic_bytes_per_launch": costs["attention_bytes"],
                    "mfma_frac": round(att_tfs / BF16_PEAK_TFLOPS, 4)}
    roofline.update({"traffic": traffic, "kernel": kernel, "avg_launch_ms": round(att_ms, 5)})
    # the step's floor: each phase at the larger of its HBM time and its MFMA time at peak
    t_roof = sum(max(costs[f"{p}_bytes"] / (HBM_PEAK_GBS * 1e9),
                     costs[f"{p}_flops"] / (BF16_PEAK_TFLOPS * 1e12)) for p in ("index", "attention"))
    if cfg.form == "latent":
        attn_desc = (f"MLA {cfg.H} heads over FP8 latent rows (656 B: {cfg.Dv} e4m3fn + 4 "
                     f"block scales + {cfg.Dr} bf16 rope)" if fp8_lat else
                     f"MLA {cfg.H} heads over bf16 latent {cfg.Dv}+{cfg.Dr}")
    else:
        attn_desc = f"MHA {cfg.H} heads, bf16 qk {cfg.Dqk} / v {cfg.Dv}"
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: B={cfg.B}, context {cfg.Lmax} per sequence, T={cfg.T}, "
                               f"indexer {cfg.H_I}x{cfg.D_I} FP8, top-{cfg.k}, {attn_desc}",
                   "B": cfg.B, "context": cfg.Lmax, "T": cfg.T, "topk": cfg.k, "H_I": cfg.H_I,
                   "d_I": cfg.D_I, "H": cfg.H, "q_width": cfg.Dq, "input_sets": args.sets,
                   "latent_cache": args.latent if cfg.form == "latent" else None,
                   "hip_graph": bool(args.graph)},
        "step_ms_p10_p50_p90": [round(pct(0.1), 5), round(pct(0.5), 5), round(pct(0.9), 5)],
        "token_layer_steps_per_s": round(cfg.B * cfg.T * value, 1),
        "keys_scored_per_s": round(costs["keys"] * value, 1),
        "keys_per_step": costs["keys"],
        "step_roofline_frac": round(t_roof / (ms_per_step * 1e-3), 4),
        "phases_avg_ms": {k: (round(v, 5) if v is not None else None) for k, v in phase_ms.items()},
        "index_scores": {"achieved_GBs": round(idx_gbs, 1), "hbm_frac": round(idx_gbs / HBM_PEAK_GBS, 4),
                         "achieved_TFLOPs": round(idx_tfs, 1),
                         "mfma_frac": round(idx_tfs / BF16_PEAK_TFLOPS, 4),
                         "keys_per_s": round(costs["keys"] / (idx_ms * 1e-3), 1)},
        "roofline": roofline,
        "indexer_prep": prep,
        "cpu_baseline": None if args.no_cpu else cpu_baseline(cfg, args.cpu_seqs, args.cpu_seconds,
                                                              args.latent),
    }
    print(json.dumps(result))


if __name__ == "__main__":
    main()
