"""Benchmark of one DSA layer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config decode_v32]

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


def _sha(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def algorithmic_costs(cfg, lens):
    """Bytes and flops the method must move / execute per step, per phase.

    Indexer: 132 B (128 FP8 + 4 B scale) and 2*H_I*d_I flops per visible (row, key),
    plus the row's q (H_I*d_I B), weights and q scales (8*H_I B).  Attention: 1152 B
    (576 bf16) per selected latent row, shared by all heads, 2*H*(576+512) flops per
    (head, selected row), plus the row's q (H*576*2 B) and output (H*512*2 B)."""
    import dsa_synth as S
    T = cfg.T
    keys = S.visible_keys(cfg, lens)
    rows = cfg.B * T
    sel = 0
    for L in lens:
        for t in range(T):
            sel += min(cfg.k, int(L) - T + t + 1)
    idx_bytes = keys * (cfg.D_I + 4) + rows * (cfg.H_I * cfg.D_I + 8 * cfg.H_I)
    idx_flops = keys * 2 * cfg.H_I * cfg.D_I
    row_bytes = cfg.Dq * 2
    att_bytes = sel * row_bytes + rows * (cfg.H * cfg.Dq * 2 + cfg.H * cfg.Dv * 2)
    att_flops = sel * 2 * cfg.H * (cfg.Dq + cfg.Dv)
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


def cpu_baseline(cfg, n_seqs: int):
    import numpy as np

    import dsa_synth as S
    import oracle as orc
    orc.build(force=False)
    seqs = list(range(min(n_seqs, cfg.B)))
    c = S.make_case(cfg, seqs=seqs)
    t0 = time.perf_counter()
    if cfg.form == "latent":
        orc.layer_step_latent(c["q_i"], c["q_scale"], c["w"], c["k_i"], c["k_scale"], c["lens"],
                              cfg.sm_scale_i, cfg.k, c["q"], c["latent"], cfg.Dv, cfg.sm_scale)
    else:
        orc.layer_step_mha(c["q_i"], c["q_scale"], c["w"], c["k_i"], c["k_scale"], cfg.sm_scale_i,
                           cfg.k, c["q"], c["k"], c["v"], cfg.sm_scale)
    dt = time.perf_counter() - t0
    frac = len(seqs) / cfg.B
    rows = len(seqs) * cfg.T
    return {"value": frac / dt, "unit": "layer-steps/s", "cores": min(orc.max_threads(), rows),
            "kind": "oracle",
            "sample": f"{len(seqs)} of {cfg.B} sequences of the same workload (full index scan, "
                      f"top-k and attention per sequence), {dt:.2f} s wall, scaled by "
                      f"{cfg.B}/{len(seqs)}; threads available {orc.max_threads()}",
            "keys_scored_per_s": float(np.sum(c["lens"])) / dt}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="decode_v32")
    ap.add_argument("--sets", type=int, default=4, help="independent input sets cycled")
    ap.add_argument("--graph", action="store_true", help="replay each step from a HIP graph")
    ap.add_argument("--cpu-seqs", type=int, default=16, help="sequences in the CPU-oracle sample")
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import torch

    import deepseek_dsa_indexer_amd as D
    import dsa_synth as S

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    D.load()
    cfg = S.CONFIGS[args.config]
    lens = S.lengths(cfg)
    costs = algorithmic_costs(cfg, lens)

    steps = []
    t_gen = time.perf_counter()
    for i in range(args.sets):
        c = S.make_case(dataclasses.replace(cfg, seed=cfg.seed + 1000 * i) if i else cfg)
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

    # second pass of the same steps with the library's per-phase HIP events
    D.profile_begin(args.steps)
    for i in range(args.steps):
        steps[i % len(steps)]()
    prof = D.profile_end()
    torch.cuda.synchronize()
    phase_ms = {k: (v[0] / v[1] if v[1] else None) for k, v in prof.items()}
    print(f"[bench] phases (avg ms): {phase_ms}", file=sys.stderr, flush=True)

    att_ms = phase_ms["attention"]
    idx_ms = phase_ms["index_scores"]
    att_gbs = costs["attention_bytes"] / (att_ms * 1e-3) / 1e9
    idx_gbs = costs["index_bytes"] / (idx_ms * 1e-3) / 1e9
    traffic = read_traffic("sparse_mla_decode", cfg.name, ATTN_SOURCE)
    roofline = {"bound": "hbm", "achieved": round(att_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(att_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "mla_decode_mfma_kernel",
                "algorithmic_bytes_per_launch": costs["attention_bytes"],
                "avg_launch_ms": round(att_ms, 5),
                "mfma_frac": round(costs["attention_flops"] / (att_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    t_roof = (costs["index_bytes"] + costs["attention_bytes"]) / (HBM_PEAK_GBS * 1e9)
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
                               f"indexer {cfg.H_I}x{cfg.D_I} FP8, top-{cfg.k}, MLA {cfg.H} heads over "
                               f"bf16 latent {cfg.Dv}+{cfg.Dr}",
                   "B": cfg.B, "context": cfg.Lmax, "T": cfg.T, "topk": cfg.k, "H_I": cfg.H_I,
                   "d_I": cfg.D_I, "H": cfg.H, "latent": cfg.Dq, "input_sets": args.sets,
                   "hip_graph": bool(args.graph)},
        "keys_scored_per_s": round(costs["keys"] * value, 1),
        "keys_per_step": costs["keys"],
        "step_hbm_roofline_frac": round(t_roof / (ms_per_step * 1e-3), 4),
        "phases_avg_ms": {k: (round(v, 5) if v is not None else None) for k, v in phase_ms.items()},
        "index_scores": {"achieved_GBs": round(idx_gbs, 1), "frac": round(idx_gbs / HBM_PEAK_GBS, 4),
                         "keys_per_s": round(costs["keys"] / (idx_ms * 1e-3), 1)},
        "roofline": roofline,
        "cpu_baseline": None if args.no_cpu else cpu_baseline(cfg, args.cpu_seqs),
    }
    print(json.dumps(result))


if __name__ == "__main__":
    main()
