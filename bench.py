"""Benchmark of one DSA layer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config decode_v32] [--latent fp8] [--graph]

A step is one call of dsa_layer_step over the whole batch: index scores over every
cached key of every sequence, top-k, sparse attention over the selected latent rows.
Inputs are seeded synthetic tensors of the configuration's shapes, resident in HBM
before the timed region; several independent input sets are cycled so that the
256 MB Infinity Cache cannot serve a step from the previous one.

Before each workload's W warm-up steps, its steps run untimed for --ramp-seconds (0.3 s)
so that the GPU's clocks have left the idle state that input generation leaves them in;
the timed steps are eager calls of dsa_layer_step (the library enqueueing each kernel);
the same steps replayed from one HIP graph per input set are timed as well and reported
as graph_ms_per_step (``--graph`` makes them the headline).

Prints one JSON line: layer-steps/s (value) of the headline workload (decode_v32 by
default), keys scored/s, the roofline of the dominant kernel (the sparse attention)
from HIP events that the library records as part of each kernel's dispatch during a
second pass of the same steps (kernel execution only, comparable with a rocprofv3
kernel trace), the HBM traffic measured by rocprofv3 counters (from profiles/, when
they match the current kernel source), the CPU oracle timed on a bounded sample, and
the same measurements for the other workloads as sub-objects (``--only`` skips them).
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
RAMP_S = 0.3                     # untimed steps before each workload's warm-up (seconds)
FP8_PEAK_TFLOPS = 5000.0         # MI355X dense FP8 MFMA, published
METRIC = "DSA decode layer-steps/s and indexer keys scored/s; % of HBM/MFMA roofline"
ATTN_SOURCE = os.path.join(ROOT, "deepseek_dsa_indexer_amd", "csrc", "sparse_mla_decode32.hip")
ATTN_FP8_SOURCE = os.path.join(ROOT, "deepseek_dsa_indexer_amd", "csrc", "sparse_mla_decode32_fp8.hip")
ATTN_GENERIC_SOURCE = os.path.join(ROOT, "deepseek_dsa_indexer_amd", "csrc", "sparse_attn.hip")
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


def latent_32x32_kernel(cfg, fp8_rows: bool) -> bool:
    """Whether the library's latent attention plan takes its 32x32x16 kernel for this
    workload: 64 heads per workgroup, enough key splits to give 256 workgroups, tiles of
    32 bf16 rows (at most 16 per split) or 64 FP8 rows (at most 8), and all of them in one
    wave of at most 256 workgroups (mla_plan in sparse_attn.hip)."""
    if cfg.H not in (64, 128) or cfg.Dv != 512:
        return False
    rows = cfg.B * cfg.T
    parts = cfg.H // 64
    kt, tmax = (64, 8) if fp8_rows else (32, 16)
    n_tiles = -(-cfg.k // kt)
    wg = rows * parts
    s = 1 if wg >= 256 else -(-256 // wg)
    s = max(min(s, 16), -(-n_tiles // tmax))
    s = max(1, min(s, n_tiles))
    return wg * s <= 256


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


def read_rocprof_avg_ms(kernels, workload: str, source: str):
    """Average duration of the kernel named ``kernels`` (a name, or a tuple of names, up to
    the template arguments) in the committed
    rocprofv3 kernel-trace summary profiles/kernels_<workload>.txt; None when absent or
    when the summary was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"kernels_{workload}.txt")
    if not os.path.exists(path):
        return None
    src = os.path.basename(source)
    ok = False
    for line in open(path):
        if line.startswith("# kernel sources"):
            ok = f"{src} {_sha(source)}" in line
        elif ok and not line.startswith("#"):
            name = line.split("calls=")[0].strip()
            if any(name == k or name.startswith(k + "<") for k in
                   ((kernels,) if isinstance(kernels, str) else kernels)):
                return float(line.split("avg_ns=")[1].split()[0]) * 1e-6
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
    res = {"value": reps * frac / dt, "unit": "layer-steps/s", "cores": threads, "kind": "oracle",
           "sample": sample + f"; threads available {orc.max_threads()}",
           "keys_scored_per_s": keys / dt, "cpu_model": cpu_model()}
    if cfg.form == "latent" and cfg.T == 1:
        # the same oracle on one thread, over the first two sequences
        n1 = min(2, cfg.B)
        c1 = S.make_case(cfg, seqs=list(range(n1)), latent_form=latent_form)
        all_threads = orc.max_threads()
        orc.set_threads(1)
        try:
            reps1, t1 = 0, time.perf_counter()
            while True:
                orc.layer_step_latent(c1["q_i"], c1["q_scale"], c1["w"], c1["k_i"], c1["k_scale"],
                                      c1["lens"], cfg.sm_scale_i, cfg.k, c1["q"], c1["latent"], cfg.Dv,
                                      cfg.sm_scale)
                reps1 += 1
                d1 = time.perf_counter() - t1
                if d1 >= min_seconds / 2:
                    break
        finally:
            orc.set_threads(all_threads)
        res["single_thread"] = {"value": reps1 * (n1 / cfg.B) / d1, "unit": "layer-steps/s",
                                "sample": f"{n1} of {cfg.B} sequences, {reps1} repetitions in "
                                          f"{d1:.1f} s on one thread, scaled by {cfg.B}/{n1}"}
    return res


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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


# input sets cycled per workload: enough distinct sets that the bytes one step touches
# (cache streams and gathered rows) exceed the 256 MB Infinity Cache before a set repeats
DEFAULT_SETS = {"tiny": 2, "decode_v32": 4, "decode_long": 2, "decode_ragged": 2,
                "prefill_chunk": 1, "prefill_chunk_latent": 1}


def measure(D, S, cfg, steps: int, warmup: int, sets: int, latent: str, graph: bool = False,
            with_prep: bool = True, ramp_s: float = RAMP_S) -> dict:
    """Time `steps` layer steps of one workload (inputs resident on the GPU, `sets` input
    sets cycled), then the same steps again with per-kernel HIP events, and return the
    figures of one JSON object."""
    import torch
    fp8_lat = latent == "fp8"
    lens = S.lengths(cfg)
    costs = algorithmic_costs(cfg, lens, latent)
    step_objs = []
    t_gen = time.perf_counter()
    for i in range(sets):
        c = S.make_case(dataclasses.replace(cfg, seed=cfg.seed + 1000 * i) if i else cfg,
                        latent_form=latent)
        d = S.to_device(c, "cuda")
        del c
        if cfg.form == "latent":
            step = D.LayerStep(d["q_i"], d["q_scale"], d["w"], d["k_i"], d["k_scale"], d["lens"],
                               cfg.sm_scale_i, cfg.k, d["q"], cfg.sm_scale, latent=d["latent"],
                               Dv=cfg.Dv)
        else:
            step = D.LayerStep(d["q_i"], d["q_scale"], d["w"], d["k_i"], d["k_scale"], d["lens"],
                               cfg.sm_scale_i, cfg.k, d["q"], cfg.sm_scale, k=d["k"], v=d["v"])
        step_objs.append(step)
    torch.cuda.synchronize()
    print(f"[bench] {cfg.name}: {sets} input sets on the GPU in "
          f"{time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    def timed(run_list):
        for i in range(warmup):
            run_list[i % len(run_list)]()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            run_list[i % len(run_list)]()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    # The GPU idles while the inputs are generated on the host, and its clocks take several
    # milliseconds of load to come back: the first windows after such a pause measured 5-15 %
    # slower than the steady state.  So the steps run untimed for ramp_s seconds first (a
    # handful of warm-up steps alone lasts a fraction of a millisecond).
    t_ramp = time.perf_counter()
    n_ramp = 0
    while time.perf_counter() - t_ramp < ramp_s:
        step_objs[n_ramp % len(step_objs)]()
        n_ramp += 1
        if n_ramp % 32 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    # eager launches (one C call per step, the library enqueueing each kernel) and the same
    # steps replayed from one HIP graph per input set (the launch sequence captured once)
    eager = list(step_objs)
    dt_eager = timed(eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for s_ in step_objs:
            s_()                                      # warm the launch path before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for s_ in step_objs:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            s_()
        graphs.append(g)
    replay = [g.replay for g in graphs]
    dt_graph = timed(replay)
    run, dt = (replay, dt_graph) if graph else (eager, dt_eager)
    ms_per_step = 1e3 * dt / steps
    value = steps / dt

    # per-step distribution: HIP events around every step (the library enqueues on the
    # current stream, which is where torch records its events)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record()
        run[i % len(run)]()
        evs[i][1].record()
    torch.cuda.synchronize()
    step_ms = sorted(a.elapsed_time(b) for a, b in evs)
    pct = lambda q: step_ms[min(len(step_ms) - 1, int(q * len(step_ms)))]

    # the same steps again, every kernel launched with a start/stop event pair recorded
    # by its own dispatch: kernel execution times without the gaps between kernels
    D.profile_begin(steps)
    for i in range(steps):
        step_objs[i % len(step_objs)]()
    prof = D.profile_end()
    torch.cuda.synchronize()
    phase_ms = {k: (v[0] / steps if v[1] else None) for k, v in prof.items()}
    att_launch_ms = prof["attention"][0] / prof["attention"][1]
    idx_launch_ms = prof["index_scores"][0] / prof["index_scores"][1]
    kernels_ms = sum(v for v in phase_ms.values() if v is not None)
    print(f"[bench] {cfg.name}: kernel time per step (ms): {phase_ms}", file=sys.stderr, flush=True)

    att_gbs = costs["attention_bytes"] / (att_launch_ms * 1e-3) / 1e9
    att_tfs = costs["attention_flops"] / (att_launch_ms * 1e-3) / 1e12
    idx_gbs = costs["index_bytes"] / (idx_launch_ms * 1e-3) / 1e9
    idx_tfs = costs["index_flops"] / (idx_launch_ms * 1e-3) / 1e12
    workload = cfg.name + ("-fp8" if fp8_lat else "")
    if cfg.form == "latent":
        tkey = "sparse_mla_decode"
        if latent_32x32_kernel(cfg, fp8_lat):
            kernel, src = (("mla_decode32_fp8_kernel", ATTN_FP8_SOURCE) if fp8_lat
                           else ("mla_decode32_kernel", ATTN_SOURCE))
        else:
            kernel, src = "mla_decode_mfma_kernel", ATTN_GENERIC_SOURCE
        if cfg.H not in (64, 128) or cfg.Dv != 512:
            kernel, src = "sparse_attn_generic_kernel", ATTN_GENERIC_SOURCE
    else:
        kernel, tkey, src = "mha_prefill_mfma_kernel", "sparse_mha_prefill", PREFILL_SOURCE
    traffic = read_traffic(tkey, workload, src)
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
    roofline.update({"traffic": traffic, "kernel": kernel, "avg_launch_ms": round(att_launch_ms, 5),
                     "timing": "HIP start/stop events recorded by each launch's dispatch "
                               "(hipExtLaunchKernel), averaged over the profiled steps"})
    # the same kernel's average in the committed rocprofv3 summary (per-dispatch timestamps
    # under the profiler), and the fraction it gives
    rp_ms = read_rocprof_avg_ms(kernel, workload, src)
    if rp_ms is not None:
        per_s = (costs["attention_flops"] / (BF16_PEAK_TFLOPS * 1e12) if mfma_bound
                 else costs["attention_bytes"] / (HBM_PEAK_GBS * 1e9))
        roofline.update({"rocprof_avg_launch_ms": round(rp_ms, 5),
                         "frac_at_rocprof_avg": round(per_s / (rp_ms * 1e-3), 4)})
    idx_rp_ms = read_rocprof_avg_ms(("index_scores_kernel", "index_scores_decode_kernel"),
                                    workload, INDEX_SOURCE)
    # the step's floor: each phase at the larger of its HBM time and its matrix-core time at
    # the peak of its own data type (the indexer's FP8 products, the attention's bf16)
    t_roof = (max(costs["index_bytes"] / (HBM_PEAK_GBS * 1e9), costs["index_flops"] / (FP8_PEAK_TFLOPS * 1e12)) +
              max(costs["attention_bytes"] / (HBM_PEAK_GBS * 1e9),
                  costs["attention_flops"] / (BF16_PEAK_TFLOPS * 1e12)))
    if cfg.form == "latent":
        attn_desc = (f"MLA {cfg.H} heads over FP8 latent rows (656 B: {cfg.Dv} e4m3fn + 4 "
                     f"block scales + {cfg.Dr} bf16 rope)" if fp8_lat else
                     f"MLA {cfg.H} heads over {cfg.attn_dtype} latent {cfg.Dv}+{cfg.Dr}")
    else:
        attn_desc = f"MHA {cfg.H} heads, bf16 qk {cfg.Dqk} / v {cfg.Dv}"
    out = {
        "value": round(value, 2),
        "unit": "layer-steps/s",
        "steps": steps,
        "warmup": warmup,
        "gpu_ramp_s": ramp_s,
        "ms_per_step": round(ms_per_step, 5),
        "eager_ms_per_step": round(1e3 * dt_eager / steps, 5),
        "graph_ms_per_step": round(1e3 * dt_graph / steps, 5),
        "dtype": cfg.attn_dtype,
        "config": {"workload": f"{cfg.name}: B={cfg.B}, context {cfg.Lmax} per sequence"
                               f"{' (' + cfg.lens + ')' if cfg.lens != 'full' else ''}, T={cfg.T}, "
                               f"indexer {cfg.H_I}x{cfg.D_I} FP8, top-{cfg.k}, {attn_desc}",
                   "B": cfg.B, "context": cfg.Lmax, "T": cfg.T, "topk": cfg.k, "H_I": cfg.H_I,
                   "d_I": cfg.D_I, "H": cfg.H, "q_width": cfg.Dq, "input_sets": sets,
                   "latent_cache": latent if cfg.form == "latent" else None,
                   "hip_graph": bool(graph)},
        "step_ms_p10_p50_p90": [round(pct(0.1), 5), round(pct(0.5), 5), round(pct(0.9), 5)],
        "token_layer_steps_per_s": round(cfg.B * cfg.T * value, 1),
        "keys_scored_per_s": round(costs["keys"] * value, 1),
        "keys_per_step": costs["keys"],
        "step_roofline_frac": round(t_roof / (ms_per_step * 1e-3), 4),
        "kernel_ms_per_step": {k: (round(v, 5) if v is not None else None) for k, v in phase_ms.items()},
        "gaps_ms_per_step": round(ms_per_step - kernels_ms, 5),
        "index_scores": {"avg_launch_ms": round(idx_launch_ms, 5),
                         "algorithmic_bytes_per_launch": costs["index_bytes"],
                         "achieved_GBs": round(idx_gbs, 1), "hbm_frac": round(idx_gbs / HBM_PEAK_GBS, 4),
                         "achieved_TFLOPs": round(idx_tfs, 1),
                         "mfma_frac_of_bf16_peak": round(idx_tfs / BF16_PEAK_TFLOPS, 4),
                         "mfma_frac_of_fp8_peak": round(idx_tfs / FP8_PEAK_TFLOPS, 4),
                         "keys_per_s": round(costs["keys"] / (idx_launch_ms * 1e-3), 1),
                         "traffic": read_traffic("index_scores", workload, INDEX_SOURCE),
                         "rocprof_avg_launch_ms": (round(idx_rp_ms, 5) if idx_rp_ms else None)},
        "roofline": roofline,
    }
    if with_prep:
        out["indexer_prep"] = measure_prep(D, S, cfg, steps)
        print(f"[bench] {cfg.name}: indexer prep {out['indexer_prep']}", file=sys.stderr, flush=True)
    del step_objs, run
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--ramp-seconds", type=float, default=RAMP_S,
                    help="untimed steps before the warm-up, to bring the GPU clocks out of idle")
    ap.add_argument("--config", default="decode_v32", help="the headline workload")
    ap.add_argument("--only", action="store_true", help="measure the headline workload only")
    ap.add_argument("--sets", type=int, default=0,
                    help="independent input sets cycled (0: the workload's default)")
    ap.add_argument("--latent", choices=["bf16", "fp8"], default="bf16",
                    help="latent cache rows: bf16 (1152 B) or the FP8 storage form (656 B: "
                         "512 e4m3fn codes, four fp32 block scales, 64 bf16 rope values)")
    ap.add_argument("--graph", action="store_true",
                    help="headline from the steps replayed from HIP graphs (default: eager calls; "
                         "both are measured and reported)")
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
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
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
    if args.latent == "fp8" and cfg.form != "latent":
        print("--latent fp8 applies to the latent (decode) workloads only", file=sys.stderr)
        sys.exit(2)
    sets = args.sets or DEFAULT_SETS.get(cfg.name, 4)
    head = measure(D, S, cfg, args.steps, args.warmup, sets, args.latent, graph=args.graph,
                   ramp_s=args.ramp_seconds)
    result = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
    }
    result.update({k: v for k, v in head.items() if k not in ("value", "unit", "steps", "warmup",
                                                               "ms_per_step", "dtype")})
    result["cpu_baseline"] = None if args.no_cpu else cpu_baseline(cfg, args.cpu_seqs, args.cpu_seconds,
                                                                  args.latent)
    if not args.only:
        others = {}
        for name in S.CONFIGS:
            if name == cfg.name:
                continue
            ocfg = S.CONFIGS[name]
            lat = args.latent if ocfg.form == "latent" and ocfg.attn_dtype == "bf16" else "bf16"
            steps = min(args.steps, 50) if ocfg.T == 1 else min(args.steps, 10)
            warm = min(args.warmup, 5)
            others[name] = measure(D, S, ocfg, steps, warm, DEFAULT_SETS.get(name, 2), lat,
                                   graph=args.graph, with_prep=False, ramp_s=args.ramp_seconds)
        result["other_workloads"] = others
    print(json.dumps(result))


if __name__ == "__main__":
    main()
