#!/usr/bin/env python3
"""Throughput of the tensor-parallel layer-shard hot path on one MI355X.

One step = one whole pass of the path on one batch of seeded synthetic input:
layer forward (LN, QKV, attention, output projection, all-reduce stand-in, LN,
fc1+GeLU, fc2, all-reduce stand-in), vocabulary-parallel cross-entropy
forward and backward, layer backward (both blocks, both phases, and the
backward all-reduce stand-ins). Inputs are resident in HBM before timing.

Prints ONE JSON line. `value` = algorithmic flops of one rank's layer shard
forward + backward (3 x the forward's contraction flops, causal attention
over visible query-key pairs only) / the median over the timed steps of the
time spent in that rank's own layer calls (both blocks' forward, both
backward phases of both blocks; event pairs around each call). The all-reduce
stand-ins (which on t GPUs are RCCL all-reduces over xGMI) and the loss are
timed and reported beside it, not in it. The default workload is the 175B
rank (the largest single-GPU workload); the other bf16 workloads are measured
in the same run and reported under `workloads`.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
       python bench.py --copy-calibration     (plain copy for PMC byte scaling)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}   # MI355X dense MFMA (AMD data sheet)
PEAK_HBM_GBS = 8000.0                           # MI355X HBM3E
MFMA_KERNELS = {"gemm_nt", "gemm_nn", "gemm_tn", "gemm_pair", "attn_fwd", "attn_bwd_dq", "attn_bwd_dkdv",
                "attn_bwd_pair"}
METRIC = "TFLOP/s per TP layer-shard fwd+bwd (bf16) and % of MI355X MFMA peak"


def step_flops(cfg, n_ranks: int) -> dict:
    """Algorithmic flops of one pass over `n_ranks` ranks of the TP group."""
    t = cfg.tp
    n, h = cfg.rows, cfg.hidden
    hr, fr, vr = h // t, cfg.ffn // t, cfg.vocab // t
    a_r, d, s, b = cfg.heads // t, cfg.head_dim, cfg.seq, cfg.micro_batch
    pairs = s * (s + 1) // 2 if cfg.causal else s * s
    fwd = 2 * n * h * 3 * hr + 4 * b * a_r * pairs * d + 2 * n * hr * h + 4 * n * h * fr
    rows = n if cfg.mask_rows is None else cfg.mask_rows
    layer = 3 * fwd * n_ranks
    xent = 6 * rows * vr * h * n_ranks
    return {"layer": layer, "xent": xent, "total": layer + xent}


def build_step(cfg):
    import synth
    from tensor_transformer_layer_03_amd.step import LayerStep
    ranks = cfg.ranks()
    rep = synth.replicated_inputs(cfg)
    shards = {r: synth.device_shard(cfg, synth.rank_shard(cfg, r)) for r in ranks}
    n_peers = cfg.tp - len(ranks)
    peers = synth.peer_partials(cfg, n_peers) if n_peers else []
    pstats = [synth.peer_stats(cfg, r) for r in range(cfg.tp) if r not in ranks]
    return LayerStep(cfg, rep, shards, peers, pstats), ranks


def time_loop(fn, steps, torch):
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def quantiles(xs):
    t = sorted(xs)
    q = lambda f: t[min(len(t) - 1, int(round(f * (len(t) - 1))))]
    return {"p10": round(q(0.1), 4), "median": round(q(0.5), 4), "p90": round(q(0.9), 4)}


class CallTimer:
    """LayerStep hook: an event pair on the current stream around every
    library call of a pass, labelled with the call's kind ("layer", "sum",
    "loss") and the step index."""

    def __init__(self, torch):
        self.torch = torch
        self.step = 0
        self.recs = []

    def __call__(self, kind, thunk):
        E = self.torch.cuda.Event
        a, b = E(enable_timing=True), E(enable_timing=True)
        a.record()
        r = thunk()
        b.record()
        self.recs.append((self.step, kind, a, b))
        return r

    def per_step(self, steps):
        """{kind: [ms of that kind's calls in step i for i < steps]} (after a sync)."""
        out = {}
        for i, kind, a, b in self.recs:
            out.setdefault(kind, [0.0] * steps)[i] += a.elapsed_time(b)
        return out


def measure(st, steps, warmup, torch):
    """Warm-up, then `steps` timed passes between two synchronisations. Each
    pass is bracketed by an event pair and each library call inside it by its
    own (CallTimer). Returns the mean step time over the timed region and the
    per-step times of the whole pass and of each call kind."""
    for _ in range(warmup):
        st.step()
    E = torch.cuda.Event
    timer = CallTimer(torch)
    st.hook = timer
    pairs = [(E(enable_timing=True), E(enable_timing=True)) for _ in range(steps)]
    t0, t1 = E(enable_timing=True), E(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i, (a, b) in enumerate(pairs):
        timer.step = i
        a.record()
        st.step()
        b.record()
    t1.record()
    torch.cuda.synchronize()
    st.hook = None
    kinds = timer.per_step(steps)
    return {"mean_step_ms": t0.elapsed_time(t1) / steps, "step": [a.elapsed_time(b) for a, b in pairs],
            "layer": kinds.get("layer", [0.0] * steps), "sum": kinds.get("sum", [0.0] * steps),
            "loss": kinds.get("loss", [0.0] * steps)}


# A workload whose layer shard is under this many flops (the 8.3B rank's
# 357.6 GF) runs about a millisecond a step, so its record times at least
# SHORT_STEPS passes to keep the median's spread small.
SHORT_LAYER_GFLOP = 400.0
SHORT_STEPS = 50


def sub_record_steps(cfg, steps: int) -> int:
    """Timed passes for a workload's record: `steps`, or SHORT_STEPS for short ones."""
    return max(steps, SHORT_STEPS) if step_flops(cfg, len(cfg.ranks()))["layer"] / 1e9 < SHORT_LAYER_GFLOP else steps


def summary(cfg, n_ranks, m, peak):
    """Throughput figures of one workload from measure()'s per-step times."""
    fl = step_flops(cfg, n_ranks)
    lq, sq, xq, tq = (quantiles(m[k]) for k in ("layer", "sum", "loss", "step"))
    tf = lambda f, ms: round(f / (ms / 1e3) / 1e12, 2)
    return {
        "layer_shard": {"tflops": tf(fl["layer"], lq["median"]),
                        "pct_of_mfma_peak": round(100 * fl["layer"] / (lq["median"] / 1e3) / 1e12 / peak, 2),
                        "ms": lq, "gflop": round(fl["layer"] / 1e9, 1),
                        "note": "the rank's own layer calls (fwd ATTN, fwd MLP, bwd MLP shard + replicated, "
                                "bwd ATTN shard + replicated), median over steps"},
        "standin_sums": {"ms": sq, "calls_per_step": 5,
                         "note": "shard_partial_sum, the all-reduce stand-in (4 per layer + the loss gradient's)"},
        "loss": {"tflops": tf(fl["xent"], xq["median"]), "ms": xq, "gflop": round(fl["xent"] / 1e9, 1),
                 "note": "vocabulary-parallel cross-entropy forward (local + finish) and backward"},
        "step": {"tflops": tf(fl["total"], tq["median"]), "ms": tq,
                 "note": "whole pass: layer, loss and the stand-in sums"},
    }


def traced_kernels(st, steps, B, dtype):
    """Per-kernel event timing of `steps` passes: {name: (launches, ms, work)}."""
    import torch
    B.tpl_trace_enable(4096)
    for _ in range(steps):
        st.step()
    torch.cuda.synchronize()
    recs = B.tpl_trace_read(4096)
    B.tpl_trace_enable(0)
    agg = {}
    for name, ms, work in recs:
        c, t, w = agg.get(name, (0, 0.0, 0.0))
        agg[name] = (c + 1, t + ms, w + work)
    return agg


def roofline(agg, dtype, workload):
    if not agg:   # no traced steps (--trace-steps 0)
        return None
    name, (count, ms, work) = max(agg.items(), key=lambda kv: kv[1][1])
    traffic = measured_traffic(name, workload)
    if name in MFMA_KERNELS:
        achieved = work / (ms / 1e3) / 1e12
        peak = PEAK_TFLOPS[dtype]
        return {"kernel": name, "bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                "launches": count, "avg_launch_us": round(ms / count * 1e3, 2),
                "flops_per_launch": work / count}
    achieved = work / (ms / 1e3) / 1e9
    return {"kernel": name, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic, "launches": count,
            "avg_launch_us": round(ms / count * 1e3, 2), "bytes_per_launch": work / count}


def cpu_baseline(cfg, seqs: int, seq_len: int, repeats: int = 3) -> dict:
    """The oracle, as it stands, on a bounded sample of the same workload:
    `seqs` sequences of `seq_len` tokens (the workload's layer, loss and
    rank split at a shorter length; every flop of that sample), median of
    `repeats` runs."""
    import dataclasses
    import oracle as O
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: report the affinity mask
        threads = len(os.sched_getaffinity(0))
    seqs = max(1, min(seqs, cfg.micro_batch))
    seq_len = max(1, min(seq_len, cfg.seq))
    rows = seqs * seq_len
    small = dataclasses.replace(cfg, micro_batch=seqs, seq=seq_len,
                                mask_rows=None if cfg.mask_rows is None else max(1, cfg.mask_rows * rows // cfg.rows))
    ranks = small.ranks()
    rep = synth.replicated_inputs(small)
    shards = {r: synth.rank_shard(small, r) for r in ranks}
    n_peers = small.tp - len(ranks)
    peers = synth.peer_partials(small, n_peers) if n_peers else []
    pstats = [synth.peer_stats(small, r) for r in range(small.tp) if r not in ranks]
    prs = {r: synth.oracle_params(small, [s], rep) for r, s in shards.items()}
    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        O.step_reference(prs, rep.x, rep.dout, rep.targets, rep.mask, seq=small.seq, causal=small.causal,
                         eps=small.ln_eps, tp=small.tp, vocab_r=small.vocab_r, peers=peers, peer_stats=pstats,
                         use_mask=small.mask_rows is not None)
        times.append(time.perf_counter() - t0)
    dt = sorted(times)[len(times) // 2]
    fl = step_flops(small, len(ranks))["total"]
    return {"value": round(fl / dt / 1e12, 4), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"oracle pass (numpy fp64: layer shard fwd+bwd and the loss) over {seqs} of "
                      f"{cfg.micro_batch} sequences at {seq_len} of {cfg.seq} tokens, median of {repeats} runs "
                      f"({fl / 1e9:.0f} GFLOP in {dt:.1f} s each)"}


def copy_calibration(torch, mib=1024, reps=5):
    """A plain device copy of known size, to scale PMC FETCH_SIZE/WRITE_SIZE."""
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": n * 4, "reps": reps}))


# ---------------------------------------------------------------- profile summaries

SOURCES = {"gemm": "gemm.hip", "attn": "attention.hip", "layernorm": "norm.hip", "colsum": "norm.hip",
           "partial": "norm.hip", "xent": "xent.hip", "embedding": "embedding.hip"}
PROFILE_CMDS = {
    "trace": "cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <out>/prof_c2 -o c2 -- "
             "python3 <repo>/bench.py --config <workload> --steps 5 --warmup 2 --cpu-seqs 0 --no-layer-only",
    "pmc": "cd /tmp && rocprofv3 --pmc <FETCH_SIZE|WRITE_SIZE> --output-format csv -d <out>/pmc_<counter> -o bench "
           "-- python3 <repo>/bench.py --config <workload> --steps 2 --warmup 1 --cpu-seqs 0 --trace-steps 1 "
           "--no-layer-only",
    "copy": "cd /tmp && rocprofv3 --pmc <FETCH_SIZE|WRITE_SIZE> --output-format csv -d <out>/pmc_<counter> -o copy "
            "-- python3 <repo>/bench.py --copy-calibration",
    "mfma": "cd /tmp && rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES --output-format csv -d <out>/pmc_mfma "
            "-o bench -- python3 <repo>/bench.py --config <workload> --steps 2 --warmup 1 --cpu-seqs 0 "
            "--trace-steps 1 --no-layer-only",
}


def kernel_family(name: str) -> str:
    """Map a rocprofv3 kernel name (mangled or demangled) to the trace names."""
    import re
    if "gemm_pair" in name:           # an activation- and a weight-gradient product in one launch
        return "gemm_pair"
    if "gemm" in name:
        m = re.search(r"gemm_\w*kernel<([^>]*)>", name)
        if m:
            flags = [t.strip() == "true" for t in m.group(1).split(",") if t.strip() in ("true", "false")]
        else:
            flags = [f == "1" for f in re.findall(r"Lb([01])E", name)]
        ak, bk = (flags + [True, True])[:2]
        return "gemm_nt" if ak and bk else ("gemm_nn" if ak else "gemm_tn")
    if "splitk_sum" in name:          # the split-K sum is part of the weight-gradient product's launch
        return "gemm_tn"
    if "splitk_reduce" in name:       # split-order sum of a split product: fp32 out = wgrad, bf16 out = dgrad
        return "gemm_tn" if ("IfE" in name or "<float>" in name) else "gemm_nn"
    if "colpart" in name:             # LN-gradient (3 outputs) or bias-gradient (1 output) column partials
        if "Li3E" in name or ", 3>" in name:
            return "layernorm_bwd_cols"
        if "Li1E" in name or ", 1>" in name:
            return "colsum"
        return "colpart"
    table = [("attn_bwd_pair", "attn_bwd_pair"), ("attn_bwd_dkdv", "attn_bwd_dkdv"), ("attn_bwd_dq", "attn_bwd_dq"),
             ("attn_bwd_pre", "attn_bwd_pre"),
             ("attn_fwd", "attn_fwd"), ("ln_bwd_cols", "layernorm_bwd_cols"), ("ln_bwd", "layernorm_bwd"),
             ("ln_fwd", "layernorm_fwd"), ("colsum_final", "colsum_final"), ("colsum", "colsum"),
             ("partial_sum", "partial_sum"), ("xent_stats", "xent_stats"), ("xent_finish", "xent_finish"),
             ("xent_dlogits", "xent_dlogits"), ("xent_merge", "xent_merge"), ("embed_fwd", "embedding_fwd"),
             ("embed_grad", "embedding_bwd"), ("embed_keys", "embedding_sort"), ("radix_sort", "embedding_sort"),
             ("embed_sort", "embedding_sort"),
             ("embed_segments", "embedding_sort")]
    for key, fam in table:
        if key in name:
            return fam
    return "other"


def attached(name: str) -> bool:
    """Dispatches that belong to a launch of their family counted once (the
    split-K sums, and the K-split tail pass that precedes a weight-gradient
    product's whole rounds): their time and bytes count, their dispatch does
    not count as a launch."""
    return "splitk_sum" in name or "splitk_reduce" in name or "tail_kernel" in name


def source_sha(family: str) -> str:
    import hashlib
    for prefix, f in SOURCES.items():
        if family.startswith(prefix):
            path = os.path.join(ROOT, "tensor_transformer_layer_03_amd", "csrc", f)
            return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]
    return ""


def recompute_bench(st, steps, torch):
    """Layer backward with the forward stash kept vs rebuilt from the block
    inputs (activation recomputation): time of each and the per-layer stash
    the recomputing form no longer has to keep (one buffer serves all layers)."""
    st.recompute = False
    bwd_ms = time_loop(st.backward, steps, torch)
    st.recompute = True
    rec_ms = time_loop(st.backward, steps, torch)
    st.recompute = False
    stash = sum(t.tensors["saved_attn"].numel() + t.tensors["saved_mlp"].numel() for t in st.states)
    return {"bwd_ms": round(bwd_ms, 4), "bwd_recompute_ms": round(rec_ms, 4),
            "stash_bytes_per_layer": int(stash)}


def embedding_bench(cfg, steps, torch, B):
    """The vocabulary-parallel input embedding on this rank's share of the
    workload (a row beside the layer step, not part of the headline): forward
    lookup and scatter-add gradient, each timed over `steps` calls."""
    import synth
    desc = B.make_desc(cfg.hidden, cfg.heads, cfg.head_dim, cfg.ffn, cfg.tp, 0, cfg.seq, cfg.micro_batch, cfg.vocab,
                       cfg.causal, cfg.dtype)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    es = 2 if cfg.dtype == "bf16" else 4
    tok = torch.from_numpy(synth.input_tokens(cfg)).cuda()
    emb = torch.randn(cfg.vocab_r, cfg.hidden, device="cuda").to(dt)
    dout = torch.randn(cfg.rows, cfg.hidden, device="cuda").to(dt)
    part = torch.empty(cfg.rows, cfg.hidden, device="cuda", dtype=dt)
    grad = torch.empty(cfg.vocab_r, cfg.hidden, device="cuda", dtype=torch.float32)
    ws = torch.empty(B.vocab_parallel_embedding_ws_bytes(desc), device="cuda", dtype=torch.uint8)
    fwd = lambda: B.vocab_parallel_embedding_fwd(desc, tok, emb, part)
    bwd = lambda: B.vocab_parallel_embedding_bwd(desc, tok, dout, grad, ws)
    for _ in range(3):
        fwd()
        bwd()
    f_ms = time_loop(fwd, steps, torch)
    b_ms = time_loop(bwd, steps, torch)
    n, h, vr = cfg.rows, cfg.hidden, cfg.vocab_r
    f_bytes = 2 * n * h * es + 4 * n                 # rows read (ids in range) + partial written + ids
    b_bytes = n * h * es + vr * h * 4 + 4 * n        # gradient rows read once + fp32 table written + ids
    return {"workload": f"{cfg.name}: ids {n}, rank rows V_r {vr} x h {h}, uniform ids",
            "fwd_us": round(f_ms * 1e3, 2), "fwd_gbs": round(f_bytes / (f_ms / 1e3) / 1e9, 1),
            "bwd_us": round(b_ms * 1e3, 2), "bwd_gbs": round(b_bytes / (b_ms / 1e3) / 1e9, 1),
            "bound": "hbm", "peak_gbs": 8000.0}


DEFAULT_WORKLOAD = "gpt_175b_t8"
BF16_WORKLOADS = ["gpt2_355m_t1", "gpt_8p3b_t8", "bert_3p9b_t4", "gpt_175b_t8"]


def profile_cmd(kind: str, workload: str) -> str:
    """A command of PROFILE_CMDS for a workload."""
    return PROFILE_CMDS[kind].replace("<workload>", workload)


def trace_cmd(workload: str) -> str:
    """The kernel-trace command of PROFILE_CMDS for a workload."""
    return profile_cmd("trace", workload)


def summarize_profiles(d: str, workload: str, trace_only: bool = False):
    import csv
    import collections
    prof = os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    # kernel trace statistics
    rows = list(csv.DictReader(open(os.path.join(d, "prof_c2", "c2_kernel_stats.csv"))))
    fam = collections.defaultdict(lambda: [0, 0.0])
    for r in rows:
        f = kernel_family(r["Name"])
        fam[f][0] += 0 if attached(r["Name"]) else int(r["Calls"])
        fam[f][1] += float(r["TotalDurationNs"])
    total = sum(v[1] for v in fam.values())
    lines = [f"# Kernel time, {workload} (rocprofv3 --kernel-trace --stats)", "",
             "Command (repo root = <repo>, output dir = <out>):", "", "    " + trace_cmd(workload), "",
             "Every launch of the run (warm-up, timed and traced steps); all are whole passes, so the mix per",
             "kernel family is the same as in one step. A weight-gradient product's split-K sum is counted",
             "in its launch (gemm_tn), as the library's own launch timing does.", "",
             "| family | launches | total ms | avg us | share |", "|---|---|---|---|---|"]
    for f, (c, t) in sorted(fam.items(), key=lambda kv: -kv[1][1]):
        lines.append(f"| {f} | {c} | {t / 1e6:.3f} | {t / c / 1e3:.1f} | {100 * t / total:.1f}% |")
    lines += ["", "Per instantiation (top 16):", "", "| kernel | calls | avg us | total ms |", "|---|---|---|---|"]
    for r in rows[:16]:
        lines.append(f"| {r['Name'][:110]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.3f} |")
    open(os.path.join(prof, f"kernel_stats_{workload}.md"), "w").write("\n".join(lines) + "\n")
    if trace_only:
        return
    # HBM bytes: FETCH_SIZE / WRITE_SIZE per dispatch, scaled by a plain copy of known size
    copy_bytes = 1024 * (1 << 20)
    per = {}
    scale = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        cp = [float(r["Counter_Value"]) for r in csv.DictReader(open(os.path.join(d, f"pmc_{c}", "copy_counter_collection.csv")))
              if "copyBuffer" in r["Kernel_Name"]]
        scale[c] = copy_bytes / (sorted(cp)[len(cp) // 2] * 1024)
        tot = collections.defaultdict(float)
        cnt = collections.defaultdict(int)
        for r in csv.DictReader(open(os.path.join(d, f"pmc_{c}", "bench_counter_collection.csv"))):
            f = kernel_family(r["Kernel_Name"])
            tot[f] += float(r["Counter_Value"]) * 1024 * scale[c]
            cnt[f] += 0 if attached(r["Kernel_Name"]) else 1
        per[c] = {k: tot[k] / max(cnt[k], 1) for k in tot}
    traffic = {f: {"fetch_bytes_per_launch": per["FETCH_SIZE"].get(f, 0.0),
                   "write_bytes_per_launch": per["WRITE_SIZE"].get(f, 0.0),
                   "bytes_per_launch": per["FETCH_SIZE"].get(f, 0.0) + per["WRITE_SIZE"].get(f, 0.0),
                   "source_sha256": source_sha(f)} for f in per["FETCH_SIZE"]}
    path = os.path.join(prof, "hbm_traffic.json")
    try:
        doc = json.load(open(path))
        doc.setdefault("workloads", {})
    except (OSError, ValueError):
        doc = {"workloads": {}}
    doc["workloads"][workload] = {"scale": scale, "kernels": traffic}
    json.dump(doc, open(path, "w"), indent=1)
    lines = [f"# HBM bytes per launch, {workload} (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)", "",
             "Commands:", "", "    " + profile_cmd("pmc", workload), "    " + PROFILE_CMDS["copy"], "",
             f"Calibration: a {copy_bytes >> 20} MiB device copy reads and writes {copy_bytes >> 20} MiB; the counters "
             f"read FETCH x{1 / scale['FETCH_SIZE']:.3f}, WRITE x{1 / scale['WRITE_SIZE']:.3f} of that, so bench "
             f"bytes are scaled by {scale['FETCH_SIZE']:.3f} (fetch) and {scale['WRITE_SIZE']:.3f} (write).", "",
             "The counters see the L2's requests to the memory side: a fetch served by the 256 MB "
             "last-level cache (MALL) counts like one from HBM, so fetch figures above a kernel's "
             "algorithmic reads are L2 misses (operand panels re-read by other XCDs or after "
             "eviction), not necessarily HBM transfers.", "",
             "| family | fetch MB/launch | write MB/launch | kernel source sha256 |", "|---|---|---|---|"]
    for f, v in sorted(traffic.items(), key=lambda kv: -kv[1]["bytes_per_launch"]):
        lines.append(f"| {f} | {v['fetch_bytes_per_launch'] / 1e6:.1f} | {v['write_bytes_per_launch'] / 1e6:.1f} | "
                     f"{v['source_sha256']} |")
    open(os.path.join(prof, f"hbm_traffic_{workload}.md"), "w").write("\n".join(lines) + "\n")
    mfma_dir = os.path.join(d, "pmc_mfma")
    if os.path.isdir(mfma_dir):
        busy = collections.defaultdict(lambda: [0.0, 0.0])
        for r in csv.DictReader(open(os.path.join(mfma_dir, "bench_counter_collection.csv"))):
            f = kernel_family(r["Kernel_Name"])
            busy[f][0 if r["Counter_Name"] == "SQ_VALU_MFMA_BUSY_CYCLES" else 1] += float(r["Counter_Value"])
        lines = [f"# MFMA busy share per kernel family, {workload} (rocprofv3 --pmc)", "",
                 "Command:", "", "    " + profile_cmd("mfma", workload), "",
                 "share = SQ_VALU_MFMA_BUSY_CYCLES / (4 x SQ_BUSY_CU_CYCLES), summed over the family's dispatches:",
                 "the fraction of SIMD cycles (4 SIMDs per CU) with the matrix unit busy while the CUs are busy.", "",
                 "| family | MFMA busy share |", "|---|---|"]
        for f, (mb, cu) in sorted(busy.items(), key=lambda kv: -kv[1][0]):
            if mb > 0:
                lines.append(f"| {f} | {mb / (4 * cu):.3f} |")
        open(os.path.join(prof, f"mfma_busy_{workload}.md"), "w").write("\n".join(lines) + "\n")
    print(f"wrote profiles for {workload}")


def measured_traffic(family: str, workload: str):
    """HBM bytes per launch of a kernel family on a workload from the committed
    counter summaries, or None if no counters were taken on that workload or
    the kernel's source changed since."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        rec = json.load(open(path))["workloads"][workload]["kernels"][family]
    except (OSError, KeyError, ValueError, TypeError):
        return None
    return rec["bytes_per_launch"] if rec.get("source_sha256") == source_sha(family) else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=DEFAULT_WORKLOAD)
    ap.add_argument("--trace-steps", type=int, default=3)
    ap.add_argument("--cpu-seqs", type=int, default=1,
                    help="sequences in the CPU-baseline sample (0 = skip)")
    ap.add_argument("--cpu-seq-len", type=int, default=512,
                    help="tokens per sequence in the CPU-baseline sample (at most the workload's)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-layer-only", dest="all_workloads", action="store_false",
                    help="time the chosen workload only (skip the other bf16 workloads' records)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write profiles/ summaries from rocprofv3 CSV output under DIR and exit")
    ap.add_argument("--trace-only", action="store_true",
                    help="with --summarize-profiles: the kernel-trace summary only (no counter passes)")
    args = ap.parse_args()

    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.config, args.trace_only)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only: the TP group's ranks are computed on one device and the "
              f"all-reduce is a local sum kernel; --gpus {args.gpus} (WORLD_SIZE={world}) is not supported.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X, gfx950)", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    import synth
    from tensor_transformer_layer_03_amd import binding as B

    cfg = synth.get_config(args.config)
    peak = PEAK_TFLOPS[cfg.dtype]
    st, ranks = build_step(cfg)
    fl = step_flops(cfg, len(ranks))
    m = measure(st, args.steps, args.warmup, torch)
    head = summary(cfg, len(ranks), m, peak)
    agg = traced_kernels(st, args.trace_steps, B, cfg.dtype)
    loss = float(st.shared["loss"][0].item())
    emb = embedding_bench(cfg, args.steps, torch, B)
    rec = recompute_bench(st, max(3, args.steps // 2), torch)
    del st
    torch.cuda.empty_cache()

    workloads = {}
    if args.all_workloads:
        for name in BF16_WORKLOADS:
            if name == cfg.name:
                workloads[name] = head
                continue
            c2 = synth.get_config(name)
            s2, r2 = build_step(c2)
            n2 = sub_record_steps(c2, args.steps)
            workloads[name] = summary(c2, len(r2), measure(s2, n2, args.warmup, torch), PEAK_TFLOPS[c2.dtype])
            workloads[name]["steps"] = n2
            del s2
            torch.cuda.empty_cache()

    value = head["layer_shard"]["tflops"]
    kernels = sorted(((k, c, t / args.trace_steps, w) for k, (c, t, w) in agg.items()), key=lambda r: -r[2])
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["mean_step_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded: activations N(0,1), weights N(0,sigma_w), uniform targets)",
        "config": {
            "workload": f"{cfg.name}: one transformer layer, hidden {cfg.hidden}, {cfg.heads} heads x "
                        f"{cfg.head_dim}, ffn {cfg.ffn}, TP t={cfg.tp} (ranks {ranks} on this GPU), "
                        f"seq {cfg.seq}, micro-batch {cfg.micro_batch}, vocab {cfg.vocab}, "
                        f"{'causal' if cfg.causal else 'bidirectional'}",
            "global_batch": cfg.micro_batch, "seq_len": cfg.seq, "parallelism": f"tp{cfg.tp} (one GPU)",
        },
        "pct_of_mfma_peak": head["layer_shard"]["pct_of_mfma_peak"],
        "value_definition": "layer-shard fwd+bwd flops / median time of the rank's own layer calls "
                            "(all-reduce stand-ins and the loss excluded; reported below)",
        "ms_per_step_definition": "mean time of a whole pass (layer, loss, stand-in sums) over the timed steps",
        "flops_per_step": fl,
        **head,
        "loss_value": round(loss, 6),
        "roofline": roofline(agg, cfg.dtype, cfg.name),
        "workloads": workloads,
        "embedding": emb,
        "recompute": rec,
        "kernels_per_step": [{"kernel": k, "launches": c // args.trace_steps, "ms": round(t, 4),
                              ("tflops" if k in MFMA_KERNELS else "gbs"):
                                  round(w / args.trace_steps / (t / 1e3) / (1e12 if k in MFMA_KERNELS else 1e9), 1)}
                             for k, c, t, w in kernels],
    }
    if args.cpu_seqs != 0:
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seqs, args.cpu_seq_len)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
