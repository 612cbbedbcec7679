#!/usr/bin/env python3
"""Benchmark of the paged-KV e4m3 decode path on one MI355X.

A step is one pass of the whole hot path over one synthetic batch:
pkv_paged_decode_attn (+ pkv_merge_splits when the plan split a sequence),
launched through the C ABI on torch's current stream. The plan is made once
(host planner) before timing, as a serving loop would. Steps rotate over
several independent KV pools (>= 1 GiB in total) so that no step finds its
cache in the 256 MB last-level cache.

Per workload: W untimed warmup steps; K eager steps with HIP events on the
launch stream around every decode and merge launch (the kernel durations and
the roofline); the same steps as HIP graph replays (one graph per pool),
first exactly K of them between two synchronisations (mean step), then
max(K, 100) back-to-back replays timed in blocks of 10 (one event between
blocks; the median over the blocks of block time / 10 is the reported step
time).

Default run (no --config): the headline workload is the fully-fp8 varlen
decode (128 sequences, q_len 1, 64 e4m3 query heads on 4 e4m3 KV heads,
d 128, 128-key pages, 90% of lengths in [1k, 4k] and 10% in [32k, 64k]);
the other workloads -- the tiny two-sequence decode, the vLLM-shaped GQA
batch, the speculative-verify batch with the causal tail and in block mode,
and the latent-record decode at 1, 2, 4, 8 and 16 query tokens -- are
measured in the same run and reported as sub-records. The streaming-read
probe (pkv_stream_read_probe) gives the achievable HBM read rate of the same
session, and the fp64 CPU oracle is timed on a bounded sample of the headline
batch over the host cores.

Printed (one JSON line on stdout): value = KV bytes per step / median step
time (GB/s, the metric), the step time, the decode kernel's roofline against
the 8 TB/s HBM peak and against the probe, the sub-records, and the CPU
baseline. Diagnostics go to stderr.

``--config 1..10`` measures one workload alone (1-5 as above; 6, 7, 8 and 10
are the fully-fp8 batch with packed fp4 (e2m1), fp6 e2m3, fp6 e3m2 and NVFP4
K/V; 9 is the sparse slot-list decode step).
"""

import argparse
import dataclasses
import json
import os
import shutil
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}  # dense
STEP_BLOCK = 10  # graph replays per timed block of the median step
MEDIAN_MIN_STEPS = 100  # >= 10 blocks of STEP_BLOCK replays
HEADLINE = 4
# sub-records of the default run: (label, workload index, overrides)
SUB_WORKLOADS = [
    ("tiny", 1, {}),
    ("gqa", 2, {}),
    ("specverify_causal", 3, {}),
    ("specverify_block", 3, {"causal": False}),
    ("latent_q1", 5, {}),
    ("latent_q2", 5, {"q_len": 2}),
    ("latent_q4", 5, {"q_len": 4}),
    ("latent_q8", 5, {"q_len": 8}),
    ("latent_q16", 5, {"q_len": 16}),
]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(batch, dec):
    """Bytes the decode kernel must move once: every visible K and V row, the
    query rows, the block-table entries, and its outputs (final bf16 O + LSE
    for unsplit sequences, fp32 partial O + (max, sum) for split ones)."""
    import numpy as np

    w = batch.spec
    lens = batch.seq_lens.cpu().numpy().astype(np.int64)
    ns = dec.n_splits.cpu().numpy().astype(np.int64)
    q_elem = 1 if w.q_format == "e4m3" else 2
    kv = batch.kv_bytes
    q = w.num_seqs * w.q_len * w.h_q * w.d_qk * q_elem
    bt = int((-(-lens // w.page_size)).sum()) * 4 * w.h_k
    rows = w.num_seqs * w.h_k * w.rows
    direct = ns <= 1
    out_direct = int(direct.sum()) * w.h_k * w.rows * (w.d_v * 2 + 4)
    out_split = int(ns[~direct].sum()) * w.h_k * w.rows * (w.d_v + 2) * 4
    # MFMA work: every (row, visible key) pair costs 2*d_qk (QK^T) + 2*d_v (PV) flops
    vis = 0
    for L in lens:
        qi = np.arange(w.q_len)
        lim = (L - w.q_len + qi) if (w.causal and w.q_len > 1) else np.full(w.q_len, L - 1)
        vis += int(np.clip(lim + 1, 0, None).sum()) * w.h_q
    flops = vis * (2 * w.d_qk + 2 * w.d_v)
    return dict(kv=kv, q=q, block_table=bt, out=out_direct + out_split, rows=rows, flops=flops,
                total=kv + q + bt + out_direct + out_split)


def profile_key(w, default_q_len):
    """Name of a workload in the committed counter summaries: the workload's
    name, with the query length when it is not the workload's own, and the
    mode when it is block attention."""
    key = w.name if w.q_len == default_q_len else f"{w.name}_q{w.q_len}"
    return key if w.causal or w.q_len == 1 else f"{key}_block"


def measured_traffic(kernel, key):
    """HBM bytes per decode launch from the committed counter summary of this
    kernel and workload, or None if there is none or the kernel source changed
    since it was taken."""
    import hashlib

    source = "decode_mla.hip" if kernel.startswith(("mla_", "sparse_")) else "decode_gqa.hip"
    path = os.path.join(ROOT, "profiles", f"{kernel.replace('_kernel', '')}_{key}_hbm_bytes.md")
    src = os.path.join(ROOT, "paged_kv_fp8_amd", "csrc", source)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            k, _, v = line.strip().partition(":")
            fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != hashlib.sha256(open(src, "rb").read()).hexdigest():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle over (sequence, kv head) units on a pool of
# host processes (one BLAS thread each). The pool is forked before the GPU is
# touched; the batch reaches the workers as memory-mapped .npy files.
# ---------------------------------------------------------------------------
_ARRAYS = {}


def _cpu_worker_init():
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover
        pass


def _arrays(files):
    import numpy as np

    for key, path in files.items():
        if _ARRAYS.get(key, (None,))[0] != path:
            _ARRAYS[key] = (path, None if path is None else np.load(path, mmap_mode="r"))
    return {k: v[1] for k, v in _ARRAYS.items() if k in files}


def _oracle_unit(task):
    """One (sequence, kv head) unit of the oracle; returns its KV bytes."""
    from oracle.attention import decode_attention, mla_decode_attention

    files, spec, b, g = task
    nb = _arrays(files)
    q_len, h_k, h_r = spec["q_len"], spec["h_k"], spec["h_r"]
    L = int(nb["seq_lens"][b])
    tok = slice(b * q_len, (b + 1) * q_len)
    if spec["kv_format"] == "mla":
        mla_decode_attention(nb["q"][tok], nb["latent"], nb["rope"], nb["scales"], nb["block_table"][b:b + 1],
                             nb["seq_lens"][b:b + 1], q_len=q_len, softmax_scale=spec["scale"], causal=spec["causal"])
        return L * 656
    heads = slice(g * h_r, (g + 1) * h_r)
    one = slice(g, g + 1)
    ks = None if nb.get("k_scale") is None else nb["k_scale"][:, :, one]
    vs = None if nb.get("v_scale") is None else nb["v_scale"][:, :, one]
    decode_attention(nb["q"][tok, heads], nb["k_cache"][:, :, one], nb["v_cache"][:, :, one],
                     nb["block_table"][b:b + 1], nb["seq_lens"][b:b + 1], nb["q_descale"][b:b + 1, one],
                     nb["k_descale"][b:b + 1, one], nb["v_descale"][b:b + 1, one], q_len=q_len, h_k=1,
                     softmax_scale=spec["scale"], causal=spec["causal"], kv_format=spec["kv_format"], k_scale=ks,
                     v_scale=vs)
    row = nb["k_cache"].shape[-1] + nb["v_cache"].shape[-1]  # stored bytes per token and head
    if ks is not None:
        row += ks.shape[-1] + vs.shape[-1]
    return L * row


def cpu_pool_size():
    """Host processes for the CPU baseline: the cores this process may run
    on, at most 16 (one GPU's share of the host)."""
    return max(1, min(len(os.sched_getaffinity(0)), 16))


def make_cpu_pool():
    """Forked before any GPU call, so the workers never inherit GPU state."""
    import multiprocessing as mp

    n = cpu_pool_size()
    return mp.get_context("fork").Pool(n, initializer=_cpu_worker_init), n


def cpu_oracle_baseline(pool, n_procs, batch, budget_s):
    """Time the fp64 oracle on (sequence, kv head) units of the batch, in
    order and cycling over the batch, on ``n_procs`` processes until
    ``budget_s`` seconds of wall time are spent; GB/s of KV bytes."""
    import numpy as np

    w = batch.spec
    nb = batch.to_numpy()
    base = "/dev/shm" if os.access("/dev/shm", os.W_OK) else None
    tmp = tempfile.mkdtemp(prefix="pkv_bench_", dir=base)
    try:
        files = {}
        for key, arr in nb.items():
            if arr is None:
                files[key] = None
                continue
            files[key] = os.path.join(tmp, key + ".npy")
            np.save(files[key], np.ascontiguousarray(arr))
        spec = dict(q_len=w.q_len, h_k=w.h_k, h_r=w.h_r, kv_format=w.kv_format, scale=w.scale, causal=w.causal)
        heads = 1 if w.kv_format == "mla" else w.h_k
        units = [(b, g) for b in range(w.num_seqs) for g in range(heads)]
        # every worker maps the arrays once before the clock starts
        pool.map(_arrays, [files] * (4 * n_procs), chunksize=1)
        pending, done, kv = [], 0, 0
        i = 0
        t0 = time.perf_counter()
        while True:
            while len(pending) < 2 * n_procs and time.perf_counter() - t0 < budget_s:
                b, g = units[i % len(units)]
                pending.append(pool.apply_async(_oracle_unit, ((files, spec, b, g),)))
                i += 1
            if not pending:
                break
            kv += pending.pop(0).get()
            done += 1
        dt = time.perf_counter() - t0
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    unit = "sequence" if heads == 1 else "(sequence, kv head)"
    return {"value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": n_procs, "kind": "oracle",
            "sample": f"{done} {unit} units of the {w.name} batch in order, cycling ({len(units)} units per pass; "
                      f"{kv} KV bytes, all rows), in {dt:.1f} s wall on {n_procs} processes, numpy fp64, "
                      f"one BLAS thread each"}


# ---------------------------------------------------------------------------
# GPU measurements
# ---------------------------------------------------------------------------
def stream_probe(args):
    """Achievable HBM read rate of this session: the streaming-read probe over
    a 2 GiB buffer (8x the last-level cache), a sweep of launch shapes, the
    best median of several launches."""
    import numpy as np
    import torch

    from paged_kv_fp8_amd import native

    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(0x5A)
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(cu * 64, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    best = None
    sweep = []
    for wg_per_cu in (4, 8, 16, 32):
        for unroll in (4, 8, 16):
            wgs = cu * wg_per_cu
            for _ in range(2):
                native.stream_read_probe(buf.data_ptr(), nbytes, wgs, unroll, sink.data_ptr(), stream)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
            for e0, e1 in ev:
                e0.record()
                native.stream_read_probe(buf.data_ptr(), nbytes, wgs, unroll, sink.data_ptr(), stream)
                e1.record()
            torch.cuda.synchronize()
            us = float(np.median([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]))
            gbs = nbytes / us / 1e3
            sweep.append({"workgroups_per_cu": wg_per_cu, "unroll": unroll, "us": round(us, 1),
                          "GB_per_s": round(gbs, 1)})
            if best is None or gbs > best["GB_per_s"]:
                best = sweep[-1]
    del buf
    log(f"streaming-read probe: best {best['GB_per_s']:.0f} GB/s ({best['workgroups_per_cu']} workgroups/CU, "
        f"unroll {best['unroll']}) over {nbytes >> 20} MiB")
    return {"kernel": "stream_read_kernel", "bytes": nbytes, "best": best, "sweep": sweep}


def replay_steps_us(graphs, n, stream):
    """Step times (us) from n back-to-back graph replays (cycling over
    ``graphs``) timed in blocks of STEP_BLOCK: one event between consecutive
    blocks, each block's time / STEP_BLOCK is one sample. An event between
    every two replays would add its own few microseconds to every step (the
    marker waits for the replay before it); here it adds that once per block."""
    import torch

    blocks = -(-n // STEP_BLOCK)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(blocks + 1)]
    ev[0].record(stream)
    i = 0
    for b in range(blocks):
        for _ in range(STEP_BLOCK):
            graphs[i % len(graphs)].replay()
            i += 1
        ev[b + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[b].elapsed_time(ev[b + 1]) * 1e3 / STEP_BLOCK for b in range(blocks)]


def measure_decode(w, args, label=None, plan_kw=None):
    """Build the batch (and its rotated pools), plan once, and time eager
    launches and graph-replayed steps. Returns the per-workload record."""
    import numpy as np
    import torch

    from paged_kv_fp8_amd import decode
    from paged_kv_fp8_amd.workloads import make_batch

    plan_kw = dict(plan_kw or {})
    first = make_batch(w, device="cuda")
    pools = args.pools or min(64, max(3, -(-(1 << 30) // max(1, first.kv_bytes))))
    lens = first.seq_lens.cpu().numpy()
    batches = [first] + [make_batch(dataclasses.replace(w, seed=w.seed + 1000 * i), device="cuda", seq_lens=lens)
                         for i in range(1, pools)]
    decs = [decode.for_batch(b, **plan_kw) for b in batches]
    info = decs[0].plan_info
    ab = algorithmic_bytes(first, decs[0])
    log(f"workload {label or w.name}: {w.num_seqs} seqs, q_len {w.q_len}, causal {w.causal}, "
        f"{int(lens.sum())} tokens, KV {ab['kv'] / 1e6:.1f} MB, pools {pools}, plan chunk={info.chunk_tiles} tiles "
        f"work={info.num_real} slots={info.slots} max_splits_used={info.max_n_splits} wg/cu={decs[0].wg_per_cu} "
        f"cu={decs[0].cu_count}")
    K, W = args.steps, args.warmup
    stream = torch.cuda.current_stream()

    for i in range(W):
        decs[i % pools].run()
    torch.cuda.synchronize()
    # eager launches, events around every decode and merge launch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(K):
        d = decs[i % pools]
        ev[i][0].record()
        d.run_decode_only()
        ev[i][1].record()
        d.run_merge_only()
        ev[i][2].record()
    end.record()
    torch.cuda.synchronize()
    eager_us_step = start.elapsed_time(end) * 1e3 / K
    dec_us = [e[0].elapsed_time(e[1]) * 1e3 for e in ev]
    # a plan that split no sequence launches no merge: the two events with
    # nothing between them would time only their own gap
    mrg_us = [e[1].elapsed_time(e[2]) * 1e3 for e in ev] if decs[0].has_splits else [0.0] * K
    # the decode kernel's duration: K decode launches back to back (pools
    # rotated) between two events, so no launch gap is counted (an event pair
    # around each launch adds the gap in front of it)
    torch.cuda.synchronize()
    start.record()
    for i in range(K):
        decs[i % pools].run_decode_only()
    end.record()
    torch.cuda.synchronize()
    b2b_us = start.elapsed_time(end) * 1e3 / K

    # graph replays: one graph per pool holding its decode + merge launches
    graphs = []
    for d in decs:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            d.run()
        graphs.append(g)
    for i in range(W):
        graphs[i % pools].replay()
    torch.cuda.synchronize()
    # exactly K steps between two synchronisations: the mean step
    t0 = time.perf_counter()
    start.record()
    for i in range(K):
        graphs[i % pools].replay()
    end.record()
    torch.cuda.synchronize()
    wall_us = (time.perf_counter() - t0) * 1e6 / K
    graph_mean_us = start.elapsed_time(end) * 1e3 / K
    # max(K, 100) back-to-back replays in blocks of 10: the median block step
    n_med = max(K, MEDIAN_MIN_STEPS)
    step_us = replay_steps_us(graphs, n_med, stream)
    step_med = float(np.median(step_us))

    dtype = "fp8" if w.q_format == "e4m3" else "bf16"
    kernel_us = b2b_us
    t_hbm = ab["total"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = ab["flops"] / (MFMA_PEAK_TFLOPS[dtype] * 1e12)
    achieved = ab["total"] / (kernel_us * 1e-6) / 1e9
    tflops = ab["flops"] / (kernel_us * 1e-6) / 1e12
    kernel = decs[0].kernel_name
    if t_mfma > t_hbm:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_PEAK_TFLOPS[dtype], "unit": "TFLOP/s",
                "frac": round(tflops / MFMA_PEAK_TFLOPS[dtype], 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof.update({"kernel": kernel, "kernel_us": round(kernel_us, 2),
                 "kernel_us_per_launch_events": round(float(np.mean(dec_us)), 2),
                 "kernel_us_median": round(float(np.median(dec_us)), 2),
                 "algorithmic_bytes_per_launch": ab["total"], "algorithmic_flops_per_launch": ab["flops"],
                 "hbm_frac": round(achieved / HBM_PEAK_GBS, 4),
                 "roofline_us": round(max(t_hbm, t_mfma) * 1e6, 2)})
    kv_gbs = ab["kv"] / (step_med * 1e-6) / 1e9
    log(f"  step {step_med:.1f} us (median over blocks of {STEP_BLOCK} of {n_med} graph replays; mean of {K}: "
        f"{graph_mean_us:.1f} us, host wall {wall_us:.1f} us; eager {eager_us_step:.1f} us); decode {kernel_us:.1f} us, merge "
        f"{float(np.mean(mrg_us)):.1f} us; KV {kv_gbs:.0f} GB/s per step; {kernel} {achieved:.0f} GB/s = "
        f"{achieved / HBM_PEAK_GBS:.3f} of HBM peak, {tflops:.1f} TFLOP/s = {tflops / MFMA_PEAK_TFLOPS[dtype]:.3f} of "
        f"{dtype} MFMA peak; roofline {roof['bound']} {max(t_hbm, t_mfma) * 1e6:.1f} us")
    rec = {
        "label": label or w.name, "workload": w.name, "q_len": w.q_len, "causal": w.causal, "dtype": dtype,
        "us_per_step": round(step_med, 2), "us_per_step_mean": round(graph_mean_us, 2),
        "us_per_step_eager": round(eager_us_step, 2), "median_of": n_med,
        "kv_bytes": ab["kv"], "kv_GB_per_s": round(kv_gbs, 2),
        "merge_us": round(float(np.mean(mrg_us)), 2),
        "roofline": roof,
        "plan": {"kind": decs[0].plan, "imbalance": decs[0].imbalance and round(decs[0].imbalance, 3),
                 "chunk_tiles": info.chunk_tiles, "work_items": info.num_real,
                 "slots": info.slots, "max_n_splits": info.max_n_splits, "wg_per_cu": decs[0].wg_per_cu,
                 "max_splits": w.max_splits, "bins": info.num_bins},
        "pools": pools, "kv_tokens": int(lens.sum()),
    }
    del graphs, decs, batches
    torch.cuda.empty_cache()
    return rec, first


def decode_line(w, rec, base_q_len, probe, cpu, K, W, as_profiled):
    """The JSON line of a decode workload record."""
    roof = dict(rec["roofline"])
    if roof["bound"] == "hbm":
        roof["traffic"] = measured_traffic(roof["kernel"], profile_key(w, base_q_len)) if as_profiled else None
        if probe:
            roof["achievable"] = probe["best"]["GB_per_s"]
            roof["frac_of_achievable"] = round(roof["achieved"] / probe["best"]["GB_per_s"], 4)
    else:
        roof["traffic"] = None
    cfg = {"workload": w.name, "num_seqs": w.num_seqs, "q_len": w.q_len, "h_q": w.h_q, "h_k": w.h_k,
           "d": w.d_qk, "page_size": w.page_size, "causal": w.causal, "kv_format": w.kv_format,
           "q_format": w.q_format, "kv_layout": w.kv_layout, "contiguous_pages": w.contiguous_pages,
           "kv_tokens": rec["kv_tokens"], "kv_bytes": rec["kv_bytes"], "max_splits": w.max_splits,
           "pools": rec["pools"], "plan": rec["plan"]}
    return {
        "metric": "achieved HBM GB/s (KV bytes / decode-step time), us per decode step",
        "value": rec["kv_GB_per_s"], "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(rec["us_per_step"] / 1e3, 5), "us_per_step": rec["us_per_step"],
        "step_stat": f"median over {rec['median_of'] // STEP_BLOCK} blocks of {STEP_BLOCK} back-to-back graph-replayed "
                     f"steps ({rec['median_of']} steps)",
        "ms_per_step_mean": round(rec["us_per_step_mean"] / 1e3, 5), "us_per_step_eager": rec["us_per_step_eager"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": rec["dtype"],
        "data": "synthetic", "config": cfg, "roofline": roof, "merge_us": rec["merge_us"],
        "streaming_probe": probe, "cpu_baseline": cpu,
    }


def sub_record(rec, probe):
    r = rec["roofline"]
    out = {"label": rec["label"], "workload": rec["workload"], "q_len": rec["q_len"], "causal": rec["causal"],
           "kernel": r["kernel"], "kernel_us": r["kernel_us"], "merge_us": rec["merge_us"],
           "step_us": rec["us_per_step"], "step_us_mean": rec["us_per_step_mean"], "kv_GB_per_s": rec["kv_GB_per_s"],
           "bound": r["bound"], "frac": r["frac"], "hbm_frac": r["hbm_frac"], "roofline_us": r["roofline_us"]}
    if probe and r["bound"] == "hbm":
        out["frac_of_achievable"] = round(r["achieved"] / probe["best"]["GB_per_s"], 4)
    return out


def bench_headline(args, pool):
    """The default run: the headline workload's line with every other decode
    workload as a sub-record, the probe and the CPU baseline."""
    from paged_kv_fp8_amd.workloads import workload

    probe = stream_probe(args)
    subs = []
    for label, idx, over in SUB_WORKLOADS:
        try:
            rec, _ = measure_decode(workload(idx, **over), args, label=label)
            subs.append(sub_record(rec, probe))
        except Exception as e:  # a failing sub-workload is reported, not fatal to the headline
            log(f"sub-workload {label} failed: {e!r}")
            subs.append({"label": label, "error": repr(e)})
    w = workload(HEADLINE)
    rec, batch = measure_decode(w, args, label="headline")
    cpu = None
    if pool is not None:
        cpu = cpu_oracle_baseline(pool[0], pool[1], batch, args.cpu_seconds)
        log(f"cpu oracle: {cpu}")
    line = decode_line(w, rec, w.q_len, probe, cpu, args.steps, args.warmup, as_profiled=not args.pools)
    line["sub_records"] = subs
    print(json.dumps(line), flush=True)


def sparse_cpu_baseline(batch, budget_s):
    """The sparse oracle on whole tokens of the batch until the budget is
    spent; GB/s of listed record bytes."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle.sparse import sparse_decode_attention

    nb = batch.to_numpy()
    done, kv = 0, 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for i in range(1 << 30):  # whole passes over the tokens until the budget is spent
            t = i % batch.spec.num_tokens
            srcs = [dict(s, slots=s["slots"][t:t + 1]) for s in nb["sources"]]
            sparse_decode_attention(nb["q"][t:t + 1], srcs, softmax_scale=batch.spec.scale, sink=nb["sink"])
            kv += sum(int((s["slots"] >= 0).sum()) for s in srcs) * 656
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
    return {"value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} tokens in order, cycling over the {batch.spec.num_tokens} of the step ({kv} record "
                      f"bytes, all heads) in {dt:.1f} s, numpy fp64, one BLAS thread"}


def bench_sparse(args):
    """The sparse slot-list decode step: tile kernel + merge per step, pools
    rotated so that the records come from HBM."""
    import numpy as np
    import torch

    from paged_kv_fp8_amd import sparse
    from paged_kv_fp8_amd.workloads import make_sparse_batch, sparse_workload

    w = sparse_workload(9)
    torch.cuda.set_device(0)
    first = make_sparse_batch(w, device="cuda")
    pool_bytes = sum(b.numel() for b in first.kv_buffers)
    pools = args.pools or min(64, max(3, -(-(1 << 30) // max(1, pool_bytes))))
    batches = [first] + [make_sparse_batch(dataclasses.replace(w, seed=w.seed + 1000 * i), device="cuda",
                                           seq_lens=first.seq_lens) for i in range(1, pools)]
    decs = [sparse.for_batch(b) for b in batches]
    T = w.num_tokens
    listed = sum(int((s["slots"] >= 0).sum().item()) for s in first.sources)
    kv = listed * 656
    widths = [s["slots"].shape[1] for s in first.sources]
    tiles = decs[0].tiles
    alg = {"kv": kv, "q": T * w.h_q * 576 * 2, "lists": T * sum(widths) * 4,
           "partials": tiles * T * w.h_q * (512 + 2) * 4}
    alg["total"] = sum(alg.values())
    flops = listed * w.h_q * (2 * 576 + 2 * 512)
    log(f"workload {w.name}: {T} tokens, {listed} listed records ({kv / 1e6:.2f} MB), tiles/token {tiles}, "
        f"pools {pools} ({pool_bytes / 1e6:.0f} MB each)")
    for i in range(args.warmup):
        decs[i % pools].run()
    torch.cuda.synchronize()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(K):
        d = decs[i % pools]
        ev[i][0].record()
        d.run_tiles_only()
        ev[i][1].record()
        d.run_merge_only()
        ev[i][2].record()
    end.record()
    torch.cuda.synchronize()
    eager_ms_step = start.elapsed_time(end) / K
    tile_events_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    mrg_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    # the tile kernel's duration: K launches back to back between two events
    torch.cuda.synchronize()
    start.record()
    for i in range(K):
        decs[i % pools].run_tiles_only()
    end.record()
    torch.cuda.synchronize()
    tile_ms = start.elapsed_time(end) / K
    graphs = []
    for d in decs:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            d.run()
        graphs.append(g)
    for i in range(args.warmup):
        graphs[i % pools].replay()
    torch.cuda.synchronize()
    gstart, gend = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gstart.record()
    for i in range(K):
        graphs[i % pools].replay()
    gend.record()
    torch.cuda.synchronize()
    graph_ms_step = gstart.elapsed_time(gend) / K
    n_med = max(K, MEDIAN_MIN_STEPS)
    ms_step = float(np.median(replay_steps_us(graphs, n_med, torch.cuda.current_stream()))) / 1e3
    value = kv / (ms_step * 1e-3) / 1e9
    achieved = alg["total"] / (tile_ms * 1e-3) / 1e9
    t_hbm = alg["total"] / (HBM_PEAK_GBS * 1e9)
    log(f"step {ms_step * 1e3:.1f} us median (tiles {tile_ms * 1e3:.1f} us, merge {mrg_ms * 1e3:.1f} us; graph mean "
        f"{graph_ms_step * 1e3:.1f}, eager {eager_ms_step * 1e3:.1f}); records {value:.0f} GB/s; tile kernel "
        f"{achieved:.0f} GB/s = {achieved / HBM_PEAK_GBS:.3f} of peak; roofline time {t_hbm * 1e6:.2f} us (hbm)")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = sparse_cpu_baseline(first, args.cpu_seconds)
        log(f"cpu oracle: {cpu}")
    kernel = "sparse_pair_kernel"
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(kernel, w.name) if not args.pools else None,
                "kernel": kernel, "kernel_us": round(tile_ms * 1e3, 2),
                "kernel_us_per_launch_events": round(tile_events_ms * 1e3, 2), "algorithmic_bytes_per_launch": alg["total"],
                "algorithmic_flops_per_launch": flops, "merge_us": round(mrg_ms * 1e3, 2)}
    line = {
        "metric": "achieved HBM GB/s (listed record bytes / decode-step time), us per decode step",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "us_per_step": round(ms_step * 1e3, 2),
        "step_stat": f"median over {n_med // STEP_BLOCK} blocks of {STEP_BLOCK} back-to-back graph-replayed steps",
        "ms_per_step_mean": round(graph_ms_step, 5),
        "us_per_step_eager": round(eager_ms_step * 1e3, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "num_tokens": T, "q_len": 1, "h_q": w.h_q, "window": w.window,
                   "topk": w.topk, "compress_ratio": w.compress_ratio, "page_size": list(w.page_size),
                   "sink": w.sink, "listed_records": listed, "kv_bytes": kv, "tiles_per_token": tiles,
                   "pools": pools},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_producers(steps):
    """Time the producers on the workloads' per-step shapes and on a
    prefill-sized write: us per call (HIP events on the launch stream) and
    algorithmic bytes / time."""
    import torch

    from paged_kv_fp8_amd import producers

    dev = "cuda"
    g = torch.Generator(device=dev).manual_seed(4242)
    cases = []

    def timed(name, fn, nbytes, shape):
        # `steps` calls captured in one graph and replayed, so the host's launch
        # cost does not sit between the kernels
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(steps):
                fn()
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        cases.append({"case": name, "shape": shape, "us_per_call": round(us, 2), "bytes": nbytes,
                      "GB_per_s": round(nbytes / us / 1e3, 1), "frac_of_hbm_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)})
        log(f"{name}: {us:.2f} us, {nbytes / us / 1e3:.0f} GB/s")

    for name, (b, t, hq, hk, d) in {"quantize_q, fully-fp8 decode step": (128, 1, 64, 4, 128),
                                    "quantize_q, speculative verify step": (32, 4, 64, 8, 128),
                                    "quantize_q, 512 sequences x 8 tokens": (512, 8, 64, 8, 128)}.items():
        q = torch.randn(b * t, hq, d, device=dev, generator=g).to(torch.bfloat16)
        q8 = torch.empty(q.shape, dtype=torch.uint8, device=dev)
        qd = torch.empty(b, hk, dtype=torch.float32, device=dev)
        nbytes = q.numel() * 2 * 2 + q.numel() + qd.numel() * 4  # q read twice (amax, codes), codes written
        timed(name, lambda: producers.quantize_q(q, b, t, hk, q8=q8, q_descale=qd), nbytes,
              {"num_seqs": b, "q_len": t, "h_q": hq, "h_k": hk, "d": d})

    for name, (b, n, hk, ps) in {"write_kv e4m3, decode step (64 x 1 token)": (64, 1, 8, 16),
                                 "write_kv e4m3, prefill (32 x 1024 tokens)": (32, 1024, 8, 16)}.items():
        d = 128
        blocks = (n + 2048) // ps + 1
        pages = b * blocks
        kc = torch.zeros(pages, ps, hk, d, dtype=torch.uint8, device=dev)
        vc = torch.zeros_like(kc)
        bt = torch.randperm(pages, device=dev, generator=g).to(torch.int32).view(b, blocks)
        lens = torch.full((b,), 2048 + n, dtype=torch.int32, device=dev)
        kn = torch.randn(b * n, hk, d, device=dev, generator=g).to(torch.bfloat16)
        vn = torch.randn(b * n, hk, d, device=dev, generator=g).to(torch.bfloat16)
        kd = torch.full((b, hk), 0.01, device=dev)
        nbytes = 2 * kn.numel() * 2 + 2 * kn.numel() + b * n * 4
        timed(name, lambda: producers.write_kv(kn, vn, bt, lens, n, kc, vc, kd, kd), nbytes,
              {"num_seqs": b, "n_new": n, "h_k": hk, "d": d, "page_size": ps})

    for name, (b, n, ps) in {"write_kv latent, decode step (32 x 1 token)": (32, 1, 64),
                             "write_kv latent, prefill (32 x 1024 tokens)": (32, 1024, 64)}.items():
        blocks = (n + 2048) // ps + 1
        pages = b * blocks
        lat = torch.zeros(pages, ps, 512, dtype=torch.uint8, device=dev)
        rope = torch.zeros(pages, ps, 64, dtype=torch.int16, device=dev)
        scl = torch.zeros(pages, ps, 4, dtype=torch.float32, device=dev)
        bt = torch.randperm(pages, device=dev, generator=g).to(torch.int32).view(b, blocks)
        lens = torch.full((b,), 2048 + n, dtype=torch.int32, device=dev)
        x = torch.randn(b * n, 576, device=dev, generator=g).to(torch.bfloat16)
        nbytes = b * n * (576 * 2 + 656 + 4)
        timed(name, lambda: producers.write_latent(x, bt, lens, n, lat, rope, scl), nbytes,
              {"num_seqs": b, "n_new": n, "page_size": ps})
    print(json.dumps({"metric": "producer kernels: us per call and algorithmic GB/s", "n_gpus": 1, "steps": steps,
                      "data": "synthetic", "cases": cases}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=None, choices=[1, 2, 3, 4, 5, 6, 7, 8, 9, 10],
                    help="one workload alone: 1-5 as specified; 6, 7, 8, 10 = workload 4 with packed fp4 (e2m1), "
                         "fp6 e2m3, fp6 e3m2, NVFP4 K/V; 9 = the sparse slot-list decode step (16 tokens, 16 heads, "
                         "128-slot window + 512 top-k slots). Default: the headline run (workload 4 with every "
                         "other decode workload as a sub-record)")
    ap.add_argument("--q-len", type=int, default=None, help="query tokens per sequence (latent workload: 1..16)")
    ap.add_argument("--causal", type=int, default=None, help="override the workload's causal flag (0/1)")
    ap.add_argument("--pools", type=int, default=0, help="KV pools to rotate (0: enough for >= 1 GiB, min 3)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="wall-time budget of the CPU oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="single-workload runs: skip the streaming-read probe")
    ap.add_argument("--wg-per-cu", type=int, default=None, help="override the occupancy the planner uses")
    ap.add_argument("--kv-layout", default=None, choices=["nhd", "hnd"],
                    help="physical cache layout (default nhd: [pages][page_size][h_k][d])")
    ap.add_argument("--max-splits", type=int, default=None, help="override the workload's split cap")
    ap.add_argument("--page-size", type=int, default=None, help="override the workload's page size")
    ap.add_argument("--contiguous-pages", action="store_true", help="hand out pages in order instead of shuffled")
    ap.add_argument("--seq-len", type=int, default=None, help="give every sequence this length")
    ap.add_argument("--plan", default="auto", choices=["auto", "wave", "even", "balanced", "queued", "paired"],
                    help="auto: wave, or balanced when pkv_plan_pick finds the wave plan's items imbalanced; "
                         "wave: one work item per workgroup (occupancy-pinned split plan); even: the same rule with "
                         "equal 32-key-block pieces per sequence; balanced: contiguous "
                         "equal shares of all keys, one per workgroup; queued: persistent workgroups, packed "
                         "static bins then a shared queue")
    ap.add_argument("--dyn-percent", type=int, default=10, help="queued plan: share of the work left to the queue")
    ap.add_argument("--pieces-per-bin", type=int, default=3, help="queued plan: pieces a bin's share is cut into")
    ap.add_argument("--producers", action="store_true",
                    help="only time the query quantisation and KV-cache write kernels (a separate JSON line)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 8 plain 256 MiB device-to-device copies (scale reference for HBM byte counters)")
    ap.add_argument("--probe-only", action="store_true", help="only run the streaming-read probe sweep")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode path has no multi-GPU leg (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    special = args.producers or args.copy_calibration or args.probe_only or args.config == 9
    # the CPU baseline's worker processes are forked now, before any GPU call
    pool = make_cpu_pool() if not (args.no_cpu_baseline or special) else None
    try:
        run(args, pool)
    finally:
        if pool is not None:
            pool[0].terminate()
            pool[0].join()


def run(args, pool):
    import torch

    torch.cuda.set_device(0)
    if args.producers:
        bench_producers(args.steps)
        return
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied 8 x 256 MiB")
        return
    if args.probe_only:
        print(json.dumps({"metric": "streaming-read probe GB/s", "n_gpus": 1, **stream_probe(args)}), flush=True)
        return
    if args.config == 9:
        return bench_sparse(args)
    if args.config is None:
        return bench_headline(args, pool)

    from paged_kv_fp8_amd.workloads import workload

    over = {} if args.causal is None else {"causal": bool(args.causal)}
    if args.q_len:
        over["q_len"] = args.q_len
    if args.kv_layout:
        over["kv_layout"] = args.kv_layout
    if args.max_splits:
        over["max_splits"] = args.max_splits
    if args.page_size:
        over["page_size"] = args.page_size
    if args.contiguous_pages:
        over["contiguous_pages"] = True
    if args.seq_len:
        over["seq_len_dist"] = ("fixed", [args.seq_len] * workload(args.config).num_seqs)
    base = workload(args.config)
    w = workload(args.config, **over)
    # counter summaries are taken on the workloads as defined (query length and mode aside)
    as_profiled = (set(over) <= {"q_len", "causal"} and not args.pools and args.wg_per_cu is None
                   and args.plan == "auto")
    plan_kw = {"wg_per_cu": args.wg_per_cu, "plan": args.plan}
    if args.plan == "queued":
        plan_kw.update(dyn_percent=args.dyn_percent, pieces_per_bin=args.pieces_per_bin)
    probe = None if args.no_probe else stream_probe(args)
    rec, batch = measure_decode(w, args, plan_kw=plan_kw)
    cpu = None
    if pool is not None:
        cpu = cpu_oracle_baseline(pool[0], pool[1], batch, args.cpu_seconds)
        log(f"cpu oracle: {cpu}")
    print(json.dumps(decode_line(w, rec, base.q_len, probe, cpu, args.steps, args.warmup, as_profiled)), flush=True)


if __name__ == "__main__":
    main()
