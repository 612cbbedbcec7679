#!/usr/bin/env python3
"""Benchmark of the paged-KV e4m3 decode path on one MI355X.

A step is one pass of the whole hot path over one synthetic batch:
pkv_paged_decode_attn (+ pkv_merge_splits when the plan split a sequence),
launched through the C ABI on torch's current stream. The plan is made once
(host planner) before timing, as a serving loop would. Steps rotate over
several independent KV pools (>= 1 GiB in total) so that no step finds its
cache in the 256 MB last-level cache. W untimed warmup steps, then exactly K
timed eager steps between two synchronisations, HIP events on the launch
stream timing every decode and merge launch; then (default) the same K steps
as HIP graph replays, one graph per pool, which give the reported step time.

Printed (one JSON line on stdout): value = KV bytes per step / time per step
(GB/s, the metric), the time per step, the decode kernel's roofline fraction
against the 8 TB/s HBM peak, and the fp64 CPU oracle timed on a bounded
sample of the same batch on the host cores. Diagnostics go to stderr.

Default workload: 64 sequences, q_len 1, 32 query heads on 8 e4m3 KV heads,
d = 128, 16-key pages, lengths uniform in [512, 8192], split-KV up to 16
chunks (``--config 2``). ``--config 1..5`` selects the other workloads; 6, 7
8 and 10 are workload 4 with packed fp4 (e2m1), fp6 e2m3, fp6 e3m2 and NVFP4 K/V; 9 is
the sparse slot-list decode step (its metric: listed record bytes per step
time).
"""

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}  # dense


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
    name, with the query length when it is not the workload's own."""
    return w.name if w.q_len == default_q_len else f"{w.name}_q{w.q_len}"


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


def cpu_oracle_baseline(batch, budget_s):
    """Time the fp64 oracle (single BLAS thread) on whole sequences of the
    batch until ``budget_s`` seconds of CPU work are spent."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle.attention import decode_attention, mla_decode_attention

    w = batch.spec
    nb = batch.to_numpy()
    lens = nb["seq_lens"]
    done, kv = 0, 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for i in range(1 << 30):  # whole passes over the batch until the budget is spent
            b = i % w.num_seqs
            sl = slice(b * w.q_len, (b + 1) * w.q_len)
            if w.kv_format == "mla":
                mla_decode_attention(nb["q"][sl], nb["latent"], nb["rope"], nb["scales"], nb["block_table"][b:b + 1],
                                     lens[b:b + 1], q_len=w.q_len, softmax_scale=w.scale, causal=w.causal)
                kv += int(lens[b]) * 656
            else:
                decode_attention(nb["q"][sl], nb["k_cache"], nb["v_cache"], nb["block_table"][b:b + 1],
                                 lens[b:b + 1], nb["q_descale"][b:b + 1], nb["k_descale"][b:b + 1],
                                 nb["v_descale"][b:b + 1], q_len=w.q_len, h_k=w.h_k, softmax_scale=w.scale,
                                 causal=w.causal, kv_format=w.kv_format, k_scale=nb.get("k_scale"),
                                 v_scale=nb.get("v_scale"))
                row_bytes = nb["k_cache"].shape[-1] + nb["v_cache"].shape[-1]  # stored bytes per token and head
                if "k_scale" in nb:
                    row_bytes += nb["k_scale"].shape[-1] + nb["v_scale"].shape[-1]
                kv += int(lens[b]) * w.h_k * row_bytes
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
    return {"value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} sequences in order, cycling over the {w.num_seqs} of the batch ({kv} KV bytes, all "
                      f"heads and rows) in {dt:.1f} s, numpy fp64, one BLAS thread"}


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
    tile_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    mrg_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
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
    ms_step = graph_ms_step if args.step_mode == "graph" else eager_ms_step
    value = kv / (ms_step * 1e-3) / 1e9
    achieved = alg["total"] / (tile_ms * 1e-3) / 1e9
    t_hbm = alg["total"] / (HBM_PEAK_GBS * 1e9)
    log(f"step {ms_step * 1e3:.1f} us (tiles {tile_ms * 1e3:.1f} us, merge {mrg_ms * 1e3:.1f} us; graph "
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
                "kernel": kernel, "kernel_us": round(tile_ms * 1e3, 2), "algorithmic_bytes_per_launch": alg["total"],
                "algorithmic_flops_per_launch": flops, "merge_us": round(mrg_ms * 1e3, 2)}
    line = {
        "metric": "achieved HBM GB/s (listed record bytes / decode-step time), us per decode step",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "us_per_step": round(ms_step * 1e3, 2), "step_mode": args.step_mode,
        "us_per_step_eager": round(eager_ms_step * 1e3, 2), "us_per_step_graph": round(graph_ms_step * 1e3, 2),
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
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5, 6, 7, 8, 9, 10],
                    help="workload: 1-5 as specified; 6, 7, 8, 10 = workload 4 with packed fp4 (e2m1), "
                         "fp6 e2m3, fp6 e3m2, NVFP4 K/V; 9 = the sparse slot-list decode step (16 tokens, 16 heads, "
                         "128-slot window + 512 top-k slots)")
    ap.add_argument("--q-len", type=int, default=None, help="query tokens per sequence (latent workload: 1..16)")
    ap.add_argument("--causal", type=int, default=None, help="override the workload's causal flag (0/1)")
    ap.add_argument("--pools", type=int, default=0, help="KV pools to rotate (0: enough for >= 1 GiB, min 3)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--wg-per-cu", type=int, default=None, help="override the occupancy the planner uses")
    ap.add_argument("--kv-layout", default=None, choices=["nhd", "hnd"],
                    help="physical cache layout (default nhd: [pages][page_size][h_k][d])")
    ap.add_argument("--max-splits", type=int, default=None, help="override the workload's split cap")
    ap.add_argument("--page-size", type=int, default=None, help="override the workload's page size")
    ap.add_argument("--contiguous-pages", action="store_true", help="hand out pages in order instead of shuffled")
    ap.add_argument("--seq-len", type=int, default=None, help="give every sequence this length")
    ap.add_argument("--plan", default="wave", choices=["wave", "even", "balanced", "queued"],
                    help="wave: one work item per workgroup (occupancy-pinned split plan); even: the same rule with "
                         "equal 32-key-block pieces per sequence; balanced: contiguous "
                         "equal shares of all keys, one per workgroup; queued: persistent workgroups, packed "
                         "static bins then a shared queue")
    ap.add_argument("--dyn-percent", type=int, default=10, help="queued plan: share of the work left to the queue")
    ap.add_argument("--pieces-per-bin", type=int, default=3, help="queued plan: pieces a bin's share is cut into")
    ap.add_argument("--fused-merge", action="store_true",
                    help="merge split sequences inside the decode kernel (last split merges) instead of a second launch")
    ap.add_argument("--step-mode", default="graph", choices=["graph", "eager"],
                    help="graph: the reported step time is K HIP graph replays of decode + merge (after an eager "
                         "pass that times each launch with events); eager: the eager pass is the step time")
    ap.add_argument("--producers", action="store_true",
                    help="only time the query quantisation and KV-cache write kernels (a separate JSON line)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 8 plain 256 MiB device-to-device copies (scale reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode path has no multi-GPU leg (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.producers:
        torch.cuda.set_device(0)
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

    if args.config == 9:
        return bench_sparse(args)

    from paged_kv_fp8_amd import decode
    from paged_kv_fp8_amd.workloads import make_batch, workload

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
    # counter summaries are taken on the workloads as defined (query length aside)
    as_profiled = (set(over) <= {"q_len"} and not args.pools and args.wg_per_cu is None and args.plan == "wave"
                   and not args.fused_merge)
    torch.cuda.set_device(0)
    first = make_batch(w, device="cuda")
    pools = args.pools or min(64, max(3, -(-(1 << 30) // max(1, first.kv_bytes))))
    lens = first.seq_lens.cpu().numpy()
    batches = [first] + [make_batch(dataclasses.replace(w, seed=w.seed + 1000 * i), device="cuda", seq_lens=lens)
                         for i in range(1, pools)]
    decs = [decode.for_batch(b, wg_per_cu=args.wg_per_cu, fused_merge=args.fused_merge, plan=args.plan,
                             **({"dyn_percent": args.dyn_percent, "pieces_per_bin": args.pieces_per_bin}
                                if args.plan == "queued" else {})) for b in batches]
    info = decs[0].plan_info
    ab = algorithmic_bytes(first, decs[0])
    log(f"workload {w.name}: {w.num_seqs} seqs, {int(lens.sum())} tokens, KV {ab['kv'] / 1e6:.1f} MB, "
        f"pools {pools}, plan chunk={info.chunk_tiles} tiles work={info.num_real} slots={info.slots} "
        f"max_splits_used={info.max_n_splits} wg/cu={decs[0].wg_per_cu} cu={decs[0].cu_count}")

    for i in range(args.warmup):
        decs[i % pools].run()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
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
    wall = time.perf_counter() - t0
    eager_ms_step = start.elapsed_time(end) / K
    dec_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    mrg_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))

    # The same K steps as HIP graph replays (one graph per KV pool, each holding
    # that pool's decode + merge launches): a serving loop replays its decode
    # step this way, without per-launch host work or the events between the
    # launches above. This is the step time the metric reports.
    graphs = []
    if args.step_mode == "graph":
        for d in decs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                d.run()
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % pools].replay()
        torch.cuda.synchronize()
        gstart, gend = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        gstart.record()
        for i in range(K):
            graphs[i % pools].replay()
        gend.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        graph_ms_step = gstart.elapsed_time(gend) / K
        ms_step = graph_ms_step
    else:
        graph_ms_step = None
        ms_step = eager_ms_step
    value = ab["kv"] / (ms_step * 1e-3) / 1e9
    dtype = "fp8" if w.q_format == "e4m3" else "bf16"
    t_hbm = ab["total"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = ab["flops"] / (MFMA_PEAK_TFLOPS[dtype] * 1e12)
    achieved = ab["total"] / (dec_ms * 1e-3) / 1e9
    tflops = ab["flops"] / (dec_ms * 1e-3) / 1e12
    if graph_ms_step is not None:
        log(f"graph-replayed step {graph_ms_step * 1e3:.1f} us, eager step {eager_ms_step * 1e3:.1f} us")
    log(f"step {ms_step * 1e3:.1f} us (decode {dec_ms * 1e3:.1f} us, merge {mrg_ms * 1e3:.1f} us), "
        f"host wall {wall / K * 1e6:.1f} us/step; KV {value:.0f} GB/s; decode kernel {achieved:.0f} GB/s "
        f"= {achieved / HBM_PEAK_GBS:.3f} of peak; {tflops:.1f} TFLOP/s = "
        f"{tflops / MFMA_PEAK_TFLOPS[dtype]:.3f} of {dtype} MFMA peak; roofline time "
        f"{max(t_hbm, t_mfma) * 1e6:.1f} us ({'mfma' if t_mfma > t_hbm else 'hbm'})")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_oracle_baseline(first, args.cpu_seconds)
        log(f"cpu oracle: {cpu}")

    kernel = decs[0].kernel_name
    if t_mfma > t_hbm:
        roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_PEAK_TFLOPS[dtype], "unit": "TFLOP/s",
                    "frac": round(tflops / MFMA_PEAK_TFLOPS[dtype], 4), "traffic": None}
    else:
        roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic(kernel, profile_key(w, base.q_len)) if as_profiled else None}
    roofline.update({"kernel": kernel, "kernel_us": round(dec_ms * 1e3, 2), "algorithmic_bytes_per_launch": ab["total"],
                     "algorithmic_flops_per_launch": ab["flops"], "merge_us": round(mrg_ms * 1e3, 2)})
    line = {
        "metric": "achieved HBM GB/s (KV bytes / decode-step time), us per decode step",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1e3, 2),
        "step_mode": args.step_mode,
        "us_per_step_eager": round(eager_ms_step * 1e3, 2),
        "us_per_step_graph": None if graph_ms_step is None else round(graph_ms_step * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "q_len": w.q_len, "h_q": w.h_q, "h_k": w.h_k,
                   "d": w.d_qk, "page_size": w.page_size, "causal": w.causal, "kv_layout": w.kv_layout,
                   "contiguous_pages": w.contiguous_pages, "kv_tokens": int(lens.sum()),
                   "kv_bytes": ab["kv"], "max_splits": w.max_splits, "pools": pools,
                   "merge": "separate launch" if not decs[0].fused_merge else "in decode kernel",
                   "plan_kind": args.plan,
                   "plan": {"chunk_tiles": info.chunk_tiles, "work_items": info.num_real, "slots": info.slots,
                            "max_n_splits": info.max_n_splits, "wg_per_cu": decs[0].wg_per_cu,
                            "bins": info.num_bins}},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
