"""Per-phase timestamps of the decode main loops (measurement only).

Builds the library with ``-DPKV_STAMPS=1`` beside the normal one
(``paged_kv_fp8_amd/libpkvfp8_stamps.so``; the normal library is not touched),
runs one workload through it and prints the mean, median and 10th / 90th
percentiles of each phase of a loop step, in shader clocks (s_memtime), over
the steps the library recorded: lane 0 of every wave of workgroups 0-15, the
first 48 steps of their first work item, the first recorded step of each wave
left out (it carries the item's start-up). ``pkv_debug_stamps`` in
``include/pkv_fp8.h`` gives the stamp points.

  python -m paged_kv_fp8_amd.stamps --build               # compile only (no GPU needed)
  python -m paged_kv_fp8_amd.stamps --config 4            # kv-head loop, fully-fp8 batch
  python -m paged_kv_fp8_amd.stamps --config 5 --q-len 16 # latent staged loop
  python -m paged_kv_fp8_amd.stamps --config 5 --q-len 1  # latent pair loop

The stamped kernels keep their phases apart with scheduling barriers, so
they run somewhat slower than the normal build, and the phases cannot
overlap there as they may in the normal build.
"""

import argparse
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
STAMP_LIB = os.path.join(HERE, "libpkvfp8_stamps.so")

PHASES = {
    0: ("kv-head one-item loop, per 32-key block", ["issue", "wait", "process"], 4),
    1: ("latent staged loop, per 32-key step", ["loads+convert", "MFMA phase", "barrier 1", "softmax", "barrier 2"], 6),
    2: ("latent pair loop, per 16-key block", ["issue", "wait", "convert+QK^T", "barrier", "softmax", "PV"], 7),
}
# the stamp buffer each loop's kernel writes (pkv_debug_stamps' loop argument):
# both latent kernels sit in one source and share one
COPY_LOOP = {0: 0, 1: 1, 2: 1}


def phases_for(kernel_name):
    return {"gqa_decode_kernel": 0, "mla_lds_kernel": 1, "mla_pair_kernel": 2}[kernel_name]


def build_stamped():
    from paged_kv_fp8_amd import build

    return build.build(extra_flags=["-DPKV_STAMPS=1"], out=STAMP_LIB)


def summarize(ts, loop):
    """Per-phase statistics of stamps int64[wg][wave][step][point] (0 = not recorded)."""
    import numpy as np

    title, names, n = PHASES[loop]
    rec = (ts[..., 0] > 0) & (ts[..., n - 1] > 0)
    # leave out each wave's first recorded step
    first = np.argmax(rec, axis=2)
    keep = rec.copy()
    wg, wv = np.nonzero(rec.any(axis=2))
    keep[wg, wv, first[wg, wv]] = False
    lines = [f"{title}: {int(keep.sum())} steps"]
    for k, name in enumerate(names):
        d = (ts[..., k + 1] - ts[..., k])[keep]
        lines.append(f"  {name:14s} mean {d.mean():8.1f}  median {np.median(d):8.1f}  "
                     f"p10 {np.percentile(d, 10):8.1f}  p90 {np.percentile(d, 90):8.1f}")
    tot = (ts[..., n - 1] - ts[..., 0])[keep]
    lines.append(f"  {'step total':14s} mean {tot.mean():8.1f}  median {np.median(tot):8.1f}")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--build", action="store_true", help="build the stamped library and exit")
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--q-len", type=int, default=None)
    ap.add_argument("--plan", default="auto")
    ap.add_argument("--runs", type=int, default=5)
    args = ap.parse_args(argv)
    if args.build:
        print(build_stamped())
        return 0
    if not os.path.exists(STAMP_LIB):
        raise SystemExit(f"{STAMP_LIB} is not built: run `python -m paged_kv_fp8_amd.stamps --build`")
    os.environ["PKV_LIB"] = STAMP_LIB  # before the binding loads a library
    import torch
    from paged_kv_fp8_amd import decode, native
    from paged_kv_fp8_amd.workloads import make_batch, workload

    assert native.LIB_PATH == STAMP_LIB, native.LIB_PATH
    over = {} if args.q_len is None else {"q_len": args.q_len}
    w = workload(args.config, **over)
    batch = make_batch(w, device="cuda")
    dec = decode.for_batch(batch, plan=args.plan)
    loop = phases_for(dec.kernel_name)
    print(f"workload {w.name} (q_len {w.q_len}), plan {dec.plan}, kernel {dec.kernel_name}, library {native.LIB_PATH}",
          flush=True)
    for _ in range(args.runs):
        dec.run()
    torch.cuda.synchronize()
    print(summarize(native.debug_stamps(COPY_LOOP[loop]), loop))
    return 0


if __name__ == "__main__":
    sys.exit(main())
