"""GPU parity of the packed narrow K/V decodes (fp4 e2m1, fp6 e2m3 and e3m2, NVFP4)
against the fp64 oracle, through the C ABI: the page's narrow KV formats with
an e4m3 query, on small variants of each format's workload (one and two
16-row blocks, causal tail and block mode, split and unsplit sequences,
ragged tails, 16-key pages), the full workload on sampled sequences, the edge
lengths, and bit-identical repeats, graph replays and the in-kernel merge. Bars as for the e4m3 cache (e4m3 P): max|dO| <= 1e-2 * max|V| at the
workload's lengths and for edge-batch sequences with L >= 1024, and the
derived short-sequence bound 0.07 * max|V| for the shorter edge lengths; each
edge case prints its measured max|dO| / max|V|."""

import numpy as np
import pytest
import torch

from helpers import O_TOL, assert_matches, compare_fp8_p, gpu_rows, max_abs_v, nan_fill_, oracle_for
from paged_kv_fp8_amd.workloads import make_batch, workload

pytestmark = pytest.mark.gpu
EDGE_LENS = [0, 1, 2, 3, 15, 16, 17, 31, 32, 33, 127, 128, 129, 255, 256, 257, 1000, 1025]
# workload index of each format: the fully-fp8 batch with that K/V format
FORMATS = {"e2m1": 6, "e2m3": 7, "e3m2": 8, "nvfp4": 10}


def _decode():
    from paged_kv_fp8_amd import decode  # loads the HIP library; fails loudly if missing
    return decode


def run(batch, **kw):
    dec = _decode().for_batch(batch, **kw)
    if dec.has_splits:
        nan_fill_(dec.workspace)
    nan_fill_(dec.o)  # every output row must be written
    nan_fill_(dec.lse)
    dec.run()
    torch.cuda.synchronize()
    return dec


def check(batch, dec, seqs=None, o_tol=O_TOL, what=""):
    spec = batch.spec
    nb = batch.to_numpy()
    o_ref, lse_ref = oracle_for(nb, spec, seqs)
    o_g, lse_g = gpu_rows(dec.o, dec.lse, spec, seqs)
    return assert_matches(o_g, lse_g, o_ref, lse_ref, max_abs_v(nb, spec, seqs), o_tol=o_tol, what=what)


SMALL = {
    "one_block": dict(num_seqs=6, seq_len_dist=("mix", 0.34, (3000, 9000), (1024, 2000))),
    "two_blocks_causal": dict(num_seqs=5, q_len=2, seq_len_dist=("uniform", 1024, 5000)),
    "two_blocks_block_mode": dict(num_seqs=5, q_len=2, causal=False, seq_len_dist=("uniform", 1024, 5000)),
    "ps16_hk8": dict(num_seqs=4, h_q=64, h_k=8, page_size=16, seq_len_dist=("uniform", 1024, 3000)),
}


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("name", list(SMALL))
def test_narrow_small_every_output(name, fmt):
    w = workload(FORMATS[fmt], **SMALL[name])
    batch = make_batch(w, device="cuda")
    dec = run(batch)
    err_o, err_l, _ = check(batch, dec, what=f"{fmt} {name}")
    print(f"{fmt} {name}: kernel={dec.kernel_name} splits={dec.plan_info.max_n_splits} "
          f"max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_narrow_full_workload_sampled(fmt):
    w = workload(FORMATS[fmt])
    batch = make_batch(w, device="cuda")
    dec = run(batch)
    lens = batch.seq_lens.cpu().numpy()
    order = np.argsort(lens)
    rng = np.random.default_rng(61)
    seqs = sorted({int(order[0]), int(order[-1])} | {int(x) for x in rng.choice(len(lens), 6, replace=False)})
    err_o, err_l, _ = check(batch, dec, seqs=seqs, what=f"{fmt} full")
    print(f"{fmt} full: work={dec.plan_info.num_real} max_splits_used={dec.plan_info.max_n_splits} "
          f"max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("q_len,causal,ps,force", [(1, True, 128, 0), (2, True, 16, 3), (2, False, 64, 0),
                                                   (1, True, 32, 5)])
def test_narrow_edge_lengths(q_len, causal, ps, force, fmt):
    w = workload(FORMATS[fmt], num_seqs=len(EDGE_LENS), q_len=q_len, page_size=ps, causal=causal,
                 seq_len_dist=("fixed", EDGE_LENS), max_splits=8)
    batch = make_batch(w, device="cuda")
    dec = run(batch, force_splits=force)
    compare_fp8_p(check, batch, dec, f"{fmt} edge q_len={q_len} causal={causal} ps={ps} force={force}")
    o = dec.o.float().cpu().numpy()
    assert np.all(o[0:q_len] == 0.0)  # L = 0: O = 0 exactly (also checked row by row above)


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_narrow_bitwise_repeats_and_graph_replay(fmt):
    w = workload(FORMATS[fmt], num_seqs=12, seq_len_dist=("mix", 0.25, (6000, 20000), (1024, 4096)))
    batch = make_batch(w, device="cuda")
    dec = run(batch)
    assert dec.has_splits
    ref_o, ref_l = dec.o.clone(), dec.lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dec.run()
    for rep in range(3):
        dec.o.zero_()
        dec.lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dec.o.view(torch.int16), ref_o.view(torch.int16)), f"replay {rep}"
        assert torch.equal(dec.lse.view(torch.int32), ref_l.view(torch.int32)), f"replay {rep}"


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_narrow_layouts_bit_identical(fmt):
    # the same codes in the head-major (HND) layout give bit-identical outputs
    lens = ("uniform", 1024, 6000)
    outs = []
    for layout in ("nhd", "hnd"):
        w = workload(FORMATS[fmt], num_seqs=6, seq_len_dist=lens, kv_layout=layout)
        batch = make_batch(w, device="cuda")
        dec = run(batch)
        outs.append((dec.o.clone(), dec.lse.clone(), batch))
    (o1, l1, b1), (o2, l2, b2) = outs
    assert torch.equal(b1.k_cache.contiguous(), b2.k_cache.contiguous())  # same codes, other strides
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
