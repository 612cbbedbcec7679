"""GPU parity of the latent-record (MLA-like) decode against the fp64 oracle.

One KV head of 656-byte records (512 e4m3 latent values, 64 bf16 rope values,
four fp32 scales, one per 128 latent values), 16 query heads, q tokens
T in {1, 2, 4, 8, 16} with the causal tail, 64-key pages. Bars as for the
GQA path: max|dO| <= 1e-2 * max|V| (V = scaled latent), max|dLSE| <= 1e-3,
empty rows exactly O = 0 / LSE = -inf.
"""

import numpy as np
import pytest
import torch

from helpers import O_TOL, assert_matches, gpu_rows, max_abs_v, nan_fill_, oracle_for
from paged_kv_fp8_amd.workloads import make_batch, workload

pytestmark = pytest.mark.gpu


def run_batch(batch, **kw):
    from paged_kv_fp8_amd import decode

    dec = decode.for_batch(batch, **kw)
    if dec.has_splits:
        nan_fill_(dec.workspace)
    nan_fill_(dec.o)  # every output row must be written
    nan_fill_(dec.lse)
    dec.run()
    torch.cuda.synchronize()
    return dec


def compare(batch, dec, seqs=None, what=""):
    spec = batch.spec
    nb = batch.to_numpy()
    o_ref, lse_ref = oracle_for(nb, spec, seqs)
    o_g, lse_g = gpu_rows(dec.o, dec.lse, spec, seqs)
    return assert_matches(o_g, lse_g, o_ref, lse_ref, max_abs_v(nb, spec, seqs), what=what)


@pytest.mark.parametrize("T,causal", [(1, True), (2, True), (3, True), (4, True), (4, False), (5, True), (5, False),
                                      (8, True), (16, True)])
def test_small_latent_every_output(T, causal):
    w = workload(5, q_len=T, causal=causal, num_seqs=4, seq_len_dist=("uniform", 40, 700))
    batch = make_batch(w, device="cuda")
    dec = run_batch(batch)
    err_o, err_l, _ = compare(batch, dec, what=f"latent T={T} causal={causal}")
    print(f"T={T} causal={causal}: splits={dec.plan_info.max_n_splits} max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")


@pytest.mark.parametrize("T", [1, 2, 4, 8, 16])
def test_full_latent_sampled(T):
    w = workload(5, q_len=T)
    batch = make_batch(w, device="cuda")
    dec = run_batch(batch)
    lens = batch.seq_lens.cpu().numpy()
    order = np.argsort(lens)
    seqs = sorted({int(order[0]), int(order[-1]), 3, 17})
    err_o, err_l, _ = compare(batch, dec, seqs=seqs, what=f"latent full T={T}")
    print(f"T={T}: seqs={seqs} splits={dec.plan_info.max_n_splits} chunk={dec.plan_info.chunk_tiles} "
          f"work={dec.plan_info.num_real} max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")


EDGE = [0, 1, 2, 15, 16, 17, 63, 64, 65, 127, 128, 129, 1000]


@pytest.mark.parametrize("T,force", [(1, 0), (2, 3), (4, 2), (8, 0), (8, 5)])
def test_latent_edge_lengths(T, force):
    w = workload(5, q_len=T, num_seqs=len(EDGE), seq_len_dist=("fixed", EDGE), max_splits=8)
    batch = make_batch(w, device="cuda")
    dec = run_batch(batch, force_splits=force)
    compare(batch, dec, what=f"latent edge T={T} force={force}")


@pytest.mark.parametrize("T", [1, 2, 4, 8])
def test_latent_edge_lengths_balanced_plan(T):
    # key-range items, among them the empty item of the L = 0 sequence (its rows: O = 0, LSE = -inf)
    w = workload(5, q_len=T, num_seqs=len(EDGE), seq_len_dist=("fixed", EDGE), max_splits=8)
    batch = make_batch(w, device="cuda")
    dec = run_batch(batch, plan="balanced")
    assert dec.plan == "balanced"
    compare(batch, dec, what=f"latent edge balanced T={T}")


@pytest.mark.parametrize("T", [2, 8])
def test_latent_repeat_bitwise(T):
    # T = 2: the pair form (two row groups, record split by d_v half); T = 8: records staged in LDS
    w = workload(5, q_len=T, num_seqs=6, seq_len_dist=("uniform", 100, 3000))
    batch = make_batch(w, device="cuda")
    dec = run_batch(batch)
    o1, l1 = dec.o.clone(), dec.lse.clone()
    for fill in (0x00, 0x7F):
        dec.workspace.fill_(fill)
        dec.run()
        torch.cuda.synchronize()
        assert torch.equal(dec.o.view(torch.int16), o1.view(torch.int16))
        assert torch.equal(dec.lse.view(torch.int32), l1.view(torch.int32))


@pytest.mark.parametrize("T", [1, 4, 16])
def test_latent_balanced_plan(T):
    w = workload(5, q_len=T, num_seqs=6, seq_len_dist=("uniform", 100, 4000))
    batch = make_batch(w, device="cuda")
    dec = run_batch(batch, plan="balanced")
    compare(batch, dec, what=f"latent balanced T={T}")


@pytest.mark.parametrize("h_q,T", [(8, 8), (8, 12), (32, 2), (32, 3)])
def test_latent_other_head_counts(h_q, T):
    # rows = T * h_q: 64, 96 (a part-filled second tile), 64, 96 with the staged form
    w = workload(5, q_len=T, h_q=h_q, num_seqs=5, seq_len_dist=("uniform", 30, 2500))
    batch = make_batch(w, device="cuda")
    dec = run_batch(batch)
    compare(batch, dec, what=f"latent h_q={h_q} T={T}")


def test_latent_staged_graph_replay():
    w = workload(5, q_len=8, num_seqs=6, seq_len_dist=("uniform", 200, 5000))
    batch = make_batch(w, device="cuda")
    dec = run_batch(batch)
    eager_o, eager_l = dec.o.clone(), dec.lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dec.run()
    for rep in range(3):
        dec.o.zero_()
        dec.lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dec.o.view(torch.int16), eager_o.view(torch.int16)), f"replay {rep}"
        assert torch.equal(dec.lse.view(torch.int32), eager_l.view(torch.int32)), f"replay {rep}"


@pytest.mark.parametrize("force", [0, 3])
def test_latent_staged_late_huge_score_restarts(force):
    # The staged form fixes each row's reference max at its first visible
    # block; a key whose score lies far above it (here ~5e4 raw units over a
    # first-block max of ~30, with the softmax scale 1/24) would push some p
    # past the kernel's bound, so the workgroup runs the item again with the
    # larger reference. The result must still be the plain softmax.
    w = workload(5, q_len=4, num_seqs=2, seq_len_dist=("fixed", [900, 700]), max_splits=8)
    batch = make_batch(w, device="cuda")
    j0 = 100  # key of sequence 0, in its fourth 32-key block
    page = int(batch.block_table[0, j0 // w.page_size])
    row = j0 % w.page_size
    q0 = batch.q[0, 0, :512].float()  # query token 0, head 0: sees keys 0 .. L - 4
    codes = (q0 / 0.02).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    batch.mla_latent[page, row, 0] = codes
    batch.mla_scales[page, row, 0] = 2.0
    dec = run_batch(batch, force_splits=force)
    assert dec.kernel_name == "mla_lds_kernel"
    err_o, err_l, _ = compare(batch, dec, what=f"latent late huge score force={force}")
    lse = dec.lse[0, 0, 0].item()
    assert lse > 1000.0, lse  # the planted key dominates row 0
    print(f"force={force}: LSE row 0 = {lse:.3f}, max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")


def _max_qk_abs_dot(batch, w):
    """max over (sequence, query row, visible key) of sum_i |q_i| |k_i| over the
    512 latent dims, k = code x block scale (float64)."""
    lat = batch.mla_latent.cpu().view(torch.float8_e4m3fn).double().reshape(-1, 4, 128)
    scl = batch.mla_scales.cpu().double().reshape(-1, 4)
    kabs = (lat * scl[:, :, None]).abs().reshape(-1, 512)
    q = batch.q.cpu().double()[..., :512].abs()
    bt = batch.block_table.cpu()
    best = 0.0
    for b, L in enumerate(batch.seq_lens.cpu().tolist()):
        if L == 0:
            continue
        keys = torch.arange(L)
        slots = bt[b, keys // w.page_size].long() * w.page_size + keys % w.page_size
        qb = q[b * w.q_len:(b + 1) * w.q_len].reshape(-1, 512)
        best = max(best, float((qb @ kabs[slots].T).max()))
    return best


@pytest.mark.parametrize("T", [4, 16])
def test_latent_staged_other_scales_round(T):
    # The record format's scales are powers of two, which the staged form folds
    # into its bf16 key rows exactly. A wave that meets any other scale takes
    # the fp32 product rounded to bf16: each dequantised value then carries a
    # relative error of at most 2^-9, so a score moves by at most
    # dS = scale * 2^-9 * sum_i |q_i| |k_i| (latent dims), the LSE by dS, and O
    # by 2^-9 max|V| from V plus 2 (e^(2 dS) - 1) max|V| from the weights.
    w = workload(5, q_len=T, num_seqs=4, seq_len_dist=("uniform", 300, 1500))
    batch = make_batch(w, device="cuda")
    sc = batch.mla_scales.view(-1, 4)
    sc[::7, 1] *= 1.3
    sc[3::11, 3] *= 0.77
    dec = run_batch(batch)
    assert dec.kernel_name == "mla_lds_kernel"
    ds = w.scale * 2.0 ** -9 * _max_qk_abs_dot(batch, w)
    o_tol = O_TOL + 2.0 ** -9 + 2.0 * np.expm1(2.0 * ds)
    lse_tol = 1e-3 + ds
    nb = batch.to_numpy()
    o_ref, lse_ref = oracle_for(nb, batch.spec)
    o_g, lse_g = gpu_rows(dec.o, dec.lse, batch.spec)
    err_o, err_l, _ = assert_matches(o_g, lse_g, o_ref, lse_ref, max_abs_v(nb, batch.spec), o_tol=o_tol,
                                     lse_tol=lse_tol, what=f"latent other scales T={T}")
    print(f"T={T}: dS bound {ds:.3e}; max|dO|={err_o:.3e} (bar {o_tol:.3e} max|V|) max|dLSE|={err_l:.3e} "
          f"(bar {lse_tol:.3e})")


@pytest.mark.parametrize("T", [1, 8])
def test_latent_split_count_at_the_library_cap(T):
    # one latent sequence of 256 tiles in 256 splits (PKV_MAX_SPLITS), one of 3 tiles in 3
    w = workload(5, q_len=T, num_seqs=2, seq_len_dist=("fixed", [32768, 300]), max_splits=256)
    batch = make_batch(w, device="cuda")
    dec = run_batch(batch, force_splits=256)
    assert dec.n_splits.cpu().tolist() == [256, 3]
    err_o, err_l, _ = compare(batch, dec, what=f"latent 256 splits T={T}")
    print(f"T={T}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")
