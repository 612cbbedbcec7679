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
