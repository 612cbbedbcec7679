"""GPU parity of the producers (pkv_quantize_q, pkv_write_kv) against the
oracle: codes and scales bit for bit (byte work), on the same seeded inputs,
including exact ties, e4m3 subnormals, saturation, NaN inputs, strided views
and sequences shorter than the new-token count."""

import numpy as np
import pytest
import torch

from oracle.producers import quantize_q as oracle_quantize_q
from oracle.producers import write_kv_e4m3, write_kv_latent
from paged_kv_fp8_amd import producers

pytestmark = pytest.mark.gpu


def bf16(x, device="cuda"):
    return torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16).to(device)


def as_f32(t):
    return t.float().cpu().numpy()


@pytest.mark.parametrize("num_seqs,q_len,h_q,h_k,d", [(4, 1, 32, 8, 128), (8, 4, 64, 4, 128), (3, 16, 16, 1, 576),
                                                      (2, 3, 6, 3, 64)])
def test_quantize_q_bitwise(num_seqs, q_len, h_q, h_k, d):
    g = torch.Generator(device="cuda").manual_seed(11 + q_len)
    q = torch.randn(num_seqs * q_len, h_q, d, device="cuda", generator=g)
    scale = torch.exp(torch.randn(num_seqs, 1, h_k, 1, device="cuda", generator=g) * 3)  # 1e-4 .. 1e4 per group
    q = (q.view(num_seqs, q_len, h_k, h_q // h_k, d) * scale[:, :, :, None]).view(q.shape).to(torch.bfloat16)
    q[:q_len, : h_q // h_k] = 0  # an all-zero group
    q8, qd = producers.quantize_q(q, num_seqs, q_len, h_k)
    torch.cuda.synchronize()
    want8, wantd = oracle_quantize_q(as_f32(q), num_seqs, q_len, h_k)
    assert np.array_equal(qd.cpu().numpy().view(np.uint32), wantd.view(np.uint32))
    assert np.array_equal(q8.cpu().numpy(), want8)


def test_quantize_q_ties_and_subnormals():
    # amax 448 -> descale exactly 1: q / descale is q itself, so midpoints of e4m3
    # values (exact in bf16) must round to the even code, and tiny values land
    # on e4m3 subnormals
    from oracle.formats import E4M3_TABLE

    fin = np.sort(np.unique(np.abs(E4M3_TABLE[np.isfinite(E4M3_TABLE)])))
    mids = (fin[1:] + fin[:-1]) / 2
    vals = np.concatenate([[448.0], mids, -mids, fin, 2.0 ** -np.arange(6, 13)])
    d = 128
    vals = np.resize(vals, (len(vals) + d - 1) // d * d).reshape(-1, d)
    q = bf16(vals[:, None, :])  # q_len rows, one head
    n = q.shape[0]
    q8, qd = producers.quantize_q(q, 1, n, 1)
    torch.cuda.synchronize()
    want8, wantd = oracle_quantize_q(as_f32(q), 1, n, 1)
    assert float(qd[0, 0]) == 1.0 and wantd[0, 0] == 1.0
    assert np.array_equal(q8.cpu().numpy(), want8)


def test_quantize_q_strided_views():
    base = torch.randn(6, 40, 256, device="cuda").to(torch.bfloat16)
    q = base[:, 4:36, 64:192]  # token stride 40*256, head stride 256, d = 128
    q8_full = torch.zeros(6, 36, 160, dtype=torch.uint8, device="cuda")
    q8 = q8_full[:, 2:34, 16:144]
    qd_full = torch.zeros(3, 16, dtype=torch.float32, device="cuda")
    qd = qd_full[:, ::4]
    producers.quantize_q(q, 3, 2, 4, q8=q8, q_descale=qd)
    torch.cuda.synchronize()
    want8, wantd = oracle_quantize_q(as_f32(q), 3, 2, 4)
    assert np.array_equal(q8.cpu().numpy(), want8)
    assert np.array_equal(qd.cpu().numpy(), wantd)
    untouched = q8_full.clone()
    untouched[:, 2:34, 16:144] = 0
    assert int(untouched.count_nonzero()) == 0


def _pool(num_seqs, lens, ps, n_extra, gen):
    blocks = [max(1, -(-int(L) // ps)) for L in lens]
    num_pages = sum(blocks) + n_extra
    perm = torch.randperm(num_pages, generator=gen).tolist()
    max_blocks = max(blocks) + 1
    bt = torch.full((num_seqs, max_blocks), num_pages - 1, dtype=torch.int32)
    i = 0
    for b, nb in enumerate(blocks):
        bt[b, :nb] = torch.tensor(perm[i:i + nb])
        i += nb
    return bt, num_pages


@pytest.mark.parametrize("n_new,ps,h_k,layout", [(1, 16, 8, "nhd"), (4, 64, 8, "nhd"), (2, 128, 4, "hnd"),
                                                 (3, 32, 2, "nhd")])
def test_write_kv_e4m3_bitwise(n_new, ps, h_k, layout):
    gen = torch.Generator().manual_seed(100 + n_new)
    num_seqs, d = 6, 128
    lens = [int(x) for x in torch.randint(n_new, 700, (num_seqs,), generator=gen)]
    lens[0] = max(1, n_new - 1)  # shorter than n_new: its first token has no slot and is skipped
    bt, num_pages = _pool(num_seqs, lens, ps, 3, gen)
    if layout == "nhd":
        k_buf = torch.randint(0, 256, (num_pages, ps, h_k, d), dtype=torch.uint8, generator=gen)
        v_buf = torch.randint(0, 256, (num_pages, ps, h_k, d), dtype=torch.uint8, generator=gen)
        kc, vc = k_buf.cuda(), v_buf.cuda()
        k_view, v_view = kc, vc
    else:  # (pages, 2, h_k, ps, d) with K/V views permuted to (pages, ps, h_k, d)
        buf = torch.randint(0, 256, (num_pages, 2, h_k, ps, d), dtype=torch.uint8, generator=gen).cuda()
        k_view, v_view = buf[:, 0].permute(0, 2, 1, 3), buf[:, 1].permute(0, 2, 1, 3)
    k_before, v_before = k_view.cpu().numpy().copy(), v_view.cpu().numpy().copy()
    kn = torch.randn(num_seqs * n_new, h_k, d, generator=gen) * 3
    vn = torch.randn(num_seqs * n_new, h_k, d, generator=gen) * 3
    kn[1, 0, :4] = float("nan")
    kd = (torch.rand(num_seqs, h_k, generator=gen) * 0.02 + 0.001).float()
    vd = (torch.rand(num_seqs, h_k, generator=gen) * 0.02 + 0.001).float()
    kd[2, 0] = 1e-4  # most of this row saturates
    kn_d, vn_d = kn.to(torch.bfloat16).cuda(), vn.to(torch.bfloat16).cuda()
    seq = torch.tensor(lens, dtype=torch.int32).cuda()
    producers.write_kv(kn_d, vn_d, bt.cuda(), seq, n_new, k_view, v_view, kd.cuda(), vd.cuda())
    torch.cuda.synchronize()
    want_k = write_kv_e4m3(k_before, as_f32(kn_d), lens, n_new, bt.numpy(), kd.numpy())
    want_v = write_kv_e4m3(v_before, as_f32(vn_d), lens, n_new, bt.numpy(), vd.numpy())
    assert np.array_equal(k_view.cpu().numpy(), want_k)
    assert np.array_equal(v_view.cpu().numpy(), want_v)


@pytest.mark.parametrize("n_new", [1, 16])
def test_write_latent_bitwise(n_new):
    gen = torch.Generator().manual_seed(200 + n_new)
    num_seqs, ps = 5, 64
    lens = [int(x) for x in torch.randint(n_new, 3000, (num_seqs,), generator=gen)]
    bt, num_pages = _pool(num_seqs, lens, ps, 2, gen)
    lat = torch.randint(0, 256, (num_pages, ps, 512), dtype=torch.uint8, generator=gen)
    rope = torch.randint(0, 65536, (num_pages, ps, 64), dtype=torch.int32, generator=gen).to(torch.int16)
    scl = torch.rand(num_pages, ps, 4, generator=gen)
    x = torch.randn(num_seqs * n_new, 576, generator=gen) * torch.exp(torch.randn(num_seqs * n_new, 1, generator=gen))
    x[0, 128:256] = 0
    x_d = x.to(torch.bfloat16).cuda()
    lat_d, rope_d, scl_d = lat.cuda(), rope.cuda(), scl.cuda()
    producers.write_latent(x_d, bt.cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), n_new, lat_d, rope_d, scl_d)
    torch.cuda.synchronize()
    xf = as_f32(x_d)
    rope_new = x_d[:, 512:].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    want_lat, want_rope, want_scl = write_kv_latent(lat.numpy(), rope.numpy().view(np.uint16), scl.numpy(),
                                                    xf[:, :512], rope_new, lens, n_new, bt.numpy())
    assert np.array_equal(lat_d.cpu().numpy(), want_lat)
    assert np.array_equal(rope_d.cpu().numpy().view(np.uint16), want_rope)
    assert np.array_equal(scl_d.cpu().numpy().view(np.uint32), want_scl.view(np.uint32))


def test_quantized_query_feeds_the_fp8_decode():
    """Quantise the fully-fp8 workload's query on the device, decode with it,
    and compare with the oracle on the same codes."""
    from helpers import assert_matches, gpu_rows, max_abs_v, oracle_for
    from paged_kv_fp8_amd.decode import for_batch
    from paged_kv_fp8_amd.workloads import make_batch, workload

    w = workload(4, num_seqs=6, seq_len_dist=("uniform", 1024, 3000))
    batch = make_batch(w, device="cuda")
    qbf = (torch.randn(batch.q.shape, device="cuda") * 2).to(torch.bfloat16)
    q8, qd = producers.quantize_q(qbf, w.num_seqs, w.q_len, w.h_k)
    batch.q.copy_(q8)
    batch.q_descale.copy_(qd)
    dec = for_batch(batch)
    dec.run()
    torch.cuda.synchronize()
    nb = batch.to_numpy()
    o_ref, lse_ref = oracle_for(nb, batch.spec, None)
    o_g, lse_g = gpu_rows(dec.o, dec.lse, batch.spec, None)
    assert_matches(o_g, lse_g, o_ref, lse_ref, max_abs_v(nb, batch.spec, None), what="quantised q -> fp8 decode")
