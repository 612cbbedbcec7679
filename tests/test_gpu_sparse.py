"""GPU parity of the sparse slot-list decode (pkv_sparse_decode) against the
fp64 oracle (``oracle.sparse``), through the C ABI: small batches element by
element (16 to 128 heads, full and padded lists, with and without the sink),
the 16-token flash-sized step of the page, the edge cases (empty lists, a
list left unused, widths that end inside a tile, slots past the pool,
duplicates), and bit-identical repeats and graph replays.

Bar (as for the latent-record decode): max|dO| <= 1e-2 * max|V| over the
listed records, max|dLSE| <= 1e-3; rows with no key and no sink exactly
O = 0, LSE = -inf."""

import numpy as np
import pytest
import torch

from oracle.attention import mla_keys_values
from oracle.sparse import gather_slots, sparse_decode_attention
from paged_kv_fp8_amd.workloads import make_sparse_batch, sparse_workload

pytestmark = pytest.mark.gpu

O_TOL, LSE_TOL = 1e-2, 1e-3


def _sparse():
    from paged_kv_fp8_amd import sparse  # loads the HIP library; fails loudly if missing
    return sparse


def run(batch, **kw):
    dec = _sparse().for_batch(batch, **kw)
    dec.workspace.fill_(255)  # poison the never-initialised workspace (NaN bytes)
    dec.run()
    torch.cuda.synchronize()
    return dec


def listed_vmax(sources):
    """max|V| over the records the lists name (absent entries name none)."""
    vmax = 0.0
    for s in sources:
        _, V = mla_keys_values(gather_slots(s["latent"], s["slots"].ravel()), gather_slots(s["rope"], s["slots"].ravel()),
                               gather_slots(s["scales"], s["slots"].ravel()))
        if V.size:
            vmax = max(vmax, float(np.abs(V).max()))
    return vmax


def check(batch, dec, what=""):
    nb = batch.to_numpy()
    w = batch.spec
    o_ref, l_ref = sparse_decode_attention(nb["q"], nb["sources"], softmax_scale=w.scale, sink=nb["sink"])
    vmax = listed_vmax(nb["sources"])
    o = dec.o.float().cpu().numpy()
    lse = dec.lse.cpu().numpy()
    assert np.all(np.isfinite(o)), what
    err_o = float(np.abs(o - o_ref).max())
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(lse), fin), what
    err_l = float(np.abs(lse[fin] - l_ref[fin]).max()) if fin.any() else 0.0
    assert err_o <= O_TOL * max(vmax, 1e-30) or (vmax == 0 and err_o == 0), f"{what}: max|dO|={err_o} vmax={vmax}"
    assert err_l <= LSE_TOL, f"{what}: max|dLSE|={err_l}"
    empty = ~fin
    assert np.all(o[empty] == 0.0), what
    return err_o, err_l, vmax


SMALL = {
    "hq16": dict(num_tokens=5, seq_len_dist=("uniform", 3000, 9000)),
    "hq32": dict(num_tokens=4, h_q=32, seq_len_dist=("uniform", 3000, 9000)),
    "hq48_padded": dict(num_tokens=6, h_q=48, seq_len_dist=("fixed", [40, 130, 700, 2100, 64, 4000])),
    "hq128_no_sink": dict(num_tokens=3, h_q=128, sink=False, seq_len_dist=("uniform", 2500, 6000)),
    "odd_widths": dict(num_tokens=4, window=100, topk=200, seq_len_dist=("fixed", [50, 400, 1000, 5000])),
    "ps16_ratio8": dict(num_tokens=4, page_size=(16, 16), compress_ratio=8, seq_len_dist=("uniform", 2000, 8000)),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_sparse_small_every_output(name):
    batch = make_sparse_batch(sparse_workload(9, **SMALL[name]), device="cuda")
    dec = run(batch)
    err_o, err_l, vmax = check(batch, dec, what=name)
    print(f"sparse {name}: tiles={dec.tiles} max|dO|={err_o:.3e} (bar {O_TOL * vmax:.3e}) max|dLSE|={err_l:.3e}")


def test_sparse_full_step():
    batch = make_sparse_batch(sparse_workload(9), device="cuda")
    dec = run(batch)
    err_o, err_l, vmax = check(batch, dec, what="full")
    print(f"sparse full: tiles={dec.tiles} max|dO|={err_o:.3e} (bar {O_TOL * vmax:.3e}) max|dLSE|={err_l:.3e}")


def test_sparse_edge_lists():
    w = sparse_workload(9, num_tokens=6, seq_len_dist=("fixed", [300, 300, 300, 300, 300, 6000]))
    batch = make_sparse_batch(w, device="cuda")
    s0, s1 = batch.sources[0]["slots"], batch.sources[1]["slots"]
    n0 = batch.sources[0]["num_pages"] * batch.sources[0]["page_size"]
    s0[0] = -1
    s1[0] = -1                  # token 0: no key, only the sink
    s0[1, 5:9] = n0             # slots past the pool: absent
    s0[1, 9] = n0 + 12345
    s1[2, 10:20] = s1[2, 0]     # duplicates count twice
    s0[3, 0::3] = -7            # scattered holes
    dec = run(batch)
    check(batch, dec, what="edge")
    lse = dec.lse.cpu().numpy()
    assert np.allclose(lse[0], batch.sink.cpu().numpy(), atol=1e-6)  # Z = exp(sink) alone
    assert np.all(dec.o[0].float().cpu().numpy() == 0.0)
    # no sink and no key: O = 0, LSE = -inf
    w2 = sparse_workload(9, num_tokens=2, sink=False, seq_len_dist=("fixed", [300, 900]))
    b2 = make_sparse_batch(w2, device="cuda")
    b2.sources[0]["slots"][0] = -1
    b2.sources[1]["slots"][0] = -1
    d2 = run(b2)
    check(b2, d2, what="empty, no sink")
    assert np.isneginf(d2.lse[0].cpu().numpy()).all()


def test_sparse_one_list_unused():
    batch = make_sparse_batch(sparse_workload(9, num_tokens=3, seq_len_dist=("uniform", 3000, 5000)), device="cuda")
    only = batch.sources[:1]
    dec = _sparse().SparseDecode(q=batch.q, lists=only, softmax_scale=batch.spec.scale, sink=batch.sink)
    dec.run()
    torch.cuda.synchronize()
    nb = batch.to_numpy()
    o_ref, l_ref = sparse_decode_attention(nb["q"], nb["sources"][:1], softmax_scale=batch.spec.scale, sink=nb["sink"])
    vmax = listed_vmax(nb["sources"][:1])
    err_o = float(np.abs(dec.o.float().cpu().numpy() - o_ref).max())
    assert err_o <= O_TOL * vmax, f"max|dO|={err_o} vmax={vmax}"
    assert np.abs(dec.lse.cpu().numpy() - l_ref).max() <= LSE_TOL


def test_sparse_bitwise_repeats_and_graph_replay():
    batch = make_sparse_batch(sparse_workload(9, num_tokens=8, h_q=32), device="cuda")
    dec = run(batch)
    ref_o, ref_l = dec.o.clone(), dec.lse.clone()
    dec.run()
    torch.cuda.synchronize()
    assert torch.equal(dec.o.view(torch.int16), ref_o.view(torch.int16))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dec.run()
    for rep in range(3):
        dec.o.zero_()
        dec.lse.zero_()
        dec.workspace.fill_(255)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dec.o.view(torch.int16), ref_o.view(torch.int16)), f"replay {rep}"
        assert torch.equal(dec.lse.view(torch.int32), ref_l.view(torch.int32)), f"replay {rep}"
