"""Test-side glue: run the fp64 oracle on a synthetic batch's bytes and
compare a GPU result with it at the stated tolerances.

Tolerances (the decode path's accuracy contract): max |O_gpu - O_oracle| <=
1e-2 * max|V| and max |LSE_gpu - LSE_oracle| <= 1e-3, with max|V| the largest
dequantised value of any visible V entry (the latent part for the latent
cache), in fp64. A row that sees no key must be exactly O = 0, LSE = -inf.
"""

import numpy as np
import torch

from oracle import attention as A
from oracle.formats import KV_DECODERS, decode_e4m3
from oracle.producers import nvfp4_kernel_values

O_TOL = 1e-2
LSE_TOL = 1e-3

# The fp8 path rounds P to e4m3(p * 448): up to 2^-4 relative error per p,
# plus the bf16 output rounding, so a row over few keys can be off by up to
# (2^-4 + 2^-9) * max|V|. Rows of sequences with at least 1024 keys (the
# shortest length of any stated workload) average those roundings out and are
# held to O_TOL; shorter ones to the derived bound.
FP8_SHORT_TOL = 0.07
FP8_LONG_LEN = 1024


def oracle_for(np_batch, spec, seqs=None, causal=None):
    """Oracle O and LSE for the sequences ``seqs`` (default: all)."""
    causal = spec.causal if causal is None else causal
    nb = np_batch
    idx = np.arange(spec.num_seqs) if seqs is None else np.asarray(seqs)
    tok = (idx[:, None] * spec.q_len + np.arange(spec.q_len)[None, :]).reshape(-1)
    if spec.kv_format == "mla":
        return A.mla_decode_attention(nb["q"][tok], nb["latent"], nb["rope"], nb["scales"], nb["block_table"][idx],
                                      nb["seq_lens"][idx], q_len=spec.q_len, softmax_scale=spec.scale, causal=causal)
    return A.decode_attention(nb["q"][tok], nb["k_cache"], nb["v_cache"], nb["block_table"][idx], nb["seq_lens"][idx],
                              nb["q_descale"][idx], nb["k_descale"][idx], nb["v_descale"][idx], q_len=spec.q_len,
                              h_k=spec.h_k, softmax_scale=spec.scale, causal=causal, kv_format=spec.kv_format,
                              k_scale=nb.get("k_scale"), v_scale=nb.get("v_scale"))


def max_abs_v(np_batch, spec, seqs=None):
    nb = np_batch
    idx = np.arange(spec.num_seqs) if seqs is None else np.asarray(seqs)
    best = 0.0
    for b in idx:
        L = int(nb["seq_lens"][b])
        if L == 0:
            continue
        for g in range(spec.h_k):
            if spec.kv_format == "mla":
                lat = A.gather_tokens(nb["latent"], nb["block_table"][b], L, 0)
                sc = A.gather_tokens(nb["scales"], nb["block_table"][b], L, 0).astype(np.float64)
                v = decode_e4m3(lat) * np.repeat(sc, 128, axis=-1)
            elif spec.kv_format == "nvfp4":
                v = nvfp4_kernel_values(A.gather_tokens(nb["v_cache"], nb["block_table"][b], L, g),
                                        A.gather_tokens(nb["v_scale"], nb["block_table"][b], L, g))
                v = v * float(nb["v_descale"][b, g])
            else:
                v = KV_DECODERS[spec.kv_format](A.gather_tokens(nb["v_cache"], nb["block_table"][b], L, g))
                v = v * float(nb["v_descale"][b, g])
            best = max(best, float(np.abs(v).max()))
    return best


def gpu_rows(o, lse, spec, seqs=None):
    """Host float64 copies of the GPU outputs of the sequences ``seqs``."""
    idx = np.arange(spec.num_seqs) if seqs is None else np.asarray(seqs)
    tok = (idx[:, None] * spec.q_len + np.arange(spec.q_len)[None, :]).reshape(-1)
    o_h = o.float().cpu().numpy().astype(np.float64)[tok]
    lse_h = lse.cpu().numpy().astype(np.float64)[idx]
    return o_h, lse_h


def rows_view(o, num_seqs, h_k):
    """O rows in the LSE's order: ``o`` is [num_seqs*q_len, h_q, d] (token,
    head); the result is [num_seqs, h_k, q_len*h_r, d] with row n = qi*h_r + hr,
    the qi-major packing of one kv head's query rows."""
    toks, h_q, d = o.shape
    q_len, h_r = toks // num_seqs, h_q // h_k
    o = o.reshape(num_seqs, q_len, h_k, h_r, d).transpose(0, 2, 1, 3, 4)
    return o.reshape(num_seqs, h_k, q_len * h_r, d)


def assert_matches(o_gpu, lse_gpu, o_ref, lse_ref, vmax, o_tol=O_TOL, lse_tol=LSE_TOL, what=""):
    """Element-wise comparison at the contract's bars. Rows with no visible key
    (oracle LSE = -inf) must be exactly O = 0 and LSE = -inf on the GPU.
    Returns (max|dO|, max|dLSE|, indices of the empty rows or None)."""
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite O"
    err_o = float(np.abs(o_gpu - o_ref).max()) if o_ref.size else 0.0
    MARGINS.append((what, err_o / vmax if vmax > 0 else 0.0, o_tol))
    assert err_o <= o_tol * vmax, f"{what}: max|dO| = {err_o:.3e} > {o_tol} * {vmax:.3e}"
    inf_ref = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), inf_ref), f"{what}: -inf rows differ"
    assert not np.any(np.isnan(lse_gpu)), f"{what}: NaN LSE"
    fin = ~inf_ref
    err_l = float(np.abs(lse_gpu[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    assert err_l <= lse_tol, f"{what}: max|dLSE| = {err_l:.3e} > {lse_tol}"
    if not inf_ref.any():
        return err_o, err_l, None
    # empty rows are exact: every element of O is +0 or -0
    o_rows = rows_view(o_gpu, lse_ref.shape[0], lse_ref.shape[1])
    empty = o_rows[inf_ref]
    assert np.all(empty == 0.0), f"{what}: {int((empty != 0).any(axis=-1).sum())} empty rows with nonzero O"
    return err_o, err_l, np.argwhere(inf_ref)


# (case, max|dO| / max|V|, bar) of every comparison made through
# assert_matches; conftest prints those held to a derived bound above O_TOL,
# and the largest ratio among the others, at the end of the run
MARGINS = []


def compare_fp8_p(compare, batch, dec, what, **kw):
    """Compare a decode whose P is e4m3(p * 448) with ``compare(batch, dec,
    seqs=..., o_tol=..., what=...)``: sequences with L >= FP8_LONG_LEN at
    O_TOL, shorter ones at FP8_SHORT_TOL; prints both margins."""
    lens = batch.seq_lens.cpu().numpy()
    groups = (([b for b, L in enumerate(lens) if L < FP8_LONG_LEN], FP8_SHORT_TOL, f"L<{FP8_LONG_LEN}"),
              ([b for b, L in enumerate(lens) if L >= FP8_LONG_LEN], O_TOL, f"L>={FP8_LONG_LEN}"))
    out = []
    for seqs, tol, tag in groups:
        if seqs:
            out.append(compare(batch, dec, seqs=seqs, o_tol=tol, what=f"{what} [{tag}]", **kw))
            case, ratio, bar = MARGINS[-1]
            print(f"{case}: max|dO|/max|V| = {ratio:.3e} (bar {bar})")
    return out


def nan_fill_(t):
    """Fill a workspace with NaN bytes (0xFF in every byte is a float NaN)."""
    t.view(torch.uint8).fill_(0xFF)
    return t
