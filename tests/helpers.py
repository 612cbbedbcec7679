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


def assert_matches(o_gpu, lse_gpu, o_ref, lse_ref, vmax, o_tol=O_TOL, lse_tol=LSE_TOL, what=""):
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite O"
    err_o = float(np.abs(o_gpu - o_ref).max()) if o_ref.size else 0.0
    assert err_o <= o_tol * vmax, f"{what}: max|dO| = {err_o:.3e} > {o_tol} * {vmax:.3e}"
    inf_ref = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), inf_ref), f"{what}: -inf rows differ"
    assert not np.any(np.isnan(lse_gpu)), f"{what}: NaN LSE"
    fin = ~inf_ref
    err_l = float(np.abs(lse_gpu[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    assert err_l <= lse_tol, f"{what}: max|dLSE| = {err_l:.3e} > {lse_tol}"
    # empty rows are exact
    if inf_ref.any():
        rows = np.argwhere(inf_ref)
        return err_o, err_l, rows
    return err_o, err_l, None


def nan_fill_(t):
    """Fill a workspace with NaN bytes (0xFF in every byte is a float NaN)."""
    t.view(torch.uint8).fill_(0xFF)
    return t
