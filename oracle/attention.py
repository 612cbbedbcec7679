"""Paged-KV decode attention: the plain fp64 definition.

Test infrastructure only (see ``oracle/__init__``).

What is computed ([T5] module docstring; the softmax and epilogue of its
``decode`` kernel; the exact branch of ``emulate_decode``; [VLLM] Kernel
design for the latent-record variant). For sequence b, KV head g and packed
query row n = qi * h_r + hr (qi-major, h_r = h_q / h_k):

  1. row n may see keys j = 0 .. lim(n), with lim(n) = L - q_len + qi under
     the causal tail when q_len > 1, and lim(n) = L - 1 otherwise (q_len == 1,
     or block attention with causal=False); L = seq_lens[b] counts the new
     tokens too.
  2. q = dec(Q[b*q_len + qi, g*h_r + hr]) * qd[b, g]    (qd = 1 for bf16 Q)
  3. key j lives in page block_table[b, j // PS], row j % PS:
     k_j = dec(K[page, row, g]) * kd[b, g],  v_j = dec(V[page, row, g]) * vd[b, g]
  4. s_j = softmax_scale * <q, k_j>;  M = max_j s_j;  l = sum_j exp(s_j - M)
  5. O[n] = o_scale * sum_j exp(s_j - M) v_j / l;  LSE[n] = M + ln l
  6. a row that sees no key has O = 0 and LSE = -inf (the epilogue's empty
     row guard and the combine's zero-weight rule).

Nothing is blocked, tiled, split or rounded: the method on the GPU reaches
this result up to rounding order and its documented roundings of P.

Layouts ([T5] module docstring):
  q           (num_seqs * q_len, h_q, d)   bf16 bit patterns (uint16) or e4m3 (uint8)
  k/v cache   (num_pages, page_size, h_k, d) uint8 e4m3, any strides (logical view);
              kv_format "e2m1": (num_pages, page_size, h_k, d/2) packed fp4 bytes
  block_table (num_seqs, max_blocks)        int32
  seq_lens    (num_seqs,)                   int32
  descales    broadcastable to (num_seqs, h_k), float32
  returns O   (num_seqs * q_len, h_q, d_v)  float64
          LSE (num_seqs, h_k, q_len * h_r)  float64, natural log

Latent-record variant ([VLLM] Kernel design; the record layout is a reading,
stated where ``mla_decode_attention`` is defined): one KV head, a token's key
is its 512 e4m3 latent values times one fp32 scale per 128-value block,
followed by 64 bf16 rope values; its value is the scaled latent part.

Pins (tests/test_oracle.py): pure-Python brute force on tiny inputs, a single
key, constant V, q = 0, the two-key sigmoid, torch's fp64
scaled_dot_product_attention on densely gathered K/V, split invariance
through ``oracle.merge``, page-permutation invariance, causal and block-mode
reductions to q_len = 1, GQA = MHA with replicated K/V, and the latent
variant against the generic core on the explicitly assembled 576-wide keys.
"""

import numpy as np

from .formats import KV_DECODERS, decode_bf16, decode_e4m3, kv_row_elems


def _decode_q(q):
    q = np.asarray(q)
    if q.dtype == np.uint16:
        return decode_bf16(q)
    if q.dtype == np.uint8:
        return decode_e4m3(q)
    raise TypeError(f"q must hold bf16 bits (uint16) or e4m3 codes (uint8), got {q.dtype}")


def _per_seq_head(t, num_seqs, h_k):
    """Descale -> float64 (num_seqs, h_k) by broadcasting: one value per
    tensor, one per kv head (h_k,), or one per (sequence, kv head)."""
    return np.broadcast_to(np.asarray(t, dtype=np.float64), (num_seqs, h_k))


def row_limits(L, q_len, h_r, causal):
    """Last visible key of every packed row n = qi * h_r + hr (step 1)."""
    qi = np.arange(q_len * h_r) // h_r
    if causal and q_len > 1:
        return L - q_len + qi
    return np.full(q_len * h_r, L - 1)


def gather_tokens(cache, block_table_row, L, g):
    """Rows 0 .. L-1 of head g of one sequence, gathered page by page through
    its block-table row (step 3). Only blocks < ceil(L / PS) are looked up and
    only rows < L are taken."""
    ps = cache.shape[1]
    n_blk = -(-L // ps)
    if L == 0:
        return cache[:0, 0, g]
    pages = np.asarray(block_table_row[:n_blk], dtype=np.int64)
    return cache[pages][:, :, g].reshape(n_blk * ps, cache.shape[-1])[:L]


def attend(qrows, K, V, limits, softmax_scale, o_scale):
    """Steps 4-6 for one (sequence, kv head): qrows (N, d_qk), K (L, d_qk),
    V (L, d_v) all float64; limits (N,) last visible key per row."""
    n_rows = qrows.shape[0]
    d_v = V.shape[1]
    out = np.zeros((n_rows, d_v))
    lse = np.full(n_rows, -np.inf)
    for n in range(n_rows):
        vis = int(limits[n]) + 1
        if vis <= 0:
            continue
        s = softmax_scale * (K[:vis] @ qrows[n])
        m = s.max()
        w = np.exp(s - m)
        den = w.sum()
        out[n] = o_scale * (w @ V[:vis]) / den
        lse[n] = m + np.log(den)
    return out, lse


def decode_attention(q, k_cache, v_cache, block_table, seq_lens, q_descale, k_descale, v_descale,
                     *, q_len, h_k, softmax_scale, o_scale=1.0, causal=True, kv_format="e4m3", k_scale=None,
                     v_scale=None):
    """Decode attention of every sequence, KV head and packed row (steps 1-6).
    kv_format names the K/V code format (step 3's dec): "e4m3", one of the
    packed narrow formats of [T5] ("e2m1" fp4, "e2m3" / "e3m2" fp6), or
    "nvfp4" (packed e2m1 with the e4m3 group scales k_scale / v_scale,
    (pages, PS, h_k, d/16) bytes, decoded to the kernel values of
    ``producers.nvfp4_kernel_values``)."""
    if kv_format == "nvfp4":
        from .producers import nvfp4_kernel_values
        d_v = v_cache.shape[-1] * 2

        def gather_kv(cache, scales, bt, L, g):
            return nvfp4_kernel_values(gather_tokens(cache, bt, L, g), gather_tokens(scales, bt, L, g))
    else:
        dec_kv = KV_DECODERS[kv_format]
        d_v = kv_row_elems(v_cache.shape[-1], kv_format)

        def gather_kv(cache, scales, bt, L, g):
            return dec_kv(gather_tokens(cache, bt, L, g))
    q = np.asarray(q)
    seq_lens = np.asarray(seq_lens)
    num_seqs = seq_lens.shape[0]
    h_q, d = q.shape[1], q.shape[2]
    if h_q % h_k:
        raise ValueError("h_q must be a multiple of h_k")
    h_r = h_q // h_k
    n_rows = q_len * h_r
    qf = _decode_q(q)
    qd = _per_seq_head(q_descale, num_seqs, h_k) if q.dtype == np.uint8 else np.ones((num_seqs, h_k))
    kd = _per_seq_head(k_descale, num_seqs, h_k)
    vd = _per_seq_head(v_descale, num_seqs, h_k)
    o = np.zeros((num_seqs * q_len, h_q, d_v))
    lse = np.full((num_seqs, h_k, n_rows), -np.inf)
    for b in range(num_seqs):
        L = int(seq_lens[b])
        lim = row_limits(L, q_len, h_r, causal)
        for g in range(h_k):
            K = gather_kv(k_cache, k_scale, block_table[b], L, g) * kd[b, g]
            V = gather_kv(v_cache, v_scale, block_table[b], L, g) * vd[b, g]
            # packed row n = qi * h_r + hr  <-  token b*q_len + qi, head g*h_r + hr
            rows = qf[b * q_len:(b + 1) * q_len, g * h_r:(g + 1) * h_r].reshape(n_rows, d) * qd[b, g]
            ob, lb = attend(rows, K, V, lim, softmax_scale, o_scale)
            o[b * q_len:(b + 1) * q_len, g * h_r:(g + 1) * h_r] = ob.reshape(q_len, h_r, d_v)
            lse[b, g] = lb
    return o, lse


# ---------------------------------------------------------------------------
# Latent-record (MLA-like) variant
# ---------------------------------------------------------------------------
MLA_LATENT = 512
MLA_ROPE = 64
MLA_BLOCK = 128


def mla_keys_values(latent, rope, scales):
    """Dequantised keys (T, 576) and values (T, 512) of T tokens of the single
    KV head. Reading of [VLLM] Kernel design ("records dequantised exactly to
    bf16", "scales after the data"): key = latent codes times their per-128
    block scale, then the bf16 rope part; value = the scaled latent part."""
    lat = decode_e4m3(latent) * np.repeat(np.asarray(scales, dtype=np.float64), MLA_BLOCK, axis=-1)
    keys = np.concatenate([lat, decode_bf16(rope)], axis=-1)
    return keys, lat


def mla_decode_attention(q, latent, rope, scales, block_table, seq_lens, *, q_len, softmax_scale,
                         o_scale=1.0, causal=True):
    """Latent-record decode: q (num_seqs*q_len, h_q, 576) bf16 bits;
    latent (pages, PS, 1, 512) e4m3; rope (pages, PS, 1, 64) bf16 bits;
    scales (pages, PS, 1, 4) float32. Returns O (num_seqs*q_len, h_q, 512)
    and LSE (num_seqs, 1, q_len*h_q)."""
    q = np.asarray(q)
    seq_lens = np.asarray(seq_lens)
    num_seqs = seq_lens.shape[0]
    h_q = q.shape[1]
    n_rows = q_len * h_q
    qf = _decode_q(q)
    o = np.zeros((num_seqs * q_len, h_q, MLA_LATENT))
    lse = np.full((num_seqs, 1, n_rows), -np.inf)
    for b in range(num_seqs):
        L = int(seq_lens[b])
        lim = row_limits(L, q_len, h_q, causal)
        K, V = mla_keys_values(gather_tokens(latent, block_table[b], L, 0),
                               gather_tokens(rope, block_table[b], L, 0),
                               gather_tokens(scales, block_table[b], L, 0))
        rows = qf[b * q_len:(b + 1) * q_len].reshape(n_rows, -1)
        ob, lb = attend(rows, K, V, lim, softmax_scale, o_scale)
        o[b * q_len:(b + 1) * q_len] = ob.reshape(q_len, h_q, MLA_LATENT)
        lse[b, 0] = lb
    return o, lse
