"""Sparse slot-list decode over latent records, the plain definition.

Test infrastructure only (see ``oracle/__init__``).

[VLLM] "vLLM PR #62633: swap-AB CuTe DSL decode attention for DeepSeek-V4.1",
Kernel design: every decode token attends to the records named by its slot
lists, a sliding-window list and a top-k list of compressed records, each
record gathered in place from its paged cache; S = KV Q^T and O = KV^T P (the
record is both key and value); the token's partials are merged together with
the attention sink. Readings taken here (the page leaves them open):

  * A slot is a flat index into a pool of pages, page * page_size + row
    (the usual paged-cache slot mapping); a negative entry, or one past the
    pool, names no key. Entries are keys, so a slot listed twice counts
    twice.
  * The record is this package's latent record (``attention.mla_keys_values``:
    512 e4m3 codes times one fp32 scale per 128 values, then 64 bf16 rope
    values; the value is the scaled latent part); the model's own record
    format needs the model.
  * The sink of head h is a logit in the units of the scaled scores: it adds
    exp(sink_h) to the softmax denominator and nothing to the numerator.

For token t and head h, with z_s = softmax_scale * <q[t, h], key_s> over the
listed slots s of both lists:
    Z = sum_s exp(z_s) + exp(sink_h)        (no sink term when sink is None)
    O[t, h] = o_scale * sum_s exp(z_s) value_s / Z,    LSE[t, h] = log Z,
and O = 0, LSE = -inf when Z = 0 (no key and no sink).

Pins (tests/test_sparse_oracle.py): the contiguous latent decode reproduced
by listing a sequence's own slots; the closed form of the sink
(LSE' = logaddexp(LSE, sink), O' = O * exp(LSE - LSE')); a pure-Python brute
force on tiny inputs; order invariance of the lists; split invariance through
``oracle.merge`` plus one sink term; empty lists with and without a sink; an
entry past the pool equal to a negative one.
"""

import numpy as np

from .attention import _decode_q, mla_keys_values


def gather_slots(pool, slots):
    """Records of the listed slots: pool (pages, page_size, 1, w) -> (n, w)
    for the entries of `slots` inside the pool, in list order."""
    pool = np.asarray(pool)
    flat = pool.reshape(pool.shape[0] * pool.shape[1], pool.shape[-1])
    s = np.asarray(slots)
    s = s[(s >= 0) & (s < flat.shape[0])]
    return flat[s]


def sparse_decode_attention(q, sources, *, softmax_scale, o_scale=1.0, sink=None):
    """q (T, h_q, 576) bf16 bits; sources: a list of dicts with "latent"
    (pages, PS, 1, 512) e4m3, "rope" (pages, PS, 1, 64) bf16 bits, "scales"
    (pages, PS, 1, 4) float32 and "slots" (T, width) int32; sink: (h_q,) or
    None. Returns O (T, h_q, 512) and LSE (T, h_q)."""
    qf = _decode_q(q)
    T, h_q = qf.shape[0], qf.shape[1]
    o = np.zeros((T, h_q, 512))
    lse = np.full((T, h_q), -np.inf)
    for t in range(T):
        keys, vals = [], []
        for src in sources:
            k, v = mla_keys_values(gather_slots(src["latent"], src["slots"][t]),
                                   gather_slots(src["rope"], src["slots"][t]),
                                   gather_slots(src["scales"], src["slots"][t]))
            keys.append(k)
            vals.append(v)
        K = np.concatenate(keys, axis=0)
        V = np.concatenate(vals, axis=0)
        for h in range(h_q):
            z = softmax_scale * (K @ qf[t, h])
            terms = list(z) + ([float(sink[h])] if sink is not None else [])
            if not terms:
                continue
            m = max(terms)
            w = np.exp(z - m)
            Z = w.sum() + (np.exp(float(sink[h]) - m) if sink is not None else 0.0)
            o[t, h] = o_scale * (w @ V) / Z
            lse[t, h] = m + np.log(Z)
    return o, lse
