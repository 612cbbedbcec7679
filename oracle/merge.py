"""Split-KV partials and their LSE merge.

Test infrastructure only (see ``oracle/__init__``).

[T5] module docstring (split-KV scheduling, workspace) and its ``reduction``
kernel: a sequence cut into contiguous KV chunks yields, per chunk j and row,
an unnormalised output O_j = sum_{keys in chunk} exp(s - m_j) v, the chunk
max m_j (natural-log units, -inf if the row sees no key of the chunk) and
l_j = sum exp(s - m_j). The combine takes m* = max_j m_j, weights
w_j = exp(m_j - m*) (0 when m_j = -inf), and gives
  O = o_scale * sum_j w_j O_j / sum_j w_j l_j   (0 when the denominator is 0)
  LSE = m* + ln sum_j w_j l_j.

Pinned by tests/test_oracle.py: for random chunkings the merge of chunk
partials equals ``oracle.attention.attend`` on the whole sequence to 1e-12,
a one-chunk merge is the identity, and all-empty partials give O = 0 and
LSE = -inf.
"""

import numpy as np


def chunk_partial(qrow, K, V, begin, end, limit, softmax_scale):
    """(O_j, m_j, l_j) of keys begin .. end-1 for one row that sees keys
    0 .. limit."""
    stop = min(end, int(limit) + 1)
    if stop <= begin:
        return np.zeros(V.shape[1]), -np.inf, 0.0
    s = softmax_scale * (K[begin:stop] @ qrow)
    m = s.max()
    w = np.exp(s - m)
    return w @ V[begin:stop], m, w.sum()


def merge_partials(o_parts, m_parts, l_parts, o_scale=1.0):
    """Combine partials in the fixed order they are given."""
    m_parts = np.asarray(m_parts, dtype=np.float64)
    m_star = m_parts.max() if m_parts.size else -np.inf
    num = np.zeros(np.asarray(o_parts[0]).shape) if len(o_parts) else 0.0
    den = 0.0
    for o_j, m_j, l_j in zip(o_parts, m_parts, l_parts):
        if m_j == -np.inf:
            continue
        w = np.exp(m_j - m_star)
        num = num + w * np.asarray(o_j)
        den += w * l_j
    if den == 0.0:
        return np.zeros_like(num), -np.inf
    return o_scale * num / den, m_star + np.log(den)


def split_attend(qrows, K, V, limits, softmax_scale, o_scale, bounds):
    """Attention of one (sequence, kv head) computed chunk by chunk over the
    key ranges ``bounds`` = [(begin, end), ...] and merged."""
    n_rows = qrows.shape[0]
    out = np.zeros((n_rows, V.shape[1]))
    lse = np.full(n_rows, -np.inf)
    for n in range(n_rows):
        parts = [chunk_partial(qrows[n], K, V, b, e, limits[n], softmax_scale) for b, e in bounds]
        out[n], lse[n] = merge_partials([p[0] for p in parts], [p[1] for p in parts],
                                        [p[2] for p in parts], o_scale)
    return out, lse
