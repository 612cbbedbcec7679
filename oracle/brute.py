"""Pure-Python brute-force decode attention for tiny inputs.

Test infrastructure only (see ``oracle/__init__``).

A second, independent spelling of the definition in ``oracle.attention``
([T5] module docstring: tensor contract, qi-major query packing, causal
tail / block mode, per-(seq, kv-head) descales; natural-log LSE): nested
Python loops over plain lists, each e4m3 byte decoded from its bit fields
with ``math.ldexp``, bf16 from its bit fields, sums with ``math.fsum``. No
numpy arithmetic, no table, no shared helper. Used only as a pin of the
numpy oracle on inputs small enough for loops (L <= a few dozen, d <= 16).
"""

import math


def e4m3_bits_to_float(code):
    code = int(code)
    s = -1.0 if code >= 128 else 1.0
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return s * math.ldexp(m, -9)  # m/8 * 2^-6
    return s * math.ldexp(8 + m, e - 10)  # (1 + m/8) * 2^(e-7)


def bf16_bits_to_float(bits):
    bits = int(bits)
    s = -1.0 if bits & 0x8000 else 1.0
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0:
        return s * math.ldexp(m, -133)  # m/128 * 2^-126
    if e == 255:
        return math.nan if m else s * math.inf
    return s * math.ldexp(128 + m, e - 134)  # (1 + m/128) * 2^(e-127)


def e2m1_nibble_to_float(code):
    """One e2m1 code from its bit fields: sign | 2-bit exponent (bias 1) | 1-bit mantissa."""
    code = int(code)
    s = -1.0 if code & 8 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        return s * math.ldexp(m, -1)  # m/2 * 2^0
    return s * math.ldexp(2 + m, e - 2)  # (1 + m/2) * 2^(e-1)


def fp4_row_to_floats(row):
    """A packed fp4 row (d/2 bytes) -> d floats: the low nibble of byte i is
    element 2i, the high nibble element 2i+1."""
    out = []
    for byte in row:
        byte = int(byte)
        out.append(e2m1_nibble_to_float(byte & 15))
        out.append(e2m1_nibble_to_float(byte >> 4))
    return out


def _dec(x, fmt):
    return e4m3_bits_to_float(x) if fmt == "e4m3" else bf16_bits_to_float(x)


def brute_decode_attention(q, q_fmt, k_cache, v_cache, block_table, seq_lens, qd, kd, vd,
                           q_len, h_k, softmax_scale, o_scale, causal, kv_fmt="e4m3"):
    """All arguments are nested Python lists (or array-likes indexed one
    element at a time). qd/kd/vd are (num_seqs, h_k) nested lists; qd is
    ignored for bf16 q. Returns (o[token][head][dim], lse[seq][g][n])."""
    num_seqs = len(seq_lens)
    h_q = len(q[0])
    d = len(q[0][0])
    d_v = len(v_cache[0][0][0]) * (2 if kv_fmt == "e2m1" else 1)
    ps = len(k_cache[0])
    h_r = h_q // h_k
    o = [[[0.0] * d_v for _ in range(h_q)] for _ in range(num_seqs * q_len)]
    lse = [[[-math.inf] * (q_len * h_r) for _ in range(h_k)] for _ in range(num_seqs)]
    for b in range(num_seqs):
        L = int(seq_lens[b])
        for g in range(h_k):
            for qi in range(q_len):
                for hr in range(h_r):
                    n = qi * h_r + hr
                    last = (L - q_len + qi) if (causal and q_len > 1) else (L - 1)
                    if last < 0:
                        continue
                    qscale = float(qd[b][g]) if q_fmt == "e4m3" else 1.0
                    qv = [_dec(q[b * q_len + qi][g * h_r + hr][i], q_fmt) * qscale for i in range(d)]
                    scores, values = [], []
                    for j in range(last + 1):
                        page = int(block_table[b][j // ps])
                        row = j % ps
                        if kv_fmt == "e2m1":
                            kv = [x * float(kd[b][g]) for x in fp4_row_to_floats(k_cache[page][row][g])]
                            vv = [x * float(vd[b][g]) for x in fp4_row_to_floats(v_cache[page][row][g])]
                        else:
                            kv = [e4m3_bits_to_float(k_cache[page][row][g][i]) * float(kd[b][g]) for i in range(d)]
                            vv = [e4m3_bits_to_float(v_cache[page][row][g][i]) * float(vd[b][g]) for i in range(d_v)]
                        scores.append(softmax_scale * math.fsum(a * c for a, c in zip(qv, kv)))
                        values.append(vv)
                    top = max(scores)
                    w = [math.exp(s - top) for s in scores]
                    den = math.fsum(w)
                    for i in range(d_v):
                        o[b * q_len + qi][g * h_r + hr][i] = o_scale * math.fsum(
                            wj * vj[i] for wj, vj in zip(w, values)) / den
                    lse[b][g][n] = top + math.log(den)
    return o, lse
