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


def fp6_code_to_float(code, kv_fmt):
    """One 6-bit code from its bit fields: e2m3 = sign | 2-bit exponent (bias 1)
    | 3-bit mantissa; e3m2 = sign | 3-bit exponent (bias 3) | 2-bit mantissa."""
    code = int(code)
    s = -1.0 if code & 32 else 1.0
    if kv_fmt == "e2m3":
        e, m = (code >> 3) & 3, code & 7
        return s * (math.ldexp(m, -3) if e == 0 else math.ldexp(8 + m, e - 4))
    e, m = (code >> 2) & 7, code & 3
    return s * (math.ldexp(m, -4) if e == 0 else math.ldexp(4 + m, e - 5))


def fp6_row_to_floats(row, kv_fmt):
    """A packed fp6 row (3d/4 bytes) -> d floats: the whole row read as one
    little-endian integer, element i = bits 6i .. 6i+5."""
    n = int.from_bytes(bytes(int(x) for x in row), "little")
    return [fp6_code_to_float((n >> (6 * i)) & 63, kv_fmt) for i in range(len(row) * 8 // 6)]


def e4m3_round_brute(x):
    """The e4m3 value nearest to x (finite, |x| <= 448), ties to the even
    code: a search over all 127 non-negative finite codes."""
    best = None
    for code in range(0x7F):
        v = e4m3_bits_to_float(code)
        d = abs(abs(x) - v)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code, v)
    return math.copysign(best[2], x)


def nvfp4_row_to_floats(row, scales):
    """A packed NVFP4 row (d/2 bytes) with its e4m3 group scales (d/16 bytes)
    -> the d kernel values e4m3(code * scale / 8)."""
    codes = fp4_row_to_floats(row)
    return [e4m3_round_brute(c * e4m3_bits_to_float(scales[i // 16]) / 8.0) for i, c in enumerate(codes)]


def _row_floats(row, kv_fmt):
    if kv_fmt == "e2m1":
        return fp4_row_to_floats(row)
    if kv_fmt in ("e2m3", "e3m2"):
        return fp6_row_to_floats(row, kv_fmt)
    return [e4m3_bits_to_float(x) for x in row]


def _dec(x, fmt):
    return e4m3_bits_to_float(x) if fmt == "e4m3" else bf16_bits_to_float(x)


def brute_decode_attention(q, q_fmt, k_cache, v_cache, block_table, seq_lens, qd, kd, vd,
                           q_len, h_k, softmax_scale, o_scale, causal, kv_fmt="e4m3", k_scale=None, v_scale=None):
    """All arguments are nested Python lists (or array-likes indexed one
    element at a time). qd/kd/vd are (num_seqs, h_k) nested lists; qd is
    ignored for bf16 q. Returns (o[token][head][dim], lse[seq][g][n])."""
    num_seqs = len(seq_lens)
    h_q = len(q[0])
    d = len(q[0][0])
    d_v = len(v_cache[0][0][0]) * 8 // {"e2m1": 4, "nvfp4": 4, "e2m3": 6, "e3m2": 6}.get(kv_fmt, 8)
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
                        if kv_fmt == "nvfp4":
                            kr = nvfp4_row_to_floats(k_cache[page][row][g], k_scale[page][row][g])
                            vr = nvfp4_row_to_floats(v_cache[page][row][g], v_scale[page][row][g])
                        else:
                            kr = _row_floats(k_cache[page][row][g], kv_fmt)
                            vr = _row_floats(v_cache[page][row][g], kv_fmt)
                        kv = [x * float(kd[b][g]) for x in kr]
                        vv = [x * float(vd[b][g]) for x in vr]
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


def brute_sparse_decode(q, sources, softmax_scale, o_scale, sink):
    """Slot-list decode over latent records with nested loops: q[t][h][576]
    bf16 bits; each source a dict of nested lists "latent" [page][row][0][512]
    e4m3 codes, "rope" [page][row][0][64] bf16 bits, "scales" [page][row][0][4]
    floats and "slots" [t][width]; sink [h] or None. A slot s is row s % PS of
    page s // PS; negative entries and entries past the pool are skipped.
    Returns (o[t][h][512],
    lse[t][h])."""
    T, h_q = len(q), len(q[0])
    o = [[[0.0] * 512 for _ in range(h_q)] for _ in range(T)]
    lse = [[-math.inf] * h_q for _ in range(T)]
    for t in range(T):
        recs = []  # (key 576 floats, value 512 floats)
        for src in sources:
            ps = len(src["latent"][0])
            for s in src["slots"][t]:
                s = int(s)
                if s < 0 or s >= len(src["latent"]) * ps:
                    continue
                page, row = s // ps, s % ps
                sc = [float(x) for x in src["scales"][page][row][0]]
                lat = [e4m3_bits_to_float(src["latent"][page][row][0][i]) * sc[i // 128] for i in range(512)]
                rope = [bf16_bits_to_float(x) for x in src["rope"][page][row][0]]
                recs.append((lat + rope, lat))
        for h in range(h_q):
            qv = [bf16_bits_to_float(x) for x in q[t][h]]
            z = [softmax_scale * math.fsum(a * b for a, b in zip(k, qv)) for k, _ in recs]
            terms = z + ([float(sink[h])] if sink is not None else [])
            if not terms:
                continue
            m = max(terms)
            w = [math.exp(x - m) for x in z]
            Z = math.fsum(w + ([math.exp(float(sink[h]) - m)] if sink is not None else []))
            for d in range(512):
                o[t][h][d] = o_scale * math.fsum(w[j] * recs[j][1][d] for j in range(len(recs))) / Z
            lse[t][h] = m + math.log(Z)
    return o, lse
