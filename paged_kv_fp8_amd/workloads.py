"""Seeded synthetic decode batches in the paged-KV tensor contract.

This module only draws random numbers and stores them in the formats the
contract names: sequence lengths, a shuffled page pool with a block table,
bf16 or e4m3 queries, e4m3 K/V codes with per-(sequence, kv-head) descales,
or latent records with per-128 block scales. It holds none of the attention
arithmetic. Both sides of a parity check (the HIP path and the CPU oracle)
receive the same bytes from here.

Tensor contract ("mjolnir-kernel 0.1.0 wheel: mjolnir/t5_decode.py", module
docstring; "MiniMax MSA fmha_sm100/cute README", Paged FP8 Decode):
  q           (num_seqs * q_len, h_q, d)     bf16, or e4m3 codes (uint8) + q_descale
  k/v cache   (num_pages, page_size, h_k, d) e4m3 codes (uint8), any strides, d contiguous
  block_table (num_seqs, max_blocks)         int32
  seq_lens    (num_seqs,)                    int32, including the new tokens
  descales    (num_seqs, h_k)                float32

Data recipe (following the t5_decode page's harness, ``run``):
  * seq_lens from the workload's distribution, drawn with numpy PCG64;
  * num_pages = used + max(4, used // 4); pages handed out from a seeded
    random permutation (or in order for ``contiguous_pages``);
  * every byte of a page no sequence references, and every row at or past
    L in a sequence's last page, holds the e4m3 NaN 0x7F, so a stray read
    shows up as NaN; block-table entries past a sequence's last block point
    at such a poisoned page (never out of bounds);
  * Q ~ N(0, 1) rounded to bf16; for e4m3 Q, quantised per (sequence, kv
    head) with descale = max(amax over (q_len, h_r, d), 1e-6) / 448
    (the page's ``quantize_q_fp8``);
  * K, V ~ N(0, 1) quantised per (sequence, kv head): descale = max(amax over
    that sequence's L tokens and d, 1e-6) / 448, codes = e4m3(x / descale)
    (round to nearest even, |x / descale| <= 448 by construction);
  * latent records: 512 latent values ~ N(0, 1) with one scale per token
    and 128-value block, the smallest power of two >= max(amax, 1e-6) / 448
    (so that code x scale is exact in bf16), 64 rope values ~ N(0, 1) in bf16;
  * packed e2m1 (fp4) K/V (the page's narrow KV formats): x ~ N(0, 1) per
    (sequence, kv head) with descale = max(amax, 1e-6) / 6 and the code of
    the nearest e2m1 magnitude (ties to the smaller, as the page's
    ``minifloat_quantize``), packed two per byte, element 2i in the low
    nibble; unused pages and tail rows hold 0x77 (there is no fp4 NaN);
  * packed e2m3 / e3m2 (fp6) K/V, the same list: descale = max(amax, 1e-6) /
    7.5 (e2m3) or / 28 (e3m2), nearest magnitude with ties to the smaller,
    four codes per three bytes (element i at bits 6i .. 6i+5 of the row);
    unused pages and tail rows hold the largest positive code 0x1F;
  * NVFP4 K/V (the page's "nvfp4" and ``nvfp4_quantize``): per (sequence,
    kv head) a global scale gs = max(amax, 1e-12) / (6 * 448); per 16
    head-dim values an e4m3 scale e4m3(min(amax_16 / 6 / gs, 448)); codes =
    nearest e2m1 of x / (scale * gs) (ties to the smaller), packed as fp4;
    the descale passed to the kernel is 8 * gs (the page folds the 2^3 of
    its conversion into it); unused rows hold code 0x77 and scale 0x7E.
Random tensors come from a torch generator on the target device, seeded per
workload, so a GPU batch is generated on the GPU.
"""

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

E4M3_MAX = 448.0
E4M3_NAN = 0x7F
E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)  # codes 0..7
E2M1_FILL = 0x77


def _minifloat_magnitudes(exp_bits, man_bits):
    """Non-negative values of a sign-magnitude minifloat with no inf/NaN
    (OCP MX style), in code order: bias 2^(E-1) - 1, exponent 0 subnormal."""
    bias = (1 << (exp_bits - 1)) - 1
    out = []
    for code in range(1 << (exp_bits + man_bits)):
        e, m = code >> man_bits, code & ((1 << man_bits) - 1)
        frac = m / (1 << man_bits)
        out.append(math.ldexp(frac, 1 - bias) if e == 0 else math.ldexp(1.0 + frac, e - bias))
    return tuple(out)


# magnitudes in code order, sign bit, bits per code, fill byte pattern of a row
NARROW_FORMATS = {
    "e2m1": (E2M1_MAGNITUDES, 0x8, 4, (E2M1_FILL,)),
    "e2m3": (_minifloat_magnitudes(2, 3), 0x20, 6, (0xDF, 0xF7, 0x7D)),  # 0x1F in all four slots
    "e3m2": (_minifloat_magnitudes(3, 2), 0x20, 6, (0xDF, 0xF7, 0x7D)),
}
MLA_LATENT, MLA_ROPE, MLA_BLOCK = 512, 64, 128
MLA_RECORD_BYTES = MLA_LATENT + 2 * MLA_ROPE + 4 * (MLA_LATENT // MLA_BLOCK)  # 656


@dataclass(frozen=True)
class Workload:
    name: str
    num_seqs: int
    q_len: int
    h_q: int
    h_k: int
    d_qk: int
    d_v: int
    page_size: int
    seq_len_dist: tuple  # ("fixed", [..]) | ("uniform", lo, hi) | ("lognormal", median, sigma, lo, hi) | ("mix", ...)
    max_splits: int = 16
    q_format: str = "bf16"  # "bf16" | "e4m3"
    kv_format: str = "e4m3"  # "e4m3" | "mla" | "e2m1" (packed fp4) | "e2m3" / "e3m2" (packed fp6) | "nvfp4"
    causal: bool = True
    seed: int = 1111
    num_pages: int = 0  # 0: used + max(4, used // 4)
    softmax_scale: float = 0.0  # 0: 1 / sqrt(d_qk)
    kv_layout: str = "nhd"  # "nhd" (pages, PS, h_k, d) or "hnd" (pages, 2, h_k, PS, d)
    contiguous_pages: bool = False

    @property
    def h_r(self):
        return self.h_q // self.h_k

    @property
    def rows(self):  # packed query rows per (sequence, kv head)
        return self.q_len * self.h_r

    @property
    def scale(self):
        s = self.softmax_scale or 1.0 / math.sqrt(self.d_qk)
        return float(np.float32(s))


# The five synthetic workloads the decode path is specified on.
WORKLOADS = {
    1: Workload("tiny_gqa_b2_hq8_hk1_ps16", 2, 1, 8, 1, 128, 128, 16, ("fixed", [37, 100]),
                max_splits=1, seed=1112, num_pages=16),
    2: Workload("gqa_b64_hq32_hk8_d128_ps16_L512-8192", 64, 1, 32, 8, 128, 128, 16,
                ("uniform", 512, 8192), max_splits=16, seed=1113),
    3: Workload("specverify_b32_q4_hq64_hk8_d128_ps64_lognormal4096", 32, 4, 64, 8, 128, 128, 64,
                ("lognormal", 4096, 1.0, 256, 32768), max_splits=16, seed=1114),
    4: Workload("fp8_b128_hq64_hk4_d128_ps128_mix1k-4k_32k-64k", 128, 1, 64, 4, 128, 128, 128,
                ("mix", 0.1, (32768, 65536), (1024, 4096)), max_splits=64, q_format="e4m3", seed=1115),
    5: Workload("mla_b32_hq16_hk1_d576-512_ps64_L2k-16k", 32, 1, 16, 1, 576, 512, 64,
                ("uniform", 2048, 16384), max_splits=64, kv_format="mla", seed=1116),
    # the fully-fp8 workload with packed fp4 (e2m1) K/V: the page's narrow KV formats
    6: Workload("fp4kv_b128_hq64_hk4_d128_ps128_mix1k-4k_32k-64k", 128, 1, 64, 4, 128, 128, 128,
                ("mix", 0.1, (32768, 65536), (1024, 4096)), max_splits=64, q_format="e4m3", kv_format="e2m1",
                seed=1115),
    # ... and with packed fp6 K/V (e2m3, the page's harness default narrow format; e3m2)
    7: Workload("fp6e2m3kv_b128_hq64_hk4_d128_ps128_mix1k-4k_32k-64k", 128, 1, 64, 4, 128, 128, 128,
                ("mix", 0.1, (32768, 65536), (1024, 4096)), max_splits=64, q_format="e4m3", kv_format="e2m3",
                seed=1115),
    8: Workload("fp6e3m2kv_b128_hq64_hk4_d128_ps128_mix1k-4k_32k-64k", 128, 1, 64, 4, 128, 128, 128,
                ("mix", 0.1, (32768, 65536), (1024, 4096)), max_splits=64, q_format="e4m3", kv_format="e3m2",
                seed=1115),
    # ... and with NVFP4 K/V (packed e2m1 codes + one e4m3 scale per 16 head-dim values)
    10: Workload("nvfp4kv_b128_hq64_hk4_d128_ps128_mix1k-4k_32k-64k", 128, 1, 64, 4, 128, 128, 128,
                 ("mix", 0.1, (32768, 65536), (1024, 4096)), max_splits=64, q_format="e4m3", kv_format="nvfp4",
                 seed=1115),
}


def workload(index, **overrides):
    """A named workload, optionally with fields replaced (q_len, causal,
    num_seqs, seq_len_dist, kv_layout, ...)."""
    return replace(WORKLOADS[index], **overrides)


def draw_seq_lens(w: Workload) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(w.seed))
    kind = w.seq_len_dist[0]
    b = w.num_seqs
    if kind == "fixed":
        lens = np.asarray(w.seq_len_dist[1], dtype=np.int64)
        assert lens.shape == (b,)
    elif kind == "uniform":
        lens = rng.integers(w.seq_len_dist[1], w.seq_len_dist[2] + 1, size=b)
    elif kind == "lognormal":
        _, median, sigma, lo, hi = w.seq_len_dist
        lens = np.clip(np.rint(np.exp(rng.normal(math.log(median), sigma, size=b))), lo, hi)
    elif kind == "mix":  # a fraction of long sequences at shuffled positions
        _, frac, long_rng, short_rng = w.seq_len_dist
        n_long = int(round(frac * b))
        lens = np.concatenate([rng.integers(long_rng[0], long_rng[1] + 1, size=n_long),
                               rng.integers(short_rng[0], short_rng[1] + 1, size=b - n_long)])
        lens = lens[rng.permutation(b)]
    else:
        raise ValueError(f"unknown length distribution {kind}")
    return lens.astype(np.int32)


@dataclass
class Batch:
    """One synthetic decode batch resident on ``device``."""
    spec: Workload
    seq_lens: torch.Tensor  # (b,) int32
    block_table: torch.Tensor  # (b, max_blocks) int32
    num_pages: int
    q: torch.Tensor  # (b*q_len, h_q, d_qk) bf16, or uint8 e4m3 codes
    q_descale: torch.Tensor  # (b, h_k) float32 (ones for bf16 q)
    k_cache: torch.Tensor = None  # (pages, PS, h_k, d) uint8 logical view
    v_cache: torch.Tensor = None
    k_descale: torch.Tensor = None  # (b, h_k) float32
    v_descale: torch.Tensor = None
    kv_buffer: torch.Tensor = None  # physical storage behind the views
    mla_latent: torch.Tensor = None  # (pages, PS, 1, 512) uint8 view of the records
    mla_rope: torch.Tensor = None  # (pages, PS, 1, 64) bf16 view
    mla_scales: torch.Tensor = None  # (pages, PS, 1, 4) float32 view
    k_scale: torch.Tensor = None  # nvfp4: (pages, PS, h_k, d/16) uint8 e4m3 group scales
    v_scale: torch.Tensor = None
    unused_pages: list = field(default_factory=list)

    @property
    def kv_bytes(self):
        """Bytes of cache the decode must stream: every visible token's K and
        V rows of every kv head (latent records are read once)."""
        toks = int(self.seq_lens.sum())
        w = self.spec
        if w.kv_format == "mla":
            return toks * MLA_RECORD_BYTES
        if w.kv_format in NARROW_FORMATS:
            return toks * w.h_k * (w.d_qk + w.d_v) * NARROW_FORMATS[w.kv_format][2] // 8
        if w.kv_format == "nvfp4":  # codes + one scale byte per 16 values
            return toks * w.h_k * ((w.d_qk + w.d_v) // 2 + (w.d_qk + w.d_v) // 16)
        return toks * w.h_k * (w.d_qk + w.d_v)

    def to_numpy(self):
        """Host copies in the oracle's formats: bf16 as uint16 bit patterns,
        e4m3 as uint8 codes, logical (strided) views kept."""
        def u16(t):
            return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

        out = dict(seq_lens=self.seq_lens.cpu().numpy(), block_table=self.block_table.cpu().numpy())
        out["q"] = u16(self.q) if self.q.dtype == torch.bfloat16 else self.q.cpu().numpy()
        out["q_descale"] = self.q_descale.cpu().numpy()
        if self.spec.kv_format == "mla":
            out["latent"] = self.mla_latent.contiguous().cpu().numpy()
            out["rope"] = u16(self.mla_rope)
            out["scales"] = self.mla_scales.contiguous().cpu().numpy()
        else:
            out["k_cache"] = self.k_cache.contiguous().cpu().numpy()
            out["v_cache"] = self.v_cache.contiguous().cpu().numpy()
            out["k_descale"] = self.k_descale.cpu().numpy()
            out["v_descale"] = self.v_descale.cpu().numpy()
            if self.spec.kv_format == "nvfp4":
                out["k_scale"] = self.k_scale.contiguous().cpu().numpy()
                out["v_scale"] = self.v_scale.contiguous().cpu().numpy()
        return out


def pow2_at_least(x):
    """The smallest power of two >= x, for positive normal float32 x: a
    nonzero mantissa carries into the exponent field and is then cleared."""
    bits = x.float().contiguous().view(torch.int32)
    return ((bits + 0x7FFFFF) & -0x800000).view(torch.float32)


def _page_assignment(w, lens, rng):
    ps = w.page_size
    blocks = [-(-int(L) // ps) for L in lens]
    used = sum(blocks)
    num_pages = w.num_pages or used + max(4, used // 4)
    if num_pages <= used:
        raise ValueError("page pool must hold at least one unused (poisoned) page")
    perm = np.arange(num_pages) if w.contiguous_pages else rng.permutation(num_pages)
    max_blocks = max(1, max(blocks))
    unused = [int(p) for p in perm[used:]]
    bt = np.empty((w.num_seqs, max_blocks), dtype=np.int32)
    cursor = 0
    for b, nb in enumerate(blocks):
        bt[b, :nb] = perm[cursor:cursor + nb]
        bt[b, nb:] = unused[b % len(unused)]  # padding -> a poisoned page
        cursor += nb
    return bt, num_pages, unused


def _token_slots(lens, bt, ps, device):
    """Flat (page * PS + row) slot of every token, sequences concatenated."""
    seg = np.repeat(np.arange(len(lens)), lens)
    pos = np.concatenate([np.arange(L) for L in lens]) if len(lens) else np.zeros(0, np.int64)
    slot = bt[seg, pos // ps].astype(np.int64) * ps + pos % ps
    return torch.from_numpy(seg).to(device), torch.from_numpy(slot).to(device)


def _seq_head_amax(x, seg, num_seqs):
    """Largest |x| of each (sequence, kv head) over its tokens and head dims:
    x (tokens, h_k, d), seg (tokens,) sequence of each token -> (b, h_k)."""
    out = torch.zeros(num_seqs, x.shape[1], device=x.device)
    per_token = x.abs().amax(dim=-1)  # (tokens, h_k)
    return out.scatter_reduce_(0, seg[:, None].expand_as(per_token), per_token, "amax")


def _quantise_per_seq_head(x, seg, num_seqs):
    """x (tokens, h_k, d) float32 -> (codes uint8, descale (b, h_k))."""
    desc = _seq_head_amax(x, seg, num_seqs).clamp(min=1e-6) / E4M3_MAX
    y = (x / desc[seg][:, :, None]).clamp(-E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8), desc.contiguous()


def _nearest_code(y, mags_t, sign_bit):
    """Sign-magnitude code of the magnitude nearest |y| (a tie goes to the
    smaller magnitude), the sign bit set for negative nonzero values. A value
    lies nearest magnitude i exactly when it passes i of the midpoints between
    consecutive magnitudes (and a value on a midpoint passes none of it);
    the midpoints of these dyadic tables are exact in float32."""
    mids = torch.tensor([(a + b) / 2 for a, b in zip(mags_t[:-1], mags_t[1:])], dtype=torch.float32,
                        device=y.device)
    mag = torch.searchsorted(mids, y.abs().contiguous(), right=False)  # midpoints strictly below |y|
    neg = (y < 0) & (mag > 0)
    return mag + neg.to(mag.dtype) * sign_bit


def _pack_codes(code, bits):
    """Pack codes (..., n) of 4 or 6 bits into a little-endian bitstream of
    bytes: code i occupies bits bits*i .. bits*i + bits - 1."""
    per_word = 8 // math.gcd(8, bits)  # codes per whole number of bytes: 2 (fp4) or 4 (fp6)
    nbytes = per_word * bits // 8
    c = code.view(*code.shape[:-1], code.shape[-1] // per_word, per_word)
    word = torch.zeros(c.shape[:-1], dtype=torch.int64, device=code.device)
    for i in range(per_word):
        word |= c[..., i].to(torch.int64) << (bits * i)
    out = [(word >> (8 * k)) & 0xFF for k in range(nbytes)]
    return torch.stack(out, dim=-1).flatten(-2).to(torch.uint8).contiguous()


def _quantise_narrow_per_seq_head(x, seg, num_seqs, kv_format):
    """x (tokens, h_k, d) float32 -> (packed codes uint8 (tokens, h_k, d*bits/8), descale (b, h_k))."""
    mags_t, sign_bit, bits, _ = NARROW_FORMATS[kv_format]
    top = mags_t[-1]
    desc = _seq_head_amax(x, seg, num_seqs).clamp(min=1e-6) / top
    y = (x / desc[seg][:, :, None]).clamp(-top, top)
    return _pack_codes(_nearest_code(y, mags_t, sign_bit), bits), desc.contiguous()


def _quantise_nvfp4_per_seq_head(x, seg, num_seqs):
    """x (tokens, h_k, d) float32 -> (packed codes (tokens, h_k, d/2), e4m3
    group scales (tokens, h_k, d/16) uint8, descale (b, h_k) = 8 * gs)."""
    tokens, h_k, d = x.shape
    gs = _seq_head_amax(x, seg, num_seqs).clamp(min=1e-12) / (6.0 * E4M3_MAX)  # global scale per (seq, head)
    gtok = gs[seg][:, :, None]  # (tokens, h_k, 1)
    groups = x.view(tokens, h_k, d // 16, 16)
    scale = (groups.abs().amax(dim=-1) / 6.0 / gtok).clamp(max=E4M3_MAX).to(torch.float8_e4m3fn)
    step = scale.float() * gtok  # value of one e2m1 unit in each group; 0 for an all-zero group
    live = step > 0
    y = groups / torch.where(live, step, torch.ones_like(step))[..., None] * live[..., None]
    code = _nearest_code(y.view(tokens, h_k, d).clamp(-E2M1_MAGNITUDES[-1], E2M1_MAGNITUDES[-1]),
                         E2M1_MAGNITUDES, 0x8)
    return _pack_codes(code, 4), scale.view(torch.uint8).contiguous(), (gs * 8.0).contiguous()


def _quantise_query_e4m3(q, b, q_len, h_k, h_r, d):
    """bf16 query -> (e4m3 codes, descale (b, h_k)): one descale per
    (sequence, kv head), its largest |q| over the q_len tokens, h_r heads and
    d dims (at least 1e-6) over 448."""
    groups = q.float().view(b, q_len, h_k, h_r, d).permute(0, 2, 1, 3, 4).reshape(b, h_k, -1)
    desc = (groups.abs().amax(dim=-1).clamp(min=1e-6) / E4M3_MAX).contiguous()
    codes = (groups / desc[..., None]).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    codes = codes.view(b, h_k, q_len, h_r, d).permute(0, 2, 1, 3, 4).reshape(b * q_len, h_k * h_r, d)
    return codes.view(torch.uint8).contiguous(), desc


def make_batch(w: Workload, device="cpu", seq_lens=None) -> Batch:
    """Generate the batch of workload ``w`` on ``device``."""
    rng = np.random.Generator(np.random.PCG64(w.seed + 7))
    lens = np.asarray(draw_seq_lens(w) if seq_lens is None else seq_lens, dtype=np.int32)
    assert lens.shape == (w.num_seqs,)
    bt, num_pages, unused = _page_assignment(w, lens, rng)
    gen = torch.Generator(device=device).manual_seed(w.seed)
    ps, b, h_k = w.page_size, w.num_seqs, w.h_k
    seg, slot = _token_slots(lens, bt, ps, device)
    n_tok = int(lens.sum())

    q = torch.randn(b * w.q_len, w.h_q, w.d_qk, generator=gen, device=device).to(torch.bfloat16)
    q_descale = torch.ones(b, h_k, device=device)
    if w.q_format == "e4m3":
        q, q_descale = _quantise_query_e4m3(q, b, w.q_len, h_k, w.h_r, w.d_qk)

    batch = Batch(spec=w, seq_lens=torch.from_numpy(lens).to(device),
                  block_table=torch.from_numpy(bt).to(device), num_pages=num_pages, q=q,
                  q_descale=q_descale, unused_pages=unused)

    if w.kv_format == "mla":
        rec = torch.full((num_pages * ps, MLA_RECORD_BYTES), E4M3_NAN, dtype=torch.uint8, device=device)
        lat = torch.randn(n_tok, MLA_LATENT // MLA_BLOCK, MLA_BLOCK, generator=gen, device=device)
        desc = pow2_at_least(lat.abs().amax(dim=-1).clamp(min=1e-6) / E4M3_MAX)  # (tokens, 4)
        codes = (lat / desc[:, :, None]).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
        rope = torch.randn(n_tok, MLA_ROPE, generator=gen, device=device).to(torch.bfloat16)
        rec[slot, :MLA_LATENT] = codes.view(torch.uint8).view(n_tok, MLA_LATENT)
        rec[slot, MLA_LATENT:MLA_LATENT + 2 * MLA_ROPE] = rope.view(torch.uint8).view(n_tok, 2 * MLA_ROPE)
        rec[slot, MLA_LATENT + 2 * MLA_ROPE:] = desc.float().contiguous().view(torch.uint8).view(n_tok, 16)
        rec = rec.view(num_pages, ps, 1, MLA_RECORD_BYTES)
        batch.kv_buffer = rec
        batch.mla_latent = rec[..., :MLA_LATENT]
        batch.mla_rope = rec[..., MLA_LATENT:MLA_LATENT + 2 * MLA_ROPE].view(torch.bfloat16)
        batch.mla_scales = rec[..., MLA_LATENT + 2 * MLA_ROPE:].view(torch.float32)
        return batch

    d = w.d_qk
    nv = w.kv_format == "nvfp4"
    narrow = w.kv_format in NARROW_FORMATS
    row_bytes = d * NARROW_FORMATS[w.kv_format][2] // 8 if narrow else d // 2 if nv else d
    fill = NARROW_FORMATS[w.kv_format][3] if narrow else (E2M1_FILL,) if nv else (E4M3_NAN,)
    if w.kv_layout == "nhd":
        kbuf = torch.empty((2, num_pages, ps, h_k, row_bytes), dtype=torch.uint8, device=device)
        k_view, v_view = kbuf[0], kbuf[1]
    elif w.kv_layout == "hnd":
        kbuf = torch.empty((num_pages, 2, h_k, ps, row_bytes), dtype=torch.uint8, device=device)
        k_view, v_view = kbuf[:, 0].transpose(1, 2), kbuf[:, 1].transpose(1, 2)
    else:
        raise ValueError(f"unknown kv_layout {w.kv_layout}")
    pat = torch.tensor(fill, dtype=torch.uint8, device=device)
    kbuf.view(-1, len(fill)).copy_(pat.expand(kbuf.numel() // len(fill), -1))
    if nv:  # group scales beside the codes, in the same layout; unused rows hold 448 (0x7E)
        if w.kv_layout == "nhd":
            sbuf = torch.full((2, num_pages, ps, h_k, d // 16), 0x7E, dtype=torch.uint8, device=device)
            scale_views = (sbuf[0], sbuf[1])
        else:
            sbuf = torch.full((num_pages, 2, h_k, ps, d // 16), 0x7E, dtype=torch.uint8, device=device)
            scale_views = (sbuf[:, 0].transpose(1, 2), sbuf[:, 1].transpose(1, 2))
    for view, name in ((k_view, "k"), (v_view, "v")):
        x = torch.randn(n_tok, h_k, d, generator=gen, device=device)
        if nv:
            codes, scl, desc = _quantise_nvfp4_per_seq_head(x, seg, b)
            sv = scale_views[0 if name == "k" else 1]
            sv[slot // ps, slot % ps] = scl
            setattr(batch, f"{name}_scale", sv)
        elif narrow:
            codes, desc = _quantise_narrow_per_seq_head(x, seg, b, w.kv_format)
        else:
            codes, desc = _quantise_per_seq_head(x, seg, b)
        del x
        pages, rows = slot // ps, slot % ps
        view[pages, rows] = codes
        setattr(batch, f"{name}_cache", view)
        setattr(batch, f"{name}_descale", desc)
    batch.kv_buffer = kbuf
    return batch


# ---- sparse slot-list decode ---------------------------------------------------
# Each decode token (one per sequence) attends to the records named by two
# slot lists over two latent-record pools ("vLLM PR #62633", Kernel design):
# the sliding window (the last `window` positions of its sequence, in a pool
# of `page_size[0]`-slot pages) and `topk` compressed records (one per
# `compress_ratio` positions, distinct, drawn at random: a synthetic stand-in
# for the indexer's choice, in a pool of `page_size[1]` = 128 // ratio-slot
# pages). Lists are padded with -1; pages are handed out from a seeded
# permutation, spare pages stay poisoned (e4m3 NaN bytes). Records as for the
# latent workload: 512 values ~ N(0, 1) quantised per 128-value block
# (power-of-two scale >= amax / 448), 64 rope values ~ N(0, 1) in bf16. Sink logits ~ N(0, 1) per
# head. Query ~ N(0, 1) in bf16, one token per sequence.
@dataclass(frozen=True)
class SparseWorkload:
    name: str
    num_tokens: int
    h_q: int
    window: int
    topk: int
    compress_ratio: int
    page_size: tuple
    seq_len_dist: tuple
    sink: bool = True
    seed: int = 1120

    @property
    def scale(self):
        return 1.0 / math.sqrt(MLA_LATENT + MLA_ROPE)


SPARSE_WORKLOADS = {
    # a small decode step of the page's flash configuration: 16 tokens, 16 live
    # heads, a 128-slot window plus 512 compressed slots (ten 64-slot tiles per token)
    9: SparseWorkload("sparse_t16_hq16_win128_top512_ratio4_L4k-64k", 16, 16, 128, 512, 4, (64, 32),
                      ("uniform", 4096, 65536)),
}


def sparse_workload(index, **overrides):
    return replace(SPARSE_WORKLOADS[index], **overrides)


@dataclass
class SparseBatch:
    spec: SparseWorkload
    seq_lens: np.ndarray
    q: torch.Tensor                 # (T, h_q, 576) bf16
    sources: list                   # per list: dict(latent, rope, scales views, slots (T, width) int32, page_size, num_pages)
    sink: torch.Tensor = None       # (h_q,) float32 or None
    kv_buffers: list = field(default_factory=list)

    @property
    def kv_bytes(self):
        """Record bytes the decode must read: every listed (non-negative) slot."""
        return sum(int((s["slots"] >= 0).sum().item()) for s in self.sources) * MLA_RECORD_BYTES

    def to_numpy(self):
        def u16(t):
            return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        out = {"q": u16(self.q), "sink": None if self.sink is None else self.sink.cpu().numpy().astype(np.float64),
               "sources": []}
        for s in self.sources:
            out["sources"].append({"latent": s["latent"].contiguous().cpu().numpy(), "rope": u16(s["rope"]),
                                   "scales": s["scales"].contiguous().cpu().numpy(),
                                   "slots": s["slots"].cpu().numpy()})
        return out


def _latent_pool(gen, pages, ps, device):
    """A record pool of `pages` pages of `ps` slots, every slot filled."""
    n = pages * ps
    rec = torch.empty((n, MLA_RECORD_BYTES), dtype=torch.uint8, device=device)
    lat = torch.randn(n, MLA_LATENT // MLA_BLOCK, MLA_BLOCK, generator=gen, device=device)
    desc = pow2_at_least(lat.abs().amax(dim=-1).clamp(min=1e-6) / E4M3_MAX)
    codes = (lat / desc[:, :, None]).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    rope = torch.randn(n, MLA_ROPE, generator=gen, device=device).to(torch.bfloat16)
    rec[:, :MLA_LATENT] = codes.view(torch.uint8).view(n, MLA_LATENT)
    rec[:, MLA_LATENT:MLA_LATENT + 2 * MLA_ROPE] = rope.view(torch.uint8).view(n, 2 * MLA_ROPE)
    rec[:, MLA_LATENT + 2 * MLA_ROPE:] = desc.float().contiguous().view(torch.uint8).view(n, 16)
    return rec.view(pages, ps, 1, MLA_RECORD_BYTES)


def make_sparse_batch(w: SparseWorkload, device="cpu", seq_lens=None) -> SparseBatch:
    rng = np.random.Generator(np.random.PCG64(w.seed + 7))
    if seq_lens is None:
        lens = draw_seq_lens(replace(WORKLOADS[2], num_seqs=w.num_tokens, seq_len_dist=w.seq_len_dist, seed=w.seed))
    else:
        lens = np.asarray(seq_lens, dtype=np.int32)
    assert lens.shape == (w.num_tokens,)
    gen = torch.Generator(device=device).manual_seed(w.seed)
    T = w.num_tokens
    q = torch.randn(T, w.h_q, MLA_LATENT + MLA_ROPE, generator=gen, device=device).to(torch.bfloat16)
    sources, buffers = [], []
    for which in (0, 1):
        ps = w.page_size[which]
        width = w.window if which == 0 else w.topk
        # positions each token lists: the window's last positions, or distinct compressed records
        picks = []
        for L in lens:
            L = int(L)
            if which == 0:
                picks.append(np.arange(max(0, L - w.window), L))
            else:
                n_c = L // w.compress_ratio
                picks.append(np.sort(rng.choice(n_c, size=min(w.topk, n_c), replace=False)) if n_c else
                             np.zeros(0, np.int64))
        # pages touched per token, handed out from one permutation of the pool
        touched = [np.unique(p // ps) for p in picks]
        used = sum(len(t) for t in touched)
        num_pages = used + max(4, used // 4)
        perm = rng.permutation(num_pages)
        slots = np.full((T, width), -1, dtype=np.int32)
        cursor = 0
        for t, (p, tp) in enumerate(zip(picks, touched)):
            page_of = dict(zip(tp.tolist(), perm[cursor:cursor + len(tp)].tolist()))
            cursor += len(tp)
            slots[t, :len(p)] = [page_of[int(x) // ps] * ps + int(x) % ps for x in p]
        rec = _latent_pool(gen, num_pages, ps, device)
        spare = torch.from_numpy(perm[used:].copy()).to(device)
        rec[spare] = E4M3_NAN  # poisoned, never listed
        buffers.append(rec)
        sources.append({"latent": rec[..., :MLA_LATENT],
                        "rope": rec[..., MLA_LATENT:MLA_LATENT + 2 * MLA_ROPE].view(torch.bfloat16),
                        "scales": rec[..., MLA_LATENT + 2 * MLA_ROPE:].view(torch.float32),
                        "slots": torch.from_numpy(slots).to(device), "page_size": ps, "num_pages": num_pages})
    sink = torch.randn(w.h_q, generator=gen, device=device) if w.sink else None
    return SparseBatch(spec=w, seq_lens=lens, q=q, sources=sources, sink=sink, kv_buffers=buffers)
