"""Plan-once / run-many wrapper over the C ABI for torch tensors.

Marshalling only: it reads shapes, strides and data pointers from torch
tensors into ``pkv_decode_args``, asks the library for its occupancy facts,
calls the library's host planner, uploads the work list once, allocates the
(uninitialised) split workspace, and then launches the library's kernels on
a stream. The call pattern follows the plan()/run() split of "MiniMax MSA
fmha_sm100/cute README" (Paged FP8 Decode): re-plan only when the batch
shape or the upper bound of the lengths changes.
"""

import numpy as np
import torch

from . import native
from .native import (PKV_KV_E2M1, PKV_KV_E2M3, PKV_KV_E3M2, PKV_KV_E4M3, PKV_KV_MLA, PKV_KV_NVFP4, PKV_Q_BF16,
                     PKV_Q_E4M3)

# K/V code formats by name: ABI value and bits per code
_KV_FORMATS = {"e4m3": PKV_KV_E4M3, "e2m1": PKV_KV_E2M1, "e2m3": PKV_KV_E2M3, "e3m2": PKV_KV_E3M2,
               "nvfp4": PKV_KV_NVFP4}
_KV_BITS = {"e4m3": 8, "e2m1": 4, "e2m3": 6, "e3m2": 6, "nvfp4": 4}


def _ptr(t):
    return None if t is None else t.data_ptr()


def _descale_strides(t, num_seqs, h_k):
    """(seq, head) element strides: one value per tensor, per kv head, or per
    (sequence, kv head)."""
    if t.numel() == 1:
        return 0, 0
    if t.dim() == 1 and t.shape[0] == h_k:
        return 0, t.stride(0)
    if t.dim() == 2 and t.shape == (num_seqs, h_k):
        return t.stride(0), t.stride(1)
    raise ValueError(f"descale shape {tuple(t.shape)} is not 1, ({h_k},) or ({num_seqs}, {h_k})")


class PagedDecode:
    """One decode configuration: tensors bound, split plan made, ready to run.

    q            (num_seqs*q_len, h_q, d) bf16, or uint8 e4m3 codes (then q_descale)
    k_cache/v_cache (num_pages, page_size, h_k, d) uint8 e4m3 views (any strides, d contiguous)
    For the latent-record cache pass ``latent`` (pages, PS, 1, 512) uint8,
    ``rope`` (pages, PS, 1, 64) bf16 and ``blk_scale`` (pages, PS, 1, 4) fp32
    instead of k/v caches and descales.
    o            (num_seqs*q_len, h_q, d_v) bf16 output (any token/head strides)
    lse          (num_seqs, h_k, q_len*h_r) fp32 contiguous output
    plan_seq_lens host lengths the plan is made for (default: seq_lens);
                 the device seq_lens may be shorter at run time.
    plan         "auto" (default): what pkv_plan_pick picks: the one-wave
                 plan, the balanced plan when its items are imbalanced, or
                 the paired plan (four kv heads, one 16-row block; the
                 one-wave plan when no chunk pairs the batch);
                 force_splits / pad_to / min_chunk_tiles keep the one-wave
                 plan. Or "wave", "even", "balanced", "queued", "paired".
    """

    def __init__(self, *, q, block_table, seq_lens, o, lse, q_len, softmax_scale, k_cache=None, v_cache=None,
                 q_descale=None, k_descale=None, v_descale=None, latent=None, rope=None, blk_scale=None,
                 num_pages=None, causal=True, o_scale=1.0, max_splits=16, force_splits=0, min_chunk_tiles=1,
                 pad_to=0, wg_per_cu=None, plan_seq_lens=None, plan="auto", pieces_per_bin=3,
                 dyn_percent=10, plan_cu_count=None, kv_format="e4m3", k_group_scale=None, v_group_scale=None):
        mla = latent is not None
        a = native.DecodeArgs()
        num_seqs = seq_lens.shape[0]
        h_q = q.shape[1]
        if mla:
            h_k, d_qk, d_v, ps = 1, q.shape[2], 512, latent.shape[1]
            num_pages = num_pages or latent.shape[0]
        else:  # e4m3 codes, or packed narrow rows (fp4: d/2 bytes, fp6: 3d/4 bytes)
            bits = _KV_BITS[kv_format]
            h_k, d_qk, d_v, ps = k_cache.shape[2], q.shape[2], v_cache.shape[3] * 8 // bits, k_cache.shape[1]
            num_pages = num_pages or k_cache.shape[0]
        a.num_seqs, a.q_len, a.h_q, a.h_k, a.d_qk, a.d_v = num_seqs, q_len, h_q, h_k, d_qk, d_v
        a.page_size, a.num_pages, a.max_blocks = ps, num_pages, block_table.shape[1]
        a.causal = 1 if causal else 0
        a.q_format = PKV_Q_BF16 if q.dtype == torch.bfloat16 else PKV_Q_E4M3
        a.kv_format = PKV_KV_MLA if mla else _KV_FORMATS[kv_format]
        a.softmax_scale, a.o_scale = float(softmax_scale), float(o_scale)
        a.q, a.q_tok_stride, a.q_head_stride = _ptr(q), q.stride(0), q.stride(1)
        if mla:
            a.k, a.k_page_stride, a.k_row_stride, a.k_head_stride = (_ptr(latent), latent.stride(0),
                                                                     latent.stride(1), latent.stride(2))
            a.v = a.k
            a.k_rope, a.rope_page_stride, a.rope_row_stride = _ptr(rope), rope.stride(0), rope.stride(1)
            a.k_blk_scale, a.scale_page_stride, a.scale_row_stride = (_ptr(blk_scale), blk_scale.stride(0),
                                                                      blk_scale.stride(1))
        else:
            a.k, a.k_page_stride, a.k_row_stride, a.k_head_stride = (_ptr(k_cache), k_cache.stride(0),
                                                                     k_cache.stride(1), k_cache.stride(2))
            a.v, a.v_page_stride, a.v_row_stride, a.v_head_stride = (_ptr(v_cache), v_cache.stride(0),
                                                                     v_cache.stride(1), v_cache.stride(2))
            a.k_descale = _ptr(k_descale)
            a.kd_seq_stride, a.kd_head_stride = _descale_strides(k_descale, num_seqs, h_k)
            a.v_descale = _ptr(v_descale)
            a.vd_seq_stride, a.vd_head_stride = _descale_strides(v_descale, num_seqs, h_k)
            if k_group_scale is not None:  # NVFP4: e4m3 scale per 16 head-dim values
                a.k_group_scale, a.kgs_page_stride, a.kgs_row_stride, a.kgs_head_stride = (
                    _ptr(k_group_scale), k_group_scale.stride(0), k_group_scale.stride(1), k_group_scale.stride(2))
                a.v_group_scale, a.vgs_page_stride, a.vgs_row_stride, a.vgs_head_stride = (
                    _ptr(v_group_scale), v_group_scale.stride(0), v_group_scale.stride(1), v_group_scale.stride(2))
            if q_descale is not None:
                a.q_descale = _ptr(q_descale)
                a.qd_seq_stride, a.qd_head_stride = _descale_strides(q_descale, num_seqs, h_k)
        a.block_table, a.bt_row_stride = _ptr(block_table), block_table.stride(0)
        a.seq_lens = _ptr(seq_lens)
        a.o, a.o_tok_stride, a.o_head_stride = _ptr(o), o.stride(0), o.stride(1)
        a.lse = _ptr(lse)
        a.max_splits = max_splits

        cu, wg, n_q_tiles = native.decode_slots(a)
        cu = plan_cu_count or cu  # a smaller count plans fewer, fuller workgroups (tests)
        self.cu_count, self.wg_per_cu, self.n_q_tiles = cu, wg_per_cu or wg, n_q_tiles
        lens = seq_lens.cpu().numpy() if plan_seq_lens is None else np.asarray(plan_seq_lens)
        dev = q.device
        self.bin_offsets = None
        self.queue = None
        self.imbalance = None
        if plan == "auto":  # the one-wave plan, or the balanced or paired plan (pkv_plan_pick)
            work, n_splits, info = native.plan_split_kv(lens, h_k, n_q_tiles, cu, self.wg_per_cu, max_splits,
                                                        force_splits, min_chunk_tiles, pad_to)
            pick, self.imbalance = native.plan_pick(lens, work, a.kv_format, h_k, q_len * (h_q // h_k))
            wave_knobs = force_splits or pad_to or min_chunk_tiles != 1
            plan = "wave"
            if pick == native.PKV_PLAN_BALANCED and not wave_knobs:
                plan = "balanced"
            elif pick == native.PKV_PLAN_PAIRED and not wave_knobs:
                try:  # no chunk may pair the batch (more sequences than pairs): keep the one-wave plan
                    work, n_splits, info = native.plan_paired(lens, cu, max_splits)
                    plan = "paired"
                except native.PkvError:
                    pass
        if plan == "paired" and self.imbalance is None:  # two items per eight-wave workgroup, one per CU
            work, n_splits, info = native.plan_paired(lens, cu, max_splits)
        if plan == "paired":
            a.work_pairs = 1
        elif plan == "balanced":  # contiguous equal shares, one per resident workgroup
            work, n_splits, offs, info = native.plan_balanced(lens, h_k, n_q_tiles, cu, self.wg_per_cu, max_splits)
            self.bin_offsets = torch.from_numpy(offs).to(dev)
            a.bin_offsets, a.num_bins = _ptr(self.bin_offsets), int(info.num_bins)
        elif plan == "queued":  # persistent workgroups: packed static bins, then a shared queue
            if mla:
                raise ValueError("the queued plan is built for the e4m3 cache only")
            work, n_splits, offs, info = native.plan_queued(lens, h_k, n_q_tiles, cu, self.wg_per_cu, max_splits,
                                                            pieces_per_bin, dyn_percent)
            self.bin_offsets = torch.from_numpy(offs).to(dev)
            a.bin_offsets, a.num_bins = _ptr(self.bin_offsets), int(info.num_bins)
            # taken / retired counters per (kv-head group, q tile): zeroed once, left zero by every call
            self.queue = torch.zeros(2 * h_k * n_q_tiles, dtype=torch.int32, device=dev)
            a.queue = _ptr(self.queue)
        elif plan == "even":  # the same rule at 32-key granularity, equal pieces per sequence (key ranges)
            if mla:
                raise ValueError("the even plan is built for the e4m3 and narrow caches")
            work, n_splits, info = native.plan_even(lens, h_k, n_q_tiles, cu, self.wg_per_cu, max_splits)
            a.work_in_keys = 1
        elif plan == "wave":  # the occupancy-pinned one-wave plan
            if self.imbalance is None:
                work, n_splits, info = native.plan_split_kv(lens, h_k, n_q_tiles, cu, self.wg_per_cu, max_splits,
                                                            force_splits, min_chunk_tiles, pad_to)
        else:
            raise ValueError(f"unknown plan {plan!r}")
        self.work = torch.from_numpy(work).to(dev)
        self.n_splits = torch.from_numpy(n_splits).to(dev)
        self.plan_info = info
        self.plan_work = work
        rows = q_len * (h_q // h_k)
        ws = native.workspace_bytes(num_seqs, h_k, rows, d_v, max_splits) if max_splits > 1 else 0
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)  # never initialised
        a.work, a.num_work = _ptr(self.work), int(info.num_work)
        a.n_splits = _ptr(self.n_splits)
        a.workspace, a.workspace_bytes = _ptr(self.workspace), self.workspace.numel()
        self.args = a
        self.o, self.lse = o, lse
        # keep every bound tensor alive as long as the raw pointers are
        self._keep = (q, k_cache, v_cache, q_descale, k_descale, v_descale, latent, rope, blk_scale, block_table,
                      seq_lens, o, lse, k_group_scale, v_group_scale)
        self.plan = plan

    @property
    def kernel_name(self):
        """The device kernel run() launches for these arguments."""
        return native.decode_kernel_name(self.args)

    @property
    def has_splits(self):
        return self.plan_info.max_n_splits > 1

    def run(self, stream=None):
        """Enqueue decode (+ merge when some sequence was split) on `stream`
        (default: torch's current stream). No allocation, no sync."""
        s = (stream or torch.cuda.current_stream()).cuda_stream
        native.paged_decode_attn(self.args, s)
        if self.has_splits:
            native.merge_splits(self.args, s)

    def run_decode_only(self, stream=None):
        native.paged_decode_attn(self.args, (stream or torch.cuda.current_stream()).cuda_stream)

    def run_merge_only(self, stream=None):
        if self.has_splits:
            native.merge_splits(self.args, (stream or torch.cuda.current_stream()).cuda_stream)


def for_batch(batch, *, o=None, lse=None, **kw):
    """PagedDecode bound to a ``workloads.Batch`` (allocating o and lse if not given)."""
    w = batch.spec
    dev = batch.q.device
    if o is None:
        o = torch.empty(w.num_seqs * w.q_len, w.h_q, w.d_v, dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty(w.num_seqs, w.h_k, w.rows, dtype=torch.float32, device=dev)
    kw.setdefault("max_splits", w.max_splits)
    kw.setdefault("causal", w.causal)
    common = dict(q=batch.q, block_table=batch.block_table, seq_lens=batch.seq_lens, o=o, lse=lse, q_len=w.q_len,
                  softmax_scale=w.scale, num_pages=batch.num_pages)
    if w.kv_format == "mla":
        return PagedDecode(latent=batch.mla_latent, rope=batch.mla_rope, blk_scale=batch.mla_scales, **common, **kw)
    q_descale = batch.q_descale if w.q_format == "e4m3" else None
    kw.setdefault("kv_format", w.kv_format)
    if w.kv_format == "nvfp4":
        kw.setdefault("k_group_scale", batch.k_scale)
        kw.setdefault("v_group_scale", batch.v_scale)
    return PagedDecode(k_cache=batch.k_cache, v_cache=batch.v_cache, q_descale=q_descale, k_descale=batch.k_descale,
                       v_descale=batch.v_descale, **common, **kw)
