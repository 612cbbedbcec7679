"""Sparse slot-list decode over latent records (``pkv_sparse_decode``).

A decode step where every token attends to the records its slot lists name
(a sliding-window list and a top-k list of compressed records, each over its
own latent-record pool) plus a per-head attention sink, as the swap-AB
decode of "vLLM PR #62633" (Kernel design) does. This module marshals torch
tensors into ``pkv_sparse_args`` once; ``run()`` enqueues the library's tile
kernel and merge on a stream. Argument marshalling only: every step runs in
the library's HIP kernels.
"""

import torch

from . import native

RECORD_VALUES, ROPE_VALUES = 512, 64


def _ptr(t):
    return None if t is None else t.data_ptr()


class SparseDecode:
    """q: (T, h_q, 576) bf16; lists: up to two dicts with "latent" (pages, PS,
    1, 512) uint8 e4m3, "rope" (pages, PS, 1, 64) bf16, "scales" (pages, PS,
    1, 4) float32 views, "slots" (T, width) int32 (flat page * PS + row, < 0
    = none); list 0 is the sliding window, list 1 the top-k list (both in
    tiles of 64 slots); sink: (h_q,) float32 or None. Allocates O (T, h_q,
    512) bf16, LSE (T, h_q) float32 and the workspace once."""

    def __init__(self, *, q, lists, softmax_scale, sink=None, o_scale=1.0, o=None, lse=None):
        if len(lists) > 2:
            raise ValueError("at most two slot lists (window, top-k)")
        T, h_q = q.shape[0], q.shape[1]
        dev = q.device
        self.q, self.lists, self.sink = q, list(lists), sink
        self.o = o if o is not None else torch.empty(T, h_q, RECORD_VALUES, dtype=torch.bfloat16, device=dev)
        self.lse = lse if lse is not None else torch.empty(T, h_q, dtype=torch.float32, device=dev)
        a = native.SparseArgs()
        a.num_tokens, a.h_q = T, h_q
        a.q, a.q_tok_stride, a.q_head_stride = _ptr(q), q.stride(0), q.stride(1)
        for i, l in enumerate(self.lists):
            d = a.list[i]
            lat, rope, scl, slots = l["latent"], l["rope"], l["scales"], l["slots"]
            d.latent, d.lat_page_stride, d.lat_row_stride = _ptr(lat), lat.stride(0), lat.stride(1)
            d.rope, d.rope_page_stride, d.rope_row_stride = _ptr(rope), rope.stride(0), rope.stride(1)
            d.blk_scale, d.scale_page_stride, d.scale_row_stride = _ptr(scl), scl.stride(0), scl.stride(1)
            d.page_size, d.num_pages = lat.shape[1], lat.shape[0]
            d.slots, d.slots_row_stride, d.width = _ptr(slots), slots.stride(0), slots.shape[1]
        a.sink = _ptr(sink)
        a.softmax_scale, a.o_scale = float(softmax_scale), float(o_scale)
        a.o, a.o_tok_stride, a.o_head_stride = _ptr(self.o), self.o.stride(0), self.o.stride(1)
        a.lse = _ptr(self.lse)
        self.tiles = sum(-(-l["slots"].shape[1] // 64) for l in self.lists)
        ws = native.sparse_workspace_bytes(a)
        if ws == 0 and self.tiles > 0:
            native.sparse_decode(a)  # invalid arguments: raises with the library's reason
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)  # never initialised
        a.workspace, a.workspace_bytes = _ptr(self.workspace), self.workspace.numel()
        self.args = a

    def run(self, stream=None):
        """Enqueue the tile kernel and the merge on `stream` (default: torch's
        current stream). No allocation, no sync."""
        native.sparse_decode(self.args, (stream or torch.cuda.current_stream()).cuda_stream)

    def run_tiles_only(self, stream=None):
        native.sparse_tiles(self.args, (stream or torch.cuda.current_stream()).cuda_stream)

    def run_merge_only(self, stream=None):
        native.sparse_merge(self.args, (stream or torch.cuda.current_stream()).cuda_stream)


def for_batch(batch, **kw):
    """A SparseDecode over a ``workloads.SparseBatch``."""
    return SparseDecode(q=batch.q, lists=batch.sources, softmax_scale=batch.spec.scale, sink=batch.sink, **kw)
