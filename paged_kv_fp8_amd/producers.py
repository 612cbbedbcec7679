"""Torch-facing wrappers of the producer entry points (argument marshalling
only): pkv_quantize_q and pkv_write_kv of include/pkv_fp8.h."""

import torch

from . import native


def _ptr(t):
    return t.data_ptr() if t is not None else None


def _stream(stream):
    return (stream or torch.cuda.current_stream()).cuda_stream


def quantize_q(q, num_seqs, q_len, h_k, q8=None, q_descale=None, stream=None):
    """q bf16 [num_seqs * q_len, h_q, d] -> (q8 uint8 same shape, q_descale fp32 [num_seqs, h_k])."""
    if q.dtype != torch.bfloat16 or q.dim() != 3 or not q.is_cuda:
        raise ValueError("q must be a CUDA bf16 tensor [num_seqs * q_len, h_q, d]")
    _, h_q, d = q.shape
    if q.stride(2) != 1:
        raise ValueError("q's last dimension must be contiguous")
    q8 = torch.empty(q.shape, dtype=torch.uint8, device=q.device) if q8 is None else q8
    q_descale = torch.empty(num_seqs, h_k, dtype=torch.float32, device=q.device) if q_descale is None else q_descale
    a = native.QuantQArgs(num_seqs=num_seqs, q_len=q_len, h_q=h_q, h_k=h_k, d=d,
                          q=_ptr(q), q_tok_stride=q.stride(0), q_head_stride=q.stride(1),
                          q8=_ptr(q8), q8_tok_stride=q8.stride(0), q8_head_stride=q8.stride(1),
                          q_descale=_ptr(q_descale), qd_seq_stride=q_descale.stride(0),
                          qd_head_stride=q_descale.stride(1))
    native.quantize_q(a, _stream(stream))
    return q8, q_descale


def write_kv(k_new, v_new, block_table, seq_lens, n_new, k_cache, v_cache, k_descale, v_descale, stream=None):
    """e4m3 cache write. k_new/v_new bf16 [num_seqs * n_new, h_k, d]; caches uint8
    views [pages, page_size, h_k, d] (any strides, d contiguous); descales fp32
    [num_seqs, h_k]."""
    num_seqs = seq_lens.shape[0]
    pages, ps, h_k, d = k_cache.shape
    a = native.KvWriteArgs(num_seqs=num_seqs, n_new=n_new, h_k=h_k, d=d, page_size=ps, num_pages=pages,
                           max_blocks=block_table.shape[1], kv_format=native.PKV_KV_E4M3,
                           k_new=_ptr(k_new), kn_tok_stride=k_new.stride(0), kn_head_stride=k_new.stride(1),
                           v_new=_ptr(v_new), vn_tok_stride=v_new.stride(0), vn_head_stride=v_new.stride(1),
                           block_table=_ptr(block_table), bt_row_stride=block_table.stride(0),
                           seq_lens=_ptr(seq_lens),
                           k_descale=_ptr(k_descale), kd_seq_stride=k_descale.stride(0),
                           kd_head_stride=k_descale.stride(1),
                           v_descale=_ptr(v_descale), vd_seq_stride=v_descale.stride(0),
                           vd_head_stride=v_descale.stride(1),
                           k=_ptr(k_cache), k_page_stride=k_cache.stride(0), k_row_stride=k_cache.stride(1),
                           k_head_stride=k_cache.stride(2),
                           v=_ptr(v_cache), v_page_stride=v_cache.stride(0), v_row_stride=v_cache.stride(1),
                           v_head_stride=v_cache.stride(2))
    native.write_kv(a, _stream(stream))


def write_latent(x_new, block_table, seq_lens, n_new, latent, rope, blk_scale, stream=None):
    """Latent-record write. x_new bf16 [num_seqs * n_new, 576]; latent uint8
    [pages, page_size, 512], rope bf16 bits (uint16 or bf16) [pages, page_size,
    64], blk_scale fp32 [pages, page_size, 4] (any page/row strides)."""
    num_seqs = seq_lens.shape[0]
    pages, ps = latent.shape[0], latent.shape[1]
    a = native.KvWriteArgs(num_seqs=num_seqs, n_new=n_new, h_k=1, d=576, page_size=ps, num_pages=pages,
                           max_blocks=block_table.shape[1], kv_format=native.PKV_KV_MLA,
                           k_new=_ptr(x_new), kn_tok_stride=x_new.stride(0), kn_head_stride=0,
                           block_table=_ptr(block_table), bt_row_stride=block_table.stride(0),
                           seq_lens=_ptr(seq_lens),
                           k=_ptr(latent), k_page_stride=latent.stride(0), k_row_stride=latent.stride(1),
                           k_head_stride=0,
                           k_rope=_ptr(rope), rope_page_stride=rope.stride(0), rope_row_stride=rope.stride(1),
                           k_blk_scale=_ptr(blk_scale), scale_page_stride=blk_scale.stride(0),
                           scale_row_stride=blk_scale.stride(1))
    native.write_kv(a, _stream(stream))
