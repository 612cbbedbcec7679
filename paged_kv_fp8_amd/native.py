"""ctypes binding of libpkvfp8.so (include/pkv_fp8.h), same entry-point names.

Argument marshalling only: every step of the decode runs in the library's
HIP kernels (or, for the planner, its host C++). Importing this module loads
the library and raises ImportError if it is missing or does not match the
header's struct layout; there is no fallback path.
"""

import ctypes
import os

import numpy as np

# PKV_LIB names another build of the library (the stamped one); default: the in-tree build
LIB_PATH = os.environ.get("PKV_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkvfp8.so")

PKV_OK, PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_CAPACITY, PKV_ERR_WORKSPACE, PKV_ERR_HIP = 0, -1, -2, -3, -4, -5
PKV_Q_BF16, PKV_Q_E4M3 = 0, 1
PKV_KV_E4M3, PKV_KV_MLA, PKV_KV_E2M1, PKV_KV_E2M3, PKV_KV_E3M2, PKV_KV_NVFP4 = 0, 1, 2, 3, 4, 5
PKV_MAX_SPLITS = 256
PKV_NOALLOC_WORKSPACE_BYTES = 64 << 20

# Every function the header declares, in declaration order.
EXPORTS = ("pkv_status_string", "pkv_last_error", "pkv_version", "pkv_decode_args_size", "pkv_plan_split_kv",
           "pkv_plan_even", "pkv_plan_balanced", "pkv_plan_queued", "pkv_workspace_bytes", "pkv_decode_slots", "pkv_paged_decode_attn",
           "pkv_merge_splits", "pkv_quantize_q", "pkv_quant_q_args_size", "pkv_write_kv", "pkv_kv_write_args_size",
           "pkv_decode_kernel_name", "pkv_sparse_workspace_bytes", "pkv_sparse_decode", "pkv_sparse_tiles", "pkv_sparse_merge",
           "pkv_sparse_args_size", "pkv_paged_decode_noalloc", "pkv_stream_read_probe", "pkv_plan_pick",
           "pkv_plan_paired", "pkv_debug_stamps")


class PkvError(RuntimeError):
    def __init__(self, status, where, detail):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({detail})")


class PlanInfo(ctypes.Structure):
    _fields_ = [("num_work", ctypes.c_int32), ("num_real", ctypes.c_int32), ("chunk_tiles", ctypes.c_int32),
                ("slots", ctypes.c_int32), ("max_n_splits", ctypes.c_int32), ("num_bins", ctypes.c_int32),
                ("num_dynamic", ctypes.c_int32)]


_i32, _i64, _f32, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p


class DecodeArgs(ctypes.Structure):
    """Mirror of ``pkv_decode_args`` (field for field, same order)."""
    _fields_ = [
        ("num_seqs", _i32), ("q_len", _i32), ("h_q", _i32), ("h_k", _i32), ("d_qk", _i32), ("d_v", _i32),
        ("page_size", _i32), ("num_pages", _i32), ("max_blocks", _i32),
        ("causal", _i32), ("q_format", _i32), ("kv_format", _i32),
        ("softmax_scale", _f32), ("o_scale", _f32),
        ("q", _vp), ("q_tok_stride", _i64), ("q_head_stride", _i64),
        ("k", _vp), ("k_page_stride", _i64), ("k_row_stride", _i64), ("k_head_stride", _i64),
        ("v", _vp), ("v_page_stride", _i64), ("v_row_stride", _i64), ("v_head_stride", _i64),
        ("k_rope", _vp), ("rope_page_stride", _i64), ("rope_row_stride", _i64),
        ("k_blk_scale", _vp), ("scale_page_stride", _i64), ("scale_row_stride", _i64),
        ("block_table", _vp), ("bt_row_stride", _i64),
        ("seq_lens", _vp),
        ("q_descale", _vp), ("qd_seq_stride", _i64), ("qd_head_stride", _i64),
        ("k_descale", _vp), ("kd_seq_stride", _i64), ("kd_head_stride", _i64),
        ("v_descale", _vp), ("vd_seq_stride", _i64), ("vd_head_stride", _i64),
        ("o", _vp), ("o_tok_stride", _i64), ("o_head_stride", _i64),
        ("lse", _vp),
        ("work", _vp), ("num_work", _i32),
        ("n_splits", _vp), ("max_splits", _i32),
        ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
        ("bin_offsets", _vp), ("num_bins", _i32),
        ("queue", _vp),
        ("k_group_scale", _vp), ("kgs_page_stride", _i64), ("kgs_row_stride", _i64), ("kgs_head_stride", _i64),
        ("v_group_scale", _vp), ("vgs_page_stride", _i64), ("vgs_row_stride", _i64), ("vgs_head_stride", _i64),
        ("work_in_keys", _i32),
        ("work_pairs", _i32),
    ]


class QuantQArgs(ctypes.Structure):
    """pkv_quant_q_args"""
    _fields_ = [("num_seqs", ctypes.c_int32), ("q_len", ctypes.c_int32), ("h_q", ctypes.c_int32),
                ("h_k", ctypes.c_int32), ("d", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("q_tok_stride", ctypes.c_int64), ("q_head_stride", ctypes.c_int64),
                ("q8", ctypes.c_void_p), ("q8_tok_stride", ctypes.c_int64), ("q8_head_stride", ctypes.c_int64),
                ("q_descale", ctypes.c_void_p), ("qd_seq_stride", ctypes.c_int64), ("qd_head_stride", ctypes.c_int64)]


class KvWriteArgs(ctypes.Structure):
    """pkv_kv_write_args"""
    _fields_ = [("num_seqs", ctypes.c_int32), ("n_new", ctypes.c_int32), ("h_k", ctypes.c_int32),
                ("d", ctypes.c_int32), ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("kv_format", ctypes.c_int32),
                ("k_new", ctypes.c_void_p), ("kn_tok_stride", ctypes.c_int64), ("kn_head_stride", ctypes.c_int64),
                ("v_new", ctypes.c_void_p), ("vn_tok_stride", ctypes.c_int64), ("vn_head_stride", ctypes.c_int64),
                ("block_table", ctypes.c_void_p), ("bt_row_stride", ctypes.c_int64),
                ("seq_lens", ctypes.c_void_p),
                ("k_descale", ctypes.c_void_p), ("kd_seq_stride", ctypes.c_int64), ("kd_head_stride", ctypes.c_int64),
                ("v_descale", ctypes.c_void_p), ("vd_seq_stride", ctypes.c_int64), ("vd_head_stride", ctypes.c_int64),
                ("k", ctypes.c_void_p), ("k_page_stride", ctypes.c_int64), ("k_row_stride", ctypes.c_int64),
                ("k_head_stride", ctypes.c_int64),
                ("v", ctypes.c_void_p), ("v_page_stride", ctypes.c_int64), ("v_row_stride", ctypes.c_int64),
                ("v_head_stride", ctypes.c_int64),
                ("k_rope", ctypes.c_void_p), ("rope_page_stride", ctypes.c_int64), ("rope_row_stride", ctypes.c_int64),
                ("k_blk_scale", ctypes.c_void_p), ("scale_page_stride", ctypes.c_int64),
                ("scale_row_stride", ctypes.c_int64)]


class SparseList(ctypes.Structure):
    """Mirror of ``pkv_sparse_list``."""
    _fields_ = [
        ("latent", _vp), ("lat_page_stride", _i64), ("lat_row_stride", _i64),
        ("rope", _vp), ("rope_page_stride", _i64), ("rope_row_stride", _i64),
        ("blk_scale", _vp), ("scale_page_stride", _i64), ("scale_row_stride", _i64),
        ("page_size", _i32), ("num_pages", _i32),
        ("slots", _vp), ("slots_row_stride", _i64),
        ("width", _i32),
    ]


class SparseArgs(ctypes.Structure):
    """Mirror of ``pkv_sparse_args``."""
    _fields_ = [
        ("num_tokens", _i32), ("h_q", _i32),
        ("q", _vp), ("q_tok_stride", _i64), ("q_head_stride", _i64),
        ("list", SparseList * 2),
        ("sink", _vp),
        ("softmax_scale", _f32), ("o_scale", _f32),
        ("o", _vp), ("o_tok_stride", _i64), ("o_head_stride", _i64),
        ("lse", _vp),
        ("workspace", _vp), ("workspace_bytes", _i64),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m paged_kv_fp8_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_status_string.argtypes = [_i32]
    lib.pkv_last_error.restype = ctypes.c_char_p
    lib.pkv_last_error.argtypes = []
    lib.pkv_version.restype = _i32
    lib.pkv_decode_args_size.restype = ctypes.c_size_t
    P = ctypes.POINTER
    lib.pkv_plan_split_kv.restype = _i32
    lib.pkv_plan_split_kv.argtypes = [P(_i32), _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, P(_i32), _i32,
                                      P(_i32), P(PlanInfo)]
    lib.pkv_plan_even.restype = _i32
    lib.pkv_plan_even.argtypes = [P(_i32), _i32, _i32, _i32, _i32, _i32, _i32, P(_i32), _i32, P(_i32), P(PlanInfo)]
    lib.pkv_plan_balanced.restype = _i32
    lib.pkv_plan_balanced.argtypes = [P(_i32), _i32, _i32, _i32, _i32, _i32, _i32, P(_i32), _i32, P(_i32), P(_i32),
                                      _i32, P(PlanInfo)]
    lib.pkv_plan_queued.restype = _i32
    lib.pkv_plan_queued.argtypes = [P(_i32), _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, P(_i32), _i32, P(_i32),
                                    P(_i32), _i32, P(PlanInfo)]
    lib.pkv_plan_pick.restype = _i32
    lib.pkv_plan_pick.argtypes = [P(_i32), _i32, P(_i32), _i32, _i32, _i32, _i32, P(_i32), P(_f32)]
    lib.pkv_plan_paired.restype = _i32
    lib.pkv_plan_paired.argtypes = [P(_i32), _i32, _i32, _i32, P(_i32), _i32, P(_i32), P(PlanInfo)]
    lib.pkv_workspace_bytes.restype = ctypes.c_size_t
    lib.pkv_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32, _i32]
    lib.pkv_decode_kernel_name.restype = ctypes.c_char_p
    lib.pkv_decode_kernel_name.argtypes = [P(DecodeArgs)]
    lib.pkv_decode_slots.restype = _i32
    lib.pkv_decode_slots.argtypes = [P(DecodeArgs), P(_i32), P(_i32), P(_i32)]
    lib.pkv_paged_decode_attn.restype = _i32
    lib.pkv_paged_decode_attn.argtypes = [P(DecodeArgs), _vp]
    lib.pkv_merge_splits.restype = _i32
    lib.pkv_merge_splits.argtypes = [P(DecodeArgs), _vp]
    lib.pkv_quantize_q.restype = _i32
    lib.pkv_quantize_q.argtypes = [P(QuantQArgs), _vp]
    lib.pkv_quant_q_args_size.restype = ctypes.c_size_t
    lib.pkv_write_kv.restype = _i32
    lib.pkv_write_kv.argtypes = [P(KvWriteArgs), _vp]
    lib.pkv_kv_write_args_size.restype = ctypes.c_size_t
    lib.pkv_sparse_workspace_bytes.restype = _i64
    lib.pkv_sparse_workspace_bytes.argtypes = [P(SparseArgs)]
    for name in ("pkv_sparse_decode", "pkv_sparse_tiles", "pkv_sparse_merge"):
        getattr(lib, name).restype = _i32
        getattr(lib, name).argtypes = [P(SparseArgs), _vp]
    lib.pkv_sparse_args_size.restype = ctypes.c_size_t
    lib.pkv_paged_decode_noalloc.restype = _i32
    lib.pkv_paged_decode_noalloc.argtypes = [P(DecodeArgs), _vp]
    lib.pkv_stream_read_probe.restype = _i32
    lib.pkv_stream_read_probe.argtypes = [_vp, ctypes.c_size_t, _i32, _i32, _vp, _vp]
    lib.pkv_debug_stamps.restype = _i32
    lib.pkv_debug_stamps.argtypes = [_i32, _vp]
    for name, st in (("pkv_quant_q_args_size", QuantQArgs), ("pkv_kv_write_args_size", KvWriteArgs),
                     ("pkv_sparse_args_size", SparseArgs)):
        if getattr(lib, name)() != ctypes.sizeof(st):
            raise ImportError(f"{st.__doc__} layout mismatch: library {getattr(lib, name)()} B, "
                              f"binding {ctypes.sizeof(st)} B")
    if lib.pkv_decode_args_size() != ctypes.sizeof(DecodeArgs):
        raise ImportError(f"pkv_decode_args layout mismatch: library {lib.pkv_decode_args_size()} B, "
                          f"binding {ctypes.sizeof(DecodeArgs)} B")
    return lib


lib = _load()


def status_string(status):
    return lib.pkv_status_string(status).decode()


def last_error():
    return lib.pkv_last_error().decode()


def _check(status, where):
    if status != PKV_OK:
        raise PkvError(status, where, last_error())


def version():
    return lib.pkv_version()


def plan_split_kv(seq_lens, h_k, n_q_tiles, cu_count, wg_per_cu=1, max_splits=16, force_splits=0, min_chunk_tiles=1,
                  pad_to=0, work_cap=None):
    """Host planner. Returns (work int32[num_work, 4], n_splits int32[num_seqs], PlanInfo)."""
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    nseq = lens.shape[0]
    if work_cap is None:
        work_cap = max(pad_to, int(max(1, nseq) * max(1, max_splits)))
    work = np.zeros((max(work_cap, 1), 4), dtype=np.int32)
    ns = np.zeros(max(nseq, 1), dtype=np.int32)
    info = PlanInfo()
    P = ctypes.POINTER(_i32)
    st = lib.pkv_plan_split_kv(lens.ctypes.data_as(P), nseq, h_k, n_q_tiles, cu_count, wg_per_cu, max_splits,
                               force_splits, min_chunk_tiles, pad_to, work.ctypes.data_as(P), work_cap,
                               ns.ctypes.data_as(P), ctypes.byref(info))
    _check(st, "pkv_plan_split_kv")
    return work[:info.num_work].copy(), ns[:nseq].copy(), info


PKV_PLAN_WAVE, PKV_PLAN_BALANCED, PKV_PLAN_PAIRED = 0, 1, 2


def plan_pick(seq_lens, work, kv_format, h_k, rows):
    """pkv_plan_pick: (PKV_PLAN_*, imbalance) for a one-wave plan's work list."""
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    wk = np.ascontiguousarray(work, dtype=np.int32).reshape(-1, 4)
    plan, ratio = _i32(0), ctypes.c_float(0.0)
    P = ctypes.POINTER(_i32)
    _check(lib.pkv_plan_pick(lens.ctypes.data_as(P), len(lens), wk.ctypes.data_as(P), wk.shape[0], kv_format, h_k,
                             rows, ctypes.byref(plan), ctypes.byref(ratio)), "pkv_plan_pick")
    return plan.value, ratio.value


def plan_paired(seq_lens, pair_slots, max_splits=16, work_cap=None):
    """pkv_plan_paired: (work int32[num_work, 4] in pairs, n_splits, PlanInfo)."""
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    nseq = lens.shape[0]
    if work_cap is None:
        work_cap = 2 * pair_slots
    work = np.zeros((max(work_cap, 1), 4), dtype=np.int32)
    ns = np.zeros(max(nseq, 1), dtype=np.int32)
    info = PlanInfo()
    P = ctypes.POINTER(_i32)
    _check(lib.pkv_plan_paired(lens.ctypes.data_as(P), nseq, pair_slots, max_splits, work.ctypes.data_as(P), work_cap,
                               ns.ctypes.data_as(P), ctypes.byref(info)), "pkv_plan_paired")
    return work[:info.num_work].copy(), ns[:nseq].copy(), info


def plan_even(seq_lens, h_k, n_q_tiles, cu_count, wg_per_cu=1, max_splits=16):
    """pkv_plan_even: (work (n, 4) int32 in keys, n_splits, PlanInfo)."""
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    cap = int(max(1, -(-int(lens.max(initial=0)) // 32)) * len(lens)) + 1
    work = np.zeros((cap, 4), dtype=np.int32)
    n_splits = np.zeros(len(lens), dtype=np.int32)
    info = PlanInfo()
    P = ctypes.POINTER(_i32)
    _check(lib.pkv_plan_even(lens.ctypes.data_as(P), len(lens), h_k, n_q_tiles, cu_count, wg_per_cu, max_splits,
                             work.ctypes.data_as(P), cap, n_splits.ctypes.data_as(P), ctypes.byref(info)),
           "pkv_plan_even")
    return work[:info.num_work].copy(), n_splits, info


def plan_balanced(seq_lens, h_k, n_q_tiles, cu_count, wg_per_cu=1, max_splits=16):
    """Balanced contiguous plan. Returns (work int32[num_work, 4], n_splits,
    bin_offsets int32[num_bins + 1], PlanInfo)."""
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    nseq = lens.shape[0]
    bins_cap = max(2, int(cu_count) * int(wg_per_cu) + 1)
    work_cap = bins_cap + max(1, nseq)
    work = np.zeros((work_cap, 4), dtype=np.int32)
    ns = np.zeros(max(nseq, 1), dtype=np.int32)
    offs = np.zeros(bins_cap, dtype=np.int32)
    info = PlanInfo()
    P = ctypes.POINTER(_i32)
    st = lib.pkv_plan_balanced(lens.ctypes.data_as(P), nseq, h_k, n_q_tiles, cu_count, wg_per_cu, max_splits,
                               work.ctypes.data_as(P), work_cap, ns.ctypes.data_as(P), offs.ctypes.data_as(P),
                               bins_cap, ctypes.byref(info))
    _check(st, "pkv_plan_balanced")
    return work[:info.num_work].copy(), ns[:nseq].copy(), offs[:info.num_bins + 1].copy(), info


def plan_queued(seq_lens, h_k, n_q_tiles, cu_count, wg_per_cu=1, max_splits=16, pieces_per_bin=3, dyn_percent=10):
    """Queued plan (static bins + shared queue). Returns (work int32[num_work, 4],
    n_splits, bin_offsets int32[num_bins + 1], PlanInfo)."""
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    nseq = lens.shape[0]
    bins_cap = max(2, int(cu_count) * int(wg_per_cu) + 1)
    work_cap = int(max(1, nseq) * max(1, max_splits))
    work = np.zeros((max(work_cap, 1), 4), dtype=np.int32)
    ns = np.zeros(max(nseq, 1), dtype=np.int32)
    offs = np.zeros(bins_cap, dtype=np.int32)
    info = PlanInfo()
    P = ctypes.POINTER(_i32)
    st = lib.pkv_plan_queued(lens.ctypes.data_as(P), nseq, h_k, n_q_tiles, cu_count, wg_per_cu, max_splits,
                             pieces_per_bin, dyn_percent, work.ctypes.data_as(P), work_cap, ns.ctypes.data_as(P),
                             offs.ctypes.data_as(P), bins_cap, ctypes.byref(info))
    _check(st, "pkv_plan_queued")
    return work[:info.num_work].copy(), ns[:nseq].copy(), offs[:info.num_bins + 1].copy(), info


def workspace_bytes(num_seqs, h_k, n_rows, d_v, max_splits):
    return lib.pkv_workspace_bytes(num_seqs, h_k, n_rows, d_v, max_splits)


def decode_slots(args):
    cu, wg, nt = _i32(), _i32(), _i32()
    _check(lib.pkv_decode_slots(ctypes.byref(args), ctypes.byref(cu), ctypes.byref(wg), ctypes.byref(nt)),
           "pkv_decode_slots")
    return cu.value, wg.value, nt.value


def decode_kernel_name(args):
    """Name of the kernel pkv_paged_decode_attn launches for `args`."""
    name = lib.pkv_decode_kernel_name(ctypes.byref(args))
    if name is None:
        raise PkvError(PKV_ERR_INVALID_ARG, "pkv_decode_kernel_name", lib.pkv_last_error().decode())
    return name.decode()


def paged_decode_attn(args, stream=None):
    _check(lib.pkv_paged_decode_attn(ctypes.byref(args), stream), "pkv_paged_decode_attn")


def merge_splits(args, stream=None):
    _check(lib.pkv_merge_splits(ctypes.byref(args), stream), "pkv_merge_splits")


def quantize_q(args, stream=None):
    _check(lib.pkv_quantize_q(ctypes.byref(args), stream), "pkv_quantize_q")


def write_kv(args, stream=None):
    _check(lib.pkv_write_kv(ctypes.byref(args), stream), "pkv_write_kv")


def sparse_workspace_bytes(args):
    return int(lib.pkv_sparse_workspace_bytes(ctypes.byref(args)))


def sparse_decode(args, stream=None):
    _check(lib.pkv_sparse_decode(ctypes.byref(args), stream), "pkv_sparse_decode")


def sparse_tiles(args, stream=None):
    _check(lib.pkv_sparse_tiles(ctypes.byref(args), stream), "pkv_sparse_tiles")


def sparse_merge(args, stream=None):
    _check(lib.pkv_sparse_merge(ctypes.byref(args), stream), "pkv_sparse_merge")


def paged_decode_noalloc(args, stream=None):
    """Decode + merge with the library's own split workspace (args.workspace
    is ignored); allocates nothing."""
    _check(lib.pkv_paged_decode_noalloc(ctypes.byref(args), stream), "pkv_paged_decode_noalloc")


PKV_STAMP_WORDS = 16 * 8 * 48 * 8


def debug_stamps(loop):
    """Stamps of the last launch of `loop` (0 kv-head one-item form, 1 latent
    staged form) as int64[16 workgroups][8 waves][48 steps][8 points]; the
    library must be built with -DPKV_STAMPS=1 (PkvError UNSUPPORTED otherwise)."""
    out = np.zeros(PKV_STAMP_WORDS, dtype=np.uint64)
    _check(lib.pkv_debug_stamps(loop, out.ctypes.data_as(ctypes.c_void_p)), "pkv_debug_stamps")
    return out.astype(np.int64).reshape(16, 8, 48, 8)


def stream_read_probe(src_ptr, nbytes, workgroups, unroll, sink_ptr, stream=None):
    """One launch of the streaming-read probe over ``nbytes`` at device
    address ``src_ptr`` (measurement only)."""
    _check(lib.pkv_stream_read_probe(src_ptr, nbytes, workgroups, unroll, sink_ptr, stream), "pkv_stream_read_probe")
