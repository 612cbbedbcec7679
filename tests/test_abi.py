"""The C-ABI library on a host without a GPU: it loads, exports every
function include/pkv_fp8.h declares, its struct layout matches the binding,
its host planner equals the plan oracle bit for bit, and invalid requests
return the documented error codes before any HIP call."""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle.plan import plan_balanced as oracle_balanced
from oracle.plan import plan_queued as oracle_queued
from oracle.plan import plan_split_kv as oracle_plan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv_fp8.h")


@pytest.fixture(scope="module")
def native():
    from paged_kv_fp8_amd import native as n
    return n


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_exports(native):
    assert declared_functions() == sorted(native.EXPORTS)


def test_library_exports_every_declared_symbol(native):
    for name in declared_functions():
        assert hasattr(native.lib, name), name
        assert ctypes.cast(getattr(native.lib, name), ctypes.c_void_p).value


def test_struct_layout_and_version(native):
    assert native.lib.pkv_decode_args_size() == ctypes.sizeof(native.DecodeArgs)
    assert native.version() >= 100


def test_status_strings(native):
    names = {0: "PKV_OK", -1: "PKV_ERR_INVALID_ARG", -2: "PKV_ERR_UNSUPPORTED", -3: "PKV_ERR_CAPACITY",
             -4: "PKV_ERR_WORKSPACE", -5: "PKV_ERR_HIP", 7: "PKV_ERR_UNKNOWN"}
    for code, name in names.items():
        assert native.status_string(code) == name


@pytest.mark.parametrize("seed", range(60))
def test_library_planner_equals_plan_oracle(native, seed):
    rng = np.random.default_rng(1000 + seed)
    b = int(rng.integers(1, 130))
    kind = seed % 3
    if kind == 0:
        lens = rng.integers(0, 70000, size=b)
    elif kind == 1:
        lens = rng.integers(512, 8193, size=b)
    else:
        lens = np.where(rng.random(b) < 0.1, rng.integers(32768, 65537, size=b), rng.integers(1024, 4097, size=b))
    kw = dict(h_k=int(rng.choice([1, 2, 4, 8])), n_q_tiles=int(rng.integers(1, 3)), cu_count=256,
              wg_per_cu=int(rng.integers(1, 17)), max_splits=int(rng.choice([1, 4, 16, 64, 256])),
              force_splits=int(rng.choice([0, 0, 0, 3])), min_chunk_tiles=int(rng.choice([1, 1, 2])))
    work, ns, chunk, slots = oracle_plan(lens.tolist(), **kw)
    pad = int(rng.choice([0, len(work) + int(rng.integers(0, 9))]))
    if pad:
        work, ns, chunk, slots = oracle_plan(lens.tolist(), pad_to=pad, **kw)
    w2, ns2, info = native.plan_split_kv(lens, kw["h_k"], kw["n_q_tiles"], kw["cu_count"], kw["wg_per_cu"],
                                         kw["max_splits"], kw["force_splits"], kw["min_chunk_tiles"], pad)
    assert w2.tolist() == [list(x) for x in work]
    assert ns2.tolist() == ns
    assert (info.chunk_tiles, info.slots, info.num_work) == (chunk, slots, len(work))
    assert info.num_real == sum(1 for x in work if x[2] > x[1])
    assert info.max_n_splits == max(ns)


def test_planner_errors(native):
    PkvError = native.PkvError
    cases = [
        (dict(seq_lens=[]), -1),
        (dict(seq_lens=[10, -1]), -1),
        (dict(seq_lens=[10], h_k=0), -1),
        (dict(seq_lens=[10], max_splits=257), -2),
        (dict(seq_lens=[1000] * 4, pad_to=2), -3),
        (dict(seq_lens=[1000] * 4, work_cap=2), -3),
    ]
    for kw, code in cases:
        args = dict(h_k=1, n_q_tiles=1, cu_count=256, wg_per_cu=1, max_splits=16)
        args.update(kw)
        lens = args.pop("seq_lens")
        with pytest.raises(PkvError) as e:
            native.plan_split_kv(lens, **args)
        assert e.value.status == code, (kw, native.last_error())
        assert native.last_error()


def _valid_args(native, **over):
    """A well-formed argument block with fake (never dereferenced) aligned
    addresses: only invalid variants of it are ever passed to the library."""
    a = native.DecodeArgs()
    a.num_seqs, a.q_len, a.h_q, a.h_k, a.d_qk, a.d_v = 2, 1, 8, 1, 128, 128
    a.page_size, a.num_pages, a.max_blocks = 16, 16, 7
    a.causal, a.q_format, a.kv_format = 1, native.PKV_Q_BF16, native.PKV_KV_E4M3
    a.softmax_scale, a.o_scale = 0.088, 1.0
    base = 1 << 40
    a.q, a.q_tok_stride, a.q_head_stride = base, 8 * 128, 128
    a.k, a.k_page_stride, a.k_row_stride, a.k_head_stride = base + (1 << 30), 16 * 128, 128, 128
    a.v, a.v_page_stride, a.v_row_stride, a.v_head_stride = base + (2 << 30), 16 * 128, 128, 128
    a.block_table, a.bt_row_stride, a.seq_lens = base + (3 << 30), 7, base + (3 << 30) + 4096
    a.k_descale, a.v_descale = base + (4 << 30), base + (4 << 30) + 256
    a.o, a.o_tok_stride, a.o_head_stride = base + (5 << 30), 8 * 128, 128
    a.lse = base + (6 << 30)
    a.work, a.num_work, a.n_splits, a.max_splits = base + (7 << 30), 2, base + (7 << 30) + 4096, 1
    for k, v in over.items():
        setattr(a, k, v)
    return a


BAD = [
    (dict(h_q=6, h_k=4), -1),
    (dict(num_seqs=0), -1),
    (dict(page_size=48), -2),
    (dict(page_size=8), -2),
    (dict(d_qk=64, d_v=64), -2),
    (dict(q_format=5), -1),
    (dict(kv_format=9), -1),
    (dict(max_splits=0), -1),
    (dict(max_splits=300), -1),
    (dict(softmax_scale=float("inf")), -1),
    (dict(q=None), -1),
    (dict(o=None), -1),
    (dict(work=None), -1),
    (dict(num_work=0), -1),
    (dict(q=(1 << 40) + 8), -1),
    (dict(k_row_stride=100), -1),
    (dict(v_page_stride=-16), -1),
    (dict(o_tok_stride=12), -1),
    (dict(bt_row_stride=3), -1),
    (dict(k_descale=None), -1),
    (dict(q_format=1, q_descale=None), -1),
    (dict(max_splits=4), -4),
    (dict(max_splits=4, workspace=1 << 41, workspace_bytes=100), -4),
    (dict(kv_format=1, h_k=2, h_q=8, d_qk=576, d_v=512), -2),
    (dict(kv_format=1, h_k=1, h_q=16, d_qk=576, d_v=512, q_format=1, q_descale=1 << 42), -2),
    (dict(kv_format=1, h_k=1, h_q=16, q_len=17, d_qk=576, d_v=512), -2),
    (dict(kv_format=1, h_k=1, h_q=16, d_qk=512, d_v=512), -2),
    (dict(kv_format=1, h_k=1, h_q=16, d_qk=576, d_v=512), -1),  # v differs from k
    (dict(kv_format=1, h_k=1, h_q=16, d_qk=576, d_v=512, v=None), -1),  # no rope / scales
    (dict(kv_format=2), -2),  # packed fp4 / fp6 caches need the e4m3 query
    (dict(kv_format=3), -2),
    (dict(kv_format=4, q_format=1, q_descale=1 << 42, d_qk=64, d_v=64), -2),
    (dict(kv_format=3, q_format=1, q_descale=1 << 42, bin_offsets=1 << 43, num_bins=4), -2),  # one-wave plan only
    (dict(kv_format=5), -2),  # NVFP4 needs the e4m3 query
    (dict(kv_format=5, q_format=1, q_descale=1 << 42), -1),  # ... and its group scales
    (dict(kv_format=5, q_format=1, q_descale=1 << 42, k_group_scale=1 << 43, v_group_scale=1 << 44,
          kgs_row_stride=4), -1),
    (dict(kv_format=6), -1),
    (dict(k_page_stride=1 << 32), -2),  # page offsets are 32 x 32-bit products
    (dict(v_page_stride=(1 << 32) + 2048), -2),
]


@pytest.mark.parametrize("over,code", BAD)
def test_decode_rejects_invalid_arguments_without_touching_the_gpu(native, over, code):
    a = _valid_args(native, **over)
    for fn in (native.lib.pkv_paged_decode_attn,):
        st = fn(ctypes.byref(a), None)
        assert st == code, (over, native.status_string(st), native.last_error())
        assert native.last_error()


@pytest.mark.parametrize("over,code", [b for b in BAD if b[1] != -4])
def test_noalloc_decode_rejects_invalid_arguments_without_touching_the_gpu(native, over, code):
    st = native.lib.pkv_paged_decode_noalloc(ctypes.byref(_valid_args(native, **over)), None)
    assert st == code, (over, native.status_string(st), native.last_error())


def test_noalloc_decode_limits(native):
    big = _valid_args(native, num_seqs=64, h_q=32, h_k=8, max_splits=256)
    need = native.workspace_bytes(64, 8, 4, 128, 256)
    assert need > native.PKV_NOALLOC_WORKSPACE_BYTES
    assert native.lib.pkv_paged_decode_noalloc(ctypes.byref(big), None) == native.PKV_ERR_WORKSPACE
    assert "workspace" in native.last_error()
    a = _valid_args(native, max_splits=4, queue=1 << 43, bin_offsets=1 << 44, num_bins=4)
    assert native.lib.pkv_paged_decode_noalloc(ctypes.byref(a), None) == native.PKV_ERR_UNSUPPORTED
    assert native.lib.pkv_paged_decode_noalloc(None, None) == native.PKV_ERR_INVALID_ARG


def test_decode_kernel_name_follows_the_shapes(native):
    assert native.decode_kernel_name(_valid_args(native)) == "gqa_decode_kernel"
    mla = dict(kv_format=1, h_k=1, h_q=16, d_qk=576, d_v=512)
    # fewer than 64 query rows per sequence: the pair form; 64 and more: the staged form
    for q_len, name in ((1, "mla_pair_kernel"), (3, "mla_pair_kernel"), (4, "mla_lds_kernel"), (16, "mla_lds_kernel")):
        assert native.decode_kernel_name(_valid_args(native, q_len=q_len, **mla)) == name, q_len
    assert native.decode_kernel_name(_valid_args(native, q_len=8, **{**mla, "h_q": 8})) == "mla_lds_kernel"
    assert native.decode_kernel_name(_valid_args(native, q_len=4, **{**mla, "h_q": 8})) == "mla_pair_kernel"
    with pytest.raises(native.PkvError):
        native.decode_kernel_name(_valid_args(native, h_q=6, h_k=4))
    assert native.lib.pkv_decode_kernel_name(None) is None
    for fmt in (native.PKV_KV_E2M1, native.PKV_KV_E2M3, native.PKV_KV_E3M2, native.PKV_KV_NVFP4):
        narrow = _valid_args(native, kv_format=fmt, q_format=native.PKV_Q_E4M3, q_descale=1 << 42)
        assert native.decode_kernel_name(narrow) == "gqa_decode_kernel", fmt


def test_merge_validates_and_is_a_noop_without_splits(native):
    a = _valid_args(native)
    assert native.lib.pkv_merge_splits(ctypes.byref(a), None) == 0  # max_splits == 1: nothing launched
    a = _valid_args(native, max_splits=8)
    assert native.lib.pkv_merge_splits(ctypes.byref(a), None) == -4
    assert native.lib.pkv_merge_splits(None, None) == -1


def test_workspace_bytes_formula(native):
    n = native.workspace_bytes(64, 8, 4, 128, 16)
    floats = 16 * 64 * 8 * 4 * (128 + 2)
    assert n == (floats * 4 + 255) // 256 * 256
    assert native.workspace_bytes(0, 8, 4, 128, 16) == 0


@pytest.mark.parametrize("seed", range(40))
def test_library_balanced_planner_equals_oracle(native, seed):
    rng = np.random.default_rng(3000 + seed)
    b = int(rng.integers(1, 130))
    lens = np.where(rng.random(b) < 0.15, rng.integers(8192, 70000, size=b), rng.integers(0, 5000, size=b))
    kw = dict(h_k=int(rng.choice([1, 2, 4, 8])), n_q_tiles=int(rng.integers(1, 3)), cu_count=256,
              wg_per_cu=int(rng.integers(1, 9)), max_splits=int(rng.choice([2, 8, 16, 64, 256])))
    work, ns, offs, bins = oracle_balanced(lens.tolist(), **kw)
    w2, ns2, offs2, info = native.plan_balanced(lens, kw["h_k"], kw["n_q_tiles"], kw["cu_count"], kw["wg_per_cu"],
                                                kw["max_splits"])
    assert w2.tolist() == [list(x) for x in work]
    assert ns2.tolist() == ns and offs2.tolist() == offs
    assert (info.num_bins, info.num_work, info.max_n_splits) == (bins, len(work), max(ns))


@pytest.mark.parametrize("seed", range(40))
def test_library_even_planner_equals_oracle(native, seed):
    from oracle.plan import plan_even
    rng = np.random.default_rng(5000 + seed)
    b = int(rng.integers(1, 130))
    lens = np.where(rng.random(b) < 0.15, rng.integers(8192, 70000, size=b), rng.integers(0, 5000, size=b))
    kw = dict(h_k=int(rng.choice([1, 2, 4, 8])), n_q_tiles=int(rng.integers(1, 3)), cu_count=256,
              wg_per_cu=int(rng.integers(1, 9)), max_splits=int(rng.choice([1, 2, 8, 16, 64, 256])))
    work, ns, c, slots = plan_even(lens.tolist(), **kw)
    w2, ns2, info = native.plan_even(lens, kw["h_k"], kw["n_q_tiles"], kw["cu_count"], kw["wg_per_cu"],
                                     kw["max_splits"])
    assert w2.tolist() == [list(x) for x in work]
    assert ns2.tolist() == ns
    assert (info.chunk_tiles, info.slots, info.num_work, info.max_n_splits) == (c, slots, len(work), max(ns))


@pytest.mark.parametrize("seed", range(60))
def test_library_paired_planner_equals_oracle(native, seed):
    from oracle.plan import plan_paired
    rng = np.random.default_rng(6000 + seed)
    b = int(rng.integers(1, 200))
    lens = np.where(rng.random(b) < 0.15, rng.integers(8192, 70000, size=b), rng.integers(0, 5000, size=b))
    pair_slots = int(rng.choice([8, 64, 128, 256]))
    max_splits = int(rng.choice([1, 2, 8, 16, 64, 256]))
    try:
        work, ns, c = plan_paired(lens.tolist(), pair_slots, max_splits)
    except ValueError:
        with pytest.raises(native.PkvError) as e:
            native.plan_paired(lens, pair_slots, max_splits)
        assert e.value.status == native.PKV_ERR_UNSUPPORTED
        return
    w2, ns2, info = native.plan_paired(lens, pair_slots, max_splits)
    assert w2.tolist() == [list(x) for x in work]
    assert ns2.tolist() == ns
    assert (info.chunk_tiles, info.num_work, info.num_real, info.slots, info.max_n_splits) == (
        c, len(work), sum(1 for x in work if x[2] > x[1]), 2 * pair_slots, max(ns))


def test_paired_planner_errors(native):
    lens = np.array([100, 200], dtype=np.int32)
    for args in ((lens, 0), (np.array([-5], dtype=np.int32), 4), (lens, 4, 0)):
        with pytest.raises(native.PkvError) as e:
            native.plan_paired(*args)
        assert e.value.status == native.PKV_ERR_INVALID_ARG
    with pytest.raises(native.PkvError) as e:
        native.plan_paired(lens, 4, native.PKV_MAX_SPLITS + 1)
    assert e.value.status == native.PKV_ERR_UNSUPPORTED
    with pytest.raises(native.PkvError) as e:  # five one-tile sequences never fit two pairs
        native.plan_paired(np.full(5, 128, np.int32), 2)
    assert e.value.status == native.PKV_ERR_UNSUPPORTED
    with pytest.raises(native.PkvError) as e:  # the work array is too small for the pairs
        native.plan_paired(lens, 4, work_cap=1)
    assert e.value.status == native.PKV_ERR_CAPACITY


def test_even_planner_errors(native):
    lens = np.array([100, 200], dtype=np.int32)
    with pytest.raises(native.PkvError):
        native.plan_even(lens, 0, 1, 256)
    with pytest.raises(native.PkvError):
        native.plan_even(np.array([-5], dtype=np.int32), 1, 1, 256)
    with pytest.raises(native.PkvError):
        native.plan_even(lens, 1, 1, 256, max_splits=native.PKV_MAX_SPLITS + 1)


def test_decode_rejects_bad_work_units(native):
    for over, code in ((dict(work_in_keys=2), -1), (dict(work_in_keys=1, kv_format=1, h_k=1, h_q=16, d_qk=576,
                                                             d_v=512, v=None), -2)):
        st = native.lib.pkv_paged_decode_attn(ctypes.byref(_valid_args(native, **over)), None)
        assert st == code, (over, native.last_error())


@pytest.mark.parametrize("seed", range(30))
def test_library_queued_planner_equals_oracle(native, seed):
    rng = np.random.default_rng(4000 + seed)
    b = int(rng.integers(1, 130))
    lens = np.where(rng.random(b) < 0.15, rng.integers(8192, 70000, size=b), rng.integers(0, 5000, size=b))
    kw = dict(h_k=int(rng.choice([1, 2, 4, 8])), n_q_tiles=int(rng.integers(1, 3)), cu_count=256,
              wg_per_cu=int(rng.integers(1, 9)), max_splits=int(rng.choice([2, 8, 16, 64, 256])),
              pieces_per_bin=int(rng.integers(1, 5)), dyn_percent=int(rng.integers(0, 60)))
    work, ns, offs, bins, nq = oracle_queued(lens.tolist(), **kw)
    w2, ns2, offs2, info = native.plan_queued(lens, kw["h_k"], kw["n_q_tiles"], kw["cu_count"], kw["wg_per_cu"],
                                              kw["max_splits"], kw["pieces_per_bin"], kw["dyn_percent"])
    assert w2.tolist() == [list(x) for x in work]
    assert ns2.tolist() == ns and offs2.tolist() == offs
    assert (info.num_bins, info.num_work, info.max_n_splits, info.num_dynamic) == (bins, len(work), max(ns), nq)


def test_queued_planner_errors(native):
    lens = np.array([100, 200], dtype=np.int32)
    for over, code in (({"pieces_per_bin": 0}, native.PKV_ERR_INVALID_ARG),
                       ({"dyn_percent": -1}, native.PKV_ERR_INVALID_ARG),
                       ({"dyn_percent": 91}, native.PKV_ERR_INVALID_ARG),
                       ({"max_splits": native.PKV_MAX_SPLITS + 1}, native.PKV_ERR_UNSUPPORTED)):
        args = dict(h_k=1, n_q_tiles=1, cu_count=4, wg_per_cu=1, max_splits=4, pieces_per_bin=2, dyn_percent=10)
        args.update(over)
        with pytest.raises(native.PkvError) as e:
            native.plan_queued(lens, **args)
        assert e.value.status == code


def test_queued_plan_needs_bin_offsets_and_the_e4m3_cache(native):
    a = _valid_args(native)
    a.queue = 1 << 41
    assert native.lib.pkv_paged_decode_attn(ctypes.byref(a), None) == native.PKV_ERR_INVALID_ARG


# ---------------------------------------------------------------------------
# producers: argument checks run before any HIP call
# ---------------------------------------------------------------------------
def _quant_args(native, **over):
    base = 1 << 40
    a = native.QuantQArgs(num_seqs=2, q_len=1, h_q=8, h_k=2, d=128, q=base, q_tok_stride=8 * 128,
                          q_head_stride=128, q8=base + (1 << 30), q8_tok_stride=8 * 128, q8_head_stride=128,
                          q_descale=base + (2 << 30), qd_seq_stride=2, qd_head_stride=1)
    for k, v in over.items():
        setattr(a, k, v)
    return a


def _write_args(native, **over):
    base = 1 << 40
    a = native.KvWriteArgs(num_seqs=2, n_new=1, h_k=2, d=128, page_size=16, num_pages=8, max_blocks=4,
                           kv_format=native.PKV_KV_E4M3, k_new=base, kn_tok_stride=256, kn_head_stride=128,
                           v_new=base + (1 << 30), vn_tok_stride=256, vn_head_stride=128,
                           block_table=base + (2 << 30), bt_row_stride=4, seq_lens=base + (2 << 30) + 4096,
                           k_descale=base + (3 << 30), kd_seq_stride=2, kd_head_stride=1,
                           v_descale=base + (3 << 30) + 256, vd_seq_stride=2, vd_head_stride=1,
                           k=base + (4 << 30), k_page_stride=16 * 256, k_row_stride=256, k_head_stride=128,
                           v=base + (5 << 30), v_page_stride=16 * 256, v_row_stride=256, v_head_stride=128)
    for k, v in over.items():
        setattr(a, k, v)
    return a


LAT = dict(kv_format=1, h_k=1, d=576, kn_tok_stride=576, kn_head_stride=0, v_new=None, v=None, k_descale=None,
           v_descale=None, k_page_stride=16 * 512, k_row_stride=512, k_head_stride=0, k_rope=(1 << 40) + (6 << 30),
           rope_page_stride=16 * 64, rope_row_stride=64, k_blk_scale=(1 << 40) + (7 << 30), scale_page_stride=64,
           scale_row_stride=4)

BAD_QUANT = [
    (dict(num_seqs=0), -1), (dict(h_q=6, h_k=4), -1), (dict(d=100), -1), (dict(d=4), -1), (dict(q=None), -1),
    (dict(q8=None), -1), (dict(q_descale=None), -1), (dict(q=(1 << 40) + 8), -1), (dict(q_tok_stride=100), -1),
    (dict(q8=(1 << 40) + (1 << 30) + 4), -1), (dict(q8_head_stride=12), -1), (dict(qd_seq_stride=-1), -1),
]

BAD_WRITE = [
    (dict(num_seqs=0), -1), (dict(n_new=0), -1), (dict(page_size=24), -2), (dict(kv_format=4), -2),
    (dict(k_new=None), -1), (dict(block_table=None), -1), (dict(seq_lens=None), -1), (dict(bt_row_stride=2), -1),
    (dict(k_new=(1 << 40) + 8), -1), (dict(kn_head_stride=100), -1), (dict(k_row_stride=100), -1),
    (dict(v=None), -1), (dict(v_descale=None), -1), (dict(vd_head_stride=-2), -1), (dict(d=100), -1),
    (dict(LAT, h_k=2), -1), (dict(LAT, d=512), -1), (dict(LAT, k_rope=None), -1), (dict(LAT, k_blk_scale=None), -1),
    (dict(LAT, k_rope=(1 << 40) + (6 << 30) + 2), -1),
]


@pytest.mark.parametrize("over,code", BAD_QUANT)
def test_quantize_q_rejects_invalid_arguments(native, over, code):
    st = native.lib.pkv_quantize_q(ctypes.byref(_quant_args(native, **over)), None)
    assert st == code, (over, native.status_string(st), native.last_error())
    assert native.last_error()


@pytest.mark.parametrize("over,code", BAD_WRITE)
def test_write_kv_rejects_invalid_arguments(native, over, code):
    st = native.lib.pkv_write_kv(ctypes.byref(_write_args(native, **over)), None)
    assert st == code, (over, native.status_string(st), native.last_error())
    assert native.last_error()


def test_producers_reject_null_args(native):
    assert native.lib.pkv_quantize_q(None, None) == -1
    assert native.lib.pkv_write_kv(None, None) == -1


def _sparse_args(native, **over):
    """A well-formed sparse argument block with fake (never dereferenced)
    aligned addresses; list fields are set with keys "l0_<field>" / "l1_<field>"."""
    a = native.SparseArgs()
    base = 1 << 40
    a.num_tokens, a.h_q = 4, 16
    a.q, a.q_tok_stride, a.q_head_stride = base, 16 * 576, 576
    for i, width in ((0, 128), (1, 512)):
        l = a.list[i]
        off = base + ((i + 1) << 32)
        l.latent, l.lat_page_stride, l.lat_row_stride = off, 64 * 656, 656
        l.rope, l.rope_page_stride, l.rope_row_stride = off + 512, 64 * 328, 328
        l.blk_scale, l.scale_page_stride, l.scale_row_stride = off + 640, 64 * 164, 164
        l.page_size, l.num_pages = 64, 100
        l.slots, l.slots_row_stride, l.width = off + (1 << 31), width, width
    a.sink = base + (3 << 32)
    a.softmax_scale, a.o_scale = 0.04, 1.0
    a.o, a.o_tok_stride, a.o_head_stride = base + (4 << 32), 16 * 512, 512
    a.lse = base + (5 << 32)
    a.workspace = base + (6 << 32)
    for k, v in over.items():
        if k.startswith("l0_") or k.startswith("l1_"):
            setattr(a.list[int(k[1])], k[3:], v)
        else:
            setattr(a, k, v)
    a.workspace_bytes = over.get("workspace_bytes", native.sparse_workspace_bytes(a) or 1)
    return a


def test_sparse_workspace_formula(native):
    a = _sparse_args(native)
    tiles = 128 // 64 + 512 // 64
    assert native.sparse_workspace_bytes(a) == tiles * 4 * 16 * (512 + 2) * 4
    a = _sparse_args(native, l0_width=65, l1_width=0)
    assert native.sparse_workspace_bytes(a) == 2 * 4 * 16 * 514 * 4
    assert native.sparse_workspace_bytes(_sparse_args(native, h_q=24)) == 0  # invalid: 0


SPARSE_BAD = [
    (dict(num_tokens=0), -1), (dict(num_tokens=70000), -2), (dict(h_q=24), -2), (dict(h_q=144), -2), (dict(q=None), -1),
    (dict(q=(1 << 40) + 8), -1), (dict(o_head_stride=510), -1), (dict(lse=None), -1), (dict(sink=(1 << 40) + 2), -1),
    (dict(softmax_scale=float("nan")), -1), (dict(l0_width=-1), -1), (dict(l1_width=5000), -2),
    (dict(l0_page_size=48), -2), (dict(l1_num_pages=0), -1), (dict(l0_slots=None), -1),
    (dict(l1_latent=(1 << 40) + (2 << 32) + 8), -1), (dict(l0_lat_row_stride=650), -1),
    (dict(l1_scale_row_stride=163), -1), (dict(l0_slots_row_stride=100), -1),
    (dict(workspace=None), -4), (dict(workspace_bytes=64), -4),
]


@pytest.mark.parametrize("over,code", SPARSE_BAD)
def test_sparse_decode_rejects_invalid_arguments_without_touching_the_gpu(native, over, code):
    for fn in (native.lib.pkv_sparse_decode, native.lib.pkv_sparse_tiles, native.lib.pkv_sparse_merge):
        st = fn(ctypes.byref(_sparse_args(native, **over)), None)
        assert st == code, (over, native.status_string(st), native.last_error())
        assert native.last_error()


def test_sparse_null_args(native):
    assert native.lib.pkv_sparse_decode(None, None) == native.PKV_ERR_INVALID_ARG
    assert native.lib.pkv_sparse_workspace_bytes(None) == 0


@pytest.mark.parametrize("src,nbytes,wg,unroll,sink", [
    (None, 4096 * 8, 64, 8, 256), (256, 4096 * 8, 64, 8, None),   # NULL pointers
    (264, 4096 * 8, 64, 8, 256), (256, 4096 * 8, 64, 8, 258),     # misaligned
    (256, 4096 * 8, 64, 6, 256), (256, 4096 * 8, 0, 8, 256),      # unroll, workgroups
    (256, 4096 * 8 + 16, 64, 8, 256), (256, 0, 64, 8, 256)])      # size not a whole number of chunks
def test_stream_read_probe_rejects_invalid_arguments_without_touching_the_gpu(native, src, nbytes, wg, unroll, sink):
    # fake (never dereferenced) addresses: every check runs before any HIP call
    st = native.lib.pkv_stream_read_probe(src, nbytes, wg, unroll, sink, None)
    assert st == native.PKV_ERR_INVALID_ARG, native.last_error()
    assert native.last_error()


def test_debug_stamps_normal_build_and_argument_errors(native):
    # the in-tree library is the normal build: no stamps; arguments are
    # checked first, and no HIP call is made on any of these paths
    buf = np.zeros(native.PKV_STAMP_WORDS, dtype=np.uint64)
    ptr = buf.ctypes.data_as(ctypes.c_void_p)
    assert native.lib.pkv_debug_stamps(0, ptr) == native.PKV_ERR_UNSUPPORTED
    assert "PKV_STAMPS" in native.last_error()
    assert native.lib.pkv_debug_stamps(1, ptr) == native.PKV_ERR_UNSUPPORTED
    assert native.lib.pkv_debug_stamps(2, ptr) == native.PKV_ERR_INVALID_ARG
    assert native.lib.pkv_debug_stamps(0, None) == native.PKV_ERR_INVALID_ARG
    with pytest.raises(native.PkvError) as e:
        native.debug_stamps(0)
    assert e.value.status == native.PKV_ERR_UNSUPPORTED
    # the header's layout constant matches the binding's
    text = open(HEADER).read()
    assert re.search(r"#define PKV_STAMP_WORDS \(16 \* 8 \* 48 \* 8\)", text)
    assert native.PKV_STAMP_WORDS == 16 * 8 * 48 * 8


def test_plan_pick_by_hand(native):
    # items in 32-key blocks of existing keys: seq 0 tiles 0..2 of L = 256 -> 8 blocks;
    # seq 1 tile 0 of L = 100 -> ceil(100 / 32) = 4; a padding entry (-1, 0, 0, 0) is skipped
    lens = [256, 100]
    work = [[0, 0, 2, 0], [1, 0, 1, 0], [-1, 0, 0, 0]]
    plan, ratio = native.plan_pick(lens, work, native.PKV_KV_E4M3, 8, 4)
    assert ratio == pytest.approx(8 / 6) and plan == native.PKV_PLAN_WAVE  # 1.33 < 1.5
    plan, _ = native.plan_pick(lens, work, native.PKV_KV_MLA, 1, 64)
    assert plan == native.PKV_PLAN_BALANCED  # latent multi-token form: 1.33 >= 1.12
    plan, _ = native.plan_pick(lens, work, native.PKV_KV_MLA, 1, 32)
    assert plan == native.PKV_PLAN_WAVE  # latent pair form: the page's 1.5
    # seq 0 alone against three one-block items: 8 / ((8 + 3) / 4) = 2.9
    lens = [256, 10, 1, 0]
    work = [[0, 0, 2, 0], [1, 0, 1, 0], [2, 0, 1, 0], [3, 0, 1, 0]]
    plan, ratio = native.plan_pick(lens, work, native.PKV_KV_E4M3, 8, 16)
    assert ratio == pytest.approx(8 * 4 / 11) and plan == native.PKV_PLAN_BALANCED
    for fmt in (native.PKV_KV_E2M1, native.PKV_KV_E2M3, native.PKV_KV_E3M2, native.PKV_KV_NVFP4):
        assert native.plan_pick(lens, work, fmt, 8, 16)[0] == native.PKV_PLAN_WAVE  # one-item form only
    # four kv heads and at most 16 rows: the paired plan, whatever the imbalance (e4m3, fp4, fp6, NVFP4 caches)
    for fmt in (native.PKV_KV_E4M3, native.PKV_KV_E2M1, native.PKV_KV_E2M3, native.PKV_KV_E3M2, native.PKV_KV_NVFP4):
        assert native.plan_pick(lens, work, fmt, 4, 16)[0] == native.PKV_PLAN_PAIRED
        assert native.plan_pick([256, 256], [[0, 0, 2, 0], [1, 0, 2, 0]], fmt, 4, 1)[0] == native.PKV_PLAN_PAIRED
    assert native.plan_pick(lens, work, native.PKV_KV_E4M3, 4, 32)[0] == native.PKV_PLAN_BALANCED  # two row blocks
    assert native.plan_pick(lens, work, native.PKV_KV_E4M3, 2, 16)[0] == native.PKV_PLAN_BALANCED  # two kv heads
    # a chunk past the runtime length counts its existing keys: tiles 1..2 of L = 200 -> 72 keys, 3 blocks
    plan, ratio = native.plan_pick([200, 300], [[0, 1, 2, 1], [1, 0, 3, 0]], native.PKV_KV_E4M3, 8, 4)
    assert ratio == pytest.approx(10 / 6.5)
    assert native.plan_pick([5], np.zeros((0, 4), np.int32), native.PKV_KV_E4M3, 8, 4)[1] == 1.0
    P = ctypes.POINTER(ctypes.c_int32)
    out = ctypes.c_int32()
    assert native.lib.pkv_plan_pick(None, 1, None, 0, 0, 8, 4, ctypes.byref(out), None) == native.PKV_ERR_INVALID_ARG
    lens_a = np.array([5], np.int32)
    assert native.lib.pkv_plan_pick(lens_a.ctypes.data_as(P), 1, lens_a.ctypes.data_as(P), 0, 0, 8, 0,
                                    ctypes.byref(out), None) == native.PKV_ERR_INVALID_ARG
    assert native.lib.pkv_plan_pick(lens_a.ctypes.data_as(P), 1, lens_a.ctypes.data_as(P), 0, 0, 0, 4,
                                    ctypes.byref(out), None) == native.PKV_ERR_INVALID_ARG
