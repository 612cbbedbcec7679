"""pkv_paged_decode_noalloc (decode + merge on the library's own per-device
split workspace) against the existing entry points (pkv_paged_decode_attn +
pkv_merge_splits with a caller workspace), through the C ABI: bit-identical
O and LSE on two calls in a row, the second on a smaller batch, for the e4m3
cache (bf16 and e4m3 queries) and the latent-record cache. The array keeps
the previous call's contents, so the second call also shows that nothing
depends on it."""

import ctypes

import pytest
import torch

from helpers import nan_fill_
from paged_kv_fp8_amd.workloads import make_batch, workload

pytestmark = pytest.mark.gpu


def _reference(batch):
    from paged_kv_fp8_amd import decode  # loads the HIP library; fails loudly if missing

    dec = decode.for_batch(batch)
    if dec.has_splits:
        nan_fill_(dec.workspace)
    dec.run()
    torch.cuda.synchronize()
    return dec


def _noalloc(dec, batch):
    from paged_kv_fp8_amd import native

    w = batch.spec
    o = torch.full((w.num_seqs * w.q_len, w.h_q, w.d_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((w.num_seqs, w.h_k, w.rows), float("nan"), dtype=torch.float32, device="cuda")
    args = native.DecodeArgs.from_buffer_copy(dec.args)
    args.o, args.o_tok_stride, args.o_head_stride = o.data_ptr(), o.stride(0), o.stride(1)
    args.lse = lse.data_ptr()
    args.workspace, args.workspace_bytes = None, 0  # ignored: the library's own array is used
    before = torch.cuda.memory_allocated()
    native.paged_decode_noalloc(args, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return o, lse


CASES = {
    "e4m3_cache_bf16_q": ((2, dict(num_seqs=12, seq_len_dist=("uniform", 300, 6000))),
                          (2, dict(num_seqs=5, seq_len_dist=("uniform", 100, 2000)))),
    "e4m3_cache_fp8_q": ((4, dict(num_seqs=10, seq_len_dist=("mix", 0.3, (6000, 12000), (1024, 3000)))),
                         (4, dict(num_seqs=4, seq_len_dist=("uniform", 1024, 3000)))),
    "latent_cache": ((5, dict(num_seqs=6, q_len=2, seq_len_dist=("uniform", 500, 4000))),
                     (5, dict(num_seqs=3, q_len=1, seq_len_dist=("uniform", 100, 1500)))),
}


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_equals_workspace_entry_points_twice(name):
    for call, (idx, over) in enumerate(CASES[name]):
        batch = make_batch(workload(idx, **over), device="cuda")
        ref = _reference(batch)
        if call == 0:
            assert ref.has_splits  # the first call uses the array
        o, lse = _noalloc(ref, batch)
        assert torch.equal(o.view(torch.int16), ref.o.view(torch.int16)), f"{name} call {call}: O differs"
        assert torch.equal(lse.view(torch.int32), ref.lse.view(torch.int32)), f"{name} call {call}: LSE differs"
        print(f"{name} call {call}: {batch.spec.num_seqs} seqs, splits {ref.plan_info.max_n_splits}: bit-identical")


def test_noalloc_rejects_a_workspace_beyond_the_array():
    from paged_kv_fp8_amd import native

    batch = make_batch(workload(2, num_seqs=8, seq_len_dist=("uniform", 300, 3000)), device="cuda")
    ref = _reference(batch)
    args = native.DecodeArgs.from_buffer_copy(ref.args)
    args.max_splits = 256
    args.num_seqs = 64  # a larger batch shape than the array holds (checked before any launch)
    st = native.lib.pkv_paged_decode_noalloc(ctypes.byref(args), None)
    assert st == native.PKV_ERR_WORKSPACE, native.last_error()
