"""The opt-in per-phase timestamps end to end, in this process: the stamped
library (built beside the normal one by ``python -m paged_kv_fp8_amd.stamps
--build``) is loaded next to the normal one and its decode entry point runs on
the arguments the binding built. Its stamps must be those of real loop steps
(every phase non-negative, the steps counted), and its O and LSE must equal
the normal library's bit for bit: the stamps and their scheduling barriers
only move instructions. Skipped when the stamped library has not been built."""
import ctypes
import os

import numpy as np
import pytest
import torch

from paged_kv_fp8_amd import decode, native
from paged_kv_fp8_amd.stamps import COPY_LOOP, PHASES, STAMP_LIB, phases_for, summarize
from paged_kv_fp8_amd.workloads import make_batch, workload


def _stamped():
    if not os.path.exists(STAMP_LIB):
        pytest.skip("stamped library not built (python -m paged_kv_fp8_amd.stamps --build)")
    lib = ctypes.CDLL(STAMP_LIB)
    lib.pkv_paged_decode_attn.restype = ctypes.c_int32
    lib.pkv_paged_decode_attn.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.pkv_merge_splits.restype = ctypes.c_int32
    lib.pkv_merge_splits.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.pkv_debug_stamps.restype = ctypes.c_int32
    lib.pkv_debug_stamps.argtypes = [ctypes.c_int32, ctypes.c_void_p]
    return lib


@pytest.mark.gpu
@pytest.mark.parametrize("cfg,over,loop", [(2, {}, 0), (5, {"q_len": 4}, 1), (5, {"q_len": 1}, 2)])
def test_stamped_library_records_phases_and_matches(cfg, over, loop):
    lib = _stamped()
    batch = make_batch(workload(cfg, **over), device="cuda")
    dec = decode.for_batch(batch)
    assert phases_for(dec.kernel_name) == loop, dec.kernel_name
    dec.run()
    torch.cuda.synchronize()
    ref_o, ref_l = dec.o.clone(), dec.lse.clone()
    dec.o.zero_()
    dec.lse.zero_()
    s = torch.cuda.current_stream().cuda_stream
    assert lib.pkv_paged_decode_attn(ctypes.byref(dec.args), s) == native.PKV_OK
    if dec.has_splits:
        assert lib.pkv_merge_splits(ctypes.byref(dec.args), s) == native.PKV_OK
    torch.cuda.synchronize()
    assert torch.equal(dec.o.view(torch.int16), ref_o.view(torch.int16)), "stamped build changed O"
    assert torch.equal(dec.lse, ref_l), "stamped build changed LSE"
    buf = np.zeros(native.PKV_STAMP_WORDS, dtype=np.uint64)
    assert lib.pkv_debug_stamps(COPY_LOOP[loop], buf.ctypes.data_as(ctypes.c_void_p)) == native.PKV_OK
    ts = buf.astype(np.int64).reshape(16, 8, 48, 8)
    n = PHASES[loop][2]
    rec = (ts[..., 0] > 0) & (ts[..., n - 1] > 0)
    assert rec.sum() > 100
    d = np.diff(ts[rec][:, :n], axis=1)
    assert (d >= 0).all(), "stamps of a step out of order"
    print(summarize(ts, loop))
