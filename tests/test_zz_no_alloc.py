"""The allocation-free decode entry point (nvfp4_paged_decode_attn_noalloc,
called through the C ABI) against nvfp4_paged_decode_attn with a caller
workspace on the same inputs: two calls in a row -- the second with a smaller
input, so it finds the first call's partials in the shared scratch -- give
outputs identical to the workspace entry point's, and both agree with the
oracle to 1e-3.  The contexts are long enough that every (sequence, kv head)
unit is split across workgroups, so the scratch's counters and partials are
used."""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_cases import ATTN_TOL, build_cache, host_f32, row_rel_err
from synthetic import synth

pytestmark = pytest.mark.gpu

SM = 1 / math.sqrt(128)


def _run(nk, lens, H, Hq, q_dtype, seed):
    print(f"case: no-alloc decode lens={lens} H={H} Hq={Hq} {q_dtype}", flush=True)
    cache = build_cache(lens, H, torch.bfloat16, "sparse6", 0.005, False, seed=seed)
    B = len(lens)
    msl = max(lens)
    bt = np.ascontiguousarray(cache.bt)
    bt_d = torch.from_numpy(bt).cuda()
    sl_d = torch.tensor(lens, dtype=torch.int32, device="cuda")
    q = synth.queries(B, Hq, q_dtype, "cuda", seed, 1).contiguous()
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    c = cache.layer.c_struct()
    st = nk.lib.nvfp4_paged_decode_attn_noalloc(
        ctypes.byref(c), ctypes.c_void_p(q.data_ptr()), nk._dtype_code(q), B, Hq, ctypes.c_void_p(bt_d.data_ptr()),
        bt.shape[1], ctypes.c_void_p(sl_d.data_ptr()), msl, ctypes.c_float(SM), ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == nk.NVFP4_OK, nk.status_string(st)
    ref_ws = nk.paged_decode_attn(cache.layer, q, bt_d, sl_d, msl, SM)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_ws), float((out - ref_ws).abs().max())
    ref = oracle.decode_attention(cache.planes, cache.g_k, cache.g_v, host_f32(q), cache.bt,
                                  np.array(lens, np.int32), float(np.float32(SM)))
    err = float(row_rel_err(out.cpu().numpy(), ref).max())
    print(f"  identical to the workspace entry point; max row rel err vs oracle {err:.2e}", flush=True)
    assert err <= ATTN_TOL
    return out


def test_noalloc_decode_two_calls_second_smaller():
    import nvfp4_quantized_paged_kv_amd as nk

    # every unit spans several workgroups' shares (split, merged through the scratch)
    assert nk.decode_workspace_bytes(3, 32, 4, 5000) > 0
    _run(nk, [5000, 3001, 4095], 4, 32, torch.bfloat16, seed=71)
    _run(nk, [1500, 17], 2, 8, torch.float32, seed=72)
    # and once more at the first shape: the counters were left at zero
    _run(nk, [5000, 3001, 4095], 4, 32, torch.bfloat16, seed=73)
