"""GPU parity of bulk quantize-append (the streaming kernel that walks the
jobs with a grid-wide stride and loads the next step's inputs ahead): whole
code and scale planes bit-exact against the oracle, for bf16 and float32
inputs, plain and Hadamard-rotated K, with a token count that is not a
multiple of 16, several grid strides per thread, and skipped slots (negative
or past the pool)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from synthetic import synth
from tests.gpu_cases import host_f32, planes_equal

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("hadamard", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_bulk_append_bitexact(dtype, hadamard):
    import nvfp4_quantized_paged_kv_amd as nk

    H, T = 8, 12007  # 12016 * 8 * 8 = 769,024 block jobs: the streaming path, about 3 grid strides
    _say(f"case: bulk append {dtype} hadamard={hadamard} T={T} H={H}")
    k = synth.kv_values(T, H, "chan50", 0.0, 0, torch.float32, "cpu", 91, 0)
    v = synth.kv_values(T, H, "sparse6", 0.005, 1, torch.float32, "cpu", 91, 0)
    if hadamard and dtype == torch.float32:
        # float32 rows rotate exactly (float64 sums) when their values span at
        # most 22 binades: keep magnitudes at or above 2^-12
        k = torch.where(k.abs() < 2.0 ** -12, torch.copysign(torch.full_like(k, 2.0 ** -12), k), k)
    k, v = k.to(dtype), v.to(dtype)
    pool = (T + 15) // 16 + 40
    rng = np.random.default_rng(5)
    slots = rng.permutation(pool * 16)[:T].astype(np.int32)
    slots[::97] = -1
    slots[11] = pool * 16 + 3  # past the pool: skipped
    ok = slots.copy()
    ok[ok >= pool * 16] = -1
    k_host = host_f32(k)
    k_in = oracle.rotate_k(k_host) if hadamard else k_host
    g_k = synth.global_scale(float(np.abs(k_in).max()))
    g_v = synth.global_scale(float(v.float().abs().max()))
    planes = oracle.Planes(pool, H)
    oracle.quantize_append(planes, k_in, host_f32(v), ok, g_k, g_v)
    layer = nk.KVCacheLayer.allocate(pool, H, g_k, g_v)
    nk.quantize_append(layer, k.cuda(), v.cuda(), torch.from_numpy(slots).cuda(), hadamard=hadamard)
    torch.cuda.synchronize()
    assert planes_equal(layer, planes) == []
