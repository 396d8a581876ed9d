"""CPU oracle for the NVFP4 paged KV cache -- TEST INFRASTRUCTURE ONLY.

Thin ctypes/numpy marshalling around ``nvfp4_oracle.c`` (plain scalar C in
float64; every function there cites the page passage it follows).  Only the
test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never imports, links or
calls it, and the two share no code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_DEFAULT_LIB = os.path.join(_HERE, "libnvfp4_oracle.so")
# NVFP4_ORACLE_LIBRARY: another build of the same source (the tests' sanitizer build)
_LIB_PATH = os.environ.get("NVFP4_ORACLE_LIBRARY") or _DEFAULT_LIB
_lib = None

_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_int = ctypes.c_int
_flt = ctypes.c_float
_dbl = ctypes.c_double


def build() -> str:
    """Compile the oracle with gcc (strict IEEE: no contraction, no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-Wall",
           "-shared", "-fPIC", _SRC, "-o", _DEFAULT_LIB + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(_DEFAULT_LIB + ".tmp", _DEFAULT_LIB)
    return _DEFAULT_LIB


def build_sanitized(out: str, clang: str) -> str:
    """The same source under AddressSanitizer and UBSan (clang, no OpenMP), for
    the host sanitizer test; the runtime is preloaded by the process that loads it."""
    cmd = [clang, "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fno-fast-math", "-Wall",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared", "-fPIC", _SRC,
           "-o", out + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(out + ".tmp", out)
    return out


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        if _LIB_PATH != _DEFAULT_LIB:
            raise ImportError(f"NVFP4_ORACLE_LIBRARY={_LIB_PATH} does not exist")
        build()
    L = ctypes.CDLL(_LIB_PATH)
    L.nvfp4o_e2m1_value.argtypes = [_int]
    L.nvfp4o_e2m1_value.restype = _dbl
    L.nvfp4o_e4m3_value.argtypes = [_int]
    L.nvfp4o_e4m3_value.restype = _dbl
    L.nvfp4o_e4m3_encode.argtypes = [_dbl]
    L.nvfp4o_e4m3_encode.restype = _int
    L.nvfp4o_e2m1_encode.argtypes = [_dbl]
    L.nvfp4o_e2m1_encode.restype = _int
    L.nvfp4o_quantize_rows.argtypes = [_f32p, _i64, _flt, _u8p, _u8p]
    L.nvfp4o_quantize_rows.restype = None
    L.nvfp4o_dequantize_rows.argtypes = [_u8p, _u8p, _i64, _flt, _f64p]
    L.nvfp4o_dequantize_rows.restype = None
    L.nvfp4o_mla_quantize_rows.argtypes = [_f32p, _i64, _flt, _u8p, _u8p]
    L.nvfp4o_mla_quantize_rows.restype = None
    L.nvfp4o_mla_sparse_decode.argtypes = [_u8p, _u8p, _i64, _flt, _f32p, _i64, _int, _i32p, _int, _flt, _f64p]
    L.nvfp4o_mla_sparse_decode.restype = None
    L.nvfp4o_scatter_rows.argtypes = [_u8p, _u8p, _i64, _int, _i32p, _int, _u8p, _u8p]
    L.nvfp4o_scatter_rows.restype = None
    L.nvfp4o_gather_rows.argtypes = [_u8p, _u8p, _i64, _int, _i32p, _int, _u8p, _u8p]
    L.nvfp4o_gather_rows.restype = None
    L.nvfp4o_decode_attention.argtypes = [_u8p, _u8p, _u8p, _u8p, _int, _flt, _flt, _f32p, _int, _i32p, _int,
                                          _i32p, _flt, _i64p, _i64, _f64p]
    L.nvfp4o_decode_attention.restype = None
    L.nvfp4o_fp8_workspace.argtypes = [_u8p, _u8p, _int, _int, _flt, _i32p, _int, _int, _i32p, _i32p, _flt, _u8p]
    L.nvfp4o_fp8_workspace.restype = None
    L.nvfp4o_fp8_quantize_rows.argtypes = [_f32p, _i64, _i64, _int, _i32p, _flt, _u8p]
    L.nvfp4o_fp8_quantize_rows.restype = None
    L.nvfp4o_extend_attention.argtypes = [_u8p, _u8p, _int, _flt, _flt, _f32p, _int, _int, _i32p, _i32p, _i32p, _flt,
                                          _i64p, _i64, _f64p]
    L.nvfp4o_extend_attention.restype = None
    L.nvfp4o_extend_attention_fp8.argtypes = L.nvfp4o_extend_attention.argtypes + [_f64p]
    L.nvfp4o_extend_attention_fp8.restype = None
    L.nvfp4o_e8m0_value.argtypes = [_int]
    L.nvfp4o_e8m0_value.restype = _dbl
    L.nvfp4o_e8m0_scale_for.argtypes = [_dbl]
    L.nvfp4o_e8m0_scale_for.restype = _int
    L.nvfp4o_mx_quantize_rows.argtypes = [_f32p, _i64, _u8p, _u8p]
    L.nvfp4o_mx_quantize_rows.restype = None
    L.nvfp4o_mx_dequantize_rows.argtypes = [_u8p, _u8p, _i64, _f64p]
    L.nvfp4o_mx_dequantize_rows.restype = None
    L.nvfp4o_mx_scatter_rows.argtypes = [_u8p, _u8p, _i64, _int, _i32p, _int, _u8p, _u8p]
    L.nvfp4o_mx_scatter_rows.restype = None
    L.nvfp4o_mx_gather_rows.argtypes = [_u8p, _u8p, _i64, _int, _i32p, _int, _u8p, _u8p]
    L.nvfp4o_mx_gather_rows.restype = None
    L.nvfp4o_mx_decode_attention.argtypes = [_u8p, _u8p, _u8p, _u8p, _int, _f32p, _int, _i32p, _int, _i32p, _flt,
                                             _i64p, _i64, _f64p]
    L.nvfp4o_mx_decode_attention.restype = None
    L.nvfp4o_hadamard_rows.argtypes = [_f64p, _i64, _dbl, _f64p]
    L.nvfp4o_hadamard_rows.restype = None
    L.nvfp4o_unrounded_block_dequant.argtypes = [_f64p, _i64, _i64, _f64p]
    L.nvfp4o_unrounded_block_dequant.restype = None
    L.nvfp4o_bytes_per_token_head.argtypes = []
    L.nvfp4o_bytes_per_token_head.restype = _i64
    L.nvfp4o_max_threads.argtypes = []
    L.nvfp4o_max_threads.restype = _int
    _lib = L
    return L


# ------------------------------------------------------------------ formats
def e2m1_value(code: int) -> float:
    return lib().nvfp4o_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return lib().nvfp4o_e4m3_value(int(byte))


def e4m3_encode(r: float) -> int:
    return lib().nvfp4o_e4m3_encode(float(r))


def e2m1_encode(y: float) -> int:
    return lib().nvfp4o_e2m1_encode(float(y))


# ------------------------------------------------------------- quantization
def quantize_rows(x: np.ndarray, g: float):
    """x: float32 [..., 128] -> (codes uint8 [n, 64], scales uint8 [n, 8])."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, 128)
    n = x.shape[0]
    codes = np.zeros((n, 64), np.uint8)
    scales = np.zeros((n, 8), np.uint8)
    lib().nvfp4o_quantize_rows(x, n, float(np.float32(g)), codes, scales)
    return codes, scales


def dequantize_rows(codes: np.ndarray, scales: np.ndarray, g: float) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1, 64)
    scales = np.ascontiguousarray(scales, dtype=np.uint8).reshape(-1, 8)
    out = np.zeros((codes.shape[0], 128), np.float64)
    lib().nvfp4o_dequantize_rows(codes, scales, codes.shape[0], float(np.float32(g)), out)
    return out


class Planes:
    """One layer's paged NVFP4 cache as four byte planes (host memory)."""

    def __init__(self, num_pages: int, num_kv_heads: int):
        self.num_pages = int(num_pages)
        self.H = int(num_kv_heads)
        self.k_codes = np.zeros(self.num_pages * self.H * 1024, np.uint8)
        self.k_scales = np.zeros(self.num_pages * self.H * 128, np.uint8)
        self.v_codes = np.zeros(self.num_pages * self.H * 1024, np.uint8)
        self.v_scales = np.zeros(self.num_pages * self.H * 128, np.uint8)


def scatter_rows(codes, scales, slot_mapping, H: int, is_v: bool, code_plane, scale_plane):
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int32)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    assert codes.size == slots.size * H * 64 and scales.size == slots.size * H * 8
    lib().nvfp4o_scatter_rows(codes, scales, slots.size, int(H), slots, int(bool(is_v)), code_plane, scale_plane)


def gather_rows(code_plane, scale_plane, slot_mapping, H: int, is_v: bool):
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int32)
    codes = np.zeros((slots.size * H, 64), np.uint8)
    scales = np.zeros((slots.size * H, 8), np.uint8)
    lib().nvfp4o_gather_rows(code_plane, scale_plane, slots.size, int(H), slots, int(bool(is_v)), codes, scales)
    return codes, scales


def quantize_append(planes: Planes, k: np.ndarray, v: np.ndarray, slot_mapping, g_k: float, g_v: float):
    """Quantize new tokens k, v (float32 [T, H, 128]) and write them at their slots."""
    H = planes.H
    kc, ks = quantize_rows(k, g_k)
    vc, vs = quantize_rows(v, g_v)
    scatter_rows(kc, ks, slot_mapping, H, False, planes.k_codes, planes.k_scales)
    scatter_rows(vc, vs, slot_mapping, H, True, planes.v_codes, planes.v_scales)
    return kc, ks, vc, vs


# --------------------------------------------------------- decode attention
def decode_attention(planes: Planes, g_k: float, g_v: float, q: np.ndarray, block_table: np.ndarray,
                     seq_lens: np.ndarray, sm_scale: float, rows=None) -> np.ndarray:
    """q: float32 [B, Hq, 128]; rows: flat indices b*Hq + qh (default: all).

    Returns float64 [len(rows), 128]."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    B, Hq, D = q.shape
    assert D == 128 and Hq % planes.H == 0
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    assert bt.shape[0] == B
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    if rows is None:
        rows = np.arange(B * Hq, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, 128), np.float64)
    lib().nvfp4o_decode_attention(planes.k_codes, planes.k_scales, planes.v_codes, planes.v_scales, planes.H,
                                  float(np.float32(g_k)), float(np.float32(g_v)), q, Hq, bt, bt.shape[1], sl,
                                  float(np.float32(sm_scale)), rows, rows.size, out)
    return out


def fp8_workspace(planes: Planes, is_v: bool, g: float, block_table, prefix_lens, ws_offsets, ws_scale: float,
                  total_tokens: int) -> np.ndarray:
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    pl = np.ascontiguousarray(prefix_lens, dtype=np.int32)
    wo = np.ascontiguousarray(ws_offsets, dtype=np.int32)
    out = np.zeros(int(total_tokens) * planes.H * 128, np.uint8)
    cp, sp = (planes.v_codes, planes.v_scales) if is_v else (planes.k_codes, planes.k_scales)
    lib().nvfp4o_fp8_workspace(cp, sp, int(bool(is_v)), planes.H, float(np.float32(g)), bt, bt.shape[1], pl.size,
                               pl, wo, float(np.float32(ws_scale)), out)
    return out.reshape(int(total_tokens), planes.H, 128)


def fp8_quantize_rows(x: np.ndarray, rows, ws_scale: float, ws: np.ndarray) -> None:
    """Store x [T, H, 128] (float32 values) as E4M3 into ws [capacity, H, 128] uint8 at ws rows `rows` (in place)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    T, H, D = x.shape
    assert D == 128 and ws.dtype == np.uint8 and ws.flags.c_contiguous and ws.shape[1:] == (H, 128)
    r = np.ascontiguousarray(rows, dtype=np.int32)
    assert r.size == T and (r < ws.shape[0]).all()
    lib().nvfp4o_fp8_quantize_rows(x, T, H * 128, H, r, float(np.float32(ws_scale)), ws.reshape(-1))


def extend_attention(ws_k: np.ndarray, ws_v: np.ndarray, k_ws_scale: float, v_ws_scale: float, q: np.ndarray,
                     q_offsets, ws_offsets, prefix_lens, sm_scale: float, rows=None) -> np.ndarray:
    """q: float32 [Tq, Hq, 128]; ws_k/ws_v: uint8 [capacity, H, 128]; rows: flat indices qrow*Hq + qh.

    Returns float64 [len(rows), 128]."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    Tq, Hq, D = q.shape
    H = ws_k.shape[1]
    assert D == 128 and Hq % H == 0 and ws_k.shape == ws_v.shape
    qo = np.ascontiguousarray(q_offsets, dtype=np.int32)
    wo = np.ascontiguousarray(ws_offsets, dtype=np.int32)
    pl = np.ascontiguousarray(prefix_lens, dtype=np.int32)
    n = pl.size
    assert qo.size == n + 1 and wo.size >= n and qo[-1] == Tq
    assert all(wo[i] + pl[i] + (qo[i + 1] - qo[i]) <= ws_k.shape[0] for i in range(n))
    if rows is None:
        rows = np.arange(Tq * Hq, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, 128), np.float64)
    lib().nvfp4o_extend_attention(np.ascontiguousarray(ws_k).reshape(-1), np.ascontiguousarray(ws_v).reshape(-1), H,
                                  float(np.float32(k_ws_scale)), float(np.float32(v_ws_scale)), q, Hq, n, qo, wo, pl,
                                  float(np.float32(sm_scale)), rows, rows.size, out)
    return out


def extend_attention_fp8(ws_k: np.ndarray, ws_v: np.ndarray, k_ws_scale: float, v_ws_scale: float, q: np.ndarray,
                         q_offsets, ws_offsets, prefix_lens, sm_scale: float, rows=None):
    """extend_attention in FP8 arithmetic (reading R11: Q and the softmax weights rounded to E4M3).

    Returns (out float64 [len(rows), 128], tol float64 [len(rows)]): tol bounds the
    difference to a kernel computing the same with float32 logits, an integer running
    maximum and FP8 matrix cores (see the C source)."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    Tq, Hq, D = q.shape
    H = ws_k.shape[1]
    assert D == 128 and Hq % H == 0 and ws_k.shape == ws_v.shape
    qo = np.ascontiguousarray(q_offsets, dtype=np.int32)
    wo = np.ascontiguousarray(ws_offsets, dtype=np.int32)
    pl = np.ascontiguousarray(prefix_lens, dtype=np.int32)
    n = pl.size
    assert qo.size == n + 1 and wo.size >= n and qo[-1] == Tq
    assert all(wo[i] + pl[i] + (qo[i + 1] - qo[i]) <= ws_k.shape[0] for i in range(n))
    if rows is None:
        rows = np.arange(Tq * Hq, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, 128), np.float64)
    tol = np.zeros(rows.size, np.float64)
    lib().nvfp4o_extend_attention_fp8(np.ascontiguousarray(ws_k).reshape(-1), np.ascontiguousarray(ws_v).reshape(-1),
                                      H, float(np.float32(k_ws_scale)), float(np.float32(v_ws_scale)), q, Hq, n, qo,
                                      wo, pl, float(np.float32(sm_scale)), rows, rows.size, out, tol)
    return out, tol


# -------------------------------------------------------------------- MXFP4
def e8m0_value(byte: int) -> float:
    return lib().nvfp4o_e8m0_value(int(byte))


def e8m0_scale_for(amax: float) -> int:
    return lib().nvfp4o_e8m0_scale_for(float(amax))


def mx_quantize_rows(x: np.ndarray):
    """x: float32 [..., 128] -> (codes uint8 [n, 64], E8M0 scales uint8 [n, 4])."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, 128)
    n = x.shape[0]
    codes = np.zeros((n, 64), np.uint8)
    scales = np.zeros((n, 4), np.uint8)
    lib().nvfp4o_mx_quantize_rows(x, n, codes, scales)
    return codes, scales


def mx_dequantize_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1, 64)
    scales = np.ascontiguousarray(scales, dtype=np.uint8).reshape(-1, 4)
    out = np.zeros((codes.shape[0], 128), np.float64)
    lib().nvfp4o_mx_dequantize_rows(codes, scales, codes.shape[0], out)
    return out


class MxPlanes:
    """One layer's paged MXFP4 cache: 1 KiB code tiles (K as NVFP4 K; V with each
    slot's nibbles in bytes of its own), 64-byte scale tiles."""

    def __init__(self, num_pages: int, num_kv_heads: int):
        self.num_pages = int(num_pages)
        self.H = int(num_kv_heads)
        self.k_codes = np.zeros(self.num_pages * self.H * 1024, np.uint8)
        self.k_scales = np.zeros(self.num_pages * self.H * 64, np.uint8)
        self.v_codes = np.zeros(self.num_pages * self.H * 1024, np.uint8)
        self.v_scales = np.zeros(self.num_pages * self.H * 64, np.uint8)


def mx_quantize_append(planes: MxPlanes, k: np.ndarray, v: np.ndarray, slot_mapping):
    """Quantize new tokens k, v (float32 [T, H, 128]) to MXFP4 and write them at their slots."""
    H = planes.H
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int32)
    out = []
    for x, is_v, cp, sp in ((k, 0, planes.k_codes, planes.k_scales), (v, 1, planes.v_codes, planes.v_scales)):
        c, s = mx_quantize_rows(x)
        assert c.shape[0] == slots.size * H
        lib().nvfp4o_mx_scatter_rows(c, s, slots.size, H, slots, is_v, cp, sp)
        out += [c, s]
    return tuple(out)


def mx_gather_rows(code_plane, scale_plane, slot_mapping, H: int, is_v: bool):
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int32)
    codes = np.zeros((slots.size * H, 64), np.uint8)
    scales = np.zeros((slots.size * H, 4), np.uint8)
    lib().nvfp4o_mx_gather_rows(code_plane, scale_plane, slots.size, int(H), slots, int(bool(is_v)), codes, scales)
    return codes, scales


def mx_decode_attention(planes: MxPlanes, q: np.ndarray, block_table: np.ndarray, seq_lens: np.ndarray,
                        sm_scale: float, rows=None) -> np.ndarray:
    """Decode attention over MXFP4 pages; q: float32 [B, Hq, 128]. Returns float64 [len(rows), 128]."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    B, Hq, D = q.shape
    assert D == 128 and Hq % planes.H == 0
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    assert bt.shape[0] == B
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    if rows is None:
        rows = np.arange(B * Hq, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, 128), np.float64)
    lib().nvfp4o_mx_decode_attention(planes.k_codes, planes.k_scales, planes.v_codes, planes.v_scales, planes.H, q, Hq,
                                     bt, bt.shape[1], sl, float(np.float32(sm_scale)), rows, rows.size, out)
    return out


# ------------------------------------------------------- Hadamard rotation
K_ROT_SCALE = 2.0 ** -4   # K' = H k / 16
Q_ROT_SCALE = 2.0 ** -3   # q' = H q / 8, so q'.k' = q.k


def hadamard_rows(x, scale: float) -> np.ndarray:
    """scale * H x for each 128-value row of x (float64 result, same leading shape)."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    shape = a.shape
    assert shape[-1] == 128
    a = a.reshape(-1, 128)
    out = np.zeros_like(a)
    lib().nvfp4o_hadamard_rows(a, a.shape[0], float(scale), out)
    return out.reshape(shape)


def rotate_k(k) -> np.ndarray:
    """K rows as stored by the rotated append: float32 nearest to H k / 16."""
    return hadamard_rows(k, K_ROT_SCALE).astype(np.float32)


def rotate_q(q) -> np.ndarray:
    """Queries as the rotated decode uses them: H q / 8 (float64)."""
    return hadamard_rows(q, Q_ROT_SCALE)


# ---------------------------------------------------- Sparse-MLA latent cache
MLA_D = 576          # latent (512) + rotary key (64) values per token row
MLA_DV = 512         # values the output sums (the latent part)
MLA_CODE_BYTES = MLA_D // 2
MLA_SCALE_BYTES = MLA_D // 16


class MlaPlanes:
    """The oracle's latent cache: codes [num_slots][288], scales [num_slots][36]."""

    def __init__(self, num_slots: int):
        self.num_slots = int(num_slots)
        self.codes = np.zeros((self.num_slots, MLA_CODE_BYTES), np.uint8)
        self.scales = np.zeros((self.num_slots, MLA_SCALE_BYTES), np.uint8)


def mla_quantize_rows(x, g: float):
    """Latent rows float32 [n, 576] -> (codes [n, 288], scales [n, 36])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.ndim == 2 and x.shape[1] == MLA_D
    n = x.shape[0]
    codes = np.zeros((n, MLA_CODE_BYTES), np.uint8)
    scales = np.zeros((n, MLA_SCALE_BYTES), np.uint8)
    lib().nvfp4o_mla_quantize_rows(x, n, float(np.float32(g)), codes, scales)
    return codes, scales


def mla_quantize_append(planes: MlaPlanes, x, slots, g: float) -> None:
    """Quantize rows x [n, 576] into their slots (slots outside the cache are skipped)."""
    codes, scales = mla_quantize_rows(x, g)
    slots = np.asarray(slots, np.int64)
    ok = (slots >= 0) & (slots < planes.num_slots)
    planes.codes[slots[ok]] = codes[ok]
    planes.scales[slots[ok]] = scales[ok]


def mla_dequantize_rows(codes, scales, g: float) -> np.ndarray:
    """codes [n, 288], scales [n, 36] -> float64 [n, 576] through the GQA row
    dequantizer (a 576-row is 36 independent 16-value blocks)."""
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    n = codes.shape[0]
    pc = np.zeros((n, 320), np.uint8)
    psc = np.zeros((n, 40), np.uint8)
    pc[:, :MLA_CODE_BYTES] = codes
    psc[:, :MLA_SCALE_BYTES] = scales
    out = dequantize_rows(pc.reshape(n * 5, 64), psc.reshape(n * 5, 8), g).reshape(n, 640)
    return out[:, :MLA_D]


def mla_sparse_decode(planes: MlaPlanes, g: float, q, indices, sm_scale: float) -> np.ndarray:
    """q float32 [T, Hq, 576], indices int32 [T, topk] (cache slots) -> float64 [T, Hq, 512]."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    T, Hq, D = q.shape
    assert D == MLA_D
    idx = np.ascontiguousarray(indices, dtype=np.int32)
    assert idx.ndim == 2 and idx.shape[0] == T
    out = np.zeros((T, Hq, MLA_DV), np.float64)
    lib().nvfp4o_mla_sparse_decode(planes.codes, planes.scales, planes.num_slots, float(np.float32(g)), q, T, Hq,
                                   idx, idx.shape[1], float(np.float32(sm_scale)), out)
    return out


# ------------------------------------------ the page's two-level comparison
def unrounded_block_dequant(x, block: int) -> np.ndarray:
    """Two-level scaling with an unrounded per-block scale amax/6 and no tensor
    scale (block = x.size: one global scale): the values read back, float64."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    lib().nvfp4o_unrounded_block_dequant(x, x.size, int(block), out)
    return out


def bytes_per_token_head() -> int:
    return int(lib().nvfp4o_bytes_per_token_head())


def max_threads() -> int:
    return int(lib().nvfp4o_max_threads())
