"""NVFP4 paged KV cache for MI355X (gfx950): Python binding of ``libnvfp4kv.so``.

Argument marshalling only: every step of quantize-append, decode attention and
the FP8 workspace dequant runs in the library's HIP kernels.  The functions
take torch tensors (device memory) and enqueue on torch's current HIP stream.
The C ABI and the cache layout are documented in ``include/nvfp4_kv.h``.

Importing this module raises if the library has not been built (there is no
fallback implementation).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# NVFP4KV_LIBRARY: another build of the same sources (the tests' host-sanitizer build)
LIB_PATH = os.environ.get("NVFP4KV_LIBRARY") or os.path.join(_PKG_DIR, "libnvfp4kv.so")

HEAD_DIM = 128
PAGE_SIZE = 16
TILE_CODE_BYTES = 1024
TILE_SCALE_BYTES = 128
MX_TILE_SCALE_BYTES = 64

NVFP4_OK = 0
NVFP4_ERR_INVALID_ARGUMENT = 1
NVFP4_ERR_UNSUPPORTED = 2
NVFP4_ERR_WORKSPACE_TOO_SMALL = 3
NVFP4_ERR_HIP = 4

DTYPE_F32 = 0
DTYPE_BF16 = 1

# Every function the public header declares.
EXPORTED_SYMBOLS = (
    "nvfp4_kv_quantize_append",
    "nvfp4_paged_decode_workspace_bytes",
    "nvfp4_paged_decode_attn",
    "nvfp4_paged_decode_attn_noalloc",
    "nvfp4_paged_decode_multi_workspace_bytes",
    "nvfp4_paged_decode_attn_multi",
    "nvfp4_paged_decode_step",
    "nvfp4_dequant_to_fp8_workspace",
    "nvfp4_fp8_rows_to_workspace",
    "nvfp4_fp8_extend_attn",
    "nvfp4_fp8_extend_attn_split_workspace_bytes",
    "nvfp4_fp8_extend_attn_split",
    "nvfp4_fp8_extend_attn_f8_workspace_bytes",
    "nvfp4_fp8_extend_attn_f8",
    "mxfp4_kv_quantize_append",
    "mxfp4_paged_decode_attn",
    "nvfp4_kv_quantize_append_hadamard",
    "nvfp4_paged_decode_attn_hadamard",
    "mxfp4_kv_quantize_append_hadamard",
    "mxfp4_paged_decode_attn_hadamard",
    "nvfp4_mla_quantize_append",
    "nvfp4_mla_sparse_decode_workspace_bytes",
    "nvfp4_mla_sparse_decode",
    "nvfp4_status_string",
)


class CKVLayer(ctypes.Structure):
    """Mirror of ``nvfp4_kv_layer_t``."""

    _fields_ = [
        ("k_codes", ctypes.c_void_p),
        ("k_scales", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p),
        ("v_scales", ctypes.c_void_p),
        ("num_pages", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("k_global", ctypes.c_float),
        ("v_global", ctypes.c_float),
    ]


class CMxLayer(ctypes.Structure):
    """Mirror of ``mxfp4_kv_layer_t``."""

    _fields_ = [
        ("k_codes", ctypes.c_void_p),
        ("k_scales", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p),
        ("v_scales", ctypes.c_void_p),
        ("num_pages", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
    ]


class CMlaLayer(ctypes.Structure):
    """Mirror of ``nvfp4_mla_layer_t``."""

    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("num_slots", ctypes.c_int32),
        ("latent_dim", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32),
        ("global_scale", ctypes.c_float),
    ]


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python nvfp4_quantized_paged_kv_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lp = ctypes.POINTER(CKVLayer)
    L.nvfp4_kv_quantize_append.argtypes = [lp, vp, vp, ctypes.c_int, i32, i64, vp, vp]
    L.nvfp4_kv_quantize_append.restype = ctypes.c_int
    L.nvfp4_paged_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.nvfp4_paged_decode_workspace_bytes.restype = sz
    L.nvfp4_paged_decode_attn.argtypes = [lp, vp, ctypes.c_int, i32, i32, vp, i32, vp, i32, f32, vp, vp, sz, vp]
    L.nvfp4_paged_decode_attn.restype = ctypes.c_int
    L.nvfp4_paged_decode_attn_noalloc.argtypes = [lp, vp, ctypes.c_int, i32, i32, vp, i32, vp, i32, f32, vp, vp]
    L.nvfp4_paged_decode_attn_noalloc.restype = ctypes.c_int
    L.nvfp4_paged_decode_multi_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.nvfp4_paged_decode_multi_workspace_bytes.restype = sz
    L.nvfp4_paged_decode_attn_multi.argtypes = [lp, vp, ctypes.c_int, i32, i32, i32, vp, i32, vp, i32, f32, vp, vp, sz,
                                                vp]
    L.nvfp4_paged_decode_attn_multi.restype = ctypes.c_int
    L.nvfp4_paged_decode_step.argtypes = [lp, vp, vp, vp, ctypes.c_int, i32, i32, i32, vp, i32, vp, i32, f32, vp, vp,
                                          sz, vp]
    L.nvfp4_paged_decode_step.restype = ctypes.c_int
    L.nvfp4_dequant_to_fp8_workspace.argtypes = [lp, vp, i32, i32, vp, vp, i32, f32, f32, vp, vp, i32, vp]
    L.nvfp4_dequant_to_fp8_workspace.restype = ctypes.c_int
    L.nvfp4_fp8_rows_to_workspace.argtypes = [vp, vp, ctypes.c_int, i32, i64, i32, vp, f32, f32, vp, vp, i32, vp]
    L.nvfp4_fp8_rows_to_workspace.restype = ctypes.c_int
    L.nvfp4_fp8_extend_attn.argtypes = [vp, ctypes.c_int, i32, i32, i32, i32, vp, vp, vp, i32, vp, vp, i32, f32, f32,
                                        f32, vp, vp]
    L.nvfp4_fp8_extend_attn.restype = ctypes.c_int
    L.nvfp4_fp8_extend_attn_split_workspace_bytes.argtypes = [ctypes.c_int, i32, i32, i32, i32, i32, i32]
    L.nvfp4_fp8_extend_attn_split_workspace_bytes.restype = sz
    L.nvfp4_fp8_extend_attn_split.argtypes = [vp, ctypes.c_int, i32, i32, i32, i32, vp, vp, vp, i32, i32, vp, vp, i32,
                                              f32, f32, f32, vp, vp, sz, vp]
    L.nvfp4_fp8_extend_attn_split.restype = ctypes.c_int
    L.nvfp4_fp8_extend_attn_f8_workspace_bytes.argtypes = L.nvfp4_fp8_extend_attn_split_workspace_bytes.argtypes
    L.nvfp4_fp8_extend_attn_f8_workspace_bytes.restype = sz
    L.nvfp4_fp8_extend_attn_f8.argtypes = L.nvfp4_fp8_extend_attn_split.argtypes
    L.nvfp4_fp8_extend_attn_f8.restype = ctypes.c_int
    mp = ctypes.POINTER(CMxLayer)
    L.mxfp4_kv_quantize_append.argtypes = [mp, vp, vp, ctypes.c_int, i32, i64, vp, vp]
    L.mxfp4_kv_quantize_append.restype = ctypes.c_int
    L.mxfp4_paged_decode_attn.argtypes = [mp, vp, ctypes.c_int, i32, i32, vp, i32, vp, i32, f32, vp, vp, sz, vp]
    L.mxfp4_paged_decode_attn.restype = ctypes.c_int
    for f in ("nvfp4_kv_quantize_append_hadamard",):
        getattr(L, f).argtypes = L.nvfp4_kv_quantize_append.argtypes
    for f in ("nvfp4_paged_decode_attn_hadamard",):
        getattr(L, f).argtypes = L.nvfp4_paged_decode_attn.argtypes
    L.mxfp4_kv_quantize_append_hadamard.argtypes = L.mxfp4_kv_quantize_append.argtypes
    L.mxfp4_paged_decode_attn_hadamard.argtypes = L.mxfp4_paged_decode_attn.argtypes
    for f in ("nvfp4_kv_quantize_append_hadamard", "nvfp4_paged_decode_attn_hadamard",
              "mxfp4_kv_quantize_append_hadamard", "mxfp4_paged_decode_attn_hadamard"):
        getattr(L, f).restype = ctypes.c_int
    mlp = ctypes.POINTER(CMlaLayer)
    L.nvfp4_mla_quantize_append.argtypes = [mlp, vp, ctypes.c_int, i32, i64, vp, vp]
    L.nvfp4_mla_quantize_append.restype = ctypes.c_int
    L.nvfp4_mla_sparse_decode_workspace_bytes.argtypes = [i32, i32, i32]
    L.nvfp4_mla_sparse_decode_workspace_bytes.restype = sz
    L.nvfp4_mla_sparse_decode.argtypes = [mlp, vp, ctypes.c_int, i32, i32, vp, i32, f32, vp, vp, sz, vp]
    L.nvfp4_mla_sparse_decode.restype = ctypes.c_int
    L.nvfp4_status_string.argtypes = [ctypes.c_int]
    L.nvfp4_status_string.restype = ctypes.c_char_p
    return L


lib = _load()


def status_string(status: int) -> str:
    return lib.nvfp4_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != NVFP4_OK:
        raise NVFP4Error(status, what)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _zeros_on(nbytes: int, device, stream) -> torch.Tensor:
    """A zero-filled byte buffer whose fill is queued on `stream` (torch's
    current stream when None), so a kernel launched there sees the zeros."""
    if stream is None:
        return torch.zeros(nbytes, dtype=torch.uint8, device=device)
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream), device=device)
    with torch.cuda.stream(s):
        return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _dev_i32(t: torch.Tensor, name: str):
    if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 device tensor")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise ValueError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


@dataclass
class KVCacheLayer:
    """One layer's paged NVFP4 cache: four byte planes in device memory."""

    k_codes: torch.Tensor
    k_scales: torch.Tensor
    v_codes: torch.Tensor
    v_scales: torch.Tensor
    num_pages: int
    num_kv_heads: int
    k_global: float
    v_global: float

    @staticmethod
    def allocate(num_pages: int, num_kv_heads: int, k_global: float, v_global: float,
                 device="cuda") -> "KVCacheLayer":
        n = int(num_pages) * int(num_kv_heads)
        z = lambda per: torch.zeros(n * per, dtype=torch.uint8, device=device)
        return KVCacheLayer(z(TILE_CODE_BYTES), z(TILE_SCALE_BYTES), z(TILE_CODE_BYTES), z(TILE_SCALE_BYTES),
                            int(num_pages), int(num_kv_heads), float(k_global), float(v_global))

    def c_struct(self) -> CKVLayer:
        return CKVLayer(self.k_codes.data_ptr(), self.k_scales.data_ptr(), self.v_codes.data_ptr(),
                        self.v_scales.data_ptr(), self.num_pages, self.num_kv_heads, HEAD_DIM, PAGE_SIZE,
                        self.k_global, self.v_global)

    @property
    def nbytes(self) -> int:
        return sum(t.numel() for t in (self.k_codes, self.k_scales, self.v_codes, self.v_scales))


def _check_new_kv(layer, k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor) -> int:
    """Validate new K/V and their slots; returns the token stride in elements."""
    if k.shape != v.shape or k.dtype != v.dtype or k.stride() != v.stride():
        raise ValueError("k and v must have the same shape, dtype and strides")
    T = k.shape[0]
    _dev_i32(slot_mapping, "slot_mapping")
    if slot_mapping.numel() != T:
        raise ValueError("slot_mapping must have one entry per token")
    if k.dim() == 3:
        if (k.shape[1:] != (layer.num_kv_heads, HEAD_DIM) or k.stride(2) != 1
                or (k.shape[1] > 1 and k.stride(1) != HEAD_DIM)):
            raise ValueError("k/v must be [T, H, 128] with contiguous heads")
    elif k.dim() != 2 or k.shape[1] != layer.num_kv_heads * HEAD_DIM or k.stride(1) != 1:
        raise ValueError("k/v must be [T, H, 128] or [T, H*128]")
    return k.stride(0) if T > 0 else layer.num_kv_heads * HEAD_DIM


def quantize_append(layer: KVCacheLayer, k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                    stream=None, hadamard: bool = False) -> None:
    """Quantize k, v ([T, H, 128] or [T, H*128], bf16/f32, token-strided) into their slots.

    hadamard: rotate the K rows (H k / 16) before quantization; read such a cache with hadamard=True."""
    stride = _check_new_kv(layer, k, v, slot_mapping)
    c = layer.c_struct()
    name = "nvfp4_kv_quantize_append_hadamard" if hadamard else "nvfp4_kv_quantize_append"
    st = getattr(lib, name)(ctypes.byref(c), _ptr(k), _ptr(v), _dtype_code(k), k.shape[0], stride,
                            _ptr(slot_mapping), _stream(stream))
    _check(st, name)


def decode_workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int, max_seq_len: int) -> int:
    return int(lib.nvfp4_paged_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, max_seq_len))


def decode_workspace(batch: int, num_q_heads: int, num_kv_heads: int, max_seq_len: int, device="cuda",
                     stream=None) -> torch.Tensor:
    """A zero-filled decode workspace (the library keeps it zeroed between calls),
    filled on `stream` (torch's current stream when None).  Allocate it once and
    pass it to every call on that stream."""
    need = max(decode_workspace_bytes(batch, num_q_heads, num_kv_heads, max_seq_len), 256)
    return _zeros_on(need, device, stream)


def paged_decode_attn(layer: KVCacheLayer, q: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                      max_seq_len: int, sm_scale: float, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, stream=None, hadamard: bool = False) -> torch.Tensor:
    """Decode attention of q [B, Hq, 128] (bf16/f32) over the cache; returns f32 [B, Hq, 128].

    hadamard: the cache holds rotated K (quantize_append(..., hadamard=True)); q is rotated alike."""
    out, workspace, ws_bytes = _decode_args(layer, q, block_table, seq_lens, max_seq_len, out, workspace, stream)
    c = layer.c_struct()
    name = "nvfp4_paged_decode_attn_hadamard" if hadamard else "nvfp4_paged_decode_attn"
    st = getattr(lib, name)(ctypes.byref(c), _ptr(q), _dtype_code(q), q.shape[0], q.shape[1],
                            _ptr(block_table), block_table.shape[1], _ptr(seq_lens), int(max_seq_len),
                            float(sm_scale), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, name)
    return out


def paged_decode_attn_noalloc(layer: KVCacheLayer, q: torch.Tensor, block_table: torch.Tensor,
                              seq_lens: torch.Tensor, max_seq_len: int, sm_scale: float, out: torch.Tensor,
                              stream=None) -> torch.Tensor:
    """paged_decode_attn with the library's own device scratch as its workspace:
    nothing is allocated (out [B, Hq, 128] float32 is the caller's).  Calls on
    one GPU share that scratch and must be ordered."""
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Hq, 128] tensor")
    B, Hq, _ = q.shape
    _dev_i32(block_table, "block_table")
    _dev_i32(seq_lens, "seq_lens")
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.numel() != B:
        raise ValueError("block_table must be [B, stride] and seq_lens [B]")
    if out.dtype != torch.float32 or not out.is_contiguous() or out.shape != (B, Hq, HEAD_DIM):
        raise ValueError("out must be a contiguous float32 [B, Hq, 128] tensor")
    c = layer.c_struct()
    st = lib.nvfp4_paged_decode_attn_noalloc(ctypes.byref(c), _ptr(q), _dtype_code(q), B, Hq, _ptr(block_table),
                                             block_table.shape[1], _ptr(seq_lens), int(max_seq_len),
                                             float(sm_scale), _ptr(out), _stream(stream))
    _check(st, "nvfp4_paged_decode_attn_noalloc")
    return out


def _decode_args(layer, q, block_table, seq_lens, max_seq_len, out, workspace, stream):
    """Validate one-token decode arguments; allocate out / workspace when not given
    (a fresh workspace is zero-filled on the call's stream)."""
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Hq, 128] tensor")
    B, Hq, _ = q.shape
    _dev_i32(block_table, "block_table")
    _dev_i32(seq_lens, "seq_lens")
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.numel() != B:
        raise ValueError("block_table must be [B, stride] and seq_lens [B]")
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or not out.is_contiguous() or out.shape != (B, Hq, HEAD_DIM):
        raise ValueError("out must be a contiguous float32 [B, Hq, 128] tensor")
    need = decode_workspace_bytes(B, Hq, layer.num_kv_heads, max_seq_len)
    if workspace is None and need > 0:
        workspace = decode_workspace(B, Hq, layer.num_kv_heads, max_seq_len, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return out, workspace, ws_bytes


def decode_multi_workspace_bytes(batch: int, q_per_seq: int, num_q_heads: int, num_kv_heads: int,
                                 max_seq_len: int) -> int:
    return int(lib.nvfp4_paged_decode_multi_workspace_bytes(batch, q_per_seq, num_q_heads, num_kv_heads, max_seq_len))


def paged_decode_attn_multi(layer: KVCacheLayer, q: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                            max_seq_len: int, sm_scale: float, out: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Decode of q [B, T, Hq, 128] (T new tokens per sequence, causal among them); returns f32 [B, T, Hq, 128]."""
    if q.dim() != 4 or q.shape[3] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, T, Hq, 128] tensor")
    B, T, Hq, _ = q.shape
    _dev_i32(block_table, "block_table")
    _dev_i32(seq_lens, "seq_lens")
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.numel() != B:
        raise ValueError("block_table must be [B, stride] and seq_lens [B]")
    if out is None:
        out = torch.empty((B, T, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or not out.is_contiguous() or out.shape != (B, T, Hq, HEAD_DIM):
        raise ValueError("out must be a contiguous float32 [B, T, Hq, 128] tensor")
    need = decode_multi_workspace_bytes(B, T, Hq, layer.num_kv_heads, max_seq_len)
    if workspace is None and need > 0:
        workspace = _zeros_on(max(need, 256), q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    c = layer.c_struct()
    st = lib.nvfp4_paged_decode_attn_multi(ctypes.byref(c), _ptr(q), _dtype_code(q), B, T, Hq, _ptr(block_table),
                                           block_table.shape[1], _ptr(seq_lens), int(max_seq_len), float(sm_scale),
                                           _ptr(out), _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "nvfp4_paged_decode_attn_multi")
    return out


def paged_decode_step(layer: KVCacheLayer, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                      block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, sm_scale: float,
                      out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """One decode step in one call: append k_new, v_new [B, T, H, 128] at the last T positions
    (seq_lens counts them) and attend with q [B, T, Hq, 128]; returns f32 [B, T, Hq, 128]."""
    if q.dim() != 4 or q.shape[3] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, T, Hq, 128] tensor")
    B, T, Hq, _ = q.shape
    for x in (k_new, v_new):
        if x.shape != (B, T, layer.num_kv_heads, HEAD_DIM) or x.dtype != q.dtype or not x.is_contiguous():
            raise ValueError("k_new / v_new must be contiguous [B, T, H, 128] tensors of the query's dtype")
    _dev_i32(block_table, "block_table")
    _dev_i32(seq_lens, "seq_lens")
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.numel() != B:
        raise ValueError("block_table must be [B, stride] and seq_lens [B]")
    if out is None:
        out = torch.empty((B, T, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or not out.is_contiguous() or out.shape != (B, T, Hq, HEAD_DIM):
        raise ValueError("out must be a contiguous float32 [B, T, Hq, 128] tensor")
    need = decode_multi_workspace_bytes(B, T, Hq, layer.num_kv_heads, max_seq_len)
    if workspace is None and need > 0:
        workspace = _zeros_on(max(need, 256), q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    c = layer.c_struct()
    st = lib.nvfp4_paged_decode_step(ctypes.byref(c), _ptr(k_new), _ptr(v_new), _ptr(q), _dtype_code(q), B, T, Hq,
                                     _ptr(block_table), block_table.shape[1], _ptr(seq_lens), int(max_seq_len),
                                     float(sm_scale), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "nvfp4_paged_decode_step")
    return out


def dequant_to_fp8_workspace(layer: KVCacheLayer, block_table: torch.Tensor, prefix_lens: torch.Tensor,
                             ws_offsets: torch.Tensor, max_prefix_len: int, k_ws_scale: float, v_ws_scale: float,
                             ws_k: torch.Tensor, ws_v: torch.Tensor, stream=None) -> None:
    """Dequantize the cached prefixes into the FP8 E4M3 workspace pair ws_k, ws_v [cap, H, 128] (uint8)."""
    _dev_i32(block_table, "block_table")
    _dev_i32(prefix_lens, "prefix_lens")
    _dev_i32(ws_offsets, "ws_offsets")
    n = prefix_lens.numel()
    if block_table.dim() != 2 or block_table.shape[0] != n or ws_offsets.numel() != n + 1:
        raise ValueError("block_table [n, stride], prefix_lens [n], ws_offsets [n+1]")
    for w in (ws_k, ws_v):
        if w.dtype not in (torch.uint8, torch.float8_e4m3fn) or not w.is_contiguous():
            raise ValueError("workspace must be contiguous uint8 / float8_e4m3fn")
        if w.dim() != 3 or w.shape[1:] != (layer.num_kv_heads, HEAD_DIM):
            raise ValueError("workspace must be [capacity, H, 128]")
    if ws_k.shape != ws_v.shape:
        raise ValueError("ws_k and ws_v must have the same shape")
    c = layer.c_struct()
    st = lib.nvfp4_dequant_to_fp8_workspace(ctypes.byref(c), _ptr(block_table), block_table.shape[1], n,
                                            _ptr(prefix_lens), _ptr(ws_offsets), int(max_prefix_len),
                                            float(k_ws_scale), float(v_ws_scale), _ptr(ws_k), _ptr(ws_v),
                                            ws_k.shape[0], _stream(stream))
    _check(st, "nvfp4_dequant_to_fp8_workspace")


def _check_ws_pair(ws_k: torch.Tensor, ws_v: torch.Tensor):
    for w in (ws_k, ws_v):
        if w.dtype not in (torch.uint8, torch.float8_e4m3fn) or not w.is_contiguous():
            raise ValueError("workspace must be contiguous uint8 / float8_e4m3fn")
        if w.dim() != 3 or w.shape[2] != HEAD_DIM:
            raise ValueError("workspace must be [capacity, H, 128]")
    if ws_k.shape != ws_v.shape:
        raise ValueError("ws_k and ws_v must have the same shape")


def fp8_rows_to_workspace(k: torch.Tensor, v: torch.Tensor, ws_rows: torch.Tensor, k_ws_scale: float,
                          v_ws_scale: float, ws_k: torch.Tensor, ws_v: torch.Tensor, stream=None) -> None:
    """Store new tokens' k, v ([T, H, 128], bf16/f32, token-strided) as E4M3 rows ws_rows of ws_k, ws_v."""
    if k.shape != v.shape or k.dtype != v.dtype or k.stride() != v.stride():
        raise ValueError("k and v must have the same shape, dtype and strides")
    _check_ws_pair(ws_k, ws_v)
    _dev_i32(ws_rows, "ws_rows")
    T = k.shape[0]
    if k.dim() != 3 or k.shape[1:] != (ws_k.shape[1], HEAD_DIM) or k.stride(2) != 1 or \
            (k.shape[1] > 1 and k.stride(1) != HEAD_DIM):
        raise ValueError("k/v must be [T, H, 128] with contiguous heads, H matching the workspace")
    if ws_rows.numel() != T:
        raise ValueError("ws_rows must have one entry per token")
    st = lib.nvfp4_fp8_rows_to_workspace(_ptr(k), _ptr(v), _dtype_code(k), T,
                                         k.stride(0) if T > 0 else ws_k.shape[1] * HEAD_DIM, ws_k.shape[1],
                                         _ptr(ws_rows), float(k_ws_scale), float(v_ws_scale), _ptr(ws_k), _ptr(ws_v),
                                         ws_k.shape[0], _stream(stream))
    _check(st, "nvfp4_fp8_rows_to_workspace")


def _extend_args(q, q_offsets, ws_offsets, prefix_lens, ws_k, ws_v, out):
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [Tq, Hq, 128] tensor")
    _check_ws_pair(ws_k, ws_v)
    for t, name in ((q_offsets, "q_offsets"), (ws_offsets, "ws_offsets"), (prefix_lens, "prefix_lens")):
        _dev_i32(t, name)
    n = prefix_lens.numel()
    if q_offsets.numel() != n + 1 or ws_offsets.numel() != n:
        raise ValueError("q_offsets [n+1], ws_offsets [n], prefix_lens [n]")
    Tq, Hq, _ = q.shape
    if out is None:
        out = torch.empty((Tq, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or not out.is_contiguous() or out.shape != (Tq, Hq, HEAD_DIM):
        raise ValueError("out must be a contiguous float32 [Tq, Hq, 128] tensor")
    return n, Tq, Hq, out


def fp8_extend_attn(q: torch.Tensor, q_offsets: torch.Tensor, ws_offsets: torch.Tensor, prefix_lens: torch.Tensor,
                    max_chunk_len: int, ws_k: torch.Tensor, ws_v: torch.Tensor, k_ws_scale: float, v_ws_scale: float,
                    sm_scale: float, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Causal attention of chunk queries q [Tq, Hq, 128] over FP8 workspace rows; returns f32 [Tq, Hq, 128]."""
    n, Tq, Hq, out = _extend_args(q, q_offsets, ws_offsets, prefix_lens, ws_k, ws_v, out)
    st = lib.nvfp4_fp8_extend_attn(_ptr(q), _dtype_code(q), Tq, Hq, ws_k.shape[1], n, _ptr(q_offsets),
                                   _ptr(ws_offsets), _ptr(prefix_lens), int(max_chunk_len), _ptr(ws_k), _ptr(ws_v),
                                   ws_k.shape[0], float(k_ws_scale), float(v_ws_scale), float(sm_scale), _ptr(out),
                                   _stream(stream))
    _check(st, "nvfp4_fp8_extend_attn")
    return out


def fp8_extend_attn_split_workspace_bytes(q_dtype: torch.dtype, num_q_tokens: int, num_q_heads: int,
                                          num_kv_heads: int, num_seqs: int, max_chunk_len: int,
                                          max_prefix_len: int) -> int:
    code = {torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_F32}.get(q_dtype)
    if code is None:
        raise ValueError(f"unsupported q dtype {q_dtype} (bfloat16 or float32)")
    return int(lib.nvfp4_fp8_extend_attn_split_workspace_bytes(code, num_q_tokens, num_q_heads, num_kv_heads,
                                                                num_seqs, max_chunk_len, max_prefix_len))


def fp8_extend_attn_f8_workspace_bytes(q_dtype: torch.dtype, num_q_tokens: int, num_q_heads: int,
                                       num_kv_heads: int, num_seqs: int, max_chunk_len: int,
                                       max_prefix_len: int) -> int:
    code = {torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_F32}.get(q_dtype)
    if code is None:
        raise ValueError(f"unsupported q dtype {q_dtype} (bfloat16 or float32)")
    return int(lib.nvfp4_fp8_extend_attn_f8_workspace_bytes(code, num_q_tokens, num_q_heads, num_kv_heads,
                                                             num_seqs, max_chunk_len, max_prefix_len))


def fp8_extend_attn_f8(q: torch.Tensor, q_offsets: torch.Tensor, ws_offsets: torch.Tensor, prefix_lens: torch.Tensor,
                       max_chunk_len: int, max_prefix_len: int, ws_k: torch.Tensor, ws_v: torch.Tensor,
                       k_ws_scale: float, v_ws_scale: float, sm_scale: float, out: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """fp8_extend_attn in FP8 arithmetic (Q and the softmax weights rounded to E4M3, FP8 MFMA);
    workspace: device bytes of fp8_extend_attn_f8_workspace_bytes (allocated when needed and not given)."""
    n, Tq, Hq, out = _extend_args(q, q_offsets, ws_offsets, prefix_lens, ws_k, ws_v, out)
    need = fp8_extend_attn_f8_workspace_bytes(q.dtype, Tq, Hq, ws_k.shape[1], n, int(max_chunk_len),
                                              int(max_prefix_len))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.nvfp4_fp8_extend_attn_f8(_ptr(q), _dtype_code(q), Tq, Hq, ws_k.shape[1], n, _ptr(q_offsets),
                                      _ptr(ws_offsets), _ptr(prefix_lens), int(max_chunk_len), int(max_prefix_len),
                                      _ptr(ws_k), _ptr(ws_v), ws_k.shape[0], float(k_ws_scale), float(v_ws_scale),
                                      float(sm_scale), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "nvfp4_fp8_extend_attn_f8")
    return out


def fp8_extend_attn_split(q: torch.Tensor, q_offsets: torch.Tensor, ws_offsets: torch.Tensor,
                          prefix_lens: torch.Tensor, max_chunk_len: int, max_prefix_len: int, ws_k: torch.Tensor,
                          ws_v: torch.Tensor, k_ws_scale: float, v_ws_scale: float, sm_scale: float,
                          out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                          stream=None) -> torch.Tensor:
    """fp8_extend_attn with each tile's keys shared among workgroups when the chunks are few tiles
    (short chunks over long prefixes); workspace: device bytes of fp8_extend_attn_split_workspace_bytes."""
    n, Tq, Hq, out = _extend_args(q, q_offsets, ws_offsets, prefix_lens, ws_k, ws_v, out)
    need = fp8_extend_attn_split_workspace_bytes(q.dtype, Tq, Hq, ws_k.shape[1], n, int(max_chunk_len),
                                                 int(max_prefix_len))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.nvfp4_fp8_extend_attn_split(_ptr(q), _dtype_code(q), Tq, Hq, ws_k.shape[1], n, _ptr(q_offsets),
                                         _ptr(ws_offsets), _ptr(prefix_lens), int(max_chunk_len), int(max_prefix_len),
                                         _ptr(ws_k), _ptr(ws_v), ws_k.shape[0], float(k_ws_scale), float(v_ws_scale),
                                         float(sm_scale), _ptr(out), _ptr(workspace),
                                         ws_bytes, _stream(stream))
    _check(st, "nvfp4_fp8_extend_attn_split")
    return out


# -------------------------------------------------------------------- MXFP4
@dataclass
class MxKVCacheLayer:
    """One layer's paged MXFP4 cache: NVFP4-layout code planes and 64-byte E8M0 scale tiles."""

    k_codes: torch.Tensor
    k_scales: torch.Tensor
    v_codes: torch.Tensor
    v_scales: torch.Tensor
    num_pages: int
    num_kv_heads: int

    @staticmethod
    def allocate(num_pages: int, num_kv_heads: int, device="cuda") -> "MxKVCacheLayer":
        n = int(num_pages) * int(num_kv_heads)
        z = lambda per: torch.zeros(n * per, dtype=torch.uint8, device=device)
        return MxKVCacheLayer(z(TILE_CODE_BYTES), z(MX_TILE_SCALE_BYTES), z(TILE_CODE_BYTES), z(MX_TILE_SCALE_BYTES),
                              int(num_pages), int(num_kv_heads))

    def c_struct(self) -> CMxLayer:
        return CMxLayer(self.k_codes.data_ptr(), self.k_scales.data_ptr(), self.v_codes.data_ptr(),
                        self.v_scales.data_ptr(), self.num_pages, self.num_kv_heads, HEAD_DIM, PAGE_SIZE)

    @property
    def nbytes(self) -> int:
        return sum(t.numel() for t in (self.k_codes, self.k_scales, self.v_codes, self.v_scales))


def mx_quantize_append(layer: MxKVCacheLayer, k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                       stream=None, hadamard: bool = False) -> None:
    """MXFP4 quantize-append of k, v (shapes as quantize_append) into their slots."""
    stride = _check_new_kv(layer, k, v, slot_mapping)
    c = layer.c_struct()
    name = "mxfp4_kv_quantize_append_hadamard" if hadamard else "mxfp4_kv_quantize_append"
    st = getattr(lib, name)(ctypes.byref(c), _ptr(k), _ptr(v), _dtype_code(k), k.shape[0], stride,
                            _ptr(slot_mapping), _stream(stream))
    _check(st, name)


def mx_paged_decode_attn(layer: MxKVCacheLayer, q: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                         max_seq_len: int, sm_scale: float, out: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None, stream=None, hadamard: bool = False) -> torch.Tensor:
    """Decode attention of q [B, Hq, 128] over MXFP4 pages; returns f32 [B, Hq, 128]."""
    out, workspace, ws_bytes = _decode_args(layer, q, block_table, seq_lens, max_seq_len, out, workspace, stream)
    c = layer.c_struct()
    name = "mxfp4_paged_decode_attn_hadamard" if hadamard else "mxfp4_paged_decode_attn"
    st = getattr(lib, name)(ctypes.byref(c), _ptr(q), _dtype_code(q), q.shape[0], q.shape[1],
                            _ptr(block_table), block_table.shape[1], _ptr(seq_lens), int(max_seq_len),
                            float(sm_scale), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, name)
    return out


# --------------------------------------------------- Sparse-MLA latent cache
MLA_DIM = 576            # latent (512) + rotary key (64) values per token row
MLA_LATENT = 512
MLA_ROW_CODE_BYTES = 288
MLA_ROW_SCALE_BYTES = 36


@dataclass
class MlaCacheLayer:
    """One layer's NVFP4 latent cache: codes [num_slots, 288] and scales [num_slots, 36] (device)."""

    codes: torch.Tensor
    scales: torch.Tensor
    num_slots: int
    global_scale: float

    @staticmethod
    def allocate(num_slots: int, global_scale: float, device="cuda") -> "MlaCacheLayer":
        n = int(num_slots)
        return MlaCacheLayer(torch.zeros((n, MLA_ROW_CODE_BYTES), dtype=torch.uint8, device=device),
                             torch.zeros((n, MLA_ROW_SCALE_BYTES), dtype=torch.uint8, device=device),
                             n, float(global_scale))

    def c_struct(self) -> CMlaLayer:
        return CMlaLayer(self.codes.data_ptr(), self.scales.data_ptr(), self.num_slots, MLA_LATENT,
                         MLA_DIM - MLA_LATENT, self.global_scale)


def mla_quantize_append(layer: MlaCacheLayer, kv: torch.Tensor, slot_mapping: torch.Tensor, stream=None) -> None:
    """Quantize latent rows kv [T, 576] (bf16/f32, token-strided) into their slots."""
    if kv.dim() != 2 or kv.shape[1] != MLA_DIM or kv.stride(1) != 1:
        raise ValueError("kv must be [T, 576] with contiguous rows")
    _dev_i32(slot_mapping, "slot_mapping")
    if slot_mapping.numel() != kv.shape[0]:
        raise ValueError("slot_mapping must have one entry per token")
    c = layer.c_struct()
    T = kv.shape[0]
    st = lib.nvfp4_mla_quantize_append(ctypes.byref(c), _ptr(kv), _dtype_code(kv), T,
                                       kv.stride(0) if T > 0 else MLA_DIM, _ptr(slot_mapping), _stream(stream))
    _check(st, "nvfp4_mla_quantize_append")


def mla_sparse_decode_workspace_bytes(num_q_tokens: int, num_q_heads: int, topk: int) -> int:
    return int(lib.nvfp4_mla_sparse_decode_workspace_bytes(num_q_tokens, num_q_heads, topk))


def mla_sparse_decode(layer: MlaCacheLayer, q: torch.Tensor, indices: torch.Tensor, sm_scale: float,
                      out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """Sparse MLA decode of q [T, Hq, 576] (bf16) over the cache slots indices [T, topk];
    returns f32 [T, Hq, 512]."""
    if q.dim() != 3 or q.shape[2] != MLA_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [T, Hq, 576] tensor")
    T, Hq, _ = q.shape
    _dev_i32(indices, "indices")
    if indices.dim() != 2 or indices.shape[0] != T:
        raise ValueError("indices must be [T, topk]")
    if out is None:
        out = torch.empty((T, Hq, MLA_LATENT), dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or not out.is_contiguous() or out.shape != (T, Hq, MLA_LATENT):
        raise ValueError("out must be a contiguous float32 [T, Hq, 512] tensor")
    need = mla_sparse_decode_workspace_bytes(T, Hq, indices.shape[1])
    if workspace is None and need > 0:  # partials of split lists: no initial contents needed
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    c = layer.c_struct()
    st = lib.nvfp4_mla_sparse_decode(ctypes.byref(c), _ptr(q), _dtype_code(q), T, Hq, _ptr(indices),
                                     indices.shape[1], float(sm_scale), _ptr(out), _ptr(workspace), ws_bytes,
                                     _stream(stream))
    _check(st, "nvfp4_mla_sparse_decode")
    return out
