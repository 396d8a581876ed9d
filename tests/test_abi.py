"""The C ABI without a GPU: the library loads, exports every function the
public header declares, and every argument check returns its status before
any HIP call (so these run on a machine with no GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4_kv.h")


def _lib():
    import nvfp4_quantized_paged_kv_amd as nk

    return nk


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"NVFP4_API\s+[\w\s\*]+?\b((?:nvfp4|mxfp4)_\w+)\s*\(", text)))


def test_header_declares_the_three_entry_points():
    fns = _declared_functions()
    for f in ("nvfp4_kv_quantize_append", "nvfp4_paged_decode_attn", "nvfp4_dequant_to_fp8_workspace"):
        assert f in fns


def test_library_exports_every_declared_symbol():
    nk = _lib()
    raw = ctypes.CDLL(nk.LIB_PATH)
    for f in _declared_functions():
        assert hasattr(raw, f), f
    assert set(_declared_functions()) == set(nk.EXPORTED_SYMBOLS)


def test_status_strings():
    nk = _lib()
    for s in range(5):
        assert nk.status_string(s) and nk.status_string(s) != "unknown status"
    assert nk.status_string(99) == "unknown status"


# A fake layer with plausible (never dereferenced) aligned addresses.
FAKE = 0x7F0000000000


def _layer(nk, **kw):
    d = dict(k_codes=FAKE, k_scales=FAKE + 0x100000, v_codes=FAKE + 0x200000, v_scales=FAKE + 0x300000,
             num_pages=10, num_kv_heads=8, head_dim=128, page_size=16, k_global=0.01, v_global=0.02)
    d.update(kw)
    return nk.CKVLayer(**d)


def _append(nk, layer, k=FAKE, v=FAKE, dtype=1, T=4, stride=1024, slots=FAKE):
    return nk.lib.nvfp4_kv_quantize_append(ctypes.byref(layer) if layer is not None else None,
                                           ctypes.c_void_p(k), ctypes.c_void_p(v), dtype, T, stride,
                                           ctypes.c_void_p(slots), None)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), 2), (dict(page_size=32), 2), (dict(k_codes=0), 1), (dict(num_pages=0), 1),
    (dict(num_kv_heads=0), 1), (dict(k_global=0.0), 1), (dict(v_global=float("inf")), 1),
    (dict(k_global=float("nan")), 1), (dict(k_global=1e-35), 1), (dict(k_codes=FAKE + 8), 2),
    (dict(v_scales=FAKE + 2), 2), (dict(num_pages=1 << 28), 2),
])
def test_layer_checks(kw, status):
    nk = _lib()
    assert _append(nk, _layer(nk, **kw)) == status


def test_append_checks():
    nk = _lib()
    L = _layer(nk)
    assert nk.lib.nvfp4_kv_quantize_append(None, None, None, 1, 1, 1024, None, None) == 1
    assert _append(nk, L, T=0, k=0, v=0, slots=0) == 0  # empty append is a no-op
    assert _append(nk, L, T=-1) == 1
    assert _append(nk, L, dtype=7) == 1
    assert _append(nk, L, k=0) == 1
    assert _append(nk, L, slots=0) == 1
    assert _append(nk, L, stride=1023) == 1  # < H*128
    assert _append(nk, L, k=FAKE + 4) == 2  # misaligned input
    assert _append(nk, L, stride=1028, dtype=1) == 2  # token stride not a multiple of 16 bytes


def _decode(nk, layer, q=FAKE, qdt=1, B=2, Hq=64, bt=FAKE, bts=4, sl=FAKE, msl=64, sm=0.088, out=FAKE,
            ws=FAKE, wsb=1 << 30):
    return nk.lib.nvfp4_paged_decode_attn(ctypes.byref(layer), ctypes.c_void_p(q), qdt, B, Hq, ctypes.c_void_p(bt),
                                          bts, ctypes.c_void_p(sl), msl, sm, ctypes.c_void_p(out),
                                          ctypes.c_void_p(ws), wsb, None)


def test_decode_checks():
    nk = _lib()
    L = _layer(nk)
    assert _decode(nk, L, Hq=60) == 1          # not a multiple of num_kv_heads
    assert _decode(nk, L, Hq=8 * 17) == 2      # more than 16 q heads per kv head
    assert _decode(nk, L, qdt=3) == 1
    assert _decode(nk, L, B=-1) == 1
    assert _decode(nk, L, B=0, q=0, bt=0, sl=0, out=0) == 0  # empty batch
    assert _decode(nk, L, q=0) == 1
    assert _decode(nk, L, out=0) == 1
    assert _decode(nk, L, bts=3) == 1          # 3*16 < max_seq_len 64
    assert _decode(nk, L, sm=float("inf")) == 1
    assert _decode(nk, L, q=FAKE + 2) == 2
    assert _decode(nk, L, B=4097, bts=4) == 2  # more sequences than one launch handles
    assert _decode(nk, L, B=4096, msl=1 << 20, bts=1 << 16) == 2  # 2^31 (sequence, head, page) items
    assert _decode(nk, L, ws=FAKE + 16) == 1   # workspace must be 256-byte aligned
    # workspace: too small, or missing when needed
    need = nk.decode_workspace_bytes(1, 64, 8, 1 << 20)
    assert need > 0
    assert _decode(nk, L, B=1, msl=1 << 20, bts=1 << 16, wsb=need - 1) == 3
    assert _decode(nk, L, B=1, msl=1 << 20, bts=1 << 16, ws=0, wsb=need) == 1


def test_decode_workspace_size_rules():
    nk = _lib()
    assert nk.decode_workspace_bytes(0, 64, 8, 8192) == 0
    assert nk.decode_workspace_bytes(32, 64, 8, 0) > 0               # counters even for an empty context
    assert nk.decode_workspace_bytes(32, 60, 8, 8192) == 0          # invalid grouping
    assert nk.decode_workspace_bytes(4097, 64, 8, 8192) == 0        # batch limit
    assert nk.decode_workspace_bytes(4096, 64, 8, 1 << 20) == 0     # over 2^30 work slots
    assert nk.decode_workspace_bytes(2000, 64, 8, 1 << 20) > 0      # just under 2^30 work slots
    assert nk.decode_workspace_bytes(1, 96, 8, 2_000_000) > 0        # a long context needs split partials
    # monotone in the context bound for a fixed batch
    sizes = [nk.decode_workspace_bytes(4, 32, 8, n) for n in (1 << 14, 1 << 16, 1 << 18, 1 << 20)]
    assert sizes == sorted(sizes)


def _ws(nk, layer, bt=FAKE, bts=8, n=2, pl=FAKE, wo=FAKE, mpl=100, ks=1.0, vs=1.0, wk=FAKE, wv=FAKE, cap=1000):
    return nk.lib.nvfp4_dequant_to_fp8_workspace(ctypes.byref(layer), ctypes.c_void_p(bt), bts, n,
                                                 ctypes.c_void_p(pl), ctypes.c_void_p(wo), mpl, ks, vs,
                                                 ctypes.c_void_p(wk), ctypes.c_void_p(wv), cap, None)


def test_workspace_dequant_checks():
    nk = _lib()
    L = _layer(nk)
    assert _ws(nk, L, n=-1) == 1
    assert _ws(nk, L, mpl=-1) == 1
    assert _ws(nk, L, cap=-1) == 1
    assert _ws(nk, L, ks=0.0) == 1
    assert _ws(nk, L, vs=float("nan")) == 1
    assert _ws(nk, L, n=0, bt=0, pl=0, wo=0, wk=0, wv=0) == 0  # nothing to do
    assert _ws(nk, L, wk=0) == 1
    assert _ws(nk, L, bts=6) == 1                              # 6*16 < 100
    assert _ws(nk, L, wv=FAKE + 4) == 2


def _rows(nk, k=FAKE, v=FAKE, dtype=1, T=4, stride=1024, H=8, rows=FAKE, ks=1.0, vs=1.0, wk=FAKE, wv=FAKE, cap=100):
    return nk.lib.nvfp4_fp8_rows_to_workspace(ctypes.c_void_p(k), ctypes.c_void_p(v), dtype, T, stride, H,
                                              ctypes.c_void_p(rows), ks, vs, ctypes.c_void_p(wk), ctypes.c_void_p(wv),
                                              cap, None)


def test_fp8_rows_checks():
    nk = _lib()
    assert _rows(nk, dtype=7) == 1
    assert _rows(nk, T=-1) == 1
    assert _rows(nk, H=0) == 1
    assert _rows(nk, cap=-1) == 1
    assert _rows(nk, ks=float("inf")) == 1
    assert _rows(nk, vs=-1.0) == 1
    assert _rows(nk, T=0, k=0, v=0, rows=0, wk=0, wv=0) == 0    # nothing to do
    assert _rows(nk, cap=0, k=0, v=0, rows=0, wk=0, wv=0) == 0  # nothing can be written
    assert _rows(nk, rows=0) == 1
    assert _rows(nk, stride=1000) == 1                           # < H*128
    assert _rows(nk, k=FAKE + 8) == 2
    assert _rows(nk, stride=1028) == 2                           # rows not 16-byte aligned
    assert _rows(nk, wv=FAKE + 2) == 2


def _ext(nk, q=FAKE, dt=1, nq=64, hq=64, h=8, n=2, qo=FAKE, wo=FAKE, pl=FAKE, mc=32, wk=FAKE, wv=FAKE, cap=1000,
         ks=1.0, vs=1.0, sm=0.088, out=FAKE):
    return nk.lib.nvfp4_fp8_extend_attn(ctypes.c_void_p(q), dt, nq, hq, h, n, ctypes.c_void_p(qo), ctypes.c_void_p(wo),
                                        ctypes.c_void_p(pl), mc, ctypes.c_void_p(wk), ctypes.c_void_p(wv), cap, ks, vs,
                                        sm, ctypes.c_void_p(out), None)


def test_fp8_extend_checks():
    nk = _lib()
    assert _ext(nk, dt=3) == 1
    assert _ext(nk, hq=60) == 1                 # not a multiple of the kv heads
    assert _ext(nk, hq=8 * 17) == 2             # more than 16 query heads per kv head
    assert _ext(nk, h=70000, hq=70000) == 2     # grid limit
    assert _ext(nk, n=70000) == 2
    assert _ext(nk, n=-1) == 1
    assert _ext(nk, mc=-1) == 1
    assert _ext(nk, ks=0.0) == 1
    assert _ext(nk, sm=float("nan")) == 1
    assert _ext(nk, sm=3e38, ks=1e30) == 1      # logit scale overflows float32
    assert _ext(nk, n=0, q=0, qo=0, wo=0, pl=0, wk=0, wv=0, out=0) == 0
    assert _ext(nk, mc=0, q=0, out=0) == 0
    assert _ext(nk, out=0) == 1
    assert _ext(nk, pl=0) == 1
    assert _ext(nk, q=FAKE + 4) == 2
    assert _ext(nk, wk=FAKE + 8) == 2


def _ext_split(nk, q=FAKE, nq=64, hq=64, h=8, n=2, mc=4, mp=8192, ks=1.0, out=FAKE, ws=FAKE, wsb=1 << 26):
    return nk.lib.nvfp4_fp8_extend_attn_split(ctypes.c_void_p(q), 1, nq, hq, h, n, ctypes.c_void_p(FAKE),
                                              ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), mc, mp,
                                              ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), 1000, ks, 1.0, 0.088,
                                              ctypes.c_void_p(out), ctypes.c_void_p(ws), wsb, None)


def test_fp8_extend_split_checks_and_sizes():
    import torch

    nk = _lib()

    def size(*a, dtype=torch.bfloat16):
        return nk.fp8_extend_attn_split_workspace_bytes(dtype, *a)

    # short chunks over long prefixes: a split, one partial row of 132 floats per split, token and head
    need = size(64, 64, 8, 2, 4, 8192)
    assert need > 0 and need % 256 == 0
    splits = need // (64 * 64 * 132 * 4)
    assert 2 <= splits <= 256 and need == -(-splits * 64 * 64 * 132 * 4 // 256) * 256
    assert size(64, 64, 8, 2, 4, 0) == 0              # a 4-token chunk alone: not worth a split
    assert size(8192, 64, 8, 2, 4096, 8192) == 0      # enough tiles without one
    assert size(64, 60, 8, 2, 4, 8192) == 0           # invalid grouping
    assert size(0, 64, 8, 2, 4, 8192) == 0
    assert size(64, 64, 8, 2, 4, 1 << 16) >= need     # longer prefixes: no fewer splits
    # one round of resident workgroups: 3 per CU for bf16 queries, 2 for float32 ones
    assert size(64, 64, 8, 2, 4, 1 << 20) == 768 // 16 * 64 * 64 * 132 * 4
    assert size(64, 64, 8, 2, 4, 1 << 20, dtype=torch.float32) == 512 // 16 * 64 * 64 * 132 * 4
    assert nk.lib.nvfp4_fp8_extend_attn_split_workspace_bytes(7, 64, 64, 8, 2, 4, 8192) == 0  # no such dtype
    assert size(64, 8 * 17, 8, 2, 4, 8192) == 0       # more than 16 query heads per kv head
    # argument checks, all before any HIP call
    assert _ext_split(nk, mp=-1) == 1
    assert _ext_split(nk, ks=0.0) == 1
    assert _ext_split(nk, hq=60) == 1
    assert _ext_split(nk, q=FAKE + 4) == 2
    assert _ext_split(nk, out=0) == 1
    assert _ext_split(nk, wsb=need - 1) == 3           # workspace too small
    assert _ext_split(nk, ws=0) == 1                   # a needed workspace missing
    assert _ext_split(nk, ws=FAKE + 4) == 2            # misaligned workspace
    assert _ext_split(nk, n=0, q=0, out=0, ws=0, wsb=0) == 0


def test_fp8_extend_f8_checks_and_sizes():
    import torch

    nk = _lib()

    def size(*a, dtype=torch.bfloat16):
        return nk.fp8_extend_attn_f8_workspace_bytes(dtype, *a)

    need = size(64, 64, 8, 2, 4, 8192)
    assert need > 0 and need % 256 == 0
    # one round of resident workgroups: two 4-wave workgroups per CU (2 waves per SIMD)
    assert size(64, 64, 8, 2, 4, 1 << 20) == 512 // 16 * 64 * 64 * 132 * 4
    assert size(64, 128, 8, 2, 4, 1 << 20) == 256 // 16 * 64 * 128 * 132 * 4  # 8-wave workgroups: one per CU
    assert size(64, 64, 8, 2, 4, 0) == 0
    assert size(8192, 64, 8, 2, 4096, 8192) == 0
    assert size(64, 60, 8, 2, 4, 8192) == 0
    assert nk.lib.nvfp4_fp8_extend_attn_f8_workspace_bytes(7, 64, 64, 8, 2, 4, 8192) == 0

    def call(q=FAKE, hq=64, mp=8192, ks=1.0, out=FAKE, ws=FAKE, wsb=1 << 26, n=2):
        return nk.lib.nvfp4_fp8_extend_attn_f8(ctypes.c_void_p(q), 1, 64, hq, 8, n, ctypes.c_void_p(FAKE),
                                               ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), 4, mp,
                                               ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), 1000, ks, 1.0, 0.088,
                                               ctypes.c_void_p(out), ctypes.c_void_p(ws), wsb, None)
    assert call(mp=-1) == 1
    assert call(ks=0.0) == 1
    assert call(hq=60) == 1
    assert call(hq=8 * 17) == 2
    assert call(q=FAKE + 4) == 2
    assert call(out=0) == 1
    assert call(wsb=need - 1) == 3
    assert call(ws=0) == 1
    assert call(ws=FAKE + 4) == 2
    assert call(n=0, q=0, out=0, ws=0, wsb=0) == 0


def test_multi_token_decode_checks_and_sizes():
    nk = _lib()
    L = _layer(nk)

    def call(T=2, hq=64, ws=1 << 20, q=FAKE, dtype=1, batch=4):
        return nk.lib.nvfp4_paged_decode_attn_multi(ctypes.byref(L), ctypes.c_void_p(q), dtype, batch, T, hq,
                                                    ctypes.c_void_p(FAKE), 8, ctypes.c_void_p(FAKE), 100, 0.088,
                                                    ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), ws, None)
    assert call(T=0) == 1
    assert call(T=3) == 2            # 8 heads per kv head x 3 tokens > 16 rows
    assert call(hq=60) == 1
    assert call(q=FAKE + 4) == 2
    assert call(ws=16) == 3          # workspace too small
    assert call(batch=0) == 0
    m = nk.decode_multi_workspace_bytes
    assert m(32, 1, 64, 8, 8192) == nk.decode_workspace_bytes(32, 64, 8, 8192)
    assert m(32, 2, 64, 8, 8192) > nk.decode_workspace_bytes(32, 64, 8, 8192)   # 16 partial rows per unit, not 8
    assert m(32, 3, 64, 8, 8192) == 0 and m(32, 0, 64, 8, 8192) == 0
    assert m(4, 16, 16, 16, 100) > 0                                               # one head per kv head, 16 tokens


def test_decode_step_checks():
    nk = _lib()
    L = _layer(nk)

    def call(k=FAKE, v=FAKE, T=1, ws=1 << 20, batch=4):
        return nk.lib.nvfp4_paged_decode_step(ctypes.byref(L), ctypes.c_void_p(k), ctypes.c_void_p(v),
                                              ctypes.c_void_p(FAKE), 1, batch, T, 64, ctypes.c_void_p(FAKE), 8,
                                              ctypes.c_void_p(FAKE), 100, 0.088, ctypes.c_void_p(FAKE),
                                              ctypes.c_void_p(FAKE), ws, None)
    assert call(k=0) == 1 and call(v=0) == 1     # the new tokens are required
    assert call(k=FAKE + 4) == 2                   # alignment
    assert call(T=3) == 2                          # 8 heads per kv head x 3 tokens > 16 rows
    assert call(ws=16) == 3
    assert call(batch=0, k=0, v=0) == 0


# ---------------------------------------------------------------- MXFP4
def _mx_layer(nk, **kw):
    d = dict(k_codes=FAKE, k_scales=FAKE + 0x100000, v_codes=FAKE + 0x200000, v_scales=FAKE + 0x300000,
             num_pages=10, num_kv_heads=8, head_dim=128, page_size=16)
    d.update(kw)
    return nk.CMxLayer(**d)


def test_header_declares_the_mxfp4_entry_points():
    fns = _declared_functions()
    assert "mxfp4_kv_quantize_append" in fns and "mxfp4_paged_decode_attn" in fns


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), 2), (dict(page_size=32), 2), (dict(k_codes=0), 1), (dict(v_scales=0), 1),
    (dict(num_pages=0), 1), (dict(num_kv_heads=0), 1), (dict(k_codes=FAKE + 8), 2), (dict(k_scales=FAKE + 1), 2),
    (dict(num_pages=1 << 28), 2),
])
def test_mx_layer_checks(kw, status):
    nk = _lib()
    L = _mx_layer(nk, **kw)
    st = nk.lib.mxfp4_kv_quantize_append(ctypes.byref(L), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), 1, 4, 1024,
                                         ctypes.c_void_p(FAKE), None)
    assert st == status


def test_mx_append_and_decode_checks():
    nk = _lib()
    L = _mx_layer(nk)

    def app(k=FAKE, dtype=1, T=4, stride=1024, slots=FAKE):
        return nk.lib.mxfp4_kv_quantize_append(ctypes.byref(L), ctypes.c_void_p(k), ctypes.c_void_p(FAKE), dtype, T,
                                               stride, ctypes.c_void_p(slots), None)

    def dec(q=FAKE, B=2, Hq=64, bts=4, msl=64, sm=0.088, out=FAKE, ws=FAKE, wsb=1 << 30):
        return nk.lib.mxfp4_paged_decode_attn(ctypes.byref(L), ctypes.c_void_p(q), 1, B, Hq, ctypes.c_void_p(FAKE),
                                              bts, ctypes.c_void_p(FAKE), msl, sm, ctypes.c_void_p(out),
                                              ctypes.c_void_p(ws), wsb, None)

    assert nk.lib.mxfp4_kv_quantize_append(None, None, None, 1, 1, 1024, None, None) == 1
    assert app(T=0, k=0, slots=0) == 0
    assert app(T=-1) == 1 and app(dtype=7) == 1 and app(k=0) == 1 and app(slots=0) == 1
    assert app(stride=1023) == 1 and app(k=FAKE + 4) == 2 and app(stride=1028) == 2
    assert nk.lib.mxfp4_paged_decode_attn(None, None, 1, 1, 8, None, 1, None, 16, 0.1, None, None, 0, None) == 1
    assert dec(Hq=60) == 1 and dec(Hq=8 * 17) == 2 and dec(B=-1) == 1
    assert dec(B=0, q=0, out=0) == 0
    assert dec(q=0) == 1 and dec(out=0) == 1 and dec(bts=3) == 1 and dec(sm=float("nan")) == 1
    assert dec(q=FAKE + 2) == 2 and dec(B=4097) == 2 and dec(ws=FAKE + 16) == 1
    need = nk.decode_workspace_bytes(1, 64, 8, 1 << 20)
    assert dec(B=1, msl=1 << 20, bts=1 << 16, wsb=need - 1) == 3


def test_hadamard_entry_points_check_like_their_plain_twins():
    nk = _lib()
    L, M = _layer(nk), _mx_layer(nk)
    for f, lay in (("nvfp4_kv_quantize_append_hadamard", L), ("mxfp4_kv_quantize_append_hadamard", M)):
        fn = getattr(nk.lib, f)
        assert fn(None, None, None, 1, 1, 1024, None, None) == 1
        assert fn(ctypes.byref(lay), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), 1, 0, 1024, None, None) == 0
        assert fn(ctypes.byref(lay), ctypes.c_void_p(FAKE + 4), ctypes.c_void_p(FAKE), 1, 4, 1024,
                  ctypes.c_void_p(FAKE), None) == 2
    for f, lay in (("nvfp4_paged_decode_attn_hadamard", L), ("mxfp4_paged_decode_attn_hadamard", M)):
        fn = getattr(nk.lib, f)

        def dec(q=FAKE, B=2, Hq=64, bts=4, msl=64, ws=FAKE, wsb=1 << 30):
            return fn(ctypes.byref(lay), ctypes.c_void_p(q), 1, B, Hq, ctypes.c_void_p(FAKE), bts,
                      ctypes.c_void_p(FAKE), msl, 0.088, ctypes.c_void_p(FAKE), ctypes.c_void_p(ws), wsb, None)
        assert dec(Hq=60) == 1 and dec(Hq=8 * 17) == 2 and dec(bts=3) == 1 and dec(q=FAKE + 2) == 2
        assert dec(B=0, q=0) == 0 and dec(ws=FAKE + 16) == 1
        need = nk.decode_workspace_bytes(1, 64, 8, 1 << 20)
        assert dec(B=1, msl=1 << 20, bts=1 << 16, wsb=need - 1) == 3



def _decode_noalloc(nk, layer, q=FAKE, qdt=1, B=2, Hq=64, bt=FAKE, bts=4, sl=FAKE, msl=64, sm=0.088, out=FAKE):
    return nk.lib.nvfp4_paged_decode_attn_noalloc(ctypes.byref(layer), ctypes.c_void_p(q), qdt, B, Hq,
                                                  ctypes.c_void_p(bt), bts, ctypes.c_void_p(sl), msl, sm,
                                                  ctypes.c_void_p(out), None)


def test_noalloc_decode_checks_and_limit():
    """The allocation-free decode checks its arguments like nvfp4_paged_decode_attn
    and rejects calls whose partials exceed its 8 MiB scratch, all before any HIP call."""
    nk = _lib()
    L = _layer(nk)
    assert _decode_noalloc(nk, L, Hq=60) == 1
    assert _decode_noalloc(nk, L, Hq=8 * 17) == 2
    assert _decode_noalloc(nk, L, qdt=3) == 1
    assert _decode_noalloc(nk, L, B=0, q=0, bt=0, sl=0, out=0) == 0  # empty batch: nothing enqueued
    assert _decode_noalloc(nk, L, q=0) == 1
    assert _decode_noalloc(nk, L, out=0) == 1
    assert _decode_noalloc(nk, L, bts=3) == 1
    assert _decode_noalloc(nk, L, sm=float("inf")) == 1
    assert _decode_noalloc(nk, L, q=FAKE + 2) == 2

    # the limit: partials = workspace bytes past the counters <= 8 MiB - 64 KiB
    def partial_bytes(B, Hq, msl):
        return nk.decode_workspace_bytes(B, Hq, 8, msl) - (B * 8 * 4 + 255) // 256 * 256
    limit = (8 << 20) - (64 << 10)
    ok_b = max(b for b in range(1, 1024) if partial_bytes(b, 64, 8192) <= limit)
    assert ok_b >= 200  # about 218 sequences of 8 kv heads at 8 q heads per kv head
    assert _decode_noalloc(nk, L, B=ok_b + 1, Hq=64, msl=8192, bts=512) == 3
    assert _decode_noalloc(nk, L, B=4096, Hq=128, msl=64, bts=4) == 3  # too many units for the counters


def _mla_layer(nk, **kw):
    d = dict(codes=FAKE, scales=FAKE + 0x100000, num_slots=100, latent_dim=512, rope_dim=64, global_scale=0.01)
    d.update(kw)
    return nk.CMlaLayer(**d)


def _mla_decode(nk, layer, q=FAKE, qdt=1, T=2, Hq=64, idx=FAKE, topk=32, sm=0.07, out=FAKE, ws=FAKE, wsb=1 << 30):
    return nk.lib.nvfp4_mla_sparse_decode(ctypes.byref(layer), ctypes.c_void_p(q), qdt, T, Hq, ctypes.c_void_p(idx),
                                          topk, sm, ctypes.c_void_p(out), ctypes.c_void_p(ws), wsb, None)


def test_mla_checks():
    """The Sparse-MLA entry points check their arguments before any HIP call."""
    nk = _lib()
    L = _mla_layer(nk)
    app = lambda layer, x=FAKE, dt=1, T=4, stride=576, sl=FAKE: nk.lib.nvfp4_mla_quantize_append(
        ctypes.byref(layer), ctypes.c_void_p(x), dt, T, stride, ctypes.c_void_p(sl), None)
    assert app(_mla_layer(nk, latent_dim=256)) == 2
    assert app(_mla_layer(nk, rope_dim=0)) == 2
    assert app(_mla_layer(nk, codes=0)) == 1
    assert app(_mla_layer(nk, codes=FAKE + 8)) == 2
    assert app(_mla_layer(nk, num_slots=0)) == 1
    assert app(_mla_layer(nk, global_scale=float("nan"))) == 1
    assert app(L, T=0, x=0, sl=0) == 0
    assert app(L, T=-1) == 1
    assert app(L, stride=575) == 1
    assert app(L, x=FAKE + 4) == 2
    assert app(L, stride=580, dt=1) == 2          # 1160-byte rows: not a multiple of 16 bytes
    assert app(L, sl=0) == 1
    assert _mla_decode(nk, L, qdt=0) == 2         # float32 queries: not supported
    assert _mla_decode(nk, L, qdt=5) == 1
    assert _mla_decode(nk, L, Hq=40) == 2         # not a multiple of 16
    assert _mla_decode(nk, L, Hq=96) == 2         # above 64: a multiple of 64
    assert _mla_decode(nk, L, topk=(1 << 20) + 1) == 2
    assert _mla_decode(nk, L, T=-1) == 1
    assert _mla_decode(nk, L, T=0, q=0, idx=0, out=0) == 0
    assert _mla_decode(nk, L, q=0) == 1
    assert _mla_decode(nk, L, idx=0) == 1
    assert _mla_decode(nk, L, q=FAKE + 8) == 2
    assert _mla_decode(nk, L, sm=float("inf")) == 1
    need = nk.mla_sparse_decode_workspace_bytes(2, 64, 2048)  # few tokens: lists split, partials needed
    assert need > 256 and _mla_decode(nk, L, topk=2048, wsb=need - 1) == 3
    assert _mla_decode(nk, L, topk=2048, ws=FAKE + 16) == 1
    assert _mla_decode(nk, L, topk=2048, ws=0, wsb=need) == 1
    assert nk.mla_sparse_decode_workspace_bytes(0, 64, 2048) == 0
    assert nk.mla_sparse_decode_workspace_bytes(512, 128, 2048) == 0  # 1024 (token, head block) units: no split
