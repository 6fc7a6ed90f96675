"""The C ABI on the CPU: the library loads, exports every symbol include/kvq.h
declares, its host helpers compute the documented sizes, and invalid
arguments are rejected on the host before any launch (no GPU needed: every
call here returns before touching the HIP runtime)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


@pytest.fixture(scope="module")
def kvq():
    import fp8_quantized_kv_amd as m
    return m


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(kvq):
    names = _declared()
    assert set(names) >= {"kvq_store", "kvq_rotate_q", "kvq_decode_attn", "kvq_merge"}
    raw = ctypes.CDLL(kvq.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), f"libkvq.so does not export {n}"
    assert set(names) == set(kvq.EXPORTED)


def test_size_helpers(kvq):
    L = kvq.lib
    assert L.kvq_row_bytes(kvq.FMT_Q4_H32, 256, 0) == 144
    assert L.kvq_row_bytes(kvq.FMT_Q4_H32, 128, 0) == 72
    assert L.kvq_row_bytes(kvq.FMT_Q4_H32, 100, 0) == 0
    assert L.kvq_row_bytes(kvq.FMT_Q8_H32, 256, 0) == 272       # 1.0625 bytes per element
    assert L.kvq_row_bytes(kvq.FMT_Q6_H32, 256, 0) == 208
    assert L.kvq_row_bytes(kvq.FMT_Q6_H32, 64, 0) == 52
    q8 = kvq.KvqCacheDesc(kvq.FMT_Q8_H32, 4, 256, 0, 16, 1024, 0x1000, 0x2000, None)
    assert L.kvq_pool_bytes(ctypes.byref(q8)) == 2 * 1024 * 16 * 4 * 272
    assert L.kvq_row_bytes(kvq.FMT_FP8_E4M3_ROW, 576, 64) == 576
    assert L.kvq_row_bytes(7, 256, 0) == 0
    assert L.kvq_num_splits(262144, 2048) == 128
    assert L.kvq_num_splits(262145, 2048) == 129
    assert L.kvq_num_splits(0, 512) == 1
    assert L.kvq_num_splits(100, 0) == 0
    d = kvq.KvqCacheDesc(kvq.FMT_Q4_H32, 4, 256, 0, 16, 16384, 0x1000, 0x2000, None)
    assert L.kvq_pool_bytes(ctypes.byref(d)) == 2 * 16384 * 16 * 4 * 144   # K and V pools
    e = kvq.KvqCacheDesc(kvq.FMT_FP8_E4M3_ROW, 1, 576, 64, 16, 16384, 0x1000, None, 0x2000)
    assert L.kvq_pool_bytes(ctypes.byref(e)) == 16384 * 16 * 584
    assert L.kvq_status_string(-2) == b"unsupported shape or format"


# Fake, aligned device addresses: every call below must be rejected on the
# host before it could be dereferenced.
A = 0x7F0000000000


def _q4(kvq, **kw):
    f = dict(format=kvq.FMT_Q4_H32, num_kv_heads=4, head_dim=256, rope_dim=0, page_size=16, num_pages=64,
             k_pool=A, v_pool=A + 0x100000, scale_pool=None)
    f.update(kw)
    return kvq.KvqCacheDesc(**f)


def _fp8(kvq, **kw):
    f = dict(format=kvq.FMT_FP8_E4M3_ROW, num_kv_heads=1, head_dim=576, rope_dim=64, page_size=16, num_pages=64,
             k_pool=A, v_pool=None, scale_pool=A + 0x100000)
    f.update(kw)
    return kvq.KvqCacheDesc(**f)


INVALID, UNSUPPORTED = -1, -2


@pytest.mark.parametrize("desc_kw,expect", [
    (dict(format=9), INVALID),
    (dict(head_dim=100), INVALID),
    (dict(head_dim=96), UNSUPPORTED),
    (dict(page_size=0), INVALID),
    (dict(num_pages=0), INVALID),
    (dict(k_pool=A + 4), INVALID),
    (dict(v_pool=None), INVALID),
    (dict(scale_pool=A), INVALID),
    (dict(rope_dim=64), INVALID),
])
def test_store_rejects_bad_q4_cache(kvq, desc_kw, expect):
    d = _q4(kvq, **desc_kw)
    rc = kvq.lib.kvq_store(ctypes.byref(d), ctypes.c_void_p(A), ctypes.c_void_p(A), 0, ctypes.c_void_p(A), 4, None)
    assert rc == expect


@pytest.mark.parametrize("desc_kw,expect", [
    (dict(num_kv_heads=2), INVALID),
    (dict(rope_dim=0), INVALID),
    (dict(head_dim=320, rope_dim=64), UNSUPPORTED),
    (dict(v_pool=A), INVALID),
    (dict(scale_pool=None), INVALID),
])
def test_store_rejects_bad_fp8_cache(kvq, desc_kw, expect):
    d = _fp8(kvq, **desc_kw)
    rc = kvq.lib.kvq_store(ctypes.byref(d), ctypes.c_void_p(A), None, 0, ctypes.c_void_p(A), 4, None)
    assert rc == expect


def test_store_argument_checks(kvq):
    d = _q4(kvq)
    P = ctypes.c_void_p
    assert kvq.lib.kvq_store(None, P(A), P(A), 0, P(A), 4, None) == INVALID
    assert kvq.lib.kvq_store(ctypes.byref(d), P(A), P(A), 7, P(A), 4, None) == INVALID      # dtype
    assert kvq.lib.kvq_store(ctypes.byref(d), P(A), P(A), 0, P(A), -1, None) == INVALID     # n_tokens
    assert kvq.lib.kvq_store(ctypes.byref(d), P(A + 2), P(A), 0, P(A), 4, None) == INVALID  # misaligned k
    assert kvq.lib.kvq_store(ctypes.byref(d), P(A), P(A), 0, P(A + 4), 4, None) == INVALID  # misaligned slots
    assert kvq.lib.kvq_store(ctypes.byref(d), P(A), P(A), 0, P(A), 0, None) == 0            # no-op
    f = _fp8(kvq)
    assert kvq.lib.kvq_store(ctypes.byref(f), P(A), P(A), 0, P(A), 4, None) == INVALID      # fp8 takes no v


def test_rotate_argument_checks(kvq):
    P = ctypes.c_void_p
    r = kvq.lib.kvq_rotate_q
    assert r(P(A), 0, P(A), 4, 100, None) == INVALID      # head_dim % 32
    assert r(P(A), 1, P(A), 4, 256, None) == INVALID      # in place needs f32
    assert r(P(A + 8), 0, P(A), 4, 256, None) == INVALID
    assert r(P(A), 0, P(A), 0, 256, None) == 0


def test_store_rotate_argument_checks(kvq):
    P = ctypes.c_void_p
    r = kvq.lib.kvq_store_rotate_q
    d = _q4(kvq)
    args = lambda **kw: [ctypes.byref(kw.get("d", d)), P(kw.get("k", A)), P(A), kw.get("kdt", 0), P(kw.get("sl", A)),
                         kw.get("n", 4), P(kw.get("q", A)), kw.get("qdt", 0), P(kw.get("qr", A + 4096)),
                         kw.get("rows", 24), None]
    assert r(*args(d=_fp8(kvq))) == INVALID          # 4-bit cache only
    assert r(*args(kdt=7)) == INVALID                 # kv dtype
    assert r(*args(qdt=5)) == INVALID                 # q dtype
    assert r(*args(n=-1)) == INVALID
    assert r(*args(rows=-1)) == INVALID
    assert r(*args(k=A + 2)) == INVALID               # misaligned k
    assert r(*args(sl=A + 4)) == INVALID              # misaligned slots
    assert r(*args(q=A + 8)) == INVALID               # misaligned q
    assert r(*args(qr=A, qdt=1)) == INVALID           # in place needs f32
    assert r(*args(d=_q4(kvq, head_dim=100))) == INVALID
    assert r(*args(n=0, rows=0)) == 0                 # nothing to do: no launch


def test_decode_sel_argument_checks(kvq):
    P = ctypes.c_void_p
    r = kvq.lib.kvq_decode_attn_sel
    f = _fp8(kvq)
    args = lambda **kw: [ctypes.byref(kw.get("d", f)), P(A), kw.get("h", 128), P(A), 64, P(kw.get("sel", A)), P(A),
                         kw.get("b", 1), kw.get("ms", 4096), ctypes.c_float(kw.get("sm", 0.04)), kw.get("split", 1024),
                         P(A), P(A), P(A), None]
    assert r(*args(d=_q4(kvq))) == UNSUPPORTED           # fp8 latent only
    assert r(*args(split=1000)) == INVALID                # split_keys % 32
    assert r(*args(split=0)) == INVALID
    assert r(*args(split=4096)) == UNSUPPORTED            # the matrix-core kernel takes <= 2048
    assert r(*args(sel=A + 2)) == INVALID                 # misaligned list
    assert r(*args(ms=-1)) == INVALID
    assert r(*args(sm=float("nan"))) == INVALID
    assert r(*args(b=0)) == 0                             # nothing to do: no launch


def test_stream_read_argument_checks(kvq):
    P = ctypes.c_void_p
    r = kvq.lib.kvq_stream_read
    assert r(P(A + 4), 16384, 1, P(A), None) == INVALID     # misaligned source
    assert r(P(A), 16384 + 16, 1, P(A), None) == INVALID    # not a multiple of 16 KiB
    assert r(P(A), 0, 1, P(A), None) == INVALID
    assert r(P(A), 16384, 2, P(A), None) == INVALID         # policy flag
    assert r(P(A), 16384, 0, P(A + 2), None) == INVALID     # misaligned result


def _decode(kvq, d, **kw):
    P = ctypes.c_void_p
    a = dict(q=P(A), n_q_heads=24, page_table=P(A), max_pages=64, seq_lens=P(A), batch=1, max_seq_len=1024,
             sm_scale=0.0625, split_keys=512, part_acc=P(A), part_m=P(A), part_z=P(A))
    a.update(kw)
    return kvq.lib.kvq_decode_attn(ctypes.byref(d), a["q"], a["n_q_heads"], a["page_table"], a["max_pages"],
                                   a["seq_lens"], a["batch"], a["max_seq_len"], a["sm_scale"], a["split_keys"],
                                   a["part_acc"], a["part_m"], a["part_z"], None)


def test_decode_argument_checks(kvq):
    d = _q4(kvq)
    assert _decode(kvq, d, split_keys=500) == INVALID
    assert _decode(kvq, d, split_keys=0) == INVALID
    assert _decode(kvq, d, n_q_heads=23) == INVALID          # not a multiple of the KV heads
    assert _decode(kvq, d, n_q_heads=4 * 17) == UNSUPPORTED  # group of 17
    assert _decode(kvq, d, max_seq_len=64 * 16 + 1) == INVALID  # beyond the page table
    assert _decode(kvq, d, max_pages=0) == INVALID
    assert _decode(kvq, d, sm_scale=float("nan")) == INVALID
    assert _decode(kvq, d, q=ctypes.c_void_p(A + 4)) == INVALID
    assert _decode(kvq, d, part_acc=None) == INVALID
    assert _decode(kvq, d, batch=-1) == INVALID
    assert _decode(kvq, d, batch=0) == 0


def test_merge_argument_checks(kvq):
    P = ctypes.c_void_p
    m = kvq.lib.kvq_merge
    d, f = _q4(kvq), _fp8(kvq)
    assert m(ctypes.byref(d), P(A), P(A), P(A), P(A), 1, 24, 1024, 512, 0, P(A), None, None) == INVALID  # Q4 rotates
    assert m(ctypes.byref(f), P(A), P(A), P(A), P(A), 1, 16, 1024, 512, 1, P(A), None, None) == INVALID  # fp8 does not
    assert m(ctypes.byref(d), P(A), P(A), P(A), P(A), 1, 24, 1024, 1000, 1, P(A), None, None) == INVALID
    assert m(ctypes.byref(d), P(A), P(A), P(A), P(A), 1, 24, 1024, 48, 1, P(A), None, None) == INVALID  # % 32
    assert m(ctypes.byref(d), P(A), P(A), P(A), P(A), 1, 24, 1024, 512, 1, P(A + 8), None, None) == INVALID
    assert m(ctypes.byref(d), P(A), P(A), P(A), P(A), 0, 24, 1024, 512, 1, P(A), None, None) == 0


def test_python_binding_checks_tensors(kvq):
    import torch
    with pytest.raises(ValueError):
        kvq.kvq_rotate_q(torch.zeros(4, 256))    # a CPU tensor is refused: no CPU path exists


def test_latent_split_granularity_and_tq_rotation_checks(kvq):
    """The latent formats split at any multiple of the 32-key tile, the
    Hadamard-32 formats only at the 512-key chunk; the TQ4 merge rotates
    back (inverse_rotate = 1); kvq_tq_rotate_q validates its arguments
    (batch 0 / 0 rows return before any launch)."""
    P = ctypes.c_void_p
    q4, f8 = _q4(kvq), _fp8(kvq)
    tq = _fp8(kvq, format=kvq.FMT_TQ4_LATENT)
    assert _decode(kvq, q4, split_keys=256, batch=0) == INVALID
    for d in (f8, tq):
        assert _decode(kvq, d, n_q_heads=16, split_keys=256, batch=0) == 0
        assert _decode(kvq, d, n_q_heads=16, split_keys=32, batch=0) == 0
        assert _decode(kvq, d, n_q_heads=16, split_keys=48, batch=0) == INVALID
    m = kvq.lib.kvq_merge
    assert m(ctypes.byref(tq), P(A), P(A), P(A), P(A), 1, 16, 1024, 512, 0, P(A), None, None) == INVALID
    assert m(ctypes.byref(tq), P(A), P(A), P(A), P(A), 0, 16, 1024, 512, 1, P(A), None, None) == 0
    r = kvq.lib.kvq_tq_rotate_q
    assert r(P(A), P(A), -1, None) == INVALID
    assert r(P(A + 4), P(A), 1, None) == INVALID
    assert r(P(A), P(A + 8), 1, None) == INVALID
    assert r(P(A), P(A), 0, None) == 0


def test_rows_argument_checks(kvq):
    """kvq_decode_attn_rows: the Hadamard-32 formats only, the 512-key chunk,
    at most 64 rows; 0 rows return before any launch."""
    P = ctypes.c_void_p
    r = kvq.lib.kvq_decode_attn_rows

    def call(d, n_rows=0, split=512, H=24):
        return r(ctypes.byref(d), P(A), H, P(A), 64, P(A), n_rows, 1024, 0.0625, split, P(A), P(A), P(A), None)

    assert call(_q4(kvq)) == 0
    assert call(_q4(kvq), split=256) == INVALID
    assert call(_q4(kvq), n_rows=65) == UNSUPPORTED
    assert call(_q4(kvq), n_rows=-1) == INVALID
    assert call(_fp8(kvq), H=16) == UNSUPPORTED
    assert call(_fp8(kvq, format=kvq.FMT_TQ4_LATENT), H=16) == UNSUPPORTED


def test_attend_workspace_and_argument_checks(kvq):
    """kvq_attend: the workspace size helper's layout (partials, then m, then z,
    each rounded up to 256 bytes) and the host checks of the call itself."""
    L = kvq.lib
    P = ctypes.c_void_p
    d = _q4(kvq)
    # 262144 positions, split 2048: S = 128; 24 heads x 128 x 256 f32, then 2 x 24 x 128 f32
    acc = 24 * 128 * 256 * 4
    mz = ((24 * 128 * 4 + 255) // 256) * 256
    big = _q4(kvq, num_pages=16384)
    assert L.kvq_attend_workspace_bytes(ctypes.byref(big), 1, 24, 262144, 2048) == acc + 2 * mz
    e = _fp8(kvq, num_pages=16384)
    assert L.kvq_attend_workspace_bytes(ctypes.byref(e), 1, 128, 262144, 2048) == (128 * 128 * 512 * 4 +
                                                                                    2 * 128 * 128 * 4)
    assert L.kvq_attend_workspace_bytes(None, 1, 24, 1024, 512) == 0
    assert L.kvq_attend_workspace_bytes(ctypes.byref(d), 1, 0, 1024, 512) == 0
    need = L.kvq_attend_workspace_bytes(ctypes.byref(d), 2, 24, 1024, 512)
    assert need > 0
    f = ctypes.c_float(0.0625)

    def call(ws=A + 0x200000, nbytes=need, out=A + 0x300000, lse=A + 0x400000, split=512, batch=2, desc=d):
        return L.kvq_attend(ctypes.byref(desc), P(A), 24, P(A), 64, P(A), batch, 1024, f, split, P(ws), nbytes,
                            P(out), P(lse), None)
    assert call(nbytes=need - 1) == INVALID          # workspace too small
    assert call(ws=A + 0x200010) == INVALID          # workspace not 256-byte aligned
    assert call(out=A + 8) == INVALID                # misaligned out
    assert call(split=500) == INVALID                # split_keys % 512
    assert call(batch=0) == 0                        # nothing to do


def test_decode_step_argument_checks(kvq):
    """kvq_decode_step: the host checks and the configurations without a step
    kernel, all refused before any launch (Q4 at head_dim 128, groups of 12
    heads, the fp8 latent rows with a V pointer, a non-f32 query or splits past
    the matrix-core kernel's 2048 keys, the TQ4 latent format)."""
    L = kvq.lib
    P = ctypes.c_void_p
    f = ctypes.c_float(0.0625)

    def call(desc, v=A + 0x10000, qdt=0, heads=24, split=512, ws=A + 0x200000, nbytes=None, batch=2, out=A + 0x300000):
        if nbytes is None:
            nbytes = L.kvq_attend_workspace_bytes(ctypes.byref(desc), batch, heads, 1024, split)
        return L.kvq_decode_step(ctypes.byref(desc), P(A), None if v is None else P(v), 1, P(A + 0x20000), qdt,
                                 heads, P(A + 0x30000), 64, P(A + 0x40000), batch, 1024, f, split, P(ws), nbytes,
                                 P(out), P(A + 0x400000), None)
    d = _q4(kvq)
    assert call(d, nbytes=L.kvq_attend_workspace_bytes(ctypes.byref(d), 2, 24, 1024, 512) - 1) == INVALID
    assert call(d, ws=A + 0x200010) == INVALID           # workspace not 256-byte aligned
    assert call(d, out=A + 8) == INVALID                 # misaligned out
    assert call(d, v=A + 4) == INVALID                   # misaligned v
    assert call(d, qdt=7) == INVALID                     # unknown query dtype
    assert call(d, batch=0) == 0                         # nothing to do
    assert call(_q4(kvq, head_dim=128)) == UNSUPPORTED   # the step forms are built for head_dim 256
    assert call(d, heads=48) == UNSUPPORTED              # groups of 12 query heads
    e = _fp8(kvq)
    assert call(e, heads=128) == INVALID                 # latent rows take no V
    assert call(e, v=None, heads=128, qdt=1) == INVALID  # the latent query is f32
    assert call(e, v=None, heads=128, split=4096) == UNSUPPORTED
    assert call(e, v=None, heads=128, batch=0) == 0
    t = kvq.KvqCacheDesc(format=kvq.FMT_TQ4_LATENT, num_kv_heads=1, head_dim=576, rope_dim=64, page_size=16,
                         num_pages=64, k_pool=A, v_pool=None, scale_pool=A + 0x100000)
    assert call(t, v=None, heads=128) == UNSUPPORTED
