"""CPU oracle for the sub-byte KV cache -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct implementation of what the GPU library
computes: the 4-bit Hadamard-32 row codec (and its 6- and 8-bit variants),
the fp8 e4m3 latent codec, the rotated-int4 + Lloyd-Max latent codec, and
decode attention over these caches in fp64.  The arithmetic lives in
kvq_oracle.c (see its header for the pages and readings it follows); this
module only marshals numpy arrays through ctypes.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product library (fp8_quantized_kv_amd) never imports it,
and the two share no code.

Parity pins: every function here is pinned by tests/test_oracle_*.py to
values fixed by the pages or by mathematics (exact-scale example, exhaustive
e4m3 and binary16 checks, Hadamard orthogonality, brute-force fp64
attention, the Lloyd-Max optimality conditions by numerical integration, the
page's 0.096 round-trip error, SplitMix64's published outputs); none is
"parity unpinned".
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVQ_ORACLE_LIB names another build of the same source (the sanitizer test
# runs the pins against an -fsanitize=address,undefined build this way).
_LIB_PATH = os.environ.get("KVQ_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_D = ctypes.c_double


def lib():
    """Load liboracle.so, building it first if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        sig = {
            "kvqo_num_threads": ([], _I),
            "kvqo_f32_to_f16": ([ctypes.c_float], ctypes.c_uint16),
            "kvqo_f16_to_f32": ([ctypes.c_uint16], ctypes.c_float),
            "kvqo_e4m3_encode": ([ctypes.c_float], ctypes.c_uint8),
            "kvqo_e4m3_decode": ([ctypes.c_uint8], _D),
            "kvqo_q4_row_bytes": ([_I], ctypes.c_size_t),
            "kvqo_blk_row_bytes": ([_I, _I], ctypes.c_size_t),
            "kvqo_q4_encode_row": ([_P, _I, _P], _I),
            "kvqo_blk_encode_rows": ([_I, _P, _I64, _I, _P], _I),
            "kvqo_blk_decode_rows": ([_I, _P, _I64, _I, _P], None),
            "kvqo_hadamard32_f32_rows": ([_P, _I64], None),
            "kvqo_rotate_f64": ([_P, _P, _I], None),
            "kvqo_blk_store": ([_I, _P, _P, _I, _I, _I, _I, _P, _P, _P, _I], _I),
            "kvqo_blk_attention": ([_I, _P, _P, _I, _I, _I, _I, _P, _I, _P, _I, _P, _I, _D, _P, _P], _I),
            "kvqo_blk_attention_chunked": ([_I, _P, _P, _I, _I, _I, _I, _P, _I, _P, _I, _P, _I, _D, _I, _I,
                                            _P, _P, _P, _P, _P], _I),
            "kvqo_fp8_encode_part": ([_P, _I, _P, _P], None),
            "kvqo_fp8_store": ([_P, _P, _I, _I, _I64, _P, _P, _I], _I),
            "kvqo_mla_attention": ([_P, _P, _I, _I, _I, _I, _P, _I, _P, _I, _P, _I, _D, _P, _P], _I),
            "kvqo_mla_attention_chunked": ([_P, _P, _I, _I, _I, _I, _P, _I, _P, _I, _P, _I, _D, _I, _I,
                                            _P, _P, _P, _P, _P], _I),
            "kvqo_mla_attention_sel": ([_P, _P, _I, _I, _I, _I, _P, _I, _P, _I, _P, _I, _P, _I, _D, _P, _P], _I),
            "kvqo_f32_to_f16_array": ([_P, _P, _I64], None),
            "kvqo_splitmix64": ([ctypes.c_uint64, _I, _P], None),
            "kvqo_tq_signs": ([_I, _I, _P], None),
            "kvqo_lloyd_max_gauss": ([_I, _P], _I),
            "kvqo_tq_tables": ([_P, _P], None),
            "kvqo_tq_quantize": ([_P, _I, _P], None),
            "kvqo_tq_rotate_f32": ([_P, _I, _I], None),
            "kvqo_tq_unrotate_f64": ([_P, _I, _I], None),
            "kvqo_tq_encode_part": ([_P, _I, _I, _P, _P], None),
            "kvqo_tq_store": ([_P, _P, _I64, _P, _P, _I], _I),
            "kvqo_tq_decode_rows": ([_P, _P, _I64, _P], None),
            "kvqo_tq_attention": ([_P, _P, _I, _I, _P, _I, _P, _I, _P, _I, _D, _P, _P], _I),
            "kvqo_e4m3_encode_array": ([_P, _P, _I64], None),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with status {rc}")


def num_threads():
    return lib().kvqo_num_threads()


# ---------------------------------------------------------------- scalars

def f32_to_f16_bits(x):
    """binary16 bits of float32 values, round to nearest even (array)."""
    x = _c(x, np.float32)
    y = np.empty(x.shape, np.uint16)
    lib().kvqo_f32_to_f16_array(_ptr(x), _ptr(y), x.size)
    return y


def f16_bits_to_f32(h):
    return np.array([lib().kvqo_f16_to_f32(int(v)) for v in np.ravel(h)], np.float32).reshape(np.shape(h))


def e4m3_encode(x):
    """e4m3 codes of float32 values (array), saturating, NaN -> 0."""
    x = _c(x, np.float32)
    y = np.empty(x.shape, np.uint8)
    lib().kvqo_e4m3_encode_array(_ptr(x), _ptr(y), x.size)
    return y


def e4m3_decode(codes):
    return np.array([lib().kvqo_e4m3_decode(int(c)) for c in np.ravel(codes)], np.float64).reshape(np.shape(codes))


# ---------------------------------------------------------------- block codecs (4-, 6-, 8-bit)
#
# Every function below takes bits = 4 (the 144-byte-row format), 6 or 8: the
# same rotated groups of 32 values and fp16 scale, with codes of that width.

def q4_row_bytes(D, bits=4):
    return int(lib().kvqo_blk_row_bytes(bits, D))


def hadamard32_f32(x):
    """The fp32 storage rotation applied to every 32-group of x (returns a copy)."""
    x = np.array(x, dtype=np.float32, order="C", copy=True)
    assert x.size % 32 == 0
    lib().kvqo_hadamard32_f32_rows(_ptr(x), x.size // 32)
    return x


def rotate_f64(x):
    """H32 applied to every 32-group of the last axis, fp64 (returns a copy)."""
    x = _c(x, np.float64)
    D = x.shape[-1]
    flat = x.reshape(-1, D)
    y = np.empty_like(flat)
    for r in range(flat.shape[0]):
        lib().kvqo_rotate_f64(_ptr(flat[r]), _ptr(y[r]), D)
    return y.reshape(x.shape)


def q4_encode_rows(x, bits=4):
    """x [..., D] float32 -> packed rows [..., row_bytes] uint8 (4 bits: D/2 + 2*D/32)."""
    x = _c(x, np.float32)
    D = x.shape[-1]
    n = x.size // D
    out = np.empty(x.shape[:-1] + (q4_row_bytes(D, bits),), np.uint8)
    _check(lib().kvqo_blk_encode_rows(bits, _ptr(x), n, D, _ptr(out)), "blk_encode_rows")
    return out


def q4_decode_rows(rows, D, bits=4):
    """packed rows [..., row_bytes] -> dequantized rotated values [..., D] fp64."""
    rows = _c(rows, np.uint8)
    n = rows.size // q4_row_bytes(D, bits)
    out = np.empty(rows.shape[:-1] + (D,), np.float64)
    lib().kvqo_blk_decode_rows(bits, _ptr(rows), n, D, _ptr(out))
    return out


def q4_chunk_attention(k_pool, v_pool, q, page_row, row_lens, sm_scale):
    """Attention of several query rows of ONE sequence over its paged cache
    (a prompt chunk: TensorFold issue "qwen27 CUDA: an opt-in 4-bit attention
    cache", "What it is" -- prompt chunks are packed, then attended over the
    decoded slots): row i attends positions [0, row_lens[i]) of the sequence
    whose page-table row is page_row; for a chunk starting at position P,
    row_lens[i] = P + i + 1 (causal within the chunk).  This is
    q4_attention with the page-table row repeated for every row.
    q: [C][H_q][D] float32 (unrotated).  Returns (o [C][H_q][D], lse [C][H_q])."""
    q = _c(q, np.float32)
    page_row = _c(page_row, np.int32).reshape(-1)
    pt = np.ascontiguousarray(np.broadcast_to(page_row, (q.shape[0], page_row.size)))
    return q4_attention(k_pool, v_pool, q, pt, _c(row_lens, np.int32), sm_scale)


def q4_pool_shape(num_pages, n_kv_heads, page_size, D, bits=4):
    return (num_pages, n_kv_heads, page_size, q4_row_bytes(D, bits))


def _bits_of_pool(pool, D):
    rb = pool.shape[-1]
    for bits in (4, 6, 8):
        if q4_row_bytes(D, bits) == rb:
            return bits
    raise ValueError(f"row of {rb} bytes matches no block format at D={D}")


def q4_store(k_pool, v_pool, k, v, slots, page_size):
    """Encode K and V [n_tok][H_kv][D] into the paged pools (in place)."""
    num_pages, H, ps, rb = k_pool.shape
    assert ps == page_size and v_pool.shape == k_pool.shape
    assert k_pool.flags.c_contiguous and v_pool.flags.c_contiguous
    k = _c(k, np.float32)
    v = _c(v, np.float32)
    slots = _c(slots, np.int64)
    D = k.shape[-1]
    bits = _bits_of_pool(k_pool, D)
    _check(lib().kvqo_blk_store(bits, _ptr(k_pool), _ptr(v_pool), H, D, page_size, num_pages, _ptr(k), _ptr(v),
                                _ptr(slots), len(slots)), "blk_store")


def q4_attention(k_pool, v_pool, q, page_table, seq_lens, sm_scale, chunk=None, n_chunks=None,
                 return_partials=False):
    """fp64 decode attention over a paged block-format cache (the format is
    read off the pools' row size).

    q: [B][H_q][D] float32 (unrotated).  Returns (o [B][H_q][D], lse [B][H_q]),
    plus (acc, m, z) chunk partials when chunk is given and return_partials.
    """
    num_pages, H_kv, ps, rb = k_pool.shape
    q = _c(q, np.float32)
    B, H_q, D = q.shape
    bits = _bits_of_pool(k_pool, D)
    pt = _c(page_table, np.int32)
    sl = _c(seq_lens, np.int32)
    out = np.empty((B, H_q, D), np.float64)
    lse = np.empty((B, H_q), np.float64)
    if chunk is None:
        _check(lib().kvqo_blk_attention(bits, _ptr(k_pool), _ptr(v_pool), H_kv, D, ps, num_pages, _ptr(q), H_q,
                                        _ptr(pt), pt.shape[1], _ptr(sl), B, float(sm_scale), _ptr(out),
                                        _ptr(lse)), "blk_attention")
        return out, lse
    if n_chunks is None:
        n_chunks = max(1, -(-int(sl.max()) // chunk)) if B else 1
    pa = np.empty((B, H_q, n_chunks, D), np.float64) if return_partials else None
    pm = np.empty((B, H_q, n_chunks), np.float64) if return_partials else None
    pz = np.empty((B, H_q, n_chunks), np.float64) if return_partials else None
    _check(lib().kvqo_blk_attention_chunked(bits, _ptr(k_pool), _ptr(v_pool), H_kv, D, ps, num_pages, _ptr(q),
                                            H_q, _ptr(pt), pt.shape[1], _ptr(sl), B, float(sm_scale), chunk,
                                            n_chunks, _ptr(pa), _ptr(pm), _ptr(pz), _ptr(out), _ptr(lse)),
           "blk_attention_chunked")
    if return_partials:
        return out, lse, (pa, pm, pz)
    return out, lse


# ---------------------------------------------------------------- fp8 latent codec

def fp8_encode_part(x):
    """One row part -> (codes uint8 [n], scale float32)."""
    x = _c(x, np.float32)
    codes = np.empty(x.shape, np.uint8)
    sc = np.zeros(1, np.float32)
    lib().kvqo_fp8_encode_part(_ptr(x), x.size, _ptr(codes), _ptr(sc))
    return codes, sc[0]


def fp8_store(codes_pool, scale_pool, x, slots, rope_dim):
    """Encode latent rows x [n_tok][D] into codes_pool [n_slots][D], scale_pool [n_slots][2]."""
    n_slots, D = codes_pool.shape
    assert scale_pool.shape == (n_slots, 2) and scale_pool.dtype == np.float32
    x = _c(x, np.float32)
    slots = _c(slots, np.int64)
    _check(lib().kvqo_fp8_store(_ptr(codes_pool), _ptr(scale_pool), D, rope_dim, n_slots, _ptr(x), _ptr(slots),
                                len(slots)), "fp8_store")


def mla_attention(codes_pool, scale_pool, q, page_table, seq_lens, sm_scale, rope_dim, page_size, chunk=None,
                  n_chunks=None, return_partials=False):
    """fp64 absorbed attention over the fp8 latent cache.  q: [B][H][D]."""
    n_slots, D = codes_pool.shape
    num_pages = n_slots // page_size
    q = _c(q, np.float32)
    B, H, Dq = q.shape
    assert Dq == D
    L = D - rope_dim
    pt = _c(page_table, np.int32)
    sl = _c(seq_lens, np.int32)
    out = np.empty((B, H, L), np.float64)
    lse = np.empty((B, H), np.float64)
    if chunk is None:
        _check(lib().kvqo_mla_attention(_ptr(codes_pool), _ptr(scale_pool), D, rope_dim, page_size, num_pages,
                                        _ptr(q), H, _ptr(pt), pt.shape[1], _ptr(sl), B, float(sm_scale), _ptr(out),
                                        _ptr(lse)), "mla_attention")
        return out, lse
    if n_chunks is None:
        n_chunks = max(1, -(-int(sl.max()) // chunk)) if B else 1
    pa = np.empty((B, H, n_chunks, L), np.float64) if return_partials else None
    pm = np.empty((B, H, n_chunks), np.float64) if return_partials else None
    pz = np.empty((B, H, n_chunks), np.float64) if return_partials else None
    _check(lib().kvqo_mla_attention_chunked(_ptr(codes_pool), _ptr(scale_pool), D, rope_dim, page_size, num_pages,
                                            _ptr(q), H, _ptr(pt), pt.shape[1], _ptr(sl), B, float(sm_scale), chunk,
                                            n_chunks, _ptr(pa), _ptr(pm), _ptr(pz), _ptr(out), _ptr(lse)),
           "mla_attention_chunked")
    if return_partials:
        return out, lse, (pa, pm, pz)
    return out, lse


def mla_attention_sel(codes_pool, scale_pool, q, page_table, sel, n_sel, sm_scale, rope_dim, page_size):
    """fp64 absorbed attention over the selected rows of the fp8 latent cache (DSA gather).
    sel: int32 [B][max_sel] absolute positions (entries outside the page capacity, e.g. -1,
    are absent); n_sel: int32 [B] entries used per sequence.  Returns (out [B][H][L], lse [B][H])."""
    n_slots, D = codes_pool.shape
    num_pages = n_slots // page_size
    q = _c(q, np.float32)
    B, H, Dq = q.shape
    assert Dq == D
    L = D - rope_dim
    pt = _c(page_table, np.int32)
    sl = _c(sel, np.int32)
    ns = _c(n_sel, np.int32)
    assert sl.ndim == 2 and sl.shape[0] == B and ns.shape == (B,)
    out = np.empty((B, H, L), np.float64)
    lse = np.empty((B, H), np.float64)
    _check(lib().kvqo_mla_attention_sel(_ptr(codes_pool), _ptr(scale_pool), D, rope_dim, page_size, num_pages,
                                        _ptr(q), H, _ptr(pt), pt.shape[1], _ptr(sl), sl.shape[1], _ptr(ns), B,
                                        float(sm_scale), _ptr(out), _ptr(lse)), "mla_attention_sel")
    return out, lse


# ---------------------------------------------------------------- rotated-int4 + Lloyd-Max latent codec
#
# colibri pull request "KV cache quantization: fp8 (KV8) + 4-bit TurboQuant
# (KV_TQ)", Summary "Why rotated-int4 for the 4-bit tier": randomized
# Hadamard rotation, 16-level Lloyd-Max codebook for N(0,1) scaled by
# radius/sqrt(n), one radius per row part.  Readings: kvq_oracle.c.

TQ_ROW_BYTES = 288      # 256 code bytes of the 512-wide latent part, 32 of the 64-wide rope part
TQ_PARTS = ((0, 512), (1, 64))


def splitmix64(seed, n):
    out = np.empty(n, np.uint64)
    lib().kvqo_splitmix64(int(seed), n, _ptr(out))
    return out


def tq_signs(part, n):
    sig = np.empty(n, np.float32)
    lib().kvqo_tq_signs(part, n, _ptr(sig))
    return sig


def lloyd_max_gauss(nlev=16):
    """Levels (fp64, ascending) and the number of Lloyd iterations run."""
    lev = np.empty(nlev, np.float64)
    it = lib().kvqo_lloyd_max_gauss(nlev, _ptr(lev))
    return lev, it


def tq_tables():
    """The codec's fp32 levels (16) and thresholds (15)."""
    lev, thr = np.empty(16, np.float32), np.empty(15, np.float32)
    lib().kvqo_tq_tables(_ptr(lev), _ptr(thr))
    return lev, thr


def tq_quantize(u):
    u = _c(u, np.float32)
    codes = np.empty(u.shape, np.uint8)
    lib().kvqo_tq_quantize(_ptr(u), u.size, _ptr(codes))
    return codes


def tq_rotate_f32(x, part):
    """The fp32 storage rotation of one part (returns a copy)."""
    x = np.array(x, dtype=np.float32, order="C", copy=True)
    lib().kvqo_tq_rotate_f32(_ptr(x), x.size, part)
    return x


def tq_unrotate_f64(y, part):
    y = np.array(y, dtype=np.float64, order="C", copy=True)
    lib().kvqo_tq_unrotate_f64(_ptr(y), y.size, part)
    return y


def tq_encode_part(x, part):
    x = _c(x, np.float32)
    out = np.empty(x.size // 2, np.uint8)
    r = np.empty(1, np.float32)
    lib().kvqo_tq_encode_part(_ptr(x), x.size, part, _ptr(out), _ptr(r))
    return out, float(r[0])


def tq_pool_shape(num_pages, page_size):
    return (num_pages * page_size, TQ_ROW_BYTES), (num_pages * page_size, 2)


def tq_store(codes_pool, radius_pool, x, slots):
    """Store latent rows x [n][576] at slots (in place on the two pools)."""
    assert codes_pool.flags.c_contiguous and radius_pool.flags.c_contiguous
    x = _c(x, np.float32)
    slots = _c(slots, np.int64)
    _check(lib().kvqo_tq_store(_ptr(codes_pool), _ptr(radius_pool), codes_pool.shape[0], _ptr(x), _ptr(slots),
                               len(slots)), "tq_store")


def tq_decode_rows(codes, radii):
    """Dequantized, rotated-back rows [n][576] (fp64)."""
    codes = _c(codes, np.uint8).reshape(-1, TQ_ROW_BYTES)
    radii = _c(radii, np.float32).reshape(-1, 2)
    out = np.empty((codes.shape[0], 576), np.float64)
    lib().kvqo_tq_decode_rows(_ptr(codes), _ptr(radii), codes.shape[0], _ptr(out))
    return out


def tq_attention(codes_pool, radius_pool, q, page_table, seq_lens, sm_scale, page_size):
    """fp64 absorbed attention over the TQ4 cache: (out [B][H][512], lse [B][H])."""
    q = _c(q, np.float32)
    B, H, D = q.shape
    assert D == 576
    pt = _c(page_table, np.int32)
    sl = _c(seq_lens, np.int32)
    out = np.empty((B, H, 512), np.float64)
    lse = np.empty((B, H), np.float64)
    num_pages = codes_pool.shape[0] // page_size
    _check(lib().kvqo_tq_attention(_ptr(_c(codes_pool, np.uint8)), _ptr(_c(radius_pool, np.float32)), page_size,
                                   num_pages, _ptr(q), H, _ptr(pt), pt.shape[1], _ptr(sl), B, float(sm_scale),
                                   _ptr(out), _ptr(lse)), "tq_attention")
    return out, lse

