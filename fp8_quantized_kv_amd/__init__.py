"""fp8_quantized_kv_amd -- sub-byte KV cache and split-K decode attention on MI355X.

A thin Python binding over libkvq.so (C ABI in include/kvq.h).  The
functions carry the C names -- kvq_store, kvq_rotate_q, kvq_decode_attn,
kvq_merge -- and only marshal arguments: they check device, dtype, shape
and contiguity of torch tensors, then pass raw pointers and torch's current
HIP stream.  Every step of the computation runs in the library's HIP
kernels; there is no CPU path.  Importing this package without a built
libkvq.so raises ImportError.

Method: TensorFold issue "qwen27 CUDA: an opt-in 4-bit attention cache"
("What it is"), FreeToken pull request "feat(kvcache): add reliable
quantized KV cache", colibri pull request "KV cache quantization: fp8 (KV8)
+ 4-bit TurboQuant (KV_TQ)" (KV8 and split-T commits).
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KVQ_OK = 0
KVQ_ERR_INVALID_ARG = -1
KVQ_ERR_UNSUPPORTED = -2
KVQ_ERR_LAUNCH = -3

FMT_Q4_H32 = 1
FMT_Q8_H32 = 3
FMT_Q6_H32 = 4
H32_FORMATS = (FMT_Q4_H32, FMT_Q8_H32, FMT_Q6_H32)
FMT_FP8_E4M3_ROW = 2
FMT_TQ4_LATENT = 5
ROTATED_FORMATS = H32_FORMATS + (FMT_TQ4_LATENT,)   # the merge rotates the context back

DT_F32, DT_BF16, DT_F16 = 0, 1, 2
_DTYPES = {torch.float32: DT_F32, torch.bfloat16: DT_BF16, torch.float16: DT_F16}

EXPORTED = ("kvq_status_string", "kvq_row_bytes", "kvq_pool_bytes", "kvq_num_splits", "kvq_store",
            "kvq_rotate_q", "kvq_store_rotate_q", "kvq_decode_attn", "kvq_decode_attn_rows", "kvq_decode_attn_sel", "kvq_merge",
            "kvq_tq_rotate_q", "kvq_stream_read", "kvq_attend_workspace_bytes", "kvq_attend",
            "kvq_attend_noalloc", "kvq_prefill_attn", "kvq_decode_step")


class KvqCacheDesc(ctypes.Structure):
    """Mirror of struct kvq_cache."""
    _fields_ = [("format", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("rope_dim", ctypes.c_int32), ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p), ("scale_pool", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python fp8_quantized_kv_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    C = ctypes.POINTER(KvqCacheDesc)
    sig = {
        "kvq_status_string": ([I32], ctypes.c_char_p),
        "kvq_row_bytes": ([I32, I32, I32], ctypes.c_size_t),
        "kvq_pool_bytes": ([C], ctypes.c_size_t),
        "kvq_num_splits": ([I32, I32], I32),
        "kvq_store": ([C, P, P, I32, P, I32, P], I32),
        "kvq_rotate_q": ([P, I32, P, I32, I32, P], I32),
        "kvq_store_rotate_q": ([C, P, P, I32, P, I32, P, I32, P, I32, P], I32),
        "kvq_decode_attn": ([C, P, I32, P, I32, P, I32, I32, F, I32, P, P, P, P], I32),
        "kvq_decode_attn_rows": ([C, P, I32, P, I32, P, I32, I32, F, I32, P, P, P, P], I32),
        "kvq_merge": ([C, P, P, P, P, I32, I32, I32, I32, I32, P, P, P], I32),
        "kvq_tq_rotate_q": ([P, P, I32, P], I32),
        "kvq_stream_read": ([P, ctypes.c_size_t, I32, P, P], I32),
        "kvq_decode_attn_sel": ([C, P, I32, P, I32, P, P, I32, I32, F, I32, P, P, P, P], I32),
        "kvq_attend_workspace_bytes": ([C, I32, I32, I32, I32], ctypes.c_size_t),
        "kvq_attend": ([C, P, I32, P, I32, P, I32, I32, F, I32, P, ctypes.c_size_t, P, P, P], I32),
        "kvq_attend_noalloc": ([C, P, I32, P, I32, P, I32, I32, F, I32, P, P, P], I32),
        "kvq_prefill_attn": ([C, P, I32, P, I32, P, I32, I32, F, I32, P, P, P, P], I32),
        "kvq_decode_step": ([C, P, P, I32, P, I32, I32, P, I32, P, I32, I32, F, I32, P, ctypes.c_size_t, P, P, P],
                            I32),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    return L


lib = _load()


class KvqError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {lib.kvq_status_string(status).decode()} ({status})")


def _check(status, what):
    if status != KVQ_OK:
        raise KvqError(status, what)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t, name, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def kvq_row_bytes(fmt, head_dim, rope_dim=0):
    return int(lib.kvq_row_bytes(fmt, head_dim, rope_dim))


def kvq_num_splits(max_seq_len, split_keys):
    return int(lib.kvq_num_splits(max_seq_len, split_keys))


class Q4Cache:
    """Paged Hadamard-32 K and V pools: [num_pages][H_kv][page_size][row_bytes] uint8 -- the
    4-bit format by default, or fmt=FMT_Q8_H32 / FMT_Q6_H32."""

    def __init__(self, num_pages, num_kv_heads, head_dim, page_size=16, device="cuda", fmt=FMT_Q4_H32):
        if fmt not in H32_FORMATS:
            raise ValueError(f"not a Hadamard-32 format: {fmt}")
        self.fmt = fmt
        rb = kvq_row_bytes(fmt, head_dim)
        if rb == 0:
            raise ValueError(f"head_dim {head_dim} is not a multiple of 32")
        shape = (num_pages, num_kv_heads, page_size, rb)
        self.k_pool = torch.zeros(shape, dtype=torch.uint8, device=device)
        self.v_pool = torch.zeros(shape, dtype=torch.uint8, device=device)
        self.num_kv_heads, self.head_dim, self.page_size, self.num_pages = num_kv_heads, head_dim, page_size, num_pages
        self.rope_dim = 0
        self.dv = head_dim
        self.desc = KvqCacheDesc(fmt, num_kv_heads, head_dim, 0, page_size, num_pages,
                                 self.k_pool.data_ptr(), self.v_pool.data_ptr(), None)

    @property
    def device(self):
        return self.k_pool.device

    def pool_bytes(self):
        return int(lib.kvq_pool_bytes(ctypes.byref(self.desc)))


class Fp8Cache:
    """Paged fp8 e4m3 latent rows: codes [num_pages*page_size][head_dim] uint8, scales [..][2] f32."""

    fmt = FMT_FP8_E4M3_ROW

    def __init__(self, num_pages, head_dim=576, rope_dim=64, page_size=16, device="cuda"):
        slots = num_pages * page_size
        self.codes = torch.zeros((slots, head_dim), dtype=torch.uint8, device=device)
        self.scales = torch.zeros((slots, 2), dtype=torch.float32, device=device)
        self.num_kv_heads, self.head_dim, self.rope_dim = 1, head_dim, rope_dim
        self.page_size, self.num_pages = page_size, num_pages
        self.dv = head_dim - rope_dim
        self.desc = KvqCacheDesc(FMT_FP8_E4M3_ROW, 1, head_dim, rope_dim, page_size, num_pages,
                                 self.codes.data_ptr(), None, self.scales.data_ptr())

    @property
    def device(self):
        return self.codes.device

    def pool_bytes(self):
        return int(lib.kvq_pool_bytes(ctypes.byref(self.desc)))


class TqCache:
    """Paged rotated-int4 + Lloyd-Max latent rows: codes [num_pages*page_size][288] uint8 (nibbles of the
    512 latent and 64 rope values), radii [..][2] f32.  Stores and decodes as Fp8Cache does: kvq_store
    takes k [n_tokens][576] and v None; kvq_decode_attn takes the unrotated query."""

    fmt = FMT_TQ4_LATENT

    def __init__(self, num_pages, page_size=16, device="cuda"):
        slots = num_pages * page_size
        self.codes = torch.zeros((slots, 288), dtype=torch.uint8, device=device)
        self.scales = torch.zeros((slots, 2), dtype=torch.float32, device=device)
        self.num_kv_heads, self.head_dim, self.rope_dim = 1, 576, 64
        self.page_size, self.num_pages = page_size, num_pages
        self.dv = 512
        self.desc = KvqCacheDesc(FMT_TQ4_LATENT, 1, 576, 64, page_size, num_pages, self.codes.data_ptr(), None,
                                 self.scales.data_ptr())

    @property
    def device(self):
        return self.codes.device

    def pool_bytes(self):
        return int(lib.kvq_pool_bytes(ctypes.byref(self.desc)))


def kvq_store(cache, k, v, slot_mapping):
    """Quantize new rows into the cache.

    Q4: k, v [n_tokens][H_kv][head_dim] (f32/bf16/f16).  FP8: k [n_tokens][head_dim], v None.
    slot_mapping: int64 [n_tokens] (negative slots are skipped)."""
    n = int(slot_mapping.shape[0])
    dt = _DTYPES.get(k.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {k.dtype}")
    if cache.fmt in H32_FORMATS:
        shape = (n, cache.num_kv_heads, cache.head_dim)
        kp = _dev(k, "k", shape=shape)
        vp = _dev(v, "v", dtype=k.dtype, shape=shape)
    else:
        if v is not None:
            raise ValueError("the latent caches take no v")
        kp = _dev(k, "k", shape=(n, cache.head_dim))
        vp = None
    sp = _dev(slot_mapping, "slot_mapping", dtype=torch.int64)
    _check(lib.kvq_store(ctypes.byref(cache.desc), kp, vp, dt, sp, n, _stream(k)), "kvq_store")


def kvq_rotate_q(q, out=None):
    """q_rot = H32 q for every 32-group of the last axis; returns an f32 tensor of q's shape."""
    dt = _DTYPES.get(q.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    D = int(q.shape[-1])
    rows = q.numel() // D if D else 0
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    qp = _dev(q, "q")
    op = _dev(out, "out", dtype=torch.float32, shape=q.shape)
    _check(lib.kvq_rotate_q(qp, dt, op, rows, D, _stream(q)), "kvq_rotate_q")
    return out


def kvq_tq_rotate_q(q, out=None):
    """The TQ4 latent format's query rotation of f32 rows [..., 576]; returns an f32 tensor of q's shape
    (out may be q itself)."""
    if q.dtype != torch.float32 or int(q.shape[-1]) != 576:
        raise ValueError("kvq_tq_rotate_q takes f32 rows of 576")
    rows = q.numel() // 576
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    qp = _dev(q, "q")
    op = _dev(out, "out", dtype=torch.float32, shape=q.shape)
    _check(lib.kvq_tq_rotate_q(qp, op, rows, _stream(q)), "kvq_tq_rotate_q")
    return out


def kvq_store_rotate_q(cache, k, v, slot_mapping, q, out=None):
    """kvq_store(cache, k, v, slot_mapping) and the query rotation in one launch; returns the rotated
    query (f32, q's shape).  Hadamard-32 caches: kvq_rotate_q(q).  TQ4 cache: v is None, q is f32
    [..., 576] and the rotation is kvq_tq_rotate_q(q)."""
    if cache.fmt == FMT_TQ4_LATENT:
        if v is not None:
            raise ValueError("the latent caches take no v")
        if q.dtype != torch.float32 or int(q.shape[-1]) != 576:
            raise ValueError("the TQ4 query rotation takes f32 rows of 576")
        n = int(slot_mapping.shape[0])
        kdt = _DTYPES.get(k.dtype)
        if kdt is None:
            raise ValueError(f"unsupported dtype {k.dtype}")
        kp = _dev(k, "k", shape=(n, cache.head_dim))
        sp = _dev(slot_mapping, "slot_mapping", dtype=torch.int64)
        rows = q.numel() // 576
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        qp = _dev(q, "q")
        op = _dev(out, "out", dtype=torch.float32, shape=q.shape)
        _check(lib.kvq_store_rotate_q(ctypes.byref(cache.desc), kp, None, kdt, sp, n, qp, DT_F32, op, rows,
                                      _stream(q)), "kvq_store_rotate_q")
        return out
    if cache.fmt not in H32_FORMATS:
        raise ValueError("kvq_store_rotate_q takes a Hadamard-32 or TQ4 cache")
    n = int(slot_mapping.shape[0])
    kdt, qdt = _DTYPES.get(k.dtype), _DTYPES.get(q.dtype)
    if kdt is None or qdt is None:
        raise ValueError(f"unsupported dtype {k.dtype if kdt is None else q.dtype}")
    shape = (n, cache.num_kv_heads, cache.head_dim)
    kp = _dev(k, "k", shape=shape)
    vp = _dev(v, "v", dtype=k.dtype, shape=shape)
    sp = _dev(slot_mapping, "slot_mapping", dtype=torch.int64)
    if int(q.shape[-1]) != cache.head_dim:
        raise ValueError(f"q rows must have the cache's head_dim {cache.head_dim}")
    rows = q.numel() // cache.head_dim
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    qp = _dev(q, "q")
    op = _dev(out, "out", dtype=torch.float32, shape=q.shape)
    _check(lib.kvq_store_rotate_q(ctypes.byref(cache.desc), kp, vp, kdt, sp, n, qp, qdt, op, rows, _stream(q)),
           "kvq_store_rotate_q")
    return out


def partial_shapes(cache, batch, n_q_heads, max_seq_len, split_keys):
    S = kvq_num_splits(max_seq_len, split_keys)
    return (batch, n_q_heads, S, cache.dv), (batch, n_q_heads, S)


def kvq_decode_attn(cache, q, page_table, seq_lens, max_seq_len, sm_scale, split_keys, part_acc=None, part_m=None,
                    part_z=None):
    """Split-K decode attention; returns the partials (acc, m, z).

    q: f32 [B][H_q][head_dim] (for Q4 already rotated with kvq_rotate_q);
    page_table: int32 [B][max_pages]; seq_lens: int32 [B]."""
    B, Hq, D = q.shape
    acc_shape, mz_shape = partial_shapes(cache, B, Hq, max_seq_len, split_keys)
    if part_acc is None:
        part_acc = torch.empty(acc_shape, dtype=torch.float32, device=q.device)
        part_m = torch.empty(mz_shape, dtype=torch.float32, device=q.device)
        part_z = torch.empty(mz_shape, dtype=torch.float32, device=q.device)
    qp = _dev(q, "q", dtype=torch.float32, shape=(B, Hq, cache.head_dim))
    ptp = _dev(page_table, "page_table", dtype=torch.int32)
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table must be [batch][max_pages]")
    slp = _dev(seq_lens, "seq_lens", dtype=torch.int32, shape=(B,))
    pa = _dev(part_acc, "part_acc", dtype=torch.float32, shape=acc_shape)
    pm = _dev(part_m, "part_m", dtype=torch.float32, shape=mz_shape)
    pz = _dev(part_z, "part_z", dtype=torch.float32, shape=mz_shape)
    _check(lib.kvq_decode_attn(ctypes.byref(cache.desc), qp, Hq, ptp, int(page_table.shape[1]), slp, B,
                               int(max_seq_len), float(sm_scale), int(split_keys), pa, pm, pz, _stream(q)),
           "kvq_decode_attn")
    return part_acc, part_m, part_z


def kvq_decode_attn_rows(cache, q, page_table, seq_lens, max_seq_len, sm_scale, split_keys, part_acc=None,
                         part_m=None, part_z=None):
    """Split-K decode attention for R query rows of one sequence (drafted rows): row r attends
    positions [0, seq_lens[r]) of the sequence with page-table row `page_table`; returns the partials
    (acc, m, z), the same bits kvq_decode_attn gives with that row repeated R times.

    q: f32 [R][H_q][head_dim] rotated with kvq_rotate_q; page_table: int32 [max_pages];
    seq_lens: int32 [R].  Merge with kvq_merge(cache, ..., seq_lens, ...)."""
    R, Hq, D = q.shape
    acc_shape, mz_shape = partial_shapes(cache, R, Hq, max_seq_len, split_keys)
    if part_acc is None:
        part_acc = torch.empty(acc_shape, dtype=torch.float32, device=q.device)
        part_m = torch.empty(mz_shape, dtype=torch.float32, device=q.device)
        part_z = torch.empty(mz_shape, dtype=torch.float32, device=q.device)
    qp = _dev(q, "q", dtype=torch.float32, shape=(R, Hq, cache.head_dim))
    if page_table.dim() != 1:
        raise ValueError("page_table must be one row [max_pages]")
    ptp = _dev(page_table, "page_table", dtype=torch.int32)
    slp = _dev(seq_lens, "seq_lens", dtype=torch.int32, shape=(R,))
    pa = _dev(part_acc, "part_acc", dtype=torch.float32, shape=acc_shape)
    pm = _dev(part_m, "part_m", dtype=torch.float32, shape=mz_shape)
    pz = _dev(part_z, "part_z", dtype=torch.float32, shape=mz_shape)
    _check(lib.kvq_decode_attn_rows(ctypes.byref(cache.desc), qp, Hq, ptp, int(page_table.shape[0]), slp, R,
                                    int(max_seq_len), float(sm_scale), int(split_keys), pa, pm, pz, _stream(q)),
           "kvq_decode_attn_rows")
    return part_acc, part_m, part_z


def kvq_prefill_attn(cache, q, page_table, row_lens, max_seq_len, sm_scale, split_keys, part_acc=None, part_m=None,
                     part_z=None):
    """Attention of a prompt chunk's rows over their sequence's 4-bit cache, as partials: row r
    attends positions [0, row_lens[r]) of the sequence with page-table row `page_table`.

    q: f32 [R][H_q][head_dim] rotated with kvq_rotate_q; page_table: int32 [max_pages];
    row_lens: int32 [R].  Merge with kvq_merge(cache, ..., row_lens, max_seq_len, split_keys)."""
    R, Hq, D = q.shape
    acc_shape, mz_shape = partial_shapes(cache, R, Hq, max_seq_len, split_keys)
    if part_acc is None:
        part_acc = torch.empty(acc_shape, dtype=torch.float32, device=q.device)
        part_m = torch.empty(mz_shape, dtype=torch.float32, device=q.device)
        part_z = torch.empty(mz_shape, dtype=torch.float32, device=q.device)
    qp = _dev(q, "q", dtype=torch.float32, shape=(R, Hq, cache.head_dim))
    if page_table.dim() != 1:
        raise ValueError("page_table must be one row [max_pages]")
    ptp = _dev(page_table, "page_table", dtype=torch.int32)
    rlp = _dev(row_lens, "row_lens", dtype=torch.int32, shape=(R,))
    pa = _dev(part_acc, "part_acc", dtype=torch.float32, shape=acc_shape)
    pm = _dev(part_m, "part_m", dtype=torch.float32, shape=mz_shape)
    pz = _dev(part_z, "part_z", dtype=torch.float32, shape=mz_shape)
    _check(lib.kvq_prefill_attn(ctypes.byref(cache.desc), qp, Hq, ptp, int(page_table.shape[0]), rlp, R,
                                int(max_seq_len), float(sm_scale), int(split_keys), pa, pm, pz, _stream(q)),
           "kvq_prefill_attn")
    return part_acc, part_m, part_z


def kvq_decode_attn_sel(cache, q, page_table, sel, n_sel, sm_scale, split_keys, part_acc=None, part_m=None,
                        part_z=None):
    """Decode attention over selected rows of the fp8 latent cache; returns the partials (acc, m, z).

    sel: int32 [B][max_sel] absolute positions (entries outside the page capacity, e.g. -1, are
    absent); n_sel: int32 [B] entries used.  Merge with kvq_merge(cache, ..., n_sel, max_sel, split_keys)."""
    B, H, D = q.shape
    max_sel = int(sel.shape[1])
    acc_shape, mz_shape = partial_shapes(cache, B, H, max_sel, split_keys)
    if part_acc is None:
        part_acc = torch.empty(acc_shape, dtype=torch.float32, device=q.device)
        part_m = torch.empty(mz_shape, dtype=torch.float32, device=q.device)
        part_z = torch.empty(mz_shape, dtype=torch.float32, device=q.device)
    qp = _dev(q, "q", dtype=torch.float32, shape=(B, H, cache.head_dim))
    ptp = _dev(page_table, "page_table", dtype=torch.int32)
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table must be [batch][max_pages]")
    sp = _dev(sel, "sel", dtype=torch.int32, shape=(B, max_sel))
    np_ = _dev(n_sel, "n_sel", dtype=torch.int32, shape=(B,))
    pa = _dev(part_acc, "part_acc", dtype=torch.float32, shape=acc_shape)
    pm = _dev(part_m, "part_m", dtype=torch.float32, shape=mz_shape)
    pz = _dev(part_z, "part_z", dtype=torch.float32, shape=mz_shape)
    _check(lib.kvq_decode_attn_sel(ctypes.byref(cache.desc), qp, H, ptp, int(page_table.shape[1]), sp, np_, B,
                                   max_sel, float(sm_scale), int(split_keys), pa, pm, pz, _stream(q)),
           "kvq_decode_attn_sel")
    return part_acc, part_m, part_z


def kvq_merge(cache, part_acc, part_m, part_z, seq_lens, max_seq_len, split_keys, out=None, lse=None,
              want_lse=True):
    """Log-sum-exp merge of the partials, then (Q4, Q8, Q6, TQ4) the inverse rotation.  Returns (out, lse)."""
    B, Hq, S, Dv = part_acc.shape
    if out is None:
        out = torch.empty((B, Hq, Dv), dtype=torch.float32, device=part_acc.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=part_acc.device)
    acc_shape, mz_shape = partial_shapes(cache, B, Hq, max_seq_len, split_keys)
    pa = _dev(part_acc, "part_acc", dtype=torch.float32, shape=acc_shape)
    pm = _dev(part_m, "part_m", dtype=torch.float32, shape=mz_shape)
    pz = _dev(part_z, "part_z", dtype=torch.float32, shape=mz_shape)
    slp = _dev(seq_lens, "seq_lens", dtype=torch.int32, shape=(B,))
    op = _dev(out, "out", dtype=torch.float32, shape=(B, Hq, Dv))
    lp = _dev(lse, "lse", dtype=torch.float32, shape=(B, Hq)) if lse is not None else None
    _check(lib.kvq_merge(ctypes.byref(cache.desc), pa, pm, pz, slp, B, Hq, int(max_seq_len), int(split_keys),
                         1 if cache.fmt in ROTATED_FORMATS else 0, op, lp, _stream(part_acc)), "kvq_merge")
    return out, lse


def kvq_attend_workspace_bytes(cache, batch, n_q_heads, max_seq_len, split_keys):
    return int(lib.kvq_attend_workspace_bytes(ctypes.byref(cache.desc), batch, n_q_heads, int(max_seq_len),
                                              int(split_keys)))


def kvq_attend(cache, q, page_table, seq_lens, max_seq_len, sm_scale, split_keys, workspace=None, out=None, lse=None,
               want_lse=True):
    """Decode attention and merge in one call (kvq_decode_attn + kvq_merge, the partials in `workspace`,
    a uint8 device tensor of at least kvq_attend_workspace_bytes bytes).  Returns (out, lse)."""
    B, Hq, D = q.shape
    need = kvq_attend_workspace_bytes(cache, B, Hq, max_seq_len, split_keys)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, cache.dv), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    qp = _dev(q, "q", dtype=torch.float32, shape=(B, Hq, cache.head_dim))
    ptp = _dev(page_table, "page_table", dtype=torch.int32)
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table must be [batch][max_pages]")
    slp = _dev(seq_lens, "seq_lens", dtype=torch.int32, shape=(B,))
    wp = _dev(workspace, "workspace", dtype=torch.uint8)
    op = _dev(out, "out", dtype=torch.float32, shape=(B, Hq, cache.dv))
    lp = _dev(lse, "lse", dtype=torch.float32, shape=(B, Hq)) if lse is not None else None
    _check(lib.kvq_attend(ctypes.byref(cache.desc), qp, Hq, ptp, int(page_table.shape[1]), slp, B, int(max_seq_len),
                          float(sm_scale), int(split_keys), wp, workspace.numel(), op, lp, _stream(q)), "kvq_attend")
    return out, lse


def kvq_decode_step(cache, k, v, q, page_table, seq_lens, max_seq_len, sm_scale, split_keys, workspace=None,
                    out=None, lse=None, want_lse=True):
    """A decode step in two launches: token b's K and V rows (k, v: [batch][num_kv_heads][head_dim]) stored
    at position seq_lens[b] - 1 of sequence b through the page table, the query q ([batch][n_q_heads]
    [head_dim], before rotation) rotated, attention and merge.  Returns (out, lse), the same bits as
    kvq_store_rotate_q + kvq_attend.  Fp8Cache: k is the latent rows [batch][head_dim], v None, q f32
    (the same bits as kvq_store + kvq_attend)."""
    B, Hq, D = q.shape
    need = kvq_attend_workspace_bytes(cache, B, Hq, max_seq_len, split_keys)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, cache.dv), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    kdt, qdt = _DTYPES.get(k.dtype), _DTYPES.get(q.dtype)
    if kdt is None or qdt is None:
        raise ValueError(f"unsupported dtype {k.dtype if kdt is None else q.dtype}")
    if cache.fmt in H32_FORMATS:
        shape = (B, cache.num_kv_heads, cache.head_dim)
        kp = _dev(k, "k", shape=shape)
        vp = _dev(v, "v", dtype=k.dtype, shape=shape)
    else:
        if v is not None:
            raise ValueError("the latent caches take no v")
        kp = _dev(k, "k", shape=(B, cache.head_dim))
        vp = None
    qp = _dev(q, "q", shape=(B, Hq, cache.head_dim))
    ptp = _dev(page_table, "page_table", dtype=torch.int32)
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table must be [batch][max_pages]")
    slp = _dev(seq_lens, "seq_lens", dtype=torch.int32, shape=(B,))
    wp = _dev(workspace, "workspace", dtype=torch.uint8)
    op = _dev(out, "out", dtype=torch.float32, shape=(B, Hq, cache.dv))
    lp = _dev(lse, "lse", dtype=torch.float32, shape=(B, Hq)) if lse is not None else None
    _check(lib.kvq_decode_step(ctypes.byref(cache.desc), kp, vp, kdt, qp, qdt, Hq, ptp, int(page_table.shape[1]),
                               slp, B, int(max_seq_len), float(sm_scale), int(split_keys), wp, workspace.numel(),
                               op, lp, _stream(q)), "kvq_decode_step")
    return out, lse


NOALLOC_SCRATCH_BYTES = 64 << 20   # KVQ_NOALLOC_SCRATCH_BYTES


def kvq_attend_noalloc(cache, q, page_table, seq_lens, max_seq_len, sm_scale, split_keys, out, lse=None):
    """kvq_attend with the partials in the library's static per-GPU scratch (no workspace argument,
    nothing allocated; out and lse must be given).  Calls that overlap on one GPU race on the scratch."""
    B, Hq, D = q.shape
    qp = _dev(q, "q", dtype=torch.float32, shape=(B, Hq, cache.head_dim))
    ptp = _dev(page_table, "page_table", dtype=torch.int32)
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table must be [batch][max_pages]")
    slp = _dev(seq_lens, "seq_lens", dtype=torch.int32, shape=(B,))
    op = _dev(out, "out", dtype=torch.float32, shape=(B, Hq, cache.dv))
    lp = _dev(lse, "lse", dtype=torch.float32, shape=(B, Hq)) if lse is not None else None
    _check(lib.kvq_attend_noalloc(ctypes.byref(cache.desc), qp, Hq, ptp, int(page_table.shape[1]), slp, B,
                                  int(max_seq_len), float(sm_scale), int(split_keys), op, lp, _stream(q)),
           "kvq_attend_noalloc")
    return out, lse


def kvq_stream_read(src, non_temporal=True, xor_out=None):
    """Reads the device buffer `src` (bytes a multiple of 16 KiB) once through LDS DMA -- the
    read-bandwidth measurement.  Returns the int32 device tensor holding the XOR of the 32-bit words
    of its final 16 KiB block."""
    if xor_out is None:
        xor_out = torch.zeros((1,), dtype=torch.int32, device=src.device)
    sp = _dev(src, "src")
    xp = _dev(xor_out, "xor_out", dtype=torch.int32, shape=(1,))
    _check(lib.kvq_stream_read(sp, src.numel() * src.element_size(), 1 if non_temporal else 0, xp, _stream(src)),
           "kvq_stream_read")
    return xor_out


def decode_step(cache, q, page_table, seq_lens, max_seq_len, sm_scale, split_keys, bufs=None, new_kv=None):
    """[store the step's rows] -> rotate (Q4, TQ4) -> decode -> merge on preallocated buffers; returns (out, lse).

    new_kv = (k, v, slot_mapping) stores those rows first (for the 4-bit cache in the same launch as the
    query rotation, kvq_store_rotate_q; v is None for the fp8 cache)."""
    q_rot = None if bufs is None else bufs.get("q_rot")
    if cache.fmt in H32_FORMATS:
        if new_kv is not None:
            q = kvq_store_rotate_q(cache, *new_kv, q, out=q_rot)
        else:
            q = kvq_rotate_q(q, out=q_rot)
    elif cache.fmt == FMT_TQ4_LATENT:
        if new_kv is not None:
            q = kvq_store_rotate_q(cache, *new_kv, q, out=q_rot)
        else:
            q = kvq_tq_rotate_q(q, out=q_rot)
    elif new_kv is not None:
        kvq_store(cache, *new_kv)
    pa, pm, pz = kvq_decode_attn(cache, q, page_table, seq_lens, max_seq_len, sm_scale, split_keys,
                                 *(() if bufs is None else (bufs["part_acc"], bufs["part_m"], bufs["part_z"])))
    return kvq_merge(cache, pa, pm, pz, seq_lens, max_seq_len, split_keys,
                     out=None if bufs is None else bufs.get("out"), lse=None if bufs is None else bufs.get("lse"))
