"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Bar: cache codes and scales bit-exact; attention output within 2e-3 of the
oracle's fp64 result (max abs error / max abs reference value, per sequence
and head); outputs bit-identical between a sequence run alone and inside a
batch.  Sizes here run in seconds and still span several tiles, several
splits and ragged tails; test_gpu_full_size.py covers the full workloads.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from helpers import TOL, MlaCase, Q4Case, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvq():
    assert torch.cuda.is_available(), "no GPU"
    import fp8_quantized_kv_amd as m
    return m


def _say(*a):
    print(*a, flush=True)


# ----------------------------------------------------------------- store

@pytest.mark.parametrize("D", [64, 128, 256, 512])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_store_q4_bit_exact(kvq, D, dtype):
    _say(f"store_q4 D={D} dtype={dtype}")
    g = torch.Generator().manual_seed(D)
    n_tok, H, ps, pages = 300, 3, 16, 40
    k = (torch.randn((n_tok, H, D), generator=g) * torch.exp(torch.randn((n_tok, H, 1), generator=g))).to(dtype)
    v = torch.randn((n_tok, H, D), generator=g).to(dtype)
    k[5, 1, 3] = 40.0
    k[7] = 0.0                          # all-zero rows: scale 0, codes 0
    slots = torch.randperm(pages * ps, generator=g)[:n_tok].to(torch.int64)
    slots[::17] = -1                    # skipped tokens
    cache = kvq.Q4Cache(pages, H, D, ps)
    kvq.kvq_store(cache, k.cuda(), v.cuda(), slots.cuda())
    kref = np.zeros(cache.k_pool.shape, np.uint8)
    vref = np.zeros_like(kref)
    oracle.q4_store(kref, vref, k.float().numpy(), v.float().numpy(), slots.numpy(), ps)
    torch.cuda.synchronize()
    assert np.array_equal(cache.k_pool.cpu().numpy(), kref)
    assert np.array_equal(cache.v_pool.cpu().numpy(), vref)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_store_q4_subnormal_scales_bit_exact(kvq, dtype):
    """Rows of magnitude 2^-12 .. 2^-30: group scales amax/8 fall among the
    binary16 subnormals (m * 2^-24) or round to 0 (inert groups); codes and
    scales bit-exact against the oracle."""
    _say(f"store_q4 subnormal scales dtype={dtype}")
    g = torch.Generator().manual_seed(77)
    n_tok, H, D, ps, pages = 400, 2, 256, 16, 30
    mag = torch.pow(2.0, -torch.randint(12, 31, (n_tok, H, 1), generator=g).float())
    k = (torch.randn((n_tok, H, D), generator=g) * mag).to(dtype)
    v = (torch.randn((n_tok, H, D), generator=g) * mag.flip(0)).to(dtype)
    slots = torch.randperm(pages * ps, generator=g)[:n_tok].to(torch.int64)
    cache = kvq.Q4Cache(pages, H, D, ps)
    kvq.kvq_store(cache, k.cuda(), v.cuda(), slots.cuda())
    kref = np.zeros(cache.k_pool.shape, np.uint8)
    vref = np.zeros_like(kref)
    oracle.q4_store(kref, vref, k.float().numpy(), v.float().numpy(), slots.numpy(), ps)
    torch.cuda.synchronize()
    sc = kref[..., D // 2:].copy().view(np.float16).astype(np.float32)
    assert np.count_nonzero((sc > 0) & (sc < 2.0 ** -14)) > 1000 and np.count_nonzero(sc == 0) > 1000
    assert np.array_equal(cache.k_pool.cpu().numpy(), kref)
    assert np.array_equal(cache.v_pool.cpu().numpy(), vref)


@pytest.mark.parametrize("split", [512, 2048])
def test_decode_q4_subnormal_scales(kvq, split):
    """Attention over a cache whose every group scale is a binary16 subnormal
    (K and V scaled by 2^-17, the query by 2^17): within the tolerance of the
    oracle's fp64 attention, on both matrix-core kernels (split 512: the
    wave-pair kernel; 2048: the four-wave kernel)."""
    w = wl.shrink(wl.GQA_32K, n_layers=1, batch=2, seq_len=0)
    case = Q4Case(w, [3000, 1500], kv_scale=2.0 ** -17)
    sc = case.k_ref[..., w.head_dim // 2:].copy().view(np.float16).astype(np.float32)
    used = sc[sc != 0]
    assert used.size > 10000 and np.all(used < 2.0 ** -14)
    _say(f"decode_q4 subnormal scales split={split}")
    o, lse = case.gpu_attention(split)
    ro, rl = case.ref_attention()
    err = rel_err(o, ro)
    _say(f"  max_rel_err={err.max():.2e}")
    assert np.all(np.isfinite(o)) and err.max() < TOL
    assert np.max(np.abs(lse - rl)) < 1e-3 * max(1.0, np.abs(rl).max())


@pytest.mark.parametrize("bits", [6, 8])
@pytest.mark.parametrize("D", [64, 128, 256, 512])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_store_blk_bit_exact(kvq, bits, D, dtype):
    """The 6- and 8-bit block formats: codes and scales bit-exact against the
    oracle, with skipped slots, an all-zero row and a large value."""
    _say(f"store bits={bits} D={D} dtype={dtype}")
    g = torch.Generator().manual_seed(D + bits)
    n_tok, H, ps, pages = 300, 3, 16, 40
    k = (torch.randn((n_tok, H, D), generator=g) * torch.exp(torch.randn((n_tok, H, 1), generator=g))).to(dtype)
    v = torch.randn((n_tok, H, D), generator=g).to(dtype)
    k[5, 1, 3] = 40.0
    k[7] = 0.0
    slots = torch.randperm(pages * ps, generator=g)[:n_tok].to(torch.int64)
    slots[::17] = -1
    fmt = kvq.FMT_Q8_H32 if bits == 8 else kvq.FMT_Q6_H32
    cache = kvq.Q4Cache(pages, H, D, ps, fmt=fmt)
    kvq.kvq_store(cache, k.cuda(), v.cuda(), slots.cuda())
    kref = np.zeros(cache.k_pool.shape, np.uint8)
    vref = np.zeros_like(kref)
    oracle.q4_store(kref, vref, k.float().numpy(), v.float().numpy(), slots.numpy(), ps)
    torch.cuda.synchronize()
    assert np.array_equal(cache.k_pool.cpu().numpy(), kref)
    assert np.array_equal(cache.v_pool.cpu().numpy(), vref)


@pytest.mark.parametrize("bits", [6, 8])
def test_blk_decode_matches_oracle(kvq, bits):
    """Decode + merge over the 6- and 8-bit caches (the matrix-core kernel at
    head_dim 256): a ragged batch with tails and an empty sequence, splits of
    512 and 2048, the one-launch store + rotation of a new token, and batch
    invariance."""
    import fp8_quantized_kv_amd as kvq_mod
    w = wl.shrink(wl.RAGGED, prefill_chunk=0, bits=bits)
    lens = [3000, 17, 0, 1100]
    case = Q4Case(w, lens)
    assert np.array_equal(case.cache.k_pool.cpu().numpy(), case.k_ref)
    ro, rl = case.ref_attention()
    for split in (512, 2048):
        o, lse = case.gpu_attention(split)
        err = rel_err(o, ro)
        _say(f"  bits={bits} split={split} max_rel_err={err.max():.2e}")
        assert err.max() < TOL
        fin = np.isfinite(rl)
        assert np.array_equal(fin, np.isfinite(lse)) and np.max(np.abs(lse[fin] - rl[fin])) < 1e-3 * max(1.0, np.abs(rl[fin]).max())
        assert np.all(o[2] == 0)
    # alone == in the batch, bit for bit
    o_b, l_b = case.gpu_attention(512)
    q_rot = kvq_mod.kvq_rotate_q(case.q)
    for b in (0, 3):
        pa, pm, pz = kvq_mod.kvq_decode_attn(case.cache, q_rot[b:b + 1].contiguous(), case.page_table[b:b + 1].contiguous(),
                                             case.seq_lens[b:b + 1].contiguous(), case.max_seq_len, w.sm_scale, 512)
        o1, l1 = kvq_mod.kvq_merge(case.cache, pa, pm, pz, case.seq_lens[b:b + 1].contiguous(), case.max_seq_len, 512)
        assert np.array_equal(o1.cpu().numpy()[0], o_b[b]) and np.array_equal(l1.cpu().numpy()[0], l_b[b])
    # one-launch store + rotation on this format equals the two calls
    gk = torch.Generator(device="cuda").manual_seed(5)
    kn = torch.randn((1, w.n_kv_heads, w.head_dim), generator=gk, device="cuda").to(torch.bfloat16)
    vn = torch.randn((1, w.n_kv_heads, w.head_dim), generator=gk, device="cuda").to(torch.bfloat16)
    sl = torch.tensor([int(case.lay.page_table[0, 0]) * w.page_size + 2], dtype=torch.int64, device="cuda")
    before_k, before_v = case.cache.k_pool.clone(), case.cache.v_pool.clone()
    qr2 = kvq_mod.kvq_store_rotate_q(case.cache, kn, vn, sl, case.q)
    fused_k, fused_v = case.cache.k_pool.clone(), case.cache.v_pool.clone()
    case.cache.k_pool.copy_(before_k)
    case.cache.v_pool.copy_(before_v)
    kvq_mod.kvq_store(case.cache, kn, vn, sl)
    torch.cuda.synchronize()
    assert torch.equal(qr2, q_rot)
    assert torch.equal(case.cache.k_pool, fused_k) and torch.equal(case.cache.v_pool, fused_v)


@pytest.mark.parametrize("bits", [6, 8])
@pytest.mark.parametrize("G", [1, 6, 8, 12])
def test_blk_mfma_edges(kvq, G, bits):
    """The 8- and 6-bit formats on the matrix-core kernel: group sizes on both
    sides of the packed hi/lo columns (G <= 8 packed, 12 not), lengths at
    sub-tile, 16-row run and wave-quarter boundaries, splits of 512, 1024 and
    2048 keys."""
    w = wl.shrink(wl.RAGGED, prefill_chunk=0, bits=bits, n_q_heads=4 * G)
    lens = [1, 31, 32, 33, 129, 1024 + 16, 2048 + 5]
    case = Q4Case(w, lens)
    ro, rl = case.ref_attention()
    for split in (512, 1024, 2048):
        o, lse = case.gpu_attention(split)
        err = rel_err(o, ro)
        _say(f"  bits={bits} G={G} split={split} max_rel_err={err.max():.2e}")
        assert err.max() < TOL
        fin = np.isfinite(rl)
        assert np.array_equal(fin, np.isfinite(lse)) and np.max(np.abs(lse[fin] - rl[fin])) < 1e-3 * max(1.0, np.abs(rl[fin]).max())


@pytest.mark.parametrize("bits", [6, 8])
def test_blk_mfma_pages_and_order(kvq, bits):
    """8- and 6-bit matrix-core decode with 64-token pages drawn in shuffled
    order: parity with the oracle, and a sequence decoded alone equals the
    same sequence inside the batch, bit for bit."""
    import fp8_quantized_kv_amd as kvq_mod
    w = wl.shrink(wl.RAGGED, prefill_chunk=0, bits=bits, page_size=64, shuffle_pages=True)
    lens = [5000, 64, 1, 3333]
    case = Q4Case(w, lens)
    assert np.array_equal(case.cache.k_pool.cpu().numpy(), case.k_ref)
    assert np.array_equal(case.cache.v_pool.cpu().numpy(), case.v_ref)
    ro, rl = case.ref_attention()
    o, lse = case.gpu_attention(2048)
    err = rel_err(o, ro)
    _say(f"  bits={bits} page=64 max_rel_err={err.max():.2e}")
    assert err.max() < TOL
    q_rot = kvq_mod.kvq_rotate_q(case.q)
    for b in (0, 3):
        pa, pm, pz = kvq_mod.kvq_decode_attn(case.cache, q_rot[b:b + 1].contiguous(), case.page_table[b:b + 1].contiguous(),
                                             case.seq_lens[b:b + 1].contiguous(), case.max_seq_len, w.sm_scale, 2048)
        o1, l1 = kvq_mod.kvq_merge(case.cache, pa, pm, pz, case.seq_lens[b:b + 1].contiguous(), case.max_seq_len, 2048)
        assert np.array_equal(o1.cpu().numpy()[0], o[b]) and np.array_equal(l1.cpu().numpy()[0], lse[b])


def test_store_q4_token_by_token_equals_bulk(kvq):
    """Storing a sequence one token per call gives the same bytes as one call."""
    w = wl.TINY
    a = Q4Case(w, [w.seq_len], build_oracle=False)
    b = Q4Case(w, [w.seq_len], store_chunk=1, build_oracle=False)
    torch.cuda.synchronize()
    assert torch.equal(a.cache.k_pool, b.cache.k_pool) and torch.equal(a.cache.v_pool, b.cache.v_pool)


def test_store_q4_exact_scale_example(kvq):
    """Rotated-domain integers with amax 8 store scale 1.0 and codes equal to
    the integers (FreeToken test-fix commit, exact-scale example)."""
    import scipy.linalg
    H = scipy.linalg.hadamard(32) / np.sqrt(32.0)
    rng = np.random.default_rng(0)
    c = rng.integers(-8, 8, size=(64, 32))
    c[:, 0] = -8
    x = torch.from_numpy((c @ H.T).astype(np.float32)).reshape(64, 1, 32).repeat(1, 1, 2)
    cache = kvq.Q4Cache(4, 1, 64, 16)
    kvq.kvq_store(cache, x.cuda().contiguous(), x.cuda().contiguous(), torch.arange(64, dtype=torch.int64).cuda())
    rows = cache.k_pool.cpu().numpy().reshape(64, 36)
    assert np.all(rows[:, 32:36].copy().view(np.uint16) == 0x3C00)
    lo = (rows[:, :16].astype(np.int16) & 0xF)
    hi = (rows[:, :16].astype(np.int16) >> 4)
    codes = np.empty((64, 32), np.int16)
    codes[:, 0::2] = np.where(lo > 7, lo - 16, lo)
    codes[:, 1::2] = np.where(hi > 7, hi - 16, hi)
    assert np.array_equal(codes, c)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_store_fp8_bit_exact(kvq, dtype):
    _say(f"store_fp8 dtype={dtype}")
    g = torch.Generator().manual_seed(3)
    n_tok, pages, ps = 200, 16, 16
    x = (torch.randn((n_tok, 576), generator=g) * torch.exp(2 * torch.randn((n_tok, 1), generator=g)))
    x[3] = 0.0                     # inert
    x[4, 7] = float("nan")         # NaN element -> 0x00, ignored by amax
    x[5, 544] = float("inf")       # non-finite amax -> inert rope part
    x[6, :512] = 1e-39             # 448/amax overflows -> inert latent part
    x[7, 100] = 1e6                # one huge element: the scale follows it
    x = x.to(dtype)
    slots = torch.randperm(pages * ps, generator=g)[:n_tok].to(torch.int64)
    slots[::13] = -1
    cache = kvq.Fp8Cache(pages, 576, 64, ps)
    kvq.kvq_store(cache, x.cuda(), None, slots.cuda())
    cref = np.zeros((pages * ps, 576), np.uint8)
    sref = np.zeros((pages * ps, 2), np.float32)
    oracle.fp8_store(cref, sref, x.float().numpy(), slots.numpy(), 64)
    torch.cuda.synchronize()
    assert np.array_equal(cache.codes.cpu().numpy(), cref)
    assert np.array_equal(cache.scales.cpu().numpy().view(np.uint32), sref.view(np.uint32))


# ----------------------------------------------------------------- rotate

def test_rotate_q_matches_oracle_butterfly(kvq):
    """kvq_rotate_q is the fp32 butterfly: bit-identical to the oracle's, and
    within fp32 rounding of the exact fp64 rotation."""
    q = torch.randn((24, 256), generator=torch.Generator().manual_seed(1))
    got = kvq.kvq_rotate_q(q.cuda()).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), oracle.hadamard32_f32(q.numpy()).view(np.uint32))
    ref = oracle.rotate_f64(q.double().numpy())
    assert np.max(np.abs(got - ref)) < 1e-5
    qq = q.cuda().clone()
    kvq.kvq_rotate_q(qq, out=qq)            # in place
    assert np.array_equal(qq.cpu().numpy(), got)


@pytest.mark.parametrize("D,kdt,qdt", [(256, torch.float32, torch.float32), (256, torch.bfloat16, torch.float32),
                                        (128, torch.float16, torch.bfloat16), (64, torch.bfloat16, torch.float16)])
def test_store_rotate_q_one_launch(kvq, D, kdt, qdt):
    """kvq_store_rotate_q stores the same bytes as the oracle's store and
    rotates q bit-identically to the oracle's butterfly; either part may be
    empty, and q may be rotated in place."""
    _say(f"store_rotate D={D} kv={kdt} q={qdt}")
    g = torch.Generator().manual_seed(D + 7)
    n_tok, H, ps, pages = 300, 3, 16, 40
    k = (torch.randn((n_tok, H, D), generator=g) * torch.exp(torch.randn((n_tok, H, 1), generator=g))).to(kdt)
    v = torch.randn((n_tok, H, D), generator=g).to(kdt)
    k[9] = 0.0
    slots = torch.randperm(pages * ps, generator=g)[:n_tok].to(torch.int64)
    slots[::13] = -1
    q = torch.randn((5, 24 // 5 + 1, D), generator=g).to(qdt)   # 25 rows: the last workgroup is ragged
    cache = kvq.Q4Cache(pages, H, D, ps)
    q_rot = kvq.kvq_store_rotate_q(cache, k.cuda(), v.cuda(), slots.cuda(), q.cuda())
    kref = np.zeros(cache.k_pool.shape, np.uint8)
    vref = np.zeros_like(kref)
    oracle.q4_store(kref, vref, k.float().numpy(), v.float().numpy(), slots.numpy(), ps)
    qref = oracle.hadamard32_f32(q.float().numpy().reshape(-1, D)).reshape(q.shape)
    torch.cuda.synchronize()
    assert np.array_equal(cache.k_pool.cpu().numpy(), kref)
    assert np.array_equal(cache.v_pool.cpu().numpy(), vref)
    assert np.array_equal(q_rot.cpu().numpy().view(np.uint32), qref.view(np.uint32))
    # rotation only (no tokens), store only (no rows), and in place
    cache2 = kvq.Q4Cache(pages, H, D, ps)
    none = torch.empty((0,), dtype=torch.int64, device="cuda")
    kv0 = torch.empty((0, H, D), dtype=kdt, device="cuda")
    r2 = kvq.kvq_store_rotate_q(cache2, kv0, kv0, none, q.cuda())
    kvq.kvq_store_rotate_q(cache2, k.cuda(), v.cuda(), slots.cuda(), torch.empty((0, D), dtype=qdt, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(r2, q_rot)
    assert torch.equal(cache2.k_pool, cache.k_pool) and torch.equal(cache2.v_pool, cache.v_pool)
    if qdt == torch.float32:
        qq = q.cuda().clone()
        kvq.kvq_store_rotate_q(cache2, k.cuda(), v.cuda(), slots.cuda(), qq, out=qq)
        torch.cuda.synchronize()
        assert torch.equal(qq, q_rot)


@pytest.mark.parametrize("non_temporal", [True, False])
def test_stream_read_reads_every_word(kvq, non_temporal):
    """The read-ceiling measurement: its fold is the XOR of the final 16 KiB
    block, for a buffer shorter and one longer than the grid."""
    for blocks in (37, 2048 + 333):
        _say(f"stream_read nt={non_temporal} blocks={blocks}")
        x = torch.randint(0, 256, (blocks * 16384,), dtype=torch.uint8, generator=torch.Generator().manual_seed(5))
        tail = x.numpy()[(blocks - 1) * 16384:]
        want = np.bitwise_xor.reduce(tail.view(np.uint32))
        got = kvq.kvq_stream_read(x.cuda(), non_temporal=non_temporal)
        torch.cuda.synchronize()
        assert int(got.cpu().numpy().view(np.uint32)[0]) == int(want)


# ----------------------------------------------------------------- 4-bit decode

def _check_q4(case, split_keys, chunked_partials=False):
    o, lse = case.gpu_attention(split_keys)
    ro, rl = case.ref_attention()
    err = rel_err(o, ro)
    _say(f"  {case.w.name} lens={case.lens[:6]} split={split_keys} max_rel_err={err.max():.2e}")
    assert err.max() < TOL, err.max()
    for b, T in enumerate(case.lens):
        if T == 0:
            assert np.all(o[b] == 0) and np.all(np.isneginf(lse[b]))
        else:
            assert np.max(np.abs(lse[b] - rl[b])) < 1e-3 * max(1.0, np.abs(rl[b]).max())


def test_tiny_workload(kvq):
    """The tiny 4-bit workload in full: D=128, 4 query heads on 1 KV head, T=1024."""
    w = wl.TINY
    case = Q4Case(w, [w.seq_len])
    assert np.array_equal(case.cache.k_pool.cpu().numpy(), case.k_ref)
    assert np.array_equal(case.cache.v_pool.cpu().numpy(), case.v_ref)
    _check_q4(case, 512)
    _check_q4(case, 1024)


def test_tiny_partials_match_oracle_chunks(kvq):
    """The GPU partials at 512-key splits match the oracle's 512-key chunk
    partials.  A partial (m, z, acc) may use any reference m (the kernels
    move m lazily), so compare what does not depend on it: the chunk's
    log-sum-exp m + log z and its normalized context acc / z."""
    w = wl.TINY
    case = Q4Case(w, [w.seq_len])
    _, _, (pa, pm, pz) = case.gpu_attention(512, want_partials=True)
    _, _, (ra, rm, rz) = case.ref_attention(chunk=512, return_partials=True)
    assert np.max(np.abs((pm + np.log(pz)) - (rm + np.log(rz)))) < 1e-3
    na, nr = pa / pz[..., None], ra / rz[..., None]
    assert rel_err(na, nr).max() < TOL


@pytest.mark.parametrize("split_keys", [512, 1024, 2048, 8192])
def test_gqa_several_splits_and_tail(kvq, split_keys):
    """Splits of 512 and 1024 keys run on the wave-pair kernel, 2048 and 8192
    on the single-wave one (four waves of 512 and 2048 keys)."""
    w = wl.shrink(wl.GQA_32K, n_layers=1, seq_len=5000)
    case = Q4Case(w, [5000])
    assert np.array_equal(case.cache.k_pool.cpu().numpy(), case.k_ref)
    _check_q4(case, split_keys)


def test_planted_key_recalled(kvq):
    """The planted key (K = the group's first query) dominates its heads."""
    w = wl.shrink(wl.GQA_262K, n_layers=1, seq_len=6000, plant_at=3000)
    case = Q4Case(w, [6000])
    o, _ = case.gpu_attention(2048)
    ro, _ = case.ref_attention()
    assert rel_err(o, ro).max() < TOL
    # the output of each group's first head is close to the planted value
    vrow = case.v_ref[3000 // 16, :, 3000 % 16]
    v_planted = oracle.rotate_f64(oracle.q4_decode_rows(vrow, w.head_dim))
    for g in range(w.n_kv_heads):
        h = g * w.group
        assert np.linalg.norm(o[0, h] - v_planted[g]) < 0.25 * np.linalg.norm(v_planted[g])


def test_ragged_batch_paged(kvq):
    """Ragged lengths (incl. 0, 1, page and split edges) over a shuffled page table."""
    w = wl.shrink(wl.RAGGED, prefill_chunk=0)
    lens = [0, 1, 16, 17, 511, 512, 513, 2047, 2048, 2049, 4100, 777]
    case = Q4Case(w, lens)
    assert np.array_equal(case.cache.k_pool.cpu().numpy(), case.k_ref)
    _check_q4(case, 512)
    _check_q4(case, 2048)


def test_rows_past_the_end_are_ignored(kvq):
    """Pool bytes past a sequence's last position -- here 0xFF, whose fp16
    scale is a NaN -- never reach the output, also inside a partial 16-row
    run and a partial tile."""
    w = wl.shrink(wl.RAGGED, prefill_chunk=0)
    lens = [1000, 17, 2049, 530]
    case = Q4Case(w, lens, fill=0xFF)
    for split in (512, 2048):
        o, lse = case.gpu_attention(split)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
        ro, rl = case.ref_attention()
        err = rel_err(o, ro)
        _say(f"  split={split} max_rel_err={err.max():.2e}")
        assert err.max() < TOL


def test_batch_invariance(kvq):
    """A sequence's output does not depend on the batch around it: solo and
    batched runs are bit-identical (TensorFold "What it is": concurrent
    replies equal solo runs)."""
    w = wl.shrink(wl.RAGGED, prefill_chunk=0)
    lens = [3000, 700, 4500]
    batch = Q4Case(w, lens, build_oracle=False)
    ob, lb = batch.gpu_attention(1024)
    import fp8_quantized_kv_amd as kvq_mod
    for b, T in enumerate(lens):
        pt = batch.page_table[b:b + 1].contiguous()
        sl = batch.seq_lens[b:b + 1].contiguous()
        q_rot = kvq_mod.kvq_rotate_q(batch.q[b:b + 1].contiguous())
        # solo run with a larger max_seq_len than needed: still identical
        for max_len in (T, max(lens)):
            pa, pm, pz = kvq_mod.kvq_decode_attn(batch.cache, q_rot, pt, sl, max_len, w.sm_scale, 1024)
            o, l = kvq_mod.kvq_merge(batch.cache, pa, pm, pz, sl, max_len, 1024)
            assert np.array_equal(o.cpu().numpy()[0], ob[b]) and np.array_equal(l.cpu().numpy()[0], lb[b])


@pytest.mark.parametrize("split_keys", [512, 2048])
def test_drafted_rows_equal_serial(kvq, split_keys):
    """Drafted output equals serial output (TensorFold issue "qwen27 CUDA: an
    opt-in 4-bit attention cache", section "What it is", contracts).  Three
    drafted tokens after a 2900-token prefix: the three rows decoded in one
    call (one batch entry per row on the same page table, lengths L+1..L+3,
    after storing the three tokens) equal, bit for bit, the rows decoded one
    after another at those lengths.  512-key splits run the wave-pair kernel,
    2048-key splits the single-wave one."""
    import fp8_quantized_kv_amd as kvq_mod
    w = wl.shrink(wl.RAGGED, prefill_chunk=0)
    L, R = 2900, 3
    case = Q4Case(w, [L + R], build_oracle=False)  # prefix and drafted tokens stored
    gen = torch.Generator(device="cuda").manual_seed(21)
    q = torch.randn((R, w.n_q_heads, w.head_dim), generator=gen, device="cuda")
    q_rot = kvq_mod.kvq_rotate_q(q)
    lens = torch.arange(L + 1, L + R + 1, dtype=torch.int32, device="cuda")
    pt = case.page_table.expand(R, -1).contiguous()
    pa, pm, pz = kvq_mod.kvq_decode_attn(case.cache, q_rot, pt, lens, L + R, w.sm_scale, split_keys)
    o_draft, l_draft = kvq_mod.kvq_merge(case.cache, pa, pm, pz, lens, L + R, split_keys)
    for r in range(R):
        sl = lens[r:r + 1].contiguous()
        pa, pm, pz = kvq_mod.kvq_decode_attn(case.cache, q_rot[r:r + 1].contiguous(), case.page_table, sl, L + r + 1,
                                             w.sm_scale, split_keys)
        o, lse = kvq_mod.kvq_merge(case.cache, pa, pm, pz, sl, L + r + 1, split_keys)
        assert torch.equal(o[0], o_draft[r]) and torch.equal(lse[0], l_draft[r]), f"row {r}"


def test_mha_and_large_group(kvq):
    """Group sizes 1 (plain multi-head) and 16 (the largest the kernels take)."""
    for hq, hkv in ((3, 3), (16, 1)):
        w = wl.shrink(wl.GQA_32K, n_layers=1, seq_len=1500, n_q_heads=hq, n_kv_heads=hkv, heavy_channels=8)
        _check_q4(Q4Case(w, [1500]), 512)


@pytest.mark.parametrize("D,page_size,hq,hkv", [(512, 16, 8, 2), (256, 8, 12, 2), (64, 16, 4, 4), (128, 32, 10, 1),
                                                 (256, 64, 32, 4)])
def test_other_shapes(kvq, D, page_size, hq, hkv):
    """Head sizes and page sizes on both kernel paths (the matrix-core kernel
    takes head_dim 128/256 with pages of a multiple of 16 tokens; the others
    run on the plain kernel)."""
    w = wl.shrink(wl.RAGGED, prefill_chunk=0, head_dim=D, page_size=page_size, n_q_heads=hq, n_kv_heads=hkv,
                  heavy_channels=D // 16)
    _check_q4(Q4Case(w, [1300, 2600, 40]), 1024)


@pytest.mark.parametrize("hq,hkv,page_size,split", [(4, 4, 16, 512), (8, 4, 32, 512), (16, 4, 64, 1024),
                                                     (8, 1, 16, 1024)])
def test_pair_kernel_edges(kvq, hq, hkv, page_size, split):
    """The wave-pair kernel (head_dim 256, groups of up to 8 heads, splits of
    up to 1024 keys): group sizes 1, 2, 4 and 8 and lengths around its tile
    (32 keys) and pair-quarter (split / 4 keys) boundaries, where the pairs
    of a workgroup run different numbers of tiles and idle pairs only join
    the barriers."""
    w = wl.shrink(wl.RAGGED, prefill_chunk=0, n_q_heads=hq, n_kv_heads=hkv, page_size=page_size)
    q = split // 4
    lens = [1, 31, 32, 33, q - 1, q, q + 1, 2 * q + 17, 3 * q + 31, split - 1, split, split + 1, 2 * split + q + 5]
    _check_q4(Q4Case(w, lens), split)


def test_pool_beyond_4gib(kvq):
    """Byte offsets above 2^32: a sequence whose pages sit at the far end of
    a pool of more than 4 GiB per K and V (the oracle sees the same rows in a
    compact pool through its own page table)."""
    w = wl.shrink(wl.GQA_32K, n_layers=1, seq_len=3000)
    T, ps = w.seq_len, w.page_size
    page_bytes = w.n_kv_heads * ps * w.row_bytes
    n_far = (1 << 32) // page_bytes + 64            # pages past the 4 GiB mark
    n_used = -(-T // ps)
    num_pages = n_far + n_used
    _say(f"pool of {num_pages} pages = {num_pages * page_bytes / 2**30:.2f} GiB per K and V")
    cache = kvq.Q4Cache(num_pages, w.n_kv_heads, w.head_dim, ps, "cuda")
    pt_far = torch.arange(n_far, n_far + n_used, dtype=torch.int32).flip(0).unsqueeze(0)  # reversed order
    k, v = wl.q4_kv_tokens(w, 0, 0, T, "cuda")
    q = wl.q4_query(w, 0, "cuda")
    slots = wl.slots_for(pt_far[0], np.arange(T), ps)
    kvq.kvq_store(cache, k, v, slots.cuda())
    pt_d, sl = pt_far.cuda(), torch.tensor([T], dtype=torch.int32, device="cuda")
    q_rot = kvq.kvq_rotate_q(q)
    pa, pm, pz = kvq.kvq_decode_attn(cache, q_rot, pt_d, sl, T, w.sm_scale, 512)
    o, _ = kvq.kvq_merge(cache, pa, pm, pz, sl, T, 512)
    torch.cuda.synchronize()
    # the same rows in a compact pool for the oracle
    pt_c = torch.arange(n_used, dtype=torch.int32).unsqueeze(0)
    shape = oracle.q4_pool_shape(n_used, w.n_kv_heads, ps, w.head_dim)
    kref, vref = np.zeros(shape, np.uint8), np.zeros(shape, np.uint8)
    oracle.q4_store(kref, vref, k.float().cpu().numpy(), v.float().cpu().numpy(),
                    wl.slots_for(pt_c[0], np.arange(T), ps).numpy(), ps)
    far = pt_far[0].to(torch.int64).cuda()
    assert np.array_equal(cache.k_pool[far].cpu().numpy(), kref)
    assert np.array_equal(cache.v_pool[far].cpu().numpy(), vref)
    ro, _ = oracle.q4_attention(kref, vref, q.cpu().numpy(), pt_c.numpy(), np.array([T], np.int32), w.sm_scale)
    err = rel_err(o.cpu().numpy(), ro)
    _say(f"  max_rel_err={err.max():.2e}")
    assert err.max() < TOL
    del cache
    torch.cuda.empty_cache()


def test_empty_splits_are_written_empty(kvq):
    w = wl.shrink(wl.RAGGED, prefill_chunk=0)
    case = Q4Case(w, [600, 3000], build_oracle=False)
    import fp8_quantized_kv_amd as kvq_mod
    q_rot = kvq_mod.kvq_rotate_q(case.q)
    pa, pm, pz = kvq_mod.kvq_decode_attn(case.cache, q_rot, case.page_table, case.seq_lens, 3000, w.sm_scale, 512)
    pa, pm, pz = pa.cpu(), pm.cpu(), pz.cpu()
    assert torch.all(pz[0, :, 2:] == 0) and torch.all(torch.isneginf(pm[0, :, 2:])) and torch.all(pa[0, :, 2:] == 0)
    assert torch.all(pz[0, :, :2] >= 1) and torch.all(pz[1] >= 1)


# ----------------------------------------------------------------- fp8 latent decode

def test_mla_small(kvq):
    w = wl.shrink(wl.MLA_262K, n_heads=20, seq_len=0)
    lens = [3000, 1, 0, 1025]
    case = MlaCase(w, lens)
    assert np.array_equal(case.cache.codes.cpu().numpy(), case.codes_ref)
    for split in (1024, 2048):
        o, lse = case.gpu_attention(split)
        ro, rl = case.ref_attention()
        err = rel_err(o, ro)
        _say(f"  mla lens={lens} split={split} max_rel_err={err.max():.2e}")
        assert err.max() < TOL
        fin = np.isfinite(rl)
        assert np.array_equal(fin, np.isfinite(lse)) and np.max(np.abs(lse[fin] - rl[fin])) < 1e-3
        assert np.all(o[2] == 0)


@pytest.mark.parametrize("n_heads", [16, 40, 128])
def test_mla_heads_splits_and_tails(kvq, n_heads):
    """Head counts that fill a 64-head workgroup partly or fully, splits of
    512-4096 keys (the last on the plain kernel), lengths with partial 16-row
    runs and tiles, and pool bytes past each sequence's end set to 0xFF (NaN
    codes and NaN scales) that must never reach the output."""
    w = wl.shrink(wl.MLA_262K, n_heads=n_heads, seq_len=0)
    lens = [17, 2100, 33, 1000]
    case = MlaCase(w, lens, fill=0xFF)
    ro, rl = case.ref_attention()
    for split in (512, 1024, 2048, 4096):
        o, lse = case.gpu_attention(split)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
        err = rel_err(o, ro)
        _say(f"  mla heads={n_heads} split={split} max_rel_err={err.max():.2e}")
        assert err.max() < TOL
        assert np.max(np.abs(lse - rl)) < 1e-3 * max(1.0, np.abs(rl).max())


def test_mla_batch_invariance(kvq):
    """An fp8-latent sequence's output is bit-identical alone and in a batch."""
    w = wl.shrink(wl.MLA_262K, n_heads=64, seq_len=0)
    lens = [1500, 300, 2500]
    batch = MlaCase(w, lens, build_oracle=False)
    ob, lb = batch.gpu_attention(1024)
    import fp8_quantized_kv_amd as kvq_mod
    for b, T in enumerate(lens):
        pt = batch.page_table[b:b + 1].contiguous()
        sl = batch.seq_lens[b:b + 1].contiguous()
        q = batch.q[b:b + 1].contiguous()
        pa, pm, pz = kvq_mod.kvq_decode_attn(batch.cache, q, pt, sl, max(lens), w.sm_scale, 1024)
        o, l = kvq_mod.kvq_merge(batch.cache, pa, pm, pz, sl, max(lens), 1024)
        assert np.array_equal(o.cpu().numpy()[0], ob[b]) and np.array_equal(l.cpu().numpy()[0], lb[b])


@pytest.mark.parametrize("fmt", ["q4", "fp8"])
def test_merge_few_splits_equals_merge_many(kvq, fmt):
    """Partials of at most 64 splits over at least 256 (row, channel block)
    items are merged one wave per item; the result is bit-identical to the
    four-wave merge that larger split counts use.  The same partials are
    merged once from a buffer of 100 splits per row (four-wave merge, only
    the used splits are read) and once from a copy holding the first 64
    (one-wave merge)."""
    import fp8_quantized_kv_amd as kvq_mod
    split = 512
    if fmt == "q4":
        w = wl.shrink(wl.RAGGED, prefill_chunk=0)
        lens = [31000, 700, 32768, 1]  # 4 x 24 heads x 4 blocks = 384 items
        case = Q4Case(w, lens, build_oracle=False)
        q = kvq_mod.kvq_rotate_q(case.q)
    else:
        w = wl.shrink(wl.MLA_262K, n_heads=40, seq_len=0)
        lens = [30000, 513, 0]  # 3 x 40 heads x 8 blocks = 960 items
        case = MlaCase(w, lens, build_oracle=False)
        q = case.q
    big = 100 * split
    pt = torch.zeros((len(lens), big // w.page_size), dtype=torch.int32, device="cuda")  # room for 100 splits
    pt[:, :case.page_table.shape[1]] = case.page_table
    pa, pm, pz = kvq_mod.kvq_decode_attn(case.cache, q, pt, case.seq_lens, big, w.sm_scale, split)
    o1, l1 = kvq_mod.kvq_merge(case.cache, pa, pm, pz, case.seq_lens, big, split)
    pa2, pm2, pz2 = (x[:, :, :64].contiguous() for x in (pa, pm, pz))
    o2, l2 = kvq_mod.kvq_merge(case.cache, pa2, pm2, pz2, case.seq_lens, 64 * split, split)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ------------------------------------------------- fp8 latent, selected rows (DSA gather)

@pytest.mark.parametrize("n_heads,n_sel,max_sel,split", [(128, [1000, 300, 0], 1024, 512), (40, [2049, 4096, 17], 4096, 2048),
                                                         (16, [4096, 1536], 4096, 1024), (64, [100], 512, 512),
                                                         (128, [2048, 33], 2048, 128), (24, [4096, 95], 4096, 32)])
def test_mla_sel_matches_oracle(kvq, n_heads, n_sel, max_sel, split):
    """Selected rows of a paged cache whose bytes past each sequence are 0xFF
    (NaN codes and scales): seeded distinct positions in random order, padded
    with -1, plus absent and repeated entries written into the lists."""
    w = wl.shrink(wl.MLA_262K, n_heads=n_heads, seq_len=0)
    lens = [6000, 4200, 5000][:len(n_sel)]
    case = MlaCase(w, lens, fill=0xFF)
    sel, ns = wl.dsa_selection(w, lens, n_sel, max_sel)
    cap = case.page_table.shape[1] * w.page_size
    if n_sel[0] > 40:
        sel[0, 3], sel[0, 20] = -1, cap + 7     # absent entries inside the list
        sel[0, 30] = sel[0, 31]                 # a repeat
    _say(f"mla_sel heads={n_heads} n_sel={n_sel} max_sel={max_sel} split={split}")
    o, lse = case.gpu_attention_sel(sel, ns, split)
    ro, rl = case.ref_attention_sel(sel, ns)
    assert np.all(np.isfinite(o))
    err = rel_err(o, ro)
    _say(f"  max_rel_err={err.max():.2e}")
    assert err.max() < TOL
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(lse)) and np.max(np.abs(lse[fin] - rl[fin])) < 1e-3 * max(1.0, np.abs(rl[fin]).max())
    for b, n in enumerate(n_sel):
        if n == 0:
            assert np.all(o[b] == 0) and np.all(np.isneginf(lse[b]))


@pytest.mark.parametrize("split", [64, 512, 1024])
def test_mla_sel_absent_tiles_splits_and_rows(kvq, split):
    """Fixed-size lists (n_sel = max_sel) whose -1 padding covers whole key
    tiles and whole splits, including the first tile of a split, and one
    sequence whose list is absent throughout: outputs match the oracle, stay
    finite, an all-absent row gives out = 0 and lse = -inf, and every split
    without a present entry is an empty partial (m = -inf, z = 0, acc = 0)."""
    import fp8_quantized_kv_amd as kvq_mod
    w = wl.shrink(wl.MLA_262K, n_heads=32, seq_len=0)
    lens = [5000, 3000, 4000]
    case = MlaCase(w, lens, fill=0xFF)
    max_sel = 2048
    sel, ns = wl.dsa_selection(w, lens, [max_sel, max_sel, 100], max_sel)
    sel[0, 0:32] = -1            # the first tile of split 0
    sel[0, 512:1024] = -1        # whole splits at 64 and 512, half of one at 1024
    sel[0, 1056:1100] = -1       # a tile and a half inside a split
    sel[1, :] = -1               # every entry absent
    sel[2, 100:] = -1            # the list's -1 padding, counted in n_sel
    ns[:] = max_sel
    _say(f"mla_sel_absent split={split}")
    pa, pm, pz = kvq_mod.kvq_decode_attn_sel(case.cache, case.q, case.page_table, sel.cuda(), ns.cuda(),
                                             w.sm_scale, split)
    o, lse = kvq_mod.kvq_merge(case.cache, pa, pm, pz, ns.cuda(), max_sel, split)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    pa, pm, pz = pa.cpu().numpy(), pm.cpu().numpy(), pz.cpu().numpy()
    assert np.all(np.isfinite(pa)) and np.all(np.isfinite(pz)) and not np.any(np.isnan(pm))
    present = (sel.numpy() >= 0).reshape(3, -1, split).any(axis=2)  # [B][S]
    for b in range(3):
        for s_ in range(present.shape[1]):
            if not present[b, s_]:
                assert np.all(pz[b, :, s_] == 0) and np.all(np.isneginf(pm[b, :, s_])) and np.all(pa[b, :, s_] == 0)
    assert np.all(np.isfinite(o))
    assert np.all(o[1] == 0) and np.all(np.isneginf(lse[1]))
    ro, rl = case.ref_attention_sel(sel, ns)
    err = rel_err(o, ro)
    _say(f"  max_rel_err={err.max():.2e}")
    assert err.max() < TOL
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - rl[fin])) < 1e-3 * max(1.0, np.abs(rl[fin]).max())


def test_mla_sel_every_position_equals_dense(kvq):
    """Selecting positions 0..T-1 in order reproduces the dense decode's
    partials bit for bit: the staged tiles are the same bytes."""
    import fp8_quantized_kv_amd as kvq_mod
    w = wl.shrink(wl.MLA_262K, n_heads=128, seq_len=0)
    lens = [3000, 1234]
    case = MlaCase(w, lens, build_oracle=False)
    T = max(lens)
    sel = torch.full((2, T), -1, dtype=torch.int32)
    for b, n in enumerate(lens):
        sel[b, :n] = torch.arange(n, dtype=torch.int32)
    ns = torch.tensor(lens, dtype=torch.int32)
    for split in (512, 2048):
        d = kvq_mod.kvq_decode_attn(case.cache, case.q, case.page_table, case.seq_lens, T, w.sm_scale, split)
        s_ = kvq_mod.kvq_decode_attn_sel(case.cache, case.q, case.page_table, sel.cuda(), ns.cuda(), w.sm_scale, split)
        torch.cuda.synchronize()
        for x, y in zip(d, s_):
            assert torch.equal(x, y)


def test_mla_sel_batch_invariance(kvq):
    """A sequence's selection gives bit-identical output alone and in a batch."""
    import fp8_quantized_kv_amd as kvq_mod
    w = wl.shrink(wl.MLA_262K, n_heads=64, seq_len=0)
    lens = [5000, 3000, 4000]
    case = MlaCase(w, lens, build_oracle=False)
    sel, ns = wl.dsa_selection(w, lens, [2048, 700, 1500], 2048)
    ob, lb = case.gpu_attention_sel(sel, ns, 1024)
    for b in range(3):
        pa, pm, pz = kvq_mod.kvq_decode_attn_sel(case.cache, case.q[b:b + 1].contiguous(),
                                                 case.page_table[b:b + 1].contiguous(), sel[b:b + 1].cuda(),
                                                 ns[b:b + 1].cuda(), w.sm_scale, 1024)
        o, l = kvq_mod.kvq_merge(case.cache, pa, pm, pz, ns[b:b + 1].cuda(), 2048, 1024)
        assert np.array_equal(o.cpu().numpy()[0], ob[b]) and np.array_equal(l.cpu().numpy()[0], lb[b])


def test_mla_nan_codes_read_zero(kvq):
    """Codes 0x7F/0xFF (e4m3 NaN) in a cache read as 0 (colibri correctness
    commit: the CPU table reads 0 for NaN codes)."""
    w = wl.shrink(wl.MLA_262K, n_heads=16, seq_len=0)
    case = MlaCase(w, [700])
    case.cache.codes[5, 10] = 0x7F
    case.cache.codes[9, 537] = 0xFF
    case.codes_ref[5, 10] = 0x7F
    case.codes_ref[9, 537] = 0xFF
    o, _ = case.gpu_attention(1024)
    ro, _ = case.ref_attention()
    assert rel_err(o, ro).max() < TOL
    assert np.all(np.isfinite(o))
