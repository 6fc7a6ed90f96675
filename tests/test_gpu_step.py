"""kvq_decode_step (the new token's store and the query rotation inside the
decode launch, then the merge) against kvq_store_rotate_q + kvq_attend, bit
for bit: the pools, the partials, out and lse; and the step's output against
the oracle after the oracle stores the same token.  Both 4-bit matrix-core
kernels and the 8- and 6-bit block formats, both places the store can take
(before the first copies when the new row's sub-tile is copied at once,
later otherwise), every input dtype, an empty sequence, a page outside the
pool, and the configurations the step does not carry.  The fp8 latent format
against kvq_store + kvq_attend the same way: the new row in the first tile,
the second or third (stored before the later copies), or later, with one
and two head blocks of 64 heads."""
import ctypes

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


def _new_token(case, kv_dtype, seed):
    """Token b's K and V rows [batch][H][D] (seeded, N(0,1)) in kv_dtype."""
    w = case.w
    g = torch.Generator(device="cpu").manual_seed(seed)
    shape = (len(case.lens), w.n_kv_heads, w.head_dim)
    k = torch.randn(shape, generator=g).to(kv_dtype).cuda()
    v = torch.randn(shape, generator=g).to(kv_dtype).cuda()
    return k, v


def _step_slots(case):
    """Slot of position T_b - 1 through the page table (-1 for T_b = 0 or a page outside the pool)."""
    pt = case.page_table.cpu().numpy()
    ps = case.w.page_size
    out = []
    for b, T in enumerate(case.lens):
        if T == 0:
            out.append(-1)
            continue
        page = int(pt[b, (T - 1) // ps])
        out.append(page * ps + (T - 1) % ps if 0 <= page < case.lay.num_pages else -1)
    return torch.tensor(out, dtype=torch.int64)


def _clone_cache(kvq, case):
    w = case.w
    fmt = {4: kvq.FMT_Q4_H32, 6: kvq.FMT_Q6_H32, 8: kvq.FMT_Q8_H32}[w.bits]
    c = kvq.Q4Cache(case.lay.num_pages, w.n_kv_heads, w.head_dim, w.page_size, "cuda", fmt=fmt)
    c.k_pool.copy_(case.cache.k_pool)
    c.v_pool.copy_(case.cache.v_pool)
    return c


def _partials(kvq, ws, case, split, Hq=None):
    """part_acc, part_m, part_z inside a workspace (the layout kvq.h states)."""
    B, Hq, D = len(case.lens), Hq or case.w.n_q_heads, case.cache.dv
    S = kvq.kvq_num_splits(case.max_seq_len, split)
    up = lambda x: (x + 255) // 256 * 256
    n = B * Hq * S
    m0 = up(n * D * 4)
    z0 = m0 + up(n * 4)
    f = ws.view(torch.uint8)
    return f[:n * D * 4], f[m0:m0 + n * 4], f[z0:z0 + n * 4]


def _both_paths(kvq, case, split, kv_dtype=torch.bfloat16, q_dtype=torch.float32, seed=7):
    k, v = _new_token(case, kv_dtype, seed)
    q = case.q.to(q_dtype).contiguous()
    B, Hq = len(case.lens), case.w.n_q_heads
    need = kvq.kvq_attend_workspace_bytes(case.cache, B, Hq, case.max_seq_len, split)
    cache_b = _clone_cache(kvq, case)
    # three launches: store + rotation, decode, merge
    slots = _step_slots(case)
    q_rot = kvq.kvq_store_rotate_q(case.cache, k, v, slots.cuda(), q)
    ws_a = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    o_a, l_a = kvq.kvq_attend(case.cache, q_rot, case.page_table, case.seq_lens, case.max_seq_len, case.w.sm_scale,
                              split, workspace=ws_a)
    # the step: two launches
    ws_b = torch.full((need,), 0x00, dtype=torch.uint8, device="cuda")
    o_b, l_b = kvq.kvq_decode_step(cache_b, k, v, q, case.page_table, case.seq_lens, case.max_seq_len,
                                   case.w.sm_scale, split, workspace=ws_b)
    torch.cuda.synchronize()
    assert torch.equal(case.cache.k_pool, cache_b.k_pool), "K pool differs"
    assert torch.equal(case.cache.v_pool, cache_b.v_pool), "V pool differs"
    for x, y, what in zip(_partials(kvq, ws_a, case, split), _partials(kvq, ws_b, case, split), ("acc", "m", "z")):
        assert torch.equal(x, y), f"partials {what} differ"
    assert torch.equal(o_a, o_b) and torch.equal(l_a, l_b)
    return k, v, slots, o_b, l_b


# (split, lens): split 512 runs on the wave-pair kernel; T = 3000 puts the new
# row in the second sub-tile of a pair's range (stored after the first
# copies), T = 5000 in the first (stored before them, then a barrier), T = 0
# stores nothing.  Split 2048 runs on the single-wave kernel: T = 33000 (sub-
# tile 7 of wave 0's range), T = 1 and T = 4097 (sub-tile 0), T = 2048 (the
# last sub-tile of wave 3's range).
CASES = [(512, [3000, 0, 5000]), (2048, [33000, 1, 4097, 2048]), (1024, [700, 16385, 1024, 1])]


@pytest.mark.parametrize("split,lens", CASES)
def test_step_equals_store_rotate_then_attend(kvq, split, lens):
    w = wl.shrink(wl.GQA_32K, n_layers=1, batch=len(lens), seq_len=0)
    case = Q4Case(w, lens, build_oracle=False)
    _say(f"step split={split} lens={lens}")
    _both_paths(kvq, case, split)


@pytest.mark.parametrize("bits", [8, 6])
@pytest.mark.parametrize("split,lens", [(512, [3000, 0, 5000]), (2048, [33000, 1, 4097, 2048])])
def test_step_block_formats(kvq, bits, split, lens):
    """The 8- and 6-bit block formats (the single-wave kernel, 4 waves at every split)."""
    w = wl.shrink(wl.GQA_32K, n_layers=1, batch=len(lens), seq_len=0, bits=bits)
    case = Q4Case(w, lens, build_oracle=False)
    _say(f"step bits={bits} split={split} lens={lens}")
    _both_paths(kvq, case, split, seed=19)


@pytest.mark.parametrize("kv_dtype,q_dtype", [(torch.float32, torch.float32), (torch.float16, torch.bfloat16),
                                              (torch.bfloat16, torch.float16)])
def test_step_dtypes(kvq, kv_dtype, q_dtype):
    w = wl.shrink(wl.GQA_32K, n_layers=1, batch=2, seq_len=0)
    case = Q4Case(w, [2500, 9000], build_oracle=False)
    for split in (512, 2048):
        _say(f"step dtypes {kv_dtype} {q_dtype} split={split}")
        _both_paths(kvq, case, split, kv_dtype=kv_dtype, q_dtype=q_dtype, seed=11)


def test_step_page_outside_pool_is_not_stored(kvq):
    """The page of position T - 1 is -1 for one sequence: neither path stores
    that row (kvq_store skips the slot), and both read the same bytes."""
    w = wl.shrink(wl.GQA_32K, n_layers=1, batch=2, seq_len=0)
    case = Q4Case(w, [4000, 6000], build_oracle=False)
    pt = case.page_table.clone()
    pt[1, (6000 - 1) // w.page_size] = -1
    case.page_table = pt
    for split in (512, 2048):
        _say(f"step page outside the pool, split={split}")
        _both_paths(kvq, case, split, seed=13)


@pytest.mark.parametrize("split", [512, 2048])
def test_step_matches_oracle(kvq, split):
    """The step's out against the oracle's attention after the oracle stores
    the same token at the same slots (codes bit-exact, attention within the bar)."""
    w = wl.shrink(wl.GQA_32K, n_layers=1, batch=2, seq_len=0)
    case = Q4Case(w, [3000, 4100])
    _say(f"step vs oracle, split={split}")
    k, v, slots, out, lse = _both_paths(kvq, case, split, seed=17)
    oracle.q4_store(case.k_ref, case.v_ref, k.float().cpu().numpy(), v.float().cpu().numpy(), slots.numpy(),
                    w.page_size)
    assert np.array_equal(case.cache.k_pool.cpu().numpy(), case.k_ref)
    assert np.array_equal(case.cache.v_pool.cpu().numpy(), case.v_ref)
    ro, rl = case.ref_attention()
    err = rel_err(out.cpu().numpy(), ro)
    _say(f"  max rel err {err.max():.2e}")
    assert err.max() < TOL
    assert np.max(np.abs(lse.cpu().numpy() - rl)) < 1e-3 * max(1.0, np.abs(rl).max())


def test_step_unsupported_configurations(kvq):
    """Configurations without a step kernel are refused before any launch."""
    for w, lens in ((wl.shrink(wl.TINY, batch=1, seq_len=0), [1000]),  # head_dim 128
                    (wl.shrink(wl.GQA_32K, n_layers=1, batch=1, seq_len=0, n_q_heads=48), [1000])):  # 12 heads a group
        case = Q4Case(w, lens, build_oracle=False)
        k, v = _new_token(case, torch.bfloat16, 3)
        with pytest.raises(kvq.KvqError) as e:
            kvq.kvq_decode_step(case.cache, k, v, case.q, case.page_table, case.seq_lens, case.max_seq_len,
                                w.sm_scale, 512)
        assert e.value.status == kvq.KVQ_ERR_UNSUPPORTED


# ----------------------------------------------------------------- fp8 latent rows

def _both_paths_latent(kvq, case, split, kv_dtype=torch.bfloat16, seed=23):
    """kvq_store of the new rows + kvq_attend against kvq_decode_step, bit for bit."""
    w = case.w
    B, Hq = len(case.lens), w.n_heads
    g = torch.Generator(device="cpu").manual_seed(seed)
    k = torch.randn((B, w.head_dim), generator=g).to(kv_dtype).cuda()
    need = kvq.kvq_attend_workspace_bytes(case.cache, B, Hq, case.max_seq_len, split)
    cache_b = kvq.Fp8Cache(case.lay.num_pages, w.head_dim, w.rope_dim, w.page_size, "cuda")
    cache_b.codes.copy_(case.cache.codes)
    cache_b.scales.copy_(case.cache.scales)
    slots = _step_slots(case)
    kvq.kvq_store(case.cache, k, None, slots.cuda())
    ws_a = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    o_a, l_a = kvq.kvq_attend(case.cache, case.q, case.page_table, case.seq_lens, case.max_seq_len, w.sm_scale,
                              split, workspace=ws_a)
    ws_b = torch.full((need,), 0x00, dtype=torch.uint8, device="cuda")
    o_b, l_b = kvq.kvq_decode_step(cache_b, k, None, case.q, case.page_table, case.seq_lens, case.max_seq_len,
                                   w.sm_scale, split, workspace=ws_b)
    torch.cuda.synchronize()
    assert torch.equal(case.cache.codes, cache_b.codes), "codes differ"
    assert torch.equal(case.cache.scales, cache_b.scales), "scales differ"
    for x, y, what in zip(_partials(kvq, ws_a, case, split, Hq), _partials(kvq, ws_b, case, split, Hq),
                          ("acc", "m", "z")):
        assert torch.equal(x, y), f"partials {what} differ"
    assert torch.equal(o_a, o_b) and torch.equal(l_a, l_b)
    return k, slots, o_b, l_b


# (split, lens): 32-key tiles.  Split 2048: T = 2049 and T = 1 put the new
# row in tile 0 of its split, T = 2048 + 50 and T = 90 in tiles 1 and 2, T =
# 3000 in tile 29; split 512: T = 520 (tile 0), T = 1100 (tile 2), T = 700
# (tile 5); T = 0 stores nothing.
LATENT_CASES = [(2048, [2049, 1, 2098, 90, 3000]), (512, [520, 0, 1100, 700])]


@pytest.mark.parametrize("n_heads", [20, 128])
@pytest.mark.parametrize("split,lens", LATENT_CASES)
def test_step_latent_equals_store_then_attend(kvq, n_heads, split, lens):
    w = wl.shrink(wl.MLA_262K, n_heads=n_heads, seq_len=0)
    case = MlaCase(w, lens, build_oracle=False)
    _say(f"step latent heads={n_heads} split={split} lens={lens}")
    _both_paths_latent(kvq, case, split)


def test_step_latent_dtypes_and_page_outside_pool(kvq):
    w = wl.shrink(wl.MLA_262K, n_heads=64, seq_len=0)
    case = MlaCase(w, [1500, 2090], build_oracle=False)
    for kv_dtype in (torch.float32, torch.float16, torch.bfloat16):
        _say(f"step latent dtype {kv_dtype}")
        _both_paths_latent(kvq, case, 1024, kv_dtype=kv_dtype, seed=29)
    pt = case.page_table.clone()
    pt[1, (2090 - 1) // w.page_size] = -1
    case.page_table = pt
    _say("step latent, page outside the pool")
    _both_paths_latent(kvq, case, 1024, seed=31)


def test_step_latent_matches_oracle(kvq):
    """The step's out against the oracle's attention after the oracle stores
    the same rows at the same slots (codes and scales bit-exact)."""
    w = wl.shrink(wl.MLA_262K, n_heads=24, seq_len=0)
    case = MlaCase(w, [2100, 60])
    _say("step latent vs oracle")
    k, slots, out, lse = _both_paths_latent(kvq, case, 2048, kv_dtype=torch.float32, seed=37)
    oracle.fp8_store(case.codes_ref, case.scales_ref, k.cpu().numpy(), slots.numpy(), w.rope_dim)
    assert np.array_equal(case.cache.codes.cpu().numpy(), case.codes_ref)
    assert np.array_equal(case.cache.scales.cpu().numpy(), case.scales_ref)
    ro, rl = case.ref_attention()
    err = rel_err(out.cpu().numpy(), ro)
    _say(f"  max rel err {err.max():.2e}")
    assert err.max() < TOL
    assert np.max(np.abs(lse.cpu().numpy() - rl)) < 1e-3 * max(1.0, np.abs(rl).max())


def test_step_latent_argument_errors(kvq):
    """A v row or a non-f32 query is refused for the latent format; the TQ4 latent format has no step."""
    w = wl.shrink(wl.MLA_262K, n_heads=16, seq_len=0)
    case = MlaCase(w, [100], build_oracle=False)
    k = torch.zeros((1, w.head_dim), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((kvq.kvq_attend_workspace_bytes(case.cache, 1, 16, 100, 512),), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((1, 16, case.cache.dv), dtype=torch.float32, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    args = lambda v, qdt: (ctypes.byref(case.cache.desc), P(k), v, kvq.DT_BF16, P(case.q), qdt, 16,
                           P(case.page_table), int(case.page_table.shape[1]), P(case.seq_lens), 1, 100,
                           float(w.sm_scale), 512, P(ws), ws.numel(), P(out), None, None)
    assert kvq.lib.kvq_decode_step(*args(P(k), kvq.DT_F32)) == kvq.KVQ_ERR_INVALID_ARG
    assert kvq.lib.kvq_decode_step(*args(None, kvq.DT_BF16)) == kvq.KVQ_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        kvq.kvq_decode_step(case.cache, k, k, case.q, case.page_table, case.seq_lens, 100, w.sm_scale, 512)
    t = kvq.TqCache(case.lay.num_pages, w.page_size, "cuda")
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_step(t, k, None, case.q, case.page_table, case.seq_lens, 100, w.sm_scale, 512)
    assert e.value.status == kvq.KVQ_ERR_UNSUPPORTED
