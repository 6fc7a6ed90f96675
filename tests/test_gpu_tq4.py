"""GPU parity of the rotated-int4 + Lloyd-Max latent codec (TQ4; colibri
pull request "KV cache quantization: fp8 (KV8) + 4-bit TurboQuant (KV_TQ)",
Summary "Why rotated-int4 for the 4-bit tier") against the oracle: stored
codes and radii bit-exact, absorbed attention within 2e-3."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from helpers import TOL, TqCase, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvq():
    assert torch.cuda.is_available(), "no GPU"
    import fp8_quantized_kv_amd as m
    return m


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_tq4_store_bit_exact(kvq, dtype):
    """Latent rows of the fp8 workload plus edge rows (zero, NaN, infinite,
    huge, tiny, a single spike): codes and radii equal the oracle's."""
    _say(f"tq4 store dtype={dtype}")
    w = wl.MLA_262K
    n = 300
    x = wl.mla_rows(w, 0, 0, n, "cuda").to(dtype)
    x[3] = 0
    x[4, 7] = float("nan")
    x[5, 600 % 576] = float("inf")
    x[6] *= 1e30 if dtype == torch.float32 else 1e20
    x[7] *= 1e-30 if dtype == torch.float32 else 1e-20
    x[8] = 0
    x[8, 511] = 3.0
    x[9, 512:] = 0
    cache = kvq.TqCache(n // 16 + 2, 16, "cuda")
    slots = torch.randperm(cache.codes.shape[0], generator=torch.Generator().manual_seed(1))[:n].to(torch.int64)
    slots[10] = -1  # skipped
    kvq.kvq_store(cache, x, None, slots.cuda())
    torch.cuda.synchronize()
    codes = np.zeros(tuple(cache.codes.shape), np.uint8)
    radii = np.zeros(tuple(cache.scales.shape), np.float32)
    oracle.tq_store(codes, radii, x.float().cpu().numpy(), slots.numpy())
    gc, gr = cache.codes.cpu().numpy(), cache.scales.cpu().numpy()
    bad = np.nonzero(np.any(gc != codes, axis=1) | np.any(gr.view(np.uint32) != radii.view(np.uint32), axis=1))[0]
    assert bad.size == 0, f"rows differ: {bad[:10]}"


def test_tq4_decode_matches_oracle(kvq):
    """Rotate + decode + merge over a ragged batch (one position, a tail, an
    empty sequence, several splits), 16 heads, splits of 512 and 2048 keys
    (matrix cores) and 4096 (beyond the matrix-core kernel's split limit: the
    plain kernel); a sequence alone equals the same sequence in the batch,
    bit for bit."""
    w = wl.MLA_262K
    lens = [1, 300, 0, 1100]
    case = TqCase(w, lens, n_heads=16)
    assert np.array_equal(case.cache.codes.cpu().numpy(), case.codes_ref)
    ro, rl = case.ref_attention()
    for split in (512, 2048, 4096):
        o, lse = case.gpu_attention(split)
        err = rel_err(o, ro)
        _say(f"  split={split} max_rel_err={err.max():.2e}")
        assert err.max() < TOL
        fin = np.isfinite(rl)
        assert np.array_equal(fin, np.isfinite(lse)) and np.max(np.abs(lse[fin] - rl[fin])) < 1e-3 * max(1.0, np.abs(rl[fin]).max())
        assert np.all(o[2] == 0)
    o_b, l_b = case.gpu_attention(512)
    for b in (1, 3):
        q1 = kvq.kvq_tq_rotate_q(case.q[b:b + 1].contiguous())
        pa, pm, pz = kvq.kvq_decode_attn(case.cache, q1, case.page_table[b:b + 1].contiguous(),
                                         case.seq_lens[b:b + 1].contiguous(), case.max_seq_len, w.sm_scale, 512)
        o1, l1 = kvq.kvq_merge(case.cache, pa, pm, pz, case.seq_lens[b:b + 1].contiguous(), case.max_seq_len, 512)
        assert np.array_equal(o1.cpu().numpy()[0], o_b[b]) and np.array_equal(l1.cpu().numpy()[0], l_b[b])


def test_tq4_decode_all_heads(kvq):
    """All 128 heads of the workload (eight head blocks) over one sequence."""
    w = wl.MLA_262K
    case = TqCase(w, [700])
    ro, rl = case.ref_attention()
    o, lse = case.gpu_attention(512)
    err = rel_err(o, ro)
    _say(f"  128 heads max_rel_err={err.max():.2e}")
    assert err.max() < TOL


def test_tq_rotate_q_bit_exact(kvq):
    """kvq_tq_rotate_q equals the oracle's fp32 rotation of each part, bit for
    bit (same butterfly order, same final multiply), also in place."""
    g = torch.Generator().manual_seed(21)
    q = torch.randn((3, 5, 576), generator=g)
    q[0, 0] = 0
    q[1, 2, 100] = 1e30
    q[2, 4, 513] = -7.5e-39
    ref = np.empty((3, 5, 576), np.float32)
    qn = q.numpy()
    for b in range(3):
        for h in range(5):
            ref[b, h, :512] = oracle.tq_rotate_f32(qn[b, h, :512], 0)
            ref[b, h, 512:] = oracle.tq_rotate_f32(qn[b, h, 512:], 1)
    qd = q.cuda()
    out = kvq.kvq_tq_rotate_q(qd)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    kvq.kvq_tq_rotate_q(qd, out=qd)
    torch.cuda.synchronize()
    assert np.array_equal(qd.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_tq4_store_rotate_one_launch(kvq):
    """kvq_store_rotate_q on a TQ4 cache equals kvq_store + kvq_tq_rotate_q,
    bit for bit (codes, radii, rotated query), with rows only, tokens only,
    and both."""
    w = wl.MLA_262K
    n = 40
    x = wl.mla_rows(w, 0, 0, n, "cuda").to(torch.bfloat16)
    q = wl.mla_query(wl.shrink(w, batch=2), 0, "cuda")[:, :24].contiguous()
    slots = torch.randperm(n * 2, generator=torch.Generator().manual_seed(3))[:n].to(torch.int64).cuda()
    slots[5] = -1
    a, b = kvq.TqCache(5, 16, "cuda"), kvq.TqCache(5, 16, "cuda")
    kvq.kvq_store(a, x, None, slots)
    qa = kvq.kvq_tq_rotate_q(q)
    qb = kvq.kvq_store_rotate_q(b, x, None, slots, q)
    torch.cuda.synchronize()
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales.view(torch.int32), b.scales.view(torch.int32))
    assert torch.equal(qa.view(torch.int32), qb.view(torch.int32))
    c = kvq.TqCache(5, 16, "cuda")
    qc = kvq.kvq_store_rotate_q(c, x[:0], None, slots[:0], q)      # rows only
    kvq.kvq_store_rotate_q(c, x, None, slots, q[:0])               # tokens only
    torch.cuda.synchronize()
    assert torch.equal(qc.view(torch.int32), qa.view(torch.int32))
    assert torch.equal(c.codes, a.codes) and torch.equal(c.scales.view(torch.int32), a.scales.view(torch.int32))


def _unrotate_f32(y):
    """The codec's inverse rotation of 512-wide rows in fp32, stage by stage
    (colibri pull request, Summary "Why rotated-int4 for the 4-bit tier"):
    the Sylvester butterfly (a + b, a - b) for h = 1 .. 256, times
    fp32(1/sqrt(512)), times the part's signs.  numpy float32 rounds each
    step as the kernel does."""
    v = np.array(y, dtype=np.float32).reshape(-1, 512).copy()
    h = 1
    while h < 512:
        x = v.reshape(-1, 512 // (2 * h), 2, h)
        a, b = x[:, :, 0, :].copy(), x[:, :, 1, :].copy()
        x[:, :, 0, :] = a + b
        x[:, :, 1, :] = a - b
        v = x.reshape(-1, 512)
        h *= 2
    c = np.float32(1.0 / np.sqrt(512.0))
    return ((v * c) * oracle.tq_signs(0, 512)).astype(np.float32)


# (split, lens): 33000 positions at split 32 give 1032 splits (the merge's
# maximum past 1024, Z terms past 256, partial batches past 128 splits a
# lane); an empty sequence gives a zero context, rotated like any other.
@pytest.mark.parametrize("split,lens", [(2048, [3000, 0, 700, 33]), (32, [33000, 9000, 1])])
def test_tq4_merge_rotates_back_in_one_launch(kvq, split, lens):
    """kvq_merge on a TQ4 cache (merge and inverse rotation in one launch)
    against the plain merge of the same partials (an FP8 cache descriptor,
    no rotation) followed by the inverse rotation in numpy fp32: out and lse
    bit for bit."""
    w = wl.shrink(wl.MLA_262K, n_heads=20, seq_len=0)
    t = TqCase(w, lens, build_oracle=False, n_heads=20)
    _say(f"tq4 merge split={split} lens={lens}")
    q_rot = kvq.kvq_tq_rotate_q(t.q)
    pa, pm, pz = kvq.kvq_decode_attn(t.cache, q_rot, t.page_table, t.seq_lens, t.max_seq_len, w.sm_scale, split)
    out, lse = kvq.kvq_merge(t.cache, pa, pm, pz, t.seq_lens, t.max_seq_len, split)
    plain = kvq.Fp8Cache(1, 576, 64, w.page_size, "cuda")  # the same merge without a rotation
    o_plain, l_plain = kvq.kvq_merge(plain, pa, pm, pz, t.seq_lens, t.max_seq_len, split)
    torch.cuda.synchronize()
    ref = _unrotate_f32(o_plain.cpu().numpy()).reshape(tuple(out.shape))
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    assert torch.equal(lse.view(torch.int32), l_plain.view(torch.int32))
