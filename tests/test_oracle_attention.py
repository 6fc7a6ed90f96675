"""Pins for the oracle's attention: brute-force fp64 softmax attention written
with numpy/scipy primitives on small inputs, closed forms, and the
equivalence of the rotated-space formulation with plain attention over the
reconstructed (unrotated) cache.

Pages: TensorFold issue "qwen27 CUDA: an opt-in 4-bit attention cache"
("What it is": rotate the query once, attend in rotated space over 512-key
chunks plus each row's tail, merge in order, rotate the output back once);
colibri pull request "KV cache quantization: fp8 (KV8) + 4-bit TurboQuant"
(KV8 commit: absorbed attention, latent is key and value; split-T commit:
partials (cl[K], m, z) merged by log-sum-exp, checked against double
references).
"""
import numpy as np
import pytest
import scipy.linalg
import scipy.special
import torch

import oracle
import workloads as wl


def _h32():
    return scipy.linalg.hadamard(32).astype(np.float64) / np.sqrt(32.0)


def _rot(x):
    """Blockwise H32 along the last axis (scipy's matrix)."""
    H = _h32()
    s = x.shape
    return (x.reshape(-1, 32) @ H.T).reshape(s)


def _np_decode_q4(rows, D):
    """Dequantized rotated values of 4-bit rows, decoded with numpy alone:
    code bytes (element 2k low nibble, 2k+1 high, two's complement), then the
    D/32 fp16 scales widened by numpy; value = code * scale of its group."""
    rows = np.ascontiguousarray(rows, np.uint8)
    c = rows[..., :D // 2].astype(np.int16)
    codes = np.empty(rows.shape[:-1] + (D,), np.float64)
    codes[..., 0::2] = ((c & 0xF) ^ 8) - 8
    codes[..., 1::2] = ((c >> 4) ^ 8) - 8
    scales = rows[..., D // 2:].copy().view(np.float16).astype(np.float64)
    return codes * np.repeat(scales, 32, axis=-1)


def _build_q4(w, lens, seed=0, scale=None):
    """Oracle-built paged caches for a small workload (inputs from workloads)."""
    lay = wl.page_layout(w, lens)
    num_pages = lay.num_pages
    shape = oracle.q4_pool_shape(num_pages, w.n_kv_heads, w.page_size, w.head_dim)
    kp = np.zeros(shape, np.uint8)
    vp = np.zeros(shape, np.uint8)
    off = 0
    for b, T in enumerate(lens):
        if T == 0:
            continue
        k, v = wl.q4_kv_tokens(w, 0, off, T)
        off += T
        k, v = k.float().numpy(), v.float().numpy()
        if scale is not None:  # tiny rows: every group's scale a binary16 subnormal
            k, v = k * np.float32(scale), v * np.float32(scale)
        slots = wl.slots_for(lay.page_table[b], np.arange(T), w.page_size).numpy()
        oracle.q4_store(kp, vp, k, v, slots, w.page_size)
    q = wl.q4_query(w, 0).numpy()
    return kp, vp, q, lay.page_table.numpy(), np.array(lens, np.int32)


def _brute_q4(kp, vp, q, pt, lens, w):
    """numpy fp64: gather dequantized rows, softmax, weighted sum, rotate back."""
    B, Hq, D = q.shape
    G = Hq // w.n_kv_heads
    o = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        T = lens[b]
        if T == 0:
            continue
        j = np.arange(T)
        slots = pt[b, j // w.page_size].astype(np.int64) * w.page_size + j % w.page_size
        pages, offs = slots // w.page_size, slots % w.page_size
        for h in range(Hq):
            g = h // G
            K = _np_decode_q4(kp[pages, g, offs], D)
            V = _np_decode_q4(vp[pages, g, offs], D)
            s = w.sm_scale * (K @ _rot(q[b, h].astype(np.float64)))
            p = scipy.special.softmax(s)
            o[b, h] = _rot(p @ V)
            lse[b, h] = scipy.special.logsumexp(s)
    return o, lse


SMALL = wl.shrink(wl.GQA_32K, n_layers=1, batch=3, seq_len=0, len_range=(1, 700), shuffle_pages=True,
                  n_q_heads=6, n_kv_heads=2)


@pytest.mark.parametrize("lens", [[37], [512, 1, 700], [0, 16, 513], [1023]])
def test_q4_attention_matches_brute_force(lens):
    w = wl.shrink(SMALL, batch=len(lens))
    kp, vp, q, pt, sl = _build_q4(w, lens)
    o, lse = oracle.q4_attention(kp, vp, q, pt, sl, w.sm_scale)
    ob, lb = _brute_q4(kp, vp, q, pt, sl, w)
    assert np.max(np.abs(o - ob)) < 1e-12
    fin = np.isfinite(lb)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - lb[fin]), initial=0) < 1e-12
    for b, T in enumerate(lens):
        if T == 0:
            assert np.all(o[b] == 0)


def test_q4_attention_subnormal_scales_matches_brute_force():
    """Rows scaled by 2^-17 put every group's fp16 scale among the binary16
    subnormals (amax/8 < 2^-14); the oracle's attention over them equals the
    numpy brute force (whose scales come from numpy's float16 widening).
    The query is scaled up by 2^17 so the scores keep their spread."""
    lens = [300, 77]
    w = wl.shrink(SMALL, batch=len(lens))
    kp, vp, q, pt, sl = _build_q4(w, lens, scale=2.0 ** -17)
    scales = kp[..., w.head_dim // 2:].copy().view(np.float16)
    used = scales[scales != 0]
    assert used.size > 1000 and np.all(np.abs(used.astype(np.float32)) < 2.0 ** -14)
    q = (q * np.float32(2.0 ** 17)).astype(np.float32)
    o, lse = oracle.q4_attention(kp, vp, q, pt, sl, w.sm_scale)
    ob, lb = _brute_q4(kp, vp, q, pt, sl, w)
    den = np.abs(ob).max(axis=-1, keepdims=True)
    assert np.max(np.abs(o - ob) / den) < 1e-12
    assert np.max(np.abs(lse - lb)) < 1e-9


@pytest.mark.parametrize("P,C", [(300, 40), (0, 33), (1000, 1)])
def test_chunk_attention_matches_causal_brute_force(P, C):
    """A prompt chunk of C rows at positions P .. P + C - 1 (TensorFold "What
    it is": prompt chunks are packed, then attended over the decoded slots):
    numpy in matrix form -- all scores at once, the causal mask j > P + i set
    to -inf, a row softmax, the weighted sum, the inverse rotation -- against
    the oracle's chunk attention."""
    T = P + C
    w = wl.shrink(SMALL, batch=1)
    kp, vp, _, pt, _ = _build_q4(w, [T])
    g = np.random.default_rng(P + C)
    q = g.standard_normal((C, w.n_q_heads, w.head_dim)).astype(np.float32)
    lens = P + 1 + np.arange(C, dtype=np.int32)
    o, lse = oracle.q4_chunk_attention(kp, vp, q, pt[0], lens, w.sm_scale)
    j = np.arange(T)
    slots = pt[0, j // w.page_size].astype(np.int64) * w.page_size + j % w.page_size
    pages, offs = slots // w.page_size, slots % w.page_size
    mask = j[None, :] > (P + np.arange(C))[:, None]              # [C][T]
    for h in range(w.n_q_heads):
        g_kv = h // w.group
        K = _np_decode_q4(kp[pages, g_kv, offs], w.head_dim)     # [T][D], rotated space
        V = _np_decode_q4(vp[pages, g_kv, offs], w.head_dim)
        S = w.sm_scale * (_rot(q[:, h].astype(np.float64)) @ K.T)  # [C][T]
        S[mask] = -np.inf
        Pm = scipy.special.softmax(S, axis=1)
        ob = _rot(Pm @ V)
        lb = scipy.special.logsumexp(S, axis=1)
        assert np.max(np.abs(o[:, h] - ob)) < 1e-12 * max(1.0, np.abs(ob).max())
        assert np.max(np.abs(lse[:, h] - lb)) < 1e-12 * max(1.0, np.abs(lb).max())


def test_rotated_space_equals_original_space():
    """Attending with H q over rotated rows, then rotating back, equals plain
    attention of q over the reconstructed rows x = H y."""
    w = wl.shrink(SMALL, batch=1)
    kp, vp, q, pt, sl = _build_q4(w, [300])
    o, _ = oracle.q4_attention(kp, vp, q, pt, sl, w.sm_scale)
    T = 300
    j = np.arange(T)
    for h in range(w.n_q_heads):
        g = h // w.group
        K = _rot(oracle.q4_decode_rows(kp[pt[0, j // 16], g, j % 16], w.head_dim))
        V = _rot(oracle.q4_decode_rows(vp[pt[0, j // 16], g, j % 16], w.head_dim))
        p = scipy.special.softmax(w.sm_scale * (K @ q[0, h].astype(np.float64)))
        assert np.max(np.abs(o[0, h] - p @ V)) < 1e-12


@pytest.mark.parametrize("chunk", [16, 512, 2048])
def test_chunked_merge_equals_direct(chunk):
    """Chunk partials at absolute multiples of the chunk size, merged in order,
    reproduce the direct softmax (ragged tails, empty sequences, T < chunk)."""
    lens = [0, 1, 15, 16, 17, 511, 512, 513, 1100]
    w = wl.shrink(SMALL, batch=len(lens), len_range=(0, 0))
    kp, vp, q, pt, sl = _build_q4(w, lens)
    o, lse = oracle.q4_attention(kp, vp, q, pt, sl, w.sm_scale)
    oc, lc, (pa, pm, pz) = oracle.q4_attention(kp, vp, q, pt, sl, w.sm_scale, chunk=chunk, return_partials=True)
    assert np.max(np.abs(o - oc)) < 1e-12
    fin = np.isfinite(lse)
    assert np.array_equal(fin, np.isfinite(lc)) and np.max(np.abs(lse[fin] - lc[fin])) < 1e-12
    # chunks past each sequence's end are empty
    for b, T in enumerate(lens):
        used = -(-T // chunk)
        assert np.all(pz[b, :, used:] == 0) and np.all(np.isneginf(pm[b, :, used:]))
        assert np.all(pa[b, :, used:] == 0)
        assert np.all(pz[b, :, :used] >= 1.0)   # each chunk's max term contributes exp(0)


def test_single_chunk_partial_is_normalized_output():
    """T <= chunk: one partial whose acc/z, rotated back, is the output."""
    w = wl.shrink(SMALL, batch=1)
    kp, vp, q, pt, sl = _build_q4(w, [400])
    o, lse, (pa, pm, pz) = oracle.q4_attention(kp, vp, q, pt, sl, w.sm_scale, chunk=512, return_partials=True)
    assert pa.shape[2] == 1
    assert np.max(np.abs(_rot(pa[0, :, 0] / pz[0, :, 0:1]) - o[0])) < 1e-12
    assert np.max(np.abs(pm[0, :, 0] + np.log(pz[0, :, 0]) - lse[0])) < 1e-12


def test_equal_keys_give_mean_of_values():
    """All keys identical -> uniform weights -> output = mean of the values."""
    D, T = 64, 200
    x = np.random.default_rng(3).standard_normal((1, 1, D)).astype(np.float32)
    k = np.repeat(x, T, axis=0)
    v = np.random.default_rng(4).standard_normal((T, 1, D)).astype(np.float32)
    pages = -(-T // 16)
    kp = np.zeros(oracle.q4_pool_shape(pages, 1, 16, D), np.uint8)
    vp = np.zeros_like(kp)
    oracle.q4_store(kp, vp, k, v, np.arange(T), 16)
    q = np.random.default_rng(5).standard_normal((1, 3, D)).astype(np.float32)
    pt = np.arange(pages, dtype=np.int32)[None]
    o, _ = oracle.q4_attention(kp, vp, q, pt, np.array([T], np.int32), 0.3)
    vrec = _rot(oracle.q4_decode_rows(vp.reshape(-1, kp.shape[-1])[:T], D))
    for h in range(3):
        assert np.max(np.abs(o[0, h] - vrec.mean(0))) < 1e-12


def test_mha_when_heads_equal():
    """H_q = H_kv: every query head reads only its own KV head."""
    w = wl.shrink(SMALL, batch=1, n_q_heads=2, n_kv_heads=2)
    kp, vp, q, pt, sl = _build_q4(w, [200])
    o, _ = oracle.q4_attention(kp, vp, q, pt, sl, w.sm_scale)
    ob, _ = _brute_q4(kp, vp, q, pt, sl, w)
    assert np.max(np.abs(o - ob)) < 1e-12
    # swapping head 1's cache changes only head 1
    kp2 = kp.copy()
    kp2[:, 1] = np.random.default_rng(0).integers(0, 256, kp2[:, 1].shape, dtype=np.uint8) & 0x77
    o2, _ = oracle.q4_attention(kp2, vp, q, pt, sl, w.sm_scale)
    assert np.array_equal(o2[0, 0], o[0, 0]) and not np.allclose(o2[0, 1], o[0, 1])


def test_planted_needle():
    """A key equal to the query dominates the softmax (TensorFold's planted-code
    recall, scaled down): the weight of the planted position is the argmax and
    the output is close to that position's value."""
    w = wl.shrink(wl.GQA_262K, n_layers=1, seq_len=4096, plant_at=1000)
    T = w.seq_len
    k, v = wl.q4_kv_tokens(w, 0, 0, T)
    q = wl.q4_query(w, 0)
    assert wl.plant(w, k, q, 0)
    lay = wl.page_layout(w, [T])
    shape = oracle.q4_pool_shape(lay.num_pages, w.n_kv_heads, w.page_size, w.head_dim)
    kp, vp = np.zeros(shape, np.uint8), np.zeros(shape, np.uint8)
    oracle.q4_store(kp, vp, k.float().numpy(), v.float().numpy(), np.arange(T), w.page_size)
    o, _ = oracle.q4_attention(kp, vp, q.numpy(), lay.page_table.numpy(), np.array([T], np.int32), w.sm_scale)
    for g in range(w.n_kv_heads):
        h = g * w.group
        j = np.arange(T)
        K = oracle.q4_decode_rows(kp[j // 16, g, j % 16], w.head_dim)
        s = w.sm_scale * (K @ _rot(q[0, h].double().numpy()))
        p = scipy.special.softmax(s)
        assert np.argmax(p) == 1000 and p[1000] > 0.9
        vrec = _rot(oracle.q4_decode_rows(vp[1000 // 16, g, 1000 % 16], w.head_dim))
        assert np.linalg.norm(o[0, h] - vrec) < 0.2 * np.linalg.norm(vrec)


# ----------------------------------------------------------------- fp8 latent

def _build_mla(w, lens):
    lay = wl.page_layout(w, lens)
    n_slots = lay.num_pages * w.page_size
    codes = np.zeros((n_slots, w.head_dim), np.uint8)
    scales = np.zeros((n_slots, 2), np.float32)
    off = 0
    for b, T in enumerate(lens):
        x = wl.mla_rows(w, 0, off, T).numpy()
        off += T
        slots = wl.slots_for(lay.page_table[b], np.arange(T), w.page_size).numpy()
        oracle.fp8_store(codes, scales, x, slots, w.rope_dim)
    q = wl.mla_query(wl.shrink(w, batch=len(lens)), 0).numpy()
    return codes, scales, q, lay.page_table.numpy(), np.array(lens, np.int32)


MLA_SMALL = wl.shrink(wl.MLA_262K, n_heads=8, seq_len=0)


def test_mla_attention_matches_brute_force():
    w = MLA_SMALL
    lens = [300, 45]
    codes, scales, q, pt, sl = _build_mla(w, lens)
    o, lse = oracle.mla_attention(codes, scales, q, pt, sl, w.sm_scale, w.rope_dim, w.page_size)
    deq = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    L = w.kv_lora
    for b, T in enumerate(lens):
        j = np.arange(T)
        slots = pt[b, j // 16].astype(np.int64) * 16 + j % 16
        lat = deq[slots, :L] * scales[slots, 0:1]
        rope = deq[slots, L:] * scales[slots, 1:2]
        for h in range(w.n_heads):
            s = w.sm_scale * (lat @ q[b, h, :L].astype(np.float64) + rope @ q[b, h, L:].astype(np.float64))
            p = scipy.special.softmax(s)
            ref = p @ lat
            assert np.max(np.abs(o[b, h] - ref)) < 1e-12 * max(1.0, np.abs(ref).max())
            assert abs(lse[b, h] - scipy.special.logsumexp(s)) < 1e-12


def test_mla_chunked_equals_direct():
    w = MLA_SMALL
    lens = [1, 1024, 1500, 0]
    codes, scales, q, pt, sl = _build_mla(w, lens)
    o, lse = oracle.mla_attention(codes, scales, q, pt, sl, w.sm_scale, w.rope_dim, w.page_size)
    oc, lc = oracle.mla_attention(codes, scales, q, pt, sl, w.sm_scale, w.rope_dim, w.page_size, chunk=512)
    assert np.max(np.abs(o - oc)) < 1e-12
    fin = np.isfinite(lse)
    assert np.array_equal(fin, np.isfinite(lc)) and np.max(np.abs(lse[fin] - lc[fin])) < 1e-12
    assert np.all(o[3] == 0) and np.all(np.isneginf(lse[3]))


def test_mla_row_bytes_match_the_page():
    """584 bytes per position (colibri VRAM-budget commit: ~CTX*584 B/layer):
    576 e4m3 codes plus two f32 scales."""
    w = wl.MLA_262K
    assert w.head_dim + 2 * 4 == 584
    assert w.seq_len * 584 == 153092096


# ------------------------------------------------ fp8 latent, selected rows (DSA gather)

def _brute_mla_sel(codes, scales, q, pt, sel, n_sel, w):
    """numpy fp64 over an explicit key list: decoded rows gathered with torch's
    e4m3 decoder, softmax by scipy, entries outside the page capacity skipped."""
    deq = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    deq[np.isnan(deq)] = 0.0
    L = w.kv_lora
    cap = pt.shape[1] * w.page_size
    B, H, _ = q.shape
    o = np.zeros((B, H, L))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        pos = np.array([p for p in sel[b, :n_sel[b]] if 0 <= p < cap], np.int64)
        if pos.size == 0:
            continue
        slots = pt[b, pos // w.page_size].astype(np.int64) * w.page_size + pos % w.page_size
        lat = deq[slots, :L] * scales[slots, 0:1]
        rope = deq[slots, L:] * scales[slots, 1:2]
        for h in range(H):
            s = w.sm_scale * (lat @ q[b, h, :L].astype(np.float64) + rope @ q[b, h, L:].astype(np.float64))
            o[b, h] = scipy.special.softmax(s) @ lat
            lse[b, h] = scipy.special.logsumexp(s)
    return o, lse


def test_mla_sel_all_positions_equals_dense():
    """Selecting every position 0..T-1 in order is the dense attention, bit for bit."""
    w = MLA_SMALL
    lens = [700, 33]
    codes, scales, q, pt, sl = _build_mla(w, lens)
    o, lse = oracle.mla_attention(codes, scales, q, pt, sl, w.sm_scale, w.rope_dim, w.page_size)
    sel = np.full((2, 800), -1, np.int32)
    for b, T in enumerate(lens):
        sel[b, :T] = np.arange(T)
    os_, ls = oracle.mla_attention_sel(codes, scales, q, pt, sel, sl, w.sm_scale, w.rope_dim, w.page_size)
    assert np.array_equal(o, os_) and np.array_equal(lse, ls)


def test_mla_sel_matches_brute_force():
    """A shuffled selection with repeats, padding (-1) and out-of-capacity
    entries against the numpy brute force; an empty selection gives 0 / -inf."""
    w = MLA_SMALL
    lens = [900, 400, 50]
    codes, scales, q, pt, sl = _build_mla(w, lens)
    rng = np.random.default_rng(3)
    cap = pt.shape[1] * w.page_size
    sel = np.full((3, 300), -1, np.int32)
    sel[0, :250] = rng.integers(0, 900, 250)                 # repeats likely
    sel[0, 7], sel[0, 8] = cap, cap + 5                      # outside the capacity: absent
    sel[1, :300] = rng.permutation(400)[:300]
    n_sel = np.array([260, 300, 0], np.int32)                # entries 250..259 of row 0 are padding
    o, lse = oracle.mla_attention_sel(codes, scales, q, pt, sel, n_sel, w.sm_scale, w.rope_dim, w.page_size)
    ro, rl = _brute_mla_sel(codes, scales, q, pt, sel, n_sel, w)
    for b in range(3):
        for h in range(w.n_heads):
            assert np.max(np.abs(o[b, h] - ro[b, h])) < 1e-12 * max(1.0, np.abs(ro[b, h]).max())
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(lse)) and np.max(np.abs(lse[fin] - rl[fin])) < 1e-12
    assert np.all(o[2] == 0) and np.all(np.isneginf(lse[2]))


def test_mla_sel_absent_throughout_is_empty():
    """A fixed-size list counted in full (n_sel = max_sel) whose entries are
    all absent attends no key: out = 0 and lse = -inf, as the brute force
    (which drops absent entries) gives; a list whose leading 64 entries are
    absent equals the list without them."""
    w = MLA_SMALL
    codes, scales, q, pt, sl = _build_mla(w, [500, 500])
    sel = np.full((2, 256), -1, np.int32)
    sel[1, 64:] = np.random.default_rng(9).permutation(500)[:192]
    n_sel = np.array([256, 256], np.int32)
    o, lse = oracle.mla_attention_sel(codes, scales, q, pt, sel, n_sel, w.sm_scale, w.rope_dim, w.page_size)
    ro, rl = _brute_mla_sel(codes, scales, q, pt, sel, n_sel, w)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0])) and np.all(np.isneginf(rl[0]))
    assert np.max(np.abs(o[1] - ro[1])) < 1e-12 * max(1.0, np.abs(ro[1]).max())
    tail = np.ascontiguousarray(sel[1:, 64:])
    o2, l2 = oracle.mla_attention_sel(codes, scales, q[1:].copy(), pt[1:].copy(), tail, np.array([192], np.int32),
                                      w.sm_scale, w.rope_dim, w.page_size)
    assert np.array_equal(o2[0], o[1]) and np.array_equal(l2[0], lse[1])


def test_mla_sel_order_and_duplicates():
    """Softmax attention is a function of the key multiset: reversing the list
    changes nothing beyond rounding, and listing every key twice changes
    nothing (each weight doubles, so does the normalizer) except lse += ln 2."""
    w = MLA_SMALL
    codes, scales, q, pt, sl = _build_mla(w, [600])
    sel = np.random.default_rng(4).permutation(600)[:400].astype(np.int32)[None, :]
    n = np.array([400], np.int32)
    a = oracle.mla_attention_sel(codes, scales, q, pt, sel, n, w.sm_scale, w.rope_dim, w.page_size)
    r = oracle.mla_attention_sel(codes, scales, q, pt, sel[:, ::-1].copy(), n, w.sm_scale, w.rope_dim, w.page_size)
    d = oracle.mla_attention_sel(codes, scales, q, pt, np.concatenate([sel, sel], 1), n * 2, w.sm_scale,
                                 w.rope_dim, w.page_size)
    assert np.max(np.abs(a[0] - r[0])) < 1e-12 and np.max(np.abs(a[1] - r[1])) < 1e-12
    assert np.max(np.abs(a[0] - d[0])) < 1e-12 and np.max(np.abs(a[1] + np.log(2.0) - d[1])) < 1e-12
