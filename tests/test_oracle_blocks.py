"""Pins for the oracle's 6- and 8-bit block formats (the q6_0 / q8_0
variants of the same skeleton): row sizes the pages print, the exact-scale
example, library fp16 scales, brute-force nearest codes, hand-computed byte
layouts, exhaustive decodes, and a brute-force attention.

Pages: FreeToken pull request "feat(kvcache): add reliable quantized KV
cache" (PR description: q8_0 at 1.0625 bytes per element beside the 4-bit
layout, one spec for all schemes; test-fix commit: the exact-scale amax is
31.0 for q6_0, whose divisor is its largest magnitude 31).
"""
import ctypes

import numpy as np
import pytest
import scipy.linalg
import scipy.special
import torch

import oracle

DIV = {6: 31.0, 8: 127.0}
GB = {4: 16, 6: 24, 8: 32}


def _h32():
    return scipy.linalg.hadamard(32).astype(np.float64) / np.sqrt(32.0)


def _scales(rows, D, bits):
    G = D // 32
    return rows[..., GB[bits] * G:].copy().view(np.uint16)


def _unpack(rows, D, bits):
    """Codes per the stated layouts, in numpy (independent of the C decoder)."""
    G = D // 32
    out = np.empty(rows.shape[:-1] + (D,), np.int64)
    for g in range(G):
        c = rows[..., GB[bits] * g: GB[bits] * (g + 1)].astype(np.int64)
        if bits == 8:
            out[..., 32 * g: 32 * g + 32] = np.where(c > 127, c - 256, c)
            continue
        lo = np.empty(c.shape[:-1] + (32,), np.int64)
        lo[..., 0::2] = c[..., :16] & 0xF
        lo[..., 1::2] = c[..., :16] >> 4
        hi = np.empty_like(lo)
        for i in range(4):
            hi[..., i::4] = (c[..., 16:24] >> (2 * i)) & 3
        v = lo | (hi << 4)
        out[..., 32 * g: 32 * g + 32] = np.where(v > 31, v - 64, v)
    return out


def test_row_sizes():
    """q8_0: 1.0625 bytes per element (FreeToken PR description); 6-bit: 0.8125."""
    assert oracle.q4_row_bytes(256, 8) == 272 and oracle.q4_row_bytes(256, 8) / 256 == 1.0625
    assert oracle.q4_row_bytes(256, 6) == 208 and oracle.q4_row_bytes(256, 6) / 256 == 0.8125
    assert oracle.q4_row_bytes(128, 6) == 104 and oracle.q4_row_bytes(64, 8) == 68


@pytest.mark.parametrize("bits", [6, 8])
def test_exact_scale_example(bits):
    """With amax equal to the divisor (31.0 for q6_0, as the test-fix commit
    states; 127 for 8 bits) the scale is exactly 1.0 and the codes equal the
    rotated-domain integers (x = H c rounded to fp32)."""
    m = int(DIV[bits])
    rng = np.random.default_rng(bits)
    n = 400
    c = rng.integers(-m, m + 1, size=(n, 32))
    c[np.arange(n), rng.integers(0, 32, n)] = np.where(rng.random(n) < 0.5, -m, m)
    x = (c.astype(np.float64) @ _h32().T).astype(np.float32)
    rows = oracle.q4_encode_rows(x, bits)
    assert np.all(_scales(rows, 32, bits) == 0x3C00)
    assert np.array_equal(_unpack(rows, 32, bits), c)
    assert np.array_equal(oracle.q4_decode_rows(rows, 32, bits), c.astype(np.float64))


def test_byte_layouts_by_hand():
    """Bytes written out by hand from the stated layouts."""
    H = _h32()
    c = np.zeros((1, 32))
    c[0, :4] = [-31, 31, 5, -1]
    r6 = oracle.q4_encode_rows((c @ H.T).astype(np.float32), 6)[0]
    want6 = np.zeros(26, np.uint8)
    want6[0], want6[1] = 0xF1, 0xF5           # low nibbles (-31 -> 0x1, 31 -> 0xF, 5, -1 -> 0xF)
    want6[16] = 0xC6                          # high two bits 2, 1, 0, 3 at bit pairs 0, 1, 2, 3
    want6[24], want6[25] = 0x00, 0x3C         # scale 1.0
    assert np.array_equal(r6, want6)
    c8 = np.zeros((1, 32))
    c8[0, :3] = [-127, 127, -1]
    r8 = oracle.q4_encode_rows((c8 @ H.T).astype(np.float32), 8)[0]
    want8 = np.zeros(34, np.uint8)
    want8[:3] = [0x81, 0x7F, 0xFF]
    want8[32], want8[33] = 0x00, 0x3C
    assert np.array_equal(r8, want8)


def test_decode_exhaustive():
    """6 bits: all 64 codes at every nibble and two-bit position, against the
    int32 arithmetic-shift sign extension; 8 bits: all 256 bytes against
    numpy's int8 view."""
    rows = np.zeros((64, 4, 26), np.uint8)
    rows[..., 24:26] = np.frombuffer(np.uint16(0x3C00).tobytes(), np.uint8)
    for v in range(64):
        for i in range(4):             # element i of the group
            rows[v, i, i // 2] = (v & 0xF) << (4 * (i & 1))
            rows[v, i, 16] = (v >> 4) << (2 * i)
    vals = oracle.q4_decode_rows(rows, 32, 6)
    for v in range(64):
        want = ctypes.c_int32(v << 26).value >> 26
        for i in range(4):
            assert vals[v, i, i] == want and np.count_nonzero(vals[v, i]) == (want != 0)
    r8 = np.zeros((256, 34), np.uint8)
    r8[:, 5] = np.arange(256)
    r8[:, 32:34] = np.frombuffer(np.uint16(0x3C00).tobytes(), np.uint8)
    v8 = oracle.q4_decode_rows(r8, 32, 8)
    assert np.array_equal(v8[:, 5], np.arange(256).astype(np.uint8).view(np.int8).astype(np.float64))


@pytest.mark.parametrize("bits", [6, 8])
def test_scale_is_library_fp16(bits):
    rng = np.random.default_rng(30 + bits)
    x = (rng.standard_normal((1500, 256)) * np.exp(rng.standard_normal((1500, 1)) * 3)).astype(np.float32)
    rows = oracle.q4_encode_rows(x, bits)
    y = oracle.hadamard32_f32(x).reshape(1500, 8, 32)
    amax = np.abs(y).max(axis=2).astype(np.float32)
    ref = torch.from_numpy(amax / np.float32(DIV[bits])).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(_scales(rows, 256, bits), ref)


@pytest.mark.parametrize("bits", [6, 8])
def test_codes_are_nearest_in_range(bits):
    """Each code is the integer of the signed range nearest to y/scale (ties
    to even), by brute force over every code of the width."""
    rng = np.random.default_rng(40 + bits)
    x = rng.standard_normal((1500, 64)).astype(np.float32)
    x[::7] *= 1e-3
    x[1::11, 5] *= 40
    rows = oracle.q4_encode_rows(x, bits)
    y = oracle.hadamard32_f32(x).reshape(-1, 2, 32)
    s = _scales(rows, 64, bits).view(np.float16).astype(np.float32)
    codes = _unpack(rows, 64, bits).reshape(-1, 2, 32).astype(np.float64)
    r = (y / s[..., None].astype(np.float32)).astype(np.float64)        # the fp32 quotient
    cand = np.arange(-(1 << (bits - 1)), 1 << (bits - 1), dtype=np.float64)
    dist = np.abs(r[..., None] - cand)
    ties = dist == dist.min(-1, keepdims=True)
    multi = ties.sum(-1, keepdims=True) > 1
    pick = np.where(multi, np.where(ties & (cand % 2 == 0), cand, np.nan), np.where(ties, cand, np.nan))
    assert np.all(s > 0)
    assert np.array_equal(codes, np.nanmax(pick, axis=-1))
    m = DIV[bits]
    assert np.abs(codes).max() <= m   # |y| <= amax and the fp16 scale is within 2^-11 of amax/m


@pytest.mark.parametrize("bits,lo,hi", [(6, 0.015, 0.03), (8, 0.003, 0.008)])
def test_roundtrip_error(bits, lo, hi):
    """Soft sanity: uniform quantization with step amax/divisor (amax of 32
    Gaussian values is ~2.5 sigma) leaves relative L2 error ~(2.5/m)/sqrt(12)."""
    rng = np.random.default_rng(50 + bits)
    x = rng.standard_normal((3000, 256)).astype(np.float32)
    rec = oracle.rotate_f64(oracle.q4_decode_rows(oracle.q4_encode_rows(x, bits), 256, bits))
    rel = np.linalg.norm(rec - x) / np.linalg.norm(x)
    assert lo < rel < hi, rel


@pytest.mark.parametrize("bits", [6, 8])
def test_attention_matches_brute_force(bits):
    """The oracle's fp64 decode attention over 6- and 8-bit pools against
    numpy: rows unpacked per the stated layout, softmax by scipy, output
    rotated back with scipy's Hadamard matrix."""
    rng = np.random.default_rng(60 + bits)
    H_kv, G, D, ps = 2, 3, 64, 16
    lens = [70, 33]
    pages = [(T + ps - 1) // ps for T in lens]
    num_pages = sum(pages)
    perm = rng.permutation(num_pages).astype(np.int32)
    pt = np.zeros((2, max(pages)), np.int32)
    pt[0, :pages[0]] = perm[:pages[0]]
    pt[1, :pages[1]] = perm[pages[0]:]
    shape = oracle.q4_pool_shape(num_pages, H_kv, ps, D, bits)
    kp, vp = np.zeros(shape, np.uint8), np.zeros(shape, np.uint8)
    for b, T in enumerate(lens):
        k = rng.standard_normal((T, H_kv, D)).astype(np.float32)
        v = rng.standard_normal((T, H_kv, D)).astype(np.float32)
        j = np.arange(T)
        oracle.q4_store(kp, vp, k, v, pt[b, j // ps].astype(np.int64) * ps + j % ps, ps)
    q = rng.standard_normal((2, H_kv * G, D)).astype(np.float32)
    o, lse = oracle.q4_attention(kp, vp, q, pt, np.array(lens, np.int32), 0.125)
    Hm = scipy.linalg.hadamard(32) / np.sqrt(32.0)
    rot = lambda a: (a.reshape(-1, 32) @ Hm.T).reshape(a.shape)
    for b, T in enumerate(lens):
        j = np.arange(T)
        pg, off = pt[b, j // ps], j % ps
        for h in range(H_kv * G):
            g = h // G
            def deq(pool):
                rows = pool[pg, g, off]
                s = _scales(rows, D, bits).view(np.float16).astype(np.float64)
                return _unpack(rows, D, bits) * np.repeat(s, 32, axis=-1)
            K, V = deq(kp), deq(vp)
            sc = 0.125 * (K @ rot(q[b, h].astype(np.float64)))
            ref = rot(scipy.special.softmax(sc) @ V)
            assert np.max(np.abs(o[b, h] - ref)) < 1e-12 * max(1.0, np.abs(ref).max())
            assert abs(lse[b, h] - scipy.special.logsumexp(sc)) < 1e-12
