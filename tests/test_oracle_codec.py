"""Pins for the oracle's codecs: each test checks the oracle against something
other than itself -- a library routine, an exhaustive brute-force search,
a closed form, or a value the pages print.

Pages: TensorFold issue "qwen27 CUDA: an opt-in 4-bit attention cache"
("What it is"); FreeToken pull request "feat(kvcache): add reliable quantized
KV cache" (PR description, test-fix commit); colibri pull request "KV cache
quantization: fp8 (KV8) + 4-bit TurboQuant (KV_TQ)" (KV8 commit, Validation).
"""
import ctypes
import os
import struct
from decimal import Decimal, getcontext

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _h32():
    return scipy.linalg.hadamard(32).astype(np.float64) / np.sqrt(32.0)


# ----------------------------------------------------------------- binary16

def test_inv_sqrt32_is_correctly_rounded():
    """The fp32 rotation constant is the nearest single to 1/sqrt(32)."""
    getcontext().prec = 60
    exact = Decimal(1) / Decimal(32).sqrt()
    x = np.zeros(32, np.float32)
    x[0] = 1.0
    c = oracle.hadamard32_f32(x)[0]          # H e0 = c * ones
    up = np.nextafter(c, np.float32(1))
    dn = np.nextafter(c, np.float32(0))
    err = abs(Decimal(float(c)) - exact)
    assert err < abs(Decimal(float(up)) - exact) and err < abs(Decimal(float(dn)) - exact)
    assert struct.unpack("<I", struct.pack("<f", float(c)))[0] == 0x3E3504F3


# Rounding a float32 to a format that keeps its top k mantissa bits depends on
# those bits, the next (round) bit and whether any bit below it is set.  For
# binary16 (k <= 10) and e4m3 (k <= 3) the round bit is bit 12 or higher, so
# bits 0..6 only ever act as sticky bits: the float32 patterns whose low 7
# bits are 0, 1, 0x40 or 0x7F, with every higher bit pattern enumerated,
# contain every rounding case of every float32 (64 times fewer values than
# all of them).
_LOW7 = np.array([0x00, 0x01, 0x40, 0x7F], np.uint32)


def _rounding_classes(lo, hi, chunk=1 << 22):
    """Chunks of float32 bit patterns in [lo, hi) with low 7 bits in _LOW7."""
    for h0 in range(lo >> 7, (hi + 127) >> 7, chunk):
        high = np.arange(h0, min(h0 + chunk, (hi + 127) >> 7), dtype=np.uint32)
        bits = ((high[:, None] << np.uint32(7)) | _LOW7[None, :]).ravel()
        yield bits[(bits >= lo) & (bits < hi)]


def test_f16_exhaustive_against_library():
    """binary16 RNE of every rounding case of a positive float32 in the
    binades where rounding is not trivially 0 or infinity (2^-26 .. 2^16),
    against torch's cast."""
    lo, hi = 0x32800000, 0x47800000  # 2^-26 .. 2^16
    n = 0
    for bits in _rounding_classes(lo, hi):
        x = bits.view(np.float32)
        ours = oracle.f32_to_f16_bits(x)
        ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
        bad = np.nonzero(ours != ref)[0]
        assert bad.size == 0, f"f16 mismatch at {x[bad[:4]]}"
        n += bits.size
    assert n == (hi - lo) // 32


def test_f16_decode_every_pattern_against_library():
    """binary16 -> float32 widening of all 65536 bit patterns (zeros, the
    1023 subnormals per sign, normals, infinities, NaNs) against numpy's
    float16 -> float32 conversion: identical bits, NaN for NaN."""
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_bits_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 * 1023
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    # subnormals are m * 2^-24 exactly, by a closed form too
    m = np.arange(1, 1024)
    assert np.array_equal(oracle.f16_bits_to_f32(m.astype(np.uint16)).astype(np.float64), np.ldexp(m, -24))
    assert np.array_equal(oracle.f16_bits_to_f32((m | 0x8000).astype(np.uint16)).astype(np.float64),
                          -np.ldexp(m, -24))


def test_f16_sign_and_specials():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    ours = oracle.f32_to_f16_bits(x)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    sp = np.array([0.0, -0.0, np.inf, -np.inf, 65504, 65519.99, 65520, 2 ** -24, 2 ** -25, 3 * 2 ** -25],
                  np.float32)
    assert np.array_equal(oracle.f32_to_f16_bits(sp),
                          torch.from_numpy(sp).to(torch.float16).view(torch.int16).numpy().view(np.uint16))


# ----------------------------------------------------------------- Hadamard

def test_rotation_is_orthonormal_sylvester():
    """The fp64 rotation is the Sylvester Hadamard matrix / sqrt(32) (scipy's),
    orthonormal and its own inverse (colibri Validation: rotation self-inverse)."""
    eye = np.eye(32)
    Hcols = oracle.rotate_f64(eye)           # row i = H e_i = column i of H
    H = _h32()
    assert np.max(np.abs(Hcols - H.T)) < 1e-15
    assert np.max(np.abs(H @ H.T - eye)) < 1e-15
    x = np.random.default_rng(0).standard_normal((7, 256))
    assert np.max(np.abs(oracle.rotate_f64(oracle.rotate_f64(x)) - x)) < 1e-13


def test_rotated_dot_equals_unrotated_dot():
    """(Hq).(Hk) = q.k: attention in rotated space needs no other change."""
    rng = np.random.default_rng(1)
    q = rng.standard_normal((50, 256))
    k = rng.standard_normal((50, 256))
    lhs = np.sum(oracle.rotate_f64(q) * oracle.rotate_f64(k), axis=1)
    assert np.max(np.abs(lhs - np.sum(q * k, axis=1))) < 1e-12


def test_fp32_butterfly_matches_matrix():
    """The fp32 storage butterfly is the same transform within fp32 rounding."""
    x = np.random.default_rng(2).standard_normal((1000, 32)).astype(np.float32)
    y32 = oracle.hadamard32_f32(x).astype(np.float64)
    y64 = x.astype(np.float64) @ _h32().T
    assert np.max(np.abs(y32 - y64)) < 4e-6


# ----------------------------------------------------------------- 4-bit rows

def _scales(rows, D):
    return rows[..., D // 2:].copy().view(np.uint16)


def _codes(rows, D):
    """Signed codes unpacked with numpy, independently of the oracle: byte k of
    the code bytes holds element 2k in its low nibble and 2k+1 in its high
    nibble, two's complement (FreeToken test-fix commit: int32 sign extension)."""
    c = rows[..., :D // 2].astype(np.int16)
    out = np.empty(rows.shape[:-1] + (D,), np.float64)
    out[..., 0::2] = ((c & 0xF) ^ 8) - 8
    out[..., 1::2] = ((c >> 4) ^ 8) - 8
    return out


def _np_scales(rows, D):
    """The fp16 scales widened by numpy (the library's binary16 decoding)."""
    return _scales(rows, D).view(np.float16).astype(np.float64)


def test_row_sizes():
    """144 bytes per row at head_dim 256 (TensorFold "What it is"); 0.5625 B/element (FreeToken)."""
    assert oracle.q4_row_bytes(256) == 144
    assert oracle.q4_row_bytes(128) == 72
    assert oracle.q4_row_bytes(256) / 256 == 0.5625


def test_nibble_sign_extension_exhaustive():
    """Every byte decodes to (low nibble, high nibble) as the int32
    arithmetic-shift sign extension defines them (FreeToken test-fix commit)."""
    D = 32
    rows = np.zeros((256, 18), np.uint8)
    rows[:, 0] = np.arange(256)
    rows[:, 16:18] = np.frombuffer(np.uint16(0x3C00).tobytes(), np.uint8)
    vals = oracle.q4_decode_rows(rows, D)
    for b in range(256):
        lo = ctypes.c_int32(b << 28).value >> 28
        hi = ctypes.c_int32((b >> 4) << 28).value >> 28
        assert vals[b, 0] == lo and vals[b, 1] == hi
        assert np.all(vals[b, 2:] == 0)


@pytest.mark.parametrize("trial_seed", range(4))
def test_exact_scale_example(trial_seed):
    """FreeToken test-fix commit: with amax 8 the scale is exactly 1.0 and the
    codes equal the inputs.  Here the integers live in the rotated domain:
    the row is x = H c (c in [-8,7]^32 with -8 present), rounded to fp32."""
    rng = np.random.default_rng(100 + trial_seed)
    H = _h32()
    n = 500
    c = rng.integers(-8, 8, size=(n, 32))
    c[np.arange(n), rng.integers(0, 32, n)] = -8
    x = (c.astype(np.float64) @ H.T).astype(np.float32)
    rows = oracle.q4_encode_rows(x)
    assert np.all(_scales(rows, 32) == 0x3C00)
    assert np.array_equal(_codes(rows, 32), c.astype(np.float64))


@pytest.mark.parametrize("trial_seed", range(3))
def test_exact_scale_example_subnormal_scales(trial_seed):
    """The exact-scale example at binary16 subnormal scales: rotated-domain
    rows y = c * s with c in [-8, 7]^32 (-8 present) and s = m * 2^-24 a
    subnormal (m < 1024), so amax/8 = s exactly; the stored scale must be the
    subnormal bit pattern m, the codes c, and the dequantized values c * s
    (numpy's float16 widening of the stored bits)."""
    rng = np.random.default_rng(300 + trial_seed)
    H = _h32()
    n = 600
    m = rng.integers(1, 1024, size=n)
    m[:4] = [1, 2, 1023, 512]
    c = rng.integers(-8, 8, size=(n, 32))
    c[np.arange(n), rng.integers(0, 32, n)] = -8
    y = c.astype(np.float64) * np.ldexp(m, -24)[:, None]
    x = (y @ H.T).astype(np.float32)
    rows = oracle.q4_encode_rows(x)
    assert np.array_equal(_scales(rows, 32)[:, 0], m.astype(np.uint16))
    assert np.array_equal(_codes(rows, 32), c.astype(np.float64))
    deq = oracle.q4_decode_rows(rows, 32)
    assert np.array_equal(deq, c * _np_scales(rows, 32))
    assert np.array_equal(deq, y)


def test_tiny_groups_round_to_subnormal_or_zero_scale():
    """Groups whose amax/8 falls below 2^-14 get the nearest subnormal scale
    (numpy's binary16 rounding of amax/8), codes nearest in [-8, 7]; below
    2^-25 the scale rounds to 0 and the group is inert."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((800, 64)).astype(np.float32)
    mag = np.ldexp(1.0, -rng.integers(12, 30, size=(800, 1))).astype(np.float32)
    x = x * mag
    rows = oracle.q4_encode_rows(x)
    y = oracle.hadamard32_f32(x).reshape(800, 2, 32)
    amax = np.abs(y).max(axis=2).astype(np.float32)
    ref = (amax / np.float32(8)).astype(np.float16)
    assert np.array_equal(_scales(rows, 64), ref.view(np.uint16))
    sub = (ref > 0) & (ref < np.float16(2.0 ** -14))
    assert sub.sum() > 200 and (ref == 0).sum() > 50  # both regimes are exercised
    s = _np_scales(rows, 64)
    codes = _codes(rows, 64).reshape(800, 2, 32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (y / s[..., None].astype(np.float32)).astype(np.float64)
    expect = np.clip(np.round(r), -8, 7)  # numpy rounds half to even
    live = s > 0
    assert np.array_equal(codes[live], expect[live])
    assert np.all(codes[~live] == 0)
    deq = oracle.q4_decode_rows(rows, 64).reshape(800, 2, 32)
    assert np.array_equal(deq, codes * s[..., None])


def test_plus_eight_clamps_to_seven():
    """+amax maps to +8, which the [-8, 7] code range clamps to 7."""
    H = _h32()
    c = np.zeros((1, 32))
    c[0, 3] = 8.0
    c[0, 9] = -5.0
    x = (c @ H.T).astype(np.float32)
    rows = oracle.q4_encode_rows(x)
    assert _scales(rows, 32)[0, 0] == 0x3C00
    got = _codes(rows, 32)[0]
    assert got[3] == 7 and got[9] == -5 and np.count_nonzero(got) == 2


def test_scale_is_library_fp16_of_amax_over_8():
    """Scale = binary16(amax/8) of the rotated group, binary16 by torch's cast."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((2000, 256)) * np.exp(rng.standard_normal((2000, 1)) * 3)).astype(np.float32)
    rows = oracle.q4_encode_rows(x)
    y = oracle.hadamard32_f32(x).reshape(2000, 8, 32)
    amax = np.abs(y).max(axis=2).astype(np.float32)
    ref = torch.from_numpy(amax / np.float32(8)).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(_scales(rows, 256), ref)


def test_codes_are_nearest_in_range():
    """Each code is the integer in [-8, 7] nearest to y/scale (ties to even),
    found by brute force over all 16 codes."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3000, 64)).astype(np.float32)
    x[::7] *= 1e-3
    x[1::11, 5] *= 40
    rows = oracle.q4_encode_rows(x)
    y = oracle.hadamard32_f32(x).reshape(-1, 2, 32).astype(np.float64)
    s = _np_scales(rows, 64)
    codes = _codes(rows, 64).reshape(-1, 2, 32)
    r = (y.astype(np.float32) / s[..., None].astype(np.float32)).astype(np.float64)  # fp32 quotient
    cand = np.arange(-8, 8, dtype=np.float64)
    dist = np.abs(r[..., None] - cand)
    best = dist.min(-1, keepdims=True)
    ties = (dist == best)
    # nearest; on a tie the even candidate
    multi = ties.sum(-1, keepdims=True) > 1
    pick = np.where(multi, np.where(ties & (cand % 2 == 0), cand, np.nan), np.where(ties, cand, np.nan))
    expect = np.nanmax(pick, axis=-1)
    assert np.all(s > 0)
    assert np.array_equal(codes, expect)


def test_zero_group_is_inert():
    x = np.zeros((2, 64), np.float32)
    x[1, 32:] = 1e-12        # amax/8 underflows binary16 -> scale 0
    rows = oracle.q4_encode_rows(x)
    assert np.all(rows == 0)


def test_out_of_domain_rejected():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = np.nan
    with pytest.raises(ValueError):
        oracle.q4_encode_rows(x)
    x[0, 0] = 1e7            # rotated amax/8 beyond binary16
    with pytest.raises(ValueError):
        oracle.q4_encode_rows(x)


def test_roundtrip_error_statistics():
    """Soft sanity: 4-bit Hadamard-32 round trip on N(0,1) has relative L2
    error near 0.09, and the rotation beats no rotation on heavy tails
    (FreeToken reports ~0.13 unrotated on kurtotic data)."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((4000, 256)).astype(np.float32)
    rows = oracle.q4_encode_rows(x)
    rec = oracle.rotate_f64(oracle.q4_decode_rows(rows, 256))
    rel = np.linalg.norm(rec - x) / np.linalg.norm(x)
    assert 0.08 < rel < 0.105, rel
    t = rng.standard_t(3, size=(4000, 256)).astype(np.float32)
    rec_t = oracle.rotate_f64(oracle.q4_decode_rows(oracle.q4_encode_rows(t), 256))
    rel_t = np.linalg.norm(rec_t - t) / np.linalg.norm(t)
    assert rel_t < 0.11, rel_t


# ----------------------------------------------------------------- e4m3

def _torch_e4m3_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_all_codes():
    """The 256-code table against torch's float8_e4m3fn; NaN codes read 0."""
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = (codes & 0x7F) == 0x7F
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all(ours[nan] == 0.0)
    assert ours.max() == 448.0 and ours.min() == -448.0


def test_e4m3_roundtrip_every_code():
    """enc(dec(c)) = c for every non-NaN code, including -0 -> 0x80 (colibri
    KV8 commit: exhaustive round trip, signed zero kept)."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    vals[codes == 0x80] = np.float32(-0.0)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


def test_e4m3_ties_and_saturation():
    """Round-to-nearest-even ties, including the binade-boundary carry, and
    saturation at +-448 (colibri KV8 commit)."""
    cases = [(0.96875, 0x38), (1.9375, 0x40), (7.5 * 2 ** -9, 0x08), (2 ** -10, 0x00), (3 * 2 ** -10, 0x02),
             (448.0, 0x7E), (464.0, 0x7E), (1e30, 0x7E), (np.inf, 0x7E), (-np.inf, 0xFE), (-448.5, 0xFE),
             (np.nan, 0x00), (-0.0, 0x80), (0.0, 0x00)]
    x = np.array([v for v, _ in cases], np.float32)
    assert [int(c) for c in oracle.e4m3_encode(x)] == [c for _, c in cases]


def test_e4m3_exhaustive_against_library():
    """Every rounding case of a float32 with |v| <= 448 (see _rounding_classes)
    against torch's RNE cast; float32 values in (448, 2^31) saturate.
    Negative values on the same bits with the sign set."""
    top = 0x43E00000  # 448.0
    for bits in _rounding_classes(0, top + 1):
        for sign in (0, 0x80000000):
            x = (bits | np.uint32(sign)).view(np.float32)
            ours = oracle.e4m3_encode(x)
            ref = _torch_e4m3_bits(x)
            bad = np.nonzero(ours != ref)[0]
            assert bad.size == 0, f"e4m3 mismatch at {x[bad[:4]]}: {ours[bad[:4]]} vs {ref[bad[:4]]}"
    big = np.arange(top + 1, 0x4F000000, 4099, dtype=np.uint32).view(np.float32)
    assert np.all(oracle.e4m3_encode(big) == 0x7E)


def test_e4m3_nearest_value_search():
    """Brute force: the code's value is the nearest e4m3 value (ties to the
    even mantissa) over a random sample of all float32 bit patterns."""
    table = oracle.e4m3_decode(np.arange(128, dtype=np.uint8))[:127]   # 0 .. 448, ascending
    rng = np.random.default_rng(8)
    bits = rng.integers(0x00000000, 0x43E00001, size=400000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32).astype(np.float64)
    codes = oracle.e4m3_encode(x.astype(np.float32))
    d = np.abs(x[:, None] - table[None, :])
    best = d.min(1, keepdims=True)
    tie = (d == best)
    even = (np.arange(127) % 2 == 0)[None, :]
    pick = np.where(tie.sum(1) > 1, np.argmax(tie & even, axis=1), np.argmax(tie, axis=1))
    assert np.array_equal(codes, pick.astype(np.uint8))


# ----------------------------------------------------------------- fp8 rows

def test_fp8_row_scale_and_codes():
    """Per-row scale amax/448 and codes e4m3(x * 448/amax) (colibri KV8 commit)."""
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(512) * 3).astype(np.float32)
    codes, scale = oracle.fp8_encode_part(x)
    amax = np.float32(np.abs(x).max())
    assert scale == np.float32(amax / np.float32(448))
    inv = np.float32(np.float32(448) / amax)
    assert np.array_equal(codes, _torch_e4m3_bits(x * inv))
    rec = oracle.e4m3_decode(codes) * scale
    assert np.max(np.abs(rec - x)) <= amax * 2 ** -4 + 1e-30


@pytest.mark.parametrize("kind", ["zero", "inf", "tiny"])
def test_fp8_inert_rows(kind):
    """Rows with amax 0, a non-finite amax, or 448/amax overflowing are stored
    inert: scale 0, all codes 0 (colibri KV8 commit, subnormal-amax guard)."""
    x = np.zeros(64, np.float32)
    if kind == "inf":
        x[3] = np.inf
        x[4] = 2.0
    if kind == "tiny":
        x[5] = np.float32(1e-39)
    codes, scale = oracle.fp8_encode_part(x)
    assert scale == 0.0 and np.all(codes == 0)


def test_fp8_nan_element_stored_as_zero():
    x = np.linspace(-2, 2, 64).astype(np.float32)
    x[10] = np.nan
    codes, scale = oracle.fp8_encode_part(x)
    assert codes[10] == 0x00 and scale == np.float32(np.float32(2.0) / np.float32(448))
