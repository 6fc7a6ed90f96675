"""Pins of the oracle's rotated-int4 + Lloyd-Max latent codec (colibri pull
request "KV cache quantization: fp8 (KV8) + 4-bit TurboQuant (KV_TQ)",
Summary "Why rotated-int4 for the 4-bit tier": randomized Hadamard rotation,
a fixed 16-level Lloyd-Max codebook optimal for N(0,1) scaled by
radius/sqrt(n), one radius per row part, ~0.096 relative L2 error at 4 bits,
radius-0 rows decode to zero).  Each pin is fixed by something other than
the oracle's own formulas: published generator outputs, numerical
integration by a library routine, the page's printed error figure, exact
scaling laws, brute force."""
import math

import numpy as np
import pytest

import oracle


def test_splitmix64_known_answers():
    # The first outputs of SplitMix64 from seed 0, as published with the
    # generator's reference implementation.
    assert [int(v) for v in oracle.splitmix64(0, 3)] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                                         0x06C45D188009454F]


def test_signs_are_plus_minus_one_and_balanced():
    for part, n in oracle.TQ_PARTS:
        s = oracle.tq_signs(part, n)
        assert set(np.unique(s)) <= {-1.0, 1.0}
        neg = int((s < 0).sum())
        assert abs(neg - n / 2) < 4 * math.sqrt(n / 4)   # binomial, 4 sigma
    assert not np.array_equal(oracle.tq_signs(0, 64), oracle.tq_signs(1, 64))


def test_lloyd_max_optimality_by_integration():
    """Each level is the mean of N(0,1) over its cell (checked by adaptive
    quadrature, a library routine independent of the oracle's closed form),
    the cells meet at midpoints, the levels are symmetric, and the mean
    squared error is the textbook 16-level figure 0.009497 (Max 1960)."""
    from scipy import integrate
    lev, it = oracle.lloyd_max_gauss(16)
    assert it < 100000
    assert np.all(np.diff(lev) > 0)
    assert np.array_equal(lev, -lev[::-1])
    pdf = lambda x: math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)
    edges = [-math.inf] + [0.5 * (lev[k] + lev[k + 1]) for k in range(15)] + [math.inf]
    mse = 0.0
    for k in range(16):
        a, b = edges[k], edges[k + 1]
        p = integrate.quad(pdf, a, b, epsabs=1e-14, epsrel=1e-13)[0]
        m1 = integrate.quad(lambda x: x * pdf(x), a, b, epsabs=1e-14, epsrel=1e-13)[0]
        assert abs(m1 / p - lev[k]) < 1e-9
        mse += integrate.quad(lambda x: (x - lev[k]) ** 2 * pdf(x), a, b, epsabs=1e-14, epsrel=1e-13)[0]
    assert abs(mse - 0.009497) < 5e-6


def test_tables_are_the_levels_in_fp32():
    lev64, _ = oracle.lloyd_max_gauss(16)
    lev, thr = oracle.tq_tables()
    assert np.array_equal(lev, lev64.astype(np.float32))
    assert np.array_equal(thr, (0.5 * (lev64[:-1] + lev64[1:])).astype(np.float32))
    assert thr[7] == 0.0


def test_quantize_is_the_nearest_level():
    """Brute force: the code is the index of the nearest fp32 level."""
    lev, thr = oracle.tq_tables()
    rng = np.random.default_rng(11)
    u = np.concatenate([rng.standard_normal(100000) * 1.5, [-9.0, 9.0, 0.0, -0.0, 1e-30, -1e-30]]).astype(np.float32)
    # keep away from the thresholds themselves, where both neighbours are nearest
    u = u[np.min(np.abs(u[:, None].astype(np.float64) - thr[None, :].astype(np.float64)), axis=1) > 1e-6]
    codes = oracle.tq_quantize(u)
    brute = np.argmin(np.abs(u[:, None].astype(np.float64) - lev[None, :].astype(np.float64)), axis=1)
    assert np.array_equal(codes, brute)
    # exactly on a threshold: the lower code
    assert list(oracle.tq_quantize(thr)) == list(range(15))


@pytest.mark.parametrize("part,n", oracle.TQ_PARTS)
def test_rotation_orthonormal_and_inverted(part, n):
    """R = H diag(s) / sqrt(n): R^T R = I; the fp64 inverse undoes the fp32
    forward rotation; R is the Sylvester Hadamard matrix (entries
    (-1)^popcount(i & j) / sqrt(n)) times the signs."""
    eye = np.eye(n, dtype=np.float32)
    R = np.stack([oracle.tq_rotate_f32(eye[j], part) for j in range(n)], axis=1).astype(np.float64)
    assert np.max(np.abs(R.T @ R - np.eye(n))) < 1e-6
    i = np.arange(n)
    H = np.array([[(-1) ** bin(a & b).count("1") for b in i] for a in i], np.float64) / math.sqrt(n)
    assert np.max(np.abs(R - H * oracle.tq_signs(part, n)[None, :])) < 1e-7
    x = np.random.default_rng(part).standard_normal(n).astype(np.float32)
    assert np.max(np.abs(oracle.tq_unrotate_f64(oracle.tq_rotate_f32(x, part), part) - x)) < 1e-5


def test_round_trip_error_is_the_pages_figure():
    """Gaussian latent rows: relative L2 round-trip error ~0.096 at 4 bits
    (the page's figure; sqrt of the quantizer's MSE, 0.0975, for a radius
    that matches the rotated row's spread)."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((200, 576)).astype(np.float32)
    codes = np.zeros((200, 288), np.uint8)
    radii = np.zeros((200, 2), np.float32)
    oracle.tq_store(codes, radii, x, np.arange(200))
    xh = oracle.tq_decode_rows(codes, radii)
    rel = np.linalg.norm(xh[:, :512] - x[:, :512], axis=1) / np.linalg.norm(x[:, :512], axis=1)
    assert 0.09 < rel.mean() < 0.10
    # the radius is the row part's Euclidean norm
    assert np.allclose(radii[:, 0], np.linalg.norm(x[:, :512].astype(np.float64), axis=1), rtol=1e-7)
    assert np.allclose(radii[:, 1], np.linalg.norm(x[:, 512:].astype(np.float64), axis=1), rtol=1e-7)


def test_power_of_two_scaling_keeps_codes():
    """Scaling a row by 2^k scales the rotation and the radius exactly, so
    the codes stay and the radius scales by 2^k exactly."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal(512).astype(np.float32)
    c0, r0 = oracle.tq_encode_part(x, 0)
    for k in (-20, -3, 1, 7, 30):
        c, r = oracle.tq_encode_part(x * np.float32(2.0 ** k), 0)
        assert np.array_equal(c, c0) and r == np.float32(r0 * 2.0 ** k)


def test_inert_rows():
    """Zero, NaN or infinite rows: radius 0, codes 0, decoded to zero."""
    for v in (0.0, np.nan, np.inf):
        x = np.zeros(576, np.float32)
        x[5] = v
        codes = np.full((1, 288), 0xAB, np.uint8)
        radii = np.full((1, 2), 7.0, np.float32)
        oracle.tq_store(codes, radii, x[None], np.array([0]))
        assert np.all(codes[0, :256] == 0) and radii[0, 0] == 0.0
        assert np.all(oracle.tq_decode_rows(codes, radii)[0, :512] == 0.0)


def test_nibble_order_and_scale():
    """Hand-written bytes: byte k holds element 2k (low nibble) and 2k+1
    (high nibble); an element decodes (before the inverse rotation) to its
    level times radius / sqrt(n)."""
    lev, _ = oracle.tq_tables()
    codes = np.zeros((1, 288), np.uint8)
    codes[0, :256] = 0x3C          # elements: 12, 3, 12, 3, ...
    codes[0, 256:] = 0xF0          # rope elements: 0, 15, ...
    radii = np.array([[math.sqrt(512.0) * 2.0, 8.0]], np.float32)
    x = oracle.tq_decode_rows(codes, radii)[0]
    yl = oracle.tq_rotate_f32(x[:512].astype(np.float32), 0).astype(np.float64)
    yr = oracle.tq_rotate_f32(x[512:].astype(np.float32), 1).astype(np.float64)
    assert np.allclose(yl[0::2], 2.0 * lev[12], atol=1e-5) and np.allclose(yl[1::2], 2.0 * lev[3], atol=1e-5)
    assert np.allclose(yr[0::2], lev[0], atol=1e-5) and np.allclose(yr[1::2], lev[15], atol=1e-5)


def test_attention_brute_force_and_rotated_space():
    """The oracle's attention equals a numpy softmax attention over its own
    decoded rows, and scores taken in rotated space (rotated query against
    levels x radius/sqrt(n)) equal those in the original space."""
    rng = np.random.default_rng(9)
    ps, n_pages, H = 16, 6, 5
    codes = np.zeros((ps * n_pages, 288), np.uint8)
    radii = np.zeros((ps * n_pages, 2), np.float32)
    lens = [37, 64, 0]
    pt = np.stack([rng.permutation(n_pages)[:4] for _ in lens]).astype(np.int32)
    used = set()
    for b, T in enumerate(lens):
        slots = np.array([pt[b, j // ps] * ps + j % ps for j in range(T)], np.int64)
        keep = [i for i, s in enumerate(slots) if s not in used]
        used.update(slots.tolist())
        x = (rng.standard_normal((T, 576)) * np.where(np.arange(576) % 50 == 0, 8.0, 1.0)).astype(np.float32)
        if keep:
            oracle.tq_store(codes, radii, x[keep], slots[keep])
    q = rng.standard_normal((len(lens), H, 576)).astype(np.float32)
    sm = 576 ** -0.5
    out, lse = oracle.tq_attention(codes, radii, q, pt, np.array(lens, np.int32), sm, ps)
    rows = oracle.tq_decode_rows(codes, radii)
    lev, _ = oracle.tq_tables()
    for b, T in enumerate(lens):
        if T == 0:
            assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b]))
            continue
        slots = np.array([pt[b, j // ps] * ps + j % ps for j in range(T)])
        K = rows[slots]
        s = sm * (q[b].astype(np.float64) @ K.T)
        p = np.exp(s - s.max(1, keepdims=True))
        ref = (p / p.sum(1, keepdims=True)) @ K[:, :512]
        assert np.max(np.abs(out[b] - ref)) < 1e-12 * max(1.0, np.abs(ref).max())
        assert np.allclose(lse[b], s.max(1) + np.log(p.sum(1)), rtol=0, atol=1e-12)
        # rotated space: q~ = R q per part, key = levels[codes] * r / sqrt(n)
        for part, lo, n in ((0, 0, 512), (1, 512, 64)):
            Rq = np.stack([oracle.tq_rotate_f32(q[b, h, lo:lo + n], part) for h in range(H)]).astype(np.float64)
            by = codes[slots][:, (0 if part == 0 else 256):(0 if part == 0 else 256) + n // 2]
            idx = np.stack([by & 15, by >> 4], axis=2).reshape(T, n)
            Y = lev[idx].astype(np.float64) * (radii[slots, part].astype(np.float64) / math.sqrt(n))[:, None]
            un = q[b, :, lo:lo + n].astype(np.float64) @ K[:, lo:lo + n].T
            assert np.max(np.abs(Rq @ Y.T - un)) < 2e-5 * max(1.0, np.abs(un).max())
