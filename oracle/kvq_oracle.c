/*
 * kvq_oracle.c -- plain, slow CPU oracle for the sub-byte KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  This file states what the GPU library has to
 * compute, as literally as possible, so that tests can compare the GPU
 * results with it.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load it.  The GPU library neither links nor calls it, and
 * the two share no source: no headers, helpers, tables or constants.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC.
 * Every float operation below is a single IEEE operation in the stated
 * precision (fp32 for the codecs, fp64 for attention); nothing is fused.
 *
 * Sources (web pages, cited by title and the section the fact is in):
 *   [TF]  TensorFold issue "qwen27 CUDA: an opt-in 4-bit attention cache
 *         (262K on a 24 GB card)": section "What it is" (144-byte rows of
 *         Hadamard-rotated 32-value groups, 4-bit codes plus an fp16 scale;
 *         rotate the query once, attend in rotated space over 512-key
 *         chunks and each row's tail, merge in order, rotate the output back).
 *   [FT]  FreeToken pull request "feat(kvcache): add reliable quantized KV
 *         cache": PR description (32 values -> 16 bytes + one fp16 scale,
 *         0.5625 B/element) and the test-fix commit (scale = amax/8, the
 *         exact-scale example, int32 arithmetic-shift sign extension).
 *   [CO]  colibri pull request "KV cache quantization: fp8 (KV8) + 4-bit
 *         TurboQuant (KV_TQ) on CPU, CUDA, and Metal": KV8 commit (e4m3
 *         rows with a per-row f32 amax/448 scale, round-to-nearest-even
 *         encoder saturating at +-448 with signed zero kept and NaN stored as
 *         0, a guard for an amax so small that 448/amax overflows, absorbed
 *         attention where the latent is key and value), split-T commit
 *         (partials (cl[K], m, z) and a log-sum-exp merge), the
 *         correctness/performance commit (NaN codes read as 0), and the
 *         Summary "Why rotated-int4 for the 4-bit tier" (the TQ4 codec at
 *         the end of this file, with its own readings).
 *
 * Readings of points the pages leave open (each one is listed in the design
 * notes with its reason):
 *   - Hadamard: Sylvester order, orthonormal (entries +-1/sqrt(32)), no random
 *     signs; it is its own inverse.
 *   - fp32 butterfly in stages h = 1,2,4,8,16, then one multiply by
 *     fp32(1/sqrt(32)) = 0x3E3504F3.
 *   - scale = fp16_rne(amax/8); codes divide by that stored scale widened to
 *     fp32; round half to even; clamp to [-8, 7]; scale 0 gives all-zero codes.
 *   - element 2k in the low nibble, 2k+1 in the high nibble, two's complement.
 *   - a row is D/2 bytes of codes (group after group), then D/32 fp16 scales,
 *     little-endian.
 *   - fp8 latent rows keep two scales per position: one for the 512-wide
 *     latent part, one for the 64-wide rope part.
 *   - an fp8 row whose amax is 0, non-finite, or so small that 448/amax is not
 *     finite is stored inert: scale 0 and every code 0x00.
 *   - the chunk partition of a sequence depends only on its length; chunks
 *     are merged in ascending order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KVQO_OK 0
#define KVQO_EDOMAIN (-1)
#define KVQO_ERANGE (-2)
#define KVQO_EARG (-3)

int kvqo_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* IEEE binary16, round to nearest even ([TF] "What it is": fp16 scale) */
/* ------------------------------------------------------------------ */

/* Nearest binary16 value of f, ties to even mantissa, overflow to infinity.
 * Written as "pick the nearest multiple of the binade's spacing" rather than
 * as bit manipulation. */
uint16_t kvqo_f32_to_f16(float f) {
    double v = (double)f;
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isnan(v)) return (uint16_t)(sign | 0x7E00u);
    if (isinf(v)) return (uint16_t)(sign | 0x7C00u);
    if (a == 0.0) return sign;
    if (a < ldexp(1.0, -14)) {
        /* subnormal binade: spacing 2^-24; n == 1024 is the smallest normal */
        double n = nearbyint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)n);
    }
    int e2;
    frexp(a, &e2);          /* a in [2^(e2-1), 2^e2) */
    int E = e2 - 1;         /* a in [2^E, 2^(E+1)) */
    double n = nearbyint(ldexp(a, 10 - E)); /* in [1024, 2048] */
    if (n == 2048.0) { n = 1024.0; E += 1; }
    if (E > 15) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)(((E + 15) << 10) | ((int)n - 1024)));
}

float kvqo_f16_to_f32(uint16_t h) {
    int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), e - 25);
    return (float)(s ? -v : v);
}

/* ------------------------------------------------------------------ */
/* Hadamard-32                                                         */
/* ------------------------------------------------------------------ */

/* fp32(1/sqrt(32)): the correctly rounded single of 0.17677669529663688... */
static float kvqo_inv_sqrt32_f32(void) {
    uint32_t bits = 0x3E3504F3u;
    float c;
    memcpy(&c, &bits, 4);
    return c;
}

/* The storage rotation of one 32-value group, in fp32 ([TF] "What it is":
 * rows are Hadamard-rotated in groups of 32).  Stages h = 1,2,4,8,16; each
 * stage replaces (t_i, t_{i+h}) by (t_i + t_{i+h}, t_i - t_{i+h}) for every i
 * with bit h clear; then every element is multiplied by fp32(1/sqrt(32)). */
void kvqo_hadamard32_f32(float t[32]) {
    for (int h = 1; h < 32; h <<= 1) {
        for (int i = 0; i < 32; ++i) {
            if (i & h) continue;
            float a = t[i], b = t[i + h];
            t[i] = a + b;
            t[i + h] = a - b;
        }
    }
    float c = kvqo_inv_sqrt32_f32();
    for (int i = 0; i < 32; ++i) t[i] = t[i] * c;
}

/* Entry (i, j) of the orthonormal Sylvester Hadamard matrix of order 32. */
static double kvqo_h32(int i, int j) {
    return (__builtin_popcount((unsigned)(i & j)) & 1) ? -1.0 / sqrt(32.0) : 1.0 / sqrt(32.0);
}

/* y = H32 x for every 32-group of a length-n vector, in fp64, as a plain
 * matrix-vector product.  H32 is symmetric and orthonormal, so the same call
 * rotates the query ([TF] "rotate the queries once") and rotates the output
 * back ("rotate the output back once"). */
void kvqo_rotate_f64(const double* x, double* y, int n) {
    for (int g = 0; g < n / 32; ++g) {
        for (int i = 0; i < 32; ++i) {
            double acc = 0.0;
            for (int j = 0; j < 32; ++j) acc += kvqo_h32(i, j) * x[32 * g + j];
            y[32 * g + i] = acc;
        }
    }
}

/* ------------------------------------------------------------------ */
/* 4-bit Hadamard-32 row codec                                         */
/* ------------------------------------------------------------------ */

/* Block formats of the same skeleton (rotated groups of 32 values, one fp16
 * scale per group, codes of `bits` bits): 4 (the format above), 6 and 8.
 * [FT] PR description: the q4_0 layout sits beside q8_0 (1.0625 bytes per
 * element: 32 one-byte codes + one fp16 scale) in one spec, and a further
 * scheme is a one-line change; test-fix commit: the exact-scale amax is 8.0
 * for q4_0 and 31.0 for q6_0 (q6_0 divides by its largest magnitude 31).
 * Readings (the pages give neither the q8 divisor nor any 6-bit layout):
 *   divisor (largest magnitude): 8 (4-bit), 31 (6-bit), 127 (8-bit, as q8_0);
 *   codes clamp to the signed range [-2^(bits-1), 2^(bits-1) - 1];
 *   8-bit: code i is byte i of the group (two's complement);
 *   6-bit: 16 bytes of low nibbles laid out as the 4-bit codes, then 8 bytes
 *   of the high two bits, code 4j+i in bits 2i..2i+1 of byte j;
 *   a row is the codes of all groups, then the fp16 scales. */
static int kvqo_blk_group_bytes(int bits) { return bits == 4 ? 16 : (bits == 6 ? 24 : 32); }
static float kvqo_blk_divisor(int bits) { return bits == 4 ? 8.0f : (bits == 6 ? 31.0f : 127.0f); }

size_t kvqo_blk_row_bytes(int bits, int D) { return (size_t)(kvqo_blk_group_bytes(bits) * (D / 32) + 2 * (D / 32)); }

size_t kvqo_q4_row_bytes(int D) { return kvqo_blk_row_bytes(4, D); }

/* Encode one row of D values (D % 32 == 0).
 * [TF] "What it is": rotated groups of 32, 4-bit codes plus an fp16 scale;
 * [FT] PR description: 32 values -> 16 bytes + one fp16 scale;
 * [FT] test-fix commit: scale = amax/8 (4-bit), amax/31 (6-bit).
 * Returns KVQO_EDOMAIN for a non-finite value or a scale beyond fp16 range. */
int kvqo_blk_encode_row(int bits, const float* x, int D, uint8_t* row) {
    if (D <= 0 || D % 32) return KVQO_EARG;
    if (bits != 4 && bits != 6 && bits != 8) return KVQO_EARG;
    const int G = D / 32, GB = kvqo_blk_group_bytes(bits);
    const float qmax = (float)((1 << (bits - 1)) - 1), qmin = -(float)(1 << (bits - 1));
    uint8_t* scales = row + GB * G;
    for (int g = 0; g < G; ++g) {
        float t[32];
        for (int i = 0; i < 32; ++i) {
            t[i] = x[32 * g + i];
            if (!isfinite(t[i])) return KVQO_EDOMAIN;
        }
        kvqo_hadamard32_f32(t);
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i) {
            float a = fabsf(t[i]);
            if (a > amax) amax = a;
        }
        uint16_t s16 = kvqo_f32_to_f16(amax / kvqo_blk_divisor(bits));
        if ((s16 & 0x7C00u) == 0x7C00u) return KVQO_EDOMAIN;
        float s = kvqo_f16_to_f32(s16);
        int q[32];
        for (int i = 0; i < 32; ++i) {
            if (s == 0.0f) { q[i] = 0; continue; }
            float r = t[i] / s;           /* one correctly rounded fp32 divide */
            float n = nearbyintf(r);      /* half to even */
            if (n > qmax) n = qmax;
            if (n < qmin) n = qmin;
            q[i] = (int)n;
        }
        uint8_t* c = row + GB * g;
        if (bits == 8) {
            for (int i = 0; i < 32; ++i) c[i] = (uint8_t)(q[i] & 0xFF);
        } else {
            for (int k = 0; k < 16; ++k) c[k] = (uint8_t)((q[2 * k] & 0xF) | ((q[2 * k + 1] & 0xF) << 4));
            if (bits == 6)
                for (int j = 0; j < 8; ++j)
                    c[16 + j] = (uint8_t)(((q[4 * j] >> 4) & 3) | (((q[4 * j + 1] >> 4) & 3) << 2) |
                                          (((q[4 * j + 2] >> 4) & 3) << 4) | (((q[4 * j + 3] >> 4) & 3) << 6));
        }
        scales[2 * g] = (uint8_t)(s16 & 0xFF);
        scales[2 * g + 1] = (uint8_t)(s16 >> 8);
    }
    return KVQO_OK;
}

int kvqo_q4_encode_row(const float* x, int D, uint8_t* row) { return kvqo_blk_encode_row(4, x, D, row); }

/* Signed value of an n-bit two's-complement field v (0 <= v < 2^n). */
static int kvqo_signed(unsigned v, int n) { return (v & (1u << (n - 1))) ? (int)v - (1 << n) : (int)v; }

/* Dequantized row in the rotated domain: v_i = scale_g * code_i, exact in fp64. */
void kvqo_blk_decode_row(int bits, const uint8_t* row, int D, double* out) {
    const int G = D / 32, GB = kvqo_blk_group_bytes(bits);
    const uint8_t* scales = row + GB * G;
    for (int g = 0; g < G; ++g) {
        uint16_t s16 = (uint16_t)(scales[2 * g] | (scales[2 * g + 1] << 8));
        double s = (double)kvqo_f16_to_f32(s16);
        const uint8_t* c = row + GB * g;
        for (int i = 0; i < 32; ++i) {
            int code;
            if (bits == 8) {
                code = kvqo_signed(c[i], 8);
            } else {
                unsigned lo = (c[i / 2] >> (4 * (i & 1))) & 0xFu;
                if (bits == 4) code = kvqo_signed(lo, 4);
                else code = kvqo_signed(lo | (((c[16 + i / 4] >> (2 * (i & 3))) & 3u) << 4), 6);
            }
            out[32 * g + i] = s * code;
        }
    }
}

void kvqo_q4_decode_row(const uint8_t* row, int D, double* out) { kvqo_blk_decode_row(4, row, D, out); }

/* Byte offset of the row of (slot, kv head) in a pool laid out as
 * [num_pages][n_kv_heads][page_size][row_bytes]. */
static size_t kvqo_row_offset(int64_t slot, int head, int n_kv_heads, int page_size, size_t row_bytes) {
    int64_t page = slot / page_size, off = slot % page_size;
    return (size_t)(((page * n_kv_heads + head) * page_size + off) * (int64_t)row_bytes);
}

/* Write K and V rows of n_tokens tokens into paged pools of a block format.
 * k, v: [n_tokens][n_kv_heads][D] fp32.  slot < 0 skips the token. */
int kvqo_blk_store(int bits, uint8_t* k_pool, uint8_t* v_pool, int n_kv_heads, int D, int page_size,
                   int num_pages, const float* k, const float* v, const int64_t* slots, int n_tokens) {
    const size_t rb = kvqo_blk_row_bytes(bits, D);
    const int64_t n_slots = (int64_t)num_pages * page_size;
    int err = KVQO_OK;
    for (int t = 0; t < n_tokens; ++t)
        if (slots[t] >= n_slots) return KVQO_ERANGE;
#pragma omp parallel for schedule(static) reduction(min : err)
    for (int t = 0; t < n_tokens; ++t) {
        if (slots[t] < 0) continue;
        for (int h = 0; h < n_kv_heads; ++h) {
            size_t src = ((size_t)t * n_kv_heads + h) * D;
            size_t dst = kvqo_row_offset(slots[t], h, n_kv_heads, page_size, rb);
            int e1 = kvqo_blk_encode_row(bits, k + src, D, k_pool + dst);
            int e2 = kvqo_blk_encode_row(bits, v + src, D, v_pool + dst);
            if (e1 < err) err = e1;
            if (e2 < err) err = e2;
        }
    }
    return err;
}

int kvqo_q4_store(uint8_t* k_pool, uint8_t* v_pool, int n_kv_heads, int D, int page_size, int num_pages,
                  const float* k, const float* v, const int64_t* slots, int n_tokens) {
    return kvqo_blk_store(4, k_pool, v_pool, n_kv_heads, D, page_size, num_pages, k, v, slots, n_tokens);
}

/* ------------------------------------------------------------------ */
/* Decode attention over a block-format cache                          */
/* ------------------------------------------------------------------ */

/* Slot of logical position j of sequence b (16-token or other pages). */
static int64_t kvqo_slot(const int32_t* page_table, int max_pages, int b, int64_t j, int page_size) {
    return (int64_t)page_table[(int64_t)b * max_pages + j / page_size] * page_size + j % page_size;
}

/* Decode attention over the 4-bit cache, as the definition states it
 * ([TF] "What it is", decode rounds): q_rot = H q; for query head h of
 * sequence b, KV head g = h / (n_q_heads / n_kv_heads), T = seq_lens[b]:
 *   s_j = sm_scale * <q_rot, k_j>  over dequantized rotated keys, j < T
 *   p = softmax(s)                  (fp64, max subtracted)
 *   o = H * sum_j p_j v_j           (the output rotated back)
 *   lse = max_j s_j + log(sum_j exp(s_j - max))
 * T = 0 gives o = 0 and lse = -inf.  q: [B][n_q_heads][D] fp32, unrotated.
 * out: [B][n_q_heads][D], lse: [B][n_q_heads] (may be NULL). */
int kvqo_blk_attention(int bits, const uint8_t* k_pool, const uint8_t* v_pool, int n_kv_heads, int D,
                       int page_size, int num_pages, const float* q, int n_q_heads, const int32_t* page_table,
                       int max_pages, const int32_t* seq_lens, int B, double sm_scale, double* out, double* lse) {
    if (n_q_heads % n_kv_heads) return KVQO_EARG;
    const int G = n_q_heads / n_kv_heads;
    const size_t rb = kvqo_blk_row_bytes(bits, D);
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] < 0 || (int64_t)seq_lens[b] > (int64_t)max_pages * page_size) return KVQO_ERANGE;
    int err = KVQO_OK;
#pragma omp parallel for schedule(dynamic, 1) reduction(min : err)
    for (int bh = 0; bh < B * n_q_heads; ++bh) {
        const int b = bh / n_q_heads, h = bh % n_q_heads, g = h / G;
        const int64_t T = seq_lens[b];
        double* o = out + (size_t)bh * D;
        double* qd = malloc(sizeof(double) * D);
        double* qr = malloc(sizeof(double) * D);
        double* row = malloc(sizeof(double) * D);
        double* orot = calloc((size_t)D, sizeof(double));
        double* s = malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
        int st = KVQO_OK;
        for (int i = 0; i < D; ++i) qd[i] = q[(size_t)bh * D + i];
        kvqo_rotate_f64(qd, qr, D);
        double m = -INFINITY;
        for (int64_t j = 0; j < T; ++j) {
            int64_t slot = kvqo_slot(page_table, max_pages, b, j, page_size);
            if (slot < 0 || slot >= (int64_t)num_pages * page_size) { st = KVQO_ERANGE; break; }
            kvqo_blk_decode_row(bits, k_pool + kvqo_row_offset(slot, g, n_kv_heads, page_size, rb), D, row);
            double dot = 0.0;
            for (int i = 0; i < D; ++i) dot += qr[i] * row[i];
            s[j] = sm_scale * dot;
            if (s[j] > m) m = s[j];
        }
        double z = 0.0;
        if (st == KVQO_OK) {
            for (int64_t j = 0; j < T; ++j) {
                int64_t slot = kvqo_slot(page_table, max_pages, b, j, page_size);
                double w = exp(s[j] - m);
                z += w;
                kvqo_blk_decode_row(bits, v_pool + kvqo_row_offset(slot, g, n_kv_heads, page_size, rb), D, row);
                for (int i = 0; i < D; ++i) orot[i] += w * row[i];
            }
        }
        if (T > 0) {
            for (int i = 0; i < D; ++i) orot[i] /= z;
            kvqo_rotate_f64(orot, o, D);
        } else {
            for (int i = 0; i < D; ++i) o[i] = 0.0;
        }
        if (lse) lse[bh] = T > 0 ? m + log(z) : -INFINITY;
        if (st < err) err = st;
        free(qd); free(qr); free(row); free(orot); free(s);
    }
    return err;
}

int kvqo_q4_attention(const uint8_t* k_pool, const uint8_t* v_pool, int n_kv_heads, int D, int page_size,
                      int num_pages, const float* q, int n_q_heads, const int32_t* page_table, int max_pages,
                      const int32_t* seq_lens, int B, double sm_scale, double* out, double* lse) {
    return kvqo_blk_attention(4, k_pool, v_pool, n_kv_heads, D, page_size, num_pages, q, n_q_heads, page_table,
                              max_pages, seq_lens, B, sm_scale, out, lse);
}

/* The same attention in the method's own structure ([TF] "What it is":
 * chunks at absolute multiples of `chunk` keys, the last partial chunk being
 * the row's tail, merged in order; [CO] split-T commit: each chunk yields
 * (acc, m, z), combined by a log-sum-exp merge).  Per chunk c:
 *   m_c = max s_j, z_c = sum exp(s_j - m_c), acc_c = sum exp(s_j - m_c) v_j
 * (rotated domain, natural-log units of the scaled score); chunks past the
 * end of a sequence are empty: m = -inf, z = 0, acc = 0.  Merge, ascending c:
 *   M = max m_c, Z = sum z_c exp(m_c - M), o = H (sum acc_c exp(m_c - M)) / Z.
 * part_acc [B][n_q_heads][n_chunks][D], part_m/part_z [B][n_q_heads][n_chunks]
 * may be NULL; n_chunks = ceil(max(seq_lens) / chunk) when given. */
int kvqo_blk_attention_chunked(int bits, const uint8_t* k_pool, const uint8_t* v_pool, int n_kv_heads, int D,
                               int page_size, int num_pages, const float* q, int n_q_heads,
                               const int32_t* page_table, int max_pages, const int32_t* seq_lens, int B,
                               double sm_scale, int chunk, int n_chunks, double* part_acc, double* part_m,
                               double* part_z, double* out, double* lse) {
    if (n_q_heads % n_kv_heads || chunk <= 0) return KVQO_EARG;
    const int G = n_q_heads / n_kv_heads;
    const size_t rb = kvqo_blk_row_bytes(bits, D);
    for (int b = 0; b < B; ++b) {
        if (seq_lens[b] < 0 || (int64_t)seq_lens[b] > (int64_t)max_pages * page_size) return KVQO_ERANGE;
        if (((int64_t)seq_lens[b] + chunk - 1) / chunk > n_chunks) return KVQO_EARG;
    }
    int err = KVQO_OK;
#pragma omp parallel for schedule(dynamic, 1) reduction(min : err)
    for (int bh = 0; bh < B * n_q_heads; ++bh) {
        const int b = bh / n_q_heads, h = bh % n_q_heads, g = h / G;
        const int64_t T = seq_lens[b];
        double* qd = malloc(sizeof(double) * D);
        double* qr = malloc(sizeof(double) * D);
        double* row = malloc(sizeof(double) * D);
        double* acc = malloc(sizeof(double) * (size_t)n_chunks * D);
        double* cm = malloc(sizeof(double) * (size_t)n_chunks);
        double* cz = malloc(sizeof(double) * (size_t)n_chunks);
        double* s = malloc(sizeof(double) * (size_t)chunk);
        int st = KVQO_OK;
        for (int i = 0; i < D; ++i) qd[i] = q[(size_t)bh * D + i];
        kvqo_rotate_f64(qd, qr, D);
        for (int c = 0; c < n_chunks; ++c) {
            double* a = acc + (size_t)c * D;
            for (int i = 0; i < D; ++i) a[i] = 0.0;
            int64_t j0 = (int64_t)c * chunk, j1 = j0 + chunk < T ? j0 + chunk : T;
            double m = -INFINITY, z = 0.0;
            for (int64_t j = j0; j < j1; ++j) {
                int64_t slot = kvqo_slot(page_table, max_pages, b, j, page_size);
                if (slot < 0 || slot >= (int64_t)num_pages * page_size) { st = KVQO_ERANGE; j1 = j; break; }
                kvqo_blk_decode_row(bits, k_pool + kvqo_row_offset(slot, g, n_kv_heads, page_size, rb), D, row);
                double dot = 0.0;
                for (int i = 0; i < D; ++i) dot += qr[i] * row[i];
                s[j - j0] = sm_scale * dot;
                if (s[j - j0] > m) m = s[j - j0];
            }
            for (int64_t j = j0; j < j1; ++j) {
                int64_t slot = kvqo_slot(page_table, max_pages, b, j, page_size);
                double w = exp(s[j - j0] - m);
                z += w;
                kvqo_blk_decode_row(bits, v_pool + kvqo_row_offset(slot, g, n_kv_heads, page_size, rb), D, row);
                for (int i = 0; i < D; ++i) a[i] += w * row[i];
            }
            cm[c] = m;
            cz[c] = z;
        }
        double M = -INFINITY;
        for (int c = 0; c < n_chunks; ++c) if (cm[c] > M) M = cm[c];
        double Z = 0.0;
        double* orot = calloc((size_t)D, sizeof(double));
        if (M > -INFINITY) {
            for (int c = 0; c < n_chunks; ++c) {
                if (cz[c] == 0.0) continue;
                double f = exp(cm[c] - M);
                Z += cz[c] * f;
                for (int i = 0; i < D; ++i) orot[i] += acc[(size_t)c * D + i] * f;
            }
            for (int i = 0; i < D; ++i) orot[i] /= Z;
            kvqo_rotate_f64(orot, out + (size_t)bh * D, D);
        } else {
            for (int i = 0; i < D; ++i) out[(size_t)bh * D + i] = 0.0;
        }
        if (lse) lse[bh] = M > -INFINITY ? M + log(Z) : -INFINITY;
        if (part_m) for (int c = 0; c < n_chunks; ++c) part_m[(size_t)bh * n_chunks + c] = cm[c];
        if (part_z) for (int c = 0; c < n_chunks; ++c) part_z[(size_t)bh * n_chunks + c] = cz[c];
        if (part_acc) memcpy(part_acc + (size_t)bh * n_chunks * D, acc, sizeof(double) * (size_t)n_chunks * D);
        if (st < err) err = st;
        free(qd); free(qr); free(row); free(acc); free(cm); free(cz); free(s); free(orot);
    }
    return err;
}

int kvqo_q4_attention_chunked(const uint8_t* k_pool, const uint8_t* v_pool, int n_kv_heads, int D, int page_size,
                              int num_pages, const float* q, int n_q_heads, const int32_t* page_table,
                              int max_pages, const int32_t* seq_lens, int B, double sm_scale, int chunk,
                              int n_chunks, double* part_acc, double* part_m, double* part_z, double* out,
                              double* lse) {
    return kvqo_blk_attention_chunked(4, k_pool, v_pool, n_kv_heads, D, page_size, num_pages, q, n_q_heads,
                                      page_table, max_pages, seq_lens, B, sm_scale, chunk, n_chunks, part_acc,
                                      part_m, part_z, out, lse);
}

/* ------------------------------------------------------------------ */
/* fp8 e4m3 (OCP "fn": bias 7, max 448, 0x7F/0xFF are NaN)              */
/* ------------------------------------------------------------------ */

/* Value of an e4m3 code; the two NaN codes read as 0 ([CO] correctness
 * commit: the CPU table reads 0 for NaN codes). */
double kvqo_e4m3_decode(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return 0.0;
    double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* Nearest e4m3 code of v ([CO] KV8 commit: round to nearest even,
 * saturating at +-448, signed zero kept, NaN stored as 0).  The nearest
 * value is found as the nearest multiple of the binade's spacing. */
uint8_t kvqo_e4m3_encode(float v) {
    if (isnan(v)) return 0x00;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    if (a < ldexp(1.0, -6)) {
        /* subnormal binade: spacing 2^-9; n == 8 is the smallest normal 0x08 */
        double n = nearbyint(ldexp(a, 9));
        return (uint8_t)(sign | (uint8_t)n);
    }
    int e2;
    frexp(a, &e2);
    int E = e2 - 1;                         /* a in [2^E, 2^(E+1)), E in [-6, 8] */
    double n = nearbyint(ldexp(a, 3 - E));  /* in [8, 16] */
    if (n == 16.0) { n = 8.0; E += 1; }
    /* E + 7 <= 15 here; E + 7 == 15 with n - 8 == 7 would be 480, which the
     * a >= 448 test excludes (values in [448, 464] already returned). */
    return (uint8_t)(sign | (uint8_t)(((E + 7) << 3) | ((int)n - 8)));
}

/* One fp8 row part of n values -> n codes and an f32 scale ([CO] KV8 commit:
 * per-row f32 scale amax/448; codes = e4m3(x * (448/amax))). */
void kvqo_fp8_encode_part(const float* x, int n, uint8_t* codes, float* scale) {
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;          /* NaN compares false: ignored */
    }
    float inv = 448.0f / amax;
    if (amax == 0.0f || !isfinite(amax) || !isfinite(inv)) {
        for (int i = 0; i < n; ++i) codes[i] = 0x00;
        *scale = 0.0f;
        return;
    }
    for (int i = 0; i < n; ++i) codes[i] = kvqo_e4m3_encode(x[i] * inv);
    *scale = amax / 448.0f;
}

/* Store latent rows: x [n_tokens][D] with D = kv_lora + rope_dim.  Codes go
 * to codes_pool[slot][D], scales to scale_pool[slot][2] = {latent, rope}. */
int kvqo_fp8_store(uint8_t* codes_pool, float* scale_pool, int D, int rope_dim, int64_t n_slots,
                   const float* x, const int64_t* slots, int n_tokens) {
    if (rope_dim < 0 || rope_dim >= D) return KVQO_EARG;
    for (int t = 0; t < n_tokens; ++t)
        if (slots[t] >= n_slots) return KVQO_ERANGE;
    const int L = D - rope_dim;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < n_tokens; ++t) {
        if (slots[t] < 0) continue;
        const float* r = x + (size_t)t * D;
        uint8_t* c = codes_pool + (size_t)slots[t] * D;
        float* sc = scale_pool + (size_t)slots[t] * 2;
        kvqo_fp8_encode_part(r, L, c, &sc[0]);
        if (rope_dim > 0) kvqo_fp8_encode_part(r + L, rope_dim, c + L, &sc[1]);
        else sc[1] = 0.0f;
    }
    return KVQO_OK;
}

/* Absorbed latent attention over the fp8 cache ([CO] KV8 commit: the latent
 * is both key and value; split-T commit: the context cl[K]).  For head h of
 * sequence b, T = seq_lens[b], latent width L = D - rope_dim:
 *   s_j = sm_scale * (scL_j <qL_h, dec(Lc_j)> + scR_j <qR_h, dec(Rc_j)>)
 *   p = softmax(s), cl_h = sum_j p_j scL_j dec(Lc_j)
 * q: [B][n_heads][D] fp32; out: [B][n_heads][L]; lse: [B][n_heads]. */
int kvqo_mla_attention(const uint8_t* codes_pool, const float* scale_pool, int D, int rope_dim, int page_size,
                       int num_pages, const float* q, int n_heads, const int32_t* page_table, int max_pages,
                       const int32_t* seq_lens, int B, double sm_scale, double* out, double* lse) {
    const int L = D - rope_dim;
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] < 0 || (int64_t)seq_lens[b] > (int64_t)max_pages * page_size) return KVQO_ERANGE;
    int err = KVQO_OK;
#pragma omp parallel for schedule(dynamic, 1) reduction(min : err)
    for (int bh = 0; bh < B * n_heads; ++bh) {
        const int b = bh / n_heads;
        const int64_t T = seq_lens[b];
        const float* qh = q + (size_t)bh * D;
        double* o = out + (size_t)bh * L;
        double* s = malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
        int st = KVQO_OK;
        double m = -INFINITY;
        for (int64_t j = 0; j < T; ++j) {
            int64_t slot = kvqo_slot(page_table, max_pages, b, j, page_size);
            if (slot < 0 || slot >= (int64_t)num_pages * page_size) { st = KVQO_ERANGE; break; }
            const uint8_t* c = codes_pool + (size_t)slot * D;
            double dl = 0.0, dr = 0.0;
            for (int i = 0; i < L; ++i) dl += (double)qh[i] * kvqo_e4m3_decode(c[i]);
            for (int i = L; i < D; ++i) dr += (double)qh[i] * kvqo_e4m3_decode(c[i]);
            s[j] = sm_scale * ((double)scale_pool[2 * slot] * dl + (double)scale_pool[2 * slot + 1] * dr);
            if (s[j] > m) m = s[j];
        }
        for (int i = 0; i < L; ++i) o[i] = 0.0;
        double z = 0.0;
        if (st == KVQO_OK) {
            for (int64_t j = 0; j < T; ++j) {
                int64_t slot = kvqo_slot(page_table, max_pages, b, j, page_size);
                const uint8_t* c = codes_pool + (size_t)slot * D;
                double w = exp(s[j] - m);
                z += w;
                double ws = w * (double)scale_pool[2 * slot];
                for (int i = 0; i < L; ++i) o[i] += ws * kvqo_e4m3_decode(c[i]);
            }
        }
        if (T > 0) for (int i = 0; i < L; ++i) o[i] /= z;
        if (lse) lse[bh] = T > 0 ? m + log(z) : -INFINITY;
        if (st < err) err = st;
        free(s);
    }
    return err;
}

/* The latent attention split into chunks of `chunk` positions with partials
 * (acc, m, z) and the in-order log-sum-exp merge ([CO] split-T commit). */
int kvqo_mla_attention_chunked(const uint8_t* codes_pool, const float* scale_pool, int D, int rope_dim,
                               int page_size, int num_pages, const float* q, int n_heads,
                               const int32_t* page_table, int max_pages, const int32_t* seq_lens, int B,
                               double sm_scale, int chunk, int n_chunks, double* part_acc, double* part_m,
                               double* part_z, double* out, double* lse) {
    const int L = D - rope_dim;
    if (chunk <= 0) return KVQO_EARG;
    for (int b = 0; b < B; ++b) {
        if (seq_lens[b] < 0 || (int64_t)seq_lens[b] > (int64_t)max_pages * page_size) return KVQO_ERANGE;
        if (((int64_t)seq_lens[b] + chunk - 1) / chunk > n_chunks) return KVQO_EARG;
    }
    int err = KVQO_OK;
#pragma omp parallel for schedule(dynamic, 1) reduction(min : err)
    for (int bh = 0; bh < B * n_heads; ++bh) {
        const int b = bh / n_heads;
        const int64_t T = seq_lens[b];
        const float* qh = q + (size_t)bh * D;
        double* acc = calloc((size_t)n_chunks * L, sizeof(double));
        double* cm = malloc(sizeof(double) * (size_t)n_chunks);
        double* cz = malloc(sizeof(double) * (size_t)n_chunks);
        double* s = malloc(sizeof(double) * (size_t)chunk);
        int st = KVQO_OK;
        for (int c = 0; c < n_chunks; ++c) {
            int64_t j0 = (int64_t)c * chunk, j1 = j0 + chunk < T ? j0 + chunk : T;
            double m = -INFINITY, z = 0.0;
            for (int64_t j = j0; j < j1; ++j) {
                int64_t slot = kvqo_slot(page_table, max_pages, b, j, page_size);
                if (slot < 0 || slot >= (int64_t)num_pages * page_size) { st = KVQO_ERANGE; j1 = j; break; }
                const uint8_t* cc = codes_pool + (size_t)slot * D;
                double dl = 0.0, dr = 0.0;
                for (int i = 0; i < L; ++i) dl += (double)qh[i] * kvqo_e4m3_decode(cc[i]);
                for (int i = L; i < D; ++i) dr += (double)qh[i] * kvqo_e4m3_decode(cc[i]);
                s[j - j0] = sm_scale * ((double)scale_pool[2 * slot] * dl + (double)scale_pool[2 * slot + 1] * dr);
                if (s[j - j0] > m) m = s[j - j0];
            }
            double* a = acc + (size_t)c * L;
            for (int64_t j = j0; j < j1; ++j) {
                int64_t slot = kvqo_slot(page_table, max_pages, b, j, page_size);
                const uint8_t* cc = codes_pool + (size_t)slot * D;
                double w = exp(s[j - j0] - m);
                z += w;
                double ws = w * (double)scale_pool[2 * slot];
                for (int i = 0; i < L; ++i) a[i] += ws * kvqo_e4m3_decode(cc[i]);
            }
            cm[c] = m;
            cz[c] = z;
        }
        double M = -INFINITY, Z = 0.0;
        for (int c = 0; c < n_chunks; ++c) if (cm[c] > M) M = cm[c];
        double* o = out + (size_t)bh * L;
        for (int i = 0; i < L; ++i) o[i] = 0.0;
        if (M > -INFINITY) {
            for (int c = 0; c < n_chunks; ++c) {
                if (cz[c] == 0.0) continue;
                double f = exp(cm[c] - M);
                Z += cz[c] * f;
                for (int i = 0; i < L; ++i) o[i] += acc[(size_t)c * L + i] * f;
            }
            for (int i = 0; i < L; ++i) o[i] /= Z;
        }
        if (lse) lse[bh] = M > -INFINITY ? M + log(Z) : -INFINITY;
        if (part_m) for (int c = 0; c < n_chunks; ++c) part_m[(size_t)bh * n_chunks + c] = cm[c];
        if (part_z) for (int c = 0; c < n_chunks; ++c) part_z[(size_t)bh * n_chunks + c] = cz[c];
        if (part_acc) memcpy(part_acc + (size_t)bh * n_chunks * L, acc, sizeof(double) * (size_t)n_chunks * L);
        if (st < err) err = st;
        free(acc); free(cm); free(cz); free(s);
    }
    return err;
}

/* Latent attention over a selection of cached rows ([CO] split-T commit,
 * DSA gather: attend the selected rows, given as absolute positions).  For
 * sequence b the keys are the positions sel[b * max_sel + k], k < n_sel[b],
 * in list order; an entry outside [0, max_pages * page_size) -- e.g. the -1
 * that pads a fixed-size list -- is absent, and a position listed twice is
 * attended twice.  Per head, exactly the formula of kvqo_mla_attention over
 * those keys; no key gives out = 0 and lse = -inf. */
int kvqo_mla_attention_sel(const uint8_t* codes_pool, const float* scale_pool, int D, int rope_dim, int page_size,
                           int num_pages, const float* q, int n_heads, const int32_t* page_table, int max_pages,
                           const int32_t* sel, int max_sel, const int32_t* n_sel, int B, double sm_scale,
                           double* out, double* lse) {
    const int L = D - rope_dim;
    const int64_t cap = (int64_t)max_pages * page_size;
    for (int b = 0; b < B; ++b)
        if (n_sel[b] < 0 || n_sel[b] > max_sel) return KVQO_ERANGE;
    int err = KVQO_OK;
#pragma omp parallel for schedule(dynamic, 1) reduction(min : err)
    for (int bh = 0; bh < B * n_heads; ++bh) {
        const int b = bh / n_heads;
        const int n = n_sel[b];
        const int32_t* list = sel + (size_t)b * max_sel;
        const float* qh = q + (size_t)bh * D;
        double* o = out + (size_t)bh * L;
        double* s = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        int64_t* slots = malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
        int st = KVQO_OK, kept = 0;
        double m = -INFINITY;
        for (int k = 0; k < n; ++k) {
            slots[k] = -1;
            if (list[k] < 0 || (int64_t)list[k] >= cap) continue;  /* absent entry */
            int64_t slot = kvqo_slot(page_table, max_pages, b, list[k], page_size);
            if (slot < 0 || slot >= (int64_t)num_pages * page_size) { st = KVQO_ERANGE; break; }
            slots[k] = slot;
            const uint8_t* c = codes_pool + (size_t)slot * D;
            double dl = 0.0, dr = 0.0;
            for (int i = 0; i < L; ++i) dl += (double)qh[i] * kvqo_e4m3_decode(c[i]);
            for (int i = L; i < D; ++i) dr += (double)qh[i] * kvqo_e4m3_decode(c[i]);
            s[k] = sm_scale * ((double)scale_pool[2 * slot] * dl + (double)scale_pool[2 * slot + 1] * dr);
            if (s[k] > m) m = s[k];
            ++kept;
        }
        for (int i = 0; i < L; ++i) o[i] = 0.0;
        double z = 0.0;
        if (st == KVQO_OK && kept > 0) {
            for (int k = 0; k < n; ++k) {
                if (slots[k] < 0) continue;
                const uint8_t* c = codes_pool + (size_t)slots[k] * D;
                double w = exp(s[k] - m);
                z += w;
                double ws = w * (double)scale_pool[2 * slots[k]];
                for (int i = 0; i < L; ++i) o[i] += ws * kvqo_e4m3_decode(c[i]);
            }
            for (int i = 0; i < L; ++i) o[i] /= z;
        }
        if (lse) lse[bh] = kept > 0 ? m + log(z) : -INFINITY;
        if (st < err) err = st;
        free(s); free(slots);
    }
    return err;
}

/* Batch helpers for the tests: element-wise codecs over arrays. */
void kvqo_f32_to_f16_array(const float* x, uint16_t* y, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) y[i] = kvqo_f32_to_f16(x[i]);
}

void kvqo_e4m3_encode_array(const float* x, uint8_t* y, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) y[i] = kvqo_e4m3_encode(x[i]);
}

/* Encode/decode many rows at once: x [n_rows][D] -> rows [n_rows][row_bytes]. */
int kvqo_blk_encode_rows(int bits, const float* x, int64_t n_rows, int D, uint8_t* rows) {
    const size_t rb = kvqo_blk_row_bytes(bits, D);
    int err = KVQO_OK;
#pragma omp parallel for schedule(static) reduction(min : err)
    for (int64_t r = 0; r < n_rows; ++r) {
        int e = kvqo_blk_encode_row(bits, x + (size_t)r * D, D, rows + (size_t)r * rb);
        if (e < err) err = e;
    }
    return err;
}

void kvqo_blk_decode_rows(int bits, const uint8_t* rows, int64_t n_rows, int D, double* out) {
    const size_t rb = kvqo_blk_row_bytes(bits, D);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; ++r) kvqo_blk_decode_row(bits, rows + (size_t)r * rb, D, out + (size_t)r * D);
}

void kvqo_hadamard32_f32_rows(float* x, int64_t n_groups) {
    for (int64_t g = 0; g < n_groups; ++g) kvqo_hadamard32_f32(x + 32 * g);
}

/* ======================================================================
 * Rotated-int4 + Lloyd-Max codec for the latent ([CO] PR description and
 * Summary, "Why rotated-int4 for the 4-bit tier": a randomized-Hadamard
 * rotation, then a fixed 16-level Lloyd-Max codebook, optimal for N(0,1),
 * scaled by radius/sqrt(n); the rotation leaves the radius unchanged, so one
 * scale per row survives; a radius-0 row decodes to the zero vector).
 *
 * Readings of points the page leaves open:
 *   - each part of a latent row (the 512-wide latent, the 64-wide rope part)
 *     is coded on its own, with its own radius, as the fp8 rows keep two
 *     scales;
 *   - rotation of a part of n values: v_i = s_i * x_i with signs s_i = +-1,
 *     then the Sylvester butterfly in fp32 (stages h = 1, 2, ..., n/2), then
 *     one multiply by fp32(1/sqrt(n)); orthonormal, and its inverse is the
 *     butterfly, the multiply, then the signs;
 *   - signs: s_i = -1 where bit 63 of the i-th output of SplitMix64 (Steele,
 *     Lea and Flood, "Fast splittable pseudorandom number generators", 2014)
 *     is set, from seed 0x4C41544E ("LATN") for the latent part and
 *     0x524F5045 ("ROPE") for the rope part;
 *   - radius r = fp32(sqrt(S)), S the fp64 sum of the squared inputs taken as
 *     sums of 8 consecutive squares, those sums then added in order;
 *   - u_i = y_i * fp32(fp32(sqrt(n)) / r); code = the number of the 15
 *     fp32 thresholds (midpoints of neighbouring fp64 levels, rounded) that
 *     u_i exceeds (0..15, ties to the lower code); levels = Lloyd's iteration
 *     on N(0,1) run to convergence in fp64, made exactly symmetric (so the
 *     middle threshold is exactly 0), kept as fp32;
 *   - a row whose r is 0 or not finite, or whose sqrt(n)/r is not finite, is
 *     inert: radius 0 and every code 0;
 *   - codes are nibble-packed, element 2k low, 2k+1 high: a row is 256 code
 *     bytes of the latent part, then 32 of the rope part (288 bytes), and
 *     its two radii are kept as f32 [slot][2].
 * ====================================================================== */

#define KVQO_TQ_LEVELS 16

static uint64_t kvqo_splitmix64_next(uint64_t* state) {
    uint64_t z = (*state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* First n outputs of SplitMix64 from `seed` (exposed for its known-answer test). */
void kvqo_splitmix64(uint64_t seed, int n, uint64_t* out) {
    uint64_t s = seed;
    for (int i = 0; i < n; ++i) out[i] = kvqo_splitmix64_next(&s);
}

static uint64_t kvqo_tq_seed(int part) { return part == 0 ? 0x4C41544Eull : 0x524F5045ull; }

/* Signs of a part: +1 or -1 as floats. */
void kvqo_tq_signs(int part, int n, float* sig) {
    uint64_t s = kvqo_tq_seed(part);
    for (int i = 0; i < n; ++i) sig[i] = (kvqo_splitmix64_next(&s) >> 63) ? -1.0f : 1.0f;
}

static double kvqo_npdf(double x) { return exp(-0.5 * x * x) / sqrt(2.0 * 3.14159265358979323846); }
static double kvqo_ncdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

/* Lloyd-Max quantizer of N(0,1) with `nlev` levels: alternate the two
 * optimality conditions (thresholds at midpoints of neighbouring levels;
 * each level the mean of N(0,1) over its cell, (pdf(a) - pdf(b)) /
 * (cdf(b) - cdf(a))) from evenly spaced levels until no level moves by more
 * than 1e-15.  Returns the number of iterations; lev ascending. */
int kvqo_lloyd_max_gauss(int nlev, double* lev) {
    for (int k = 0; k < nlev; ++k) lev[k] = -3.0 + 6.0 * (k + 0.5) / nlev;
    int it = 0;
    for (; it < 100000; ++it) {
        double move = 0.0;
        double prev_t = -INFINITY;
        double nl[64];
        for (int k = 0; k < nlev; ++k) {
            const double t = k + 1 < nlev ? 0.5 * (lev[k] + lev[k + 1]) : INFINITY;
            const double pa = isinf(prev_t) ? 0.0 : kvqo_npdf(prev_t), pb = isinf(t) ? 0.0 : kvqo_npdf(t);
            const double ca = isinf(prev_t) ? 0.0 : kvqo_ncdf(prev_t), cb = isinf(t) ? 1.0 : kvqo_ncdf(t);
            nl[k] = (pa - pb) / (cb - ca);
            prev_t = t;
        }
        for (int k = 0; k < nlev; ++k) {
            const double d = fabs(nl[k] - lev[k]);
            if (d > move) move = d;
            lev[k] = nl[k];
        }
        if (move <= 1e-15) break;
    }
    /* N(0,1) is symmetric: make the levels exactly so (the middle threshold
     * is then exactly 0), averaging the two magnitudes of each pair. */
    for (int k = 0; k < nlev / 2; ++k) {
        const double a = 0.5 * (lev[nlev - 1 - k] - lev[k]);
        lev[k] = -a;
        lev[nlev - 1 - k] = a;
    }
    return it;
}

/* The codec's tables: fp32 levels and the 15 fp32 thresholds (computed once). */
void kvqo_tq_tables(float* lev32, float* thr32) {
    static float s_lev[KVQO_TQ_LEVELS], s_thr[KVQO_TQ_LEVELS - 1];
    static int s_done = 0;
#pragma omp critical(kvqo_tq_tables)
    {
        if (!s_done) {
            double lev[KVQO_TQ_LEVELS];
            kvqo_lloyd_max_gauss(KVQO_TQ_LEVELS, lev);
            for (int k = 0; k < KVQO_TQ_LEVELS; ++k) s_lev[k] = (float)lev[k];
            for (int k = 0; k + 1 < KVQO_TQ_LEVELS; ++k) s_thr[k] = (float)(0.5 * (lev[k] + lev[k + 1]));
            s_done = 1;
        }
    }
    memcpy(lev32, s_lev, sizeof(s_lev));
    memcpy(thr32, s_thr, sizeof(s_thr));
}

/* Code of one rotated, normalized value: how many thresholds it exceeds. */
static int kvqo_tq_code(float u, const float* thr32) {
    int q = 0;
    for (int k = 0; k + 1 < KVQO_TQ_LEVELS; ++k) q += u > thr32[k];
    return q;
}

void kvqo_tq_quantize(const float* u, int n, uint8_t* codes) {
    float lev32[KVQO_TQ_LEVELS], thr32[KVQO_TQ_LEVELS - 1];
    kvqo_tq_tables(lev32, thr32);
    for (int i = 0; i < n; ++i) codes[i] = (uint8_t)kvqo_tq_code(u[i], thr32);
}

/* The forward rotation of a part (n a power of two), fp32, in place. */
void kvqo_tq_rotate_f32(float* v, int n, int part) {
    float sig[512];
    kvqo_tq_signs(part, n, sig);
    for (int i = 0; i < n; ++i) v[i] = v[i] * sig[i];
    for (int h = 1; h < n; h <<= 1)
        for (int i = 0; i < n; ++i)
            if ((i & h) == 0) {
                const float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
    const float c = (float)(1.0 / sqrt((double)n));
    for (int i = 0; i < n; ++i) v[i] = v[i] * c;
}

/* Inverse rotation of a part in fp64 (the butterfly, 1/sqrt(n), the signs). */
void kvqo_tq_unrotate_f64(double* v, int n, int part) {
    float sig[512];
    kvqo_tq_signs(part, n, sig);
    for (int h = 1; h < n; h <<= 1)
        for (int i = 0; i < n; ++i)
            if ((i & h) == 0) {
                const double a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
    const double c = 1.0 / sqrt((double)n);
    for (int i = 0; i < n; ++i) v[i] = v[i] * c * (double)sig[i];
}

/* Encode one part of n values (n = 512 or 64) -> n/2 code bytes, radius. */
void kvqo_tq_encode_part(const float* x, int n, int part, uint8_t* bytes, float* radius) {
    double S = 0.0;
    for (int b = 0; b < n; b += 8) {
        double s8 = 0.0;
        for (int i = b; i < b + 8; ++i) s8 += (double)x[i] * (double)x[i];
        S += s8;
    }
    const float r = (float)sqrt(S);
    const float kn = (float)sqrt((double)n);
    const float inv = kn / r;
    if (!(r > 0.0f) || !isfinite(r) || !isfinite(inv)) {
        memset(bytes, 0, (size_t)n / 2);
        *radius = 0.0f;
        return;
    }
    float y[512];
    memcpy(y, x, sizeof(float) * (size_t)n);
    kvqo_tq_rotate_f32(y, n, part);
    float lev32[KVQO_TQ_LEVELS], thr32[KVQO_TQ_LEVELS - 1];
    kvqo_tq_tables(lev32, thr32);
    for (int k = 0; k < n / 2; ++k) {
        const int q0 = kvqo_tq_code(y[2 * k] * inv, thr32), q1 = kvqo_tq_code(y[2 * k + 1] * inv, thr32);
        bytes[k] = (uint8_t)(q0 | (q1 << 4));
    }
    *radius = r;
}

/* Dequantize one part to the unrotated fp64 values. */
void kvqo_tq_decode_part(const uint8_t* bytes, float radius, int n, int part, double* out) {
    float lev32[KVQO_TQ_LEVELS], thr32[KVQO_TQ_LEVELS - 1];
    kvqo_tq_tables(lev32, thr32);
    const double sc = (double)radius / sqrt((double)n);
    for (int i = 0; i < n; ++i) {
        const int q = (bytes[i / 2] >> (4 * (i & 1))) & 15;
        out[i] = (double)lev32[q] * sc;
    }
    kvqo_tq_unrotate_f64(out, n, part);
}

/* Store latent rows x [n_tokens][576] (512 latent + 64 rope) into
 * codes_pool [slot][288] and radius_pool [slot][2]; slot < 0 skips. */
int kvqo_tq_store(uint8_t* codes_pool, float* radius_pool, int64_t n_slots, const float* x,
                  const int64_t* slots, int n_tokens) {
    for (int t = 0; t < n_tokens; ++t)
        if (slots[t] >= n_slots) return KVQO_ERANGE;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < n_tokens; ++t) {
        if (slots[t] < 0) continue;
        const float* r = x + (size_t)t * 576;
        uint8_t* c = codes_pool + (size_t)slots[t] * 288;
        float* rad = radius_pool + (size_t)slots[t] * 2;
        kvqo_tq_encode_part(r, 512, 0, c, &rad[0]);
        kvqo_tq_encode_part(r + 512, 64, 1, c + 256, &rad[1]);
    }
    return KVQO_OK;
}

/* Decode rows of the pool: out [n][576] fp64 (unrotated). */
void kvqo_tq_decode_rows(const uint8_t* codes_pool, const float* radius_pool, int64_t n, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        kvqo_tq_decode_part(codes_pool + (size_t)j * 288, radius_pool[2 * j], 512, 0, out + (size_t)j * 576);
        kvqo_tq_decode_part(codes_pool + (size_t)j * 288 + 256, radius_pool[2 * j + 1], 64, 1,
                            out + (size_t)j * 576 + 512);
    }
}

/* Absorbed latent attention over the TQ4 cache, by its definition: every
 * position's latent row is dequantized and rotated back (fp64), then
 *   s_j = sm_scale * <q_h, x_j> over all 576 values, p = softmax(s),
 *   cl_h = sum_j p_j x_j[0:512];
 * q: [B][n_heads][576] fp32; out: [B][n_heads][512]; lse: [B][n_heads]. */
int kvqo_tq_attention(const uint8_t* codes_pool, const float* radius_pool, int page_size, int num_pages,
                      const float* q, int n_heads, const int32_t* page_table, int max_pages,
                      const int32_t* seq_lens, int B, double sm_scale, double* out, double* lse) {
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] < 0 || (int64_t)seq_lens[b] > (int64_t)max_pages * page_size) return KVQO_ERANGE;
    int err = KVQO_OK;
    for (int b = 0; b < B; ++b) {
        const int64_t T = seq_lens[b];
        double* rows = malloc(sizeof(double) * 576 * (size_t)(T > 0 ? T : 1));
        int st = KVQO_OK;
        for (int64_t j = 0; j < T && st == KVQO_OK; ++j) {
            const int64_t slot = kvqo_slot(page_table, max_pages, b, j, page_size);
            if (slot < 0 || slot >= (int64_t)num_pages * page_size) { st = KVQO_ERANGE; break; }
            kvqo_tq_decode_rows(codes_pool + (size_t)slot * 288, radius_pool + 2 * slot, 1, rows + (size_t)j * 576);
        }
#pragma omp parallel for schedule(dynamic, 1)
        for (int h = 0; h < n_heads; ++h) {
            const float* qh = q + ((size_t)b * n_heads + h) * 576;
            double* o = out + ((size_t)b * n_heads + h) * 512;
            double* s = malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
            double m = -INFINITY;
            for (int64_t j = 0; j < T && st == KVQO_OK; ++j) {
                double d = 0.0;
                for (int i = 0; i < 576; ++i) d += (double)qh[i] * rows[(size_t)j * 576 + i];
                s[j] = sm_scale * d;
                if (s[j] > m) m = s[j];
            }
            for (int i = 0; i < 512; ++i) o[i] = 0.0;
            double z = 0.0;
            if (st == KVQO_OK)
                for (int64_t j = 0; j < T; ++j) {
                    const double w = exp(s[j] - m);
                    z += w;
                    for (int i = 0; i < 512; ++i) o[i] += w * rows[(size_t)j * 576 + i];
                }
            if (T > 0) for (int i = 0; i < 512; ++i) o[i] /= z;
            if (lse) lse[(size_t)b * n_heads + h] = T > 0 ? m + log(z) : -INFINITY;
            free(s);
        }
        if (st < err) err = st;
        free(rows);
    }
    return err;
}
