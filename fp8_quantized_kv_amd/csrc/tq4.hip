// tq4.hip -- the rotated-int4 + Lloyd-Max codec for the MLA latent (TQ4):
// store (rotate, radius, quantize, pack) and a plain split-T decode.
//
// Method: colibri pull request "KV cache quantization: fp8 (KV8) + 4-bit
// TurboQuant (KV_TQ)", Summary "Why rotated-int4 for the 4-bit tier": a
// randomized Hadamard rotation, then a fixed 16-level Lloyd-Max codebook
// optimal for N(0,1), scaled by radius/sqrt(n); the rotation keeps the
// radius, so one scale per row part survives; a radius-0 row decodes to 0.
// The latent is both key and value (absorbed attention, KV8 commit), and
// the split-T partials (cl[K], m, z) are merged by the log-sum-exp kernel.
//
// Format (per position): the 512-wide latent part and the 64-wide rope part
// are each rotated and coded apart: v = s (.) x with signs s_i = -1 where bit
// 63 of the i-th SplitMix64 output (Steele, Lea and Flood 2014) from the
// part's seed is set, the Sylvester butterfly in fp32 (stages h = 1 .. n/2),
// times fp32(1/sqrt(n)).  Radius r = fp32(sqrt(S)), S the fp64 sum of the
// squared inputs as sums of 8 consecutive squares added in order.  Code =
// how many of the 15 fp32 thresholds y_i * fp32(fp32(sqrt(n)) / r) exceeds.
// Nibbles packed element 2k low, 2k + 1 high: 256 + 32 bytes per position;
// radii f32 [slot][2].  A zero, NaN or infinite row is stored inert (radius
// 0, codes 0).
//
// Attention runs in rotated space, as for the 4-bit cache ("rotate the
// queries once ... rotate the output back once"): the query rows are rotated
// by tq_rotate_rows (kvq_tq_rotate), the decode scores and accumulates
// against levels x radius/sqrt(n), the partials and their merge are those of
// the fp8 latent cache, and the merged 512-wide context is rotated back by
// tq_rotate_rows (inverse).  The decode here is the plain fp32 kernel, for
// the shapes the matrix-core kernel (decode_fp8_mfma.hip) does not take.
#include "internal.h"

#include <cmath>

namespace kvq {

namespace {

// ---- codebook: Lloyd's iteration on the positive half of N(0,1) ----------
// Levels c_0 < .. < c_7 > 0 (the negative half mirrors them); cell k is
// (t_k, t_k+1) with t_0 = 0, t_k = (c_k-1 + c_k) / 2, t_8 = inf; each level
// moves to the mean of N(0,1) over its cell, (pdf(a) - pdf(b)) / (Q(a) -
// Q(b)) with Q the upper tail, until no level moves by more than 1e-15.
double npdf(double x) { return std::exp(-0.5 * x * x) * 0.39894228040143267794; }
double upper_tail(double x) { return 0.5 * std::erfc(x * 0.70710678118654752440); }

TqTables make_tables() {
    double c[8];
    for (int k = 0; k < 8; ++k) c[k] = 0.35 * (k + 0.5);
    for (int it = 0; it < 100000; ++it) {
        double t[9];
        t[0] = 0.0;
        for (int k = 1; k < 8; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
        t[8] = INFINITY;
        double move = 0.0;
        for (int k = 0; k < 8; ++k) {
            const double a = t[k], b = t[k + 1];
            const double num = npdf(a) - (std::isinf(b) ? 0.0 : npdf(b));
            const double den = upper_tail(a) - (std::isinf(b) ? 0.0 : upper_tail(b));
            const double nc = num / den;
            move = std::fmax(move, std::fabs(nc - c[k]));
            c[k] = nc;
        }
        if (move <= 1e-15) break;
    }
    TqTables tb;
    for (int k = 0; k < 8; ++k) {
        tb.lev[8 + k] = float(c[k]);
        tb.lev[7 - k] = -float(c[k]);
    }
    tb.thr[7] = 0.0f;
    for (int k = 0; k < 7; ++k) {
        tb.thr[8 + k] = float(0.5 * (c[k] + c[k + 1]));
        tb.thr[6 - k] = -tb.thr[8 + k];
    }
    return tb;
}

constexpr uint64_t kSeedLatent = 0x4C41544Eull, kSeedRope = 0x524F5045ull;

__device__ __forceinline__ int clamp_int(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Sign of element i of a part: bit 63 of SplitMix64 output i (counter-based:
// output i mixes seed + (i + 1) * golden gamma).
__device__ __forceinline__ float tq_sign(uint64_t seed, int i) {
    uint64_t z = seed + uint64_t(i + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (z >> 63) ? -1.0f : 1.0f;
}

template <InType DT>
__device__ __forceinline__ float load_x(const void* x, int64_t i) {
    if constexpr (DT == InType::F32) return static_cast<const float*>(x)[i];
    else if constexpr (DT == InType::BF16) return __uint_as_float(uint32_t(static_cast<const uint16_t*>(x)[i]) << 16);
    else return __half2float(static_cast<const __half*>(x)[i]);
}

// ---- store: one wave per token; lane l holds elements 8l .. 8l + 7 -------
// The butterfly stages below 8 run inside a lane, the others between lanes
// (partner lane l ^ (h / 8)); each stage is (a + b, a - b) with a the element
// whose index has bit h clear, in fp32, as the format states.
template <int N>
__device__ __forceinline__ void encode_part(float (&v)[8], int lane, uint64_t seed, const TqTables& tb,
                                            double* red, uint8_t* out, float* radius) {
    constexpr int LANES = N / 8;
    const bool on = lane < LANES;
    // radius: per-lane sums of 8 squares (fp64), then added in lane order
    double s8 = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) s8 += double(v[e]) * double(v[e]);
    if (on) red[lane] = s8;
    __syncthreads();
    double S = 0.0;
    for (int l = 0; l < LANES; ++l) S += red[l];
    __syncthreads();
    const float r = float(std::sqrt(S));
    const float inv = float(std::sqrt(double(N))) / r;
    const bool inert = !(r > 0.0f) || !isfinite(r) || !isfinite(inv);
    // rotation
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = v[e] * tq_sign(seed, 8 * lane + e);
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if ((e & h) == 0) {
                const float a = v[e], b = v[e + h];
                v[e] = a + b;
                v[e + h] = a - b;
            }
#pragma unroll
    for (int hl = 1; hl < LANES; hl <<= 1) {
        const bool low = (lane & hl) == 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float o = __shfl_xor(v[e], hl, 64);
            v[e] = low ? v[e] + o : o - v[e];
        }
    }
    const float c = float(1.0 / std::sqrt(double(N)));
    uint32_t word = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float u = (v[e] * c) * inv;
        uint32_t q = 0u;
#pragma unroll
        for (int k = 0; k < 15; ++k) q += u > tb.thr[k] ? 1u : 0u;
        word |= (inert ? 0u : q) << (4 * e);
    }
    if (on) reinterpret_cast<uint32_t*>(out)[lane] = word;
    if (lane == 0) *radius = inert ? 0.0f : r;
}

// Token t of x into its slot (one wave; a skipped slot is uniform over it).
template <InType DT>
__device__ __forceinline__ void store_token(const void* __restrict__ x, const int64_t* __restrict__ slots, int t,
                                            int lane, uint8_t* __restrict__ codes, float* __restrict__ radii,
                                            int64_t n_slots, const TqTables& tb, double* red) {
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= n_slots) return;
    const int64_t base = int64_t(t) * 576;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = load_x<DT>(x, base + 8 * lane + e);
    encode_part<512>(v, lane, kSeedLatent, tb, red, codes + slot * 288, radii + slot * 2);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = lane < 8 ? load_x<DT>(x, base + 512 + 8 * lane + e) : 0.0f;
    encode_part<64>(v, lane, kSeedRope, tb, red, codes + slot * 288 + 256, radii + slot * 2 + 1);
}

template <InType DT>
__global__ __launch_bounds__(64) void store_tq4_kernel(const void* __restrict__ x, const int64_t* __restrict__ slots,
                                                       int n_tokens, uint8_t* __restrict__ codes,
                                                       float* __restrict__ radii, int64_t n_slots, TqTables tb) {
    __shared__ double red[64];
    store_token<DT>(x, slots, blockIdx.x, threadIdx.x, codes, radii, n_slots, tb, red);
}

// ---- decode: plain fp32, split-T --------------------------------------------
constexpr int kTT = 256;     // threads
constexpr int kTHB = 16;     // heads per workgroup
constexpr int kTTile = 16;   // keys per tile
constexpr int kTL = 512, kTR = 64, kTD = 576;

// Rotation of rows by one wave each (kvq_tq_rotate): row_len 576 (a query:
// both parts) or 512 (a context: the latent part).  Forward: signs, the
// butterfly, 1/sqrt(n); inverse: the butterfly, 1/sqrt(n), the signs.  Lane
// l holds elements 8l .. 8l + 7 of the 512-wide part and lanes 0..7 those of
// the 64-wide part, as in the store.
template <int N>
__device__ __forceinline__ void rotate_part(float (&v)[8], int lane, uint64_t seed, bool inverse) {
    constexpr int LANES = N / 8;
    if (!inverse) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = v[e] * tq_sign(seed, 8 * lane + e);
    }
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if ((e & h) == 0) {
                const float a = v[e], b = v[e + h];
                v[e] = a + b;
                v[e + h] = a - b;
            }
#pragma unroll
    for (int hl = 1; hl < LANES; hl <<= 1) {
        const bool low = (lane & hl) == 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float o = __shfl_xor(v[e], hl, 64);
            v[e] = low ? v[e] + o : o - v[e];
        }
    }
    const float c = float(1.0 / std::sqrt(double(N)));
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = inverse ? (v[e] * c) * tq_sign(seed, 8 * lane + e) : v[e] * c;
}

// Row r of x (row_len 576: both parts; 512: the latent part) into y.
__device__ __forceinline__ void rotate_row(const float* __restrict__ x, float* __restrict__ y, int64_t r, int row_len,
                                           bool inverse, int lane) {
    const float* xr = x + r * row_len;
    float* yr = y + r * row_len;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = xr[8 * lane + e];
    rotate_part<kTL>(v, lane, kSeedLatent, inverse);
#pragma unroll
    for (int e = 0; e < 8; ++e) yr[8 * lane + e] = v[e];
    if (row_len == kTD) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = lane < 8 ? xr[kTL + 8 * lane + e] : 0.0f;
        rotate_part<kTR>(v, lane, kSeedRope, inverse);
        if (lane < 8) {
#pragma unroll
            for (int e = 0; e < 8; ++e) yr[kTL + 8 * lane + e] = v[e];
        }
    }
}

__global__ __launch_bounds__(64) void tq_rotate_rows(const float* __restrict__ x, float* __restrict__ y, int64_t n_rows,
                                                     int row_len, int inverse) {
    if (int64_t(blockIdx.x) >= n_rows) return;
    rotate_row(x, y, blockIdx.x, row_len, inverse != 0, threadIdx.x);
}

// The step's store and the query rotation in one launch (kvq_store_rotate_q
// on a TQ4 cache): workgroups 0 .. n_tokens - 1 store a token each, the rest
// rotate a query row each; the two sets touch disjoint memory.
template <InType DT>
__global__ __launch_bounds__(64) void store_rotate_tq4_kernel(const void* __restrict__ x,
                                                              const int64_t* __restrict__ slots, int n_tokens,
                                                              uint8_t* __restrict__ codes, float* __restrict__ radii,
                                                              int64_t n_slots, TqTables tb, const float* __restrict__ q,
                                                              float* __restrict__ q_rot, int n_rows) {
    __shared__ double red[64];
    const int b = blockIdx.x;
    if (b < n_tokens)
        store_token<DT>(x, slots, b, threadIdx.x, codes, radii, n_slots, tb, red);
    else if (b - n_tokens < n_rows)
        rotate_row(q, q_rot, b - n_tokens, kTD, false, threadIdx.x);
}

__global__ __launch_bounds__(kTT) void decode_tq4_simple(const uint8_t* __restrict__ codes,
                                                         const float* __restrict__ radii, int page_size,
                                                         int num_pages, DecodeArgs a, TqTables tb) {
    constexpr int DW = 288 / 4;  // code words per row
    constexpr int CPT = kTL / kTT;
    const int s = blockIdx.x, hblk = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int h0 = hblk * kTHB;
    const int nh = min(kTHB, a.n_q_heads - h0);
    const int T = clamp_int(a.seq_lens[b], 0, a.max_seq_len);
    const int j0 = s * a.split_keys;
    const int j1 = min(j0 + a.split_keys, T);
    const int64_t hb = int64_t(b) * a.n_q_heads + h0;
    const int S = a.n_splits;

    if (j0 >= j1) {
        for (int i = tid; i < nh * kTL; i += kTT) a.part_acc[((hb + i / kTL) * S + s) * kTL + i % kTL] = 0.0f;
        if (tid < nh) {
            a.part_m[(hb + tid) * S + s] = -INFINITY;
            a.part_z[(hb + tid) * S + s] = 0.0f;
        }
        return;
    }

    __shared__ float qs[kTHB][kTD];
    __shared__ uint32_t ct[kTTile * DW];
    __shared__ float scl[kTTile], scr[kTTile];
    __shared__ float part[16][kTHB][kTTile];
    __shared__ float p[kTHB][kTTile];
    __shared__ float m_s[kTHB], z_s[kTHB], alpha_s[kTHB];
    __shared__ float lev[16];

    if (tid < 16) lev[tid] = tb.lev[tid];
    for (int i = tid; i < kTHB * kTD; i += kTT) {
        const int h = i / kTD;
        qs[h][i % kTD] = h < nh ? a.q[(hb + h) * kTD + i % kTD] : 0.0f;
    }
    if (tid < kTHB) {
        m_s[tid] = -INFINITY;
        z_s[tid] = 0.0f;
    }
    __syncthreads();
    // the (rotated) query, pre-scaled by sm_scale * log2(e)
    const float qscale = a.sm_scale * kLog2e;
    for (int i = tid; i < kTHB * kTD; i += kTT) qs[i / kTD][i % kTD] *= qscale;

    float acc[CPT][kTHB];
#pragma unroll
    for (int ci = 0; ci < CPT; ++ci)
#pragma unroll
        for (int h = 0; h < kTHB; ++h) acc[ci][h] = 0.0f;
    __syncthreads();

    const float cL = float(1.0 / std::sqrt(512.0)), cR = 0.125f;
    const int32_t* pt = a.page_table + int64_t(b) * a.max_pages;
    auto code_at = [&](int kk, int c) -> float {  // level of element c (0..575) of tile row kk
        const int byte = c < kTL ? c / 2 : 256 + (c - kTL) / 2;
        const uint32_t w = ct[kk * DW + byte / 4];
        return lev[(w >> (8 * (byte & 3) + 4 * (c & 1))) & 15u];
    };
    for (int t0 = j0; t0 < j1; t0 += kTTile) {
        const int n = min(kTTile, j1 - t0);
        for (int i = tid; i < n * DW; i += kTT) {
            const int kk = i / DW, w = i % DW;
            const int pos = t0 + kk;
            const int page = clamp_int(pt[pos / page_size], 0, num_pages - 1);
            const int64_t slot = int64_t(page) * page_size + pos % page_size;
            ct[i] = reinterpret_cast<const uint32_t*>(codes + slot * 288)[w];
        }
        if (tid < n) {
            const int pos = t0 + tid;
            const int page = clamp_int(pt[pos / page_size], 0, num_pages - 1);
            const int64_t slot = int64_t(page) * page_size + pos % page_size;
            scl[tid] = radii[slot * 2] * cL;
            scr[tid] = radii[slot * 2 + 1] * cR;
        }
        __syncthreads();
        {
            // thread (key kk, part_i): latent channels 32 part_i .. +31, rope 4 part_i .. +3
            const int kk = tid & (kTTile - 1), part_i = tid / kTTile;
            float dl[kTHB], dr[kTHB];
#pragma unroll
            for (int h = 0; h < kTHB; ++h) dl[h] = dr[h] = 0.0f;
            if (kk < n) {
                for (int c = 32 * part_i; c < 32 * part_i + 32; ++c) {
                    const float v = code_at(kk, c);
#pragma unroll
                    for (int h = 0; h < kTHB; ++h) dl[h] = fmaf(qs[h][c], v, dl[h]);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = kTL + 4 * part_i + e;
                    const float v = code_at(kk, c);
#pragma unroll
                    for (int h = 0; h < kTHB; ++h) dr[h] = fmaf(qs[h][c], v, dr[h]);
                }
            }
            const float sl = kk < n ? scl[kk] : 0.0f, sr = kk < n ? scr[kk] : 0.0f;
#pragma unroll
            for (int h = 0; h < kTHB; ++h) part[part_i][h][kk] = fmaf(sl, dl[h], sr * dr[h]);
        }
        __syncthreads();
        {
            const int wave = tid >> 6, lane = tid & 63;
            const int h = wave * 4 + (lane >> 4), kk = lane & 15;
            float sc = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) sc += part[i][h][kk];
            sc = kk < n ? sc : -INFINITY;
            float tmax = sc;
#pragma unroll
            for (int m = 8; m >= 1; m >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, m, 64));
            const float m_old = m_s[h];
            const float m_new = fmaxf(m_old, tmax);
            const float e = kk < n ? exp2f(sc - m_new) : 0.0f;
            float sum = e;
#pragma unroll
            for (int m = 8; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, 64);
            p[h][kk] = e * (kk < n ? scl[kk] : 0.0f);  // the value is level x radius / sqrt(512)
            __syncthreads();  // every lane has read m_s[h] before lane 0 of the head writes it
            if (kk == 0) {
                const float al = exp2f(m_old - m_new);
                alpha_s[h] = al;
                z_s[h] = z_s[h] * al + sum;
                m_s[h] = m_new;
            }
        }
        __syncthreads();
#pragma unroll
        for (int ci = 0; ci < CPT; ++ci) {
            const int c = tid + ci * kTT;
#pragma unroll
            for (int h = 0; h < kTHB; ++h) acc[ci][h] *= alpha_s[h];
            for (int kk = 0; kk < n; ++kk) {
                const float v = code_at(kk, c);
#pragma unroll
                for (int h = 0; h < kTHB; ++h) acc[ci][h] = fmaf(p[h][kk], v, acc[ci][h]);
            }
        }
        __syncthreads();
    }
    // the split's context, in rotated space
#pragma unroll
    for (int ci = 0; ci < CPT; ++ci)
#pragma unroll
        for (int h = 0; h < kTHB; ++h)
            if (h < nh) a.part_acc[((hb + h) * S + s) * kTL + tid + ci * kTT] = acc[ci][h];
    if (tid < nh) {
        a.part_m[(hb + tid) * S + s] = m_s[tid] * kLn2;
        a.part_z[(hb + tid) * S + s] = z_s[tid];
    }
}

// ---- merge + inverse rotation in one launch ------------------------------
// The log-sum-exp merge of the split-T partials (colibri pull request,
// split-T commit) followed by rotating the merged latent context back
// ("rotate the output back once"), for one (sequence x query head) row per
// workgroup of 16 waves.  The merge's arithmetic is merge_kernel's, term
// for term: M is the exact maximum of the used splits' m; w_s = exp(m_s - M)
// for z_s > 0, else 0; Z sums z_s w_s over s = lane, lane + 64, ... in
// ascending order per lane, then a lane-xor butterfly (every wave alike);
// wave w sums acc_s[c] w_s over s = (w & 3) + 4k ascending, for channels
// 128 (w >> 2) + lane and 128 (w >> 2) + 64 + lane, as merge_kernel's wave
// w & 3 does for the 64-channel block holding c; the four sums are added in
// order and divided by Z.  (One 8-byte load per lane and split for two
// adjacent channels instead ran slower: 9.7 against 8.4 us per launch.)  Wave 0 then rotates the row back with
// rotate_part (lane l: elements 8l .. 8l + 7), as tq_rotate_rows does on
// merge_kernel's output, so out and lse have the bits of the two launches.
constexpr int kMtWaves = 16;
constexpr int kMtBatch = 32;  // partial loads in flight per lane and channel
constexpr int kMtZPre = 4;    // z_s preloaded per lane (s < 256)

__global__ __launch_bounds__(kMtWaves * 64) void merge_tq_kernel(const float* __restrict__ part_acc,
                                                                 const float* __restrict__ part_m,
                                                                 const float* __restrict__ part_z,
                                                                 const int32_t* __restrict__ seq_lens, int n_q_heads,
                                                                 int max_seq_len, int S, int split_keys,
                                                                 float* __restrict__ out, float* __restrict__ lse) {
    extern __shared__ float w[];  // [S] split weights
    __shared__ float part[4][kTL];
    __shared__ float red[kMtWaves];

    const int bh = blockIdx.x;
    const int b = bh / n_q_heads;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int sw = wave & 3, cb = wave >> 2;
    const float* pm = part_m + int64_t(bh) * S;
    const float* pz = part_z + int64_t(bh) * S;
    const float* pa = part_acc + int64_t(bh) * S * kTL + 128 * cb + lane;

    // loads that do not need the sequence length (one memory round trip)
    int T = seq_lens[b];
    float v0[kMtBatch], v1[kMtBatch];
#pragma unroll
    for (int k = 0; k < kMtBatch; ++k) {
        const int sk = sw + 4 * k;
        v0[k] = sk < S ? pa[int64_t(sk) * kTL] : 0.0f;
        v1[k] = sk < S ? pa[int64_t(sk) * kTL + 64] : 0.0f;
    }
    const float my_m = tid < S ? pm[tid] : -INFINITY;
    const float my_z = tid < S ? pz[tid] : 0.0f;
    float zl[kMtZPre];
#pragma unroll
    for (int k = 0; k < kMtZPre; ++k) zl[k] = lane + 64 * k < S ? pz[lane + 64 * k] : 0.0f;

    T = T < 0 ? 0 : (T > max_seq_len ? max_seq_len : T);
    const int n = (T + split_keys - 1) / split_keys;  // workgroup-uniform
    float M = -INFINITY, z = 0.0f;
    if (n > 0) {
        float mx = tid < n ? my_m : -INFINITY;
        for (int s = tid + kMtWaves * 64; s < n; s += kMtWaves * 64) mx = fmaxf(mx, pm[s]);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
        if (lane == 0) red[wave] = mx;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kMtWaves; ++i) M = fmaxf(M, red[i]);  // exact: any order
        if (tid < n) w[tid] = my_z > 0.0f ? expf(my_m - M) : 0.0f;
        for (int s = tid + kMtWaves * 64; s < n; s += kMtWaves * 64) w[s] = pz[s] > 0.0f ? expf(pm[s] - M) : 0.0f;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kMtZPre; ++k)
            if (lane + 64 * k < n) z += zl[k] * w[lane + 64 * k];
        for (int s = lane + 64 * kMtZPre; s < n; s += 64) z += pz[s] * w[s];
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) z += __shfl_xor(z, m, 64);
        float acc0 = 0.0f, acc1 = 0.0f;
        for (int k0 = 0; sw + 4 * k0 < n; k0 += kMtBatch) {
            if (k0 > 0) {
#pragma unroll
                for (int k = 0; k < kMtBatch; ++k) {
                    const int sk = sw + 4 * (k0 + k);
                    v0[k] = sk < n ? pa[int64_t(sk) * kTL] : 0.0f;
                    v1[k] = sk < n ? pa[int64_t(sk) * kTL + 64] : 0.0f;
                }
            }
#pragma unroll
            for (int k = 0; k < kMtBatch; ++k) {
                const int sk = sw + 4 * (k0 + k);
                if (sk < n) {
                    acc0 += v0[k] * w[sk];
                    acc1 += v1[k] * w[sk];
                }
            }
        }
        part[sw][128 * cb + lane] = acc0;
        part[sw][128 * cb + 64 + lane] = acc1;
    }
    __syncthreads();
    if (wave != 0) return;
    // Z = 0 (no split holds a key) and T = 0 give a zero context, rotated like any other
    const bool any = n > 0 && z > 0.0f;
    float r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int j = 8 * lane + e;
        r[e] = any ? (((part[0][j] + part[1][j]) + part[2][j]) + part[3][j]) / z : 0.0f;
    }
    rotate_part<kTL>(r, lane, kSeedLatent, true);
    float* o = out + int64_t(bh) * kTL + 8 * lane;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = r[e];
    if (lse && lane == 0) lse[bh] = any ? M + logf(z) : -INFINITY;
}

}  // namespace

// The value of a double rounded to the nearest f16 (ties to even), for
// positive values in the f16 normal range.
static double round_f16(double v) {
    int e;
    std::frexp(v, &e);                            // v = m 2^e, m in [0.5, 1)
    const double quantum = std::ldexp(1.0, e - 11);  // 10 fraction bits after the leading one
    return std::nearbyint(v / quantum) * quantum;
}

// The matrix-core decode reads the levels as f16.  Scaling all of them by a
// common c (undone in the radius multipliers) lets the 16 values sit closer
// to the f16 grid: c is the multiple of 2^-16 in [1, 2) with the smallest
// largest relative deviation (about 9.5e-5, against 3.2e-4 at c = 1).
static TqMfmaTable make_mfma_table() {
    const TqTables& tb = tq_tables();
    double best_c = 1.0, best = 1.0;
    for (int i = 0; i < 65536; ++i) {
        const double c = 1.0 + i / 65536.0;
        double dev = 0.0;
        for (int k = 0; k < 16; ++k) {
            const double v = c * std::fabs(double(tb.lev[k]));
            dev = std::fmax(dev, std::fabs(round_f16(v) - v) / v);
        }
        if (dev < best) {
            best = dev;
            best_c = c;
        }
    }
    TqMfmaTable t{};
    for (int k = 0; k < 16; ++k) {
        // f16 bits of the rounded value: sign, biased exponent, 10 fraction bits
        const double v = round_f16(best_c * std::fabs(double(tb.lev[k])));
        int e;
        const double m = std::frexp(v, &e);  // v = m 2^e, m in [0.5, 1)
        const uint32_t frac = uint32_t(std::ldexp(m, 11)) - 1024u;
        const uint32_t bits = (tb.lev[k] < 0.0f ? 0x8000u : 0u) | (uint32_t(e - 1 + 15) << 10) | frac;
        t.lo[k / 4] |= uint32_t(bits & 0xFF) << (8 * (k % 4));
        t.hi[k / 4] |= uint32_t(bits >> 8) << (8 * (k % 4));
    }
    t.f_latent = float(1.0 / (best_c * std::sqrt(512.0)));
    t.f_rope = float(1.0 / (best_c * 8.0));
    t.c = float(best_c);
    t.max_dev = float(best);
    return t;
}

const TqMfmaTable& tq_mfma_table() {
    static const TqMfmaTable t = make_mfma_table();
    return t;
}

const TqTables& tq_tables() {
    static const TqTables tb = make_tables();
    return tb;
}

hipError_t launch_store_tq4(const Fp8Pool& pool, const void* x, InType dt, const int64_t* slots, int n_tokens,
                            hipStream_t s) {
    const int64_t n_slots = int64_t(pool.num_pages) * pool.page_size;
    const dim3 grid(static_cast<unsigned>(n_tokens)), block(64);
    const TqTables& tb = tq_tables();
    switch (dt) {
        case InType::F32:
            store_tq4_kernel<InType::F32><<<grid, block, 0, s>>>(x, slots, n_tokens, pool.codes, pool.scales, n_slots, tb);
            break;
        case InType::BF16:
            store_tq4_kernel<InType::BF16><<<grid, block, 0, s>>>(x, slots, n_tokens, pool.codes, pool.scales, n_slots, tb);
            break;
        case InType::F16:
            store_tq4_kernel<InType::F16><<<grid, block, 0, s>>>(x, slots, n_tokens, pool.codes, pool.scales, n_slots, tb);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_store_rotate_tq4(const Fp8Pool& pool, const void* x, InType dt, const int64_t* slots, int n_tokens,
                                   const float* q, float* q_rot, int n_rows, hipStream_t s) {
    const int64_t n_slots = int64_t(pool.num_pages) * pool.page_size;
    const dim3 grid(static_cast<unsigned>(n_tokens + n_rows)), block(64);
    const TqTables& tb = tq_tables();
    switch (dt) {
        case InType::F32:
            store_rotate_tq4_kernel<InType::F32><<<grid, block, 0, s>>>(x, slots, n_tokens, pool.codes, pool.scales,
                                                                        n_slots, tb, q, q_rot, n_rows);
            break;
        case InType::BF16:
            store_rotate_tq4_kernel<InType::BF16><<<grid, block, 0, s>>>(x, slots, n_tokens, pool.codes, pool.scales,
                                                                         n_slots, tb, q, q_rot, n_rows);
            break;
        case InType::F16:
            store_rotate_tq4_kernel<InType::F16><<<grid, block, 0, s>>>(x, slots, n_tokens, pool.codes, pool.scales,
                                                                        n_slots, tb, q, q_rot, n_rows);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_tq_rotate(const float* x, float* y, int64_t n_rows, int row_len, bool inverse, hipStream_t s) {
    if (n_rows == 0) return hipSuccess;
    tq_rotate_rows<<<dim3(unsigned(n_rows)), dim3(64), 0, s>>>(x, y, n_rows, row_len, inverse ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_merge_tq(const MergeArgs& a, hipStream_t s) {
    if (a.batch == 0) return hipSuccess;
    if (a.dv != kTL || a.rotate) return hipErrorInvalidValue;
    merge_tq_kernel<<<dim3(unsigned(a.batch * a.n_q_heads)), dim3(kMtWaves * 64), sizeof(float) * size_t(a.n_splits),
                      s>>>(a.part_acc, a.part_m, a.part_z, a.seq_lens, a.n_q_heads, a.max_seq_len, a.n_splits,
                           a.split_keys, a.out, a.lse);
    return hipGetLastError();
}

hipError_t launch_decode_tq4_simple(const Fp8Pool& pool, const DecodeArgs& a, hipStream_t s) {
    const int n_hblk = (a.n_q_heads + kTHB - 1) / kTHB;
    const dim3 grid(unsigned(a.n_splits), unsigned(n_hblk), unsigned(a.batch)), block(kTT);
    decode_tq4_simple<<<grid, block, 0, s>>>(pool.codes, pool.scales, pool.page_size, pool.num_pages, a, tq_tables());
    return hipGetLastError();
}

}  // namespace kvq
