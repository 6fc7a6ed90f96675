// decode_simple.hip -- split-K decode attention with plain fp32 vector math.
//
// One workgroup per (split, KV head or head block, sequence) -- the
// flash-decoding grid of the colibri pull request "KV cache quantization:
// fp8 (KV8) + 4-bit TurboQuant", split-T commit (partial online-softmax
// blocks, one per (head, split), each writing (cl[K], m, z)).  Keys are
// consumed in tiles staged through LDS; scores go through an online softmax
// in log2 units; partial m is written in natural-log units.
//
// These kernels favour clarity over speed; they serve any head_dim the
// format allows and are the reference point the MFMA kernels are measured
// against.
#include "internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;
constexpr int kMaxG = 16;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Signed value of nibble `e` (0..7) of a code word.
__device__ __forceinline__ float nibble(uint32_t w, int e) { return float(int32_t(w << (28 - 4 * e)) >> 28); }

// Code c of a 6- or 8-bit row (the layouts of blk_group_bytes).
template <int BITS>
__device__ __forceinline__ float blk_code(const uint8_t* row, int c) {
    const uint8_t* grp = row + (c >> 5) * blk_group_bytes(BITS);
    const int i = c & 31;
    if (BITS == 8) return float(int8_t(grp[i]));
    const uint32_t lo = (uint32_t(grp[i >> 1]) >> (4 * (i & 1))) & 0xFu;
    const uint32_t hi = (uint32_t(grp[16 + (i >> 2)]) >> (2 * (i & 3))) & 3u;
    return float(int32_t((lo | (hi << 4)) << 26) >> 26);
}

// ---------------------------------------------------------------- 4-bit
//
// Workgroup (split s, KV head g, sequence b) serves the G query heads of g.
// Per tile: rows -> LDS; each thread dots one key against a quarter of the
// channels for all G heads; the four quarters are summed in LDS; one wave per
// head runs the online softmax over the tile's 64 keys; then each thread
// accumulates its channel(s) of p * v for all heads.
// (BITS = 6, 8: the same kernel over the 6- and 8-bit block formats.)
template <int D, int BITS>
__global__ __launch_bounds__(kThreads) void decode_q4_simple(const uint8_t* __restrict__ k_pool,
                                                             const uint8_t* __restrict__ v_pool, int H,
                                                             int page_size, int num_pages, DecodeArgs a) {
    constexpr int RB = blk_row_bytes(BITS, D);
    constexpr int SCALE_OFF = (D / 32) * blk_group_bytes(BITS);  // byte offset of the fp16 scales
    constexpr int RW = RB / 4;
    constexpr int CQ = D / 4;
    constexpr int CPT = (D + kThreads - 1) / kThreads;
    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int G = a.n_q_heads / H;
    const int tid = threadIdx.x;
    const int T = clampi(a.seq_lens[b], 0, a.max_seq_len);
    const int j0 = s * a.split_keys;
    const int j1 = min(j0 + a.split_keys, T);
    const int64_t hb = int64_t(b) * a.n_q_heads + int64_t(g) * G;  // first query head (flat)
    const int S = a.n_splits;

    if (j0 >= j1) {  // split past the end: an empty partial
        for (int i = tid; i < G * D; i += kThreads)
            a.part_acc[((hb + i / D) * S + s) * D + i % D] = 0.0f;
        if (tid < G) {
            a.part_m[(hb + tid) * S + s] = -INFINITY;
            a.part_z[(hb + tid) * S + s] = 0.0f;
        }
        return;
    }

    __shared__ float qs[kMaxG][D];
    __shared__ uint32_t kt[kTile * RW];
    __shared__ uint32_t vt[kTile * RW];
    __shared__ float part[4][kMaxG][kTile];
    __shared__ float p[kMaxG][kTile];
    __shared__ float m_s[kMaxG], z_s[kMaxG], alpha_s[kMaxG];

    const float qscale = a.sm_scale * kLog2e;
    for (int i = tid; i < G * D; i += kThreads) qs[i / D][i % D] = a.q[hb * D + i] * qscale;
    if (tid < kMaxG) {
        m_s[tid] = -INFINITY;
        z_s[tid] = 0.0f;
    }
    float acc[CPT][kMaxG];
#pragma unroll
    for (int ci = 0; ci < CPT; ++ci)
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) acc[ci][h] = 0.0f;
    __syncthreads();

    const int32_t* pt = a.page_table + int64_t(b) * a.max_pages;
    for (int t0 = j0; t0 < j1; t0 += kTile) {
        const int n = min(kTile, j1 - t0);
        for (int i = tid; i < n * RW; i += kThreads) {
            const int kk = i / RW, w = i % RW;
            const int pos = t0 + kk;
            const int page = clampi(pt[pos / page_size], 0, num_pages - 1);
            const int64_t row = ((int64_t(page) * H + g) * page_size + pos % page_size) * RB;
            kt[i] = reinterpret_cast<const uint32_t*>(k_pool + row)[w];
            vt[i] = reinterpret_cast<const uint32_t*>(v_pool + row)[w];
        }
        __syncthreads();
        {
            const int kk = tid & (kTile - 1), qq = tid / kTile;
            float d[kMaxG];
#pragma unroll
            for (int h = 0; h < kMaxG; ++h) d[h] = 0.0f;
            if (kk < n) {
                for (int c0 = qq * CQ; c0 < (qq + 1) * CQ; c0 += 8) {
                    const uint8_t* krow = reinterpret_cast<const uint8_t*>(kt + kk * RW);
                    const int grp = c0 / 32;
                    const float sc = __half2float(__ushort_as_half(reinterpret_cast<const uint16_t*>(krow + SCALE_OFF)[grp]));
                    float v8[8];
                    if constexpr (BITS == 4) {
                        const uint32_t w = kt[kk * RW + c0 / 8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) v8[e] = nibble(w, e) * sc;
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) v8[e] = blk_code<BITS>(krow, c0 + e) * sc;
                    }
#pragma unroll
                    for (int h = 0; h < kMaxG; ++h) {
                        if (h < G) {
#pragma unroll
                            for (int e = 0; e < 8; ++e) d[h] = fmaf(qs[h][c0 + e], v8[e], d[h]);
                        }
                    }
                }
            }
#pragma unroll
            for (int h = 0; h < kMaxG; ++h)
                if (h < G) part[qq][h][kk] = d[h];
        }
        __syncthreads();
        {
            const int wave = tid >> 6, lane = tid & 63;
            for (int h = wave; h < G; h += kThreads / 64) {
                const float sc =
                    lane < n ? (part[0][h][lane] + part[1][h][lane]) + (part[2][h][lane] + part[3][h][lane]) : -INFINITY;
                const float m_old = m_s[h];
                const float m_new = fmaxf(m_old, wave_max(sc));
                const float e = lane < n ? exp2f(sc - m_new) : 0.0f;
                const float sum = wave_sum(e);
                p[h][lane] = e;
                if (lane == 0) {
                    const float al = exp2f(m_old - m_new);
                    alpha_s[h] = al;
                    z_s[h] = z_s[h] * al + sum;
                    m_s[h] = m_new;
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int ci = 0; ci < CPT; ++ci) {
            const int c = tid + ci * kThreads;
            if (c < D) {
#pragma unroll
                for (int h = 0; h < kMaxG; ++h)
                    if (h < G) acc[ci][h] *= alpha_s[h];
                const int grp = c / 32;
                for (int kk = 0; kk < n; ++kk) {
                    const uint8_t* vrow = reinterpret_cast<const uint8_t*>(vt + kk * RW);
                    const float sc = __half2float(__ushort_as_half(reinterpret_cast<const uint16_t*>(vrow + SCALE_OFF)[grp]));
                    float vv;
                    if constexpr (BITS == 4) vv = nibble(vt[kk * RW + c / 8], c & 7) * sc;
                    else vv = blk_code<BITS>(vrow, c) * sc;
#pragma unroll
                    for (int h = 0; h < kMaxG; ++h)
                        if (h < G) acc[ci][h] = fmaf(p[h][kk], vv, acc[ci][h]);
                }
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int ci = 0; ci < CPT; ++ci) {
        const int c = tid + ci * kThreads;
        if (c < D) {
#pragma unroll
            for (int h = 0; h < kMaxG; ++h)
                if (h < G) a.part_acc[((hb + h) * S + s) * D + c] = acc[ci][h];
        }
    }
    if (tid < G) {
        a.part_m[(hb + tid) * S + s] = m_s[tid] * kLn2;
        a.part_z[(hb + tid) * S + s] = z_s[tid];
    }
}

// ---------------------------------------------------------------- fp8 latent
//
// Workgroup (split s, block of 16 heads, sequence b).  Tiles of 16 keys;
// each of 16 thread groups dots the tile's keys against 1/16 of the channels
// for all 16 heads; scales are applied per key (latent and rope separately);
// the 16 partial dots are summed in LDS; one wave handles 4 heads' online
// softmax; each thread accumulates 2 latent channels for all 16 heads.

// Value of an e4m3 code; the NaN codes 0x7F/0xFF read as 0.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float v = e == 0u ? float(m) * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
    v = (c & 0x7Fu) == 0x7Fu ? 0.0f : v;
    return (c & 0x80u) ? -v : v;
}

constexpr int kHB = 16;
constexpr int kFTile = 16;

template <int L, int R>
__global__ __launch_bounds__(kThreads) void decode_fp8_simple(const uint8_t* __restrict__ codes,
                                                              const float* __restrict__ scales, int page_size,
                                                              int num_pages, DecodeArgs a) {
    constexpr int D = L + R;
    constexpr int DW = D / 4;
    constexpr int LP = L / 16;  // latent channels per thread group
    constexpr int RP = R / 16;  // rope channels per thread group
    constexpr int CPT = L / kThreads;
    static_assert(L % kThreads == 0 && R % 16 == 0 && LP % 4 == 0, "latent/rope split");
    const int s = blockIdx.x, hblk = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int h0 = hblk * kHB;
    const int nh = min(kHB, a.n_q_heads - h0);
    const int T = clampi(a.seq_lens[b], 0, a.max_seq_len);
    const int j0 = s * a.split_keys;
    const int j1 = min(j0 + a.split_keys, T);
    const int64_t hb = int64_t(b) * a.n_q_heads + h0;
    const int S = a.n_splits;

    if (j0 >= j1) {
        for (int i = tid; i < nh * L; i += kThreads) a.part_acc[((hb + i / L) * S + s) * L + i % L] = 0.0f;
        if (tid < nh) {
            a.part_m[(hb + tid) * S + s] = -INFINITY;
            a.part_z[(hb + tid) * S + s] = 0.0f;
        }
        return;
    }

    __shared__ float qs[kHB][D];
    __shared__ uint32_t ct[kFTile * DW];
    __shared__ float scl[kFTile], scr[kFTile];
    __shared__ float part[16][kHB][kFTile];
    __shared__ float p[kHB][kFTile];
    __shared__ float m_s[kHB], z_s[kHB], alpha_s[kHB];

    const float qscale = a.sm_scale * kLog2e;
    for (int i = tid; i < kHB * D; i += kThreads) {
        const int h = i / D;
        qs[h][i % D] = h < nh ? a.q[(hb + h) * D + i % D] * qscale : 0.0f;
    }
    if (tid < kHB) {
        m_s[tid] = -INFINITY;
        z_s[tid] = 0.0f;
    }
    float acc[CPT][kHB];
#pragma unroll
    for (int ci = 0; ci < CPT; ++ci)
#pragma unroll
        for (int h = 0; h < kHB; ++h) acc[ci][h] = 0.0f;
    __syncthreads();

    const int32_t* pt = a.page_table + int64_t(b) * a.max_pages;
    for (int t0 = j0; t0 < j1; t0 += kFTile) {
        const int n = min(kFTile, j1 - t0);
        for (int i = tid; i < n * DW; i += kThreads) {
            const int kk = i / DW, w = i % DW;
            const int pos = t0 + kk;
            const int page = clampi(pt[pos / page_size], 0, num_pages - 1);
            const int64_t slot = int64_t(page) * page_size + pos % page_size;
            ct[i] = reinterpret_cast<const uint32_t*>(codes + slot * D)[w];
        }
        if (tid < n) {
            const int pos = t0 + tid;
            const int page = clampi(pt[pos / page_size], 0, num_pages - 1);
            const int64_t slot = int64_t(page) * page_size + pos % page_size;
            scl[tid] = scales[slot * 2];
            scr[tid] = scales[slot * 2 + 1];
        }
        __syncthreads();
        {
            const int kk = tid & (kFTile - 1), part_i = tid / kFTile;
            float dl[kHB], dr[kHB];
#pragma unroll
            for (int h = 0; h < kHB; ++h) dl[h] = dr[h] = 0.0f;
            if (kk < n) {
                const int cl0 = part_i * LP;
                for (int c = cl0; c < cl0 + LP; c += 4) {
                    const uint32_t w = ct[kk * DW + c / 4];
                    float v4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v4[e] = e4m3_value((w >> (8 * e)) & 0xFFu);
#pragma unroll
                    for (int h = 0; h < kHB; ++h)
#pragma unroll
                        for (int e = 0; e < 4; ++e) dl[h] = fmaf(qs[h][c + e], v4[e], dl[h]);
                }
                const int cr0 = L + part_i * RP;
#pragma unroll
                for (int e = 0; e < RP; ++e) {
                    const int c = cr0 + e;
                    const float v = e4m3_value((ct[kk * DW + c / 4] >> (8 * (c & 3))) & 0xFFu);
#pragma unroll
                    for (int h = 0; h < kHB; ++h) dr[h] = fmaf(qs[h][c], v, dr[h]);
                }
            }
            const float sl = kk < n ? scl[kk] : 0.0f, sr = kk < n ? scr[kk] : 0.0f;
#pragma unroll
            for (int h = 0; h < kHB; ++h) part[part_i][h][kk] = fmaf(sl, dl[h], sr * dr[h]);
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
            p[h][kk] = e * (kk < n ? scl[kk] : 0.0f);  // the value is scL * dec(Lc)
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
            const int c = tid + ci * kThreads;
#pragma unroll
            for (int h = 0; h < kHB; ++h) acc[ci][h] *= alpha_s[h];
            for (int kk = 0; kk < n; ++kk) {
                const float v = e4m3_value((ct[kk * DW + c / 4] >> (8 * (c & 3))) & 0xFFu);
#pragma unroll
                for (int h = 0; h < kHB; ++h) acc[ci][h] = fmaf(p[h][kk], v, acc[ci][h]);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int ci = 0; ci < CPT; ++ci) {
        const int c = tid + ci * kThreads;
#pragma unroll
        for (int h = 0; h < kHB; ++h)
            if (h < nh) a.part_acc[((hb + h) * S + s) * L + c] = acc[ci][h];
    }
    if (tid < nh) {
        a.part_m[(hb + tid) * S + s] = m_s[tid] * kLn2;
        a.part_z[(hb + tid) * S + s] = z_s[tid];
    }
}

}  // namespace

template <int BITS>
hipError_t launch_blk_simple(const Q4Pool& pool, const DecodeArgs& a, hipStream_t s) {
    const dim3 grid(unsigned(a.n_splits), unsigned(pool.n_kv_heads), unsigned(a.batch)), block(kThreads);
    const int H = pool.n_kv_heads, P = pool.page_size, N = pool.num_pages;
    switch (pool.head_dim) {
        case 64: decode_q4_simple<64, BITS><<<grid, block, 0, s>>>(pool.k, pool.v, H, P, N, a); break;
        case 128: decode_q4_simple<128, BITS><<<grid, block, 0, s>>>(pool.k, pool.v, H, P, N, a); break;
        case 256: decode_q4_simple<256, BITS><<<grid, block, 0, s>>>(pool.k, pool.v, H, P, N, a); break;
        case 512: decode_q4_simple<512, BITS><<<grid, block, 0, s>>>(pool.k, pool.v, H, P, N, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode_q4_simple(const Q4Pool& pool, const DecodeArgs& a, hipStream_t s) {
    if (pool.bits == 8) return launch_blk_simple<8>(pool, a, s);
    if (pool.bits == 6) return launch_blk_simple<6>(pool, a, s);
    return launch_blk_simple<4>(pool, a, s);
}

hipError_t launch_decode_fp8_simple(const Fp8Pool& pool, const DecodeArgs& a, hipStream_t s) {
    const int n_hblk = (a.n_q_heads + kHB - 1) / kHB;
    const dim3 grid(unsigned(a.n_splits), unsigned(n_hblk), unsigned(a.batch)), block(kThreads);
    if (pool.head_dim == 576 && pool.rope_dim == 64) {
        decode_fp8_simple<512, 64><<<grid, block, 0, s>>>(pool.codes, pool.scales, pool.page_size, pool.num_pages, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kvq
