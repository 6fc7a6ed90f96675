// decode_q4_chunk.hip -- split-K attention of several query rows of one
// sequence (a prompt chunk) over its 4-bit Hadamard-32 cache, on matrix cores.
//
// Method: TensorFold issue "qwen27 CUDA: an opt-in 4-bit attention cache",
// section "What it is": prompt chunks are packed into the 4-bit cache and
// then attended over the decoded slots, in rotated space; colibri pull
// request "KV cache quantization: fp8 (KV8) + 4-bit TurboQuant", split-T
// commit: partial blocks (cl[K], m, z) merged by a log-sum-exp kernel.  Row
// i attends positions [0, row_lens[i]) (a chunk starting at position P:
// row_lens[i] = P + i + 1), and the partials are the decode's, so kvq_merge
// with the same row lengths completes the attention.
//
// Why a kernel of its own: a decode reads every cache byte for one query row
// (6 heads), so it is bound by HBM; a chunk of C rows attends the same bytes
// C times, so the rows must share each staged tile.  Workgroup = 8 waves =
// (split s, KV head g, group of 8 consecutive rows), one row per wave.  Waves
// 0..3 each copy one 16-row run of every 32-key tile (K runs 0, 1, V runs 0,
// 1) with LDS DMA into a ring of 4 tiles shared by the workgroup, three tiles
// ahead; one workgroup barrier per tile both publishes the tile and frees the
// slot the next copy overwrites.  Every wave then runs the single-row decode
// kernel's tile step on the shared tile (decode_q4_mfma.hip): scores and
// context on v_mfma_f32_16x16x32_f16 with the codes as f16 subnormals, the
// query's f16 hi and lo parts in B columns 0..7 and 8..15, the fp16 scales
// hoisted out of the 32-element dots, a lazily moving running maximum, and
// the context operand's power-of-two exponent window for the V scales.  Keys
// at or past a row's own length are masked in that row's scores; V scales of
// rows past the group's last key are zeroed in LDS, so stale bytes cannot
// meet p = 0.  Each wave writes its row's partial from registers.
#include "mfma_common.h"

namespace kvq {
namespace {

using namespace mx;

constexpr int kRowsWG = 8;         // query rows per workgroup, one per wave
constexpr int kWaves = kRowsWG;
constexpr int kSub = 32;           // keys per tile
constexpr int kSlots = 4;          // tiles in the shared ring (three in flight)
constexpr float kRescale = 6.0f;   // log2 headroom before the running max moves

template <int D>
struct ChunkShape {
    static constexpr int NG = D / 32;                       // 32-channel groups per row
    static constexpr int RB = D / 2 + D / 16;               // row bytes (144 at D = 256)
    static constexpr int SOFF = D / 2;                      // the scales' offset in a row
    static constexpr int NB = D / 16;                       // 16-channel output blocks
    static constexpr int RUN = 16 * RB;                     // bytes of a 16-row run
    static constexpr int RUN_INSTR = (RUN / 16 + 63) / 64;  // 16-byte DMA instructions per run
    static constexpr int TILE = kSub * RB;                  // one pool's tile
    static constexpr int SLOT = 2 * TILE;                   // K tile, then V tile
    static constexpr int LDS = kSlots * SLOT;
};

// Copies one 16-row run (RUN bytes) from global to LDS, default cache policy:
// the other row groups of the same split read these bytes again.
template <int D>
__device__ __forceinline__ void chunk_dma_run(const uint8_t* src, uint32_t lds, int lane) {
    using S = ChunkShape<D>;
#pragma unroll
    for (int i = 0; i < S::RUN_INSTR; ++i) {
        const int chunk = i * 64 + lane;
        if (i + 1 < S::RUN_INSTR || chunk < S::RUN / 16) dma16<false>(src, uint32_t(chunk * 16), lds + uint32_t(i * 1024));
    }
}

__device__ __forceinline__ void barrier_lds_only() {
    // LDS writes of every wave visible, the copies in flight not waited for.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Grid: (splits, KV heads, row groups).  Groups of at most 8 query heads per
// KV head (the packed hi / lo B columns), head_dim 128 or 256, pages of a
// multiple of 16 tokens.
template <int D>
__global__ __launch_bounds__(kWaves * 64, 1) void decode_q4_chunk(const uint8_t* __restrict__ k_pool,
                                                                 const uint8_t* __restrict__ v_pool, int H,
                                                                 int page_size, int num_pages, DecodeArgs a) {
    using S = ChunkShape<D>;
    constexpr int NG = S::NG, RB = S::RB, NB = S::NB, SOFF = S::SOFF;
    constexpr float kOff = 8.0f;
    // (+16: the 16-byte scale reads of the last row run 8 bytes past it at head_dim 128)
    __shared__ __attribute__((aligned(16))) uint8_t smem[S::LDS + 16];

    const int s = blockIdx.x, g = blockIdx.y, rg = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, q4 = lane >> 4;
    const int G = a.n_q_heads / H;
    const int Sn = a.n_splits;
    const int j0 = s * a.split_keys;
    const int row = rg * kRowsWG + wave;  // this wave's query row
    const bool has_row = row < a.batch;

    // Row lengths: this wave's (wave-uniform) and the group's largest.
    auto clamp_len = [&](int T) { return T < 0 ? 0 : (T > a.max_seq_len ? a.max_seq_len : T); };
    int L = 0, Lg = 0;
    {
        const int r = rg * kRowsWG + (lane & 7);
        const int T = r < a.batch ? clamp_len(a.seq_lens[r]) : 0;
        L = __builtin_amdgcn_readfirstlane(__shfl(T, wave, 64));
        int m = T;
#pragma unroll
        for (int k = 1; k < 8; k <<= 1) m = max(m, __shfl_xor(m, k, 64));
        Lg = __builtin_amdgcn_readfirstlane(m);
    }
    const int64_t hb = int64_t(row) * a.n_q_heads + int64_t(g) * G;

    const int jg1 = min(j0 + a.split_keys, Lg);  // the group's keys in this split: [j0, jg1)
    const int n_tiles = jg1 > j0 ? (jg1 - j0 + kSub - 1) / kSub : 0;
    const int n_keys = has_row ? max(0, min(j0 + a.split_keys, L) - j0) : 0;  // this row's keys here
    auto write_empty = [&]() {
        if (!has_row) return;
        for (int i = lane; i < G * D; i += 64) a.part_acc[((hb + i / D) * Sn + s) * D + i % D] = 0.0f;
        if (lane < G) {
            a.part_m[(hb + lane) * Sn + s] = -INFINITY;
            a.part_z[(hb + lane) * Sn + s] = 0.0f;
        }
    };
    if (n_tiles == 0) {  // no row of the group reaches this split: the whole workgroup leaves
        write_empty();
        return;
    }

    // DMA duty: waves 0, 1 copy K runs 0, 1 of every tile, waves 2, 3 the V runs.
    const bool copier = wave < 4;
    const uint8_t* pool = wave < 2 ? k_pool : v_pool;
    const int run = wave & 1;
    const int32_t* pt = a.page_table;
    const int last_pos = a.max_seq_len > 0 ? (a.max_seq_len - 1) & ~15 : 0;
    // Position of this wave's run of tile t (clamped to the run holding
    // max_seq_len - 1, so every copy stays in bounds; rows past the end are
    // masked) and its page (a scalar load: the index is wave-uniform).
    auto run_pos = [&](int t) { return min(j0 + kSub * t + 16 * run, last_pos); };
    auto run_page = [&](int t) {
        const int page = pt[run_pos(t) / page_size];
        return page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
    };
    auto issue = [&](int t, int page) {  // this wave's run of tile t into ring slot t % kSlots
        const int pos = run_pos(t);
        const int64_t off = ((int64_t(page) * H + g) * page_size + pos % page_size) * RB;
        const uint32_t dst = lds_addr(smem) + uint32_t((t % kSlots) * S::SLOT + (wave >> 1) * S::TILE + run * 16 * RB);
        chunk_dma_run<D>(pool + off, dst, lane);
    };
    int next_page = 0;  // the page of the next tile to issue, loaded one tile ahead
    if (copier) {
#pragma unroll
        for (int t = 0; t < kSlots - 1; ++t)
            if (t < n_tiles) issue(t, run_page(t));
        if (kSlots - 1 < n_tiles) next_page = run_page(kSlots - 1);
    }

    // The query of head hcol for B column n16: hi part in columns 0..7, lo in 8..15.
    const int hcol = n16 & 7;
    const bool live = has_row && hcol < G;
    const float* qh = a.q + ((has_row ? hb : 0) + (live ? hcol : 0)) * D;
    half8_t bq_hi[NG];
    f32x4 cbias[NG];
    {
        const float qscale = a.sm_scale * kLog2e;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            const float4 lo4 = *reinterpret_cast<const float4*>(qh + 32 * gi + 8 * q4);
            const float4 hi4 = *reinterpret_cast<const float4*>(qh + 32 * gi + 8 * q4 + 4);
            const float c8[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
            constexpr int order[8] = {0, 4, 1, 5, 2, 6, 3, 7};
            float sum = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float f = (k & 2) ? 0.0625f : 1.0f;
                const float v = live ? c8[order[k]] * qscale * f : 0.0f;
                const _Float16 h = _Float16(v);
                const _Float16 l = _Float16(v - float(h));
                bq_hi[gi][k] = (n16 & 8) ? l : h;
                sum += (float(h) + float(l)) * ((k & 2) ? 16.0f : 1.0f);
            }
            sum = quad_sum(sum);
            const float cb = (n16 & 8) ? 0.0f : -kOff * sum / kTwo24;  // the offset once, in the hi column
            cbias[gi] = f32x4{cb, cb, cb, cb};
        }
    }
    half8_t bconst;
#pragma unroll
    for (int k = 0; k < 8; ++k) bconst[k] = _Float16((k & 2) ? -16.0f * kOff / kTwo24 : -kOff / kTwo24);

    f32x4 o[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) o[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    f32x4 ro[NG / 2];  // the +8 offset of the V codes, per pair of groups
#pragma unroll
    for (int i = 0; i < NG / 2; ++i) ro[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, z_run = 0.0f;
    int a_exp = 0;  // the context operand's exponent (mfma_common.h); wave-uniform
    uint32_t win_lo = f16_bits_pow2(-8), win_hi = f16_bits_pow2(9);

    // ds_read_b64_tr_b4 row of this lane: key K(q4, e) for e = n16 & 7,
    // K(q, e) = 4q + e (e < 4) or 16 + 4q + e - 4, channel half n16 >> 3.
    const int e7 = n16 & 7;
    const int tr_key = e7 < 4 ? 4 * q4 + e7 : 16 + 4 * q4 + e7 - 4;
    const int tr_off = tr_key * RB + 8 * (n16 >> 3);
    const uint32_t psel_pair = (n16 & 8) ? 0x07060302u : 0x05040100u;

    for (int t = 0; t < n_tiles; ++t) {
        const int t0 = j0 + kSub * t;  // first key of the tile
        uint8_t* kt = smem + (t % kSlots) * S::SLOT;
        uint8_t* vt = kt + S::TILE;
        if (copier) {
            // own run of tile t landed: at most the later tiles' copies are outstanding
            if (t + 2 < n_tiles) wait_vmcnt<2 * S::RUN_INSTR>();
            else if (t + 1 < n_tiles) wait_vmcnt<S::RUN_INSTR>();
            else wait_vmcnt<0>();
            // rows past the group's last key may hold any bytes (a NaN scale among
            // them) that must not meet p = 0: zero their V scales (own run only)
            if (wave >= 2) {
                const int r = 16 * run + lane;
                if (lane < 16 && t0 + r >= jg1) {
#pragma unroll
                    for (int i = 0; i < D / 16; i += 4) *reinterpret_cast<uint32_t*>(vt + r * RB + SOFF + i) = 0u;
                }
            }
        }
        barrier_lds_only();  // tile t staged for every wave; every wave is done with tile t - 1
        if (copier && t + kSlots - 1 < n_tiles) {
            issue(t + kSlots - 1, next_page);  // into the slot of tile t - 1
            if (t + kSlots < n_tiles) next_page = run_page(t + kSlots);
        }
        const int valid = min(kSub, L - t0);
        if (!has_row || valid <= 0) continue;  // this row's keys end before the tile (the others' do not)

        // ---- scores: two 16-key blocks; lane holds keys 16 kb + 4 q4 + i of head column n16
        float sc[2][4];
        {
            u32x4 ks[2][4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    ks[kb][i] = *reinterpret_cast<const u32x4*>(kt + (16 * kb + 4 * q4 + i) * RB + SOFF);
            uint32_t kc[2][NG];
#pragma unroll
            for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    kc[kb][gi] = *reinterpret_cast<const uint32_t*>(kt + (16 * kb + n16) * RB + 16 * gi + 4 * q4);
            float acc[2][4] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
            f32x4 dprev[2];
#pragma unroll
            for (int gi = 0; gi <= NG; ++gi) {
                f32x4 dcur[2];
                if (gi < NG) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) dcur[kb] = mfma(unpack8(kc[kb][gi]), bq_hi[gi], cbias[gi]);
                }
                if (gi > 0) {
                    const int gp = gi - 1;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const uint32_t sw = ks[kb][i][gp >> 1];
                            acc[kb][i] = fmaf(dprev[kb][i], (gp & 1) ? hi_half(sw) : lo_half(sw), acc[kb][i]);
                        }
                }
                if (gi < NG) {
                    dprev[0] = dcur[0];
                    dprev[1] = dcur[1];
                }
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[kb][i] = row_xor8(acc[kb][i]) + acc[kb][i];  // hi + lo columns
        }
        if (valid < kSub) {  // keys at or past this row's length
            asm volatile("" ::: "memory");
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * kb + 4 * q4 + i >= valid) sc[kb][i] = -INFINITY;
        }

        // ---- V operands and scales of the tile
        i32x2 cv[NG];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
            cv[gi] = __builtin_amdgcn_ds_read_tr4_b64_v2i32((__attribute__((address_space(3))) i32x2*)(vt + tr_off + 16 * gi));
        u32x4 vsa[4], vsb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            vsa[r] = *reinterpret_cast<const u32x4*>(vt + (4 * q4 + r) * RB + SOFF);
            vsb[r] = *reinterpret_cast<const u32x4*>(vt + (16 + 4 * q4 + r) * RB + SOFF);
        }
        const uint32_t vmax = [&] {
            const u32x2 w = *reinterpret_cast<const u32x2*>(vt + (lane >> 1) * RB + SOFF + (NG >= 8 ? 8 * (lane & 1) : 0));
            return max4_u16(w[0], w[1]);
        }();

        // ---- online softmax (log2 units; the maximum moves by more than 2^6 only)
        const float tmax = quad_max_nonan(max8f(sc)) * kTwo24;  // finite: valid >= 1
        const bool move = tmax > m_run + kRescale;              // the first tile moves it from -inf
        const bool rebase = outside_window(vmax, win_lo, win_hi);
        if (__builtin_amdgcn_ballot_w64(move) != 0ull || rebase) {
            const int a_new = rebase ? v_exponent_for(vmax, a_exp) : a_exp;
            const float m_new = move ? fmaxf(m_run, tmax) : m_run;
            const float alpha = (move ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f) * pow2i(a_new - a_exp);
            if (rebase) {
                a_exp = __builtin_amdgcn_readfirstlane(a_new);
                win_lo = __builtin_amdgcn_readfirstlane(f16_bits_pow2(-8 - a_exp));
                win_hi = __builtin_amdgcn_readfirstlane(f16_bits_pow2(9 - a_exp));
            }
            z_run *= alpha;
            m_run = m_new;
            float al[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * q4 + i, 64);  // rows 4 q4 + i are heads
#pragma unroll
            for (int blk = 0; blk < NB; ++blk)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[blk][i] *= al[i];
#pragma unroll
            for (int gp = 0; gp < NG / 2; ++gp)
#pragma unroll
                for (int i = 0; i < 4; ++i) ro[gp][i] *= al[i];
        }
        float p[2][4];
        const float nm0 = float(a_exp) - m_run, nm4 = nm0 - 4.0f;  // p * 2^a_exp; slots 2,3,6,7 / 16
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[kb][i] = __builtin_amdgcn_exp2f(fmaf(sc[kb][i], kTwo24, (i & 1) ? nm4 : nm0));
                z_run = (i & 1) ? fmaf(16.0f, p[kb][i], z_run) : z_run + p[kb][i];
            }

        // ---- context: rows 0..7 carry the even group of a pair, 8..15 the odd
        half8_t av;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            if ((gi & 1) == 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t pair = __builtin_amdgcn_perm(vsb[r][gi >> 1], vsa[r][gi >> 1], psel_pair);
                    const half2_t w = ctx_weights(p[0][r], p[1][r], pair);
                    av[2 * r] = w[0];
                    av[2 * r + 1] = w[1];
                }
                ro[gi >> 1] = mfma(av, bconst, ro[gi >> 1]);
            }
            o[2 * gi] = mfma(av, unpack8(uint32_t(cv[gi][0])), o[2 * gi]);
            o[2 * gi + 1] = mfma(av, unpack8(uint32_t(cv[gi][1])), o[2 * gi + 1]);
        }
    }

    // ---- this row's partial, straight from registers: o rows 4 q4 + i are
    // head (row & 7), group blk / 2 read from rows 0..7 if even, 8..15 if odd
    if (!has_row) return;
    if (n_keys == 0) {
        write_empty();
        return;
    }
    z_run = quad_sum(z_run);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int orow = 4 * q4 + i, h = orow & 7;
        if (h < G) {
            float* dst = a.part_acc + ((hb + h) * Sn + s) * D + n16;
#pragma unroll
            for (int blk = 0; blk < NB; ++blk)
                if (((blk >> 1) & 1) == (orow >> 3)) dst[16 * blk] = (o[blk][i] + ro[blk >> 2][i]) * kTwo24;
        }
    }
    if (q4 == 0 && n16 < G) {
        a.part_m[(hb + n16) * Sn + s] = (m_run - float(a_exp)) * kLn2;
        a.part_z[(hb + n16) * Sn + s] = z_run;
    }
}

}  // namespace

bool decode_q4_chunk_supported(const Q4Pool& pool, const DecodeArgs& a) {
    const int G = a.n_q_heads / pool.n_kv_heads;
    return pool.bits == 4 && (pool.head_dim == 128 || pool.head_dim == 256) && G >= 1 && G <= 8 &&
           pool.page_size % 16 == 0 && a.split_keys % kSub == 0;
}

// a.batch = the chunk's rows, a.seq_lens = their lengths, a.page_table = the
// sequence's one page-table row.
hipError_t launch_decode_q4_chunk(const Q4Pool& pool, const DecodeArgs& a, hipStream_t s) {
    const dim3 grid(unsigned(a.n_splits), unsigned(pool.n_kv_heads), unsigned((a.batch + kRowsWG - 1) / kRowsWG));
    switch (pool.head_dim) {
        case 128:
            decode_q4_chunk<128><<<grid, dim3(kWaves * 64), 0, s>>>(pool.k, pool.v, pool.n_kv_heads, pool.page_size,
                                                                   pool.num_pages, a);
            break;
        case 256:
            decode_q4_chunk<256><<<grid, dim3(kWaves * 64), 0, s>>>(pool.k, pool.v, pool.n_kv_heads, pool.page_size,
                                                                   pool.num_pages, a);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kvq
