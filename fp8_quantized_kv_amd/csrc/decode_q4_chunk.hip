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
// C times, so the rows must share each staged tile, and per row the work is
// matrix-core and vector-ALU work, not bytes.  Workgroup = 8 waves = (split
// s, KV head g, group of 16 consecutive rows), two rows per wave, two waves
// per SIMD.  Waves 0..3 each copy one 16-row run of every 32-key tile (K runs
// 0, 1, V runs 0, 1) with LDS DMA into a ring of 4 tiles shared by the
// workgroup, three tiles ahead; one workgroup barrier per tile both
// publishes the tile and frees the slot the next copy overwrites.
//
// A wave's two rows share the MFMA columns: column n = (row n / G, head
// n % G), 2 G <= 16 of them, so every unpacked K or V code operand and every
// staged scale a wave reads serves both rows.  Per tile, on
// v_mfma_f32_16x16x32_f16 with the codes as f16 subnormals (code + 8) 2^-24:
//  * scores: per 32-channel group, the query's f16 hi part (registers) and
//    lo part (this wave's LDS area) in one MFMA chain, the group's fp16 scale
//    applied to the chain's result with one FMA; the +8 offset, summed over
//    the groups with the key's scales, is one more MFMA per 16 keys (A = the
//    key's scales, B = -8 2^-24 x each group's query sum, x 2^16 as f16 hi +
//    lo);
//  * softmax per column in log2 units, a lazily moving running maximum, the
//    context operand's power-of-two exponent window for the V scales;
//  * context per group: A = p x the keys' V scale of the group, formed in
//    fp32 and rounded to f16 once (v_fma_mix), B = the V codes; the +8 offset
//    of the V codes is one accumulator for all groups, group gi's sum in its
//    column gi (B = the offset constant in column gi only, from an LDS table).
// Keys at or past a column's row length are masked in its scores; V scales
// of rows past the group's last key are zeroed in LDS, so stale bytes cannot
// meet p = 0.  Each wave writes its rows' partials from registers.
#include "mfma_common.h"

namespace kvq {
namespace {

using namespace mx;

constexpr int kRowsWG = 16;        // query rows per workgroup
constexpr int kRowsWave = 2;       // query rows per wave: 2 G <= 16 MFMA columns
constexpr int kWaves = kRowsWG / kRowsWave;
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
    static constexpr int RING = kSlots * SLOT;
    static constexpr int BQLO = RING;                       // per wave: the query's lo parts, [gi][lane] x 16 bytes
    static constexpr int BRO = BQLO + kWaves * NG * 1024;   // [gi][lane] x 16 bytes: the V offset constant in column gi
    static constexpr int LDS = BRO + NG * 1024;
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

// Context weights of two keys for one group: p0 times the f16 V scale in
// half H of sa (low half, 0, or high half, 1) and p1 times that of sb, each
// formed in fp32 and rounded to f16 once, as one f16 pair.
template <int H>
__device__ __forceinline__ uint32_t ctx_pair(float p0, float p1, uint32_t sa, uint32_t sb) {
    uint32_t r;  // mixlo writes the low half; mixhi then the high half
    if (H == 0) {
        asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=v"(r) : "v"(p0), "v"(sa));
        asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "+v"(r) : "v"(p1), "v"(sb));
    } else {
        asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(r) : "v"(p0), "v"(sa));
        asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "+v"(r) : "v"(p1), "v"(sb));
    }
    return r;
}

// Grid: (splits, KV heads, row groups).  Groups of at most 8 query heads per
// KV head (two rows' heads share the MFMA columns), head_dim 128 or 256,
// pages of a multiple of 16 tokens.
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

    // MFMA column n16 = (row rr, head h) of this wave: rr = n16 / G, h = n16 % G
    // (columns 2 G .. 15 unused).
    const int c_rr = n16 >= G ? 1 : 0;
    const int c_h = n16 - c_rr * G;
    const bool c_used = n16 < kRowsWave * G;

    // Row lengths: this wave's two rows' (wave-uniform) and the group's largest.
    auto clamp_len = [&](int T) { return T < 0 ? 0 : (T > a.max_seq_len ? a.max_seq_len : T); };
    int L[kRowsWave], Lg = 0;
    {
        const int r = rg * kRowsWG + (lane & 15);
        const int T = r < a.batch ? clamp_len(a.seq_lens[r]) : 0;
#pragma unroll
        for (int rr = 0; rr < kRowsWave; ++rr) L[rr] = __builtin_amdgcn_readfirstlane(__shfl(T, kRowsWave * wave + rr, 64));
        int m = T;
#pragma unroll
        for (int k = 1; k < 16; k <<= 1) m = max(m, __shfl_xor(m, k, 64));
        Lg = __builtin_amdgcn_readfirstlane(m);
    }
    const int row0 = rg * kRowsWG + kRowsWave * wave;
    auto has_row = [&](int rr) { return row0 + rr < a.batch; };
    auto hbase = [&](int rr) { return int64_t(row0 + rr) * a.n_q_heads + int64_t(g) * G; };
    auto n_keys = [&](int rr) { return has_row(rr) ? max(0, min(j0 + a.split_keys, L[rr]) - j0) : 0; };
    const int Lc = c_rr ? L[1] : L[0];  // this lane's column's row length

    const int jg1 = min(j0 + a.split_keys, Lg);  // the group's keys in this split: [j0, jg1)
    const int n_tiles = jg1 > j0 ? (jg1 - j0 + kSub - 1) / kSub : 0;
    auto write_empty = [&](int rr) {
        if (!has_row(rr)) return;
        const int64_t hb = hbase(rr);
        for (int i = lane; i < G * D; i += 64) a.part_acc[((hb + i / D) * Sn + s) * D + i % D] = 0.0f;
        if (lane < G) {
            a.part_m[(hb + lane) * Sn + s] = -INFINITY;
            a.part_z[(hb + lane) * Sn + s] = 0.0f;
        }
    };
    if (n_tiles == 0) {  // no row of the group reaches this split: the whole workgroup leaves
        write_empty(0);
        write_empty(1);
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

    // B operands: column n16's query (row c_rr, head c_h) x sm_scale x log2(e)
    // as f16 hi and lo parts, k-slots in the unpacked codes' order (slots 2,
    // 3, 6, 7 carry the x16 high nibbles: their query is / 16).  The hi parts
    // stay in registers, the lo parts go to this wave's LDS area.  The +8
    // offset of the codes, -8 * 2^-24 * (the group's query sum), times the
    // key's group scale and summed over the groups, is one more MFMA per key
    // block: A = the key's scales (k-slots 0..7 in lanes 0..31), B = the
    // offsets x 2^16 as f16 hi (slots 0..7, lanes 0..15) and lo parts
    // (lanes 16..31).
    half8_t bq_hi[NG];
    half8_t bcb = {};
    uint8_t* bqlo_lds = smem + S::BQLO + wave * NG * 1024 + lane * 16;
    {
        const bool live = c_used && has_row(c_rr);
        const float* qh = a.q + (live ? hbase(c_rr) + c_h : 0) * D;
        const float qscale = a.sm_scale * kLog2e;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            const float4 lo4 = *reinterpret_cast<const float4*>(qh + 32 * gi + 8 * q4);
            const float4 hi4 = *reinterpret_cast<const float4*>(qh + 32 * gi + 8 * q4 + 4);
            const float c8[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
            constexpr int order[8] = {0, 4, 1, 5, 2, 6, 3, 7};
            float sum = 0.0f;
            half8_t lo8;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float f = (k & 2) ? 0.0625f : 1.0f;
                const float v = live ? c8[order[k]] * qscale * f : 0.0f;
                const _Float16 h = _Float16(v);
                const _Float16 l = _Float16(v - float(h));
                bq_hi[gi][k] = h;
                lo8[k] = l;
                sum += (float(h) + float(l)) * ((k & 2) ? 16.0f : 1.0f);
            }
            *reinterpret_cast<half8_t*>(bqlo_lds + gi * 1024) = lo8;
            sum = quad_sum(sum);
            const float cb = -kOff * sum * (65536.0f / kTwo24);  // x 2^16: f16 normal range
            const _Float16 cb_hi = _Float16(cb), cb_lo = _Float16(cb - float(cb_hi));
            if (q4 == 0) bcb[gi] = cb_hi;
            if (q4 == 1) bcb[gi] = cb_lo;
        }
    }
    {  // B operands of the V-offset MFMA: the offset constant in column gi only
       // (written by wave 0, published by the first barrier)
        half8_t bc;
#pragma unroll
        for (int k = 0; k < 8; ++k) bc[k] = _Float16((k & 2) ? -16.0f * kOff / kTwo24 : -kOff / kTwo24);
        const half8_t zero = {};
        if (wave == 0)
            for (int gi = 0; gi < NG; ++gi)
                *reinterpret_cast<half8_t*>(smem + S::BRO + gi * 1024 + lane * 16) = n16 == gi ? bc : zero;
    }
    f32x4 o[NB];   // rows 4 q4 + i: the columns (row, head) 4 q4 + i
    f32x4 ro = {0.0f, 0.0f, 0.0f, 0.0f};  // column gi: the +8 offset of group gi's V codes
#pragma unroll
    for (int i = 0; i < NB; ++i) o[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, z_run = 0.0f;  // column n16's
    int a_exp = 0;  // the context operand's exponent (mfma_common.h); wave-uniform
    uint32_t win_lo = f16_bits_pow2(-8), win_hi = f16_bits_pow2(9);

    // ds_read_b64_tr_b4 row of this lane: key K(q4, e) for e = n16 & 7,
    // K(q, e) = 4q + e (e < 4) or 16 + 4q + e - 4, channel half n16 >> 3.
    const int e7 = n16 & 7;
    const int tr_key = e7 < 4 ? 4 * q4 + e7 : 16 + 4 * q4 + e7 - 4;
    const int tr_off = tr_key * RB + 8 * (n16 >> 3);

    for (int t = 0; t < n_tiles; ++t) {
        const int t0 = j0 + kSub * t;  // first key of the tile
        uint8_t* kt = smem + (t % kSlots) * S::SLOT;
        uint8_t* vt = kt + S::TILE;
        if (copier) {
            // own run of tile t landed: at most the later tiles' copies are outstanding
            if (t + 2 < n_tiles) wait_vmcnt<2 * S::RUN_INSTR>();
            else if (t + 1 < n_tiles) wait_vmcnt<S::RUN_INSTR>();
            else wait_vmcnt<0>();
        }
        // rows past the group's last key may hold any bytes (a NaN scale among
        // them) that must not meet p = 0: zero their V scales (own run only)
        if (wave == 2 || wave == 3) {
            const int r = 16 * run + lane;
            if (lane < 16 && t0 + r >= jg1) {
#pragma unroll
                for (int i = 0; i < D / 16; i += 4) *reinterpret_cast<uint32_t*>(vt + r * RB + SOFF + i) = 0u;
            }
        }
        barrier_lds_only();  // tile t staged for every wave; every wave is done with tile t - 1
        if (copier && t + kSlots - 1 < n_tiles) {
            issue(t + kSlots - 1, next_page);  // into the slot of tile t - 1
            if (t + kSlots < n_tiles) next_page = run_page(t + kSlots);
        }
        const int vmin = min(L[0] - t0, has_row(1) ? L[1] - t0 : kSub);  // fewest valid keys of the two rows
        const int vmax_rows = max(L[0] - t0, has_row(1) ? L[1] - t0 : 0);
        if (!has_row(0) || vmax_rows <= 0) continue;  // both rows' keys end before the tile

        // ---- scores: two 16-key blocks; lane holds keys 16 kb + 4 q4 + i of
        // column n16; hi and lo parts accumulate in one MFMA chain per group
        float sc[2][4];
        {
            uint32_t kc[2][NG];
#pragma unroll
            for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    kc[kb][gi] = *reinterpret_cast<const uint32_t*>(kt + (16 * kb + n16) * RB + 16 * gi + 4 * q4);
            u32x4 ks[2][4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    ks[kb][i] = *reinterpret_cast<const u32x4*>(kt + (16 * kb + 4 * q4 + i) * RB + SOFF);
            float acc[2][4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {  // the offset term: sum over groups of scale x offset
                u32x4 sk = *reinterpret_cast<const u32x4*>(kt + (16 * kb + n16) * RB + SOFF);
                if (NG < 8) sk = u32x4{sk[0], sk[1], 0u, 0u};
                const f32x4 b = mfma(__builtin_bit_cast(half8_t, sk), bcb, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[kb][i] = b[i] * (1.0f / 65536.0f);
            }
            f32x4 dprev[2];
#pragma unroll
            for (int gi = 0; gi <= NG; ++gi) {
                f32x4 dcur[2];
                if (gi < NG) {
                    const half8_t blo = *reinterpret_cast<const half8_t*>(bqlo_lds + gi * 1024);
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        const half8_t ka = unpack8(kc[kb][gi]);
                        dcur[kb] = mfma(ka, blo, mfma(ka, bq_hi[gi], f32x4{0.0f, 0.0f, 0.0f, 0.0f}));
                    }
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
                for (int i = 0; i < 4; ++i) sc[kb][i] = acc[kb][i];
        }
        if (vmin < kSub) {  // keys at or past the lane's row's length
            asm volatile("" ::: "memory");
            const int valid = Lc - t0;
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

        // ---- online softmax per column (log2 units; the maximum moves by more
        // than 2^6 only); a column whose row has no key in the tile keeps its
        // state (its scores are all -inf)
        const float tmax = quad_max_nonan(max8f(sc)) * kTwo24;
        const bool move = tmax > m_run + kRescale;  // the first tile with keys moves it from -inf
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
            for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * q4 + i, 64);  // o rows 4 q4 + i are columns
#pragma unroll
            for (int blk = 0; blk < NB; ++blk)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[blk][i] *= al[i];
#pragma unroll
            for (int i = 0; i < 4; ++i) ro[i] *= al[i];
        }
        float p[2][4];
        {
            // while a column's maximum is -inf all its scores so far are -inf: p = 0
            const float m_ref = m_run == -INFINITY ? 0.0f : m_run;
            const float nm0 = float(a_exp) - m_ref, nm4 = nm0 - 4.0f;  // p * 2^a_exp; slots 2,3,6,7 / 16
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[kb][i] = __builtin_amdgcn_exp2f(fmaf(sc[kb][i], kTwo24, (i & 1) ? nm4 : nm0));
                    z_run = (i & 1) ? fmaf(16.0f, p[kb][i], z_run) : z_run + p[kb][i];
                }
        }

        // ---- context per group: A = the columns' weights times the keys' V
        // scales of the group (slot 2 r: key 4 q4 + r, slot 2 r + 1: key
        // 16 + 4 q4 + r), B = the group's V codes
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            u32x4 w;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                w[r] = (gi & 1) ? ctx_pair<1>(p[0][r], p[1][r], vsa[r][gi >> 1], vsb[r][gi >> 1])
                                : ctx_pair<0>(p[0][r], p[1][r], vsa[r][gi >> 1], vsb[r][gi >> 1]);
            const half8_t av = __builtin_bit_cast(half8_t, w);
            ro = mfma(av, *reinterpret_cast<const half8_t*>(smem + S::BRO + gi * 1024 + lane * 16), ro);
            o[2 * gi] = mfma(av, unpack8(uint32_t(cv[gi][0])), o[2 * gi]);
            o[2 * gi + 1] = mfma(av, unpack8(uint32_t(cv[gi][1])), o[2 * gi + 1]);
        }
    }

    // ---- the partials, straight from registers: o rows 4 q4 + i are the
    // columns (row, head) 4 q4 + i
#pragma unroll
    for (int rr = 0; rr < kRowsWave; ++rr)
        if (has_row(rr) && n_keys(rr) == 0) write_empty(rr);
    z_run = quad_sum(z_run);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int col = 4 * q4 + i;
        float rov[NG];  // group gi's offset of row col: column gi of ro
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) rov[gi] = __shfl(ro[i], 16 * q4 + gi, 64);
        const int rr = col >= G ? 1 : 0, h = col - rr * G;
        if (col < kRowsWave * G && has_row(rr) && n_keys(rr) > 0) {
            float* dst = a.part_acc + ((hbase(rr) + h) * Sn + s) * D + n16;
#pragma unroll
            for (int blk = 0; blk < NB; ++blk) dst[16 * blk] = (o[blk][i] + rov[blk >> 1]) * kTwo24;
        }
    }
    if (q4 == 0 && c_used && has_row(c_rr) && n_keys(c_rr) > 0) {
        const int64_t hb = hbase(c_rr);
        a.part_m[(hb + c_h) * Sn + s] = (m_run - float(a_exp)) * kLn2;
        a.part_z[(hb + c_h) * Sn + s] = z_run;
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
