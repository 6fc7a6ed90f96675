// decode_q4_mfma.hip -- split-K decode over the 4-bit Hadamard-32 cache with
// matrix cores (gfx950 v_mfma_f32_16x16x32_f16).
//
// Method: TensorFold issue "qwen27 CUDA: an opt-in 4-bit attention cache",
// section "What it is" (attend in rotated space over the 4-bit cache in
// chunks, merge in order); colibri pull request "KV cache quantization: fp8
// (KV8) + 4-bit TurboQuant", split-T commit (partial blocks per (head,
// split) writing (cl[K], m, z)).  The query arrives rotated (kvq_rotate_q).
//
// Why matrix cores: per (key, KV head) the G = 6 query heads of a group need
// 2 x 6 x 256 multiply-adds against only 288 bytes of cache, which the fp32
// vector units cannot keep up with at HBM speed.  With the heads as the
// 16-wide M dimension the score and context products become 16x16x32 MFMAs,
// and the vector units are left with unpacking, scaling and the softmax.
//
// Workgroup = 4 (or, for splits of at most 1024 keys, 8) waves = (split s,
// KV head g, sequence b); each wave streams its own contiguous share of the
// split in 32-key sub-tiles and keeps its own online softmax; the waves'
// results are merged in LDS at the end into one partial.
//
// Per sub-tile:
//  * DMA: the sub-tile's K and V rows (two 16-row page runs per pool) are
//    copied global -> LDS with global_load_lds_dwordx4 (non-temporal: each
//    row is read once) into per-wave K and V rings of two sub-tiles each.
//    A slot is refilled with sub-tile t + 2 as soon as everything the
//    scores (K) or the context (V) read from it is in registers, so about
//    two sub-tiles per pool are in flight; completion is awaited with
//    s_waitcnt vmcnt.  The byte offsets of the wave's page runs are resolved
//    in the prologue into lane registers (lane r holds run r) and read back
//    with readlane when a copy is issued; the query is loaded after the
//    first copies are issued, so they wait for the page table only.
//  * Scores: for each 16-key block and 32-channel group, A = the keys' codes
//    (lane (key n, quarter q) holds code dword 4*group + q of key n), B = the
//    pre-scaled query split into f16 hi + lo parts (for groups of at most 8
//    heads, hi in B columns 0..7 and lo in 8..15: one MFMA).  Codes enter
//    as f16 subnormals: (nibble ^ 8) masked into place is (code + 8) * 2^-24
//    (or x16 for the high nibble of a byte, compensated in B), so unpacking a
//    dword of 8 codes takes 5 integer ops.  The +8 offset is removed by the
//    MFMA's C input (-8 * 2^-24 * sum of the group's query), and the group's
//    fp16 scale is applied per key with one mixed-precision FMA.  Both key
//    blocks' MFMAs of a group are issued before the previous group's FMAs.
//  * Softmax: lane (head h, quarter q) holds 8 scores of head h; the running
//    maximum only moves when a tile exceeds it by more than 2^6, so the
//    accumulators are rescaled a handful of times per split, not per tile.
//  * Context: ds_read_b64_tr_b4 transposes a 16x16 tile of nibbles so that
//    lane (channel n, quarter q) receives channel n of the 8 keys it needs
//    as MFMA k-slots; the same unpack makes the B operand.  A = P times the
//    keys' V scale (f16).  For groups of at most 8 heads A rows 8..15 repeat
//    heads 0..7, so one A operand carries the scales of a pair of groups
//    (rows 0..7 the even group, 8..15 the odd), and the +8 offset is summed
//    in one accumulator per pair (an MFMA against a constant B) and added
//    to the output once, at the end.
#include "mfma_common.h"

namespace kvq {
namespace {

using namespace mx;

constexpr int kEightWaveSplit = 1024;  // splits up to this many keys use 8-wave workgroups
constexpr int kSub = 32;          // keys per sub-tile
constexpr int kMaxRuns = 128;     // 16-key runs per wave (split_keys <= 8192)
constexpr float kRescale = 6.0f;  // log2 headroom before the running max moves

template <int D, int W, int BITS = 4>
struct Shape {
    static constexpr int NG = D / 32;               // 32-channel groups per row
    static constexpr int GB = 4 * BITS;             // code bytes of a group (16, 24 or 32)
    static constexpr int SOFF = NG * GB;            // byte offset of the fp16 scales in a row
    static constexpr int RB = SOFF + D / 16;        // row bytes
    static constexpr int NB = D / 16;               // 16-channel output blocks
    static constexpr int RUN = 16 * RB;             // bytes of 16 rows (one run)
    static constexpr int RUN_INSTR = (RUN / 16 + 63) / 64;  // 16-byte DMA instructions per run
    static constexpr int TILE = kSub * RB;          // bytes of a sub-tile, one pool
    static constexpr int HALF = 2 * RUN_INSTR;      // DMA instructions of a sub-tile, one pool
    static constexpr int WAVE_LDS = 4 * TILE;       // K ring (2 tiles) then V ring (2 tiles)
    static constexpr int LDS = W * WAVE_LDS;
};

// Copies one 16-row run (RUN bytes) from global to LDS.
template <int D, int BITS>
__device__ __forceinline__ void dma_run(const uint8_t* src, uint32_t lds, int lane) {
    using S = Shape<D, 4, BITS>;  // the run geometry does not depend on the wave count
#pragma unroll
    for (int i = 0; i < S::RUN_INSTR; ++i) {
        const int chunk = i * 64 + lane;
        if (i + 1 < S::RUN_INSTR || chunk < S::RUN / 16)
            dma16<true>(src, uint32_t(chunk * 16), lds + uint32_t(i * 1024));  // each row is read once
    }
}

// 8 codes of an 8-bit row as MFMA k-slots (e0,e4) (e1,e5) (e2,e6) (e3,e7),
// element e = byte e of the two dwords, each the f16 subnormal
// (code + 128) * 2^-24: flipping bit 7 turns two's complement into offset
// binary, and a byte permute puts each byte under a zero byte.
__device__ __forceinline__ half8_t unpack8_b8(u32x2 w) {
    const uint32_t x0 = w[0] ^ 0x80808080u, x1 = w[1] ^ 0x80808080u;
    const u32x4 r = {__builtin_amdgcn_perm(x1, x0, 0x0C040C00u), __builtin_amdgcn_perm(x1, x0, 0x0C050C01u),
                     __builtin_amdgcn_perm(x1, x0, 0x0C060C02u), __builtin_amdgcn_perm(x1, x0, 0x0C070C03u)};
    return __builtin_bit_cast(half8_t, r);
}

// 8 codes of a 6-bit row as MFMA k-slots (c0,c4) (c1,c5)x16 (c2,c6) (c3,c7)x16
// (the 4-bit order), each the f16 subnormal (code + 32) * 2^-24 (x16 where
// marked): w holds the codes' low nibbles laid out as 4-bit codes (unsigned
// here), hb their high two-bit fields (code i at bits 2i..2i+1; flipping
// bit 1 of a field turns two's complement into offset binary), placed above
// each nibble.
__device__ __forceinline__ half8_t unpack8_b6(uint32_t w, uint32_t hb) {
    const uint32_t w2 = w >> 8;
    const uint32_t e = __builtin_amdgcn_perm(0u, hb ^ 0xAAAAu, 0x0C010C00u);  // fields of codes 0-3 | 4-7 << 16
    const u32x4 r = {(w & 0x000F000Fu) | ((e << 4) & 0x00300030u), (w & 0x00F000F0u) | ((e << 6) & 0x03000300u),
                     (w2 & 0x000F000Fu) | (e & 0x00300030u), (w2 & 0x00F000F0u) | ((e << 2) & 0x03000300u)};
    return __builtin_bit_cast(half8_t, r);
}

// The same for the context operand: nib = 8 keys' low nibbles of one channel
// (element e in nibble e, as ds_read_b64_tr_b4 delivers them), h0 / h1 = the
// same keys' two-bit fields, offset binary, in bits 0..1 of byte e of h0
// (e < 4) or of byte e - 4 of h1.
__device__ __forceinline__ half8_t unpack8_b6_ctx(uint32_t nib, uint32_t h0, uint32_t h1) {
    const uint32_t n2 = nib >> 8;
    const u32x4 r = {(__builtin_amdgcn_perm(h1, h0, 0x0C040C00u) << 4) | (nib & 0x000F000Fu),
                     (__builtin_amdgcn_perm(h1, h0, 0x0C050C01u) << 8) | (nib & 0x00F000F0u),
                     (__builtin_amdgcn_perm(h1, h0, 0x0C060C02u) << 4) | (n2 & 0x000F000Fu),
                     (__builtin_amdgcn_perm(h1, h0, 0x0C070C03u) << 8) | (n2 & 0x00F000F0u)};
    return __builtin_bit_cast(half8_t, r);
}

// BITS = 4: the 4-bit format; BITS = 8: the 8-bit block format (byte codes,
// same rows of codes then fp16 scales, same arithmetic with offset 128);
// BITS = 6: the 6-bit block format (per group 16 bytes of low nibbles laid
// out as the 4-bit codes, then 8 bytes of high two-bit fields; offset 32).
// STEP (kvq_decode_step): the query arrives unrotated and is rotated here,
// and the wave whose key range holds position seq_lens[b] - 1 first stores
// token b's K and V rows there (the store kernel's encoder, so the bytes are
// the same), before its own copy of that row: each wave copies only its own
// rows, so no other wave of the launch reads them.
template <int D, int W, bool PACK, int BITS, bool STEP = false>
__global__ __launch_bounds__(W * 64, BITS == 4 ? 2 : 1) void decode_q4_mfma(const uint8_t* __restrict__ k_pool,
                                                                  const uint8_t* __restrict__ v_pool, int H,
                                                                  int page_size, int num_pages, DecodeArgs a) {
    using S = Shape<D, W, BITS>;
    constexpr int NG = S::NG, RB = S::RB, NB = S::NB, SOFF = S::SOFF, GB = S::GB;
    static_assert(BITS == 4 || BITS == 6 || BITS == 8, "4-, 6- or 8-bit codes");
    constexpr float kOff = BITS == 4 ? 8.0f : (BITS == 6 ? 32.0f : 128.0f);  // code offset of the f16 subnormals
    constexpr bool X16 = BITS != 8;  // 4 and 6 bits: k-slots 2,3,6,7 carry x16 (nibble in bits 4..7)
    __shared__ __attribute__((aligned(16))) uint8_t smem[S::LDS];

    int s, g, b;
    if (!decode_block(a, H, s, g, b)) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches per wave
    const int n16 = lane & 15, q4 = lane >> 4;  // MFMA column / row-quarter of this lane
    const int G = a.n_q_heads / H;
    const int Sn = a.n_splits;
    const int j0 = s * a.split_keys;
    const int64_t hb = int64_t(b) * a.n_q_heads + int64_t(g) * G;

    // This wave's keys: a contiguous quarter of the split.
    const int kq = a.split_keys / W;
    const int w0 = j0 + wave * kq;
    int T = a.seq_lens[b];  // first: its latency overlaps the loads below

    // Byte offset (within a pool) of each 16-row run of this wave's quarter:
    // lane l holds run l in the first register and run 64 + l in the second.
    // Resolved before the sequence length is known: positions are clamped to
    // the start of the 16-row run holding max_seq_len - 1 (a run never
    // crosses a page, page_size being a multiple of 16) and pages to the
    // pool, so every copy stays in bounds; rows past the sequence's end are
    // masked in the scores.
    const int32_t* pt = a.page_table + (a.rows ? 0 : int64_t(b) * a.max_pages);
    const int n_runs = kq / 16;
    const int last_pos = a.max_seq_len > 0 ? (a.max_seq_len - 1) & ~15 : 0;
    int64_t roff[2] = {0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (h == 1 && n_runs <= 64) break;
        const int r = min(lane + 64 * h, n_runs - 1);  // lanes past the last run repeat it
        const int pos = min(w0 + 16 * r, last_pos);
        int page = pt[pos / page_size];
        page = page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
        roff[h] = ((int64_t(page) * H + g) * page_size + pos % page_size) * RB;
    }

    T = T < 0 ? 0 : (T > a.max_seq_len ? a.max_seq_len : T);
    const int j1 = min(j0 + a.split_keys, T);
    if (j0 >= j1) {  // split past the end: an empty partial
        for (int i = tid; i < G * D; i += W * 64) a.part_acc[((hb + i / D) * Sn + s) * D + i % D] = 0.0f;
        if (tid < G) {
            a.part_m[(hb + tid) * Sn + s] = -INFINITY;
            a.part_z[(hb + tid) * Sn + s] = 0.0f;
        }
        return;
    }
    const int w1 = min(w0 + kq, j1);
    const int n_keys = w1 > w0 ? w1 - w0 : 0;
    const int n_sub = (n_keys + kSub - 1) / kSub;

    // STEP: store token b's K and V rows at position T - 1 if this wave's
    // keys hold it; the row must be in the L2 (the stores acknowledged:
    // vmcnt(0)) before this wave copies it.  vmcnt counts stores too, but an
    // older store still outstanding can only make the copies' count-based
    // waits wait longer, never let one pass early: a load completes before
    // every later load, so while it is outstanding all later loads are too.
    // A position whose page is outside the pool is not stored (kvq_store
    // skips such a slot too).
    const int pos_new = T - 1;
    const bool storer = STEP && T > 0 && pos_new >= w0 && pos_new < w1;  // wave-uniform
    const int t_new = storer ? (pos_new - w0) / kSub : -1;              // the row's sub-tile
    auto store_token = [&](bool wait) {
        const int page = pt[pos_new / page_size];
        if (page >= 0 && page < num_pages) {
            const int64_t row = (int64_t(page) * H + g) * page_size + pos_new % page_size;
            const int64_t src = (int64_t(b) * H + g) * D + 4 * lane;
            const void* const ptr[2] = {a.step_k, a.step_v};
            const int64_t idx[2] = {src, src};
            float x[2][4];
            load4n_dyn<2>(a.step_kv_dt, ptr, idx, x);
            encode_blk_quad<BITS>(x[0], const_cast<uint8_t*>(k_pool) + row * RB, D, lane, lane);
            encode_blk_quad<BITS>(x[1], const_cast<uint8_t*>(v_pool) + row * RB, D, lane, lane);
        }
        if (wait) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
    // Rows of sub-tiles 0 and 1 are copied just below: store and wait first.
    if (storer && t_new <= 1) store_token(true);

    uint8_t* ring = smem + wave * S::WAVE_LDS;  // K tiles 0, 1 then V tiles 0, 1
    const uint32_t lds0 = lds_addr(ring);
    auto run_at = [&](int r) -> int64_t {  // r is wave-uniform
        const int64_t v = r < 64 ? roff[0] : roff[1];
        const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(v), r & 63);
        const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(uint64_t(v) >> 32), r & 63);
        return int64_t((uint64_t(hi) << 32) | lo);
    };
    // One pool's half of sub-tile t (two runs) into ring slot t & 1.
    auto issue = [&](const uint8_t* pool, int t, uint32_t ring_base) {
        const uint32_t dst = ring_base + uint32_t((t & 1) * S::TILE);
        const int64_t r0 = run_at(2 * t), r1 = run_at(2 * t + 1);
        wait_lgkm0();  // earlier LDS reads of this slot have completed
        dma_run<D, BITS>(pool + r0, dst, lane);
        dma_run<D, BITS>(pool + r1, dst + S::RUN, lane);
    };
    const uint32_t k_ring = lds0, v_ring = lds0 + uint32_t(2 * S::TILE);
    if (n_sub > 0) {
        issue(k_pool, 0, k_ring);
        issue(v_pool, 0, v_ring);
    }
    if (n_sub > 1) {
        issue(k_pool, 1, k_ring);
        issue(v_pool, 1, v_ring);
    }

    // The query of head n16 (log2-scaled later), loaded after the first
    // copies are issued: the copies then wait only for the page-table
    // reads, not for the query's 16 KB per wave from L2 as well (when the
    // query is used, the first copies are needed anyway).
    // PACK (groups of at most 8 heads): B columns 0..7 carry the query's f16
    // hi part and columns 8..15 its lo part, so one MFMA per group does both.
    const int hcol = PACK ? (n16 & 7) : n16;  // the head this lane's B column holds
    const bool live = hcol < G;
    float4 qv[NG][2];
    if constexpr (STEP) {  // rotated here, bit for bit as kvq_rotate_q rotates it (PACK only)
        static_assert(!STEP || PACK, "the step's rotation uses the packed columns");
        // lane column n16 loads groups 2k + (n16 >> 3): the two column halves
        // hold the same head (PACK), so each rotates half the groups
        const int64_t qrow = (hb + (live ? hcol : 0)) * D + 32 * (n16 >> 3);
        const void* ptr[NG];
        int64_t idx[NG];
#pragma unroll
        for (int n = 0; n < NG; ++n) {
            ptr[n] = a.step_q;
            idx[n] = qrow + 64 * (n >> 1) + 8 * q4 + 4 * (n & 1);
        }
        float xl[NG][4];
        load4n_dyn<NG>(a.step_q_dt, ptr, idx, xl);
        float x[NG / 2][8], y[NG][8];
#pragma unroll
        for (int k = 0; k < NG / 2; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[k][i] = xl[2 * k][i];
                x[k][4 + i] = xl[2 * k + 1][i];
            }
        rotate_q_packed<NG>(x, y, lane);
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            qv[gi][0] = make_float4(y[gi][0], y[gi][1], y[gi][2], y[gi][3]);
            qv[gi][1] = make_float4(y[gi][4], y[gi][5], y[gi][6], y[gi][7]);
        }
    } else {
        const float* qh = a.q + (hb + (live ? hcol : 0)) * D;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            qv[gi][0] = *reinterpret_cast<const float4*>(qh + 32 * gi + 8 * q4);
            qv[gi][1] = *reinterpret_cast<const float4*>(qh + 32 * gi + 8 * q4 + 4);
        }
    }
    // STEP, a later sub-tile holds the new row: store it now, while the first
    // copies land; the acknowledgement is awaited just before that sub-tile's
    // copy is issued (two sub-tiles ahead, in the loop).
    if (storer && t_new > 1) store_token(false);

    // B operands of the score MFMAs: pre-scaled query (log2 units) of head
    // n16 for the 8 channels that k-slots (q4, 0..7) of each group hold,
    // split into f16 hi + lo.  Slot order (c0,c4,c1,c5,c2,c6,c3,c7) of the
    // dword 8*q4..8*q4+7 of the group; slots 2,3,6,7 carry x16 in A, so /16 here.
    half8_t bq_hi[NG], bq_lo[PACK ? 1 : NG];
    f32x4 cbias[NG];
    {
        const float qscale = a.sm_scale * kLog2e;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            const float4 lo4 = qv[gi][0], hi4 = qv[gi][1];
            const float c8[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
            constexpr int order[8] = {0, 4, 1, 5, 2, 6, 3, 7};
            float sum = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float f = (X16 && (k & 2)) ? 0.0625f : 1.0f;
                const float v = live ? c8[order[k]] * qscale * f : 0.0f;
                const _Float16 h = _Float16(v);
                const _Float16 l = _Float16(v - float(h));
                if (PACK) {
                    bq_hi[gi][k] = (n16 & 8) ? l : h;
                } else {
                    bq_hi[gi][k] = h;
                    bq_lo[gi][k] = l;
                }
                sum += (float(h) + float(l)) * ((X16 && (k & 2)) ? 16.0f : 1.0f);
            }
            sum = quad_sum(sum);
            const float bias = -kOff * sum / kTwo24;
            const float cb = (PACK && (n16 & 8)) ? 0.0f : bias;  // the offset once, in the hi column
            cbias[gi] = f32x4{cb, cb, cb, cb};
        }
    }
    // Constant B of the context offset MFMA: -8 * 2^-24 (x16 on slots 2,3,6,7).
    half8_t bconst;
#pragma unroll
    for (int k = 0; k < 8; ++k) bconst[k] = _Float16((X16 && (k & 2)) ? -16.0f * kOff / kTwo24 : -kOff / kTwo24);

    f32x4 o[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) o[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // PACK: the +8 offset of the V codes, summed apart from o per pair of
    // groups (one MFMA per pair and sub-tile against the constant B; every
    // column of it holds the same value) and added to o once at the end.
    f32x4 ro[PACK ? NG / 2 : 1];
#pragma unroll
    for (int i = 0; i < (PACK ? NG / 2 : 1); ++i) ro[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY;  // running max (log2 units) of head n16
    float z_run = 0.0f;       // this lane's share of the running sum (of p * 2^a_exp)
    // The f16 context operand's exponent (mfma_common.h): p enters as p * 2^a_exp,
    // so the partial's maximum is m_run - a_exp.  Wave-uniform.
    int a_exp = 0;
    uint32_t win_lo = f16_bits_pow2(-8), win_hi = f16_bits_pow2(9);

    // tr_b4 row address of this lane: key K(q4, e) for e = n16 & 7, where
    // K(q, e) = 4q + e (e < 4) or 16 + 4q + e - 4, at channel half n16 >> 3.
    // (tr_b8: lane j of a 16-lane group receives byte j of the 8-byte reads of
    // lanes 2e + (j >> 3), e = 0..7, as its element e; so lane n16 reads key
    // K(q4, n16 >> 1) at channel offset 8 * (n16 & 1).)
    const int e7 = BITS != 8 ? (n16 & 7) : (n16 >> 1);
    const int tr_key = e7 < 4 ? 4 * q4 + e7 : 16 + 4 * q4 + e7 - 4;
    const int tr_off = tr_key * RB + (BITS != 8 ? 8 * (n16 >> 3) : 8 * (n16 & 1));
    // 6 bits: a tr_b8 read of the high-field block (8 bytes per key) whose
    // two source lanes 2e, 2e + 1 both read key K(q4, e) leaves byte n16 & 7
    // of each key's block in lane n16; lane n16 of block b takes it from lane
    // 4b + (n16 >> 2) of its 16 (byte 4b + (n16 >> 2) holds its channel's field,
    // at bits 2 * (n16 & 3)).
    const int e8 = n16 >> 1;
    const int hi_off = (e8 < 4 ? 4 * q4 + e8 : 16 + 4 * q4 + e8 - 4) * RB + 16;
    const int hi_src0 = 4 * ((lane & ~15) + (n16 >> 2));  // ds_bpermute byte address, block 0
    const uint32_t hi_shift = 2u * uint32_t(n16 & 3);

    // Waves that are further along drop their issue priority, so the two
    // workgroups on a CU stream their copies at the same pace to the end.
    __builtin_amdgcn_s_setprio(3);
    for (int t = 0; t < n_sub; ++t) {
        if (4 * t == n_sub) __builtin_amdgcn_s_setprio(2);
        if (2 * t == n_sub) __builtin_amdgcn_s_setprio(1);
        if (4 * t == 3 * n_sub) __builtin_amdgcn_s_setprio(0);
        // K of sub-tile t has landed once at most the halves issued after it
        // are outstanding: V_t, K_t+1, V_t+1.
        if (t + 1 < n_sub) wait_vmcnt<3 * S::HALF>();
        else wait_vmcnt<S::HALF>();
        const uint8_t* kt = ring + (t & 1) * S::TILE;
        uint8_t* vt = ring + (2 + (t & 1)) * S::TILE;
        const int valid = min(kSub, n_keys - t * kSub);

        // ---- scores: two 16-key blocks; lane holds keys 16*kb + 4*q4 + i of head n16.
        // Both blocks' MFMAs of group gi are issued before the scale FMAs of
        // group gi - 1 consume the previous results, so the matrix-core
        // latency is covered by independent work; each acc still sums the
        // groups in ascending order.
        float sc[2][4];
        {
            u32x4 ks[2][4];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    ks[kb][i] = *reinterpret_cast<const u32x4*>(kt + (16 * kb + 4 * q4 + i) * RB + SOFF);
            // 8 codes: 4 bits a dword of nibbles, 8 bits two dwords of bytes,
            // 6 bits a dword of low nibbles and 16 bits of high fields
            using KW = std::conditional_t<BITS == 8, u32x2, uint32_t>;
            KW kc[2][NG];
            uint32_t kh[2][BITS == 6 ? NG : 1];
#pragma unroll
            for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const uint8_t* rowp = kt + (16 * kb + n16) * RB + GB * gi;
                    if constexpr (BITS == 6) {
                        kc[kb][gi] = *reinterpret_cast<const uint32_t*>(rowp + 4 * q4);
                        kh[kb][gi] = *reinterpret_cast<const uint16_t*>(rowp + 16 + 2 * q4);
                    } else {
                        kc[kb][gi] = *reinterpret_cast<const KW*>(rowp + (GB / 4) * q4);
                    }
                }
            // Everything the scores read from the K slot is now in registers
            // (the copy's lgkmcnt wait sees to that): refill the slot with
            // sub-tile t + 2 before the MFMAs rather than after them.
            if (STEP && t + 2 == t_new) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the new row stored
            if (t + 2 < n_sub) issue(k_pool, t + 2, k_ring);
            float acc[2][4] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
            f32x4 dprev[2];
#pragma unroll
            for (int gi = 0; gi <= NG; ++gi) {
                f32x4 dcur[2];
                if (gi < NG) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        half8_t av;
                        if constexpr (BITS == 4) av = unpack8(kc[kb][gi]);
                        else if constexpr (BITS == 6) av = unpack8_b6(kc[kb][gi], kh[kb][BITS == 6 ? gi : 0]);
                        else av = unpack8_b8(kc[kb][gi]);
                        dcur[kb] = mfma(av, bq_hi[gi], cbias[gi]);
                        if (!PACK) dcur[kb] = mfma(av, bq_lo[PACK ? 0 : gi], dcur[kb]);
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
                for (int i = 0; i < 4; ++i) {
                    // PACK: column n16 ^ 8 holds the other part of the same head
                    // (DPP row rotate by 8, folded into the add as its first
                    // operand); a + b = b + a, so both columns agree.
                    sc[kb][i] = PACK ? row_xor8(acc[kb][i]) + acc[kb][i] : acc[kb][i];  // log2 units / 2^24
                }
        }
        if (valid < kSub) {  // only the last tile of a wave can be partial
            asm volatile("" ::: "memory");  // a real branch: keep the full tiles free of selects
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * kb + 4 * q4 + i >= valid) sc[kb][i] = -INFINITY;
        }

        // V of sub-tile t has landed once at most K_t+1, V_t+1, K_t+2 are outstanding.
        if (t + 2 < n_sub) wait_vmcnt<3 * S::HALF>();
        else if (t + 1 < n_sub) wait_vmcnt<2 * S::HALF>();
        else wait_vmcnt<0>();

        // In a partial tile (only a wave's last) the rows past the sequence's
        // end may hold any bytes -- a NaN scale among them -- which must not
        // meet p = 0 in the context products: zero their V scales in LDS.
        if (valid < kSub) {
            const int row = valid + lane;
            if (row < kSub) {
                uint8_t* srow = vt + row * RB + SOFF;
#pragma unroll
                for (int i = 0; i < D / 16; i += 4) *reinterpret_cast<uint32_t*>(srow + i) = 0u;
            }
        }

        // Everything the context reads from the V slot, into registers; the
        // slot is then refilled with sub-tile t + 2 before the softmax and
        // the context products run.
        i32x2 cv[NG][BITS == 4 ? 1 : 2];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            if constexpr (BITS == 4) {
                cv[gi][0] = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
                    (__attribute__((address_space(3))) i32x2*)(vt + tr_off + 16 * gi));
            } else if constexpr (BITS == 6) {
                cv[gi][0] = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
                    (__attribute__((address_space(3))) i32x2*)(vt + tr_off + GB * gi));
                cv[gi][1] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) i32x2*)(vt + hi_off + GB * gi));
            } else {
#pragma unroll
                for (int hb2 = 0; hb2 < 2; ++hb2)
                    cv[gi][hb2 % (BITS == 4 ? 1 : 2)] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (__attribute__((address_space(3))) i32x2*)(vt + tr_off + 32 * gi + 16 * hb2));
            }
        }
        // V scales of keys 4q+r and 16+4q+r, r = 0..3: all groups of each row
        u32x4 vsa[4], vsb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            vsa[r] = *reinterpret_cast<const u32x4*>(vt + (4 * q4 + r) * RB + SOFF);
            vsb[r] = *reinterpret_cast<const u32x4*>(vt + (16 + 4 * q4 + r) * RB + SOFF);
        }
        // The tile's largest V scale (lane: 4 scales of row lane / 2), for the
        // context operand's exponent window.
        const uint32_t vmax = [&] {
            const u32x2 w = *reinterpret_cast<const u32x2*>(vt + (lane >> 1) * RB + SOFF + (NG >= 8 ? 8 * (lane & 1) : 0));
            return max4_u16(w[0], w[1]);
        }();
        if (t + 2 < n_sub) issue(v_pool, t + 2, v_ring);

        // ---- online softmax over the tile (per head = per column n16)
        // scores are finite or -inf (valid rows have finite scales), never NaN
        const float tmax = quad_max_nonan(max8f(sc)) * kTwo24;
        const bool move = tmax > m_run + kRescale || m_run == -INFINITY;
        const bool rebase = outside_window(vmax, win_lo, win_hi);  // rare: scales far from 1
        if (__builtin_amdgcn_ballot_w64(move) != 0ull || rebase) {
            const int a_new = rebase ? v_exponent_for(vmax, a_exp) : a_exp;
            const float m_new = move ? fmaxf(m_run, tmax) : m_run;
            // 0 when m_run = -inf; x 2^(a_new - a_exp) (x 1 when the exponent stays)
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new) * pow2i(a_new - a_exp);
            if (rebase) {  // wave-uniform values: kept in scalar registers
                a_exp = __builtin_amdgcn_readfirstlane(a_new);
                win_lo = __builtin_amdgcn_readfirstlane(f16_bits_pow2(-8 - a_exp));
                win_hi = __builtin_amdgcn_readfirstlane(f16_bits_pow2(9 - a_exp));
            }
            z_run *= alpha;
            m_run = m_new;
            float al[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * q4 + i, 64);  // rows 4*q4+i are heads
#pragma unroll
            for (int blk = 0; blk < NB; ++blk)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[blk][i] *= al[i];
            if (PACK) {
#pragma unroll
                for (int gp = 0; gp < NG / 2; ++gp)
#pragma unroll
                    for (int i = 0; i < 4; ++i) ro[gp][i] *= al[i];
            }
        }
        // p for keys of slots 2,3,6,7 (i = 1, 3) is taken /16 to undo the x16
        // those V codes carry.
        float p[2][4];
        const float nm0 = float(a_exp) - m_run, nm4 = nm0 - 4.0f;  // p * 2^a_exp
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool x16 = X16 && (i & 1);  // 4- and 6-bit slots 2,3,6,7 carry x16 in B
                p[kb][i] = __builtin_amdgcn_exp2f(fmaf(sc[kb][i], kTwo24, x16 ? nm4 : nm0));
                z_run = x16 ? fmaf(16.0f, p[kb][i], z_run) : z_run + p[kb][i];
            }
        half2_t pp[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pp[r] = half2_t{_Float16(p[0][r]), _Float16(p[1][r])};

        // ---- context: per group, two 16-channel blocks.  A row n16 holds head
        // n16 (or, PACK, head n16 & 7: rows 8..15 repeat heads 0..7).  PACK
        // gives rows 0..7 the scales of the even group of a pair and rows
        // 8..15 those of the odd group, so one A operand serves both groups:
        // an even group's outputs are read from rows 0..7, an odd group's
        // from rows 8..15, and the other rows are discarded.
        const uint32_t psel_pair = (n16 & 8) ? 0x07060302u : 0x05040100u;
        half8_t av;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            // scale pair (key 4q+r, key 16+4q+r) of group gi, r = 0..3
            if (!PACK || (gi & 1) == 0) {
                const uint32_t psel = PACK ? psel_pair : ((gi & 1) ? 0x07060302u : 0x05040100u);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t pair = __builtin_amdgcn_perm(vsb[r][gi >> 1], vsa[r][gi >> 1], psel);
                    const half2_t w = pp[r] * __builtin_bit_cast(half2_t, pair);
                    av[2 * r] = w[0];
                    av[2 * r + 1] = w[1];
                }
                if (PACK) ro[gi >> 1] = mfma(av, bconst, ro[gi >> 1]);
            }
            half8_t b0, b1;
            if constexpr (BITS == 4) {
                b0 = unpack8(uint32_t(cv[gi][0][0]));
                b1 = unpack8(uint32_t(cv[gi][0][1]));
            } else if constexpr (BITS == 6) {
                // high fields of block b from lane 4b + (n16 >> 2) of this 16,
                // the field of channel n16 & 3 of its byte, offset binary
                uint32_t hf[2][2];
#pragma unroll
                for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const uint32_t v = uint32_t(
                            __builtin_amdgcn_ds_bpermute(hi_src0 + 16 * b2, int(cv[gi][BITS == 6 ? 1 : 0][k])));
                        hf[b2][k] = ((v >> hi_shift) & 0x03030303u) ^ 0x02020202u;
                    }
                b0 = unpack8_b6_ctx(uint32_t(cv[gi][0][0]), hf[0][0], hf[0][1]);
                b1 = unpack8_b6_ctx(uint32_t(cv[gi][0][1]), hf[1][0], hf[1][1]);
            } else {
                b0 = unpack8_b8(__builtin_bit_cast(u32x2, cv[gi][0]));
                b1 = unpack8_b8(__builtin_bit_cast(u32x2, cv[gi][BITS == 4 ? 0 : 1]));
            }
            o[2 * gi] = mfma(av, b0, o[2 * gi]);
            if (!PACK) o[2 * gi] = mfma(av, bconst, o[2 * gi]);
            o[2 * gi + 1] = mfma(av, b1, o[2 * gi + 1]);
            if (!PACK) o[2 * gi + 1] = mfma(av, bconst, o[2 * gi + 1]);
        }
    }

    // ---- per-wave results: m (log2), z per head; o rows = heads 4*q4 + i.
    // Each wave puts its G live head rows, m and z in its own ring (its
    // copies have all landed and it has read them: no barrier needed before
    // the writes); after one barrier every thread forms the weights
    // exp2(m_w - M) of its head and sums each output channel over the waves
    // in wave order.
    static_assert(16 * D * 4 + 2 * 16 * 4 <= S::WAVE_LDS, "per-wave results fit the wave's ring");
    z_run = quad_sum(z_run);
    auto wo = [&](int w) { return reinterpret_cast<float*>(smem + w * S::WAVE_LDS); };  // [16][D]
    auto wm = [&](int w) { return wo(w) + 16 * D; };                                     // [16]
    auto wz = [&](int w) { return wo(w) + 16 * D + 16; };                                // [16]
    {
        float* mine = wo(wave);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * q4 + i, h = PACK ? (row & 7) : row;
            if (h < G) {
#pragma unroll
                for (int blk = 0; blk < NB; ++blk) {
                    // PACK: group blk / 2 is read from rows 0..7 if even, 8..15 if odd
                    if (!PACK || ((blk >> 1) & 1) == (row >> 3))
                        mine[h * D + 16 * blk + n16] = (PACK ? o[blk][i] + ro[blk >> 2][i] : o[blk][i]) * kTwo24;
                }
            }
        }
        if (lane < 16) {
            wm(wave)[lane] = n_keys > 0 ? m_run - float(a_exp) : -INFINITY;
            wz(wave)[lane] = n_keys > 0 ? z_run : 0.0f;
        }
    }
    __syncthreads();
    for (int i = tid; i < G * D; i += W * 64) {
        const int h = i / D, c = i % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w) M = fmaxf(M, wm(w)[h]);
        float acc = 0.0f, Z = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const float zw = wz(w)[h];
            const float f = zw > 0.0f ? __builtin_amdgcn_exp2f(wm(w)[h] - M) : 0.0f;
            acc += wo(w)[h * D + c] * f;
            Z += zw * f;
        }
        store_wt(&a.part_acc[((hb + h) * Sn + s) * D + c], acc);
        if (c == 0) {
            store_wt(&a.part_m[(hb + h) * Sn + s], M * kLn2);
            store_wt(&a.part_z[(hb + h) * Sn + s], Z);
        }
    }
}

}  // namespace

bool decode_q4_mfma_supported(const Q4Pool& pool, const DecodeArgs& a) {
    const int G = a.n_q_heads / pool.n_kv_heads;
    // 8- and 6-bit rows are 272 and 208 bytes at head_dim 256 (16-byte aligned scale chunks)
    const bool dims = pool.bits == 4 ? (pool.head_dim == 128 || pool.head_dim == 256)
                                     : ((pool.bits == 8 || pool.bits == 6) && pool.head_dim == 256);
    return dims && G >= 1 && G <= 16 && pool.page_size % 16 == 0 && a.split_keys % 128 == 0 &&
           a.split_keys / 4 <= 16 * kMaxRuns;
}

// Workgroups of 4 waves, each streaming a quarter of a split of more than
// 1024 keys; splits of 512 or 1024 keys (short contexts, where fewer and
// larger splits would leave CUs idle) are shared by 8 waves, so each wave
// has half as many tiles and a short context's copies are all in flight at
// once.  The 8- and 6-bit formats always use 4 waves: their rings take 34 and
// 26 KB per wave.  The choice depends on split_keys and the format alone, never on the
// batch, so a sequence's partials do not depend on the sequences beside it.
bool decode_q4_mfma_step_supported(const Q4Pool& pool, const DecodeArgs& a) {
    // 4 bits: the 4-wave kernel (splits over 1024 keys); 8 and 6 bits always run on 4 waves
    return decode_q4_mfma_supported(pool, a) && pool.head_dim == 256 && a.n_q_heads / pool.n_kv_heads <= 8 &&
           (pool.bits != 4 || a.split_keys > kEightWaveSplit) && a.rows == 0;
}

hipError_t launch_decode_q4_mfma(const Q4Pool& pool, const DecodeArgs& a, hipStream_t s) {
    const dim3 grid = decode_grid(a, pool.n_kv_heads);
    const bool eight = a.split_keys <= kEightWaveSplit;
    const bool pack = a.n_q_heads / pool.n_kv_heads <= 8;
    if (a.step_k) {  // kvq_decode_step: head_dim 256, packed columns, 4 waves (the caller checks it)
        if (!decode_q4_mfma_step_supported(pool, a)) return hipErrorInvalidValue;
        if (pool.bits == 8)
            decode_q4_mfma<256, 4, true, 8, true><<<grid, dim3(4 * 64), 0, s>>>(pool.k, pool.v, pool.n_kv_heads,
                                                                                pool.page_size, pool.num_pages, a);
        else if (pool.bits == 6)
            decode_q4_mfma<256, 4, true, 6, true><<<grid, dim3(4 * 64), 0, s>>>(pool.k, pool.v, pool.n_kv_heads,
                                                                                pool.page_size, pool.num_pages, a);
        else
            decode_q4_mfma<256, 4, true, 4, true><<<grid, dim3(4 * 64), 0, s>>>(pool.k, pool.v, pool.n_kv_heads,
                                                                                pool.page_size, pool.num_pages, a);
        return hipGetLastError();
    }
#define KVQ_LAUNCH(D_, W_, P_, B_)                                                                             \
    decode_q4_mfma<D_, W_, P_, B_><<<grid, dim3((W_) * 64), 0, s>>>(pool.k, pool.v, pool.n_kv_heads,          \
                                                                     pool.page_size, pool.num_pages, a)
#define KVQ_LAUNCH_W(D_, P_)             \
    if (eight) KVQ_LAUNCH(D_, 8, P_, 4); \
    else KVQ_LAUNCH(D_, 4, P_, 4)
    if (pool.bits == 8 || pool.bits == 6) {
        if (pool.head_dim != 256) return hipErrorInvalidValue;
        if (pool.bits == 8) {
            if (pack) KVQ_LAUNCH(256, 4, true, 8);
            else KVQ_LAUNCH(256, 4, false, 8);
        } else {
            if (pack) KVQ_LAUNCH(256, 4, true, 6);
            else KVQ_LAUNCH(256, 4, false, 6);
        }
        return hipGetLastError();
    }
    switch (pool.head_dim) {
        case 128:
            if (pack) { KVQ_LAUNCH_W(128, true); }
            else { KVQ_LAUNCH_W(128, false); }
            break;
        case 256:
            if (pack) { KVQ_LAUNCH_W(256, true); }
            else { KVQ_LAUNCH_W(256, false); }
            break;
        default: return hipErrorInvalidValue;
    }
#undef KVQ_LAUNCH_W
#undef KVQ_LAUNCH
    return hipGetLastError();
}

}  // namespace kvq
