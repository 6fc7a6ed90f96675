// decode_q4_pair.hip -- split-K decode over the 4-bit Hadamard-32 cache for
// head_dim 256 and groups of up to 8 query heads, with wave pairs that
// share each key tile by channel halves.
//
// Method: TensorFold issue "qwen27 CUDA: an opt-in 4-bit attention cache",
// section "What it is" (attend in rotated space over the 4-bit cache in
// chunks, merge in order); colibri pull request "KV cache quantization: fp8
// (KV8) + 4-bit TurboQuant", split-T commit (partial blocks per (head,
// split) writing (cl[K], m, z)).  The query arrives rotated (kvq_rotate_q).
//
// The single-wave design (decode_q4_mfma.hip) keeps a whole 256-channel
// context accumulator, the query operands of 8 groups and a 4-tile LDS ring
// of full 144-byte rows per wave, which caps it at two waves per SIMD; its
// per-tile work is a chain of dependent unpack -> MFMA -> FMA steps that two
// waves cannot hide.  Here a pair of waves shares each 32-key sub-tile: wave
// half h owns channels 128h .. 128h + 127 (groups 4h .. 4h + 3), so it copies
// only its 64 code bytes of each row plus the 16-byte scale chunk (80 of the
// 144 bytes), computes partial scores over its four groups, and keeps the
// context accumulator of its 128 channels.  The two partial score sets meet
// in LDS (each wave writes its own into the K slot it has just consumed),
// and both waves add them in the same order (half 0's + half 1's), so both
// run the identical online softmax.  Registers and LDS per wave halve, and
// four waves per SIMD fit.
//
// Where it pays: a pair spends more instructions per key than a single wave
// (both halves run the softmax, and the exchange adds LDS traffic and a
// barrier per tile), so once every CU is full of work the single-wave
// kernel, with fewer instructions per key, is as fast or faster (measured:
// 65 vs 61 us for a 262144-token, 2048-key-split layer).  For short splits
// (up to 1024 keys, e.g. 32K contexts) the doubled occupancy wins (16.2 vs
// 18.8 us for a 32768-token, 512-key-split layer), and the launcher takes
// this kernel there.  The choice depends on split_keys alone, never on the
// batch.
//
// Workgroup = 4 pairs = 8 waves = (split s, KV head g, sequence b); pair p
// streams the p-th quarter of the split, and the four pairs' results are
// combined in LDS at the end into one partial.  Per sub-tile and wave the
// steps are those of the single-wave kernel restricted to the wave's four
// groups: LDS DMA of the half-rows into K and V rings of two sub-tiles
// (the next sub-tile's K copied after the exchange, its V after the
// context: one sub-tile ahead, see the copy schedule below),
// score MFMAs with the codes as f16 subnormals and the +8 offset removed in
// the accumulator input, a lazily moving running maximum, and context MFMAs
// on ds_read_b64_tr_b4-transposed V codes.
#include "mfma_common.h"

namespace kvq {
namespace {

using namespace mx;

constexpr int kD = 256;
constexpr int kRB = 144;                    // row bytes in the pool
constexpr int kPitch = 80;                  // LDS row: 64 code bytes + the 16-byte scale chunk
constexpr int kSub = 32;                    // keys per sub-tile
constexpr int kSlot = kSub * kPitch;        // one sub-tile of one pool, one wave
constexpr int kWaveLds = 4 * kSlot;         // K slots 0, 1 then V slots 0, 1
constexpr int kPairs = 4;                   // pairs per workgroup
constexpr int kWaves = 2 * kPairs;
constexpr int kLds = kWaves * kWaveLds;     // 81920: two workgroups per CU
constexpr int kHalfInstr = 4;               // DMA instructions per sub-tile, one pool
constexpr int kMaxSplit = 1024;             // longer splits run on the single-wave kernel
constexpr int kMaxRuns = kMaxSplit / kPairs / 16;  // 16-key runs per pair
static_assert(kMaxRuns <= 64, "one lane register per run");
constexpr float kRescale = 6.0f;            // log2 headroom before the running max moves

// Epilogue scratch (reuses the rings once every pair is done).
constexpr int kEpiRows = 8;
static_assert(kPairs * kEpiRows * kD * 4 + 5 * kPairs * 16 * 4 <= kLds, "epilogue fits the rings");

__device__ __forceinline__ void barrier_lds() {
    // LDS writes of both waves visible, outstanding cache copies not waited for.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// STEP (kvq_decode_step): the query arrives unrotated and is rotated here,
// and the pair whose key range holds position seq_lens[b] - 1 first stores
// token b's K row (wave 0 of the pair) and V row (wave 1) there (the store
// kernel's encoder, so the bytes are the same).  Both waves of that pair
// copy both rows, so both stores complete before either copy: before the
// workgroup's first barrier if the row's sub-tile is copied in the
// prologue, else before the exchange barrier after which that sub-tile is
// copied.
template <bool STEP>
__global__ __attribute__((amdgpu_flat_work_group_size(kWaves * 64, kWaves * 64), amdgpu_waves_per_eu(4, 4)))
void decode_q4_pair(const uint8_t* __restrict__ k_pool, const uint8_t* __restrict__ v_pool, int H,
                    int page_size, int num_pages, DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];

    int s, g, b;
    if (!decode_block(a, H, s, g, b)) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = wave >> 1, h = wave & 1;  // channel half of this wave
    const int n16 = lane & 15, q4 = lane >> 4;
    const int G = a.n_q_heads / H;
    const int Sn = a.n_splits;
    const int j0 = s * a.split_keys;
    const int64_t hb = int64_t(b) * a.n_q_heads + int64_t(g) * G;

    const int kp = a.split_keys / kPairs;  // keys of this pair: a contiguous quarter
    const int w0 = j0 + pair * kp;
    int T = a.seq_lens[b];

    // Query of head hcol for this wave's groups; B columns 0..7 carry the
    // f16 hi part and 8..15 the lo part.
    const int hcol = n16 & 7;
    const bool live = hcol < G;
    float4 qv[4][2];
    // STEP: the unrotated query, rotated after the first copies are issued;
    // column n16 loads groups 2k + (n16 >> 3) of this half (columns n16 and
    // n16 ^ 8 hold the same head, so each rotates half the groups)
    float qraw[4][4];
    if constexpr (STEP) {
        const int64_t qrow = (hb + (live ? hcol : 0)) * kD + 128 * h + 32 * (n16 >> 3);
        const void* ptr[4];
        int64_t idx[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            ptr[n] = a.step_q;
            idx[n] = qrow + 64 * (n >> 1) + 8 * q4 + 4 * (n & 1);
        }
        load4n_dyn<4>(a.step_q_dt, ptr, idx, qraw);
    } else {
        const float* qh = a.q + (hb + (live ? hcol : 0)) * kD + 128 * h;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            qv[j][0] = *reinterpret_cast<const float4*>(qh + 32 * j + 8 * q4);
            qv[j][1] = *reinterpret_cast<const float4*>(qh + 32 * j + 8 * q4 + 4);
        }
    }

    // Pool row index of the first row of each 16-row run of the pair's
    // quarter (lane r: run r), clamped into the table and the pool as in the
    // single-wave kernel.  A row index fits 32 bits for pools up to 2^32 rows
    // (the launcher checks), so one register holds it; the byte offset is
    // formed in scalar registers when a copy is issued.
    const int32_t* pt = a.page_table + (a.rows ? 0 : int64_t(b) * a.max_pages);
    const int n_runs = kp / 16;
    const int last_pos = a.max_seq_len > 0 ? (a.max_seq_len - 1) & ~15 : 0;
    uint32_t rrow;
    {
        const int r = min(lane, n_runs - 1);
        const int pos = min(w0 + 16 * r, last_pos);
        int page = pt[pos / page_size];
        page = page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
        rrow = (uint32_t(page) * uint32_t(H) + uint32_t(g)) * uint32_t(page_size) + uint32_t(pos % page_size);
    }

    T = T < 0 ? 0 : (T > a.max_seq_len ? a.max_seq_len : T);
    const int j1 = min(j0 + a.split_keys, T);
    if (j0 >= j1) {  // split past the end: an empty partial
        for (int i = tid; i < G * kD; i += kWaves * 64) a.part_acc[((hb + i / kD) * Sn + s) * kD + i % kD] = 0.0f;
        if (tid < G) {
            a.part_m[(hb + tid) * Sn + s] = -INFINITY;
            a.part_z[(hb + tid) * Sn + s] = 0.0f;
        }
        return;
    }
    const int p1 = min(w0 + kp, j1);
    const int n_keys = p1 > w0 ? p1 - w0 : 0;  // pair-uniform
    const int n_sub = (n_keys + kSub - 1) / kSub;
    // s_barrier spans the workgroup, so every wave runs the loop as often as
    // pair 0 (which has the most keys); a pair past its own tiles only takes
    // part in the barriers.
    const int n_loop = (min(kp, j1 - j0) + kSub - 1) / kSub;

    // DMA of one 16-row run's half-rows: chunk c = 5 * row + part, part 0..3
    // the code bytes 64h + 16 part, part 4 the scale chunk (bytes 128..143).
    // Lanes 0..63 copy chunks 0..63, lanes 0..15 chunks 64..79; the LDS
    // destination of chunk c is 16c, so rows land at a pitch of 80 bytes.
    auto chunk_src = [&](int c) {
        const int row = c / 5, part = c % 5;
        return uint32_t(row * kRB + (part < 4 ? 64 * h + 16 * part : 128));
    };
    const uint32_t src_off0 = chunk_src(lane);
    uint8_t* ring = smem + wave * kWaveLds;
    uint8_t* pring = smem + (wave ^ 1) * kWaveLds;  // the other half's ring
    const uint32_t lds0 = lds_addr(ring);
    const uint32_t k_ring = lds0, v_ring = lds0 + uint32_t(2 * kSlot);
    auto run_at = [&](int r) -> uint64_t {  // r is wave-uniform
        return uint64_t(uint32_t(__builtin_amdgcn_readlane(rrow, r))) * kRB;
    };
    auto issue = [&](const uint8_t* pool, int t, uint32_t ring_base) {
        const uint32_t dst = ring_base + uint32_t((t & 1) * kSlot);
        const uint8_t* r0 = pool + run_at(2 * t);
        const uint8_t* r1 = pool + run_at(2 * t + 1);
        // The offset of chunks 64..79 is recomputed at each copy from a lane id
        // the compiler cannot hoist: kept across the loop it would be one
        // register too many and spill (a reload waits for every copy in flight).
        int l16 = lane & 15;
        asm volatile("" : "+v"(l16));
        const uint32_t src_off1 = chunk_src(64 + l16);
        wait_lgkm0();  // earlier LDS reads of this slot have completed
        // Code bytes are read once (non-temporal); the scale chunk is read by
        // both waves of the pair, the second time from the caches.
        dma16<true>(r0, src_off0, dst);
        if (lane < 16) dma16<false>(r0, src_off1, dst + 1024u);
        dma16<true>(r1, src_off0, dst + 1280u);
        if (lane < 16) dma16<false>(r1, src_off1, dst + 2304u);
    };
    // STEP: the new row (position T - 1) and the pair that stores it (wave h
    // of the pair: the K row if h = 0, the V row if h = 1); the stores must be
    // acknowledged (vmcnt(0)) before either wave of the pair copies the row.  vmcnt counts stores too, but an older store still
    // outstanding can only make the copies' count-based waits wait longer,
    // never let one pass early (a load completes before every later load).
    // A position whose page is outside the pool is not stored (kvq_store
    // skips such a slot too).
    const int pos_new = T - 1;
    const bool holds = STEP && T > 0 && pos_new >= j0 && pos_new < j1;  // workgroup-uniform
    const int t_new = holds ? ((pos_new - j0) % kp) / kSub : -1;       // the row's sub-tile
    const bool early = holds && t_new == 0;                            // copied in the prologue
    const bool storer = holds && pair == (pos_new - j0) / kp;  // both waves of the pair
    auto store_token = [&](bool wait) {
        const int page = pt[pos_new / page_size];
        if (page >= 0 && page < num_pages) {
            const int64_t row = (int64_t(page) * H + g) * page_size + pos_new % page_size;
            const int64_t src = (int64_t(b) * H + g) * kD + 4 * lane;
            const void* const ptr[1] = {h ? a.step_v : a.step_k};
            const int64_t idx[1] = {src};
            float x[1][4];
            load4n_dyn<1>(a.step_kv_dt, ptr, idx, x);
            encode_blk_quad<4>(x[0], const_cast<uint8_t*>(h ? v_pool : k_pool) + row * kRB, kD, lane, lane);
        }
        if (wait) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
    if (early) {  // both waves of the pair copy the row below: store, then a workgroup barrier
        if (storer) store_token(true);
        __syncthreads();
    }

    // Copy schedule: one sub-tile ahead.  Sub-tile 0 is copied here; sub-tile
    // t + 1's K after sub-tile t's exchange and its V after sub-tile t's
    // context.  A copy instruction stalls its wave until the memory system
    // accepts it, and at a launch's start every wave queues its copies at
    // once: with two sub-tiles ahead each wave waited ~4 us behind its 20 KB
    // before its first scores, though its first K had landed ~0.5 us after
    // issue.  With one ahead the first scores start once sub-tile 0 is
    // accepted (32768 keys at split 512: 14.1 vs 15.0 us per layer; 131072
    // keys at split 1024: 39.0 vs 40.5 us; the same bits).
    if (n_sub > 0) {
        issue(k_pool, 0, k_ring);
        issue(v_pool, 0, v_ring);
    }

    if constexpr (STEP) {  // rotated here, bit for bit as kvq_rotate_q rotates it
        float x[2][8], y[4][8];
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[k][i] = qraw[2 * k][i];
                x[k][4 + i] = qraw[2 * k + 1][i];
            }
        rotate_q_packed<4>(x, y, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            qv[j][0] = make_float4(y[j][0], y[j][1], y[j][2], y[j][3]);
            qv[j][1] = make_float4(y[j][4], y[j][5], y[j][6], y[j][7]);
        }
    }

    // Score B operands (pre-scaled query in log2 units, hi/lo by column) and
    // the accumulator input that removes the codes' +8 offset.
    half8_t bq[4];
    f32x4 cbias[4];
    {
        const float qscale = a.sm_scale * kLog2e;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 lo4 = qv[j][0], hi4 = qv[j][1];
            const float c8[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
            constexpr int order[8] = {0, 4, 1, 5, 2, 6, 3, 7};
            float sum = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float f = (k & 2) ? 0.0625f : 1.0f;
                const float v = live ? c8[order[k]] * qscale * f : 0.0f;
                const _Float16 hv = _Float16(v);
                const _Float16 lv = _Float16(v - float(hv));
                bq[j][k] = (n16 & 8) ? lv : hv;
                sum += (float(hv) + float(lv)) * ((k & 2) ? 16.0f : 1.0f);
            }
            sum = quad_sum(sum);
            const float cb = (n16 & 8) ? 0.0f : -8.0f * sum / kTwo24;
            cbias[j] = f32x4{cb, cb, cb, cb};
        }
    }
    half8_t bconst;
#pragma unroll
    for (int k = 0; k < 8; ++k) bconst[k] = _Float16((k & 2) ? -128.0f / kTwo24 : -8.0f / kTwo24);
    // STEP, a later sub-tile holds the new row: store it now; the
    // acknowledgement is awaited before the exchange barrier after which both
    // waves of the pair copy that sub-tile.
    if (storer && !early) store_token(false);

    f32x4 o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY;
    float z_run = 0.0f;  // of p * 2^a_exp
    // The f16 context operand's exponent (mfma_common.h): p enters as p * 2^a_exp
    // and the partial's maximum is m_run - a_exp.  Both halves of a pair copy the
    // row's whole scale chunk, so they take the same a_exp.
    int a_exp = 0;
    uint32_t win_lo = f16_bits_pow2(-8), win_hi = f16_bits_pow2(9);

    const int e7 = n16 & 7;
    const int tr_key = e7 < 4 ? 4 * q4 + e7 : 16 + 4 * q4 + e7 - 4;
    const int tr_off = tr_key * kPitch + 8 * (n16 >> 3);

    for (int t = 0; t < n_loop; ++t) {
        const bool act = t < n_sub;  // wave-uniform
        uint8_t* kt = ring + (t & 1) * kSlot;
        const uint8_t* vt = ring + (2 + (t & 1)) * kSlot;
        const int valid = min(kSub, n_keys - t * kSub);

        // ---- partial scores over this half's four groups (K of sub-tile t has
        // landed once at most V_t is outstanding)
        float sc[2][4];
        if (act) {
            wait_vmcnt<kHalfInstr>();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const uint8_t* arow = kt + (16 * kb + n16) * kPitch;
                float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {  // groups 2jj, 2jj + 1 share a scale dword
                    uint32_t ks[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        ks[i] = *reinterpret_cast<const uint32_t*>(kt + (16 * kb + 4 * q4 + i) * kPitch + 64 + 8 * h +
                                                                   4 * jj);
#pragma unroll
                    for (int j = 2 * jj; j < 2 * jj + 2; ++j) {
                        const uint32_t w = *reinterpret_cast<const uint32_t*>(arow + 16 * j + 4 * q4);
                        const f32x4 d = mfma(unpack8(w), bq[j], cbias[j]);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            acc[i] = fmaf(d[i], (j & 1) ? hi_half(ks[i]) : lo_half(ks[i]), acc[i]);
                    }
                }
                // column n16 ^ 8 holds the other (hi or lo) part of the same head
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[kb][i] = acc[i] + row_xor8(acc[i]);
            }
        }
        // ---- exchange through the consumed K slot; both halves add half 0's first
        float* mine = reinterpret_cast<float*>(kt);
        // The partner's slot, addressed from a lane id the compiler cannot hoist
        // (a hoisted address is one register too many across the loop).
        int lx = lane;
        asm volatile("" : "+v"(lx));
        const float* other = reinterpret_cast<const float*>(pring + (t & 1) * kSlot) + lx;
        if (act) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) mine[(4 * kb + i) * 64 + lane] = sc[kb][i];
        }
        if (STEP && storer && t + 1 == t_new) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // new row stored
        // One barrier per sub-tile: both halves' scores are in LDS, and each
        // half has finished reading the other's sub-tile t - 1 exchange (its
        // reads completed before it reached this barrier), so the slot of
        // sub-tile t - 1 may take sub-tile t + 1's K below.  Sub-tile t's
        // exchange (slot t & 1) is refilled only after the next barrier.
        barrier_lds();
        if (act) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x = other[(4 * kb + i) * 64];
                    sc[kb][i] = h == 0 ? sc[kb][i] + x : x + sc[kb][i];
                }
        }
        if (!act) continue;
        if (t + 1 < n_sub) issue(k_pool, t + 1, k_ring);  // into the slot of sub-tile t - 1

        if (valid < kSub) {
            asm volatile("" ::: "memory");
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * kb + 4 * q4 + i >= valid) sc[kb][i] = -INFINITY;
        }

        // V of sub-tile t has landed once at most K_t+1 is outstanding.
        if (t + 1 < n_sub) wait_vmcnt<kHalfInstr>();
        else wait_vmcnt<0>();

        if (valid < kSub) {  // rows past the end: zero their V scales
            const int row = valid + lane;
            if (row < kSub) {
                uint32_t* srow = reinterpret_cast<uint32_t*>(ring + (2 + (t & 1)) * kSlot + row * kPitch + 64);
#pragma unroll
                for (int i = 0; i < 4; ++i) srow[i] = 0u;
            }
        }
        // The tile's largest V scale, for the context operand's exponent window:
        // lane reads the scales of groups 4 (n16 >> 3) .. +3 of the key its
        // transposed code reads address (tr_off covers every key and half once;
        // reusing its address register costs no register across the loop).
        const uint32_t vmax = [&] {
            const u32x2 w = *reinterpret_cast<const u32x2*>(vt + tr_off + 64);
            return max4_u16(w[0], w[1]);
        }();

        // ---- online softmax (identical in both halves)
        float tmax = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                           fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
        tmax = quad_max(tmax) * kTwo24;
        const bool move = tmax > m_run + kRescale || m_run == -INFINITY;
        const bool rebase = outside_window(vmax, win_lo, win_hi);  // rare: scales far from 1
        if (__builtin_amdgcn_ballot_w64(move) != 0ull || rebase) {
            const int a_new = rebase ? v_exponent_for(vmax, a_exp) : a_exp;
            const float m_new = move ? fmaxf(m_run, tmax) : m_run;
            // x 2^(a_new - a_exp): x 1 when the exponent stays
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
            for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * q4 + i, 64);
#pragma unroll
            for (int blk = 0; blk < 8; ++blk)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[blk][i] *= al[i];
        }
        float p[2][4];
        const float nm0 = float(a_exp) - m_run, nm4 = nm0 - 4.0f;  // p * 2^a_exp
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[kb][i] = __builtin_amdgcn_exp2f(fmaf(sc[kb][i], kTwo24, (i & 1) ? nm4 : nm0));
                z_run = (i & 1) ? fmaf(16.0f, p[kb][i], z_run) : z_run + p[kb][i];
            }
        half2_t pp[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pp[r] = half2_t{_Float16(p[0][r]), _Float16(p[1][r])};

        // ---- context over this half's four groups
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int gi = 4 * h + j;  // group in the row (wave-uniform)
            const i32x2 cv = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
                (__attribute__((address_space(3))) i32x2*)(vt + tr_off + 16 * j));
            half8_t av;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t sa = *reinterpret_cast<const uint32_t*>(vt + (4 * q4 + r) * kPitch + 64 + 4 * (gi >> 1));
                const uint32_t sb =
                    *reinterpret_cast<const uint32_t*>(vt + (16 + 4 * q4 + r) * kPitch + 64 + 4 * (gi >> 1));
                const uint32_t pr = (j & 1) ? __builtin_amdgcn_perm(sb, sa, 0x07060302u)
                                            : __builtin_amdgcn_perm(sb, sa, 0x05040100u);
                const half2_t w = pp[r] * __builtin_bit_cast(half2_t, pr);
                av[2 * r] = w[0];
                av[2 * r + 1] = w[1];
            }
            o[2 * j] = mfma(av, unpack8(uint32_t(cv[0])), o[2 * j]);
            o[2 * j] = mfma(av, bconst, o[2 * j]);
            o[2 * j + 1] = mfma(av, unpack8(uint32_t(cv[1])), o[2 * j + 1]);
            o[2 * j + 1] = mfma(av, bconst, o[2 * j + 1]);
        }
        if (t + 1 < n_sub) issue(v_pool, t + 1, v_ring);  // into the slot of sub-tile t - 1
    }

    // ---- combine the four pairs.  Each wave leaves its live head rows (its
    // channel half) and, in half 0, m and z in its own V ring (read by no
    // other wave); after one barrier every thread forms its head's weights
    // exp2(m_p - M) and sums each channel over the pairs in pair order.
    static_assert(kEpiRows * 128 * 4 + 2 * 16 * 4 <= 2 * kSlot, "per-wave results fit the wave's V ring");
    z_run = quad_sum(z_run);
    auto wo = [&](int w) { return reinterpret_cast<float*>(smem + w * kWaveLds + 2 * kSlot); };  // [8][128]
    auto wm = [&](int w) { return wo(w) + kEpiRows * 128; };                                       // [16]
    auto wz = [&](int w) { return wo(w) + kEpiRows * 128 + 16; };                                  // [16]
    {
        float* mine = wo(wave);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * q4 + i;
            if (row < G) {
#pragma unroll
                for (int blk = 0; blk < 8; ++blk) mine[row * 128 + 16 * blk + n16] = o[blk][i] * kTwo24;
            }
        }
        if (h == 0 && lane < 16) {
            wm(wave)[lane] = n_keys > 0 ? m_run - float(a_exp) : -INFINITY;
            wz(wave)[lane] = n_keys > 0 ? z_run : 0.0f;
        }
    }
    __syncthreads();
    for (int i = tid; i < G * kD; i += kWaves * 64) {
        const int hd = i / kD, c = i % kD, half = c >> 7;
        float M = -INFINITY;
#pragma unroll
        for (int q = 0; q < kPairs; ++q) M = fmaxf(M, wm(2 * q)[hd]);
        float acc = 0.0f, Z = 0.0f;
#pragma unroll
        for (int q = 0; q < kPairs; ++q) {
            const float zq = wz(2 * q)[hd];
            const float f = zq > 0.0f ? __builtin_amdgcn_exp2f(wm(2 * q)[hd] - M) : 0.0f;
            acc += wo(2 * q + half)[hd * 128 + (c & 127)] * f;
            Z += zq * f;
        }
        store_wt(&a.part_acc[((hb + hd) * Sn + s) * kD + c], acc);
        if (c == 0) {
            store_wt(&a.part_m[(hb + hd) * Sn + s], M * kLn2);
            store_wt(&a.part_z[(hb + hd) * Sn + s], Z);
        }
    }
}

}  // namespace

bool decode_q4_pair_supported(const Q4Pool& pool, const DecodeArgs& a) {
    const int G = a.n_q_heads / pool.n_kv_heads;
    const int64_t rows = int64_t(pool.num_pages) * pool.n_kv_heads * pool.page_size;
    return pool.bits == 4 && pool.head_dim == kD && G >= 1 && G <= 8 && pool.page_size % 16 == 0 &&
           a.split_keys % (32 * kPairs) == 0 &&
           a.split_keys <= kMaxSplit && rows <= (int64_t(1) << 32);
}

hipError_t launch_decode_q4_pair(const Q4Pool& pool, const DecodeArgs& a, hipStream_t s) {
    const dim3 grid = decode_grid(a, pool.n_kv_heads);
    if (a.step_k)
        decode_q4_pair<true><<<grid, dim3(kWaves * 64), 0, s>>>(pool.k, pool.v, pool.n_kv_heads, pool.page_size,
                                                                pool.num_pages, a);
    else
        decode_q4_pair<false><<<grid, dim3(kWaves * 64), 0, s>>>(pool.k, pool.v, pool.n_kv_heads, pool.page_size,
                                                                 pool.num_pages, a);
    return hipGetLastError();
}

}  // namespace kvq
