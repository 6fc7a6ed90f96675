// decode_fp8_mfma.hip -- split-T decode over the fp8 e4m3 MLA latent cache
// with matrix cores (gfx950 v_mfma_f32_16x16x32_f16).
//
// Method: colibri pull request "KV cache quantization: fp8 (KV8) + 4-bit
// TurboQuant", KV8 commit (latent rows of kv_lora + rope e4m3 codes with a
// per-row f32 amax/448 scale each; absorbed attention, where the latent is
// both key and value) and split-T commit (partials (cl[K], m, z) per (head,
// split), merged by a log-sum-exp kernel); its correctness notes (e4m3 NaN
// codes read as 0, where a GPU convert would read NaN).
//
// Per position j and head h:
//   s_hj = sm_scale * (scL_j <qL_h, dec(Lc_j)> + scR_j <qR_h, dec(Rc_j)>),
//   acc_h = sum_j exp(s_hj - m_h) scL_j dec(Lc_j),  z_h = sum_j exp(s_hj - m_h).
// 128 heads x (576 + 512) multiply-adds per 584 cached bytes: the work is
// bound by the matrix cores, not by HBM.
//
// Workgroup = 8 waves = 4 pairs x 16 heads (the MFMA's 16-wide dimension)
// x one split of the context; both head blocks of a split read the same
// tiles (the second read is served by the caches).  The two waves of a pair
// split the channels: each takes 9 of the 18 groups of 32 score channels
// (the second the last 7 latent groups and the 2 rope groups) and 256 of the
// 512 latent output channels, so a wave holds half the query and half the
// accumulators and two waves fit on a SIMD.  Per 32-key tile:
//  * Staging: the tile's rows (two 16-row page runs of 576 code bytes) and
//    their scales are copied raw by LDS DMA three tiles ahead of use, into a
//    ring of three raw stages; one iteration ahead of use every thread
//    converts its chunks of the raw tile into one of two f16 stages.  On the
//    way, codes 0x7F / 0xFF (NaN) are zeroed with byte-wise integer
//    arithmetic and every code is converted to f16 by
//    v_cvt_scalef32_pk_f16_fp8 (exact: every e4m3 value is an f16), once
//    per workgroup: the four pairs that use a code read it converted.
//    (Selected rows go global -> registers -> LDS, one row at a time.)  Rows
//    are 1168 bytes apart in LDS (576 f16 + 16), with the keys permuted
//    within each 16-row block (lds_row), so a score read and a context read
//    each touch every bank once.
//  * Scores: A = 16 keys x 32 channels (16 bytes of f16 per lane), B = the
//    query pre-scaled by sm_scale*log2(e), split into f16 hi + lo parts; the
//    latent and rope parts meet their scales in fp32.  The pair exchanges
//    its two partial scores through LDS and both add them in the same order,
//    so both hold bit-identical scores and softmax state.  Output lane
//    (head n, quarter q) holds keys 4q+i and 16+4q+i.
//  * Softmax in log2 units with a lazily moving maximum (moves only when a
//    tile exceeds it by more than 2^6).
//  * Context: A = p * scL for the lane's 8 keys (exactly the score lane's
//    own keys, so no exchange is needed) in f16, scaled by 2^-E with E a
//    running exponent of the largest latent scale seen, which keeps A inside
//    the f16 range whatever the rows' magnitude; B = 8 keys x 1 channel of
//    the latent gathered by two ds_read_b64_tr_b16 (source lane 4e + m of a
//    16-lane group addresses key slot e at channels 4m .. 4m + 3, so lane j
//    receives channel j of keys e = 0..3; the second read takes slots 4..7).
//
// The rotated-int4 + Lloyd-Max latent cache (the same pull request, Summary
// "Why rotated-int4 for the 4-bit tier": 288 nibble bytes and two radii per
// row) runs through the same kernel in rotated space: the query arrives
// rotated, the staging turns each nibble into the f16 value of c * lev[code]
// (two byte tables looked up with v_perm_b32, the code's bit 3 choosing
// between the halves of the table) and the row's scales become r_L / (c
// sqrt(512)) and r_R / (c sqrt(64)), so everything after the staging is the
// fp8 code.  c is the scale in [1, 2) that brings the 16 levels closest to
// the f16 grid (largest relative deviation under 1e-4, against 3.2e-4 at
// c = 1); the partials are the rotated context, rotated back after the merge.
//
// Selected rows (colibri split-T commit, DSA gather: attend the selected
// rows, given as absolute positions): the keys of a split are entries
// j0 .. j1-1 of the sequence's list instead of positions j0 .. j1-1.  The
// workgroup first resolves every entry of its split to a cache slot (list,
// then page table) into an LDS table; each staged row is then addressed on
// its own, and entries outside the page capacity (the -1 of a padded list)
// are masked like rows past the end.  Everything after the staging is the
// same code.
#include "mfma_common.h"

namespace kvq {
namespace {

using namespace mx;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int kL = 512, kR = 64, kD = kL + kR;  // latent, rope, row
constexpr int kWaves = 8;                            // 4 pairs
constexpr int kThreads = kWaves * 64;
constexpr int kHeadsWG = 16 * (kWaves / 2);
constexpr int kTile = 32;                            // keys per tile
constexpr int kPitch = 1168;                         // LDS bytes per row: 576 f16 + 16
constexpr int kScaleOff = kTile * kPitch;            // scales after the rows
constexpr int kStage = kScaleOff + kTile * 8;        // 37632 bytes
constexpr int kXOff = 2 * kStage;                    // partial-score exchange: [wave][lane][8] f32
constexpr int kLds = kXOff + kWaves * 64 * 8 * 4;
constexpr int kSelOff = kLds;                        // selected rows: the split's slot table
constexpr int kLdsSel = kSelOff + 2048 * 4;          // int32 per entry, split_keys <= 2048
// Code bytes per row, 16-byte chunks per row and per tile, chunks per thread:
// fp8 576, 36, 1152, 3 (the third for 128 threads); TQ4 288, 18, 576, 2 (the
// second for 64 threads).  Threads 128..143 own the scale chunks in their last
// slot in both.
template <bool TQ> struct Rows {
    static constexpr int kBytes = TQ ? kD / 2 : kD;
    static constexpr int kChunkRow = kBytes / 16;
    static constexpr int kChunks = kTile * kChunkRow;
    static constexpr int kPerThread = (kChunks + kThreads - 1) / kThreads;
};
// Rows staged by LDS DMA (dense rows): a tile's two 16-row page runs are two
// contiguous blocks of 16 rows in the pool, copied raw into one of three raw
// stages (run a, run b, then both runs' scale pairs) two tiles ahead of the
// conversion.  DMA instruction j of a tile (64 lanes x 16 bytes) is issued by
// wave j mod 8; the scale pairs of run a / b by waves 2 / 3.
template <bool TQ> struct Raw {
    static constexpr int kRunBytes = 16 * Rows<TQ>::kBytes;       // fp8 9216, TQ4 4608
    static constexpr int kRunInstr = (kRunBytes / 16 + 63) / 64;   // 9, 5 (the fifth: 32 lanes)
    static constexpr int kInstr = 2 * kRunInstr;
    static constexpr int kScaleOff = 2 * kRunBytes;
    static constexpr int kStage = kScaleOff + kTile * 8;
    // DMA instructions a wave issues per tile
    static constexpr int count(int w) { return (kInstr - w + 7) / 8 + (w == 2 || w == 3 ? 1 : 0); }
    static constexpr int kFirst = count(0);  // waves 0..3
    static constexpr int kLast = count(4);   // waves 4..7
    static_assert(count(1) == kFirst && count(2) == kFirst && count(3) == kFirst && count(5) == kLast &&
                  count(7) == kLast && kInstr <= 24, "per-wave DMA counts");
};
constexpr int kRawStages = 3;
constexpr int kRawOff = kLds;
template <bool TQ> constexpr int kLdsDense = kRawOff + kRawStages * Raw<TQ>::kStage;
constexpr int kMaxRuns = 128;                        // 16-key runs per split (split_keys <= 2048)
constexpr int kQG = 9;                               // score channel groups (of 32) per wave
constexpr int kNBW = kL / 16 / 2;                    // 16 output blocks of 16 channels per wave
constexpr float kRescale = 6.0f;

// 8 e4m3 codes (two dwords, byte order = k-slot order) as 8 f16 values.
__device__ __forceinline__ half8_t cvt8(uint32_t w0, uint32_t w1) {
    const half2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
    const half2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
    const half2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
    const half2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
    return half8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Zero the bytes of w that are e4m3 NaN codes (low 7 bits all ones).
__device__ __forceinline__ uint32_t clear_nan_codes(uint32_t w) {
    const uint32_t t = ((w & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;  // bit 7 set where low 7 bits were 0x7F
    return w & ~(t | (t - (t >> 7)));
}

// 8 TQ4 codes (one dword: byte k holds code 2k in its low nibble, 2k+1 in its
// high nibble) as the 8 f16 values c * lev[code], in element order.  lo / hi
// hold the low / high bytes of the 16 f16 table entries (entry k is byte k of
// the 16-byte table): v_perm_b32 looks up codes 0..7 in one 8-byte half and
// 8..15 in the other, and the code's bit 3 picks the result byte-wise.
__device__ __forceinline__ void tq_cvt8(uint32_t w, const uint32_t (&lo)[4], const uint32_t (&hi)[4], uint32_t* d) {
    const uint32_t ce = w & 0x07070707u, co = (w >> 4) & 0x07070707u;          // codes & 7: even / odd elements
    const uint32_t me = ((w >> 3) & 0x01010101u) * 0xFFu, mo = ((w >> 7) & 0x01010101u) * 0xFFu;  // bit 3
    const uint32_t le = __builtin_amdgcn_perm(lo[1], lo[0], ce), le8 = __builtin_amdgcn_perm(lo[3], lo[2], ce);
    const uint32_t he = __builtin_amdgcn_perm(hi[1], hi[0], ce), he8 = __builtin_amdgcn_perm(hi[3], hi[2], ce);
    const uint32_t lO = __builtin_amdgcn_perm(lo[1], lo[0], co), lO8 = __builtin_amdgcn_perm(lo[3], lo[2], co);
    const uint32_t hO = __builtin_amdgcn_perm(hi[1], hi[0], co), hO8 = __builtin_amdgcn_perm(hi[3], hi[2], co);
    const uint32_t Le = (le & ~me) | (le8 & me), He = (he & ~me) | (he8 & me);  // bytes of elements 0, 2, 4, 6
    const uint32_t Lo = (lO & ~mo) | (lO8 & mo), Ho = (hO & ~mo) | (hO8 & mo);  // bytes of elements 1, 3, 5, 7
    const uint32_t e01 = __builtin_amdgcn_perm(He, Le, 0x05010400u);  // f16 of elements 0, 2
    const uint32_t e23 = __builtin_amdgcn_perm(He, Le, 0x07030602u);  // elements 4, 6
    const uint32_t o01 = __builtin_amdgcn_perm(Ho, Lo, 0x05010400u);  // elements 1, 3
    const uint32_t o23 = __builtin_amdgcn_perm(Ho, Lo, 0x07030602u);  // elements 5, 7
    d[0] = __builtin_amdgcn_perm(o01, e01, 0x05040100u);  // elements 0, 1
    d[1] = __builtin_amdgcn_perm(o01, e01, 0x07060302u);  // 2, 3
    d[2] = __builtin_amdgcn_perm(o23, e23, 0x05040100u);  // 4, 5
    d[3] = __builtin_amdgcn_perm(o23, e23, 0x07060302u);  // 6, 7
}

// LDS row of key k of a tile.  Rows are kPitch = 292 dwords apart, so row r
// starts at bank 36 r mod 64: the even rows of a 16-row block start at banks
// 0, 8, ..., 56 and the odd rows at 4, 12, ..., 60 (mod 64), each set tiling
// the 64 banks with 8-dword spans.  A context read (ds_read_b64_tr_b16, 32
// lanes per pass) takes 8 keys x 8 bytes; keys 0..7 of a 16-key block sit
// on the even rows and keys 8..15 on the odd ones, so each pass touches one
// set and no bank twice.  A score read (16 keys x 16 bytes) still touches
// 16 distinct rows, all at distinct 4-dword spans.
__device__ __forceinline__ int lds_row(int k) { return (k & 16) | ((k & 7) << 1) | ((k >> 3) & 1); }

// 2^e for an integer e in [-126, 127], exactly.
__device__ __forceinline__ float exp2i(int e) { return __uint_as_float(uint32_t(e + 127) << 23); }

// STEP (kvq_decode_step, fp8 rows over consecutive positions): wave 0 of
// each workgroup whose split holds position seq_lens[b] - 1 first stores
// token b's latent row there, with the store kernel's arithmetic per element
// (amax per part over fabsf, 448 / amax, e4m3_encode), so the bytes are the
// same.  Both head-block workgroups of that split store the row, writing the
// same bytes; each copies the row only after its own store is acknowledged:
// at once when the row's tile is copied first (then a workgroup barrier), by
// the prologue's full wait before tiles 1 and 2 are copied (then a barrier if
// the row is in one of them), else long before (the barriers that follow).
template <bool SEL, bool TQ, bool STEP = false>
__global__ __launch_bounds__(kThreads) void decode_fp8_mfma(const uint8_t* __restrict__ codes,
                                                            const float* __restrict__ scales, int page_size,
                                                            int num_pages, DecodeArgs a, TqMfmaTable tab) {
    using R = Rows<TQ>;
    constexpr int kRowB = R::kBytes, kChunkRow = R::kChunkRow, kChunks = R::kChunks, kPerThread = R::kPerThread;
    __shared__ __attribute__((aligned(16))) uint8_t smem[SEL ? kLdsSel : kLdsDense<TQ>];

    const int s = blockIdx.x, hblk = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = wave & 1;                       // channel half of the pair
    const int n16 = lane & 15, q4 = lane >> 4;
    const int H = a.n_q_heads, Sn = a.n_splits;
    const int j0 = s * a.split_keys;
    const int h_pair = hblk * kHeadsWG + (wave >> 1) * 16;  // first head of this pair
    const int g0 = half * kQG;                       // first score group of this wave
    int T = a.seq_lens[b];

    // Query of head h_pair + n16, channels 32 (g0 + gl) + 8 q4 .. +7.
    const int hq = h_pair + n16;
    const bool live = hq < H;
    const float* qh = a.q + (int64_t(b) * H + (live ? hq : 0)) * kD + 32 * g0 + 8 * q4;
    float4 qv[kQG][2];
#pragma unroll
    for (int gl = 0; gl < kQG; ++gl) {
        qv[gl][0] = *reinterpret_cast<const float4*>(qh + 32 * gl);
        qv[gl][1] = *reinterpret_cast<const float4*>(qh + 32 * gl + 4);
    }

    // Slot of the first row of each 16-row run of the split: lane l holds run
    // l in the first register and run 64 + l in the second.  Positions are
    // clamped to the start of the run holding max_seq_len - 1 and pages to
    // the pool, so every read stays in bounds; rows past the end are masked.
    const int32_t* pt = a.page_table + int64_t(b) * a.max_pages;
    const int n_runs = a.split_keys / 16;
    const int last_pos = a.max_seq_len > 0 ? (a.max_seq_len - 1) & ~15 : 0;
    int64_t rslot[2] = {0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (SEL || (h == 1 && n_runs <= 64)) break;
        const int r = min(lane + 64 * h, n_runs - 1);
        const int pos = min(j0 + 16 * r, last_pos);
        int page = pt[pos / page_size];
        page = page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
        rslot[h] = int64_t(page) * page_size + pos % page_size;
    }

    T = T < 0 ? 0 : (T > a.max_seq_len ? a.max_seq_len : T);
    const int j1 = min(j0 + a.split_keys, T);
    if (j0 >= j1) {  // split past the end: empty partials for this workgroup's heads
        const int nh = max(0, min(kHeadsWG, H - hblk * kHeadsWG));
        const int64_t hb = int64_t(b) * H + hblk * kHeadsWG;
        for (int i = tid; i < nh * kL; i += kThreads) a.part_acc[((hb + i / kL) * Sn + s) * kL + i % kL] = 0.0f;
        if (tid < nh) {
            a.part_m[(hb + tid) * Sn + s] = -INFINITY;
            a.part_z[(hb + tid) * Sn + s] = 0.0f;
        }
        return;
    }
    const int n_keys = j1 - j0;
    const int n_tiles = (n_keys + kTile - 1) / kTile;

    const int pos_new = T - 1;
    const bool holds = STEP && T > 0 && pos_new >= j0 && pos_new < j1;  // workgroup-uniform
    const int t_new = holds ? (pos_new - j0) / kTile : -1;               // the row's tile
    // Wave 0: the token's row (lane: latent elements lane + 64 k, k < 8, and
    // rope element lane) into its slot; a page outside the pool is not
    // stored (kvq_store skips such a slot too).
    auto store_token = [&](bool wait) {
        float xv[9];
        const int64_t base = int64_t(b) * kD + lane;
        const void* x = a.step_k;
        if (a.step_kv_dt == InType::F32) {
#pragma unroll
            for (int k = 0; k < 9; ++k) xv[k] = load_elem<InType::F32>(x, base + 64 * k);
        } else if (a.step_kv_dt == InType::BF16) {
#pragma unroll
            for (int k = 0; k < 9; ++k) xv[k] = load_elem<InType::BF16>(x, base + 64 * k);
        } else {
#pragma unroll
            for (int k = 0; k < 9; ++k) xv[k] = load_elem<InType::F16>(x, base + 64 * k);
        }
        const int page = pt[pos_new / page_size];
        if (page >= 0 && page < num_pages) {
            const int64_t slot = int64_t(page) * page_size + pos_new % page_size;
            uint8_t* out = const_cast<uint8_t*>(codes) + slot * kD;
#pragma unroll
            for (int part = 0; part < 2; ++part) {
                const int k0 = part ? 8 : 0, nk = part ? 1 : 8;
                float amax = 0.0f;
                for (int k = k0; k < k0 + nk; ++k) amax = fmaxf(amax, fabsf(xv[k]));  // NaN ignored
#pragma unroll
                for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
                const float inv = 448.0f / amax;
                const bool inert = !(amax > 0.0f) || !isfinite(amax) || !isfinite(inv);
                for (int k = k0; k < k0 + nk; ++k)
                    out[lane + 64 * k] = inert ? uint8_t(0) : uint8_t(e4m3_encode(xv[k] * inv));
                if (lane == 0) const_cast<float*>(scales)[slot * 2 + part] = inert ? 0.0f : amax / 448.0f;
            }
        }
        if (wait) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };

    auto run_slot = [&](int r) -> int64_t {  // r is wave-uniform
        const int64_t v = r < 64 ? rslot[0] : rslot[1];
        const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(v), r & 63);
        const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(uint64_t(v) >> 32), r & 63);
        return int64_t((uint64_t(hi) << 32) | lo);
    };

    // ---- selected rows: slot of every entry of the split (-1: absent entry;
    // entries past the split's end point at slot 0 and are masked by `valid`).
    int32_t* slot_tab = reinterpret_cast<int32_t*>(smem + kSelOff);
    bool any_absent = false;
    if constexpr (SEL) {
        const int32_t* list = a.sel + int64_t(b) * a.sel_stride + j0;
        const int64_t cap = int64_t(a.max_pages) * page_size;
        for (int k = tid; k < n_tiles * kTile; k += kThreads) {
            int32_t slot = 0;
            if (k < n_keys) {
                const int32_t pos = list[k];
                if (pos >= 0 && pos < cap) {
                    int page = pt[pos / page_size];
                    page = page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
                    slot = page * page_size + pos % page_size;
                } else {
                    slot = -1;
                    any_absent = true;
                }
            }
            slot_tab[k] = slot;
        }
        any_absent = __syncthreads_or(any_absent);  // also publishes the table
    }

    // ---- staging: thread tid owns code chunks tid + 512 i (i < 3 while
    // < 1152); threads 128..143 own the 16 scale chunks instead of a third
    // (selected rows: threads 128..159 the 32 rows' scale pairs).
    u32x4 stg[kPerThread];
    const bool has_scale = tid >= 128 && tid < (SEL ? 160 : 144);
    auto chunk_row = [&](int i) { return (tid + kThreads * i) / kChunkRow; };
    auto chunk_col = [&](int i) { return (tid + kThreads * i) % kChunkRow; };
    auto load_tile = [&](int t) {
        if constexpr (SEL) {
            const int32_t* tab = slot_tab + t * kTile;
#pragma unroll
            for (int i = 0; i < kPerThread; ++i) {
                if (tid + kThreads * i < kChunks) {
                    const int64_t sl = max(tab[chunk_row(i)], 0);
                    stg[i] = *reinterpret_cast<const u32x4*>(codes + sl * kRowB + 16 * chunk_col(i));
                } else if (has_scale) {
                    const int64_t sl = max(tab[tid - 128], 0);
                    const uint2 v = *reinterpret_cast<const uint2*>(scales + sl * 2);
                    stg[i] = u32x4{v.x, v.y, 0u, 0u};
                }
            }
            return;
        }
        const int64_t ra = run_slot(2 * t), rb = run_slot(2 * t + 1);
        const uint8_t* ca = codes + ra * kRowB;
        const uint8_t* cb = codes + rb * kRowB;
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            if (tid + kThreads * i < kChunks) {
                const int kr = chunk_row(i);
                stg[i] = *reinterpret_cast<const u32x4*>((kr >= 16 ? cb : ca) + (kr & 15) * kRowB + 16 * chunk_col(i));
            } else if (has_scale) {
                const int key = 2 * (tid - 128);  // keys key, key + 1
                stg[i] = *reinterpret_cast<const u32x4*>(scales + ((key >= 16 ? rb : ra) + (key & 15)) * 2);
            }
        }
    };
    auto store_tile = [&](int t) {
        uint8_t* st = smem + (t & 1) * kStage;
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            if (TQ && tid + kThreads * i < kChunks) {
                uint32_t d[16];
#pragma unroll
                for (int e = 0; e < 4; ++e) tq_cvt8(stg[i][e], tab.lo, tab.hi, d + 4 * e);
                u32x4* dst = reinterpret_cast<u32x4*>(st + lds_row(chunk_row(i)) * kPitch + 64 * chunk_col(i));
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[e] = u32x4{d[4 * e], d[4 * e + 1], d[4 * e + 2], d[4 * e + 3]};
            } else if (tid + kThreads * i < kChunks) {
                u32x4 w = stg[i];
                // NaN codes are rare: test the chunk, clear only if one is present.
                uint32_t any = 0u;
#pragma unroll
                for (int e = 0; e < 4; ++e) any |= (w[e] & 0x7F7F7F7Fu) + 0x01010101u;
                if (any & 0x80808080u) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = clear_nan_codes(w[e]);
                }
                half8_t* d = reinterpret_cast<half8_t*>(st + lds_row(chunk_row(i)) * kPitch + 32 * chunk_col(i));
                d[0] = cvt8(w[0], w[1]);
                d[1] = cvt8(w[2], w[3]);
            } else if (has_scale) {
                if (SEL)
                    *reinterpret_cast<uint2*>(st + kScaleOff + 8 * (tid - 128)) = make_uint2(stg[i][0], stg[i][1]);
                else if (TQ)  // radii (latent, rope) of two keys -> the table values' multipliers
                    *reinterpret_cast<float4*>(st + kScaleOff + 16 * (tid - 128)) =
                        make_float4(__uint_as_float(stg[i][0]) * tab.f_latent, __uint_as_float(stg[i][1]) * tab.f_rope,
                                    __uint_as_float(stg[i][2]) * tab.f_latent, __uint_as_float(stg[i][3]) * tab.f_rope);
                else
                    *reinterpret_cast<u32x4*>(st + kScaleOff + 16 * (tid - 128)) = stg[i];
            }
        }
    };

    // Dense rows: DMA of tile t's raw rows into raw stage t % 3 (no registers).
    auto issue_tile = [&](int t) {
        using RW = Raw<TQ>;
        const int64_t ra = run_slot(2 * t), rb = run_slot(2 * t + 1);
        const uint32_t raw = lds_addr(smem + kRawOff + (t % kRawStages) * RW::kStage);
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            const int j = wave + 8 * m;
            if (j < RW::kInstr) {
                const int run = j >= RW::kRunInstr ? 1 : 0;
                const int k = j - run * RW::kRunInstr;
                const int chunk = 64 * k + lane;
                if (chunk < RW::kRunBytes / 16)
                    dma16<false>(codes + (run ? rb : ra) * kRowB, uint32_t(16 * chunk),
                                 raw + uint32_t(run * RW::kRunBytes + 1024 * k));
            }
        }
        if (wave == 2 || wave == 3) {
            const int run = wave - 2;
            if (lane < 8)
                dma16<false>(reinterpret_cast<const uint8_t*>(scales + (run ? rb : ra) * 2), uint32_t(16 * lane),
                             raw + uint32_t(RW::kScaleOff + 128 * run));
        }
    };
    // Dense rows, the conversion split so that it can sit between the context
    // MFMAs: every thread reads its kFull chunks (tid + 512 i, always in the
    // tile), the first kRemWaves waves one more code chunk, threads 128..143 a
    // scale chunk (wave-uniform conditions but for that one), all before any
    // is used; NaN codes are cleared in one test over all of a thread's chunks
    // (clear_nan_codes leaves chunks without one as they are, so the bytes are
    // those of the per-chunk test); then each chunk is converted on its own.
    constexpr int kFull = R::kChunks / kThreads, kRemWaves = (R::kChunks % kThreads) / 64;
    static_assert(R::kChunks % 64 == 0 && kRemWaves <= 2 && kFull + 1 == kPerThread, "dense chunk mapping");
    auto dense_read = [&](int t) {
        using RW = Raw<TQ>;
        const uint8_t* rw = smem + kRawOff + (t % kRawStages) * RW::kStage;
#pragma unroll
        for (int i = 0; i < kFull; ++i) stg[i] = *reinterpret_cast<const u32x4*>(rw + 16 * (tid + kThreads * i));
        if (wave < kRemWaves)
            stg[kFull] = *reinterpret_cast<const u32x4*>(rw + 16 * (tid + kThreads * kFull));
        else if (has_scale)
            stg[kFull] = *reinterpret_cast<const u32x4*>(rw + RW::kScaleOff + 16 * (tid - 128));
    };
    auto dense_clear_nan = [&]() {
        if constexpr (!TQ) {
            uint32_t any = 0u;
#pragma unroll
            for (int i = 0; i < kPerThread; ++i)
                if (i < kFull || wave < kRemWaves) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) any |= (stg[i][e] & 0x7F7F7F7Fu) + 0x01010101u;
                }
            if (any & 0x80808080u) {  // rare
#pragma unroll
                for (int i = 0; i < kPerThread; ++i)
                    if (i < kFull || wave < kRemWaves) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) stg[i][e] = clear_nan_codes(stg[i][e]);
                    }
            }
        }
    };
    // slot i of this thread into f16 stage t & 1 (slot kFull: the remainder code chunk or the scales)
    auto dense_convert = [&](int t, int i) {
        uint8_t* st = smem + (t & 1) * kStage;
        const bool code = i < kFull || wave < kRemWaves;
        if (code && TQ) {
            uint32_t d[16];
#pragma unroll
            for (int e = 0; e < 4; ++e) tq_cvt8(stg[i][e], tab.lo, tab.hi, d + 4 * e);
            u32x4* dst = reinterpret_cast<u32x4*>(st + lds_row(chunk_row(i)) * kPitch + 64 * chunk_col(i));
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[e] = u32x4{d[4 * e], d[4 * e + 1], d[4 * e + 2], d[4 * e + 3]};
        } else if (code) {
            half8_t* d = reinterpret_cast<half8_t*>(st + lds_row(chunk_row(i)) * kPitch + 32 * chunk_col(i));
            d[0] = cvt8(stg[i][0], stg[i][1]);
            d[1] = cvt8(stg[i][2], stg[i][3]);
        } else if (has_scale) {
            if (SEL)  // selected rows: one row's scale pair a thread
                *reinterpret_cast<uint2*>(st + kScaleOff + 8 * (tid - 128)) = make_uint2(stg[i][0], stg[i][1]);
            else if (TQ)
                *reinterpret_cast<float4*>(st + kScaleOff + 16 * (tid - 128)) =
                    make_float4(__uint_as_float(stg[i][0]) * tab.f_latent, __uint_as_float(stg[i][1]) * tab.f_rope,
                                __uint_as_float(stg[i][2]) * tab.f_latent, __uint_as_float(stg[i][3]) * tab.f_rope);
            else
                *reinterpret_cast<u32x4*>(st + kScaleOff + 16 * (tid - 128)) = stg[i];
        }
    };

    // Own DMAs of the tile before the newest landed (the newest may be in flight).
    auto wait_own = [&](bool newest_in_flight) {
        if (!newest_in_flight) wait_vmcnt<0>();
        else if (wave < 4) wait_vmcnt<Raw<TQ>::kFirst>();
        else wait_vmcnt<Raw<TQ>::kLast>();
    };

    if constexpr (SEL) {
        load_tile(0);
    } else {
        if (STEP && holds && wave == 0) store_token(t_new == 0);
        if (STEP && holds && t_new == 0) __syncthreads();  // the row's tile is copied next
        issue_tile(0);  // tiles 1 and 2 after the query is in registers (its wait covers tile 0 only)
    }

    // B operands of the score MFMAs: the pre-scaled query split into f16 hi + lo.
    half8_t bq_hi[kQG], bq_lo[kQG];
    {
        const float qscale = a.sm_scale * kLog2e;
#pragma unroll
        for (int gl = 0; gl < kQG; ++gl) {
            const float c8[8] = {qv[gl][0].x, qv[gl][0].y, qv[gl][0].z, qv[gl][0].w,
                                 qv[gl][1].x, qv[gl][1].y, qv[gl][1].z, qv[gl][1].w};
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float v = live ? c8[k] * qscale : 0.0f;
                const _Float16 hi = _Float16(v);
                bq_hi[gl][k] = hi;
                bq_lo[gl][k] = _Float16(v - float(hi));
            }
        }
    }

    if constexpr (SEL) {
        store_tile(0);
        if (n_tiles > 1) load_tile(1);
    } else {
        wait_vmcnt<0>();  // (wave 0 of a STEP workgroup: also its stores of the new row)
        if (STEP && holds && (t_new == 1 || t_new == 2)) __syncthreads();
        if (n_tiles > 1) issue_tile(1);
        if (n_tiles > 2) issue_tile(2);
        __syncthreads();  // tile 0 staged raw
        dense_read(0);
        dense_clear_nan();
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) dense_convert(0, i);
    }
    __syncthreads();

    f32x4 o[kNBW];
#pragma unroll
    for (int i = 0; i < kNBW; ++i) o[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY;  // running max (log2 units) of head n16
    float z_run = 0.0f;       // this lane's share of the running sum
    int e_run = -1000;        // running exponent of the largest latent scale (unset)

    // tr_b16 source of this lane: key slot n16 >> 2 of its quarter (key
    // 4 q4 + (n16 >> 2), then 16 + the same for slots 4..7) at channels
    // 4 (n16 & 3) .. +3 of the 16-channel block, this wave's latent half.
    const int tr_off = lds_row(4 * q4 + (n16 >> 2)) * kPitch + 2 * (4 * (n16 & 3) + half * (kL / 2));
    float* xmine = reinterpret_cast<float*>(smem + kXOff) + (wave * 64 + lane) * 8;
    const float* xpart = reinterpret_cast<const float*>(smem + kXOff) + ((wave ^ 1) * 64 + lane) * 8;

    for (int t = 0; t < n_tiles; ++t) {
        const uint8_t* st = smem + (t & 1) * kStage;
        const int valid = min(kTile, n_keys - t * kTile);

        // ---- partial scores over this wave's 9 groups: two 16-key blocks;
        // lane holds keys 16 kb + 4 q4 + i of head n16.  Groups 0..6 are
        // latent for both halves; 7 and 8 are latent (first half) or rope.
        // The 18 A operands are read from LDS kAhead steps ahead of their
        // MFMAs (the order is pinned by scheduling barriers: left to itself
        // the compiler read two and waited for them before each pair of
        // groups), and both blocks' scale factors are applied after all 36
        // MFMAs are issued, so that work overlaps the last ones.
        float part[2][4], scl[2][4];
        {
            constexpr int kSteps = 2 * kQG, kAhead = 3;
            const float4* sp = reinterpret_cast<const float4*>(st + kScaleOff + 8 * (4 * q4));
            const float4 s01[2] = {sp[0], sp[8]}, s23[2] = {sp[1], sp[9]};  // keys 16 kb + 4 q4 + 0..3 (8 bytes a key)
            const uint8_t* krow[2] = {st + lds_row(n16) * kPitch + 2 * (32 * g0 + 8 * q4),
                                      st + lds_row(16 + n16) * kPitch + 2 * (32 * g0 + 8 * q4)};
            half8_t av[kSteps];
            // Raised issue priority while this wave feeds its score MFMAs (the other wave
            // of the SIMD is then mostly in its vector work): 151 vs 152.6 us at 262K;
            // raising it for the context MFMAs as well was slower (155 us).
            __builtin_amdgcn_s_setprio(2);
#pragma unroll
            for (int j = 0; j < kAhead; ++j) av[j] = *reinterpret_cast<const half8_t*>(krow[j / kQG] + 64 * (j % kQG));
            f32x4 acc[2][3];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int c = 0; c < 3; ++c) acc[kb][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int j = 0; j < kSteps; ++j) {
                if (j + kAhead < kSteps)
                    av[j + kAhead] = *reinterpret_cast<const half8_t*>(krow[(j + kAhead) / kQG] +
                                                                       64 * ((j + kAhead) % kQG));
                const int kb = j / kQG, gl = j % kQG;
                const int c = gl >= 7 ? 2 : (gl & 1);  // chains: even groups, odd groups, groups 7 and 8
                acc[kb][c] = mfma(av[j], bq_hi[gl], acc[kb][c]);
                acc[kb][c] = mfma(av[j], bq_lo[gl], acc[kb][c]);
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_s_setprio(0);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const float sl[4] = {s01[kb].x, s01[kb].z, s23[kb].x, s23[kb].z};
                const float sr[4] = {s01[kb].y, s01[kb].w, s23[kb].y, s23[kb].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    part[kb][i] = fmaf(half ? sr[i] : sl[i], acc[kb][2][i], sl[i] * (acc[kb][0][i] + acc[kb][1][i]));
                    scl[kb][i] = sl[i];
                }
            }
        }
        // ---- the pair's scores: first half's partial + second half's, in both waves
        {
            float4* xm = reinterpret_cast<float4*>(xmine);
            xm[0] = make_float4(part[0][0], part[0][1], part[0][2], part[0][3]);
            xm[1] = make_float4(part[1][0], part[1][1], part[1][2], part[1][3]);
        }
        if (!SEL && t + 1 < n_tiles) wait_own(t + 2 < n_tiles);  // tile t + 1 raw, own part
        __syncthreads();  // partial scores exchanged (dense rows: tile t + 1 staged raw)
        if (!SEL && !TQ && t + 1 < n_tiles) dense_read(t + 1);  // converted between the context MFMAs
        float sc[2][4];
        {
            const float4* xp = reinterpret_cast<const float4*>(xpart);
            const float4 o0 = xp[0], o1 = xp[1];
            const float other[2][4] = {{o0.x, o0.y, o0.z, o0.w}, {o1.x, o1.y, o1.z, o1.w}};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sc[kb][i] = half ? other[kb][i] + part[kb][i] : part[kb][i] + other[kb][i];
        }
        if (valid < kTile) {  // only the last tile can be partial
            asm volatile("" ::: "memory");  // a real branch: keep the full tiles free of selects
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * kb + 4 * q4 + i >= valid) {
                        sc[kb][i] = -INFINITY;
                        scl[kb][i] = 0.0f;  // rows past the end may hold any scale
                    }
        }
        if (SEL && any_absent) {  // absent entries of the list: slot 0 was staged in their place
            asm volatile("" ::: "memory");
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (slot_tab[t * kTile + 16 * kb + 4 * q4 + i] < 0) {
                        sc[kb][i] = -INFINITY;
                        scl[kb][i] = 0.0f;
                    }
        }

        // ---- running maximum (per head) and running scale exponent (uniform)
        // (scores are finite or -inf, scales finite or 0: no NaN reaches these maxima)
        const float tmax = quad_max_nonan(max8f(sc));
        const float smax = quad_max_nonan(max8f(scl));  // the same in every lane: scales belong to keys
        const int e_tile = smax > 0.0f ? int((__float_as_uint(smax) >> 23) & 0xFF) - 127 : -1000;
        const int e_new = __builtin_amdgcn_readfirstlane(
            e_run == -1000 ? max(e_tile, -100) : (e_tile > e_run + 4 ? e_tile : e_run));
        // The maximum moves to the first finite tile maximum (-inf + 6 = -inf), then
        // by more than 2^6.  A tile whose keys are all masked (absent entries of a
        // selection) while the maximum is still -inf does not move it, and its p
        // are 0 below, so no -inf - -inf = NaN reaches z or the accumulators.
        const bool move = tmax > m_run + kRescale;
        if (__builtin_amdgcn_ballot_w64(move) != 0ull || e_new != e_run) {
            const float m_new = move ? fmaxf(m_run, tmax) : m_run;
            const float alpha = move ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;  // 0 when m_run = -inf
            z_run *= alpha;
            m_run = m_new;
            const float f = e_run == -1000 ? 1.0f : exp2i(max(e_run - e_new, -126));
            e_run = e_new;
            float al[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * q4 + i, 64) * f;  // rows 4 q4 + i are heads
#pragma unroll
            for (int blk = 0; blk < kNBW; ++blk)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[blk][i] *= al[i];
        }
        const float sfac = exp2i(-e_run);
        // while the maximum is -inf every score of the tile is -inf: p = 2^-inf = 0
        const float m_ref = m_run == -INFINITY ? 0.0f : m_run;

        // ---- weights: p for z, p * scL * 2^-E (f16) for the context
        half8_t av;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = __builtin_amdgcn_exp2f(sc[kb][i] - m_ref);
                z_run += p;
                av[4 * kb + i] = _Float16(p * (scl[kb][i] * sfac));
            }

        // ---- context: this wave's 16 blocks of 16 latent channels (each
        // block's two transposed reads issued kAhead blocks before its MFMA)
        {
            constexpr int kAhead = 4;
            i16x4 v0[kNBW], v1[kNBW];
            auto read_blk = [&](int cb) {
                v0[cb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4*)(st + tr_off + 32 * cb));
                v1[cb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4*)(st + tr_off + 16 * kPitch + 32 * cb));
            };
            // fp8 rows (dense, or selected: loaded into registers an iteration ahead): tile
            // t + 1 is converted here (the TQ4 levels' heavier conversion measured slower
            // between the MFMAs, 173.7 vs 159.8 us, and runs after them)
            const bool next = !TQ && t + 1 < n_tiles;
            if (next) dense_clear_nan();
#pragma unroll
            for (int cb = 0; cb < kAhead; ++cb) read_blk(cb);
#pragma unroll
            for (int cb = 0; cb < kNBW; ++cb) {
                if (cb + kAhead < kNBW) read_blk(cb + kAhead);
                if (next && cb % 5 == 2 && cb / 5 < kPerThread) dense_convert(t + 1, cb / 5);
                const half8_t bv = __builtin_bit_cast(
                    half8_t, i16x8{v0[cb][0], v0[cb][1], v0[cb][2], v0[cb][3], v1[cb][0], v1[cb][1], v1[cb][2], v1[cb][3]});
                o[cb] = mfma(av, bv, o[cb]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // ---- next tile: registers -> LDS (the other stage), then the one after into registers
        if constexpr (SEL) {
            if (t + 2 < n_tiles) load_tile(t + 2);  // (tile t + 1 was converted between the context MFMAs)
        } else {
            if (TQ && t + 1 < n_tiles) {
                dense_read(t + 1);
#pragma unroll
                for (int i = 0; i < kPerThread; ++i) dense_convert(t + 1, i);
            }
            if (t + 3 < n_tiles) issue_tile(t + 3);  // into the raw stage of tile t, converted before  // into the raw stage of tile t, converted before
        }
        __syncthreads();
    }

    // ---- partials: o rows are heads 4 q4 + i, columns channels 256 half + 16 cb + n16
    z_run = quad_sum(z_run);
    const float back = e_run == -1000 ? 0.0f : exp2i(e_run);
    const int64_t hrow = int64_t(b) * H + h_pair;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = 4 * q4 + i;
        if (h_pair + h < H) {
            float* dst = a.part_acc + ((hrow + h) * Sn + s) * kL + half * (kL / 2) + n16;
#pragma unroll
            for (int cb = 0; cb < kNBW; ++cb) dst[16 * cb] = o[cb][i] * back;
        }
    }
    if (half == 0 && q4 == 0 && live) {
        a.part_m[(hrow + n16) * Sn + s] = m_run * kLn2;
        a.part_z[(hrow + n16) * Sn + s] = z_run;
    }
}

}  // namespace

bool decode_fp8_mfma_supported(const Fp8Pool& pool, const DecodeArgs& a) {
    return pool.head_dim == kD && pool.rope_dim == kR && pool.page_size % 16 == 0 && a.split_keys % kTile == 0 &&
           a.split_keys / 16 <= kMaxRuns;
}

hipError_t launch_decode_fp8_mfma(const Fp8Pool& pool, const DecodeArgs& a, hipStream_t s) {
    const dim3 grid(unsigned(a.n_splits), unsigned((a.n_q_heads + kHeadsWG - 1) / kHeadsWG), unsigned(a.batch));
    const TqMfmaTable none{};
    if (a.step_k) {  // kvq_decode_step: dense rows only
        if (a.sel) return hipErrorInvalidValue;
        decode_fp8_mfma<false, false, true><<<grid, dim3(kThreads), 0, s>>>(pool.codes, pool.scales, pool.page_size,
                                                                            pool.num_pages, a, none);
        return hipGetLastError();
    }
    if (a.sel)
        decode_fp8_mfma<true, false><<<grid, dim3(kThreads), 0, s>>>(pool.codes, pool.scales, pool.page_size,
                                                                     pool.num_pages, a, none);
    else
        decode_fp8_mfma<false, false><<<grid, dim3(kThreads), 0, s>>>(pool.codes, pool.scales, pool.page_size,
                                                                      pool.num_pages, a, none);
    return hipGetLastError();
}

hipError_t launch_decode_tq4_mfma(const Fp8Pool& pool, const DecodeArgs& a, hipStream_t s) {
    if (a.sel) return hipErrorInvalidValue;
    const dim3 grid(unsigned(a.n_splits), unsigned((a.n_q_heads + kHeadsWG - 1) / kHeadsWG), unsigned(a.batch));
    decode_fp8_mfma<false, true><<<grid, dim3(kThreads), 0, s>>>(pool.codes, pool.scales, pool.page_size,
                                                                 pool.num_pages, a, tq_mfma_table());
    return hipGetLastError();
}

}  // namespace kvq
