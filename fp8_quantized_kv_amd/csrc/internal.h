// internal.h -- declarations shared by the kernels and the C-ABI layer of
// libkvq (not installed; the public interface is include/kvq.h).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace kvq {

// Element types a store or rotation may read.
enum class InType : int { F32 = 0, BF16 = 1, F16 = 2 };

// Rows of the 4-bit format: D/2 code bytes then D/32 fp16 scales.
__host__ __device__ constexpr int q4_row_bytes(int D) { return D / 2 + 2 * (D / 32); }

// Block formats of the same skeleton with codes of BITS = 4, 6 or 8 bits:
// per 32-value group 16, 24 or 32 code bytes (6 bits: 16 bytes of low
// nibbles laid out as the 4-bit codes, then 8 bytes holding the high two bits
// of codes 4j..4j+3 in byte j); a row is all groups' codes, then the fp16
// scales; scale = fp16(amax / divisor), codes clamped to the signed range.
__host__ __device__ constexpr int blk_group_bytes(int bits) { return bits == 4 ? 16 : (bits == 6 ? 24 : 32); }
__host__ __device__ constexpr int blk_row_bytes(int bits, int D) { return (blk_group_bytes(bits) + 2) * (D / 32); }

// ln(2) and log2(e) in fp32.
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

// fp32(1/sqrt(32)) = 0x3E3504F3, the Hadamard-32 normalisation.
__device__ __forceinline__ float inv_sqrt32() { return __uint_as_float(0x3E3504F3u); }

template <InType T>
__device__ __forceinline__ float load_elem(const void* p, int64_t i);

template <>
__device__ __forceinline__ float load_elem<InType::F32>(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
}
template <>
__device__ __forceinline__ float load_elem<InType::BF16>(const void* p, int64_t i) {
    return __uint_as_float(uint32_t(static_cast<const uint16_t*>(p)[i]) << 16);
}
template <>
__device__ __forceinline__ float load_elem<InType::F16>(const void* p, int64_t i) {
    return __half2float(__ushort_as_half(static_cast<const uint16_t*>(p)[i]));
}

// Four consecutive elements i .. i+3 (i a multiple of 4, the row 16-byte
// aligned) widened to fp32.
template <InType T>
__device__ __forceinline__ void load4(const void* p, int64_t i, float (&x)[4]);

template <>
__device__ __forceinline__ void load4<InType::F32>(const void* p, int64_t i, float (&x)[4]) {
    const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    x[0] = v.x;
    x[1] = v.y;
    x[2] = v.z;
    x[3] = v.w;
}
template <>
__device__ __forceinline__ void load4<InType::BF16>(const void* p, int64_t i, float (&x)[4]) {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
    x[0] = __uint_as_float(w.x << 16);
    x[1] = __uint_as_float(w.x & 0xFFFF0000u);
    x[2] = __uint_as_float(w.y << 16);
    x[3] = __uint_as_float(w.y & 0xFFFF0000u);
}
template <>
__device__ __forceinline__ void load4<InType::F16>(const void* p, int64_t i, float (&x)[4]) {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
    x[0] = __half2float(__ushort_as_half(uint16_t(w.x)));
    x[1] = __half2float(__ushort_as_half(uint16_t(w.x >> 16)));
    x[2] = __half2float(__ushort_as_half(uint16_t(w.y)));
    x[3] = __half2float(__ushort_as_half(uint16_t(w.y >> 16)));
}

// Unnormalised Hadamard-32 butterfly of a group spread over 8 consecutive
// lanes (8-aligned within the wave): lane j = lane & 7 holds elements
// 4j .. 4j+3.  Stages 1 and 2 pair elements inside a lane, stages 4, 8 and
// 16 pair lane j with lane j ^ 1, ^ 2, ^ 4.  Every pair (a, b), a the lower
// element, becomes (a + b, a - b) exactly as in the one-lane butterfly.
__device__ __forceinline__ void h32_butterfly_lanes8(float (&x)[4], int lane) {
    float a = x[0], b = x[1];
    x[0] = a + b;
    x[1] = a - b;
    a = x[2];
    b = x[3];
    x[2] = a + b;
    x[3] = a - b;
    a = x[0];
    b = x[2];
    x[0] = a + b;
    x[2] = a - b;
    a = x[1];
    b = x[3];
    x[1] = a + b;
    x[3] = a - b;
#pragma unroll
    for (int m = 1; m <= 4; m <<= 1) {
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float o = __shfl_xor(x[i], m, 64);
            x[i] = upper ? o - x[i] : x[i] + o;
        }
    }
}

// Query rotation, one lane per 4 consecutive values i .. i+3 of q (i = 4 *
// quad; a 32-group is 8 lanes, 8-aligned in the wave): the butterfly above,
// then x fp32(1/sqrt(32)) -- the transform the store applies to K and V, in
// the same order.  Each value is read and written by the same lane, so q may
// alias q_rot.  Every lane of a group must call it (the lanes exchange values).
template <InType DT>
__device__ __forceinline__ void rotate_q_quad(const void* q, float* q_rot, int64_t quad, int lane) {
    float x[4];
    load4<DT>(q, 4 * quad, x);
    h32_butterfly_lanes8(x, lane);
    const float c = inv_sqrt32();
    *reinterpret_cast<float4*>(q_rot + 4 * quad) = make_float4(x[0] * c, x[1] * c, x[2] * c, x[3] * c);
}

// N load4s (elements i[n] .. i[n] + 3 of p[n]) with the element type chosen
// at run time (uniform across the wave): one branch around all N, so the
// loads are issued together and waited for once.
template <int N>
__device__ __forceinline__ void load4n_dyn(InType dt, const void* const (&p)[N], const int64_t (&i)[N],
                                           float (&x)[N][4]) {
    if (dt == InType::F32) {
#pragma unroll
        for (int n = 0; n < N; ++n) load4<InType::F32>(p[n], i[n], x[n]);
    } else if (dt == InType::BF16) {
#pragma unroll
        for (int n = 0; n < N; ++n) load4<InType::BF16>(p[n], i[n], x[n]);
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) load4<InType::F16>(p[n], i[n], x[n]);
    }
}

// The query rotation above for the decode kernels' lane layout: lane (n, q)
// = n + 16 q holds elements 8q .. 8q + 7 of a 32-group (q = 0..3), i.e. the
// quads 2q and 2q + 1 of rotate_q_quad.  The same stages in the same order
// on the same operands: stages 1 and 2 inside each quad, stage 4 between the
// lane's two quads, stages 8 and 16 with lane ^ 16 and lane ^ 32; every pair
// (a, b), a the lower element, becomes (a + b, a - b); then x
// fp32(1/sqrt(32)).  So y equals kvq_rotate_q's output bit for bit.  The
// cross-lane stages take the partner's value with the permlane swaps (of the
// pair they return, element 0 is the lower lane's value, element 1 the upper
// lane's) and form lo + s * hi with s = +1 (lower lane) or -1 (upper lane) in
// one fma: s * hi is exact, so the single rounding gives lo + hi or lo - hi
// exactly.  Every lane of the four q-lanes of a group must call it.
__device__ __forceinline__ void rotate_q_lanes4(float (&y)[8], int lane) {
#pragma unroll
    for (int h = 0; h < 8; h += 4) {
        float a = y[h], b = y[h + 1];
        y[h] = a + b;
        y[h + 1] = a - b;
        a = y[h + 2];
        b = y[h + 3];
        y[h + 2] = a + b;
        y[h + 3] = a - b;
        a = y[h];
        b = y[h + 2];
        y[h] = a + b;
        y[h + 2] = a - b;
        a = y[h + 1];
        b = y[h + 3];
        y[h + 1] = a + b;
        y[h + 3] = a - b;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = y[i], b = y[i + 4];
        y[i] = a + b;
        y[i + 4] = a - b;
    }
    const float s16 = (lane & 16) ? -1.0f : 1.0f, s32 = (lane & 32) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(y[i]), __float_as_uint(y[i]), false, false);
        y[i] = fmaf(s16, __uint_as_float(p[1]), __uint_as_float(p[0]));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(y[i]), __float_as_uint(y[i]), false, false);
        y[i] = fmaf(s32, __uint_as_float(p[1]), __uint_as_float(p[0]));
    }
    const float c = inv_sqrt32();
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = y[i] * c;
}

// The rotated query for the packed B layout (columns n and n ^ 8 of a
// 16-lane row hold the same head): lane n of a row rotates the groups of
// parity n >> 3 of each pair (2k, 2k + 1) -- x[k] holds its 8 raw values of
// group 2k + (n >> 3) -- and the two halves swap the results (row_ror:8), so
// every lane ends with all NG groups of its head, NG / 2 rotations each.
template <int NG>
__device__ __forceinline__ void rotate_q_packed(float (&x)[NG / 2][8], float (&q)[NG][8], int lane) {
    const bool odd = (lane & 8) != 0;
#pragma unroll
    for (int k = 0; k < NG / 2; ++k) {
        rotate_q_lanes4(x[k], lane);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float other =
                __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x[k][i]), 0x128, 0xF, 0xF, true));
            q[2 * k][i] = odd ? other : x[k][i];
            q[2 * k + 1][i] = odd ? x[k][i] : other;
        }
    }
}

// The block-format encoder of one lane's 4 consecutive values x of a row
// (lane-in-row e: values 4e .. 4e + 3; a 32-group is 8 lanes, 8-aligned in
// the wave): the Hadamard-32 butterfly, x fp32(1/sqrt(32)), the group's amax,
// scale = fp16_rne(amax / divisor) and codes round-half-even(x / scale)
// clamped to the signed BITS-bit range, written into `row` (a row of
// blk_row_bytes(BITS, D) bytes).  Every step is one IEEE fp32 operation in a
// fixed order (compiled without contraction, with the correctly rounded
// divide), so the stored bytes do not depend on which kernel calls it.
template <int BITS>
__device__ __forceinline__ void encode_blk_quad(float (&x)[4], uint8_t* __restrict__ row, int D, int e, int lane) {
    h32_butterfly_lanes8(x, lane);
    const float c = inv_sqrt32();
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = x[i] * c;
        amax = fmaxf(amax, fabsf(x[i]));
    }
#pragma unroll
    for (int m = 1; m <= 4; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    // scale = fp16_rne(amax / divisor); for 4 bits amax * 0.125 is the same
    // exactly rounded value as amax / 8.
    const __half s16 = __float2half_rn(BITS == 4 ? amax * 0.125f : amax / (BITS == 6 ? 31.0f : 127.0f));
    const float s = __half2float(s16);
    constexpr float kMax = float((1 << (BITS - 1)) - 1), kMin = -float(1 << (BITS - 1));
    int q[4] = {0, 0, 0, 0};
    if (s != 0.0f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float n = rintf(x[i] / s);  // correctly rounded divide, then half-to-even
            n = fminf(fmaxf(n, kMin), kMax);
            q[i] = int(n);
        }
    }
    // Values 4j .. 4j+3 of group g (j = e & 7, g = e >> 3).
    const int g = e >> 3, j = e & 7;
    uint8_t* grp = row + g * blk_group_bytes(BITS);
    if (BITS == 8) {
        uint32_t w = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) w |= (uint32_t(q[i]) & 0xFFu) << (8 * i);
        reinterpret_cast<uint32_t*>(grp)[j] = w;
    } else {
        // value 2k in the low nibble of byte k, value 2k+1 in the high nibble
        uint32_t nib = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) nib |= (uint32_t(q[i]) & 0xFu) << (4 * i);
        reinterpret_cast<uint16_t*>(grp)[j] = uint16_t(nib);
        if (BITS == 6) {
            uint32_t top = 0u;  // high two bits of value 4j + i in bits 2i .. 2i+1 of byte j
#pragma unroll
            for (int i = 0; i < 4; ++i) top |= ((uint32_t(q[i]) >> 4) & 3u) << (2 * i);
            grp[16 + j] = uint8_t(top);
        }
    }
    if (j == 0) reinterpret_cast<uint16_t*>(row + (D / 32) * blk_group_bytes(BITS))[g] = __half_as_ushort(s16);
}

// e4m3 ("fn": bias 7, max 448) code of v, round to nearest even, saturating
// to +-448, NaN -> 0x00, signed zero kept.  Bit manipulation on the fp32
// encoding: the top 3 mantissa bits survive and the 20 below decide rounding.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return 0u;                 // NaN
    if (a >= 0x43E00000u) return sign | 0x7Eu;      // |v| >= 448, incl. infinity
    if (a < 0x3C800000u) {                          // |v| < 2^-6: spacing 2^-9
        const float n = rintf(__uint_as_float(a) * 512.0f);  // exact scaling, then RNE
        return sign | uint32_t(n);                  // n == 8 is the smallest normal
    }
    uint32_t code = ((((a >> 23) - 127u + 7u)) << 3) | ((a >> 20) & 7u);
    const uint32_t rem = a & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) code += 1u;  // carry may bump the exponent
    return sign | code;
}

// ------------------------------------------------------------------ launchers
// Each returns the hipError_t of its launch; shapes are validated by the caller.

struct Q4Pool {
    uint8_t* k;
    uint8_t* v;
    int n_kv_heads;
    int head_dim;
    int page_size;
    int num_pages;
    int bits = 4;  // code width of the block format (4, 6 or 8)
};

struct Fp8Pool {
    uint8_t* codes;   // [slots][head_dim]
    float* scales;    // [slots][2]
    int head_dim;
    int rope_dim;
    int page_size;
    int num_pages;
};

hipError_t launch_store_q4(const Q4Pool& pool, const void* k, const void* v, InType dt, const int64_t* slots,
                           int n_tokens, hipStream_t s);
hipError_t launch_store_fp8(const Fp8Pool& pool, const void* x, InType dt, const int64_t* slots, int n_tokens,
                            hipStream_t s);
hipError_t launch_rotate_q(const void* q, InType dt, float* q_rot, int n_rows, int head_dim, hipStream_t s);
// The 4-bit store and the query rotation (q rows of the pool's head_dim) as
// one launch; the same results as the two launches above.
hipError_t launch_store_rotate_q4(const Q4Pool& pool, const void* k, const void* v, InType dt, const int64_t* slots,
                                  int n_tokens, const void* q, InType q_dt, float* q_rot, int n_rows, hipStream_t s);

struct DecodeArgs {
    const float* q;
    int n_q_heads;
    const int32_t* page_table;
    int max_pages;
    const int32_t* seq_lens;
    int batch;
    int max_seq_len;
    int n_splits;
    float sm_scale;
    int split_keys;
    float* part_acc;
    float* part_m;
    float* part_z;
    // Selected rows (fp8 latent only): when set, the keys of sequence b are
    // the positions sel[b * sel_stride + k], k < seq_lens[b] (max_seq_len is
    // the list capacity); entries outside the page capacity are absent.
    const int32_t* sel = nullptr;
    int sel_stride = 0;
    // Drafted rows (4-bit formats, kvq_decode_attn_rows): when rows > 0 the
    // batch entries are `rows` query rows of one sequence, sharing one
    // page-table row, and the grid is the row layout of decode_block.
    int rows = 0;
    // Decode step (kvq_decode_step, 4-bit format): when step_k is set, q is
    // unused and step_q holds the query before rotation ([batch][n_q_heads]
    // [D], type step_q_dt), which each workgroup rotates for the heads it
    // reads; and token b's K and V rows (step_k, step_v: [batch][H][D], type
    // step_kv_dt) are stored at position seq_lens[b] - 1 of sequence b by the
    // one wave whose key range holds that position, before any copy of it.
    const void* step_k = nullptr;
    const void* step_v = nullptr;
    const void* step_q = nullptr;
    InType step_kv_dt = InType::F32;
    InType step_q_dt = InType::F32;
};

// Block coordinates (split s, KV head g, batch entry b) of this workgroup.
// Plain launches: the grid is (splits, KV heads, batch).  Row launches
// (a.rows > 0): a 1-D grid whose workgroup L runs on XCD L % 8 (the
// dispatcher's round robin) as that XCD's (L / 8)-th; each run of a.rows
// consecutive workgroups on an XCD takes the rows of one (split, KV head), so
// they are dispatched together and the rows after the first find the tiles
// in that XCD's L2.  Returns false for the padding workgroups of the last
// round (the whole workgroup then exits before any barrier).
__device__ __forceinline__ bool decode_block(const DecodeArgs& a, int n_kv_heads, int& s, int& g, int& b) {
    if (a.rows == 0) {
        s = blockIdx.x;
        g = blockIdx.y;
        b = blockIdx.z;
        return true;
    }
    const unsigned L = blockIdx.x, xcd = L % 8u, k = L / 8u;
    const unsigned sg = (k / unsigned(a.rows)) * 8u + xcd;
    b = int(k % unsigned(a.rows));
    if (sg >= unsigned(a.n_splits) * unsigned(n_kv_heads)) return false;
    s = int(sg % unsigned(a.n_splits));
    g = int(sg / unsigned(a.n_splits));
    return true;
}

// The launch grid matching decode_block.
inline dim3 decode_grid(const DecodeArgs& a, int n_kv_heads) {
    if (a.rows == 0) return dim3(unsigned(a.n_splits), unsigned(n_kv_heads), unsigned(a.batch));
    const unsigned n_sg = unsigned(a.n_splits) * unsigned(n_kv_heads);
    return dim3(8u * unsigned(a.rows) * ((n_sg + 7u) / 8u));
}

// Matrix-core kernel for the 4-bit cache (head_dim 128/256, pages of a
// multiple of 16 tokens, groups of up to 16 query heads, split_keys <= 8192).
bool decode_q4_mfma_supported(const Q4Pool& pool, const DecodeArgs& a);
hipError_t launch_decode_q4_mfma(const Q4Pool& pool, const DecodeArgs& a, hipStream_t s);
// The STEP form of it (a.step_k set): head_dim 256, 4 bits, groups of up to
// 8 query heads, splits of more than 1024 keys, no drafted rows.
bool decode_q4_mfma_step_supported(const Q4Pool& pool, const DecodeArgs& a);

// Matrix-core kernel for head_dim 256 and groups of up to 8 query heads, a
// pair of waves sharing each key tile by channel halves (split_keys a
// multiple of 128, at most 1024).
bool decode_q4_pair_supported(const Q4Pool& pool, const DecodeArgs& a);
hipError_t launch_decode_q4_pair(const Q4Pool& pool, const DecodeArgs& a, hipStream_t s);
// Both forms (plain and STEP) run wherever decode_q4_pair_supported holds.

// Matrix-core kernel for the fp8 latent cache (512 + 64, pages of a
// multiple of 16 tokens, split_keys <= 2048), over consecutive positions or
// (a.sel set) over a list of selected positions.
bool decode_fp8_mfma_supported(const Fp8Pool& pool, const DecodeArgs& a);
hipError_t launch_decode_fp8_mfma(const Fp8Pool& pool, const DecodeArgs& a, hipStream_t s);

// Matrix-core kernel for several query rows of one sequence (a prompt chunk):
// a.batch rows with lengths a.seq_lens over the one page-table row
// a.page_table; head_dim 128/256, groups of up to 8 query heads, pages of a
// multiple of 16 tokens, split_keys a multiple of 32.
bool decode_q4_chunk_supported(const Q4Pool& pool, const DecodeArgs& a);
hipError_t launch_decode_q4_chunk(const Q4Pool& pool, const DecodeArgs& a, hipStream_t s);

// Plain fp32 vector-math kernels (any supported head_dim).
hipError_t launch_decode_q4_simple(const Q4Pool& pool, const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_fp8_simple(const Fp8Pool& pool, const DecodeArgs& a, hipStream_t s);

// Rotated-int4 + Lloyd-Max latent codec (tq4.hip): fp32 levels and the 15
// thresholds between them, derived once per process on the host.  The pool
// is an Fp8Pool whose codes are 288-byte nibble rows and whose scales are the
// two radii.
struct TqTables {
    float lev[16];
    float thr[15];
};
const TqTables& tq_tables();
hipError_t launch_store_tq4(const Fp8Pool& pool, const void* x, InType dt, const int64_t* slots, int n_tokens,
                            hipStream_t s);
hipError_t launch_decode_tq4_simple(const Fp8Pool& pool, const DecodeArgs& a, hipStream_t s);
// The levels as the matrix-core decode uses them: f16 of c * lev[k] split into
// low / high bytes (entry k is byte k), and the radius multipliers
// 1 / (c sqrt(512)), 1 / (c sqrt(64)).
struct TqMfmaTable {
    uint32_t lo[4];
    uint32_t hi[4];
    float f_latent;
    float f_rope;
    float c;          // the scale (host-side record)
    float max_dev;    // max_k |f16(c lev[k]) - c lev[k]| / |c lev[k]|
};
const TqMfmaTable& tq_mfma_table();
hipError_t launch_decode_tq4_mfma(const Fp8Pool& pool, const DecodeArgs& a, hipStream_t s);
hipError_t launch_tq_rotate(const float* x, float* y, int64_t n_rows, int row_len, bool inverse, hipStream_t s);
hipError_t launch_store_rotate_tq4(const Fp8Pool& pool, const void* x, InType dt, const int64_t* slots, int n_tokens,
                                   const float* q, float* q_rot, int n_rows, hipStream_t s);

struct MergeArgs {
    const float* part_acc;
    const float* part_m;
    const float* part_z;
    const int32_t* seq_lens;
    int batch;
    int n_q_heads;
    int max_seq_len;
    int n_splits;
    int split_keys;
    int dv;
    bool rotate;
    float* out;
    float* lse;
};

hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
// TQ4 latent rows (dv 512, a.rotate false): the merge and the inverse rotation
// of the merged context in one launch, the bits of launch_merge followed by
// launch_tq_rotate(out, out, rows, 512, inverse).
hipError_t launch_merge_tq(const MergeArgs& a, hipStream_t s);

// Read-bandwidth measurement (bytes a multiple of 16 KiB): XOR of every
// 32-bit word of src folded into *xor_out.
hipError_t launch_stream_read(const void* src, size_t bytes, bool non_temporal, uint32_t* xor_out, hipStream_t s);

}  // namespace kvq
