// store.hip -- quantize new K/V rows into the paged caches.
//
// 4-bit Hadamard-32 rows (TensorFold issue "qwen27 CUDA: an opt-in 4-bit
// attention cache", section "What it is"; FreeToken pull request
// "feat(kvcache): add reliable quantized KV cache", PR description and
// test-fix commit: 16 code bytes + one fp16 scale per 32 values, scale =
// amax/8) and fp8 e4m3 latent rows (colibri pull request "KV cache
// quantization: fp8 (KV8) + 4-bit TurboQuant", KV8 commit: per-row f32
// scale amax/448, RNE, saturating, NaN stored as 0, guard for an amax whose
// 448/amax overflows).
//
// The codes are bit-exact by construction: every step is one IEEE fp32
// operation in a fixed order (this file is compiled without contraction and
// with the correctly rounded fp32 divide), and binary16 conversion is the
// hardware's round-to-nearest-even convert.
#include "internal.h"

#pragma clang fp contract(off)

namespace kvq {
namespace {

// One lane per 4 consecutive values of a row, so a 32-group is 8 lanes and a
// head_dim-256 row is one wave: loads and code stores are contiguous across
// lanes.  Lanes of a group exchange values for the butterfly's upper stages
// and the amax; each lane then packs its 4 codes into 2 bytes.  Rows are
// ordered K rows first, then V rows, each (token, head) major.
// idx is the lane's global index; lane its index in the wave.  BITS: the
// code width (4, 6, 8); the scale divides amax by 8, 31 or 127 and the codes
// clamp to [-2^(BITS-1), 2^(BITS-1) - 1].
template <InType DT, int BITS>
__device__ __forceinline__ void store_q4_quad(const void* __restrict__ k, const void* __restrict__ v,
                                              const int64_t* __restrict__ slots, int n_tokens,
                                              uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool, int H,
                                              int D, int page_size, int64_t n_slots, int64_t idx, int lane) {
    const int per_row = D / 4;
    const int64_t nth = int64_t(n_tokens) * H;
    if (idx >= 2 * nth * per_row) return;
    const int e = int(idx % per_row);  // lane-in-row: values 4e .. 4e+3
    int64_t r = idx / per_row;
    const int which = r >= nth ? 1 : 0;
    r -= which * nth;                   // r = t * H + h
    const int64_t t = r / H;
    const int h = int(r % H);
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= n_slots) return;  // the whole row (all 8 lanes of each group) leaves

    float x[4];
    load4<DT>(which ? v : k, r * D + 4 * e, x);
    const int64_t page = slot / page_size, off = slot % page_size;
    uint8_t* row = (which ? v_pool : k_pool) + ((page * H + h) * page_size + off) * blk_row_bytes(BITS, D);
    encode_blk_quad<BITS>(x, row, D, e, lane);
}

template <InType DT, int BITS>
__global__ __launch_bounds__(256) void store_q4_kernel(const void* __restrict__ k, const void* __restrict__ v,
                                                       const int64_t* __restrict__ slots, int n_tokens,
                                                       uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
                                                       int H, int D, int page_size, int64_t n_slots) {
    store_q4_quad<DT, BITS>(k, v, slots, n_tokens, k_pool, v_pool, H, D, page_size, n_slots,
                            int64_t(blockIdx.x) * blockDim.x + threadIdx.x, threadIdx.x & 63);
}

// The store's lanes in the first store_blocks workgroups, the query
// rotation's in the rest: the two steps that precede the decode of a step
// are independent, and one launch costs less than two.  A workgroup runs one
// role only, and each role keeps its 8-lane groups whole.
template <InType DK, InType DQ, int BITS>
__global__ __launch_bounds__(256) void store_rotate_q4_kernel(const void* __restrict__ k, const void* __restrict__ v,
                                                              const int64_t* __restrict__ slots, int n_tokens,
                                                              uint8_t* __restrict__ k_pool,
                                                              uint8_t* __restrict__ v_pool, int H, int D,
                                                              int page_size, int64_t n_slots, unsigned store_blocks,
                                                              const void* q, float* q_rot, int64_t n_quads) {
    const int lane = threadIdx.x & 63;
    if (blockIdx.x < store_blocks) {
        store_q4_quad<DK, BITS>(k, v, slots, n_tokens, k_pool, v_pool, H, D, page_size, n_slots,
                                int64_t(blockIdx.x) * blockDim.x + threadIdx.x, lane);
        return;
    }
    const int64_t i = int64_t(blockIdx.x - store_blocks) * blockDim.x + threadIdx.x;
    if (i >= n_quads) return;  // n_quads is a multiple of 8: whole groups leave
    rotate_q_quad<DQ>(q, q_rot, i, lane);
}


// One wave per token: the latent part (L values) and the rope part (R values)
// each get their own amax, reduced across the wave, then every lane encodes
// the elements it strides over.
template <InType DT>
__global__ __launch_bounds__(64) void store_fp8_kernel(const void* __restrict__ x, const int64_t* __restrict__ slots,
                                                       int n_tokens, uint8_t* __restrict__ codes,
                                                       float* __restrict__ scales, int D, int R, int64_t n_slots) {
    const int t = blockIdx.x;
    const int lane = threadIdx.x;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= n_slots) return;
    const int L = D - R;
    const int64_t base = int64_t(t) * D;
    uint8_t* out = codes + slot * D;
#pragma unroll 1
    for (int part = 0; part < 2; ++part) {
        const int lo = part ? L : 0, n = part ? R : L;
        float amax = 0.0f;
        for (int i = lane; i < n; i += 64) amax = fmaxf(amax, fabsf(load_elem<DT>(x, base + lo + i)));  // NaN ignored
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
        const float inv = 448.0f / amax;
        const bool inert = !(amax > 0.0f) || !isfinite(amax) || !isfinite(inv);
        for (int i = lane; i < n; i += 64) {
            const float e = load_elem<DT>(x, base + lo + i);
            out[lo + i] = inert ? uint8_t(0) : uint8_t(e4m3_encode(e * inv));
        }
        if (lane == 0) scales[slot * 2 + part] = inert ? 0.0f : amax / 448.0f;
    }
}

}  // namespace

namespace {
template <int BITS>
void store_blk(dim3 grid, hipStream_t s, const Q4Pool& pool, const void* k, const void* v, InType dt,
               const int64_t* slots, int n_tokens, int64_t n_slots) {
    const int H = pool.n_kv_heads, D = pool.head_dim, P = pool.page_size;
    switch (dt) {
        case InType::F32:
            store_q4_kernel<InType::F32, BITS><<<grid, 256, 0, s>>>(k, v, slots, n_tokens, pool.k, pool.v, H, D, P, n_slots);
            break;
        case InType::BF16:
            store_q4_kernel<InType::BF16, BITS><<<grid, 256, 0, s>>>(k, v, slots, n_tokens, pool.k, pool.v, H, D, P, n_slots);
            break;
        case InType::F16:
            store_q4_kernel<InType::F16, BITS><<<grid, 256, 0, s>>>(k, v, slots, n_tokens, pool.k, pool.v, H, D, P, n_slots);
            break;
    }
}

template <InType DK, int BITS>
void store_rotate_dq(dim3 grid, hipStream_t s, const Q4Pool& pool, const void* k, const void* v, const int64_t* slots,
                     int n_tokens, int64_t n_slots, unsigned store_blocks, const void* q, InType q_dt, float* q_rot,
                     int64_t n_quads) {
    const int H = pool.n_kv_heads, D = pool.head_dim, P = pool.page_size;
    switch (q_dt) {
        case InType::F32:
            store_rotate_q4_kernel<DK, InType::F32, BITS><<<grid, 256, 0, s>>>(
                k, v, slots, n_tokens, pool.k, pool.v, H, D, P, n_slots, store_blocks, q, q_rot, n_quads);
            break;
        case InType::BF16:
            store_rotate_q4_kernel<DK, InType::BF16, BITS><<<grid, 256, 0, s>>>(
                k, v, slots, n_tokens, pool.k, pool.v, H, D, P, n_slots, store_blocks, q, q_rot, n_quads);
            break;
        case InType::F16:
            store_rotate_q4_kernel<DK, InType::F16, BITS><<<grid, 256, 0, s>>>(
                k, v, slots, n_tokens, pool.k, pool.v, H, D, P, n_slots, store_blocks, q, q_rot, n_quads);
            break;
    }
}

template <int BITS>
void store_rotate_blk(dim3 grid, hipStream_t s, const Q4Pool& pool, const void* k, const void* v, InType dt,
                      const int64_t* slots, int n_tokens, int64_t n_slots, unsigned store_blocks, const void* q,
                      InType q_dt, float* q_rot, int64_t n_quads) {
    switch (dt) {
        case InType::F32:
            store_rotate_dq<InType::F32, BITS>(grid, s, pool, k, v, slots, n_tokens, n_slots, store_blocks, q, q_dt,
                                               q_rot, n_quads);
            break;
        case InType::BF16:
            store_rotate_dq<InType::BF16, BITS>(grid, s, pool, k, v, slots, n_tokens, n_slots, store_blocks, q, q_dt,
                                                q_rot, n_quads);
            break;
        case InType::F16:
            store_rotate_dq<InType::F16, BITS>(grid, s, pool, k, v, slots, n_tokens, n_slots, store_blocks, q, q_dt,
                                               q_rot, n_quads);
            break;
    }
}
}  // namespace

hipError_t launch_store_q4(const Q4Pool& pool, const void* k, const void* v, InType dt, const int64_t* slots,
                           int n_tokens, hipStream_t s) {
    const int64_t total = int64_t(n_tokens) * pool.n_kv_heads * 2 * (pool.head_dim / 4);
    if (total == 0) return hipSuccess;
    const dim3 grid(unsigned((total + 255) / 256));
    const int64_t n_slots = int64_t(pool.num_pages) * pool.page_size;
    if (pool.bits == 8) store_blk<8>(grid, s, pool, k, v, dt, slots, n_tokens, n_slots);
    else if (pool.bits == 6) store_blk<6>(grid, s, pool, k, v, dt, slots, n_tokens, n_slots);
    else store_blk<4>(grid, s, pool, k, v, dt, slots, n_tokens, n_slots);
    return hipGetLastError();
}

hipError_t launch_store_rotate_q4(const Q4Pool& pool, const void* k, const void* v, InType dt, const int64_t* slots,
                                  int n_tokens, const void* q, InType q_dt, float* q_rot, int n_rows, hipStream_t s) {
    const int64_t store_lanes = int64_t(n_tokens) * pool.n_kv_heads * 2 * (pool.head_dim / 4);
    const int64_t n_quads = int64_t(n_rows) * (pool.head_dim / 4);
    const unsigned store_blocks = unsigned((store_lanes + 255) / 256);
    const unsigned rot_blocks = unsigned((n_quads + 255) / 256);
    if (store_blocks + rot_blocks == 0) return hipSuccess;
    const dim3 grid(store_blocks + rot_blocks);
    const int64_t n_slots = int64_t(pool.num_pages) * pool.page_size;
    if (pool.bits == 8)
        store_rotate_blk<8>(grid, s, pool, k, v, dt, slots, n_tokens, n_slots, store_blocks, q, q_dt, q_rot, n_quads);
    else if (pool.bits == 6)
        store_rotate_blk<6>(grid, s, pool, k, v, dt, slots, n_tokens, n_slots, store_blocks, q, q_dt, q_rot, n_quads);
    else
        store_rotate_blk<4>(grid, s, pool, k, v, dt, slots, n_tokens, n_slots, store_blocks, q, q_dt, q_rot, n_quads);
    return hipGetLastError();
}

hipError_t launch_store_fp8(const Fp8Pool& pool, const void* x, InType dt, const int64_t* slots, int n_tokens,
                            hipStream_t s) {
    if (n_tokens == 0) return hipSuccess;
    const int64_t n_slots = int64_t(pool.num_pages) * pool.page_size;
    const dim3 block(64), grid(static_cast<unsigned>(n_tokens));
    switch (dt) {
        case InType::F32:
            store_fp8_kernel<InType::F32><<<grid, block, 0, s>>>(x, slots, n_tokens, pool.codes, pool.scales,
                                                                 pool.head_dim, pool.rope_dim, n_slots);
            break;
        case InType::BF16:
            store_fp8_kernel<InType::BF16><<<grid, block, 0, s>>>(x, slots, n_tokens, pool.codes, pool.scales,
                                                                  pool.head_dim, pool.rope_dim, n_slots);
            break;
        case InType::F16:
            store_fp8_kernel<InType::F16><<<grid, block, 0, s>>>(x, slots, n_tokens, pool.codes, pool.scales,
                                                                 pool.head_dim, pool.rope_dim, n_slots);
            break;
    }
    return hipGetLastError();
}

}  // namespace kvq
