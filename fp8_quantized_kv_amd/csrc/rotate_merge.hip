// rotate_merge.hip -- the query rotation and the log-sum-exp merge.
//
// TensorFold issue "qwen27 CUDA: an opt-in 4-bit attention cache", section
// "What it is": rotate the queries once, merge the chunk partials in order,
// rotate the output back once.  colibri pull request "KV cache quantization:
// fp8 (KV8) + 4-bit TurboQuant", split-T commit: partials (cl[K], m, z) and
// a log-sum-exp merge kernel.
#include "internal.h"

namespace kvq {
namespace {

// One lane per 4 consecutive query values (a 32-group is 8 lanes, a row of
// 256 values one wave); q may alias q_rot.
template <InType DT>
__global__ __launch_bounds__(256) void rotate_q_kernel(const void* q, float* q_rot, int64_t n_quads) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n_quads) return;  // n_quads is a multiple of 8: whole groups leave
    rotate_q_quad<DT>(q, q_rot, i, threadIdx.x & 63);
}

constexpr int kMergeWaves = 4;
constexpr int kMergeCh = 64;     // output channels per workgroup (two Hadamard groups)
constexpr int kMergeBatch = 32;  // partial loads in flight per lane

// Workgroup (sequence x query head, 64-channel block).  Weights w_s =
// exp(m_s - M) are formed per used split s < n; wave w sums acc_s[c] * w_s
// over the splits s = w, w + 4, w + 8, ... in ascending order, and the four
// sums are added in wave order, so the result depends only on the sequence's
// own partials.  Because that order does not depend on n, every load is
// issued before the sequence length arrives (for all S allocated splits,
// masked afterwards): one memory round trip instead of two.  Z = sum_s z_s
// w_s runs over s = lane, lane + 64, ... ascending, then a butterfly; every
// wave forms it from the z_s it loaded up front (splits past 256 are read in
// the loop), so no barrier hands it over.
// For the 4-bit cache the normalized rotated-domain vector is rotated back
// with H32 (its own inverse): out[c] = sum_j H[c%32][j] * O[32*(c/32) + j],
// H[i][j] = (-1)^popcount(i&j) / sqrt(32).
constexpr int kMergeZPre = 4;  // z_s preloaded per lane: s = lane + 64 k, k < 4 (s < 256)

__global__ __launch_bounds__(kMergeWaves * 64) void merge_kernel(const float* __restrict__ part_acc,
                                                                 const float* __restrict__ part_m,
                                                                 const float* __restrict__ part_z,
                                                                 const int32_t* __restrict__ seq_lens,
                                                                 int n_q_heads, int max_seq_len, int S,
                                                                 int split_keys, int dv, int rotate,
                                                                 float* __restrict__ out, float* __restrict__ lse) {
    extern __shared__ float w[];  // [S] split weights
    __shared__ float part[kMergeWaves][kMergeCh];
    __shared__ float red[kMergeWaves];

    const int bh = blockIdx.x, c0 = blockIdx.y * kMergeCh;
    const int b = bh / n_q_heads;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const float* pm = part_m + int64_t(bh) * S;
    const float* pz = part_z + int64_t(bh) * S;
    const float* pa = part_acc + int64_t(bh) * S * dv + c0 + lane;

    // Loads that do not need the sequence length: this wave's first batch of
    // partials, (m, z) of the split this thread forms the weight of, and the
    // z_s of this lane's first Z terms.
    int T = seq_lens[b];
    float v[kMergeBatch];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
        const int sk = wave + kMergeWaves * k;
        v[k] = sk < S ? pa[int64_t(sk) * dv] : 0.0f;
    }
    const float my_m = tid < S ? pm[tid] : -INFINITY;
    const float my_z = tid < S ? pz[tid] : 0.0f;
    float zl[kMergeZPre];
#pragma unroll
    for (int k = 0; k < kMergeZPre; ++k) zl[k] = lane + 64 * k < S ? pz[lane + 64 * k] : 0.0f;

    T = T < 0 ? 0 : (T > max_seq_len ? max_seq_len : T);
    const int n = (T + split_keys - 1) / split_keys;
    float* o = out + int64_t(bh) * dv;
    if (n == 0) {
        if (tid < kMergeCh) o[c0 + tid] = 0.0f;
        if (lse && blockIdx.y == 0 && tid == 0) lse[bh] = -INFINITY;
        return;
    }

    // M = max over the used splits (exact, so the reduction order is moot).
    float mx = tid < n ? my_m : -INFINITY;
    for (int s = tid + kMergeWaves * 64; s < n; s += kMergeWaves * 64) mx = fmaxf(mx, pm[s]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (tid < n) w[tid] = my_z > 0.0f ? expf(my_m - M) : 0.0f;
    for (int s = tid + kMergeWaves * 64; s < n; s += kMergeWaves * 64) w[s] = pz[s] > 0.0f ? expf(pm[s] - M) : 0.0f;
    __syncthreads();
    // Z: lane-strided partial sums in ascending order, then a fixed butterfly (every wave alike)
    float z = 0.0f;
#pragma unroll
    for (int k = 0; k < kMergeZPre; ++k)
        if (lane + 64 * k < n) z += zl[k] * w[lane + 64 * k];
    for (int s = lane + 64 * kMergeZPre; s < n; s += 64) z += pz[s] * w[s];
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) z += __shfl_xor(z, m, 64);
    // this wave's splits wave + 4k < n, ascending
    float acc = 0.0f;
    for (int k0 = 0; wave + kMergeWaves * k0 < n; k0 += kMergeBatch) {
        if (k0 > 0) {
#pragma unroll
            for (int k = 0; k < kMergeBatch; ++k) {
                const int sk = wave + kMergeWaves * (k0 + k);
                v[k] = sk < n ? pa[int64_t(sk) * dv] : 0.0f;
            }
        }
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) {
            const int sk = wave + kMergeWaves * (k0 + k);
            if (sk < n) acc += v[k] * w[sk];
        }
    }
    part[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    // Z = 0: no split holds a key (every entry of a selection absent): out = 0, lse = -inf
    const float orot = z > 0.0f ? (((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane]) / z : 0.0f;
    if (rotate) {  // within wave 0: its own LDS row, a wave barrier
        float* o_rot = part[0];
        __builtin_amdgcn_wave_barrier();
        o_rot[lane] = orot;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const float* blk = o_rot + (lane & ~31);
        const int i = lane & 31;
        float r = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; ++j) r += (__popc(unsigned(i & j)) & 1) ? -blk[j] : blk[j];
        o[c0 + lane] = r * inv_sqrt32();
    } else {
        o[c0 + lane] = orot;
    }
    if (lse && blockIdx.y == 0 && lane == 0) lse[bh] = z > 0.0f ? M + logf(z) : -INFINITY;
}

// Partials with at most 64 splits (short contexts, short selections, many
// rows): one wave per (sequence x query head, 64-channel block), four items
// per workgroup, instead of four waves on one item.  Same arithmetic in the
// same order as merge_kernel: lane s < n forms w_s = exp(m_s - M); Z is the
// same lane-strided sum (one term per lane here) and butterfly; the context
// keeps the four partial sums of the splits s = 0, 1, 2, 3 (mod 4), each in
// ascending s, and adds them in that order -- so the bits equal merge_kernel's.
constexpr int kSmallS = 64;

__global__ __launch_bounds__(kMergeWaves * 64) void merge_small_kernel(const float* __restrict__ part_acc,
                                                                       const float* __restrict__ part_m,
                                                                       const float* __restrict__ part_z,
                                                                       const int32_t* __restrict__ seq_lens,
                                                                       int n_q_heads, int max_seq_len, int S,
                                                                       int split_keys, int dv, int rotate,
                                                                       int64_t n_items, float* __restrict__ out,
                                                                       float* __restrict__ lse) {
    __shared__ float o_rot[kMergeWaves][kMergeCh];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t item = int64_t(blockIdx.x) * kMergeWaves + wave;
    if (item >= n_items) return;  // a whole wave; no workgroup barrier below
    const int n_blk = dv / kMergeCh;
    const int64_t bh = item / n_blk;
    const int c0 = int(item % n_blk) * kMergeCh;
    const int b = int(bh / n_q_heads);
    const float* pa = part_acc + bh * S * dv + c0 + lane;

    int T = seq_lens[b];
    float v[kSmallS];
#pragma unroll
    for (int k = 0; k < kSmallS; ++k) v[k] = k < S ? pa[int64_t(k) * dv] : 0.0f;
    const float my_m = lane < S ? part_m[bh * S + lane] : -INFINITY;
    const float my_z = lane < S ? part_z[bh * S + lane] : 0.0f;

    T = T < 0 ? 0 : (T > max_seq_len ? max_seq_len : T);
    const int n = (T + split_keys - 1) / split_keys;
    float* o = out + bh * dv;
    if (n == 0) {
        o[c0 + lane] = 0.0f;
        if (lse && c0 == 0 && lane == 0) lse[bh] = -INFINITY;
        return;
    }
    float M = lane < n ? my_m : -INFINITY;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
    const float w = lane < n ? (my_z > 0.0f ? expf(my_m - M) : 0.0f) : 0.0f;
    float z = lane < n ? my_z * w : 0.0f;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) z += __shfl_xor(z, m, 64);

    float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < kSmallS; ++k) {
        if (k < n) {
            const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));
            p[k & 3] += v[k] * wk;
        }
    }
    // z = 0: no split holds a key (every entry of a selection absent): out = 0, lse = -inf
    const float orot = z > 0.0f ? (((p[0] + p[1]) + p[2]) + p[3]) / z : 0.0f;
    if (rotate) {
        o_rot[wave][lane] = orot;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const float* blk = &o_rot[wave][lane & ~31];
        const int i = lane & 31;
        float r = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; ++j) r += (__popc(unsigned(i & j)) & 1) ? -blk[j] : blk[j];
        o[c0 + lane] = r * inv_sqrt32();
    } else {
        o[c0 + lane] = orot;
    }
    if (lse && c0 == 0 && lane == 0) lse[bh] = z > 0.0f ? M + logf(z) : -INFINITY;
}

}  // namespace

hipError_t launch_rotate_q(const void* q, InType dt, float* q_rot, int n_rows, int head_dim, hipStream_t s) {
    const int64_t n_quads = int64_t(n_rows) * (head_dim / 4);
    if (n_quads == 0) return hipSuccess;
    const dim3 block(256), grid(unsigned((n_quads + 255) / 256));
    switch (dt) {
        case InType::F32: rotate_q_kernel<InType::F32><<<grid, block, 0, s>>>(q, q_rot, n_quads); break;
        case InType::BF16: rotate_q_kernel<InType::BF16><<<grid, block, 0, s>>>(q, q_rot, n_quads); break;
        case InType::F16: rotate_q_kernel<InType::F16><<<grid, block, 0, s>>>(q, q_rot, n_quads); break;
    }
    return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
    if (a.batch == 0) return hipSuccess;
    // One wave per item pays off once there are enough items to fill the GPU
    // (measured: 384 items 5.7 vs 6.0 us, 16384 items 13.7 vs 35 us; 96 items
    // 5.9 vs 5.0 us).  Both kernels give the same bits, so the choice is free.
    const int64_t n_items = int64_t(a.batch) * a.n_q_heads * (a.dv / kMergeCh);
    if (a.n_splits <= kSmallS && n_items >= 256) {
        const dim3 grid(unsigned((n_items + kMergeWaves - 1) / kMergeWaves));
        merge_small_kernel<<<grid, dim3(kMergeWaves * 64), 0, s>>>(
            a.part_acc, a.part_m, a.part_z, a.seq_lens, a.n_q_heads, a.max_seq_len, a.n_splits, a.split_keys, a.dv,
            a.rotate ? 1 : 0, n_items, a.out, a.lse);
        return hipGetLastError();
    }
    const size_t shm = sizeof(float) * size_t(a.n_splits);
    const dim3 grid(unsigned(a.batch * a.n_q_heads), unsigned(a.dv / kMergeCh));
    merge_kernel<<<grid, dim3(kMergeWaves * 64), shm, s>>>(
        a.part_acc, a.part_m, a.part_z, a.seq_lens, a.n_q_heads, a.max_seq_len, a.n_splits, a.split_keys, a.dv,
        a.rotate ? 1 : 0, a.out, a.lse);
    return hipGetLastError();
}

}  // namespace kvq
