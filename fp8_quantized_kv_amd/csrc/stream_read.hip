// stream_read.hip -- the HBM read ceiling the decode kernels are measured
// against: every 16-byte chunk of a buffer copied once into LDS with the
// same LDS-DMA instruction the 4-bit decode kernels stream their cache rows
// with, with or without the non-temporal hint; the final 16 KiB block is
// folded into one XOR, a result the caller can check.
#include "internal.h"
#include "mfma_common.h"

namespace kvq {
namespace {

using namespace mx;

constexpr int kStreamWaves = 4;
constexpr int kStreamU = 4;        // 1 KiB DMA instructions per wave and step
constexpr int kStreamGrid = 2048;  // workgroups (16 KiB of LDS each)

// The buffer is n_steps steps of 16 KiB (the caller checks that bytes is a
// multiple of 16 KiB, so every copy is in bounds).  Workgroup w takes steps
// w, w + gridDim.x, ...; wave v copies KiB 4v .. 4v + 3 of a step into its
// LDS slot and waits for it before the next step (reading the slot back
// every step would leave the memory pipe idle meanwhile).  The workgroup
// whose last step is the buffer's final 16 KiB block folds that block into
// the result: four atomics in all (one per wave of every workgroup piled up
// on the one address at the end of the launch and cost ~15% of the rate).
template <bool NT>
__global__ __launch_bounds__(kStreamWaves * 64) void stream_read_kernel(const uint8_t* __restrict__ src,
                                                                        int64_t n_steps, uint32_t* xor_out) {
    constexpr int kSlot = kStreamU * 1024;
    __shared__ __attribute__((aligned(16))) uint8_t smem[kStreamWaves * kSlot];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint8_t* slot = smem + wave * kSlot;
    const uint32_t lds = lds_addr(slot);
    constexpr int64_t kStep = int64_t(kStreamWaves) * kSlot;  // bytes per workgroup step
    // Held in a register: the copies' memory clobber would otherwise reload it every step.
    const int64_t stride = gridDim.x;
    for (int64_t st = blockIdx.x; st < n_steps; st += stride) {
        const uint8_t* base = src + st * kStep + int64_t(wave) * kSlot;
#pragma unroll
        for (int u = 0; u < kStreamU; ++u) dma16<NT>(base, uint32_t(u * 1024 + lane * 16), lds + uint32_t(u * 1024));
        wait_vmcnt<0>();
    }
    if (int64_t(blockIdx.x) != (n_steps - 1) % stride) return;
    uint32_t x = 0;
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(slot + u * 1024 + lane * 16);
        x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x ^= uint32_t(__shfl_xor(int(x), m, 64));
    if (lane == 0) atomicXor(xor_out, x);
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, bool non_temporal, uint32_t* xor_out, hipStream_t s) {
    constexpr size_t kStep = size_t(kStreamWaves) * kStreamU * 1024;
    const int64_t n_steps = int64_t(bytes / kStep);
    if (n_steps == 0) return hipSuccess;
    const unsigned grid = unsigned(n_steps < kStreamGrid ? n_steps : kStreamGrid);
    const uint8_t* p = static_cast<const uint8_t*>(src);
    if (non_temporal)
        stream_read_kernel<true><<<grid, kStreamWaves * 64, 0, s>>>(p, n_steps, xor_out);
    else
        stream_read_kernel<false><<<grid, kStreamWaves * 64, 0, s>>>(p, n_steps, xor_out);
    return hipGetLastError();
}

}  // namespace kvq
