// kvq_api.hip -- the C ABI (include/kvq.h): argument validation on the host,
// then kernel launches on the caller's stream.  Nothing here allocates,
// frees or synchronizes.
#include "kvq.h"

#include <mutex>

#include "internal.h"

// kvq_attend_noalloc's workspace (see device_scratch below).
static_assert(KVQ_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte blocks");
static __device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_SCRATCH_BYTES];

namespace {

using kvq::InType;

constexpr uintptr_t kAlign = 16;

constexpr int64_t kMaxLaunchThreads = 0xFFFFFF00LL;  // grid x block of a 1-D launch
constexpr int32_t kMaxDraftRows = 64;                 // rows per kvq_decode_attn_rows call

bool aligned(const void* p, uintptr_t a = kAlign) { return p && (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool q4_dim_ok(int32_t D) { return D == 64 || D == 128 || D == 256 || D == 512; }

// The Hadamard-32 block formats (K and V pools, rows of codes then fp16 scales).
bool is_h32(int32_t format) {
    return format == KVQ_FMT_Q4_H32 || format == KVQ_FMT_Q8_H32 || format == KVQ_FMT_Q6_H32;
}
int h32_bits(int32_t format) { return format == KVQ_FMT_Q8_H32 ? 8 : (format == KVQ_FMT_Q6_H32 ? 6 : 4); }

// Validates a descriptor; returns KVQ_OK or the status to report.
kvq_status check_cache(const kvq_cache* c) {
    if (!c) return KVQ_ERR_INVALID_ARG;
    if (c->page_size < 1 || c->num_pages < 1 || c->num_kv_heads < 1 || c->head_dim < 1) return KVQ_ERR_INVALID_ARG;
    if (int64_t(c->num_pages) * c->page_size > INT32_MAX) return KVQ_ERR_UNSUPPORTED;
    if (is_h32(c->format)) {
        if (c->head_dim % 32 || c->rope_dim != 0) return KVQ_ERR_INVALID_ARG;
        if (!q4_dim_ok(c->head_dim)) return KVQ_ERR_UNSUPPORTED;
        if (!aligned(c->k_pool) || !aligned(c->v_pool) || c->scale_pool) return KVQ_ERR_INVALID_ARG;
        return KVQ_OK;
    }
    if (c->format == KVQ_FMT_TQ4_LATENT) {
        if (c->num_kv_heads != 1 || c->head_dim != 576 || c->rope_dim != 64) return KVQ_ERR_INVALID_ARG;
        if (!aligned(c->k_pool) || c->v_pool || !aligned(c->scale_pool)) return KVQ_ERR_INVALID_ARG;
        return KVQ_OK;
    }
    if (c->format == KVQ_FMT_FP8_E4M3_ROW) {
        if (c->num_kv_heads != 1 || c->rope_dim <= 0 || c->rope_dim >= c->head_dim) return KVQ_ERR_INVALID_ARG;
        if (c->head_dim % 16 || (c->head_dim - c->rope_dim) % 64) return KVQ_ERR_INVALID_ARG;
        if (c->head_dim - c->rope_dim != 512 || c->rope_dim != 64) return KVQ_ERR_UNSUPPORTED;
        if (!aligned(c->k_pool) || c->v_pool || !aligned(c->scale_pool)) return KVQ_ERR_INVALID_ARG;
        return KVQ_OK;
    }
    return KVQ_ERR_INVALID_ARG;
}

bool dtype_ok(int32_t dt) { return dt == KVQ_DT_F32 || dt == KVQ_DT_BF16 || dt == KVQ_DT_F16; }

kvq::Q4Pool q4_pool(const kvq_cache* c) {
    return kvq::Q4Pool{static_cast<uint8_t*>(c->k_pool), static_cast<uint8_t*>(c->v_pool), c->num_kv_heads,
                       c->head_dim, c->page_size, c->num_pages, h32_bits(c->format)};
}

kvq::Fp8Pool fp8_pool(const kvq_cache* c) {
    return kvq::Fp8Pool{static_cast<uint8_t*>(c->k_pool), static_cast<float*>(c->scale_pool), c->head_dim,
                        c->rope_dim, c->page_size, c->num_pages};
}

kvq_status launched(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH; }

// Shared checks of kvq_decode_attn / kvq_decode_attn_sel / kvq_merge arguments; split_keys must be a
// positive multiple of split_unit (512 for decode over positions, 32 for selections and the merge).
kvq_status check_seq_args(const kvq_cache* c, int32_t n_q_heads, const int32_t* seq_lens, int32_t batch,
                          int32_t max_seq_len, int32_t split_keys, int32_t split_unit) {
    if (n_q_heads < 1 || batch < 0 || max_seq_len < 0 || split_keys < split_unit || split_keys % split_unit)
        return KVQ_ERR_INVALID_ARG;
    if (n_q_heads % c->num_kv_heads) return KVQ_ERR_INVALID_ARG;
    if (batch > 0 && !aligned(seq_lens, 4)) return KVQ_ERR_INVALID_ARG;
    if (batch > 65535) return KVQ_ERR_UNSUPPORTED;
    if (is_h32(c->format) && n_q_heads / c->num_kv_heads > 16) return KVQ_ERR_UNSUPPORTED;
    if (kvq_num_splits(max_seq_len, split_keys) > 16384) return KVQ_ERR_UNSUPPORTED;  // merge keeps one weight per split in LDS
    return KVQ_OK;
}

// The decode kernel kvq_decode_attn runs for these (validated) arguments.
kvq_status launch_decode_for(const kvq_cache* cache, const kvq::DecodeArgs& a, hipStream_t stream) {
    if (is_h32(cache->format)) {
        const kvq::Q4Pool pool = q4_pool(cache);
        if (pool.bits == 4 && kvq::decode_q4_pair_supported(pool, a))
            return launched(kvq::launch_decode_q4_pair(pool, a, stream));
        if (kvq::decode_q4_mfma_supported(pool, a)) return launched(kvq::launch_decode_q4_mfma(pool, a, stream));
        return launched(kvq::launch_decode_q4_simple(pool, a, stream));
    }
    const kvq::Fp8Pool pool = fp8_pool(cache);
    if (cache->format == KVQ_FMT_TQ4_LATENT) {
        if (kvq::decode_fp8_mfma_supported(pool, a)) return launched(kvq::launch_decode_tq4_mfma(pool, a, stream));
        return launched(kvq::launch_decode_tq4_simple(pool, a, stream));
    }
    if (kvq::decode_fp8_mfma_supported(pool, a)) return launched(kvq::launch_decode_fp8_mfma(pool, a, stream));
    return launched(kvq::launch_decode_fp8_simple(pool, a, stream));
}

// Checks shared by kvq_decode_attn and kvq_attend, after check_cache.
kvq_status check_decode_args(const kvq_cache* cache, int32_t n_q_heads, int32_t max_pages, const int32_t* seq_lens,
                             int32_t batch, int32_t max_seq_len, float sm_scale, int32_t split_keys) {
    // Hadamard-32 formats split at the 512-key chunk; the latent formats at any 32-key tile
    kvq_status st = check_seq_args(cache, n_q_heads, seq_lens, batch, max_seq_len, split_keys,
                                   is_h32(cache->format) ? 512 : 32);
    if (st != KVQ_OK) return st;
    if (max_pages < 1 || int64_t(max_seq_len) > int64_t(max_pages) * cache->page_size) return KVQ_ERR_INVALID_ARG;
    if (!(sm_scale == sm_scale) || sm_scale == INFINITY || sm_scale == -INFINITY) return KVQ_ERR_INVALID_ARG;
    return KVQ_OK;
}

// Output channels of a cache's attention (the merge's Dv).
int32_t value_dim(const kvq_cache* c) { return is_h32(c->format) ? c->head_dim : c->head_dim - c->rope_dim; }

// The merge (and, for TQ4, the inverse rotation in the same launch) of validated arguments.
kvq_status launch_merge_for(const kvq_cache* cache, const kvq::MergeArgs& a, hipStream_t stream) {
    if (cache->format == KVQ_FMT_TQ4_LATENT) return launched(kvq::launch_merge_tq(a, stream));
    return launched(kvq::launch_merge(a, stream));
}

// Partials of kvq_attend inside its workspace: part_acc [B][H_q][S][Dv], then
// part_m and part_z [B][H_q][S], all f32, each starting on a 256-byte boundary.
struct AttendLayout {
    size_t acc, m, z, total;
};
AttendLayout attend_layout(int64_t batch, int64_t n_q_heads, int64_t S, int64_t dv) {
    auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
    AttendLayout l{};
    const size_t n_mz = size_t(batch) * size_t(n_q_heads) * size_t(S);
    l.acc = 0;
    l.m = up(n_mz * size_t(dv) * sizeof(float));
    l.z = l.m + up(n_mz * sizeof(float));
    l.total = l.z + up(n_mz * sizeof(float));
    return l;
}

// kvq_attend's work on a validated workspace of at least attend_layout().total bytes.
kvq_status attend_on(const kvq_cache* cache, const float* q, int32_t n_q_heads, const int32_t* page_table,
                     int32_t max_pages, const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, float sm_scale,
                     int32_t split_keys, uint8_t* ws, float* out, float* lse, hipStream_t stream) {
    const int32_t S = kvq_num_splits(max_seq_len, split_keys);
    const AttendLayout l = attend_layout(batch, n_q_heads, S, value_dim(cache));
    float* pa = reinterpret_cast<float*>(ws + l.acc);
    float* pm = reinterpret_cast<float*>(ws + l.m);
    float* pz = reinterpret_cast<float*>(ws + l.z);
    const kvq::DecodeArgs d{q, n_q_heads, page_table, max_pages, seq_lens, batch, max_seq_len, S, sm_scale,
                            split_keys, pa, pm, pz};
    kvq_status st = launch_decode_for(cache, d, stream);
    if (st != KVQ_OK) return st;
    const kvq::MergeArgs m{pa, pm, pz, seq_lens, batch, n_q_heads, max_seq_len, S, split_keys, value_dim(cache),
                           is_h32(cache->format), out, lse};
    return launch_merge_for(cache, m, stream);
}

// Argument checks of kvq_attend (and its variants) before the workspace.
kvq_status check_attend_args(const kvq_cache* cache, const float* q, int32_t n_q_heads, const int32_t* page_table,
                             int32_t max_pages, const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                             float sm_scale, int32_t split_keys, const float* out, const float* lse) {
    kvq_status st = check_cache(cache);
    if (st != KVQ_OK) return st;
    st = check_decode_args(cache, n_q_heads, max_pages, seq_lens, batch, max_seq_len, sm_scale, split_keys);
    if (st != KVQ_OK) return st;
    if (batch == 0) return KVQ_OK;
    if (!aligned(q) || !aligned(page_table, 4) || !aligned(out) || (lse && !aligned(lse, 4)))
        return KVQ_ERR_INVALID_ARG;
    if (int64_t(batch) * n_q_heads > INT32_MAX) return KVQ_ERR_UNSUPPORTED;
    return KVQ_OK;
}

// ------------------------------------------------------------ static scratch
// kvq_attend_noalloc's workspace: a file-scope device array, one copy per GPU
// the library runs on, held until the process ends.  In host code `scratch`
// is only a host-side stand-in for the symbol; the device address of each
// GPU's copy comes from hipGetSymbolAddress, taken once per device (with that
// device current) on the entry point's first call there, and only that
// address is ever passed to a kernel.
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
uint8_t* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The current device's copy of the scratch array (nullptr if the runtime cannot give it).
uint8_t* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? static_cast<uint8_t*>(p) : nullptr;
    });
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* kvq_status_string(kvq_status s) {
    switch (s) {
        case KVQ_OK: return "ok";
        case KVQ_ERR_INVALID_ARG: return "invalid argument";
        case KVQ_ERR_UNSUPPORTED: return "unsupported shape or format";
        case KVQ_ERR_LAUNCH: return "kernel launch failed";
        case KVQ_ERR_TOO_LARGE: return "request exceeds the static scratch of kvq_attend_noalloc";
    }
    return "unknown status";
}

size_t kvq_row_bytes(int32_t format, int32_t head_dim, int32_t rope_dim) {
    if (is_h32(format)) {
        if (head_dim <= 0 || head_dim % 32 || rope_dim != 0) return 0;
        return size_t(kvq::blk_row_bytes(h32_bits(format), head_dim));
    }
    if (format == KVQ_FMT_FP8_E4M3_ROW) {
        if (head_dim <= 0 || rope_dim <= 0 || rope_dim >= head_dim) return 0;
        return size_t(head_dim);
    }
    if (format == KVQ_FMT_TQ4_LATENT) return head_dim == 576 && rope_dim == 64 ? 288 : 0;
    return 0;
}

size_t kvq_pool_bytes(const kvq_cache* c) {
    if (!c || c->page_size < 1 || c->num_pages < 1 || c->num_kv_heads < 1) return 0;
    const size_t rb = kvq_row_bytes(c->format, c->head_dim, c->rope_dim);
    if (!rb) return 0;
    const size_t slots = size_t(c->num_pages) * size_t(c->page_size);
    if (is_h32(c->format)) return 2 * slots * size_t(c->num_kv_heads) * rb;
    return slots * (rb + 2 * sizeof(float));
}

int32_t kvq_num_splits(int32_t max_seq_len, int32_t split_keys) {
    if (max_seq_len < 0 || split_keys <= 0) return 0;
    const int32_t n = int32_t((int64_t(max_seq_len) + split_keys - 1) / split_keys);
    return n < 1 ? 1 : n;
}

kvq_status kvq_store(const kvq_cache* cache, const void* k, const void* v, int32_t dtype,
                     const int64_t* slot_mapping, int32_t n_tokens, hipStream_t stream) {
    kvq_status st = check_cache(cache);
    if (st != KVQ_OK) return st;
    if (!dtype_ok(dtype) || n_tokens < 0) return KVQ_ERR_INVALID_ARG;
    if (n_tokens == 0) return KVQ_OK;
    if (!aligned(slot_mapping, 8)) return KVQ_ERR_INVALID_ARG;
    const InType dt = static_cast<InType>(dtype);
    if (is_h32(cache->format)) {
        if (!aligned(k) || !aligned(v)) return KVQ_ERR_INVALID_ARG;
        // one lane per 4 values: the launch must stay under 2^32 threads
        if (int64_t(n_tokens) * cache->num_kv_heads * 2 * (cache->head_dim / 4) > kMaxLaunchThreads)
            return KVQ_ERR_UNSUPPORTED;
        return launched(kvq::launch_store_q4(q4_pool(cache), k, v, dt, slot_mapping, n_tokens, stream));
    }
    if (!aligned(k) || v) return KVQ_ERR_INVALID_ARG;
    if (cache->format == KVQ_FMT_TQ4_LATENT)
        return launched(kvq::launch_store_tq4(fp8_pool(cache), k, dt, slot_mapping, n_tokens, stream));
    return launched(kvq::launch_store_fp8(fp8_pool(cache), k, dt, slot_mapping, n_tokens, stream));
}

kvq_status kvq_rotate_q(const void* q, int32_t dtype, float* q_rot, int32_t n_rows, int32_t head_dim,
                        hipStream_t stream) {
    if (!dtype_ok(dtype) || n_rows < 0 || head_dim <= 0 || head_dim % 32) return KVQ_ERR_INVALID_ARG;
    if (n_rows == 0) return KVQ_OK;
    if (!aligned(q) || !aligned(q_rot)) return KVQ_ERR_INVALID_ARG;
    if (q == q_rot && dtype != KVQ_DT_F32) return KVQ_ERR_INVALID_ARG;
    if (int64_t(n_rows) * (head_dim / 4) > kMaxLaunchThreads) return KVQ_ERR_UNSUPPORTED;
    return launched(kvq::launch_rotate_q(q, static_cast<InType>(dtype), q_rot, n_rows, head_dim, stream));
}

kvq_status kvq_store_rotate_q(const kvq_cache* cache, const void* k, const void* v, int32_t kv_dtype,
                              const int64_t* slot_mapping, int32_t n_tokens, const void* q, int32_t q_dtype,
                              float* q_rot, int32_t n_rows, hipStream_t stream) {
    kvq_status st = check_cache(cache);
    if (st != KVQ_OK) return st;
    if (cache->format == KVQ_FMT_TQ4_LATENT) {  // latent rows + f32 query rows of 576
        if (!dtype_ok(kv_dtype) || q_dtype != KVQ_DT_F32 || n_tokens < 0 || n_rows < 0 || v) return KVQ_ERR_INVALID_ARG;
        if (n_tokens > 0 && (!aligned(slot_mapping, 8) || !aligned(k))) return KVQ_ERR_INVALID_ARG;
        if (n_rows > 0 && (!aligned(q) || !aligned(q_rot))) return KVQ_ERR_INVALID_ARG;
        if (n_tokens == 0 && n_rows == 0) return KVQ_OK;
        if (int64_t(n_tokens) + n_rows > INT32_MAX) return KVQ_ERR_UNSUPPORTED;
        return launched(kvq::launch_store_rotate_tq4(fp8_pool(cache), k, static_cast<InType>(kv_dtype), slot_mapping,
                                                     n_tokens, static_cast<const float*>(q), q_rot, n_rows, stream));
    }
    if (!is_h32(cache->format)) return KVQ_ERR_INVALID_ARG;
    if (!dtype_ok(kv_dtype) || !dtype_ok(q_dtype) || n_tokens < 0 || n_rows < 0) return KVQ_ERR_INVALID_ARG;
    if (n_tokens > 0 && (!aligned(slot_mapping, 8) || !aligned(k) || !aligned(v))) return KVQ_ERR_INVALID_ARG;
    if (n_rows > 0) {
        if (!aligned(q) || !aligned(q_rot)) return KVQ_ERR_INVALID_ARG;
        if (q == q_rot && q_dtype != KVQ_DT_F32) return KVQ_ERR_INVALID_ARG;
    }
    if (n_tokens == 0 && n_rows == 0) return KVQ_OK;
    // one lane per 4 values in each role, each role rounded up to whole 256-lane workgroups
    const int64_t quads = cache->head_dim / 4;
    const int64_t store_lanes = (int64_t(n_tokens) * cache->num_kv_heads * 2 * quads + 255) / 256 * 256;
    const int64_t rot_lanes = (int64_t(n_rows) * quads + 255) / 256 * 256;
    if (store_lanes + rot_lanes > kMaxLaunchThreads) return KVQ_ERR_UNSUPPORTED;
    return launched(kvq::launch_store_rotate_q4(q4_pool(cache), k, v, static_cast<InType>(kv_dtype), slot_mapping,
                                                n_tokens, q, static_cast<InType>(q_dtype), q_rot, n_rows, stream));
}

kvq_status kvq_decode_attn(const kvq_cache* cache, const float* q, int32_t n_q_heads, const int32_t* page_table,
                           int32_t max_pages, const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                           float sm_scale, int32_t split_keys, float* part_acc, float* part_m, float* part_z,
                           hipStream_t stream) {
    kvq_status st = check_cache(cache);
    if (st != KVQ_OK) return st;
    st = check_decode_args(cache, n_q_heads, max_pages, seq_lens, batch, max_seq_len, sm_scale, split_keys);
    if (st != KVQ_OK) return st;
    if (batch == 0) return KVQ_OK;
    if (!aligned(q) || !aligned(page_table, 4) || !aligned(part_acc) || !aligned(part_m, 4) || !aligned(part_z, 4))
        return KVQ_ERR_INVALID_ARG;
    const kvq::DecodeArgs a{q, n_q_heads, page_table, max_pages, seq_lens, batch, max_seq_len,
                            kvq_num_splits(max_seq_len, split_keys), sm_scale, split_keys, part_acc, part_m, part_z};
    return launch_decode_for(cache, a, stream);
}

kvq_status kvq_decode_attn_rows(const kvq_cache* cache, const float* q, int32_t n_q_heads, const int32_t* page_table,
                                int32_t max_pages, const int32_t* seq_lens, int32_t n_rows, int32_t max_seq_len,
                                float sm_scale, int32_t split_keys, float* part_acc, float* part_m, float* part_z,
                                hipStream_t stream) {
    kvq_status st = check_cache(cache);
    if (st != KVQ_OK) return st;
    if (!is_h32(cache->format)) return KVQ_ERR_UNSUPPORTED;
    st = check_seq_args(cache, n_q_heads, seq_lens, n_rows, max_seq_len, split_keys, 512);
    if (st != KVQ_OK) return st;
    if (max_pages < 1 || int64_t(max_seq_len) > int64_t(max_pages) * cache->page_size) return KVQ_ERR_INVALID_ARG;
    if (!(sm_scale == sm_scale) || sm_scale == INFINITY || sm_scale == -INFINITY) return KVQ_ERR_INVALID_ARG;
    if (n_rows > kMaxDraftRows) return KVQ_ERR_UNSUPPORTED;
    if (n_rows == 0) return KVQ_OK;
    if (!aligned(q) || !aligned(page_table, 4) || !aligned(part_acc) || !aligned(part_m, 4) || !aligned(part_z, 4))
        return KVQ_ERR_INVALID_ARG;
    kvq::DecodeArgs a{q, n_q_heads, page_table, max_pages, seq_lens, n_rows, max_seq_len,
                      kvq_num_splits(max_seq_len, split_keys), sm_scale, split_keys, part_acc, part_m, part_z};
    a.rows = n_rows;
    // the row layout is one 1-D grid of workgroups of at most 512 threads
    const int64_t n_sg = int64_t(a.n_splits) * cache->num_kv_heads;
    if (8 * int64_t(n_rows) * ((n_sg + 7) / 8) * 512 > kMaxLaunchThreads) return KVQ_ERR_UNSUPPORTED;
    // the kernel kvq_decode_attn would choose for the same rows, so the partials are the same bits
    const kvq::Q4Pool pool = q4_pool(cache);
    if (pool.bits == 4 && kvq::decode_q4_pair_supported(pool, a)) return launched(kvq::launch_decode_q4_pair(pool, a, stream));
    if (kvq::decode_q4_mfma_supported(pool, a)) return launched(kvq::launch_decode_q4_mfma(pool, a, stream));
    return KVQ_ERR_UNSUPPORTED;
}

kvq_status kvq_prefill_attn(const kvq_cache* cache, const float* q, int32_t n_q_heads, const int32_t* page_table,
                            int32_t max_pages, const int32_t* row_lens, int32_t n_rows, int32_t max_seq_len,
                            float sm_scale, int32_t split_keys, float* part_acc, float* part_m, float* part_z,
                            hipStream_t stream) {
    kvq_status st = check_cache(cache);
    if (st != KVQ_OK) return st;
    if (cache->format != KVQ_FMT_Q4_H32) return KVQ_ERR_UNSUPPORTED;
    st = check_seq_args(cache, n_q_heads, row_lens, n_rows, max_seq_len, split_keys, 32);
    if (st != KVQ_OK) return st;
    if (max_pages < 1 || int64_t(max_seq_len) > int64_t(max_pages) * cache->page_size) return KVQ_ERR_INVALID_ARG;
    if (!(sm_scale == sm_scale) || sm_scale == INFINITY || sm_scale == -INFINITY) return KVQ_ERR_INVALID_ARG;
    if (n_rows == 0) return KVQ_OK;
    if (!aligned(q) || !aligned(page_table, 4) || !aligned(part_acc) || !aligned(part_m, 4) || !aligned(part_z, 4))
        return KVQ_ERR_INVALID_ARG;
    const kvq::DecodeArgs a{q, n_q_heads, page_table, max_pages, row_lens, n_rows, max_seq_len,
                            kvq_num_splits(max_seq_len, split_keys), sm_scale, split_keys, part_acc, part_m, part_z};
    const kvq::Q4Pool pool = q4_pool(cache);
    if (!kvq::decode_q4_chunk_supported(pool, a)) return KVQ_ERR_UNSUPPORTED;
    return launched(kvq::launch_decode_q4_chunk(pool, a, stream));
}

kvq_status kvq_decode_attn_sel(const kvq_cache* cache, const float* q, int32_t n_q_heads, const int32_t* page_table,
                               int32_t max_pages, const int32_t* sel, const int32_t* n_sel, int32_t batch,
                               int32_t max_sel, float sm_scale, int32_t split_keys, float* part_acc, float* part_m,
                               float* part_z, hipStream_t stream) {
    kvq_status st = check_cache(cache);
    if (st != KVQ_OK) return st;
    if (cache->format != KVQ_FMT_FP8_E4M3_ROW) return KVQ_ERR_UNSUPPORTED;
    st = check_seq_args(cache, n_q_heads, n_sel, batch, max_sel, split_keys, 32);
    if (st != KVQ_OK) return st;
    if (max_pages < 1) return KVQ_ERR_INVALID_ARG;
    if (!(sm_scale == sm_scale) || sm_scale == INFINITY || sm_scale == -INFINITY) return KVQ_ERR_INVALID_ARG;
    if (batch == 0) return KVQ_OK;
    if (!aligned(q) || !aligned(page_table, 4) || !aligned(sel, 4) || !aligned(part_acc) || !aligned(part_m, 4) ||
        !aligned(part_z, 4))
        return KVQ_ERR_INVALID_ARG;
    kvq::DecodeArgs a{q, n_q_heads, page_table, max_pages, n_sel, batch, max_sel,
                      kvq_num_splits(max_sel, split_keys), sm_scale, split_keys, part_acc, part_m, part_z,
                      sel, max_sel};
    const kvq::Fp8Pool pool = fp8_pool(cache);
    if (!kvq::decode_fp8_mfma_supported(pool, a)) return KVQ_ERR_UNSUPPORTED;
    return launched(kvq::launch_decode_fp8_mfma(pool, a, stream));
}

kvq_status kvq_merge(const kvq_cache* cache, const float* part_acc, const float* part_m, const float* part_z,
                     const int32_t* seq_lens, int32_t batch, int32_t n_q_heads, int32_t max_seq_len,
                     int32_t split_keys, int32_t inverse_rotate, float* out, float* lse, hipStream_t stream) {
    kvq_status st = check_cache(cache);
    if (st != KVQ_OK) return st;
    st = check_seq_args(cache, n_q_heads, seq_lens, batch, max_seq_len, split_keys, 32);
    if (st != KVQ_OK) return st;
    const bool q4 = is_h32(cache->format);  // Hadamard-32 formats: inverse rotation in the merge, Dv = head_dim
    const bool tq = cache->format == KVQ_FMT_TQ4_LATENT;  // inverse rotation after the merge
    if (inverse_rotate != (q4 || tq ? 1 : 0)) return KVQ_ERR_INVALID_ARG;
    if (batch == 0) return KVQ_OK;
    if (!aligned(part_acc) || !aligned(part_m, 4) || !aligned(part_z, 4) || !aligned(out) ||
        (lse && !aligned(lse, 4)))
        return KVQ_ERR_INVALID_ARG;
    if (int64_t(batch) * n_q_heads > INT32_MAX) return KVQ_ERR_UNSUPPORTED;
    const kvq::MergeArgs a{part_acc, part_m, part_z, seq_lens, batch, n_q_heads, max_seq_len,
                           kvq_num_splits(max_seq_len, split_keys), split_keys, value_dim(cache), q4, out, lse};
    return launch_merge_for(cache, a, stream);
}

size_t kvq_attend_workspace_bytes(const kvq_cache* cache, int32_t batch, int32_t n_q_heads, int32_t max_seq_len,
                                  int32_t split_keys) {
    if (check_cache(cache) != KVQ_OK || batch < 0 || n_q_heads < 1 || max_seq_len < 0 || split_keys < 1) return 0;
    return attend_layout(batch, n_q_heads, kvq_num_splits(max_seq_len, split_keys), value_dim(cache)).total;
}

kvq_status kvq_attend(const kvq_cache* cache, const float* q, int32_t n_q_heads, const int32_t* page_table,
                      int32_t max_pages, const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, float sm_scale,
                      int32_t split_keys, void* workspace, size_t workspace_bytes, float* out, float* lse,
                      hipStream_t stream) {
    kvq_status st = check_attend_args(cache, q, n_q_heads, page_table, max_pages, seq_lens, batch, max_seq_len,
                                      sm_scale, split_keys, out, lse);
    if (st != KVQ_OK || batch == 0) return st;
    const size_t need =
        attend_layout(batch, n_q_heads, kvq_num_splits(max_seq_len, split_keys), value_dim(cache)).total;
    if (!aligned(workspace, 256) || workspace_bytes < need) return KVQ_ERR_INVALID_ARG;
    return attend_on(cache, q, n_q_heads, page_table, max_pages, seq_lens, batch, max_seq_len, sm_scale, split_keys,
                     static_cast<uint8_t*>(workspace), out, lse, stream);
}

kvq_status kvq_decode_step(const kvq_cache* cache, const void* k, const void* v, int32_t kv_dtype, const void* q,
                           int32_t q_dtype, int32_t n_q_heads, const int32_t* page_table, int32_t max_pages,
                           const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, float sm_scale,
                           int32_t split_keys, void* workspace, size_t workspace_bytes, float* out, float* lse,
                           hipStream_t stream) {
    kvq_status st = check_cache(cache);
    if (st != KVQ_OK) return st;
    st = check_decode_args(cache, n_q_heads, max_pages, seq_lens, batch, max_seq_len, sm_scale, split_keys);
    if (st != KVQ_OK) return st;
    if (!dtype_ok(kv_dtype) || !dtype_ok(q_dtype)) return KVQ_ERR_INVALID_ARG;
    const bool latent = cache->format == KVQ_FMT_FP8_E4M3_ROW;  // one latent row a token, the f32 query as is
    if (!latent && !is_h32(cache->format)) return KVQ_ERR_UNSUPPORTED;  // TQ4: no step form
    if (latent && (v || q_dtype != KVQ_DT_F32)) return KVQ_ERR_INVALID_ARG;
    if (batch == 0) return KVQ_OK;
    if (!aligned(k) || (!latent && !aligned(v)) || !aligned(q) || !aligned(page_table, 4) || !aligned(out) ||
        (lse && !aligned(lse, 4)))
        return KVQ_ERR_INVALID_ARG;
    if (int64_t(batch) * n_q_heads > INT32_MAX) return KVQ_ERR_UNSUPPORTED;
    const int32_t S = kvq_num_splits(max_seq_len, split_keys);
    const AttendLayout l = attend_layout(batch, n_q_heads, S, value_dim(cache));
    if (!aligned(workspace, 256) || workspace_bytes < l.total) return KVQ_ERR_INVALID_ARG;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    float* pa = reinterpret_cast<float*>(ws + l.acc);
    float* pm = reinterpret_cast<float*>(ws + l.m);
    float* pz = reinterpret_cast<float*>(ws + l.z);
    kvq::DecodeArgs d{nullptr, n_q_heads, page_table, max_pages, seq_lens, batch, max_seq_len, S, sm_scale,
                      split_keys, pa, pm, pz};
    d.step_k = k;
    d.step_v = v;
    d.step_q = q;
    d.step_kv_dt = static_cast<InType>(kv_dtype);
    d.step_q_dt = static_cast<InType>(q_dtype);
    // The kernel kvq_decode_attn would run (launch_decode_for), in its STEP form.
    if (latent) {
        d.q = static_cast<const float*>(q);
        const kvq::Fp8Pool pool = fp8_pool(cache);
        if (!kvq::decode_fp8_mfma_supported(pool, d)) return KVQ_ERR_UNSUPPORTED;
        st = launched(kvq::launch_decode_fp8_mfma(pool, d, stream));
    } else {
        const kvq::Q4Pool pool = q4_pool(cache);
        if (pool.bits == 4 && kvq::decode_q4_pair_supported(pool, d))
            st = launched(kvq::launch_decode_q4_pair(pool, d, stream));
        else if (kvq::decode_q4_mfma_step_supported(pool, d))
            st = launched(kvq::launch_decode_q4_mfma(pool, d, stream));
        else return KVQ_ERR_UNSUPPORTED;
    }
    if (st != KVQ_OK) return st;
    const kvq::MergeArgs m{pa, pm, pz, seq_lens, batch, n_q_heads, max_seq_len, S, split_keys, value_dim(cache),
                           is_h32(cache->format), out, lse};
    return launch_merge_for(cache, m, stream);
}

kvq_status kvq_attend_noalloc(const kvq_cache* cache, const float* q, int32_t n_q_heads, const int32_t* page_table,
                              int32_t max_pages, const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                              float sm_scale, int32_t split_keys, float* out, float* lse, hipStream_t stream) {
    kvq_status st = check_attend_args(cache, q, n_q_heads, page_table, max_pages, seq_lens, batch, max_seq_len,
                                      sm_scale, split_keys, out, lse);
    if (st != KVQ_OK || batch == 0) return st;
    const size_t need =
        attend_layout(batch, n_q_heads, kvq_num_splits(max_seq_len, split_keys), value_dim(cache)).total;
    if (need > KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ERR_TOO_LARGE;
    uint8_t* ws = device_scratch();
    if (!ws) return KVQ_ERR_LAUNCH;
    // The partials are written in full by the decode before the merge reads
    // them, so what an earlier call left in the array needs no clearing.
    return attend_on(cache, q, n_q_heads, page_table, max_pages, seq_lens, batch, max_seq_len, sm_scale, split_keys,
                     ws, out, lse, stream);
}

kvq_status kvq_tq_rotate_q(const float* q, float* q_rot, int32_t n_rows, hipStream_t stream) {
    if (n_rows < 0) return KVQ_ERR_INVALID_ARG;
    if (n_rows == 0) return KVQ_OK;
    if (!aligned(q) || !aligned(q_rot)) return KVQ_ERR_INVALID_ARG;
    return launched(kvq::launch_tq_rotate(q, q_rot, n_rows, 576, false, stream));
}

kvq_status kvq_stream_read(const void* src, size_t bytes, int32_t non_temporal, uint32_t* xor_out,
                           hipStream_t stream) {
    if (!aligned(src) || !aligned(xor_out, 4) || bytes == 0 || bytes % 16384) return KVQ_ERR_INVALID_ARG;
    if (non_temporal != 0 && non_temporal != 1) return KVQ_ERR_INVALID_ARG;
    return launched(kvq::launch_stream_read(src, bytes, non_temporal == 1, xor_out, stream));
}

}  // extern "C"
