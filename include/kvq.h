/*
 * kvq.h -- C ABI of the MI355X (gfx950) sub-byte KV cache library.
 *
 * Quantize new K/V rows into a paged sub-byte cache and run decode attention
 * directly over it, split-K (flash-decoding) style, then merge the partials.
 *
 * Method (web pages, cited by title and section):
 *  - TensorFold issue "qwen27 CUDA: an opt-in 4-bit attention cache (262K on
 *    a 24 GB card)", section "What it is": each (position, KV head) row is
 *    Hadamard-rotated in groups of 32 and stored as 4-bit codes plus an fp16
 *    scale (144 bytes at head_dim 256); a decode round packs the new keys and
 *    values, rotates the queries once, attends over the 4-bit cache in
 *    rotated space in shared 512-key chunks plus each row's tail with an
 *    in-order merge, and rotates the output back once.
 *  - FreeToken pull request "feat(kvcache): add reliable quantized KV cache":
 *    PR description (32 values -> 16 bytes + one fp16 scale; one layout
 *    constant shared by pool, store and attention) and its CLI-plumbing
 *    commit (head_dim must be divisible by the 32-value block; unsupported
 *    pools are refused at configuration time); test-fix commit (scale =
 *    amax/8, codes sign-extended as int32).
 *  - colibri pull request "KV cache quantization: fp8 (KV8) + 4-bit
 *    TurboQuant (KV_TQ) on CPU, CUDA, and Metal": KV8 commit (latent rows
 *    of kv_lora + rope values stored as e4m3 with a per-row f32 amax/448
 *    scale, RNE, saturating at +-448, NaN stored as 0; absorbed attention
 *    where the latent is both key and value) and split-T commit (partial
 *    blocks per (head, split) holding (cl[K], m, z), then a log-sum-exp
 *    merge kernel).
 *
 * Conventions for every entry point:
 *  - Ownership: the caller allocates and owns every buffer (device memory
 *    unless stated).  The library never allocates, frees or synchronizes,
 *    and keeps no mutable global state, so calls are thread-safe -- except
 *    kvq_attend_noalloc, whose partials live in a static per-GPU array.
 *  - Asynchrony: work is enqueued on `stream` (0 = the null stream).  The
 *    returned status covers argument validation, done on the host before any
 *    launch, and the launch itself; a device fault surfaces at the caller's
 *    next synchronization.
 *  - Validation: an invalid argument returns KVQ_ERR_INVALID_ARG (or
 *    KVQ_ERR_UNSUPPORTED for a valid but unimplemented shape) and launches
 *    nothing.  There is no fallback path.
 *  - Determinism: the split partition of a sequence, and the order in which
 *    the kernels combine its keys, depend only on its own length, head_dim and
 *    split_keys, the merge adds the partials in a fixed order that
 *    depends only on the number of splits, and no atomics are used, so outputs
 *    are bit-reproducible and independent of the other sequences in the
 *    batch.
 *  - Device pointers must be 16-byte aligned unless stated otherwise.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KVQ_OK = 0,
    KVQ_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, bad size or pairing */
    KVQ_ERR_UNSUPPORTED = -2,  /* valid request the library does not implement */
    KVQ_ERR_LAUNCH = -3,       /* the HIP runtime rejected a launch */
    KVQ_ERR_TOO_LARGE = -4     /* kvq_attend_noalloc: partials beyond its static scratch */
} kvq_status;

typedef enum {
    KVQ_FMT_Q4_H32 = 1,        /* 4-bit Hadamard-32 groups + fp16 scale, K and V pools */
    KVQ_FMT_FP8_E4M3_ROW = 2,  /* e4m3 latent rows + f32 scales (latent, rope) */
    KVQ_FMT_Q8_H32 = 3,        /* the same skeleton with 8-bit codes */
    KVQ_FMT_Q6_H32 = 4,        /* the same skeleton with 6-bit codes */
    KVQ_FMT_TQ4_LATENT = 5     /* rotated-int4 + Lloyd-Max latent rows + f32 radii (latent, rope) */
} kvq_format;

typedef enum {
    KVQ_DT_F32 = 0,
    KVQ_DT_BF16 = 1,
    KVQ_DT_F16 = 2
} kvq_dtype;

/* A paged cache.  A slot is page * page_size + offset.
 *
 * KVQ_FMT_Q4_H32 (the "What it is" row of the TensorFold issue):
 *   head_dim D, a multiple of 32 (64, 128, 256 or 512); rope_dim = 0.
 *   k_pool and v_pool: [num_pages][num_kv_heads][page_size][row_bytes] bytes,
 *   row_bytes = D/2 + 2*(D/32).  A row is the D/2 code bytes, group after
 *   group (byte k of a group holds element 2k in its low nibble and element
 *   2k+1 in its high nibble, two's complement), then the D/32 fp16 scales,
 *   little-endian.  scale_pool = NULL.
 * KVQ_FMT_Q8_H32, KVQ_FMT_Q6_H32 (FreeToken pull request "feat(kvcache):
 *   add reliable quantized KV cache": the q4_0 layout sits beside q8_0, 1.0625
 *   bytes per element, in one spec; q6_0 divides by 31): the same pools,
 *   rotation and fp16 scale per group, with scale = fp16(amax/127) and codes
 *   in [-128, 127] (8-bit) or fp16(amax/31) and [-32, 31] (6-bit).  A row is
 *   the codes of every group, then the D/32 fp16 scales: 32 bytes per group
 *   (code i in byte i) or 24 bytes per group (16 bytes of low nibbles laid
 *   out as the 4-bit codes, then 8 bytes holding the high two bits of code
 *   4j+i in bits 2i..2i+1 of byte j).  row_bytes = 34*(D/32) or 26*(D/32);
 *   head_dim 64, 128, 256 or 512.  At head_dim 256 the decode runs on matrix
 *   cores; other head sizes run a plain vector kernel.
 * KVQ_FMT_FP8_E4M3_ROW (the KV8 commit of the colibri pull request):
 *   num_kv_heads = 1 (one latent shared by all heads), head_dim = kv_lora +
 *   rope_dim (a multiple of 16; kv_lora a multiple of 64), rope_dim > 0.
 *   k_pool: e4m3 codes [num_pages*page_size][head_dim]; v_pool = NULL;
 *   scale_pool: f32 [num_pages*page_size][2] = {latent scale, rope scale}.
 * KVQ_FMT_TQ4_LATENT (the colibri pull request's Summary, "Why rotated-int4
 *   for the 4-bit tier"): num_kv_heads = 1, head_dim = 576, rope_dim = 64.
 *   Each part (512 latent, 64 rope values) is rotated by a randomized
 *   Hadamard transform (signs from SplitMix64, seeds 0x4C41544E and
 *   0x524F5045), normalized by its radius (Euclidean norm) times sqrt(n),
 *   and coded as the index of the nearest of 16 Lloyd-Max levels of N(0,1).
 *   k_pool: codes [num_pages*page_size][288] (256 latent + 32 rope bytes,
 *   element 2k in the low nibble); v_pool = NULL; scale_pool: f32
 *   [num_pages*page_size][2] = {latent radius, rope radius}; radius 0 marks an
 *   inert (zero) row.  Attention runs in rotated space (the same Summary:
 *   rotate the queries once, the output back once): q for kvq_decode_attn
 *   is the query rotated by kvq_tq_rotate_q, the partials hold the rotated
 *   context, and kvq_merge rotates the merged context back (inverse_rotate
 *   = 1).  The decode runs on matrix cores when the page size is a multiple
 *   of 16 and split_keys at most 2048, else on a plain vector kernel.
 */
typedef struct kvq_cache {
    int32_t format;        /* kvq_format */
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t rope_dim;
    int32_t page_size;     /* tokens per page, >= 1 */
    int32_t num_pages;
    void* k_pool;
    void* v_pool;
    void* scale_pool;
} kvq_cache;

/* ---------------------------------------------------------------- helpers */

/* Human-readable name of a status (static storage). */
const char* kvq_status_string(kvq_status s);

/* Bytes of one stored row: Q4 -> D/2 + 2*D/32 (144 at D = 256, the TensorFold
 * "What it is" figure); FP8 -> head_dim (codes only; scales are separate).
 * Returns 0 for an invalid format or size.  Host only. */
size_t kvq_row_bytes(int32_t format, int32_t head_dim, int32_t rope_dim);

/* Bytes of the pool(s) a cache descriptor needs: k_pool + v_pool (Q4), or
 * codes + scales (FP8).  0 if the descriptor is invalid.  Host only. */
size_t kvq_pool_bytes(const kvq_cache* cache);

/* Number of splits (partials per head) for sequences up to max_seq_len:
 * ceil(max_seq_len / split_keys), at least 1.  0 on invalid input.  Host only. */
int32_t kvq_num_splits(int32_t max_seq_len, int32_t split_keys);

/* ---------------------------------------------------------------- store */

/* Quantize n_tokens new rows into the cache (TensorFold "What it is": pack
 * the window's new keys and values; colibri KV8 commit: the producer
 * quantizes the fresh row).
 *
 * Q4:  k, v: [n_tokens][num_kv_heads][head_dim] of `dtype` (f32, bf16, f16).
 *      Per row and group of 32: fp32 Hadamard butterfly (stages 1,2,4,8,16)
 *      then x fp32(1/sqrt(32)); amax; scale = fp16_rne(amax/8); codes =
 *      clamp(round_half_even(y / scale), -8, 7), all codes 0 when the scale
 *      is 0.  Rows whose scale would overflow fp16 or that hold NaN/Inf are
 *      outside the format's domain; their stored bytes are unspecified.
 * FP8: k: [n_tokens][head_dim] of `dtype`, v = NULL.  Latent part and rope
 *      part are quantized separately: amax (NaN ignored); if amax is 0 or
 *      not finite or 448/amax is not finite, scale 0 and codes 0x00;
 *      otherwise codes = e4m3_rne_saturating(x * (448/amax)) with NaN -> 0x00,
 *      scale = amax/448.
 * slot_mapping: device int64 [n_tokens] (8-byte aligned); a token whose slot
 * is negative or >= num_pages * page_size is skipped (nothing is written for
 * it and no error is reported).  n_tokens = 0 is a no-op. */
kvq_status kvq_store(const kvq_cache* cache, const void* k, const void* v, int32_t dtype,
                     const int64_t* slot_mapping, int32_t n_tokens, hipStream_t stream);

/* ---------------------------------------------------------------- rotate */

/* q_rot = H32 q for every 32-group of every row (TensorFold "What it is":
 * rotate the queries once), H32 the orthonormal Sylvester Hadamard matrix,
 * computed as the fp32 butterfly then x fp32(1/sqrt(32)).
 * q: [n_rows][head_dim] of `dtype`; q_rot: [n_rows][head_dim] f32.  In place
 * (q == q_rot) is allowed for f32.  Q4 only; head_dim % 32 == 0. */
kvq_status kvq_rotate_q(const void* q, int32_t dtype, float* q_rot, int32_t n_rows, int32_t head_dim,
                        hipStream_t stream);

/* ---------------------------------------------------------------- store + rotate */

/* kvq_store of n_tokens rows into a Q4 cache and kvq_rotate_q of n_rows query
 * rows of the cache's head_dim, as one launch (TensorFold "What it is": the
 * step packs the window's new keys and values and rotates the queries once
 * before attending; the two are independent, so a decode step can issue them
 * together and pay for one launch instead of two).
 * Every argument means what it means for kvq_store (kv_dtype for `dtype`)
 * and kvq_rotate_q (q_dtype for `dtype`, head_dim = cache->head_dim); the
 * stored bytes and q_rot are bit-identical to those two calls.  Either count
 * may be 0 (that part is skipped and its pointers are not read).  q_rot must
 * not overlap k, v or the pools; q == q_rot is allowed for f32.
 * Hadamard-32 formats (Q4, Q8, Q6), and TQ4: there k is the latent rows
 * [n_tokens][576] (v = NULL), q f32 [n_rows][576] (q_dtype KVQ_DT_F32) and
 * q_rot kvq_tq_rotate_q's result, bit for bit.  KVQ_ERR_INVALID_ARG for an FP8
 * cache. */
kvq_status kvq_store_rotate_q(const kvq_cache* cache, const void* k, const void* v, int32_t kv_dtype,
                              const int64_t* slot_mapping, int32_t n_tokens, const void* q, int32_t q_dtype,
                              float* q_rot, int32_t n_rows, hipStream_t stream);

/* ---------------------------------------------------------------- decode */

/* Split-K decode attention over the cache, writing one partial per
 * (sequence, query head, split) (colibri split-T commit: (cl[K], m, z)).
 *
 * Split s of sequence b covers positions [s*split_keys, min((s+1)*split_keys,
 * T_b)), T_b = seq_lens[b]; splits at or past the end are written empty
 * (m = -inf, z = 0, acc = 0).  Position j lives at slot
 * page_table[b*max_pages + j/page_size]*page_size + j%page_size.
 * Scores are natural-log units: s_j = sm_scale * <q, k_j>.
 *   m = max_j s_j, z = sum_j exp(s_j - m), acc = sum_j exp(s_j - m) v_j.
 *
 * Q4:  q = q_rot [batch][n_q_heads][head_dim] f32 (already rotated); query
 *      head h reads KV head h / (n_q_heads / num_kv_heads); k_j, v_j are the
 *      dequantized rotated rows (scale * code), acc is in the rotated domain.
 *      Dv = head_dim.
 * TQ4: q = the rotated query (kvq_tq_rotate_q) [batch][n_q_heads][576] f32;
 *      k_j = lev[code] * radius / sqrt(n) per part, in rotated space; the
 *      latent is the value, acc is in rotated space; Dv = 512.
 * FP8: q = [batch][n_q_heads][head_dim] f32 (latent part then rope part);
 *      s_j = sm_scale*(scL_j <qL, dec(Lc_j)> + scR_j <qR, dec(Rc_j)>),
 *      v_j = scL_j dec(Lc_j) (the latent is the value); Dv = head_dim -
 *      rope_dim.  NaN codes (0x7F, 0xFF) read as 0.
 * page_table: device int32 [batch][max_pages]; seq_lens: device int32
 * [batch], each in [0, max_seq_len]; max_seq_len <= max_pages*page_size.
 * split_keys: a positive multiple of 512 (the TensorFold chunk size) for the
 * Hadamard-32 formats, of 32 (the latent kernels' key tile) for FP8 and TQ4 --
 * short splits give a short context more workgroups; at most 16384 splits per
 * sequence.
 * part_acc: [batch][n_q_heads][S][Dv] f32, part_m / part_z: [batch][n_q_heads][S]
 * f32 with S = kvq_num_splits(max_seq_len, split_keys).
 * Requires n_q_heads % num_kv_heads == 0 and a group of at most 16 query
 * heads per KV head (Hadamard-32 formats); Q8 and Q6 run on matrix cores at
 * head_dim 256 and on a plain vector kernel at other head sizes. */
kvq_status kvq_decode_attn(const kvq_cache* cache, const float* q, int32_t n_q_heads, const int32_t* page_table,
                           int32_t max_pages, const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                           float sm_scale, int32_t split_keys, float* part_acc, float* part_m, float* part_z,
                           hipStream_t stream);

/* Split-K decode attention for several query rows of ONE sequence -- drafted
 * rows, or a short prompt chunk, attending the cache they were just stored
 * into (TensorFold "What it is": drafted rows reuse the cache's full chunks and
 * stay bit-identical to decoding the rows one at a time).  Row r attends
 * positions [0, seq_lens[r]) of the sequence whose page-table row is
 * page_table[0 .. max_pages); every other argument, the partials' layout and
 * the merge (kvq_merge with batch = n_rows and the same seq_lens) are those of
 * kvq_decode_attn with batch = n_rows and that page-table row repeated, and
 * the partials are the same bits (the same kernel, the same per-row work).
 * The difference is the schedule: the workgroups of all rows of one split and
 * KV head are dispatched together on one XCD, so the rows after the first
 * read the split's tiles from that XCD's L2 instead of HBM.
 * Hadamard-32 formats (Q4, Q8, Q6) on the matrix-core kernels: head_dim 256
 * (Q4 also 128), page_size a multiple of 16, groups of at most 16 query
 * heads; other shapes or formats give KVQ_ERR_UNSUPPORTED, as does n_rows >
 * 64.  q: [n_rows][n_q_heads][head_dim] f32, rotated (kvq_rotate_q);
 * seq_lens: device int32 [n_rows], each in [0, max_seq_len]. */
kvq_status kvq_decode_attn_rows(const kvq_cache* cache, const float* q, int32_t n_q_heads, const int32_t* page_table,
                                int32_t max_pages, const int32_t* seq_lens, int32_t n_rows, int32_t max_seq_len,
                                float sm_scale, int32_t split_keys, float* part_acc, float* part_m, float* part_z,
                                hipStream_t stream);

/* Attention of a prompt chunk's query rows over their sequence's 4-bit cache
 * (TensorFold "What it is": prompt chunks are packed into the 4-bit cache --
 * kvq_store -- and then attended over the decoded slots, in rotated space),
 * split into the decode's partials: row r attends positions [0, row_lens[r])
 * of the sequence whose page-table row is page_table[0 .. max_pages); for a
 * chunk of n_rows rows starting at position P (stored before the call),
 * row_lens[r] = P + r + 1 (causal within the chunk).  q: [n_rows][n_q_heads]
 * [head_dim] f32, rotated (kvq_rotate_q); row_lens: device int32 [n_rows],
 * each in [0, max_seq_len]; split_keys: a positive multiple of 32 (long
 * splits write fewer partials; short ones give a short context more
 * workgroups); the partials [n_rows][n_q_heads][S][head_dim] and
 * [n_rows][n_q_heads][S] (S = kvq_num_splits(max_seq_len, split_keys)) are
 * those of kvq_decode_attn with batch = n_rows, and kvq_merge(cache, ...,
 * row_lens, n_rows, n_q_heads, max_seq_len, split_keys, 1, out, lse)
 * completes the attention.  Eight rows share every staged key tile, so the
 * work is bound by the matrix cores, not by HBM (kvq_decode_attn_rows serves
 * a few drafted rows with the decode kernels' arithmetic instead).
 * KVQ_FMT_Q4_H32 caches, head_dim 128 or 256, groups of up to 8 query heads,
 * page_size a multiple of 16, n_rows <= 65535; KVQ_ERR_UNSUPPORTED otherwise. */
kvq_status kvq_prefill_attn(const kvq_cache* cache, const float* q, int32_t n_q_heads, const int32_t* page_table,
                            int32_t max_pages, const int32_t* row_lens, int32_t n_rows, int32_t max_seq_len,
                            float sm_scale, int32_t split_keys, float* part_acc, float* part_m, float* part_z,
                            hipStream_t stream);

/* Split decode attention over SELECTED rows of an FP8 latent cache (colibri
 * split-T commit, DSA gather: attend the selected rows, given as absolute
 * positions; a list of 1024 or more entries is split into partials and
 * merged).  Sequence b attends the positions sel[b*max_sel + k] for
 * k < n_sel[b], in list order; an entry outside [0, max_pages*page_size)
 * (e.g. -1 padding a fixed-size list) is absent, and a position listed
 * twice is attended twice.  Split s covers list entries [s*split_keys,
 * min((s+1)*split_keys, n_sel[b])); everything else -- q, the scores, the
 * partials (S = kvq_num_splits(max_sel, split_keys)) -- is as for
 * kvq_decode_attn on an FP8 cache, and kvq_merge(cache, ..., n_sel, batch,
 * n_q_heads, max_sel, split_keys, 0, out, lse) completes the attention.
 * sel: device int32 [batch][max_sel]; n_sel: device int32 [batch], each in
 * [0, max_sel]; split_keys: a positive multiple of 32 (the key tile), at
 * most 2048 -- short lists run faster with short splits, which give more
 * workgroups; the cache's page_size a multiple of 16.  A Q4 cache gives
 * KVQ_ERR_UNSUPPORTED. */
kvq_status kvq_decode_attn_sel(const kvq_cache* cache, const float* q, int32_t n_q_heads, const int32_t* page_table,
                               int32_t max_pages, const int32_t* sel, const int32_t* n_sel, int32_t batch,
                               int32_t max_sel, float sm_scale, int32_t split_keys, float* part_acc, float* part_m,
                               float* part_z, hipStream_t stream);

/* ---------------------------------------------------------------- merge */

/* Log-sum-exp merge of the partials (colibri split-T commit), in a fixed
 * order (TensorFold "What it is": an in-order merge): split s goes to partial
 * sum s mod 4, each partial sum runs over its splits in ascending order, and
 * the four are added in order 0, 1, 2, 3;
 * followed for Q4 by the single inverse rotation (H32 is its own inverse):
 *   M = max_s m_s, Z = sum_s z_s exp(m_s - M),
 *   out = R( sum_s acc_s exp(m_s - M) / Z ),  R = H32 (Q4/Q8/Q6), the inverse
 *   of the latent part's randomized Hadamard transform (TQ4, in the same
 *   launch: one workgroup per row) or identity (FP8),
 *   lse = M + log Z.
 * A sequence with T = 0 gives out = 0 and lse = -inf.  Only the splits that
 * cover [0, T_b) are read.  inverse_rotate must be 1 for the rotated formats
 * (Q4, Q8, Q6, TQ4) and 0 for FP8.
 * seq_lens, max_seq_len and split_keys are those of the decode call that
 * wrote the partials (for kvq_decode_attn_sel: n_sel and max_sel); split_keys
 * is a positive multiple of 32.
 * out: [batch][n_q_heads][Dv] f32; lse: [batch][n_q_heads] f32 or NULL. */
kvq_status kvq_merge(const kvq_cache* cache, const float* part_acc, const float* part_m, const float* part_z,
                     const int32_t* seq_lens, int32_t batch, int32_t n_q_heads, int32_t max_seq_len,
                     int32_t split_keys, int32_t inverse_rotate, float* out, float* lse, hipStream_t stream);

/* ---------------------------------------------------------------- decode + merge */

/* Bytes of the workspace kvq_attend needs for these sizes: the partials
 * [batch][n_q_heads][S][Dv] f32 and two [batch][n_q_heads][S] f32 arrays,
 * each rounded up to 256 bytes (S = kvq_num_splits(max_seq_len, split_keys),
 * Dv as for kvq_decode_attn).  0 on invalid input.  Host only. */
size_t kvq_attend_workspace_bytes(const kvq_cache* cache, int32_t batch, int32_t n_q_heads, int32_t max_seq_len,
                                  int32_t split_keys);

/* The attention of a decode step in one call (TensorFold "What it is": attend
 * over the 4-bit cache in chunks, merge in order, rotate the output back once;
 * colibri split-T commit: partials (cl[K], m, z), then the log-sum-exp merge):
 * kvq_decode_attn with its partials in `workspace`, then kvq_merge of them into
 * out / lse (with the inverse rotation of the rotated formats).  Every argument
 * means what it means for those two calls; out and lse are the same bits as
 * the two calls give.  q is the rotated query for the rotated formats.
 * workspace: device, 256-byte aligned, at least kvq_attend_workspace_bytes()
 * bytes, owned by the caller; its contents on entry do not matter and on
 * return are the partials (layout: part_acc, then part_m, then part_z, each
 * at a 256-byte boundary).  out: [batch][n_q_heads][Dv] f32; lse:
 * [batch][n_q_heads] f32 or NULL.  KVQ_ERR_INVALID_ARG for a workspace that
 * is too small or misaligned. */
kvq_status kvq_attend(const kvq_cache* cache, const float* q, int32_t n_q_heads, const int32_t* page_table,
                      int32_t max_pages, const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, float sm_scale,
                      int32_t split_keys, void* workspace, size_t workspace_bytes, float* out, float* lse,
                      hipStream_t stream);

/* A whole decode step of the 4-bit cache in two launches (TensorFold "What
 * it is": the step packs the new key and value, rotates the query once,
 * attends over the cache in chunks, merges them in order and rotates the
 * output back once): the store and the query rotation run inside the decode
 * launch, then the merge.  Token b's K and V rows (k, v: device
 * [batch][num_kv_heads][head_dim] of kv_dtype) are stored at position
 * T_b - 1 of sequence b, T_b = seq_lens[b], i.e. at slot
 * page_table[b*max_pages + (T_b-1)/page_size]*page_size + (T_b-1)%page_size
 * (a page outside the pool is not stored, as kvq_store skips such a slot;
 * a sequence with T_b = 0 stores nothing); q ([batch][n_q_heads][head_dim]
 * of q_dtype) is the query BEFORE rotation; every other argument means what
 * it means for kvq_attend.  The stored bytes and out / lse are bit-identical
 * to kvq_store_rotate_q (that slot mapping, n_tokens = batch, n_rows =
 * batch * n_q_heads) followed by kvq_attend on the rotated query, and the
 * workspace holds the same partials.  The positions T_b - 1 of different
 * sequences must map to different slots, and none of those slots may be one
 * that another sequence of the batch reads (a page shared below its length).
 * k, v, q, out: 16-byte aligned.
 * FP8 (the KV8 commit of the colibri pull request: one e4m3 latent row per
 * token, no rotation): k is the latent rows [batch][head_dim] of kv_dtype,
 * v is NULL, q is [batch][n_q_heads][head_dim] f32 (q_dtype KVQ_DT_F32) as
 * kvq_attend takes it; the stored bytes and scales and out / lse are
 * bit-identical to kvq_store (that slot mapping) followed by kvq_attend.
 * KVQ_ERR_INVALID_ARG for a non-NULL v or another q_dtype with FP8.
 * KVQ_ERR_UNSUPPORTED outside the kernels that carry the step (formats Q4,
 * Q8 and Q6 at head_dim 256, groups of at most 8 query heads, pages of a
 * multiple of 16 tokens, split_keys at most 8192; FP8 at head_dim 576 with
 * rope_dim 64, pages of a multiple of 16 tokens, split_keys at most 2048;
 * not TQ4): call kvq_store_rotate_q (kvq_store) and kvq_attend instead. */
kvq_status kvq_decode_step(const kvq_cache* cache, const void* k, const void* v, int32_t kv_dtype, const void* q,
                           int32_t q_dtype, int32_t n_q_heads, const int32_t* page_table, int32_t max_pages,
                           const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, float sm_scale,
                           int32_t split_keys, void* workspace, size_t workspace_bytes, float* out, float* lse,
                           hipStream_t stream);

/* kvq_attend for callers that cannot allocate device memory -- code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc:
 * the same work with the partials in a static device array of
 * KVQ_NOALLOC_SCRATCH_BYTES (64 MiB) held on each GPU the library runs on
 * until the process ends, instead of a workspace argument.  The entry point
 * calls no allocating routine; the first call on a device looks the array's
 * address up once (hipGetSymbolAddress).  Every argument, the outputs and
 * their bits are those of kvq_attend.  A request whose partials
 * (kvq_attend_workspace_bytes) exceed the array returns KVQ_ERR_TOO_LARGE
 * before any launch.  All calls on one GPU share its array: calls that
 * overlap in time on one GPU (different streams, or threads) race on it and
 * must be serialized by the caller; calls on one stream are ordered.  The
 * array keeps the last call's partials; nothing in it needs clearing, since
 * every call writes the partials it reads. */
#define KVQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
kvq_status kvq_attend_noalloc(const kvq_cache* cache, const float* q, int32_t n_q_heads, const int32_t* page_table,
                              int32_t max_pages, const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                              float sm_scale, int32_t split_keys, float* out, float* lse, hipStream_t stream);

/* Query rotation of the TQ4 latent format (the colibri pull request's
 * Summary, "Why rotated-int4 for the 4-bit tier": the query is rotated once,
 * with the rotation the rows were stored with): each row's 512 latent values
 * and 64 rope values are rotated by their parts' randomized Hadamard
 * transforms, y = H (s * x) / sqrt(n) (signs s from SplitMix64 with the
 * seeds above, H the Sylvester Hadamard matrix), in fp32 (the butterfly, then
 * x fp32(1/sqrt(n))).
 * q, q_rot: device f32 [n_rows][576], 16-byte aligned; q == q_rot is
 * allowed (in place); other overlap is not. */
kvq_status kvq_tq_rotate_q(const float* q, float* q_rot, int32_t n_rows, hipStream_t stream);

/* ---------------------------------------------------------------- measurement */

/* The HBM read ceiling the decode kernels are measured against (not a step of
 * the method): every 16-byte chunk of src is copied once into LDS with the
 * LDS-DMA load the 4-bit decode kernels use for cache rows, with the
 * non-temporal hint (non_temporal = 1) or the default cache policy (0).  As
 * a checkable result, the XOR of the little-endian 32-bit words of the final
 * 16 KiB block of src is XOR-ed into *xor_out; the caller sets it first,
 * e.g. to 0.
 * src: device, 16-byte aligned; bytes: a positive multiple of 16384;
 * xor_out: device, 4-byte aligned.  Timing is the caller's (events around
 * the call on `stream`). */
kvq_status kvq_stream_read(const void* src, size_t bytes, int32_t non_temporal, uint32_t* xor_out,
                           hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
