/*
 * pa.h -- C ABI of libpa.so: paged decode attention for AMD Instinct MI355X
 * (CDNA4, gfx950).
 *
 * What it computes is fixed by three web pages on vLLM's PagedAttention:
 *   - "读 vLLM 的 PagedAttention kernel" (inference-learning-path.pages.dev):
 *     §3.1 the paged K/V pool layouts, §3.2 the slot_mapping cache write,
 *     §3.3 the kernel inputs and the v1/v2 PARTITION_SIZE split, §2 and §3.4
 *     the block-table walk with an online-softmax fold;
 *   - "KV Cache与PagedAttention内存管理" (aiqz.cc), section 自回归推理 for
 *     softmax(QK^T/sqrt(d_k))V and section 分页机制 for the page map;
 *   - "vLLM 的 PagedAttention：KV cache 为什么要分页" (bhhxx.wiki), §4.3 for
 *     the per-block kernel loop, §2 for prefill and decode.
 *
 * Conventions shared by every call
 *   - Every pointer argument is a DEVICE pointer into memory the caller owns
 *     (allocated by the caller, e.g. through PyTorch).  The library never
 *     allocates, frees or synchronises; it validates its host-side arguments,
 *     enqueues kernels on `stream` (a hipStream_t; NULL = the null stream) and
 *     returns.  Calls keep no state between them that affects their results
 *     (pa_decode_v2 caches each device's compute-unit count and its kernels'
 *     occupancy, read-only properties, in thread-safe process-wide slots) and
 *     may be made from several host threads.
 *   - Element types: q, key, value, k_cache and v_cache hold IEEE fp16; out,
 *     tmp_out, exp_sums and max_logits hold fp32; block_tables and seq_lens
 *     int32; slot_mapping and cu_seq_lens int64.  All tensors are dense
 *     row-major with the shapes given below, except key/value rows, whose
 *     token stride is an argument.
 *   - block_size must be 16 and head_size 64 or 128 (PA_ERR_UNSUPPORTED
 *     otherwise).  x = 16 bytes / element size: 8 for fp16 pools, 16 for fp8.
 *   - kv_cache_dtype selects the pools' element type (§3.2 of the kernel
 *     page names kv_cache_dtype, k_scale and v_scale but defines no scheme;
 *     the one taken here): PA_KV_FP16, or PA_KV_FP8_E4M3 -- one byte per
 *     element in the OCP FP8 E4M3 format (sign, 4 exponent bits with bias 7,
 *     3 mantissa bits, no infinity, S.1111.111 = NaN, largest finite 448),
 *     with one fp32 scale per pool: the cache write stores
 *     code = E4M3(fp32(x) / k_scale) (nearest, ties to even, finite values
 *     beyond 448 saturated, NaN -> 0x7F) and attention reads K as
 *     code * k_scale and V as code * v_scale.  For fp16 pools the scales are
 *     ignored; for fp8 they must be finite and > 0.  Another dtype value is
 *     PA_ERR_UNSUPPORTED.
 *   - Return value: PA_OK, or a negative pa_status before anything is
 *     enqueued.  PA_ERR_LAUNCH reports a failed launch.  A kernel fault shows
 *     up at the caller's next synchronisation, as HIP does.
 *   - Values the host cannot see (block ids, seq_lens, slots) are checked on
 *     the device so that no bad value turns into an out-of-bounds access:
 *     a sequence whose walk over a partition (v2) or over its whole table
 *     (v1) meets a block id outside [0, num_blocks), or whose length is
 *     longer than its block-table row, gets NaN in that walk's output rows
 *     (every head of the KV group) instead of a read; the cache write skips
 *     slots outside the pool.
 */
#ifndef PA_MI355X_PA_H
#define PA_MI355X_PA_H

#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define PA_API __attribute__((visibility("default")))
#else
#define PA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_kv_dtype {
    PA_KV_FP16 = 0,           /* IEEE binary16 elements                         */
    PA_KV_FP8_E4M3 = 1        /* OCP FP8 E4M3 codes with per-pool fp32 scales   */
} pa_kv_dtype;

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = -1,  /* null pointer, non-positive or inconsistent size */
    PA_ERR_UNSUPPORTED = -2,  /* head_size not 64/128, block_size not 16        */
    PA_ERR_MISALIGNED = -3,   /* a pointer or stride breaks 16-byte alignment    */
    PA_ERR_LAUNCH = -4,       /* the HIP runtime refused a launch               */
    PA_ERR_NO_SPACE = -5,     /* block manager: too few free blocks / output too small */
    PA_ERR_SCRATCH_TOO_SMALL = -6  /* pa_decode_v2_noalloc: partials exceed its fixed scratch */
} pa_status;

/* Version of this ABI (bumped on any signature change). */
PA_API int pa_abi_version(void);

/* Human-readable text for a pa_status value (static storage). */
PA_API const char* pa_status_str(int status);

/*
 * pa_decode_v1 -- unpartitioned paged decode attention.
 *
 * For every sequence s and query head h (KV head kvh = h / (num_heads /
 * num_kv_heads)): walk block_tables[s] in logical order over the
 * ceil(L/16) blocks of L = seq_lens[s] tokens, load each block's K and V from
 * the pools (§3.1), and return
 *     out[s,h,:] = sum_t softmax_t(scale * q[s,h,:] . K_t) V_t
 * computed block by block with an online softmax (running max, normaliser
 * and accumulator, §2 flowchart / §3.3), fp32 accumulation.  With an fp8
 * cache, K_t and V_t are the scaled codes (see kv_cache_dtype above); they
 * are converted to fp16 exactly, and k_scale and v_scale are applied to the
 * logits and to the final normalisation.
 *
 *   out          [num_seqs, num_heads, head_size] fp32, written
 *   q            [num_seqs, num_heads, head_size] fp16
 *   k_cache      [num_blocks, num_kv_heads, head_size/x, 16, x] (x = 8 fp16,
 *                16 fp8)
 *   v_cache      [num_blocks, num_kv_heads, head_size, 16]
 *   block_tables [num_seqs, max_blocks_per_seq] int32: physical block ids;
 *                entries past ceil(L/16) are never read
 *   seq_lens     [num_seqs] int32: L <= 0 gives an all-zero row; slots past L
 *                in the last block are never read (any bits, NaN included)
 *   num_heads must be a multiple of num_kv_heads; scale must be finite and > 0.
 */
PA_API int pa_decode_v1(float* out, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* seq_lens,
                 int num_seqs, int num_heads, int num_kv_heads, int head_size,
                 int block_size, int max_blocks_per_seq, int num_blocks,
                 float scale, int kv_cache_dtype, float k_scale, float v_scale,
                 void* stream);

/* ceil(max_seq_len / partition_size): the number of PARTITION_SIZE token
 * ranges the longest sequence is cut into (kernel page §3.3, the v2 split),
 * i.e. the partition count the v2 scratch is sized for; -1 if an argument is
 * not positive. */
PA_API int pa_v2_max_partitions(int max_seq_len, int partition_size);

/*
 * pa_decode_v2 -- partitioned paged decode attention, first pass (§3.3: a
 * PARTITION_SIZE > 0 cuts a long sequence into partitions computed in
 * parallel and merged afterwards).
 *
 * Partition p of sequence s covers tokens [p*PS, min((p+1)*PS, L)),
 * p < ceil(L/PS).  For each query head h it writes
 *     max_logits[s,p,h] = m_p = max_t z_t          (z_t = scale * q . K_t,
 *                                                   K_t scaled for fp8)
 *     exp_sums[s,p,h]   = l_p = sum_t exp(z_t - m_p)
 *     tmp_out[s,p,h,:]  = sum_t exp(z_t - m_p) V_t / l_p
 * in natural-log units.  Entries with p >= ceil(L/PS) are not written.
 * pa_reduce merges them into the final output.  The partition index comes
 * before the head index so that the query heads of one KV group -- the
 * results of one work unit -- are one contiguous run of whole cache lines:
 * writes scattered through the K/V read stream cost DRAM read/write
 * turnarounds.
 *
 *   tmp_out     [num_seqs, max_num_partitions, num_heads, head_size] fp32 scratch
 *   exp_sums    [num_seqs, max_num_partitions, num_heads] fp32 scratch
 *   max_logits  [num_seqs, max_num_partitions, num_heads] fp32 scratch
 *   other arguments as in pa_decode_v1;
 *   partition_size: a positive multiple of 16;
 *   max_num_partitions: >= ceil(L/PS) for every sequence (a longer sequence
 *   gets NaN partials).
 */
PA_API int pa_decode_v2(float* tmp_out, float* exp_sums, float* max_logits,
                 const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* seq_lens,
                 int num_seqs, int num_heads, int num_kv_heads, int head_size,
                 int block_size, int max_blocks_per_seq, int num_blocks,
                 int max_num_partitions, int partition_size, float scale,
                 int kv_cache_dtype, float k_scale, float v_scale, void* stream);

/*
 * pa_decode_v2_shared -- pa_decode_v2 for batches whose sequences share K/V
 * blocks ("vLLM 的 PagedAttention：KV cache 为什么要分页", §4.2: parallel
 * sampling and beam search point several sequences' block tables at the same
 * physical blocks, and copy-on-write gives each its own copy of a partly
 * filled block it writes).  Same arguments, outputs, validation and error
 * codes as pa_decode_v2, for any batch.
 *
 * With G = num_heads / num_kv_heads in {2, 4, 8} and partition_size <= 1024,
 * aligned sets of 16/G sequences are taken together: the sequences of a set
 * whose token range in a partition and block-table entries over it equal the
 * set's first sequence's (the partition's last entry may differ) are computed
 * in one walk of the shared blocks, split over two waves, each sequence's
 * own last block folded into its own rows; every other sequence alone, with
 * the same two-wave split.  A sequence's results are bit for bit the same
 * whether its blocks are shared or private copies.  Other G or partition
 * sizes: exactly pa_decode_v2.  On batches that share nothing it is correct
 * but slower than pa_decode_v2 when the lengths in a set differ (a set's
 * sequences run one after another in one workgroup).
 */
PA_API int pa_decode_v2_shared(float* tmp_out, float* exp_sums, float* max_logits,
                 const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* seq_lens,
                 int num_seqs, int num_heads, int num_kv_heads, int head_size,
                 int block_size, int max_blocks_per_seq, int num_blocks,
                 int max_num_partitions, int partition_size, float scale,
                 int kv_cache_dtype, float k_scale, float v_scale, void* stream);

/*
 * pa_reduce -- v2 second pass: log-sum-exp merge of the partials (the pages
 * say only "merged afterwards"; this is the exact merge).
 *
 * With n = ceil(L/PS), M = max_{p<n} m_p and w_p = l_p exp(m_p - M):
 *     out[s,h,:] = sum_{p<n} (w_p / sum_q w_q) tmp_out[s,p,h,:]
 * n = 0 gives zeros; n > max_num_partitions gives NaN.
 *
 *   out [num_seqs, num_heads, head_size] fp32, written; the other arrays as
 *   written by pa_decode_v2 with the same num_heads, head_size,
 *   max_num_partitions and partition_size.
 */
PA_API int pa_reduce(float* out, const float* tmp_out, const float* exp_sums,
              const float* max_logits, const int32_t* seq_lens,
              int num_seqs, int num_heads, int head_size,
              int max_num_partitions, int partition_size, void* stream);

/*
 * pa_decode_v2_noalloc -- pa_decode_v2 followed by pa_reduce, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the partials live in a
 * fixed array of PA_NOALLOC_SCRATCH_BYTES inside the library's device code
 * (one per GPU, held until the process ends) instead of caller scratch.
 * The call allocates nothing; the caller passes the inputs and the output.
 *
 *   out  [num_seqs, num_heads, head_size] fp32, written (as pa_reduce)
 *   other arguments as in pa_decode_v2.
 * The partials take S*P*H*D*4 bytes plus 2*S*P*H*4 (P = max_num_partitions,
 * each part rounded up to 256 bytes); more than PA_NOALLOC_SCRATCH_BYTES
 * returns PA_ERR_SCRATCH_TOO_SMALL before anything is enqueued.  The first
 * call on a GPU looks up the device address of that GPU's array.  Every call
 * on a GPU uses the same array, so calls that overlap on one GPU (two
 * streams, two host threads) race; calls in one stream are ordered.
 */
#define PA_NOALLOC_SCRATCH_BYTES (48ull * 1024ull * 1024ull)

PA_API int pa_decode_v2_noalloc(float* out, const void* q, const void* k_cache,
                 const void* v_cache, const int32_t* block_tables, const int32_t* seq_lens,
                 int num_seqs, int num_heads, int num_kv_heads, int head_size,
                 int block_size, int max_blocks_per_seq, int num_blocks,
                 int max_num_partitions, int partition_size, float scale,
                 int kv_cache_dtype, float k_scale, float v_scale, void* stream);

/*
 * pa_prefill -- multi-token queries over the paged cache with a causal mask
 * (prefill, chunked prefill, speculative verify: the phases around decode).
 *
 * Sequence s holds L = seq_lens[s] cached tokens (its K/V already written,
 * the new tokens' included); its last n = query_start_loc[s+1] -
 * query_start_loc[s] tokens have queries, rows query_start_loc[s] + j of q
 * and out.  Query j sits at position p = L - n + j and attends keys 0..p:
 *     out[r,h,:] = sum_{t<=p} softmax_t(scale * q[r,h,:] . K_t) V_t
 * with the same head mapping, dtypes and fp8 scaling as pa_decode_v1.  n = 1
 * is a decode step, n = L a full prefill.
 *
 *   out             [total_q, num_heads, head_size] fp32, written
 *   q               [total_q, num_heads, head_size] fp16
 *   query_start_loc [num_seqs + 1] int32, non-decreasing, starting at 0;
 *                   a sequence whose range [query_start_loc[s],
 *                   query_start_loc[s+1]) runs backwards or leaves
 *                   [0, total_q) is bad: the part of it inside [0, total_q)
 *                   is set to NaN and nothing outside is read or written
 *   total_q         rows of q and out (>= 0; 0 enqueues nothing)
 *   max_query_len   >= every n (sizes the grid; 0 enqueues nothing); rows of a
 *                   sequence beyond the first max_query_len, rounded up to
 *                   the tile of 4 x 32/G query tokens (4 x 2 for G >= 16),
 *                   are set to NaN
 *   other arguments as in pa_decode_v1.  n > L or L beyond the table row
 *   gives NaN rows for that sequence; a block id outside the pool gives NaN
 *   rows for the queries that attend over that block (with the other
 *   queries of their wave's tile of 32/G tokens, 2 for G >= 16).
 */
PA_API int pa_prefill(float* out, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, const int32_t* seq_lens,
               const int32_t* query_start_loc, int num_seqs, int total_q, int num_heads,
               int num_kv_heads, int head_size, int block_size, int max_blocks_per_seq,
               int num_blocks, int max_query_len, float scale, int kv_cache_dtype,
               float k_scale, float v_scale, void* stream);

/*
 * pa_reshape_and_cache -- the pages' reshape_and_cache: scatter new tokens'
 * K and V into the pools through
 * slot_mapping (§3.2: a flat physical slot = block id * block_size + offset
 * in the block; the write is the same indirection as the read, in the other
 * direction).
 *
 * For token i with slot = slot_mapping[i], b = slot / 16, o = slot % 16:
 *     k_cache[b, h, d/x, o, d%x] = key[i, h, d]
 *     v_cache[b, h, d, o]        = value[i, h, d]     for every h, d,
 * a bit-exact copy into fp16 pools, or the E4M3 codes of key / k_scale and
 * value / v_scale into fp8 pools (kv_cache_dtype above).  slot < 0 skips
 * the token (padding); a slot at or past num_blocks*16 is skipped too.  Two
 * tokens with the same slot race.
 *
 *   key, value   [num_tokens, num_kv_heads, head_size] fp16, token stride
 *                key_stride / value_stride elements (a multiple of 8, at
 *                least num_kv_heads*head_size)
 *   k_cache, v_cache  as in pa_decode_v1, updated in place
 *   slot_mapping [num_tokens] int64
 * With num_tokens == 0 nothing is enqueued and key, value and slot_mapping
 * may be NULL.
 */
PA_API int pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                         int head_size, int block_size, int num_blocks,
                         int64_t key_stride, int64_t value_stride,
                         int kv_cache_dtype, float k_scale, float v_scale, void* stream);

/*
 * pa_gather_kv -- the read-side indirection alone: every sequence's K and V
 * copied bit-exactly, in logical token order, to contiguous arrays of the
 * pools' element type (fp16 values or fp8 codes).  It is the cache write of
 * kernel page §3.2 run in the other direction -- logical token t of a
 * sequence is slot t % 16 of physical block block_tables[s][t / 16] (§3.4,
 * the block-table walk; memory page 分页机制, the page map) -- with no
 * attention arithmetic, so a test can check the walk bit for bit.
 *
 *   k_out, v_out [sum_s L_s, num_kv_heads, head_size] elements, written:
 *                token t of sequence s goes to row cu_seq_lens[s] + t
 *   cu_seq_lens  [num_seqs] int64: starting row of each sequence
 *   other arguments as in pa_decode_v1 (kv_cache_dtype: element type only).
 *   A bad block id writes NaN rows.
 */
PA_API int pa_gather_kv(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* seq_lens,
                 const int64_t* cu_seq_lens, int num_seqs, int num_kv_heads,
                 int head_size, int block_size, int max_blocks_per_seq, int num_blocks,
                 int kv_cache_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_MI355X_PA_H */
