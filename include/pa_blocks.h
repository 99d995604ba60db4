/*
 * pa_blocks.h -- host-side block manager of the paged KV cache, and the
 * device block copy its copy-on-writes need (part of libpa.so).
 *
 * What it manages is fixed by two web pages:
 *   - "vLLM 的 PagedAttention：KV cache 为什么要分页" (bhhxx.wiki), §4.1: a
 *     sequence's logical blocks map to physical blocks anywhere in a global
 *     pool through its block table, and blocks are allocated as the sequence
 *     grows; §4.2: sequences with the same prefix (parallel sampling) share
 *     physical blocks, a not-yet-diverged last block included, and a write
 *     into a shared block whose reference count is above one copies it to a
 *     new block first, while a count of one writes in place;
 *   - "KV Cache与PagedAttention内存管理" (aiqz.cc), section 分页机制 and the
 *     prefix-sharing paragraph after it: a pool of fixed-size blocks handed
 *     out on demand and returned on release, shared blocks carrying a
 *     reference count.
 * A token at logical position t of a sequence lives in the flat slot
 * table[t / block_size] * block_size + t % block_size, the slot_mapping
 * convention of reshape_and_cache ("读 vLLM 的 PagedAttention kernel", §3.2).
 *
 * Rules where the pages are silent:
 *   - the free list is a stack: it starts as ids num_blocks-1 .. 0, so the
 *     first allocations return 0, 1, 2, ...; released blocks are pushed in
 *     the order of the releasing table, so the last one is reused first;
 *   - a decode step appends one token to each listed sequence, in list order;
 *     a sequence may appear once per step;
 *   - a token at a position that is a multiple of block_size opens a new
 *     block and never copies;
 *   - an operation that would need more free blocks than there are fails as
 *     a whole (PA_ERR_NO_SPACE) and changes nothing;
 *   - a copy duplicates the whole block, every slot of every KV head.
 *
 * The block manager is plain host memory; none of its calls touch the GPU.
 * A manager is not thread-safe: calls on one manager must not overlap.
 * Different managers are independent.  Integer results: PA_OK or a negative
 * pa_status (pa.h).
 */
#ifndef PA_MI355X_PA_BLOCKS_H
#define PA_MI355X_PA_BLOCKS_H

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/* A manager of num_blocks blocks of block_size tokens (both > 0), all free.
 * Returns NULL on bad sizes or when host memory runs out.  Owned by the
 * caller; release with pa_bm_destroy. */
PA_API pa_block_manager* pa_bm_create(int num_blocks, int block_size);

/* Releases the manager (NULL is ignored). */
PA_API void pa_bm_destroy(pa_block_manager* bm);

/* A new sequence seq_id holding num_tokens >= 0 tokens (its prompt):
 * allocates ceil(num_tokens / block_size) blocks in logical order.  If
 * slots_out is not NULL it receives the slot of every token
 * ([num_tokens] int64, caller-owned).  PA_ERR_INVALID_ARG if seq_id exists
 * or num_tokens < 0; PA_ERR_NO_SPACE if too few blocks are free. */
PA_API int pa_bm_add_sequence(pa_block_manager* bm, int64_t seq_id, int num_tokens,
                              int64_t* slots_out);

/* child starts as a copy of parent's table and length; every block of it
 * gains one reference.  PA_ERR_INVALID_ARG if parent is unknown or child
 * exists. */
PA_API int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child);

/* Drops seq_id; each of its blocks loses one reference and returns to the
 * free list at zero.  PA_ERR_INVALID_ARG if unknown. */
PA_API int pa_bm_free_sequence(pa_block_manager* bm, int64_t seq_id);

/* One decode step: one new token for each of seq_ids[0..num_seqs) in order.
 *   slots_out   [num_seqs] int64: slot of each new token (reshape_and_cache's
 *               slot_mapping)
 *   copies_out  [max_copies][2] int32: (source, destination) block pairs of
 *               the step's copy-on-writes, in order (copy_blocks' input;
 *               apply them before writing the step's tokens); at most
 *               num_seqs pairs are ever needed
 *   num_copies  out: number of pairs written
 * PA_ERR_INVALID_ARG for an unknown or repeated id, or when the step needs
 * more than max_copies pairs; PA_ERR_NO_SPACE if too few blocks are free.
 * On any error nothing changes. */
PA_API int pa_bm_append_slots(pa_block_manager* bm, const int64_t* seq_ids, int num_seqs,
                              int64_t* slots_out, int32_t* copies_out, int max_copies,
                              int* num_copies);

/* Block tables and lengths of a batch, ready for pa_decode_v1/v2:
 *   tables_out   [num_seqs][width] int32: row i = the table of seq_ids[i],
 *                padded with `pad`; PA_ERR_NO_SPACE if a table is wider
 *   seq_lens_out [num_seqs] int32 (may be NULL)
 * PA_ERR_INVALID_ARG for an unknown id. */
PA_API int pa_bm_block_tables(const pa_block_manager* bm, const int64_t* seq_ids, int num_seqs,
                              int32_t* tables_out, int width, int32_t pad,
                              int32_t* seq_lens_out);

/* Introspection: free blocks; live sequences; tokens of seq_id (-1 if
 * unknown); references to block (-1 if out of range). */
PA_API int pa_bm_num_free_blocks(const pa_block_manager* bm);
PA_API int pa_bm_num_sequences(const pa_block_manager* bm);
PA_API int pa_bm_seq_len(const pa_block_manager* bm, int64_t seq_id);
PA_API int pa_bm_refcount(const pa_block_manager* bm, int block);

/*
 * pa_copy_blocks -- the device side of copy-on-write: for each pair i,
 * block block_pairs[2i+1] of both pools becomes a bit-exact copy of block
 * block_pairs[2i] (all KV heads, all slots).  Pairs are independent (a
 * destination must not be another pair's source or destination, which
 * pa_bm_append_slots never produces); a pair naming an id outside
 * [0, num_blocks) is skipped on the device.
 *
 *   k_cache, v_cache  the pools of pa_decode_v1 (device, updated in place),
 *                     of element type kv_cache_dtype (pa.h)
 *   block_pairs       [num_pairs][2] int32 (device; may be NULL when
 *                     num_pairs == 0, which enqueues nothing)
 * Enqueued on `stream`; PA_ERR_* as in pa.h for bad host arguments.
 */
PA_API int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs, int num_pairs,
                          int num_kv_heads, int head_size, int block_size, int num_blocks,
                          int kv_cache_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_MI355X_PA_BLOCKS_H */
