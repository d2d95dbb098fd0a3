/*
 * pa_blocks.h - block management for the paged KV cache: a host-side block
 * manager (C++, in libpa.so) and the device copy that copy-on-write needs.
 *
 * The cache is a pool of fixed-size physical blocks and each sequence's table
 * maps its logical positions to blocks. Blocks are taken only as tokens are
 * generated, so only a sequence's last block has unused slots, and a finished
 * sequence's blocks return to the pool at once (How vLLM gets real throughput
 * on H100s, "PagedAttention borrows from operating systems" and "Continuous
 * batching removes straggler bubbles"; vLLM architecture, memory and
 * benchmarks deep dive, "PagedAttention: a 1960s idea for modern GPUs").
 * Sequences forked from one prompt point at the prompt's blocks; a shared
 * block is duplicated only when a sequence writes into it (copy-on-write:
 * Dissecting vLLM, "PagedAttention: Virtual Memory for KV Cache").
 *
 * Policy, fixed so that results are reproducible:
 *   - the free pool is a stack: initially block 0 is taken first, then 1, 2,
 *     ...; afterwards the most recently freed block is reused first;
 *   - pa_bm_free releases a sequence's blocks from its last logical block to
 *     its first, and a block whose count reaches zero goes onto the stack;
 *   - pa_bm_append of k tokens to a sequence of n tokens takes a new block at
 *     every position p with p % block_size == 0; if n % block_size != 0 and
 *     the last block is shared, that block is first copied to a new block
 *     (the pair is queued for pa_copy_blocks) and the table entry moved to
 *     the copy. An append succeeds whole or changes nothing.
 *
 * Threading: a manager is not thread-safe; one thread (a scheduler) owns it.
 * Status codes are those of pa.h plus PA_ERR_OUT_OF_BLOCKS (the pool lacks
 * the blocks an append needs) and PA_ERR_STATE (unknown sequence, or a
 * sequence id already in use).
 */
#ifndef PA_BLOCKS_H
#define PA_BLOCKS_H

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/* A manager of num_blocks blocks of block_size tokens (any block_size >= 1);
 * a sequence holds at most max_blocks_per_seq blocks. PA_ERR_SHAPE for a
 * non-positive size or num_blocks above 2^31 - 1; *out is NULL on error. */
pa_status_t pa_bm_create(int64_t num_blocks, int32_t block_size,
                         int32_t max_blocks_per_seq, pa_block_manager** out);
void pa_bm_destroy(pa_block_manager* bm);

/* New empty sequence `seq` (any int64 id not in use). */
pa_status_t pa_bm_add(pa_block_manager* bm, int64_t seq);

/* `child` (not in use) gets parent's table and length; every block of it
 * gains one reference. */
pa_status_t pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child);

/* Reserve num_tokens >= 0 positions after seq's last; slots[i] (host array of
 * num_tokens) receives the cache slot block * block_size + offset of position
 * length + i, the value the scatter's slot_mapping takes. PA_ERR_SHAPE if the
 * table would exceed max_blocks_per_seq, PA_ERR_OUT_OF_BLOCKS if the pool is
 * short; neither changes anything. */
pa_status_t pa_bm_append(pa_block_manager* bm, int64_t seq, int32_t num_tokens,
                         int64_t* slots);

/* Drop seq; its blocks lose one reference each. */
pa_status_t pa_bm_free(pa_block_manager* bm, int64_t seq);

int64_t pa_bm_num_free(const pa_block_manager* bm);
/* Tokens of seq, or -1 if unknown. */
int64_t pa_bm_length(const pa_block_manager* bm, int64_t seq);
/* Blocks an append of num_tokens to seq would take from the pool (new blocks
 * plus a copy-on-write block), or -1 if seq is unknown. */
int64_t pa_bm_blocks_needed(const pa_block_manager* bm, int64_t seq, int32_t num_tokens);
/* References to block, or -1 if out of range. */
int32_t pa_bm_refcount(const pa_block_manager* bm, int64_t block);

/* seq's block table: writes min(blocks, capacity) entries to out and pads up
 * to capacity with -1; returns the number of blocks, or -1 if unknown. */
int32_t pa_bm_table(const pa_block_manager* bm, int64_t seq, int32_t* out, int32_t capacity);

/* Block tables and lengths of num_seqs sequences for one step: row i of
 * tables (row_stride int32 entries, row_stride >= max_blocks_per_seq) is
 * seqs[i]'s table padded with -1, context_lens[i] its length. Host arrays. */
pa_status_t pa_bm_tables(const pa_block_manager* bm, const int64_t* seqs, int32_t num_seqs,
                         int32_t* tables, int32_t row_stride, int32_t* context_lens);

/* Move queued copy-on-write pairs (src, dst) into pairs (host, 2 * max_pairs
 * int64) and return how many. Only a run of pairs that one pa_copy_blocks
 * call may apply together is returned: it stops before a pair that writes a
 * block an earlier pair of the run reads or writes, or reads a block an
 * earlier pair writes. A caller loops (take, copy) until 0 comes back, and
 * runs the copies before the scatter of the step's new tokens. Pairs come in
 * the order the appends made them. */
int64_t pa_bm_take_copies(pa_block_manager* bm, int64_t* pairs, int64_t max_pairs);

/*
 * Copy-on-write groups of a decode batch, for pa_decode_shared, from its block
 * tables and lengths (host arrays; the block manager hands forked sequences
 * the same physical blocks for their shared prompt): maximal runs of
 * consecutive sequences whose tables start with the same blocks as the run's
 * first sequence, for at least min_blocks blocks within every member's
 * context. A run's prefix is the number of leading blocks every member shares
 * with the first, times block_size. Runs of one sequence are not groups;
 * sequences between two runs become one group with prefix 0. Writes
 * cu_groups[0 .. G] (capacity num_seqs + 1), prefix_lens[0 .. G - 1]
 * (capacity num_seqs), and the largest member count and prefix of the groups
 * with a non-zero prefix; returns G (0: nothing shared), or -1 for invalid
 * arguments.
 */
int32_t pa_find_shared_prefixes(const int32_t* block_tables, const int32_t* context_lens,
                                int32_t num_seqs, int32_t max_blocks_per_seq,
                                int32_t block_size, int32_t min_blocks, int32_t* cu_groups,
                                int32_t* prefix_lens, int32_t* max_group_size,
                                int32_t* max_prefix_len);

/*
 * Device copy of whole blocks, K and V: for each pair (src, dst) of
 * pairs[num_pairs][2] (int64, device), block dst of both caches (all heads,
 * all rows) receives block src's bytes. A pair with an index outside
 * [0, num_blocks) is skipped. Pairs of one call must be independent (no
 * destination is also a source or a second destination), which
 * pa_bm_take_copies guarantees. Caches as in pa.h; dtype F32, BF16 or
 * PA_DTYPE_FP8_E4M3.
 */
pa_status_t pa_copy_blocks(void* key_cache, void* value_cache, const int64_t* pairs,
                           int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int64_t num_blocks, pa_dtype_t dtype,
                           void* stream);

/*
 * Swapping for preemption: when memory runs short a running sequence's blocks
 * are moved to host memory and its device blocks freed; it resumes later
 * with its context intact (Dissecting vLLM, "Continuous Batching: Breaking
 * the Sequence Barrier"). Both calls copy whole blocks, K and V, for each
 * pair of pairs[num_pairs][2] (int64; device memory or pinned host memory):
 *   pa_swap_out: pair (device block, host block), device caches -> host pools
 *   pa_swap_in:  pair (host block, device block), host pools -> device caches
 * host_key, host_value: [num_host_blocks, num_kv_heads, block_size, head_dim]
 * in pinned host memory (hipHostMalloc, or torch pin_memory), which the kernel
 * reads or writes directly, one launch per batch. Pointer kinds are checked
 * before any launch: pageable host memory or device memory as a host pool is
 * PA_ERR_UNSUPPORTED. A pair outside the pools is skipped. Pairs of one call
 * must be independent (the scheduler's plans are). Asynchronous on stream:
 * the host pool may be read only after the stream has drained.
 */
pa_status_t pa_swap_out(const void* key_cache, const void* value_cache, void* host_key,
                        void* host_value, const int64_t* pairs, int32_t num_pairs,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int64_t num_blocks, int64_t num_host_blocks, pa_dtype_t dtype,
                        void* stream);
pa_status_t pa_swap_in(void* key_cache, void* value_cache, const void* host_key,
                       const void* host_value, const int64_t* pairs, int32_t num_pairs,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int64_t num_blocks, int64_t num_host_blocks, pa_dtype_t dtype,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCKS_H */
