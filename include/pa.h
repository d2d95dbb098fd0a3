/*
 * pa.h - paged attention on AMD Instinct MI355X (gfx950): C ABI.
 *
 * The KV cache is cut into fixed-size physical blocks of 16 or 32 tokens and a
 * per-sequence block table maps each logical token position to the physical
 * block that holds it (How vLLM gets real throughput on H100s, "PagedAttention
 * borrows from operating systems"; vLLM architecture, memory and benchmarks
 * deep dive, "PagedAttention: a 1960s idea for modern GPUs"). The attention
 * kernels walk that table at run time and gather K/V from the scattered blocks
 * (Dissecting vLLM, "PagedAttention: Virtual Memory for KV Cache").
 *
 * Layouts (all row-major, contiguous, element type given by pa_dtype_t):
 *   key_cache, value_cache  [num_blocks, num_kv_heads, block_size, head_dim]
 *       one (block, head) tile of block_size rows of head_dim elements is
 *       contiguous; token slot s lives in block s / block_size, row
 *       s % block_size.
 *   block_tables            int32 [num_seqs, max_blocks_per_seq]; entry j is
 *       the physical block of logical tokens j*block_size .. (j+1)*block_size-1.
 *       Several sequences may name the same physical block (copy-on-write
 *       sharing of a prompt: How vLLM gets real throughput on H100s,
 *       "PagedAttention borrows from operating systems").
 *   context_lens            int32 [num_seqs]; tokens attended, new token
 *       included (it is written by pa_reshape_and_cache first).
 *   query                   [num_seqs, num_q_heads, head_dim] (decode) or
 *                           [total_q, num_q_heads, head_dim] (prefill chunk)
 *   out                     float32, same leading shape as query.
 * Query head h reads KV head h / (num_q_heads / num_kv_heads) (grouped-query
 * attention, as in the pages' example of 4 KV heads of dimension 256).
 *
 * Ownership and threading: every pointer argument except `stream` is a device
 * pointer owned by the caller. The library allocates no device memory, keeps
 * no pointer after a call returns, and never synchronizes: each call enqueues
 * its kernels on `stream` (a hipStream_t; NULL means the null stream) and
 * returns. The caller keeps every buffer alive until the stream has drained.
 * Calls are reentrant; concurrent calls must not share output or workspace
 * buffers.
 *
 * Errors: a negative count is PA_ERR_SHAPE and a zero count of tokens /
 * sequences / rows is a successful no-op; both are decided first. The other
 * host-visible arguments are then checked before any HIP call, in this order,
 * and the first failure is returned:
 *   PA_ERR_NULL         a required pointer is NULL
 *   PA_ERR_SHAPE        a size is negative or zero where it must be positive,
 *                       or num_q_heads is not a multiple of num_kv_heads
 *   PA_ERR_UNSUPPORTED  block_size not 16/32, head_dim not 64/128/256, query
 *                       group size not 1/2/4/8, or a dtype the entry point
 *                       does not take
 *   PA_ERR_ALIGN        a tensor or workspace pointer is not 16-byte aligned,
 *                       or an index or scale array is not aligned to its
 *                       element size
 *   PA_ERR_WORKSPACE    the workspace is smaller than the size query returns
 *   PA_ERR_HIP          a kernel launch failed (hipGetLastError after launch)
 * Device-resident values (table entries, lengths, slots) are not checked on
 * the host, since that would need a synchronization. The kernels never read or
 * write outside the buffers the sizes describe: a table entry outside
 * [0, num_blocks) makes its tokens contribute nothing, a length above
 * max_blocks_per_seq * block_size (or above max_context_len) is clamped, and a
 * slot outside [0, num_blocks * block_size) is skipped; the results for such
 * rows are then unspecified. Duplicate non-negative slots in one scatter call
 * leave either token's bits in that slot.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_DTYPE_F32 = 0,   /* IEEE binary32 */
  PA_DTYPE_BF16 = 1,  /* bfloat16: the top 16 bits of a binary32 */
  PA_DTYPE_FP8_E4M3 = 2  /* OCP E4M3 codes (block copies only; see the FP8 entry points) */
} pa_dtype_t;

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,
  PA_ERR_SHAPE = 2,
  PA_ERR_UNSUPPORTED = 3,
  PA_ERR_ALIGN = 4,
  PA_ERR_WORKSPACE = 5,
  PA_ERR_HIP = 6,
  PA_ERR_OUT_OF_BLOCKS = 7,  /* block manager: the pool lacks the blocks asked for */
  PA_ERR_STATE = 8,          /* block manager: unknown or duplicate sequence id */
  PA_ERR_NOMEM = 9           /* host side: an allocation failed (no C++ exception
                                ever crosses this ABI; see pa_blocks.h) */
} pa_status_t;

/*
 * Cache-write scatter. Blocks fill as tokens are generated (How vLLM gets real
 * throughput on H100s, "PagedAttention borrows from operating systems"): for
 * every token t with s = slot_mapping[t] in [0, num_blocks*block_size),
 *   key_cache  [s / block_size, h, s % block_size, :] = key  [t, h, :]
 *   value_cache[s / block_size, h, s % block_size, :] = value[t, h, :]
 * for all h. A bit copy: no conversion, no rounding. A negative slot skips the
 * token.
 *   key, value      [num_tokens, num_kv_heads, head_dim], element type dtype
 *   slot_mapping    int64 [num_tokens]
 * dtype: PA_DTYPE_F32 or PA_DTYPE_BF16 (the cache's own type).
 */
pa_status_t pa_reshape_and_cache(const void* key, const void* value,
                                 void* key_cache, void* value_cache,
                                 const int64_t* slot_mapping,
                                 int32_t num_tokens, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size,
                                 int64_t num_blocks, pa_dtype_t dtype,
                                 void* stream);

/*
 * Bytes of device workspace pa_decode needs for these sizes: a 256-byte head
 * (plan summary and work-queue counters), then split-context partial results.
 * The partials are bounded by the batch, not by max_context_len alone: about
 * one slot per sequence plus a fixed spare of 2048 (per query head, head_dim
 * + 2 floats each), unless the largest partitions (8192 tokens) need more;
 * capped by the slots of 256-token partitions. Depends only on the
 * arguments; 0 never occurs for positive sizes. Returns 0 for arguments
 * pa_decode would reject.
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int32_t max_context_len);

/*
 * Zero-fills the head of a decode workspace (its first 256 bytes, or all of
 * it if smaller) on `stream`, with a fill kernel so that it can be captured
 * in a graph. A workspace must be initialised once before its first
 * pa_decode; every pa_decode leaves the head at zero again (the last
 * partition workgroup resets the counters), whatever happens to later
 * launches. Any zero fill (for example a buffer allocated zeroed) serves
 * equally.
 */
pa_status_t pa_decode_workspace_init(void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * Decode attention: one new query per sequence over its whole paged context
 * (decode re-reads the KV cache at every step and is bound by memory
 * bandwidth: How vLLM gets real throughput on H100s, "Decode is a memory
 * problem, not a math problem"). For sequence b with n = context_lens[b] and
 * query head h of KV group g = h / G:
 *   out[b,h,:] = sum_{j<n} softmax_j(scale * q[b,h,:] . k_j) v_j
 * where k_j, v_j are KV head g's rows at logical position j, found through
 * block_tables[b, j / block_size]. n == 0 gives a zero row. Accumulation is
 * float32; out is float32 and fully overwritten (never read).
 *   query           [num_seqs, num_q_heads, head_dim], element type dtype
 *   workspace       device buffer of at least pa_decode_workspace_size(...)
 *                   bytes, initialised before its first use (see
 *                   pa_decode_workspace_init) and then left to the library
 *                   between calls. Its head holds a work-queue counter that
 *                   the call takes with atomics and sets back to zero, so two
 *                   calls that overlap on one workspace race (stream order
 *                   is fine). A workspace that was never initialised gives
 *                   wrong results but no out-of-bounds access.
 *   max_context_len upper bound of context_lens (sizes the launch grid).
 * dtype: PA_DTYPE_F32 or PA_DTYPE_BF16 for query and both caches.
 */
pa_status_t pa_decode(float* out, const void* query,
                      const void* key_cache, const void* value_cache,
                      const int32_t* block_tables, const int32_t* context_lens,
                      int32_t num_seqs, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t max_blocks_per_seq,
                      int64_t num_blocks, int32_t max_context_len,
                      float scale, pa_dtype_t dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode without a workspace, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments, result and errors as pa_decode, less
 * the workspace: the split-context partials and the work-queue counters live
 * in a static device array of pa_decode_noalloc_max_bytes() bytes (64 MiB)
 * inside the library, one per GPU, held until the process ends. Sizes whose
 * pa_decode_workspace_size exceeds it return PA_ERR_WORKSPACE before any HIP
 * call (64 sequences x 8192 tokens at 16 query heads, d 256, fit: 32.3 MiB).
 * Each call first clears the array's head (a fill kernel) and then runs the
 * decode kernels on it; it calls no allocating routine. Every call on one GPU
 * shares the array, so calls that overlap on one GPU (other streams, other
 * threads) race; calls in one stream's order are fine.
 */
pa_status_t pa_decode_noalloc(float* out, const void* query,
                              const void* key_cache, const void* value_cache,
                              const int32_t* block_tables,
                              const int32_t* context_lens, int32_t num_seqs,
                              int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size,
                              int32_t max_blocks_per_seq, int64_t num_blocks,
                              int32_t max_context_len, float scale,
                              pa_dtype_t dtype, void* stream);

/* Size of pa_decode_noalloc's static scratch, in bytes. */
size_t pa_decode_noalloc_max_bytes(void);

/*
 * Decode of a batch that holds copy-on-write groups: sequences forked from
 * one prompt point at the prompt's physical blocks (How vLLM gets real
 * throughput on H100s, "PagedAttention borrows from operating systems";
 * Dissecting vLLM, "PagedAttention: Virtual Memory for KV Cache"), so the
 * shared blocks need to be read once per group, not once per member. The
 * result is pa_decode's (pa_decode_fp8's for an E4M3 cache); only the order
 * of the arithmetic differs:
 *   1. a shared-prefix pass on the matrix cores: for each group, its members'
 *      queries (G heads each) are the rows of one product over the group's
 *      shared blocks, read through the FIRST member's table; member b sees
 *      positions below min(prefix, n_b);
 *   2. the decode kernels over each member's private tail (positions from
 *      the prefix on), and over every ungrouped sequence in full;
 *   3. the merge of both partial results by log-sum-exp.
 * Groups (device int32 arrays):
 *   cu_groups    [num_groups + 1], non-decreasing, within [0, num_seqs]:
 *                group g is sequences cu_groups[g] .. cu_groups[g+1] - 1
 *                (sequences outside [cu_groups[0], cu_groups[num_groups])
 *                are in no group); bounds outside the batch are clamped;
 *   prefix_lens  [num_groups]: positions 0 .. prefix_lens[g] - 1 hold the same
 *                K/V in every member (their blocks are shared). Only whole
 *                blocks count: the prefix is rounded down to a multiple of
 *                block_size (a partly filled last prompt block is attended
 *                with each tail). 0 = nothing shared.
 *   max_group_size  upper bound of the members of any group whose prefix is
 *                at least one block; max_prefix_len upper bound of
 *                prefix_lens. Both size the launch (host values).
 * Other arguments as pa_decode / pa_decode_fp8: cache_dtype is
 * PA_DTYPE_BF16 (k_scale, v_scale ignored) or PA_DTYPE_FP8_E4M3 (scales
 * required); the query is BF16. At most 4096 sequences per call. num_groups
 * = 0 is a plain decode. The workspace is pa_decode_shared_workspace_size
 * bytes (a decode workspace, initialised once as with pa_decode_workspace_init,
 * followed by the prefix pass's partials).
 */
size_t pa_decode_shared_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t max_context_len,
                                       int32_t num_groups, int32_t max_group_size,
                                       int32_t max_prefix_len);

pa_status_t pa_decode_shared(float* out, const void* query,
                             const void* key_cache, const void* value_cache,
                             const float* k_scale, const float* v_scale,
                             const int32_t* block_tables,
                             const int32_t* context_lens,
                             const int32_t* cu_groups, const int32_t* prefix_lens,
                             int32_t num_groups, int32_t max_group_size,
                             int32_t max_prefix_len, int32_t num_seqs,
                             int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size,
                             int32_t max_blocks_per_seq, int64_t num_blocks,
                             int32_t max_context_len, float scale,
                             pa_dtype_t cache_dtype, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * FP8 KV cache. Quantizing the cache to FP8 halves the bytes every decode
 * step re-reads, which the pages count as doubling the effective memory
 * bandwidth (vLLM architecture, memory and benchmarks deep dive,
 * "Hardware-level optimizations"). They fix no format; the one used here:
 *   codes     OCP E4M3: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits;
 *             exponent 0 is subnormal (m/8 * 2^-6); no infinities;
 *             S.1111.111 is NaN; largest magnitude 448. One byte per element,
 *             same cache layout as above.
 *   scales    float32 device arrays k_scale, v_scale [num_kv_heads]: the value
 *             of K code c of head h is E4M3(c) * k_scale[h] (V likewise).
 *             They must be positive and finite (not checked: device memory).
 *
 * pa_reshape_and_cache_fp8: the scatter above, writing codes
 *   code = E4M3(x / scale[h])
 * with x widened to float32 and divided in IEEE float32, rounded to nearest
 * with ties to even, magnitudes above 448 (infinity included) saturated to
 * +-448, NaN kept as NaN with its sign, the sign of zero kept.
 *   key, value   [num_tokens, num_kv_heads, head_dim], src_dtype F32 or BF16
 *   key_cache, value_cache  uint8 codes [num_blocks, num_kv_heads, block_size, head_dim]
 */
pa_status_t pa_reshape_and_cache_fp8(const void* key, const void* value,
                                     void* key_cache, void* value_cache,
                                     const int64_t* slot_mapping,
                                     const float* k_scale, const float* v_scale,
                                     int32_t num_tokens, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size,
                                     int64_t num_blocks, pa_dtype_t src_dtype,
                                     void* stream);

/*
 * pa_decode over an FP8 cache: the attention of pa_decode with k_j and v_j
 * the dequantized rows (code value times the head's scale). The products
 * q . k_j are exact in float32 (E4M3 values are BF16 values), so the result
 * differs from pa_decode on the dequantized cache only by float32 rounding.
 * The workspace is the one pa_decode_workspace_size / pa_decode_workspace_init
 * describe for the same sizes (the two entry points may share it in stream
 * order).
 * query_dtype: PA_DTYPE_BF16 only.
 */
pa_status_t pa_decode_fp8(float* out, const void* query,
                          const void* key_cache, const void* value_cache,
                          const float* k_scale, const float* v_scale,
                          const int32_t* block_tables, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t max_blocks_per_seq,
                          int64_t num_blocks, int32_t max_context_len,
                          float scale, pa_dtype_t query_dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace pa_prefill_chunk needs for these sizes; may be 0.
 */
size_t pa_prefill_chunk_workspace_size(int32_t num_seqs, int32_t total_q,
                                       int32_t max_q_len, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size,
                                       int32_t max_context_len);

/*
 * Causal chunk of a prompt against the paged cache. Prefill is a dense
 * matrix product (How vLLM gets real throughput on H100s, "Decode is a memory
 * problem, not a math problem") and chunked prefill cuts a long prompt into
 * pieces interleaved with decode tokens (vLLM architecture, memory and
 * benchmarks deep dive, "Hardware-level optimizations"). Rows
 * cu_q_lens[b] .. cu_q_lens[b+1]-1 of query are sequence b's chunk of
 * L = cu_q_lens[b+1] - cu_q_lens[b] rows; its K/V are already in the cache and
 * n = context_lens[b] counts prefix plus chunk, so row i sits at position
 * n - L + i and attends keys 0 .. n - L + i:
 *   out[r,h,:] = sum_{j <= n-L+i} softmax_j(scale * q[r,h,:] . k_j) v_j
 * QK^T and PV run on the matrix cores in BF16 with float32 accumulation; each
 * softmax weight enters the PV product as the sum of two BF16 values (about
 * 16 significant bits).
 *   query      BF16 [total_q, num_q_heads, head_dim]
 *   cu_q_lens  int32 [num_seqs + 1], device, non-decreasing, cu[0] = 0,
 *              cu[num_seqs] = total_q; each chunk length <= max_q_len and
 *              <= its context length.
 *   workspace  at least pa_prefill_chunk_workspace_size(...) bytes.
 * dtype: PA_DTYPE_BF16 only.
 */
pa_status_t pa_prefill_chunk(float* out, const void* query,
                             const void* key_cache, const void* value_cache,
                             const int32_t* block_tables,
                             const int32_t* context_lens,
                             const int32_t* cu_q_lens,
                             int32_t num_seqs, int32_t total_q,
                             int32_t max_q_len, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t max_blocks_per_seq,
                             int64_t num_blocks, int32_t max_context_len,
                             float scale, pa_dtype_t dtype,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * pa_prefill_chunk over an FP8 cache (codes and per-head scales as for
 * pa_decode_fp8): the causal chunk attention of pa_prefill_chunk with k_j and
 * v_j the dequantized rows. The pages name the FP8 cache and chunked prefill
 * together as levers of one serving step (vLLM architecture, memory and
 * benchmarks deep dive, "Hardware-level optimizations"). The codes are
 * converted exactly to BF16 as the K/V tiles are staged for the matrix cores;
 * the K scale folds into the softmax scale and the V scale into the output.
 * The workspace is the one pa_prefill_chunk_workspace_size describes for the
 * same sizes.
 * query_dtype: PA_DTYPE_BF16 only.
 */
pa_status_t pa_prefill_chunk_fp8(float* out, const void* query,
                                 const void* key_cache, const void* value_cache,
                                 const float* k_scale, const float* v_scale,
                                 const int32_t* block_tables,
                                 const int32_t* context_lens,
                                 const int32_t* cu_q_lens,
                                 int32_t num_seqs, int32_t total_q,
                                 int32_t max_q_len, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t max_blocks_per_seq,
                                 int64_t num_blocks, int32_t max_context_len,
                                 float scale, pa_dtype_t query_dtype,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Static, NUL-terminated description of a status code. */
const char* pa_status_string(pa_status_t status);

/* Library version as major*10000 + minor*100 + patch. */
int32_t pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
