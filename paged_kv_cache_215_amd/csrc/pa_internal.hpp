// Host-side interfaces between the C ABI (pa_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Head of a decode workspace: the plan summary the partition kernel writes for
// the merge kernel, and the work-queue counters. The counters are zero between
// calls: the last partition workgroup to leave the queue resets them.
struct DecodePlan {
  int part_tokens;   // tokens per partition chosen for this batch
  int max_nparts;    // largest partition count of any sequence
  int ticket;        // next ticketed unit; 0 between calls
  int done;          // workgroups that have left the queue; 0 between calls
  int full_total;    // full partitions of the plan (their slots come first)
  int pad[3];
};

struct DecodeArgs {
  float* out;            // [S, Hq, D] float32
  // Copy-on-write groups (num_groups > 0): group g is sequences
  // cu_groups[g] .. cu_groups[g+1] - 1 sharing their first prefix_lens[g]
  // tokens (rounded down to whole blocks). Their shared part was attended by
  // the prefix pass (partials pre_o / pre_ml, [S, Hq, pre_splits]); this
  // launch attends each member's tail from that position on and the merge
  // combines both.
  const int32_t* cu_groups;
  const int32_t* prefix_lens;
  int num_groups;
  int pre_splits;
  float* pre_o;          // [S, Hq, pre_splits, D]
  float* pre_ml;         // [S, Hq, pre_splits, 2]
  int* seq_start;        // [S] first tail position of each group member (written by
                         // the prefix pass; sequences outside every group start at 0)
  float* part_o;         // [unit_slots, Hq, D] normalised partial outputs
  float* part_ml;        // [unit_slots, Hq, 2] (max in log2 units, sum)
  int* full_pre;         // [S] first slot of each sequence's full partitions
                         // (its last partition's slot is full_total + seq)
  const void* query;     // [S, Hq, D]
  const void* key_cache;    // [num_blocks, Hkv, bs, D]
  const void* value_cache;
  const int32_t* block_tables;  // [S, max_blocks_per_seq]
  const int32_t* context_lens;  // [S]
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int head_dim;
  int block_size_log2;
  int max_blocks_per_seq;
  int64_t num_blocks;
  int ctx_limit;         // min(max_context_len, max_blocks_per_seq * block_size)
  DecodePlan* plan;      // workspace head: plan summary for the merge kernel
  int plan_cus;          // CUs of the device (sizes the plan)
  int plan_units_per_cu; // target units per CU for ragged batches that share blocks
  int plan_units_unshared; // the same when no two consecutive sequences share their first block
  int part_floor;        // smallest partition size the plan may choose
  int part_cap;          // largest partition size the plan may choose
  int waves;             // waves per partition workgroup (4 or 8)
  int max_parts;         // ceil(max_context_len / part_floor): most partitions of a sequence
  float scale_log2;      // softmax scale * log2(e)
  const float* k_scale;  // [Hkv] FP8 cache: K = code value * k_scale (else null)
  const float* v_scale;  // [Hkv] FP8 cache: V = code value * v_scale (else null)
};

struct ScatterArgs {
  const void* key;       // [T, Hkv, D]
  const void* value;
  void* key_cache;       // [num_blocks, Hkv, bs, D]
  void* value_cache;
  const int64_t* slot_mapping;  // [T]
  int num_tokens;
  int num_kv_heads;
  int row_chunks;        // D * elem_bytes / 16
  int block_size;
  int64_t num_slots;     // num_blocks * block_size
};

struct ScatterFp8Args {
  const void* key;       // [T, Hkv, D] BF16 or float32
  const void* value;
  void* key_cache;       // [num_blocks, Hkv, bs, D] E4M3 codes
  void* value_cache;
  const int64_t* slot_mapping;  // [T]
  const float* k_scale;  // [Hkv]
  const float* v_scale;  // [Hkv]
  int num_tokens;
  int num_kv_heads;
  int head_dim;
  int block_size;
  int64_t num_slots;     // num_blocks * block_size
  bool src_bf16;         // source rows are BF16 (else float32)
};

// Whole-block copies from a source pool to a destination pool (the same
// cache for copy-on-write; the device cache and a pinned host pool for swaps).
struct CopyArgs {
  const void* src_key;   // [src_blocks, Hkv, bs, D]
  const void* src_value;
  void* dst_key;         // [dst_blocks, Hkv, bs, D]
  void* dst_value;
  const int64_t* pairs;  // [num_pairs][2] (src, dst), device-accessible
  int64_t num_pairs;
  int64_t src_blocks;
  int64_t dst_blocks;
  int64_t block_chunks;  // 16-byte chunks per block of one cache
};

struct PrefillArgs {
  float* out;            // [total_q, Hq, D] float32
  float* part_o;         // split-context partials (may be unused)
  float* part_ml;
  const void* query;     // BF16 [total_q, Hq, D]
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* cu_q_lens;     // [S + 1]
  int num_seqs;
  int total_q;
  int max_q_len;
  int num_q_heads;
  int num_kv_heads;
  int head_dim;
  int block_size_log2;
  int max_blocks_per_seq;
  int64_t num_blocks;
  int ctx_limit;
  int kv_splits;         // context splits per row tile (1 = no partials)
  int xcd_remap;         // group workgroups of one (KV head, split) on one XCD
  float scale_log2;
  bool kv_fp8;           // caches hold E4M3 codes (else BF16)
  const float* k_scale;  // [Hkv] E4M3 cache: K = code value * k_scale (else null)
  const float* v_scale;  // [Hkv] E4M3 cache: V = code value * v_scale (else null)
  // Prefix mode (the shared-prefix pass of a grouped decode): "sequence" g is
  // a copy-on-write group whose rows are its members' decode queries
  // (cu_q_lens = group bounds over the decode batch), context_lens holds the
  // groups' shared prefix lengths, the blocks are read through the first
  // member's table, no causal mask applies, row r sees keys below its own
  // member_lens entry, and partials are always written (part_o / part_ml
  // indexed by (member, query head, split)) for the decode merge.
  int prefix_mode;
  const int32_t* member_lens;   // [S] decode context lengths (prefix mode)
  int* seq_start;        // [S] prefix mode: written with each member's tail start
  int min_waves;         // waves per workgroup at least (0: the default for the group)
};

struct DecodeLaunch {
  int part_floor;        // smallest partition size: one that keeps the plan's
                         // partitions within unit_slots
  int part_cap;
  int max_parts;
  int waves;
  int64_t unit_slots;    // partition slots of the workspace (per query head)
};

int decode_waves_per_workgroup();
DecodeLaunch decode_launch_shape(int num_seqs, int num_kv_heads, int block_size,
                                 int max_context_len);
enum class KvType { F32, BF16, FP8 };
hipError_t launch_decode(const DecodeArgs& a, KvType kv, hipStream_t stream);
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream);
hipError_t launch_scatter(const ScatterArgs& a, hipStream_t stream);
hipError_t launch_scatter_fp8(const ScatterFp8Args& a, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream);

int prefill_kv_splits(int num_seqs, int max_q_len, int num_q_heads, int num_kv_heads,
                      int head_dim, int max_context_len);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
int prefix_pass_splits(int num_groups, int max_group_size, int num_q_heads, int num_kv_heads,
                       int max_prefix_len);

}  // namespace pa
