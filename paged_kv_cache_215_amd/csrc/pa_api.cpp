// C ABI of the paged-attention library: argument validation (before any HIP
// call), launch geometry, workspace carving. Declarations and the contract of
// every entry point are in include/pa.h.

#include "pa.h"
#include "pa_blocks.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdlib>

#include "pa_internal.hpp"

namespace pa {

int decode_waves_per_workgroup() {
  static const int waves = [] {
    const char* s = std::getenv("PA_DECODE_WAVES");
    const int v = s ? std::atoi(s) : 0;
    return v == 4 ? 4 : 8;
  }();
  return waves;
}

}  // namespace pa

// Decode scratch for pa_decode_noalloc: a fixed device array that every call
// on a GPU shares (each GPU the library runs on holds its own copy until the
// process ends). In host code `scratch` only names the symbol: its device
// address comes from hipGetSymbolAddress, once per device, and only that
// address is ever passed to a kernel or a fill.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_block(int32_t bs) { return bs == 16 || bs == 32; }
bool supported_dim(int32_t d) { return d == 64 || d == 128 || d == 256; }
bool supported_group(int32_t hq, int32_t hkv) {
  const int32_t g = hq / hkv;
  return g == 1 || g == 2 || g == 4 || g == 8;
}
int log2_exact(int32_t v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}
int elem_bytes(pa_dtype_t t) { return t == PA_DTYPE_BF16 ? 2 : 4; }

int32_t ctx_limit(int32_t max_ctx, int32_t max_blocks, int32_t bs) {
  const int64_t cap = (int64_t)max_blocks * bs;
  return (int32_t)(cap < max_ctx ? cap : max_ctx);
}

struct DecodeGeometry {
  pa::DecodeLaunch launch;
  size_t full_pre_off;
  size_t part_o_off;
  size_t part_ml_off;
  size_t bytes;
};

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace: plan summary and work-queue counters (256 bytes) | first slot of
// each sequence's partitions | partial outputs | partial (m, l). Launches of
// at most 4096 sequences each reuse it in stream order.
constexpr size_t kDecodeHeadBytes = 256;

DecodeGeometry decode_geometry(int32_t num_seqs, int32_t hq, int32_t hkv, int32_t d, int32_t bs,
                               int32_t max_ctx) {
  DecodeGeometry g;
  g.launch = pa::decode_launch_shape(num_seqs, hkv, bs, max_ctx);
  const size_t seqs = num_seqs < 4096 ? (size_t)num_seqs : 4096;
  const size_t rows = (size_t)g.launch.unit_slots * hq;
  g.full_pre_off = kDecodeHeadBytes;
  g.part_o_off = round_up(g.full_pre_off + seqs * sizeof(int32_t), 256);
  g.part_ml_off = round_up(g.part_o_off + rows * d * sizeof(float), 256);
  g.bytes = round_up(g.part_ml_off + rows * 2 * sizeof(float), 256);
  return g;
}

pa_status_t from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

int64_t dtype_bytes(pa_dtype_t t) { return t == PA_DTYPE_F32 ? 4 : t == PA_DTYPE_BF16 ? 2 : 1; }

// Device-visible address of p: device memory as is, pinned host memory
// through its mapping; nullptr for memory a kernel cannot reach (pageable
// host memory, unknown pointers). The query's error, if any, is cleared so
// that it cannot be reported by a later launch check.
const void* device_view(const void* p, bool allow_device) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (attr.type == hipMemoryTypeDevice) return allow_device ? p : nullptr;
  if (attr.type != hipMemoryTypeHost || !attr.devicePointer) return nullptr;
  const char* base_h = static_cast<const char*>(attr.hostPointer ? attr.hostPointer : p);
  return static_cast<const char*>(attr.devicePointer) + (static_cast<const char*>(p) - base_h);
}

// Swap of whole blocks between the device caches and pinned host pools:
// out = device -> host, else host -> device. Pointer kinds are checked
// before any launch.
pa_status_t swap_impl(const void* key_cache, const void* value_cache, const void* host_key,
                      const void* host_value, const int64_t* pairs, int32_t num_pairs,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int64_t num_blocks, int64_t num_host_blocks, pa_dtype_t dtype,
                      void* stream, bool out) {
  if (num_pairs < 0) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!key_cache || !value_cache || !host_key || !host_value || !pairs) return PA_ERR_NULL;
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0 ||
      num_host_blocks <= 0)
    return PA_ERR_SHAPE;
  if (!supported_block(block_size) || !supported_dim(head_dim) ||
      (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16 && dtype != PA_DTYPE_FP8_E4M3))
    return PA_ERR_UNSUPPORTED;
  if (!aligned(key_cache, 16) || !aligned(value_cache, 16) || !aligned(host_key, 16) ||
      !aligned(host_value, 16) || !aligned(pairs, 8))
    return PA_ERR_ALIGN;
  const void* hk = device_view(host_key, false);
  const void* hv = device_view(host_value, false);
  const void* pp = device_view(pairs, true);
  const void* dk = device_view(key_cache, true);
  const void* dv = device_view(value_cache, true);
  if (!hk || !hv || !pp || !dk || !dv) return PA_ERR_UNSUPPORTED;  // host pools must be pinned
  key_cache = dk;
  value_cache = dv;
  pa::CopyArgs a;
  a.src_key = out ? key_cache : hk;
  a.src_value = out ? value_cache : hv;
  a.dst_key = const_cast<void*>(out ? hk : key_cache);
  a.dst_value = const_cast<void*>(out ? hv : value_cache);
  a.pairs = static_cast<const int64_t*>(pp);
  a.num_pairs = num_pairs;
  a.src_blocks = out ? num_blocks : num_host_blocks;
  a.dst_blocks = out ? num_host_blocks : num_blocks;
  a.block_chunks = (int64_t)num_kv_heads * block_size * head_dim * dtype_bytes(dtype) / 16;
  return from_hip(pa::launch_copy_blocks(a, static_cast<hipStream_t>(stream)));
}

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device, looked up on the first
// call there (nullptr if the lookup fails; its error is cleared).
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
    (void)hipGetLastError();
    return nullptr;
  }
  scratch_ptr[dev].store(p, std::memory_order_release);  // the same value on every race
  return p;
}

// Copy-on-write groups of a grouped decode (pa_decode_shared).
struct GroupSpec {
  const int32_t* cu_groups;
  const int32_t* prefix_lens;
  int32_t num_groups;
  int32_t max_group_size;
  int32_t max_prefix_len;
};

// Workspace of a grouped decode: the decode workspace, then each sequence's
// tail start, then the prefix pass's partials [S, Hq, splits, D] and
// [S, Hq, splits, 2].
struct SharedGeometry {
  DecodeGeometry dec;
  int splits;
  size_t seq_start_off;
  size_t pre_o_off;
  size_t pre_ml_off;
  size_t bytes;
};

SharedGeometry shared_geometry(int32_t num_seqs, int32_t hq, int32_t hkv, int32_t d, int32_t bs,
                               int32_t max_ctx, const GroupSpec& gs) {
  SharedGeometry g;
  g.dec = decode_geometry(num_seqs, hq, hkv, d, bs, max_ctx);
  g.splits = gs.num_groups > 0 ? pa::prefix_pass_splits(gs.num_groups, gs.max_group_size, hq, hkv,
                                                        gs.max_prefix_len)
                               : 0;
  const size_t rows = (size_t)num_seqs * hq * g.splits;
  g.seq_start_off = round_up(g.dec.bytes, 256);
  g.pre_o_off = round_up(g.seq_start_off + (size_t)num_seqs * sizeof(int32_t), 256);
  g.pre_ml_off = round_up(g.pre_o_off + rows * d * sizeof(float), 256);
  g.bytes = round_up(g.pre_ml_off + rows * 2 * sizeof(float), 256);
  return g;
}

// Validation (NULL -> SHAPE -> UNSUPPORTED -> ALIGN -> WORKSPACE) and launch of
// a decode over a cache of type kv. type_ok is the caller's check of its
// element types (reported as UNSUPPORTED); an FP8 cache also needs its two
// scale arrays. With use_scratch the decode runs on the static scratch
// instead of a caller's workspace (workspace and workspace_bytes are then
// ignored): the sizes must fit kScratchBytes, and the scratch head is cleared
// with a fill kernel before the launch.
pa_status_t decode_impl(float* out, const void* query, const void* key_cache,
                        const void* value_cache, const float* k_scale, const float* v_scale,
                        const int32_t* block_tables, const int32_t* context_lens,
                        int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                        int64_t num_blocks, int32_t max_context_len, float scale, pa::KvType kv,
                        bool type_ok, void* workspace, size_t workspace_bytes, void* stream,
                        bool use_scratch = false, const GroupSpec* groups = nullptr) {
  const bool scaled = kv == pa::KvType::FP8;
  const bool grouped = groups && groups->num_groups > 0;
  if (num_seqs < 0 || (groups && groups->num_groups < 0)) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens ||
      (!workspace && !use_scratch) || (scaled && (!k_scale || !v_scale)) ||
      (grouped && (!groups->cu_groups || !groups->prefix_lens)))
    return PA_ERR_NULL;
  if (num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      max_blocks_per_seq <= 0 || num_blocks <= 0 || max_context_len < 0 ||
      num_q_heads % num_kv_heads != 0 || !std::isfinite(scale) ||
      (grouped && (groups->max_group_size <= 0 || groups->max_prefix_len < 0)))
    return PA_ERR_SHAPE;
  if (!supported_block(block_size) || !supported_dim(head_dim) ||
      !supported_group(num_q_heads, num_kv_heads) || !type_ok || (groups && num_seqs > 4096))
    return PA_ERR_UNSUPPORTED;
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(key_cache, 16) ||
      !aligned(value_cache, 16) || (!use_scratch && !aligned(workspace, 16)) ||
      !aligned(block_tables, 4) ||
      !aligned(context_lens, 4) || (scaled && (!aligned(k_scale, 4) || !aligned(v_scale, 4))) ||
      (grouped && (!aligned(groups->cu_groups, 4) || !aligned(groups->prefix_lens, 4))))
    return PA_ERR_ALIGN;
  const GroupSpec none{nullptr, nullptr, 0, 0, 0};
  const SharedGeometry sgeo = shared_geometry(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                              block_size, max_context_len,
                                              grouped ? *groups : none);
  const DecodeGeometry& geo = sgeo.dec;
  const size_t need = groups ? sgeo.bytes : geo.bytes;
  if ((use_scratch ? kScratchBytes : workspace_bytes) < need) return PA_ERR_WORKSPACE;
  if (use_scratch) {
    workspace = scratch_on_current_device();
    if (!workspace) return PA_ERR_HIP;
    if (pa::launch_zero_fill(workspace, kDecodeHeadBytes, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
      return PA_ERR_HIP;
  }

  pa::DecodeArgs a;
  char* ws = static_cast<char*>(workspace);
  a.out = out;
  a.plan = reinterpret_cast<pa::DecodePlan*>(ws);
  a.plan_cus = 0;
  a.plan_units_per_cu = 0;
  a.plan_units_unshared = 0;
  a.part_o = reinterpret_cast<float*>(ws + geo.part_o_off);
  a.part_ml = reinterpret_cast<float*>(ws + geo.part_ml_off);
  a.full_pre = reinterpret_cast<int*>(ws + geo.full_pre_off);
  a.query = query;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size_log2 = log2_exact(block_size);
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.ctx_limit = ctx_limit(max_context_len, max_blocks_per_seq, block_size);
  a.part_floor = geo.launch.part_floor;
  a.part_cap = geo.launch.part_cap;
  a.waves = geo.launch.waves;
  a.max_parts = geo.launch.max_parts;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.cu_groups = nullptr;
  a.prefix_lens = nullptr;
  a.num_groups = 0;
  a.pre_splits = 0;
  a.pre_o = nullptr;
  a.pre_ml = nullptr;
  a.seq_start = nullptr;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (grouped) {
    a.cu_groups = groups->cu_groups;
    a.prefix_lens = groups->prefix_lens;
    a.num_groups = groups->num_groups;
    a.pre_splits = sgeo.splits;
    a.pre_o = reinterpret_cast<float*>(ws + sgeo.pre_o_off);
    a.pre_ml = reinterpret_cast<float*>(ws + sgeo.pre_ml_off);
    a.seq_start = reinterpret_cast<int*>(ws + sgeo.seq_start_off);
    // The shared-prefix pass on the matrix cores: each group's members are
    // the query rows of one causal-free chunk over the group's whole shared
    // blocks; its partials go to pre_o / pre_ml for the merge.
    pa::PrefillArgs p;
    p.out = nullptr;
    p.part_o = a.pre_o;
    p.part_ml = a.pre_ml;
    p.query = query;
    p.key_cache = key_cache;
    p.value_cache = value_cache;
    p.block_tables = block_tables;
    p.context_lens = groups->prefix_lens;
    p.cu_q_lens = groups->cu_groups;
    p.num_seqs = groups->num_groups;
    p.total_q = num_seqs;
    p.max_q_len = groups->max_group_size;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = num_kv_heads;
    p.head_dim = head_dim;
    p.block_size_log2 = a.block_size_log2;
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.num_blocks = num_blocks;
    p.ctx_limit = a.ctx_limit;
    p.kv_splits = sgeo.splits;
    p.xcd_remap = 1;
    p.scale_log2 = a.scale_log2;
    p.kv_fp8 = scaled;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.prefix_mode = 1;
    p.member_lens = context_lens;
    p.seq_start = a.seq_start;
    p.min_waves = 4;
    const hipError_t err = pa::launch_prefill(p, st);
    if (err != hipSuccess) return PA_ERR_HIP;
  }
  return from_hip(pa::launch_decode(a, kv, st));
}

// Validation (NULL -> SHAPE -> UNSUPPORTED -> ALIGN -> WORKSPACE) and launch of
// a prefill chunk over a BF16 cache, or an E4M3 one with its two scale arrays.
pa_status_t prefill_impl(float* out, const void* query, const void* key_cache,
                         const void* value_cache, const float* k_scale, const float* v_scale,
                         const int32_t* block_tables, const int32_t* context_lens,
                         const int32_t* cu_q_lens, int32_t num_seqs, int32_t total_q,
                         int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                         int64_t num_blocks, int32_t max_context_len, float scale, bool fp8,
                         bool type_ok, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs < 0 || total_q < 0) return PA_ERR_SHAPE;
  if (num_seqs == 0 || total_q == 0) return PA_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens ||
      !cu_q_lens || (fp8 && (!k_scale || !v_scale)))
    return PA_ERR_NULL;
  if (max_q_len <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || max_context_len < 0 ||
      num_q_heads % num_kv_heads != 0 || !std::isfinite(scale))
    return PA_ERR_SHAPE;
  if (!supported_block(block_size) || !supported_dim(head_dim) ||
      !supported_group(num_q_heads, num_kv_heads) || !type_ok)
    return PA_ERR_UNSUPPORTED;
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(key_cache, 16) ||
      !aligned(value_cache, 16) || !aligned(block_tables, 4) || !aligned(context_lens, 4) ||
      !aligned(cu_q_lens, 4) || (workspace && !aligned(workspace, 16)) ||
      (fp8 && (!aligned(k_scale, 4) || !aligned(v_scale, 4))))
    return PA_ERR_ALIGN;
  const size_t need = pa_prefill_chunk_workspace_size(num_seqs, total_q, max_q_len, num_q_heads,
                                                      num_kv_heads, head_dim, block_size,
                                                      max_context_len);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PA_ERR_WORKSPACE;

  pa::PrefillArgs a;
  a.out = out;
  a.xcd_remap = 1;
  a.kv_splits = pa::prefill_kv_splits(num_seqs, max_q_len, num_q_heads, num_kv_heads, head_dim,
                                             max_context_len);
  if (a.kv_splits < 1) a.kv_splits = 1;
  const size_t rows = (size_t)total_q * num_q_heads * a.kv_splits;
  a.part_o = need ? static_cast<float*>(workspace) : nullptr;
  a.part_ml = need ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                              rows * head_dim * sizeof(float))
                   : nullptr;
  a.query = query;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.cu_q_lens = cu_q_lens;
  a.num_seqs = num_seqs;
  a.total_q = total_q;
  a.max_q_len = max_q_len;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size_log2 = log2_exact(block_size);
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.ctx_limit = ctx_limit(max_context_len, max_blocks_per_seq, block_size);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.kv_fp8 = fp8;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.prefix_mode = 0;
  a.member_lens = nullptr;
  a.seq_start = nullptr;
  a.min_waves = 0;
  return from_hip(pa::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

pa_status_t pa_reshape_and_cache(const void* key, const void* value, void* key_cache,
                                 void* value_cache, const int64_t* slot_mapping,
                                 int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int64_t num_blocks, pa_dtype_t dtype,
                                 void* stream) {
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PA_ERR_NULL;
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_ERR_SHAPE;
  if (!supported_block(block_size) || !supported_dim(head_dim) ||
      (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16))
    return PA_ERR_UNSUPPORTED;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(key_cache, 16) ||
      !aligned(value_cache, 16) || !aligned(slot_mapping, 8))
    return PA_ERR_ALIGN;
  pa::ScatterArgs a;
  a.key = key;
  a.value = value;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_kv_heads = num_kv_heads;
  a.row_chunks = head_dim * elem_bytes(dtype) / 16;
  a.block_size = block_size;
  a.num_slots = num_blocks * block_size;
  return from_hip(pa::launch_scatter(a, static_cast<hipStream_t>(stream)));
}

pa_status_t pa_reshape_and_cache_fp8(const void* key, const void* value, void* key_cache,
                                     void* value_cache, const int64_t* slot_mapping,
                                     const float* k_scale, const float* v_scale,
                                     int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t block_size, int64_t num_blocks,
                                     pa_dtype_t src_dtype, void* stream) {
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping || !k_scale || !v_scale)
    return PA_ERR_NULL;
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_ERR_SHAPE;
  if (!supported_block(block_size) || !supported_dim(head_dim) ||
      (src_dtype != PA_DTYPE_F32 && src_dtype != PA_DTYPE_BF16))
    return PA_ERR_UNSUPPORTED;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(key_cache, 16) ||
      !aligned(value_cache, 16) || !aligned(slot_mapping, 8) || !aligned(k_scale, 4) ||
      !aligned(v_scale, 4))
    return PA_ERR_ALIGN;
  pa::ScatterFp8Args a;
  a.key = key;
  a.value = value;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.slot_mapping = slot_mapping;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.num_tokens = num_tokens;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.num_slots = num_blocks * block_size;
  a.src_bf16 = src_dtype == PA_DTYPE_BF16;
  return from_hip(pa::launch_scatter_fp8(a, static_cast<hipStream_t>(stream)));
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t max_context_len) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0 ||
      num_q_heads % num_kv_heads || !supported_block(block_size) || !supported_dim(head_dim) ||
      !supported_group(num_q_heads, num_kv_heads))
    return 0;
  return decode_geometry(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                         max_context_len)
      .bytes;
}

pa_status_t pa_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace_bytes == 0) return PA_OK;
  if (!workspace) return PA_ERR_NULL;
  if (!aligned(workspace, 16)) return PA_ERR_ALIGN;
  // only the head (the work-queue counters) has to start at zero: partials are
  // always written before they are read
  const size_t n = workspace_bytes < kDecodeHeadBytes ? workspace_bytes : kDecodeHeadBytes;
  return from_hip(pa::launch_zero_fill(workspace, n & ~(size_t)15,
                                       static_cast<hipStream_t>(stream)));
}

pa_status_t pa_decode(float* out, const void* query, const void* key_cache,
                      const void* value_cache, const int32_t* block_tables,
                      const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
                      float scale, pa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                      void* stream) {
  const bool type_ok = dtype == PA_DTYPE_F32 || dtype == PA_DTYPE_BF16;
  return decode_impl(out, query, key_cache, value_cache, nullptr, nullptr, block_tables,
                     context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     max_blocks_per_seq, num_blocks, max_context_len, scale,
                     dtype == PA_DTYPE_BF16 ? pa::KvType::BF16 : pa::KvType::F32, type_ok,
                     workspace, workspace_bytes, stream);
}

pa_status_t pa_decode_noalloc(float* out, const void* query, const void* key_cache,
                              const void* value_cache, const int32_t* block_tables,
                              const int32_t* context_lens, int32_t num_seqs,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t max_blocks_per_seq,
                              int64_t num_blocks, int32_t max_context_len, float scale,
                              pa_dtype_t dtype, void* stream) {
  const bool type_ok = dtype == PA_DTYPE_F32 || dtype == PA_DTYPE_BF16;
  return decode_impl(out, query, key_cache, value_cache, nullptr, nullptr, block_tables,
                     context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     max_blocks_per_seq, num_blocks, max_context_len, scale,
                     dtype == PA_DTYPE_BF16 ? pa::KvType::BF16 : pa::KvType::F32, type_ok,
                     nullptr, 0, stream, /*use_scratch=*/true);
}

size_t pa_decode_noalloc_max_bytes(void) { return kScratchBytes; }

size_t pa_decode_shared_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                       int32_t max_context_len, int32_t num_groups,
                                       int32_t max_group_size, int32_t max_prefix_len) {
  if (num_seqs <= 0 || num_seqs > 4096 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      max_context_len < 0 || num_q_heads % num_kv_heads || !supported_block(block_size) ||
      !supported_dim(head_dim) || !supported_group(num_q_heads, num_kv_heads) ||
      num_groups < 0 || (num_groups > 0 && (max_group_size <= 0 || max_prefix_len < 0)))
    return 0;
  const GroupSpec gs{nullptr, nullptr, num_groups, max_group_size, max_prefix_len};
  return shared_geometry(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                         max_context_len, gs)
      .bytes;
}

pa_status_t pa_decode_shared(float* out, const void* query, const void* key_cache,
                             const void* value_cache, const float* k_scale, const float* v_scale,
                             const int32_t* block_tables, const int32_t* context_lens,
                             const int32_t* cu_groups, const int32_t* prefix_lens,
                             int32_t num_groups, int32_t max_group_size, int32_t max_prefix_len,
                             int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                             int64_t num_blocks, int32_t max_context_len, float scale,
                             pa_dtype_t cache_dtype, void* workspace, size_t workspace_bytes,
                             void* stream) {
  const bool fp8 = cache_dtype == PA_DTYPE_FP8_E4M3;
  const bool type_ok = fp8 || cache_dtype == PA_DTYPE_BF16;
  const GroupSpec gs{cu_groups, prefix_lens, num_groups, max_group_size, max_prefix_len};
  return decode_impl(out, query, key_cache, value_cache, fp8 ? k_scale : nullptr,
                     fp8 ? v_scale : nullptr, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                     max_context_len, scale, fp8 ? pa::KvType::FP8 : pa::KvType::BF16, type_ok,
                     workspace, workspace_bytes, stream, false, &gs);
}

pa_status_t pa_decode_fp8(float* out, const void* query, const void* key_cache,
                          const void* value_cache, const float* k_scale, const float* v_scale,
                          const int32_t* block_tables, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                          int64_t num_blocks, int32_t max_context_len, float scale,
                          pa_dtype_t query_dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return decode_impl(out, query, key_cache, value_cache, k_scale, v_scale, block_tables,
                     context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     max_blocks_per_seq, num_blocks, max_context_len, scale, pa::KvType::FP8,
                     query_dtype == PA_DTYPE_BF16, workspace, workspace_bytes, stream);
}

size_t pa_prefill_chunk_workspace_size(int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                       int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size,
                                       int32_t max_context_len) {
  if (num_seqs <= 0 || total_q <= 0 || max_q_len <= 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || num_q_heads % num_kv_heads || max_context_len < 0 ||
      !supported_block(block_size) || !supported_dim(head_dim) ||
      !supported_group(num_q_heads, num_kv_heads))
    return 0;
  const int splits = pa::prefill_kv_splits(num_seqs, max_q_len, num_q_heads, num_kv_heads, head_dim,
                                             max_context_len);
  if (splits <= 1) return 0;
  const size_t rows = (size_t)total_q * num_q_heads * splits;
  return rows * head_dim * sizeof(float) + rows * 2 * sizeof(float);
}

pa_status_t pa_prefill_chunk(float* out, const void* query, const void* key_cache,
                             const void* value_cache, const int32_t* block_tables,
                             const int32_t* context_lens, const int32_t* cu_q_lens,
                             int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t max_blocks_per_seq,
                             int64_t num_blocks, int32_t max_context_len, float scale,
                             pa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return prefill_impl(out, query, key_cache, value_cache, nullptr, nullptr, block_tables,
                      context_lens, cu_q_lens, num_seqs, total_q, max_q_len, num_q_heads,
                      num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                      max_context_len, scale, false, dtype == PA_DTYPE_BF16, workspace,
                      workspace_bytes, stream);
}

pa_status_t pa_prefill_chunk_fp8(float* out, const void* query, const void* key_cache,
                                 const void* value_cache, const float* k_scale,
                                 const float* v_scale, const int32_t* block_tables,
                                 const int32_t* context_lens, const int32_t* cu_q_lens,
                                 int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t max_blocks_per_seq,
                                 int64_t num_blocks, int32_t max_context_len, float scale,
                                 pa_dtype_t query_dtype, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return prefill_impl(out, query, key_cache, value_cache, k_scale, v_scale, block_tables,
                      context_lens, cu_q_lens, num_seqs, total_q, max_q_len, num_q_heads,
                      num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                      max_context_len, scale, true, query_dtype == PA_DTYPE_BF16, workspace,
                      workspace_bytes, stream);
}

pa_status_t pa_copy_blocks(void* key_cache, void* value_cache, const int64_t* pairs,
                           int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int64_t num_blocks, pa_dtype_t dtype,
                           void* stream) {
  if (num_pairs < 0) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!key_cache || !value_cache || !pairs) return PA_ERR_NULL;
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_ERR_SHAPE;
  if (!supported_block(block_size) || !supported_dim(head_dim) ||
      (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16 && dtype != PA_DTYPE_FP8_E4M3))
    return PA_ERR_UNSUPPORTED;
  if (!aligned(key_cache, 16) || !aligned(value_cache, 16) || !aligned(pairs, 8))
    return PA_ERR_ALIGN;
  pa::CopyArgs a;
  a.src_key = key_cache;
  a.src_value = value_cache;
  a.dst_key = key_cache;
  a.dst_value = value_cache;
  a.pairs = pairs;
  a.num_pairs = num_pairs;
  a.src_blocks = num_blocks;
  a.dst_blocks = num_blocks;
  a.block_chunks = (int64_t)num_kv_heads * block_size * head_dim * dtype_bytes(dtype) / 16;
  return from_hip(pa::launch_copy_blocks(a, static_cast<hipStream_t>(stream)));
}

pa_status_t pa_swap_out(const void* key_cache, const void* value_cache, void* host_key,
                        void* host_value, const int64_t* pairs, int32_t num_pairs,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int64_t num_blocks, int64_t num_host_blocks, pa_dtype_t dtype,
                        void* stream) {
  return swap_impl(key_cache, value_cache, host_key, host_value, pairs, num_pairs, num_kv_heads,
                   head_dim, block_size, num_blocks, num_host_blocks, dtype, stream, true);
}

pa_status_t pa_swap_in(void* key_cache, void* value_cache, const void* host_key,
                       const void* host_value, const int64_t* pairs, int32_t num_pairs,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int64_t num_blocks, int64_t num_host_blocks, pa_dtype_t dtype,
                       void* stream) {
  return swap_impl(key_cache, value_cache, host_key, host_value, pairs, num_pairs, num_kv_heads,
                   head_dim, block_size, num_blocks, num_host_blocks, dtype, stream, false);
}

const char* pa_status_string(pa_status_t status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "invalid size or shape";
    case PA_ERR_UNSUPPORTED: return "unsupported block size, head dim, group size or dtype";
    case PA_ERR_ALIGN: return "misaligned pointer (tensors need 16 bytes, index arrays their element size)";
    case PA_ERR_WORKSPACE: return "workspace too small";
    case PA_ERR_HIP: return "HIP launch failed";
    case PA_ERR_OUT_OF_BLOCKS: return "the block pool lacks the blocks asked for";
    case PA_ERR_STATE: return "unknown or duplicate sequence id, or an object left unusable";
    case PA_ERR_NOMEM: return "host memory could not be allocated";
  }
  return "unknown status";
}

int32_t pa_version(void) { return 100; }

}  // extern "C"
