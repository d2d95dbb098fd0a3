// Cache-write scatter for gfx950: token t's K and V rows go to slot
// slot_mapping[t] of the paged cache (How vLLM gets real throughput on H100s,
// "PagedAttention borrows from operating systems": blocks fill as tokens
// arrive). A pure bit copy in 16-byte vectors; one thread per 16-byte chunk of
// a (token, KV head) row, K and V handled by the same thread.

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

__global__ __launch_bounds__(256) void scatter_kernel(ScatterArgs a) {
  const int64_t per_token = (int64_t)a.num_kv_heads * a.row_chunks;
  const int64_t total = (int64_t)a.num_tokens * per_token;
  const uint4* key = reinterpret_cast<const uint4*>(a.key);
  const uint4* value = reinterpret_cast<const uint4*>(a.value);
  uint4* kc = reinterpret_cast<uint4*>(a.key_cache);
  uint4* vc = reinterpret_cast<uint4*>(a.value_cache);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / per_token;
    const int64_t rest = i - t * per_token;          // head * row_chunks + chunk
    const int64_t slot = a.slot_mapping[t];
    if (slot < 0 || slot >= a.num_slots) continue;   // skipped or out of range
    const int64_t blk = slot / a.block_size;
    const int64_t off = slot - blk * a.block_size;
    const int64_t head = rest / a.row_chunks;
    const int64_t chunk = rest - head * a.row_chunks;
    const int64_t dst = ((blk * a.num_kv_heads + head) * a.block_size + off) * a.row_chunks + chunk;
    kc[dst] = key[i];
    vc[dst] = value[i];
  }
}

hipError_t launch_scatter(const ScatterArgs& a, hipStream_t stream) {
  const int64_t total = (int64_t)a.num_tokens * a.num_kv_heads * a.row_chunks;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65535) blocks = 65535;
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
