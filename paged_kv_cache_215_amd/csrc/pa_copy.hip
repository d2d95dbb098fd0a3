// Whole-block copies of the paged KV cache on gfx950.
//
// Copy-on-write: a block shared by sequences forked from one prompt is
// duplicated when one of them writes into it (Dissecting vLLM,
// "PagedAttention: Virtual Memory for KV Cache"; How vLLM gets real
// throughput on H100s, "PagedAttention borrows from operating systems").
// Swapping: a preempted sequence's blocks move to host memory and back
// (Dissecting vLLM, "Continuous Batching: Breaking the Sequence Barrier");
// the host pool is pinned memory the kernel reads or writes directly, so a
// batch of scattered blocks moves in one launch.
//
// One block of one cache is num_kv_heads * block_size * head_dim elements,
// contiguous, so a copy is a flat 16-byte-vector copy, K and V by the same
// thread.

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

// grid.x walks the 16-byte chunks of a block, grid.y the pairs.
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyArgs a) {
  const int64_t p = blockIdx.y;
  const int64_t src = a.pairs[2 * p], dst = a.pairs[2 * p + 1];
  if (src < 0 || src >= a.src_blocks || dst < 0 || dst >= a.dst_blocks) return;
  const int64_t n = a.block_chunks;
  const uint4* ks = reinterpret_cast<const uint4*>(a.src_key) + src * n;
  const uint4* vs = reinterpret_cast<const uint4*>(a.src_value) + src * n;
  uint4* kd = reinterpret_cast<uint4*>(a.dst_key) + dst * n;
  uint4* vd = reinterpret_cast<uint4*>(a.dst_value) + dst * n;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n; c += (int64_t)gridDim.x * 256) {
    kd[c] = ks[c];
    vd[c] = vs[c];
  }
}

hipError_t launch_copy_blocks(const CopyArgs& a_in, hipStream_t stream) {
  const int64_t per_block_wgs = (a_in.block_chunks + 255) / 256;
  const unsigned gx = (unsigned)(per_block_wgs < 64 ? per_block_wgs : 64);
  constexpr int64_t kMaxY = 65535;  // grid.y limit: pairs go in launches of at most this many
  for (int64_t p0 = 0; p0 < a_in.num_pairs; p0 += kMaxY) {
    CopyArgs a = a_in;
    a.pairs = a_in.pairs + 2 * p0;
    const int64_t np = a_in.num_pairs - p0 < kMaxY ? a_in.num_pairs - p0 : kMaxY;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(gx, (unsigned)np), dim3(256), 0, stream, a);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace pa
