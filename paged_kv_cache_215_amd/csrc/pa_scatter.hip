// Cache-write scatter for gfx950: token t's K and V rows go to slot
// slot_mapping[t] of the paged cache (How vLLM gets real throughput on H100s,
// "PagedAttention borrows from operating systems": blocks fill as tokens
// arrive). For a cache of the source's own type it is a pure bit copy in
// 16-byte vectors, one thread per 16-byte chunk of a (token, KV head) row, K
// and V handled by the same thread; for an FP8 cache each thread quantizes 16
// elements into one 16-byte chunk of codes.

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
    // the rows are read before the slot is tested, so that their loads and
    // the slot's are in flight together
    const uint4 kv = key[i];
    const uint4 vv = value[i];
    if (slot < 0 || slot >= a.num_slots) continue;   // skipped or out of range
    const int64_t blk = slot / a.block_size;
    const int64_t off = slot - blk * a.block_size;
    const int64_t head = rest / a.row_chunks;
    const int64_t chunk = rest - head * a.row_chunks;
    const int64_t dst = ((blk * a.num_kv_heads + head) * a.block_size + off) * a.row_chunks + chunk;
    kc[dst] = kv;
    vc[dst] = vv;
  }
}

// ---------------------------------------------------------------------------
// FP8 (E4M3) cache write. The pages name FP8 as the lever that doubles the
// effective bandwidth (vLLM architecture, memory and benchmarks deep dive,
// "Hardware-level optimizations") without fixing a format; the one used is
// the OCP E4M3 encoding (bias 7, no infinities, S.1111.111 = NaN, largest
// magnitude 448), with one float32 scale per KV head for K and one for V.
// Code = E4M3(x / s): x widened to float32, divided by s (IEEE float32
// division), rounded to nearest with ties to even, saturated at +-448; NaN
// stays NaN with its sign.

__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;  // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;  // |y| >= 448, infinity included
  if (a >= 0x3c800000u) {
    // normal range (|y| >= 2^-6): round the 23 mantissa bits to 3, ties to
    // even; a carry moves into the exponent, and the float32 exponent bias
    // 127 becomes the E4M3 bias 7
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    return sign | ((r >> 20) - (120u << 3));
  }
  // subnormal range: multiples of 2^-9; the scaling by 2^9 is exact and
  // rint rounds ties to even (8 * 2^-9 = 2^-6 is code 0x08)
  return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.f);
}

// Four float32 values -> four codes packed little-endian in one word.
__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d, float s) {
  return e4m3_code(__fdiv_rn(a, s)) | (e4m3_code(__fdiv_rn(b, s)) << 8) |
         (e4m3_code(__fdiv_rn(c, s)) << 16) | (e4m3_code(__fdiv_rn(d, s)) << 24);
}

// 4 source elements starting at element e of a row -> 4 codes in one word.
__device__ __forceinline__ uint32_t quantize4(const void* src, int64_t e, bool bf16, float s) {
  if (bf16) {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(src) + e);
    return pack4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y), s);
  }
  const float4 w = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + e);
  return pack4(w.x, w.y, w.z, w.w, s);
}

// One thread per 4 codes of a (token, KV head) row: the first half of the
// threads write K, the second half V. (Each code takes an IEEE division, so
// a thread's work is a serial chain; short chains on many threads finish
// sooner than 32 divisions on each of a few.)
__global__ __launch_bounds__(256) void scatter_fp8_kernel(ScatterFp8Args a) {
  const int row_words = a.head_dim / 4;
  const int64_t per_token = (int64_t)a.num_kv_heads * row_words;
  const int64_t total = (int64_t)a.num_tokens * per_token;  // words per cache
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < 2 * total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const bool is_v = i >= total;
    const int64_t j = is_v ? i - total : i;
    const int64_t t = j / per_token;
    const int64_t rest = j - t * per_token;  // head * row_words + word
    const int64_t slot = a.slot_mapping[t];
    const int64_t head = rest / row_words;
    const int64_t word = rest - head * row_words;
    // the codes are formed before the slot is tested, so that the source
    // loads and the slot's are in flight together
    const uint32_t codes = quantize4(is_v ? a.value : a.key, j * 4, a.src_bf16,
                                     is_v ? a.v_scale[head] : a.k_scale[head]);
    if (slot < 0 || slot >= a.num_slots) continue;  // skipped or out of range
    const int64_t blk = slot / a.block_size;
    const int64_t off = slot - blk * a.block_size;
    const int64_t dst = ((blk * a.num_kv_heads + head) * a.block_size + off) * row_words + word;
    static_cast<uint32_t*>(is_v ? a.value_cache : a.key_cache)[dst] = codes;
  }
}

hipError_t launch_scatter_fp8(const ScatterFp8Args& a, hipStream_t stream) {
  const int64_t total = 2 * (int64_t)a.num_tokens * a.num_kv_heads * (a.head_dim / 4);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65535) blocks = 65535;
  hipLaunchKernelGGL(scatter_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_scatter(const ScatterArgs& a, hipStream_t stream) {
  const int64_t total = (int64_t)a.num_tokens * a.num_kv_heads * a.row_chunks;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65535) blocks = 65535;
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
