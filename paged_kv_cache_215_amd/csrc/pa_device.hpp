// Device-side helpers shared by the paged-attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kWave = 64;

// Element-type tags of the KV cache. The cache stores binary32, bfloat16 (the
// top half of a binary32) or FP8 E4M3 codes, all moved through 16-byte
// vectors; Query is the element type of the queries that attend to it.
struct F32 {
  static constexpr int kBytes = 4;
  using Query = F32;
};
struct BF16 {
  static constexpr int kBytes = 2;
  using Query = BF16;
};
struct FP8 {
  static constexpr int kBytes = 1;
  using Query = BF16;
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

// 16-byte load marked nontemporal (global_load_dwordx4 ... nt): for data read
// exactly once per launch, such as the K/V rows of a decode step, so that the
// stream does not displace reusable lines in L2 and the Infinity Cache.
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
// The same for an 8-byte chunk (global_load_dwordx2 ... nt).
__device__ __forceinline__ uint2 load_stream(const uint2* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}
// The load of a K/V chunk a work unit uses: nontemporal (each byte is read
// once), or ordinary when the blocks are shared between sequences (rollouts
// of one prompt), where the caches' reuse across work units matters. The
// choice is a template argument: two forms in one function body get merged
// by the compiler into the ordinary one.
template <bool Keep, typename C>
__device__ __forceinline__ C load_kv(const C* p) {
  if constexpr (Keep) {
    return *p;
  } else {
    return load_stream(p);
  }
}
__device__ __forceinline__ void zero_chunk(uint4& v) { v = make_uint4(0, 0, 0, 0); }
__device__ __forceinline__ void zero_chunk(uint2& v) { v = make_uint2(0, 0); }

// Widen the low / high bfloat16 of a packed pair: a bfloat16 is the high half
// of the binary32 with the same value, so widening is a shift or a mask.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// a.lo*b.lo + a.hi*b.hi + c on packed bfloat16 pairs (v_dot2_f32_bf16): the
// products of two bfloat16 are exact in binary32 and the sum accumulates in
// binary32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Dot product of one 16-byte chunk of K with the matching chunk of q.
__device__ __forceinline__ float dot_chunk(BF16, const uint4& k, const uint4& q, float c) {
  c = dot2_bf16(k.x, q.x, c);
  c = dot2_bf16(k.y, q.y, c);
  c = dot2_bf16(k.z, q.z, c);
  c = dot2_bf16(k.w, q.w, c);
  return c;
}
__device__ __forceinline__ float dot_chunk(F32, const uint4& k, const uint4& q, float c) {
  c = __builtin_fmaf(__uint_as_float(k.x), __uint_as_float(q.x), c);
  c = __builtin_fmaf(__uint_as_float(k.y), __uint_as_float(q.y), c);
  c = __builtin_fmaf(__uint_as_float(k.z), __uint_as_float(q.z), c);
  c = __builtin_fmaf(__uint_as_float(k.w), __uint_as_float(q.w), c);
  return c;
}

// A 16-byte K chunk in the query's element type: BF16 and binary32 chunks
// are used as they are; 16 E4M3 codes become 16 bfloat16 (two chunks) with
// the hardware conversion (v_cvt_scalef32_pk_bf16_fp8 at scale 1), which is
// exact: every E4M3 value is a bfloat16 value.
template <bool Hi>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, Hi));
}
__device__ __forceinline__ void k_as_query(F32, const uint4& k, uint4* out) { out[0] = k; }
__device__ __forceinline__ void k_as_query(BF16, const uint4& k, uint4* out) { out[0] = k; }
__device__ __forceinline__ void k_as_query(FP8, const uint4& k, uint4* out) {
  out[0] = make_uint4(fp8x2_to_bf16x2<false>(k.x), fp8x2_to_bf16x2<true>(k.x),
                      fp8x2_to_bf16x2<false>(k.y), fp8x2_to_bf16x2<true>(k.y));
  out[1] = make_uint4(fp8x2_to_bf16x2<false>(k.z), fp8x2_to_bf16x2<true>(k.z),
                      fp8x2_to_bf16x2<false>(k.w), fp8x2_to_bf16x2<true>(k.w));
}

// Widen one 16-byte chunk to binary32 (16 E4M3, 8 bfloat16 or 4 binary32
// values), or an 8-byte chunk of 8 E4M3 codes. E4M3 uses v_cvt_pk_f32_fp8,
// exact for every code.
__device__ __forceinline__ void widen_chunk(BF16, const uint4& v, float* out) {
  out[0] = bf16_lo(v.x); out[1] = bf16_hi(v.x);
  out[2] = bf16_lo(v.y); out[3] = bf16_hi(v.y);
  out[4] = bf16_lo(v.z); out[5] = bf16_hi(v.z);
  out[6] = bf16_lo(v.w); out[7] = bf16_hi(v.w);
}
__device__ __forceinline__ void widen_chunk(FP8, const uint4& v, float* out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
    out[4 * i] = a[0]; out[4 * i + 1] = a[1];
    out[4 * i + 2] = b[0]; out[4 * i + 3] = b[1];
  }
}
__device__ __forceinline__ void widen_chunk(FP8, const uint2& v, float* out) {
  const uint32_t w[2] = {v.x, v.y};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
    out[4 * i] = a[0]; out[4 * i + 1] = a[1];
    out[4 * i + 2] = b[0]; out[4 * i + 3] = b[1];
  }
}
__device__ __forceinline__ void widen_chunk(F32, const uint4& v, float* out) {
  out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
  out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
}

// ---------------------------------------------------------------------------
// Cross-lane exchange. xor_lane<M>(x) returns x from lane (lane ^ M).
//   M = 1, 2 : DPP quad permutation (VALU, no LDS traffic)
//   M = 8    : DPP row rotate by 8 within a 16-lane row, which is lane ^ 8
//   M = 4, 16: ds_swizzle in xor mode (within 32 lanes)
//   M = 32   : ds_bpermute
template <int M>
__device__ __forceinline__ float xor_lane(float x) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "mask");
  int v = __float_as_int(x);
  if constexpr (M == 1) {
    v = __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    v = __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  } else if constexpr (M == 8) {
    v = __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else if constexpr (M == 4 || M == 16) {
    v = __builtin_amdgcn_ds_swizzle(v, 0x1F | (M << 10));           // and 0x1F, xor M
  } else {
    v = __builtin_amdgcn_ds_bpermute((int)((__lane_id() ^ 32u) << 2), v);
  }
  return __int_as_float(v);
}

// Partner for the transposing reduction at lane bit log2(M): any involution
// that flips bit log2(M) and keeps every higher bit works there, because the
// lower bits are resolved afterwards. Bit 2 uses the DPP half-row mirror
// (lane ^ 7), which stays on the VALU.
template <int M>
__device__ __forceinline__ float reduce_partner(float x) {
  if constexpr (M == 4) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
  } else {
    return xor_lane<M>(x);
  }
}

// Lane exchange across 16- or 32-lane halves on the VALU
// (v_permlane16_swap / v_permlane32_swap, gfx950). swap_halves<M>(a, b)
// returns {r0, r1}: a lane with bit M clear gets r0 = a[l], r1 = a[l ^ M];
// a lane with bit M set gets r0 = b[l ^ M], r1 = b[l] (checked on the
// hardware). So with a = b = x every lane holds the pair {x[l], x[l ^ M]},
// and with a = the lower lanes' kept value / the upper lanes' sent value, r0 +
// r1 is a lane's kept value plus its partner's sent one.
template <int M>
__device__ __forceinline__ void swap_halves(float a, float b, float& r0, float& r1) {
  static_assert(M == 16 || M == 32, "half-wave swaps only");
  if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    r0 = __uint_as_float(r[0]);
    r1 = __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    r0 = __uint_as_float(r[0]);
    r1 = __uint_as_float(r[1]);
  }
}

// max / sum of x over lanes l and l ^ M.
template <int M>
__device__ __forceinline__ float pair_max(float x) {
  if constexpr (M == 16 || M == 32) {
    float r0, r1;
    swap_halves<M>(x, x, r0, r1);
    return fmaxf(r0, r1);
  } else {
    return fmaxf(x, xor_lane<M>(x));
  }
}
template <int M>
__device__ __forceinline__ float pair_sum(float x) {
  if constexpr (M == 16 || M == 32) {
    float r0, r1;
    swap_halves<M>(x, x, r0, r1);
    return r0 + r1;
  } else {
    return x + xor_lane<M>(x);
  }
}

__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa
