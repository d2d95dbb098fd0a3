// Chunked-prefill attention against the paged cache, on the gfx950 matrix
// cores (v_mfma_f32_16x16x32_bf16).
//
// What is computed (How vLLM gets real throughput on H100s, "Decode is a
// memory problem, not a math problem": prefill is a dense matrix product;
// vLLM architecture, memory and benchmarks deep dive, "Hardware-level
// optimizations": long prompts are cut into chunks that run against the
// cache between decode steps): chunk row i of a sequence with context n and
// chunk length L sits at position n - L + i and attends keys 0 .. n - L + i,
// whose K/V are gathered through the block table.
//
// Work decomposition. A workgroup owns (sequence, KV head, 16*R query rows,
// context split); its NW = max(4, G) waves each take 16 query rows of one
// query head of the group, so every K/V tile staged in LDS serves all G heads.
// Per 32-key tile and wave:
//   S^T[32 x 16] = K[32 x D] . Q^T[D x 16]   A = K rows (LDS, chunk-swizzled),
//                                             B = Q^T (this lane's query row,
//                                             held in registers)
//   O^T[D x 16] += V^T[D x 32] . P^T[32 x 16] A = V^T (LDS, transposed when the
//                                             tile is staged), B = P^T (this
//                                             lane's own softmax weights)
// With the accumulator layout of the 16x16 MFMA (lane l holds rows
// 4*(l/16)+i of column l%16) both S^T and O^T keep a query row in the lanes
// l%16 == row, so the online softmax is lane-local up to a 4-lane reduction.
// P enters the PV product as two BF16 terms (hi + lo, 16 significant bits)
// and the running sum uses the same split weights. The B operand of PV takes
// the 8 weights a lane holds for
// keys {4q..4q+3, 16+4q..16+4q+3} (q = l/16); V^T columns are stored in that
// same key order, so the contraction pairs every weight with its key's row.

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kKeyTile = 32;      // keys per staged tile
constexpr int kVtStride = 40;     // bf16 per V^T row in LDS (32 keys + 8 pad: 80-byte rows)

// LDS column of key k (0..31) in a V^T row: keys 4q..4q+3 -> 8q..8q+3,
// keys 16+4q..16+4q+3 -> 8q+4..8q+7.
__device__ __forceinline__ int vt_slot(int k) {
  return (k < 16) ? (8 * (k >> 2) + (k & 3)) : (8 * ((k - 16) >> 2) + 4 + (k & 3));
}

__device__ __forceinline__ uint32_t pack_lo(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);  // lo16(x) | lo16(y) << 16
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);  // hi16(x) | hi16(y) << 16
}

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  return (uint32_t)__builtin_bit_cast(unsigned short, static_cast<__bf16>(f));
}

template <int D, int G>
struct PrefillShape {
  static constexpr int NW = G >= 4 ? G : 4;       // waves per workgroup
  static constexpr int RT = NW / G;               // 16-row sub-tiles per workgroup
  static constexpr int ROWS = 16 * RT;            // query rows per workgroup
  static constexpr int NT = NW * kWave;           // threads
  static constexpr int DCH = D / 8;               // 16-byte chunks per K/V row
  static constexpr int SWZ = (DCH < 16 ? DCH : 16) - 1;  // K chunk swizzle mask
  static constexpr int KSTEPS = D / 32;           // MFMA k-steps of QK^T
  static constexpr int DTILES = D / 16;           // 16-row tiles of O^T
  static constexpr int KCHUNKS = kKeyTile * DCH;  // K chunks per tile
  static constexpr int VJOBS = (kKeyTile / 4) * (D / 8);  // 4-key x 8-dim V jobs
};

template <int D, int G>
__global__ __launch_bounds__((PrefillShape<D, G>::NT)) void prefill_kernel(PrefillArgs a) {
  using S = PrefillShape<D, G>;
  constexpr int DCH = S::DCH;
  __shared__ uint4 k_lds[kKeyTile * DCH];                   // swizzled K rows
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * kVtStride];  // V^T

  const int row_tile = blockIdx.x, kvh = blockIdx.y;
  const int seq = blockIdx.z / a.kv_splits, split = blockIdx.z % a.kv_splits;
  const int q0 = a.cu_q_lens[seq];
  const int L = a.cu_q_lens[seq + 1] - q0;
  const int r0 = row_tile * S::ROWS;
  if (r0 >= L) return;
  int n = a.context_lens[seq];
  n = n > a.ctx_limit ? a.ctx_limit : n;
  if (L > n) return;  // malformed chunk (longer than its context): nothing defined to compute
  const int bs_log2 = a.block_size_log2;
  const int bs = 1 << bs_log2;
  const int base_pos = n - L;  // position of chunk row 0

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int lrow = lane % 16, lq = lane / 16;
  const int head = kvh * G + wave % G;
  const int rsub = wave / G;
  const int my_row = r0 + rsub * 16 + lrow;          // chunk row of this lane's query
  const int qrow = my_row < L ? my_row : L - 1;       // clamp padding rows (not written)

  // Q^T operand: query row my_row, dims 32*ks + 8*lq .. +8
  bf16x8_t qop[S::KSTEPS];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(a.query) +
                      ((int64_t)(q0 + qrow) * a.num_q_heads + head) * DCH;
#pragma unroll
    for (int ks = 0; ks < S::KSTEPS; ++ks) qop[ks] = __builtin_bit_cast(bf16x8_t, qp[4 * ks + lq]);
  }

  // Key range of this split: keys visible to some row of the workgroup.
  const int last_row = min(r0 + S::ROWS, L) - 1;
  const int kmax = base_pos + last_row + 1;
  const int ntiles = (kmax + kKeyTile - 1) / kKeyTile;
  const int per_split = (ntiles + a.kv_splits - 1) / a.kv_splits;
  const int kt_begin = split * per_split;
  const int kt_end = min(ntiles, kt_begin + per_split);

  const uint4* kcache = reinterpret_cast<const uint4*>(a.key_cache);
  const uint4* vcache = reinterpret_cast<const uint4*>(a.value_cache);
  const int64_t block_stride = (int64_t)a.num_kv_heads * bs * DCH;
  const int64_t head_off = (int64_t)kvh * bs * DCH;
  const int32_t* bt = a.block_tables + (int64_t)seq * a.max_blocks_per_seq;

  // Global chunk offset of key k's row, or -1 if the key is past the context
  // or its table entry is outside the pool.
  auto row_offset = [&](int k) -> int64_t {
    if (k >= n) return -1;
    const int e = bt[k >> bs_log2];
    if (e < 0 || (int64_t)e >= a.num_blocks) return -1;
    return (int64_t)e * block_stride + head_off + (int64_t)(k & (bs - 1)) * DCH;
  };

  f32x4_t acc[S::DTILES];
#pragma unroll
  for (int i = 0; i < S::DTILES; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // this lane's query row, log2 units
  float l_part = 0.f;       // sum of this lane's rounded weights

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int key0 = kt * kKeyTile;
    __syncthreads();  // previous tile fully consumed
    // ---- stage K (row-chunk swizzle: chunk c of row r lives at c ^ (r & SWZ),
    // so the 16 rows one MFMA operand read touches fall in distinct banks)
    for (int idx = tid; idx < S::KCHUNKS; idx += S::NT) {
      const int r = idx / DCH, c = idx % DCH;
      const int64_t off = row_offset(key0 + r);
      const uint4 v = off >= 0 ? kcache[off + c] : make_uint4(0, 0, 0, 0);
      k_lds[r * DCH + (c ^ (r & S::SWZ))] = v;
    }
    // ---- stage V^T: each job transposes 4 keys x 8 dims
    for (int job = tid; job < S::VJOBS; job += S::NT) {
      const int kg = job % (kKeyTile / 4), dg = job / (kKeyTile / 4);
      uint4 rows[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t off = row_offset(key0 + 4 * kg + r);
        rows[r] = off >= 0 ? vcache[off + dg] : make_uint4(0, 0, 0, 0);
      }
      const int slot = vt_slot(4 * kg);
      const uint32_t* w0 = &rows[0].x;
      const uint32_t* w1 = &rows[1].x;
      const uint32_t* w2 = &rows[2].x;
      const uint32_t* w3 = &rows[3].x;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint2 even, odd;  // dims 8*dg + 2c and 8*dg + 2c + 1, keys 4kg..4kg+3
        even.x = pack_lo(w0[c], w1[c]);
        even.y = pack_lo(w2[c], w3[c]);
        odd.x = pack_hi(w0[c], w1[c]);
        odd.y = pack_hi(w2[c], w3[c]);
        const int d = 8 * dg + 2 * c;
        *reinterpret_cast<uint2*>(&vt_lds[d * kVtStride + slot]) = even;
        *reinterpret_cast<uint2*>(&vt_lds[(d + 1) * kVtStride + slot]) = odd;
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T for keys key0..key0+31 (two 16-key halves)
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < S::KSTEPS; ++ks) {
      const int c = 4 * ks + lq;
      const bf16x8_t k0 =
          __builtin_bit_cast(bf16x8_t, k_lds[lrow * DCH + (c ^ (lrow & S::SWZ))]);
      const bf16x8_t k1 =
          __builtin_bit_cast(bf16x8_t, k_lds[(16 + lrow) * DCH + (c ^ ((16 + lrow) & S::SWZ))]);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qop[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qop[ks], s1, 0, 0, 0);
    }

    // ---- scale and causal / context mask (lane: keys 4lq+i and 16+4lq+i)
    float sv[8];
    const int limit = base_pos + my_row;  // last key this row may see
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = s0[i] * a.scale_log2;
      sv[4 + i] = s1[i] * a.scale_log2;
    }
    const bool diag = key0 + kKeyTile - 1 > base_pos + r0 || key0 + kKeyTile > n;
    if (diag) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ka = key0 + 4 * lq + i, kb = key0 + 16 + 4 * lq + i;
        sv[i] = (ka <= limit && ka < n) ? sv[i] : -INFINITY;
        sv[4 + i] = (kb <= limit && kb < n) ? sv[4 + i] : -INFINITY;
      }
    }

    // ---- online softmax over this lane's query row
    float mx = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
    mx = fmaxf(mx, xor_lane<16>(mx));
    mx = fmaxf(mx, xor_lane<32>(mx));
    const float m_new = fmaxf(m_run, mx);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < S::DTILES; ++i) acc[i] *= alpha;
      m_run = m_new;
    }
    // Each weight p is carried as p_hi + p_lo, both BF16 (p_hi = RNE(p),
    // p_lo = RNE(p - p_hi)): 16 significant bits instead of 8, so the PV
    // product on the BF16 matrix cores keeps the weights' float32 accuracy to
    // about 2^-17 relative. The running sum uses the same p_hi + p_lo.
    const float moff = m_run == -INFINITY ? 0.f : m_run;
    uint32_t ph[8], pl[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float pf = fast_exp2(sv[i] - moff);
      ph[i] = bf16_bits_rne(pf);
      const float hi = __uint_as_float(ph[i] << 16);
      pl[i] = bf16_bits_rne(pf - hi);
      l_part += hi + __uint_as_float(pl[i] << 16);
    }
    uint4 wh, wl;
    wh.x = ph[0] | (ph[1] << 16);
    wh.y = ph[2] | (ph[3] << 16);
    wh.z = ph[4] | (ph[5] << 16);
    wh.w = ph[6] | (ph[7] << 16);
    wl.x = pl[0] | (pl[1] << 16);
    wl.y = pl[2] | (pl[3] << 16);
    wl.z = pl[4] | (pl[5] << 16);
    wl.w = pl[6] | (pl[7] << 16);
    const bf16x8_t pop_hi = __builtin_bit_cast(bf16x8_t, wh);
    const bf16x8_t pop_lo = __builtin_bit_cast(bf16x8_t, wl);

    // ---- O^T += V^T (P_hi + P_lo)^T
#pragma unroll
    for (int dt = 0; dt < S::DTILES; ++dt) {
      const bf16x8_t vop = __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const uint4*>(&vt_lds[(16 * dt + lrow) * kVtStride + 8 * lq]));
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop_hi, acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop_lo, acc[dt], 0, 0, 0);
    }
  }

  // ---- row totals and output
  float l_row = l_part + xor_lane<16>(l_part);
  l_row += xor_lane<32>(l_row);
  if (my_row >= L) return;
  const int64_t orow = (int64_t)(q0 + my_row) * a.num_q_heads + head;
  if (a.kv_splits == 1) {
    const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
    float4* o = reinterpret_cast<float4*>(a.out + orow * D);
#pragma unroll
    for (int dt = 0; dt < S::DTILES; ++dt)
      o[4 * dt + lq] = make_float4(acc[dt][0] * inv, acc[dt][1] * inv, acc[dt][2] * inv,
                                   acc[dt][3] * inv);
  } else {
    const int64_t slot = orow * a.kv_splits + split;
    const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
    float4* o = reinterpret_cast<float4*>(a.part_o + slot * D);
#pragma unroll
    for (int dt = 0; dt < S::DTILES; ++dt)
      o[4 * dt + lq] = make_float4(acc[dt][0] * inv, acc[dt][1] * inv, acc[dt][2] * inv,
                                   acc[dt][3] * inv);
    if (lq == 0) {
      a.part_ml[2 * slot] = m_run;
      a.part_ml[2 * slot + 1] = l_row;
    }
  }
}

// Merge of the context splits of one (row, query head):
// out = sum_s w_s o_s / sum_s w_s with w_s = l_s * 2^(m_s - max_s m_s).
template <int D>
__global__ __launch_bounds__(kWave) void prefill_merge_kernel(PrefillArgs a) {
  constexpr int PER = D / kWave;
  const int h = blockIdx.x, row = blockIdx.y;
  const int64_t orow = (int64_t)row * a.num_q_heads + h;
  const float* ml = a.part_ml + 2 * orow * a.kv_splits;
  float M = -INFINITY;
  for (int s = 0; s < a.kv_splits; ++s) M = fmaxf(M, ml[2 * s]);
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  float L = 0.f;
  const float* po = a.part_o + orow * a.kv_splits * D + threadIdx.x * PER;
  for (int s = 0; s < a.kv_splits; ++s) {
    const float l = ml[2 * s + 1];
    if (l == 0.f) continue;  // a split that saw no key of this row
    const float w = l * fast_exp2(ml[2 * s] - M);
    L += w;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = __builtin_fmaf(w, po[(int64_t)s * D + e], o[e]);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float* out = a.out + orow * D + threadIdx.x * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) out[e] = o[e] * inv;
}

// ---------------------------------------------------------------------------
// Host side.

int prefill_kv_splits(int num_seqs, int max_q_len, int num_kv_heads, int max_context_len) {
  // Split the keys of each row tile until the launch has about two
  // workgroups per CU, keeping at least 8 key tiles per split.
  const int rows = 16;  // the smallest row tile (group size 4 or 8)
  const int64_t wgs = (int64_t)num_seqs * num_kv_heads * ((max_q_len + rows - 1) / rows);
  int splits = 1;
  while (splits < 8 && wgs * splits < 512 &&
         (max_context_len / kKeyTile) / (2 * splits) >= 8)
    splits *= 2;
  return splits;
}

template <int D, int G>
static hipError_t launch_pf(const PrefillArgs& a, hipStream_t stream) {
  using S = PrefillShape<D, G>;
  dim3 grid((a.max_q_len + S::ROWS - 1) / S::ROWS, a.num_kv_heads, a.num_seqs * a.kv_splits);
  hipLaunchKernelGGL((prefill_kernel<D, G>), grid, dim3(S::NT), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.kv_splits == 1) return err;
  hipLaunchKernelGGL((prefill_merge_kernel<D>), dim3(a.num_q_heads, a.total_q), dim3(kWave), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_pg(const PrefillArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_pf<D, 1>(a, stream);
    case 2: return launch_pf<D, 2>(a, stream);
    case 4: return launch_pf<D, 4>(a, stream);
    case 8: return launch_pf<D, 8>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: return launch_pg<64>(a, stream);
    case 128: return launch_pg<128>(a, stream);
    case 256: return launch_pg<256>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
