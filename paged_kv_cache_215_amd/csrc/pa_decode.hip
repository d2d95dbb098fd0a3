// Paged decode attention for gfx950: split-context partition kernel plus a
// separate merge kernel.
//
// What is computed (How vLLM gets real throughput on H100s, "Decode is a
// memory problem, not a math problem" and "PagedAttention borrows from
// operating systems"; Dissecting vLLM, "PagedAttention: Virtual Memory for KV
// Cache"): for each sequence b and query head h, softmax-weighted sum of the V
// rows of KV head h / G over the sequence's n logical positions, the K/V rows
// being gathered through the block table at run time.
//
// Work decomposition. A workgroup (4 waves) owns one (sequence, KV head,
// context partition of P tokens). Its waves take interleaved 16-token tiles of
// the partition; a tile never crosses a physical block (block sizes 16, 32).
// Each wave keeps an online softmax (running max m, running sum l, unnormalised
// accumulator) per query head of the GQA group, the 4 waves are merged in LDS,
// and the workgroup writes one normalised partial (o, m, l) per query head. A
// sequence that needs one partition writes its output directly; otherwise the
// merge kernel combines the partials. Decode moves ~4 FLOP per byte of KV, far
// below the matrix-core ridge, so the contractions stay on the VALU.
//
// Register layout of a 16-token tile (per wave):
//   K: each row (token) is spread over KL lanes that each hold KCH 16-byte
//      chunks; 64/KL rows per load instruction, so a load instruction reads
//      whole 128-byte segments. Each lane multiplies its chunks with the
//      matching q chunks of all G heads (v_dot2_f32_bf16 for BF16), leaving
//      NGK*G partial dots that a transposing butterfly over the KL lanes turns
//      into one finished score per lane (G heads x 16 tokens spread over the
//      wave) without any LDS traffic.
//   V: each row is spread over RC lanes (one 16-byte chunk each, a fully
//      coalesced row read); every lane accumulates its head-dim slice for all
//      G heads from the same registers, so V is read once per KV head however
//      many query heads share it. Softmax weights reach the V lanes through a
//      64-float LDS slot per wave.

#include "pa_device.hpp"
#include "pa_internal.hpp"

#include <type_traits>

namespace pa {

constexpr int kTile = 16;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;

constexpr int choose_k_lanes(int row_chunks, int group) {
  // Enough lanes per K row that the q chunks held per lane (group * KCH
  // 16-byte chunks) fit in 32 VGPRs, at least 4 so that a tile holds whole
  // load groups.
  int need = group * row_chunks / 8;
  if (need < 4) need = 4;
  int kl = 4;
  while (kl < need) kl *= 2;
  return kl > row_chunks ? row_chunks : kl;
}

template <typename T, int D, int G>
struct DecodeShape {
  static constexpr int E = 16 / T::kBytes;          // elements per 16-byte chunk
  static constexpr int RC = D * T::kBytes / 16;     // chunks per row
  static constexpr int KL = choose_k_lanes(RC, G);  // lanes per K row
  static constexpr int KCH = RC / KL;               // chunks per lane per K row
  static constexpr int RK = kWave / KL;             // K rows per load instruction
  static constexpr int NGK = kTile / RK;            // K load groups per tile
  static constexpr int NV = NGK * G;                // partial dots per lane
  static constexpr int NVF = NV >= KL ? NV / KL : 1;  // finished scores per lane
  static constexpr int REP = NV >= KL ? 1 : KL / NV;  // lanes holding the same score
  static constexpr int VL = RC;                     // lanes per V row
  static constexpr int RV = kWave / VL;             // V rows per load instruction
  static constexpr int NGV = kTile / RV;            // V load groups per tile
  static constexpr int NHS = NVF < G ? NVF : G;     // distinct heads among a lane's scores
  static_assert(RC <= kWave && RK <= kTile && RV <= kTile, "tile shape");
  static_assert((KL & (KL - 1)) == 0 && KL >= 4, "K lanes");

  // Score slot j of lane l after the transposing reduction holds partial-dot
  // index i = grp * G + g (grp = K load group, g = head in the group).
  static constexpr int slot_index(int l, int j) {
    return NV >= KL ? NVF * (l % KL) + j : (l % KL) / REP;
  }
  static constexpr int slot_head(int l, int j) { return slot_index(l, j) % G; }
  static constexpr int slot_token(int l, int j) { return (slot_index(l, j) / G) * RK + l / KL; }
  // Lane bit b is head-neutral when flipping it never changes a slot's head.
  static constexpr bool bit_neutral(int b) {
    for (int l = 0; l < kWave; ++l)
      for (int j = 0; j < NVF; ++j)
        if (slot_head(l, j) != slot_head(l ^ (1 << b), j)) return false;
    return true;
  }
  // A lane and slot that hold head g (for wave-uniform broadcasts).
  static constexpr int rep_lane(int g) {
    for (int l = 0; l < kWave; ++l)
      for (int j = 0; j < NHS; ++j)
        if (slot_head(l, j) == g) return l;
    return -1;
  }
  static constexpr int rep_slot(int g) {
    for (int l = 0; l < kWave; ++l)
      for (int j = 0; j < NHS; ++j)
        if (slot_head(l, j) == g) return j;
    return -1;
  }
};

// Transposing butterfly over lane bits M, M/2, .., 1: while a lane holds more
// than one value, pairs (v[i], v[i+N/2]) are split so that the lane keeps one
// half and receives its partner's copy of the same half; once one value is
// left it is summed with the partner's.
template <int N, int M>
__device__ __forceinline__ void transpose_reduce(float* v) {
  if constexpr (M >= 1) {
    if constexpr (N > 1) {
      const bool upper = (__lane_id() & M) != 0;
#pragma unroll
      for (int i = 0; i < N / 2; ++i) {
        const float a = v[i], b = v[i + N / 2];
        const float keep = upper ? b : a;
        const float send = upper ? a : b;
        v[i] = keep + reduce_partner<M>(send);
      }
      transpose_reduce<N / 2, M / 2>(v);
    } else {
      v[0] += reduce_partner<M>(v[0]);
      transpose_reduce<1, M / 2>(v);
    }
  }
}

// All-reduce (max or sum) over the head-neutral lane bits.
template <typename Shape, bool IsMax>
__device__ __forceinline__ float reduce_neutral(float x) {
#define PA_STEP(B)                                                    \
  if constexpr (Shape::bit_neutral(B)) {                              \
    const float y = xor_lane<(1 << B)>(x);                            \
    x = IsMax ? fmaxf(x, y) : x + y;                                  \
  }
  PA_STEP(0) PA_STEP(1) PA_STEP(2) PA_STEP(3) PA_STEP(4) PA_STEP(5)
#undef PA_STEP
  return x;
}

template <typename Shape>
__device__ __forceinline__ void load_k(const uint4* __restrict__ kbase, int lane,
                                       uint4 (&kb)[Shape::NGK][Shape::KCH]) {
  constexpr int RC = Shape::RC, KL = Shape::KL, RK = Shape::RK;
  const int krow = lane / KL, kc = lane % KL;
#pragma unroll
  for (int gk = 0; gk < Shape::NGK; ++gk)
#pragma unroll
    for (int i = 0; i < Shape::KCH; ++i)
      kb[gk][i] = load_stream(kbase + (gk * RK + krow) * RC + kc + KL * i);
}

template <typename Shape>
__device__ __forceinline__ void load_v(const uint4* __restrict__ vbase, int lane,
                                       uint4 (&vb)[Shape::NGV]) {
  constexpr int RC = Shape::RC, VL = Shape::VL, RV = Shape::RV;
  const int vrow = lane / VL, vc = lane % VL;
#pragma unroll
  for (int gv = 0; gv < Shape::NGV; ++gv) vb[gv] = load_stream(vbase + (gv * RV + vrow) * RC + vc);
}

template <typename T, int D, int G>
__global__ __launch_bounds__(kThreads) void decode_partition_kernel(DecodeArgs a) {
  using S = DecodeShape<T, D, G>;
  constexpr int RC = S::RC, KL = S::KL, KCH = S::KCH, NGK = S::NGK, NV = S::NV,
                NVF = S::NVF, NGV = S::NGV, VL = S::VL, RV = S::RV, E = S::E;

  __shared__ float s_p[kWaves][kTile * G];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ float4 s_acc[kWaves][RV][G][D / 4];

  const int part = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
  const int bs_log2 = a.block_size_log2;
  const int bs = 1 << bs_log2;
  int n = a.context_lens[seq];
  n = n < 0 ? 0 : n;
  n = n > a.ctx_limit ? a.ctx_limit : n;
  const int start = part * a.part_tokens;
  if (start >= n) return;
  const int end = min(start + a.part_tokens, n);
  const int nparts = (n + a.part_tokens - 1) / a.part_tokens;

  const int tid = threadIdx.x;
  // wave index as a scalar, so that all tile bookkeeping below is uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;

  // q of the G heads of this KV group, in the K-lane layout.
  uint4 q[G][KCH];
  {
    const uint4* qb = reinterpret_cast<const uint4*>(a.query) +
                      ((int64_t)seq * a.num_q_heads + (int64_t)kvh * G) * RC;
    const int kc = lane % KL;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < KCH; ++i) q[g][i] = qb[g * RC + kc + KL * i];
  }

  // Block-table entries of this partition: lane i holds entry blk0 + i
  // (at most 64 blocks per partition by construction of part_tokens).
  const int blk0 = start >> bs_log2;
  const int nblk = ((end - start) + bs - 1) >> bs_log2;
  int my_block = -1;
  if (lane < nblk) {
    const int e = a.block_tables[(int64_t)seq * a.max_blocks_per_seq + blk0 + lane];
    my_block = (e >= 0 && (int64_t)e < a.num_blocks) ? e : -1;
  }

  const uint4* kcache = reinterpret_cast<const uint4*>(a.key_cache);
  const uint4* vcache = reinterpret_cast<const uint4*>(a.value_cache);
  const int64_t block_stride = (int64_t)a.num_kv_heads * bs * RC;  // in 16-byte chunks
  const int64_t head_off = (int64_t)kvh * bs * RC;

  float m_run[G];     // running max per head (log2 domain), wave-uniform
  float acc[G][E];    // unnormalised PV accumulator, this lane's head-dim slice
  float l_slot[NVF];  // running sum of this lane's own score slots
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[g][e] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < NVF; ++j) l_slot[j] = 0.f;

  const int ntiles = (end - start + kTile - 1) / kTile;
  float* p_lds = s_p[wave];

  // Physical block of tile t (a scalar read of the table entry held by lane
  // t*16/bs); an entry outside the pool reads block 0 and the tile is masked.
  auto tile_block = [&](int t) -> int {
    return __builtin_amdgcn_readlane(my_block, (t * kTile) >> bs_log2);
  };
  auto tile_offset = [&](int t, int blk) -> int64_t {
    return (int64_t)(blk < 0 ? 0 : blk) * block_stride + head_off +
           (int64_t)((start + t * kTile) & (bs - 1)) * RC;
  };

  // Software pipeline over this wave's tiles t = wave, wave + 4, ...: the K
  // registers are refilled for the next tile as soon as the scores are done,
  // the V registers as soon as the PV update is done, so one tile's loads are
  // always in flight behind the current tile's arithmetic. All branches are
  // wave-uniform; the last tile is peeled so that every pipelined iteration
  // prefetches unconditionally.
  uint4 kb[NGK][KCH];
  uint4 vb[NGV];

  auto process = [&](int t, int blk, int64_t off_next, auto prefetch) {
    constexpr bool kPrefetch = decltype(prefetch)::value;
    const int tok0 = start + t * kTile;
    const bool valid = blk >= 0;  // invalid table entry: these tokens contribute nothing

    // ---- scores: partial dots, then transposing reduction over KL lanes
    float sc[NV];
#pragma unroll
    for (int gk = 0; gk < NGK; ++gk)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float c = 0.f;
#pragma unroll
        for (int i = 0; i < KCH; ++i) c = dot_chunk(T{}, kb[gk][i], q[g][i], c);
        sc[gk * G + g] = c;
      }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kPrefetch) load_k<S>(kcache + off_next, lane, kb);
    __builtin_amdgcn_sched_barrier(0);
    transpose_reduce<NV, KL / 2>(sc);

    // rows past the context (or of an invalid block) are masked; they may
    // hold anything, NaN included
    const bool masked_tile = (tok0 + kTile > n) || !valid;
    float s[NVF];
#pragma unroll
    for (int j = 0; j < NVF; ++j) {
      s[j] = sc[j] * a.scale_log2;
      if (masked_tile) {
        const int tok = tok0 + S::slot_token(lane, j);
        s[j] = (valid && tok < n) ? s[j] : -INFINITY;
      }
    }
    if (masked_tile) {
      const int vrow = lane / VL;
#pragma unroll
      for (int gv = 0; gv < NGV; ++gv)
        if (!valid || tok0 + gv * RV + vrow >= n) vb[gv] = make_uint4(0, 0, 0, 0);
    }

    // ---- online softmax: tile max per head, rescale on increase
    float mh[S::NHS];
#pragma unroll
    for (int j = 0; j < S::NHS; ++j) {
      float x = s[j];
#pragma unroll
      for (int jj = j + G; jj < NVF; jj += G) x = fmaxf(x, s[jj]);
      mh[j] = reduce_neutral<S, true>(x);
    }
    float m_new[G];
    bool grow = false;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float tm = readlane_f(mh[S::rep_slot(g)], S::rep_lane(g));
      m_new[g] = fmaxf(m_run[g], tm);
      grow |= m_new[g] > m_run[g];
    }
    if (grow) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float alpha = fast_exp2(m_run[g] - m_new[g]);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[g][e] *= alpha;
      }
#pragma unroll
      for (int j = 0; j < NVF; ++j) {
        // this slot's head, selected from the uniform per-head values
        float mo = m_run[0], mn = m_new[0];
#pragma unroll
        for (int g = 1; g < G; ++g) {
          const bool hit = S::slot_head(lane, j) == g;
          mo = hit ? m_run[g] : mo;
          mn = hit ? m_new[g] : mn;
        }
        l_slot[j] *= fast_exp2(mo - mn);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) m_run[g] = m_new[g];
    }

    // ---- weights: exp2, running sums, hand to the V lanes through LDS. A
    // head whose every score so far is masked has m = -inf: its weights are 0.
#pragma unroll
    for (int j = 0; j < NVF; ++j) {
      float mh_j = m_run[0];
#pragma unroll
      for (int g = 1; g < G; ++g) mh_j = S::slot_head(lane, j) == g ? m_run[g] : mh_j;
      mh_j = mh_j == -INFINITY ? 0.f : mh_j;
      const float p = fast_exp2(s[j] - mh_j);
      l_slot[j] += p;
      p_lds[S::slot_token(lane, j) * G + S::slot_head(lane, j)] = p;
    }
    __builtin_amdgcn_wave_barrier();

    // ---- PV over this lane's head-dim slice, all G heads
    const int vrow = lane / VL;
#pragma unroll
    for (int gv = 0; gv < NGV; ++gv) {
      const int trow = gv * RV + vrow;
      float pw[G];
#pragma unroll
      for (int g = 0; g < G; ++g) pw[g] = p_lds[trow * G + g];
      float v[E];
      widen_chunk(T{}, vb[gv], v);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[g][e] = __builtin_fmaf(pw[g], v[e], acc[g][e]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kPrefetch) load_v<S>(vcache + off_next, lane, vb);
    __builtin_amdgcn_sched_barrier(0);
  };

  int t = wave;
  if (t < ntiles) {
    int blk = tile_block(t);
    const int64_t off = tile_offset(t, blk);
    load_k<S>(kcache + off, lane, kb);
    load_v<S>(vcache + off, lane, vb);
    for (; t + kWaves < ntiles; t += kWaves) {
      const int blk_next = tile_block(t + kWaves);
      process(t, blk, tile_offset(t + kWaves, blk_next), std::true_type{});
      blk = blk_next;
    }
    process(t, blk, 0, std::false_type{});
  }

  // ---- wave totals: l per head (each score counted once), m per head
  float l_head[G];
#pragma unroll
  for (int g = 0; g < G; ++g) l_head[g] = 0.f;
#pragma unroll
  for (int j = 0; j < S::NHS; ++j) {
    float x = l_slot[j];
#pragma unroll
    for (int jj = j + G; jj < NVF; jj += G) x += l_slot[jj];
    x = reduce_neutral<S, false>(x);
#pragma unroll
    for (int g = 0; g < G; ++g)
      if (S::rep_slot(g) == j) l_head[g] = readlane_f(x, S::rep_lane(g)) / (float)S::REP;
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      s_m[wave][g] = m_run[g];
      s_l[wave][g] = l_head[g];
    }
  }
  {
    const int r = lane / VL, c = lane % VL;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e4 = 0; e4 < E / 4; ++e4)
        s_acc[wave][r][g][c * (E / 4) + e4] =
            make_float4(acc[g][4 * e4], acc[g][4 * e4 + 1], acc[g][4 * e4 + 2], acc[g][4 * e4 + 3]);
  }
  __syncthreads();

  // ---- merge the 4 waves and write o (normalised), m, l
  for (int idx = tid; idx < G * D / 4; idx += kThreads) {
    const int g = idx / (D / 4), d4 = idx % (D / 4);
    float M = s_m[0][g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][g]);
    float L = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float sw = fast_exp2(s_m[w][g] - M);
      L += sw * s_l[w][g];
#pragma unroll
      for (int r = 0; r < RV; ++r) {
        const float4 x = s_acc[w][r][g][d4];
        o.x += sw * x.x; o.y += sw * x.y; o.z += sw * x.z; o.w += sw * x.w;
      }
    }
    const float inv = 1.f / L;
    o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
    const int64_t head = (int64_t)seq * a.num_q_heads + (int64_t)kvh * G + g;
    if (nparts == 1) {
      reinterpret_cast<float4*>(a.out)[head * (D / 4) + d4] = o;
    } else {
      const int64_t slot = head * a.max_parts + part;
      reinterpret_cast<float4*>(a.part_o)[slot * (D / 4) + d4] = o;
      if (d4 == 0) {
        a.part_ml[2 * slot] = M;
        a.part_ml[2 * slot + 1] = L;
      }
    }
  }
}

// Merge of the per-partition partials of one (sequence, query head):
// out = sum_p w_p o_p / sum_p w_p with w_p = l_p * 2^(m_p - max_p m_p).
template <int D>
__global__ __launch_bounds__(kWave) void decode_merge_kernel(DecodeArgs a) {
  constexpr int PER = D / kWave;  // 1, 2 or 4 floats per lane
  const int h = blockIdx.x, seq = blockIdx.y;
  int n = a.context_lens[seq];
  n = n < 0 ? 0 : n;
  n = n > a.ctx_limit ? a.ctx_limit : n;
  const int nparts = (n + a.part_tokens - 1) / a.part_tokens;
  const int64_t head = (int64_t)seq * a.num_q_heads + h;
  float* out = a.out + head * D + threadIdx.x * PER;
  if (nparts == 1) return;  // the partition kernel wrote this row
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  if (nparts > 1) {
    const float* ml = a.part_ml + 2 * head * a.max_parts;
    float M = -INFINITY;
    for (int p = 0; p < nparts; ++p) M = fmaxf(M, ml[2 * p]);
    float L = 0.f;
    const float* po = a.part_o + head * a.max_parts * D + threadIdx.x * PER;
    for (int p = 0; p < nparts; ++p) {
      const float w = ml[2 * p + 1] * fast_exp2(ml[2 * p] - M);
      L += w;
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] = __builtin_fmaf(w, po[(int64_t)p * D + e], o[e]);
    }
    const float inv = 1.f / L;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] *= inv;
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) out[e] = o[e];
}

// ---------------------------------------------------------------------------
// Host side.

int decode_part_tokens(int num_seqs, int num_kv_heads, int block_size, int max_context_len) {
  // Largest partition (a multiple of 64 tokens, at most 64 blocks) that still
  // gives the launch enough workgroups to fill 256 CUs several times over.
  const int target = decode_target_workgroups();
  int best = 64;
  const int cap = 64 * block_size;
  for (int p = 64; p <= cap; p *= 2) {
    const int64_t parts = (max_context_len + p - 1) / p;
    if ((int64_t)num_seqs * num_kv_heads * parts >= target) best = p;
  }
  return best;
}

template <typename T, int D, int G>
static hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  if (a.max_parts > 0) {  // every context empty: only the merge kernel runs (zero rows)
    dim3 grid(a.max_parts, a.num_kv_heads, a.num_seqs);
    hipLaunchKernelGGL((decode_partition_kernel<T, D, G>), grid, dim3(kThreads), 0, stream, a);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(a.num_q_heads, a.num_seqs), dim3(kWave), 0,
                     stream, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_g(const DecodeArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_t<T, D, 1>(a, stream);
    case 2: return launch_t<T, D, 2>(a, stream);
    case 4: return launch_t<T, D, 4>(a, stream);
    case 8: return launch_t<T, D, 8>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_d(const DecodeArgs& a, int group, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: return launch_g<T, 64>(a, group, stream);
    case 128: return launch_g<T, 128>(a, group, stream);
    case 256: return launch_g<T, 256>(a, group, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, bool bf16, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  return bf16 ? launch_d<BF16>(a, group, stream) : launch_d<F32>(a, group, stream);
}

}  // namespace pa
