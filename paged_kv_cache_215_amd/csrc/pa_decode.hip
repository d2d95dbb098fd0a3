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
// Work decomposition. A work unit is one (sequence, KV head, context
// partition of P tokens); the partition size comes from a plan that every
// workgroup derives from the context lengths at the start of the launch. The
// grid is persistent (a few workgroups per CU): each workgroup (NW waves, 8
// for the BF16 d 256 shapes) loops over units. In a unit the waves take
// interleaved 16-token tiles of the partition; a tile never crosses a
// physical block (block sizes 16, 32). Each wave keeps an online softmax
// (running max m, running sum l, unnormalised accumulator) per query head of
// the GQA group, the waves are merged in LDS, and the unit writes one
// normalised partial (o, m, l) per query head. A sequence that needs one
// partition writes its output directly; otherwise the merge kernel combines
// the partials. Decode moves ~4 FLOP per byte of KV for groups of up to 4
// query heads, far below the matrix-core ridge, so those contractions stay on
// the VALU; groups of 8 over BF16 caches (about 8 FLOP per byte, enough to
// stall the VALU) run on the matrix cores in decode_mfma_kernel below, with
// the same plan, units and merge. E4M3 caches, whose codes must be converted
// before any arithmetic, take the matrix cores for groups of 8 and for groups
// of 4 at d >= 128 as well.
//
// The plan also tests whether consecutive sequences start on the same
// physical block (copy-on-write rollouts of one prompt). If fewer than half
// of the live sequences do, it aims at one unit per CU and the K/V loads are
// nontemporal: each byte is read once. Otherwise it aims at two units per
// CU, dealt in lockstep, and the dealt partitions (the shared prompt) use
// ordinary loads so that the rollouts reading the same blocks find them in
// the caches.
//
// Register layout of a 16-token tile (per wave):
//   K: each row (token) is spread over KL lanes that each hold KCH 16-byte
//      chunks; 64/KL rows per load instruction, so a load instruction reads
//      whole 128-byte segments. Each lane multiplies its chunks with the
//      matching q chunks of all G heads (v_dot2_f32_bf16 for BF16), leaving
//      NGK*G partial dots that a transposing butterfly over the KL lanes turns
//      into one finished score per lane (G heads x 16 tokens spread over the
//      wave) without any LDS traffic.
//   V: each row is spread over VL lanes (one 16-byte chunk each, 8 bytes for
//      E4M3: a fully coalesced row read); every lane accumulates its
//      head-dim slice for all
//      G heads from the same registers, so V is read once per KV head however
//      many query heads share it. Softmax weights reach the V lanes through a
//      64-float LDS slot per wave.

#include "pa_device.hpp"
#include "pa_internal.hpp"

#include <cstdlib>
#include <type_traits>

namespace pa {

constexpr int kTile = 16;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
constexpr int kMaxPartBlocks = 512;  // table entries staged per partition

constexpr int choose_k_lanes(int row_chunks, int group) {
  // Enough lanes per K row that the q chunks held per lane (group * KCH
  // 16-byte chunks, times the q chunks per K chunk) fit in 32 VGPRs, at
  // least 4 so that a tile holds whole load groups.
  int need = group * row_chunks / 8;
  if (need < 4) need = 4;
  int kl = 4;
  while (kl < need) kl *= 2;
  return kl > row_chunks ? row_chunks : kl;
}

template <typename T, int D, int G>
struct DecodeShape {
  // V is read in VB-byte chunks, one per lane and row: 16 bytes, or 8 for
  // E4M3, whose 16-byte chunk would need 16 accumulators per head and lane.
  static constexpr int VB = T::kBytes == 1 ? 8 : 16;
  static constexpr int E = VB / T::kBytes;          // V elements per lane (8, 8, 4)
  using VChunk = typename std::conditional<VB == 16, uint4, uint2>::type;
  static constexpr int RC = D * T::kBytes / 16;     // chunks per row
  static constexpr int QCH = T::Query::kBytes / T::kBytes;  // q chunks per K chunk
  static constexpr int QRC = RC * QCH;              // q chunks per row
  static constexpr int KL = choose_k_lanes(RC, G * QCH);  // lanes per K row
  static constexpr int KCH = RC / KL;               // chunks per lane per K row
  static constexpr int RK = kWave / KL;             // K rows per load instruction
  static constexpr int NGK = kTile / RK;            // K load groups per tile
  static constexpr int NV = NGK * G;                // partial dots per lane
  static constexpr int NVF = NV >= KL ? NV / KL : 1;  // finished scores per lane
  static constexpr int REP = NV >= KL ? 1 : KL / NV;  // lanes holding the same score
  static constexpr int VL = D * T::kBytes / VB;     // lanes per V row
  static constexpr int RV = kWave / VL;             // V rows per load instruction
  static constexpr int NGV = kTile / RV;            // V load groups per tile
  static constexpr int NHS = NVF < G ? NVF : G;     // distinct heads among a lane's scores
  static_assert(RC <= kWave && RK <= kTile && RV <= kTile, "tile shape");
  static_assert(VL >= 4, "the V row-group sum covers at most 16 row groups");
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

// v[h] for a per-lane index h < 8, as a tree of selects on the bits of h.
// Used for groups of 8 heads only: there the compiler turns a chain of
// compares against 1..7 into an indexed load from scratch memory (for
// smaller groups the chain stays in registers and is used as is).
template <int G>
__device__ __forceinline__ float pick_head(const float (&v)[G], int h) {
  float t[G];
#pragma unroll
  for (int g = 0; g < G; ++g) t[g] = v[g];
#pragma unroll
  for (int w = 1; w < G; w <<= 1) {
    const bool up = (h & w) != 0;
#pragma unroll
    for (int g = 0; g + w < G; g += 2 * w) t[g] = up ? t[g + w] : t[g];
  }
  return t[0];
}

// Transposing butterfly over lane bits M, M/2, .., 1: while a lane holds more
// than one value, pairs (v[i], v[i+N/2]) are split so that the lane keeps one
// half and receives its partner's copy of the same half; once one value is
// left it is summed with the partner's.
template <int N, int M>
__device__ __forceinline__ void transpose_reduce(float* v) {
  if constexpr (M >= 1) {
    if constexpr (N > 1) {
      if constexpr (M >= 16) {
        // the half-wave swap keeps a for lower lanes and b for upper lanes and
        // brings in the partner's other one: exactly keep + partner's send
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
          float r0, r1;
          swap_halves<M>(v[i], v[i + N / 2], r0, r1);
          v[i] = r0 + r1;
        }
      } else {
        const bool upper = (__lane_id() & M) != 0;
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
          const float a = v[i], b = v[i + N / 2];
          const float keep = upper ? b : a;
          const float send = upper ? a : b;
          v[i] = keep + reduce_partner<M>(send);
        }
      }
      transpose_reduce<N / 2, M / 2>(v);
    } else {
      if constexpr (M >= 16) {
        v[0] = pair_sum<M>(v[0]);
      } else {
        v[0] += reduce_partner<M>(v[0]);
      }
      transpose_reduce<1, M / 2>(v);
    }
  }
}

// All-reduce (max or sum) over the head-neutral lane bits.
template <typename Shape, bool IsMax>
__device__ __forceinline__ float reduce_neutral(float x) {
#define PA_STEP(B)                                                    \
  if constexpr (Shape::bit_neutral(B)) {                              \
    x = IsMax ? pair_max<(1 << B)>(x) : pair_sum<(1 << B)>(x);        \
  }
  PA_STEP(0) PA_STEP(1) PA_STEP(2) PA_STEP(3) PA_STEP(4) PA_STEP(5)
#undef PA_STEP
  return x;
}

template <typename Shape, bool Keep>
__device__ __forceinline__ void load_k(const uint4* __restrict__ kbase, int lane,
                                       uint4 (&kb)[Shape::NGK][Shape::KCH]) {
  constexpr int RC = Shape::RC, KL = Shape::KL, RK = Shape::RK;
  const int krow = lane / KL, kc = lane % KL;
#pragma unroll
  for (int gk = 0; gk < Shape::NGK; ++gk)
#pragma unroll
    for (int i = 0; i < Shape::KCH; ++i)
      kb[gk][i] = load_kv<Keep>(kbase + (gk * RK + krow) * RC + kc + KL * i);
}

template <typename Shape, bool Keep>
__device__ __forceinline__ void load_v(const uint4* __restrict__ vbase, int lane,
                                       typename Shape::VChunk (&vb)[Shape::NGV]) {
  using VC = typename Shape::VChunk;
  constexpr int VL = Shape::VL, RV = Shape::RV;  // a row is VL chunks of VC
  const VC* base = reinterpret_cast<const VC*>(vbase);
  const int vrow = lane / VL, vc = lane % VL;
#pragma unroll
  for (int gv = 0; gv < Shape::NGV; ++gv) vb[gv] = load_kv<Keep>(base + (gv * RV + vrow) * VL + vc);
}

// ---------------------------------------------------------------------------
// Plan of one decode call. Every partition workgroup derives the same plan
// from the context lengths: the partition size is one partition per sequence
// for a batch of equal lengths (when that alone gives every CU a unit),
// otherwise about units_per_cu units per CU; units are every full partition
// first, then each sequence's last (shorter) one, and a single unit for an
// empty context (its zero row). A launch covers at most kPlanSeqs sequences.
constexpr int kPlanSeqs = 4096;

__device__ __forceinline__ long long wave_sum_ll(long long x) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) x += __shfl_xor(x, m);
  return x;
}
__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) x = min(x, __shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) x = max(x, __shfl_xor(x, m));
  return x;
}
// inclusive prefix sum across the wave
__device__ __forceinline__ int wave_scan(int x) {
  const int lane = __lane_id();
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    const int y = __shfl_up(x, m);
    if (lane >= m) x += y;
  }
  return x;
}

constexpr int kTailClasses = 16;  // size classes of the last partitions (P / 16 tokens each)

struct PlanLds {
  int lens[kPlanSeqs];        // tokens to attend: clamped context lengths, less a
                              // copy-on-write group member's shared prefix
  int starts[kPlanSeqs];      // first position attended (the shared prefix's end)
  int full_pre[kPlanSeqs];    // exclusive prefix of full-partition counts
  unsigned short tail_order[kPlanSeqs];  // sequences by the size of their last partition
  int cls_cnt[8][kTailClasses];          // per wave: last partitions of each size class
  long long red_sum[16];
  int red_a[16], red_b[16], red_c[16], red_d[16];
  int part_tokens, full_total, max_nparts;
  int ranked;                 // tail_order holds the order (else: sequence order)
  int shared;                 // at least half of the live sequences start on their
                              // predecessor's first block (copy-on-write rollouts)
  int ticket;                 // this workgroup's current unit
};

// Fills the plan for the whole workgroup (NW waves); ends with a barrier.
template <int NW>
__device__ void build_plan(const DecodeArgs& a, PlanLds& pl) {
  static_assert(NW <= 8 && kPlanSeqs <= 65536, "plan storage");
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int S = a.num_seqs;
  constexpr int kT = NW * kWave;
  const int chunk = (S + kT - 1) / kT;
  const int b0 = min(S, tid * chunk), b1 = min(S, b0 + chunk);
  long long sum = 0;
  int mn = 0x7fffffff, mx = 0;
  // shared: sequences that start on the same physical block as the one
  // before them (copy-on-write rollouts of one prompt are consecutive);
  // live: sequences with a non-empty context. The batch counts as sharing
  // blocks when at least half of its live sequences do.
  // (an entry is read whatever the length, so that its load does not wait on
  // the length's; it counts only for a non-empty context)
  int shared = 0, live = 0;
  int prev_first = -1;
  if (b0 > 0 && b0 < b1) {
    const int n = a.context_lens[b0 - 1];
    const int e = a.block_tables[(int64_t)(b0 - 1) * a.max_blocks_per_seq];
    if (n > 0 && a.ctx_limit > 0) prev_first = e;
  }
  const int grouped_lo = a.num_groups > 0 ? max(a.cu_groups[0], 0) : 0;
  const int grouped_hi = a.num_groups > 0 ? min(a.cu_groups[a.num_groups], S) : 0;
  for (int b = b0; b < b1; ++b) {
    int n = a.context_lens[b];
    const int e = a.block_tables[(int64_t)b * a.max_blocks_per_seq];
    n = n < 0 ? 0 : n;
    n = n > a.ctx_limit ? a.ctx_limit : n;
    // copy-on-write group member: its shared prefix was attended by the
    // prefix pass, which recorded where its tail starts; this launch takes
    // the tail (sequences outside [cu_groups[0], cu_groups[num_groups]) are
    // in no group)
    const int start = (b >= grouped_lo && b < grouped_hi) ? a.seq_start[b] : 0;
    pl.starts[b] = start;
    n = n > start ? n - start : 0;
    pl.lens[b] = n;
    sum += n;
    mn = min(mn, n);
    mx = max(mx, n);
    const int first = n > 0 ? e : -1;
    shared += first >= 0 && first == prev_first;
    live += n > 0;
    prev_first = first;
  }
  sum = wave_sum_ll(sum);
  mn = wave_min(mn);
  mx = wave_max(mx);
  shared = (int)wave_sum_ll(shared);
  live = (int)wave_sum_ll(live);
  if (lane == 0) {
    pl.red_sum[wave] = sum;
    pl.red_a[wave] = mn;
    pl.red_b[wave] = mx;
    pl.red_c[wave] = shared;
    pl.red_d[wave] = live;
  }
  __syncthreads();
  if (wave == 0) {
    sum = lane < NW ? pl.red_sum[lane] : 0;
    mn = lane < NW ? pl.red_a[lane] : 0x7fffffff;
    mx = lane < NW ? pl.red_b[lane] : 0;
    shared = lane < NW ? pl.red_c[lane] : 0;
    live = lane < NW ? pl.red_d[lane] : 0;
    sum = wave_sum_ll(sum);
    mn = wave_min(mn);
    mx = wave_max(mx);
    shared = (int)wave_sum_ll(shared);
    live = (int)wave_sum_ll(live);
    // (members of copy-on-write groups attend only their private tails here)
    shared = a.num_groups == 0 && live > 0 && 2 * shared >= live;
    if (lane == 0) {
      int P = a.part_floor;
      if (mx > 0 && mn == mx) {
        for (int p = a.part_floor; p <= a.part_cap; p *= 2)
          if ((long long)S * a.num_kv_heads * ((mx + p - 1) / p) >= a.plan_cus) P = p;
      } else if (mx > 0) {
        // Ragged lengths: each CU's share of the tokens, rounded up to a
        // multiple of 128 (whole 16-token tiles for every wave, whole
        // blocks), within [part_floor, part_cap]. Rounded down to a power
        // of two instead, a CU's share was one full partition plus scraps
        // for the ticketed tails to fill: ragged 32-sequence layer 106.5 ->
        // 101.7 us, over FP8 67.8 -> 62.7 us, mixed step 303.5 -> 298.4 us.
        const int units = shared ? a.plan_units_per_cu : a.plan_units_unshared;
        const long long budget =
            sum * a.num_kv_heads / ((long long)a.plan_cus * units);
        long long p = (budget + 127) / 128 * 128;
        p = p < a.part_floor ? a.part_floor : p;
        p = p > a.part_cap ? a.part_cap : p;
        P = (int)p;
      }
      pl.part_tokens = P;
      pl.ranked = mn != mx;  // equal lengths: equal last partitions, already in order
      pl.shared = shared;
    }
  }
  __syncthreads();
  const int P = pl.part_tokens;
  int full = 0, most = 0;
  for (int b = b0; b < b1; ++b) {
    const int np = max(1, (pl.lens[b] + P - 1) / P);
    full += np - 1;
    most = max(most, np);
  }
  const int incl = wave_scan(full);
  most = wave_max(most);
  __syncthreads();  // the reduction slots are reused below
  if (lane == kWave - 1) pl.red_a[wave] = incl;
  if (lane == 0) pl.red_b[wave] = most;
  __syncthreads();
  if (wave == 0) {
    const int c = lane < NW ? pl.red_a[lane] : 0;
    const int ci = wave_scan(c);
    const int mp = wave_max(lane < NW ? pl.red_b[lane] : 0);
    if (lane < NW) pl.red_a[lane] = ci - c;
    if (lane == kWave - 1) {
      pl.full_total = ci;
      pl.max_nparts = mp;
    }
  }
  __syncthreads();
  int run = pl.red_a[wave] + incl - full;
  for (int b = b0; b < b1; ++b) {
    pl.full_pre[b] = run;
    run += max(1, (pl.lens[b] + P - 1) / P) - 1;
  }

  // Order of the last partitions, which the ticket counter hands out: the
  // longest first, so that the shortest ones fill the gaps at the end (longest
  // processing time first). Lengths go into kTailClasses classes of P / 16
  // tokens; within a class the order is the sequence order, so every
  // workgroup derives the same permutation. Wave w ranks the sequences of
  // its own contiguous range with ballots. A batch of equal lengths keeps the
  // sequence order and skips this.
  if (!pl.ranked) {
    __syncthreads();
    return;
  }
  const int per_wave = (S + NW - 1) / NW;
  const int w0 = min(S, wave * per_wave), w1 = min(S, w0 + per_wave);
  auto tail_class = [&](int b) {
    const int n = pl.lens[b];
    const int tail = n - (max(1, (n + P - 1) / P) - 1) * P;
    return tail <= 0 ? 0 : (tail - 1) * kTailClasses / P;
  };
  int cnt = 0;  // lane k < kTailClasses: sequences of class k in this wave's range
  for (int c0 = w0; c0 < w1; c0 += kWave) {
    const int b = c0 + lane;
    const int c = b < w1 ? tail_class(b) : -1;
#pragma unroll
    for (int k = 0; k < kTailClasses; ++k) {
      const int m = __builtin_popcountll(__builtin_amdgcn_ballot_w64(c == k));
      if (lane == k) cnt += m;
    }
  }
  if (lane < kTailClasses) pl.cls_cnt[wave][lane] = cnt;
  __syncthreads();
  {  // lane k < kTailClasses: first position of (class k, this wave)
    int total = 0, earlier = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int x = lane < kTailClasses ? pl.cls_cnt[w][lane] : 0;
      total += x;
      earlier += w < wave ? x : 0;
    }
    const int incl_cls = wave_scan(total);  // classes 0..k
    const int all = __builtin_amdgcn_readlane(incl_cls, kTailClasses - 1);
    cnt = all - incl_cls + earlier;  // larger classes, then this class in earlier waves
  }
  for (int c0 = w0; c0 < w1; c0 += kWave) {
    const int b = c0 + lane;
    const int c = b < w1 ? tail_class(b) : -1;
    int pos = 0;
#pragma unroll
    for (int k = 0; k < kTailClasses; ++k) {
      const unsigned long long m = __builtin_amdgcn_ballot_w64(c == k);
      const int next = __builtin_amdgcn_readlane(cnt, k);
      const int below = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
      if (c == k) pos = next + below;
      if (lane == k) cnt += __builtin_popcountll(m);
    }
    if (b < w1) pl.tail_order[pos] = (unsigned short)b;
  }
  __syncthreads();
}

// Unit e of the plan -> (sequence, partition).
__device__ __forceinline__ int2 plan_unit(const PlanLds& pl, int S, int e) {
  if (e >= pl.full_total) {
    const int b = pl.ranked ? pl.tail_order[e - pl.full_total] : e - pl.full_total;
    const int P = pl.part_tokens;
    return make_int2(b, max(1, (pl.lens[b] + P - 1) / P) - 1);
  }
  int lo = 0, hi = S - 1;  // last b with full_pre[b] <= e
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pl.full_pre[mid] <= e) lo = mid; else hi = mid - 1;
  }
  return make_int2(lo, e - pl.full_pre[lo]);
}

// The plan summary the merge kernel needs, written by workgroup 0: partition
// size, largest partition count, and (only when some sequence has several
// partitions) where each sequence's partial slots start.
template <int NT>
__device__ __forceinline__ void publish_plan(const DecodeArgs& a, const PlanLds& pl) {
  if (blockIdx.x != 0) return;
  if (threadIdx.x == 0) {
    a.plan->part_tokens = pl.part_tokens;
    a.plan->max_nparts = pl.max_nparts;
    a.plan->full_total = pl.full_total;
  }
  if (pl.max_nparts > 1)
    for (int b = threadIdx.x; b < a.num_seqs; b += NT) a.full_pre[b] = pl.full_pre[b];
}

// Partial slot of (sequence, partition, query head): full partitions take
// slots [0, full_total) in plan order, a sequence's last partition slot
// full_total + seq; each slot holds one row per query head.
__device__ __forceinline__ int64_t partial_slot(const DecodeArgs& a, const PlanLds& pl, int seq,
                                                int part, int nparts, int head) {
  const int e = part < nparts - 1 ? pl.full_pre[seq] + part : pl.full_total + seq;
  return (int64_t)e * a.num_q_heads + head;
}

// Persistent loop over the plan's units, shared by the partition kernels.
// Full partitions (all of one size) go round-robin, so the grid walks them in
// lockstep rounds: sequences that share prompt blocks (copy-on-write rollouts
// are consecutive) read those blocks at about the same time. The last
// partitions, whose sizes are ragged, are then taken from the ticket counter
// in the workspace head so that they balance across CUs. The last workgroup
// to leave the queue sets the counters back to zero for the next call (every
// other workgroup has taken its last ticket by then), so a workspace is left
// ready whatever happens to later launches. `keep` selects ordinary rather
// than nontemporal K/V loads for a batch that shares blocks;
// unit(seq, kvh, part, tag) runs one unit with the load kind as a type tag.
template <int KvBytes, typename Unit>
__device__ __forceinline__ void run_units(const DecodeArgs& a, PlanLds& pl, bool keep,
                                          Unit&& unit) {
  const int tid = threadIdx.x;
  const int n_full = pl.full_total * a.num_kv_heads;
  const int n_units = (pl.full_total + a.num_seqs) * a.num_kv_heads;
  for (int u = blockIdx.x; u < n_full; u += gridDim.x) {
    const int2 e = plan_unit(pl, a.num_seqs, u / a.num_kv_heads);
    if (keep) unit(e.x, u % a.num_kv_heads, e.y, std::true_type{});
    else unit(e.x, u % a.num_kv_heads, e.y, std::false_type{});
    __syncthreads();  // LDS is reused by the next unit
  }
  for (;;) {
    if (tid == 0) pl.ticket = atomicAdd(&a.plan->ticket, 1);
    __syncthreads();
    const int u = n_full + pl.ticket;
    __syncthreads();  // every thread has read the ticket before it is reused
    if (u < n_full || u >= n_units) break;  // (below n_full: workspace never zero-filled)
    const int2 e = plan_unit(pl, a.num_seqs, u / a.num_kv_heads);
    // last partitions are private tails even in a shared batch: nontemporal
    // for BF16 / float32 caches (shared-prompt batch 245 -> 231 us), ordinary
    // for E4M3 ones, which measured faster that way (146 vs 154 us)
    if (KvBytes == 1 && keep) unit(e.x, u % a.num_kv_heads, e.y, std::true_type{});
    else unit(e.x, u % a.num_kv_heads, e.y, std::false_type{});
    __syncthreads();
  }
  // (No fence before the count: each workgroup consumed the value its last
  // ticket fetch returned before it got here, so that fetch has been
  // performed. A device-scope fence would also write this XCD's L2 back,
  // which cost the C2-shaped ragged layer about 10 %.)
  if (tid == 0) {
    if (atomicAdd(&a.plan->done, 1) == (int)gridDim.x - 1) {
      atomicExch(&a.plan->ticket, 0);
      atomicExch(&a.plan->done, 0);
    }
  }
}

template <typename T, int D, int G, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_partition_kernel(DecodeArgs a) {
  using S = DecodeShape<T, D, G>;
  constexpr int kWaves = NW;
  constexpr int kThreads = NW * kWave;
  constexpr int RC = S::RC, KL = S::KL, KCH = S::KCH, NGK = S::NGK, NV = S::NV,
                NVF = S::NVF, NGV = S::NGV, VL = S::VL, RV = S::RV, E = S::E;

  __shared__ PlanLds s_plan;
  __shared__ int s_bt[kMaxPartBlocks];
  __shared__ float s_p[kWaves][kTile * G];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ float4 s_acc[kWaves][G][D / 4];
  __shared__ int s_prog[kWaves];  // tiles each wave has finished in this unit

  const int bs_log2 = a.block_size_log2;
  const int bs = 1 << bs_log2;
  const int tid = threadIdx.x;
  build_plan<NW>(a, s_plan);
  const int P = s_plan.part_tokens;
  // blocks shared between sequences: K/V through ordinary loads (see load_kv)
  const bool keep = __builtin_amdgcn_readfirstlane(s_plan.shared) != 0;
  publish_plan<kThreads>(a, s_plan);

  // One work unit: (sequence, KV head, partition) of the plan.
  auto unit = [&](const int seq, const int kvh, const int part, auto keep_tag) {
  constexpr bool kKeep = decltype(keep_tag)::value;
  // n: tokens this launch attends (a copy-on-write group member's tail, from
  // position pos0 on; the whole context otherwise)
  const int n = s_plan.lens[seq];
  const int pos0 = s_plan.starts[seq];
  const bool has_prefix = pos0 > 0;
  const int start = part * P;
  if (n == 0) {
    if (has_prefix) {  // empty tail: an empty partial for the merge
      if (tid < G) {
        const int64_t slot = partial_slot(a, s_plan, seq, 0, 1, kvh * G + tid);
        a.part_ml[2 * slot] = -INFINITY;
        a.part_ml[2 * slot + 1] = 0.f;
      }
      return;
    }
    for (int idx = tid; idx < G * D / 4; idx += kThreads)  // empty context: a zero row
      reinterpret_cast<float4*>(a.out)[((int64_t)seq * a.num_q_heads + (int64_t)kvh * G) * (D / 4) + idx] =
          make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  if (start >= n) return;
  const int end = min(start + P, n);
  const int nparts = (n + P - 1) / P;

  // wave index as a scalar, so that all tile bookkeeping below is uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;

  // q of the G heads of this KV group, in the K-lane layout.
  constexpr int QCH = S::QCH, QRC = S::QRC;
  using QT = typename T::Query;
  uint4 q[G][KCH][QCH];
  {
    const uint4* qb = reinterpret_cast<const uint4*>(a.query) +
                      ((int64_t)seq * a.num_q_heads + (int64_t)kvh * G) * QRC;
    const int kc = lane % KL;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < KCH; ++i)
#pragma unroll
        for (int j = 0; j < QCH; ++j) q[g][i][j] = qb[g * QRC + (kc + KL * i) * QCH + j];
  }
  // FP8 cache: the per-head K scale folds into the score scale, the V scale
  // into the output normalisation
  constexpr bool kScaled = std::is_same<T, FP8>::value;
  const float score_scale = kScaled ? a.scale_log2 * a.k_scale[kvh] : a.scale_log2;
  const float out_scale = kScaled ? a.v_scale[kvh] : 1.f;

  // Block-table entries of this partition, staged in LDS (at most
  // kMaxPartBlocks by construction of part_tokens); -1 marks an entry outside
  // the pool.
  const int blk0 = (pos0 + start) >> bs_log2;  // pos0 is a whole number of blocks
  const int nblk = ((end - start) + bs - 1) >> bs_log2;
  for (int i = tid; i < nblk; i += kThreads) {
    const int e = a.block_tables[(int64_t)seq * a.max_blocks_per_seq + blk0 + i];
    s_bt[i] = (e >= 0 && (int64_t)e < a.num_blocks) ? e : -1;
  }
  if (lane == 0) s_prog[wave] = 0;
  __syncthreads();

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

  // Physical block of tile t (one broadcast LDS read, made scalar); an entry
  // outside the pool reads block 0 and the tile is masked.
  auto tile_block = [&](int t) -> int {
    return __builtin_amdgcn_readfirstlane(s_bt[(t * kTile) >> bs_log2]);
  };
  auto tile_offset = [&](int t, int blk) -> int64_t {
    return (int64_t)(blk < 0 ? 0 : blk) * block_stride + head_off +
           (int64_t)((start + t * kTile) & (bs - 1)) * RC;
  };

  // Software pipeline over this wave's tiles t = wave, wave + NW, ...: the K
  // registers are refilled for the next tile as soon as the scores are done,
  // the V registers as soon as the PV update is done, so one tile's loads are
  // always in flight behind the current tile's arithmetic. All branches are
  // wave-uniform; the last tile is peeled so that every pipelined iteration
  // prefetches unconditionally.
  uint4 kb[NGK][KCH];
  typename S::VChunk vb[NGV];

  auto process = [&](int t, int blk, int64_t off_next, auto prefetch) {
    constexpr bool kPrefetch = decltype(prefetch)::value;
    const int tok0 = start + t * kTile;
    const bool valid = blk >= 0;  // invalid table entry: these tokens contribute nothing

    // ---- scores: partial dots, then transposing reduction over KL lanes
    float sc[NV];
    if constexpr (QCH == 1) {  // K chunks are used as they are
#pragma unroll
      for (int gk = 0; gk < NGK; ++gk)
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float c = 0.f;
#pragma unroll
          for (int i = 0; i < KCH; ++i) c = dot_chunk(QT{}, kb[gk][i], q[g][i][0], c);
          sc[gk * G + g] = c;
        }
    } else {  // each K chunk is converted once for all G heads
#pragma unroll
      for (int gk = 0; gk < NGK; ++gk) {
#pragma unroll
        for (int g = 0; g < G; ++g) sc[gk * G + g] = 0.f;
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
          uint4 kq[QCH];
          k_as_query(T{}, kb[gk][i], kq);
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int j = 0; j < QCH; ++j)
              sc[gk * G + g] = dot_chunk(QT{}, kq[j], q[g][i][j], sc[gk * G + g]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kPrefetch) load_k<S, kKeep>(kcache + off_next, lane, kb);
    __builtin_amdgcn_sched_barrier(0);
    transpose_reduce<NV, KL / 2>(sc);

    // rows past the context (or of an invalid block) are masked; they may
    // hold anything, NaN included
    const bool masked_tile = (tok0 + kTile > n) || !valid;
    float s[NVF];
#pragma unroll
    for (int j = 0; j < NVF; ++j) {
      s[j] = sc[j] * score_scale;
      if (masked_tile) {
        const int tok = tok0 + S::slot_token(lane, j);
        s[j] = (valid && tok < n) ? s[j] : -INFINITY;
      }
    }
    if (masked_tile) {
      const int vrow = lane / VL;
#pragma unroll
      for (int gv = 0; gv < NGV; ++gv)
        if (!valid || tok0 + gv * RV + vrow >= n) zero_chunk(vb[gv]);
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
        if constexpr (G == 8) {
          const int h = S::slot_head(lane, j);
          mo = pick_head<G>(m_run, h);
          mn = pick_head<G>(m_new, h);
        } else {
#pragma unroll
          for (int g = 1; g < G; ++g) {
            const bool hit = S::slot_head(lane, j) == g;
            mo = hit ? m_run[g] : mo;
            mn = hit ? m_new[g] : mn;
          }
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
      if constexpr (G == 8) {
        mh_j = pick_head<G>(m_run, S::slot_head(lane, j));
      } else {
#pragma unroll
        for (int g = 1; g < G; ++g) mh_j = S::slot_head(lane, j) == g ? m_run[g] : mh_j;
      }
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
    if constexpr (kPrefetch) load_v<S, kKeep>(vcache + off_next, lane, vb);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Waves w and w + 4 share a SIMD, and of two waves the older one wins the
  // issue arbitration: with equal tile counts waves 0-3 finished their tiles
  // in about 74 % of the time waves 4-7 took, so for the last quarter of
  // every unit one wave per SIMD streamed alone. Each wave posts its
  // progress after every tile, and the one that is behind its partner takes
  // the higher priority. (Which wave attends which tile does not change, so
  // results stay bit-identical run to run.)
  int t = wave;
  if (t < ntiles) {
    int blk = tile_block(t);
    const int64_t off = tile_offset(t, blk);
    load_k<S, kKeep>(kcache + off, lane, kb);
    load_v<S, kKeep>(vcache + off, lane, vb);
    for (; t + kWaves < ntiles; t += kWaves) {
      if constexpr (kWaves == 8) {
        __builtin_amdgcn_sched_barrier(0);
        const int done = (t - wave) / kWaves;  // tiles this wave has finished
        if (lane == 0) s_prog[wave] = done;
        const int partner = __builtin_amdgcn_readfirstlane(s_prog[wave ^ 4]);
        if (done > partner) __builtin_amdgcn_s_setprio(0);
        else __builtin_amdgcn_s_setprio(1);
        __builtin_amdgcn_sched_barrier(0);
      }
      const int blk_next = tile_block(t + kWaves);
      process(t, blk, tile_offset(t + kWaves, blk_next), std::true_type{});
      blk = blk_next;
    }
    process(t, blk, 0, std::false_type{});
    if constexpr (kWaves == 8) __builtin_amdgcn_s_setprio(0);
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
    // sum the RV row groups of the wave (lanes l, l + VL, ...) in registers
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float x = acc[g][e];
        if constexpr (VL <= 32 && RV > 1) x = pair_sum<32>(x);
        if constexpr (VL <= 16 && RV > 2) x = pair_sum<16>(x);
        if constexpr (VL <= 8 && RV > 4) x += xor_lane<(VL <= 8 ? 8 : 1)>(x);
        if constexpr (VL <= 4 && RV > 8) x += xor_lane<(VL <= 4 ? 4 : 1)>(x);
        acc[g][e] = x;
      }
    if (lane < VL) {
      const int c = lane;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e4 = 0; e4 < E / 4; ++e4)
          s_acc[wave][g][c * (E / 4) + e4] =
              make_float4(acc[g][4 * e4], acc[g][4 * e4 + 1], acc[g][4 * e4 + 2], acc[g][4 * e4 + 3]);
    }
  }
  __syncthreads();

  // ---- merge the waves and write o (normalised), m, l
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
      const float4 x = s_acc[w][g][d4];
      o.x += sw * x.x; o.y += sw * x.y; o.z += sw * x.z; o.w += sw * x.w;
    }
    const float inv = out_scale / L;
    o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
    const int64_t head = (int64_t)seq * a.num_q_heads + (int64_t)kvh * G + g;
    if (nparts == 1 && !has_prefix) {
      reinterpret_cast<float4*>(a.out)[head * (D / 4) + d4] = o;
    } else {
      const int64_t slot = partial_slot(a, s_plan, seq, part, nparts, kvh * G + g);
      reinterpret_cast<float4*>(a.part_o)[slot * (D / 4) + d4] = o;
      if (d4 == 0) {
        a.part_ml[2 * slot] = M;
        a.part_ml[2 * slot + 1] = L;
      }
    }
  }
  };  // unit

  run_units<T::kBytes>(a, s_plan, keep, unit);
}

// ---------------------------------------------------------------------------
// Matrix-core partition kernel for groups of 8 query heads over BF16 caches,
// and for groups of 4 and 8 over E4M3 caches.
//
// With 8 query heads per KV head the VALU kernel spends 4 * 8 * d flops per
// (token, KV head) against 4 d bytes of K and V: about 8 flops per byte,
// enough to make it wait on its own arithmetic (about 61 % of the HBM rate at
// d = 128). An E4M3 cache halves the bytes for the same arithmetic and adds
// the code conversions, so groups of 4 hit the same wall there. Here the
// contractions run on v_mfma instructions, with the G heads as the first G
// of the 16 columns of a 16 x 16 product (the rest are padding):
//   S^T[16 keys x 16] = K[16 keys x d] . Q^T[d x 16]   (16x16x32, d/32 steps)
//     A = K rows straight from HBM: lane l reads 16 bytes of key l % 16 at
//         dims 32 ks + 8 (l / 16) .. + 7, the A operand layout (E4M3: 16
//         codes at dims 16 (l / 16 + 4 j), converted exactly to BF16 and
//         used as k-steps 2 j and 2 j + 1);
//     B = Q^T: lane l holds head l % 16 at the same dims (registers).
//   O^T[16 dims x 16] += V^T[16 dims x 16 keys] . P^T[16 keys x 16]  (16x16x16;
//     an E4M3 V tile is converted to BF16 as it is written to LDS)
//     B = P^T: lane l holds the weights of keys 4 (l / 16) .. + 3 for head
//         l % 16, which is where the score product left those scores;
//     A = V^T: the V tile goes through this wave's LDS region row-major and
//         is read with ds_read_b64_tr_b16 (lane layout checked on the
//         hardware): output lane i of a 16-lane group q gets V[4q + k][d0 + i]
//         for k = 0..3 when lane j of the group supplies key row 4q + j/4 at
//         dims d0 + 4 (j % 4).
// The weights enter PV as BF16 hi + lo terms (16 significant bits), as in
// the prefill kernel, and the running sum uses the same split values. The
// plan, the work units, the persistent loop, the partials and the merge
// kernel are those of the VALU kernel. The per-head E4M3 scales fold into
// the score scale (K) and the output normalisation (V).
template <typename T, int D, int G, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_mfma_kernel(DecodeArgs a) {
  constexpr bool kFp8 = std::is_same<T, FP8>::value;
  static_assert(kFp8 || std::is_same<T, BF16>::value, "BF16 or E4M3 caches");
  static_assert(G <= 16, "heads are columns of a 16-wide product");
  constexpr int kWaves = NW;
  constexpr int kThreads = NW * kWave;
  constexpr int DCH = D / 8;                   // 16-byte BF16 chunks per row
  constexpr int CCH = D * T::kBytes / 16;      // 16-byte chunks per cache row
  constexpr int KSTEPS = D / 32;               // k-steps of the score product
  constexpr int KLD = kFp8 ? KSTEPS / 2 : KSTEPS;  // K loads per lane per tile
  constexpr int DT = D / 16;                   // 16-dim tiles of the output
  constexpr int SWZ = (DCH < 16 ? DCH : 16) - 1;
  constexpr int VPL = kTile * CCH / kWave;     // V cache chunks per lane per tile
  static_assert(VPL >= 1 && kTile * CCH % kWave == 0 && KLD >= 1, "tile shape");
  // a wave's V tile (kTile rows of D bf16) and its share of the final merge
  // (G heads of D floats) are both 32 D bytes; the merge reuses the region
  static_assert(kTile * DCH * 16 >= G * D * 4, "the merge fits the V region");

  __shared__ PlanLds s_plan;
  __shared__ int s_bt[kMaxPartBlocks];
  __shared__ __attribute__((aligned(16))) uint4 s_region[kWaves][kTile * DCH];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ int s_prog[kWaves];  // tiles each wave has finished in this unit

  const int bs_log2 = a.block_size_log2;
  const int bs = 1 << bs_log2;
  const int tid = threadIdx.x;
  build_plan<NW>(a, s_plan);
  const int P = s_plan.part_tokens;
  // blocks shared between sequences: K/V through ordinary loads (see load_kv)
  const bool keep = __builtin_amdgcn_readfirstlane(s_plan.shared) != 0;
  publish_plan<kThreads>(a, s_plan);

  auto unit = [&](const int seq, const int kvh, const int part, auto keep_tag) {
  constexpr bool kKeep = decltype(keep_tag)::value;
  // n: tokens this launch attends (a copy-on-write group member's tail, from
  // position pos0 on; the whole context otherwise)
  const int n = s_plan.lens[seq];
  const int pos0 = s_plan.starts[seq];
  const bool has_prefix = pos0 > 0;
  const int start = part * P;
  if (n == 0) {
    if (has_prefix) {  // empty tail: an empty partial for the merge
      if (tid < G) {
        const int64_t slot = partial_slot(a, s_plan, seq, 0, 1, kvh * G + tid);
        a.part_ml[2 * slot] = -INFINITY;
        a.part_ml[2 * slot + 1] = 0.f;
      }
      return;
    }
    for (int idx = tid; idx < G * D / 4; idx += kThreads)  // empty context: a zero row
      reinterpret_cast<float4*>(a.out)[((int64_t)seq * a.num_q_heads + (int64_t)kvh * G) * (D / 4) + idx] =
          make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  if (start >= n) return;
  const int end = min(start + P, n);
  const int nparts = (n + P - 1) / P;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  int lane = tid % kWave;
  // E4M3: the lane's address offsets are recomputed in each unit rather than
  // held across the whole kernel (28 VGPRs, which kept d = 256 above the 256
  // of an 8-wave workgroup)
  if constexpr (kFp8) asm volatile("" : "+v"(lane));
  const int col = lane % 16, grp = lane / 16;

  // Q^T operand: head col of the group (zero for the padding columns)
  // (k-step ks covers BF16 chunk 4 ks + grp; for E4M3, k-steps 2 j + h cover
  // chunk 2 (grp + 4 j) + h, the dims of the lane's 16 codes)
  bf16x8_t qop[KSTEPS];
  {
    const uint4* qb = reinterpret_cast<const uint4*>(a.query) +
                      ((int64_t)seq * a.num_q_heads + (int64_t)kvh * G + (col < G ? col : 0)) * DCH;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int chunk = kFp8 ? 2 * (grp + 4 * (ks / 2)) + ks % 2 : 4 * ks + grp;
      const uint4 v = qb[chunk];
      qop[ks] = __builtin_bit_cast(bf16x8_t, col < G ? v : make_uint4(0, 0, 0, 0));
    }
  }
  const float score_scale = kFp8 ? a.scale_log2 * a.k_scale[kvh] : a.scale_log2;
  const float out_scale = kFp8 ? a.v_scale[kvh] : 1.f;

  const int blk0 = (pos0 + start) >> bs_log2;  // pos0 is a whole number of blocks
  const int nblk = ((end - start) + bs - 1) >> bs_log2;
  for (int i = tid; i < nblk; i += kThreads) {
    const int e = a.block_tables[(int64_t)seq * a.max_blocks_per_seq + blk0 + i];
    s_bt[i] = (e >= 0 && (int64_t)e < a.num_blocks) ? e : -1;
  }
  if (lane == 0) s_prog[wave] = 0;
  __syncthreads();

  const uint4* kcache = reinterpret_cast<const uint4*>(a.key_cache);
  const uint4* vcache = reinterpret_cast<const uint4*>(a.value_cache);
  const int64_t block_stride = (int64_t)a.num_kv_heads * bs * CCH;  // 16-byte chunks
  const int64_t head_off = (int64_t)kvh * bs * CCH;
  const int ntiles = (end - start + kTile - 1) / kTile;
  uint4* vt = s_region[wave];

  auto tile_block = [&](int t) -> int {
    return __builtin_amdgcn_readfirstlane(s_bt[(t * kTile) >> bs_log2]);
  };
  auto tile_offset = [&](int t, int blk) -> int64_t {
    return (int64_t)(blk < 0 ? 0 : blk) * block_stride + head_off +
           (int64_t)((start + t * kTile) & (bs - 1)) * CCH;
  };

  f32x4_t acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // head col, log2 units (the same in the 4 lanes of a column)
  float l_part = 0.f;       // sum of this lane's own weights

  // K operand and V chunks of a tile, one tile ahead of the arithmetic
  uint4 kop[KLD];
  uint4 vreg[VPL];
  auto load_k = [&](int64_t off) {
#pragma unroll
    for (int j = 0; j < KLD; ++j)
      kop[j] = load_kv<kKeep>(kcache + off + col * CCH + (kFp8 ? grp + 4 * j : 4 * j + grp));
  };
  auto load_v = [&](int64_t off) {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int idx = lane + kWave * i;
      vreg[i] = load_kv<kKeep>(vcache + off + (idx / CCH) * CCH + idx % CCH);
    }
  };

  auto process = [&](int t, int blk, int64_t off_next, auto prefetch) {
    constexpr bool kPrefetch = decltype(prefetch)::value;
    const int tok0 = start + t * kTile;
    const bool valid = blk >= 0;

    // V rows of the tile into this wave's region (chunk c of row r at
    // c ^ (r & SWZ)); rows past the context (or of an invalid block) are
    // zeroed, they may hold anything, NaN included
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int idx = lane + kWave * i;
      const int r = idx / CCH, c = idx % CCH;
      const uint4 v = (valid && tok0 + r < n) ? vreg[i] : make_uint4(0, 0, 0, 0);
      if constexpr (kFp8) {  // 16 codes -> BF16 chunks 2c, 2c + 1 (exact), one chunk at a time
        uint4 w[2];
        k_as_query(FP8{}, v, w);
        vt[r * DCH + ((2 * c) ^ (r & SWZ))] = w[0];
        vt[r * DCH + ((2 * c + 1) ^ (r & SWZ))] = w[1];
        __builtin_amdgcn_sched_barrier(0);
      } else {
        vt[r * DCH + (c ^ (r & SWZ))] = v;
      }
    }

    // scores of keys tok0 + 4 grp + i for head col
    f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KLD; ++j) {
      if constexpr (kFp8) {
        uint4 kq[2];
        k_as_query(FP8{}, kop[j], kq);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kq[0]),
                                                    qop[2 * j], sc, 0, 0, 0);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kq[1]),
                                                    qop[2 * j + 1], sc, 0, 0, 0);
      } else {
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kop[j]), qop[j],
                                                    sc, 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kPrefetch) {
      load_k(off_next);
      load_v(off_next);
    }
    __builtin_amdgcn_sched_barrier(0);

    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = tok0 + 4 * grp + i;
      sv[i] = (valid && tok < n) ? sc[i] * score_scale : -INFINITY;
    }
    // online softmax per head: the column's 16 scores sit in lanes col,
    // col + 16, col + 32, col + 48 (4 each)
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = pair_max<16>(mx);
    mx = pair_max<32>(mx);
    // rescale only when a head's maximum grew by more than 2^8 (weights of
    // up to 2^8 stay far from float32 / BF16 overflow)
    const float m_new = fmaxf(m_run, mx);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run + 8.f) != 0) {
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
      l_part *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
      m_run = m_new;
    }
    const float moff = m_run == -INFINITY ? 0.f : m_run;
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pf = fast_exp2(sv[i] - moff);
      ph[i] = (uint32_t)__builtin_bit_cast(unsigned short, static_cast<__bf16>(pf));
      const float hi = __uint_as_float(ph[i] << 16);
      pl[i] = (uint32_t)__builtin_bit_cast(unsigned short, static_cast<__bf16>(pf - hi));
      l_part += hi + __uint_as_float(pl[i] << 16);
    }
    const i16x4_t p_hi = __builtin_bit_cast(i16x4_t, make_uint2(ph[0] | (ph[1] << 16), ph[2] | (ph[3] << 16)));
    const i16x4_t p_lo = __builtin_bit_cast(i16x4_t, make_uint2(pl[0] | (pl[1] << 16), pl[2] | (pl[3] << 16)));

    // O^T += V^T P^T over the tile's 16 keys, 16 dims at a time
    const int vrow = 4 * grp + col / 4;  // the key row this lane supplies
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int dim = 16 * dt + 4 * (col % 4);
      const int c = dim / 8, half = (dim / 4) & 1;
      const char* src = reinterpret_cast<const char*>(vt + vrow * DCH + (c ^ (vrow & SWZ))) + 8 * half;
      const i16x4_t vop = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)src);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, p_hi, acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, p_lo, acc[dt], 0, 0, 0);
    }
  };

  int t = wave;
  if (t < ntiles) {
    int blk = tile_block(t);
    load_k(tile_offset(t, blk));
    load_v(tile_offset(t, blk));
    for (; t + kWaves < ntiles; t += kWaves) {
      if constexpr (kWaves == 8) {  // the priority rule of the VALU kernel
        __builtin_amdgcn_sched_barrier(0);
        const int done = (t - wave) / kWaves;
        if (lane == 0) s_prog[wave] = done;
        const int partner = __builtin_amdgcn_readfirstlane(s_prog[wave ^ 4]);
        if (done > partner) __builtin_amdgcn_s_setprio(0);
        else __builtin_amdgcn_s_setprio(1);
        __builtin_amdgcn_sched_barrier(0);
      }
      const int blk_next = tile_block(t + kWaves);
      process(t, blk, tile_offset(t + kWaves, blk_next), std::true_type{});
      blk = blk_next;
    }
    process(t, blk, 0, std::false_type{});
    if constexpr (kWaves == 8) __builtin_amdgcn_s_setprio(0);
  }

  // ---- wave totals per head, into this wave's region (its V rows are done)
  float l_col = pair_sum<16>(l_part);
  l_col = pair_sum<32>(l_col);
  if (grp == 0 && col < G) {
    s_m[wave][col] = m_run;
    s_l[wave][col] = l_col;
  }
  float4* s_acc = reinterpret_cast<float4*>(vt);  // [G][D / 4]
  if (col < G) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      s_acc[col * (D / 4) + 4 * dt + grp] = make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
  }
  __syncthreads();

  // ---- merge the waves and write o (normalised), m, l
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
      const float4 x = reinterpret_cast<const float4*>(s_region[w])[g * (D / 4) + d4];
      o.x += sw * x.x; o.y += sw * x.y; o.z += sw * x.z; o.w += sw * x.w;
    }
    const float inv = out_scale / L;
    o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
    const int64_t head = (int64_t)seq * a.num_q_heads + (int64_t)kvh * G + g;
    if (nparts == 1 && !has_prefix) {
      reinterpret_cast<float4*>(a.out)[head * (D / 4) + d4] = o;
    } else {
      const int64_t slot = partial_slot(a, s_plan, seq, part, nparts, kvh * G + g);
      reinterpret_cast<float4*>(a.part_o)[slot * (D / 4) + d4] = o;
      if (d4 == 0) {
        a.part_ml[2 * slot] = M;
        a.part_ml[2 * slot + 1] = L;
      }
    }
  }
  };  // unit

  run_units<T::kBytes>(a, s_plan, keep, unit);
}

// Merge of the per-partition partials of one (sequence, query head):
// out = sum_p w_p o_p / sum_p w_p with w_p = l_p * 2^(m_p - max_p m_p), over
// partials with l_p > 0 (a partial that saw no key adds nothing; if none saw
// one the row is zero). A copy-on-write group member's partials are its
// shared-prefix splits (from the prefix pass) followed by its tail's
// partitions. Persistent over rows; when the plan gave every sequence one
// partition and there are no groups, the partition kernel already wrote every
// row and the launch ends at once.
template <int D>
__global__ __launch_bounds__(kWave) void decode_merge_kernel(DecodeArgs a) {
  constexpr int PER = D / kWave;  // 1, 2 or 4 floats per lane
  constexpr int kBatch = 8;       // entries whose outputs are loaded together
  const int P = a.plan->part_tokens;
  if (a.plan->max_nparts <= 1 && a.num_groups == 0) return;
  const int full_total = a.plan->full_total;
  const int rows = a.num_seqs * a.num_q_heads;
  const int lane = threadIdx.x;
  for (int row = blockIdx.x; row < rows; row += gridDim.x) {
    const int seq = row / a.num_q_heads, h = row % a.num_q_heads;
    // (the first slot is read whatever the partition count turns out to be,
    // so that its load does not wait on the length's; it is used only for
    // a sequence of several partitions, for which the plan wrote it)
    int n = a.context_lens[seq];
    const int first_slot = a.full_pre[seq];
    n = n < 0 ? 0 : n;
    n = n > a.ctx_limit ? a.ctx_limit : n;
    const bool grouped = a.num_groups > 0 && seq >= a.cu_groups[0] &&
                         seq < a.cu_groups[a.num_groups];
    const int pos0 = grouped ? a.seq_start[seq] : 0;
    n = n > pos0 ? n - pos0 : 0;
    const int nparts = (n + P - 1) / P;          // tail partitions (0 for an empty tail)
    const int npre = pos0 > 0 ? a.pre_splits : 0;  // shared-prefix splits
    if (npre == 0 && nparts <= 1) continue;  // written by the partition kernel
    const int total = npre + (nparts > 0 ? nparts : 1);
    const int first = nparts > 1 ? first_slot : 0;
    // (m, l) and partial output of entry k: prefix splits, then tail partitions
    auto ml_of = [&](int k) -> const float* {
      if (k < npre) return a.pre_ml + 2 * (((int64_t)seq * a.num_q_heads + h) * npre + k);
      const int p = k - npre;
      const int e = p < nparts - 1 ? first + p : full_total + seq;
      return a.part_ml + 2 * ((int64_t)e * a.num_q_heads + h);
    };
    auto o_of = [&](int k) -> const float* {
      if (k < npre) return a.pre_o + (((int64_t)seq * a.num_q_heads + h) * npre + k) * D;
      const int p = k - npre;
      const int e = p < nparts - 1 ? first + p : full_total + seq;
      return a.part_o + ((int64_t)e * a.num_q_heads + h) * D;
    };
    // The first kBatch entries' outputs go out together with the (m, l)
    // loads (lane k: entry k), so that the row costs two dependent loads.
    // An empty partial (l = 0) may leave its output unwritten: it enters by
    // a select, never as a product with zero.
    float ob[kBatch][PER];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float* po = o_of(j < total ? j : 0) + lane * PER;
#pragma unroll
      for (int e = 0; e < PER; ++e) ob[j][e] = po[e];
    }
    float M = -INFINITY;
    for (int k = lane; k < total; k += kWave) {
      const float* ml = ml_of(k);
      if (ml[1] > 0.f) M = fmaxf(M, ml[0]);
    }
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) M = fmaxf(M, __shfl_xor(M, m));
    float o[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = 0.f;
    float L = 0.f;
    for (int k0 = 0; k0 < total; k0 += kWave) {
      const int k = k0 + lane;
      float w_lane = 0.f;
      if (k < total) {
        const float* ml = ml_of(k);
        w_lane = ml[1] > 0.f ? ml[1] * fast_exp2(ml[0] - M) : 0.f;
      }
      L += w_lane;
      const int cnt = total - k0 < kWave ? total - k0 : kWave;
      for (int j0 = 0; j0 < cnt; j0 += kBatch) {
        if (k0 + j0 > 0) {  // later batches: their outputs, loaded together
#pragma unroll
          for (int j = 0; j < kBatch; ++j) {
            const float* po = o_of(j0 + j < cnt ? k0 + j0 + j : k0) + lane * PER;
#pragma unroll
            for (int e = 0; e < PER; ++e) ob[j][e] = po[e];
          }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const float w = __shfl(w_lane, j0 + j < cnt ? j0 + j : 0);
          const bool use = j0 + j < cnt && w > 0.f;
#pragma unroll
          for (int e = 0; e < PER; ++e) o[e] = use ? __builtin_fmaf(w, ob[j][e], o[e]) : o[e];
        }
      }
    }
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) L += __shfl_xor(L, m);
    const float inv = L > 0.f ? 1.f / L : 0.f;
    float* out = a.out + (int64_t)row * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) out[e] = o[e] * inv;
  }
}

// Zero fill of a decode workspace (a kernel rather than a memset, so that it
// can be captured in a graph).
__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * 256)
    p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<uint4*>(p), n16);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Host side.

// Partial slots a workspace holds beyond one per sequence. The plan aims at
// one or two units per CU; the partitions it makes stay below this many more
// than one per sequence for any batch (and far below for 256 CUs).
constexpr int64_t kSpareSlots = 2048;

DecodeLaunch decode_launch_shape(int num_seqs, int num_kv_heads, int block_size,
                                 int max_context_len) {
  // The plan picks the partition size per call between part_floor and
  // part_cap. The workspace holds unit_slots partial slots; part_floor is the
  // smallest size (a power-of-two multiple of 256) at which every batch
  // within max_context_len fits them: a sequence of n tokens takes
  // max(1, ceil(n / P)) slots. unit_slots is the partition count at 256
  // tokens, capped at a modest figure unless the largest partitions need more.
  (void)num_kv_heads;
  DecodeLaunch r;
  r.waves = decode_waves_per_workgroup();
  r.part_cap = kMaxPartBlocks * block_size < 8192 ? kMaxPartBlocks * block_size : 8192;
  const int64_t seqs = num_seqs < kPlanSeqs ? num_seqs : kPlanSeqs;
  const int64_t ctx = max_context_len > 1 ? max_context_len : 1;
  auto parts_at = [&](int64_t p) { return seqs * ((ctx + p - 1) / p); };
  const int64_t at_cap = parts_at(r.part_cap);
  int64_t slots = seqs + kSpareSlots > at_cap ? seqs + kSpareSlots : at_cap;
  if (parts_at(256) < slots) slots = parts_at(256);
  r.unit_slots = slots;
  int p = 256;  // a multiple of 16 * 8 waves
  while (p < r.part_cap && parts_at(p) > slots) p *= 2;
  r.part_floor = p;
  r.max_parts = (int)((ctx + p - 1) / p);
  return r;
}

namespace {

int device_cus() {
  static int cus[64] = {0};  // per device, filled on first use
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    cus[dev] = (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) ==
                    hipSuccess && v > 0)
                   ? v
                   : 256;
  }
  return cus[dev];
}

// Work units per CU the plan aims for on ragged batches: fewer, larger
// partitions cost less per unit, more give the ticketed tail finer grain.
// Batches whose sequences share prompt blocks take 2 (with 1, every sequence
// of the shared-prompt batch is a single ticketed unit, and rollouts no
// longer read their shared blocks together: 170 -> 205 us); others take 1
// (ragged 32-sequence layer 108.5 -> 106.5 us, E4M3 70.7 -> 66.7 us, mixed
// step 305 -> 300 us). The environment override (both cases) exists for
// tuning sweeps only.
static int units_override() {
  static const int v = [] {
    const char* s = std::getenv("PA_DECODE_UNITS_PER_CU");
    const int x = s ? std::atoi(s) : 0;
    return x > 0 ? x : 0;
  }();
  return v;
}
int units_per_cu() { return units_override() ? units_override() : 2; }
int units_per_cu_unshared() { return units_override() ? units_override() : 1; }

template <typename Kernel>
int resident_per_cu(Kernel k, int threads) {
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k, threads, 0) != hipSuccess ||
      blocks < 1)
    blocks = 1;
  return blocks;
}

}  // namespace

// Launch of a partition kernel (NW waves per workgroup) and the merge kernel.
template <int D, int QueryBytes, int NW, auto Kernel>
static hipError_t launch_kernel(const DecodeArgs& a, hipStream_t stream) {
  static const int per_cu = resident_per_cu(Kernel, NW * kWave);
  const int cus = device_cus();
  // Batches above kPlanSeqs sequences run as consecutive launches of at most
  // kPlanSeqs sequences each, sharing the workspace in stream order.
  for (int s0 = 0; s0 < a.num_seqs; s0 += kPlanSeqs) {
    DecodeArgs c = a;
    c.num_seqs = a.num_seqs - s0 < kPlanSeqs ? a.num_seqs - s0 : kPlanSeqs;
    c.out = a.out + (int64_t)s0 * a.num_q_heads * D;
    c.query = static_cast<const char*>(a.query) + (int64_t)s0 * a.num_q_heads * D * QueryBytes;
    c.block_tables = a.block_tables + (int64_t)s0 * a.max_blocks_per_seq;
    c.context_lens = a.context_lens + s0;
    c.plan_cus = cus;
    c.plan_units_per_cu = units_per_cu();
    c.plan_units_unshared = units_per_cu_unshared();
    const int64_t most_units = (int64_t)c.num_seqs * c.num_kv_heads * c.max_parts;
    const int64_t slots = (int64_t)cus * per_cu;
    const int64_t grid = most_units < slots ? most_units : slots;
    hipLaunchKernelGGL(Kernel, dim3((unsigned)grid), dim3(NW * kWave), 0, stream, c);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t rows = (int64_t)c.num_seqs * c.num_q_heads;
    // up to 8 one-wave workgroups per CU: each row is a short chain of
    // dependent loads, so rows run side by side rather than in turn
    const int64_t mgrid = rows < 8 * (int64_t)cus ? rows : 8 * (int64_t)cus;
    hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)mgrid), dim3(kWave), 0, stream, c);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

template <typename T, int D, int G, int NW>
static hipError_t launch_nw(const DecodeArgs& a, hipStream_t stream) {
  return launch_kernel<D, T::Query::kBytes, NW, decode_partition_kernel<T, D, G, NW>>(a, stream);
}

template <typename T, int D, int G>
static hipError_t launch_t(const DecodeArgs& a, int waves, hipStream_t stream) {
  // Groups of 8 query heads over BF16 caches, and groups of 8 (and of 4 at
  // d >= 128) over E4M3 caches, run on the matrix cores (their VALU forms
  // wait on their own arithmetic). BF16 at d = 256 exceeds the 256 VGPRs of
  // an 8-wave workgroup and uses 4 waves.
  constexpr bool kFp8 = std::is_same<T, FP8>::value;
  constexpr bool kMfma = (std::is_same<T, BF16>::value && G == 8) ||
                         (kFp8 && (G == 8 || (G == 4 && D >= 128)));
  if constexpr (kMfma) {
    constexpr int kNw = (!kFp8 && D > 128) ? 4 : 8;
    return launch_kernel<D, 2, kNw, decode_mfma_kernel<T, D, G, kNw>>(a, stream);
  } else {
    // 8-wave workgroups are limited to 256 VGPRs per lane; the d = 256 shapes
    // with 8 query heads per KV head or float32 data, float32 at d = 128 with
    // 8 query heads, and FP8 with 8 query heads per KV head (16 accumulators
    // per head and lane) need more and use 4 waves.
    constexpr bool kFits8 = !(D == 256 && (G == 8 || T::kBytes == 4)) &&
                            !(D == 128 && G == 8 && T::kBytes == 4) && G * (16 / T::kBytes) <= 64;
    if constexpr (kFits8) {
      if (waves == 8) return launch_nw<T, D, G, 8>(a, stream);
    }
    return launch_nw<T, D, G, 4>(a, stream);
  }
}

template <typename T, int D>
static hipError_t launch_g(const DecodeArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_t<T, D, 1>(a, a.waves, stream);
    case 2: return launch_t<T, D, 2>(a, a.waves, stream);
    case 4: return launch_t<T, D, 4>(a, a.waves, stream);
    case 8: return launch_t<T, D, 8>(a, a.waves, stream);
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

hipError_t launch_decode(const DecodeArgs& a, KvType kv, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  switch (kv) {
    case KvType::BF16: return launch_d<BF16>(a, group, stream);
    case KvType::F32: return launch_d<F32>(a, group, stream);
    case KvType::FP8: return launch_d<FP8>(a, group, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
