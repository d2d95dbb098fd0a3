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
// Per tile of KT keys (64 for 8-wave workgroups, else 32) and wave:
//   S^T[KT x 16] = K[KT x D] . Q^T[D x 16]   A = K rows (LDS, chunk-swizzled),
//                                             B = Q^T (this lane's query row,
//                                             held in registers)
//   O^T[D x 16] += V^T[D x KT] . P^T[KT x 16] A = V^T (LDS, transposed when the
//                                             tile is staged), B = P^T (this
//                                             lane's own softmax weights)
// With the accumulator layout of the 16x16 MFMA (lane l holds rows
// 4*(l/16)+i of column l%16) both S^T and O^T keep a query row in the lanes
// l%16 == row, so the online softmax is lane-local up to a 4-lane reduction.
// P enters the PV product as two BF16 terms (hi + lo, 16 significant bits);
// the running sum takes the float32 weights. In each 32-key step of PV the
// B operand takes the 8 weights a lane holds for keys
// {4q..4q+3, 16+4q..16+4q+3} (q = l/16) of that step; V^T columns are stored
// in that same key order, so the contraction pairs every weight with its
// key's row.

#include "pa_device.hpp"
#include "pa_internal.hpp"

#include <cstdlib>
#include <type_traits>

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// LDS column of key k of a tile in a V^T row. Each 32-key step of the PV
// product keeps its own 32 columns, in which keys 4q..4q+3 -> 8q..8q+3 and
// keys 16+4q..16+4q+3 -> 8q+4..8q+7.
__device__ __forceinline__ int vt_slot(int k) {
  const int j = k & 31;
  return (k & ~31) + ((j < 16) ? (8 * (j >> 2) + (j & 3)) : (8 * ((j - 16) >> 2) + 4 + (j & 3)));
}

__device__ __forceinline__ uint32_t pack_lo(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);  // lo16(x) | lo16(y) << 16
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);  // hi16(x) | hi16(y) << 16
}


// Schedule of a run of NR operand reads from LDS, each feeding M matrix
// products: the first kAhead reads go out together and every read after
// them follows the products of the read kAhead before it, so kAhead reads
// are in flight while the products run.
constexpr int kAhead = 4;
template <int NR, int M>
__device__ __forceinline__ void interleave_reads() {
  __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);  // LDS reads
#pragma unroll
  for (int i = 0; i < NR - kAhead; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, M, 0);     // matrix products
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, M * kAhead, 0);
}

template <int D, int G, int HPW, int MW, int KT>
struct PrefillShape {
  static_assert(KT == 32 || KT == 64, "key tile");
  static constexpr int HG = G / HPW;              // head groups (waves across heads)
  static constexpr int NW = HG >= MW ? HG : MW;   // waves per workgroup (at least MW)
  static constexpr int RT = NW / HG;              // 16-row sub-tiles per workgroup
  static constexpr int ROWS = 16 * RT;            // query rows per workgroup
  static constexpr int NT = NW * kWave;           // threads
  static constexpr int DCH = D / 8;               // 16-byte chunks per K/V row
  static constexpr int SWZ = (DCH < 16 ? DCH : 16) - 1;  // K chunk swizzle mask
  static constexpr int KSTEPS = D / 32;           // MFMA k-steps of QK^T
  static constexpr int DTILES = D / 16;           // 16-row tiles of O^T
  static constexpr int QB = KT / 16;              // 16-key row blocks of S^T per tile
  static constexpr int PSTEPS = KT / 32;          // 32-key k-steps of PV per tile
  // bf16 per V^T row in LDS: 64-key rows take 16 pad elements (8 left a
  // nine-fold count of LDS bank conflicts); 32-key rows keep 8, so that two
  // 4-wave workgroups still fit in a CU's LDS
  static constexpr int VT_STRIDE = KT == 64 ? KT + 16 : KT + 8;
  static constexpr int KCHUNKS = KT * DCH;        // K chunks per tile
  static constexpr int VJOBS = (KT / 4) * (D / 8);  // 4-key x 8-dim V jobs
  // K staging: TPR threads per key row, each loading KPT chunks of that row
  static constexpr int TPR = (NT / KT) < DCH ? (NT / KT) : DCH;
  static constexpr int KPT = DCH / TPR;
  static constexpr int VPT = (VJOBS + NT - 1) / NT;       // V jobs per thread
  // Two register stages of staged tiles, for one head per wave at d <= 128
  // and for 4-wave workgroups (at d = 256 the 8-wave shape ran slower with
  // the second set: 248 VGPRs)
  static constexpr bool kDeep = HPW == 1 && (D <= 128 || NW == 4);
  static constexpr bool kAllV = VJOBS % NT == 0;  // every thread has VPT jobs
};

constexpr int kPfMaxBlocks = 1024;  // table entries one context split may span

// Workgroup barrier that orders LDS only: global loads in flight (the
// prefetch of later tiles) stay in flight across it, where __syncthreads()
// would wait for them.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// 8 E4M3 codes (an 8-byte cache chunk) as 8 bfloat16 (a 16-byte LDS chunk):
// exact, every E4M3 value being a bfloat16 value.
__device__ __forceinline__ u32x4_t fp8x8_to_bf16x8(const uint2& c) {
  u32x4_t r;
  r.x = fp8x2_to_bf16x2<false>(c.x);
  r.y = fp8x2_to_bf16x2<true>(c.x);
  r.z = fp8x2_to_bf16x2<false>(c.y);
  r.w = fp8x2_to_bf16x2<true>(c.y);
  return r;
}

// T: cache element type, BF16 or FP8 (E4M3 codes). An E4M3 cache is staged
// through the same LDS layout: every 16-byte BF16 chunk of a row (8 dims)
// corresponds to an 8-byte chunk of 8 codes at the same chunk index, which is
// loaded and converted on its way to LDS.
template <typename T, int D, int G, int HPW, int MW, int KT>
__global__ __launch_bounds__((PrefillShape<D, G, HPW, MW, KT>::NT))
__attribute__((amdgpu_waves_per_eu(1, 2))) void prefill_kernel(PrefillArgs a) {
  using S = PrefillShape<D, G, HPW, MW, KT>;
  constexpr bool kFp8 = std::is_same<T, FP8>::value;
  // cache chunk: 16 bytes of 8 bfloat16, or 8 bytes of 8 codes
  using CC = typename std::conditional<kFp8, uint2, uint4>::type;
  constexpr int DCH = S::DCH;
  constexpr int kKeyTile = KT;
  constexpr int kVtStride = S::VT_STRIDE;
  __shared__ uint4 k_lds[2][kKeyTile * DCH];                          // swizzled K rows
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[2][D * kVtStride];  // V^T
  __shared__ int s_bt[kPfMaxBlocks];

  // XCD-aware order: the hardware deals consecutive workgroup ids to the 8
  // XCDs in turn, so ids are regrouped so that all row tiles of one (KV head,
  // split) run on one XCD and share its L2 copy of that split's K/V.
  const int n_rt = gridDim.x;
  const int total = n_rt * gridDim.y * gridDim.z;
  int lin = blockIdx.x + n_rt * (blockIdx.y + gridDim.y * blockIdx.z);
  if (a.xcd_remap && total % 8 == 0) lin = (lin % 8) * (total / 8) + lin / 8;
  const int row_tile = lin % n_rt;
  const int kvh = (lin / n_rt) % gridDim.y;
  const int zz = lin / (n_rt * gridDim.y);
  const int seq = zz / a.kv_splits, split = zz % a.kv_splits;
  int q0 = a.cu_q_lens[seq];
  int L = a.cu_q_lens[seq + 1] - q0;
  if (a.prefix_mode) {  // group bounds kept within the decode batch
    const int q1 = min(max(q0 + L, 0), a.total_q);
    q0 = min(max(q0, 0), a.total_q);
    L = max(q1 - q0, 0);
  }
  const int r0 = row_tile * S::ROWS;
  const int bs_log2 = a.block_size_log2;
  const int bs = 1 << bs_log2;
  int n = a.context_lens[seq];
  n = n > a.ctx_limit ? a.ctx_limit : n;
  if (a.prefix_mode) {
    // shared prefix of a copy-on-write group: its whole blocks only. One
    // workgroup per group records where each member's tail starts, for the
    // decode of the tails and the merge that follow in stream order.
    n = n < 0 ? 0 : n & ~(bs - 1);
    if (row_tile == 0 && kvh == 0 && split == 0)
      for (int r = threadIdx.x; r < L; r += S::NT) a.seq_start[q0 + r] = n;
  } else if (L > n) {
    return;  // malformed chunk (longer than its context): nothing defined to compute
  }
  if (r0 >= L) return;
  const int base_pos = n - L;  // position of chunk row 0 (causal chunks)

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int lrow = lane % 16, lq = lane / 16;
  // this wave: HPW query heads of the group, one 16-row sub-tile; every K/V
  // operand read from LDS feeds one product per head
  const int head0 = kvh * G + (wave % S::HG) * HPW;
  const int rsub = wave / S::HG;
  const int my_row = r0 + rsub * 16 + lrow;          // chunk row of this lane's query
  const int qrow = my_row < L ? my_row : L - 1;       // clamp padding rows (not written)

  // Q^T operands: query row my_row, dims 32*ks + 8*lq .. +8, per head. The
  // scores are scaled inside the exponent by c = |scale * log2(e)|; for a
  // negative scale the query's sign bits are flipped instead (exact), and a
  // zero scale becomes the smallest normal float, whose products with finite
  // scores round the weights to exactly 1, as the zero scale would.
  // (E4M3 cache: the head's positive K scale multiplies every score, so it
  // folds into c; the V scale multiplies the output.)
  const uint32_t qflip = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  const float k_scale = kFp8 ? a.k_scale[kvh] : 1.f;
  const float v_scale = kFp8 ? a.v_scale[kvh] : 1.f;
  const float c_exp = fmaxf(fabsf(a.scale_log2) * k_scale, 1.17549435e-38f);
  bf16x8_t qop[HPW][S::KSTEPS];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(a.query) +
                        ((int64_t)(q0 + qrow) * a.num_q_heads + head0 + hh) * DCH;
#pragma unroll
    for (int ks = 0; ks < S::KSTEPS; ++ks)
      qop[hh][ks] = __builtin_bit_cast(bf16x8_t, qp[4 * ks + lq] ^ qflip);
  }

  // Key range of this split: keys visible to some row of the workgroup.
  const int last_row = min(r0 + S::ROWS, L) - 1;
  const int kmax = a.prefix_mode ? n : base_pos + last_row + 1;
  // Prefix mode: row my_row (member q0 + my_row) sees keys below both the
  // shared prefix and its own context; a wave with a row that stops short of
  // the prefix masks every tile.
  int member_limit = n - 1;
  if (a.prefix_mode) {
    int nm = a.member_lens[q0 + qrow];
    nm = nm < 0 ? 0 : (nm > a.ctx_limit ? a.ctx_limit : nm);
    member_limit = min(n, nm) - 1;
  }
  const bool wave_short =
      a.prefix_mode && __builtin_amdgcn_ballot_w64(member_limit < n - 1) != 0;
  const int ntiles = (kmax + kKeyTile - 1) / kKeyTile;
  const int per_split = (ntiles + a.kv_splits - 1) / a.kv_splits;
  const int kt_begin = split * per_split;
  const int kt_end = min(ntiles, kt_begin + per_split);

  // (in cache chunks: DCH per row for either element type)
  const CC* kcache = reinterpret_cast<const CC*>(a.key_cache);
  const CC* vcache = reinterpret_cast<const CC*>(a.value_cache);
  const int64_t block_stride = (int64_t)a.num_kv_heads * bs * DCH;
  const int64_t head_off = (int64_t)kvh * bs * DCH;

  // Table entries of the split's keys, staged once (-1: outside the pool).
  const int blk_first = (kt_begin * kKeyTile) >> bs_log2;
  {
    const int key_end = min(kt_end * kKeyTile, n);
    const int nblk = key_end > kt_begin * kKeyTile ? ((key_end + bs - 1) >> bs_log2) - blk_first : 0;
    // (prefix mode: the group's first member holds the shared blocks)
    const int32_t* bt =
        a.block_tables + (int64_t)(a.prefix_mode ? q0 : seq) * a.max_blocks_per_seq + blk_first;
    for (int i = tid; i < nblk && i < kPfMaxBlocks; i += S::NT) {
      const int e = bt[i];
      s_bt[i] = (e >= 0 && (int64_t)e < a.num_blocks) ? e : -1;
    }
  }
  __syncthreads();

  // Global chunk offset of key k's row. Keys past the context (and entries
  // outside the pool) read block 0 instead: their scores are masked and
  // their V rows zeroed, so the address only has to be valid.
  auto row_base = [&](int k) -> int64_t {
    const int i = (k >> bs_log2) - blk_first;
    const int e = (k < n && i < kPfMaxBlocks) ? s_bt[i] : -1;  // split rule keeps i in range
    return (int64_t)(e < 0 ? 0 : e) * block_stride + head_off + (int64_t)(k & (bs - 1)) * DCH;
  };

  // Tile staging, split in two so that later tiles' global loads are in
  // flight while the current tile's products run: load_into issues them into
  // a register set, store_from writes a set (K swizzled, V transposed) into
  // an LDS buffer.
  // K: thread t stages chunks (t % TPR) + TPR * i of key row t / TPR.
  // V: a job stages 4 consecutive keys (one block) x 8 dims.
  // (threads beyond the tile's rows, which only some shapes have, load a
  // duplicate row and store nothing; the loads stay unconditional so that the
  // staging registers are never placed in scratch memory)
  const int k_row = tid / S::TPR, k_c0 = tid % S::TPR;
  const bool k_active = k_row < kKeyTile;
  const int k_row_c = k_active ? k_row : kKeyTile - 1;
  // (K staging uses native vectors: copied as plain structs, the registers
  // ended up in scratch memory)
  using KRegs = u32x4_t[S::KPT];
  using VRegs = CC[S::VPT][4];
  KRegs kreg;
  VRegs vreg;
  auto load_into = [&](int kt, KRegs& kr, VRegs& vr) {
    const int key0 = kt * kKeyTile;
    {
      const CC* src = kcache + row_base(key0 + k_row_c) + k_c0;
#pragma unroll
      for (int i = 0; i < S::KPT; ++i) {
        if constexpr (kFp8) {
          const u32x2_t c = *reinterpret_cast<const u32x2_t*>(src + S::TPR * i);
          kr[i] = u32x4_t{c.x, c.y, 0u, 0u};  // converted when stored
        } else {
          kr[i] = *reinterpret_cast<const u32x4_t*>(src + S::TPR * i);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < S::VPT; ++j) {
      const int job = tid + j * S::NT;
      if (S::kAllV || job < S::VJOBS) {
        const int kg = job % (kKeyTile / 4), dg = job / (kKeyTile / 4);
        const CC* src = vcache + row_base(key0 + 4 * kg) + dg;
#pragma unroll
        for (int r = 0; r < 4; ++r) vr[j][r] = src[r * DCH];
      }
    }
  };
  auto store_from = [&](int buf, int kt, KRegs& kr, VRegs& vr) {
    const int key0 = kt * kKeyTile;
    if (key0 + kKeyTile > n) {  // tail tile: V rows past the context may hold NaN
#pragma unroll
      for (int j = 0; j < S::VPT; ++j) {
        const int job = tid + j * S::NT;
        const int kg = job % (kKeyTile / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (key0 + 4 * kg + r >= n) zero_chunk(vr[j][r]);
      }
    }
    // K: chunk c of row r lives at c ^ (r & SWZ), so the 16 rows one MFMA
    // operand read touches fall in distinct banks
    if (k_active) {
#pragma unroll
      for (int i = 0; i < S::KPT; ++i) {
        const int c = k_c0 + S::TPR * i;
        u32x4_t w = kr[i];
        if constexpr (kFp8) w = fp8x8_to_bf16x8(make_uint2(w.x, w.y));
        *reinterpret_cast<u32x4_t*>(&k_lds[buf][k_row * DCH + (c ^ (k_row & S::SWZ))]) = w;
      }
    }
    // V^T: each job transposes 4 keys x 8 dims
#pragma unroll
    for (int j = 0; j < S::VPT; ++j) {
      const int job = tid + j * S::NT;
      if (S::kAllV || job < S::VJOBS) {
        const int kg = job % (kKeyTile / 4), dg = job / (kKeyTile / 4);
        const int slot = vt_slot(4 * kg);
        uint4 rows[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (kFp8) {
            const u32x4_t w = fp8x8_to_bf16x8(vr[j][r]);
            rows[r] = make_uint4(w.x, w.y, w.z, w.w);
          } else {
            rows[r] = vr[j][r];
          }
        }
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
          *reinterpret_cast<uint2*>(&vt_lds[buf][d * kVtStride + slot]) = even;
          *reinterpret_cast<uint2*>(&vt_lds[buf][(d + 1) * kVtStride + slot]) = odd;
        }
      }
    }
  };

  f32x4_t acc[HPW][S::DTILES];
  float m_run[HPW];   // this lane's query row, per head, log2 units
  float l_part[HPW];  // sum of this lane's weights, per head
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
#pragma unroll
    for (int i = 0; i < S::DTILES; ++i) acc[hh][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[hh] = -INFINITY;
    l_part[hh] = 0.f;
  }

  // One key tile in LDS buffer buf: S^T products, then after_scores() (where
  // the caller issues later tiles' loads), the masked online softmax and the
  // PV products.
  auto attend_tile = [&](int kt, int buf, auto&& after_scores) {
    const int key0 = kt * kKeyTile;

    // ---- S^T = K Q^T for keys key0..key0+KT-1 (16-key row blocks), per head
    f32x4_t sc[HPW][S::QB];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
      for (int qb = 0; qb < S::QB; ++qb) sc[hh][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Waves raise their priority while they issue matrix products: of the
    // two waves sharing a SIMD, the one that reaches its products first
    // keeps the matrix unit while the other runs its softmax.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < S::KSTEPS; ++ks) {
      const int c = 4 * ks + lq;
#pragma unroll
      for (int qb = 0; qb < S::QB; ++qb) {
        const int kr = 16 * qb + lrow;
        const bf16x8_t kop = __builtin_bit_cast(bf16x8_t, k_lds[buf][kr * DCH + (c ^ (kr & S::SWZ))]);
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh)
          sc[hh][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[hh][ks], sc[hh][qb], 0, 0, 0);
      }
    }
    interleave_reads<S::KSTEPS * S::QB, HPW>();

    __builtin_amdgcn_s_setprio(0);
    // Later tiles' global loads go out once the score products have been
    // issued: issued before them, the compiler made those products wait for
    // the loads.
    after_scores();

    // last key this row may see; tiles that need the mask
    const int limit = a.prefix_mode ? member_limit : base_pos + my_row;
    const bool diag = a.prefix_mode
                          ? (wave_short || key0 + kKeyTile > n)
                          : (key0 + kKeyTile - 1 > base_pos + r0 || key0 + kKeyTile > n);
    bf16x8_t pop_hi[HPW][S::PSTEPS], pop_lo[HPW][S::PSTEPS];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      // ---- causal / context mask on the unscaled scores (lane: keys 16qb + 4lq + i)
      float sv[4 * S::QB];
#pragma unroll
      for (int qb = 0; qb < S::QB; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[4 * qb + i] = sc[hh][qb][i];
      if (diag) {
#pragma unroll
        for (int qb = 0; qb < S::QB; ++qb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int k = key0 + 16 * qb + 4 * lq + i;
            sv[4 * qb + i] = (k <= limit && k < n) ? sv[4 * qb + i] : -INFINITY;
          }
      }

      // ---- online softmax over this lane's query row, in log2 units (c_exp > 0,
      // so the largest scaled score is c_exp times the largest score)
      float mx = sv[0];
#pragma unroll
      for (int i = 1; i < 4 * S::QB; ++i) mx = fmaxf(mx, sv[i]);
      mx = pair_max<16>(mx);
      mx = pair_max<32>(mx);
      mx *= c_exp;
      // Rescale only when some row's maximum grew by more than 2^8: the
      // softmax does not depend on the offset subtracted, and weights of up
      // to 2^8 are far from float32 / BF16 overflow. This keeps the rescale
      // of the accumulators off almost every tile.
      const float m_new = fmaxf(m_run[hh], mx);
      if (__builtin_amdgcn_ballot_w64(m_new > m_run[hh] + 8.f) != 0) {
        const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run[hh] - m_new);
        l_part[hh] *= alpha;
#pragma unroll
        for (int i = 0; i < S::DTILES; ++i) acc[hh][i] *= alpha;
        m_run[hh] = m_new;
      }
      // Each weight p is carried as p_hi + p_lo, both BF16 (p_hi = RNE(p),
      // p_lo = RNE(p - p_hi)): 16 significant bits instead of 8, so the PV
      // product on the BF16 matrix cores keeps the weights' float32 accuracy
      // to about 2^-17 relative; the running sum takes p itself. Weights are
      // rounded in pairs (one packed conversion per pair). PV step j takes
      // the weights of row blocks 2j and 2j + 1.
      const float moff = m_run[hh] == -INFINITY ? 0.f : m_run[hh];
#pragma unroll
      for (int j = 0; j < S::PSTEPS; ++j) {
        uint32_t wh[4], wl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x2_t pf;
          pf.x = fast_exp2(__builtin_fmaf(sv[8 * j + 2 * i], c_exp, -moff));
          pf.y = fast_exp2(__builtin_fmaf(sv[8 * j + 2 * i + 1], c_exp, -moff));
          wh[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pf, bf16x2_t));
          f32x2_t r;
          r.x = pf.x - __uint_as_float(wh[i] << 16);
          r.y = pf.y - __uint_as_float(wh[i] & 0xffff0000u);
          wl[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2_t));
          l_part[hh] += pf.x + pf.y;
        }
        pop_hi[hh][j] = __builtin_bit_cast(bf16x8_t, make_uint4(wh[0], wh[1], wh[2], wh[3]));
        pop_lo[hh][j] = __builtin_bit_cast(bf16x8_t, make_uint4(wl[0], wl[1], wl[2], wl[3]));
      }
    }

    // ---- O^T += V^T (P_hi + P_lo)^T, one V^T operand read for all heads
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int dt = 0; dt < S::DTILES; ++dt) {
#pragma unroll
      for (int j = 0; j < S::PSTEPS; ++j) {
        const bf16x8_t vop = __builtin_bit_cast(
            bf16x8_t,
            *reinterpret_cast<const uint4*>(&vt_lds[buf][(16 * dt + lrow) * kVtStride + 32 * j + 8 * lq]));
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
          acc[hh][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop_hi[hh][j], acc[hh][dt], 0, 0, 0);
          acc[hh][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop_lo[hh][j], acc[hh][dt], 0, 0, 0);
        }
      }
    }
    interleave_reads<S::DTILES * S::PSTEPS, 2 * HPW>();
    __builtin_amdgcn_s_setprio(0);
  };

  if constexpr (S::kDeep) {
    // Two register stages, so that two tiles are in flight behind the one
    // being attended: step i attends tile i, writes tile i + 1 (set c, loaded
    // one step earlier) into the other buffer and loads tile i + 2 into set
    // n; the sets swap roles every step. The per-step barrier orders LDS only
    // (lds_barrier), so set n's loads stay in flight across it.
    KRegs kreg2;
    VRegs vreg2;
    const int ntl = kt_end - kt_begin;
    if (ntl > 0) {
      load_into(kt_begin, kreg, vreg);
      store_from(0, kt_begin, kreg, vreg);
    }
    if (ntl > 1) load_into(kt_begin + 1, kreg, vreg);
    lds_barrier();
    auto step = [&](int i, KRegs& kc, VRegs& vc, KRegs& kn, VRegs& vn) {
      // (the last two steps load the split's last tile again into a set
      // that is never stored: issued unconditionally, the loads keep the
      // wait counts static, so waiting for set c never waits for set n)
      attend_tile(kt_begin + i, i & 1, [&] {
        load_into(kt_begin + min(i + 2, ntl - 1), kn, vn);
      });
      if (i + 1 < ntl) store_from((i & 1) ^ 1, kt_begin + i + 1, kc, vc);
      lds_barrier();  // next buffer complete; this one free for reuse
    };
    int i = 0;
    for (; i + 1 < ntl; i += 2) {
      step(i, kreg, vreg, kreg2, vreg2);
      step(i + 1, kreg2, vreg2, kreg, vreg);
    }
    if (i < ntl) step(i, kreg, vreg, kreg2, vreg2);
  } else {
    if (kt_begin < kt_end) {
      load_into(kt_begin, kreg, vreg);
      store_from(0, kt_begin, kreg, vreg);
    }
    __syncthreads();
    for (int kt = kt_begin; kt < kt_end; ++kt) {
      const int buf = (kt - kt_begin) & 1;
      const bool has_next = kt + 1 < kt_end;
      attend_tile(kt, buf, [&] {
        if (has_next) load_into(kt + 1, kreg, vreg);
      });
      if (has_next) store_from(buf ^ 1, kt + 1, kreg, vreg);
      __syncthreads();  // next buffer complete; this one free for reuse
    }
  }

  // ---- row totals and output, per head
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    float l_row = pair_sum<16>(l_part[hh]);
    l_row = pair_sum<32>(l_row);
    if (my_row >= L) continue;
    const int64_t orow = (int64_t)(q0 + my_row) * a.num_q_heads + head0 + hh;
    const float inv = l_row > 0.f ? v_scale / l_row : 0.f;
    float* dst;
    if (a.kv_splits == 1 && !a.prefix_mode) {
      dst = a.out + orow * D;
    } else {
      const int64_t slot = orow * a.kv_splits + split;
      dst = a.part_o + slot * D;
      if (lq == 0) {
        a.part_ml[2 * slot] = m_run[hh];
        a.part_ml[2 * slot + 1] = l_row;
      }
    }
    float4* o = reinterpret_cast<float4*>(dst);
#pragma unroll
    for (int dt = 0; dt < S::DTILES; ++dt)
      o[4 * dt + lq] = make_float4(acc[hh][dt][0] * inv, acc[hh][dt][1] * inv,
                                   acc[hh][dt][2] * inv, acc[hh][dt][3] * inv);
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

// Heads of a GQA group one wave holds (the environment override exists for
// tuning sweeps only).
int prefill_heads_per_wave(int group) {
  static const int want = [] {
    const char* s = std::getenv("PA_PREFILL_HPW");
    const int v = s ? std::atoi(s) : 0;
    return v == 1 || v == 2 || v == 4 ? v : 1;
  }();
  int h = want < group ? want : group;
  return h < 1 ? 1 : h;
}

// Least waves per workgroup: more waves give a workgroup more 16-row
// sub-tiles, so each staged K/V tile serves more query rows. Groups of 4
// query heads take 8 waves (two sub-tiles of 16 rows per head), which
// measured faster than 4 waves on a 512-row chunk against a 4096-token
// context; other groups keep 4. The environment override exists for tuning
// sweeps only.
int prefill_min_waves(int group) {
  static const int v = [] {
    const char* s = std::getenv("PA_PREFILL_WAVES");
    const int x = s ? std::atoi(s) : 0;
    return x == 4 || x == 8 ? x : 0;
  }();
  return v ? v : (group == 4 ? 8 : 4);
}

// Heads per wave for this group and head size: four heads of d = 256 exceed
// the register file, and with 8 waves per workgroup (at most 256 VGPRs) a
// wave holds at most 256 / d heads.
int prefill_group_heads_per_wave(int group, int head_dim) {
  const int mw = prefill_min_waves(group);
  int hpw = prefill_heads_per_wave(group);
  if (head_dim > 128 && hpw > 2) hpw = 2;
  while (mw == 8 && hpw * head_dim > 256) hpw /= 2;
  return hpw;
}

int prefill_rows_per_workgroup(int group, int head_dim) {
  const int mw = prefill_min_waves(group);
  const int hpw = prefill_group_heads_per_wave(group, head_dim);
  const int hg = group / hpw;
  const int nw = hg >= mw ? hg : mw;
  return 16 * (nw / hg);
}

// Keys per staged tile: 64 for 8-wave workgroups of at most 2 heads per
// wave (the per-tile barrier, softmax reductions and staging then serve twice
// the matrix work), else 32: 4-wave workgroups would double their staging
// registers, and 4 heads per wave would spill. The environment override
// exists for tuning sweeps only.
int prefill_key_tile(int group, int head_dim) {
  static const int v = [] {
    const char* s = std::getenv("PA_PREFILL_KEYTILE");
    const int x = s ? std::atoi(s) : 0;
    return x == 32 || x == 64 ? x : 0;
  }();
  if (prefill_min_waves(group) != 8 || prefill_group_heads_per_wave(group, head_dim) > 2) return 32;
  return v ? v : 64;
}

int prefill_kv_splits(int num_seqs, int max_q_len, int num_q_heads, int num_kv_heads,
                      int head_dim, int max_context_len) {
  // Split the keys of each row tile until the launch has about 2048 waves
  // (two per SIMD on 256 CUs), keeping at least 8 key tiles per split.
  const int group = num_q_heads / num_kv_heads;
  const int rows = prefill_rows_per_workgroup(group, head_dim);
  const int kt = prefill_key_tile(group, head_dim);
  const int64_t wgs = (int64_t)num_seqs * num_kv_heads * ((max_q_len + rows - 1) / rows);
  const int waves = (rows / 16) * (group / prefill_group_heads_per_wave(group, head_dim));
  static const int env_target = [] {
    const char* s = std::getenv("PA_PREFILL_TARGET_WGS");
    const int v = s ? std::atoi(s) : 0;
    return v > 0 ? v : 0;
  }();
  const int target = env_target ? env_target : 2048 / waves;
  int splits = 1;
  while (splits < 8 && wgs * splits < target && (max_context_len / 32) / (2 * splits) >= 8)
    splits *= 2;
  // Each split's keys must fit the staged table. A split holds at most
  // ceil(ntiles / splits) tiles of kt keys, starting on a tile boundary: at
  // most max_context_len / splits + 2 * kt keys, i.e. at most
  // max_context_len / (16 * splits) + 2 * kt / 16 + 1 blocks of 16 tokens.
  const int64_t span = (int64_t)(kPfMaxBlocks - 2 * kt / 16 - 2) * 16;
  while ((int64_t)splits * span < max_context_len) ++splits;
  return splits;
}

// Context splits of the shared-prefix pass of a grouped decode. Its
// workgroups are 4-wave ones (rows per workgroup: 16 per wave and head of the
// group, 64 / G rows when G <= 4) over whole 32-key tiles; the prefix of each
// group is split until the launch has about kPrefixTargetWgs workgroups,
// keeping at least 256 keys per split, then further if a split's keys would
// not fit the staged table. Fewer splits mean fewer partials for the merge to
// read; the environment override exists for tuning sweeps only.
int prefix_pass_splits(int num_groups, int max_group_size, int num_q_heads, int num_kv_heads,
                       int max_prefix_len) {
  static const int target = [] {
    const char* s = std::getenv("PA_PREFIX_TARGET_WGS");
    const int v = s ? std::atoi(s) : 0;
    return v > 0 ? v : 256;
  }();
  const int group = num_q_heads / num_kv_heads;
  const int nw = group > 4 ? group : 4;
  const int rows = 16 * (nw / group);
  const int64_t wgs =
      (int64_t)num_groups * num_kv_heads * ((max_group_size + rows - 1) / rows);
  int splits = 1;
  while (splits < 32 && wgs * splits < target && max_prefix_len / (2 * splits) >= 256)
    splits *= 2;
  const int64_t span = (int64_t)(kPfMaxBlocks - 6) * 16;
  while ((int64_t)splits * span < max_prefix_len) ++splits;
  return splits;
}

template <typename T, int D, int G, int HPW, int MW, int KT>
static hipError_t launch_pf(const PrefillArgs& a_in, hipStream_t stream) {
  static const int remap = [] {
    const char* s = std::getenv("PA_PREFILL_XCD");
    return s ? std::atoi(s) : 1;
  }();
  PrefillArgs a = a_in;
  a.xcd_remap = remap;
  using S = PrefillShape<D, G, HPW, MW, KT>;
  dim3 grid((a.max_q_len + S::ROWS - 1) / S::ROWS, a.num_kv_heads, a.num_seqs * a.kv_splits);
  hipLaunchKernelGGL((prefill_kernel<T, D, G, HPW, MW, KT>), grid, dim3(S::NT), 0, stream, a);
  hipError_t err = hipGetLastError();
  // (prefix mode: the decode merge combines these partials with the tails')
  if (err != hipSuccess || a.kv_splits == 1 || a.prefix_mode) return err;
  hipLaunchKernelGGL((prefill_merge_kernel<D>), dim3(a.num_q_heads, a.total_q), dim3(kWave), 0,
                     stream, a);
  return hipGetLastError();
}

template <typename T, int D, int G, int HPW, int MW>
static hipError_t launch_pk(const PrefillArgs& a, hipStream_t stream) {
  if constexpr (MW == 8 && HPW <= 2) {
    if (prefill_key_tile(G, D) == 64) return launch_pf<T, D, G, HPW, MW, 64>(a, stream);
  }
  return launch_pf<T, D, G, HPW, MW, 32>(a, stream);
}

template <typename T, int D, int G, int MW>
static hipError_t launch_ph(const PrefillArgs& a, hipStream_t stream) {
  const int hpw = prefill_group_heads_per_wave(G, D);
  if constexpr (G >= 4 && D <= 128 && (MW == 4 || 4 * D <= 256)) {
    if (hpw == 4) return launch_pk<T, D, G, 4, MW>(a, stream);
  }
  if constexpr (G >= 2 && (MW == 4 || 2 * D <= 256)) {
    if (hpw == 2) return launch_pk<T, D, G, 2, MW>(a, stream);
  }
  return launch_pk<T, D, G, 1, MW>(a, stream);
}

template <typename T, int D, int G>
static hipError_t launch_pw(const PrefillArgs& a, hipStream_t stream) {
  const int mw = a.min_waves ? a.min_waves : prefill_min_waves(G);
  if (mw == 8) return launch_ph<T, D, G, 8>(a, stream);
  return launch_ph<T, D, G, 4>(a, stream);
}

template <typename T, int D>
static hipError_t launch_pg(const PrefillArgs& a, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_pw<T, D, 1>(a, stream);
    case 2: return launch_pw<T, D, 2>(a, stream);
    case 4: return launch_pw<T, D, 4>(a, stream);
    case 8: return launch_pw<T, D, 8>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_pd(const PrefillArgs& a, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: return launch_pg<T, 64>(a, stream);
    case 128: return launch_pg<T, 128>(a, stream);
    case 256: return launch_pg<T, 256>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  return a.kv_fp8 ? launch_pd<FP8>(a, stream) : launch_pd<BF16>(a, stream);
}

}  // namespace pa
