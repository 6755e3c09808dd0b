// Backward of the fused attention forward pass on gfx950: dQ, dK and dV of
// O = softmax(scale * Q K^T + mask) V for an upstream gradient dO.
//
// The CUTLASS Blackwell FMHA walk-through (trdm.cn, "CUTLASS Blackwell FMHA 示例完全解析",
// section "FMHA for Blackwell: Backward") splits the backward into a row sum of O * dO, a main
// pass that recomputes the probabilities from the forward's LSE and forms dQ, dK and dV (in a
// dK/dV kernel and a dQ kernel), and a conversion of dQ from fp32 to the output type.  With
// P = exp(scale * S - LSE) recomputed tile by tile:
//
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - delta),   delta_i = sum_d O_id dO_id,
//     dQ = scale * dS K,   dK = scale * dS^T Q,
//
// masked positions carrying P = 0 (the backward mask of the walk-through's fusion-point
// section: the forward masks with the causal offset 0 or Sk - Sq).
//
// CDNA4 design (two kernels, no atomics, deterministic; e4m3 inputs add a widening pass first):
// * dq_kernel: a workgroup owns 256 query rows of one (sequence, head), 32 per wave, with its Q
//   and dO rows held as MFMA B operands in registers.  It first forms the rows' statistics,
//   delta_i and LSE_i * log2(e) (+inf for a row with no key), from its dO fragment and the same
//   fragment of O (the walk-through's row sum of O * dO, so it needs no kernel of its own), and
//   stores them in a workspace of 64-row blocks [lse2[64], -delta[64]] for the dK/dV kernel; the
//   rows past a sequence's end in its last block get +inf and 0, so that kernel reads whole
//   blocks and padding rows yield P = 0.  64-key K/V tiles stream through a 3-stage
//   LDS ring (LDS-direct loads, one barrier per tile).  S^T = K Q^T and dP^T = V dO^T run on
//   v_mfma_f32_32x32x16 with K and V read row-wise from LDS; the accumulator layout of dS^T is
//   the B operand of dQ^T += K^T dS^T, whose A operand is K read transposed with
//   ds_read_b64_tr_b16 (the key order of the accumulator rows).  dQ is owned by one wave, so it
//   is scaled and converted in registers and stored once: the fp32 conversion step of the
//   walk-through folds into the epilogue.
// * dkdv_kernel: a workgroup owns 128 keys of one (sequence, K/V head) in four 32-key blocks,
//   each served by two waves on one SIMD: a P-wave holding K and a dS-wave holding V as B
//   operands in registers.  64-row Q/dO tiles (and their row statistics) stream through LDS
//   for every query head of the GQA group.  S = Q K^T and dP = dO V^T put the wave's keys in
//   the accumulator columns, so P and dS are directly the B operands of dV^T += dO^T P
//   (P-wave) and dK^T += Q^T dS (dS-wave), with dO^T and Q^T read transposed from LDS; P
//   passes from the P-wave to the dS-wave through LDS, one step behind.  dK and dV of a K/V
//   head sum over its group's query heads inside one workgroup.
// Masks, varlen and GQA follow fmha_fwd: buffer descriptors bounded to the sequence (rows past
// either end read 0 and are not written), the causal offset Sk_b - Sq_b for causal-qend, and
// tiles that no row of a wave sees skipped by that wave.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "fmha.h"
#include "fmha_device.h"

namespace fmha {
namespace bwd {

constexpr int kAuxRows = 64;                 // rows per block of the row-statistics workspace
constexpr int kAuxBlock = 2 * kAuxRows * 4;  // bytes per block: lse2[64], then -delta[64]
constexpr int kStages = 3;                   // LDS ring depth of both main kernels

constexpr int kKvBlocks = 4;            // dK/dV kernel: 32-key blocks per workgroup
constexpr int kKvWaves = 2 * kKvBlocks; // a P-wave and a dS-wave per key block
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int kKvN = 32 * kKvBlocks;    // keys per workgroup
constexpr int kKvM = kAuxRows;          // query rows per streamed tile

constexpr int kQWaves = 8;              // dQ kernel: waves per workgroup, 32 query rows each
constexpr int kQThreads = 64 * kQWaves;
constexpr int kQM = 32 * kQWaves;       // query rows per workgroup
constexpr int kQN = 64;                 // keys per streamed tile

constexpr int kSchedMfma = 0x008;  // scheduling-group masks of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedDsRead = 0x100;
constexpr int kPrefetch = 6;       // LDS reads kept in flight ahead of the MFMAs
constexpr int kChunksAhead = 1;    // dK/dV kernel: 16-row chunks of transposed reads in flight

struct Params {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* aux;            // workspace: row-statistics blocks
  uint32_t aux_bytes;
  const int32_t* cu_q;   // null for dense batches
  const int32_t* cu_k;
  int32_t B, Sq, Sk, H, H_kv, group;
  int32_t total_q;       // packed: LSE row length; dense: 0
  int32_t aux_bstride;   // dense: blocks per sequence (H * ceil(Sq / 64)); packed: 0
  int32_t aux_hstride;   // blocks between consecutive heads of one sequence
  int32_t n_tiles;       // dq: q tiles per sequence; dkdv: key tiles
  int32_t xcd_per;       // (sequence, head) pairs per XCD when their count is a multiple of 8
  int32_t rank_seqs;     // packed batch of at most 64 sequences: sequences taken longest first
  int32_t causal, qend;
  float scale, scale_log2;
};

struct Seq {
  int q_row0, Sq_b, k_row0, Sk_b;
};

__device__ inline Seq seq_bounds(const Params& p, int b) {
  Seq s;
  if (p.cu_q) {
    s.q_row0 = p.cu_q[b];
    s.Sq_b = p.cu_q[b + 1] - s.q_row0;
    s.k_row0 = p.cu_k[b];
    s.Sk_b = p.cu_k[b + 1] - s.k_row0;
  } else {
    s.q_row0 = b * p.Sq;
    s.Sq_b = p.Sq;
    s.k_row0 = b * p.Sk;
    s.Sk_b = p.Sk;
  }
  return s;
}

// First statistics block of sequence b (head 0).  Packed batches give sequence b the blocks
// from floor(cu_q[b] / 64) + b on, which never overlap the next sequence's.
__device__ inline int aux_seq_base(const Params& p, int b, int q_row0) {
  return p.cu_q ? (q_row0 >> 6) + b : b * p.aux_bstride;
}

// (pair, group) of a workgroup: round-robin dispatch puts workgroup x on XCD x % 8, so the
// pairs are dealt out per XCD and the workgroups of one pair share that XCD's L2.  Packed
// batches of at most 64 sequences (rank_seqs) take the sequences longest first, by query rows
// (by_q: the dK/dV kernel, whose key blocks see them) or by keys (the dQ kernel), with all the
// workgroups of a pair side by side; in batch order a long sequence's tiles can land behind every
// other sequence's and run one after another on one compute unit.
__device__ inline void decode_unit(const Params& p, int npairs, int* pair, int* grp, bool by_q) {
  const int x = blockIdx.x;
  if (p.rank_seqs) {
    int pr;
    if (p.xcd_per) {
      const int slot = x >> 3;
      pr = (slot / p.n_tiles) * 8 + (x & 7);
      *grp = slot % p.n_tiles;
    } else {
      pr = x / p.n_tiles;
      *grp = x % p.n_tiles;
    }
    const int heads = npairs / p.B;
    const int r = pr / heads;
    const int lane = threadIdx.x & 63;
    const int32_t* cu = by_q ? p.cu_q : p.cu_k;
    const int len_l = lane < p.B ? cu[lane + 1] - cu[lane] : -1;  // lane i: sequence i (B <= 64)
    int rank = 0;
    for (int j = 0; j < p.B; ++j) {
      const int len_j = __builtin_amdgcn_readlane(len_l, j);
      rank += (len_j > len_l) | ((len_j == len_l) & (j < lane));
    }
    const uint64_t of_r = __ballot(lane < p.B && rank == r);  // one lane: the ranks are 0 .. B-1
    *pair = (int)__builtin_ctzll(of_r) * heads + (pr - r * heads);
  } else if (p.xcd_per) {
    const int slot = x >> 3;
    *grp = slot / p.xcd_per;
    *pair = (x & 7) * p.xcd_per + slot % p.xcd_per;
  } else {
    *grp = x / npairs;
    *pair = x % npairs;
  }
}

__device__ inline i32x4 load_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// A operand of v_mfma_f32_32x32x16 read transposed from a row-major LDS tile: element
// (m = dim 32 db + l32, k = one of 16 tile rows starting at `rows`), the rows in the order of a
// 32x32 accumulator's rows (4 h32 + 0..3, then 8 + 4 h32 + 0..3).
__device__ inline i32x4 read_tr(uint32_t lane0, uint32_t lane1, int db, uint32_t rows) {
  const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)((lane0 ^ (64 * db)) + rows));
  const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)((lane1 ^ (64 * db)) + rows));
  const i32x4 a = {__builtin_bit_cast(int, __builtin_shufflevector(v0, v0, 0, 1)),
                   __builtin_bit_cast(int, __builtin_shufflevector(v0, v0, 2, 3)),
                   __builtin_bit_cast(int, __builtin_shufflevector(v1, v1, 0, 1)),
                   __builtin_bit_cast(int, __builtin_shufflevector(v1, v1, 2, 3))};
  return a;
}

// Stores a 32x32 accumulator block times f as 16-bit values, 16 bytes per lane: the block's
// rows are 32 consecutive dims of the output row given by the lane's column (lane l32, h32 holds
// rows 8 g + 4 h32 + 0..3).  A lane swap across the halves gives each lane dims 16 gp + 8 h32 ..
// + 7, which it writes at at + 2 * that dim; rows outside the descriptor are dropped.
template <int DT>
__device__ inline void store_block(const f32x16& a, float f, __amdgpu_buffer_rsrc_t r, uint32_t at, int h32) {
  typedef Elem<DT> T;
#pragma unroll
  for (int gp = 0; gp < 2; ++gp) {
    const int g0 = 2 * gp, g1 = 2 * gp + 1;
    auto r0 = __builtin_amdgcn_permlane32_swap(T::pack(a[4 * g0] * f, a[4 * g0 + 1] * f),
                                               T::pack(a[4 * g1] * f, a[4 * g1 + 1] * f), false, false);
    auto r1 = __builtin_amdgcn_permlane32_swap(T::pack(a[4 * g0 + 2] * f, a[4 * g0 + 3] * f),
                                               T::pack(a[4 * g1 + 2] * f, a[4 * g1 + 3] * f), false, false);
    const i32x4 w = {(int)r0[0], (int)r1[0], (int)r0[1], (int)r1[1]};
    __builtin_amdgcn_raw_buffer_store_b128(w, r, at + (uint32_t)(16 * gp + 8 * h32) * 2, 0, 0);
  }
}

// NC chains of v_mfma_f32_32x32x16 over the head dimension, interleaved: c[j] += sum_ks
// A_j[ks] B_j[ks], A_j[ks] the 16-byte row-wise LDS read at base[j] ^ (32 ks) (chunk 2 ks + h32 of
// the lane's row) and B_j = bj[ks] (j = 0, 2 take b0; 1, 3 take b1).  The reads run kPrefetch
// ahead of their MFMAs (pinned with scheduling groups: left alone, the compiler waits for each
// read right before its MFMA, and the matrix core idles for the LDS latency).
template <int DT, int KS, int NC>
__device__ inline void row_chains(f32x16 (&c)[NC], const uint32_t (&base)[NC], const i32x4 (&b0)[KS],
                                  const i32x4 (&b1)[KS]) {
  typedef Elem<DT> T;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const i32x4 a = *(const lds_i32x4*)(uintptr_t)(base[j] ^ (32 * ks));
      c[j] = T::mma(a, (j & 1) ? b1[ks] : b0[ks], c[j]);
    }
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kPrefetch, 0);
#pragma unroll
  for (int i = 0; i < NC * KS; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
  }
}

// ------------------------------------------------------------------------------------------
// dQ kernel: grid = B * H * n_tiles workgroups of kQThreads
// ------------------------------------------------------------------------------------------
template <int DT, int D, bool WIDE>
__global__ __launch_bounds__(kQThreads, 1) void dq_kernel(const Params p) {
  constexpr int E = 2;
  constexpr int RB = D * E;          // bytes per row
  constexpr int CPR = RB / 16;       // 16-byte chunks per row
  constexpr int TILE = kQN * RB;     // bytes per K or V tile
  constexpr int TBLK = TILE / 1024;  // 1 KiB LDS-direct loads per tile
  constexpr int LPW = 2 * TBLK / kQWaves;  // loads per wave per step (K and V)
  constexpr int STAGE = 2 * TILE;
  constexpr int KS = D / 16;
  constexpr int NDB = D / 32;
  static_assert(TILE % 1024 == 0 && (2 * TBLK) % kQWaves == 0 && LPW >= 1, "whole loads per wave");
  static_assert(LPW < 32, "vmcnt range");
  typedef Elem<DT> T;

  __shared__ __attribute__((aligned(1024))) char lds[kStages * STAGE];
  const uint32_t ring = (uint32_t)(uintptr_t)(lds_void*)lds;

  const int lane = threadIdx.x & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int l32 = lane & 31;
  const int h32 = lane >> 5;

  int bh, grp;
  decode_unit(p, p.B * p.H, &bh, &grp, false);
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int kvh = h / p.group;
  const Seq sq = seq_bounds(p, b);
  const int qt0 = (p.n_tiles - 1 - grp) * kQM;  // heaviest (latest rows) first
  if (qt0 >= sq.Sq_b) return;
  const int off = p.qend ? sq.Sk_b - sq.Sq_b : 0;
  const int q_last = min(qt0 + kQM, sq.Sq_b) - 1;
  const int k_end = p.causal ? min(sq.Sk_b, q_last + off + 1) : sq.Sk_b;
  const int n_steps = k_end > 0 ? (k_end + kQN - 1) / kQN : 0;

  const int qw0 = qt0 + 32 * wave_u;  // this wave's rows
  const int qi = qw0 + l32;           // this lane's row
  const bool wave_on = qw0 < sq.Sq_b;
  // last visible key of this lane's row, of the wave's first row, and of its last row
  const int lim_q = p.causal ? min(sq.Sk_b - 1, qi + off) : sq.Sk_b - 1;
  const int wave_lim = p.causal ? min(sq.Sk_b - 1, qw0 + off) : sq.Sk_b - 1;
  const int wave_max = p.causal ? min(sq.Sk_b - 1, qw0 + 31 + off) : sq.Sk_b - 1;

  // Byte offsets stay 32-bit however long the sequence: the Q, dO, O and dQ descriptors start
  // at the workgroup's first row, and each K/V tile load gets descriptors that start at its tile.
  const uint32_t qstride = (uint32_t)p.H * RB;
  const uint32_t kstride = (uint32_t)p.H_kv * RB;
  const size_t q_base = ((size_t)sq.q_row0 + qt0) * qstride;
  const size_t k_base = ((size_t)sq.k_row0 * p.H_kv + kvh) * RB;
  const uint32_t q_bytes = (uint32_t)min(sq.Sq_b - qt0, kQM) * qstride;
  const size_t k_len = sq.Sk_b > 0 ? (size_t)(sq.Sk_b - 1) * kstride + RB : 0;  // bytes from k_base
  const auto rq = make_rsrc((const char*)p.q + q_base, q_bytes);
  const auto rdo = make_rsrc((const char*)p.dout + q_base, q_bytes);
  const auto rdq = make_rsrc((const char*)p.dq + q_base, q_bytes);

  // the wave's Q and dO rows as B operands (row l32, dims 16 ks + 8 h32 ..); rows past the
  // sequence read 0
  i32x4 qf[KS], dof[KS];
  const uint32_t frag = (uint32_t)(qi - qt0) * qstride + (uint32_t)h * RB + 16 * h32;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = load_b128(rq, frag + 32 * ks);
    dof[ks] = load_b128(rdo, frag + 32 * ks);
  }
  // The row's statistics: delta = sum over the head dimension of O * dO (this lane holds half
  // the dims of its row, lane l ^ 32 the other half) and the LSE in log2 units.  Every lane of
  // the lower half stores its row into the workspace block of the dK/dV kernel when the block
  // holds a row of the sequence, as +inf and 0 past the sequence's end.
  float lse2 = __builtin_inff(), delta = 0.0f;
  {
    const auto ro = make_rsrc((const char*)p.o + q_base, q_bytes);
    float s = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const i32x4 of = load_b128(ro, frag + 32 * ks);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        s = __builtin_fmaf(T::lo((uint32_t)of[u]), T::lo((uint32_t)dof[ks][u]), s);
        s = __builtin_fmaf(T::hi((uint32_t)of[u]), T::hi((uint32_t)dof[ks][u]), s);
      }
    }
    s = wave_row_sum(s);
    if (qi < sq.Sq_b) {
      const float L = p.lse[p.cu_q ? (size_t)h * p.total_q + sq.q_row0 + qi : ((size_t)b * p.H + h) * p.Sq + qi];
      lse2 = L == -__builtin_inff() ? __builtin_inff() : L * 1.4426950408889634f;
      delta = s;
    }
    if (h32 == 0 && (qi & ~(kAuxRows - 1)) < sq.Sq_b) {
      float* blk = p.aux + (size_t)(aux_seq_base(p, b, sq.q_row0) + h * p.aux_hstride + qi / kAuxRows) * (kAuxBlock / 4);
      blk[qi % kAuxRows] = lse2;
      blk[kAuxRows + qi % kAuxRows] = -delta;
    }
  }

  // tile loads: load g of a step (0 .. 2 TBLK - 1; K first, then V) is wave g % kQWaves's
  uint32_t ld_off[LPW], ld_dst[LPW];
  bool ld_v[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int g = wave_u + kQWaves * i;
    const int gi = g % TBLK;
    const int pos = 64 * gi + lane;
    const int j = pos / CPR;
    ld_off[i] = (uint32_t)j * kstride + (((pos % CPR) ^ swz<CPR>(j)) * 16);
    ld_v[i] = g >= TBLK;
    ld_dst[i] = (uint32_t)((g >= TBLK ? TILE : 0) + 1024 * gi);
  }
  // K/V tiles: one descriptor pair over the sequence's keys when the host has seen that their
  // byte offsets fit 31 bits; otherwise (WIDE) descriptors placed at each tile, a few scalar
  // instructions more per tile (done always, they cost ~2% of the whole backward).
  i32x4 rk_seq = {}, rv_seq = {};
  if constexpr (!WIDE) {
    rk_seq = make_rsrc_words((const char*)p.k + k_base, (uint32_t)k_len);
    rv_seq = make_rsrc_words((const char*)p.v + k_base, (uint32_t)k_len);
  }
  auto load_step = [&](int n) __attribute__((always_inline)) {
    const uint32_t st = ring + (uint32_t)((n % kStages) * STAGE);
    if constexpr (!WIDE) {
      const uint32_t key0 = (uint32_t)(n * kQN) * kstride;
#pragma unroll
      for (int i = 0; i < LPW; ++i) lds_load16(ld_v[i] ? rv_seq : rk_seq, key0 + ld_off[i], st + ld_dst[i]);
    } else {  // descriptors over this tile's keys (rows past the sequence read 0)
      const size_t key0 = (size_t)(n * kQN) * kstride;
      const uint32_t bytes = k_len > key0 ? (uint32_t)min(k_len - key0, (size_t)kQN * kstride) : 0;
      const i32x4 rk = make_rsrc_words((const char*)p.k + k_base + key0, bytes);
      const i32x4 rv = make_rsrc_words((const char*)p.v + k_base + key0, bytes);
#pragma unroll
      for (int i = 0; i < LPW; ++i) lds_load16(ld_v[i] ? rv : rk, ld_off[i], st + ld_dst[i]);
    }
  };
  if (n_steps > 0) load_step(0);
  if (n_steps > 1) load_step(1);

  // per-lane LDS offsets: row-wise A reads of K and V (row l32, chunk 2 ks + h32), and the
  // transposed K reads (as the V^T reads of the forward kernel)
  const uint32_t k_lane = l32 * RB + ((h32 ^ swz<CPR>(l32)) * 16);
  const int g16 = (lane >> 4) & 1;
  const int s16 = lane & 15;
  const int t_row0 = 4 * h32 + (s16 >> 2);
  const int t_part = 2 * g16 + ((s16 & 3) >> 1);
  const uint32_t t_lane0 = t_row0 * RB + ((t_part ^ swz<CPR>(t_row0)) * 16) + 8 * (s16 & 1);
  const uint32_t t_lane1 = (t_row0 + 8) * RB + ((t_part ^ swz<CPR>(t_row0 + 8)) * 16) + 8 * (s16 & 1);

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  const float sl2 = p.scale_log2;

  for (int n = 0; n < n_steps; ++n) {
    if (n + 1 < n_steps)
      wait_vmcnt<LPW>();
    else
      wait_vmcnt<0>();
    phase_barrier();  // tile n is in LDS for every wave; stage (n + 2) % 3 is free
    if (n + 2 < n_steps) load_step(n + 2);
    const int kb = n * kQN;
    if (!wave_on || kb > wave_max) continue;  // no row of this wave sees a key of the tile
    const uint32_t st = ring + (uint32_t)((n % kStages) * STAGE);

    // S^T = K Q^T and dP^T = V dO^T: element r of block kb2 is key kb + 32 kb2 + 4 h32 +
    // 8 (r / 4) + r % 4, row qi
    f32x16 c4[4] = {};  // S^T block 0, dP^T block 0, S^T block 1, dP^T block 1
    {
      const uint32_t k0 = st + k_lane, k1 = k0 + (uint32_t)(32 * RB);
      const uint32_t base[4] = {k0, k0 + TILE, k1, k1 + TILE};
      row_chains<DT, KS, 4>(c4, base, qf, dof);
    }
    const f32x16 s[2] = {c4[0], c4[2]}, dp[2] = {c4[1], c4[3]};
    // P = exp2(scale log2(e) s - lse2) (0 where masked), dS = P (dP - delta), packed
    const bool special = kb + kQN - 1 > wave_lim;
    const int lim = lim_q - kb - 4 * h32;
    uint32_t pk[8 * 2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      float d[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb2][e], sl2, -lse2));
        if (special) pr = 32 * kb2 + 8 * (e >> 2) + (e & 3) <= lim ? pr : 0.0f;
        d[e] = pr * (dp[kb2][e] - delta);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) pk[8 * kb2 + i] = T::pack(d[2 * i], d[2 * i + 1]);
    }
    // dQ^T += K^T dS^T, 16 keys per MFMA (two transposed reads each, kept ahead of the MFMAs)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const i32x4 bp = {(int)pk[4 * c], (int)pk[4 * c + 1], (int)pk[4 * c + 2], (int)pk[4 * c + 3]};
      const uint32_t rows = (uint32_t)(16 * c * RB);
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] = T::mma(read_tr(st + t_lane0, st + t_lane1, db, rows), bp, acc[db]);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kPrefetch, 0);
#pragma unroll
    for (int i = 0; i < 4 * NDB; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
  }

  // dQ = scale * acc: lane holds row qi (rows past the sequence are dropped by the descriptor)
  if (!wave_on) return;
  const uint32_t at = (uint32_t)(qi - qt0) * qstride + (uint32_t)h * RB;
#pragma unroll
  for (int db = 0; db < NDB; ++db) store_block<DT>(acc[db], p.scale, rdq, at + 64 * db, h32);
}

// ------------------------------------------------------------------------------------------
// dK/dV kernel: grid = B * H_kv * n_tiles workgroups of kKvThreads
// ------------------------------------------------------------------------------------------
// Two waves share each SIMD and the same 32 keys.  The P-wave (waves 0-3) holds K and forms
// S = Q K^T, P and dV^T += dO^T P; it leaves P, rounded to the 16-bit type as the dV product
// consumes it, in LDS.  The dS-wave (waves 4-7) holds V and forms dP - delta = dO V^T - delta
// (the MFMAs accumulate onto -delta, read from the statistics block straight into the
// accumulators); one step later, after the barrier that publishes P, it forms
// dS = P (dP - delta) and dK^T += Q^T dS.  Each
// wave thus runs half of the four products of a tile (32 MFMAs per 64-row step), and the
// vector work of one wave (the exponentials, or the dS products) issues while the other
// wave's MFMAs run.  Q tiles stay in LDS one step longer than dO tiles for the dS-wave's
// transposed reads: 4 Q slots, 3 dO slots, 2 P slots.
template <int DT, int D, bool WIDE>
__global__ __launch_bounds__(kKvThreads, 1) void dkdv_kernel(const Params p) {
  constexpr int E = 2;
  constexpr int RB = D * E;
  constexpr int CPR = RB / 16;
  constexpr int TILE = kKvM * RB;    // bytes per Q or dO tile
  constexpr int TBLK = TILE / 1024;
  constexpr int LPW = 2 * TBLK / kKvWaves;  // Q and dO loads per wave per step
  constexpr int QSLOTS = 4, DOSLOTS = 3;
  constexpr int AUX_AT = (QSLOTS + DOSLOTS) * TILE;  // 4 statistics blocks of 1 KiB
  constexpr int P_AT = AUX_AT + 4 * 1024;            // 2 slots of P: 32 keys x 64 rows per key block
  constexpr int PBLK = 32 * kKvM * E;
  constexpr int PSLOT = kKvBlocks * PBLK;
  constexpr int KS = D / 16;
  constexpr int NDB = D / 32;
  static_assert(TILE % 1024 == 0 && (2 * TBLK) % kKvWaves == 0 && LPW >= 1, "whole loads per wave");
  static_assert(LPW + 1 < 32, "vmcnt range");
  typedef Elem<DT> T;

  __shared__ __attribute__((aligned(1024))) char lds[P_AT + 2 * PSLOT];
  const uint32_t ring = (uint32_t)(uintptr_t)(lds_void*)lds;

  const int lane = threadIdx.x & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int l32 = lane & 31;
  const int h32 = lane >> 5;
  const bool ds_wave = wave_u >= kKvBlocks;  // wave-uniform role
  const int kblk = wave_u & (kKvBlocks - 1);

  int bkv, grp;
  decode_unit(p, p.B * p.H_kv, &bkv, &grp, true);
  const int b = bkv / p.H_kv;
  const int kvh = bkv - b * p.H_kv;
  const Seq sq = seq_bounds(p, b);
  const int kb0 = grp * kKvN;  // key tile 0 sees the most rows: heaviest first
  if (kb0 >= sq.Sk_b) return;
  const int off = p.qend ? sq.Sk_b - sq.Sq_b : 0;
  const int kw0 = kb0 + 32 * kblk;  // this wave's keys
  const int key = kw0 + l32;        // this lane's key
  // rows below kb0 - off see no key of the workgroup
  const int qt_first = p.causal ? max(0, kb0 - off) / kKvM : 0;
  const int n_qt = (sq.Sq_b + kKvM - 1) / kKvM;
  const int nq = max(0, n_qt - qt_first);
  const int n_steps = nq * p.group;

  // Byte offsets stay 32-bit however long the sequence: the K, V, dK and dV descriptors start at
  // the workgroup's first key, and each Q/dO tile load gets descriptors that start at its tile.
  const uint32_t qstride = (uint32_t)p.H * RB;
  const uint32_t kstride = (uint32_t)p.H_kv * RB;
  const size_t q_base = (size_t)sq.q_row0 * qstride;
  const size_t k_base = ((size_t)sq.k_row0 + kb0) * kstride + (size_t)kvh * RB;
  const uint32_t k_bytes = (uint32_t)(min(sq.Sk_b - kb0, kKvN) - 1) * kstride + RB;
  const i32x4 raux = make_rsrc_words(p.aux, p.aux_bytes);
  // Q/dO tiles: one descriptor pair over the sequence's rows when the host has seen that their
  // byte offsets fit 31 bits; otherwise (WIDE) descriptors placed at each tile
  i32x4 rq_seq = {}, rdo_seq = {};
  if constexpr (!WIDE) {
    const uint32_t q_len = (uint32_t)sq.Sq_b * qstride;
    rq_seq = make_rsrc_words((const char*)p.q + q_base, q_len);
    rdo_seq = make_rsrc_words((const char*)p.dout + q_base, q_len);
  }

  // tile loads: load g of a step (0 .. 2 TBLK - 1; Q first, then dO) is wave g % kKvWaves's;
  // wave 0 also copies the step's statistics block (and the next one, unused) into LDS
  uint32_t ld_off[LPW], ld_dst[LPW];
  bool ld_do[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int g = wave_u + kKvWaves * i;
    const int gi = g % TBLK;
    const int pos = 64 * gi + lane;
    const int j = pos / CPR;
    ld_off[i] = (uint32_t)j * qstride + (((pos % CPR) ^ swz<CPR>(j)) * 16);
    ld_do[i] = g >= TBLK;
    ld_dst[i] = (uint32_t)(1024 * gi);
  }
  const int aux_b = aux_seq_base(p, b, sq.q_row0);
  auto q_slot = [&](int t) __attribute__((always_inline)) { return ring + (uint32_t)((t % QSLOTS) * TILE); };
  auto do_slot = [&](int t) __attribute__((always_inline)) {
    return ring + (uint32_t)((QSLOTS + t % DOSLOTS) * TILE);
  };
  auto aux_slot = [&](int t) __attribute__((always_inline)) { return ring + (uint32_t)(AUX_AT + (t % 4) * 1024); };
  auto p_slot = [&](int t) __attribute__((always_inline)) {
    return ring + (uint32_t)(P_AT + (t & 1) * PSLOT + kblk * PBLK);
  };
  auto load_step = [&](int t) __attribute__((always_inline)) {
    const int hi = t / nq;
    const int qt = qt_first + t - hi * nq;
    const int hq = kvh * p.group + hi;
    const uint32_t sq_ = q_slot(t), sd = do_slot(t);
    if constexpr (!WIDE) {
      const uint32_t base = (uint32_t)(qt * kKvM) * qstride + (uint32_t)hq * RB;
#pragma unroll
      for (int i = 0; i < LPW; ++i)
        lds_load16(ld_do[i] ? rdo_seq : rq_seq, base + ld_off[i], (ld_do[i] ? sd : sq_) + ld_dst[i]);
    } else {  // descriptors over the tile's rows of query head hq (rows past the sequence read 0)
      const size_t base = q_base + (size_t)(qt * kKvM) * qstride + (size_t)hq * RB;
      const uint32_t bytes = (uint32_t)(min(sq.Sq_b - qt * kKvM, kKvM) - 1) * qstride + RB;
      const i32x4 rq = make_rsrc_words((const char*)p.q + base, bytes);
      const i32x4 rdo = make_rsrc_words((const char*)p.dout + base, bytes);
#pragma unroll
      for (int i = 0; i < LPW; ++i) lds_load16(ld_do[i] ? rdo : rq, ld_off[i], (ld_do[i] ? sd : sq_) + ld_dst[i]);
    }
    if (wave_u == 0) {
      const uint32_t blk = (uint32_t)(aux_b + hq * p.aux_hstride + qt);
      lds_load16(raux, blk * kAuxBlock + 16 * lane, aux_slot(t));
    }
  };
  // first row of step t's tile, and whether no row of it sees this wave's keys
  auto step_q0 = [&](int t) __attribute__((always_inline)) { return (qt_first + t % nq) * kKvM; };
  auto skipped = [&](int t) __attribute__((always_inline)) {
    return p.causal && step_q0(t) + kKvM - 1 + off < kw0;
  };
  if (n_steps > 0) load_step(0);
  if (n_steps > 1) load_step(1);

  // the wave's K (P-wave) or V (dS-wave) rows as B operands (key l32, dims 16 ks + 8 h32 ..);
  // keys past the sequence read 0 (their columns are never stored).  They are waited for
  // here, together with the first two tiles: the compiler does not count the tile loads, so a
  // wait it placed inside the loop would drain the tiles in flight at every step.
  i32x4 kvf[KS];
  {
    const auto rkv = make_rsrc((const char*)(ds_wave ? p.v : p.k) + k_base, k_bytes);
    const uint32_t frag = (uint32_t)(key - kb0) * kstride + 16 * h32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kvf[ks] = load_b128(rkv, frag + 32 * ks);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(kvf[ks]));
  }

  // per-lane LDS offsets: row-wise A reads of Q and dO, transposed reads of both, and this
  // lane's 32 bytes of a 32-row half of P (two 1 KiB planes of 16 bytes per lane)
  const uint32_t r_lane = l32 * RB + ((h32 ^ swz<CPR>(l32)) * 16);
  const int g16 = (lane >> 4) & 1;
  const int s16 = lane & 15;
  const int t_row0 = 4 * h32 + (s16 >> 2);
  const int t_part = 2 * g16 + ((s16 & 3) >> 1);
  const uint32_t t_lane0 = t_row0 * RB + ((t_part ^ swz<CPR>(t_row0)) * 16) + 8 * (s16 & 1);
  const uint32_t t_lane1 = (t_row0 + 8) * RB + ((t_part ^ swz<CPR>(t_row0 + 8)) * 16) + 8 * (s16 & 1);
  const uint32_t p_lane = 16 * lane;

  f32x16 acc[NDB];  // dV^T (P-wave) or dK^T (dS-wave): 32 dims x the wave's 32 keys per block
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  const float sl2 = p.scale_log2;

  // Element r of a half qb's 32x32 block of S, dP, P or dS is row q0 + 32 qb + 4 h32 +
  // 8 (r / 4) + r % 4, key `key`.  MFMAs over one 16-row chunk of a half take P or dS packed in
  // that order, against the matching transposed read of dO or Q.  The reads of chunk
  // c + kChunksAhead are issued before the MFMAs of chunk c (pinned by scheduling barriers:
  // left alone, the compiler reuses one set of registers and waits for each read right before
  // its MFMA).
  auto chunk_mma = [&](uint32_t tile, const uint32_t (&pk)[16]) __attribute__((always_inline)) {
    constexpr int CA = kChunksAhead;
    i32x4 a[CA + 1][NDB];
#pragma unroll
    for (int c = 0; c < CA; ++c)
#pragma unroll
      for (int db = 0; db < NDB; ++db) a[c][db] = read_tr(tile + t_lane0, tile + t_lane1, db, (uint32_t)(16 * c * RB));
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c + CA < 4) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          a[(c + CA) % (CA + 1)][db] = read_tr(tile + t_lane0, tile + t_lane1, db, (uint32_t)(16 * (c + CA) * RB));
      }
      __builtin_amdgcn_sched_barrier(0);
      const i32x4 bp = {(int)pk[4 * c], (int)pk[4 * c + 1], (int)pk[4 * c + 2], (int)pk[4 * c + 3]};
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] = T::mma(a[c % (CA + 1)][db], bp, acc[db]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (!ds_wave) {
    // ---- P-wave: S, P (to LDS), dV ------------------------------------------------------
    for (int t = 0; t < n_steps; ++t) {
      if (t + 1 < n_steps) {
        if (wave_u == 0) wait_vmcnt<LPW + 1>(); else wait_vmcnt<LPW>();
      } else {
        wait_vmcnt<0>();
      }
      phase_barrier();  // step t is in LDS; the slots of step t + 2 are free
      if (t + 2 < n_steps) load_step(t + 2);
      if (skipped(t)) continue;
      const int q0 = step_q0(t);
      const uint32_t sq_ = q_slot(t);
      f32x16 c2[2] = {};  // S of the two halves
      {
        const uint32_t base[2] = {sq_ + r_lane, sq_ + r_lane + (uint32_t)(32 * RB)};
        row_chains<DT, KS, 2>(c2, base, kvf, kvf);
      }
      // P = exp2(scale log2(e) s - lse2), 0 where masked (padding rows: lse2 = +inf)
      const bool special = p.causal && q0 < kw0 + 31 - off;
      const int lim = key - off - q0 - 4 * h32;  // keep element r iff 32 qb + 8 (r / 4) + r % 4 >= lim
      const uint32_t sa = aux_slot(t);
      const uint32_t ps = p_slot(t);
      uint32_t pp[16];
      auto softmax = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const i32x4 l4 = *(const lds_i32x4*)(uintptr_t)(sa + 4 * (32 * qb + 8 * g + 4 * h32));
            float pr[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              pr[u] = __builtin_amdgcn_exp2f(
                  __builtin_fmaf(c2[qb][4 * g + u], sl2, -__builtin_bit_cast(float, (int)l4[u])));
              if constexpr (decltype(masked)::value) pr[u] = 32 * qb + 8 * g + u >= lim ? pr[u] : 0.0f;
            }
            pp[8 * qb + 2 * g] = T::pack(pr[0], pr[1]);
            pp[8 * qb + 2 * g + 1] = T::pack(pr[2], pr[3]);
          }
        }
      };
      if (special)
        softmax(std::true_type{});
      else
        softmax(std::false_type{});
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int pl = 0; pl < 2; ++pl) {
          const i32x4 w = {(int)pp[8 * qb + 4 * pl], (int)pp[8 * qb + 4 * pl + 1], (int)pp[8 * qb + 4 * pl + 2],
                           (int)pp[8 * qb + 4 * pl + 3]};
          *(lds_i32x4*)(uintptr_t)(ps + (uint32_t)(2048 * qb + 1024 * pl) + p_lane) = w;
        }
      chunk_mma(do_slot(t), pp);  // dV^T += dO^T P
    }
    if (n_steps > 0) phase_barrier();  // the dS-wave's last step reads the last P
  } else {
    // ---- dS-wave: dP, then one step later dS and dK ---------------------------------------
    f32x16 dp[2] = {};  // dP - delta of the previous step's tile
    auto ds_step = [&](int t) __attribute__((always_inline)) {  // dS and dK of step t's tile
      const uint32_t ps = p_slot(t);
      uint32_t pd[16];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        uint32_t pr[8];
#pragma unroll
        for (int pl = 0; pl < 2; ++pl) {
          const i32x4 w = *(const lds_i32x4*)(uintptr_t)(ps + (uint32_t)(2048 * qb + 1024 * pl) + p_lane);
#pragma unroll
          for (int i = 0; i < 4; ++i) pr[4 * pl + i] = (uint32_t)w[i];
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t a = pr[2 * g], c = pr[2 * g + 1];
          pd[8 * qb + 2 * g] = T::pack(T::lo(a) * dp[qb][4 * g], T::hi(a) * dp[qb][4 * g + 1]);
          pd[8 * qb + 2 * g + 1] = T::pack(T::lo(c) * dp[qb][4 * g + 2], T::hi(c) * dp[qb][4 * g + 3]);
        }
      }
      chunk_mma(q_slot(t), pd);  // dK^T += Q^T dS
    };
    for (int t = 0; t < n_steps; ++t) {
      if (t + 1 < n_steps)
        wait_vmcnt<LPW>();
      else
        wait_vmcnt<0>();
      phase_barrier();  // step t is in LDS, and P of step t - 1
      if (t + 2 < n_steps) load_step(t + 2);
      if (t > 0 && !skipped(t - 1)) ds_step(t - 1);
      if (skipped(t)) continue;
      const uint32_t sd = do_slot(t);
      const uint32_t sa = aux_slot(t) + 4 * kAuxRows;  // -delta of the tile's rows
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const i32x4 d4 = *(const lds_i32x4*)(uintptr_t)(sa + 4 * (32 * qb + 8 * g + 4 * h32));
#pragma unroll
          for (int u = 0; u < 4; ++u) dp[qb][4 * g + u] = __builtin_bit_cast(float, (int)d4[u]);
        }
      const uint32_t base[2] = {sd + r_lane, sd + r_lane + (uint32_t)(32 * RB)};
      row_chains<DT, KS, 2>(dp, base, kvf, kvf);
    }
    if (n_steps > 0) {
      phase_barrier();
      if (!skipped(n_steps - 1)) ds_step(n_steps - 1);
    }
  }

  // dK = scale * acc (dS-wave), dV = acc (P-wave): lane holds key `key` (keys past the
  // sequence are dropped by the descriptor)
  const auto rout = make_rsrc((char*)(ds_wave ? p.dk : p.dv) + k_base, k_bytes);
  const float f = ds_wave ? p.scale : 1.0f;
  const uint32_t at = (uint32_t)(key - kb0) * kstride;
#pragma unroll
  for (int db = 0; db < NDB; ++db) store_block<DT>(acc[db], f, rout, at + 64 * db, h32);
}

// ------------------------------------------------------------------------------------------
// e4m3 inputs: widened to bf16 in the workspace before the two kernels (exact: every e4m3fn
// value, subnormals and NaN included, is a bf16 value).  Tensor blockIdx.y of the table.  A wave
// takes 2 KiB of input per step as four 512-byte rows, lane j bytes 8j .. 8j + 7 of each, and
// writes each row's 1 KiB of bf16 with one contiguous store; a tail of fewer than 2 KiB goes 16
// bytes per thread.
// ------------------------------------------------------------------------------------------
constexpr int kWidenTensors = 5;  // q, o, dO, k, v
constexpr int kWidenThreads = 256;
constexpr int kWidenRows = 4;     // 512-byte input rows per wave and step

struct Widen {
  const void* src[kWidenTensors];
  void* dst[kWidenTensors];
  uint64_t n16[kWidenTensors];  // 16-byte chunks of e4m3 input (0: nothing to widen)
};

template <bool HI>
__device__ inline int widen2(int x) {  // e4m3 bytes 2 HI, 2 HI + 1 of x -> two bf16
  return __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, HI));
}

__global__ __launch_bounds__(kWidenThreads) void widen_e4m3_kernel(const Widen w) {
  const int t = blockIdx.y;
  const uint64_t n = w.n16[t];
  const char* src = (const char*)w.src[t];
  char* dst = (char*)w.dst[t];
  const int lane = threadIdx.x & 63;
  const uint64_t n_steps = n / (kWidenRows * 32);  // whole 2 KiB input steps
  const uint64_t waves = (uint64_t)gridDim.x * (kWidenThreads / 64);
  for (uint64_t u = ((uint64_t)blockIdx.x * kWidenThreads + threadIdx.x) / 64; u < n_steps; u += waves) {
    i32x2 x[kWidenRows];
#pragma unroll
    for (int r = 0; r < kWidenRows; ++r) x[r] = *(const i32x2*)(src + (u * kWidenRows + r) * 512 + 8 * lane);
#pragma unroll
    for (int r = 0; r < kWidenRows; ++r)
      *(i32x4*)(dst + (u * kWidenRows + r) * 1024 + 16 * lane) =
          i32x4{widen2<false>(x[r][0]), widen2<true>(x[r][0]), widen2<false>(x[r][1]), widen2<true>(x[r][1])};
  }
  const i32x4* src16 = (const i32x4*)src;
  i32x4* dst16 = (i32x4*)dst;
  for (uint64_t i = n_steps * kWidenRows * 32 + (uint64_t)blockIdx.x * kWidenThreads + threadIdx.x; i < n;
       i += (uint64_t)gridDim.x * kWidenThreads) {
    const i32x4 x = src16[i];
    dst16[2 * i] = i32x4{widen2<false>(x[0]), widen2<true>(x[0]), widen2<false>(x[1]), widen2<true>(x[1])};
    dst16[2 * i + 1] = i32x4{widen2<false>(x[2]), widen2<true>(x[2]), widen2<false>(x[3]), widen2<true>(x[3])};
  }
}

template <int DT, int D>
hipError_t launch(Params p, int n_q_tiles, int n_k_tiles, bool have_q, bool have_k, bool wide_k, bool wide_q,
                  hipStream_t stream) {
  if (have_q) {  // dQ and the row statistics; the dK/dV kernel after it reads the statistics
    const int64_t pairs = (int64_t)p.B * p.H;
    p.n_tiles = n_q_tiles;
    p.xcd_per = pairs % 8 == 0 ? (int32_t)(pairs / 8) : 0;
    if (wide_k)
      hipLaunchKernelGGL((dq_kernel<DT, D, true>), dim3((unsigned)(pairs * n_q_tiles)), dim3(kQThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((dq_kernel<DT, D, false>), dim3((unsigned)(pairs * n_q_tiles)), dim3(kQThreads), 0, stream, p);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (have_k) {
    const int64_t pairs = (int64_t)p.B * p.H_kv;
    p.n_tiles = n_k_tiles;
    p.xcd_per = pairs % 8 == 0 ? (int32_t)(pairs / 8) : 0;
    if (wide_q)
      hipLaunchKernelGGL((dkdv_kernel<DT, D, true>), dim3((unsigned)(pairs * n_k_tiles)), dim3(kKvThreads), 0, stream,
                         p);
    else
      hipLaunchKernelGGL((dkdv_kernel<DT, D, false>), dim3((unsigned)(pairs * n_k_tiles)), dim3(kKvThreads), 0, stream,
                         p);
    return hipGetLastError();
  }
  return hipSuccess;
}

// Shape checks and workspace size.  Fills the layout fields of p.
fmha_status plan(int32_t B, int32_t Sq, int32_t Sk, int32_t H, int32_t H_kv, int32_t D, const fmha_varlen* varlen,
                 Params* p, size_t* ws_bytes) {
  const bool packed = varlen != nullptr;
  if (B < 0 || Sq < 0 || Sk < 0 || H < 0 || H_kv < 0) return FMHA_ERR_INVALID_SHAPE;
  if (H > 0 && (H_kv < 1 || H % H_kv != 0)) return FMHA_ERR_INVALID_SHAPE;
  if (D != 32 && D != 64 && D != 128) return FMHA_ERR_INVALID_SHAPE;
  if (packed && (varlen->total_length_q < 0 || varlen->total_length_k < 0)) return FMHA_ERR_INVALID_SHAPE;
  const int64_t lim = (int64_t)1 << 31;
  // the kernels address one workgroup's rows (or one tile's) from a descriptor placed at them:
  // those byte offsets fit 31 bits; a sequence may be any length
  if ((int64_t)kQM * H * D * 2 >= lim || (int64_t)kKvN * H_kv * D * 2 >= lim ||
      (int64_t)kKvM * H * D * 2 >= lim)
    return FMHA_ERR_UNSUPPORTED;
  const int64_t nqb = (Sq + kAuxRows - 1) / kAuxRows;
  int64_t blocks;
  if (packed) {
    const int64_t hb = (int64_t)(varlen->total_length_q >> 6) + B + 1;
    if (hb >= lim) return FMHA_ERR_UNSUPPORTED;
    p->aux_hstride = (int32_t)hb;
    p->aux_bstride = 0;
    blocks = hb * H;
  } else {
    p->aux_hstride = (int32_t)nqb;
    if (nqb * H >= lim) return FMHA_ERR_UNSUPPORTED;
    p->aux_bstride = (int32_t)(nqb * H);
    blocks = (int64_t)B * H * nqb;
  }
  // the statistics loads read one block past the last
  if ((blocks + 1) * kAuxBlock >= lim) return FMHA_ERR_UNSUPPORTED;
  *ws_bytes = (size_t)blocks * kAuxBlock;
  p->B = B;
  p->Sq = Sq;
  p->Sk = Sk;
  p->H = H;
  p->H_kv = H_kv;
  p->group = H > 0 ? H / H_kv : 1;
  p->total_q = packed ? varlen->total_length_q : 0;
  return FMHA_OK;
}

// Workspace layout: the row-statistics blocks first, then, for e4m3 inputs, bf16 copies of q, o,
// dO, k and v (in that order), each at a 256-byte boundary.
struct WsLayout {
  size_t off[kWidenTensors];
  uint64_t n16[kWidenTensors];  // 16-byte chunks of e4m3 input per copy (0: no copy)
  size_t total;
};

inline WsLayout ws_layout(size_t stats_bytes, bool f8, int64_t rows_q, int64_t rows_k, int64_t H, int64_t H_kv,
                          int64_t D) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const uint64_t elems[kWidenTensors] = {(uint64_t)(rows_q * H * D), (uint64_t)(rows_q * H * D),
                                         (uint64_t)(rows_q * H * D), (uint64_t)(rows_k * H_kv * D),
                                         (uint64_t)(rows_k * H_kv * D)};
  WsLayout w;
  size_t at = up(stats_bytes);
  for (int t = 0; t < kWidenTensors; ++t) {
    w.off[t] = at;
    w.n16[t] = f8 ? elems[t] / 16 : 0;  // D is a multiple of 16
    if (f8) at += up(2 * (size_t)elems[t]);
  }
  w.total = f8 ? at : stats_bytes;
  return w;
}

}  // namespace bwd
}  // namespace fmha

// --------------------------------------------------------------------------------------
// C ABI
// --------------------------------------------------------------------------------------
extern "C" {

size_t fmha_bwd_workspace_size(int32_t B, int32_t Sq, int32_t Sk, int32_t H, int32_t H_kv, int32_t D,
                               fmha_dtype dtype, const fmha_varlen* varlen) {
  using namespace fmha::bwd;
  if ((int)dtype < 0 || (int)dtype > 2) return 0;
  Params p;
  size_t bytes = 0;
  if (plan(B, Sq, Sk, H, H_kv, D, varlen, &p, &bytes) != FMHA_OK) return 0;
  const int64_t rows_q = varlen ? varlen->total_length_q : (int64_t)B * Sq;
  const int64_t rows_k = varlen ? varlen->total_length_k : (int64_t)B * Sk;
  return ws_layout(bytes, dtype == FMHA_DTYPE_F8E4M3, rows_q, rows_k, H, H_kv, D).total;
}

fmha_status fmha_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                     void* dq, void* dk, void* dv, int32_t B, int32_t Sq, int32_t Sk, int32_t H, int32_t H_kv,
                     int32_t D, float scale, fmha_mask mask, fmha_dtype dtype, const fmha_varlen* varlen,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  using namespace fmha::bwd;
  const bool packed = varlen != nullptr;
  if (packed && (!varlen->cu_seqlens_q != !varlen->cu_seqlens_k)) return FMHA_ERR_NULL_POINTER;
  if (packed && !varlen->cu_seqlens_q) return FMHA_ERR_NULL_POINTER;
  Params p;
  size_t need = 0;
  const fmha_status st = plan(B, Sq, Sk, H, H_kv, D, varlen, &p, &need);
  if (st != FMHA_OK) return st;
  if ((int)dtype < 0 || (int)dtype > 2) return FMHA_ERR_UNSUPPORTED;
  if ((int)mask < 0 || (int)mask > 3) return FMHA_ERR_UNSUPPORTED;
  const bool f8 = dtype == FMHA_DTYPE_F8E4M3;
  const bool have_q = B > 0 && H > 0 && (packed ? varlen->total_length_q > 0 : Sq > 0);
  const bool have_k = B > 0 && H > 0 && (packed ? varlen->total_length_k > 0 : Sk > 0);
  if (have_q && (!q || !o || !dout || !lse || !dq)) return FMHA_ERR_NULL_POINTER;
  if (have_k && (!k || !v || !dk || !dv)) return FMHA_ERR_NULL_POINTER;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout | (uintptr_t)dq |
       (uintptr_t)dk | (uintptr_t)dv) & 15)
    return FMHA_ERR_MISALIGNED;
  if ((uintptr_t)lse & 3) return FMHA_ERR_MISALIGNED;
  if (!(scale > 0.0f) || !isfinite(scale)) return FMHA_ERR_INVALID_ARGUMENT;
  if (!have_q && !have_k) return FMHA_OK;
  // the dK/dV kernel reads the statistics of every row it visits; e4m3 inputs are widened into
  // the workspace first
  const int64_t rows_q = packed ? varlen->total_length_q : (int64_t)B * Sq;
  const int64_t rows_k = packed ? varlen->total_length_k : (int64_t)B * Sk;
  const WsLayout wl = ws_layout(need, f8, have_q ? rows_q : 0, have_k ? rows_k : 0, H, H_kv, D);
  const bool need_ws = have_q || f8;
  if (need_ws && !workspace) return FMHA_ERR_NULL_POINTER;
  if ((uintptr_t)workspace & 15) return FMHA_ERR_MISALIGNED;
  if (need_ws && workspace_bytes < wl.total) return FMHA_ERR_INVALID_ARGUMENT;
  const int64_t n_q = (Sq + kQM - 1) / kQM;
  const int64_t n_k = (Sk + kKvN - 1) / kKvN;
  const int64_t lim = (int64_t)1 << 31;
  if ((int64_t)B * H * n_q >= lim || (int64_t)B * H_kv * n_k >= lim)
    return FMHA_ERR_UNSUPPORTED;

  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.aux = (float*)workspace;
  p.aux_bytes = (uint32_t)need;
  p.cu_q = packed ? varlen->cu_seqlens_q : nullptr;
  p.cu_k = packed ? varlen->cu_seqlens_k : nullptr;
  p.causal = mask == FMHA_MASK_CAUSAL_QBEGIN || mask == FMHA_MASK_CAUSAL_QEND;
  p.qend = mask == FMHA_MASK_CAUSAL_QEND;
  p.scale = scale;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  p.xcd_per = 0;
  p.n_tiles = 0;
  p.rank_seqs = packed && B <= 64 ? 1 : 0;

  // Streams whose byte offsets from the start of one sequence could pass 31 bits (one tile to
  // spare; packed batches bounded by their totals) take the kernels that place descriptors at
  // every streamed tile: K/V in the dQ kernel, Q/dO in the dK/dV kernel.
  const int64_t seq_q = packed ? varlen->total_length_q : Sq;
  const int64_t seq_k = packed ? varlen->total_length_k : Sk;
  const bool wide_k = (seq_k + kKvN) * H_kv * D * 2 >= lim;
  const bool wide_q = (seq_q + kKvN) * H * D * 2 >= lim;

  if (f8) {  // bf16 copies of the e4m3 inputs; the gradients are computed and written in bf16
    char* ws = (char*)workspace;
    const void* src[kWidenTensors] = {q, o, dout, k, v};
    const void** use[kWidenTensors] = {&p.q, &p.o, &p.dout, &p.k, &p.v};
    Widen w;
    uint64_t most = 0;
    for (int t = 0; t < kWidenTensors; ++t) {
      w.src[t] = src[t];
      w.dst[t] = ws + wl.off[t];
      w.n16[t] = wl.n16[t];
      if (wl.n16[t]) *use[t] = w.dst[t];
      most = wl.n16[t] > most ? wl.n16[t] : most;
    }
    if (most) {  // one wave per 2 KiB step of the largest tensor, at most 2048 workgroups per tensor
      const uint64_t blocks = (most + 4 * kWidenRows * 32 - 1) / (4 * kWidenRows * 32);
      hipLaunchKernelGGL(widen_e4m3_kernel, dim3((unsigned)(blocks < 2048 ? blocks : 2048), kWidenTensors),
                         dim3(kWidenThreads), 0, stream, w);
      if (hipGetLastError() != hipSuccess) return FMHA_ERR_HIP;
    }
  }

  hipError_t err = hipSuccess;
  const int nq = (int)n_q, nk = (int)n_k;
  if (dtype == FMHA_DTYPE_BF16 || f8) {
    if (D == 32) err = launch<fmha::kBF16, 32>(p, nq, nk, have_q, have_k, wide_k, wide_q, stream);
    if (D == 64) err = launch<fmha::kBF16, 64>(p, nq, nk, have_q, have_k, wide_k, wide_q, stream);
    if (D == 128) err = launch<fmha::kBF16, 128>(p, nq, nk, have_q, have_k, wide_k, wide_q, stream);
  } else {
    if (D == 32) err = launch<fmha::kF16, 32>(p, nq, nk, have_q, have_k, wide_k, wide_q, stream);
    if (D == 64) err = launch<fmha::kF16, 64>(p, nq, nk, have_q, have_k, wide_k, wide_q, stream);
    if (D == 128) err = launch<fmha::kF16, 128>(p, nq, nk, have_q, have_k, wide_k, wide_q, stream);
  }
  return err == hipSuccess ? FMHA_OK : FMHA_ERR_HIP;
}

}  // extern "C"
