// Fused multi-head attention forward pass for gfx950 (AMD Instinct MI355X, CDNA4).
//
// O = softmax(scale * Q K^T + mask) V, computed one K/V tile at a time with an online
// softmax, so S and P live only in registers (the method of the wingedge777 article
// "[CUDA 优化实战] fmha sm120: 超越 torch.sdpa(flash-attention-2)", sections
// "1. flash attention" and "2. fmha 实现").  Masks, packed variable-length batches, GQA
// and the LSE output follow the CUTLASS Blackwell FMHA example as the trdm.cn
// walk-through "CUTLASS Blackwell FMHA 示例完全解析" describes it (sections on the fusion
// point fmha_fusion.hpp, variable sequence length, verification, GQA/MQA strides).
//
// CDNA4 design (the pages' TMA / ldmatrix / mma.sync machinery has no counterpart here):
//
// * One workgroup = 4 waves of 64 lanes = 128 query rows (32 per wave) of one
//   (sequence, head).  K/V tiles of 64 keys stream through LDS, double buffered, filled
//   by buffer loads that write LDS directly (no VGPR staging).  The buffer descriptor
//   bounds every load to the rows of the current sequence: rows past the end read as 0,
//   which is how ragged tails and packed sequences are handled without touching
//   neighbouring memory.
// * Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_{bf16,f16}:
//   A = 32 keys x 16 dims read from LDS, B = 16 dims x 32 queries held in VGPRs for the
//   whole loop.  In the accumulator layout lane l then owns query l%32, and lanes l and
//   l^32 together own all 32 keys of the block, so a row max or sum is an in-lane reduction
//   plus one v_permlane32_swap.
// * The same accumulator layout is, key for key, the B operand layout of the second
//   product O^T += V^T P^T: the probabilities are converted in registers (v_cvt_pk_*)
//   and fed straight back to the matrix cores (the counterpart of the article's section
//   "Ps 寄存器重排").  The V^T operand comes from the row-major V tile through
//   ds_read_b64_tr_b16 transpose reads.
// * exp2 with scale*log2(e) folded into one FMA per score.  The running maximum is only
//   raised when a tile's maximum exceeds it by more than 2^8 (a lazy rescale in the spirit
//   of the article's section "lazy rescale": probabilities stay <= 256, far inside the
//   range of the 16-bit and fp8 operand types, and the O rescale is skipped for most tiles).
// * The row sum l: on tiles that need the mask (the causal diagonal, the ragged tail) it
//   adds the rounded 16-bit probabilities the matrix cores see, so a row with few visible
//   keys is normalised by exactly the weights of its numerator; on fully visible tiles it
//   adds the fp32 probabilities (as the FlashAttention papers do), two VALU operations
//   cheaper per pair.  Both use two independent partial sums per lane.  (v_dot2 against
//   1.0 would sum the rounded values in one operation, but on gfx950 the dot instructions
//   wait behind the MFMAs of the wave that shares the SIMD: the softmax phase took 15%
//   longer with them.)
//   fp8 sums on the matrix cores instead (an all-ones operand against the probability
//   operand of the PV product: one more MFMA per tile, exact sums of the rounded values),
//   since its matrix phase is the short one; with an LSE it also keeps the fp32 sum.
// * Tiles are split into fully visible ones, which run no mask code, and boundary tiles
//   (causal diagonal, ragged tail), the trip-count split of the CUTLASS fusion point.
// * Work order: heaviest q-tiles first (causal), and workgroups of one (sequence, head
//   group) land on the same XCD so they share K/V in that XCD's L2.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include <type_traits>

#include "fmha.h"

namespace fmha {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 64;           // keys per K/V tile
constexpr float kRescaleThreshold = 8.0f;  // log2 units: raise the running max only past 2^8
// fp8 probabilities are shifted up by 2^kF8Shift before the e4m3 conversion (and the running
// max is raised past 2^kF8Threshold), so they span [2^-9, 2^8] with e4m3 normals covering
// down to 2^-6 below the running max of the row, instead of most of a long row's weights
// landing among the subnormals.  The shift cancels in O = sum p v / sum p; the LSE removes it.
constexpr float kF8Shift = 6.0f;
constexpr float kF8Threshold = 2.0f;
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // gfx9 buffer descriptor: raw 32-bit dwords
constexpr int kSchedMfma = 0x008;    // scheduling-group masks of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedDsRead = 0x100;
constexpr int kPrefetch = 6;         // LDS reads kept in flight ahead of the MFMAs
constexpr int kWaitVmcnt0 = 0x0F70;           // s_waitcnt vmcnt(0), expcnt and lgkmcnt left at their maxima

enum : int { kF16 = 0, kBF16 = 1, kF8 = 2 };

struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* cu_q;  // null for dense batches
  const int32_t* cu_k;
  int32_t B, Sq, Sk, H, H_kv, group;  // Sq / Sk: lengths (packed: maxima)
  int32_t total_q;                    // packed: rows of q (LSE row length)
  int32_t n_qtiles;
  int32_t causal;   // 1 for both causal masks
  int32_t qend;     // causal aligned to the last key
  int32_t xcd_per;  // (sequence, head) pairs per XCD when B*H % 8 == 0, else 0
  float scale_log2; // scale * log2(e)
  float o_scale;
};

// ------------------------------------------------------------------------------------
// device primitives
// ------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}

// Same descriptor as raw SGPR words, for the inline-asm LDS-direct load below.
__device__ inline i32x4 make_rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  const i32x4 r = {__builtin_amdgcn_readfirstlane((int)(uint32_t)a), __builtin_amdgcn_readfirstlane((int)(a >> 32)),
                   __builtin_amdgcn_readfirstlane((int)bytes), (int)kRsrcWord3};
  return r;
}

// 16 bytes per lane from a buffer straight into LDS at lds_addr + 16 * lane (lds_addr is
// wave-uniform).  Written as inline asm so the compiler does not track it: it would
// otherwise wait for these loads before LDS reads it cannot prove disjoint, which undoes the
// prefetch; the phase schedule waits for them explicitly.  No memory clobber: the LDS reads
// of the current stage may move across it (it only ever writes the other stage), while the
// volatile asm statements (loads, waits, barriers) keep their order.  M0 is saved and restored.
__device__ inline void lds_load16(i32x4 rsrc, uint32_t voff, uint32_t lds_addr) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(lds_addr));
}

__device__ inline float wave_row_max(float x) {  // max of lanes l and l^32
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                            false, false);
  return __builtin_fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ inline float wave_row_sum(float x) {  // sum of lanes l and l^32
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                            false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Workgroup barrier for the phase schedule.  Unlike __syncthreads() it carries no release
// fence, which would also wait for the K/V loads still in flight for a later phase; the only
// ordering needed is that this wave's LDS reads have returned (lgkmcnt(0)) before another
// wave may overwrite the buffer, and the loads are waited for explicitly (vmcnt) where due.
__device__ inline void phase_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N)
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 16-byte chunk swizzle of a K/V tile row j in LDS (CPR chunks per row).  Rows 0..15 map
// to distinct chunks, so the 32-row b128 reads of K spread over all banks; four
// consecutive rows move whole chunk pairs, so the 4-row transpose reads of V do too.
template <int CPR>
__device__ inline int swz(int j) {
  return (2 * (j & 3) + ((j >> 2) & 1) + 8 * ((j >> 3) & 1)) & (CPR - 1);
}

template <int DT>
struct Elem;
template <>
struct Elem<kBF16> {
  typedef bf16x8 frag;
  __device__ static inline uint32_t pack(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};  // v_cvt_pk_bf16_f32, round to nearest even
    return __builtin_bit_cast(uint32_t, v);
  }
  // the two packed values as fp32 (exact)
  __device__ static inline float lo(uint32_t pk) { return __builtin_bit_cast(float, pk << 16); }
  __device__ static inline float hi(uint32_t pk) { return __builtin_bit_cast(float, pk & 0xFFFF0000u); }
  __device__ static inline f32x16 mma(i32x4 a, i32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
  }
};
template <>
struct Elem<kF16> {
  typedef f16x8 frag;
  __device__ static inline uint32_t pack(float a, float b) {
    f16x2 v = {(_Float16)a, (_Float16)b};  // v_cvt_pk_f16_f32, round to nearest even
    return __builtin_bit_cast(uint32_t, v);
  }
  // the two packed values as fp32 (exact)
  __device__ static inline float lo(uint32_t pk) { return (float)__builtin_bit_cast(f16x2, pk)[0]; }
  __device__ static inline float hi(uint32_t pk) { return (float)__builtin_bit_cast(f16x2, pk)[1]; }
  __device__ static inline f32x16 mma(i32x4 a, i32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                 0, 0);
  }
};

// fp8 e4m3 (OCP e4m3fn): S^T and O^T on the 32x32x64 f8f6f4 MFMA, unit block scales
// (E8M0 127 = 2^0) since the per-tensor scales are folded into scale and o_scale.
__device__ inline f32x16 mma_f8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// four fp32 values -> four e4m3 bytes (round to nearest even; inputs within +-448)
__device__ inline uint32_t pack_f8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}
template <int I>
__device__ inline float f8_byte(uint32_t w) { return __builtin_amdgcn_cvt_f32_fp8((int)w, I); }

// 16-byte chunk swizzle of an 8-bit K/V tile row j in LDS (CPR chunks per row, P = 256 / row
// bytes rows per 256-byte bank window).  The 16 rows of a b128 K read land in 16 distinct
// chunk slots of the bank window, and so do the 8 rows x 2 chunks of a transposed 8-bit V read.
template <int CPR>
__device__ inline int swz8(int j) {
  constexpr int P = 256 / (16 * CPR);
  return 2 * ((j / P) % (CPR / 2)) + ((j >> 3) & 1);
}

// ------------------------------------------------------------------------------------
// the kernel (fp16 / bf16 / fp8 e4m3)
// ------------------------------------------------------------------------------------
// Phase schedule.  The 8 waves form two groups, A = waves 0-3 and B = waves 4-7, so every
// SIMD holds one wave of each.  Time is cut into phases separated by workgroup barriers.
// In phase 2t group A runs the matrix work of tile t (S(t) = K(t) Q^T and O += V(t-1) P(t-1))
// while group B runs the softmax of tile t-1; in phase 2t+1 the roles swap.  Each SIMD thus
// always has one wave feeding its matrix core and one wave on the vector ALU (the two-tile
// ping-pong of the CUTLASS design, built here from the single workgroup barrier).
// K(t+1) and V(t) are requested at the start of phase 2t and waited for at the end of phase
// 2t+1, two phases ahead of their first use.
template <int DT, int D, bool LSE_SUM>
__global__ __launch_bounds__(kThreads, 1) void fmha_fwd_kernel(const Params p) {
  constexpr bool F8 = DT == kF8;
  constexpr int E = F8 ? 1 : 2;    // bytes per element
  constexpr int RB = D * E;        // bytes per K/V row, in memory and in LDS (swizzled)
  constexpr int CPR = RB / 16;     // 16-byte chunks per row
  constexpr int TILE = kBN * RB;   // LDS bytes per K or V tile
  constexpr int KBLK = TILE / 1024;  // 1 KiB LDS-direct loads (64 lanes x 16 B) per K or V tile
  constexpr int NBLK = 2 * KBLK;
  constexpr int NSTAGE = 3;          // K/V tile pairs resident in LDS: in use, landed, landing
  constexpr int STAGE = 2 * TILE;    // LDS bytes per stage: K tile, then V tile
  constexpr int LPP = (NBLK + 15) / 16;  // loads one wave issues per phase
  static_assert(NBLK % 8 == 0, "every wave issues the same number of tile loads");
  static_assert(!F8 || D >= 64, "fp8 needs D >= 64 (one 64-deep MFMA k-step)");
  constexpr int KS = F8 ? D / 64 : D / 16;  // MFMA k-steps over the head dimension
  constexpr int NDB = D / 32;      // 32-wide blocks of the head dimension in O
  typedef Elem<DT == kF8 ? kBF16 : DT> T;  // (fp8 uses the helpers above instead)
  auto sw = [](int j) __attribute__((always_inline)) { return F8 ? swz8<CPR>(j) : swz<CPR>(j); };

  // The tile loads are inline assembly the compiler cannot see, so it inserts no waits for
  // them: every wait on them below is explicit.
  __shared__ __attribute__((aligned(1024))) char kv_lds[NSTAGE * STAGE];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)kv_lds;  // LDS address of stage 0

  const int lane = threadIdx.x & 63;
  // (Left as a per-lane value on purpose: branches on the wave group then compile to exec
  // masks over one register assignment; as scalar branches, they make the register
  // allocator copy the accumulators at every join.)
  const int wave = threadIdx.x >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // the same, in a scalar register
  const int l32 = lane & 31;
  const int h32 = lane >> 5;
  const int group = wave >> 2;             // 0 = A, 1 = B
  const int rblk = 2 * (wave & 3) + group; // 32-row block of the workgroup tile owned by this wave

  // ---- which (sequence, head, q-tile) this workgroup owns ---------------------------
  const int BH = p.B * p.H;
  const int x = blockIdx.x;
  int bh, qt_rev;
  if (p.xcd_per) {  // round-robin dispatch puts workgroup x on XCD x % 8
    const int slot = x >> 3;
    qt_rev = slot / p.xcd_per;
    bh = (x & 7) * p.xcd_per + slot % p.xcd_per;
  } else {
    qt_rev = x / BH;
    bh = x % BH;
  }
  const int qt = p.n_qtiles - 1 - qt_rev;  // heaviest causal tiles first
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int kvh = h / p.group;

  int q_row0, Sq_b, k_row0, Sk_b;
  if (p.cu_q) {
    q_row0 = p.cu_q[b];
    Sq_b = p.cu_q[b + 1] - q_row0;
    k_row0 = p.cu_k[b];
    Sk_b = p.cu_k[b + 1] - k_row0;
  } else {
    q_row0 = b * p.Sq;
    Sq_b = p.Sq;
    k_row0 = b * p.Sk;
    Sk_b = p.Sk;
  }
  const int q0 = qt * kBM;
  if (q0 >= Sq_b) return;
  const int off = p.qend ? Sk_b - Sq_b : 0;
  // keys visible to the last valid row of a row range, as an exclusive end
  auto key_end = [&](int last_row) { return p.causal ? min(Sk_b, last_row + off + 1) : Sk_b; };
  const int wg_end = key_end(min(Sq_b, q0 + kBM) - 1);
  const int n_tiles = wg_end > 0 ? (wg_end + kBN - 1) / kBN : 0;
  // per wave: the first tile that some row of the wave does not see completely (the mask
  // is applied from there on)
  const int qw0 = q0 + 32 * rblk;
  int w_full = 0;
  if (qw0 < Sq_b) {
    const int first_sees = p.causal ? min(Sk_b, qw0 + off + 1) : Sk_b;
    w_full = first_sees > 0 ? first_sees / kBN : 0;
  }

  const uint32_t qstride = (uint32_t)p.H * D * E;     // bytes between rows of one head
  const uint32_t kstride = (uint32_t)p.H_kv * D * E;
  const size_t q_base = ((size_t)q_row0 * p.H + h) * D * E;
  const size_t k_base = ((size_t)k_row0 * p.H_kv + kvh) * D * E;
  const uint32_t q_bytes = Sq_b > 0 ? (uint32_t)(Sq_b - 1) * qstride + RB : 0;
  const uint32_t k_bytes = Sk_b > 0 ? (uint32_t)(Sk_b - 1) * kstride + RB : 0;
  const auto rq = make_rsrc((const char*)p.q + q_base, q_bytes);
  const i32x4 rk = make_rsrc_words((const char*)p.k + k_base, k_bytes);
  const i32x4 rv = make_rsrc_words((const char*)p.v + k_base, k_bytes);
  const auto ro = make_rsrc((const char*)p.o + q_base, q_bytes);

  // ---- Q fragment: B operand of S^T = K Q^T, lane owns query l32, dims 8*h32.. of each k-step
  const int qi = qw0 + l32;  // query row inside the sequence
  // (fp8: 32 bytes, dims 64 ks + 32 h32 .., per 64-deep k-step, in qf[2 ks], qf[2 ks + 1])
  constexpr int NQF = F8 ? 2 * KS : KS;
  i32x4 qf[NQF];
#pragma unroll
  for (int i = 0; i < NQF; ++i)
    qf[i] = __builtin_amdgcn_raw_buffer_load_b128(
        rq, (uint32_t)qi * qstride + (F8 ? 64 * (i >> 1) + 32 * h32 + 16 * (i & 1) : (16 * i + 8 * h32) * E), 0, 0);
  // (Q is waited for in the prologue below, together with the first two K/V tiles.)

  // ---- K/V tile loads straight into LDS, one 1 KiB block (64 lanes x 16 B) per instruction.
  // Block b of a tile covers rows 64b/CPR.. of it; lane l fills LDS chunk (64b + l) % CPR of
  // its row j with memory chunk ((64b + l) % CPR) ^ swz(j).
  //
  // Step t consumes L(t) = {K(t), V(t-1)} from LDS stage t % 3.  L(t+2) is requested during
  // phases 2t and 2t+1 by all 8 waves: block b of its NBLK blocks (K first, then V) by wave
  // b % 8 in the phase of parity (b / 8) % 2, spread over that wave's MFMA or softmax work.
  // (Issued in bursts, or by fewer waves, the loads queue at the CU's vector-memory path and
  // stall the issuing waves for hundreds of cycles.)  A load of a tile past either end of
  // the sequence reads zeros, so each wave issues the same NBLK / 8 loads every step, and
  // the number it has in flight at a step's end is that constant.
  auto tile_off = [&](int t) __attribute__((always_inline)) -> uint32_t { return (uint32_t)(t * kBN) * kstride; };
  uint32_t ld_off[2][LPP];  // per-lane byte offsets inside a tile of this wave's blocks
#pragma unroll
  for (int pp = 0; pp < 2; ++pp)
#pragma unroll
    for (int i = 0; i < LPP; ++i) {
      const int b = 16 * i + 8 * pp + wave_u;
      const int pos = (b % KBLK) * 64 + lane;  // 16-byte chunk position inside the tile
      const int j = pos / CPR;
      ld_off[pp][i] = (uint32_t)j * kstride + (((pos % CPR) ^ sw(j)) * 16);
    }
  // load i of phase parity pp for L(tl), tl >= 0, into stage tl % 3
  auto load_unit = [&](int tl, int pp, int i) __attribute__((always_inline)) {
    const int b0 = 16 * i + 8 * pp;  // first block of this (pp, i) over the 8 waves
    if (b0 >= NBLK) return;          // compile-time after unrolling
    const bool is_k = b0 + 8 <= KBLK ? true : b0 >= KBLK ? false : b0 + wave_u < KBLK;
    const uint32_t goff = (is_k ? tile_off(tl) : tile_off(tl - 1)) + ld_off[pp][i];
    const uint32_t lds_addr = lds0 + (uint32_t)((tl % NSTAGE) * STAGE + (b0 + wave_u) * 1024);
    lds_load16(is_k ? rk : rv, goff, __builtin_amdgcn_readfirstlane(lds_addr));
  };

  f32x16 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
  f32x16 s[2];                      // scores of the tile between its matrix and softmax phases
  constexpr int NPK = F8 ? 4 : 8;   // packed probability registers per 32-key block
  uint32_t pk[2][NPK] = {};         // probabilities of the tile between its softmax and PV phases
  float m_run = -__builtin_inff();  // running max of scale*log2(e)*s for query l32
  // fp8 row sums on the matrix cores: an all-ones A operand against the probability
  // operand of the PV product, so every element of acc_l holds the row sum of this lane's
  // query over the rounded probabilities that O is built from (exact in fp32).  (The fp8
  // matrix phase is half as long as the softmax, so the MFMA is the cheap place for it; the
  // 16-bit paths keep it on the vector ALU, where their longer matrix phase hides it.)
  f32x16 acc_l = {};
  float l_run = 0.0f;  // this lane's part of the VALU row sum (l_run + l_run2)
  float l_run2 = 0.0f;
  constexpr bool VSUM = !F8 || LSE_SUM;  // keep the VALU row sum
  const float sl2 = p.scale_log2;
  // last key visible to this lane's query, less the lane's key offset 4 h32 inside a tile
  const int vis_last = (p.causal ? min(Sk_b - 1, qi + off) : Sk_b - 1) - 4 * h32;

  // Per-lane LDS byte offsets.  The swizzle only touches chunk bits that the k-step (K) or
  // the d-block (V) index leaves clear, so every read address is one of these bases XOR a
  // compile-time constant, plus an immediate row offset.
  //   16-bit: K row l32, chunk 2 ks + h32; fp8: K row l32, chunks 4 ks + 2 h32 (+1).
  const int k_lane = l32 * RB + (((F8 ? 2 * h32 : h32) ^ sw(l32)) * 16);
  const int k_lane2 = l32 * RB + (((2 * h32 + 1) ^ sw(l32)) * 16);  // fp8 only
  const int g16 = (lane >> 4) & 1;
  const int s16 = lane & 15;
  // 16-bit V transpose read (ds_read_b64_tr_b16): row 4 h32 + s16 / 4 of a 16-row group (and
  // that row + 8), 8 bytes at column 16 g16 + 4 (s16 % 4).
  // fp8 (ds_read_b64_tr_b8, which hands lane j of each 16-lane group byte j % 8 of the words
  // of lanes j / 8, j / 8 + 2, ..): lane l supplies row 8 h32 + s16 / 2 of a 16-row chunk,
  // 8 bytes at column 16 g16 + 8 (s16 % 2), and gets column l32 of rows 8 h32 + 0..7.
  const int v_row0 = F8 ? 8 * h32 + (s16 >> 1) : 4 * h32 + (s16 >> 2);
  const int v_part = F8 ? g16 : 2 * g16 + ((s16 & 3) >> 1);
  const int v_lane0 = TILE + v_row0 * RB + ((v_part ^ sw(v_row0)) * 16) + 8 * (s16 & 1);
  const int v_lane1 = TILE + (v_row0 + 8) * RB + ((v_part ^ sw(v_row0 + 8)) * 16) + 8 * (s16 & 1);

  // one QK^T MFMA of the tile: k-step ks of key block jb (ka, kb: k_lane, k_lane2 + the
  // stage's address)
  auto qk_mma = [&](uint32_t ka, uint32_t kb, int i) __attribute__((always_inline)) {
    const int jb = i & 1, ks = i >> 1;
    if constexpr (F8) {
      const i32x4 a0 = *(const lds_i32x4*)(uintptr_t)((ka ^ (64 * ks)) + 32 * jb * RB);
      const i32x4 a1 = *(const lds_i32x4*)(uintptr_t)((kb ^ (64 * ks)) + 32 * jb * RB);
      const i32x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
      const i32x8 b = __builtin_shufflevector(qf[2 * ks], qf[2 * ks + 1], 0, 1, 2, 3, 4, 5, 6, 7);
      s[jb] = mma_f8(a, b, s[jb]);
    } else {
      const i32x4 a = *(const lds_i32x4*)(uintptr_t)((ka ^ (32 * ks)) + 32 * jb * RB);
      s[jb] = T::mma(a, qf[ks], s[jb]);
    }
  };
  // one PV MFMA.  16-bit: d-block db, 16-key chunk (jb, c).  fp8: d-block i, all 64 keys; byte
  // 8 c + r of either operand is key 16 c + 8 h32 + r (the probabilities are regrouped to
  // this order at the end of the softmax, and the transposed V reads deliver it).
  auto pv_mma = [&](uint32_t va0, uint32_t va1, int i) __attribute__((always_inline)) {
    if constexpr (F8) {
      i32x2 t[4];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        t[c] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(uintptr_t)((va0 ^ (32 * i)) + 16 * c * RB));
      const i32x8 a = {t[0][0], t[0][1], t[1][0], t[1][1], t[2][0], t[2][1], t[3][0], t[3][1]};
      const i32x8 b = {(int)pk[0][0], (int)pk[0][1], (int)pk[0][2], (int)pk[0][3],
                       (int)pk[1][0], (int)pk[1][1], (int)pk[1][2], (int)pk[1][3]};
      acc_o[i] = mma_f8(a, b, acc_o[i]);
      if (i == NDB - 1) {  // row sums: e4m3 1.0 = 0x38
        const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                            0x38383838, 0x38383838, 0x38383838, 0x38383838};
        acc_l = mma_f8(ones, b, acc_l);
      }
      return;
    }
    const int db = i % NDB, jc = i / NDB, jb = jc >> 1, c = jc & 1;
    const uint32_t rows = (32 * jb + 16 * c) * RB;
    const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)((va0 ^ (64 * db)) + rows));
    const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)((va1 ^ (64 * db)) + rows));
    const i32x4 a = {__builtin_bit_cast(int, __builtin_shufflevector(v0, v0, 0, 1)),
                     __builtin_bit_cast(int, __builtin_shufflevector(v0, v0, 2, 3)),
                     __builtin_bit_cast(int, __builtin_shufflevector(v1, v1, 0, 1)),
                     __builtin_bit_cast(int, __builtin_shufflevector(v1, v1, 2, 3))};
    const i32x4 bp = {(int)pk[jb][4 * c], (int)pk[jb][4 * c + 1], (int)pk[jb][4 * c + 2], (int)pk[jb][4 * c + 3]};
    acc_o[db] = T::mma(a, bp, acc_o[db]);
  };
  constexpr int NQK = 2 * KS;                // MFMAs of S^T for one tile
  constexpr int NPV = F8 ? NDB : 4 * NDB;    // MFMAs of O^T += V^T P^T for one tile
  constexpr int RQK = F8 ? 2 : 1;            // LDS reads per S^T MFMA
  constexpr int RPV = F8 ? 4 : 2;            // LDS reads per O^T MFMA

  // matrix phase of tile t: S(t) = K(t) Q^T and O += V(t-1) P(t-1), from LDS stage t % 3;
  // hook(j), j < LPP, issues this wave's loads of the phase.  Every wave runs every tile of
  // the workgroup: past a wave's last visible tile its probabilities are zero, and the
  // phase takes as long as the busiest wave of the group anyway.
  auto matrix_phase = [&](int t, auto& hook) __attribute__((always_inline)) {
    constexpr int N = NQK > NPV ? NQK : NPV;
    const uint32_t st = lds0 + (uint32_t)((t % NSTAGE) * STAGE);
    uint32_t ka = k_lane + st, kb = k_lane2 + st, va0 = v_lane0 + st, va1 = v_lane1 + st;
    // keep derived addresses out of loop-invariant code
    if constexpr (F8)
      asm volatile("" : "+v"(ka), "+v"(kb), "+v"(va0));
    else
      asm volatile("" : "+v"(ka), "+v"(va0), "+v"(va1));
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (i < NQK) qk_mma(ka, kb, i);
      if (i < NPV) pv_mma(va0, va1, i);
#pragma unroll
      for (int j = 0; j < LPP; ++j)  // load j goes after step j * N / LPP
        if ((j * N) / LPP == i) hook(j);
    }
    // The LDS reads run kPrefetch reads ahead of the MFMAs that consume them (pinned with
    // scheduling groups: the compiler alone keeps only one or two in flight, which leaves
    // the matrix core waiting on LDS latency).
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kPrefetch, 0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (i < NQK) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, RQK, 0);
      }
      if (i < NPV) {
        if (F8 && i == NDB - 1)  // this step also adds the row sums
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
        else
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, RPV, 0);
      }
    }
  };

  // softmax phase of tile t: mask, running max, lazy rescale, probabilities; hook(j), j <
  // LPP, issues this wave's loads of the phase, spread over the exponentials
  auto softmax_phase = [&](int t, auto& hook) __attribute__((always_inline)) {
    if (t >= w_full) {  // some key of the tile is hidden from some row of the wave
      // score (jb, r) belongs to key t kBN + 4 h32 + 32 jb + 8 (r / 4) + r % 4
      const int lim = vis_last - t * kBN;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[jb][r] = 32 * jb + 8 * (r >> 2) + (r & 3) <= lim ? s[jb][r] : -__builtin_inff();
    }
    float mx = s[0][0];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[jb][r]);
    mx = wave_row_max(mx);
    const float m_cand = mx * sl2;
    if (__any(m_cand > m_run + (F8 ? kF8Threshold : kRescaleThreshold))) {
      const float m_new = __builtin_fmaxf(m_run, m_cand);
      const float alpha = m_new == -__builtin_inff() ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      if constexpr (F8) acc_l[0] *= alpha;  // (the only element read)
      if constexpr (VSUM) {
        l_run *= alpha;
        l_run2 *= alpha;
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc_o[db] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -__builtin_inff() ? 0.0f : m_run) - (F8 ? kF8Shift : 0.0f);
    // exponentials, packing and (VALU) row sums.  16-bit ROUNDED: sum the 16-bit values the
    // matrix cores see, else the fp32 ones (see the row-sum note at the top of this file);
    // fp8 with an LSE: the fp32 ones.
    auto exps = [&](auto rounded_tag) __attribute__((always_inline)) {
      constexpr bool ROUNDED = decltype(rounded_tag)::value;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {  // scores 4 qd .. 4 qd + 3: keys 8 qd + 4 h32 + 0..3
          float e[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) e[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[jb][4 * qd + u], sl2, -m_use));
          if constexpr (F8) {
            pk[jb][qd] = pack_f8x4(e[0], e[1], e[2], e[3]);
          } else {
            pk[jb][2 * qd] = T::pack(e[0], e[1]);
            pk[jb][2 * qd + 1] = T::pack(e[2], e[3]);
          }
          if constexpr (!F8 && ROUNDED) {
            l_run += T::lo(pk[jb][2 * qd]) + T::lo(pk[jb][2 * qd + 1]);
            l_run2 += T::hi(pk[jb][2 * qd]) + T::hi(pk[jb][2 * qd + 1]);
          } else if constexpr (VSUM) {
            l_run += e[0] + e[2];
            l_run2 += e[1] + e[3];
          }
#pragma unroll
          for (int j = 0; j < LPP; ++j)  // load j goes after exponential quad j * 8 / LPP
            if ((j * 8) / LPP == 4 * jb + qd) hook(j);
        }
    };
    if constexpr (F8) {
      exps(std::false_type{});
    } else {
      if (t >= w_full)
        exps(std::true_type{});
      else
        exps(std::false_type{});
    }
    if constexpr (F8) {
      // Regroup to 8 consecutive keys per lane and 16-key chunk (the fp8 PV operand order):
      // lane h32 = 0 trades its keys 8..11 of each chunk for keys 4..7 of lane l + 32.
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          auto r = __builtin_amdgcn_permlane32_swap(pk[jb][2 * m], pk[jb][2 * m + 1], false, false);
          pk[jb][2 * m] = r[0];
          pk[jb][2 * m + 1] = r[1];
        }
    }
    // Pin the results here: the compiler may otherwise sink the tail of this arithmetic past
    // the phase barrier, into the matrix phase that follows on this wave.
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int q = 0; q < NPK; ++q) asm volatile("" : "+v"(pk[jb][q]));
    asm volatile("" : "+v"(m_run));
    if constexpr (VSUM) asm volatile("" : "+v"(l_run), "+v"(l_run2));
  };

  // The matrix work runs at raised wave priority so the SIMD issues its MFMAs ahead of the
  // softmax VALU work of the other group's wave.
  auto matrix_prio = [&](int t, auto& hook) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    matrix_phase(t, hook);
    __builtin_amdgcn_s_setprio(0);
  };
  // The loads of phase ph request part ph % 2 of L(ph / 2 + 2).  At the end of an odd phase
  // 2t+1, L(t+1) must have landed for step t+1; only this wave's requests for L(t+2) may
  // still be in flight.
  auto even_end = [&]() __attribute__((always_inline)) { phase_barrier(); };
  auto odd_end = [&]() __attribute__((always_inline)) {
    wait_vmcnt<NBLK / 8>();
    phase_barrier();
  };
  auto no_work = [&](int tl, auto pp_tag) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LPP; ++i) load_unit(tl, decltype(pp_tag)::value, i);
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;

  // prologue: L(0) (K(0) and the zero V(-1)) and L(1) into stages 0 and 1
  no_work(0, P0{});
  no_work(0, P1{});
  no_work(1, P0{});
  no_work(1, P1{});
  // Wait for Q and the tiles with the builtin (whose effect the compiler tracks): otherwise
  // it keeps partial vmcnt waits for Q inside the loop, and those would also stall on the
  // K/V loads.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  phase_barrier();
  // Phases 0 .. 2 n_tiles + 1.  Group A: matrix(t) in phase 2t, softmax(t) in 2t+1.  Group B:
  // softmax(t-1) in phase 2t, matrix(t) in 2t+1.  Each group runs its own straight loop
  // (the two meet at the same barriers), so no phase body branches on the group.
  if (group == 0) {
    for (int t = 0; t < n_tiles; ++t) {
      auto h0 = [&](int i) __attribute__((always_inline)) { load_unit(t + 2, 0, i); };
      auto h1 = [&](int i) __attribute__((always_inline)) { load_unit(t + 2, 1, i); };
      matrix_prio(t, h0);
      even_end();
      softmax_phase(t, h1);
      odd_end();
    }
    {
      auto h0 = [&](int i) __attribute__((always_inline)) { load_unit(n_tiles + 2, 0, i); };
      matrix_prio(n_tiles, h0);  // O += V(n-1) P(n-1)
      even_end();
      no_work(n_tiles + 2, P1{});
      odd_end();
    }
  } else {
    no_work(2, P0{});
    even_end();
    for (int t = 0; t < n_tiles; ++t) {
      auto h1 = [&](int i) __attribute__((always_inline)) { load_unit(t + 2, 1, i); };
      auto h0 = [&](int i) __attribute__((always_inline)) { load_unit(t + 3, 0, i); };
      matrix_prio(t, h1);
      odd_end();
      softmax_phase(t, h0);
      even_end();
    }
    {
      auto h1 = [&](int i) __attribute__((always_inline)) { load_unit(n_tiles + 2, 1, i); };
      matrix_prio(n_tiles, h1);
      odd_end();
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the requests past the end (they write LDS)

  // ---- epilogue: normalise, scale, convert; stage each wave's 32 x D tile of O through LDS
  // (free now) so the stores write whole rows, 16 bytes per lane, instead of 16-byte pieces
  // of 32 rows.  Rows past the sequence fall outside the O descriptor and are dropped.
  phase_barrier();  // every wave's requests past the end have landed and its reads are done
  const float l_tot = F8 ? acc_l[0] : wave_row_sum(l_run + l_run2);
  const float inv = l_tot > 0.0f ? p.o_scale / l_tot : 0.0f;
  constexpr int OST = RB + 16;  // LDS bytes per staged O row (padded against bank conflicts)
  static_assert(kWaves * 32 * OST <= NSTAGE * STAGE, "O staging fits in the K/V stages");
  char* const ot = kv_lds + wave * 32 * OST;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * db + 8 * g + 4 * h32;
      if constexpr (F8) {  // saturate to the largest finite e4m3 value, then round
        float x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = __builtin_fminf(__builtin_fmaxf(acc_o[db][4 * g + u] * inv, -448.0f), 448.0f);
        *(uint32_t*)(ot + l32 * OST + d) = pack_f8x4(x[0], x[1], x[2], x[3]);
      } else {
        const i32x2 w = {(int)T::pack(acc_o[db][4 * g] * inv, acc_o[db][4 * g + 1] * inv),
                         (int)T::pack(acc_o[db][4 * g + 2] * inv, acc_o[db][4 * g + 3] * inv)};
        *(i32x2*)(ot + l32 * OST + d * E) = w;
      }
    }
  constexpr int RPI = 64 / CPR;  // rows per store instruction
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int row = i * RPI + lane / CPR, chunk = lane % CPR;
    const i32x4 w = *(const i32x4*)(ot + row * OST + chunk * 16);
    __builtin_amdgcn_raw_buffer_store_b128(w, ro, (uint32_t)(qw0 + row) * qstride + chunk * 16, 0, 0);
  }
  // (fp8: the LSE takes the fp32 sum, which a 3-bit-mantissa rounding would move by up to ~0.06)
  const float l_exact = F8 && LSE_SUM ? wave_row_sum(l_run + l_run2) : l_tot;  // (all lanes: a lane swap)
  if (p.lse && h32 == 0 && qi < Sq_b) {
    const float lse = l_tot > 0.0f ? (m_run + __builtin_amdgcn_logf(l_exact) - (F8 ? kF8Shift : 0.0f)) *
                                         0.69314718055994531f
                                   : -__builtin_inff();
    const size_t idx = p.cu_q ? (size_t)h * p.total_q + q_row0 + qi : ((size_t)b * p.H + h) * p.Sq + qi;
    p.lse[idx] = lse;
  }
}
template <int DT, int D>
hipError_t launch(const Params& p, int grid, hipStream_t stream) {
  // fp8 keeps an fp32 row sum beside the matrix-core one when an LSE is wanted (see the kernel)
  if constexpr (DT == kF8) {
    if (p.lse) {
      hipLaunchKernelGGL((fmha_fwd_kernel<DT, D, true>), dim3(grid), dim3(kThreads), 0, stream, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((fmha_fwd_kernel<DT, D, false>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fmha

// --------------------------------------------------------------------------------------
// C ABI
// --------------------------------------------------------------------------------------
extern "C" {

const char* fmha_status_string(fmha_status s) {
  switch (s) {
    case FMHA_OK: return "ok";
    case FMHA_ERR_NULL_POINTER: return "null pointer (q, k, v, o, or only one of the cu_seqlens pointers)";
    case FMHA_ERR_INVALID_SHAPE: return "invalid shape (negative size, H % H_kv != 0, D not in {32, 64, 128})";
    case FMHA_ERR_UNSUPPORTED: return "unsupported (dtype or mask out of range, or tensor too large for 32-bit offsets)";
    case FMHA_ERR_MISALIGNED: return "misaligned pointer (q, k, v, o need 16 bytes, lse needs 4)";
    case FMHA_ERR_INVALID_ARGUMENT: return "invalid argument (scale must be finite and > 0, o_scale finite)";
    case FMHA_ERR_HIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

int32_t fmha_version(void) { return 100; }

fmha_status fmha_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B, int32_t Sq,
                     int32_t Sk, int32_t H, int32_t H_kv, int32_t D, float scale, fmha_mask mask, fmha_dtype dtype,
                     float o_scale, const fmha_varlen* varlen, hipStream_t stream) {
  using namespace fmha;
  const bool packed = varlen != nullptr;
  const bool no_keys = packed ? varlen->total_length_k == 0 : Sk == 0;  // k and v may then be NULL
  if (!q || !o || (!no_keys && (!k || !v))) return FMHA_ERR_NULL_POINTER;
  if (packed && (!varlen->cu_seqlens_q != !varlen->cu_seqlens_k)) return FMHA_ERR_NULL_POINTER;
  if (packed && !varlen->cu_seqlens_q) return FMHA_ERR_NULL_POINTER;
  if (B < 0 || Sq < 0 || Sk < 0 || H < 0 || H_kv < 0) return FMHA_ERR_INVALID_SHAPE;
  if (H > 0 && (H_kv < 1 || H % H_kv != 0)) return FMHA_ERR_INVALID_SHAPE;
  if (D != 32 && D != 64 && D != 128) return FMHA_ERR_INVALID_SHAPE;
  if (packed && (varlen->total_length_q < 0 || varlen->total_length_k < 0)) return FMHA_ERR_INVALID_SHAPE;
  if ((int)dtype < 0 || (int)dtype > 2) return FMHA_ERR_UNSUPPORTED;
  if ((int)mask < 0 || (int)mask > 3) return FMHA_ERR_UNSUPPORTED;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return FMHA_ERR_MISALIGNED;
  if ((uintptr_t)lse & 3) return FMHA_ERR_MISALIGNED;
  if (!(scale > 0.0f) || !isfinite(scale) || !isfinite(o_scale)) return FMHA_ERR_INVALID_ARGUMENT;
  if (dtype == FMHA_DTYPE_F8E4M3 && D == 32) return FMHA_ERR_UNSUPPORTED;  // fp8 MFMA k-step is 64 deep

  const int64_t esz = dtype == FMHA_DTYPE_F8E4M3 ? 1 : 2;
  // every per-sequence byte offset must fit the 31-bit range of a buffer descriptor
  const int64_t rows_q = packed ? varlen->total_length_q : Sq;
  const int64_t rows_k = packed ? varlen->total_length_k : Sk;
  const int64_t lim = (int64_t)1 << 31;
  if (rows_q * H * D * esz >= lim || rows_k * H_kv * D * esz >= lim) return FMHA_ERR_UNSUPPORTED;
  // tiles requested one before and two past the keys must not wrap the 32-bit offset
  if ((int64_t)3 * kBN * H_kv * D * esz >= lim) return FMHA_ERR_UNSUPPORTED;
  if (B == 0 || H == 0 || Sq == 0 || (packed && varlen->total_length_q == 0)) return FMHA_OK;

  Params p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.cu_q = packed ? varlen->cu_seqlens_q : nullptr;
  p.cu_k = packed ? varlen->cu_seqlens_k : nullptr;
  p.B = B;
  p.Sq = Sq;
  p.Sk = Sk;
  p.H = H;
  p.H_kv = H_kv;
  p.group = H / H_kv;
  p.total_q = packed ? varlen->total_length_q : 0;
  p.n_qtiles = (Sq + kBM - 1) / kBM;
  p.causal = mask == FMHA_MASK_CAUSAL_QBEGIN || mask == FMHA_MASK_CAUSAL_QEND;
  p.qend = mask == FMHA_MASK_CAUSAL_QEND;
  const int64_t BH = (int64_t)B * H;
  const int64_t grid = BH * p.n_qtiles;
  if (grid >= lim) return FMHA_ERR_UNSUPPORTED;
  p.xcd_per = (BH % 8 == 0) ? (int32_t)(BH / 8) : 0;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  p.o_scale = o_scale;

  hipError_t err = hipSuccess;
  if (dtype == FMHA_DTYPE_F8E4M3) {
    if (D == 64) err = launch<kF8, 64>(p, (int)grid, stream);
    if (D == 128) err = launch<kF8, 128>(p, (int)grid, stream);
  } else if (dtype == FMHA_DTYPE_BF16) {
    if (D == 32) err = launch<kBF16, 32>(p, (int)grid, stream);
    if (D == 64) err = launch<kBF16, 64>(p, (int)grid, stream);
    if (D == 128) err = launch<kBF16, 128>(p, (int)grid, stream);
  } else {
    if (D == 32) err = launch<kF16, 32>(p, (int)grid, stream);
    if (D == 64) err = launch<kF16, 64>(p, (int)grid, stream);
    if (D == 128) err = launch<kF16, 128>(p, (int)grid, stream);
  }
  return err == hipSuccess ? FMHA_OK : FMHA_ERR_HIP;
}

}  // extern "C"
