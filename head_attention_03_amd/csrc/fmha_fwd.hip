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
// * One workgroup = 8 waves of 64 lanes; a q-tile is 256 query rows (32 per wave) of one
//   (sequence, head).  The two halves of the workgroup ping-pong between the matrix cores
//   and the vector ALU (the phase schedule above the kernel).  K/V tiles of 64 keys (fp8:
//   128, the same bytes) stream through three LDS stages, filled by buffer loads that write
//   LDS directly (no VGPR staging).  The buffer descriptor bounds every load to the rows of the current
//   sequence: rows past the end read as 0, which is how ragged tails and packed sequences
//   are handled without touching neighbouring memory.
// * A workgroup runs up to 8 q-tiles of one (sequence, head) back to back as a single K/V
//   stream: the next q-tile's Q rows and first K/V tiles load while the current one still
//   computes, and its output is written while the other half of the workgroup works the
//   matrix cores, so no q-tile waits for its inputs from memory after the first.
// * Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_{bf16,f16}:
//   A = 32 keys x 16 dims read from LDS, B = 16 dims x 32 queries held in VGPRs for the
//   whole q-tile.  In the accumulator layout lane l then owns query l%32, and lanes l and
//   l^32 together own all 32 keys of the block, so a row max or sum is an in-lane reduction
//   plus one v_permlane32_swap.
// * The same accumulator layout is, key for key, the B operand layout of the second
//   product O^T += V^T P^T: the probabilities are converted in registers (v_cvt_pk_*)
//   and fed straight back to the matrix cores (the counterpart of the article's section
//   "Ps 寄存器重排").  The V^T operand comes from the row-major V tile through
//   ds_read_b64_tr_b16 transpose reads.
// * exp2 with scale*log2(e) folded into one FMA per score (fp8 without an LSE: that FMA
//   builds the fp32 bit pattern of 2^x, kF8ExpCentre below).  The running maximum is only
//   raised when a tile's maximum exceeds it by more than 2^8 (a lazy rescale in the spirit
//   of the article's section "lazy rescale": probabilities stay <= 256, far inside the
//   range of the 16-bit and fp8 operand types, and the O rescale is skipped for most tiles).
// * The row sum l: on tiles that need the mask (the causal diagonal, the ragged tail) the
//   matrix cores add the rounded probabilities they multiply (a selecting all-ones operand
//   against the probability operand of the PV product: 4 more 16x16x32 MFMAs per 64-key
//   tile, exact in fp32), so a row with few visible keys is normalised by exactly the
//   weights of its numerator; on fully visible tiles the vector ALU adds the fp32
//   probabilities (as the FlashAttention papers do), with two independent partial sums per
//   lane.  Summing every tile on the matrix cores cost more than it saved once the VALU and
//   MFMA phases are balanced; v_dot2 against 1.0 waits behind the other wave's MFMAs on
//   gfx950.  fp8 sums every tile on the matrix cores (two 16x16x128 MFMAs per 128-key tile);
//   with an LSE it also keeps the fp32 sum.
// * Steps over tiles that every row sees completely run a build with no mask code at all;
//   boundary tiles (causal diagonal, ragged tail) run the masked build, the trip-count
//   split of the CUTLASS fusion point.
// * Work order: with several q-tiles per workgroup, causal q-tiles are paired heavy with
//   light (n-1-j with j) so every workgroup gets the same number of K/V tiles; with one,
//   heaviest first.  Workgroups of one (sequence, head group) land on the same XCD so they
//   share K/V in that XCD's L2; with several q-tiles each, the workgroups of one (sequence,
//   head) are dispatched side by side, so they run at the same time and stream its K/V tiles
//   together, and the host lowers the q-tiles per workgroup where that keeps the K/V streamed
//   by an XCD's resident workgroups inside its L2.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include <type_traits>

#include "fmha.h"
#include "fmha_device.h"

namespace fmha {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 64;           // keys per K/V tile (16-bit; fp8 tiles hold 2 kBN keys, the same bytes)
// fp8 probabilities are shifted up by 2^kF8Shift before the e4m3 conversion (and the running
// max is raised past 2^kF8Threshold), so they span [2^-9, 2^8] with e4m3 normals covering
// down to 2^-6 below the running max of the row, instead of most of a long row's weights
// landing among the subnormals.  The shift cancels in O = sum p v / sum p; the LSE removes it.
constexpr float kF8Shift = 6.0f;
constexpr float kF8Threshold = 2.0f;
// fp8 without an LSE forms 2^x from its fp32 bit pattern (Schraudolph's exponential: N. N.
// Schraudolph, "A fast, compact approximation of the exponential function", Neural
// Computation 11(4), 1999).  The integer 2^23 (x + 127 - c), read as a float, is
// 2^floor(x - c) (1 + frac(x - c)): 2^x with the mantissa interpolated linearly between
// powers of two, within a factor 1.0615 of it; c = log2(sqrt(1.0615)) centres that error at
// +-3.03%.  The e4m3 conversion that follows rounds to 3 mantissa bits anyway (+-6.25%), so
// each probability stays within 9.4% of 2^x, subnormals included, for one FMA and one
// float-to-integer conversion instead of an FMA and a v_exp_f32 (8 cycles per wave64
// instruction on gfx950, twice an FMA).  With an LSE the exact v_exp_f32 path is kept: the
// LSE takes the fp32 row sum of the probabilities.
constexpr float kF8ExpCentre = 0.0430357f;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Row-sum MFMAs on the 16x16 shapes: the selecting all-ones operand (see rowsum_lane in the
// kernel) against the probability operand of the PV product; C element 0 of every lane is the
// sum of its query's probabilities over the operand's keys.
__device__ inline f32x4 rowsum_f8(i32x8 ones, i32x8 p, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, p, c, 0, 0, 0, 127, 0, 127);
}
template <int DT>
__device__ inline f32x4 rowsum_16(i32x4 ones, i32x4 p, f32x4 c) {
  if constexpr (DT == kBF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ones), __builtin_bit_cast(bf16x8, p), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, ones), __builtin_bit_cast(f16x8, p), c, 0,
                                                  0, 0);
}

// pack_f8x4 written over an old register value: both halves are replaced, so the register
// needs no zeroing move first.
__device__ inline uint32_t pack_f8x4_over(uint32_t old, float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}
constexpr int kSchedMfma = 0x008;    // scheduling-group masks of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedDsRead = 0x100;
constexpr int kPrefetch = 6;         // fp8: LDS reads kept in flight ahead of the MFMAs
constexpr int kKLead = 4;            // 16-bit: K operand reads issued this many S^T MFMAs ahead
constexpr int kVLead = 2;            // 16-bit: V^T operand reads issued this many PV MFMAs ahead

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
  int32_t ipw;      // q-tiles run by one workgroup, one after the other
  int32_t causal;   // 1 for both causal masks
  int32_t qend;     // causal aligned to the last key
  int32_t xcd_per;  // (sequence, head) pairs per XCD when B*H % 8 == 0, else 0
  int32_t ngrp;     // workgroups per (sequence, head)
  int32_t rank_seqs;  // packed batch of at most 64 sequences: sequences taken longest (in keys) first
  float scale_log2; // scale * log2(e)
  float o_scale;
};

// ------------------------------------------------------------------------------------
// the kernel (fp16 / bf16 / fp8 e4m3)
// ------------------------------------------------------------------------------------
// Phase schedule.  The 8 waves form two groups, A = waves 0-3 and B = waves 4-7, so every
// SIMD holds one wave of each.  Time is cut into phases separated by workgroup barriers.
// In phase 2t group A runs the matrix work of tile t (S(t) = K(t) Q^T and O += V(t-1) P(t-1))
// while group B runs the softmax of tile t-1; in phase 2t+1 the roles swap.  Each SIMD thus
// always has one wave feeding its matrix core and one wave on the vector ALU (the two-tile
// ping-pong of the CUTLASS design, built here from the single workgroup barrier).
// K(t+2) and V(t+1) are requested during phases 2t and 2t+1 and waited for at the end of
// phase 2t+3, before their first use in phase 2t+4.
template <int DT, int D, bool LSE_SUM>
__global__ __launch_bounds__(kThreads, 1) void fmha_fwd_kernel(const Params p) {
  constexpr bool F8 = DT == kF8;
  constexpr int E = F8 ? 1 : 2;    // bytes per element
  constexpr int RB = D * E;        // bytes per K/V row, in memory and in LDS (swizzled)
  constexpr int CPR = RB / 16;     // 16-byte chunks per row
  constexpr int BN = F8 ? 2 * kBN : kBN;  // keys per K/V tile
  constexpr int NJB = BN / 32;     // 32-key blocks of a tile (S^T accumulators per wave)
  constexpr int TILE = BN * RB;    // LDS bytes per K or V tile
  constexpr int KBLK = TILE / 1024;  // 1 KiB LDS-direct loads (64 lanes x 16 B) per K or V tile
  constexpr int NBLK = 2 * KBLK;
  constexpr int NSTAGE = 3;          // K/V tile pairs resident in LDS: in use, landed, landing
  constexpr int STAGE = 2 * TILE;    // LDS bytes per stage: K tile, then V tile
  constexpr int LPP = (NBLK + 15) / 16;  // loads one wave issues per phase
  static_assert(NBLK % 8 == 0, "every wave issues the same number of tile loads");
  // fp8 with D = 32: one 64-deep MFMA k-step whose upper 32 dims are zero (the lanes that
  // supply them hold a zero Q operand and reread the K bytes of the lower half)
  constexpr bool F8_HALF = F8 && D == 32;
  constexpr int KS = F8 ? (D + 63) / 64 : D / 16;  // MFMA k-steps over the head dimension
  constexpr int NDB = D / 32;      // 32-wide blocks of the head dimension in O
  typedef Elem<DT == kF8 ? kBF16 : DT> T;  // (fp8 uses the helpers above instead)
  auto sw = [](int j) __attribute__((always_inline)) { return F8 ? swz8<CPR>(j) : swz<CPR>(j); };

  // The tile loads are inline assembly the compiler cannot see, so it inserts no waits for
  // them: every wait on them below is explicit.
  // LDS: the K/V stages, then one block of 32 Q rows per wave
  __shared__ __attribute__((aligned(1024))) char kv_lds[NSTAGE * STAGE + kWaves * 32 * RB];
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

  // ---- which (sequence, head) and which of its q-tiles this workgroup owns ------------
  const int BH = p.B * p.H;
  const int x = blockIdx.x;
  int bh, grp;
  if (p.rank_seqs) {
    // Packed batch: (sequence, head) pairs in the order of the sequences' key counts, longest
    // first, so that the longest streams start in the first round of workgroups (in batch order
    // a long sequence's q-tiles can land behind every other sequence's and run one after another
    // on one compute unit).  The pairs are dealt to the XCDs in turn and the workgroups of one
    // pair sit side by side on its XCD; lane i ranks sequence i (B <= 64).
    int pr;
    if (p.xcd_per) {
      const int slot = x >> 3;
      pr = (slot / p.ngrp) * 8 + (x & 7);
      grp = slot % p.ngrp;
    } else {
      pr = x / p.ngrp;
      grp = x % p.ngrp;
    }
    const int r = pr / p.H;
    const int hh = pr - r * p.H;
    const int sk_l = lane < p.B ? p.cu_k[lane + 1] - p.cu_k[lane] : -1;
    int rank = 0;
    for (int j = 0; j < p.B; ++j) {
      const int sk_j = __builtin_amdgcn_readlane(sk_l, j);
      rank += (sk_j > sk_l) | ((sk_j == sk_l) & (j < lane));
    }
    const uint64_t of_r = __ballot(lane < p.B && rank == r);  // one lane: the ranks are 0 .. B-1
    bh = (int)__builtin_ctzll(of_r) * p.H + hh;
  } else if (p.xcd_per) {  // round-robin dispatch puts workgroup x on XCD x % 8
    const int slot = x >> 3;
    if (p.ipw > 1) {  // the workgroups of one (sequence, head) side by side
      grp = slot % p.ngrp;
      bh = (x & 7) * p.xcd_per + slot / p.ngrp;
    } else {  // the heaviest q-tile of every (sequence, head) first
      grp = slot / p.xcd_per;
      bh = (x & 7) * p.xcd_per + slot % p.xcd_per;
    }
  } else {
    grp = x / BH;
    bh = x % BH;
  }
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
  // The workgroup runs the q-tiles ("items") in slots grp * ipw .. of its sequence one after
  // the other, as one stream of K/V tiles: the first tiles of an item are requested during
  // the last steps of the one before, its Q rows are loaded while that one still runs, and
  // the output of an item is written during the next item's first softmax phase, while the
  // other wave group keeps the matrix cores busy.  Slot order: one item per workgroup,
  // heaviest causal tile first; several, pairs of q-tiles n-1-j and j, whose causal tile
  // counts add up to the same total for every pair.
  const int nq_b = (Sq_b + kBM - 1) / kBM;  // q-tiles of this sequence
  const int slot0 = grp * p.ipw;
  if (slot0 >= nq_b) return;
  const int n_items = min(p.ipw, nq_b - slot0);
  const int off = p.qend ? Sk_b - Sq_b : 0;
  // keys visible to the last valid row of a row range, as an exclusive end
  auto key_end = [&](int last_row) { return p.causal ? min(Sk_b, last_row + off + 1) : Sk_b; };
  auto item_q0 = [&](int k) __attribute__((always_inline)) {  // first query row of item k
    const int s = slot0 + k;
    return kBM * (p.ipw == 1 ? nq_b - 1 - s : (s & 1) ? s >> 1 : nq_b - 1 - (s >> 1));
  };
  // K/V tiles of item k: those some row of it sees, and at least one (a row that sees no key
  // gets a tile of masked scores, hence O = 0 and LSE = -inf)
  auto item_tiles = [&](int k) __attribute__((always_inline)) {
    const int e = key_end(min(Sq_b, item_q0(k) + kBM) - 1);
    return e > 0 ? (e + BN - 1) / BN : 1;
  };
  int n_stream = 0;  // K/V tiles of the whole stream
  for (int k = 0; k < n_items; ++k) n_stream += item_tiles(k);

  // Buffer descriptors are rebased as the work moves: Q and O per q-tile (at its first row), K
  // and V per tile window (at the tile a load cursor stands on), each bounded by the end of the
  // sequence, so every in-descriptor offset stays small however long the sequence is.
  const uint32_t qstride = (uint32_t)p.H * D * E;     // bytes between rows of one head
  const uint32_t kstride = (uint32_t)p.H_kv * D * E;
  const char* q_seq = (const char*)p.q + ((size_t)q_row0 * p.H + h) * D * E;
  char* o_seq = (char*)p.o + ((size_t)q_row0 * p.H + h) * D * E;
  const size_t k_base = ((size_t)k_row0 * p.H_kv + kvh) * D * E;
  const char* k_seq = (const char*)p.k + k_base;
  const char* v_seq = (const char*)p.v + k_base;
  const uint64_t q_bytes = Sq_b > 0 ? (uint64_t)(Sq_b - 1) * qstride + RB : 0;
  const uint64_t k_bytes = Sk_b > 0 ? (uint64_t)(Sk_b - 1) * kstride + RB : 0;
  // bytes of a sequence from byte `from` on (0 past its end; a bound of 2^31 is far beyond the
  // three tiles or one q-tile a descriptor is ever used for)
  auto rest = [](uint64_t bytes, uint64_t from) __attribute__((always_inline)) {
    const uint64_t r = from < bytes ? bytes - from : 0;
    return (uint32_t)(r < 0x80000000ull ? r : 0x80000000ull);
  };
  auto q_rsrc = [&](int row0) __attribute__((always_inline)) {  // Q rows from row0 on
    const uint64_t from = (uint64_t)row0 * qstride;
    return make_rsrc_words(q_seq + from, rest(q_bytes, from));
  };
  auto o_rsrc = [&](int row0) __attribute__((always_inline)) {  // O rows from row0 on
    const uint64_t from = (uint64_t)row0 * qstride;
    return make_rsrc(o_seq + from, rest(q_bytes, from));
  };
  auto kv_rsrc = [&](const char* seq, uint64_t from) __attribute__((always_inline)) {  // K or V from byte `from`
    return make_rsrc_words(seq + from, rest(k_bytes, from));
  };

  // per item and wave: first row, this lane's query row, the first tile that some row of
  // the wave does not see completely (the mask is applied from there on), and the last key
  // visible to this lane's query, less the lane's key offset 4 h32 inside a tile.  The first
  // row of an item sees the fewest keys, so item_full(k), the first tile that some row of
  // the item does not see completely, is the least w_full of its waves.
  int iq0, qw0, qi, w_full, vis_last;
  auto set_rows = [&](int k) __attribute__((always_inline)) {
    iq0 = item_q0(k);
    qw0 = item_q0(k) + 32 * rblk;
    qi = qw0 + l32;
    w_full = 0x7fffffff;  // a wave with no row in the sequence: its output is dropped anyway
    if (qw0 < Sq_b) {
      const int first_sees = p.causal ? min(Sk_b, qw0 + off + 1) : Sk_b;
      w_full = first_sees > 0 ? first_sees / BN : 0;
    }
    vis_last = (p.causal ? min(Sk_b - 1, qi + off) : Sk_b - 1) - 4 * h32;
  };
  set_rows(0);
  auto item_full = [&](int k) __attribute__((always_inline)) {
    const int first_sees = p.causal ? min(Sk_b, item_q0(k) + off + 1) : Sk_b;
    return first_sees > 0 ? first_sees / BN : 0;
  };

  // ---- Q: each wave's 32 rows of an item land in its own LDS block (LDS-direct loads,
  // swizzled like a K tile) and are read from there into the B operand of S^T = K Q^T: lane
  // owns query l32, dims 8 h32.. of each k-step (fp8: 32 bytes, dims 64 ks + 32 h32 .., per
  // 64-deep k-step, in qf[2 ks], qf[2 ks + 1]).  The block then takes the next item's rows.
  constexpr int NQF = F8 ? 2 * KS : KS;
  constexpr int QBLK = 32 * RB / 1024;  // 1 KiB loads per wave for its rows of an item
  static_assert(QBLK * 1024 == 32 * RB, "a wave's Q rows are whole 1 KiB loads");
  const uint32_t q_lds = lds0 + (uint32_t)(NSTAGE * STAGE + wave_u * 32 * RB);
  const int rblk_u = 2 * (wave_u & 3) + (wave_u >> 2);  // rblk, in a scalar register
  auto load_q = [&](int k) __attribute__((always_inline)) {
    const i32x4 rq = q_rsrc(item_q0(k));
    const uint32_t row0 = (uint32_t)(32 * rblk_u) * qstride;
#pragma unroll
    for (int i = 0; i < QBLK; ++i) {
      const int pos = 64 * i + lane;  // 16-byte chunk position inside the wave's block
      const int j = pos / CPR;
      lds_load16(rq, row0 + (uint32_t)j * qstride + (((pos % CPR) ^ sw(j)) * 16), q_lds + 1024 * i);
    }
  };
  i32x4 qf[NQF];

  // ---- K/V tile loads straight into LDS, one 1 KiB block (64 lanes x 16 B) per instruction.
  // Block b of a tile covers rows 64b/CPR.. of it; lane l fills LDS chunk (64b + l) % CPR of
  // its row j with memory chunk ((64b + l) % CPR) ^ swz(j).
  //
  // Step u of the stream consumes L(u) = {K tile of stream tile u, V tile of stream tile u-1}
  // from LDS stage u % 3 (so the step that starts an item also holds the last V tile of the
  // item before).  L(u+2) is requested during phases 2u and 2u+1 by all 8 waves: block b of
  // its NBLK blocks (K first, then V) by wave b % 8 in the phase of parity (b / 8) % 2, spread
  // over that wave's MFMA or softmax work.  (Issued in bursts, or by fewer waves, the loads
  // queue at the CU's vector-memory path and stall the issuing waves for hundreds of
  // cycles.)  A load of a tile past either end of the sequence reads zeros, so each wave
  // issues the same NBLK / 8 loads every step.  The waits count this wave's requests: "at
  // most N in flight" covers every request older than the N newest, so the Q loads and O
  // stores that some steps add can only make a wait stricter, never looser.
  // Request cursor, at L(c): K tile lt of item litem (ln tiles), V tile of the item of L(c-1)
  // (tile -1 before the first; past the last item the K tile index runs on past its end), as
  // byte offsets in the K/V rows, and the LDS address of stage c % 3 plus this wave's first
  // block.  Kept as running sums: the loop carries no multiplies or remainders for them.
  const uint32_t tile_bytes = (uint32_t)BN * kstride;
  constexpr uint32_t kStages = NSTAGE * STAGE;
  static_assert(7 * 1024 < STAGE, "a wave's block offset stays inside the first stage");
  // The K descriptor starts at byte k_at of the sequence's K rows and the cursor's K tile lies
  // lk_off bytes past it; k_at only moves when lk_off reaches 2^30 (sequences past 1 GiB), and
  // back to 0 at a q-tile change after such a move.  V follows K one tile behind: at each advance
  // it takes over K's offset, and its descriptor is the V one at K's base of the step before.
  // These moves happen in special steps only; a plain step finds both bases unchanged.
  int lt = 0, ln = item_tiles(0), litem = 0;
  uint64_t k_at = 0;
  uint32_t lk_off = 0, lv_off = 0u - tile_bytes;  // (V before the first tile: out of bounds)
  i32x4 rk = kv_rsrc(k_seq, 0), rv = kv_rsrc(v_seq, 0), rv_next = rv;
  bool k_base_moved = false;                 // the last advance moved K's base
  constexpr uint32_t kRebase = 0x40000000u;  // far below 2^31 less three tiles
  uint32_t l_st = lds0 + (uint32_t)wave_u * 1024;
  auto advance = [&]() __attribute__((always_inline)) {
    lv_off = lk_off;
    rv = rv_next;
    l_st += STAGE;
    if (l_st >= lds0 + kStages) l_st -= kStages;
    k_base_moved = false;
    if ((lt + 1 < ln) | (litem + 1 >= n_items)) {
      ++lt;
      lk_off += tile_bytes;
    } else {
      ++litem;
      lt = 0;
      lk_off = 0;
      ln = item_tiles(litem);
      k_base_moved = k_at != 0;
      k_at = 0;
    }
    if (lk_off >= kRebase) {
      k_at += lk_off;
      lk_off = 0;
      k_base_moved = true;
    }
    if (k_base_moved) {
      rk = kv_rsrc(k_seq, k_at);
      rv_next = kv_rsrc(v_seq, k_at);
    }
  };
  uint32_t ld_off[2][LPP];  // per-lane byte offsets inside a tile of this wave's blocks
#pragma unroll
  for (int pp = 0; pp < 2; ++pp)
#pragma unroll
    for (int i = 0; i < LPP; ++i) {
      const int b = 16 * i + 8 * pp + wave_u;
      const int pos = (b % KBLK) * 64 + lane;  // 16-byte chunk position inside the tile
      const int j = pos / CPR;
      // fp8 V tiles: LDS row j holds key row j with bits 2 and 3 swapped, so that the
      // transposed reads hand each lane the keys of its own probabilities (see pv_mma).
      const int jg = (F8 && b >= KBLK && (((j >> 2) ^ (j >> 3)) & 1)) ? j ^ 12 : j;
      ld_off[pp][i] = (uint32_t)jg * kstride + (((pos % CPR) ^ sw(j)) * 16);
    }
  // load i of phase parity pp for the cursor's L(c) into stage c % 3
  auto load_unit = [&](int pp, int i) __attribute__((always_inline)) {
    const int b0 = 16 * i + 8 * pp;  // first block of this (pp, i) over the 8 waves
    if (b0 >= NBLK) return;          // compile-time after unrolling
    const bool is_k = b0 + 8 <= KBLK ? true : b0 >= KBLK ? false : b0 + wave_u < KBLK;
    const uint32_t goff = (is_k ? lk_off : lv_off) + ld_off[pp][i];
    lds_load16(is_k ? rk : rv, goff, __builtin_amdgcn_readfirstlane(l_st + b0 * 1024));
  };

  f32x16 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
  f32x16 s[NJB];                    // scores of the tile between its matrix and softmax phases
  constexpr int NPK = F8 ? 4 : 8;   // packed probability registers per 32-key block
  uint32_t pk[NJB][NPK] = {};       // probabilities of the tile between its softmax and PV phases
  bool pk_masked = false;           // 16-bit: pk holds a masked tile, whose row sum the matrix cores add
  float m_run = -__builtin_inff();  // running max of scale*log2(e)*s for query l32
  // Row sums on the matrix cores: a selecting all-ones A operand against the probability
  // operand of the PV product, so element 0 of acc_l holds the row sum of this lane's query
  // over the rounded probabilities that O is built from (exact in fp32).  fp8 sums every tile
  // there (one 16x16x128 MFMA per 64 keys, see pv_mma); the 16-bit paths only the tiles that
  // needed the mask (one 16x16x32 MFMA per 16 keys after the tile's PV product), where a row
  // with few visible keys must be normalised by exactly the weights of its numerator, and add
  // the fp32 probabilities of fully visible tiles on the vector ALU (l_run + l_run2), where the
  // longer 16-bit matrix phase hides them.
  f32x4 acc_l = {};
  // The A operand of those 16x16 MFMAs: lane l holds A row l % 16 over k-block l / 16 and
  // receives C rows 4 (l / 16) + 0..3 of column l % 16.  The probability operand puts query
  // q = l % 32 in column q % 16 of k-blocks (q / 16) + {0, 2}, so A rows 0 and 8 take blocks 0
  // and 2 (queries 0..15), rows 4 and 12 blocks 1 and 3 (queries 16..31), all other rows
  // nothing, and every lane's C element 0 is its own query's sum.
  const bool rowsum_lane = ((lane & 3) == 0) && (((lane >> 2) ^ (lane >> 4)) & 1) == 0;
  const int f8_ones = rowsum_lane ? 0x38383838 : 0;
  float l_run = 0.0f;  // this lane's part of the VALU row sum (l_run + l_run2)
  float l_run2 = 0.0f;
  constexpr bool VSUM = !F8 || LSE_SUM;  // keep the VALU row sum
  const float sl2 = p.scale_log2;
  const float sl2_bits = 8388608.0f * sl2;  // fp8 without an LSE: 2^23 scale log2(e)

  // Per-lane LDS byte offsets.  The swizzle only touches chunk bits that the k-step (K) or
  // the d-block (V) index leaves clear, so every read address is one of these bases XOR a
  // compile-time constant, plus an immediate row offset.
  //   16-bit: K row l32, chunk 2 ks + h32; fp8: K row l32, chunks 4 ks + 2 h32 (+1).
  const int k_lane = l32 * RB + (((F8 ? (F8_HALF ? 0 : 2 * h32) : h32) ^ sw(l32)) * 16);
  const int k_lane2 = l32 * RB + ((((F8_HALF ? 0 : 2 * h32) + 1) ^ sw(l32)) * 16);  // fp8 only
  const int g16 = (lane >> 4) & 1;
  const int s16 = lane & 15;
  // 16-bit V transpose read (ds_read_b64_tr_b16): row 4 h32 + s16 / 4 of a 16-row group (and
  // that row + 8), 8 bytes at column 16 g16 + 4 (s16 % 4).
  // fp8 (ds_read_b64_tr_b8, which hands lane j of each 16-lane group byte j % 8 of the words
  // of lanes j / 8, j / 8 + 2, ..): lane l supplies LDS row 8 h32 + s16 / 2 of a 16-row chunk,
  // 8 bytes at column 16 g16 + 8 (s16 % 2), and gets column l32 of LDS rows 8 h32 + 0..7
  // (keys 8 (r / 4) + 4 h32 + r % 4, r = 0..7, of the chunk: the V rows are stored permuted).
  const int v_row0 = F8 ? 8 * h32 + (s16 >> 1) : 4 * h32 + (s16 >> 2);
  const int v_part = F8 ? g16 : 2 * g16 + ((s16 & 3) >> 1);
  const int v_lane0 = TILE + v_row0 * RB + ((v_part ^ sw(v_row0)) * 16) + 8 * (s16 & 1);
  const int v_lane1 = TILE + (v_row0 + 8) * RB + ((v_part ^ sw(v_row0 + 8)) * 16) + 8 * (s16 & 1);

  // Q fragment from the wave's LDS block (the K read addresses: the rows are swizzled alike).
  // The values are pinned before the block may take the next item's rows.
  auto read_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NQF; ++i) {
      if constexpr (F8)
        qf[i] = *(const lds_i32x4*)(uintptr_t)(((i & 1) ? q_lds + k_lane2 : q_lds + k_lane) ^ (64 * (i >> 1)));
      else
        qf[i] = *(const lds_i32x4*)(uintptr_t)((q_lds + k_lane) ^ (32 * i));
    }
    if constexpr (F8_HALF) {  // dims 32..63 of the k-step do not exist
#pragma unroll
      for (int i = 0; i < NQF; ++i) qf[i] = h32 ? i32x4{} : qf[i];
    }
#pragma unroll
    for (int i = 0; i < NQF; ++i) asm volatile("" : "+v"(qf[i]));
  };

  // fp8: one QK^T MFMA of the tile, k-step ks of key block jb (ka, kb: k_lane, k_lane2 + the
  // stage's address).  (The 16-bit matrix phase has its own operand pipeline below.)
  auto qk_mma = [&](uint32_t ka, uint32_t kb, int i) __attribute__((always_inline)) {
    const int jb = i % NJB, ks = i / NJB;
    const i32x4 a0 = *(const lds_i32x4*)(uintptr_t)((ka ^ (64 * ks)) + 32 * jb * RB);
    const i32x4 a1 = *(const lds_i32x4*)(uintptr_t)((kb ^ (64 * ks)) + 32 * jb * RB);
    const i32x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
    const i32x8 b = __builtin_shufflevector(qf[2 * ks], qf[2 * ks + 1], 0, 1, 2, 3, 4, 5, 6, 7);
    s[jb] = mma_f8(a, b, s[jb]);
  };
  // fp8: one PV MFMA, d-block i % NDB and 64-key half kh = i / NDB of the 128-key tile; byte
  // 8 c + r of either operand is key 64 kh + 16 c + 8 (r / 4) + 4 h32 + r % 4: the order in
  // which the softmax packs the probabilities (4 per register, straight from the accumulator
  // layout).  Transposed read c hands lane l column l32 of LDS rows 16 c + 8 h32 + 0..7, and
  // the V tile stores key row j at LDS row j with bits 2 and 3 swapped, so those LDS rows hold
  // exactly these keys, and the probabilities need no exchange between lanes.
  auto pv_mma = [&](uint32_t va0, int i) __attribute__((always_inline)) {
    const int db = i % NDB, kh = i / NDB;
    i32x2 t[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      t[c] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (lds_i32x2*)(uintptr_t)((va0 ^ (32 * db)) + (64 * kh + 16 * c) * RB));
    const i32x8 a = {t[0][0], t[0][1], t[1][0], t[1][1], t[2][0], t[2][1], t[3][0], t[3][1]};
    const i32x8 b = {(int)pk[2 * kh][0], (int)pk[2 * kh][1], (int)pk[2 * kh][2], (int)pk[2 * kh][3],
                     (int)pk[2 * kh + 1][0], (int)pk[2 * kh + 1][1], (int)pk[2 * kh + 1][2], (int)pk[2 * kh + 1][3]};
    acc_o[db] = mma_f8(a, b, acc_o[db]);
    if (db == NDB - 1) {  // row sums of this half (e4m3 1.0 = 0x38): see f8_ones
      const i32x8 ones = {f8_ones, f8_ones, f8_ones, f8_ones, f8_ones, f8_ones, f8_ones, f8_ones};
      acc_l = rowsum_f8(ones, b, acc_l);
    }
  };
  constexpr int NQK = NJB * KS;              // MFMAs of S^T for one tile
  constexpr int NPV = F8 ? 2 * NDB : 4 * NDB;  // MFMAs of O^T += V^T P^T for one tile
  constexpr int RQK = F8 ? 2 : 1;            // LDS reads per S^T MFMA
  constexpr int RPV = F8 ? 4 : 2;            // LDS reads per O^T MFMA

  auto pin_l = [&]() __attribute__((always_inline)) {
    asm volatile("" : "+v"(acc_l));
  };
  // matrix phase of stream tile u: S(u) = K(u) Q^T and O += V(u-1) P(u-1), from the LDS stage
  // at st (stage u % 3); hook(j), j < LPP, issues this wave's loads of the phase.  Every wave runs every tile of
  // the workgroup: past a wave's last visible tile its probabilities are zero, and the
  // phase takes as long as the busiest wave of the group anyway.
  // MASKABLE (special steps): the previous tile may have been masked, and then its row sums
  // are added here.
  auto matrix_phase = [&](uint32_t st, auto& hook, auto maskable_tag) __attribute__((always_inline)) {
    constexpr bool MASKABLE = decltype(maskable_tag)::value;
    constexpr int N = NQK > NPV ? NQK : NPV;
    uint32_t ka = k_lane + st, kb = k_lane2 + st, va0 = v_lane0 + st, va1 = v_lane1 + st;
    // keep derived addresses out of loop-invariant code
    if constexpr (F8)
      asm volatile("" : "+v"(ka), "+v"(kb), "+v"(va0));
    else
      asm volatile("" : "+v"(ka), "+v"(va0), "+v"(va1));
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) s[jb] = f32x16{};
    if constexpr (!F8) {
      // 16-bit: an explicit software pipeline.  Each b128 K read is issued kKLead S^T MFMAs
      // before its use (four 4-register buffers), each pair of V^T transpose reads kVLead PV
      // MFMAs before.  (Left to the compiler with a plain read-ahead count, the K buffers
      // alternated between two, each refilled right after the MFMA that freed it; the deeper
      // K lead measured ~1% faster.  The operand reads still cost the matrix phase time: the
      // b128 K reads far more per byte than the b64 transpose reads of V.)
      constexpr int KL = kKLead < NQK ? kKLead : NQK;
      constexpr int VL = kVLead < NPV ? kVLead : NPV;
      auto rdk = [&](int i) __attribute__((always_inline)) {  // A operand of S^T MFMA i
        const int jb = i & 1, ks = i >> 1;
        return *(const lds_i32x4*)(uintptr_t)((ka ^ (32 * ks)) + 32 * jb * RB);
      };
      auto rdv = [&](int i) __attribute__((always_inline)) {  // A operand of PV MFMA i
        const int db = i % NDB, jc = i / NDB, jb = jc >> 1, c = jc & 1;
        const uint32_t rows = (32 * jb + 16 * c) * RB;
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)((va0 ^ (64 * db)) + rows));
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)((va1 ^ (64 * db)) + rows));
        return i32x4{__builtin_bit_cast(int, __builtin_shufflevector(v0, v0, 0, 1)),
                     __builtin_bit_cast(int, __builtin_shufflevector(v0, v0, 2, 3)),
                     __builtin_bit_cast(int, __builtin_shufflevector(v1, v1, 0, 1)),
                     __builtin_bit_cast(int, __builtin_shufflevector(v1, v1, 2, 3))};
      };
      i32x4 kbuf[KL], vbuf[VL];
#pragma unroll
      for (int j = 0; j < KL; ++j) kbuf[j] = rdk(j);
#pragma unroll
      for (int j = 0; j < VL; ++j) vbuf[j] = rdv(j);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        if (i < NQK) {
          s[i & 1] = T::mma(kbuf[i % KL], qf[i >> 1], s[i & 1]);
          if (i + KL < NQK) kbuf[i % KL] = rdk(i + KL);
        }
        if (i < NPV) {
          const int db = i % NDB, jc = i / NDB, jb = jc >> 1, c = jc & 1;
          const i32x4 bp = {(int)pk[jb][4 * c], (int)pk[jb][4 * c + 1], (int)pk[jb][4 * c + 2], (int)pk[jb][4 * c + 3]};
          acc_o[db] = T::mma(vbuf[i % VL], bp, acc_o[db]);
          if (i + VL < NPV) vbuf[i % VL] = rdv(i + VL);
        }
#pragma unroll
        for (int j = 0; j < LPP; ++j)  // load j goes after step j * N / LPP
          if ((j * N) / LPP == i) hook(j);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, KL + 2 * VL, 0);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        if (i < NQK) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          if (i + KL < NQK) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        if (i < NPV) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          if (i + VL < NPV) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
      }
    } else {
      // fp8: the S^T MFMAs first, then the PV MFMAs, so the tile's row max (in the softmax code,
      // free to move here) runs on the vector ALU while the PV products execute: an fp8 phase
      // has half the MFMA time of a 16-bit one per key, so the vector work beside it matters more.
#pragma unroll
      for (int i = 0; i < NQK; ++i) qk_mma(ka, kb, i);
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        pv_mma(va0, i);
#pragma unroll
        for (int j = 0; j < LPP; ++j)  // load j goes after PV step j * NPV / LPP
          if ((j * NPV) / LPP == i) hook(j);
      }
      // The LDS reads run kPrefetch reads ahead of the MFMAs that consume them (pinned with
      // scheduling groups: the compiler alone keeps only one or two in flight, which leaves
      // the matrix core waiting on LDS latency).
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kPrefetch, 0);
#pragma unroll
      for (int i = 0; i < NQK; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, RQK, 0);
      }
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        if (i % NDB == NDB - 1)  // this step also adds the row sums of its 64 keys
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
        else
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, RPV, 0);
      }
    }
    // Pin the products here: the compiler may otherwise sink MFMAs past the phase barrier,
    // into the softmax or the epilogue of an item that follows on this wave.
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) asm volatile("" : "+v"(s[jb]));
#pragma unroll
    for (int db = 0; db < NDB; ++db) asm volatile("" : "+v"(acc_o[db]));
    if constexpr (!F8 && MASKABLE) {
      if (pk_masked) {
        const int one = rowsum_lane ? (DT == kBF16 ? 0x3F803F80 : 0x3C003C00) : 0;
        const i32x4 ones = {one, one, one, one};
#pragma unroll
        for (int jc = 0; jc < 4; ++jc) {
          const i32x4 bp = {(int)pk[jc >> 1][4 * (jc & 1)], (int)pk[jc >> 1][4 * (jc & 1) + 1],
                            (int)pk[jc >> 1][4 * (jc & 1) + 2], (int)pk[jc >> 1][4 * (jc & 1) + 3]};
          acc_l = rowsum_16<DT>(ones, bp, acc_l);
        }
      }
    }
    pin_l();
  };

  // softmax phase of tile t: mask, running max, lazy rescale, probabilities; hook(j), j <
  // LPP, issues this wave's loads of the phase, spread over the exponentials.  Not MASKABLE
  // (plain steps): every row of every wave sees the whole tile.
  auto softmax_phase = [&](int t, auto& hook, auto maskable_tag) __attribute__((always_inline)) {
    constexpr bool MASKABLE = decltype(maskable_tag)::value;
    // 16-bit: the scores are pinned again here, after the phase barrier, so that the row max
    // (which waits for the last S^T MFMA) cannot be hoisted into the matrix phase: there it
    // held the wave back from the barrier while its last MFMAs drained, and the other group's
    // matrix work started only after that.  Issued MFMAs complete across a barrier by
    // themselves.  (fp8 issues its S^T MFMAs first and lets the max move up.)
    if constexpr (!F8) asm volatile("" : "+v"(s[0]), "+v"(s[1]));
    if (MASKABLE && t >= w_full) {  // some key of the tile is hidden from some row of the wave
      // score (jb, r) belongs to key t BN + 4 h32 + 32 jb + 8 (r / 4) + r % 4
      const int lim = vis_last - t * BN;
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[jb][r] = 32 * jb + 8 * (r >> 2) + (r & 3) <= lim ? s[jb][r] : -__builtin_inff();
    }
    float mx = s[0][0];
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[jb][r]);
    mx = wave_row_max(mx);
    const float m_cand = mx * sl2;
    if (__any(m_cand > m_run + (F8 ? kF8Threshold : kRescaleThreshold))) {
      const float m_new = __builtin_fmaxf(m_run, m_cand);
      const float alpha = m_new == -__builtin_inff() ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      acc_l[0] *= alpha;  // (the only element read)
      if constexpr (VSUM) {
        l_run *= alpha;
        l_run2 *= alpha;
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc_o[db] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -__builtin_inff() ? 0.0f : m_run) - (F8 ? kF8Shift : 0.0f);
    const float bits_add = 8388608.0f * (127.0f - kF8ExpCentre - m_use);
    // exponentials, packing and VALU row sums (fp32; none for a masked 16-bit tile, which the
    // matrix cores sum; fp8: only for an LSE)
    auto exps = [&](auto masked_tag) __attribute__((always_inline)) {
      constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {  // scores 4 qd .. 4 qd + 3: keys 8 qd + 4 h32 + 0..3
          float e[4];
          if constexpr (F8 && !VSUM && !MASKED) {
            // 2^x from the bits 2^23 (x + 127 - c) (kF8ExpCentre).  v_cvt_u32_f32 saturates: a
            // score far below the row max gives +0.  (Tiles that some row of the wave sees only
            // in part take the exact exponential below: a row with few keys has all of them
            // there, and its few weights would not average the approximation out.)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const float y = __builtin_fmaf(s[jb][4 * qd + u], sl2_bits, bits_add);
              uint32_t bits;
              asm("v_cvt_u32_f32 %0, %1" : "=v"(bits) : "v"(y));
              e[u] = __builtin_bit_cast(float, bits);
            }
          } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) e[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[jb][4 * qd + u], sl2, -m_use));
          }
          if constexpr (F8) {  // (the old value is overwritten whole: no zeroing move)
            pk[jb][qd] = pack_f8x4_over(pk[jb][qd], e[0], e[1], e[2], e[3]);
          } else {
            pk[jb][2 * qd] = T::pack(e[0], e[1]);
            pk[jb][2 * qd + 1] = T::pack(e[2], e[3]);
          }
          if constexpr (VSUM && !(!F8 && MASKED)) {
            l_run += e[0] + e[2];
            l_run2 += e[1] + e[3];
          }
#pragma unroll
          for (int j = 0; j < LPP; ++j)  // load j goes after exponential quad j * 4 NJB / LPP
            if ((j * 4 * NJB) / LPP == 4 * jb + qd) hook(j);
        }
    };
    if constexpr (F8 && (VSUM || !MASKABLE)) {
      exps(std::false_type{});
    } else if constexpr (F8) {
      if (__builtin_amdgcn_readfirstlane(t >= w_full))
        exps(std::true_type{});
      else
        exps(std::false_type{});
    } else if constexpr (MASKABLE) {
      pk_masked = __builtin_amdgcn_readfirstlane(t >= w_full);
      if (pk_masked)
        exps(std::true_type{});
      else
        exps(std::false_type{});
    } else {
      pk_masked = false;
      exps(std::false_type{});
    }
    // Pin the results here: the compiler may otherwise sink the tail of this arithmetic past
    // the phase barrier, into the matrix phase that follows on this wave.
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
      for (int q = 0; q < NPK; ++q) asm volatile("" : "+v"(pk[jb][q]));
    asm volatile("" : "+v"(m_run));
    if constexpr (VSUM) asm volatile("" : "+v"(l_run), "+v"(l_run2));
  };

  // The matrix work runs at raised wave priority so the SIMD issues its MFMAs ahead of the
  // softmax VALU work of the other group's wave.
  auto matrix_prio = [&](uint32_t st, auto& hook, auto maskable_tag) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    matrix_phase(st, hook, maskable_tag);
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
  auto no_work = [&](auto pp_tag) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LPP; ++i) load_unit(decltype(pp_tag)::value, i);
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;

  // ---- epilogue of an item: normalise, scale, convert, store; LSE.  A lane swap with lane
  // l^32 gives every lane 8 consecutive head dims of its row (16 bytes for 16-bit O).  Rows
  // past the sequence fall outside the O descriptor and are dropped.  Issues NST stores of O
  // (and one LSE store where due) and clears the item state.
  constexpr int NST = 2 * NDB;
  auto epilogue = [&]() __attribute__((always_inline)) {
    const auto ro = o_rsrc(iq0);
    const uint32_t orow = (uint32_t)(qi - iq0) * qstride;  // this lane's row inside the q-tile
    const float l_tot = F8 ? acc_l[0] : acc_l[0] + wave_row_sum(l_run + l_run2);
    const float inv = l_tot > 0.0f ? p.o_scale / l_tot : 0.0f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        // quads g = 2 gp (dims 16 gp + 4 h32 ..) and 2 gp + 1 (dims 16 gp + 8 + 4 h32 ..): after
        // the swap the lane holds dims 32 db + 16 gp + 8 h32 + 0..7
        const int g0 = 2 * gp, g1 = 2 * gp + 1;
        const uint32_t byte = (uint32_t)(32 * db + 16 * gp + 8 * h32) * E;
        if constexpr (F8) {  // saturate to the largest finite e4m3 value, then round
          float x0[4], x1[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            x0[u] = __builtin_fminf(__builtin_fmaxf(acc_o[db][4 * g0 + u] * inv, -448.0f), 448.0f);
            x1[u] = __builtin_fminf(__builtin_fmaxf(acc_o[db][4 * g1 + u] * inv, -448.0f), 448.0f);
          }
          auto r = __builtin_amdgcn_permlane32_swap(pack_f8x4(x0[0], x0[1], x0[2], x0[3]),
                                                    pack_f8x4(x1[0], x1[1], x1[2], x1[3]), false, false);
          const i32x2 w = {(int)r[0], (int)r[1]};
          __builtin_amdgcn_raw_buffer_store_b64(w, ro, orow + byte, 0, 0);
        } else {
          auto r0 = __builtin_amdgcn_permlane32_swap(T::pack(acc_o[db][4 * g0] * inv, acc_o[db][4 * g0 + 1] * inv),
                                                     T::pack(acc_o[db][4 * g1] * inv, acc_o[db][4 * g1 + 1] * inv),
                                                     false, false);
          auto r1 = __builtin_amdgcn_permlane32_swap(
              T::pack(acc_o[db][4 * g0 + 2] * inv, acc_o[db][4 * g0 + 3] * inv),
              T::pack(acc_o[db][4 * g1 + 2] * inv, acc_o[db][4 * g1 + 3] * inv), false, false);
          const i32x4 w = {(int)r0[0], (int)r1[0], (int)r0[1], (int)r1[1]};
          __builtin_amdgcn_raw_buffer_store_b128(w, ro, orow + byte, 0, 0);
        }
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
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
    acc_l = f32x4{};
    l_run = 0.0f;
    l_run2 = 0.0f;
    m_run = -__builtin_inff();
  };

  // ---- prologue: Q of the first item, L(0) (K of its first tile and the zero V(-1)) and L(1)
  // into stages 0 and 1; the phases start once L(0) and group A's Q rows are in (L(1) is waited
  // for at the end of phase 1, like every later tile).  Group B runs no matrix work before phase
  // 1, so its waves request their Q rows after L(0) and read them at the end of phase 0: the
  // first phase waits for half the Q bytes.  Then each block takes the second item's Q rows.
  const bool grp_b = wave_u >= 4;  // (scalar: the branches below hold no accumulators)
  if (!grp_b) load_q(0);
  no_work(P0{});
  no_work(P1{});
  advance();
  if (grp_b) load_q(0);
  no_work(P0{});
  no_work(P1{});
  advance();
  if (grp_b)
    wait_vmcnt<NBLK / 8 + QBLK>();  // L(0); Q and L(1) may be in flight
  else
    wait_vmcnt<NBLK / 8>();  // Q and L(0)
  phase_barrier();
  if (!grp_b) {
    read_q();
    if (n_items > 1) load_q(1);
  }

  // Phases 0 .. 2 n_stream + 1.  Group A: matrix(u) in phase 2u, softmax(u) in 2u+1.  Group
  // B: softmax(u-1) in phase 2u, matrix(u) in 2u+1.  Each group runs its own straight loop
  // (the two meet at the same barriers), so no phase body branches on the group.  Item
  // changes: matrix(u) of the first tile u of item k multiplies item k's Q and adds the last
  // PV product of item k-1, so item k-1 is written out at the start of softmax(u); item k's Q
  // is read from LDS at the end of softmax(u-1) (its rows were requested at least one step
  // earlier, so at least NBLK / 8 newer requests stand behind them there).
  // compute cursor: item, tile inside it, its tiles, LDS address of stage u % 3
  int k = 0, t = 0, nt = item_tiles(0), nfull = item_full(0);
  uint32_t c_st = lds0;
  auto next_tile = [&]() __attribute__((always_inline)) {
    c_st += STAGE;
    if (c_st >= lds0 + kStages) c_st -= kStages;
    if (++t == nt) {
      ++k;
      t = 0;
      nt = item_tiles(k);
      nfull = item_full(k);
    }
  };
  // Steps come in two builds.  A plain step neither starts nor ends an item, neither of its
  // requests moves the cursor into the next item, and every row of the item sees its whole
  // tile: it runs without any of that control and mask code (in the softmax phase every
  // extra instruction costs issue time).  The others (the first tile of an item after the
  // first, the last three tiles of an item before the last, and tiles from item_full on) are
  // special steps with the full bookkeeping.  plain_end() is the end of the run of plain
  // steps that starts at step u (u itself when step u is special).
  auto plain_end = [&](int u) __attribute__((always_inline)) {
    if (((t == 0) & (k > 0)) | k_base_moved) return u;
    int lim = k + 1 == n_items ? n_stream : u - t + nt - 3;
    lim = min(lim, u - t + nfull);
    // the K offset stays below the rebase point through the run (a special step rebases)
    lim = min(lim, u + (int)((kRebase - 1 - lk_off) / tile_bytes));
    return lim > u ? lim : u;
  };
  auto plain_advance = [&]() __attribute__((always_inline)) {
    lv_off = lk_off;
    lk_off += tile_bytes;
    ++lt;
    l_st += STAGE;
    if (l_st >= lds0 + kStages) l_st -= kStages;
  };
  auto plain_next_tile = [&]() __attribute__((always_inline)) {
    ++t;
    c_st += STAGE;
    if (c_st >= lds0 + kStages) c_st -= kStages;
  };
  auto h0 = [&](int i) __attribute__((always_inline)) { load_unit(0, i); };
  auto h1 = [&](int i) __attribute__((always_inline)) { load_unit(1, i); };
  if (group == 0) {
    auto step = [&](auto special_tag) __attribute__((always_inline)) {
      constexpr bool SPECIAL = decltype(special_tag)::value;
      matrix_prio(c_st, h0, special_tag);
      even_end();
      const bool first = SPECIAL && (t == 0) & (k > 0);
      if (first) {
        epilogue();
        set_rows(k);
      }
      softmax_phase(t, h1, special_tag);
      // At the end of the phase L(u+1) must have landed.  The newest requests are this step's
      // NBLK / 8 for L(u+2), and after an epilogue also its NST stores of O.
      if (first)
        wait_vmcnt<NBLK / 8 + NST>();
      else
        wait_vmcnt<NBLK / 8>();
      if (SPECIAL && (t == nt - 1) & (k + 1 < n_items)) {
        read_q();
        if (k + 2 < n_items) load_q(k + 2);
      }
      phase_barrier();
      if constexpr (SPECIAL) {
        advance();
        next_tile();
      } else {
        plain_advance();
        plain_next_tile();
      }
    };
    for (int u = 0; u < n_stream;) {
      for (const int e = plain_end(u); u < e; ++u) step(std::false_type{});
      if (u < n_stream) {
        step(std::true_type{});
        ++u;
      }
    }
    matrix_prio(c_st, h0, std::true_type{});  // O += V P of the last tile
    even_end();
    no_work(P1{});
    odd_end();
  } else {
    no_work(P0{});
    // this wave's Q rows (requested after L(0), before L(1)): only L(1) and this phase's loads
    // may still be in flight
    wait_vmcnt<NBLK / 8 + LPP>();
    read_q();
    if (n_items > 1) load_q(1);
    even_end();
    auto step = [&](auto special_tag) __attribute__((always_inline)) {
      constexpr bool SPECIAL = decltype(special_tag)::value;
      matrix_prio(c_st, h1, special_tag);
      odd_end();
      if constexpr (SPECIAL) {
        advance();
        if ((t == 0) & (k > 0)) {
          epilogue();
          set_rows(k);
          if (k + 1 < n_items) load_q(k + 1);
        }
      } else {
        plain_advance();
      }
      softmax_phase(t, h0, special_tag);
      if (SPECIAL && (t == nt - 1) & (k + 1 < n_items)) {
        // item k+1's rows were requested at the start of this phase (a one-tile item k > 0:
        // only this phase's LPP loads are newer) or at least one step earlier
        if (nt == 1)
          wait_vmcnt<LPP>();
        else
          wait_vmcnt<NBLK / 8>();
        read_q();
      }
      even_end();
      if constexpr (SPECIAL)
        next_tile();
      else
        plain_next_tile();
    };
    for (int u = 0; u < n_stream;) {
      for (const int e = plain_end(u); u < e; ++u) step(std::false_type{});
      if (u < n_stream) {
        step(std::true_type{});
        ++u;
      }
    }
    matrix_prio(c_st, h1, std::true_type{});
    odd_end();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the requests past the end (they write LDS)
  epilogue();
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
    case FMHA_ERR_HIP: return "HIP kernel launch failed, or the scratch array's device address is unavailable";
    case FMHA_ERR_SCRATCH_TOO_SMALL: return "shape needs more workspace than the 32 MiB static scratch array";
  }
  return "unknown status";
}

int32_t fmha_version(void) { return 200; }

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

  const int64_t esz = dtype == FMHA_DTYPE_F8E4M3 ? 1 : 2;
  // The kernel rebases its buffer descriptors per q-tile and per K/V tile window, so sequences
  // may be of any length; what one descriptor spans (three K/V tiles, one q-tile of 256 rows)
  // must stay inside the 31-bit offset range, and row indices inside int32.
  const int64_t lim = (int64_t)1 << 31;
  if ((int64_t)3 * (esz == 1 ? 2 * kBN : kBN) * H_kv * D * esz >= lim || (int64_t)kBM * H * D * esz >= lim) return FMHA_ERR_UNSUPPORTED;
  if (!packed && ((int64_t)B * Sq >= lim || (int64_t)B * Sk >= lim)) return FMHA_ERR_UNSUPPORTED;
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
  p.causal = mask == FMHA_MASK_CAUSAL_QBEGIN || mask == FMHA_MASK_CAUSAL_QEND;
  p.qend = mask == FMHA_MASK_CAUSAL_QEND;
  const int64_t BH = (int64_t)B * H;
  const int64_t n_qtiles = (Sq + kBM - 1) / kBM;  // per sequence (packed: of the longest)
  // q-tiles per workgroup: as many as leave one workgroup per compute unit or more, at most 8,
  // even when causal (pairs of a heavy and a light tile); one when there is less work
  const int cus = compute_units();
  if (cus < 1) return FMHA_ERR_HIP;
  // packed batches of up to 64 sequences are ordered by key count in the kernel, and their
  // q-tiles are counted from the total rows (at most total / 256 + B), not as B times the longest
  p.rank_seqs = packed && B <= 64 ? 1 : 0;
  int64_t qtiles_all = (int64_t)B * n_qtiles;
  if (p.rank_seqs && varlen->total_length_q / kBM + B < qtiles_all) qtiles_all = varlen->total_length_q / kBM + B;
  int64_t ipw = (int64_t)H * qtiles_all / cus;
  ipw = ipw < 1 ? 1 : ipw > 8 ? 8 : ipw;
  if (ipw > n_qtiles) ipw = n_qtiles;
  if (p.causal && ipw > 1) ipw &= ~(int64_t)1;
  p.xcd_per = (BH % 8 == 0) ? (int32_t)(BH / 8) : 0;
  if (p.xcd_per && ipw > 2) {
    // Every q-tile of a workgroup streams the whole (causal: visible) K/V of its head again,
    // and the workgroups of one head, dispatched side by side, share that stream in L2 while
    // they run together.  Fewer q-tiles per workgroup mean more workgroups per head and fewer
    // heads on an XCD at once: take the largest halving of ipw (down to 2) at which the K/V
    // heads the XCD's resident workgroups (one per CU) stream fit its 4 MiB L2, if any does.
    const int64_t per_xcd = cus / 8 > 0 ? cus / 8 : 1;
    const int64_t kv_head_bytes = (int64_t)2 * Sk * D * esz;
    for (int64_t w = ipw; w >= 2; w /= 2) {
      const int64_t we = p.causal ? (w & ~(int64_t)1) : w;
      const int64_t per_head = (n_qtiles + we - 1) / we;
      int64_t heads = (per_xcd + per_head - 1) / per_head;
      if (heads > p.xcd_per) heads = p.xcd_per;
      if ((heads + p.group - 1) / p.group * kv_head_bytes <= ((int64_t)4 << 20)) {
        ipw = we;
        break;
      }
    }
  }
  p.ipw = (int32_t)ipw;
  p.ngrp = (int32_t)((n_qtiles + ipw - 1) / ipw);
  const int64_t grid = BH * p.ngrp;
  if (grid >= lim) return FMHA_ERR_UNSUPPORTED;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  p.o_scale = o_scale;

  hipError_t err = hipSuccess;
  if (dtype == FMHA_DTYPE_F8E4M3) {
    if (D == 32) err = launch<kF8, 32>(p, (int)grid, stream);
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
