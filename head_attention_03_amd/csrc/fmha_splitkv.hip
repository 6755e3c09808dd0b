// Split-KV attention forward for few query rows per head (generation / decode) on gfx950.
//
// The same O = softmax(scale * Q K^T + mask) V and LSE as fmha_fwd, for shapes where every
// head has only a few query rows and a long key range: the keys of each (sequence, K/V head)
// are cut into splits that run on different workgroups, each writing a partial result
// (O_s normalised, LSE_s) to a caller-provided workspace, and a second kernel merges the
// splits, O = sum_s exp(LSE_s - LSE) O_s with LSE = log sum_s exp(LSE_s).  This is the
// generation kernel with its split-KV reduction that the trdm.cn walk-through "CUTLASS
// Blackwell FMHA 示例完全解析" describes (sections on the generation kernel and the
// reduction), with the query heads of a GQA group packed into the rows of one MFMA tile, as
// the CUTLASS examples/77_blackwell_fmha README does for generation ("FMHA for Blackwell:
// Generation").
//
// CDNA4 design:
// * The work is bound by HBM bandwidth (each K/V byte meets only the few query rows of its
//   group), so the kernel is built to keep loads in flight rather than to share K/V tiles:
//   each wave streams its 32-key tiles through a private ring of 4 LDS stages (LDS-direct
//   loads, three tiles = 48 KiB in flight, no barrier inside the loop).  A workgroup is one
//   wave (kWaves; with more, the waves take turns over the tiles and merge their states in
//   LDS at the end), so two workgroups share a compute unit (72 KiB of LDS each) and one's
//   start-up latency overlaps the other's stream: 3.5% faster than two waves sharing one
//   workgroup's 144 KiB.  The vector-memory counter caps a wave at 63 loads in flight, so a
//   deeper ring would need more waves, and the LDS rings cap those.
// * A workgroup covers 32 packed query rows (row r: head kv_h * group + r / Sq, query r % Sq)
//   of one (sequence, K/V head).  S^T = K Q^T and O^T += V^T P^T run on the same
//   v_mfma_f32_32x32x16 operand layouts as fmha_fwd (K and V rows XOR-swizzled in LDS, V^T
//   from ds_read_b64_tr_b16); rows past the group are zero and their output is dropped.
// * Paged caches (fmha_fwd_splitkv_paged): each 32-key tile lies in one page; the wave looks the
//   page up in the block table and bounds its descriptors to the page's rows in the sequence.
// * e4m3 caches under 16-bit queries: tiles land in LDS as bytes (fmha_fwd's fp8 row swizzle) and
//   widen exactly to the 16-bit MFMA type as the operands are read (v_cvt_scalef32_pk_*_fp8 with
//   scale 1; V^T through ds_read_b64_tr_b8, with P regrouped to its 8-consecutive-key order).
//   The 8 KiB tiles make a 40 KiB workgroup, so four share a compute unit and the split target
//   doubles: 1.55x faster than keeping two per unit, which left the SIMDs waiting.
// * Masks, varlen and GQA follow fmha_fwd: per-row last visible key, buffer descriptors
//   bounded to the sequence (rows past either end read 0), and the causal alignment offset
//   Sk_b - Sq_b for causal-qend.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include <type_traits>

#include "fmha.h"
#include "fmha_device.h"

namespace fmha {
namespace skv {

// lds_load16 with the non-temporal hint, for the K/V tiles: every cached K/V byte is read by
// one workgroup once, so nothing is gained by keeping it in the caches (measured on the decode
// workload: 18% faster over a contiguous cache; over a paged cache, together with the page
// numbers read ahead, see the kernel).  The forward kernel, whose workgroups share K/V tiles
// through L2, is 6% slower with the hint and keeps the plain load.
__device__ inline void lds_load16_stream(i32x4 rsrc, uint32_t voff, uint32_t lds_addr) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen nt lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(lds_addr));
}

constexpr int kWaves = 1;       // waves per workgroup, each streaming its own K/V tiles
constexpr int kThreads = 64 * kWaves;
constexpr int kTN = 32;         // keys per tile: one 32-key block of the MFMA
constexpr int kStages = 4;      // tiles in a wave's LDS ring (three in flight) for 16-bit K/V
constexpr int kStages8 = 4;     // the same for e4m3 K/V (8 KiB tiles: a 40 KiB workgroup, four per CU)

// s_waitcnt for "at most `ahead` tiles of NLD loads each still in flight" (ahead capped at T)
template <int NLD, int T>
__device__ inline void wait_tiles(int ahead) {
  if constexpr (T == 0) {
    wait_vmcnt<0>();
  } else {
    if (ahead >= T)
      wait_vmcnt<T * NLD>();
    else
      wait_tiles<NLD, T - 1>(ahead);
  }
}
constexpr int kRows = 32;       // packed query rows per workgroup (the MFMA N dimension)
constexpr int kMinChunk = 256;  // fewest keys per split
constexpr int kTargetWgs = 512; // split until about this many workgroups (two per compute unit)
constexpr int kTargetWgs8 = 1024;  // the same for e4m3 K/V (four per compute unit)

struct Params {
  const void* q;
  const void* k;
  const void* v;
  float* o_part;    // workspace: [n_splits][rows][D], each split's O normalised by its own sum
  float* lse_part;  // workspace: [n_splits][rows], natural log (-inf: the split saw no key)
  const int32_t* cu_q;  // null for dense batches
  const int32_t* cu_k;
  const int32_t* block_table;  // paged cache: [B][bt_stride] physical page of each logical page; null: contiguous
  const int32_t* seqlens_k;    // paged cache: keys of each sequence
  int32_t bt_stride, page_shift, num_pages;
  int32_t Sq, H, H_kv, group;  // Sq: query rows per sequence (packed: maximum)
  int32_t Sk;                  // dense: keys per sequence; paged: the most keys of any sequence
  int32_t M;                   // packed rows per K/V head: group * Sq
  int32_t mblks;               // ceil(M / kRows)
  int32_t n_splits, chunk;     // splits per (sequence, K/V head) and keys per split
  int32_t rows;                // rows of the partial arrays: query rows * H
  int32_t causal, qend;
  float scale_log2;            // scale * log2(e)
};

struct MergeParams {
  const float* o_part;
  const float* lse_part;
  void* o;
  float* lse;
  int32_t rows, n_splits, H, Sq, total_q;  // total_q > 0: packed LSE layout [H, total_q]
  float o_scale;
};

// split kernel: grid = B * H_kv * mblks * n_splits workgroups of kThreads
// KV8: K and V are e4m3 (a quantised cache); they are widened to the 16-bit type of Q exactly
// (every e4m3 value is a bf16 and an fp16 value) as the MFMA operands are read from LDS.
// Q8 (with KV8): Q is e4m3 as well, widened to bf16 (DT) the same way: e4m3 inputs throughout,
// computed on the 16-bit matrix cores with the probabilities in bf16; the merge writes e4m3.
template <int DT, int D, bool KV8, bool PAGED, bool Q8 = false>
__global__ __launch_bounds__(kThreads, 1) void split_kernel(const Params p) {
  static_assert(!Q8 || KV8, "e4m3 queries come with an e4m3 K/V");
  constexpr int E = Q8 ? 1 : 2;      // bytes per Q element
  constexpr int EK = KV8 ? 1 : 2;    // bytes per K/V element
  constexpr int RB = D * E;          // bytes per Q row
  constexpr int RBK = D * EK;        // bytes per K/V row
  constexpr int CPR = RB / 16;       // 16-byte chunks per Q row
  constexpr int CPRK = RBK / 16;     // 16-byte chunks per K/V row
  constexpr int TILE = kTN * RBK;    // bytes per K or V tile
  constexpr int TBLK = TILE / 1024;  // 1 KiB LDS-direct loads per K or V tile
  constexpr int NLD = 2 * TBLK;      // loads per tile
  constexpr int STAGE = 2 * TILE;    // K tile, then V tile
  constexpr int STG = KV8 ? kStages8 : kStages;  // ring depth
  constexpr int QB = kRows * RB;     // a wave's copy of the query rows
  constexpr int QBLK = QB / 1024;
  constexpr int KS = D / 16;         // MFMA k-steps over the head dimension
  constexpr int NDB = D / 32;        // 32-wide blocks of the head dimension in O
  static_assert(TILE % 1024 == 0 && QB % 1024 == 0, "whole 1 KiB loads");
  static_assert(!KV8 || D >= 32, "e4m3 K/V rows of at least 32 bytes (two 16-byte chunks)");
  static_assert((STG - 1) * NLD < 64, "vmcnt range");
  typedef Elem<DT> T;
  // eight e4m3 values (bytes 0..7 of w) as eight 16-bit values of the MFMA type, in order
  auto widen8 = [](i32x2 w) __attribute__((always_inline)) {
    i32x4 a;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if constexpr (DT == kBF16) {
        a[2 * h] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[h], 1.0f, false));
        a[2 * h + 1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[h], 1.0f, true));
      } else {
        a[2 * h] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[h], 1.0f, false));
        a[2 * h + 1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[h], 1.0f, true));
      }
    }
    return a;
  };

  // LDS: per wave a ring of STG {K, V} stages, then per wave a copy of the Q rows
  __shared__ __attribute__((aligned(1024))) char lds[kWaves * (STG * STAGE + QB)];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)lds;

  const int lane = threadIdx.x & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int l32 = lane & 31;
  const int h32 = lane >> 5;

  // ---- work unit: (sequence, K/V head, row block, split) ------------------------------
  int x = blockIdx.x;
  const int split = x % p.n_splits;
  x /= p.n_splits;
  const int mblk = x % p.mblks;
  x /= p.mblks;
  const int kvh = x % p.H_kv;
  const int b = x / p.H_kv;
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
  // (PAGED: the paged entry point, which always passes a block table.  The contiguous build
  // keeps the run-time test, whose code measured 4% faster than the one without it.)
  const bool paged = PAGED || p.block_table != nullptr;
  if (paged) {  // keys live in pages; no sequence has more than Sk (which the tables cover)
    k_row0 = 0;
    Sk_b = min(max(p.seqlens_k[b], 0), p.Sk);
  }
  const int off = p.qend ? Sk_b - Sq_b : 0;

  // this lane's packed row: head hq, query qi of the sequence; the keys it sees are [0, vis_end)
  const int r = mblk * kRows + l32;
  const int hq = kvh * p.group + r / p.Sq;
  const int qi = r % p.Sq;
  const bool row_ok = r < p.M && qi < Sq_b;
  const int vis_end = row_ok ? (p.causal ? min(Sk_b, qi + off + 1) : Sk_b) : 0;
  // keys of this split that some row sees, and the first key that some row does not see
  int wg_end = vis_end, wg_min = row_ok ? vis_end : 0x7fffffff;
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) {
    wg_end = max(wg_end, __shfl_xor(wg_end, o));
    wg_min = min(wg_min, __shfl_xor(wg_min, o));
  }
  const int k0 = split * p.chunk;
  const int k1 = min(min(Sk_b, k0 + p.chunk), __builtin_amdgcn_readfirstlane(wg_end));
  const int n_tiles = k1 > k0 ? (k1 - k0 + kTN - 1) / kTN : 0;
  const int n_w = n_tiles > wave_u ? (n_tiles - wave_u + kWaves - 1) / kWaves : 0;  // this wave's tiles
  // tiles from here on need the mask (some row does not see all their keys, or they run past k1)
  const int mask_from = min(__builtin_amdgcn_readfirstlane(wg_min), k1);
  const int lim_row = min(vis_end, k1) - 1 - 4 * h32;  // last key this lane keeps, less its key offset

  // ---- descriptors: bounded to the rows of this sequence; K/V start at the split's first key
  // (the host keeps a split's keys, with its last tiles, below 2^30 bytes), so a sequence's
  // K/V may be any length ------------------------------------------------------------
  const uint32_t qstride = (uint32_t)p.H * D * E;
  const uint32_t kstride = (uint32_t)p.H_kv * RBK;
  const size_t q_base = (size_t)q_row0 * p.H * D * E;
  const size_t k_base = ((size_t)k_row0 + (paged ? 0 : k0)) * kstride + (size_t)kvh * RBK;
  const uint32_t q_bytes = Sq_b > 0 ? (uint32_t)Sq_b * qstride : 0;
  const int k_rows = paged ? 0 : min(Sk_b - k0, p.chunk + kWaves * kTN * STG);  // rows from k_base
  const uint32_t k_bytes = k_rows > 0 ? (uint32_t)(k_rows - 1) * kstride + RBK : 0;
  const i32x4 rq = make_rsrc_words((const char*)p.q + q_base, q_bytes);
  const i32x4 rk = make_rsrc_words((const char*)p.k + k_base, k_bytes);
  const i32x4 rv = make_rsrc_words((const char*)p.v + k_base, k_bytes);

  const uint32_t ring = lds0 + (uint32_t)(wave_u * STG * STAGE);
  const uint32_t q_lds = lds0 + (uint32_t)(kWaves * STG * STAGE + wave_u * QB);

  // Paged cache: when the split's keys lie in at most 64 pages, lane j holds the table entry of
  // the split's j-th page, loaded once here, and each tile takes its page with a lane read
  // instead of a scalar load it would wait for.  The load is waited for once, unconditionally,
  // behind the Q rows below: the tile loads are invisible to the compiler, and a use it could
  // not prove waited for would make it drain every request in flight (vmcnt(0)) in the loop.
  const int lp_first = paged ? k0 >> p.page_shift : 0;
  const bool pre = PAGED && n_tiles > 0 && ((k1 - 1) >> p.page_shift) - lp_first < 64;
  int page_v = 0;
  if (pre && lp_first + lane <= ((k1 - 1) >> p.page_shift))
    page_v = p.block_table[(size_t)b * p.bt_stride + lp_first + lane];

  // ---- Q rows into this wave's LDS copy (swizzled like a K tile), then the B operand ----
#pragma unroll
  for (int i = 0; i < QBLK; ++i) {
    const int pos = 64 * i + lane;  // 16-byte chunk of the 32 x D block
    const int j = pos / CPR;        // packed row
    const int rj = mblk * kRows + j;
    const int hj = kvh * p.group + rj / p.Sq, qj = rj % p.Sq;
    // rows past the group, or past the sequence, fall outside the descriptor and read 0
    const int chunk = (pos % CPR) ^ (Q8 ? swz8<CPR>(j) : swz<CPR>(j));
    const uint32_t src = rj < p.M ? (uint32_t)qj * qstride + (uint32_t)hj * RB + chunk * 16
                                  : q_bytes;
    lds_load16(rq, src, q_lds + 1024 * i);
  }
  if constexpr (PAGED) asm volatile("" : "+v"(page_v));  // the one wait for page_v (and the Q rows)

  // per-lane LDS offsets: Q (and 16-bit K) row l32, chunk h32 of each k-step; V^T transpose
  // read (as fmha_fwd).  e4m3 K/V tiles use fmha_fwd's fp8 row swizzle: K row l32, 8 bytes at
  // chunk ks, half h32; V^T from ds_read_b64_tr_b8, which gives each lane column l32 of the
  // 8 consecutive rows 8 h32 + 0..7 of a 16-row chunk.
  auto swk = [](int j) __attribute__((always_inline)) { return KV8 ? swz8<CPRK>(j) : swz<CPRK>(j); };
  const int q_lane = l32 * RB + ((h32 ^ swz<CPR>(l32)) * 16);
  const int k_lane = KV8 ? l32 * RBK + (swk(l32) * 16) + 8 * h32 : q_lane;
  const int g16 = (lane >> 4) & 1;
  const int s16 = lane & 15;
  const int v_row0 = KV8 ? 8 * h32 + (s16 >> 1) : 4 * h32 + (s16 >> 2);
  const int v_part = KV8 ? g16 : 2 * g16 + ((s16 & 3) >> 1);
  const int v_lane0 = TILE + v_row0 * RBK + ((v_part ^ swk(v_row0)) * 16) + 8 * (s16 & 1);
  const int v_lane1 = TILE + (v_row0 + 8) * RBK + ((v_part ^ swk(v_row0 + 8)) * 16) + 8 * (s16 & 1);

  // loads of this wave's tile n (keys k0 + (wave + n kWaves) kTN ..) into stage n % STG
  uint32_t ld_off[TBLK];
#pragma unroll
  for (int i = 0; i < TBLK; ++i) {
    const int pos = 64 * i + lane;
    const int j = pos / CPRK;
    ld_off[i] = (uint32_t)j * kstride + (((pos % CPRK) ^ swk(j)) * 16);
  }
  // Paged cache: a tile (32 keys, page sizes are powers of two >= 32) lies inside one page; its
  // descriptors start at the page's row 0 of this K/V head and end after the page's last row
  // inside the sequence, so rows past the end read 0 as in the contiguous layout.  A table
  // entry outside [0, num_pages) gets an empty descriptor: its keys read as 0.
  auto load_tile = [&](int n) __attribute__((always_inline)) {
    const int kt = k0 + (wave_u + n * kWaves) * kTN;  // first key of the tile
    const uint32_t st = ring + (uint32_t)((n % STG) * STAGE);
    i32x4 tk = rk, tv = rv;
    uint32_t key0 = (uint32_t)(kt - k0) * kstride;  // (contiguous: from the split's first key)
    if (paged) {
      const int ps = 1 << p.page_shift;
      const int lp = kt >> p.page_shift;
      // (longer splits: a scalar load through the constant address space, waited on lgkmcnt,
      // which the tile loads in flight do not count toward)
      const int phys = pre ? __builtin_amdgcn_readlane(page_v, lp - lp_first)
                           : ((const __attribute__((address_space(4))) int32_t*)p.block_table)[(size_t)b * p.bt_stride + lp];
      const bool ok = (unsigned)phys < (unsigned)p.num_pages;
      const int valid = min(ps, Sk_b - (lp << p.page_shift));  // >= 1: the tile starts inside the sequence
      const size_t pb = ok ? ((size_t)phys * ps * p.H_kv + kvh) * RBK : 0;
      const uint32_t bytes = ok ? (uint32_t)(valid - 1) * kstride + RBK : 0;
      tk = make_rsrc_words((const char*)p.k + pb, bytes);
      tv = make_rsrc_words((const char*)p.v + pb, bytes);
      key0 = (uint32_t)(kt & (ps - 1)) * kstride;
    }
    if (PAGED || KV8 || !paged) {
#pragma unroll
      for (int i = 0; i < TBLK; ++i) lds_load16_stream(tk, key0 + ld_off[i], st + 1024 * i);
#pragma unroll
      for (int i = 0; i < TBLK; ++i) lds_load16_stream(tv, key0 + ld_off[i], st + TILE + 1024 * i);
    } else {  // (not reached: kept for the code shape of the contiguous build, above)
#pragma unroll
      for (int i = 0; i < TBLK; ++i) lds_load16(tk, key0 + ld_off[i], st + 1024 * i);
#pragma unroll
      for (int i = 0; i < TBLK; ++i) lds_load16(tv, key0 + ld_off[i], st + TILE + 1024 * i);
    }
  };
#pragma unroll
  for (int n = 0; n < STG - 1; ++n)
    if (n < n_w) load_tile(n);

  // Q landed (it is older than every tile load): read the B operand, dims 16 ks + 8 h32 ..
  wait_tiles<NLD, STG - 1>(n_w);
  i32x4 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if constexpr (Q8)  // e4m3 rows are swizzled and read like an e4m3 K tile, then widened
      qf[ks] = widen8(*(const lds_i32x2*)(uintptr_t)((q_lds + l32 * RB + swz8<CPR>(l32) * 16 + 8 * h32) ^ (16 * ks)));
    else
      qf[ks] = *(const lds_i32x4*)(uintptr_t)((q_lds + q_lane) ^ (32 * ks));
  }

  f32x16 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
  float m_run = -__builtin_inff();  // running max of scale*log2(e)*s for row l32
  float l_run = 0.0f;               // this lane's part of the row sum
  const float sl2 = p.scale_log2;

  for (int n = 0; n < n_w; ++n) {
    // tile n must have landed; the tiles requested after it may still be in flight
    wait_tiles<NLD, STG - 2>(n_w - 1 - n);
    const uint32_t st = ring + (uint32_t)((n % STG) * STAGE);
    const int kb = k0 + (wave_u + n * kWaves) * kTN;  // first key of the tile

    // S^T = K Q^T: score r of this lane is key kb + 4 h32 + 8 (r / 4) + r % 4, row l32
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      i32x4 a;
      if constexpr (KV8)
        a = widen8(*(const lds_i32x2*)(uintptr_t)((st + k_lane) ^ (16 * ks)));
      else
        a = *(const lds_i32x4*)(uintptr_t)((st + k_lane) ^ (32 * ks));
      s = T::mma(a, qf[ks], s);
    }
    if (kb + kTN > mask_from) {
      const int lim = lim_row - kb;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = 8 * (e >> 2) + (e & 3) <= lim ? s[e] : -__builtin_inff();
    }
    float mx = s[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = __builtin_fmaxf(mx, s[e]);
    mx = wave_row_max(mx);
    const float m_cand = mx * sl2;
    if (__any(m_cand > m_run + kRescaleThreshold)) {
      const float m_new = __builtin_fmaxf(m_run, m_cand);
      const float alpha = m_new == -__builtin_inff() ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc_o[db] *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == -__builtin_inff() ? 0.0f : m_run;
    uint32_t pk[8];
    float l2 = 0.0f;
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      float e4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) e4[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * qd + u], sl2, -m_use));
      pk[2 * qd] = T::pack(e4[0], e4[1]);
      pk[2 * qd + 1] = T::pack(e4[2], e4[3]);
      // the row sum takes the rounded probabilities the matrix cores multiply
      l_run += T::lo(pk[2 * qd]) + T::hi(pk[2 * qd]);
      l2 += T::lo(pk[2 * qd + 1]) + T::hi(pk[2 * qd + 1]);
    }
    l_run += l2;
    if constexpr (KV8) {
      // regroup to the order of the transposed e4m3 V read, 8 consecutive keys per lane and
      // 16-key chunk: lane h32 = 0 trades its keys 8..11 for keys 4..7 of lane l + 32
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int a = 4 * (i >> 1) + (i & 1);
        auto r = __builtin_amdgcn_permlane32_swap(pk[a], pk[a + 2], false, false);
        pk[a] = r[0];
        pk[a + 2] = r[1];
      }
    }

    // O^T += V^T P^T: 16-key chunk c, d-block db
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const i32x4 bp = {(int)pk[4 * c], (int)pk[4 * c + 1], (int)pk[4 * c + 2], (int)pk[4 * c + 3]};
      const uint32_t rows = (uint32_t)(16 * c * RBK);
      if constexpr (KV8) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const i32x2 t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(uintptr_t)(((st + v_lane0) ^ (32 * db)) + rows));
          acc_o[db] = T::mma(widen8(t), bp, acc_o[db]);
        }
        continue;
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const i16x4 v0 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(((st + v_lane0) ^ (64 * db)) + rows));
        const i16x4 v1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(((st + v_lane1) ^ (64 * db)) + rows));
        const i32x4 a = {__builtin_bit_cast(int, __builtin_shufflevector(v0, v0, 0, 1)),
                         __builtin_bit_cast(int, __builtin_shufflevector(v0, v0, 2, 3)),
                         __builtin_bit_cast(int, __builtin_shufflevector(v1, v1, 0, 1)),
                         __builtin_bit_cast(int, __builtin_shufflevector(v1, v1, 2, 3))};
        acc_o[db] = T::mma(a, bp, acc_o[db]);
      }
    }
    // stage (n - 1) % STG was read in the previous iteration: refill it with tile n + STG - 1
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (n + STG - 1 < n_w) load_tile(n + STG - 1);
  }

  // ---- merge the waves' states in LDS (the rings are free now), then write the partial --
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  const float l_tot = wave_row_sum(l_run);
  float m_all = m_run, l_all = l_tot;
  f32x16 o_all[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o_all[db] = acc_o[db];
  if constexpr (kWaves > 1) {
    __syncthreads();
    float* xm = (float*)lds;                  // [kWaves][64] running maxima
    float* xl = xm + kWaves * 64;             // [kWaves][64] row sums
    float* xo = xl + kWaves * 64;             // [kWaves][NDB * 16][64] accumulators, lane-major
    xm[wave_u * 64 + lane] = m_run;
    xl[wave_u * 64 + lane] = l_tot;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) xo[(wave_u * NDB * 16 + db * 16 + e) * 64 + lane] = acc_o[db][e];
    __syncthreads();
    if (wave_u != 0) return;
    m_all = xm[lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m_all = __builtin_fmaxf(m_all, xm[w * 64 + lane]);
    l_all = 0.0f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) o_all[db] = f32x16{};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = xm[w * 64 + lane];
      const float a = mw == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(mw - m_all);
      l_all += a * xl[w * 64 + lane];
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o_all[db][e] += a * xo[(w * NDB * 16 + db * 16 + e) * 64 + lane];
    }
  }
  if (!row_ok) return;
  const size_t row = (size_t)(q_row0 + qi) * p.H + hq;
  const size_t part = (size_t)split * p.rows + row;
  const float inv = l_all > 0.0f ? 1.0f / l_all : 0.0f;
  float* op = p.o_part + part * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {  // dims 32 db + 8 g + 4 h32 + 0..3
      const float4 w = {o_all[db][4 * g] * inv, o_all[db][4 * g + 1] * inv, o_all[db][4 * g + 2] * inv,
                        o_all[db][4 * g + 3] * inv};
      *(float4*)(op + 32 * db + 8 * g + 4 * h32) = w;
    }
  if (h32 == 0)
    p.lse_part[part] = l_all > 0.0f ? (m_all + __builtin_amdgcn_logf(l_all)) * 0.69314718055994531f : -__builtin_inff();
}

constexpr int kMergeChunk = 8;  // splits merged per round of loads

// merge kernel: D / 4 threads per row, each 4 consecutive dims.  OUT8: e4m3 output, saturated
// to the largest finite value and rounded to nearest even (as fmha_fwd's fp8 output).
template <int DT, int D, bool OUT8 = false>
__global__ __launch_bounds__(256) void merge_kernel(const MergeParams p) {
  constexpr int TPR = D / 4;
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int row = t / TPR;
  const int part = t % TPR;
  if (row >= p.rows) return;
  // Splits in chunks of kMergeChunk, each chunk's LSEs and partial rows requested together (a
  // loop of dependent loads, one split at a time, took several memory round trips per split);
  // across chunks the running sum is rescaled to the new maximum.  With one chunk this is
  // exactly the two-pass merge: the maximum first, then the weighted sum in split order.
  float mx = -__builtin_inff();
  float wsum = 0.0f;
  float4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < p.n_splits; s0 += kMergeChunk) {
    float ls[kMergeChunk];
    float4 os[kMergeChunk];
#pragma unroll
    for (int j = 0; j < kMergeChunk; ++j)
      ls[j] = s0 + j < p.n_splits ? p.lse_part[(size_t)(s0 + j) * p.rows + row] : -__builtin_inff();
#pragma unroll
    for (int j = 0; j < kMergeChunk; ++j)
      if (s0 + j < p.n_splits) os[j] = *(const float4*)(p.o_part + ((size_t)(s0 + j) * p.rows + row) * D + 4 * part);
    float cm = mx;
#pragma unroll
    for (int j = 0; j < kMergeChunk; ++j) cm = __builtin_fmaxf(cm, ls[j]);
    if (cm == -__builtin_inff()) continue;  // no split so far saw a key of this row
    if (cm != mx) {  // rescale what came before to the new maximum
      const float r = mx == -__builtin_inff() ? 0.0f : __expf(mx - cm);
      wsum *= r;
      acc.x *= r;
      acc.y *= r;
      acc.z *= r;
      acc.w *= r;
      mx = cm;
    }
#pragma unroll
    for (int j = 0; j < kMergeChunk; ++j) {
      if (ls[j] == -__builtin_inff()) continue;  // a split that saw no key of this row (or none)
      const float w = __expf(ls[j] - mx);
      wsum += w;
      acc.x += w * os[j].x;
      acc.y += w * os[j].y;
      acc.z += w * os[j].z;
      acc.w += w * os[j].w;
    }
  }
  const float f = wsum > 0.0f ? p.o_scale / wsum : 0.0f;
  if constexpr (OUT8) {
    auto sat = [](float x) { return __builtin_fminf(__builtin_fmaxf(x, -448.0f), 448.0f); };
    *(uint32_t*)((char*)p.o + (size_t)row * D + 4 * part) =
        pack_f8x4(sat(acc.x * f), sat(acc.y * f), sat(acc.z * f), sat(acc.w * f));
  } else {
    typedef Elem<DT> T;
    const uint32_t lo = T::pack(acc.x * f, acc.y * f), hi = T::pack(acc.z * f, acc.w * f);
    *(i32x2*)((char*)p.o + ((size_t)row * D + 4 * part) * 2) = i32x2{(int)lo, (int)hi};
  }
  if (p.lse && part == 0) {
    const int q = row / p.H, h = row - q * p.H;  // row = (query row) * H + head
    const size_t idx = p.total_q > 0 ? (size_t)h * p.total_q + q : ((size_t)(q / p.Sq) * p.H + h) * p.Sq + q % p.Sq;
    p.lse[idx] = wsum > 0.0f ? mx + __logf(wsum) : -__builtin_inff();
  }
}

// Splits per (sequence, K/V head) and keys per split: split until about `target` workgroups,
// but never below kMinChunk keys per split, and never above max_chunk keys (which keeps a
// split's byte offsets within 31 bits); chunks are whole wave-tile rounds.
inline void plan(int64_t units, int64_t Sk, int64_t target, int64_t max_chunk, int32_t* n_splits, int32_t* chunk) {
  int64_t n = units > 0 ? (target + units - 1) / units : 1;
  const int64_t n_max = Sk > kMinChunk ? (Sk + kMinChunk - 1) / kMinChunk : 1;
  n = n < 1 ? 1 : n > n_max ? n_max : n;
  // and at least enough splits that none exceeds max_chunk keys
  const int64_t n_min = Sk > max_chunk ? (Sk + max_chunk - 1) / max_chunk : 1;
  n = n < n_min ? n_min : n;
  constexpr int64_t round = kWaves * kTN;
  int64_t c = Sk > 0 ? (Sk + n - 1) / n : round;
  c = (c + round - 1) / round * round;
  *chunk = (int32_t)c;
  *n_splits = (int32_t)(Sk > 0 ? (Sk + c - 1) / c : 1);
}

template <int DT, int D, bool KV8 = false, bool PAGED = false, bool Q8 = false>
hipError_t launch(const Params& p, const MergeParams& mp, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((split_kernel<DT, D, KV8, PAGED, Q8>), dim3(grid), dim3(kThreads), 0, stream, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t threads = (int64_t)mp.rows * (D / 4);
  hipLaunchKernelGGL((merge_kernel<DT, D, Q8>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, mp);
  return hipGetLastError();
}


// ------------------------------------------------------------------------------------------
// Cache append: the new tokens' K and V rows into their pages (the generation kernel's default
// mode in the CUTLASS walk-through, as opposed to its --cache-only reads).  One workgroup per
// new row (sequence b, token i), 16 bytes per thread and step; new row i of sequence b is key
// seqlens_k[b] - S_new + i.  A row whose key lies before 0 or past the block table, or whose
// page number is outside [0, num_pages), is not written, so no table entry can send a store
// outside the cache.
// ------------------------------------------------------------------------------------------
struct AppendParams {
  char* k_cache;
  char* v_cache;
  const char* k_new;  // [B, S_new, H_kv, D]
  const char* v_new;
  const int32_t* block_table;
  const int32_t* seqlens_k;
  int32_t S_new, max_pages, page_size, num_pages;
  uint32_t row_bytes;  // H_kv * D * element size, a multiple of 16
};

constexpr int kAppendThreads = 256;

__global__ __launch_bounds__(kAppendThreads) void append_kernel(const AppendParams p) {
  const int b = blockIdx.x / p.S_new;
  const int i = blockIdx.x - b * p.S_new;
  const int64_t pos = (int64_t)p.seqlens_k[b] - p.S_new + i;
  if (pos < 0 || pos >= (int64_t)p.max_pages * p.page_size) return;
  const int page = p.block_table[(size_t)b * p.max_pages + (size_t)(pos / p.page_size)];
  if (page < 0 || page >= p.num_pages) return;
  const size_t dst = ((size_t)page * p.page_size + (size_t)(pos % p.page_size)) * p.row_bytes;
  const size_t src = (size_t)blockIdx.x * p.row_bytes;
  for (uint32_t off = 16u * threadIdx.x; off < p.row_bytes; off += 16u * kAppendThreads) {
    *(i32x4*)(p.k_cache + dst + off) = *(const i32x4*)(p.k_new + src + off);
    *(i32x4*)(p.v_cache + dst + off) = *(const i32x4*)(p.v_new + src + off);
  }
}

}  // namespace skv
}  // namespace fmha

// --------------------------------------------------------------------------------------
// C ABI
// --------------------------------------------------------------------------------------
// Scratch of fmha_fwd_splitkv_noalloc (see scratch_address below): 32 MiB per device.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

// The shape checks fmha_fwd makes, and the split plan.  Returns FMHA_OK with the plan filled.
fmha_status splitkv_plan(const void* q, const void* k, const void* v, const void* o, const float* lse, int32_t B,
                         int32_t Sq, int32_t Sk, int32_t H, int32_t H_kv, int32_t D, fmha_mask mask, fmha_dtype dtype,
                         const fmha_varlen* varlen, fmha::skv::Params* p, int64_t* grid, size_t* ws_bytes,
                         bool paged = false, bool kv8 = false) {
  using namespace fmha::skv;
  const bool packed = varlen != nullptr;
  if (B < 0 || Sq < 0 || Sk < 0 || H < 0 || H_kv < 0) return FMHA_ERR_INVALID_SHAPE;
  if (H > 0 && (H_kv < 1 || H % H_kv != 0)) return FMHA_ERR_INVALID_SHAPE;
  if (D != 32 && D != 64 && D != 128) return FMHA_ERR_INVALID_SHAPE;
  if (packed && (varlen->total_length_q < 0 || varlen->total_length_k < 0)) return FMHA_ERR_INVALID_SHAPE;
  if ((int)dtype < 0 || (int)dtype > 2) return FMHA_ERR_UNSUPPORTED;
  if ((int)mask < 0 || (int)mask > 3) return FMHA_ERR_UNSUPPORTED;
  // e4m3 queries (with an e4m3 K/V) run the e4m3-cache kernels
  const bool q8 = dtype == FMHA_DTYPE_F8E4M3;
  const bool k8 = kv8 || q8;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return FMHA_ERR_MISALIGNED;
  if ((uintptr_t)lse & 3) return FMHA_ERR_MISALIGNED;
  const int64_t rows_q = packed ? varlen->total_length_q : Sq;
  const int64_t lim = (int64_t)1 << 31;
  // Q byte offsets of one sequence fit 31 bits.  K/V descriptors start at each split's first key
  // and splits are capped at 2^30 bytes of K (a paged cache addresses each page on its own).
  const int64_t qe = q8 ? 1 : 2, ke = k8 ? 1 : 2;
  if (rows_q * H * D * qe >= lim) return FMHA_ERR_UNSUPPORTED;
  const int64_t k_row_bytes = (int64_t)H_kv * D * ke;
  const int64_t max_chunk = k_row_bytes > 0 ? ((int64_t)1 << 30) / k_row_bytes : ((int64_t)1 << 30);
  if (max_chunk < kMinChunk) return FMHA_ERR_UNSUPPORTED;
  const int64_t q_rows = packed ? (int64_t)varlen->total_length_q : (int64_t)B * Sq;
  const int64_t group = H > 0 ? H / H_kv : 1;
  const int64_t M = group * Sq;
  const int64_t mblks = (M + kRows - 1) / kRows;
  // The workspace is sized for the larger split target, so one size serves both cache types.
  int32_t n_splits = 1, chunk = kWaves * kTN, ws_splits = 1, ws_chunk = kWaves * kTN;
  plan((int64_t)B * H_kv * mblks, Sk, k8 ? kTargetWgs8 : kTargetWgs, max_chunk, &n_splits, &chunk);
  plan((int64_t)B * H_kv * mblks, Sk, kTargetWgs8, max_chunk, &ws_splits, &ws_chunk);
  const int64_t rows = q_rows * H;
  if (rows >= lim || (int64_t)ws_splits * rows * D >= lim * 2) return FMHA_ERR_UNSUPPORTED;
  *grid = (int64_t)B * H_kv * mblks * n_splits;
  if (*grid >= lim) return FMHA_ERR_UNSUPPORTED;
  *ws_bytes = (size_t)ws_splits * (size_t)rows * (size_t)(D + 1) * sizeof(float);
  p->Sq = Sq;
  p->Sk = Sk;
  p->H = H;
  p->H_kv = H_kv;
  p->group = (int32_t)group;
  p->M = (int32_t)M;
  p->mblks = (int32_t)mblks;
  p->n_splits = n_splits;
  p->chunk = chunk;
  p->rows = (int32_t)rows;
  p->causal = mask == FMHA_MASK_CAUSAL_QBEGIN || mask == FMHA_MASK_CAUSAL_QEND;
  p->qend = mask == FMHA_MASK_CAUSAL_QEND;
  return FMHA_OK;
}

// ------------------------------------------------------------------------------------
// scratch of the allocation-free entry point
// ------------------------------------------------------------------------------------
// The split partials of fmha_fwd_splitkv_noalloc live in this library-owned array: one copy on
// every device the library runs on, held until the process ends.  In host code `scratch` is only
// a stand-in for the symbol; its device address on the current device comes from
// hipGetSymbolAddress, resolved on the first call on each device and kept per device.
// Device address of `scratch` on the current device, or nullptr if the runtime cannot give it.
void* scratch_address() {
  static std::atomic<uintptr_t> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
  if (dev < 64) {
    const uintptr_t a = cache[dev].load(std::memory_order_acquire);
    if (a) return (void*)a;
  }
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
  if (dev < 64) cache[dev].store((uintptr_t)ptr, std::memory_order_release);
  return ptr;
}

// fmha_fwd_splitkv, with the workspace either the caller's or (library_scratch) this library's
// static array on the current device.
fmha_status splitkv_run(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B, int32_t Sq,
                        int32_t Sk, int32_t H, int32_t H_kv, int32_t D, float scale, fmha_mask mask, fmha_dtype dtype,
                        float o_scale, const fmha_varlen* varlen, void* workspace, size_t workspace_bytes,
                        bool library_scratch, hipStream_t stream) {
  using namespace fmha::skv;
  const bool packed = varlen != nullptr;
  const bool no_keys = packed ? varlen->total_length_k == 0 : Sk == 0;  // k and v may then be NULL
  if (!q || !o || (!no_keys && (!k || !v))) return FMHA_ERR_NULL_POINTER;
  if (packed && (!varlen->cu_seqlens_q != !varlen->cu_seqlens_k)) return FMHA_ERR_NULL_POINTER;
  if (packed && !varlen->cu_seqlens_q) return FMHA_ERR_NULL_POINTER;
  Params p;
  int64_t grid = 0;
  size_t need = 0;
  const fmha_status st = splitkv_plan(q, k, v, o, lse, B, Sq, Sk, H, H_kv, D, mask, dtype, varlen, &p, &grid, &need);
  if (st != FMHA_OK) return st;
  if (!(scale > 0.0f) || !isfinite(scale) || !isfinite(o_scale)) return FMHA_ERR_INVALID_ARGUMENT;
  if (B == 0 || H == 0 || Sq == 0 || (packed && varlen->total_length_q == 0)) return FMHA_OK;
  if (library_scratch) {
    if (need > kScratchBytes) return FMHA_ERR_SCRATCH_TOO_SMALL;
    workspace = scratch_address();
    if (!workspace) return FMHA_ERR_HIP;
    workspace_bytes = kScratchBytes;
  }
  if (!workspace) return FMHA_ERR_NULL_POINTER;
  if ((uintptr_t)workspace & 15) return FMHA_ERR_MISALIGNED;
  if (workspace_bytes < need) return FMHA_ERR_INVALID_ARGUMENT;

  p.q = q;
  p.k = k;
  p.v = v;
  p.o_part = (float*)workspace;
  p.lse_part = p.o_part + (size_t)p.n_splits * p.rows * D;
  p.cu_q = packed ? varlen->cu_seqlens_q : nullptr;
  p.cu_k = packed ? varlen->cu_seqlens_k : nullptr;
  p.block_table = nullptr;
  p.seqlens_k = nullptr;
  p.bt_stride = p.page_shift = p.num_pages = 0;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  MergeParams mp;
  mp.o_part = p.o_part;
  mp.lse_part = p.lse_part;
  mp.o = o;
  mp.lse = lse;
  mp.rows = p.rows;
  mp.n_splits = p.n_splits;
  mp.H = H;
  mp.Sq = Sq;
  mp.total_q = packed ? varlen->total_length_q : 0;
  mp.o_scale = o_scale;

  hipError_t err = hipSuccess;
  if (dtype == FMHA_DTYPE_F8E4M3) {  // e4m3 Q, K, V widened to bf16 for the matrix cores
    if (D == 32) err = fmha::skv::launch<fmha::kBF16, 32, true, false, true>(p, mp, (int)grid, stream);
    if (D == 64) err = fmha::skv::launch<fmha::kBF16, 64, true, false, true>(p, mp, (int)grid, stream);
    if (D == 128) err = fmha::skv::launch<fmha::kBF16, 128, true, false, true>(p, mp, (int)grid, stream);
  } else if (dtype == FMHA_DTYPE_BF16) {
    if (D == 32) err = fmha::skv::launch<fmha::kBF16, 32>(p, mp, (int)grid, stream);
    if (D == 64) err = fmha::skv::launch<fmha::kBF16, 64>(p, mp, (int)grid, stream);
    if (D == 128) err = fmha::skv::launch<fmha::kBF16, 128>(p, mp, (int)grid, stream);
  } else {
    if (D == 32) err = fmha::skv::launch<fmha::kF16, 32>(p, mp, (int)grid, stream);
    if (D == 64) err = fmha::skv::launch<fmha::kF16, 64>(p, mp, (int)grid, stream);
    if (D == 128) err = fmha::skv::launch<fmha::kF16, 128>(p, mp, (int)grid, stream);
  }
  return err == hipSuccess ? FMHA_OK : FMHA_ERR_HIP;
}

}  // namespace

extern "C" {

size_t fmha_fwd_splitkv_workspace_size(int32_t B, int32_t Sq, int32_t Sk, int32_t H, int32_t H_kv, int32_t D,
                                       const fmha_varlen* varlen) {
  fmha::skv::Params p;
  int64_t grid = 0;
  size_t bytes = 0;
  // The workspace holds per-split partial rows of Q's shape, whatever the K/V bytes: planned as
  // for a paged cache, which skips the contiguous K/V offset bound (the entry points check it).
  const fmha_status st = splitkv_plan(nullptr, nullptr, nullptr, nullptr, nullptr, B, Sq, Sk, H, H_kv, D,
                                      FMHA_MASK_NONE, FMHA_DTYPE_BF16, varlen, &p, &grid, &bytes, true);
  return st == FMHA_OK ? bytes : 0;
}

fmha_status fmha_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B, int32_t Sq,
                             int32_t Sk, int32_t H, int32_t H_kv, int32_t D, float scale, fmha_mask mask,
                             fmha_dtype dtype, float o_scale, const fmha_varlen* varlen, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  return splitkv_run(q, k, v, o, lse, B, Sq, Sk, H, H_kv, D, scale, mask, dtype, o_scale, varlen, workspace,
                     workspace_bytes, false, stream);
}

fmha_status fmha_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B,
                                     int32_t Sq, int32_t Sk, int32_t H, int32_t H_kv, int32_t D, float scale,
                                     fmha_mask mask, fmha_dtype dtype, float o_scale, const fmha_varlen* varlen,
                                     hipStream_t stream) {
  return splitkv_run(q, k, v, o, lse, B, Sq, Sk, H, H_kv, D, scale, mask, dtype, o_scale, varlen, nullptr, 0, true,
                     stream);
}

fmha_status fmha_fwd_splitkv_paged(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                                   int32_t B, int32_t Sq, int32_t Sk, int32_t H, int32_t H_kv, int32_t D, float scale,
                                   fmha_mask mask, fmha_dtype dtype, float o_scale, const fmha_paged_kv* paged,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  using namespace fmha::skv;
  if (!paged) return FMHA_ERR_NULL_POINTER;
  const bool no_keys = Sk == 0;
  if (!q || !o || (!no_keys && (!k_cache || !v_cache || !paged->block_table || !paged->seqlens_k)))
    return FMHA_ERR_NULL_POINTER;
  Params p;
  int64_t grid = 0;
  size_t need = 0;
  const bool kv8 = paged->kv_dtype == FMHA_DTYPE_F8E4M3;
  const fmha_status st = splitkv_plan(q, k_cache, v_cache, o, lse, B, Sq, Sk, H, H_kv, D, mask, dtype, nullptr, &p,
                                      &grid, &need, true, kv8);
  if (st != FMHA_OK) return st;
  const int32_t ps = paged->page_size;
  if (ps < kTN || ps > (1 << 16) || (ps & (ps - 1))) return FMHA_ERR_INVALID_SHAPE;
  if (!kv8 && paged->kv_dtype != dtype) return FMHA_ERR_UNSUPPORTED;
  const bool q8 = dtype == FMHA_DTYPE_F8E4M3;     // (e4m3 queries need an e4m3 cache)
  if (paged->max_pages_per_seq < 0 || paged->num_pages < 0) return FMHA_ERR_INVALID_SHAPE;
  if (!no_keys && (paged->num_pages < 1 || (int64_t)paged->max_pages_per_seq * ps < Sk)) return FMHA_ERR_INVALID_SHAPE;
  if ((int64_t)ps * H_kv * D * 2 >= ((int64_t)1 << 31)) return FMHA_ERR_UNSUPPORTED;
  if (!(scale > 0.0f) || !isfinite(scale) || !isfinite(o_scale)) return FMHA_ERR_INVALID_ARGUMENT;
  if (B == 0 || H == 0 || Sq == 0) return FMHA_OK;
  if (!workspace) return FMHA_ERR_NULL_POINTER;
  if ((uintptr_t)workspace & 15) return FMHA_ERR_MISALIGNED;
  if (workspace_bytes < need) return FMHA_ERR_INVALID_ARGUMENT;

  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.o_part = (float*)workspace;
  p.lse_part = p.o_part + (size_t)p.n_splits * p.rows * D;
  p.cu_q = nullptr;
  p.cu_k = nullptr;
  p.block_table = no_keys ? nullptr : paged->block_table;
  p.seqlens_k = paged->seqlens_k;
  p.bt_stride = paged->max_pages_per_seq;
  p.page_shift = __builtin_ctz((unsigned)ps);
  p.num_pages = paged->num_pages;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  MergeParams mp;
  mp.o_part = p.o_part;
  mp.lse_part = p.lse_part;
  mp.o = o;
  mp.lse = lse;
  mp.rows = p.rows;
  mp.n_splits = p.n_splits;
  mp.H = H;
  mp.Sq = Sq;
  mp.total_q = 0;
  mp.o_scale = o_scale;

  hipError_t err = hipSuccess;
  if (no_keys) {
    // An empty cache: the block table and the lengths may be NULL, and no key is read.  The
    // contiguous kernels (no table) give every row O = 0 and LSE = -inf, whatever the cache type.
    if (q8) {
      if (D == 32) err = fmha::skv::launch<fmha::kBF16, 32, true, false, true>(p, mp, (int)grid, stream);
      if (D == 64) err = fmha::skv::launch<fmha::kBF16, 64, true, false, true>(p, mp, (int)grid, stream);
      if (D == 128) err = fmha::skv::launch<fmha::kBF16, 128, true, false, true>(p, mp, (int)grid, stream);
    } else if (dtype == FMHA_DTYPE_BF16) {
      if (D == 32) err = fmha::skv::launch<fmha::kBF16, 32>(p, mp, (int)grid, stream);
      if (D == 64) err = fmha::skv::launch<fmha::kBF16, 64>(p, mp, (int)grid, stream);
      if (D == 128) err = fmha::skv::launch<fmha::kBF16, 128>(p, mp, (int)grid, stream);
    } else {
      if (D == 32) err = fmha::skv::launch<fmha::kF16, 32>(p, mp, (int)grid, stream);
      if (D == 64) err = fmha::skv::launch<fmha::kF16, 64>(p, mp, (int)grid, stream);
      if (D == 128) err = fmha::skv::launch<fmha::kF16, 128>(p, mp, (int)grid, stream);
    }
  } else if (kv8) {
    if (q8) {
      if (D == 32) err = fmha::skv::launch<fmha::kBF16, 32, true, true, true>(p, mp, (int)grid, stream);
      if (D == 64) err = fmha::skv::launch<fmha::kBF16, 64, true, true, true>(p, mp, (int)grid, stream);
      if (D == 128) err = fmha::skv::launch<fmha::kBF16, 128, true, true, true>(p, mp, (int)grid, stream);
    } else if (dtype == FMHA_DTYPE_BF16) {
      if (D == 32) err = fmha::skv::launch<fmha::kBF16, 32, true, true>(p, mp, (int)grid, stream);
      if (D == 64) err = fmha::skv::launch<fmha::kBF16, 64, true, true>(p, mp, (int)grid, stream);
      if (D == 128) err = fmha::skv::launch<fmha::kBF16, 128, true, true>(p, mp, (int)grid, stream);
    } else {
      if (D == 32) err = fmha::skv::launch<fmha::kF16, 32, true, true>(p, mp, (int)grid, stream);
      if (D == 64) err = fmha::skv::launch<fmha::kF16, 64, true, true>(p, mp, (int)grid, stream);
      if (D == 128) err = fmha::skv::launch<fmha::kF16, 128, true, true>(p, mp, (int)grid, stream);
    }
  } else if (dtype == FMHA_DTYPE_BF16) {
    if (D == 32) err = fmha::skv::launch<fmha::kBF16, 32, false, true>(p, mp, (int)grid, stream);
    if (D == 64) err = fmha::skv::launch<fmha::kBF16, 64, false, true>(p, mp, (int)grid, stream);
    if (D == 128) err = fmha::skv::launch<fmha::kBF16, 128, false, true>(p, mp, (int)grid, stream);
  } else {
    if (D == 32) err = fmha::skv::launch<fmha::kF16, 32, false, true>(p, mp, (int)grid, stream);
    if (D == 64) err = fmha::skv::launch<fmha::kF16, 64, false, true>(p, mp, (int)grid, stream);
    if (D == 128) err = fmha::skv::launch<fmha::kF16, 128, false, true>(p, mp, (int)grid, stream);
  }
  return err == hipSuccess ? FMHA_OK : FMHA_ERR_HIP;
}

fmha_status fmha_paged_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new, int32_t B,
                                 int32_t S_new, int32_t H_kv, int32_t D, const fmha_paged_kv* paged,
                                 hipStream_t stream) {
  if (!paged) return FMHA_ERR_NULL_POINTER;
  if (B < 0 || S_new < 0 || H_kv < 1) return FMHA_ERR_INVALID_SHAPE;
  if (D != 32 && D != 64 && D != 128) return FMHA_ERR_INVALID_SHAPE;
  if ((int)paged->kv_dtype < 0 || (int)paged->kv_dtype > 2) return FMHA_ERR_UNSUPPORTED;
  const int32_t ps = paged->page_size;
  if (ps < 32 || ps > 65536 || (ps & (ps - 1)) != 0 || paged->max_pages_per_seq < 1 || paged->num_pages < 1)
    return FMHA_ERR_INVALID_SHAPE;
  if (B == 0 || S_new == 0) return FMHA_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !paged->block_table || !paged->seqlens_k)
    return FMHA_ERR_NULL_POINTER;
  if (((uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)k_new | (uintptr_t)v_new) & 15) return FMHA_ERR_MISALIGNED;
  const int64_t row_bytes = (int64_t)H_kv * D * (paged->kv_dtype == FMHA_DTYPE_F8E4M3 ? 1 : 2);
  if ((int64_t)B * S_new >= ((int64_t)1 << 31) || row_bytes >= ((int64_t)1 << 31)) return FMHA_ERR_UNSUPPORTED;
  fmha::skv::AppendParams p;
  p.k_cache = (char*)k_cache;
  p.v_cache = (char*)v_cache;
  p.k_new = (const char*)k_new;
  p.v_new = (const char*)v_new;
  p.block_table = paged->block_table;
  p.seqlens_k = paged->seqlens_k;
  p.S_new = S_new;
  p.max_pages = paged->max_pages_per_seq;
  p.page_size = ps;
  p.num_pages = paged->num_pages;
  p.row_bytes = (uint32_t)row_bytes;
  hipLaunchKernelGGL(fmha::skv::append_kernel, dim3((unsigned)((int64_t)B * S_new)), dim3(fmha::skv::kAppendThreads), 0,
                     stream, p);
  return hipGetLastError() == hipSuccess ? FMHA_OK : FMHA_ERR_HIP;
}

}  // extern "C"
