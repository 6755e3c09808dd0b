/*
 * fmha.h -- fused multi-head attention on AMD Instinct MI355X (gfx950): forward pass
 * (fmha_fwd, fmha_fwd_splitkv) and backward pass (fmha_bwd).
 *
 * C ABI of libfmha.so.  One call computes, for every sequence b, query head h and
 * query row i,
 *
 *     O[b, i, h, :] = o_scale * sum_j softmax_j(scale * Q[b, i, h, :] . K[b, j, h_kv, :] + mask) * V[b, j, h_kv, :]
 *
 * with h_kv = h / (H / H_kv), tile by tile with an online softmax, so the score and
 * probability matrices never reach device memory.  This is the method of the
 * wingedge777 article "[CUDA 优化实战] fmha sm120: 超越 torch.sdpa(flash-attention-2)"
 * (sections "1. flash attention" and "2. fmha 实现"), with the masks, packed
 * variable-length batches, GQA/MQA head sharing, LSE output and fp8 output scale of
 * the CUTLASS Blackwell FMHA example (trdm.cn walk-through "CUTLASS Blackwell FMHA
 * 示例完全解析", sections on the fusion point fmha_fusion.hpp, variable sequence
 * length, verification and GQA/MQA strides; CUTLASS examples/77_blackwell_fmha
 * README, "FMHA for Blackwell: Forward").
 *
 * Ownership: every pointer is device memory owned by the caller.  The library
 * allocates nothing and keeps no pointer after a call returns.  Its only global
 * state is a per-device cache of the compute-unit count (written once, atomically,
 * with the value the runtime reports; it sizes the grid), so calls from several
 * host threads are safe.  Work is enqueued on `stream` and runs asynchronously;
 * errors inside the kernel surface at the caller's next synchronisation.  The grid
 * is sized from the current device's (hipGetDevice) compute-unit count; results do
 * not depend on it.
 */
#ifndef FMHA_H_
#define FMHA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q, K, V and O (all four share it). */
typedef enum {
  FMHA_DTYPE_F16 = 0,    /* IEEE binary16 */
  FMHA_DTYPE_BF16 = 1,   /* bfloat16 */
  FMHA_DTYPE_F8E4M3 = 2  /* OCP fp8 E4M3FN (largest finite 448, no infinities) */
} fmha_dtype;

/* Masks of the CUTLASS fusion point (trdm.cn walk-through, section on fmha_fusion.hpp).
 * Every mask also hides the keys j >= Sk_b of the sequence.
 *   NONE, RESIDUAL     query i sees every key j < Sk_b (identical results; RESIDUAL is
 *                      kept for interface parity: partial last tiles are always masked)
 *   CAUSAL_QBEGIN      query i sees key j iff j <= i                (top-left aligned)
 *   CAUSAL_QEND        query i sees key j iff j <= i + (Sk_b - Sq_b) (bottom-right aligned)
 * A query row that sees no key gets O = 0 and LSE = -inf. */
typedef enum {
  FMHA_MASK_NONE = 0,
  FMHA_MASK_RESIDUAL = 1,
  FMHA_MASK_CAUSAL_QBEGIN = 2,
  FMHA_MASK_CAUSAL_QEND = 3
} fmha_mask;

typedef enum {
  FMHA_OK = 0,
  FMHA_ERR_NULL_POINTER = 1,     /* q, o, or (when there are keys) k or v is NULL, or only one
                                    cu_seqlens pointer is set */
  FMHA_ERR_INVALID_SHAPE = 2,    /* negative sizes, H % H_kv != 0, D not in {32, 64, 128}, totals < 0 */
  FMHA_ERR_UNSUPPORTED = 3,      /* dtype/mask enum out of range, or a problem too large for the
                                    kernels' 32-bit offsets.  fmha_fwd and fmha_bwd address each
                                    workgroup's rows and each streamed tile from descriptors placed
                                    there, so sequences may be of any length: fmha_fwd refuses only
                                    three K/V tiles (192 16-bit or 384 e4m3 rows) or 256 Q rows of
                                    2^31 bytes or more, and dense B * Sq or B * Sk of 2^31 rows or
                                    more; fmha_bwd refuses 256 query rows or 128 K/V rows of 2^31
                                    bytes or more, or a statistics workspace of 2^31 bytes or more.
                                    fmha_fwd_splitkv starts its K/V descriptors at each split and
                                    splits the keys so that none spans 2^30 bytes: it refuses only
                                    one sequence's Q of 2^31 bytes or more, or a K/V row (all K/V
                                    heads of one key) of more than 4 MiB. */
  FMHA_ERR_MISALIGNED = 4,       /* q, k, v or o not 16-byte aligned, or lse not 4-byte aligned */
  FMHA_ERR_INVALID_ARGUMENT = 5, /* scale not finite and > 0, or o_scale not finite */
  FMHA_ERR_HIP = 6,              /* the kernel launch failed (hipGetLastError), or the device address
                                    of the library's scratch array could not be obtained */
  FMHA_ERR_SCRATCH_TOO_SMALL = 7 /* fmha_fwd_splitkv_noalloc: the shape needs more workspace than
                                    the library's static scratch array holds (32 MiB) */
} fmha_status;

/* Packed variable-length batch, after CUTLASS's VariableLength {max_length,
 * cumulative_length, total_length} (trdm.cn walk-through, section on variable
 * sequence length).  Sequence b owns rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) of q
 * and o and rows [cu_seqlens_k[b], cu_seqlens_k[b+1]) of k and v.
 *   cu_seqlens_q, cu_seqlens_k  device int32 arrays of B + 1 entries, non-decreasing,
 *                               entry 0 is 0 and entry B is the total; each length must
 *                               not exceed the Sq / Sk passed to fmha_fwd (the maxima).
 *                               They are read on the device only and cannot be checked.
 *   total_length_q/k            number of packed rows (= cu_seqlens[B]); sizes of the LSE
 *                               rows and the bound used for 32-bit offsets.
 * The library reads and writes only rows inside [cu[b], cu[b+1]); padding the caller
 * keeps around the packed rows is never touched. */
typedef struct {
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  int32_t total_length_q;
  int32_t total_length_k;
} fmha_varlen;

/*
 * fmha_fwd -- enqueue one attention forward pass.
 *
 *   q      [B, Sq, H, D]     dense, contiguous   |  [total_length_q, H, D]     packed
 *   k, v   [B, Sk, H_kv, D]  dense, contiguous   |  [total_length_k, H_kv, D]  packed
 *          (may be NULL when there are no keys: Sk == 0, or total_length_k == 0)
 *   o      same shape as q, written (rows outside the sequences are left untouched)
 *   lse    NULL, or fp32 [B, H, Sq] (dense) / [H, total_length_q] (packed):
 *          natural-log log-sum-exp of scale * q.k over the visible keys (-inf if none)
 *   B      number of sequences (>= 0);  Sq, Sk: lengths (packed: the maximum lengths)
 *   H, H_kv  query heads and key/value heads, H % H_kv == 0 (H_kv == 1 is MQA)
 *   D      head dimension: 32, 64 or 128
 *   scale  softmax scale (finite, > 0), applied to q.k in fp32.  For fp8 inputs the
 *          caller folds the per-tensor dequantisation scales of q and k into it.
 *   mask   see fmha_mask
 *   dtype  element type of q, k, v and o
 *   o_scale  fp32 multiplier applied to the normalised output before the conversion to
 *          dtype (fp8 output scale; for fp8 inputs the caller folds v's scale in).
 *          fp8 outputs saturate to +-448; fp16/bf16 outputs round to nearest even.
 *   varlen NULL for dense batches, else the packed description above
 *   stream HIP stream the kernel is enqueued on (0 = the null stream)
 *
 * Validation happens on the host before anything is enqueued; on error nothing is
 * launched and no memory is touched.  Sizes that give no work (B, H, Sq or a total
 * of 0) return FMHA_OK without a launch.
 */
fmha_status fmha_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int32_t B, int32_t Sq, int32_t Sk, int32_t H, int32_t H_kv, int32_t D,
                     float scale, fmha_mask mask, fmha_dtype dtype, float o_scale,
                     const fmha_varlen* varlen, hipStream_t stream);

/*
 * fmha_fwd_splitkv -- the same attention forward pass as fmha_fwd (same arguments, masks,
 * layouts, LSE and results up to rounding), built for generation / decode: few query rows
 * per head (Sq small, e.g. 1 to 16 new tokens) against a long key range.  The keys of each
 * (sequence, K/V head) are cut into splits that run on different workgroups; each writes
 * its partial O (normalised by its own row sums, fp32) and partial LSE into `workspace`,
 * and a second kernel merges them as O = sum_s exp(LSE_s - LSE) O_s, LSE = log sum_s
 * exp(LSE_s) -- the split-KV reduction of the CUTLASS generation kernel (trdm.cn
 * walk-through "CUTLASS Blackwell FMHA 示例完全解析", sections on the generation kernel and
 * the reduction; examples/77_blackwell_fmha README, "FMHA for Blackwell: Generation").  The
 * query heads of a GQA group share one K/V stream (they are packed into the rows of one
 * matrix tile).  Correct for any Sq, but fmha_fwd is the faster choice once Sq * H / H_kv
 * reaches a few hundred rows.
 *
 *   workspace        device memory owned by the caller, 16-byte aligned, at least
 *                    fmha_fwd_splitkv_workspace_size(...) bytes for the same shape; its
 *                    contents on entry do not matter and are overwritten (calls that
 *                    overlap in time must not share it)
 *   workspace_bytes  its size
 *   dtype            FMHA_DTYPE_F16, FMHA_DTYPE_BF16, or FMHA_DTYPE_F8E4M3 (D 32, 64 or 128): e4m3 q,
 *                    k, v and o, the per-tensor dequantisation scales folded into scale and o_scale as
 *                    for fmha_fwd, the output saturated to +-448.  e4m3 values widen exactly to bf16,
 *                    so the fp8 call runs on the 16-bit matrix cores with its probabilities in bf16.
 * Errors as fmha_fwd, and: workspace NULL -> FMHA_ERR_NULL_POINTER, not 16-byte aligned
 * -> FMHA_ERR_MISALIGNED, smaller than needed -> FMHA_ERR_INVALID_ARGUMENT (checked only
 * when there is work).
 */
fmha_status fmha_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                             int32_t B, int32_t Sq, int32_t Sk, int32_t H, int32_t H_kv, int32_t D,
                             float scale, fmha_mask mask, fmha_dtype dtype, float o_scale,
                             const fmha_varlen* varlen, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * fmha_fwd_splitkv_noalloc -- fmha_fwd_splitkv (same arguments without the workspace, same
 * kernels, same split plan, bit-identical results) for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The split partials go to a static array that the library owns, 32 MiB on every device it runs
 * on, held until the process ends.  The call allocates nothing (no hipMalloc, no hipFree).
 *   Shapes whose fmha_fwd_splitkv_workspace_size(...) exceeds 32 MiB -> FMHA_ERR_SCRATCH_TOO_SMALL
 *   (nothing launched); other errors as fmha_fwd_splitkv.  The first call on a device looks up the
 *   array's device address there (FMHA_ERR_HIP if the runtime cannot give it).
 * All calls on one device share its array, and each call overwrites what the last one left there
 * before reading it (no part of it needs to start at zero).  Calls enqueued on one stream run one
 * after the other; calls that may overlap in time on one device (several streams, several host
 * threads) race on the array and must not be issued.
 */
fmha_status fmha_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                     int32_t B, int32_t Sq, int32_t Sk, int32_t H, int32_t H_kv, int32_t D,
                                     float scale, fmha_mask mask, fmha_dtype dtype, float o_scale,
                                     const fmha_varlen* varlen, hipStream_t stream);

/* Workspace bytes fmha_fwd_splitkv and fmha_fwd_splitkv_paged need for this shape (host
 * arithmetic only: no device call; the packed form reads only varlen->total_length_q).  The
 * size depends on the query rows, heads, D and the split plan, not on the bytes of K and V, so a
 * contiguous K/V too large for the kernel's 32-bit offsets still gets a size (fmha_fwd_splitkv
 * then returns FMHA_ERR_UNSUPPORTED).  Returns 0 for an invalid shape, or query rows or
 * partials too large for 32-bit offsets. */
size_t fmha_fwd_splitkv_workspace_size(int32_t B, int32_t Sq, int32_t Sk, int32_t H, int32_t H_kv, int32_t D,
                                       const fmha_varlen* varlen);

/*
 * fmha_bwd -- enqueue the backward pass of fmha_fwd (o_scale 1): the gradients dq, dk, dv of
 * the forward's output for an upstream gradient dout,
 *
 *     P = exp(scale * Q K^T + mask - LSE)            (recomputed from the forward's LSE)
 *     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - delta),  delta_i = sum_d O_id dO_id,
 *     dQ = scale * dS K,  dK = scale * dS^T Q,
 *
 * per (sequence, head), after the backward of the CUTLASS Blackwell FMHA example (trdm.cn
 * walk-through "CUTLASS Blackwell FMHA 示例完全解析", section "FMHA for Blackwell: Backward":
 * a row sum of O * dO, the main dQ/dK/dV pass, dQ converted to the output type; masks as that
 * section's backward mask, i.e. the forward masks).  Two kernels run on `stream`: dQ (which
 * also forms the row statistics), then dK/dV (after a widening pass for e4m3 inputs).  No atomics: results are bitwise repeatable.  With GQA/MQA
 * (H_kv < H), dk and dv of a K/V head are the sums over its group of query heads (the
 * CUTLASS backward does not support GQA; this is the gradient of the shared head).
 *
 *   q, k, v, o   the forward's inputs and output (o written by fmha_fwd with o_scale 1)
 *   dout         dO, same shape and type as o
 *   lse          the forward's fp32 LSE (natural log), layout as in fmha_fwd; required
 *   dq           same shape as q, written
 *   dk, dv       same shapes as k and v, written (keys that no query sees get 0)
 *   B, Sq, Sk, H, H_kv, D, scale, mask, varlen   as in fmha_fwd
 *   dtype        FMHA_DTYPE_F16 or FMHA_DTYPE_BF16: every tensor above except lse has this type.
 *                FMHA_DTYPE_F8E4M3 (the walk-through lists fp8 among the backward's types):
 *                q, k, v, o and dout are e4m3 and dq, dk, dv are written as bf16, since a
 *                3-bit mantissa without a scale (the pages give none for gradients) would flush
 *                most gradient values.  The e4m3 values are taken as they are: scale is the
 *                forward's (with q's and k's dequantisation scales folded in), o is fmha_fwd's
 *                e4m3 output with o_scale 1, and a caller with per-tensor scales s_q, s_k, s_v,
 *                s_do multiplies dq by s_do s_v / s_q, dk by s_do s_v / s_k and dv by s_do.  The
 *                inputs are widened exactly to bf16 in the workspace and run the bf16 kernels.
 *   workspace    device memory owned by the caller, 16-byte aligned, at least
 *                fmha_bwd_workspace_size(...) bytes for the same shape and dtype; contents on
 *                entry do not matter (calls that overlap in time must not share it).  It holds
 *                8 bytes of row statistics per query row and head, in blocks of 64 rows, and for
 *                e4m3 the bf16 copies of q, o, dout, k and v.
 *   workspace_bytes  its size
 * The gradients are computed in fp32 with the probabilities and dS rounded to the 16-bit type
 * for the matrix cores, and written rounded to nearest even.
 * Errors as fmha_fwd (o, dout, lse and dq are required when there are query rows; k, v, dk and
 * dv when there are keys; all but lse 16-byte aligned), and: workspace NULL ->
 * FMHA_ERR_NULL_POINTER, not 16-byte aligned -> FMHA_ERR_MISALIGNED, smaller than needed ->
 * FMHA_ERR_INVALID_ARGUMENT (checked when there are query rows, and for e4m3 whenever there is
 * work).  With query rows but no keys dq is zeroed; with keys but no query rows dk and dv are
 * zeroed.  Rows and keys outside the sequences are never touched.
 */
fmha_status fmha_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                     void* dq, void* dk, void* dv, int32_t B, int32_t Sq, int32_t Sk, int32_t H, int32_t H_kv,
                     int32_t D, float scale, fmha_mask mask, fmha_dtype dtype, const fmha_varlen* varlen,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes fmha_bwd needs for this shape and dtype (host arithmetic only; the packed
 * form reads only varlen->total_length_q and total_length_k).  Returns 0 for an invalid shape or
 * dtype, or one too large for the kernels' 32-bit offsets (and for fp16/bf16 with no query rows,
 * where no workspace is used). */
size_t fmha_bwd_workspace_size(int32_t B, int32_t Sq, int32_t Sk, int32_t H, int32_t H_kv, int32_t D,
                               fmha_dtype dtype, const fmha_varlen* varlen);

/* Paged K/V cache: fixed-size pages shared by all sequences, addressed through a block table.
 * This is the KV-cache-block layout that the sm120 article's TODO section names as the core of
 * paged attention, with the per-sequence index remapping of the CUTLASS generation kernel and
 * the power-of-two pages of its MLA kernel (trdm.cn walk-through "CUTLASS Blackwell FMHA 示例完全
 * 解析", sections on the generation kernel and on MLA).
 *   k_cache, v_cache  [num_pages, page_size, H_kv, D], contiguous, 16-byte aligned
 *   block_table       device int32 [B, max_pages_per_seq]: key j of sequence b is row
 *                     j % page_size of page block_table[b * max_pages_per_seq + j / page_size].
 *                     Entries outside [0, num_pages) read as zero keys and values (no fault).
 *   seqlens_k         device int32 [B]: keys of sequence b, at most the Sk of the call
 *                     (larger values are clamped to Sk, negative ones to 0)
 *   page_size         a power of two from 32 to 65536
 *   kv_dtype          element type of the cache: the call's dtype, or FMHA_DTYPE_F8E4M3 for an
 *                     e4m3 cache under fp16/bf16 queries (the fp8/INT8 KV quantisation the sm120
 *                     article's TODO section lists).  e4m3 values widen exactly to fp16/bf16 for
 *                     the matrix cores; the caller folds the cache's per-tensor dequantisation
 *                     scales into scale (K) and o_scale (V), as for fp8 in fmha_fwd.  D 32, 64 or 128.
 * Rows of a page past its sequence's end are never read. */
typedef struct {
  const int32_t* block_table;
  const int32_t* seqlens_k;
  int32_t max_pages_per_seq;
  int32_t page_size;
  int32_t num_pages;
  fmha_dtype kv_dtype;
} fmha_paged_kv;

/*
 * fmha_fwd_splitkv_paged -- fmha_fwd_splitkv with K and V in a paged cache (see fmha_paged_kv):
 * the same split-KV kernels, reading each 32-key tile from the page that holds it.  q, o and lse
 * are dense ([B, Sq, H, D], [B, H, Sq]); Sk is the most keys of any sequence (it sizes the
 * splits, and max_pages_per_seq * page_size must reach it).  The causal-qend offset of sequence b
 * is seqlens_k[b] - Sq.  workspace: fmha_fwd_splitkv_workspace_size(B, Sq, Sk, H, H_kv, D, NULL)
 * bytes.  dtype (q and o): FMHA_DTYPE_F16 or FMHA_DTYPE_BF16, or FMHA_DTYPE_F8E4M3 over an e4m3 cache
 * (q and o e4m3 as in fmha_fwd_splitkv).
 * Errors as fmha_fwd_splitkv, and: paged NULL, or (when Sk > 0) k_cache, v_cache, block_table or
 * seqlens_k NULL -> FMHA_ERR_NULL_POINTER; page_size not a power of two in [32, 65536],
 * max_pages_per_seq * page_size < Sk, or num_pages < 1 -> FMHA_ERR_INVALID_SHAPE; kv_dtype neither
 * dtype nor FMHA_DTYPE_F8E4M3 (e4m3 queries need an e4m3 cache) -> FMHA_ERR_UNSUPPORTED.
 */
fmha_status fmha_fwd_splitkv_paged(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                                   int32_t B, int32_t Sq, int32_t Sk, int32_t H, int32_t H_kv, int32_t D, float scale,
                                   fmha_mask mask, fmha_dtype dtype, float o_scale, const fmha_paged_kv* paged,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fmha_paged_kv_append -- insert the new tokens' K and V into a paged cache, the step before a
 * decode call over it: the CUTLASS generation kernel's default mode, which inserts the new
 * tokens' K/V, as opposed to its --cache-only mode, which only reads the cache (trdm.cn
 * walk-through "CUTLASS Blackwell FMHA 示例完全解析", section on the generation kernel and its
 * options).
 *   k_cache, v_cache  the cache of paged (see fmha_paged_kv), written in place
 *   k_new, v_new      device [B, S_new, H_kv, D] dense, 16-byte aligned, of the cache's element
 *                     type paged->kv_dtype (an e4m3 cache takes e4m3 rows, quantised by the caller
 *                     with the cache's scales); bytes are copied unchanged
 *   paged->seqlens_k  keys of each sequence counting the new tokens: new row i of sequence b
 *                     becomes key seqlens_k[b] - S_new + i, so that a following
 *                     fmha_fwd_splitkv_paged call with Sq = S_new and causal-qend aligns each new
 *                     query with its own key
 * Rows whose key would lie before key 0 or past max_pages_per_seq * page_size, or whose table
 * entry is outside [0, num_pages), are not written.  Two new rows that the table maps to the same
 * cache row race (either may win).  Asynchronous on stream; nothing is allocated.
 * Errors: paged NULL, or (B * S_new > 0) k_cache, v_cache, k_new, v_new, block_table or seqlens_k
 * NULL -> FMHA_ERR_NULL_POINTER; B or S_new negative, H_kv < 1, D not 32, 64 or 128, page_size not
 * a power of two in [32, 65536], max_pages_per_seq < 1 or num_pages < 1 -> FMHA_ERR_INVALID_SHAPE;
 * kv_dtype not a fmha_dtype, B * S_new or H_kv * D * element size at or past 2^31 ->
 * FMHA_ERR_UNSUPPORTED; a pointer not 16-byte aligned -> FMHA_ERR_MISALIGNED.  B or S_new 0: FMHA_OK,
 * nothing launched.
 */
fmha_status fmha_paged_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new, int32_t B,
                                 int32_t S_new, int32_t H_kv, int32_t D, const fmha_paged_kv* paged,
                                 hipStream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fmha_status_string(fmha_status status);

/* Library version as 10000 * major + 100 * minor + patch. */
int32_t fmha_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FMHA_H_ */
