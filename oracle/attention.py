"""fp64 CPU oracle of the fused multi-head attention forward pass.

TEST INFRASTRUCTURE ONLY -- see oracle/__init__.py.

It computes, per (sequence, head), the plain three-step definition that the
wingedge777 article "[CUDA 优化实战] fmha sm120: 超越 torch.sdpa(flash-attention-2)"
gives in its section "1. flash attention": S = scale * Q K^T, P = softmax(S) along
the keys, O = P V.  S and P are materialised in full; there is no tiling, no
online softmax and no reordering.  Matrix products use numpy's fp64 matmul.

Masks (the CUTLASS Blackwell FMHA walk-through, trdm.cn, section on the fusion
point ``collective/fmha_fusion.hpp``, and the same article's causal section
"k_end 和 need_causal_mask"):

* ``none`` and ``residual``: every key j < Sk of the sequence is visible.  The
  residual mask only exists to blank the keys past Sk inside a partial last
  tile, which this untiled definition never forms, so both give the same O.
* ``causal_qbegin``: query i sees key j iff j <= i (queries aligned to the first
  key; the diagonal is kept, as the sm120 kernel's ``q >= k`` test keeps it).
* ``causal_qend``: query i sees key j iff j <= i + (Sk - Sq) (queries aligned
  to the last key; the page's ``offset_q = seqlen_k - seqlen_q``).

Masked positions get weight exactly 0.  A query row with no visible key has
O = 0 and LSE = -inf (the log of an empty sum; the pages do not say).

LSE is the natural-log log-sum-exp of the scaled scores over the visible keys,
the second output that the CUTLASS example's verification checks next to O.

GQA/MQA (the sm120 kernel's ``kv_head_id = head_id / group_size``; the
CUTLASS walk-through's section on GQA/MQA strides): query head h reads K/V head
h // (H / H_kv).

Packed variable-length batches (the CUTLASS walk-through's section on variable
sequence length): sequence b owns rows [cu[b], cu[b+1]) of the packed tensors.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

MASKS = ("none", "residual", "causal_qbegin", "causal_qend")


def visible_keys(sq: int, sk: int, mask: str, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Boolean [sq, sk] (or [len(rows), sk]): True where query i may attend to key j."""
    if mask not in MASKS:
        raise ValueError(f"unknown mask {mask!r}")
    i = (np.arange(sq) if rows is None else np.asarray(rows))[:, None]
    sq_rows = i.shape[0]
    j = np.arange(sk)[None, :]
    if mask in ("none", "residual"):
        return np.ones((sq_rows, sk), dtype=bool)
    if mask == "causal_qbegin":
        return j <= i
    return j <= i + (sk - sq)


def attention_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, mask: str,
                   return_p: bool = False):
    """One sequence and head: q [sq, D], k [sk, D], v [sk, D] (fp64).

    Returns O [sq, D], LSE [sq] and, if asked, S [sq, sk] and P [sq, sk].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    sq, sk = q.shape[0], k.shape[0]
    s = scale * (q @ k.T)
    vis = visible_keys(sq, sk, mask)
    has_key = vis.any(axis=1)
    m = np.where(has_key, np.where(vis, s, -np.inf).max(axis=1, initial=-np.inf), 0.0)
    e = np.where(vis, np.exp(np.where(vis, s, 0.0) - m[:, None]), 0.0)
    den = e.sum(axis=1)
    p = np.zeros_like(e)
    p[has_key] = e[has_key] / den[has_key, None]
    o = p @ v
    lse = np.full(sq, -np.inf)
    lse[has_key] = m[has_key] + np.log(den[has_key])
    if return_p:
        return o, lse, s, p
    return o, lse


def attention_dense(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, mask: str,
                    o_scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """BSHD layout: q [B, Sq, H, D], k/v [B, Sk, H_kv, D] -> O [B, Sq, H, D] (times o_scale), LSE [B, H, Sq]."""
    B, Sq, H, D = q.shape
    H_kv = k.shape[2]
    if H % H_kv:
        raise ValueError("H must be a multiple of H_kv")
    group = H // H_kv
    o = np.zeros((B, Sq, H, D))
    lse = np.zeros((B, H, Sq))
    for b in range(B):
        for h in range(H):
            kvh = h // group
            o[b, :, h], lse[b, h] = attention_head(q[b, :, h], k[b, :, kvh], v[b, :, kvh], scale, mask)
    return o_scale * o, lse


def attention_varlen(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_q: Sequence[int], cu_k: Sequence[int],
                     scale: float, mask: str, o_scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """Packed layout: q [total_q, H, D], k/v [total_k, H_kv, D] -> O [total_q, H, D], LSE [H, total_q]."""
    total_q, H, D = q.shape
    H_kv = k.shape[1]
    group = H // H_kv
    o = np.zeros((total_q, H, D))
    lse = np.zeros((H, total_q))
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        for h in range(H):
            kvh = h // group
            o[q0:q1, h], lse[h, q0:q1] = attention_head(q[q0:q1, h], k[k0:k1, kvh], v[k0:k1, kvh], scale, mask)
    return o_scale * o, lse


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, mask: str,
                   picks: Iterable[Tuple[int, int, int]], o_scale: float = 1.0,
                   cu_q: Optional[Sequence[int]] = None, cu_k: Optional[Sequence[int]] = None):
    """Selected output rows, one (batch b, head h, query i) at a time.

    Dense layout unless ``cu_q``/``cu_k`` are given (then i is the row inside sequence b).
    Returns O rows [n, D] (times o_scale) and LSE values [n].
    """
    picks = list(picks)
    D = q.shape[-1]
    H = q.shape[-2]
    H_kv = k.shape[-2]
    group = H // H_kv
    o = np.zeros((len(picks), D))
    lse = np.zeros(len(picks))
    for n, (b, h, i) in enumerate(picks):
        kvh = h // group
        if cu_q is None:
            sq, sk = q.shape[1], k.shape[1]
            qi = q[b, i:i + 1, h]
            kk, vv = k[b, :, kvh], v[b, :, kvh]
        else:
            q0, k0, k1 = int(cu_q[b]), int(cu_k[b]), int(cu_k[b + 1])
            sq, sk = int(cu_q[b + 1]) - q0, k1 - k0
            qi = q[q0 + i:q0 + i + 1, h]
            kk, vv = k[k0:k1, kvh], v[k0:k1, kvh]
        # the row of the mask that belongs to query i of a [sq, sk] problem
        vis = visible_keys(sq, sk, mask, rows=[i])[0]
        o_row, lse_row = attention_head(qi, kk[vis], vv[vis], scale, "none")
        o[n] = o_row[0]
        lse[n] = lse_row[0]
    return o_scale * o, lse
