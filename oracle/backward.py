"""fp64 CPU oracle of the fused multi-head attention backward pass.

TEST INFRASTRUCTURE ONLY -- see oracle/__init__.py.

The CUTLASS Blackwell FMHA walk-through (trdm.cn, "CUTLASS Blackwell FMHA 示例完全解析",
section "FMHA for Blackwell: Backward") describes the backward of the forward pass in
oracle.attention as three steps: a row sum of O * dO, the main pass producing dQ, dK and
dV, and a conversion of dQ from fp32 to the output type.  The pages print no formulas for
it, so this module takes the plainest reading: the exact gradients, by the chain rule, of
the forward definition (S = scale * Q K^T, P = softmax(S) over the visible keys, O = P V)
for a given upstream gradient dO.  Per (sequence, head), with every matrix materialised:

    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - delta),   delta_i = sum_j P_ij dP_ij     (the softmax Jacobian)
    dQ = scale * dS K
    dK = scale * dS^T Q

delta is computed from its definition; it equals sum_d O_id dO_id (the quantity the
walk-through's first kernel sums), which the pins check.  A backward pass receives O as stored
(rounded to its type, e4m3 for fp8 inputs), and its first kernel sums that O; the optional `o`
argument takes delta from a given O in the same way, so that the effect of a coarsely stored O
is part of the expected result rather than of the error.  Masked positions have P = 0,
hence dS = 0: no gradient crosses them.  A query row with no visible key has an all-zero
P row and contributes nothing.

Masks follow the backward mask of the walk-through's fusion-point section (a position is
blanked when the query position plus the alignment offset is below the key position, or
it lies outside the problem); with the offset 0 (causal_qbegin) or Sk - Sq (causal_qend)
these are exactly the forward masks of oracle.attention.visible_keys.

GQA/MQA: the walk-through notes that the CUTLASS backward ignores the K/V head count.  The
definition extends to shared K/V heads without any choice: K/V head g feeds every query
head of its group, so its gradient is the sum over that group.

Packed variable-length batches: sequence b owns rows [cu[b], cu[b+1]) as in the forward.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

from .attention import attention_head, visible_keys


def attention_head_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float,
                            mask: str, o: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One sequence and head: q, do [sq, D]; k, v [sk, D].  Returns dQ [sq, D], dK, dV [sk, D] (fp64).

    o: None, or the forward output [sq, D] as a backward pass receives it (rounded to a storage
    type).  Given, delta is the row sum of O * dO over it, the quantity the walk-through's first
    backward kernel forms from its O input, instead of sum_j P_ij dP_ij; the two are equal when
    o is the exact output."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    _, _, _, p = attention_head(q, k, v, scale, mask, return_p=True)
    dv = p.T @ do
    dp = do @ v.T
    if o is None:
        delta = (p * dp).sum(axis=1)
    else:
        delta = sum_o_do(o, do)
    ds = p * (dp - delta[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def attention_head_backward_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float,
                                 mask: str, q_rows: Sequence[int], k_rows: Sequence[int],
                                 chunk: int = 1024) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One sequence and head too long to hold S whole: the gradients of attention_head_backward
    at the query rows q_rows (dQ) and at the key rows k_rows (this head's part of dK and dV),
    with S, P and dP formed for `chunk` query rows at a time (the same steps, row block by row
    block; only the order of the sums over query rows changes).
    Returns dQ [len(q_rows), D], dK [len(k_rows), D], dV [len(k_rows), D] (fp64)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    sq, sk, D = q.shape[0], k.shape[0], q.shape[1]
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    dq_rows = np.zeros((len(q_rows), D))
    dk_rows = np.zeros((len(k_rows), D))
    dv_rows = np.zeros((len(k_rows), D))
    for r0 in range(0, sq, chunk):
        r1 = min(sq, r0 + chunk)
        # the forward's probabilities of rows r0 .. r1 - 1 (rows with no visible key: P = 0)
        s = scale * (q[r0:r1] @ k.T)
        vis = visible_keys(sq, sk, mask, rows=range(r0, r1))
        has_key = vis.any(axis=1)
        m = np.where(has_key, np.where(vis, s, -np.inf).max(axis=1, initial=-np.inf), 0.0)
        e = np.where(vis, np.exp(np.where(vis, s, 0.0) - m[:, None]), 0.0)
        den = e.sum(axis=1)
        p = np.zeros_like(e)
        p[has_key] = e[has_key] / den[has_key, None]
        # the backward steps on these rows
        dp = do[r0:r1] @ v.T
        delta_rows = (p * dp).sum(axis=1)
        ds = p * (dp - delta_rows[:, None])
        sel = np.nonzero((q_rows >= r0) & (q_rows < r1))[0]
        dq_rows[sel] = scale * (ds[q_rows[sel] - r0] @ k)
        dk_rows += scale * (ds[:, k_rows].T @ q[r0:r1])
        dv_rows += p[:, k_rows].T @ do[r0:r1]
    return dq_rows, dk_rows, dv_rows


def attention_backward_dense(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float,
                             mask: str, o: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """BSHD layout: q, do [B, Sq, H, D]; k, v [B, Sk, H_kv, D] -> dQ [B, Sq, H, D], dK, dV [B, Sk, H_kv, D].
    o: None or the forward output [B, Sq, H, D] as received (see attention_head_backward)."""
    B, Sq, H, D = q.shape
    H_kv = k.shape[2]
    if H % H_kv:
        raise ValueError("H must be a multiple of H_kv")
    group = H // H_kv
    dq = np.zeros((B, Sq, H, D))
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(B):
        for h in range(H):
            kvh = h // group
            gq, gk, gv = attention_head_backward(q[b, :, h], k[b, :, kvh], v[b, :, kvh], do[b, :, h], scale, mask,
                                                 None if o is None else o[b, :, h])
            dq[b, :, h] = gq
            dk[b, :, kvh] += gk
            dv[b, :, kvh] += gv
    return dq, dk, dv


def attention_backward_varlen(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, cu_q: Sequence[int],
                              cu_k: Sequence[int], scale: float, mask: str,
                              o: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Packed layout: q, do [total_q, H, D]; k, v [total_k, H_kv, D] -> dQ, dK, dV of the same shapes.
    o: None or the forward output [total_q, H, D] as received (see attention_head_backward)."""
    total_q, H, D = q.shape
    H_kv = k.shape[1]
    if H % H_kv:
        raise ValueError("H must be a multiple of H_kv")
    group = H // H_kv
    dq = np.zeros((total_q, H, D))
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        for h in range(H):
            kvh = h // group
            gq, gk, gv = attention_head_backward(q[q0:q1, h], k[k0:k1, kvh], v[k0:k1, kvh], do[q0:q1, h], scale,
                                                 mask, None if o is None else o[q0:q1, h])
            dq[q0:q1, h] = gq
            dk[k0:k1, kvh] += gk
            dv[k0:k1, kvh] += gv
    return dq, dk, dv


def sum_o_do(o: np.ndarray, do: np.ndarray) -> np.ndarray:
    """Row sums of O * dO over the head dimension (the walk-through's first backward kernel).

    Any layout with D last: returns o.shape[:-1].
    """
    return (np.asarray(o, dtype=np.float64) * np.asarray(do, dtype=np.float64)).sum(axis=-1)
