"""fp64 CPU oracle of attention over a paged K/V cache.

TEST INFRASTRUCTURE ONLY -- see oracle/__init__.py.

The sm120 article ("[CUDA 优化实战] fmha sm120: 超越 torch.sdpa(flash-attention-2)", section
"TODO") names attention over KV-cache blocks as the core of paged attention, which an
inference framework needs; the CUTLASS walk-through (trdm.cn, "CUTLASS Blackwell FMHA 示例完全
解析") shows the generation kernel reading the cache of each batch entry through an index
remapping (its "--remap" option, section on the generation kernel) and the MLA kernel reading
the cache in pages (page size 128, or a power of two up to 128; MLA section).  The pages fix no
layout, so this module takes the plainest one, a block table:

* the cache holds ``num_pages`` pages of ``page_size`` keys: k_cache, v_cache
  [num_pages, page_size, H_kv, D];
* sequence b owns ``seqlens_k[b]`` keys; its key j lives in physical page
  ``block_table[b, j // page_size]`` at row ``j % page_size``;
* rows of a page past the sequence end, and pages the table does not name, are not part of
  any sequence.

The attention itself is the forward definition of oracle.attention on the gathered keys.

``append_paged`` is the step before a decode call that the walk-through's generation section
describes as the kernel's default mode (its "--cache-only" option turns it off): the new tokens'
K and V are inserted into the cache.  The pages fix no positions; the reading here is that
``seqlens_k`` already counts the new tokens, so that the decode call's causal-qend offset
(seqlens_k[b] - Sq) lines the new queries up with their own keys: new row i of sequence b is key
seqlens_k[b] - S_new + i.  Rows that would land before key 0, past the block table, or in a page
number outside [0, num_pages) are dropped, like the table entries the attention reads as zeros.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

from .attention import attention_head


def gather_pages(cache: np.ndarray, block_table: np.ndarray, seqlen: int, page_size: int) -> np.ndarray:
    """Keys (or values) of one sequence, in order: [seqlen, H_kv, D] from the pages its table row names."""
    n_pages = -(-int(seqlen) // page_size)
    pages = [cache[int(block_table[i])] for i in range(n_pages)]
    if not pages:
        return np.zeros((0,) + cache.shape[2:], dtype=cache.dtype)
    return np.concatenate(pages, axis=0)[:seqlen]


def attention_paged(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_table: np.ndarray,
                    seqlens_k: Sequence[int], scale: float, mask: str,
                    o_scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """q [B, Sq, H, D] dense; caches [num_pages, page_size, H_kv, D] -> O [B, Sq, H, D], LSE [B, H, Sq]."""
    B, Sq, H, D = q.shape
    page_size, H_kv = k_cache.shape[1], k_cache.shape[2]
    if H % H_kv:
        raise ValueError("H must be a multiple of H_kv")
    group = H // H_kv
    o = np.zeros((B, Sq, H, D))
    lse = np.zeros((B, H, Sq))
    for b in range(B):
        kb = gather_pages(k_cache, block_table[b], int(seqlens_k[b]), page_size)
        vb = gather_pages(v_cache, block_table[b], int(seqlens_k[b]), page_size)
        for h in range(H):
            o[b, :, h], lse[b, h] = attention_head(q[b, :, h], kb[:, h // group], vb[:, h // group], scale, mask)
    return o_scale * o, lse


def append_paged(k_cache: np.ndarray, v_cache: np.ndarray, block_table: np.ndarray, seqlens_k: Sequence[int],
                 k_new: np.ndarray, v_new: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Caches [num_pages, page_size, H_kv, D] after inserting k_new, v_new [B, S_new, H_kv, D] (any
    element type: values are copied as they are).  Returns new arrays; the inputs are unchanged."""
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    num_pages, page_size = kc.shape[0], kc.shape[1]
    B, S_new = k_new.shape[0], k_new.shape[1]
    max_pages = block_table.shape[1]
    for b in range(B):
        for i in range(S_new):
            pos = int(seqlens_k[b]) - S_new + i  # key index of new row i
            if pos < 0 or pos >= max_pages * page_size:
                continue
            page = int(block_table[b, pos // page_size])
            if not 0 <= page < num_pages:
                continue
            kc[page, pos % page_size] = k_new[b, i]
            vc[page, pos % page_size] = v_new[b, i]
    return kc, vc
