"""Pins of the paged-cache oracle against facts that do not come from it.

Brute force with per-key page arithmetic, the dense forward oracle (pinned on its own) on a
cache laid out in order, invariance under relabelling the physical pages, independence from
memory no sequence owns, the empty sequence, and planted mistakes.  CPU only.
"""
import math
import types

import numpy as np
import pytest

from oracle import attention as oracle_attention
from oracle import paged as oracle_paged

MASKS = ("none", "residual", "causal_qbegin", "causal_qend")


def _cache(rng, num_pages, page_size, H_kv, D):
    return rng.standard_normal((num_pages, page_size, H_kv, D)), rng.standard_normal((num_pages, page_size, H_kv, D))


def _brute(q, kc, vc, bt, seqlens, scale, mask, page_size):
    """Per key j: page bt[b][j // page_size], row j % page_size; softmax written as the plain quotient."""
    B, Sq, H, D = q.shape
    H_kv = kc.shape[2]
    o = np.zeros((B, Sq, H, D))
    lse = np.zeros((B, H, Sq))
    for b in range(B):
        sk = int(seqlens[b])
        for h in range(H):
            g = h // (H // H_kv)
            for i in range(Sq):
                ws, acc = [], np.zeros(D)
                for j in range(sk):
                    if mask == "causal_qbegin" and j > i:
                        continue
                    if mask == "causal_qend" and j > i + (sk - Sq):
                        continue
                    page, row = int(bt[b][j // page_size]), j % page_size
                    w = math.exp(scale * float(np.dot(q[b, i, h], kc[page, row, g])))
                    ws.append(w)
                    acc += w * vc[page, row, g]
                den = sum(ws)
                o[b, i, h] = acc / den if ws else 0.0
                lse[b, h, i] = math.log(den) if ws else -math.inf
    return o, lse


def pin_brute_force(mod):
    rng = np.random.default_rng(21)
    ps, H, H_kv, D = 4, 4, 2, 8
    kc, vc = _cache(rng, 9, ps, H_kv, D)
    bt = np.array([[7, 2, 5], [0, 8, 1], [3, 6, 4]])
    seqlens = [10, 3, 12]
    for Sq in (1, 3):
        q = rng.standard_normal((3, Sq, H, D))
        for mask in MASKS:
            o, lse = mod.attention_paged(q, kc, vc, bt, seqlens, 0.4, mask)
            eo, el = _brute(q, kc, vc, bt, seqlens, 0.4, mask, ps)
            np.testing.assert_allclose(o, eo, rtol=1e-11, atol=1e-13)
            np.testing.assert_allclose(lse, el, rtol=1e-12)


def pin_dense_in_order(mod):
    # pages laid out in order, one table row per sequence: the dense forward oracle on the contiguous cache
    rng = np.random.default_rng(22)
    B, Sq, S, H, H_kv, D, ps = 2, 5, 24, 4, 4, 16, 8
    kc, vc = _cache(rng, B * S // ps, ps, H_kv, D)
    bt = np.arange(B * S // ps).reshape(B, S // ps)
    q = rng.standard_normal((B, Sq, H, D))
    k = kc.reshape(B, S, H_kv, D)
    v = vc.reshape(B, S, H_kv, D)
    for mask in MASKS:
        o, lse = mod.attention_paged(q, kc, vc, bt, [S] * B, 0.3, mask, o_scale=0.5)
        eo, el = oracle_attention.attention_dense(q, k, v, 0.3, mask, o_scale=0.5)
        np.testing.assert_allclose(o, eo, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse, el, rtol=1e-12)


def pin_invariants(mod):
    rng = np.random.default_rng(23)
    ps, H, H_kv, D = 8, 6, 2, 8
    kc, vc = _cache(rng, 12, ps, H_kv, D)
    bt = np.array([[3, 9, 0, 11], [5, 1, 7, 2]])
    seqlens = [29, 17]
    q = rng.standard_normal((2, 2, H, D))
    for mask in MASKS:
        o, lse = mod.attention_paged(q, kc, vc, bt, seqlens, 0.5, mask)
        # relabelling the physical pages (cache and table together) changes nothing
        perm = rng.permutation(12)
        inv = np.argsort(perm)
        o2, lse2 = mod.attention_paged(q, kc[perm], vc[perm], inv[bt], seqlens, 0.5, mask)
        np.testing.assert_array_equal(o2, o)
        np.testing.assert_array_equal(lse2, lse)
        # memory no sequence owns (other pages, rows past a sequence's end) does not enter
        kn, vn = kc.copy(), vc.copy()
        used = set()
        for b, sk in enumerate(seqlens):
            for j in range(sk):
                used.add((int(bt[b][j // ps]), j % ps))
        for pg in range(12):
            for r in range(ps):
                if (pg, r) not in used:
                    kn[pg, r] = np.nan
                    vn[pg, r] = np.nan
        o3, lse3 = mod.attention_paged(q, kn, vn, bt, seqlens, 0.5, mask)
        np.testing.assert_array_equal(o3, o)
        np.testing.assert_array_equal(lse3, lse)
    # an empty sequence: O = 0, LSE = -inf
    o, lse = mod.attention_paged(q, kc, vc, bt, [0, 17], 0.5, "none")
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))


PINS = [pin_brute_force, pin_dense_in_order, pin_invariants]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_paged_oracle_pin(pin):
    pin(oracle_paged)


MUTATIONS = {
    "page index off by one": ("pages = [cache[int(block_table[i])] for i in range(n_pages)]",
                              "pages = [cache[int(block_table[min(i + 1, len(block_table) - 1)])] for i in range(n_pages)]"),
    "whole last page kept": ("return np.concatenate(pages, axis=0)[:seqlen]", "return np.concatenate(pages, axis=0)"),
    "pages in table order ignored": ("pages = [cache[int(block_table[i])] for i in range(n_pages)]",
                                     "pages = [cache[int(p)] for p in sorted(block_table[:n_pages])]"),
    "wrong GQA head": ("kb[:, h // group], vb[:, h // group]", "kb[:, h % H_kv], vb[:, h % H_kv]"),
}


def _mutant(name):
    src = open(oracle_paged.__file__).read()
    old, new = MUTATIONS[name]
    assert old in src, f"mutation anchor for {name!r} not found"
    src = src.replace("from .attention import attention_head", "from oracle.attention import attention_head")
    mod = types.ModuleType(f"oracle_paged_mutant_{name.replace(' ', '_')}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_paged_mistake_is_caught(name):
    mod = _mutant(name)
    caught = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutation {name!r} passed every pin"
