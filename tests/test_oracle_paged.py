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


# ----------------------------------------------------------------------------------------------
# append_paged: inserting the new tokens' K/V before a decode step
# ----------------------------------------------------------------------------------------------
def test_append_hand_example():
    # 3 pages of 2 rows, one head, one dim; sequence 0 owns pages [2, 0] and 3 keys, the last two
    # of which are new: key 1 -> page 2 row 1, key 2 -> page 0 row 0 (worked out by hand)
    kc = np.arange(6, dtype=np.int16).reshape(3, 2, 1, 1)
    vc = (100 + np.arange(6, dtype=np.int16)).reshape(3, 2, 1, 1)
    bt = np.array([[2, 0]], dtype=np.int32)
    k_new = np.array([[[[10]], [[11]]]], dtype=np.int16)
    v_new = np.array([[[[20]], [[21]]]], dtype=np.int16)
    k2, v2 = oracle_paged.append_paged(kc, vc, bt, [3], k_new, v_new)
    assert k2[:, :, 0, 0].tolist() == [[11, 1], [2, 3], [4, 10]]
    assert v2[:, :, 0, 0].tolist() == [[21, 101], [102, 103], [104, 20]]
    assert kc[:, :, 0, 0].tolist() == [[0, 1], [2, 3], [4, 5]]  # inputs unchanged


@pytest.mark.parametrize("page_size", [2, 4, 8])
def test_append_then_gather_is_old_keys_then_new_rows(page_size):
    rng = np.random.default_rng(31 + page_size)
    B, S_new, H_kv, D = 3, 3, 2, 4
    seqlens = [S_new, 7, 13]  # the first sequence is all new
    n_pages = [-(-s // page_size) for s in seqlens]
    num_pages = sum(n_pages) + 2
    perm = rng.permutation(num_pages)
    bt = np.full((B, max(n_pages)), -1, dtype=np.int32)
    n = 0
    for b in range(B):
        for i in range(n_pages[b]):
            bt[b, i] = perm[n]
            n += 1
    kc, vc = _cache(rng, num_pages, page_size, H_kv, D)
    k_new, v_new = rng.standard_normal((B, S_new, H_kv, D)), rng.standard_normal((B, S_new, H_kv, D))
    k2, v2 = oracle_paged.append_paged(kc, vc, bt, seqlens, k_new, v_new)
    for b in range(B):
        L = seqlens[b]
        for new, old, cache in ((k_new, kc, k2), (v_new, vc, v2)):
            got = oracle_paged.gather_pages(cache, bt[b], L, page_size)
            before = oracle_paged.gather_pages(old, bt[b], L, page_size)
            np.testing.assert_array_equal(got[:L - S_new], before[:L - S_new])
            np.testing.assert_array_equal(got[L - S_new:], new[b])
    # pages no sequence owns, and rows past each sequence's end, are untouched
    owned = np.zeros(kc.shape[:2], dtype=bool)
    for b in range(B):
        for j in range(seqlens[b]):
            owned[bt[b, j // page_size], j % page_size] = True
    np.testing.assert_array_equal(k2[~owned], kc[~owned])
    np.testing.assert_array_equal(v2[~owned], vc[~owned])


def test_append_drops_rows_outside_the_table():
    rng = np.random.default_rng(5)
    kc, vc = _cache(rng, 4, 2, 1, 2)
    k_new, v_new = rng.standard_normal((2, 3, 1, 2)), rng.standard_normal((2, 3, 1, 2))
    # sequence 0: only one key, so new rows 0 and 1 would lie before key 0; sequence 1: its
    # second page entry is -1 and the third is past num_pages
    bt = np.array([[1, -1, 9], [3, -1, 9]], dtype=np.int32)
    k2, v2 = oracle_paged.append_paged(kc, vc, bt, [1, 5], k_new, v_new)
    exp_k = kc.copy()
    exp_k[1, 0] = k_new[0, 2]  # sequence 0, key 0
    # sequence 1: keys 2, 3 -> page -1 (dropped), key 4 -> page 9 (dropped)
    np.testing.assert_array_equal(k2, exp_k)
    exp_v = vc.copy()
    exp_v[1, 0] = v_new[0, 2]
    np.testing.assert_array_equal(v2, exp_v)


def test_append_planted_off_by_one_is_caught():
    # a version that writes new row i at seqlens_k - S_new + i + 1 breaks the gather invariant
    rng = np.random.default_rng(8)
    kc, vc = _cache(rng, 3, 4, 1, 2)
    bt = np.array([[0, 2]], dtype=np.int32)
    k_new, v_new = rng.standard_normal((1, 2, 1, 2)), rng.standard_normal((1, 2, 1, 2))
    wrong = kc.copy()
    for i in range(2):
        pos = 6 - 2 + i + 1
        wrong[bt[0, pos // 4], pos % 4] = k_new[0, i]
    right, _ = oracle_paged.append_paged(kc, vc, bt, [6], k_new, v_new)
    assert not np.array_equal(oracle_paged.gather_pages(wrong, bt[0], 6, 4)[4:], k_new[0])
    np.testing.assert_array_equal(oracle_paged.gather_pages(right, bt[0], 6, 4)[4:], k_new[0])
