"""Pins of the fp64 backward oracle against facts that do not come from the oracle itself.

Automatic differentiation (torch autograd through a materialised attention, and through
torch's scaled_dot_product_attention), central finite differences of the separately pinned
forward oracle, closed forms of special cases, invariants of the softmax, and planted
mistakes that the pins must catch.  CPU only.
"""
import types

import numpy as np
import pytest
import torch

from oracle import attention as oracle_attention
from oracle import backward as oracle_backward

MASKS = ("none", "residual", "causal_qbegin", "causal_qend")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _visible(sq, sk, mask):
    i = np.arange(sq)[:, None]
    j = np.arange(sk)[None, :]
    if mask in ("none", "residual"):
        return np.ones((sq, sk), dtype=bool)
    if mask == "causal_qbegin":
        return j <= i
    return j <= i + (sk - sq)


def _autograd_head(q, k, v, do, scale, mask):
    """Gradients of sum(O * dO) by torch autograd through an explicit fp64 forward."""
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = scale * (tq @ tk.T)
    s = s.masked_fill(~torch.from_numpy(_visible(q.shape[0], k.shape[0], mask)), float("-inf"))
    o = torch.softmax(s, dim=-1) @ tv
    (o * torch.tensor(do)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


# ----------------------------------------------------------------------------------------------
# pins, written against a module so that planted mistakes can be run through them
# ----------------------------------------------------------------------------------------------
def pin_autograd(mod):
    rng = np.random.default_rng(11)
    # every row keeps a visible key (torch's softmax of an all -inf row is NaN)
    for sq, sk in ((5, 5), (3, 7), (6, 4)):
        for mask in MASKS:
            if mask == "causal_qend" and sk < sq:
                continue
            q, k, v, do = _rand(rng, sq, 8), _rand(rng, sk, 8), _rand(rng, sk, 8), _rand(rng, sq, 8)
            ours = mod.attention_head_backward(q, k, v, do, 0.7, mask)
            ref = _autograd_head(q, k, v, do, 0.7, mask)
            for a, r in zip(ours, ref):
                np.testing.assert_allclose(a, r, rtol=1e-10, atol=1e-12)


def pin_library_sdpa(mod):
    """torch's scaled_dot_product_attention (fp64, CPU) differentiated by autograd, BSHD batches with GQA."""
    rng = np.random.default_rng(12)
    B, sq, sk, H, H_kv, D = 2, 6, 9, 4, 2, 16
    q, do = _rand(rng, B, sq, H, D), _rand(rng, B, sq, H, D)
    k, v = _rand(rng, B, sk, H_kv, D), _rand(rng, B, sk, H_kv, D)
    group = H // H_kv
    for mask in ("none", "causal_qbegin", "causal_qend"):
        tq = torch.tensor(q.transpose(0, 2, 1, 3), requires_grad=True)
        tk = torch.tensor(k.transpose(0, 2, 1, 3), requires_grad=True)
        tv = torch.tensor(v.transpose(0, 2, 1, 3), requires_grad=True)
        kk = tk.repeat_interleave(group, dim=1)
        vv = tv.repeat_interleave(group, dim=1)
        if mask == "none":
            o = torch.nn.functional.scaled_dot_product_attention(tq, kk, vv, scale=0.3)
        elif mask == "causal_qbegin":
            o = torch.nn.functional.scaled_dot_product_attention(tq, kk, vv, is_causal=True, scale=0.3)
        else:
            am = torch.from_numpy(_visible(sq, sk, mask))
            o = torch.nn.functional.scaled_dot_product_attention(tq, kk, vv, attn_mask=am, scale=0.3)
        (o * torch.tensor(do.transpose(0, 2, 1, 3))).sum().backward()
        dq, dk, dv = mod.attention_backward_dense(q, k, v, do, 0.3, mask)
        np.testing.assert_allclose(dq, tq.grad.numpy().transpose(0, 2, 1, 3), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dk, tk.grad.numpy().transpose(0, 2, 1, 3), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dv, tv.grad.numpy().transpose(0, 2, 1, 3), rtol=1e-10, atol=1e-12)


def pin_finite_differences(mod):
    """Central differences of L = sum(O * dO), O from the forward oracle (pinned on its own)."""
    rng = np.random.default_rng(13)
    sq, sk, D, scale, eps = 4, 6, 5, 0.8, 1e-6
    for mask in MASKS:
        q, k, v, do = _rand(rng, sq, D), _rand(rng, sk, D), _rand(rng, sk, D), _rand(rng, sq, D)
        grads = mod.attention_head_backward(q, k, v, do, scale, mask)

        def loss(qq, kk, vv):
            o, _ = oracle_attention.attention_head(qq, kk, vv, scale, mask)
            return float((o * do).sum())

        for which, g in enumerate(grads):
            base = [q, k, v][which]
            for idx in np.ndindex(base.shape):
                plus, minus = [x.copy() for x in (q, k, v)], [x.copy() for x in (q, k, v)]
                plus[which][idx] += eps
                minus[which][idx] -= eps
                fd = (loss(*plus) - loss(*minus)) / (2 * eps)
                assert abs(fd - g[idx]) < 1e-7, (mask, "qkv"[which], idx, fd, g[idx])


def pin_closed_forms(mod):
    rng = np.random.default_rng(14)
    D, scale = 6, 0.5
    # one key: P = 1, so dS = 0 (no gradient to q or k) and dV = sum_i dO_i
    q, k, v, do = _rand(rng, 5, D), _rand(rng, 1, D), _rand(rng, 1, D), _rand(rng, 5, D)
    dq, dk, dv = mod.attention_head_backward(q, k, v, do, scale, "none")
    np.testing.assert_allclose(dq, 0.0, atol=1e-14)
    np.testing.assert_allclose(dk, 0.0, atol=1e-14)
    np.testing.assert_allclose(dv[0], do.sum(axis=0), rtol=1e-12)
    # Q = 0: uniform weights 1/n.  dV_j = mean_i dO_i; dK = 0 (dK is a combination of Q rows);
    # dQ_i = scale / n * sum_j (dO_i . (v_j - vbar)) k_j
    n = 7
    q, k, v, do = np.zeros((4, D)), _rand(rng, n, D), _rand(rng, n, D), _rand(rng, 4, D)
    dq, dk, dv = mod.attention_head_backward(q, k, v, do, scale, "none")
    np.testing.assert_allclose(dv, np.tile(do.sum(axis=0) / n, (n, 1)), rtol=1e-12)
    np.testing.assert_allclose(dk, 0.0, atol=1e-14)
    vbar = v.mean(axis=0)
    for i in range(4):
        expect = scale / n * sum(float(do[i] @ (v[j] - vbar)) * k[j] for j in range(n))
        np.testing.assert_allclose(dq[i], expect, rtol=1e-11, atol=1e-13)
    # causal_qbegin, row 0 sees only key 0: its dQ is 0 (a single visible key)
    q, k, v, do = _rand(rng, 4, D), _rand(rng, 4, D), _rand(rng, 4, D), _rand(rng, 4, D)
    dq, _, _ = mod.attention_head_backward(q, k, v, do, scale, "causal_qbegin")
    np.testing.assert_allclose(dq[0], 0.0, atol=1e-14)
    # causal_qend with sq > sk: rows i < sq - sk see no key, get dQ = 0, and change nothing else
    q, v, do = _rand(rng, 6, D), _rand(rng, 3, D), _rand(rng, 6, D)
    k = _rand(rng, 3, D)
    dq, dk, dv = mod.attention_head_backward(q, k, v, do, scale, "causal_qend")
    np.testing.assert_allclose(dq[:3], 0.0, atol=1e-14)
    do2 = do.copy()
    do2[:3] = rng.standard_normal((3, D))
    q2 = q.copy()
    q2[:3] = rng.standard_normal((3, D))
    dq2, dk2, dv2 = mod.attention_head_backward(q2, k, v, do2, scale, "causal_qend")
    np.testing.assert_array_equal(dk2, dk)
    np.testing.assert_array_equal(dv2, dv)
    np.testing.assert_array_equal(dq2[3:], dq[3:])


def pin_invariants(mod):
    rng = np.random.default_rng(15)
    D, scale = 8, 0.6
    for sq, sk in ((5, 5), (4, 9), (9, 4)):
        for mask in MASKS:
            q, k, v, do = _rand(rng, sq, D), _rand(rng, sk, D), _rand(rng, sk, D), _rand(rng, sq, D)
            dq, dk, dv = mod.attention_head_backward(q, k, v, do, scale, mask)
            vis = _visible(sq, sk, mask)
            rows = vis.any(axis=1)
            # shifting every key by u leaves O unchanged: sum_j dK_j = 0
            np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-11)
            # adding w to every value adds w to every row with a key: sum_j dV_j = sum_(rows) dO_i
            np.testing.assert_allclose(dv.sum(axis=0), do[rows].sum(axis=0), rtol=1e-10, atol=1e-11)
            # keys that no query sees get no gradient
            dead = ~vis.any(axis=0)
            assert np.all(dk[dead] == 0) and np.all(dv[dead] == 0)
            # dO enters linearly
            g2 = mod.attention_head_backward(q, k, v, 2.0 * do, scale, mask)
            for a, b in zip(g2, (dq, dk, dv)):
                np.testing.assert_allclose(a, 2.0 * b, rtol=1e-12, atol=1e-14)
            # the row sum the first backward kernel forms: sum_d O dO equals sum_j P dP
            o, _, _, p = oracle_attention.attention_head(q, k, v, scale, mask, return_p=True)
            np.testing.assert_allclose(oracle_backward.sum_o_do(o, do), (p * (do @ v.T)).sum(axis=1),
                                       rtol=1e-10, atol=1e-12)
    # GQA: the K/V gradient of a shared head is the sum over its group (MHA on repeated heads)
    B, sq, sk, H, H_kv = 2, 5, 7, 6, 2
    q, do = _rand(rng, B, sq, H, D), _rand(rng, B, sq, H, D)
    k, v = _rand(rng, B, sk, H_kv, D), _rand(rng, B, sk, H_kv, D)
    for mask in MASKS:
        dq, dk, dv = mod.attention_backward_dense(q, k, v, do, scale, mask)
        kr, vr = np.repeat(k, H // H_kv, axis=2), np.repeat(v, H // H_kv, axis=2)
        dq1, dk1, dv1 = mod.attention_backward_dense(q, kr, vr, do, scale, mask)
        np.testing.assert_allclose(dq, dq1, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(dk, dk1.reshape(B, sk, H_kv, H // H_kv, D).sum(axis=3), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dv, dv1.reshape(B, sk, H_kv, H // H_kv, D).sum(axis=3), rtol=1e-12, atol=1e-13)
        # head h of the dense batch is the single-head call on its K/V head
        for b in range(B):
            for h in range(H):
                g = mod.attention_head_backward(q[b, :, h], k[b, :, h // 3], v[b, :, h // 3], do[b, :, h], scale, mask)
                np.testing.assert_allclose(dq[b, :, h], g[0], rtol=1e-12, atol=1e-14)
    # packed batch == per-sequence dense runs
    lq, lk = [3, 6, 0, 2], [5, 2, 4, 0]
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    H, H_kv = 4, 2
    q, do = _rand(rng, cu_q[-1], H, D), _rand(rng, cu_q[-1], H, D)
    k, v = _rand(rng, cu_k[-1], H_kv, D), _rand(rng, cu_k[-1], H_kv, D)
    for mask in MASKS:
        dq, dk, dv = mod.attention_backward_varlen(q, k, v, do, cu_q, cu_k, scale, mask)
        for b in range(len(lq)):
            q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
            gq, gk, gv = mod.attention_backward_dense(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], do[None, q0:q1],
                                                      scale, mask)
            np.testing.assert_allclose(dq[q0:q1], gq[0], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(dk[k0:k1], gk[0], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(dv[k0:k1], gv[0], rtol=1e-12, atol=1e-14)


def pin_rows_autograd(mod):
    """The row-block form (long sequences) against autograd directly, several block sizes."""
    rng = np.random.default_rng(12)
    for sq, sk in ((7, 7), (5, 9), (9, 6)):
        for mask in MASKS:
            if mask == "causal_qend" and sk < sq:
                continue
            q, k, v, do = _rand(rng, sq, 8), _rand(rng, sk, 8), _rand(rng, sk, 8), _rand(rng, sq, 8)
            ref = _autograd_head(q, k, v, do, 0.6, mask)
            rows_q, rows_k = [0, 2, sq - 1], [0, sk // 2, sk - 1]
            for chunk in (1, 3, 64):
                dq, dk, dv = mod.attention_head_backward_rows(q, k, v, do, 0.6, mask, rows_q, rows_k, chunk)
                np.testing.assert_allclose(dq, ref[0][rows_q], rtol=1e-10, atol=1e-12)
                np.testing.assert_allclose(dk, ref[1][rows_k], rtol=1e-10, atol=1e-12)
                np.testing.assert_allclose(dv, ref[2][rows_k], rtol=1e-10, atol=1e-12)


def pin_rows_keyless_rows(mod):
    """Rows that see no key (causal_qend with more queries than keys) get dQ = 0 and give no dK
    or dV; the keys' gradients equal the sums over the rows that see them (autograd on those)."""
    rng = np.random.default_rng(13)
    sq, sk = 9, 4
    q, k, v, do = _rand(rng, sq, 8), _rand(rng, sk, 8), _rand(rng, sk, 8), _rand(rng, sq, 8)
    seen = sq - sk  # rows 0 .. sq - sk - 1 see no key
    dq, dk, dv = mod.attention_head_backward_rows(q, k, v, do, 0.8, "causal_qend", list(range(sq)), list(range(sk)), 2)
    assert np.all(dq[:seen] == 0.0)
    ref = _autograd_head(q[seen:], k, v, do[seen:], 0.8, "causal_qbegin")
    np.testing.assert_allclose(dq[seen:], ref[0], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, ref[1], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, ref[2], rtol=1e-10, atol=1e-12)


def _given_o_head(q, k, v, do, scale, mask, err):
    """Expected gradients when the backward receives O + err instead of the exact O: autograd's
    exact gradients, with delta shifted by d_i = sum_d err_id dO_id.  dS moves by -P_ij d_i, so
    dQ moves by -scale d_i (P K)_i, dK by -scale (P^T diag(d) Q) and dV not at all."""
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64) for x in (q, k, v))
    s = (scale * (tq @ tk.T)).masked_fill(~torch.from_numpy(_visible(q.shape[0], k.shape[0], mask)), float("-inf"))
    p = torch.softmax(s, dim=-1).numpy()
    o = p @ v
    gq, gk, gv = _autograd_head(q, k, v, do, scale, mask)
    d = (err * do).sum(axis=1)
    return o + err, gq - scale * d[:, None] * (p @ k), gk - scale * (p * d[:, None]).T @ q, gv


def pin_given_o(mod):
    """delta from a given O (as a backward pass receives it): the exact O reproduces autograd, and
    a perturbed O moves the gradients by the closed form of _given_o_head, per head, through the
    dense wrapper with a GQA group and through the packed wrapper."""
    rng = np.random.default_rng(14)
    for sq, sk, mask in ((5, 5, "causal_qbegin"), (4, 7, "none"), (6, 6, "causal_qend")):
        q, k, v, do = _rand(rng, sq, 8), _rand(rng, sk, 8), _rand(rng, sk, 8), _rand(rng, sq, 8)
        o_exact, *ref = _given_o_head(q, k, v, do, 0.55, mask, np.zeros((sq, 8)))
        for a, r in zip(mod.attention_head_backward(q, k, v, do, 0.55, mask, o=o_exact), ref):
            np.testing.assert_allclose(a, r, rtol=1e-10, atol=1e-12)
        err = 0.05 * _rand(rng, sq, 8)
        o_pert, *ref = _given_o_head(q, k, v, do, 0.55, mask, err)
        for a, r in zip(mod.attention_head_backward(q, k, v, do, 0.55, mask, o=o_pert), ref):
            np.testing.assert_allclose(a, r, rtol=1e-10, atol=1e-12)
    # dense, H = 4 over H_kv = 2
    B, Sq, Sk, H, H_kv, D = 2, 5, 6, 4, 2, 8
    q, do = _rand(rng, B, Sq, H, D), _rand(rng, B, Sq, H, D)
    k, v = _rand(rng, B, Sk, H_kv, D), _rand(rng, B, Sk, H_kv, D)
    err = 0.05 * _rand(rng, B, Sq, H, D)
    o = np.zeros((B, Sq, H, D))
    eq, ek, ev = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for b in range(B):
        for h in range(H):
            g = h // (H // H_kv)
            o[b, :, h], gq, gk, gv = _given_o_head(q[b, :, h], k[b, :, g], v[b, :, g], do[b, :, h], 0.4, "causal_qend",
                                                   err[b, :, h])
            eq[b, :, h] = gq
            ek[b, :, g] += gk
            ev[b, :, g] += gv
    for a, r in zip(mod.attention_backward_dense(q, k, v, do, 0.4, "causal_qend", o=o), (eq, ek, ev)):
        np.testing.assert_allclose(a, r, rtol=1e-10, atol=1e-12)
    # packed: two sequences whose query and key rows start at different offsets
    cu_q, cu_k, H, H_kv = [0, 3, 7], [0, 5, 8], 2, 1
    q, do = _rand(rng, 7, H, D), _rand(rng, 7, H, D)
    k, v = _rand(rng, 8, H_kv, D), _rand(rng, 8, H_kv, D)
    err = 0.05 * _rand(rng, 7, H, D)
    o = np.zeros(q.shape)
    eq, ek, ev = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for b in range(2):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        for h in range(H):
            o[q0:q1, h], gq, gk, gv = _given_o_head(q[q0:q1, h], k[k0:k1, 0], v[k0:k1, 0], do[q0:q1, h], 0.4, "none",
                                                    err[q0:q1, h])
            eq[q0:q1, h] = gq
            ek[k0:k1, 0] += gk
            ev[k0:k1, 0] += gv
    for a, r in zip(mod.attention_backward_varlen(q, k, v, do, cu_q, cu_k, 0.4, "none", o=o), (eq, ek, ev)):
        np.testing.assert_allclose(a, r, rtol=1e-10, atol=1e-12)


PINS = [pin_autograd, pin_library_sdpa, pin_finite_differences, pin_closed_forms, pin_invariants,
        pin_rows_autograd, pin_rows_keyless_rows, pin_given_o]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_backward_oracle_pin(pin):
    pin(oracle_backward)


# ----------------------------------------------------------------------------------------------
# planted mistakes: a mutated copy of the backward oracle must fail at least one pin
# ----------------------------------------------------------------------------------------------
MUTATIONS = {
    "softmax row term dropped": ("ds = p * (dp - delta[:, None])", "ds = p * dp"),
    "softmax row term sign": ("ds = p * (dp - delta[:, None])", "ds = p * (dp + delta[:, None])"),
    "dV not transposed": ("dv = p.T @ do", "dv = (p @ do) if p.shape[0] == p.shape[1] else p.T @ do"),
    "dK not transposed": ("dk = scale * (ds.T @ q)", "dk = scale * ((ds @ q) if ds.shape[0] == ds.shape[1] else ds.T @ q)"),
    "dQ scale missing": ("dq = scale * (ds @ k)", "dq = ds @ k"),
    "dK scale squared": ("dk = scale * (ds.T @ q)", "dk = scale * scale * (ds.T @ q)"),
    "dP from K": ("dp = do @ v.T", "dp = do @ k.T"),
    "GQA overwrite": ("            dk[b, :, kvh] += gk\n", "            dk[b, :, kvh] = gk\n"),
    "wrong GQA head": ("            kvh = h // group\n            gq, gk, gv = attention_head_backward(q[b, :, h]",
                       "            kvh = h % H_kv\n            gq, gk, gv = attention_head_backward(q[b, :, h]"),
    "rows: softmax row term dropped": ("ds = p * (dp - delta_rows[:, None])", "ds = p * dp"),
    "rows: dV from dS": ("dv_rows += p[:, k_rows].T @ do[r0:r1]", "dv_rows += ds[:, k_rows].T @ do[r0:r1]"),
    "rows: dQ row off by one": ("dq_rows[sel] = scale * (ds[q_rows[sel] - r0] @ k)",
                                "dq_rows[sel] = scale * (ds[q_rows[sel] - r0 - 1] @ k)"),
    "rows: block mask from row 0": ("vis = visible_keys(sq, sk, mask, rows=range(r0, r1))",
                                    "vis = visible_keys(sq, sk, mask, rows=range(0, r1 - r0))"),
    "rows: dK without scale": ("dk_rows += scale * (ds[:, k_rows].T @ q[r0:r1])", "dk_rows += ds[:, k_rows].T @ q[r0:r1]"),
    "given O ignored": ("        delta = sum_o_do(o, do)\n", "        delta = (p * dp).sum(axis=1)\n"),
    "given O without dO": ("        delta = sum_o_do(o, do)\n", "        delta = np.asarray(o).sum(axis=1)\n"),
    "dense: given O of the K/V head": ("None if o is None else o[b, :, h])", "None if o is None else o[b, :, kvh])"),
    "varlen: given O at the key rows": ("None if o is None else o[q0:q1, h])",
                                        "None if o is None else o[k0:k0 + q1 - q0, h])"),
    "varlen key offset": ("gq, gk, gv = attention_head_backward(q[q0:q1, h], k[k0:k1, kvh], v[k0:k1, kvh]",
                          "gq, gk, gv = attention_head_backward(q[q0:q1, h], k[q0:q0 + k1 - k0, kvh], v[k0:k1, kvh]"),
}


def _mutant(name):
    src = open(oracle_backward.__file__).read()
    old, new = MUTATIONS[name]
    assert old in src, f"mutation anchor for {name!r} not found"
    src = src.replace("from .attention import attention_head", "from oracle.attention import attention_head")
    mod = types.ModuleType(f"oracle_backward_mutant_{name.replace(' ', '_')}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_backward_mistake_is_caught(name):
    mod = _mutant(name)
    caught = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutation {name!r} passed every pin"
