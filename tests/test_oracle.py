"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Brute force, a library routine, closed forms, invariants, and planted mistakes
that the pins must catch.  CPU only.
"""
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oracle_attention
from workloads import make_dense, make_varlen, to_bits

MASKS = ("none", "residual", "causal_qbegin", "causal_qend")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------------------------
# format decoders
# ----------------------------------------------------------------------------------------------
def test_decode_every_code_matches_library_casts():
    codes16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode(codes16, "f16")
    lib = codes16.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    assert np.array_equal(ours[~np.isnan(ours)], lib[~np.isnan(lib)])

    ours = oracle.decode(codes16, "bf16")
    lib = torch.from_numpy(codes16.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    assert np.array_equal(ours[~np.isnan(ours)], lib[~np.isnan(lib)])

    codes8 = np.arange(256, dtype=np.uint8)
    ours = oracle.decode(codes8, "f8e4m3")
    lib = torch.from_numpy(codes8.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    assert np.array_equal(ours[~np.isnan(ours)], lib[~np.isnan(lib)])


def test_decode_values_fixed_by_the_format_definitions():
    e4 = lambda c: float(oracle.decode(np.array([c], np.uint8), "f8e4m3")[0])  # noqa: E731
    assert e4(0x38) == 1.0 and e4(0xB8) == -1.0
    assert e4(0x7E) == 448.0  # largest finite e4m3fn
    assert math.isnan(e4(0x7F)) and math.isnan(e4(0xFF))
    assert e4(0x08) == 2.0 ** -6  # smallest normal
    assert e4(0x01) == 2.0 ** -9  # smallest subnormal
    assert e4(0x78) == 256.0
    bf = lambda c: float(oracle.decode(np.array([c], np.uint16), "bf16")[0])  # noqa: E731
    assert bf(0x3F80) == 1.0 and bf(0xC000) == -2.0 and bf(0x7F80) == math.inf
    h = lambda c: float(oracle.decode(np.array([c], np.uint16), "f16")[0])  # noqa: E731
    assert h(0x3C00) == 1.0 and h(0x7BFF) == 65504.0 and h(0x0001) == 2.0 ** -24


# ----------------------------------------------------------------------------------------------
# the pins, written against a module so that planted mistakes can be run through them
# ----------------------------------------------------------------------------------------------
def _bf_visible(mask, sq, sk):
    if mask == "causal_qbegin":
        return lambda i, j: not (j > i)
    if mask == "causal_qend":
        return lambda i, j: not (j > i + sk - sq)
    return lambda i, j: True


def _brute_force(q, k, v, scale, mask):
    """Pure-Python loops: weights exp(scale * q.k) over visible keys divided by their sum (no max shift)."""
    sq, sk, d = len(q), len(k), len(q[0])
    vis = _bf_visible(mask, sq, sk)
    out, lses = [], []
    for i in range(sq):
        w = []
        for j in range(sk):
            if vis(i, j):
                dot = 0.0
                for a in range(d):
                    dot += q[i][a] * k[j][a]
                w.append((j, math.exp(scale * dot)))
        if not w:
            out.append([0.0] * d)
            lses.append(-math.inf)
            continue
        z = sum(x for _, x in w)
        out.append([sum(x * v[j][a] for j, x in w) / z for a in range(d)])
        lses.append(math.log(z))
    return np.array(out, dtype=np.float64).reshape(sq, d), np.array(lses)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def pin_brute_force(mod):
    rng = np.random.default_rng(7)
    # dense, every mask, GQA (H=4, H_kv=2), Sq < Sk, Sq > Sk, Sq == Sk
    for sq, sk in [(5, 5), (3, 7), (7, 3), (1, 6), (6, 1), (4, 8)]:
        B, H, H_kv, D = 2, 4, 2, 5
        q, k, v = _rand(rng, B, sq, H, D), _rand(rng, B, sk, H_kv, D), _rand(rng, B, sk, H_kv, D)
        for mask in MASKS:
            o, lse = mod.attention_dense(q, k, v, 0.37, mask)
            for b in range(B):
                for h in range(H):
                    kvh = h // (H // H_kv)
                    ob, lb = _brute_force(q[b, :, h].tolist(), k[b, :, kvh].tolist(), v[b, :, kvh].tolist(), 0.37, mask)
                    np.testing.assert_allclose(o[b, :, h], ob, rtol=1e-12, atol=1e-12)
                    np.testing.assert_allclose(lse[b, h], lb, rtol=1e-12, atol=1e-12)
    # packed sequences including an empty one
    lq, lk = [3, 0, 5, 2], [4, 3, 5, 1]
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    H, H_kv, D = 2, 1, 4
    q, k, v = _rand(rng, cu_q[-1], H, D), _rand(rng, cu_k[-1], H_kv, D), _rand(rng, cu_k[-1], H_kv, D)
    for mask in MASKS:
        o, lse = mod.attention_varlen(q, k, v, cu_q, cu_k, 0.5, mask)
        for b in range(4):
            for h in range(H):
                qs, ks = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
                if lq[b] == 0:
                    continue
                ob, lb = _brute_force(q[qs, h].tolist(), k[ks, 0].tolist(), v[ks, 0].tolist(), 0.5, mask)
                np.testing.assert_allclose(o[qs, h], ob, rtol=1e-12, atol=1e-12)
                np.testing.assert_allclose(lse[h, qs], lb, rtol=1e-12, atol=1e-12)


def pin_library_sdpa(mod):
    rng = np.random.default_rng(11)
    B, H, H_kv, D = 2, 4, 2, 16
    for sq, sk in [(33, 33), (17, 40), (40, 17)]:
        q, k, v = _rand(rng, B, sq, H, D), _rand(rng, B, sk, H_kv, D), _rand(rng, B, sk, H_kv, D)
        tq = torch.from_numpy(q).permute(0, 2, 1, 3)
        tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(H // H_kv, dim=1)
        tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(H // H_kv, dim=1)
        sdpa = torch.nn.functional.scaled_dot_product_attention
        ref_none = sdpa(tq, tk, tv, scale=0.3).permute(0, 2, 1, 3).numpy()
        o, _ = mod.attention_dense(q, k, v, 0.3, "none")
        np.testing.assert_allclose(o, ref_none, rtol=1e-10, atol=1e-12)
        if sq <= sk:  # torch's is_causal is aligned to the first key; rows without keys are NaN in torch
            ref_causal = sdpa(tq, tk, tv, scale=0.3, is_causal=True).permute(0, 2, 1, 3).numpy()
            o, _ = mod.attention_dense(q, k, v, 0.3, "causal_qbegin")
            np.testing.assert_allclose(o, ref_causal, rtol=1e-10, atol=1e-12)
        if sq <= sk:
            allowed = torch.ones(sq, sk, dtype=torch.bool).tril(diagonal=sk - sq)
            ref_qend = sdpa(tq, tk, tv, scale=0.3, attn_mask=allowed).permute(0, 2, 1, 3).numpy()
            o, _ = mod.attention_dense(q, k, v, 0.3, "causal_qend")
            np.testing.assert_allclose(o, ref_qend, rtol=1e-10, atol=1e-12)
        # LSE from the library: logsumexp of the scaled scores
        s = torch.einsum("bhid,bhjd->bhij", tq, tk) * 0.3
        _, lse = mod.attention_dense(q, k, v, 0.3, "none")
        np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


def pin_closed_forms(mod):
    rng = np.random.default_rng(5)
    D = 8
    # one key: O = V[0], LSE = scale * q.k0
    q, k, v = _rand(rng, 1, 6, 2, D), _rand(rng, 1, 1, 2, D), _rand(rng, 1, 1, 2, D)
    for mask in ("none", "residual", "causal_qbegin"):
        o, lse = mod.attention_dense(q, k, v, 0.7, mask)
        assert np.array_equal(o, np.broadcast_to(v[:, :1], o.shape)), mask
        np.testing.assert_allclose(lse, 0.7 * np.einsum("bihd,bhd->bhi", q, k[:, 0]), rtol=1e-13)
    # causal-qend with one key: only the last query row sees it
    o, lse = mod.attention_dense(q, k, v, 0.7, "causal_qend")
    assert np.array_equal(o[:, -1], v[:, 0]) and not o[:, :-1].any()
    assert np.all(np.isneginf(lse[:, :, :-1]))
    # constant V rows
    q, k = _rand(rng, 1, 9, 2, D), _rand(rng, 1, 12, 2, D)
    c = _rand(rng, D)
    v = np.broadcast_to(c, (1, 12, 2, D)).copy()
    for mask in MASKS:
        o, _ = mod.attention_dense(q, k, v, 0.4, mask)
        rows = np.ones(9, bool) if mask != "causal_qend" else np.arange(9) + 3 >= 0
        np.testing.assert_allclose(o[0, rows], np.broadcast_to(c, o[0, rows].shape), rtol=1e-13, atol=1e-14)
    # causal-qbegin row 0 is V[0] exactly
    q, k, v = _rand(rng, 2, 7, 3, D), _rand(rng, 2, 10, 3, D), _rand(rng, 2, 10, 3, D)
    o, lse = mod.attention_dense(q, k, v, 0.9, "causal_qbegin")
    assert np.array_equal(o[:, 0], v[:, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.9 * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0]), rtol=1e-13)
    # Q = 0: uniform weights over the visible keys
    sq, sk = 6, 9
    q = np.zeros((1, sq, 1, D))
    k, v = _rand(rng, 1, sk, 1, D), _rand(rng, 1, sk, 1, D)
    for mask in MASKS:
        o, lse = mod.attention_dense(q, k, v, 1.3, mask)
        for i in range(sq):
            n = {"causal_qbegin": i + 1, "causal_qend": i + 1 + sk - sq}.get(mask, sk)
            np.testing.assert_allclose(o[0, i, 0], v[0, :n, 0].mean(axis=0), rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(lse[0, 0, i], math.log(n), rtol=1e-13)
    # Q = K = ones: every score is scale * D
    q, k = np.ones((1, sq, 1, D)), np.ones((1, sk, 1, D))
    for mask in MASKS:
        _, lse = mod.attention_dense(q, k, v, 0.25, mask)
        for i in range(sq):
            n = {"causal_qbegin": i + 1, "causal_qend": i + 1 + sk - sq}.get(mask, sk)
            np.testing.assert_allclose(lse[0, 0, i], 0.25 * D + math.log(n), rtol=1e-13)


def pin_invariants(mod):
    rng = np.random.default_rng(3)
    D = 6
    for sq, sk in [(8, 8), (5, 11), (11, 5)]:
        q, k, v = _rand(rng, sq, D), _rand(rng, sk, D), _rand(rng, sk, D)
        for mask in MASKS:
            o, lse, s, p = mod.attention_head(q, k, v, 0.6, mask, return_p=True)
            has = np.isfinite(lse)
            np.testing.assert_allclose(p[has].sum(axis=1), 1.0, rtol=1e-13)
            seen = np.array([[_bf_visible(mask, sq, sk)(i, j) for j in range(sk)] for i in range(sq)])
            # sum over the visible keys of exp(S - LSE) is 1
            np.testing.assert_allclose(np.where(seen, np.exp(s - np.where(has, lse, 0.0)[:, None]), 0.0)[has].sum(axis=1),
                                       1.0, rtol=1e-12)
            assert np.array_equal(has, seen.any(axis=1))
            # masked positions carry exactly zero weight, so changing K/V there leaves O bit-identical
            for i in range(sq):
                hidden = [j for j in range(sk) if not _bf_visible(mask, sq, sk)(i, j)]
                if hidden:
                    assert np.all(p[i, hidden] == 0.0)
            k2, v2 = k.copy(), v.copy()
            cols_hidden_for_all = [j for j in range(sk) if all(not _bf_visible(mask, sq, sk)(i, j) for i in range(sq))]
            k2[cols_hidden_for_all] = 1e3
            v2[cols_hidden_for_all] = -7e5
            o2, lse2 = mod.attention_head(q, k2, v2, 0.6, mask)
            assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    # permutation of keys together with their values (no mask)
    q, k, v = _rand(rng, 7, D), _rand(rng, 13, D), _rand(rng, 13, D)
    perm = rng.permutation(13)
    o1, l1 = mod.attention_head(q, k, v, 0.8, "none")
    o2, l2 = mod.attention_head(q, k[perm], v[perm], 0.8, "none")
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)
    # GQA == MHA with repeated K/V heads
    B, sq, sk, H, H_kv = 2, 5, 7, 6, 2
    q, k, v = _rand(rng, B, sq, H, D), _rand(rng, B, sk, H_kv, D), _rand(rng, B, sk, H_kv, D)
    for mask in MASKS:
        o1, l1 = mod.attention_dense(q, k, v, 0.5, mask)
        o2, l2 = mod.attention_dense(q, np.repeat(k, H // H_kv, axis=2), np.repeat(v, H // H_kv, axis=2), 0.5, mask)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # causal-qend == causal-qbegin when Sq == Sk
    q, k, v = _rand(rng, 1, 9, 2, D), _rand(rng, 1, 9, 2, D), _rand(rng, 1, 9, 2, D)
    a, la = mod.attention_dense(q, k, v, 0.5, "causal_qend")
    b, lb = mod.attention_dense(q, k, v, 0.5, "causal_qbegin")
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    # packed batch == per-sequence dense runs
    lq, lk = [4, 7, 1], [9, 3, 6]
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    q, k, v = _rand(rng, cu_q[-1], 2, D), _rand(rng, cu_k[-1], 1, D), _rand(rng, cu_k[-1], 1, D)
    for mask in MASKS:
        o, lse = mod.attention_varlen(q, k, v, cu_q, cu_k, 0.5, mask)
        for bi in range(3):
            qs, ks = slice(cu_q[bi], cu_q[bi + 1]), slice(cu_k[bi], cu_k[bi + 1])
            od, ld = mod.attention_dense(q[None, qs], k[None, ks], v[None, ks], 0.5, mask)
            assert np.array_equal(o[qs], od[0]) and np.array_equal(lse[:, qs], ld[0])
    # selected rows == full result
    B, sq, sk, H, H_kv = 2, 6, 9, 4, 2
    q, k, v = _rand(rng, B, sq, H, D), _rand(rng, B, sk, H_kv, D), _rand(rng, B, sk, H_kv, D)
    picks = [(0, 0, 0), (1, 3, 5), (0, 2, 3), (1, 1, 1)]
    for mask in MASKS:
        o, lse = mod.attention_dense(q, k, v, 0.5, mask, o_scale=0.5)
        orow, lrow = mod.attention_rows(q, k, v, 0.5, mask, picks, o_scale=0.5)
        for n, (b, h, i) in enumerate(picks):
            np.testing.assert_allclose(orow[n], o[b, i, h], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(lrow[n], lse[b, h, i], rtol=1e-12)
    # selected rows of a packed batch == the packed result
    lq, lk = [4, 7, 2], [9, 3, 6]
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    q, k, v = _rand(rng, cu_q[-1], 4, D), _rand(rng, cu_k[-1], 2, D), _rand(rng, cu_k[-1], 2, D)
    picks = [(0, 0, 3), (1, 3, 6), (2, 1, 0), (1, 2, 2), (2, 0, 1)]
    for mask in MASKS:
        o, lse = mod.attention_varlen(q, k, v, cu_q, cu_k, 0.5, mask)
        orow, lrow = mod.attention_rows(q, k, v, 0.5, mask, picks, cu_q=cu_q, cu_k=cu_k)
        for n, (b, h, i) in enumerate(picks):
            np.testing.assert_allclose(orow[n], o[cu_q[b] + i, h], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(lrow[n], lse[h, cu_q[b] + i], rtol=1e-12)


PINS = [pin_brute_force, pin_library_sdpa, pin_closed_forms, pin_invariants]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle_attention)


# ----------------------------------------------------------------------------------------------
# planted mistakes: a mutated copy of the oracle must fail at least one pin
# ----------------------------------------------------------------------------------------------
MUTATIONS = {
    "diagonal dropped": ("        return j <= i\n", "        return j < i\n"),
    "qend offset flipped": ("return j <= i + (sk - sq)", "return j <= i - (sk - sq)"),
    "wrong GQA head": ("kvh = h // group", "kvh = h % H_kv"),
    "scale missing": ("s = scale * (q @ k.T)", "s = q @ k.T"),
    "transposed scores": ("s = scale * (q @ k.T)", "s = scale * (q @ k.T).T if q.shape[0] == k.shape[0] else scale * (q @ k.T)"),
    "masked keys keep weight": ("e = np.where(vis, np.exp(np.where(vis, s, 0.0) - m[:, None]), 0.0)",
                                "e = np.exp(np.where(vis, s, 0.0) - m[:, None])"),
    "lse without max": ("lse[has_key] = m[has_key] + np.log(den[has_key])", "lse[has_key] = np.log(den[has_key])"),
    "varlen key offset": ("kk, vv = k[k0:k1, kvh], v[k0:k1, kvh]", "kk, vv = k[q0:q0 + sk, kvh], v[q0:q0 + sk, kvh]"),
    "o_scale dropped": ("return o_scale * o, lse\n\n\ndef attention_varlen", "return o, lse\n\n\ndef attention_varlen"),
}


def _mutant(name):
    src = open(oracle_attention.__file__).read()
    old, new = MUTATIONS[name]
    assert old in src, f"mutation anchor for {name!r} not found"
    mod = types.ModuleType(f"oracle_mutant_{name.replace(' ', '_')}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(name)
    caught = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutation {name!r} passed every pin"


# ----------------------------------------------------------------------------------------------
# FLOP convention against the numbers printed on the sm120 article
# ----------------------------------------------------------------------------------------------
def test_flop_convention_reproduces_printed_tflops():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "sm120_benchmark.txt")) if ln.strip() and ln[0] != "#"]
    assert len(rows) == 10
    for seq, _impl, ms, tflops in rows:
        S = int(seq)
        inp = types.SimpleNamespace(B=1, H=32, Sq=S, Sk=S, D=128, mask="causal_qbegin")
        from workloads.synth import DenseInputs
        flops = DenseInputs.flops(inp)
        assert round(flops / (float(ms) * 1e-3) / 1e12, 2) == float(tflops)


# ----------------------------------------------------------------------------------------------
# the oracle on generator output: fp8 dequantisation stays within the e4m3 rounding bound
# ----------------------------------------------------------------------------------------------
def test_fp8_inputs_dequantise_within_rounding_bound():
    inp = make_dense(99, 1, 64, 64, 2, 2, 32, "f8e4m3")
    rng = np.random.default_rng(99)
    x = rng.standard_normal(size=(1, 64, 2, 32), dtype=np.float32).astype(np.float64)
    xhat = oracle.decode(to_bits(inp.q), "f8e4m3") * inp.q_scale
    # e4m3 keeps 3 mantissa bits: relative error <= 2^-4 for normals, absolute <= 2^-10 * s below 2^-6 * s
    bound = np.maximum(np.abs(x) * 2.0 ** -4, inp.q_scale * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(np.abs(xhat - x) <= bound)
    assert np.abs(xhat).max() <= 448 * inp.q_scale * (1 + 1e-12)


def test_varlen_oracle_on_generator_output():
    inp = make_varlen(5, [3, 0, 70], [40, 5, 65], 2, 1, 16, "f16", mask="causal_qend")
    q = oracle.decode(to_bits(inp.q), "f16")
    k = oracle.decode(to_bits(inp.k), "f16")
    v = oracle.decode(to_bits(inp.v), "f16")
    o, lse = oracle.attention_varlen(q, k, v, inp.cu_q, inp.cu_k, inp.scale, inp.mask)
    assert o.shape == (73, 2, 16) and lse.shape == (2, 73)
    # sequence 2 has Sq=70 > Sk=65 under causal-qend: its first 5 rows see no key
    assert not o[3:8].any() and np.all(np.isneginf(lse[:, 3:8]))
    assert np.all(np.isfinite(lse[:, 8:]))
