"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on an MI355X.

Every case is compared element by element.  At full size the prefill (B=4, H=16, 2048²) and
fp8 (B=8, H=16, 4096²) and long-context GQA (B=2, H=32/8, 8192²) workloads are compared
whole.  Shapes span several q- and k-tiles with
ragged tails; the packed-batch shapes follow the CUTLASS example's test list (zero-length
sequences, tiny and non-divisible lengths, both causal alignments).
"""
import numpy as np
import pytest
import torch

import oracle
from harness import (TOL, compare, decoded, log, oracle_dense, oracle_dense_heads, oracle_varlen, run_dense,
                     run_varlen)
from workloads import make_config, make_dense, make_dense_sink, make_varlen, to_bits
from workloads.synth import O_SENTINEL_BITS

pytestmark = pytest.mark.gpu

MASKS = ("none", "residual", "causal_qbegin", "causal_qend")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import head_attention_03_amd as fmha
    fmha.load()  # fails loudly when libfmha.so is missing


def _dense_case(name, inp, want_lse=True):
    log(f"[case] {name} dtype={inp.dtype} B={inp.B} Sq={inp.Sq} Sk={inp.Sk} H={inp.H} H_kv={inp.H_kv} D={inp.D} "
        f"mask={inp.mask} seed={inp.seed}")
    res = run_dense(inp, want_lse=want_lse)
    assert res.status == 0
    o, lse = oracle_dense(inp)
    compare(name, res.o_bits, inp.dtype, o, res.lse, lse if want_lse else None)
    return res


def test_config1_tiny():
    _dense_case("config 1", make_config(1))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("mask", MASKS)
def test_dense_masks_dims(dtype, D, mask):
    inp = make_dense(2000 + D, 2, 200, 333, 4, 2, D, dtype, mask=mask)
    _dense_case(f"dense {dtype} D{D} {mask}", inp)


@pytest.mark.parametrize("want_lse", [True, False], ids=["lse", "nolse"])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("mask", MASKS)
def test_fp8_masks_dims(D, mask, want_lse):
    # without an LSE the kernel forms the probabilities from their fp32 bit pattern, with one
    # exact v_exp_f32 per score
    inp = make_dense(2400 + D, 2, 200, 333, 4, 2, D, "f8e4m3", mask=mask, o_scale=0.5)
    _dense_case(f"dense fp8 D{D} {mask} lse={want_lse}", inp, want_lse=want_lse)


@pytest.mark.parametrize("want_lse", [True, False], ids=["lse", "nolse"])
@pytest.mark.parametrize("sink_logit,mask", [(6.0, "none"), (9.0, "none"), (12.0, "none"), (9.0, "causal_qend")])
def test_fp8_attention_sink(sink_logit, mask, want_lse):
    # One key per row scores sink_logit nats above the rest, so much of a 4096-key row's
    # weight lies 9-20 binades below its maximum, among the e4m3 subnormals of P.
    # Probabilities that drop those weights (an e4m3 code linear in x, clipped at the
    # smallest normal) miss the tolerance here: a CPU model of them errs by ~0.16 against 0.06.
    inp = make_dense_sink(2470, 1, 64, 4096, 2, 2, 128, "f8e4m3", sink_logit, mask=mask, o_scale=0.5)
    _dense_case(f"fp8 sink {sink_logit} {mask} lse={want_lse}", inp, want_lse=want_lse)


def test_fp8_gqa_more_queries_than_keys():
    inp = make_dense(2450, 1, 333, 200, 4, 1, 128, "f8e4m3", mask="causal_qend", o_scale=0.5)
    _dense_case("fp8 MQA Sq>Sk causal_qend", inp)


@pytest.mark.parametrize("mask", ["causal_qbegin", "causal_qend", "none"])
def test_more_queries_than_keys(mask):
    # under causal-qend the first Sq - Sk rows see no key: O = 0, LSE = -inf
    inp = make_dense(2101, 1, 333, 200, 2, 2, 64, "bf16", mask=mask)
    _dense_case(f"Sq>Sk {mask}", inp)


@pytest.mark.parametrize("shape", [
    dict(B=1, H=1, H_kv=1, Sq=1013, Sk=1024, D=128, mask="causal_qend", dtype="f16"),
    dict(B=2, H=4, H_kv=4, Sq=512, Sk=512, D=64, mask="none", dtype="f16"),
    dict(B=2, H=4, H_kv=2, Sq=512, Sk=512, D=64, mask="causal_qbegin", dtype="bf16"),
    dict(B=1, H=4, H_kv=4, Sq=512, Sk=512, D=128, mask="residual", dtype="bf16"),
    dict(B=1, H=3, H_kv=1, Sq=77, Sk=1, D=64, mask="none", dtype="bf16"),
    dict(B=3, H=2, H_kv=2, Sq=1, Sk=129, D=128, mask="causal_qend", dtype="f16"),
    dict(B=1, H=2, H_kv=2, Sq=64, Sk=64, D=32, mask="causal_qbegin", dtype="f16"),
])
def test_edge_shapes(shape):
    s = dict(shape)
    inp = make_dense(2200, s.pop("B"), s.pop("Sq"), s.pop("Sk"), s.pop("H"), s.pop("H_kv"), s.pop("D"),
                     s.pop("dtype"), mask=s.pop("mask"))
    _dense_case(f"edge {shape}", inp)


def test_no_keys_gives_zero_and_neg_inf():
    inp = make_dense(2300, 1, 70, 0, 2, 2, 64, "f16", mask="none")
    res = run_dense(inp, want_lse=True)
    assert res.status == 0
    assert not oracle.decode(res.o_bits, "f16").any()
    assert np.all(np.isneginf(res.lse))


def test_gqa_equals_mha_with_repeated_heads():
    inp = make_dense(2400, 2, 300, 300, 8, 2, 128, "bf16", mask="causal_qbegin")
    rep = make_dense(2400, 2, 300, 300, 8, 2, 128, "bf16", mask="causal_qbegin")
    rep.k = inp.k.repeat_interleave(4, dim=2).contiguous()
    rep.v = inp.v.repeat_interleave(4, dim=2).contiguous()
    rep.H_kv = 8
    a, b = run_dense(inp, want_lse=True), run_dense(rep, want_lse=True)
    assert np.array_equal(a.o_bits, b.o_bits) and np.array_equal(a.lse, b.lse)


def test_mqa():
    _dense_case("mqa", make_dense(2450, 1, 257, 190, 6, 1, 64, "f16", mask="causal_qend"))


def test_bitwise_repeatable():
    inp = make_dense(2500, 2, 700, 900, 4, 4, 128, "bf16", mask="causal_qend")
    runs = [run_dense(inp, want_lse=True) for _ in range(3)]
    for r in runs[1:]:
        assert np.array_equal(r.o_bits, runs[0].o_bits) and np.array_equal(r.lse, runs[0].lse)


# ----------------------------------------------------------------------------------------------
# several q-tiles per workgroup: enough (sequence, head, q-tile) items that every workgroup runs
# two or more of them as one K/V stream (item changes, one- and two-tile items, ragged tiles)
# ----------------------------------------------------------------------------------------------
def _items_per_workgroup(B, H, Sq, mask, Sk=0, H_kv=1, D=128, esz=2, total_q=None):
    """The launch rule of the library: q-tiles of 256 rows, about one workgroup per compute unit,
    at most 8 per workgroup, pairs when causal; then, when B*H is a multiple of 8, the largest
    halving (down to 2) at which the K/V heads that an XCD's resident workgroups stream fit 4 MiB.
    Packed batches of at most 64 sequences (total_q given) count their q-tiles as at most
    total_q // 256 + B instead of B times the longest sequence's."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n_qt = (Sq + 255) // 256
    causal = mask.startswith("causal")
    qt_all = B * n_qt
    if total_q is not None and B <= 64:
        qt_all = min(qt_all, total_q // 256 + B)
    ipw = max(1, min(8, H * qt_all // cus, n_qt))
    if causal and ipw > 1:
        ipw &= ~1
    if (B * H) % 8 == 0 and ipw > 2:
        per_xcd, xcd_per, group = max(1, cus // 8), B * H // 8, H // H_kv
        w = ipw
        while w >= 2:
            we = w & ~1 if causal else w
            heads = min(xcd_per, -(-per_xcd // -(-n_qt // we)))
            if -(-heads // group) * 2 * Sk * D * esz <= 4 << 20:
                ipw = we
                break
            w //= 2
    return ipw


MULTI_ITEM = [
    # (B, Sq, Sk, H, H_kv, D, dtype, mask)
    (1, 1000, 1000, 128, 128, 64, "bf16", "causal_qbegin"),   # heavy/light pairs, ragged last q-tile
    (2, 1024, 50, 128, 32, 128, "f16", "causal_qend"),        # one-tile items (rows without keys too)
    (1, 1024, 100, 256, 64, 64, "bf16", "residual"),          # two-tile items: every step special
    (1, 1030, 230, 256, 256, 32, "f16", "causal_qbegin"),     # four-tile items, D 32
    (1, 1100, 300, 128, 8, 128, "bf16", "none"),              # five q-tiles: a lone last item
]


@pytest.mark.parametrize("case", MULTI_ITEM, ids=lambda c: f"S{c[1]}x{c[2]}-H{c[3]}/{c[4]}-D{c[5]}-{c[6]}-{c[7]}")
def test_several_qtiles_per_workgroup(case):
    B, Sq, Sk, H, H_kv, D, dtype, mask = case
    ipw = _items_per_workgroup(B, H, Sq, mask, Sk, H_kv, D, 1 if dtype == "f8e4m3" else 2)
    log(f"[multi-item] {ipw} q-tiles per workgroup")
    assert ipw >= 2, "the case no longer covers several q-tiles per workgroup"
    _dense_case(f"multi-item {case}", make_dense(2900 + Sq + Sk, B, Sq, Sk, H, H_kv, D, dtype, mask=mask))


@pytest.mark.parametrize("D", [32, 128])
@pytest.mark.parametrize("mask", ["none", "causal_qend"])
def test_several_qtiles_per_workgroup_fp8(mask, D):
    assert _items_per_workgroup(1, 128, 1100, mask, 300, 16, D, 1) >= 2
    inp = make_dense(2950 + D, 1, 1100, 300, 128, 16, D, "f8e4m3", mask=mask, o_scale=0.5)
    _dense_case(f"multi-item fp8 D{D} {mask}", inp)
    _dense_case(f"multi-item fp8 D{D} {mask} (no LSE)", inp, want_lse=False)


def test_several_qtiles_per_workgroup_repeatable():
    inp = make_dense(2960, 1, 1000, 700, 128, 32, 128, "bf16", mask="causal_qend")
    assert _items_per_workgroup(1, 128, 1000, "causal_qend", 700, 32, 128) >= 2
    runs = [run_dense(inp, want_lse=True) for _ in range(2)]
    assert np.array_equal(runs[1].o_bits, runs[0].o_bits) and np.array_equal(runs[1].lse, runs[0].lse)


# ----------------------------------------------------------------------------------------------
# packed variable-length batches
# ----------------------------------------------------------------------------------------------
def _varlen_case(name, inp, want_lse=True):
    log(f"[case] {name} dtype={inp.dtype} seqlens_q={inp.seqlens_q.tolist()} seqlens_k={inp.seqlens_k.tolist()} "
        f"H={inp.H} H_kv={inp.H_kv} D={inp.D} mask={inp.mask} seed={inp.seed}")
    res = run_varlen(inp, want_lse=want_lse)
    assert res.status == 0
    o, lse = oracle_varlen(inp)
    compare(name, res.o_bits[inp.pad_q:], inp.dtype, o, res.lse, lse if want_lse else None)
    # the leading padding of O is never written
    assert np.all(res.o_bits[:inp.pad_q] == O_SENTINEL_BITS[inp.dtype]), f"{name}: O padding was written"
    return res


@pytest.mark.parametrize("mask", ["residual", "causal_qend"])
def test_config4_varlen(mask):
    _varlen_case(f"config 4 {mask}", make_config(4, mask=mask))


CMAKE_VARLEN = [
    ([128], [128], 8, 4, 128, "none"),
    ([256, 256, 256, 256], [256, 768, 512, 512], 4, 4, 128, "none"),
    ([256, 256, 256, 256], [256, 0, 1280, 512], 4, 2, 64, "residual"),
    ([256, 0, 512, 256], [256, 256, 512, 256], 4, 2, 64, "none"),
    ([3, 2], [2, 5], 2, 2, 64, "none"),
    ([17, 10], [13, 10], 2, 1, 128, "causal_qend"),
    ([1], [1], 1, 1, 64, "causal_qbegin"),
    ([177, 845], [257, 766], 4, 4, 128, "none"),
    ([17], [257], 2, 2, 128, "causal_qbegin"),
    ([17], [257], 2, 2, 128, "causal_qend"),
    ([1013], [1024], 2, 2, 64, "causal_qend"),
    ([1024], [1035], 2, 2, 32, "causal_qend"),
]


@pytest.mark.parametrize("case", CMAKE_VARLEN, ids=lambda c: f"q{c[0]}-k{c[1]}-{c[5]}-D{c[4]}")
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_varlen_shapes(case, dtype):
    lq, lk, H, H_kv, D, mask = case
    _varlen_case(f"varlen {lq}/{lk}", make_varlen(2600, lq, lk, H, H_kv, D, dtype, mask=mask))


@pytest.mark.parametrize("case", CMAKE_VARLEN, ids=lambda c: f"q{c[0]}-k{c[1]}-{c[5]}-D{c[4]}")
def test_varlen_shapes_fp8(case):
    lq, lk, H, H_kv, D, mask = case
    _varlen_case(f"varlen fp8 {lq}/{lk}", make_varlen(2650, lq, lk, H, H_kv, D, "f8e4m3", mask=mask, o_scale=0.5))


# fp8 tiles hold 128 keys: key lengths on either side of one and two tiles, with every mask that
# ends a sequence inside a tile (the ragged tail, the causal diagonal aligned to the last key)
FP8_TILE_EDGES = [
    ([130, 128, 127, 256, 300, 1], [127, 128, 129, 255, 256, 257], 4, 2, 128, "residual"),
    ([127, 128, 129, 255, 256, 257], [127, 128, 129, 255, 256, 257], 4, 4, 64, "causal_qend"),
    ([64, 200, 129], [129, 255, 385], 2, 1, 128, "causal_qbegin"),
]


@pytest.mark.parametrize("case", FP8_TILE_EDGES, ids=lambda c: f"k{c[1]}-{c[5]}-D{c[4]}")
def test_varlen_fp8_key_tile_edges(case):
    lq, lk, H, H_kv, D, mask = case
    inp = make_varlen(2680 + len(lk), lq, lk, H, H_kv, D, "f8e4m3", mask=mask, o_scale=0.5)
    _varlen_case(f"varlen fp8 tile edges {lq}/{lk}", inp)
    # without an LSE the probabilities come from the fp32 bit pattern of 2^x
    _varlen_case(f"varlen fp8 tile edges {lq}/{lk} (no LSE)", inp, want_lse=False)


def test_varlen_poisoned_padding_never_read_fp8():
    inp = make_varlen(2750, [100, 37, 250], [90, 300, 5], 4, 2, 128, "f8e4m3", mask="causal_qend", poison_pads=True)
    _varlen_case("varlen fp8 NaN pads", inp)


def test_varlen_poisoned_padding_never_read():
    inp = make_varlen(2700, [100, 37, 250], [90, 300, 5], 4, 2, 64, "bf16", mask="causal_qend", poison_pads=True)
    _varlen_case("varlen NaN pads", inp)


def test_varlen_several_qtiles_per_workgroup():
    # q-tiles per sequence from 0 to 4 under one launch rule (4 per workgroup): workgroups of the
    # short sequences run fewer items, or none; the sequences are taken longest first
    lq = [1000, 300, 64, 1, 0, 513, 777, 256]
    lk = [900, 310, 64, 1, 5, 600, 1000, 40]
    inp = make_varlen(2970, lq, lk, 128, 16, 64, "bf16", mask="causal_qend", poison_pads=True)
    assert _items_per_workgroup(len(lq), 128, max(lq), "causal_qend", max(lk), 16, 64, 2, sum(lq)) >= 2
    _varlen_case("varlen multi-item", inp)


def test_varlen_ranked_several_qtiles_without_xcd_groups():
    # the longest-first order with four q-tiles per workgroup (pairs of heavy and light tiles)
    # and B*H not a multiple of 8 (pairs dealt in plain order, not per XCD)
    lq, lk, H, H_kv = [700, 1024, 300], [900, 1024, 1500], 170, 17
    assert (len(lq) * H) % 8 != 0
    assert _items_per_workgroup(len(lq), H, max(lq), "causal_qend", max(lk), H_kv, 64, 2, sum(lq)) >= 2
    inp = make_varlen(2980, lq, lk, H, H_kv, 64, "f16", mask="causal_qend")
    _varlen_case("varlen ranked, several q-tiles, plain order", inp)


@pytest.mark.parametrize("n_seq", [64, 65])
def test_varlen_many_sequences(n_seq):
    # up to 64 sequences the kernel takes them in the order of their key counts (ties in batch
    # order), past 64 in batch order: both work orders, with ties, empty and one-row sequences
    rng = np.random.default_rng(2990 + n_seq)
    lq = [int(x) for x in rng.integers(0, 600, size=n_seq)]
    lk = [int(x) for x in rng.choice([0, 1, 64, 300, 300, 700, 1500], size=n_seq)]
    lq[0], lq[1] = 1, 0
    inp = make_varlen(2990 + n_seq, lq, lk, 4, 2, 64, "bf16", mask="causal_qend")
    _varlen_case(f"varlen {n_seq} sequences", inp)


def test_varlen_equals_dense_runs():
    lq, lk = [130, 64, 7], [200, 64, 300]
    inp = make_varlen(2800, lq, lk, 4, 2, 128, "bf16", mask="causal_qend")
    packed = run_varlen(inp, want_lse=False)
    for b in range(3):
        qs = slice(int(inp.cu_q[b]), int(inp.cu_q[b + 1]))
        ks = slice(int(inp.cu_k[b]), int(inp.cu_k[b + 1]))
        dense = make_dense(0, 1, lq[b], lk[b], 4, 2, 128, "bf16", mask="causal_qend")
        dense.q = inp.q[qs].unsqueeze(0).contiguous()
        dense.k = inp.k[ks].unsqueeze(0).contiguous()
        dense.v = inp.v[ks].unsqueeze(0).contiguous()
        one = run_dense(dense)
        assert np.array_equal(packed.o_bits[inp.pad_q + qs.start:inp.pad_q + qs.stop], one.o_bits[0])


# ----------------------------------------------------------------------------------------------
# full-size configurations, in the launch configuration the benchmark times
# ----------------------------------------------------------------------------------------------
def _full_size_run(config_id, want_lse):
    inp = make_config(config_id)
    log(f"[case] full config {config_id}: {inp.dtype} B={inp.B} S={inp.Sq} H={inp.H}/{inp.H_kv} D={inp.D} "
        f"{inp.mask} lse={want_lse} seed={inp.seed}")
    res = run_dense(inp, want_lse=want_lse)
    assert res.status == 0
    return inp, res


@pytest.mark.parametrize("config_id", [2, 5])
def test_full_size_config_whole(config_id):
    # prefill bf16 (with LSE) and fp8: every output element against the oracle.  fp8 outputs are
    # small here (|0.5 O| < 0.12), so the plain max-abs bound holds next to the one counted
    # beyond the best e4m3 output.
    want_lse = config_id == 2
    inp, res = _full_size_run(config_id, want_lse)
    heads = [(b, h) for b in range(inp.B) for h in range(inp.H)]
    o_exp, lse_exp = oracle_dense_heads(inp, heads)  # [B*H, Sq, D]
    got = np.stack([res.o_bits[b, :, h] for b, h in heads])
    got_lse = np.stack([res.lse[b, h] for b, h in heads]) if want_lse else None
    compare(f"config {config_id} whole ({len(heads)} heads)", got, inp.dtype, o_exp, got_lse,
            lse_exp if want_lse else None, plain=True)


def test_full_size_config3_whole():
    # long-context GQA: all 64 (sequence, head) pairs, 8192 rows each, every output element, in
    # four chunks of 16 heads (four whole GQA groups each) so that progress shows
    inp, res = _full_size_run(3, False)
    heads = [(b, h) for b in range(inp.B) for h in range(inp.H)]
    for c in range(0, len(heads), 16):
        part = heads[c:c + 16]
        o_exp, _ = oracle_dense_heads(inp, part)
        got = np.stack([res.o_bits[b, :, h] for b, h in part])
        compare(f"config 3 heads {c}..{c + len(part) - 1} of {len(heads)}", got, inp.dtype, o_exp)


# ----------------------------------------------------------------------------------------------
# negative control: an oracle with a planted mistake must disagree with the HIP path
# ----------------------------------------------------------------------------------------------
def test_fp8_check_rejects_a_dropped_key_tile():
    # the fp8 bound is loose at these output magnitudes; an oracle that drops the last 64
    # keys must still fail the combined max-abs / relative-Frobenius check
    inp = make_dense(2950, 1, 512, 1024, 2, 2, 128, "f8e4m3", mask="none", o_scale=0.5)
    res = run_dense(inp)
    assert res.status == 0
    q, k, v = decoded(inp, "q"), decoded(inp, "k"), decoded(inp, "v")
    wrong, _ = oracle.attention_dense(q, k[:, :-64], v[:, :-64], inp.scale, "none", o_scale=inp.o_scale)
    right, _ = oracle.attention_dense(q, k, v, inp.scale, "none", o_scale=inp.o_scale)
    compare("fp8 reference", res.o_bits, "f8e4m3", right)
    with pytest.raises(AssertionError):
        compare("fp8 against a dropped key tile", res.o_bits, "f8e4m3", wrong)


def test_planted_oracle_mistake_is_detected():
    inp = make_dense(2900, 1, 256, 256, 2, 2, 64, "f16", mask="causal_qbegin")
    res = run_dense(inp)
    q, k, v = decoded(inp, "q"), decoded(inp, "k"), decoded(inp, "v")
    # diagonal dropped: query i sees only keys j < i
    wrong = np.zeros_like(q)
    for h in range(2):
        s = inp.scale * q[0, :, h] @ k[0, :, h].T
        vis = np.tril(np.ones((256, 256), bool), -1)
        vis[0, 0] = True
        e = np.where(vis, np.exp(s - np.where(vis, s, -np.inf).max(1, keepdims=True)), 0)
        wrong[0, :, h] = (e / e.sum(1, keepdims=True)) @ v[0, :, h]
    err = np.abs(oracle.decode(res.o_bits, "f16") - wrong).max()
    assert err > 10 * TOL["f16"], err


# ----------------------------------------------------------------------------------------------
# sequences whose tensors exceed 32-bit byte offsets (descriptors rebased per q-tile and per K/V
# tile window); inputs drawn on the device, rows checked one at a time against the oracle
# ----------------------------------------------------------------------------------------------
def _long_rows_case(name, inp, picks):
    dev = torch.device("cuda:0")
    log(f"[case] {name}: B={inp.B} Sq={inp.Sq} Sk={inp.Sk} H={inp.H}/{inp.H_kv} D={inp.D} {inp.mask} "
        f"seed={inp.seed} ({inp.k.numel() * inp.k.element_size() / 2**30:.2f} GiB per K/V tensor)")
    o = torch.empty_like(inp.q)
    lse = torch.empty((inp.B, inp.H, inp.Sq), dtype=torch.float32, device=dev)
    import head_attention_03_amd as fmha
    st = fmha.fmha_fwd(inp.q, inp.k, inp.v, o, lse, inp.B, inp.Sq, inp.Sk, inp.H, inp.H_kv, inp.D, inp.kernel_scale,
                       inp.mask, inp.dtype, 1.0, None, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert st == 0, fmha.fmha_status_string(st)
    group = inp.H // inp.H_kv
    heads = sorted({h for _, h, _ in picks})
    got, exp_o, got_lse, exp_lse = [], [], [], []
    for h in heads:  # the oracle reads back exactly the stored values of one head at a time
        rows = [(b, i) for b, hh, i in picks if hh == h]
        kvh = h // group
        k_h = oracle.decode(to_bits(inp.k[:, :, kvh:kvh + 1].cpu()), inp.dtype)
        v_h = oracle.decode(to_bits(inp.v[:, :, kvh:kvh + 1].cpu()), inp.dtype)
        q_h = oracle.decode(to_bits(inp.q[:, :, h:h + 1].cpu()), inp.dtype)
        o_rows, l_rows = oracle.attention_rows(q_h, k_h, v_h, inp.scale, inp.mask, [(b, 0, i) for b, i in rows])
        exp_o.append(o_rows)
        exp_lse.append(l_rows)
        got.append(np.stack([to_bits(o[b, i, h].cpu()) for b, i in rows]))
        got_lse.append(np.array([float(lse[b, h, i]) for b, i in rows]))
        del k_h, v_h, q_h
    compare(f"{name} ({sum(len(x) for x in got)} rows)", np.concatenate(got), inp.dtype, np.concatenate(exp_o),
            np.concatenate(got_lse), np.concatenate(exp_lse))


def test_long_prefill_131072_keys():
    # B=1, H=64, D=128, 131072 queries and keys: 2 GiB per tensor, 4 MiB rows of all heads
    from workloads import make_dense_on_device
    inp = make_dense_on_device(3300, 1, 131072, 131072, 64, 64, 128, "bf16", mask="causal_qbegin")
    S = inp.Sq
    rng = np.random.default_rng(3300)
    rows = [0, 1, 255, 256, 65535, 65536, S - 257, S - 256, S - 2, S - 1] + [int(x) for x in rng.integers(0, S, 6)]
    picks = [(0, h, i) for h in (0, 37, 63) for i in rows]
    _long_rows_case("long prefill 131072", inp, picks)
    del inp
    torch.cuda.empty_cache()


def test_keys_beyond_4gib_per_tensor():
    # 270336 keys x 64 heads x D 128 (4.1 GiB per K/V tensor): K/V offsets past 2^32, reached
    # by rows aligned to the last key
    from workloads import make_dense_on_device
    inp = make_dense_on_device(3301, 1, 1000, 270336, 64, 64, 128, "f16", mask="causal_qend")
    rng = np.random.default_rng(3301)
    rows = [0, 1, 255, 256, 511, 512, 998, 999] + [int(x) for x in rng.integers(0, 1000, 4)]
    picks = [(0, h, i) for h in (1, 62) for i in rows]
    _long_rows_case("keys beyond 4 GiB", inp, picks)
    del inp
    torch.cuda.empty_cache()
