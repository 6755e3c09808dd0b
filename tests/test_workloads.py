"""The seeded input generator: determinism, shapes, lengths, padding.  CPU only."""
import numpy as np
import torch

from workloads import CONFIGS, make_config, make_dense, make_varlen, to_bits
from workloads.synth import O_SENTINEL_BITS


def test_same_seed_same_bits():
    a = make_dense(42, 2, 33, 47, 4, 2, 64, "bf16", mask="causal_qend")
    b = make_dense(42, 2, 33, 47, 4, 2, 64, "bf16", mask="causal_qend")
    c = make_dense(43, 2, 33, 47, 4, 2, 64, "bf16", mask="causal_qend")
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        assert np.array_equal(to_bits(x), to_bits(y))
    assert not np.array_equal(to_bits(a.q), to_bits(c.q))
    assert a.q.shape == (2, 33, 4, 64) and a.k.shape == (2, 47, 2, 64) and a.q.dtype == torch.bfloat16


def test_draw_order_q_then_k_then_v():
    inp = make_dense(9, 1, 5, 6, 2, 1, 32, "f16")
    rng = np.random.default_rng(9)
    q = rng.standard_normal(size=(1, 5, 2, 32), dtype=np.float32)
    k = rng.standard_normal(size=(1, 6, 1, 32), dtype=np.float32)
    v = rng.standard_normal(size=(1, 6, 1, 32), dtype=np.float32)
    assert np.array_equal(to_bits(inp.q), to_bits(torch.from_numpy(q).half()))
    assert np.array_equal(to_bits(inp.k), to_bits(torch.from_numpy(k).half()))
    assert np.array_equal(to_bits(inp.v), to_bits(torch.from_numpy(v).half()))


def test_varlen_config_lengths_and_offsets():
    inp = make_config(4)
    c = CONFIGS[4]
    assert inp.B == 8
    assert np.all((inp.seqlens_q >= c["sq_lo"]) & (inp.seqlens_q <= c["sq_hi"]))
    extra = inp.seqlens_k - inp.seqlens_q
    assert np.all((extra >= 0) & (extra <= c["sk_extra_hi"]))
    assert inp.cu_q[0] == 0 and np.all(np.diff(inp.cu_q) == inp.seqlens_q)
    assert inp.cu_k.dtype == np.int32 and inp.cu_k[-1] == inp.total_k
    assert inp.pad_q == inp.max_q and inp.pad_k == inp.max_k
    assert inp.q_buf.shape == (inp.pad_q + inp.total_q, 16, 64)
    assert inp.k.shape == (inp.total_k, 16, 64)
    # the same seed re-draws the same lengths
    assert np.array_equal(make_config(4).seqlens_k, inp.seqlens_k)


def test_output_buffer_sentinel_and_poisoned_pads():
    inp = make_varlen(3, [5, 0, 9], [7, 2, 4], 2, 2, 32, "bf16", poison_pads=True)
    o = inp.new_output_buffer()
    assert o.shape == (9 + 14, 2, 32)
    assert np.all(to_bits(o) == O_SENTINEL_BITS["bf16"])
    assert torch.isnan(inp.q_buf[: inp.pad_q].float()).all()
    assert torch.isfinite(inp.q.float()).all() and torch.isfinite(inp.k.float()).all()


def test_fp8_scales_are_folded_for_the_kernel():
    inp = make_dense(77, 1, 16, 16, 2, 2, 128, "f8e4m3", o_scale=0.5)
    assert inp.q.dtype == torch.float8_e4m3fn
    assert abs(inp.kernel_scale - inp.scale * inp.q_scale * inp.k_scale) < 1e-15
    assert abs(inp.kernel_o_scale - 0.5 * inp.v_scale) < 1e-15
    assert float(inp.q.float().abs().max()) == 448.0  # amax maps onto the largest finite code
