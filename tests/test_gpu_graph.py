"""The entry points under HIP graph capture: a call recorded into a graph (torch.cuda.graph on the
caller's stream) and replayed must give the eager call's bits on every replay.

The library launches kernels only (no allocation, no memset, no host synchronisation), so a
call can be captured once its one-time host queries (the compute-unit count, the scratch
array's address) have run eagerly.  Each replay is preceded by other eager GPU work and a
poisoned output, and every replay is checked, not only the last.
"""
import numpy as np
import pytest
import torch

import head_attention_03_amd as fmha
from harness import log
from workloads import make_dense, make_grad, make_varlen, to_bits

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    fmha.load()  # fails loudly when libfmha.so is missing


def _replays_match(name, call, outs):
    """call(stream) launches into outs; eager once, then captured and replayed REPLAYS times."""
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        assert call(stream) == 0
    torch.cuda.synchronize()
    ref = [to_bits(t.cpu()) for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        st = call(stream)
    assert st == 0
    for r in range(REPLAYS):
        junk = torch.randn(1 << 20, device="cuda") * 2.0  # unrelated eager work between replays
        for t in outs:
            t.view(torch.uint8).fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        del junk
        for i, t in enumerate(outs):
            assert np.array_equal(to_bits(t.cpu()), ref[i]), f"{name}: replay {r} output {i} differs from the eager call"
    log(f"[graph] {name}: {REPLAYS} replays bit-identical to the eager call")


def test_fwd_captured():
    inp = make_dense(7000, 2, 700, 900, 8, 2, 128, "bf16", mask="causal_qend")
    dev = torch.device("cuda:0")
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((inp.B, inp.H, inp.Sq), dtype=torch.float32, device=dev)
    _replays_match("fmha_fwd", lambda s: fmha.fmha_fwd(q, k, v, o, lse, inp.B, inp.Sq, inp.Sk, inp.H, inp.H_kv, inp.D,
                                                     inp.kernel_scale, inp.mask, inp.dtype, 1.0, None, s), [o, lse])


def test_fwd_varlen_captured():
    inp = make_varlen(7001, [300, 64, 5], [400, 64, 900], 8, 8, 64, "f16", mask="causal_qend")
    dev = torch.device("cuda:0")
    q, k, v = inp.q_buf.to(dev), inp.k_buf.to(dev), inp.v_buf.to(dev)
    o = inp.new_output_buffer().to(dev)
    cu_q, cu_k = torch.from_numpy(inp.cu_q).to(dev), torch.from_numpy(inp.cu_k).to(dev)
    vl = fmha.make_varlen(cu_q, cu_k, inp.total_q, inp.total_k)
    pq, pk = inp.pad_q, inp.pad_k
    _replays_match("fmha_fwd varlen", lambda s: fmha.fmha_fwd(q[pq:], k[pk:], v[pk:], o[pq:], None, inp.B, inp.max_q,
                                                            inp.max_k, inp.H, inp.H_kv, inp.D, inp.kernel_scale,
                                                            inp.mask, inp.dtype, 1.0, vl, s), [o[pq:]])


def test_splitkv_noalloc_captured():
    # the allocation-free decode entry point: no workspace at all
    inp = make_dense(7002, 4, 1, 4097, 32, 8, 128, "bf16", mask="none")
    dev = torch.device("cuda:0")
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((inp.B, inp.H, inp.Sq), dtype=torch.float32, device=dev)
    _replays_match("fmha_fwd_splitkv_noalloc",
                   lambda s: fmha.fmha_fwd_splitkv_noalloc(q, k, v, o, lse, inp.B, inp.Sq, inp.Sk, inp.H, inp.H_kv,
                                                           inp.D, inp.kernel_scale, inp.mask, inp.dtype, 1.0, None, s),
                   [o, lse])


def test_bwd_captured():
    inp = make_dense(7003, 1, 300, 300, 4, 2, 64, "bf16", mask="causal_qbegin")
    dev = torch.device("cuda:0")
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((inp.B, inp.H, inp.Sq), dtype=torch.float32, device=dev)
    assert fmha.fmha_fwd(q, k, v, o, lse, inp.B, inp.Sq, inp.Sk, inp.H, inp.H_kv, inp.D, inp.kernel_scale, inp.mask,
                         inp.dtype, 1.0, None, torch.cuda.current_stream()) == 0
    do = make_grad(7004, tuple(q.shape), "bf16").to(dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    need = fmha.fmha_bwd_workspace_size(inp.B, inp.Sq, inp.Sk, inp.H, inp.H_kv, inp.D, inp.dtype, None)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    _replays_match("fmha_bwd", lambda s: fmha.fmha_bwd(q, k, v, o, do, lse, dq, dk, dv, inp.B, inp.Sq, inp.Sk, inp.H,
                                                     inp.H_kv, inp.D, inp.kernel_scale, inp.mask, inp.dtype, None, ws,
                                                     need, s), [dq, dk, dv])
