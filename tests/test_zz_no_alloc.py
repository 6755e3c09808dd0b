"""fmha_fwd_splitkv_noalloc (library-owned scratch) against fmha_fwd_splitkv (caller workspace) on an
MI355X: the same kernels and split plan, so the outputs must be bit-identical, and both within the
oracle's tolerance.  Calls in a row, the later ones smaller, so that a result depending on what an
earlier call left in the shared scratch would show."""
import numpy as np
import pytest
import torch

import head_attention_03_amd as fmha
from harness import compare, log, oracle_dense, oracle_varlen, run_dense, run_varlen
from workloads import make_dense, make_varlen, to_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    fmha.load()


def _noalloc_dense(inp):
    dev = torch.device("cuda:0")
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((inp.B, inp.H, inp.Sq), dtype=torch.float32, device=dev)
    st = fmha.fmha_fwd_splitkv_noalloc(q, k, v, o, lse, inp.B, inp.Sq, inp.Sk, inp.H, inp.H_kv, inp.D,
                                       inp.kernel_scale, inp.mask, inp.dtype, inp.kernel_o_scale, None,
                                       torch.cuda.current_stream())
    torch.cuda.synchronize()
    return st, to_bits(o.cpu()), lse.cpu().numpy()


def _noalloc_varlen(inp):
    dev = torch.device("cuda:0")
    q_buf, k_buf, v_buf = inp.q_buf.to(dev), inp.k_buf.to(dev), inp.v_buf.to(dev)
    o_buf = inp.new_output_buffer().to(dev)
    cu_q, cu_k = torch.from_numpy(inp.cu_q).to(dev), torch.from_numpy(inp.cu_k).to(dev)
    lse = torch.empty((inp.H, max(inp.total_q, 1)), dtype=torch.float32, device=dev)
    vl = fmha.make_varlen(cu_q, cu_k, inp.total_q, inp.total_k)
    st = fmha.fmha_fwd_splitkv_noalloc(q_buf[inp.pad_q:], k_buf[inp.pad_k:], v_buf[inp.pad_k:], o_buf[inp.pad_q:], lse,
                                       inp.B, inp.max_q, inp.max_k, inp.H, inp.H_kv, inp.D, inp.kernel_scale, inp.mask,
                                       inp.dtype, inp.kernel_o_scale, vl, torch.cuda.current_stream())
    torch.cuda.synchronize()
    return st, to_bits(o_buf.cpu()), lse.cpu().numpy()[:, :inp.total_q]


def test_noalloc_matches_caller_workspace_in_a_row():
    cases = [
        ("dense bf16 GQA 8x4 rows vs 3000 keys", make_dense(3100, 8, 4, 3000, 32, 8, 128, "bf16", mask="causal_qend")),
        ("dense f16 3x2 rows vs 700 keys (smaller)", make_dense(3101, 3, 2, 700, 8, 2, 64, "f16", mask="none")),
        ("packed bf16 (smaller still)", make_varlen(3102, [3, 1, 2], [500, 40, 1200], 4, 2, 32, "bf16",
                                                    mask="causal_qbegin")),
    ]
    for name, inp in cases:
        log(f"[case] noalloc {name}")
        packed = hasattr(inp, "cu_q")
        st, o_bits, lse = _noalloc_varlen(inp) if packed else _noalloc_dense(inp)
        assert st == 0, fmha.fmha_status_string(st)
        ref = run_varlen(inp, want_lse=True, splitkv=True) if packed else run_dense(inp, want_lse=True, splitkv=True)
        assert ref.status == 0
        assert np.array_equal(o_bits, ref.o_bits), f"{name}: O differs from the caller-workspace entry point"
        assert np.array_equal(lse, ref.lse), f"{name}: LSE differs from the caller-workspace entry point"
        if packed:
            o_exp, lse_exp = oracle_varlen(inp)
            compare(f"noalloc {name}", o_bits[inp.pad_q:], inp.dtype, o_exp, lse, lse_exp)
        else:
            o_exp, lse_exp = oracle_dense(inp)
            compare(f"noalloc {name}", o_bits, inp.dtype, o_exp, lse, lse_exp)


def test_noalloc_too_large_is_refused_without_launch():
    # more partials than the 32 MiB scratch: refused before anything is enqueued
    big = (64, 16, 8192, 64, 8, 128)
    assert fmha.fmha_fwd_splitkv_workspace_size(*big) > 32 << 20
    P = 0x10000
    assert fmha.fmha_fwd_splitkv_noalloc(P, P, P, P, None, *big, 0.1, "none", "bf16", 1.0, None, None) == 7
