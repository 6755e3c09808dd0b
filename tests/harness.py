"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI, run the oracle.

The HIP side only ever sees device buffers and the C entry point; the oracle side only
ever sees the generator's CPU tensors decoded to fp64.  The two meet in ``compare``.
"""
from __future__ import annotations

import dataclasses
import sys
from typing import Optional

import numpy as np
import torch

import head_attention_03_amd as fmha
import oracle
from workloads import DenseInputs, VarlenInputs, to_bits
from workloads.synth import ELEM_BYTES, TORCH_DTYPES

# Tolerances stated for the method: max-abs error on O (and LSE) for 16-bit types, and on
# the dequantised fp8 output for fp8 (CUTLASS's verification uses 1e-2 / 1e-1).
TOL = {"f16": 1e-2, "bf16": 1e-2, "f8e4m3": 6e-2}
LSE_TOL = 1e-2
# fp8 outputs of the long unmasked workload are small (|0.5 O| ~ 0.1), so the max-abs bound
# alone would pass a kernel that wrote zeros; the relative Frobenius error is checked as well,
# allowing 3 points above the relative error of the best possible e4m3 output.
REL_TOL = {"f8e4m3": 0.03}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


@dataclasses.dataclass
class GpuResult:
    o_bits: np.ndarray  # raw output bits (packed: the whole buffer including the padding)
    lse: Optional[np.ndarray]
    status: int


def _workspace(need: int):
    """Split-KV workspace, filled with NaN bit patterns: no result may depend on its contents."""
    return torch.full((max(need, 16),), 0xFF, dtype=torch.uint8, device=torch.device("cuda:0"))


def _entry(splitkv: bool, varlen, shape):
    """The C entry point to call: fmha_fwd, or fmha_fwd_splitkv with a poisoned workspace."""
    if not splitkv:
        return lambda *a: fmha.fmha_fwd(*a)
    need = fmha.fmha_fwd_splitkv_workspace_size(*shape, varlen)
    assert need > 0, "shape rejected by the split-KV plan"
    ws = _workspace(need)
    return lambda *a: fmha.fmha_fwd_splitkv(*a[:-1], ws, need, a[-1])


def run_dense(inp: DenseInputs, want_lse: bool = False, stream=None, o_init_bits: Optional[int] = None,
              splitkv: bool = False) -> GpuResult:
    dev = torch.device("cuda:0")
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    if o_init_bits is None:
        o = torch.empty_like(q)
    else:
        raw = torch.full(q.shape, o_init_bits, dtype=torch.uint8 if ELEM_BYTES[inp.dtype] == 1 else torch.int16)
        o = raw.view(TORCH_DTYPES[inp.dtype]).to(dev)
    lse = torch.empty((inp.B, inp.H, inp.Sq), dtype=torch.float32, device=dev) if want_lse else None
    call = _entry(splitkv, None, (inp.B, inp.Sq, inp.Sk, inp.H, inp.H_kv, inp.D))
    st = call(q, k, v, o, lse, inp.B, inp.Sq, inp.Sk, inp.H, inp.H_kv, inp.D, inp.kernel_scale, inp.mask,
              inp.dtype, inp.kernel_o_scale, None, stream if stream is not None else torch.cuda.current_stream())
    torch.cuda.synchronize()
    return GpuResult(o_bits=to_bits(o.cpu()), lse=lse.cpu().numpy() if want_lse else None, status=st)


def run_varlen(inp: VarlenInputs, want_lse: bool = False, stream=None, splitkv: bool = False) -> GpuResult:
    dev = torch.device("cuda:0")
    q_buf, k_buf, v_buf = inp.q_buf.to(dev), inp.k_buf.to(dev), inp.v_buf.to(dev)
    o_buf = inp.new_output_buffer().to(dev)
    cu_q = torch.from_numpy(inp.cu_q).to(dev)
    cu_k = torch.from_numpy(inp.cu_k).to(dev)
    lse = torch.empty((inp.H, max(inp.total_q, 1)), dtype=torch.float32, device=dev) if want_lse else None
    vl = fmha.make_varlen(cu_q, cu_k, inp.total_q, inp.total_k)
    call = _entry(splitkv, vl, (inp.B, inp.max_q, inp.max_k, inp.H, inp.H_kv, inp.D))
    st = call(q_buf[inp.pad_q:], k_buf[inp.pad_k:], v_buf[inp.pad_k:], o_buf[inp.pad_q:], lse, inp.B, inp.max_q,
              inp.max_k, inp.H, inp.H_kv, inp.D, inp.kernel_scale, inp.mask, inp.dtype, inp.kernel_o_scale, vl,
              stream if stream is not None else torch.cuda.current_stream())
    torch.cuda.synchronize()
    return GpuResult(o_bits=to_bits(o_buf.cpu()), lse=lse.cpu().numpy()[:, :inp.total_q] if want_lse else None,
                     status=st)


def decoded(inp, which: str) -> np.ndarray:
    """fp64 values of an input tensor, dequantised for fp8."""
    t = getattr(inp, which)
    s = {"q": inp.q_scale, "k": inp.k_scale, "v": inp.v_scale}[which]
    return oracle.decode(to_bits(t), inp.dtype) * s


def oracle_dense(inp: DenseInputs):
    return oracle.attention_dense(decoded(inp, "q"), decoded(inp, "k"), decoded(inp, "v"), inp.scale, inp.mask,
                                  o_scale=inp.o_scale)


def oracle_varlen(inp: VarlenInputs):
    return oracle.attention_varlen(decoded(inp, "q"), decoded(inp, "k"), decoded(inp, "v"), inp.cu_q, inp.cu_k,
                                   inp.scale, inp.mask, o_scale=inp.o_scale)


def _round_to(expected: np.ndarray, dtype: str) -> np.ndarray:
    """Bits of the expected values rounded to the output format (fp8: saturated to +-448)."""
    if dtype == "f8e4m3":
        t = torch.from_numpy(expected.astype(np.float32)).clamp(-448, 448).to(torch.float8_e4m3fn)
    else:
        t = torch.from_numpy(expected.astype(np.float32)).to(TORCH_DTYPES[dtype])
    return to_bits(t)


def output_floor(expected: np.ndarray, dtype: str) -> float:
    """max |round(O) - O|: the error of the best possible output in this format."""
    return float(np.abs(oracle.decode(_round_to(expected, dtype), dtype) - expected).max()) if expected.size else 0.0


def oracle_dense_heads(inp, heads, workers: int = 8):
    """Whole heads [(b, h), ...] of a dense problem from the oracle, several at a time (numpy's
    matmul and exp release the GIL; each head is the oracle's own per-head definition).
    Returns O [n, Sq, D] (times o_scale) and LSE [n, Sq]."""
    from concurrent.futures import ThreadPoolExecutor
    q, k, v = decoded(inp, "q"), decoded(inp, "k"), decoded(inp, "v")
    group = inp.H // inp.H_kv

    def one(bh):
        b, h = bh
        return oracle.attention_head(q[b, :, h], k[b, :, h // group], v[b, :, h // group], inp.scale, inp.mask)

    with ThreadPoolExecutor(max_workers=workers) as ex:
        res = list(ex.map(one, heads))
    return np.stack([r[0] for r in res]) * inp.o_scale, np.stack([r[1] for r in res])


def compare(name: str, got_bits: np.ndarray, dtype: str, expected: np.ndarray, got_lse=None, expected_lse=None,
            tol: Optional[float] = None, plain: bool = False):
    """Element-by-element check of the decoded GPU output against the oracle; returns the max error.

    plain: for fp8, also hold the raw max-abs error (not only the error beyond the best e4m3
    output) to the tolerance; used where |O| is small enough for that bound to be reachable."""
    tol = TOL[dtype] if tol is None else tol
    got = oracle.decode(got_bits, dtype)
    assert got.shape == expected.shape, (got.shape, expected.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite outputs"
    err = float(np.abs(got - expected).max()) if got.size else 0.0
    fl = output_floor(expected, dtype)
    rel = float(np.linalg.norm(got - expected) / max(np.linalg.norm(expected), 1e-30)) if got.size else 0.0
    msg = f"{name}: max|err| {err:.3e} (format floor {fl:.3e}, tol {tol:g}), rel fro {rel:.3e}"
    rel_bound = REL_TOL.get(dtype)
    if dtype == "f8e4m3" and got.size:
        # e4m3 outputs are 0.125 apart at |O| in [1, 2) and carry a 4-5% relative rounding
        # error of their own.  The max-abs bound applies to the error beyond that of the best
        # possible output (the exact O rounded to e4m3), element by element; the relative
        # Frobenius error may exceed the best output's own by REL_TOL (the e4m3 rounding of
        # the probabilities that feed the PV product, which the method prescribes).
        best = oracle.decode(_round_to(expected, dtype), dtype)
        err_beyond = float((np.abs(got - expected) - np.abs(best - expected)).max())
        rel_floor = float(np.linalg.norm(best - expected) / max(np.linalg.norm(expected), 1e-30))
        msg += f", beyond the best e4m3 output {err_beyond:.3e}, best output's rel fro {rel_floor:.3e}"
        if plain:
            assert err <= tol, msg + " (plain max-abs bound)"
        err = err_beyond
        rel_bound = rel_floor + REL_TOL[dtype]
    if got_lse is not None:
        fin = np.isfinite(expected_lse)
        assert np.array_equal(fin, np.isfinite(got_lse)), f"{name}: LSE finiteness differs"
        assert np.all(np.isneginf(got_lse[~fin])), f"{name}: rows without keys must have LSE = -inf"
        lerr = float(np.abs(got_lse[fin] - expected_lse[fin]).max()) if fin.any() else 0.0
        msg += f", lse max|err| {lerr:.3e}"
        assert lerr <= LSE_TOL, msg
    log(msg)
    assert err <= tol, msg
    if rel_bound is not None and got.size:
        assert rel <= rel_bound, msg + f" (relative Frobenius bound {rel_bound:.3e})"
    return err


# ----------------------------------------------------------------------------------------------
# backward (fmha_bwd)
# ----------------------------------------------------------------------------------------------
# Gradient tolerance, relative to the largest |gradient| of the tensor and counted beyond each
# element's own rounding to the output format.  The kernels round P and dS to the 16-bit type for
# the matrix cores and form delta from the 16-bit O; an fp64 emulation of exactly those roundings
# at these shapes stays within 3.1e-3 max|ref| (bf16) and 5e-4 (fp16), and fp32 accumulation adds
# far less, so 1e-2 leaves a factor of three.  Where the exact gradient cancels to 0 (a row with
# one visible key has dP - delta = 0), the scale is taken as 2^-8, the 16-bit rounding of the O(1)
# terms that cancel (delta is formed from the rounded O).
BWD_TOL = 1e-2
BWD_SCALE_FLOOR = 2.0 ** -8
# Sentinel written around packed gradients: the kernels must not touch rows outside the sequences.
GRAD_SENTINEL = {"f16": 0x7BAD, "bf16": 0x4B1D}


def grad_dtype(dtype: str) -> str:
    """Type fmha_bwd writes the gradients in: the input type, bf16 for e4m3 inputs."""
    return "bf16" if dtype == "f8e4m3" else dtype


def oracle_forward_inputs(inp):
    """O (rounded to the input type) and fp32 LSE from the oracle, as the backward's inputs."""
    if isinstance(inp, VarlenInputs):
        o, lse = oracle_varlen(inp)
    else:
        o, lse = oracle_dense(inp)
    o_t = torch.from_numpy(o.astype(np.float32)).to(TORCH_DTYPES[inp.dtype])
    return o_t, lse.astype(np.float32)


def _bwd_workspace(need: int):
    return _workspace(need)


def run_bwd_dense(inp: DenseInputs, do: torch.Tensor, o: torch.Tensor, lse: np.ndarray, stream=None):
    """dQ, dK, dV (CPU tensors) from fmha_bwd; o and lse are the forward's outputs (CPU)."""
    dev = torch.device("cuda:0")
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    o_d, do_d = o.to(dev), do.to(dev)
    lse_d = torch.from_numpy(np.ascontiguousarray(lse, dtype=np.float32)).to(dev)
    gt = TORCH_DTYPES[grad_dtype(inp.dtype)]
    dq, dk, dv = (torch.empty(t.shape, dtype=gt, device=dev) for t in (q, k, v))
    need = fmha.fmha_bwd_workspace_size(inp.B, inp.Sq, inp.Sk, inp.H, inp.H_kv, inp.D, inp.dtype, None)
    ws = _bwd_workspace(need)
    st = fmha.fmha_bwd(q, k, v, o_d, do_d, lse_d, dq, dk, dv, inp.B, inp.Sq, inp.Sk, inp.H, inp.H_kv, inp.D,
                       inp.kernel_scale, inp.mask, inp.dtype, None, ws, need,
                       stream if stream is not None else torch.cuda.current_stream())
    torch.cuda.synchronize()
    return st, dq.cpu(), dk.cpu(), dv.cpu()


def run_bwd_varlen(inp: VarlenInputs, do_buf: torch.Tensor, o: torch.Tensor, lse: np.ndarray):
    """Packed backward.  do_buf holds pad_q leading rows like q_buf; o and lse cover the packed rows.

    Returns the status and the whole dQ, dK, dV buffers (padding included, sentinel-initialised).
    """
    dev = torch.device("cuda:0")
    q_buf, k_buf, v_buf = inp.q_buf.to(dev), inp.k_buf.to(dev), inp.v_buf.to(dev)
    o_buf = torch.zeros_like(inp.q_buf)
    o_buf[inp.pad_q:] = o
    o_buf, do_d = o_buf.to(dev), do_buf.to(dev)
    lse_d = torch.from_numpy(np.ascontiguousarray(lse, dtype=np.float32).reshape(inp.H, -1)).to(dev)
    gd = grad_dtype(inp.dtype)
    bits = GRAD_SENTINEL[gd]
    dq = torch.full(q_buf.shape, bits, dtype=torch.int16).view(TORCH_DTYPES[gd]).to(dev)
    dk = torch.full(k_buf.shape, bits, dtype=torch.int16).view(TORCH_DTYPES[gd]).to(dev)
    dv = torch.full(v_buf.shape, bits, dtype=torch.int16).view(TORCH_DTYPES[gd]).to(dev)
    cu_q = torch.from_numpy(inp.cu_q).to(dev)
    cu_k = torch.from_numpy(inp.cu_k).to(dev)
    vl = fmha.make_varlen(cu_q, cu_k, inp.total_q, inp.total_k)
    need = fmha.fmha_bwd_workspace_size(inp.B, inp.max_q, inp.max_k, inp.H, inp.H_kv, inp.D, inp.dtype, vl)
    ws = _bwd_workspace(need)
    pq, pk = inp.pad_q, inp.pad_k
    st = fmha.fmha_bwd(q_buf[pq:], k_buf[pk:], v_buf[pk:], o_buf[pq:], do_d[pq:], lse_d, dq[pq:], dk[pk:], dv[pk:],
                       inp.B, inp.max_q, inp.max_k, inp.H, inp.H_kv, inp.D, inp.kernel_scale, inp.mask, inp.dtype, vl,
                       ws, need, torch.cuda.current_stream())
    torch.cuda.synchronize()
    return st, dq.cpu(), dk.cpu(), dv.cpu()


def compare_grad(name: str, got: torch.Tensor, dtype: str, expected: np.ndarray, tol: float = BWD_TOL) -> float:
    """Element-by-element check of a gradient against the oracle's fp64 value; returns the error."""
    g = oracle.decode(to_bits(got), dtype)
    assert g.shape == expected.shape, (g.shape, expected.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite gradients"
    if not g.size:
        return 0.0
    best = oracle.decode(_round_to(expected, dtype), dtype)
    beyond = float((np.abs(g - expected) - np.abs(best - expected)).max())
    mx = float(np.abs(expected).max())
    bound = tol * max(mx, BWD_SCALE_FLOOR)
    rel = float(np.linalg.norm(g - expected) / max(np.linalg.norm(expected), 1e-30))
    msg = (f"{name}: max|ref| {mx:.3e}, max|err| beyond the format rounding {beyond:.3e} (bound {bound:.3e}), "
           f"rel fro {rel:.3e}")
    log(msg)
    assert beyond <= bound, msg
    return beyond


# ----------------------------------------------------------------------------------------------
# paged cache (fmha_fwd_splitkv_paged)
# ----------------------------------------------------------------------------------------------
def run_paged(inp, want_lse: bool = True, block_table=None):
    """O bits and LSE of fmha_fwd_splitkv_paged (NaN-filled workspace)."""
    dev = torch.device("cuda:0")
    q, kc, vc = inp.q.to(dev), inp.k_cache.to(dev), inp.v_cache.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((inp.B, inp.H, inp.Sq), dtype=torch.float32, device=dev) if want_lse else None
    bt = torch.from_numpy(np.ascontiguousarray(inp.block_table if block_table is None else block_table)).to(dev)
    sl = torch.from_numpy(inp.seqlens_k).to(dev)
    pk = fmha.make_paged_kv(bt, sl, bt.shape[1], inp.page_size, inp.num_pages, inp.kv_dtype or inp.dtype)
    need = fmha.fmha_fwd_splitkv_workspace_size(inp.B, inp.Sq, inp.Sk, inp.H, inp.H_kv, inp.D, None)
    ws = _workspace(need)
    st = fmha.fmha_fwd_splitkv_paged(q, kc, vc, o, lse, inp.B, inp.Sq, inp.Sk, inp.H, inp.H_kv, inp.D,
                                     inp.kernel_scale, inp.mask, inp.dtype, inp.kernel_o_scale, pk, ws, need,
                                     torch.cuda.current_stream())
    torch.cuda.synchronize()
    return GpuResult(o_bits=to_bits(o.cpu()), lse=lse.cpu().numpy() if want_lse else None, status=st)


def oracle_paged(inp, block_table=None, k_cache=None):
    kvt = inp.kv_dtype or inp.dtype
    kc = oracle.decode(to_bits(inp.k_cache if k_cache is None else k_cache), kvt) * inp.k_scale
    vc = oracle.decode(to_bits(inp.v_cache), kvt) * inp.v_scale
    if k_cache is not None and kc.shape[0] > vc.shape[0]:
        vc = np.concatenate([vc, np.zeros((kc.shape[0] - vc.shape[0],) + vc.shape[1:])])
    q = oracle.decode(to_bits(inp.q), inp.dtype) * inp.q_scale
    bt = inp.block_table if block_table is None else block_table
    return oracle.attention_paged(q, kc, vc, bt, inp.seqlens_k, inp.scale, inp.mask, o_scale=inp.o_scale)
