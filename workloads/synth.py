"""Seeded synthetic Q/K/V for the attention forward pass (no attention arithmetic here).

Recipe (the same for the HIP path's tests, the benchmark and the CPU oracle):

* one ``numpy.random.default_rng(seed)`` (PCG64) stream per workload;
* for packed variable-length batches the per-sequence lengths are drawn first,
  then Q, then K, then V;
* every tensor is a full ``standard_normal`` draw in float32, converted to the
  storage type by torch's CPU round-to-nearest-even cast (fp16 / bf16);
* fp8 tensors are quantised per tensor: ``s = amax|x| / 448`` and
  ``x_q = e4m3fn(x / s)`` (torch's CPU cast, round to nearest even); the caller
  folds the scales into the softmax scale and the output scale;
* a packed batch has one leading padding sequence of valid but unused memory in
  front of Q, K, V and O (``max_seqlen`` rows each); device pointers are passed
  past it.  The O padding holds a sentinel bit pattern, the input padding holds
  random values (or NaN when ``poison_pads`` is set).

Tensors are returned on the CPU; callers move them to the device.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

TORCH_DTYPES = {
    "f16": torch.float16,
    "bf16": torch.bfloat16,
    "f8e4m3": torch.float8_e4m3fn,
}
ELEM_BYTES = {"f16": 2, "bf16": 2, "f8e4m3": 1}
E4M3_MAX = 448.0
# Bit patterns written into the output padding; a kernel that writes outside its rows changes them.
O_SENTINEL_BITS = {"f16": 0x7BAD, "bf16": 0x4B1D, "f8e4m3": 0x5A}


def config_seed(config_id: int) -> int:
    return 1000 + int(config_id)


def draw_normal(rng: np.random.Generator, shape: Sequence[int]) -> np.ndarray:
    """i.i.d. N(0, 1) in float32, drawn in C order."""
    return rng.standard_normal(size=tuple(int(s) for s in shape), dtype=np.float32)


def quantize_e4m3(x: torch.Tensor):
    """Per-tensor e4m3fn quantisation: returns (codes as float8_e4m3fn, dequantisation scale)."""
    amax = float(x.abs().max()) if x.numel() else 0.0
    s = amax / E4M3_MAX if amax > 0.0 else 1.0
    q = (x.to(torch.float32) / s).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q, s


def _to_storage(x32: np.ndarray, dtype: str):
    t = torch.from_numpy(x32)
    if dtype == "f8e4m3":
        return quantize_e4m3(t)
    return t.to(TORCH_DTYPES[dtype]), 1.0


def to_bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage bits of a CPU tensor as an unsigned numpy array (uint8 or uint16)."""
    t = t.detach().cpu().contiguous()
    if t.element_size() == 1:
        return t.view(torch.uint8).numpy()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.element_size() == 4:
        return t.view(torch.int32).numpy().view(np.uint32)
    raise TypeError(f"unsupported element size {t.element_size()}")


@dataclasses.dataclass
class DenseInputs:
    q: torch.Tensor  # [B, Sq, H, D]
    k: torch.Tensor  # [B, Sk, H_kv, D]
    v: torch.Tensor  # [B, Sk, H_kv, D]
    B: int
    Sq: int
    Sk: int
    H: int
    H_kv: int
    D: int
    dtype: str
    mask: str
    scale: float  # softmax scale in terms of the real (dequantised) values
    o_scale: float  # multiplier applied to O before the output conversion
    seed: int
    q_scale: float = 1.0  # fp8 dequantisation scales (1.0 otherwise)
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def kernel_scale(self) -> float:
        """Softmax scale handed to the kernel, with the fp8 input scales folded in."""
        return self.scale * self.q_scale * self.k_scale

    @property
    def kernel_o_scale(self) -> float:
        return self.o_scale * self.v_scale

    def flops(self) -> float:
        """4*B*H*Sq*Sk*D, halved for the causal masks (the convention of the pages' benchmark)."""
        f = 4.0 * self.B * self.H * self.Sq * self.Sk * self.D
        return f / 2 if self.mask.startswith("causal") else f


@dataclasses.dataclass
class VarlenInputs:
    q_buf: torch.Tensor  # [pad_q + total_q, H, D]; rows [pad_q, ...) are the packed sequences
    k_buf: torch.Tensor  # [pad_k + total_k, H_kv, D]
    v_buf: torch.Tensor
    seqlens_q: np.ndarray  # int64 [B]
    seqlens_k: np.ndarray
    cu_q: np.ndarray  # int32 [B + 1], cu[0] = 0
    cu_k: np.ndarray
    pad_q: int
    pad_k: int
    H: int
    H_kv: int
    D: int
    dtype: str
    mask: str
    scale: float
    o_scale: float
    seed: int
    q_scale: float = 1.0
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def B(self) -> int:
        return len(self.seqlens_q)

    @property
    def total_q(self) -> int:
        return int(self.cu_q[-1])

    @property
    def total_k(self) -> int:
        return int(self.cu_k[-1])

    @property
    def max_q(self) -> int:
        return int(self.seqlens_q.max()) if self.B else 0

    @property
    def max_k(self) -> int:
        return int(self.seqlens_k.max()) if self.B else 0

    @property
    def q(self) -> torch.Tensor:
        return self.q_buf[self.pad_q:]

    @property
    def k(self) -> torch.Tensor:
        return self.k_buf[self.pad_k:]

    @property
    def v(self) -> torch.Tensor:
        return self.v_buf[self.pad_k:]

    @property
    def kernel_scale(self) -> float:
        return self.scale * self.q_scale * self.k_scale

    @property
    def kernel_o_scale(self) -> float:
        return self.o_scale * self.v_scale

    def new_output_buffer(self) -> torch.Tensor:
        """O buffer with its own leading padding, every element set to the sentinel bits."""
        rows = self.pad_q + self.total_q
        bits = O_SENTINEL_BITS[self.dtype]
        if ELEM_BYTES[self.dtype] == 1:
            raw = torch.full((rows, self.H, self.D), bits, dtype=torch.uint8)
        else:
            raw = torch.full((rows, self.H, self.D), bits, dtype=torch.int16)
        return raw.view(TORCH_DTYPES[self.dtype])

    def flops_convention(self) -> float:
        f = 4.0 * self.H * self.D * float(np.sum(self.seqlens_q.astype(np.float64) * self.seqlens_k))
        return f / 2 if self.mask.startswith("causal") else f

    def flops_exact(self) -> float:
        """4*H*D times the number of (query, key) pairs the mask keeps."""
        pairs = 0
        for sq, sk in zip(self.seqlens_q.tolist(), self.seqlens_k.tolist()):
            if self.mask == "causal_qbegin":
                pairs += sum(min(sk, i + 1) for i in range(sq))
            elif self.mask == "causal_qend":
                off = sk - sq
                pairs += sum(max(0, min(sk, i + off + 1)) for i in range(sq))
            else:
                pairs += sq * sk
        return 4.0 * self.H * self.D * pairs


def _dense_from_rng(rng, B, Sq, Sk, H, H_kv, D, dtype):
    q, sq = _to_storage(draw_normal(rng, (B, Sq, H, D)), dtype)
    k, sk = _to_storage(draw_normal(rng, (B, Sk, H_kv, D)), dtype)
    v, sv = _to_storage(draw_normal(rng, (B, Sk, H_kv, D)), dtype)
    return q, k, v, sq, sk, sv


def make_dense(seed: int, B: int, Sq: int, Sk: int, H: int, H_kv: int, D: int, dtype: str,
               mask: str = "none", scale: Optional[float] = None, o_scale: float = 1.0) -> DenseInputs:
    rng = np.random.default_rng(seed)
    q, k, v, sq, sk, sv = _dense_from_rng(rng, B, Sq, Sk, H, H_kv, D, dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return DenseInputs(q=q, k=k, v=v, B=B, Sq=Sq, Sk=Sk, H=H, H_kv=H_kv, D=D, dtype=dtype, mask=mask,
                       scale=float(scale), o_scale=float(o_scale), seed=seed, q_scale=sq, k_scale=sk, v_scale=sv)


def make_dense_sink(seed: int, B: int, Sq: int, Sk: int, H: int, H_kv: int, D: int, dtype: str,
                    sink_logit: float, mask: str = "none", o_scale: float = 1.0) -> DenseInputs:
    """Dense inputs with an attention sink: key 0 of every sequence and K/V head scores about
    ``sink_logit`` (natural-log units, at scale 1/sqrt(D)) above the other keys for every query,
    so most of a long row's weights sit many binades below its maximum.  Q, K, V are drawn as in
    ``make_dense`` (N(0, 1), order Q, K, V); then dim 0 of every query is raised by 4 and dim 0 of
    key 0 is set to sink_logit sqrt(D) / 4, before the conversion to the storage type."""
    rng = np.random.default_rng(seed)
    q = draw_normal(rng, (B, Sq, H, D))
    k = draw_normal(rng, (B, Sk, H_kv, D))
    v = draw_normal(rng, (B, Sk, H_kv, D))
    q[..., 0] += 4.0
    if Sk > 0:
        k[:, 0, :, 0] = sink_logit * math.sqrt(D) / 4.0
    (q, sq), (k, sk), (v, sv) = (_to_storage(x, dtype) for x in (q, k, v))
    return DenseInputs(q=q, k=k, v=v, B=B, Sq=Sq, Sk=Sk, H=H, H_kv=H_kv, D=D, dtype=dtype, mask=mask,
                       scale=1.0 / math.sqrt(D), o_scale=float(o_scale), seed=seed, q_scale=sq, k_scale=sk,
                       v_scale=sv)


def make_dense_on_device(seed: int, B: int, Sq: int, Sk: int, H: int, H_kv: int, D: int, dtype: str,
                         mask: str = "none", device="cuda:0") -> DenseInputs:
    """Dense 16-bit inputs too large to draw on the host in reasonable time (gigabytes per tensor):
    i.i.d. N(0, 1) drawn in float32 by torch's seeded generator on ``device`` (Philox, in the
    order Q, K, V), rounded to the storage type (round to nearest even), and left on the device.
    A different stream from ``make_dense`` for the same seed; the tests read back the exact stored
    values of the rows they check."""
    if dtype not in ("f16", "bf16"):
        raise ValueError("device-drawn inputs are 16-bit")
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))

    def draw(shape):
        out = torch.empty(shape, dtype=TORCH_DTYPES[dtype], device=device)
        rows = max(1, (1 << 28) // max(1, int(np.prod(shape[2:])) * shape[0]))  # ~1 GiB of float32 at a time
        for r0 in range(0, shape[1], rows):
            r1 = min(shape[1], r0 + rows)
            out[:, r0:r1] = torch.randn((shape[0], r1 - r0) + tuple(shape[2:]), generator=g, device=device,
                                        dtype=torch.float32).to(TORCH_DTYPES[dtype])
        return out

    q = draw((B, Sq, H, D))
    k = draw((B, Sk, H_kv, D))
    v = draw((B, Sk, H_kv, D))
    return DenseInputs(q=q, k=k, v=v, B=B, Sq=Sq, Sk=Sk, H=H, H_kv=H_kv, D=D, dtype=dtype, mask=mask,
                       scale=1.0 / math.sqrt(D), o_scale=1.0, seed=seed)


def make_grad(seed: int, shape: Sequence[int], dtype: str) -> torch.Tensor:
    """Upstream gradient dO for the backward pass: N(0, 1) float32 from its own stream, cast to dtype."""
    t, _ = _to_storage(draw_normal(np.random.default_rng(seed), shape), dtype)
    return t


def make_grad_on_device(seed: int, shape: Sequence[int], dtype: str, device="cuda:0") -> torch.Tensor:
    """Upstream gradient dO too large to draw on the host: N(0, 1) drawn in float32 by torch's seeded
    generator on ``device`` (Philox), a row block at a time, rounded to the 16-bit storage type."""
    if dtype not in ("f16", "bf16"):
        raise ValueError("device-drawn gradients are 16-bit")
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    out = torch.empty(tuple(shape), dtype=TORCH_DTYPES[dtype], device=device)
    rows = max(1, (1 << 28) // max(1, int(np.prod(shape[2:])) * shape[0]))
    for r0 in range(0, shape[1], rows):
        r1 = min(shape[1], r0 + rows)
        out[:, r0:r1] = torch.randn((shape[0], r1 - r0) + tuple(shape[2:]), generator=g, device=device,
                                    dtype=torch.float32).to(TORCH_DTYPES[dtype])
    return out


@dataclasses.dataclass
class PagedInputs:
    q: torch.Tensor        # [B, Sq, H, D]
    k_cache: torch.Tensor  # [num_pages, page_size, H_kv, D]
    v_cache: torch.Tensor
    block_table: np.ndarray  # int32 [B, max_pages_per_seq]; unused entries -1
    seqlens_k: np.ndarray    # int32 [B]
    page_size: int
    B: int
    Sq: int
    H: int
    H_kv: int
    D: int
    dtype: str
    mask: str
    scale: float
    o_scale: float
    seed: int
    q_scale: float = 1.0
    k_scale: float = 1.0
    v_scale: float = 1.0
    kv_dtype: str = ""  # element type of the cache ("" = dtype)

    @property
    def Sk(self) -> int:
        """The most keys of any sequence."""
        return int(self.seqlens_k.max()) if len(self.seqlens_k) else 0

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    def flops(self) -> float:
        """4*B*H*Sq*Sk*D with Sk the longest cache (the decode workloads give every sequence that length)."""
        return 4.0 * self.B * self.H * self.Sq * self.Sk * self.D

    @property
    def kernel_scale(self) -> float:
        return self.scale * self.q_scale * self.k_scale

    @property
    def kernel_o_scale(self) -> float:
        return self.o_scale * self.v_scale


def make_paged(seed: int, B: int, Sq: int, seqlens_k: Sequence[int], H: int, H_kv: int, D: int, dtype: str,
               page_size: int, mask: str = "none", extra_pages: int = 3, poison: bool = True,
               scale: Optional[float] = None, o_scale: float = 1.0, kv_dtype: Optional[str] = None) -> PagedInputs:
    """Dense Q and a paged K/V cache.  Draws Q, then the whole K cache, then the V cache (N(0, 1)), then
    a random permutation that deals the physical pages out to the sequences' logical pages in order.
    ``extra_pages`` pages belong to no sequence; with ``poison`` they, and the rows of each last page
    past its sequence's end, hold NaN.  ``kv_dtype="f8e4m3"`` quantises each cache per tensor (the
    scale from the rows the sequences own)."""
    rng = np.random.default_rng(seed)
    lk = np.asarray(seqlens_k, dtype=np.int32)
    assert lk.shape == (B,)
    pages_b = [-(-int(s) // page_size) for s in lk]
    num_pages = sum(pages_b) + int(extra_pages)
    max_pages = max(pages_b + [1])
    kv_dtype = kv_dtype or dtype
    q, sq = _to_storage(draw_normal(rng, (B, Sq, H, D)), dtype)
    k32 = draw_normal(rng, (num_pages, page_size, H_kv, D))
    v32 = draw_normal(rng, (num_pages, page_size, H_kv, D))
    perm = rng.permutation(num_pages).astype(np.int32)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    used = np.zeros((num_pages, page_size), dtype=bool)
    n = 0
    for b in range(B):
        for i in range(pages_b[b]):
            pg = int(perm[n])
            n += 1
            table[b, i] = pg
            rows = min(page_size, int(lk[b]) - i * page_size)
            used[pg, :rows] = True
    sk = sv = 1.0
    if kv_dtype == "f8e4m3":
        _, sk = quantize_e4m3(torch.from_numpy(k32[used]))
        _, sv = quantize_e4m3(torch.from_numpy(v32[used]))
        kc = (torch.from_numpy(k32) / sk).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
        vc = (torch.from_numpy(v32) / sv).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    else:
        kc, _ = _to_storage(k32, kv_dtype)
        vc, _ = _to_storage(v32, kv_dtype)
    if poison:
        unused = torch.from_numpy(~used)
        if kv_dtype == "f8e4m3":  # 0x7F: e4m3fn NaN
            kc.view(torch.uint8)[unused] = 0x7F
            vc.view(torch.uint8)[unused] = 0x7F
        else:
            kc[unused] = float("nan")
            vc[unused] = float("nan")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return PagedInputs(q=q, k_cache=kc, v_cache=vc, block_table=table, seqlens_k=lk, page_size=int(page_size), B=B,
                       Sq=Sq, H=H, H_kv=H_kv, D=D, dtype=dtype, mask=mask, scale=float(scale),
                       o_scale=float(o_scale), seed=seed, q_scale=float(sq), k_scale=float(sk), v_scale=float(sv),
                       kv_dtype=kv_dtype)


def make_new_rows(seed: int, B: int, S_new: int, H_kv: int, D: int, kv_dtype: str, k_scale: float = 1.0,
                  v_scale: float = 1.0):
    """K and V rows of S_new new tokens per sequence, [B, S_new, H_kv, D] in the cache's storage type:
    N(0, 1) drawn K then V; an e4m3 cache's rows are quantised with the cache's scales."""
    rng = np.random.default_rng(seed)
    k32, v32 = draw_normal(rng, (B, S_new, H_kv, D)), draw_normal(rng, (B, S_new, H_kv, D))
    if kv_dtype == "f8e4m3":
        k = (torch.from_numpy(k32) / k_scale).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
        v = (torch.from_numpy(v32) / v_scale).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
        return k, v
    return torch.from_numpy(k32).to(TORCH_DTYPES[kv_dtype]), torch.from_numpy(v32).to(TORCH_DTYPES[kv_dtype])


def make_varlen(seed: int, seqlens_q: Sequence[int], seqlens_k: Sequence[int], H: int, H_kv: int, D: int,
                dtype: str, mask: str = "none", scale: Optional[float] = None, o_scale: float = 1.0,
                poison_pads: bool = False, rng: Optional[np.random.Generator] = None) -> VarlenInputs:
    """Packed batch with explicit lengths.  ``rng`` continues a stream that already drew the lengths."""
    if rng is None:
        rng = np.random.default_rng(seed)
    lq = np.asarray(seqlens_q, dtype=np.int64)
    lk = np.asarray(seqlens_k, dtype=np.int64)
    assert lq.shape == lk.shape and lq.ndim == 1
    cu_q = np.zeros(len(lq) + 1, dtype=np.int32)
    cu_k = np.zeros(len(lk) + 1, dtype=np.int32)
    cu_q[1:] = np.cumsum(lq)
    cu_k[1:] = np.cumsum(lk)
    pad_q = int(lq.max()) if len(lq) else 0
    pad_k = int(lk.max()) if len(lk) else 0
    q32 = draw_normal(rng, (pad_q + int(cu_q[-1]), H, D))
    k32 = draw_normal(rng, (pad_k + int(cu_k[-1]), H_kv, D))
    v32 = draw_normal(rng, (pad_k + int(cu_k[-1]), H_kv, D))
    if dtype == "f8e4m3":
        # quantise with the scale of the packed rows only, so the padding never changes the scales
        q, sq = quantize_e4m3(torch.from_numpy(q32[pad_q:]))
        k, sk = quantize_e4m3(torch.from_numpy(k32[pad_k:]))
        v, sv = quantize_e4m3(torch.from_numpy(v32[pad_k:]))
        qp = (torch.from_numpy(q32[:pad_q]) / sq).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
        kp = (torch.from_numpy(k32[:pad_k]) / sk).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
        vp = (torch.from_numpy(v32[:pad_k]) / sv).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
        q_buf, k_buf, v_buf = torch.cat([qp, q]), torch.cat([kp, k]), torch.cat([vp, v])
    else:
        q_buf = torch.from_numpy(q32).to(TORCH_DTYPES[dtype])
        k_buf = torch.from_numpy(k32).to(TORCH_DTYPES[dtype])
        v_buf = torch.from_numpy(v32).to(TORCH_DTYPES[dtype])
        sq = sk = sv = 1.0
    if poison_pads:
        q_buf[:pad_q] = float("nan")
        k_buf[:pad_k] = float("nan")
        v_buf[:pad_k] = float("nan")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return VarlenInputs(q_buf=q_buf, k_buf=k_buf, v_buf=v_buf, seqlens_q=lq, seqlens_k=lk, cu_q=cu_q, cu_k=cu_k,
                        pad_q=pad_q, pad_k=pad_k, H=H, H_kv=H_kv, D=D, dtype=dtype, mask=mask,
                        scale=float(scale), o_scale=float(o_scale), seed=seed, q_scale=sq, k_scale=sk, v_scale=sv)


# The measured workloads.  Config 4 is run twice on the same inputs (residual, then causal-qend);
# config 6 is the split-KV (decode) entry point's workload; config 7 is the backward pass (fmha_bwd)
# of config 2's shape; config 8 is config 6 over a paged cache (fmha_fwd_splitkv_paged), config 9
# the same over an e4m3 cache; config 10 is config 7 with e4m3 inputs.
CONFIGS = {
    1: dict(name="tiny dense fp16 D64 no mask", kind="dense", B=1, H=2, H_kv=2, Sq=128, Sk=128, D=64,
            dtype="f16", mask="none", lse=False, o_scale=1.0),
    2: dict(name="prefill causal-qbegin bf16 D128 + LSE", kind="dense", B=4, H=16, H_kv=16, Sq=2048, Sk=2048,
            D=128, dtype="bf16", mask="causal_qbegin", lse=True, o_scale=1.0),
    3: dict(name="GQA causal long context bf16 D128", kind="dense", B=2, H=32, H_kv=8, Sq=8192, Sk=8192, D=128,
            dtype="bf16", mask="causal_qbegin", lse=False, o_scale=1.0),
    4: dict(name="packed varlen fp16 D64 residual / causal-qend", kind="varlen", nseq=8, sq_lo=64, sq_hi=1024,
            sk_extra_hi=2048, H=16, H_kv=16, D=64, dtype="f16", masks=("residual", "causal_qend"), lse=False,
            o_scale=1.0),
    5: dict(name="fp8 e4m3 D128 no mask, output scale 0.5", kind="dense", B=8, H=16, H_kv=16, Sq=4096, Sk=4096,
            D=128, dtype="f8e4m3", mask="none", lse=False, o_scale=0.5),
    # Generation / decode, run through fmha_fwd_splitkv: one new token per sequence against an
    # 8192-key cache, GQA 32/8 (one query row per head: no mask and causal-qend coincide).
    6: dict(name="decode GQA bf16 D128, 1 token vs 8192 keys (split-KV)", kind="dense", entry="splitkv", B=16,
            H=32, H_kv=8, Sq=1, Sk=8192, D=128, dtype="bf16", mask="none", lse=True, o_scale=1.0),
    # Backward of the prefill workload: dQ, dK, dV for a N(0, 1) upstream gradient (fmha_bwd).
    7: dict(name="backward of prefill causal-qbegin bf16 D128", kind="dense", entry="bwd", B=4, H=16, H_kv=16,
            Sq=2048, Sk=2048, D=128, dtype="bf16", mask="causal_qbegin", lse=True, o_scale=1.0),
    # Decode over a paged cache: config 6's shape with 128-key pages dealt out in random order.
    8: dict(name="paged decode GQA bf16 D128, 1 token vs 8192 keys, 128-key pages", kind="paged",
            entry="splitkv_paged", B=16, H=32, H_kv=8, Sq=1, Sk=8192, D=128, page_size=128, dtype="bf16",
            mask="none", lse=True, o_scale=1.0),
    # The same over an e4m3 cache (per-tensor scales), bf16 queries and output.
    9: dict(name="paged decode GQA bf16 D128 over an e4m3 cache, 1 token vs 8192 keys, 128-key pages",
            kind="paged", entry="splitkv_paged", B=16, H=32, H_kv=8, Sq=1, Sk=8192, D=128, page_size=128,
            dtype="bf16", kv_dtype="f8e4m3", mask="none", lse=True, o_scale=1.0),
    # Backward of the prefill shape with e4m3 inputs (O from the fp8 forward with o_scale 1, an
    # e4m3 dO), gradients in bf16.
    10: dict(name="backward of prefill causal-qbegin D128, e4m3 inputs, bf16 gradients", kind="dense", entry="bwd",
             B=4, H=16, H_kv=16, Sq=2048, Sk=2048, D=128, dtype="f8e4m3", mask="causal_qbegin", lse=True,
             o_scale=1.0),
}


def make_config(config_id: int, seed: Optional[int] = None, mask: Optional[str] = None, poison_pads: bool = False):
    c = CONFIGS[config_id]
    seed = config_seed(config_id) if seed is None else seed
    if c["kind"] == "paged":
        return make_paged(seed, c["B"], c["Sq"], [c["Sk"]] * c["B"], c["H"], c["H_kv"], c["D"], c["dtype"],
                          c["page_size"], mask=mask or c["mask"], extra_pages=0, poison=False, o_scale=c["o_scale"],
                          kv_dtype=c.get("kv_dtype"))
    if c["kind"] == "dense":
        return make_dense(seed, c["B"], c["Sq"], c["Sk"], c["H"], c["H_kv"], c["D"], c["dtype"],
                          mask=mask or c["mask"], o_scale=c["o_scale"])
    rng = np.random.default_rng(seed)
    lq = rng.integers(c["sq_lo"], c["sq_hi"], size=c["nseq"], endpoint=True)
    lk = lq + rng.integers(0, c["sk_extra_hi"], size=c["nseq"], endpoint=True)
    return make_varlen(seed, lq, lk, c["H"], c["H_kv"], c["D"], c["dtype"], mask=mask or c["masks"][0],
                       o_scale=c["o_scale"], poison_pads=poison_pads, rng=rng)
