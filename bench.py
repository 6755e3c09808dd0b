#!/usr/bin/env python3
"""Benchmark of the attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--no-cpu-baseline]

A step is one fmha_fwd call (the whole hot path) over one batch of seeded synthetic
input already resident in device memory.  The default workload is the prefill
causal-qbegin bf16 D=128 problem (B=4, H=16, S=2048, LSE written).  Rank 0 prints one
JSON line with the throughput in TFLOP/s (4*B*H*Sq*Sk*D, halved for causal masks), the
roofline of the kernel (FLOPs per launch over the average launch duration: one pair of HIP
events on the launch stream around the timed launches, divided by their number; against
MI355X's dense MFMA peak for the dtype), and the
fp64 CPU oracle timed on a bounded sample of the same workload.

--config 6 is the generation / decode workload of fmha_fwd_splitkv (one split-KV call per
step, both of its kernels): bound by HBM, so its line reports GB/s of algorithmic bytes
(|Q| + |K| + |V| + |O| + |LSE|) against MI355X's 8 TB/s.

--config 8 is config 6 over a paged cache (fmha_fwd_splitkv_paged, 128-key pages dealt out in
random order), reported the same way; --config 9 is config 8 over an e4m3 cache (half the K/V
bytes; bf16 queries and output).

--config 7 is the backward pass (one fmha_bwd call per step: its two kernels, dQ with the row
statistics, then dK/dV) of the prefill shape, with O and LSE from fmha_fwd computed once before timing.  Its
FLOPs follow the 5-matmul count (S, dP, dV, dQ, dK: 2.5 times the forward's 4*B*H*Sq*Sk*D,
halved for causal masks); the roofline is taken over the whole call.  --config 10 is the same backward
with e4m3 inputs (O from the fp8 forward, an e4m3 dO) and bf16 gradients: the inputs are widened to
bf16 in the workspace by a third kernel, so its peak is the bf16 one.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import head_attention_03_amd as fmha  # noqa: E402
from workloads import CONFIGS, make_config, to_bits  # noqa: E402

# MI355X published dense peaks (TFLOP/s): 256 CUs x 2.4 GHz x {4096 fp16/bf16, 8192 fp8} FLOP/clk/CU
PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "f8e4m3": 5033.2}
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
CSRC = os.path.join(ROOT, "head_attention_03_amd", "csrc")
KERNEL_SOURCES = {"fwd": ("fmha_fwd.hip", "fmha_device.h"), "splitkv": ("fmha_splitkv.hip", "fmha_device.h"),
                  "splitkv_paged": ("fmha_splitkv.hip", "fmha_device.h"),
                  "bwd": ("fmha_bwd.hip", "fmha_device.h")}
BWD_FLOP_FACTOR = 2.5  # backward matmuls (S, dP, dV, dQ, dK) per forward matmul pair
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash(entry: str = "fwd") -> str:
    """Hash of the sources a workload's kernels are compiled from."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[entry]:
        h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()[:16]


def workload_slug(c: dict) -> str:
    """File-name tag of a workload: dtype, head dim, mask, sizes."""
    heads = f"h{c['H']}" if c["H"] == c["H_kv"] else f"h{c['H']}kv{c['H_kv']}"
    if c.get("entry") == "bwd":
        return f"bwd_{c['dtype']}_d{c['D']}_{c['mask']}_b{c['B']}_{heads}_s{c['Sq']}"
    if c.get("entry") == "splitkv_paged":
        kv = f"_kv{c['kv_dtype']}" if c.get("kv_dtype") else ""
        return (f"splitkv_paged_{c['dtype']}{kv}_d{c['D']}_{c['mask']}_b{c['B']}_{heads}_q{c['Sq']}_k{c['Sk']}"
                f"_p{c['page_size']}")
    if c.get("entry") == "splitkv":
        return f"splitkv_{c['dtype']}_d{c['D']}_{c['mask']}_b{c['B']}_{heads}_q{c['Sq']}_k{c['Sk']}"
    if c["kind"] == "dense":
        return f"{c['dtype']}_d{c['D']}_{c['mask']}_b{c['B']}_{heads}_s{c['Sq']}"
    return f"{c['dtype']}_d{c['D']}_varlen{c['nseq']}_h{c['H']}"


def measured_traffic(c: dict):
    """Bytes per launch that left the L2 (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated; Infinity
    Cache hits included, so an upper bound of the HBM traffic) from the committed counter summary of
    this workload, if it was taken on the current kernel source (else None)."""
    try:
        prefix = "fmha_" if c.get("entry") == "bwd" else "fmha_fwd_"
        rec = json.load(open(os.path.join(PROFILES, f"{prefix}{workload_slug(c)}_traffic.json")))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(c.get("entry", "fwd")):
        return None
    return rec.get("l2_miss_bytes_per_launch")


def algorithmic_bytes(inp, want_lse: bool) -> float:
    """|Q| + |K| + |V| + |O| (+ |LSE|) of a dense workload: what the path must move at least."""
    e = 1 if inp.dtype == "f8e4m3" else 2
    ek = 1 if (getattr(inp, "kv_dtype", "") or inp.dtype) == "f8e4m3" else 2
    qo = 2.0 * inp.B * inp.Sq * inp.H * inp.D * e
    kv = 2.0 * inp.B * inp.Sk * inp.H_kv * inp.D * ek
    return qo + kv + (4.0 * inp.B * inp.H * inp.Sq if want_lse else 0.0)


def cpu_baseline(config_id: int, budget_s: float):
    """The fp64 oracle as it stands, on whole (sequence, head) units of the same workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    inp = make_config(config_id)
    q = oracle.decode(to_bits(inp.q), inp.dtype) * inp.q_scale
    if CONFIGS[config_id]["kind"] == "paged":  # whole sequences through the paged oracle, gather included
        kvt = inp.kv_dtype or inp.dtype
        kc = oracle.decode(to_bits(inp.k_cache), kvt) * inp.k_scale
        vc = oracle.decode(to_bits(inp.v_cache), kvt) * inp.v_scale
        done, t0 = 0, time.perf_counter()
        for b in range(inp.B):
            oracle.attention_paged(q[b:b + 1], kc, vc, inp.block_table[b:b + 1], inp.seqlens_k[b:b + 1], inp.scale,
                                   inp.mask)
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        gbs = algorithmic_bytes(inp, bool(CONFIGS[config_id]["lse"])) * done / inp.B / dt / 1e9
        return {"value": round(gbs, 6), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
                "sample": f"{done} of {inp.B} sequences of the same workload (all heads, page gather included), "
                          f"fp64 numpy, {dt:.1f} s on {platform.processor() or platform.machine()}"}
    else:
        k = oracle.decode(to_bits(inp.k), inp.dtype) * inp.k_scale
        v = oracle.decode(to_bits(inp.v), inp.dtype) * inp.v_scale
    group = inp.H // inp.H_kv
    units = [(b, h) for b in range(inp.B) for h in range(inp.H)]
    bwd = CONFIGS[config_id].get("entry") == "bwd"
    if bwd:
        from workloads import make_grad
        do = oracle.decode(to_bits(make_grad(inp.seed + 1, (inp.B, inp.Sq, inp.H, inp.D), inp.dtype)), inp.dtype)
    done, flops, t0 = 0, 0.0, time.perf_counter()
    for b, h in units:
        if bwd:
            oracle.attention_head_backward(q[b, :, h], k[b, :, h // group], v[b, :, h // group], do[b, :, h],
                                           inp.scale, inp.mask)
            flops += BWD_FLOP_FACTOR * inp.flops() / len(units)
        else:
            oracle.attention_head(q[b, :, h], k[b, :, h // group], v[b, :, h // group], inp.scale, inp.mask)
            flops += inp.flops() / len(units)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    if CONFIGS[config_id].get("entry") in ("splitkv", "splitkv_paged"):  # GB/s of the workload's bytes, as the GPU line
        gbs = algorithmic_bytes(inp, bool(CONFIGS[config_id]["lse"])) * done / len(units) / dt / 1e9
        return {"value": round(gbs, 6), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
                "sample": f"{done} of {len(units)} (sequence, head) units of the same workload, fp64 numpy, "
                          f"{dt:.1f} s on {platform.processor() or platform.machine()}"}
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {len(units)} (sequence, head) units of the same workload, fp64 numpy, "
                      f"{dt:.1f} s on {platform.processor() or platform.machine()}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, choices=sorted(CONFIGS))
    ap.add_argument("--rotate", type=int, default=2, help="input buffer sets cycled through (defeats cache reuse)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this path has no multi-GPU mode",
              file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only; launch it without torch.distributed", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "needs a ROCm GPU"
    fmha.load()

    cid = args.config
    c = CONFIGS[cid]
    dev = torch.device("cuda:0")
    inp = make_config(cid)
    masks = [inp.mask] if c["kind"] in ("dense", "paged") else list(c["masks"])
    want_lse = bool(c["lse"])

    # device buffers: `rotate` copies of the inputs, one output (and LSE) per copy
    sets = []
    for r in range(max(1, args.rotate)):
        if c["kind"] == "paged":
            q = inp.q.to(dev)
            bt = torch.from_numpy(inp.block_table).to(dev)
            sl = torch.from_numpy(inp.seqlens_k).to(dev)
            sets.append(dict(q=q, k=inp.k_cache.to(dev), v=inp.v_cache.to(dev), o=torch.empty_like(q),
                             lse=torch.empty((inp.B, inp.H, inp.Sq), dtype=torch.float32, device=dev),
                             varlen=None, tables=(bt, sl),
                             paged=fmha.make_paged_kv(bt, sl, bt.shape[1], inp.page_size, inp.num_pages,
                                                      inp.kv_dtype or inp.dtype)))
        elif c["kind"] == "dense":
            q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
            o = torch.empty_like(q)
            lse = torch.empty((inp.B, inp.H, inp.Sq), dtype=torch.float32, device=dev) if want_lse else None
            sets.append(dict(q=q, k=k, v=v, o=o, lse=lse, varlen=None))
        else:
            q = inp.q_buf.to(dev)[inp.pad_q:]
            k, v = inp.k_buf.to(dev)[inp.pad_k:], inp.v_buf.to(dev)[inp.pad_k:]
            o = inp.new_output_buffer().to(dev)[inp.pad_q:]
            cu_q, cu_k = torch.from_numpy(inp.cu_q).to(dev), torch.from_numpy(inp.cu_k).to(dev)
            lse = torch.empty((inp.H, inp.total_q), dtype=torch.float32, device=dev) if want_lse else None
            sets.append(dict(q=q, k=k, v=v, o=o, lse=lse, cu=(cu_q, cu_k),
                             varlen=fmha.make_varlen(cu_q, cu_k, inp.total_q, inp.total_k)))
    if c["kind"] == "paged":
        B, Sq, Sk = inp.B, inp.Sq, inp.Sk
        flops_step = 4.0 * B * inp.H * Sq * Sk * inp.D
    elif c["kind"] == "dense":
        B, Sq, Sk = inp.B, inp.Sq, inp.Sk
        flops_step = inp.flops()
    else:
        B, Sq, Sk = inp.B, inp.max_q, inp.max_k
        flops_step = 0.0
        for m in masks:
            inp.mask = m
            flops_step += inp.flops_convention()

    stream = torch.cuda.Stream(device=dev)  # default priority
    paged = c.get("entry") == "splitkv_paged"
    splitkv = c.get("entry") in ("splitkv", "splitkv_paged")
    bwd = c.get("entry") == "bwd"
    if bwd:
        # the backward's inputs: dO (seeded), and O and LSE of the forward, computed once here
        from workloads import make_grad
        do_cpu = make_grad(inp.seed + 1, (inp.B, inp.Sq, inp.H, inp.D), inp.dtype)
        bws = fmha.fmha_bwd_workspace_size(B, Sq, Sk, inp.H, inp.H_kv, inp.D, inp.dtype, None)
        for s_ in sets:
            lse = s_["lse"] if s_["lse"] is not None else torch.empty((B, inp.H, Sq), dtype=torch.float32, device=dev)
            fmha.check(fmha.fmha_fwd(s_["q"], s_["k"], s_["v"], s_["o"], lse, B, Sq, Sk, inp.H, inp.H_kv, inp.D,
                                     inp.kernel_scale, inp.mask, inp.dtype, 1.0, None, stream))
            gt = torch.bfloat16 if inp.dtype == "f8e4m3" else s_["q"].dtype  # e4m3 inputs: bf16 gradients
            s_.update(lse=lse, do=do_cpu.to(dev), dq=torch.empty(s_["q"].shape, dtype=gt, device=dev),
                      dk=torch.empty(s_["k"].shape, dtype=gt, device=dev),
                      dv=torch.empty(s_["v"].shape, dtype=gt, device=dev))
        bw = torch.empty(max(bws, 16), dtype=torch.uint8, device=dev)
        flops_step = BWD_FLOP_FACTOR * flops_step
        torch.cuda.synchronize()
    ws_bytes = fmha.fmha_fwd_splitkv_workspace_size(B, Sq, Sk, inp.H, inp.H_kv, inp.D, None) if splitkv else 0
    # one workspace serves every set: the launches run one after another on one stream
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev) if splitkv else None

    def launch(i):
        s = sets[i % len(sets)]
        for m in masks:
            if bwd:
                st = fmha.fmha_bwd(s["q"], s["k"], s["v"], s["o"], s["do"], s["lse"], s["dq"], s["dk"], s["dv"], B, Sq,
                                   Sk, inp.H, inp.H_kv, inp.D, inp.kernel_scale, m, inp.dtype, None, bw, bws, stream)
            elif paged:
                st = fmha.fmha_fwd_splitkv_paged(s["q"], s["k"], s["v"], s["o"], s["lse"], B, Sq, Sk, inp.H, inp.H_kv,
                                                 inp.D, inp.kernel_scale, m, inp.dtype, inp.kernel_o_scale, s["paged"],
                                                 ws, ws_bytes, stream)
            elif splitkv:
                st = fmha.fmha_fwd_splitkv(s["q"], s["k"], s["v"], s["o"], s["lse"], B, Sq, Sk, inp.H, inp.H_kv,
                                           inp.D, inp.kernel_scale, m, inp.dtype, inp.kernel_o_scale, s["varlen"],
                                           ws, ws_bytes, stream)
            else:
                st = fmha.fmha_fwd(s["q"], s["k"], s["v"], s["o"], s["lse"], B, Sq, Sk, inp.H, inp.H_kv, inp.D,
                                   inp.kernel_scale, m, inp.dtype, inp.kernel_o_scale, s["varlen"], stream)
            if st != 0:
                raise fmha.FmhaError(st)

    torch.cuda.synchronize()
    for i in range(args.warmup):
        launch(i)
    torch.cuda.synchronize()

    # timed region: K back-to-back steps.  One pair of HIP events on the launch stream brackets
    # the launches, so the average launch duration is the stream's busy time over the region
    # divided by the launches (the dispatch gap between back-to-back launches included).  An
    # event pair around every step would put an event packet, with its cache release, between
    # consecutive kernels: that measured 7-8 us more per prefill step (about 9%), on the
    # kernels as well as on the wall clock.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        launch(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    avg_launch_s = ev0.elapsed_time(ev1) / 1e3 / args.steps / len(masks)

    value = flops_step * args.steps / elapsed / 1e12
    achieved = flops_step / len(masks) / avg_launch_s / 1e12
    # the backward computes e4m3 inputs on the bf16 matrix cores (after an exact widening)
    peak = PEAK_TFLOPS["bf16" if bwd else inp.dtype]
    traffic = measured_traffic(c)
    # the label names the workload's type, head dim and masks (the prefill workload's reads
    # "(bf16, D=128, causal)")
    mask_txt = " + ".join("causal" if m.startswith("causal") else ("no mask" if m == "none" else m) for m in masks)
    type_txt = {"f16": "f16", "bf16": "bf16", "f8e4m3": "fp8 e4m3"}[inp.dtype]
    metric = f"FMHA fwd TFLOP/s and % of MI355X dense MFMA peak ({type_txt}, D={inp.D}, {mask_txt})"
    unit, bound = "TFLOP/s", "mfma"
    if bwd:
        metric = "FMHA bwd TFLOP/s (5-matmul count) and % of MI355X dense MFMA peak (bf16, D=128, causal)"
        if inp.dtype == "f8e4m3":
            metric = ("FMHA bwd TFLOP/s (5-matmul count) and % of MI355X dense bf16 MFMA peak (e4m3 inputs widened "
                      "to bf16, D=128, causal)")
    tflops = value
    if splitkv:  # HBM-bound: GB/s of algorithmic bytes
        bytes_step = algorithmic_bytes(inp, want_lse)
        metric, unit, bound = "FMHA split-KV decode GB/s of algorithmic HBM bytes and % of MI355X HBM peak", "GB/s", "hbm"
        if paged:
            metric = "FMHA paged-KV split-KV decode GB/s of algorithmic HBM bytes and % of MI355X HBM peak"
        value = bytes_step * args.steps / elapsed / 1e9
        achieved = bytes_step / avg_launch_s / 1e9
        peak = PEAK_HBM_GBS
    cfg = {"workload": c["name"], "config_id": cid, "B": B, "Sq": Sq, "Sk": Sk, "H": inp.H, "H_kv": inp.H_kv,
           "D": inp.D, "dtype": inp.dtype, "mask": "+".join(masks), "lse": want_lse, "seed": inp.seed,
           "rotate_buffers": len(sets), "flop_per_step": flops_step}
    if splitkv:
        cfg.update(entry="fmha_fwd_splitkv_paged" if paged else "fmha_fwd_splitkv", tflops=round(tflops, 3),
                   workspace_bytes=ws_bytes)
    if paged:
        cfg.update(page_size=inp.page_size, num_pages=inp.num_pages, kv_dtype=inp.kv_dtype or inp.dtype)
    if bwd:
        cfg.update(entry="fmha_bwd", workspace_bytes=bws, flop_convention="2.5 x forward (S, dP, dV, dQ, dK)")
    out = {
        "metric": metric,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic type: the e4m3 backward computes on widened bf16 copies
        "dtype": "bf16" if bwd and inp.dtype == "f8e4m3" else {"f16": "f16", "bf16": "bf16", "f8e4m3": "fp8_e4m3"}[inp.dtype],
        "data": "synthetic (seeded N(0,1))",
        "config": cfg,
        "pct_of_peak": round(100.0 * value / peak, 2),
        "roofline": {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel_avg_us": round(avg_launch_s * 1e6, 3)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cid, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
