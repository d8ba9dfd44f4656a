"""Benchmark: fused attention forward (TFLOP/s) and split-KV decode (GB/s) on one MI355X.

One step = one pass of the whole hot path on resident synthetic inputs:
  fa_fwd on the long-prefill workload (B2 H32 S8192 d128, causal, K x4 on 1% of positions),
  then the split-KV decode (B64 Hq32 Hkv8 Skv16384 d128): chunk partials + log-sum-exp merge.
W untimed warmup steps (default 300), then K timed steps (default 200) between device
synchronisations. Every kernel is bracketed by HIP events recorded on the stream the
library launches on (torch's current stream, which is passed to the library), giving
per-kernel average durations.

Prints ONE JSON line. ``value`` is forward TFLOP/s with causal FLOPs counted as half
(4*B*Hq*Sq*Skv*d/2); the decode figures sit under ``decode``, the other prefill
workloads (B4 H16 S2048 d64; B1 Hq32 Hkv8 S32768 d128) under ``prefill_other``, each
timed on its own after the step loop. Beside the GPU figures:
  * ``ceilings``: the sustained matrix-core rate and HBM read bandwidth measured on this
    chip by the probe library, and each roofline's fraction of them;
  * ``cpu_baseline`` per workload: the fp64 oracle as it stands, spread over a process pool
    of the host's cores (one BLAS thread each), timed on a stated share of the workload;
  * ``parity`` per workload: the stated check (max-abs <= 1e-2, rel-L2 <= 4e-3 for O and
    LSE) over the same share, with the bf16 floor, the worst error in bf16 ulps and the
    same check on an fp32-output run of the forward.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd attention TFLOP/s (bf16, causal-adjusted) & % MFMA peak; decode HBM GB/s"
PEAK_MFMA_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0              # MI355X HBM3E
PEAK_MFMA_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PROFILES = os.path.join(ROOT, "profiles")
# Sources each kernel family is built from: an HBM-traffic record is used only while
# the sources it was measured on are unchanged.
KERNEL_SOURCES = {"fwd": ["fa_device.hpp", "fa_dma.hpp", "fa_launch.hpp", "fa_walk.hpp", "fa_fwd.hip"],
                  "decode": ["fa_device.hpp", "fa_launch.hpp", "fa_decode.hip"],
                  "bwd": ["fa_device.hpp", "fa_dma.hpp", "fa_bwd.hpp", "fa_bwd.hip"],
                  "fp8": ["fa_device.hpp", "fa_dma.hpp", "fa_fp8.hpp", "fa_walk.hpp", "fa_fwd_fp8.hip"],
                  "bpt": ["fa_device.hpp", "fa_dma.hpp", "fa_launch.hpp", "fa_walk.hpp", "fa_fwd.hip", "fa_bpt.hpp",
                          "fa_ffn.hip", "fa_api.hip", "fa_bwd.hpp", "fa_fp8.hpp"]}


def fwd_flops(w) -> float:
    f = 4.0 * w.B * w.Hq * w.Sq * w.Skv * w.d
    return f / 2 if w.causal else f


def fwd_bytes(w) -> int:
    q = w.B * w.Sq * w.Hq * w.d * 2
    kv = 2 * w.B * w.Skv * w.Hkv * w.d * 2
    return q + kv + q + w.B * w.Hq * w.Sq * 4


def decode_bytes(w) -> dict:
    kv = 2 * w.B * w.Skv * w.Hkv * w.d * 2
    q = w.B * w.Hq * w.d * 2
    return {"total": kv + q + q + w.B * w.Hq * 4, "split_kernel": kv + q}


def kernel_source_hash(family: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, "io_aware_exact_21_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(name: str, family: str):
    """HBM bytes per launch from the committed PMC summary, if taken on the current kernel sources."""
    path = os.path.join(PROFILES, name)
    try:
        with open(path) as f:
            rec = json.loads(next(l for l in f if l.startswith("{")))
    except (OSError, StopIteration, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash(family):
        return None
    return rec.get("hbm_bytes_per_launch")


def measured_mfma_util(name: str, family: str):
    """Matrix-core utilisation and shader clock from the committed counter summary, if taken
    on the current kernel sources."""
    path = os.path.join(PROFILES, name)
    try:
        with open(path) as f:
            rec = json.loads(next(l for l in f if l.startswith("{")))
    except (OSError, StopIteration, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash(family):
        return None
    return {"mfma_util": rec.get("mfma_util"), "shader_clock_ghz": rec.get("shader_clock_ghz"),
            "source": "rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs), sustained dispatches"}


# Share of each workload the oracle leg covers, where it is less than every (batch, head):
# none today (the whole leg, every head of every workload, takes about half a minute on
# 16 host cores). A workload listed here maps to the (batch, head) pairs to check.
ORACLE_SHARE = {}


def oracle_leg(key: str, w, q, k, v, outputs: dict) -> tuple:
    """The fp64 oracle as it stands, over a process pool of the host's cores, on the
    workload's share (ORACLE_SHARE): its rate (cpu_baseline) and the stated check of the
    device outputs on that share (parity)."""
    from oracle import fullcheck as fc
    log = lambda m: print(f"[bench] {key}: {m}", file=sys.stderr, flush=True)
    if w.decode:
        res = fc.check_decode(q, k, v, outputs, scale=w.scale, progress=log)
        share, total = w.B, w.B
        what = f"{share} of {total} sequences (every query head)"
        unit_amount = decode_bytes(w)["total"] * share / total
        value, unit = unit_amount / res["_oracle"]["wall_s"] / 1e9, "GB/s"
    else:
        heads = ORACLE_SHARE[key](w) if key in ORACLE_SHARE else None
        res = fc.check_prefill(q, k, v, outputs, causal=w.causal, scale=w.scale, heads=heads, progress=log)
        share, total = res["_oracle"]["shares"], w.B * w.Hq
        what = f"{share} of {total} (batch, query head) slices, every query row and visible key"
        value, unit = res["_oracle"]["flops"] / res["_oracle"]["wall_s"] / 1e12, "TFLOP/s"
    orc = res.pop("_oracle")
    cpu = {"value": round(value, 5), "unit": unit, "cores": orc["workers"], "kind": "oracle",
           "cpu_model": orc["cpu_model"], "wall_s": round(orc["wall_s"], 2),
           "sample": f"{what} of the {w.name} workload; fp64 NumPy oracle in {orc['workers']} worker "
                     f"processes with one BLAS thread each"}
    par = {"share": what, "label": fc.label(res["bf16"], res.get("f32")), "bf16_output": res["bf16"]}
    if "f32" in res:
        par["f32_output"] = res["f32"]
        par["f32_output_stated_check"] = "pass" if fc.stated_ok(res["f32"]) else "fail"
    return cpu, par


def probe_ceilings(dev, stream) -> dict:
    """Sustained matrix-core rate (bf16 32x32x16 products, random operands, two waves per
    SIMD) and HBM read bandwidth (non-temporal 16-byte loads over 4 GiB) on this chip."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "io_aware_exact_21_amd", "libfa_probe.so"))
    lib.fa_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.fa_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_void_p]
    sp = stream.cuda_stream
    blocks, iters = 1024, 400
    ops = torch.randn(blocks * 512 * 10 * 8, device=dev).to(torch.bfloat16)
    sink = torch.empty(blocks * 512, dtype=torch.float32, device=dev)

    def timed(fn, n):
        for _ in range(n):                      # as many untimed launches first (sustained clock)
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def mfma():
        if lib.fa_probe_mfma_bf16(ops.data_ptr(), sink.data_ptr(), blocks, iters, sp) != 0:
            raise RuntimeError("fa_probe_mfma_bf16 failed")
    ms = timed(mfma, 20)
    mfma_tf = blocks * 8 * iters * 8 * 32768.0 / (ms * 1e-3) / 1e12
    nbytes = 4 << 30
    buf = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=dev)
    rblocks = 1024                              # four waves per CU: the fastest of 512..16384 workgroups

    def read():
        if lib.fa_probe_hbm_read(buf.data_ptr(), nbytes, sink.data_ptr(), rblocks, sp) != 0:
            raise RuntimeError("fa_probe_hbm_read failed")
    ms_r = timed(read, 10)
    gbs = nbytes / (ms_r * 1e-3) / 1e9
    del buf, ops
    return {"mfma_bf16": {"value": round(mfma_tf, 1), "unit": "TFLOP/s", "frac_of_spec": round(mfma_tf / PEAK_MFMA_BF16_TFLOPS, 4),
                          "probe": "fa_probe_mfma_bf16: 1024 workgroups x 8 waves (one workgroup per CU), 400 "
                                   "rounds of 8 v_mfma_f32_32x32x16_bf16 on random operands held in registers"},
            "hbm_read": {"value": round(gbs, 1), "unit": "GB/s", "frac_of_spec": round(gbs / PEAK_HBM_GBS, 4),
                         "probe": "fa_probe_hbm_read: 4 GiB, 1024 workgroups x 128 threads, each streaming its "
                                  "own 4 MiB slice with non-temporal 16-byte loads, 8 in flight per thread"}}


def time_calls(stream, call, steps: int, warmup: int) -> float:
    """Average ms of ``call`` over ``steps`` back-to-back calls after ``warmup`` calls (HIP events)."""
    import torch
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def prefill_bench(fa, lib, stream, key: str, w, up, steps: int, warmup: int) -> tuple:
    """One more prefill workload through fa_fwd, timed on its own; returns its JSON object
    and the inputs and outputs the oracle leg compares."""
    import torch
    from synth import make_workload
    print(f"[bench] prefill workload {w.name}", file=sys.stderr, flush=True)
    q, k, v = make_workload(w)
    tq, tk, tv = up(q), up(k), up(v)
    o = torch.empty_like(tq)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=tq.device)
    sp = stream.cuda_stream

    def call():
        fa._lib.check(lib.fa_fwd(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                 w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.d, int(w.causal), w.scale, sp), "fa_fwd")
    ms = time_calls(stream, call, steps, warmup)
    flops = fwd_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    o32, l32 = fa.fwd(tq, tk, tv, causal=w.causal, scale=w.scale, out_f32=True)
    torch.cuda.synchronize()
    outs = {"bf16": (o.float().cpu().numpy(), lse.cpu().numpy()), "f32": (o32.cpu().numpy(), l32.cpu().numpy())}
    rec = {"config": {**w.describe(), "scale": w.scale, "seed": w.seed},
           "value": round(tflops, 2), "unit": "TFLOP/s", "ms": round(ms, 4),
           "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_MFMA_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_BF16_TFLOPS, 4),
                        "traffic": measured_traffic(f"fa_fwd_{key}_hbm_traffic.txt", "fwd"),
                        "kernel": "fa_fwd_kernel", "avg_kernel_ms": round(ms, 4), "algorithmic_flops": flops,
                        "algorithmic_bytes": fwd_bytes(w)},
           "note": "fa_fwd timed with HIP events around back-to-back calls on the library's stream"}
    return rec, (q, k, v, outs)


def paged_decode_bench(fa, dev, stream, steps: int, warmup: int) -> dict:
    """Paged-cache split-KV decode, timed on its own after the main step.

    GB/s counts the K and V bytes of every sequence's own tokens read once, plus q read
    and O + LSE written; the block table and the split workspace are not counted.
    """
    import numpy as np
    import torch
    from synth import PAGED_WORKLOADS, make_paged_workload

    w = PAGED_WORKLOADS["paged"]
    print(f"[bench] generating inputs: {w.name}", file=sys.stderr, flush=True)
    q, kp, vp, table, lens = make_paged_workload(w)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    tq, tk, tv = up(q), up(kp), up(vp)
    del kp, vp
    tbt = torch.from_numpy(table).to(dev)
    tsl = torch.from_numpy(lens).to(dev)
    from io_aware_exact_21_amd.api import decode_paged_default_splits
    ns = decode_paged_default_splits(w.B, w.Hkv, w.max_len, w.d)
    ws = torch.empty(fa.decode_workspace_bytes(w.B, w.Hq, w.d, ns), dtype=torch.uint8, device=dev)
    o = torch.empty((w.B, w.Hq, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)
    for _ in range(warmup):
        fa.decode_paged(tq, tk, tv, tbt, tsl, scale=w.scale, num_splits=ns, workspace=ws, out=o, lse=lse)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fa.decode_paged(tq, tk, tv, tbt, tsl, scale=w.scale, num_splits=ns, workspace=ws, out=o, lse=lse)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = int(lens.astype(np.int64).sum()) * w.Hkv * w.d * 2 * 2 + 2 * w.B * w.Hq * w.d * 2 + w.B * w.Hq * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"config": {**w.describe(), "num_splits": ns, "seed": w.seed, "mean_len": float(lens.mean())},
            "value": round(gbs, 1), "unit": "GB/s", "ms": round(ms, 4), "algorithmic_bytes": nbytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("fa_decode_paged_hbm_traffic.txt", "decode"),
                         "kernel": "fa_decode_split_kernel (paged) + fa_decode_combine_kernel"},
            "note": "fa_decode_paged (partials + merge) timed with HIP events around the whole call"}


def backward_bench(fa, lib, stream, wkey: str, w, tq, tk, tv, o, lse, steps: int, warmup: int) -> dict:
    """fa_bwd (dQ kernel + dK/dV kernel) on the forward workload, timed on its own.

    TFLOP/s counts the five products of the backward (S = Q K^T, dP = dO V^T, dV, dK,
    dQ), i.e. 2.5x the forward's FLOPs, causal halved; the kernels execute seven (S and
    dP are formed in both kernels), which the rate does not count.
    """
    import numpy as np
    import torch
    from synth import make_grad_out

    print(f"[bench] backward on {w.name}", file=sys.stderr, flush=True)
    do = make_grad_out(w.B, w.Sq, w.Hq, w.d, w.seed)
    tdo = torch.from_numpy(np.ascontiguousarray(do).view(np.int16)).view(torch.bfloat16).to(tq.device)
    del do
    dq, dk, dv = torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)
    nws = fa.bwd_workspace_bytes(w.B, w.Hq, w.Sq)
    ws = torch.empty(nws, dtype=torch.uint8, device=tq.device)
    sp = stream.cuda_stream

    def call():
        fa._lib.check(lib.fa_bwd(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                 tdo.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), w.B, w.Hq, w.Hkv,
                                 w.Sq, w.Skv, w.d, int(w.causal), w.scale, ws.data_ptr(), nws, sp), "fa_bwd")

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 2.5 * fwd_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    return {"config": {**w.describe(), "seed": w.seed, "dO": "i.i.d. N(0,1) bf16, tensor id 5"},
            "value": round(tflops, 2), "unit": "TFLOP/s", "ms": round(ms, 4),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_MFMA_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_BF16_TFLOPS, 4),
                         "traffic": measured_traffic(f"fa_bwd_{wkey}_hbm_traffic.txt", "bwd"),
                         "kernel": "fa_bwd_dq_kernel + fa_bwd_dkdv_kernel (one fa_bwd call)",
                         "algorithmic_flops": flops, "executed_products": 7, "counted_products": 5},
            "note": "fa_bwd timed with HIP events around the whole call on the library's stream"}


def fp8_bench(fa, stream, wkey: str, w, steps: int, warmup: int) -> dict:
    """fa_fwd_fp8 on the e4m3-quantised version of the forward workload, timed on its own.

    TFLOP/s counts 4 B Hq Sq Skv d (halved when causal), as for the bf16 forward; the
    peak is the dense fp8 MFMA peak.
    """
    import numpy as np
    import torch
    from synth.fp8 import make_fp8_qkv

    print(f"[bench] fp8 forward on {w.name}", file=sys.stderr, flush=True)
    q8, k8, vt8, qs, ks, vs, ldv = make_fp8_qkv(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.d, w.seed, w.k_stress_frac)
    dev = torch.device("cuda:0")
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    tq, tk, tvt, tqs, tks, tvs = to(q8), to(k8), to(vt8), to(qs), to(ks), to(vs)
    del q8, k8, vt8
    o = torch.empty((w.B, w.Sq, w.Hq, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    lib = fa._lib.load()
    sp = stream.cuda_stream

    def call():
        fa._lib.check(lib.fa_fwd_fp8(tq.data_ptr(), tk.data_ptr(), tvt.data_ptr(), tqs.data_ptr(), tks.data_ptr(),
                                     tvs.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B, w.Hq, w.Hkv, w.Sq, w.Skv,
                                     ldv, w.d, int(w.causal), w.scale, sp), "fa_fwd_fp8")

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = fwd_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    return {"config": {**w.describe(), "dtype_io": "e4m3 in, bf16 out", "layout": "q, k [B,S,H,d]; v [B,Hkv,d,S]",
                       "quantisation": "per (batch, head) scale amax/448", "seed": w.seed},
            "value": round(tflops, 2), "unit": "TFLOP/s", "ms": round(ms, 4),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_MFMA_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_FP8_TFLOPS, 4),
                         "traffic": measured_traffic(f"fa_fwd_fp8_{wkey}_hbm_traffic.txt", "fp8"),
                         "kernel": "fa_fwd_fp8_kernel", "algorithmic_flops": flops},
            "note": "fa_fwd_fp8 timed with HIP events around the call on the library's stream"}


def bpt_bench(fa, stream, wkey: str, w, tq, tk, tv, steps: int, warmup: int, block_rows: int = 2048) -> dict:
    """fa_bpt_layer (attention + feed-forward network, blockwise) on the forward workload
    with d_model = Hq d and d_ff = 4 d_model, timed on its own; also the whole-sequence
    schedule (one block per batch element) for comparison.

    TFLOP/s counts the attention (as the forward, causal halved) plus the two FFN GEMMs,
    4 B S d_model d_ff.
    """
    import numpy as np
    import torch
    from synth import make_ffn_weights

    dm, dff = w.Hq * w.d, 4 * w.Hq * w.d
    print(f"[bench] blockwise attention + FFN on {w.name}, d_ff {dff}", file=sys.stderr, flush=True)
    dev = tq.device
    up = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
    w1, b1, w2, b2 = (up(x) for x in make_ffn_weights(dm, dff, w.seed))
    y = torch.empty((w.B, w.Sq, dm), dtype=torch.bfloat16, device=dev)
    lib = fa._lib.load()
    sp = stream.cuda_stream
    flops = fwd_flops(w) + 4.0 * w.B * w.Sq * dm * dff

    def timed(rows):
        nws = fa.bpt_workspace_bytes(w.B, w.Sq, rows, w.Hq, w.d, dff)
        ws = torch.empty(nws, dtype=torch.uint8, device=dev)

        def call():
            fa._lib.check(lib.fa_bpt_layer(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), w1.data_ptr(), b1.data_ptr(),
                                           w2.data_ptr(), b2.data_ptr(), y.data_ptr(), w.B, w.Hq, w.Hkv, w.Sq, w.d,
                                           dff, int(w.causal), w.scale, rows, ws.data_ptr(), nws, sp),
                          "fa_bpt_layer")
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps, nws

    ms, nws = timed(block_rows)
    ms_full, nws_full = timed(w.Sq)
    tflops = flops / (ms * 1e-3) / 1e12
    return {"config": {**w.describe(), "d_model": dm, "d_ff": dff, "ffn": "relu(h W1 + b1) W2 + b2",
                       "block_rows": block_rows, "weights": "N(0,1)/sqrt(fan-in), bias N(0,1)/10, bf16"},
            "value": round(tflops, 2), "unit": "TFLOP/s", "ms": round(ms, 4),
            "workspace_bytes": nws,
            "whole_sequence_schedule": {"block_rows": w.Sq, "ms": round(ms_full, 4),
                                        "TFLOP/s": round(flops / (ms_full * 1e-3) / 1e12, 2),
                                        "workspace_bytes": nws_full},
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_MFMA_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_BF16_TFLOPS, 4),
                         "traffic": measured_traffic(f"fa_bpt_{wkey}_hbm_traffic.txt", "bpt"),
                         "kernel": "per block of rows of every batch element: fa_fwd_kernel + two ffn_gemm_kernel", "algorithmic_flops": flops},
            "note": "fa_bpt_layer timed with HIP events around the call on the library's stream"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The compute-bound kernels settle at their sustained clock only after a few hundred
    # milliseconds of load (forward rate per 200-step window: 1111 TFLOP/s in the first,
    # 1128-1129 from the second on, flat over 4000 steps): 300 warm-up steps (about 0.5 s)
    # precede the 200 timed ones.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--fwd-workload", default="mha8k", choices=["tiny", "mha2k", "mha8k", "gqa32k"])
    # The decode workload splits the KV length into chunks and merges them by log-sum-exp,
    # so the bench runs two chunks per sequence; at this batch (B 64, Hkv 8) the library's
    # own default (0 below) picks one chunk, since 512 unsplit workgroups already fill the chip.
    ap.add_argument("--num-splits", type=int, default=2, help="decode KV splits (0 = library heuristic)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle leg (CPU baseline and stated-check parity per workload)")
    ap.add_argument("--no-other-prefill", action="store_true", help="skip the other prefill workloads")
    ap.add_argument("--no-paged", action="store_true", help="skip the paged-cache decode measurement")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward measurement")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8 forward measurement")
    ap.add_argument("--no-bpt", action="store_true", help="skip the blockwise attention + FFN measurement")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the ceiling probes")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run plain device copies of MIB MiB (reference reading for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only; --gpus {args.gpus} is not supported (the prefill and "
              "decode kernels shard by independent heads or KV chunks, one share per GPU, with no exchange)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    oracle_on = not args.no_cpu_baseline and args.copy_calibration == 0
    if oracle_on:
        # the oracle's worker processes are spawned before this process touches the GPU
        from oracle import fullcheck
        fullcheck.start_pool()

    import io_aware_exact_21_amd as fa
    from synth import WORKLOADS, make_workload

    dev = torch.device("cuda:0")
    if args.copy_calibration > 0:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE readings per dispatch
        # convert the counters of the attention kernels into bytes.
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "dispatches": 3}))
        return 0

    wf, wd = WORKLOADS[args.fwd_workload], WORKLOADS["decode"]

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    print(f"[bench] generating inputs: {wf.name}; {wd.name}", file=sys.stderr, flush=True)
    qf, kf, vf = make_workload(wf)
    tq, tk, tv = up(qf), up(kf), up(vf)
    qd, kd, vd = make_workload(wd)
    dq, dk, dv = up(qd), up(kd), up(vd)
    if not oracle_on:
        del kd, vd
    ns = args.num_splits if args.num_splits > 0 else fa.decode_default_splits(wd.B, wd.Hkv, wd.Skv, wd.d)
    o = torch.empty_like(tq)
    lse = torch.empty((wf.B, wf.Hq, wf.Sq), dtype=torch.float32, device=dev)
    po = torch.empty((wd.B, wd.Hq, ns, wd.d), dtype=torch.float32, device=dev)
    pl = torch.empty((wd.B, wd.Hq, ns), dtype=torch.float32, device=dev)
    lib = fa._lib.load()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    od = torch.empty((wd.B, wd.Hq, wd.d), dtype=torch.bfloat16, device=dev)
    ld = torch.empty((wd.B, wd.Hq), dtype=torch.float32, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa._lib.check(lib.fa_fwd(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                 wf.B, wf.Hq, wf.Hkv, wf.Sq, wf.Skv, wf.d, int(wf.causal), wf.scale, sp), "fa_fwd")
        if ev is not None:
            ev[1].record(stream)
        fa._lib.check(lib.fa_decode_partials(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), po.data_ptr(),
                                             pl.data_ptr(), wd.B, wd.Hq, wd.Hkv, wd.Skv, wd.d, wd.scale, ns, sp),
                      "fa_decode_partials")
        if ev is not None:
            ev[2].record(stream)
        fa._lib.check(lib.fa_decode_combine(po.data_ptr(), pl.data_ptr(), od.data_ptr(), ld.data_ptr(),
                                            wd.B, wd.Hq, wd.d, ns, sp), "fa_decode_combine")
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done; timing {args.steps} steps", file=sys.stderr, flush=True)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(end)
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    split_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    comb_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))

    flops = fwd_flops(wf)
    tflops = flops / (fwd_ms * 1e-3) / 1e12
    db = decode_bytes(wd)
    dec_gbs = db["total"] / ((split_ms + comb_ms) * 1e-3) / 1e9
    split_gbs = db["split_kernel"] / (split_ms * 1e-3) / 1e9

    # outputs of the timed calls, for the oracle leg (the forward also once with fp32 output)
    outputs = {}
    if oracle_on:
        o32, l32 = fa.fwd(tq, tk, tv, causal=wf.causal, scale=wf.scale, out_f32=True)
        torch.cuda.synchronize()
        outputs[args.fwd_workload] = (wf, (qf, kf, vf), {"bf16": (o.float().cpu().numpy(), lse.cpu().numpy()),
                                                         "f32": (o32.cpu().numpy(), l32.cpu().numpy())})
        del o32, l32
        outputs["decode"] = (wd, (qd, kd, vd), {"bf16": (od.float().cpu().numpy(), ld.cpu().numpy())})

    t_fwd = measured_traffic(f"fa_fwd_{args.fwd_workload}_hbm_traffic.txt", "fwd")
    t_dec = measured_traffic("fa_decode_split_decode_hbm_traffic.txt", "decode")
    rec = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {**wf.describe(), "scale": wf.scale, "k_stress_frac": wf.k_stress_frac, "seed": wf.seed},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_MFMA_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_BF16_TFLOPS, 4), "traffic": t_fwd,
                     "kernel": "fa_fwd_kernel", "avg_kernel_ms": round(fwd_ms, 4),
                     "algorithmic_flops": flops, "algorithmic_bytes": fwd_bytes(wf),
                     "counters": measured_mfma_util("mfma_utilisation_counters.txt", "fwd")
                     if args.fwd_workload == "mha8k" else None},
        "decode": {
            "config": {**wd.describe(), "num_splits": ns, "seed": wd.seed},
            "value": round(dec_gbs, 1), "unit": "GB/s", "ms": round(split_ms + comb_ms, 4),
            "roofline": {"bound": "hbm", "achieved": round(split_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(split_gbs / PEAK_HBM_GBS, 4), "traffic": t_dec,
                         "kernel": "fa_decode_split_kernel", "avg_kernel_ms": round(split_ms, 4),
                         "algorithmic_bytes": db["split_kernel"]},
            "combine_kernel_ms": round(comb_ms, 4), "algorithmic_bytes": db["total"],
        },
        "wall_s_timed": round(t_wall, 3),
        "kernel_source_hash": {f: kernel_source_hash(f) for f in KERNEL_SOURCES},
    }
    if not args.no_other_prefill:
        rec["prefill_other"] = {}
        for key in ("mha2k", "gqa32k"):
            if key == args.fwd_workload:
                continue
            sub, data = prefill_bench(fa, lib, stream, key, WORKLOADS[key], up, args.steps, args.warmup)
            rec["prefill_other"][key] = sub
            if oracle_on:
                outputs[key] = (WORKLOADS[key], data[:3], data[3])
            del data
    if oracle_on and args.fwd_workload != "tiny":
        # the tiny exact-check workload is a parity case only: one call, no timing
        wt = WORKLOADS["tiny"]
        qt, kt, vt = make_workload(wt)
        ot, lt = fa.fwd(up(qt), up(kt), up(vt), causal=wt.causal, scale=wt.scale)
        ot32, lt32 = fa.fwd(up(qt), up(kt), up(vt), causal=wt.causal, scale=wt.scale, out_f32=True)
        torch.cuda.synchronize()
        outputs["tiny"] = (wt, (qt, kt, vt), {"bf16": (ot.float().cpu().numpy(), lt.cpu().numpy()),
                                              "f32": (ot32.cpu().numpy(), lt32.cpu().numpy())})
    if not args.no_bwd:
        rec["backward"] = backward_bench(fa, lib, stream, args.fwd_workload, wf, tq, tk, tv, o, lse, args.steps,
                                         args.warmup)
    if not args.no_bpt:
        rec["blockwise_layer"] = bpt_bench(fa, stream, args.fwd_workload, wf, tq, tk, tv, args.steps, args.warmup)
    if not args.no_fp8:
        rec["fp8_forward"] = fp8_bench(fa, stream, args.fwd_workload, wf, args.steps, args.warmup)
    if not args.no_paged:
        rec["paged_decode"] = paged_decode_bench(fa, dev, stream, args.steps, args.warmup)
    del tq, tk, tv, dq, dk, dv
    if not args.no_ceilings:
        print("[bench] ceiling probes", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        ceil = probe_ceilings(dev, stream)
        rec["ceilings"] = ceil
        rec["roofline"]["frac_of_measured_ceiling"] = round(tflops / ceil["mfma_bf16"]["value"], 4)
        rec["decode"]["roofline"]["frac_of_measured_ceiling"] = round(split_gbs / ceil["hbm_read"]["value"], 4)
        for sub in rec.get("prefill_other", {}).values():
            sub["roofline"]["frac_of_measured_ceiling"] = round(sub["value"] / ceil["mfma_bf16"]["value"], 4)

    rec["cpu_baseline"] = None
    if oracle_on:
        rec["parity"] = {}
        for key, (w, (q, k, v), outs) in outputs.items():
            print(f"[bench] oracle leg: {w.name}", file=sys.stderr, flush=True)
            cpu, par = oracle_leg(key, w, q, k, v, outs)
            if key == args.fwd_workload:
                rec["cpu_baseline"], rec["parity"] = cpu, par
            elif key == "decode":
                rec["decode"]["cpu_baseline"], rec["decode"]["parity"] = cpu, par
            elif key in rec.get("prefill_other", {}):
                rec["prefill_other"][key]["cpu_baseline"], rec["prefill_other"][key]["parity"] = cpu, par
            else:
                rec["parity_only"] = {"config": {**w.describe(), "seed": w.seed}, "parity": par}
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
