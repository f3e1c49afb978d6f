"""Benchmark: causal grouped-query attention on one MI355X.

One step = one pass of the whole hot path on the two GQA 32q/8kv d128
workloads: the causal prefill (B=4, Hq=32, Hkv=8, T=4096, bf16) through
gqa_attn_fwd, then the split-KV decode (B=64, Hq=32, Hkv=8, Tmax=8192,
lengths uniform in [1024, 8192]) through gqa_attn_decode.  Inputs are seeded
synthetic N(0,1) tensors already resident in HBM.  `value` is the prefill
throughput in TFLOP/s (algorithmic FLOPs: 2*(Dk+Dv) per visible causal
(query, key) pair per query head); the decode KV read rate is reported next
to it.  Per-kernel times come from HIP events recorded on the stream the
library launches on (torch's current stream); `value` and the roofline
figures use the median launch, the mean is reported beside it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import statistics
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
METRIC = "prefill attn TFLOP/s & %MFMA peak; decode KV GB/s & %HBM peak (GQA 32q/8kv d128)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "fwd_bf16_kernel": ["causal_grouped_query_amd/csrc/fwd_bf16.hip",
                        "causal_grouped_query_amd/csrc/device_common.h"],
    "decode_bf16_flat_kernel": ["causal_grouped_query_amd/csrc/decode_bf16.hip",
                                "causal_grouped_query_amd/csrc/combine.hip",
                                "causal_grouped_query_amd/csrc/device_common.h"],
}


def causal_pairs(Tq: int, Tk: int) -> int:
    off = Tk - Tq
    return sum(min(Tk, off + i + 1) for i in range(Tq))


def fwd_flops(w) -> float:
    return 2.0 * (w.Dk + w.Dv) * causal_pairs(w.Tq, w.Tk) * w.Hq * w.B


def varlen_flops(w) -> float:
    """Visible (query, key) pairs of a packed sliding-window workload: a query
    at position p of its sequence sees min(p + 1, window) keys."""
    win = w.extra["window"]
    pairs = 0
    for n in w.extra["lens"]:
        full = min(n, win)
        pairs += full * (full + 1) // 2 + (n - full) * win
    return 2.0 * (w.Dk + w.Dv) * pairs * w.Hq


def decode_bytes(w, lens) -> float:
    per_key = w.Dk if w.kind == "mla_decode" else (w.Dk + w.Dv)  # MLA: V is the latent prefix of K
    return float(sum(lens)) * w.Hkv * per_key * 2


def fp8_decode_bytes(w, lens) -> float:
    """Bytes an FP8-cache decode must read: one byte per cached element of K
    and V, plus one fp32 scale per K row and per V row."""
    return float(sum(lens)) * w.Hkv * ((w.Dk + w.Dv) * 1 + 2 * 4)


def topk_bytes(w, sel_rows) -> float:
    """Latent rows a top-k decode must gather: the selected positions of each
    sequence, 576 bf16 values each (the value is inside the key)."""
    return float(sum(sel_rows)) * w.Dk * 2


def decode_flops(w, lens) -> float:
    return 2.0 * (w.Dk + w.Dv) * float(sum(lens)) * w.Hq


def source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, launches_per_unit: int = 1):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel source changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_sha") != source_sha(kernel):
        return None
    return t["bytes_per_launch"]


PROFILE_WORKLOADS = ("prefill", "decode", "mqa", "mla", "topk", "topk64", "swa", "fp8", "shard", "merge", "probes")


def _profile_call(torch, gqa, W, dev, name):
    """Inputs in HBM and a zero-argument launch of one workload (for counter
    passes: one call per step, nothing else on the GPU)."""
    if name in ("prefill", "mqa"):
        w = W.GQA_PREFILL if name == "prefill" else W.MQA_SUFFIX
        sets = []
        for wv in (w, dataclasses.replace(w, seed=w.seed + 100)):
            q, k, v = (t.to(dev) for t in W.fwd_inputs(wv))
            sets.append((q, k, v, torch.empty((w.B, w.Hq, w.Tq, w.Dv), dtype=torch.bfloat16, device=dev)))
        turn = [0]

        def fn():
            q, k, v, out = sets[turn[0] % 2]
            turn[0] += 1
            gqa.attention(q, k, v, scale=w.scale, causal=True, out=out)
        return fn, {"workload": w.name, "flop_per_call": fwd_flops(w)}
    if name == "swa":
        w = W.SWA_VARLEN
        q, k, v, cu = (t.to(dev) for t in W.varlen_inputs(w))
        out = torch.empty((q.shape[0], w.Hq, w.Dv), dtype=torch.bfloat16, device=dev)
        return (lambda: gqa.attention_varlen(q, k, v, cu, cu, scale=w.scale, causal=True, window=w.extra["window"],
                                             out=out)), {"workload": w.name, "flop_per_call": varlen_flops(w)}
    if name in ("decode", "mla"):
        w = W.GQA_DECODE if name == "decode" else W.MLA_DECODE
        q, kc, vc, lens = W.decode_inputs(w, nan_tail=False)
        q, kc, lens_d = q.to(dev), kc.to(dev), lens.to(dev)
        vc = kc[..., : w.Dv] if name == "mla" else vc.to(dev)
        out = torch.empty((w.B, w.Hq, 1, w.Dv), dtype=torch.bfloat16, device=dev)
        S = gqa.decode_splits(w.B, w.Hq, w.Hkv, w.Tk, w.Dk, w.Dv, gqa.GQA_BF16)
        ws = torch.empty(gqa.decode_workspace_size(w.B, w.Hq, w.Dv, S), dtype=torch.uint8, device=dev)
        return (lambda: gqa.decode(q, kc, vc, lens_d, scale=w.scale, num_splits=S, out=out, workspace=ws)), {
            "workload": w.name, "kv_bytes_per_call": decode_bytes(w, lens.tolist()), "splits": S}
    if name == "fp8":
        w = W.GQA_DECODE_FP8
        q, kc, vc, ks, vs, lens = W.fp8_decode_inputs(w, nan_tail=False)
        lens_l = lens.tolist()
        q, kc, vc, ks, vs, lens = (t.to(dev) for t in (q, kc, vc, ks, vs, lens))
        out = torch.empty((w.B, w.Hq, 1, w.Dv), dtype=torch.bfloat16, device=dev)
        S = gqa.decode_fp8_splits(w.B, w.Hq, w.Hkv, w.Tk, w.Dk, w.Dv)
        ws = torch.empty(gqa.decode_workspace_size(w.B, w.Hq, w.Dv, S), dtype=torch.uint8, device=dev)
        return (lambda: gqa.decode_fp8(q, kc, vc, ks, vs, lens, scale=w.scale, num_splits=S, out=out,
                                       workspace=ws)), {"workload": w.name,
                                                        "kv_bytes_per_call": fp8_decode_bytes(w, lens_l)}
    if name in ("topk", "topk64"):
        w = W.MLA_TOPK if name == "topk" else W.MLA_TOPK_B64
        fn, S, sel_rows = _topk_call(torch, gqa, W, dev, w)
        return fn, {"workload": w.name, "kv_bytes_per_call": topk_bytes(w, sel_rows), "splits": S}
    if name in ("shard", "merge"):
        # one device's key shard under sequence parallelism (the heaviest: every
        # key visible to every query), and the merge of all shards' partials
        w = W.CP_SHARD
        nsh, q_pos0 = w.extra["shards"], w.extra["q_pos0"]
        q = W.fwd_inputs(w)[0].to(dev)
        outs = torch.empty((nsh, w.B, w.Hq, w.Tq, w.Dv), dtype=torch.float32, device=dev)
        lses = torch.empty((nsh, w.B, w.Hq, w.Tq), dtype=torch.float32, device=dev)
        kv0 = None
        for r in range(nsh):
            _, k, v = W.fwd_inputs(dataclasses.replace(w, seed=w.seed + 10 * r))
            k, v = k.to(dev), v.to(dev)
            gqa.attention_shard(q, k, v, q_pos0, r * w.Tk, scale=w.scale, out=outs[r], lse=lses[r])
            kv0 = kv0 or (k, v)
        if name == "shard":
            k0, v0 = kv0
            return (lambda: gqa.attention_shard(q, k0, v0, q_pos0, 0, scale=w.scale, out=outs[0], lse=lses[0])), {
                "workload": w.name, "flop_per_call": 2.0 * (w.Dk + w.Dv) * w.Tq * w.Tk * w.Hq * w.B}
        merged = torch.empty((w.B, w.Hq, w.Tq, w.Dv), dtype=torch.bfloat16, device=dev)
        mb = float(outs.numel() * 4 + lses.numel() * 4 + merged.numel() * 2)
        return (lambda: gqa.merge(outs, lses, out=merged)), {
            "workload": "context_parallel_merge_8_shards_262144_rows_d128", "kv_bytes_per_call": mb}
    raise ValueError(name)


def _topk_call(torch, gqa, W, dev, w):
    """A top-k decode call over eight selections in turn (one selection's rows
    would be served from the Infinity Cache after the first call).  Batch 16
    draws its inputs as the parity tests do; the batch-64 cache (2.4 GB) is
    drawn on the device, for timing only."""
    if w.B <= 16:
        q, kc, _, lens = W.decode_inputs(w, nan_tail=False)
        q, kc = q.to(dev), kc.to(dev)
    else:
        lens = W.decode_lengths(w)
        g = torch.Generator(device=dev).manual_seed(w.seed)
        q = torch.randn((w.B, w.Hq, 1, w.Dk), generator=g, device=dev).to(torch.bfloat16)
        kc = torch.empty((w.B, 1, w.Tk, w.Dk), dtype=torch.bfloat16, device=dev)
        for b in range(w.B):  # one sequence at a time: no 4.8 GB fp32 temporary
            kc[b].copy_(torch.randn((1, w.Tk, w.Dk), generator=g, device=dev))
    sels = [W.topk_indices(dataclasses.replace(w, seed=w.seed + 10 * i), lens).to(dev) for i in range(8)]
    sel_rows = [min(w.extra["topk"], n) for n in lens.tolist()]
    lens_d = lens.to(dev)
    out = torch.empty((w.B, w.Hq, 1, w.Dv), dtype=torch.bfloat16, device=dev)
    S = gqa.decode_topk_splits(w.B, w.Hq, w.extra["topk"], w.Dk, w.Dv, gqa.GQA_BF16)
    ws = torch.empty(gqa.decode_workspace_size(w.B, w.Hq, w.Dv, S), dtype=torch.uint8, device=dev)
    turn = [0]

    def fn():
        idx = sels[turn[0] % len(sels)]
        turn[0] += 1
        gqa.decode_topk(q, kc, lens_d, idx, scale=w.scale, num_splits=S, out=out, workspace=ws)
    return fn, S, sel_rows


def profile_one(torch, gqa, W, dev, name, steps, warmup) -> int:
    """Launch one workload warmup + steps times (nothing else), time the
    timed calls with HIP events on the launch stream, print one JSON line."""
    fn, info = _profile_call(torch, gqa, W, dev, name)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    us = [a.elapsed_time(b) * 1e3 for a, b in ev]
    med = statistics.median(us)
    info.update({"profile": name, "calls": steps, "median_us": round(med, 2), "mean_us": round(sum(us) / len(us), 2)})
    if "flop_per_call" in info:
        info["TFLOP/s"] = round(info["flop_per_call"] / med / 1e6, 1)
        info["frac_mfma_peak"] = round(info["TFLOP/s"] / PEAK_BF16_TFLOPS, 4)
    if "kv_bytes_per_call" in info:
        info["GB/s"] = round(info["kv_bytes_per_call"] / med / 1e3, 1)
        info["frac_hbm_peak"] = round(info["GB/s"] / PEAK_HBM_GBPS, 4)
    print(json.dumps(info), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the MQA-suffix / sliding-window varlen / MLA / fp32 workloads")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--profile", choices=sorted(PROFILE_WORKLOADS), default=None,
                    help="only launch this workload's kernels (warmup + steps calls, for rocprofv3 passes)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path (KV-head groups would "
              "split across GPUs without communication; key shards would exchange (o, lse) partials and "
              "merge them with gqa_attn_merge).", file=sys.stderr)
        return 2

    import torch
    import causal_grouped_query_amd as gqa
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        return 2
    gqa.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")

    if args.copy_calibration:
        # a plain copy of known size: reads 1 GiB, writes 1 GiB per launch
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return 0

    if args.profile == "probes":
        print(json.dumps(probe_context(torch, dev)), flush=True)
        return 0
    if args.profile:
        return profile_one(torch, gqa, W, dev, args.profile, args.steps, args.warmup)

    # ---------------- inputs (seeded, synthetic, resident in HBM) ----------------
    # The prefill alternates between two input sets (seeds s and s + 100) so
    # that the 256 MB Infinity Cache cannot serve a step's inputs from the
    # previous step; the decode cache (1.2 GB read per step) exceeds it anyway.
    wp, wd = W.GQA_PREFILL, W.GQA_DECODE
    pre_sets = []
    for wv in (wp, dataclasses.replace(wp, seed=wp.seed + 100)):
        q, k, v = (t.to(dev) for t in W.fwd_inputs(wv))
        pre_sets.append((q, k, v, torch.empty((wp.B, wp.Hq, wp.Tq, wp.Dv), dtype=torch.bfloat16, device=dev)))
    dq, dk, dv, lens_cpu = W.decode_inputs(wd, nan_tail=False)
    dq, dk, dv = dq.to(dev), dk.to(dev), dv.to(dev)
    lens = lens_cpu.to(dev)
    dout = torch.empty((wd.B, wd.Hq, 1, wd.Dv), dtype=torch.bfloat16, device=dev)
    S = gqa.decode_splits(wd.B, wd.Hq, wd.Hkv, wd.Tk, wd.Dk, wd.Dv, gqa.GQA_BF16)
    ws = torch.empty(gqa.decode_workspace_size(wd.B, wd.Hq, wd.Dv, S), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    step_no = [0]

    def prefill():
        q, k, v, out = pre_sets[step_no[0] % 2]
        gqa.attention(q, k, v, scale=wp.scale, causal=True, out=out)

    def decode():
        gqa.decode(dq, dk, dv, lens, scale=wd.scale, num_splits=S, out=dout, workspace=ws)

    for _ in range(args.warmup):
        prefill()
        decode()
        step_no[0] += 1
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record()
        prefill()
        ev[i][1].record()
        decode()
        ev[i][2].record()
        step_no[0] += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_pre = sum(e[0].elapsed_time(e[1]) for e in ev) / K * 1e-3
    t_dec = sum(e[1].elapsed_time(e[2]) for e in ev) / K * 1e-3
    t_pre_med = statistics.median(e[0].elapsed_time(e[1]) for e in ev) * 1e-3
    t_dec_med = statistics.median(e[1].elapsed_time(e[2]) for e in ev) * 1e-3
    ms_step = ev[0][0].elapsed_time(ev[-1][2]) / K

    F = fwd_flops(wp)
    lens_list = lens_cpu.tolist()
    DB = decode_bytes(wd, lens_list)
    # rates at the median launch (the mean is reported beside it)
    pre_tflops = F / t_pre_med / 1e12
    dec_gbps = DB / t_dec_med / 1e9

    tr = traffic_for("fwd_bf16_kernel")
    roofline = {
        "kernel": "fwd_bf16_kernel<128> (gqa_attn_fwd, one launch per step)",
        "bound": "mfma", "achieved": round(pre_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
        "frac": round(pre_tflops / PEAK_BF16_TFLOPS, 4), "traffic": tr,
        "median_launch_us": round(t_pre_med * 1e6, 2), "avg_launch_us": round(t_pre * 1e6, 2),
        "frac_at_avg": round(F / t_pre / 1e12 / PEAK_BF16_TFLOPS, 4),
        "flop_per_launch": F,
    }
    trd = traffic_for("decode_bf16_flat_kernel")
    roofline_decode = {
        "kernel": f"decode_bf16_flat_kernel<128,128> + combine_kernel (gqa_attn_decode, balanced, {S} slots)",
        "bound": "hbm", "achieved": round(dec_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
        "frac": round(dec_gbps / PEAK_HBM_GBPS, 4), "traffic": trd,
        "median_launch_us": round(t_dec_med * 1e6, 2), "avg_launch_us": round(t_dec * 1e6, 2),
        "frac_at_avg": round(DB / t_dec / 1e9 / PEAK_HBM_GBPS, 4),
        "kv_bytes_per_launch": DB, "sum_len": int(sum(lens_list)),
    }

    result = {
        "metric": METRIC,
        "value": round(pre_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), cast to bf16; decode lengths uniform [1024, 8192])",
        "config": {
            "workload": f"{wp.name} + {wd.name}",
            "prefill": {"B": wp.B, "Hq": wp.Hq, "Hkv": wp.Hkv, "Tq": wp.Tq, "Tk": wp.Tk, "D": wp.Dk,
                        "causal": True},
            "decode": {"B": wd.B, "Hq": wd.Hq, "Hkv": wd.Hkv, "Tmax": wd.Tk, "D": wd.Dk, "splits": S},
        },
        "prefill_tflops": round(pre_tflops, 2),
        "prefill_frac_mfma_peak": round(pre_tflops / PEAK_BF16_TFLOPS, 4),
        "decode_kv_GBps": round(dec_gbps, 1),
        "decode_frac_hbm_peak": round(dec_gbps / PEAK_HBM_GBPS, 4),
        "roofline": roofline,
        "roofline_decode": roofline_decode,
        "wall_s_timed": round(wall, 4),
    }

    # free the headline inputs before the extra workloads
    del pre_sets, dq, dk, dv, dout, ws
    torch.cuda.empty_cache()
    result["context"] = {"hbm_copy_GBps": copy_bandwidth(torch, dev),
                         "bf16_gemm_TFLOPs": gemm_rate(torch, dev),
                         "probes": probe_context(torch, dev),
                         "note": "plain 1 GiB device-to-device copy (reads + writes), the practical HBM rate; "
                                 "8192^3 bf16 GEMM through torch (hipBLASLt), a practical dense-MFMA rate "
                                 "under the board power limit"}

    if not args.no_extra:
        result["extra"] = extra_workloads(torch, gqa, W, dev)

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)

    print(json.dumps(result), flush=True)
    return 0


def _time(torch, fn, reps=10, warm=3):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps * 1e-3


def copy_bandwidth(torch, dev) -> float:
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    sec = _time(torch, lambda: dst.copy_(src), reps=5, warm=2)
    del src, dst
    return round(2 * n / sec / 1e9, 1)


def probe_context(torch, dev) -> dict:
    """Ceilings measured on this GPU by the probe kernels (libgqa_probes.so):
    a pure v_mfma_f32_32x32x16_bf16 loop (8 independent chains per wave, every
    CU) on seeded N(0,1) bf16 operands and on zeros, and a global_load_lds
    stream of 2 GiB through LDS with no arithmetic.  Each reports the shader
    clock it ran at (s_memtime cycles per 100 MHz s_memrealtime tick,
    median over workgroups)."""
    import ctypes
    path = os.path.join(ROOT, "causal_grouped_query_amd", "libgqa_probes.so")
    L = ctypes.CDLL(path)
    P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.gqa_probe_mfma_bf16.restype = I
    L.gqa_probe_mfma_bf16.argtypes = [P, I, P, P, I, I, I, P]
    L.gqa_probe_stream_lds.restype = I
    L.gqa_probe_stream_lds.argtypes = [P, SZ, I, I, P, P]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def clock_ghz(clk):
        c = clk.view(-1, 4).cpu().double()
        ghz = (c[:, 1] - c[:, 0]) / ((c[:, 3] - c[:, 2]) * 10.0)  # cycles per ns (realtime is 100 MHz)
        return round(float(ghz.median()), 3)

    res = {}
    n_ops = 4096
    g = torch.Generator("cpu").manual_seed(11)
    ops_rand = torch.randn(n_ops * 64 * 8, generator=g).to(torch.bfloat16).to(dev)
    ops_zero = torch.zeros_like(ops_rand)
    grid, waves, iters = 256, 8, 40000  # one resident round: 2 waves per SIMD
    out = torch.empty(grid * waves * 64, dtype=torch.float32, device=dev)
    clk = torch.zeros(grid * 4, dtype=torch.int64, device=dev)
    flop = 32768.0 * 8 * iters * grid * waves
    for name, ops in (("n01", ops_rand), ("zeros", ops_zero)):
        best = None
        for _ in range(3):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            rc = L.gqa_probe_mfma_bf16(ops.data_ptr(), n_ops, out.data_ptr(), clk.data_ptr(), grid, waves, iters,
                                       stream)
            e.record()
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError("MFMA probe launch failed")
            sec = s.elapsed_time(e) * 1e-3
            if best is None or sec < best[0]:
                best = (sec, clock_ghz(clk))
        sec, ghz = best
        tf = flop / sec / 1e12
        res[f"mfma_bf16_{name}"] = {"TFLOP/s": round(tf, 1), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                                    "shader_clock_GHz": ghz,
                                    "frac_peak_at_clock": round(tf / (PEAK_BF16_TFLOPS * ghz / 2.4), 4)}
    del ops_rand, ops_zero, out
    nbytes, grid_s = 2 << 30, 2048
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    clk = torch.zeros(grid_s * 4, dtype=torch.int64, device=dev)
    best = None
    for _ in range(4):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        rc = L.gqa_probe_stream_lds(src.data_ptr(), nbytes // grid_s, grid_s, 1, clk.data_ptr(), stream)
        e.record()
        torch.cuda.synchronize()
        if rc != 0:
            raise RuntimeError("stream probe launch failed")
        sec = s.elapsed_time(e) * 1e-3
        if best is None or sec < best[0]:
            best = (sec, clock_ghz(clk))
    res["stream_global_load_lds"] = {"GB/s": round(nbytes / best[0] / 1e9, 1),
                                     "frac_peak": round(nbytes / best[0] / 1e9 / PEAK_HBM_GBPS, 4),
                                     "shader_clock_GHz": best[1], "bytes": nbytes}
    del src
    res["note"] = ("probe kernels: dense 32x32x16 bf16 MFMA loop on every CU (2 waves per SIMD, 8 independent "
                   "chains each) and a read-only HBM -> LDS stream; shader clock from s_memtime / s_memrealtime")
    return res


def gemm_rate(torch, dev) -> float:
    n = 8192
    g = torch.Generator(device=dev).manual_seed(7)
    a = torch.randn(n, n, device=dev, generator=g).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev, generator=g).to(torch.bfloat16)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    sec = _time(torch, lambda: torch.matmul(a, b, out=c), reps=20, warm=5)
    del a, b, c
    return round(2.0 * n ** 3 / sec / 1e12, 1)


def extra_workloads(torch, gqa, W, dev):
    """The other headline shapes, timed the same way (not part of the step)."""
    res = {}
    w = W.MQA_SUFFIX
    # two input sets in turn: one set (201 MB) would fit the Infinity Cache
    sets = []
    for wv in (w, dataclasses.replace(w, seed=w.seed + 100)):
        q, k, v = (t.to(dev) for t in W.fwd_inputs(wv))
        sets.append((q, k, v, torch.empty((w.B, w.Hq, w.Tq, w.Dv), dtype=torch.bfloat16, device=dev)))
    turn = [0]

    def mqa():
        q, k, v, out = sets[turn[0] % 2]
        turn[0] += 1
        gqa.attention(q, k, v, scale=w.scale, out=out)

    sec = _time(torch, mqa)
    f = fwd_flops(w)
    res[w.name] = {"us": round(sec * 1e6, 1), "TFLOP/s": round(f / sec / 1e12, 1),
                   "frac_mfma_peak": round(f / sec / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del sets

    w = W.SWA_VARLEN
    q, k, v, cu = W.varlen_inputs(w)
    q, k, v, cu = q.to(dev), k.to(dev), v.to(dev), cu.to(dev)
    out = torch.empty((q.shape[0], w.Hq, w.Dv), dtype=torch.bfloat16, device=dev)
    sec = _time(torch, lambda: gqa.attention_varlen(q, k, v, cu, cu, scale=w.scale, causal=True,
                                                    window=w.extra["window"], out=out))
    f = varlen_flops(w)
    res[w.name] = {"us": round(sec * 1e6, 1), "TFLOP/s": round(f / sec / 1e12, 1),
                   "frac_mfma_peak": round(f / sec / 1e12 / PEAK_BF16_TFLOPS, 4),
                   "flop_per_launch": f, "sequences": list(w.extra["lens"]), "window": w.extra["window"]}
    del q, k, v, cu, out

    w = W.MLA_DECODE
    q, kc, _, lens = W.decode_inputs(w, nan_tail=False)
    q, kc, lens_d = q.to(dev), kc.to(dev), lens.to(dev)
    out = torch.empty((w.B, w.Hq, 1, w.Dv), dtype=torch.bfloat16, device=dev)
    S = gqa.decode_splits(w.B, w.Hq, w.Hkv, w.Tk, w.Dk, w.Dv, gqa.GQA_BF16)
    ws = torch.empty(gqa.decode_workspace_size(w.B, w.Hq, w.Dv, S), dtype=torch.uint8, device=dev)
    sec = _time(torch, lambda: gqa.decode(q, kc, kc[..., : w.Dv], lens_d, scale=w.scale, num_splits=S, out=out,
                                          workspace=ws))
    b = decode_bytes(w, lens.tolist())
    f = decode_flops(w, lens.tolist())
    res[w.name] = {"us": round(sec * 1e6, 1), "GB/s": round(b / sec / 1e9, 1),
                   "frac_hbm_peak": round(b / sec / 1e9 / PEAK_HBM_GBPS, 4),
                   "TFLOP/s": round(f / sec / 1e12, 1), "frac_mfma_peak": round(f / sec / 1e12 / PEAK_BF16_TFLOPS, 4),
                   "splits": S}
    del q, kc, out, ws

    # the GQA decode shape with a 4096-key sliding window (each query reads
    # only the last min(len, 4096) keys of its full-length cache)
    w, win = W.GQA_DECODE, 4096
    q, kc, vc, lens = W.decode_inputs(w, nan_tail=False)
    q, kc, vc, lens_d = q.to(dev), kc.to(dev), vc.to(dev), lens.to(dev)
    out = torch.empty((w.B, w.Hq, 1, w.Dv), dtype=torch.bfloat16, device=dev)
    S = gqa.decode_splits(w.B, w.Hq, w.Hkv, w.Tk, w.Dk, w.Dv, gqa.GQA_BF16)
    ws = torch.empty(gqa.decode_workspace_size(w.B, w.Hq, w.Dv, S), dtype=torch.uint8, device=dev)
    sec = _time(torch, lambda: gqa.decode(q, kc, vc, lens_d, scale=w.scale, num_splits=S, out=out, workspace=ws,
                                          window=win))
    wl = [min(n, win) for n in lens.tolist()]
    b = decode_bytes(w, wl)
    res["gqa_decode_swa_w4096_b64_hq32_hkv8_tmax8192_d128"] = {
        "us": round(sec * 1e6, 1), "GB/s": round(b / sec / 1e9, 1), "frac_hbm_peak": round(b / sec / 1e9 / PEAK_HBM_GBPS, 4),
        "window": win, "kv_bytes_per_launch": b}
    del q, kc, vc, out, ws

    w = W.GQA_DECODE_FP8
    q, kc, vc, ks, vs, lens = W.fp8_decode_inputs(w, nan_tail=False)
    q, kc, vc, ks, vs, lens_d = (t.to(dev) for t in (q, kc, vc, ks, vs, lens))
    out = torch.empty((w.B, w.Hq, 1, w.Dv), dtype=torch.bfloat16, device=dev)
    S = gqa.decode_fp8_splits(w.B, w.Hq, w.Hkv, w.Tk, w.Dk, w.Dv)
    ws = torch.empty(gqa.decode_workspace_size(w.B, w.Hq, w.Dv, S), dtype=torch.uint8, device=dev)
    sec = _time(torch, lambda: gqa.decode_fp8(q, kc, vc, ks, vs, lens_d, scale=w.scale, num_splits=S, out=out,
                                              workspace=ws))
    b = fp8_decode_bytes(w, lens.tolist())
    res[w.name] = {"us": round(sec * 1e6, 1), "GB/s": round(b / sec / 1e9, 1),
                   "frac_hbm_peak": round(b / sec / 1e9 / PEAK_HBM_GBPS, 4), "splits": S,
                   "kv_bytes_per_launch": b, "tokens_per_s": round(float(sum(lens.tolist())) / sec, 1)}
    del q, kc, vc, ks, vs, out, ws

    for w in (W.MLA_TOPK, W.MLA_TOPK_B64):
        topk, S, sel_rows = _topk_call(torch, gqa, W, dev, w)
        sec = _time(torch, topk, reps=16, warm=8)
        b = topk_bytes(w, sel_rows)
        f = decode_flops(w, sel_rows)
        res[w.name] = {"us": round(sec * 1e6, 1), "GB/s": round(b / sec / 1e9, 1),
                       "frac_hbm_peak": round(b / sec / 1e9 / PEAK_HBM_GBPS, 4),
                       "TFLOP/s": round(f / sec / 1e12, 2),
                       "frac_mfma_peak": round(f / sec / 1e12 / PEAK_BF16_TFLOPS, 4), "splits": S, "topk": w.extra["topk"],
                       "kv_bytes_per_launch": b}
        del topk
        torch.cuda.empty_cache()

    w = W.CP_SHARD
    nsh, q_pos0 = w.extra["shards"], w.extra["q_pos0"]
    q, _, _ = W.fwd_inputs(w)
    q = q.to(dev)
    outs = torch.empty((nsh, w.B, w.Hq, w.Tq, w.Dv), dtype=torch.float32, device=dev)
    lses = torch.empty((nsh, w.B, w.Hq, w.Tq), dtype=torch.float32, device=dev)
    shards = []
    for r in range(nsh):  # every device's shard once, for real partials to merge
        _, k, v = W.fwd_inputs(dataclasses.replace(w, seed=w.seed + 10 * r))
        k, v = k.to(dev), v.to(dev)
        gqa.attention_shard(q, k, v, q_pos0, r * w.Tk, scale=w.scale, out=outs[r], lse=lses[r])
        shards.append((k, v))
    k0, v0 = shards[0]  # the heaviest shard: every key visible to every query
    sec = _time(torch, lambda: gqa.attention_shard(q, k0, v0, q_pos0, 0, scale=w.scale, out=outs[0], lse=lses[0]))
    f = 2.0 * (w.Dk + w.Dv) * w.Tq * w.Tk * w.Hq * w.B
    merged = torch.empty((w.B, w.Hq, w.Tq, w.Dv), dtype=torch.bfloat16, device=dev)
    msec = _time(torch, lambda: gqa.merge(outs, lses, out=merged))
    mb = float(outs.numel() * 4 + lses.numel() * 4 + merged.numel() * 2)
    res[w.name] = {"shard_us": round(sec * 1e6, 1), "shard_TFLOP/s": round(f / sec / 1e12, 1),
                   "shard_frac_mfma_peak": round(f / sec / 1e12 / PEAK_BF16_TFLOPS, 4),
                   "merge_us": round(msec * 1e6, 1), "merge_GB/s": round(mb / msec / 1e9, 1),
                   "merge_frac_hbm_peak": round(mb / msec / 1e9 / PEAK_HBM_GBPS, 4), "shards": nsh,
                   "merge_bytes": mb}
    del q, outs, lses, shards, k0, v0, merged

    w = W.TINY_F32
    q, k, v = (t.to(dev) for t in W.fwd_inputs(w))
    sec = _time(torch, lambda: gqa.attention(q, k, v, scale=w.scale))
    res[w.name] = {"us": round(sec * 1e6, 1), "note": "parity-only fp32 workload"}
    torch.cuda.empty_cache()
    return res


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(target_s: float):
    """The fp64 oracle as it stands, on this host's cores, on all five headline
    workloads with the same seeded inputs: the tiny fp32 one and the GQA decode
    in full, the GQA prefill, MQA suffix and absorbed-MLA decode on a random
    row sample of about target_s / 3 seconds each.  Rates are the workload's
    algorithmic FLOPs of the rows done per second; `value` is the GQA
    prefill's, in the unit of the metric."""
    import numpy as np
    import workloads as W
    from oracle import oracle as O

    threads = O.max_threads()
    rng = np.random.default_rng(12345)
    per = {}

    def run(name, q, k, v, scale, flops_of_row, n_rows, lens=None, budget=None):
        """Rows of one workload, all of them or a sampled stream of batches
        until the budget is spent; returns the per-workload record."""
        done_rows, done_flops, elapsed, batch = 0, 0.0, 0.0, 4 * threads
        while done_rows < n_rows and (budget is None or elapsed < budget):
            if budget is None:
                rows = np.arange(n_rows, dtype=np.int64)
            else:
                rows = rng.integers(0, n_rows, size=min(batch, n_rows))
            t0 = time.perf_counter()
            O.attention(q, k, v, scale, True, kv_lens=lens, rows=rows, threads=threads)
            elapsed += time.perf_counter() - t0
            done_rows += rows.size
            done_flops += float(sum(flops_of_row(int(r)) for r in rows))
            if budget is not None:
                # next batch: twice this one, but no more than the rest of the budget at the rate so far
                rate = done_rows / elapsed
                batch = max(threads, min(2 * batch, int(rate * (budget - elapsed))))
        per[name] = {"GFLOP/s": round(done_flops / elapsed / 1e9, 3), "seconds": round(elapsed, 2),
                     "rows": int(done_rows), "rows_total": int(n_rows),
                     "sample": "all rows" if budget is None else "uniform random rows"}
        return per[name]

    def fwd_row_flops(w):
        off = w.Tk - w.Tq
        return lambda r: 2.0 * (w.Dk + w.Dv) * min(w.Tk, off + r % w.Tq + 1)

    each = target_s / 3.0
    # tiny fp32: prefill rows, then its decode step (the last query over all keys)
    w = W.TINY_F32
    q, k, v = W.fwd_inputs(w)
    run(w.name, q, k, v, w.scale, fwd_row_flops(w), w.B * w.Hq * w.Tq)
    # GQA prefill (the metric's workload): sampled rows
    w = W.GQA_PREFILL
    q, k, v = W.fwd_inputs(w)
    head = run(w.name, q, k, v, w.scale, fwd_row_flops(w), w.B * w.Hq * w.Tq, budget=each)
    del q, k, v
    # GQA decode: every (sequence, head) row over its cached length
    w = W.GQA_DECODE
    q, k, v, lens = W.decode_inputs(w, nan_tail=False)
    ll = lens.tolist()
    run(w.name, q, k, v, w.scale, lambda r: 2.0 * (w.Dk + w.Dv) * ll[r // w.Hq], w.B * w.Hq, lens=ll)
    del q, k, v
    # MQA suffix: sampled rows
    w = W.MQA_SUFFIX
    q, k, v = W.fwd_inputs(w)
    run(w.name, q, k, v, w.scale, fwd_row_flops(w), w.B * w.Hq * w.Tq, budget=each)
    del q, k, v
    # absorbed MLA decode (V is the latent prefix of K): sampled rows
    w = W.MLA_DECODE
    q, k, v, lens = W.decode_inputs(w, nan_tail=False)
    ll = lens.tolist()
    run(w.name, q, k, v, w.scale, lambda r: 2.0 * (w.Dk + w.Dv) * ll[r // w.Hq], w.B * w.Hq, lens=ll,
        budget=each)
    del q, k, v
    return {
        "value": head["GFLOP/s"] / 1e3,
        "unit": "TFLOP/s",
        "cores": threads,
        "cpu_model": _cpu_model(),
        "kind": "oracle",
        "sample": (f"{head['rows']} uniformly drawn query rows (of {head['rows_total']}) of {W.GQA_PREFILL.name}, "
                   f"fp64, {head['seconds']} s; all five workloads under 'configs'"),
        "configs": per,
    }


if __name__ == "__main__":
    sys.exit(main())
