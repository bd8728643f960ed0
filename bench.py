#!/usr/bin/env python3
"""Benchmark of the routed-expert MXFP4 MoE layer on one MI355X.

One step = the whole layer (moe_route, moe_build_bitmatrix, moe_expert_offsets,
moe_grouped_ffn_mxfp4, moe_combine) over one batch of seeded synthetic inputs
already resident in HBM.  The default workload is the speculative-decode
verify step: T = 8 tokens (1 + 7 draft), E = 256, k = 6, H = 4096, I = 2048.

Timing: W untimed warm-up steps, then exactly K steps bracketed by
torch.cuda.synchronize() and the host clock.  Inside the timed region, HIP
events recorded on the library's stream time each call and, through the
instrumented FFN entry point, the W1 and W2 kernels on their own.  Two copies
of the expert weights alternate between steps so that a step never finds the
previous step's weights in the 256 MB last-level cache (as in a real model,
where other layers run in between).

Prints ONE JSON line.  Extra fields: per-call microseconds, the roofline of
the dominant kernel (W1: gate|up product + clamped SwiGLU) against the 8 TB/s
HBM peak, and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + µs/layer; % HBM peak (decode), % MFMA peak (prefill)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


class HipEvents:
    """hipEvent_t handles from the HIP runtime (plumbing for timing only)."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.rt.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(h.value)
        return out

    def record(self, ev, stream):
        if self.rt.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b):
        f = ctypes.c_float()
        if self.rt.hipEventElapsedTime(ctypes.byref(f), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value


def measured_traffic(profile_name: str, kernel_source: str):
    """HBM bytes per launch from a committed rocprofv3 summary, or None when the
    kernel source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile_name)
    try:
        fields = dict(line.split(":", 1) for line in open(path) if line.count(":") == 1
                      and line.split(":")[0] in ("traffic_bytes_per_launch",
                                                  "kernel_source_sha256_prefix"))
        want = fields["kernel_source_sha256_prefix"].strip()
        have = hashlib.sha256(open(os.path.join(ROOT, kernel_source), "rb").read()).hexdigest()
        if not have.startswith(want):
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(inp, n_tokens):
    """The oracle, as it stands, on the first n_tokens tokens of the workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:   # pragma: no cover - threadpoolctl missing
        limiter = None
    sub = dict(inp, logits=inp["logits"][:n_tokens], x=inp["x"][:n_tokens])
    t0 = time.perf_counter()
    oracle.moe_layer(sub, 10.0)
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.restore_original_limits()
    return dict(value=n_tokens / dt, unit="tokens/s", cores=1, kind="oracle",
                sample=f"first {n_tokens} of {inp['logits'].shape[0]} tokens, whole layer "
                       f"(route..combine, dequantisation included), numpy with 1 BLAS thread, "
                       f"{dt:.1f} s")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=1, help="0..4 (default 1: decode verify)")
    ap.add_argument("--limit", type=float, default=10.0, help="SwiGLU clamp limit (<=0: off)")
    ap.add_argument("--weight-copies", type=int, default=2)
    ap.add_argument("--cpu-tokens", type=int, default=4,
                    help="tokens in the CPU oracle sample (0: skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of the layer, run a plain device-to-device copy of this many "
                         "MiB (--steps times): the reference for HBM traffic counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer is "
              "built and measured per GPU, see DESIGN.md for how it would shard", file=sys.stderr)
        sys.exit(2)

    import torch
    from mxfp4_routed_expert_route_amd import binding, inputs, layer

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": args.steps}), flush=True)
        return
    lib = binding.load()
    wl = inputs.workload(args.workload)
    T, E, k, H, I = wl.T, wl.E, wl.k, wl.H, wl.I
    print(f"[bench] workload {wl.index} {wl.name}: generating inputs", file=sys.stderr, flush=True)
    inp = inputs.make_inputs(wl.index)
    dev = layer.to_device(inp)
    copies = [dev]
    for _ in range(args.weight_copies - 1):
        copies.append({key: (v.clone() if key.startswith("w") else v) for key, v in dev.items()})
    b = layer.LayerBuffers.allocate(T, E, k, H, I)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    hip = HipEvents()
    n_ev = 8
    events = hip.create(n_ev * args.steps)
    ev_arr = (ctypes.c_void_p * 3)()

    def step(i, evs=None):
        d = copies[i % len(copies)]
        if evs is not None:
            hip.record(evs[0], sh)
        binding.moe_route(d["logits"], k, b.topk_ids, b.topk_weights, stream)
        if evs is not None:
            hip.record(evs[1], sh)
        binding.moe_build_bitmatrix(b.topk_ids, E, b.bitmatrix, stream)
        if evs is not None:
            hip.record(evs[2], sh)
        binding.moe_expert_offsets(b.bitmatrix, b.topk_ids, E, b.counts, b.offsets, b.gather,
                                   b.scatter, b.ws, stream)
        if evs is None:
            binding.moe_grouped_ffn_mxfp4(d["x"], k, d["w1"], d["w1_s"], d["w2"], d["w2_s"],
                                          b.counts, b.offsets, b.gather, args.limit, b.y_sorted,
                                          b.ws, stream)
        else:
            hip.record(evs[3], sh)
            ev_arr[0], ev_arr[1], ev_arr[2] = evs[4], evs[5], evs[6]
            rc = lib.moe_grouped_ffn_mxfp4_timed(
                ctypes.c_void_p(d["x"].data_ptr()), T, H, I, E, k, ctypes.c_void_p(d["w1"].data_ptr()),
                ctypes.c_void_p(d["w1_s"].data_ptr()), ctypes.c_void_p(d["w2"].data_ptr()),
                ctypes.c_void_p(d["w2_s"].data_ptr()), ctypes.c_void_p(b.counts.data_ptr()),
                ctypes.c_void_p(b.offsets.data_ptr()), ctypes.c_void_p(b.gather.data_ptr()),
                ctypes.c_float(args.limit), ctypes.c_void_p(b.y_sorted.data_ptr()),
                ctypes.c_void_p(b.ws.data_ptr()), ctypes.c_size_t(b.ws.numel()), ev_arr,
                ctypes.c_void_p(sh))
            if rc != 0:
                raise binding.MoeError("moe_grouped_ffn_mxfp4_timed", rc)
        binding.moe_combine(b.y_sorted, b.topk_weights, b.scatter, b.y, stream)
        if evs is not None:
            hip.record(evs[7], sh)

    lib.moe_grouped_ffn_mxfp4_timed.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32] + \
        [ctypes.c_void_p] * 7 + [ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                 ctypes.c_void_p, ctypes.c_void_p]
    lib.moe_grouped_ffn_mxfp4_timed.restype = ctypes.c_int

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i * n_ev:(i + 1) * n_ev])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # per-call and per-kernel durations (ms), averaged over the timed steps
    names = ["route", "bitmatrix", "offsets", "ffn_plan", "ffn_w1", "ffn_w2", "combine"]
    per = np.zeros((args.steps, len(names)))
    for i in range(args.steps):
        ev = events[i * n_ev:(i + 1) * n_ev]
        per[i] = [hip.ms(ev[j], ev[j + 1]) for j in range(7)]
    avg_ms = per.mean(axis=0)
    layer_ms_events = float(np.mean([hip.ms(events[i * n_ev], events[i * n_ev + 7])
                                     for i in range(args.steps)]))

    counts = b.counts.cpu().numpy()
    touched = int((counts > 0).sum())
    w1_bytes_per_expert = 2 * I * H // 2 + 2 * I * H // 32
    w2_bytes_per_expert = H * I // 2 + H * I // 32
    w1_alg = touched * w1_bytes_per_expert + T * H * 2
    w1_ms = float(avg_ms[names.index("ffn_w1")])
    achieved = w1_alg / (w1_ms * 1e-3) / 1e9
    layer_alg = touched * (w1_bytes_per_expert + w2_bytes_per_expert) + 2 * T * H * 2 + T * E * 4
    ms_per_step = elapsed * 1e3 / args.steps
    flops = 2.0 * T * k * 3 * H * I

    result = {
        "metric": METRIC,
        "value": T * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "us_per_layer": ms_per_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: T={T} E={E} k={k} H={H} I={I}, MXFP4 experts, "
                               f"seed {wl.index}",
                   "T": T, "E": E, "k": k, "H": H, "I": I, "swiglu_limit": args.limit,
                   "weight_copies": args.weight_copies, "parallelism": "single GPU"},
        "per_call_us": {n: float(v) * 1e3 for n, v in zip(names, avg_ms)},
        "layer_us_events": layer_ms_events * 1e3,
        "touched_experts": touched,
        "roofline": {"bound": "hbm", "kernel": "gemm_kernel<true> (W1 gate|up + SwiGLU)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": (measured_traffic("ffn_w1_stream_verify-1+7.md",
                                                  "mxfp4_routed_expert_route_amd/csrc/ffn.hip")
                                 if wl.index == 1 else None),
                     "algorithmic_bytes_per_launch": w1_alg},
        "layer_hbm_frac": layer_alg / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "ffn_hbm_frac": (touched * (w1_bytes_per_expert + w2_bytes_per_expert))
                        / (float(avg_ms[3:6].sum()) * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "layer_mfma_frac_bf16": flops / (ms_per_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
    }
    if args.cpu_tokens > 0:
        print(f"[bench] CPU oracle on {args.cpu_tokens} tokens", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(inp, min(args.cpu_tokens, T))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
