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


def ffn_kernel_name(T: int, E: int, k: int, H: int) -> str:
    """The W1 kernel the library picks for these sizes (its row-tile rule; the
    80-row kernel stages E8M0 scales in LDS while they fit beside the activations
    in 80 KB, the 128-row kernel while they fit in the CU's 160 KB)."""
    if T <= 16 or T * k // E <= 8:
        return "gemm_stream_kernel<true, 1, true, 2>"
    if T * k // E <= 24:
        return "gemm_stream_kernel<true, 2, true, 4>"
    if T * k // E < 96:
        lds_scales = 2 * 80 * 272 + 4 * (H // 128) * 64 * 4 <= 80 * 1024
        return f"gemm_tile_kernel<true, 5, 4, 4, {'true' if lds_scales else 'false'}>"
    lds_scales = 2 * 128 * 272 + 8 * (H // 128) * 64 * 4 <= 160 * 1024
    return f"gemm_tile_kernel<true, 8, 4, 8, {'true' if lds_scales else 'false'}>"


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
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f
                              if ln.startswith("model name")), None)
    except OSError:
        pass
    return dict(value=n_tokens / dt, unit="tokens/s", cores=1, kind="oracle",
                sample=f"first {n_tokens} of {inp['logits'].shape[0]} tokens, whole layer "
                       f"(route..combine, dequantisation included), numpy with 1 BLAS thread, "
                       f"{dt:.1f} s",
                host_cpu=cpu_model, host_cpu_count=os.cpu_count(), numpy=np.__version__)


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
    ap.add_argument("--separate-routing", action="store_true",
                    help="route with moe_route + moe_build_bitmatrix + moe_expert_offsets instead "
                         "of the fused moe_route_and_group (same outputs)")
    ap.add_argument("--event-every", type=int, default=10,
                    help="in the timed region, every n-th step runs the FFN call that records "
                         "HIP events around W1 and W2 (an event costs GPU time, so the others "
                         "run without)")
    ap.add_argument("--graph-steps", type=int, default=200,
                    help="after the timed region, replay the layer captured as HIP graphs this "
                         "many times and report graph_us_per_layer (0: skip)")
    ap.add_argument("--copy-marker-mib", type=int, default=1024,
                    help="device-to-device copy timed after the layer, as the achievable-HBM "
                         "marker of the same run (0: skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of the layer, run a plain device-to-device copy of this many "
                         "MiB (--steps times): the reference for HBM traffic counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the layer is "
              "built and measured on a single GPU; sharding it by expert across GPUs is not "
              "implemented", file=sys.stderr)
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

    # Arguments are marshalled once per weight copy, so the timed loop makes only bare
    # ctypes calls (a slower host loop would leave the GPU idle between launches).
    from ctypes import c_void_p as P, c_int64 as I64, c_int32 as I32, c_size_t as SZ, c_float as F
    for name, argt in (("moe_route", [P, I64, I32, I32, P, P, P]),
                       ("moe_build_bitmatrix", [P, I64, I32, I32, P, P]),
                       ("moe_expert_offsets", [P, P, I64, I32, I32, P, P, P, P, P, SZ, P]),
                       ("moe_route_and_group", [P, I64, I32, I32] + [P] * 8 + [SZ, P]),
                       ("moe_grouped_ffn_mxfp4_timed", [P, I64, I32, I32, I32, I32] + [P] * 7 +
                        [F, P, P, SZ, P, P]),
                       ("moe_grouped_ffn_mxfp4", [P, I64, I32, I32, I32, I32] + [P] * 7 +
                        [F, P, P, SZ, P]),
                       ("moe_forward_mxfp4", [P, P, I64, I32, I32, I32, I32, P, P, P, P, F] +
                        [P] * 10 + [SZ, P]),
                       ("moe_combine", [P, P, P, I64, I32, I32, P, P])):
        getattr(lib, name).argtypes = argt
        getattr(lib, name).restype = ctypes.c_int
    ptr = lambda t: P(t.data_ptr())
    ev_arrs = [(ctypes.c_void_p * 3)(*events[i * n_ev + 4:i * n_ev + 7]) for i in range(args.steps)]
    ev_null = (ctypes.c_void_p * 3)(*hip.create(3))
    S = P(sh)

    def marshal(d, S):
        return dict(
            route=(ptr(d["logits"]), T, E, k, ptr(b.topk_ids), ptr(b.topk_weights), S),
            bitmatrix=(ptr(b.topk_ids), T, E, k, ptr(b.bitmatrix), S),
            offsets=(ptr(b.bitmatrix), ptr(b.topk_ids), T, E, k, ptr(b.counts), ptr(b.offsets),
                     ptr(b.gather), ptr(b.scatter), ptr(b.ws), b.ws.numel(), S),
            front=(ptr(d["logits"]), T, E, k, ptr(b.topk_ids), ptr(b.topk_weights),
                   ptr(b.bitmatrix), ptr(b.counts), ptr(b.offsets), ptr(b.gather),
                   ptr(b.scatter), ptr(b.ws), b.ws.numel(), S),
            ffn=(ptr(d["x"]), T, H, I, E, k, ptr(d["w1"]), ptr(d["w1_s"]), ptr(d["w2"]),
                 ptr(d["w2_s"]), ptr(b.counts), ptr(b.offsets), ptr(b.gather), F(args.limit),
                 ptr(b.y_sorted), ptr(b.ws), b.ws.numel()),
            combine=(ptr(b.y_sorted), ptr(b.topk_weights), ptr(b.scatter), T, H, k, ptr(b.y), S),
            forward=(ptr(d["logits"]), ptr(d["x"]), T, H, I, E, k, ptr(d["w1"]), ptr(d["w1_s"]),
                     ptr(d["w2"]), ptr(d["w2_s"]), F(args.limit), ptr(b.topk_ids),
                     ptr(b.topk_weights), ptr(b.bitmatrix), ptr(b.counts), ptr(b.offsets),
                     ptr(b.gather), ptr(b.scatter), ptr(b.y_sorted), ptr(b.y), ptr(b.ws),
                     b.ws.numel(), S))

    calls = [marshal(d, S) for d in copies]
    record = hip.rt.hipEventRecord
    f_route, f_bm, f_offs = lib.moe_route, lib.moe_build_bitmatrix, lib.moe_expert_offsets
    f_front, f_ffn, f_comb = lib.moe_route_and_group, lib.moe_grouped_ffn_mxfp4_timed, lib.moe_combine
    f_ffn_plain, f_forward = lib.moe_grouped_ffn_mxfp4, lib.moe_forward_mxfp4

    def check(rc, name):
        if rc != 0:
            raise binding.MoeError(name, rc)

    def step(i, evs=None, ffn_events=None, c=None):
        """One layer.  evs: 8 events around every call (breakdown pass only);
        ffn_events: the 3 events inside the FFN call.  With neither (and the default
        routing), the layer is one moe_forward_mxfp4 call."""
        c = calls[i % len(calls)] if c is None else c
        if evs is None and ffn_events is None and not args.separate_routing:
            check(f_forward(*c["forward"]), "moe_forward_mxfp4")
            return
        if evs is not None:
            record(evs[0], S)
        if args.separate_routing:
            check(f_route(*c["route"]), "moe_route")
            if evs is not None:
                record(evs[1], S)
            check(f_bm(*c["bitmatrix"]), "moe_build_bitmatrix")
            if evs is not None:
                record(evs[2], S)
            check(f_offs(*c["offsets"]), "moe_expert_offsets")
        else:
            check(f_front(*c["front"]), "moe_route_and_group")
            if evs is not None:
                record(evs[1], S)
                record(evs[2], S)
        if evs is not None:
            record(evs[3], S)
        if ffn_events is None:
            check(f_ffn_plain(*c["ffn"], c["combine"][-1]), "moe_grouped_ffn_mxfp4")
        else:
            check(f_ffn(*c["ffn"], ffn_events, c["combine"][-1]), "moe_grouped_ffn_mxfp4_timed")
        check(f_comb(*c["combine"]), "moe_combine")
        if evs is not None:
            record(evs[7], S)

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i, ffn_events=ev_null if i % 2 else None)
    torch.cuda.synchronize()

    # Timed region: K steps.  Every event_every-th step runs the instrumented FFN
    # call, which records three events (plan | W1 | W2) on the library's stream;
    # W1 and W2 durations are averaged over those steps.
    every = max(1, args.event_every)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    ffn_ev = [(ctypes.c_void_p * 3)(*hip.create(3)) for _ in range(0, args.steps, every)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, ffn_events=ffn_ev[i // every] if i % every == 0 else None)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    w1_ms = float(np.mean([hip.ms(e[0], e[1]) for e in ffn_ev]))
    w2_ms = float(np.mean([hip.ms(e[1], e[2]) for e in ffn_ev]))

    # Graph pass (not the timed region): the layer captured once per weight copy as a
    # HIP graph on a side stream, then replayed back to back.
    graph_us = None
    if args.graph_steps > 0:
        gstream = torch.cuda.Stream()
        gcalls = [marshal(d, P(gstream.cuda_stream)) for d in copies]
        graphs = []
        for gc in gcalls:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=gstream):
                step(0, c=gc)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(min(args.warmup, 20)):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        g0 = time.perf_counter()
        for i in range(args.graph_steps):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        graph_us = (time.perf_counter() - g0) * 1e6 / args.graph_steps

    # Breakdown pass (not timed as a whole): events around every call.
    n_bd = min(args.steps, 20)
    for i in range(n_bd):
        step(i, events[i * n_ev:(i + 1) * n_ev], ev_arrs[i])
    torch.cuda.synchronize()
    names = ["route", "bitmatrix", "offsets", "ffn_plan", "ffn_w1", "ffn_w2", "combine"]
    if not args.separate_routing:   # one call for the three routing steps
        names[0:3] = ["route_and_group", "-", "-"]
    per = np.zeros((n_bd, len(names)))
    for i in range(n_bd):
        ev = events[i * n_ev:(i + 1) * n_ev]
        per[i] = [hip.ms(ev[j], ev[j + 1]) for j in range(7)]
    avg_ms = per.mean(axis=0)
    layer_ev_us = np.array([hip.ms(events[i * n_ev], events[i * n_ev + 7]) for i in range(n_bd)]) * 1e3

    # Achievable-HBM markers of the same run: a plain device copy (read + write
    # bytes over its time) and a plain streaming read (moe_read_probe).
    copy_gbs = read_gbs = None
    if args.copy_marker_mib > 0:
        n = args.copy_marker_mib << 20
        src = torch.zeros(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        c0 = time.perf_counter()
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        copy_gbs = 2 * n * 10 / (time.perf_counter() - c0) / 1e9
        del dst
        # and a plain streaming read of the same bytes (the library's read probe)
        sink = torch.empty(binding.READ_PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
        binding.moe_read_probe(src, sink)
        torch.cuda.synchronize()
        c0 = time.perf_counter()
        for _ in range(10):
            binding.moe_read_probe(src, sink)
        torch.cuda.synchronize()
        read_gbs = n * 10 / (time.perf_counter() - c0) / 1e9
        del src, sink

    counts = b.counts.cpu().numpy()
    touched = int((counts > 0).sum())
    w1_bytes_per_expert = 2 * I * H // 2 + 2 * I * H // 32
    w2_bytes_per_expert = H * I // 2 + H * I // 32
    w1_alg = touched * w1_bytes_per_expert + T * H * 2
    achieved = w1_alg / (w1_ms * 1e-3) / 1e9
    layer_alg = touched * (w1_bytes_per_expert + w2_bytes_per_expert) + 2 * T * H * 2 + T * E * 4
    ms_per_step = elapsed * 1e3 / args.steps
    flops = 2.0 * T * k * 3 * H * I
    # The W1 kernel's bound: its FLOPs per algorithmic byte against the ratio of
    # the two peaks (bf16 ridge: 312.5 FLOP/B).  Decode and the 48-row prefill sit
    # below it (HBM); experts with hundreds of rows sit above it (MFMA).
    w1_flops = 2.0 * T * k * 2 * I * H
    kname = "W1 gate|up + clamped SwiGLU (" + ffn_kernel_name(T, E, k, H) + ")"
    if w1_flops / w1_alg > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        tflops = w1_flops / (w1_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": kname, "achieved": tflops,
                    "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tflops / BF16_PEAK_TFLOPS,
                    "traffic": None, "algorithmic_flops_per_launch": w1_flops,
                    "algorithmic_bytes_per_launch": w1_alg}
    else:
        roofline = {"bound": "hbm", "kernel": kname, "achieved": achieved, "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                    "traffic": (measured_traffic("ffn_w1_stream_verify-1+7.md",
                                                 "mxfp4_routed_expert_route_amd/csrc/ffn_stream.hip")
                                if wl.index == 1 else None),
                    "algorithmic_bytes_per_launch": w1_alg}

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
                   "weight_copies": args.weight_copies, "parallelism": "single GPU",
                   "calls": ("moe_route + moe_build_bitmatrix + moe_expert_offsets + "
                             "moe_grouped_ffn_mxfp4 + moe_combine" if args.separate_routing else
                             "moe_forward_mxfp4 (every event_every-th step: moe_route_and_group + "
                             "moe_grouped_ffn_mxfp4_timed + moe_combine)")},
        "per_call_us": {n: float(v) * 1e3 for n, v in zip(names, avg_ms) if n != "-"},
        "per_call_note": "separate pass with events around every call (events add a few us each)",
        "event_every": every,
        "graph_us_per_layer": graph_us,
        "layer_us_with_events_p10_p50_p90": [float(np.percentile(layer_ev_us, q)) for q in (10, 50, 90)],
        "hbm_copy_marker_gbs": copy_gbs,
        "hbm_read_marker_gbs": read_gbs,
        "ffn_w1_us_timed": w1_ms * 1e3,
        "ffn_w2_us_timed": w2_ms * 1e3,
        "touched_experts": touched,
        "roofline": roofline,
        "layer_hbm_frac": layer_alg / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "ffn_hbm_frac": (touched * (w1_bytes_per_expert + w2_bytes_per_expert))
                        / ((w1_ms + w2_ms) * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "layer_mfma_frac_bf16": flops / (ms_per_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
    }
    if args.cpu_tokens > 0:
        print(f"[bench] CPU oracle on {args.cpu_tokens} tokens", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(inp, min(args.cpu_tokens, T))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
