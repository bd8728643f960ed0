#!/usr/bin/env python3
"""Benchmark of the routed-expert MXFP4 MoE layer on one MI355X.

One step = the whole layer (routing, bit matrix, expert offsets, grouped W1 /
SwiGLU / W2 FFN, weighted combine; one moe_forward_mxfp4 call) over one batch of
seeded synthetic inputs already resident in HBM.  The default run measures the
four full-size workloads in one process, E = 256, k = 6, H = 4096, I = 2048:

  1 verify-1+7     T = 8     one speculative-decode verify step (1 + 7 draft tokens)
  2 burst-64x8     T = 512   64 streams x 8 tokens, nearly every expert touched
  3 prefill-2048   T = 2048  a prefill chunk at a 2,048-token budget
  4 skewed-8191    T = 8191  skewed long-prompt prefill (hot experts ~ T rows)

The headline (metric value, ms_per_step, roofline) is the largest workload,
skewed-8191; the others are reported in "workloads" with their own layer time,
W1 / W2 kernel times and roofline fractions.

Timing, per workload: W untimed warm-up steps, then exactly K steps bracketed by
torch.cuda.synchronize() and the host clock.  Inside the timed region every
event_every-th step runs the instrumented one-call layer (moe_forward_mxfp4_timed:
the same kernels, plus HIP events on the library's stream around the W1 and W2
kernels); with --separate-routing, the separate calls with the instrumented FFN
entry point.  Two copies of the expert weights alternate between steps so that a
step never finds the previous step's weights in the 256 MB last-level cache (as
in a real model, where other layers run in between).

Prints ONE JSON line.  Also: the oracle (CPU) timed on a bounded sample of the
headline workload (its first 16 tokens) and on the whole verify-1+7 layer, with
every BLAS thread, and two achievable-bandwidth markers of the same run (a
device copy and a plain streaming read).
"""
from __future__ import annotations

import argparse
import ctypes
import gc
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + µs/layer; % HBM peak (decode), % MFMA peak (prefill)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
CSRC = "mxfp4_routed_expert_route_amd/csrc"

# Committed rocprofv3 summary per workload: W1 HBM bytes per launch (FETCH_SIZE and
# WRITE_SIZE, scaled by the copy calibration), valid while the digest of the
# kernel sources it names still matches.
PROFILES = {1: "ffn_gemv_verify-1+7.md", 2: "ffn_stream_burst-64x8.md",
            3: "ffn_tile_prefill-2048.md", 4: "ffn_tile_skewed-8191.md"}


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

    def destroy(self, evs):
        for e in evs:
            self.rt.hipEventDestroy(e)

    def record(self, ev, stream):
        if self.rt.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b):
        f = ctypes.c_float()
        if self.rt.hipEventElapsedTime(ctypes.byref(f), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value


def _code_only(text: str) -> str:
    """C/C++ source with comments removed and whitespace runs collapsed, so that a
    comment edit does not read as a kernel change (string literals are not
    special-cased: the kernel sources hold none with comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def sources_digest(paths) -> str:
    """sha256 over the code (comments and whitespace dropped) of the named source
    files, in the order given."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
        h.update(b"\0")
    return h.hexdigest()


def measured_traffic(profile_name: str):
    """W1 HBM bytes per launch from a committed rocprofv3 summary, or None when a
    kernel source it names has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", profile_name)
    try:
        fields = {}
        with open(path) as f:
            for line in f:
                key, sep, val = line.partition(":")
                if sep and key in ("traffic_bytes_per_launch", "kernel_sources",
                                   "kernel_sources_sha256_prefix"):
                    fields[key] = val.strip()
        want = fields["kernel_sources_sha256_prefix"]
        if not want or not sources_digest(fields["kernel_sources"].split()).startswith(want):
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def ffn_kernel_name(T: int, E: int, k: int, H: int, I: int) -> str:
    """The W1 kernel the library picks for these sizes (its row-tile rule; the
    80-row kernel stages E8M0 weight scales in LDS while they fit beside the
    activations in 80 KB, the 128-row kernel weight and activation scales while
    they fit in the CU's 160 KB)."""
    if T * k < E and H in (2048, 4096) and I in (2048, 4096):
        return f"gemv_kernel<true, {H // 2048}>"
    if T <= 16 or T * k // E <= 8:
        return "gemm_stream_kernel<true, 1, true, 2>"
    if T * k // E <= 24:
        return "gemm_stream_kernel<true, 2, true, 4>"
    if T * k // E < 96:
        lds_scales = 2 * 80 * 256 + 2 * 256 * 4 + 4 * (H // 128) * 64 * 4 <= 80 * 1024
        return f"gemm_tile_kernel<true, 5, 4, 4, false, {'true' if lds_scales else 'false'}, false>"
    tiled = H % 2048 == 0 and 2 * 128 * 256 + 128 * (H // 128 + 1) * 4 + 8 * (H // 128) * 64 * 4 <= 160 * 1024
    return f"gemm_tile_kernel<true, 8, 4, 8, false, {'true, true' if tiled else 'false, false'}>"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:   # pragma: no cover - threadpoolctl missing
        return 1


def cpu_model() -> str | None:
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                        None)
    except OSError:
        return None


def cpu_baseline(inp, n_tokens: int, one_thread_tokens: int):
    """The oracle, as it stands, on the first n_tokens tokens of the workload (the
    whole layer: routing, dequantisation, products, combine), with numpy's BLAS
    at its configured thread count; and, as a secondary figure, the same on
    one_thread_tokens tokens with one BLAS thread."""
    import oracle

    def timed(n):
        sub = dict(inp, logits=inp["logits"][:n], x=inp["x"][:n])
        t0 = time.perf_counter()
        oracle.moe_layer(sub, 10.0)
        return time.perf_counter() - t0

    threads = blas_threads()
    dt = timed(n_tokens)
    T = inp["logits"].shape[0]
    out = dict(value=n_tokens / dt, unit="tokens/s", cores=threads, kind="oracle",
               sample=(f"{'all' if n_tokens == T else 'first'} {n_tokens} of {T} tokens of "
                       f"{inp['workload'].name}, whole layer (route..combine, dequantisation "
                       f"included), numpy with {threads} BLAS threads (its elementwise steps "
                       f"run on one thread), {dt:.1f} s"),
               host_cpu=cpu_model(), host_cpu_count=os.cpu_count(), numpy=np.__version__)
    if one_thread_tokens > 0:
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1, user_api="blas"):
                dt1 = timed(one_thread_tokens)
            out["one_thread"] = dict(value=one_thread_tokens / dt1, unit="tokens/s", cores=1,
                                     sample=f"first {one_thread_tokens} tokens, {dt1:.1f} s")
        except Exception:   # pragma: no cover - threadpoolctl missing
            pass
    return out


class Runner:
    """One workload's device inputs, buffers and marshalled ctypes calls."""

    def __init__(self, lib, hip, wl, inp, args):
        import torch
        from mxfp4_routed_expert_route_amd import layer
        self.torch, self.lib, self.hip, self.wl, self.args = torch, lib, hip, wl, args
        T, E, k, H, I = wl.T, wl.E, wl.k, wl.H, wl.I
        dev = layer.to_device(inp)
        self.copies = [dev]
        for _ in range(args.weight_copies - 1):
            self.copies.append({key: (v.clone() if key.startswith("w") else v)
                                for key, v in dev.items()})
        b = self.b = layer.LayerBuffers.allocate(T, E, k, H, I)
        self.S = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self.calls = [self.marshal(d, self.S) for d in self.copies]

    def marshal(self, d, S):
        from ctypes import c_void_p as P, c_float as F
        wl, b = self.wl, self.b
        T, E, k, H, I = wl.T, wl.E, wl.k, wl.H, wl.I
        ptr = lambda t: P(t.data_ptr())
        lim = F(self.args.limit)
        return dict(
            route=(ptr(d["logits"]), T, E, k, ptr(b.topk_ids), ptr(b.topk_weights), S),
            bitmatrix=(ptr(b.topk_ids), T, E, k, ptr(b.bitmatrix), S),
            offsets=(ptr(b.bitmatrix), ptr(b.topk_ids), T, E, k, ptr(b.counts), ptr(b.offsets),
                     ptr(b.gather), ptr(b.scatter), ptr(b.ws), b.ws.numel(), S),
            front=(ptr(d["logits"]), T, E, k, ptr(b.topk_ids), ptr(b.topk_weights),
                   ptr(b.bitmatrix), ptr(b.counts), ptr(b.offsets), ptr(b.gather),
                   ptr(b.scatter), ptr(b.ws), b.ws.numel(), S),
            ffn=(ptr(d["x"]), T, H, I, E, k, ptr(d["w1"]), ptr(d["w1_s"]), ptr(d["w2"]),
                 ptr(d["w2_s"]), ptr(b.counts), ptr(b.offsets), ptr(b.gather), lim,
                 ptr(b.y_sorted), ptr(b.ws), b.ws.numel()),
            combine=(ptr(b.y_sorted), ptr(b.topk_weights), ptr(b.scatter), T, H, k, ptr(b.y), S),
            forward=(ptr(d["logits"]), ptr(d["x"]), T, H, I, E, k, ptr(d["w1"]), ptr(d["w1_s"]),
                     ptr(d["w2"]), ptr(d["w2_s"]), lim, ptr(b.topk_ids), ptr(b.topk_weights),
                     ptr(b.bitmatrix), ptr(b.counts), ptr(b.offsets), ptr(b.gather),
                     ptr(b.scatter), ptr(b.y_sorted), ptr(b.y), ptr(b.ws), b.ws.numel(), S))

    def step(self, i, evs=None, ffn_events=None, c=None):
        """One layer.  evs: 8 events around every call (breakdown pass only: the
        separate calls); ffn_events: the 3 events inside the FFN step.  Without evs
        (and with the default routing) the layer is one moe_forward_mxfp4 call, or
        one moe_forward_mxfp4_timed call with ffn_events."""
        lib, S, sep = self.lib, self.S, self.args.separate_routing
        c = self.calls[i % len(self.calls)] if c is None else c
        record = self.hip.rt.hipEventRecord

        def check(rc, name):
            if rc != 0:
                from mxfp4_routed_expert_route_amd import binding
                raise binding.MoeError(name, rc)

        if evs is None and not sep:
            if ffn_events is None:
                check(lib.moe_forward_mxfp4(*c["forward"]), "moe_forward_mxfp4")
            else:
                check(lib.moe_forward_mxfp4_timed(*c["forward"][:-1], ffn_events,
                                                  c["forward"][-1]), "moe_forward_mxfp4_timed")
            return
        if evs is not None:
            record(evs[0], S)
        if sep:
            check(lib.moe_route(*c["route"]), "moe_route")
            if evs is not None:
                record(evs[1], S)
            check(lib.moe_build_bitmatrix(*c["bitmatrix"]), "moe_build_bitmatrix")
            if evs is not None:
                record(evs[2], S)
            check(lib.moe_expert_offsets(*c["offsets"]), "moe_expert_offsets")
        else:
            check(lib.moe_route_and_group(*c["front"]), "moe_route_and_group")
            if evs is not None:
                record(evs[1], S)
                record(evs[2], S)
        if evs is not None:
            record(evs[3], S)
        if ffn_events is None:
            check(lib.moe_grouped_ffn_mxfp4(*c["ffn"], c["combine"][-1]), "moe_grouped_ffn_mxfp4")
        else:
            check(lib.moe_grouped_ffn_mxfp4_timed(*c["ffn"], ffn_events, c["combine"][-1]),
                  "moe_grouped_ffn_mxfp4_timed")
        check(lib.moe_combine(*c["combine"]), "moe_combine")
        if evs is not None:
            record(evs[7], S)

    def measure(self):
        torch, hip, args, wl = self.torch, self.hip, self.args, self.wl
        T, E, k, H, I = wl.T, wl.E, wl.k, wl.H, wl.I
        tag = f"[bench] workload {wl.index} {wl.name}"
        ev_null = (ctypes.c_void_p * 3)(*hip.create(3))
        print(f"{tag}: warmup {args.warmup} steps", file=sys.stderr, flush=True)
        for i in range(args.warmup):
            self.step(i, ffn_events=ev_null if i % 2 else None)
        torch.cuda.synchronize()

        # Timed region: exactly K steps.  Every event_every-th step runs the
        # instrumented FFN call (three events: plan | W1 | W2 on the library's stream).
        # The event steps are the last of each group of event_every (never the first
        # step after the synchronisation, which runs with the clocks still rising).
        every = max(1, args.event_every)
        ffn_ev = [(ctypes.c_void_p * 3)(*hip.create(3)) for _ in range(args.steps // every)]
        if not ffn_ev:
            ffn_ev = [(ctypes.c_void_p * 3)(*hip.create(3))]
        ev_at = {min(args.steps, every * (j + 1)) - 1: j for j in range(len(ffn_ev))}
        print(f"{tag}: timing {args.steps} steps", file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            self.step(i, ffn_events=ffn_ev[ev_at[i]] if i in ev_at else None)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        w1_ms = float(np.mean([hip.ms(e[0], e[1]) for e in ffn_ev]))
        w2_ms = float(np.mean([hip.ms(e[1], e[2]) for e in ffn_ev]))

        # Graph pass (not the timed region): the layer captured once per weight copy
        # as a HIP graph on a side stream, then replayed back to back.
        graph_us = None
        if args.graph_steps > 0:
            gstream = torch.cuda.Stream()
            gcalls = [self.marshal(d, ctypes.c_void_p(gstream.cuda_stream)) for d in self.copies]
            graphs = []
            for gc_ in gcalls:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=gstream):
                    self.step(0, c=gc_)
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
            del graphs

        # Breakdown pass (not timed as a whole): events around every call.
        n_ev = 8
        n_bd = min(args.steps, 20)
        events = hip.create(n_ev * n_bd)
        # the FFN call records its three events (plan | W1 | W2) into slots 4..6
        ev_arrs = [(ctypes.c_void_p * 3)(*events[i * n_ev + 4:i * n_ev + 7]) for i in range(n_bd)]
        for i in range(n_bd):
            self.step(i, events[i * n_ev:(i + 1) * n_ev], ev_arrs[i])
        torch.cuda.synchronize()
        names = ["route", "bitmatrix", "offsets", "ffn_plan", "ffn_w1", "ffn_w2", "combine"]
        if not args.separate_routing:   # one call for the three routing steps
            names[0:3] = ["route_and_group", "-", "-"]
        per = np.zeros((n_bd, len(names)))
        for i in range(n_bd):
            ev = events[i * n_ev:(i + 1) * n_ev]
            per[i] = [hip.ms(ev[j], ev[j + 1]) for j in range(7)]
        avg_ms = per.mean(axis=0)
        layer_ev_us = np.array([hip.ms(events[i * n_ev], events[i * n_ev + 7])
                                for i in range(n_bd)]) * 1e3
        hip.destroy(events)

        counts = self.b.counts.cpu().numpy()
        touched = int((counts > 0).sum())
        w1_pe = 2 * I * H // 2 + 2 * I * H // 32          # W1 codes + E8M0 scales per expert
        w2_pe = H * I // 2 + H * I // 32
        # + x read once, h written once (2 bytes per element; the tiled kernels' two-part
        # FP8 form adds one scale byte per 32 elements, not counted)
        w1_alg = touched * w1_pe + T * H * 2 + T * k * I * 2
        layer_alg = touched * (w1_pe + w2_pe) + 2 * T * H * 2 + T * E * 4
        ms_per_step = elapsed * 1e3 / args.steps
        w1_flops = 2.0 * T * k * 2 * I * H
        layer_flops = 2.0 * T * k * 3 * H * I
        hbm_gbs = w1_alg / (w1_ms * 1e-3) / 1e9
        tflops = w1_flops / (w1_ms * 1e-3) / 1e12
        kname = "W1 gate|up + clamped SwiGLU (" + ffn_kernel_name(T, E, k, H, I) + ")"
        traffic = measured_traffic(PROFILES[wl.index]) if wl.index in PROFILES else None
        # The W1 kernel's bound: its FLOPs per algorithmic byte against the ratio of
        # the two peaks (bf16 ridge: 312.5 FLOP/B).  Decode and the 48-row prefill
        # sit below it (HBM); experts with hundreds of rows sit above it (MFMA).
        if w1_flops / w1_alg > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
            roofline = {"bound": "mfma", "kernel": kname, "achieved": tflops,
                        "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": tflops / BF16_PEAK_TFLOPS, "traffic": traffic,
                        "algorithmic_flops_per_launch": w1_flops,
                        "algorithmic_bytes_per_launch": w1_alg}
        else:
            roofline = {"bound": "hbm", "kernel": kname, "achieved": hbm_gbs,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": hbm_gbs / HBM_PEAK_GBS,
                        "traffic": traffic, "algorithmic_bytes_per_launch": w1_alg,
                        "mfma_frac_bf16": tflops / BF16_PEAK_TFLOPS}
        out = {
            "workload": f"{wl.name}: T={T} E={E} k={k} H={H} I={I}, MXFP4 experts, seed {wl.index}",
            "T": T, "steps": args.steps, "warmup": args.warmup,
            "tokens_per_s": T * args.steps / elapsed,
            "ms_per_step": ms_per_step, "us_per_layer": ms_per_step * 1e3,
            "ffn_w1_us": w1_ms * 1e3, "ffn_w2_us": w2_ms * 1e3,
            "touched_experts": touched, "max_rows_per_expert": int(counts.max()),
            "roofline": roofline,
            "w2_hbm_frac": touched * w2_pe / (w2_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "ffn_hbm_frac": touched * (w1_pe + w2_pe) / ((w1_ms + w2_ms) * 1e-3) / 1e9
                            / HBM_PEAK_GBS,
            "layer_hbm_frac": layer_alg / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "layer_mfma_frac_bf16": layer_flops / (ms_per_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "layer_algorithmic_bytes": layer_alg, "layer_flops": layer_flops,
            "per_call_us": {n: float(v) * 1e3 for n, v in zip(names, avg_ms) if n != "-"},
            "graph_us_per_layer": graph_us,
            "layer_us_with_events_p10_p50_p90": [float(np.percentile(layer_ev_us, q))
                                                 for q in (10, 50, 90)],
        }
        print(f"{tag}: {out['us_per_layer']:.1f} us/layer, W1 {out['ffn_w1_us']:.1f} us, "
              f"W2 {out['ffn_w2_us']:.1f} us", file=sys.stderr, flush=True)
        return out

    def free(self):
        del self.copies, self.calls, self.b
        gc.collect()
        self.torch.cuda.empty_cache()


def markers(mib: int):
    """Achievable-HBM markers of the same run: a plain device copy (read + write
    bytes over its time) and the library's plain streaming read (moe_read_probe)."""
    import torch
    from mxfp4_routed_expert_route_amd import binding
    n = mib << 20
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
    sink = torch.empty(binding.READ_PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
    binding.moe_read_probe(src, sink)
    torch.cuda.synchronize()
    c0 = time.perf_counter()
    for _ in range(10):
        binding.moe_read_probe(src, sink)
    torch.cuda.synchronize()
    read_gbs = n * 10 / (time.perf_counter() - c0) / 1e9
    return copy_gbs, read_gbs


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # the clocks settle over the first few ms of steady work (verify layer: ~112 us
    # per step over the first 100 steps after setup, ~105.5 after)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workloads", default="1,2,3,4",
                    help="comma-separated workload indices 0..4 (default: the four full-size ones)")
    ap.add_argument("--workload", type=int, default=None,
                    help="measure this one workload only (same as --workloads N)")
    ap.add_argument("--headline", type=int, default=None,
                    help="the workload of the headline figures (default: the largest measured)")
    ap.add_argument("--limit", type=float, default=10.0, help="SwiGLU clamp limit (<=0: off)")
    ap.add_argument("--weight-copies", type=int, default=2)
    ap.add_argument("--cpu-tokens", type=int, default=16,
                    help="tokens of the headline workload in the CPU oracle sample (0: skip)")
    ap.add_argument("--cpu-workload", type=int, default=1,
                    help="workload whose whole layer the CPU oracle is also timed on, reported "
                         "with that workload (-1: skip)")
    ap.add_argument("--cpu-one-thread-tokens", type=int, default=4,
                    help="tokens of that workload in a secondary one-BLAS-thread sample (0: skip)")
    ap.add_argument("--separate-routing", action="store_true",
                    help="route with moe_route + moe_build_bitmatrix + moe_expert_offsets instead "
                         "of the fused moe_route_and_group (same outputs)")
    ap.add_argument("--event-every", type=int, default=10,
                    help="in the timed region, every n-th step runs the call that records "
                         "HIP events around W1 and W2 (the three event records cost ~10 us of "
                         "GPU time per instrumented step on the verify layer, so the others run "
                         "without)")
    ap.add_argument("--graph-steps", type=int, default=100,
                    help="after the timed region, replay the layer captured as HIP graphs this "
                         "many times and report graph_us_per_layer (0: skip)")
    ap.add_argument("--copy-marker-mib", type=int, default=1024,
                    help="device copy and plain read of this many MiB timed after the layers, as "
                         "the achievable-HBM markers of the same run (0: skip)")
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
    from mxfp4_routed_expert_route_amd import binding, inputs

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
                       ("moe_forward_mxfp4_timed", [P, P, I64, I32, I32, I32, I32, P, P, P, P,
                                                    F] + [P] * 10 + [SZ, P, P]),
                       ("moe_combine", [P, P, P, I64, I32, I32, P, P])):
        getattr(lib, name).argtypes = argt
        getattr(lib, name).restype = ctypes.c_int
    hip = HipEvents()

    order = [args.workload] if args.workload is not None else \
        [int(s) for s in args.workloads.split(",") if s.strip()]
    headline = args.headline if args.headline is not None else max(order)
    if headline not in order:
        order.append(headline)
    results, cpu = {}, None
    for index in order:
        wl = inputs.workload(index)
        print(f"[bench] workload {index} {wl.name}: generating inputs", file=sys.stderr,
              flush=True)
        inp = inputs.make_inputs(index)
        run = Runner(lib, hip, wl, inp, args)
        results[index] = run.measure()
        run.free()
        del run
        if index == headline and args.cpu_tokens > 0:
            n = min(args.cpu_tokens, wl.T)
            print(f"[bench] CPU oracle on {n} tokens of {wl.name}", file=sys.stderr, flush=True)
            cpu = cpu_baseline(inp, n, 0)
        if index == args.cpu_workload:
            print(f"[bench] CPU oracle on the whole {wl.name} layer", file=sys.stderr, flush=True)
            results[index]["cpu_baseline"] = cpu_baseline(
                inp, wl.T, min(args.cpu_one_thread_tokens, wl.T))
        del inp
        gc.collect()

    copy_gbs = read_gbs = None
    if args.copy_marker_mib > 0:
        copy_gbs, read_gbs = markers(args.copy_marker_mib)

    h = results[headline]
    hw = inputs.workload(headline)
    result = {
        "metric": METRIC,
        "value": h["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "us_per_layer": h["us_per_layer"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": h["workload"], "T": hw.T, "E": hw.E, "k": hw.k, "H": hw.H,
                   "I": hw.I, "swiglu_limit": args.limit, "weight_copies": args.weight_copies,
                   "parallelism": "single GPU",
                   "calls": ("moe_route + moe_build_bitmatrix + moe_expert_offsets + "
                             "moe_grouped_ffn_mxfp4 + moe_combine" if args.separate_routing else
                             "moe_forward_mxfp4 (every event_every-th step: "
                             "moe_forward_mxfp4_timed)")},
        "roofline": h["roofline"],
        "event_every": max(1, args.event_every),
        "workloads": {inputs.workload(i).name: r for i, r in results.items()},
        "hbm_copy_marker_gbs": copy_gbs,
        "hbm_read_marker_gbs": read_gbs,
    }
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
