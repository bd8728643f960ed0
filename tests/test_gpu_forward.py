"""moe_forward_mxfp4 (the whole layer in one call) against the separate calls.

Every output must match the separate-call chain (moe_route_and_group,
moe_grouped_ffn_mxfp4, moe_combine) bit for bit: the same kernels run, except
that the routing side also writes the FFN's row-tile plan in place of the FFN's
plan kernel: the one-launch front-end for T <= 64, the one-workgroup
expert-offsets kernel up to 512 tokens (two experts per thread), the
expert-offsets scan above; and on the decode GEMV path (fewer routed rows than
experts, H and I of 2048 or 4096) W2 and the weighted combine run as one launch
with the same arithmetic.  The cases cover each tile kind the plan can hold
(one-row GEMV tiles, 16- and 32-row streaming tiles, 80-row LDS tiles; 128-row
tiles, which need more than 64 tokens) on both sides of the T = 64 front-end
limit, and T = 0.  moe_forward_mxfp4_timed must give the same outputs again.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from mxfp4_routed_expert_route_amd import inputs
from tests.test_gpu_parity import tiny

pytestmark = pytest.mark.gpu

OUTPUTS = ("topk_ids", "topk_weights", "bitmatrix", "counts", "offsets", "gather", "scatter",
           "y_sorted", "y")


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _compare(inp, limit=10.0):
    from mxfp4_routed_expert_route_amd import binding, layer
    binding.load()
    wl = inp["workload"]
    T = inp["logits"].shape[0]
    print(f"[forward] T={T} E={wl.E} k={wl.k} H={wl.H} I={wl.I}", file=sys.stderr, flush=True)
    dev = layer.to_device(inp)
    a = layer.LayerBuffers.allocate(T, wl.E, wl.k, wl.H, wl.I)
    b = layer.LayerBuffers.allocate(T, wl.E, wl.k, wl.H, wl.I)
    for buf in (a, b):   # stale values must not leak into either result
        for name in OUTPUTS:
            _bits(getattr(buf, name)).fill_(-3)
        buf.ws.fill_(0x5A)
    layer.run_layer(dev, a, limit, fused=True)
    layer.run_forward(dev, b, limit)
    torch.cuda.synchronize()
    for name in OUTPUTS:
        assert torch.equal(_bits(getattr(a, name)), _bits(getattr(b, name))), name


@pytest.mark.parametrize("index", [0, 1, 2, 3, 4])   # 2: the offsets kernel writes the
                                                     # plan; 3, 4: the scan
def test_forward_matches_separate_calls_workloads(index):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _compare(inputs.make_inputs(index))


@pytest.mark.parametrize("T,E,k,H,I,seed", [
    (1, 256, 6, 256, 128, 41),       # one token, 16-row tiles
    (40, 8, 1, 128, 128, 42),        # 5 rows per expert: 16-row tiles, several per expert
    (64, 24, 7, 256, 128, 43),       # 18.7 rows per expert: 32-row tiles, front-end plan
    (64, 16, 8, 256, 256, 44),       # 32 rows per expert: 80-row LDS tiles, front-end plan,
                                     # x split by its own launch
    (65, 16, 8, 256, 256, 45),       # past the one-launch limit: the offsets kernel's plan,
                                     # x split by extra workgroups of the routing launch
    (300, 8, 3, 256, 256, 48),       # 112 rows per expert: 128-row tiles, offsets kernel
    (100, 256, 6, 256, 128, 51),     # 16-row tiles for 2.3 rows per expert, offsets kernel
    (200, 64, 6, 256, 128, 52),      # 18.75 rows per expert: 32-row tiles, offsets kernel
    (300, 32, 6, 256, 256, 53),      # 56 rows per expert: 80-row tiles, offsets kernel
    (500, 1024, 8, 128, 128, 54),    # maximum E: every thread holds two experts
    (130, 40, 5, 128, 128, 55),      # E not a multiple of 64 (odd expert count per wave)
    (600, 16, 2, 256, 256, 49),      # past one offsets block (512 tokens): the scan writes
                                     # the plan (80-row tiles)
    (1100, 8, 3, 256, 256, 50),      # three offsets blocks, 128-row tiles from the scan's plan
    (33, 1024, 8, 128, 128, 46),     # maximum E and k
    (7, 16, 2, 2048, 2048, 56),      # GEMV path: W2 + combine in one launch, k = 2
    (5, 16, 1, 2048, 2048, 57),      # GEMV path, k = 1
    (1, 16, 8, 2048, 2048, 58),      # GEMV path, k = 8 (the maximum)
    (3, 16, 3, 2048, 4096, 59),      # GEMV path, W2 over K = 4096 (two slices), k odd
    (2, 16, 5, 4096, 2048, 60),      # GEMV path, H = 4096
    (1, 16, 8, 2048, 4096, 61),      # GEMV path, W2 K = 4096 and k = 8: 64 KB of h in LDS
])
def test_forward_matches_separate_calls(T, E, k, H, I, seed):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _compare(tiny(T, E, k, H, I, seed))


def test_forward_empty_batch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mxfp4_routed_expert_route_amd import binding, layer
    binding.load()
    inp = tiny(0, 64, 6, 256, 128, 47)
    dev = layer.to_device(inp)
    b = layer.LayerBuffers.allocate(0, 64, 6, 256, 128)
    b.counts.fill_(-7)
    b.offsets.fill_(-7)
    layer.run_forward(dev, b, 10.0)
    torch.cuda.synchronize()
    assert (b.counts.cpu().numpy() == 0).all() and (b.offsets.cpu().numpy() == 0).all()


def _hip_events(n):
    import ctypes
    rt = ctypes.CDLL("libamdhip64.so")
    rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                       ctypes.c_void_p]
    rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = []
    for _ in range(n):
        h = ctypes.c_void_p()
        assert rt.hipEventCreate(ctypes.byref(h)) == 0
        evs.append(h.value)

    def ms(a, b):
        f = ctypes.c_float()
        assert rt.hipEventElapsedTime(ctypes.byref(f), a, b) == 0
        return f.value
    return rt, evs, ms


@pytest.mark.parametrize("case", ["verify", "tiled"])
def test_forward_timed_matches_forward(case):
    """The instrumented one-call layer: the same outputs bit for bit, and its three
    events in order on the stream (W1 and W2 each take a positive time)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mxfp4_routed_expert_route_amd import binding, layer
    binding.load()
    inp = inputs.make_inputs(1) if case == "verify" else tiny(300, 32, 6, 256, 256, 53)
    wl = inp["workload"]
    T = inp["logits"].shape[0]
    print(f"[forward_timed] {case} T={T}", file=sys.stderr, flush=True)
    dev = layer.to_device(inp)
    a = layer.LayerBuffers.allocate(T, wl.E, wl.k, wl.H, wl.I)
    b = layer.LayerBuffers.allocate(T, wl.E, wl.k, wl.H, wl.I)
    for buf in (a, b):
        for name in OUTPUTS:
            _bits(getattr(buf, name)).fill_(-3)
    rt, ev, ms = _hip_events(3)
    try:
        layer.run_forward(dev, a, 10.0)
        binding.moe_forward_mxfp4_timed(dev["logits"], dev["x"], b.k, dev["w1"], dev["w1_s"],
                                        dev["w2"], dev["w2_s"], 10.0, b.topk_ids, b.topk_weights,
                                        b.bitmatrix, b.counts, b.offsets, b.gather, b.scatter,
                                        b.y_sorted, b.y, b.ws, ev)
        torch.cuda.synchronize()
        for name in OUTPUTS:
            assert torch.equal(_bits(getattr(a, name)), _bits(getattr(b, name))), name
        assert ms(ev[0], ev[1]) > 0 and ms(ev[1], ev[2]) > 0
    finally:
        for e in ev:
            rt.hipEventDestroy(e)
