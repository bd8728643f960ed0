"""moe_forward_mxfp4_noalloc (static device scratch, no caller workspace) against
moe_forward_mxfp4 (caller workspace), through the C ABI.

Two calls in a row on the same GPU, the second with a smaller input, so the
second call runs on scratch that still holds the first call's contents: the
prefill-2048 workload (80-row tiled FFN, offsets kernels and scan; 68 MB of the
128 MiB scratch), then the verify-1+7 step (one-launch front-end, streaming FFN).
Every output of each call must equal the workspace entry point's, bit for bit
(the same kernels run on the same inputs; routing is also checked against the
oracle).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from mxfp4_routed_expert_route_amd import inputs

pytestmark = pytest.mark.gpu

OUTPUTS = ("topk_ids", "topk_weights", "bitmatrix", "counts", "offsets", "gather", "scatter",
           "y_sorted", "y")


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _noalloc(binding, dev, b, limit):
    binding.moe_forward_mxfp4_noalloc(dev["logits"], dev["x"], b.k, dev["w1"], dev["w1_s"],
                                      dev["w2"], dev["w2_s"], limit, b.topk_ids, b.topk_weights,
                                      b.bitmatrix, b.counts, b.offsets, b.gather, b.scatter,
                                      b.y_sorted, b.y)


def test_noalloc_matches_workspace_entry_point_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mxfp4_routed_expert_route_amd import binding, layer
    binding.load()
    for index in (3, 1):   # larger input first, then a smaller one on the used scratch
        wl = inputs.workload(index)
        assert binding.moe_workspace_bytes(wl.T, wl.E, wl.k, wl.H, wl.I) <= \
            binding.NOALLOC_SCRATCH_BYTES
        print(f"[noalloc] workload {index} ({wl.name}) T={wl.T}", file=sys.stderr, flush=True)
        inp = inputs.make_inputs(index)
        dev = layer.to_device(inp)
        a = layer.LayerBuffers.allocate(wl.T, wl.E, wl.k, wl.H, wl.I)
        b = layer.LayerBuffers.allocate(wl.T, wl.E, wl.k, wl.H, wl.I)
        for buf in (a, b):
            for name in OUTPUTS:
                _bits(getattr(buf, name)).fill_(-3)
        layer.run_forward(dev, a, 10.0)
        _noalloc(binding, dev, b, 10.0)
        torch.cuda.synchronize()
        for name in OUTPUTS:
            assert torch.equal(_bits(getattr(a, name)), _bits(getattr(b, name))), \
                f"workload {index}: {name} differs from moe_forward_mxfp4"
        ids, _ = oracle.route(inp["logits"], wl.k)
        assert np.array_equal(b.topk_ids.cpu().numpy(), ids)
        counts, offsets, gather, scatter = oracle.expert_offsets(ids, wl.E)
        assert np.array_equal(b.gather.cpu().numpy(), gather)
        del a, b, dev, inp
        torch.cuda.empty_cache()


def test_noalloc_rejects_sizes_beyond_the_scratch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mxfp4_routed_expert_route_amd import binding, layer
    binding.load()
    T, E, k, H, I = 4033, 256, 6, 4096, 2048   # just over 128 MiB of workspace
    assert binding.moe_workspace_bytes(T, E, k, H, I) > binding.NOALLOC_SCRATCH_BYTES
    small = inputs.make_inputs(0)
    logits = torch.zeros((T, E), dtype=torch.float32, device="cuda")
    x = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    w1 = torch.zeros((E, 2 * I, 16), dtype=torch.uint8, device="cuda")   # never read
    b = layer.LayerBuffers.allocate(T, E, k, H, I)
    b.counts.fill_(-7)
    with pytest.raises(binding.MoeError) as err:
        binding.moe_forward_mxfp4_noalloc(logits, x, k, w1, w1, w1, w1, 10.0, b.topk_ids,
                                          b.topk_weights, b.bitmatrix, b.counts, b.offsets,
                                          b.gather, b.scatter, b.y_sorted, b.y)
    assert err.value.code == 4   # MOE_ERR_WORKSPACE_TOO_SMALL, nothing enqueued
    torch.cuda.synchronize()
    assert (b.counts.cpu().numpy() == -7).all()
    del small
