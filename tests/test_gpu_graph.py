"""The whole layer captured as a HIP graph replays to the same bits as the eager calls.

The library's calls enqueue kernels only (no memset, no host synchronisation,
no allocation), so stream capture records the five calls as graph nodes.  Each
test replays the graph several times with the program's own eager work and
synchronisations in between (the outputs are scribbled over and the eager layer
runs on other inputs) and checks every replay against the eager result, bit for
bit, on every output of the layer.
"""
from __future__ import annotations

import sys

import pytest

torch = pytest.importorskip("torch")

from mxfp4_routed_expert_route_amd import inputs

pytestmark = pytest.mark.gpu

OUTPUTS = ("topk_ids", "topk_weights", "bitmatrix", "counts", "offsets", "gather", "scatter",
           "y_sorted", "y")


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("index,fused", [
    (0, False),       # tiny: separate routing calls, streaming FFN
    (0, True),        # tiny: one-launch front-end
    (1, True),        # decode verify, full size: streaming FFN
    (1, "forward"),   # decode verify through moe_forward_mxfp4 (front-end writes the plan)
    (3, True),        # prefill 2048, full size: three routing kernels, plan + tiled FFN
])
def test_graph_replay_matches_eager(index, fused):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mxfp4_routed_expert_route_amd import binding, layer
    binding.load()
    wl = inputs.workload(index)
    print(f"[graph] workload {index} fused={fused}", file=sys.stderr, flush=True)
    inp = inputs.make_inputs(index)
    dev = layer.to_device(inp)
    other = dict(dev, logits=torch.flip(dev["logits"], dims=[1]).contiguous())
    b = layer.LayerBuffers.allocate(wl.T, wl.E, wl.k, wl.H, wl.I)

    def run(d, limit):
        if fused == "forward":
            layer.run_forward(d, b, limit)
        else:
            layer.run_layer(d, b, limit, fused=fused)

    run(dev, 10.0)
    torch.cuda.synchronize()
    ref = {name: _bits(getattr(b, name)).clone() for name in OUTPUTS}

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        run(dev, 10.0)
    torch.cuda.synchronize()

    for rep in range(3):
        # eager work between replays: scribble over the outputs, run the layer on
        # other routing logits, synchronise
        for name in OUTPUTS:
            _bits(getattr(b, name)).fill_(-1)
        run(other, 0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name in OUTPUTS:
            assert torch.equal(_bits(getattr(b, name)), ref[name]), f"replay {rep}: {name} differs"
