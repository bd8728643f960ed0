"""moe_read_probe (the streaming-read marker of the bench) reads every byte.

The XOR of the per-workgroup sink words must equal the XOR of all 32-bit words
of the buffer, computed on the host; sizes cover a buffer smaller than the grid
(most workgroups read nothing), slabs that end inside the unrolled loop's last
step, and a large buffer.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_bytes", [16, 8192 * 16 * 37 + 48, 64 << 20])
def test_read_probe_reads_every_word(n_bytes):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mxfp4_routed_expert_route_amd import binding
    binding.load()
    print(f"[read_probe] bytes={n_bytes}", file=sys.stderr, flush=True)
    host = np.random.default_rng(n_bytes).integers(0, 256, n_bytes, dtype=np.uint8)
    buf = torch.from_numpy(host).cuda()
    sink = torch.full((binding.READ_PROBE_SINK_WORDS,), -1, dtype=torch.int32, device="cuda")
    binding.moe_read_probe(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.view(np.uint32))
    assert got == want
