"""Device buffers for one routed-expert MoE layer and the five-call chain.

PyTorch supplies device memory (torch.empty) and the stream; every step runs
in the HIP library through ``binding``.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

from . import binding


@dataclasses.dataclass
class LayerBuffers:
    T: int
    E: int
    k: int
    H: int
    I: int
    topk_ids: torch.Tensor
    topk_weights: torch.Tensor
    bitmatrix: torch.Tensor
    counts: torch.Tensor
    offsets: torch.Tensor
    gather: torch.Tensor
    scatter: torch.Tensor
    y_sorted: torch.Tensor
    y: torch.Tensor
    ws: torch.Tensor

    @classmethod
    def allocate(cls, T, E, k, H, I, device="cuda"):
        dev = torch.device(device)
        ws_bytes = binding.moe_workspace_bytes(T, E, k, H, I)
        if ws_bytes == 0:
            raise ValueError("invalid layer sizes")
        i32 = dict(dtype=torch.int32, device=dev)
        return cls(
            T, E, k, H, I,
            topk_ids=torch.empty((T, k), **i32),
            topk_weights=torch.empty((T, k), dtype=torch.float32, device=dev),
            bitmatrix=torch.empty((T, (E + 31) // 32), **i32),
            counts=torch.empty(E, **i32),
            offsets=torch.empty(E + 1, **i32),
            gather=torch.empty(T * k, **i32),
            scatter=torch.empty(T * k, **i32),
            y_sorted=torch.empty((T * k, H), dtype=torch.bfloat16, device=dev),
            y=torch.empty((T, H), dtype=torch.bfloat16, device=dev),
            ws=torch.empty(ws_bytes, dtype=torch.uint8, device=dev),
        )


def to_device(inp: dict, device="cuda") -> dict:
    """Copy one input dict (see inputs.make_inputs) to the GPU."""
    dev = torch.device(device)
    out = {}
    for key in ("logits", "x", "w1", "w1_s", "w2", "w2_s"):
        if key not in inp:
            continue
        a = np.ascontiguousarray(inp[key])
        if not a.flags.writeable:
            a = a.copy()
        if key == "x":
            a = a.view(np.int16)
        out[key] = torch.from_numpy(a).to(dev)
    if "x" in out:
        out["x"] = out["x"].view(torch.bfloat16)
    return out


def run_routing(dev: dict, b: LayerBuffers, stream=None, fused: bool = False):
    """A1-A3: three calls, or the fused front-end entry point (same outputs)."""
    if fused:
        binding.moe_route_and_group(dev["logits"], b.k, b.topk_ids, b.topk_weights, b.bitmatrix,
                                    b.counts, b.offsets, b.gather, b.scatter, b.ws, stream)
        return
    binding.moe_route(dev["logits"], b.k, b.topk_ids, b.topk_weights, stream)
    binding.moe_build_bitmatrix(b.topk_ids, b.E, b.bitmatrix, stream)
    binding.moe_expert_offsets(b.bitmatrix, b.topk_ids, b.E, b.counts, b.offsets, b.gather,
                               b.scatter, b.ws, stream)


def run_ffn(dev: dict, b: LayerBuffers, limit: float, stream=None):
    binding.moe_grouped_ffn_mxfp4(dev["x"], b.k, dev["w1"], dev["w1_s"], dev["w2"], dev["w2_s"],
                                  b.counts, b.offsets, b.gather, limit, b.y_sorted, b.ws, stream)
    binding.moe_combine(b.y_sorted, b.topk_weights, b.scatter, b.y, stream)


def run_layer(dev: dict, b: LayerBuffers, limit: float, stream=None, fused: bool = False):
    run_routing(dev, b, stream, fused)
    run_ffn(dev, b, limit, stream)


def run_forward(dev: dict, b: LayerBuffers, limit: float, stream=None):
    """The whole layer through the one-call entry point (same outputs as run_layer)."""
    binding.moe_forward_mxfp4(dev["logits"], dev["x"], b.k, dev["w1"], dev["w1_s"], dev["w2"],
                              dev["w2_s"], limit, b.topk_ids, b.topk_weights, b.bitmatrix,
                              b.counts, b.offsets, b.gather, b.scatter, b.y_sorted, b.y, b.ws,
                              stream)


def bf16_tensor_to_f32(t: torch.Tensor) -> np.ndarray:
    """Exact bf16 -> fp32 on the host (for comparisons)."""
    return t.float().cpu().numpy()
