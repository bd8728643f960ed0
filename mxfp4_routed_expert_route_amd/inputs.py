"""Seeded synthetic inputs for the routed-expert MXFP4 MoE layer.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic (no selection, no decoding, no products).  Both the CPU
oracle's tests and the GPU path take their inputs from here, so that the two
sides see the same bytes.

Workloads (sizes from the deployment the pages describe: 256 routed experts,
top-6 per token; the txtmix.com article, §1 and §3; T = 1 + 7 draft tokens for a
DSpark-7 verify step, §4 and §8; the 2,048-token scheduling budget, §8):

  0 tiny           T=16,   H=256,  I=128   logits N(0,1)
  1 verify         T=8,    H=4096, I=2048  one stream, 1 + 7 draft tokens
  2 burst          T=512,  H=4096, I=2048  64 streams x 8 tokens
  3 prefill-2048   T=2048, H=4096, I=2048  uniform routing
  4 skewed-8191    T=8191, H=4096, I=2048  per-expert bias 2*ln(1/rank) + ~1% exact ties

Common distributions: activations N(0,1) rounded to bf16 (round to nearest
even); E2M1 codes uniform over all 16 values (so packed bytes are uniform over
0..255); E8M0 scales uniform over the integers 120..126; router logits fp32
N(0,1).  One numpy PCG64 stream per workload, seed = workload index unless
given, drawn in a fixed order: logits, bias permutation, ties, x, W1 codes, W1
scales, W2 codes, W2 scales.

Layouts (row-major):
  logits  fp32  [T, E]
  x       bf16 bit patterns as uint16 [T, H]
  w1      uint8 [E, 2I, H/2]   rows 0..I-1 gate, I..2I-1 up; element 2i in the
                               low nibble of byte i, 2i+1 in the high nibble
  w1_s    uint8 [E, 2I, H/32]  one E8M0 scale per 32 consecutive elements of a row
  w2      uint8 [E, H, I/2]
  w2_s    uint8 [E, H, I/32]
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "make_inputs", "f32_to_bf16_bits",
           "bf16_bits_to_f32"]


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    T: int
    E: int
    k: int
    H: int
    I: int
    skewed: bool = False
    tie_fraction: float = 0.0

    @property
    def slots(self) -> int:
        return self.T * self.k


WORKLOADS = (
    Workload(0, "tiny", 16, 256, 6, 256, 128),
    Workload(1, "verify-1+7", 8, 256, 6, 4096, 2048),
    Workload(2, "burst-64x8", 512, 256, 6, 4096, 2048),
    Workload(3, "prefill-2048", 2048, 256, 6, 4096, 2048),
    Workload(4, "skewed-8191", 8191, 256, 6, 4096, 2048, skewed=True, tie_fraction=0.01),
)


def workload(index: int) -> Workload:
    return WORKLOADS[index]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even) and return the bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _skewed_logits(rng: np.random.Generator, T: int, E: int, k: int,
                   tie_fraction: float) -> np.ndarray:
    base = rng.standard_normal((T, E), dtype=np.float32)
    rank = rng.permutation(E) + 1                      # expert e has load rank[e] (1 = hottest)
    bias = 2.0 * np.log(1.0 / rank.astype(np.float64))
    logits = (base.astype(np.float64) + bias[None, :]).astype(np.float32)
    n_ties = int(round(tie_fraction * T * E))
    rows = rng.integers(0, T, n_ties)
    dst = rng.integers(0, E, n_ties)
    src = rng.integers(0, E, n_ties)
    boundary = rng.random(n_ties) < 0.5
    for i in range(n_ties):
        r = rows[i]
        if boundary[i]:
            # copy the row's current k-th largest value: an exact tie that straddles
            # the top-k boundary, so only the index order can decide it
            val = np.partition(logits[r], E - k)[E - k]
        else:
            val = logits[r, src[i]]
        logits[r, dst[i]] = val
    return logits


def make_inputs(wl: Workload | int, seed: int | None = None, *, weights: bool = True,
                T: int | None = None) -> dict:
    """Draw one workload's inputs.  ``T`` overrides the token count (same recipe)."""
    if isinstance(wl, int):
        wl = workload(wl)
    if T is not None:
        wl = dataclasses.replace(wl, T=T)
    rng = np.random.Generator(np.random.PCG64(wl.index if seed is None else seed))
    T, E, k, H, I = wl.T, wl.E, wl.k, wl.H, wl.I
    if wl.skewed:
        logits = _skewed_logits(rng, T, E, k, wl.tie_fraction)
    else:
        logits = rng.standard_normal((T, E), dtype=np.float32)
    x = f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    out = dict(workload=wl, logits=logits, x=x)
    if weights:
        out["w1"] = np.frombuffer(rng.bytes(E * 2 * I * H // 2), np.uint8).reshape(E, 2 * I, H // 2)
        out["w1_s"] = rng.integers(120, 127, (E, 2 * I, H // 32), dtype=np.uint8)
        out["w2"] = np.frombuffer(rng.bytes(E * H * I // 2), np.uint8).reshape(E, H, I // 2)
        out["w2_s"] = rng.integers(120, 127, (E, H, I // 32), dtype=np.uint8)
    return out
