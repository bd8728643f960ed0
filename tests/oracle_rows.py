"""The oracle's FFN on chosen sorted rows of a full-size workload.

Full-size parity cannot afford the oracle on every row (dequantising one expert
takes about a second of numpy), so the tests pick rows: all rows of a few
experts, and the rows of sampled tokens.  This module only selects rows and
calls the oracle on them: ``oracle.ffn`` restricted to one expert (its weight
slab, its rows' slot ids, offsets [0, n]) gives exactly the rows the full call
would give for that expert, because every sorted row depends only on its own
token's activations and its expert's weights.  Experts run in a thread pool
(numpy releases the GIL inside its array operations); the arithmetic is the
oracle's alone.
"""
from __future__ import annotations

import concurrent.futures
import os

import numpy as np

import oracle


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def sorted_rows(inp: dict, gather, offsets, k: int, positions, limit) -> np.ndarray:
    """Oracle y_sorted rows at `positions` (indices into the expert-major order
    given by gather/offsets), float32 [len(positions), H], in the order given."""
    positions = np.asarray(positions, dtype=np.int64)
    offsets = np.asarray(offsets, dtype=np.int64)
    gather = np.asarray(gather)
    H = inp["w2"].shape[1]
    expert_of = np.searchsorted(offsets, positions, side="right") - 1
    out = np.empty((len(positions), H), dtype=np.float32)

    def one(e):
        sel = np.nonzero(expert_of == e)[0]
        rows = oracle.ffn(inp["x"], gather[positions[sel]], np.array([0, len(sel)]), k,
                          inp["w1"][e:e + 1], inp["w1_s"][e:e + 1], inp["w2"][e:e + 1],
                          inp["w2_s"][e:e + 1], limit)
        return sel, rows

    with concurrent.futures.ThreadPoolExecutor(_workers()) as ex:
        for sel, rows in ex.map(one, np.unique(expert_of)):
            out[sel] = rows
    return out


def token_outputs(inp: dict, ref: dict, k: int, tokens, limit):
    """Oracle y for `tokens` (and their k sorted rows, slot order), from the
    oracle's own routing in `ref` (route + expert_offsets outputs)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    slots = (tokens[:, None] * k + np.arange(k)[None, :]).ravel()
    positions = np.asarray(ref["scatter"])[slots]
    ys = sorted_rows(inp, ref["gather"], ref["offsets"], k, positions, limit)
    y = oracle.combine(ys, np.asarray(ref["weights"])[tokens], np.arange(len(slots)),
                       len(tokens), k)
    return y, ys, positions
