"""The routing invariants catch the padding-lane bug the pages describe.

The txtmix.com article, §3, and the aihot.vn README translation, section
"Định tuyến MXFP4", describe a bitmatrix kernel whose lane count is padded past
the logical block it owns, and whose padding lanes were masked only by the
global bound; the fix masks them by the logical block size as well.  This is a
CPU model of such a tiled kernel (64 lanes, a logical block of floor(64/k)*k
entries, per-program histogram contributions).  With only the global mask,
lanes past the logical block count the next program's entries a second time;
the invariant checks used on the GPU outputs must flag that whenever the input
spans more than one program, and must pass when it fits in one.
"""
import numpy as np
import pytest

import oracle
from tests import invariants


def tiled_counts(ids, E, lanes=64, logical_mask=True):
    T, k = ids.shape
    n = T * k
    tokens_per_prog = lanes // k
    logical = tokens_per_prog * k
    flat = ids.reshape(-1)
    counts = np.zeros(E, np.int64)
    for p in range((T + tokens_per_prog - 1) // tokens_per_prog):
        for lane in range(lanes):
            entry = p * logical + lane
            active = entry < n
            if logical_mask:
                active = active and lane < logical
            if active:
                counts[flat[entry]] += 1
    return counts


@pytest.mark.parametrize("T", [1, 10, 11, 64, 200])
@pytest.mark.parametrize("fixed", [True, False])
def test_invariants_flag_global_only_mask(T, fixed):
    E, k = 256, 6
    logits = np.random.default_rng(T).standard_normal((T, E)).astype(np.float32)
    ids, _ = oracle.route(logits, k)
    _, _, gather, scatter = oracle.expert_offsets(ids, E)
    counts = tiled_counts(ids, E, logical_mask=fixed)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    spans_programs = T > 64 // k
    if fixed or not spans_programs:
        invariants.check_offsets(counts, offsets, gather, scatter, ids, E)
    else:
        with pytest.raises(AssertionError):
            invariants.check_offsets(counts, offsets, gather, scatter, ids, E)
