"""The row-restricted oracle helper (tests/oracle_rows.py) against the full oracle.

The full-size GPU tests compare chosen rows with oracle.ffn restricted to one
expert at a time.  Here, on small workloads, those restricted rows and the
sampled tokens' outputs must equal the full oracle call's rows and outputs (the
products run on different row subsets, so equal up to fp32 summation order).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from mxfp4_routed_expert_route_amd import inputs
from tests import oracle_rows


@pytest.mark.parametrize("limit", [10.0, None])
def test_sorted_rows_match_full_call(limit):
    inp = inputs.make_inputs(0)
    full = oracle.moe_layer(inp, limit)
    rng = np.random.default_rng(5)
    positions = rng.permutation(len(full["gather"]))[:40]
    rows = oracle_rows.sorted_rows(inp, full["gather"], full["offsets"], 6, positions, limit)
    ref = full["y_sorted"][positions]
    assert np.allclose(rows, ref, rtol=1e-5, atol=1e-5 * np.abs(ref).max())


@pytest.mark.parametrize("limit", [10.0, None])
def test_token_outputs_match_full_call(limit):
    inp = inputs.make_inputs(0)
    full = oracle.moe_layer(inp, limit)
    tokens = [0, 3, 7, 15]
    y, ys, pos = oracle_rows.token_outputs(inp, full, 6, tokens, limit)
    assert np.array_equal(pos, full["scatter"].reshape(16, 6)[tokens].ravel())
    assert np.allclose(ys, full["y_sorted"][pos], rtol=1e-5, atol=1e-5 * np.abs(ys).max())
    assert np.allclose(y, full["y"][tokens], rtol=1e-5, atol=1e-5 * np.abs(y).max())


def test_sorted_rows_skewed_multi_row_experts():
    # T = 200 skewed: some experts hold dozens of rows; every row of every expert
    inp = inputs.make_inputs(0, T=200)
    inp["logits"] = inp["logits"] + np.float32(3.0) * (np.arange(256) < 4).astype(np.float32)
    full = oracle.moe_layer(inp, None)
    assert full["counts"].max() > 100
    pos = np.arange(len(full["gather"]))
    rows = oracle_rows.sorted_rows(inp, full["gather"], full["offsets"], 6, pos, None)
    assert np.allclose(rows, full["y_sorted"], rtol=1e-5, atol=1e-5 * np.abs(rows).max())
