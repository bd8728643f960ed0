"""Pins for the CPU oracle: checks against what the MX spec and plain mathematics
fix, independent of the oracle's own code paths (CPU only)."""
from __future__ import annotations

import math
import os

import numpy as np
import pytest

import oracle
from mxfp4_routed_expert_route_amd import inputs
from tests import invariants

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_sections(path):
    sec, out = None, {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("["):
            sec = line.strip("[]")
            out[sec] = []
            continue
        out[sec].append(line.split())
    return out


def _pow2_or_nan(tok):
    if tok == "nan":
        return math.nan
    if tok.startswith("2^"):
        return math.ldexp(1.0, int(tok[2:]))
    return float(tok)


# ---------------------------------------------------------------- MX decoding

def test_e2m1_matches_spec_table():
    g = _read_sections(os.path.join(GOLDEN, "mx_codes.txt"))["e2m1"]
    assert len(g) == 16
    for code, val in g:
        got = oracle.e2m1_decode(int(code))
        want = float(val)
        assert got == want
        assert math.copysign(1.0, float(got)) == math.copysign(1.0, want), f"sign of code {code}"


def test_e8m0_matches_spec_table():
    g = _read_sections(os.path.join(GOLDEN, "mx_codes.txt"))["e8m0"]
    for code, val in g:
        got = float(oracle.e8m0_decode(int(code)))
        want = _pow2_or_nan(val)
        if math.isnan(want):
            assert math.isnan(got)
        else:
            assert got == want, code
    # every finite code is the power of two 2^(s-127): exact doubling per step
    s = np.arange(255)
    v = oracle.e8m0_decode(s)
    assert (v[1:] == 2 * v[:-1]).all()


def test_dequant_nibble_order_and_scale_blocks():
    # 64 elements: bytes pack (element 2i low nibble, element 2i+1 high nibble)
    codes = np.zeros(32, np.uint8)
    codes[0] = 0x21            # element 0 -> code 1 (0.5), element 1 -> code 2 (1.0)
    codes[16] = 0xF7           # element 32 -> code 7 (6.0), element 33 -> code 15 (-6.0)
    codes[31] = 0x90           # element 62 -> code 0, element 63 -> code 9 (-0.5)
    scales = np.array([127, 129], np.uint8)   # x1 for elements 0..31, x4 for 32..63
    d = oracle.dequant_mxfp4(codes, scales)
    assert d.dtype == np.float32 and d.shape == (64,)
    assert d[0] == 0.5 and d[1] == 1.0
    assert d[32] == 24.0 and d[33] == -24.0
    assert d[62] == 0.0 and d[63] == -2.0
    assert np.count_nonzero(d) == 5


def test_dequant_nan_scale_and_tiny_scale():
    codes = np.full(16, 0x22, np.uint8)
    d = oracle.dequant_mxfp4(codes, np.array([255], np.uint8))
    assert np.isnan(d).all()
    d = oracle.dequant_mxfp4(codes, np.array([0], np.uint8))
    assert (d == np.float32(math.ldexp(1.0, -127))).all()   # 1.0 * 2^-127, an fp32 subnormal


# ---------------------------------------------------------------- routing

def _check_topk_property(logits, ids, k):
    """Selection property, written independently of any sort: the chosen set holds
    the k largest logits, a tie at the boundary goes to lower indices, and the k
    ids are listed by (logit desc, index asc)."""
    T, E = logits.shape
    for t in range(T):
        row = logits[t].astype(np.float64)
        chosen = [int(e) for e in ids[t]]
        rest = [e for e in range(E) if e not in chosen]
        for c in chosen:
            for r in rest:
                assert row[c] > row[r] or (row[c] == row[r] and c < r), (t, c, r)
        for a, b in zip(chosen, chosen[1:]):
            assert row[a] > row[b] or (row[a] == row[b] and a < b), (t, a, b)


@pytest.mark.parametrize("T,E,k,seed", [(7, 9, 3, 0), (5, 32, 6, 1), (16, 256, 6, 2),
                                        (4, 40, 1, 3), (3, 8, 8, 4)])
def test_route_selection_property(T, E, k, seed):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    # plant exact ties, some of them straddling the boundary
    logits[:, 1] = logits[:, 0]
    logits[0, :] = np.round(logits[0, :])
    ids, w = oracle.route(logits, k)
    invariants.check_ids(ids, E, k)
    _check_topk_property(logits, ids, k)


def test_route_weights_closed_form():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((6, 20)).astype(np.float32)
    ids, w = oracle.route(logits, 4)
    for t in range(6):
        l = [float(logits[t, e]) for e in ids[t]]
        z = sum(math.exp(v - l[0]) for v in l)
        for j in range(4):
            assert abs(float(w[t, j]) - math.exp(l[j] - l[0]) / z) <= 1e-7 * float(w[t, j])
        assert abs(float(w[t].astype(np.float64).sum()) - 1.0) < 1e-6
    ids1, w1 = oracle.route(logits, 1)
    assert (w1 == 1.0).all()
    assert (ids1[:, 0] == ids[:, 0]).all()


def test_route_hand_cases():
    # all-equal row: ids 0..k-1, equal weights
    ids, w = oracle.route(np.zeros((1, 10), np.float32), 4)
    assert ids.tolist() == [[0, 1, 2, 3]]
    assert np.allclose(w, 0.25, rtol=0, atol=1e-7)
    # -0.0 and +0.0 are equal: the lower index wins either way round
    row = np.full((2, 8), -1.0, np.float32)
    row[0, 3], row[0, 5] = -0.0, 0.0
    row[1, 2], row[1, 4] = 0.0, -0.0
    ids, w = oracle.route(row, 2)
    assert ids.tolist() == [[3, 5], [2, 4]]
    assert (w == 0.5).all()
    # boundary tie: the k-th and (k+1)-th values are equal; the lower index is taken
    row = np.array([[0.0, 5.0, 1.0, 3.0, 1.0, 1.0]], np.float32)
    ids, _ = oracle.route(row, 3)
    assert ids.tolist() == [[1, 3, 2]]


def test_bitmatrix_and_offsets_bruteforce():
    rng = np.random.default_rng(7)
    for T, E, k in [(1, 40, 3), (13, 40, 6), (33, 256, 6), (64, 96, 8)]:
        logits = rng.standard_normal((T, E)).astype(np.float32)
        ids, _ = oracle.route(logits, k)
        bm = oracle.bitmatrix(ids, E)
        invariants.check_bitmatrix(bm, ids, E)
        counts, offsets, gather, scatter = oracle.expert_offsets(ids, E)
        invariants.check_offsets(counts, offsets, gather, scatter, ids, E, bm=bm)
        # brute force: count by direct comparison, rebuild gather by scanning (e, t, j)
        for e in range(E):
            assert counts[e] == int((ids == e).sum())
        g2 = [t * k + j for e in range(E) for t in range(T) for j in range(k) if ids[t, j] == e]
        assert gather.tolist() == g2


# ---------------------------------------------------------------- SwiGLU and combine

def test_swiglu_clamp_closed_form():
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))
    g = np.array([20.0, -20.0, 3.0, 0.0, 12.0], np.float32)
    u = np.array([20.0, -20.0, -4.0, 7.0, -10.5], np.float32)
    h = oracle.swiglu(g, u, 10.0)
    want = [10 * sig(10) * 10, -20 * sig(-20) * -10, 3 * sig(3) * -4, 0.0, 10 * sig(10) * -10]
    assert np.allclose(h, want, rtol=1e-6, atol=0)
    for off in (0.0, -1.0, math.inf, math.nan, None):
        h = oracle.swiglu(g, u, off)
        want = [float(a) * sig(float(a)) * float(b) for a, b in zip(g, u)]
        assert np.allclose(h, want, rtol=1e-6, atol=1e-30)
    h = oracle.swiglu(np.array([math.nan, 1.0], np.float32), np.array([1.0, math.nan], np.float32), 10.0)
    assert np.isnan(h).all()


def test_combine_closed_form():
    T, k, H = 3, 2, 4
    ys = np.arange(T * k * H, dtype=np.float32).reshape(T * k, H)
    w = np.array([[0.25, 0.75], [1.0, 0.0], [0.5, 0.5]], np.float32)
    scatter = np.array([5, 0, 1, 2, 3, 4])
    y = oracle.combine(ys, w, scatter, T, k)
    assert np.array_equal(y[0], 0.25 * ys[5] + 0.75 * ys[0])
    assert np.array_equal(y[1], ys[1])
    assert np.array_equal(y[2], 0.5 * ys[3] + 0.5 * ys[4])


# ---------------------------------------------------------------- FFN pins

def _tiny_inputs(T, E, k, H, I, seed):
    rng = np.random.default_rng(seed)
    return dict(
        workload=inputs.Workload(0, "t", T, E, k, H, I),
        logits=rng.standard_normal((T, E)).astype(np.float32),
        x=inputs.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)),
        w1=rng.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8),
        w1_s=rng.integers(120, 127, (E, 2 * I, H // 32), dtype=np.uint8),
        w2=rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8),
        w2_s=rng.integers(120, 127, (E, H, I // 32), dtype=np.uint8))


@pytest.mark.parametrize("T,E,k,H,I,seed,limit", [
    (16, 256, 6, 256, 128, 0, 10.0),
    (9, 12, 3, 64, 32, 1, 10.0),
    (40, 16, 4, 96, 64, 2, None),
    (64, 24, 8, 64, 32, 3, 2.0),
])
def test_routed_equals_dense_bruteforce(T, E, k, H, I, seed, limit):
    inp = _tiny_inputs(T, E, k, H, I, seed)
    ref = oracle.moe_layer(inp, limit)
    dense = oracle.dense_moe(inp["x"], ref["ids"], ref["weights"], inp["w1"], inp["w1_s"],
                             inp["w2"], inp["w2_s"], limit)
    scale = float(np.abs(dense).max())
    assert scale > 0
    assert float(np.abs(ref["y"] - dense).max()) <= 1e-5 * scale


def test_workload0_routed_equals_dense():
    inp = inputs.make_inputs(0)
    ref = oracle.moe_layer(inp, 10.0)
    dense = oracle.dense_moe(inp["x"], ref["ids"], ref["weights"], inp["w1"], inp["w1_s"],
                             inp["w2"], inp["w2_s"], 10.0)
    assert float(np.abs(ref["y"] - dense).max()) <= 1e-5 * float(np.abs(dense).max())


def test_ffn_one_hot_closed_form():
    """Weights with a single 1.0 (code 2) per row, all scales 1 (127) except a few x2
    (128): every output is a hand-computable function of x.  Pins the nibble order,
    the gate|up halves, the scale-block index and the clamp."""
    T, E, k, H, I = 5, 4, 2, 64, 32
    L = 1.5
    rng = np.random.default_rng(11)
    x_f = rng.standard_normal((T, H)).astype(np.float32) * 3
    x_bits = inputs.f32_to_bf16_bits(x_f)
    x = inputs.bf16_bits_to_f32(x_bits).astype(np.float64)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    w1 = np.zeros((E, 2 * I, H // 2), np.uint8)
    w1_s = np.full((E, 2 * I, H // 32), 127, np.uint8)
    w2 = np.zeros((E, H, I // 2), np.uint8)
    w2_s = np.full((E, H, I // 32), 127, np.uint8)
    a = rng.integers(0, H, (E, I))      # gate row i reads x[a]
    b = rng.integers(0, H, (E, I))      # up row i reads x[b]
    c = rng.integers(0, I, (E, H))      # output n reads h[c]
    def put(mat, e, row, col):
        mat[e, row, col // 2] |= np.uint8(0x2 << (4 * (col % 2)))
    for e in range(E):
        for i in range(I):
            put(w1, e, i, a[e, i])
            put(w1, e, I + i, b[e, i])
        for n in range(H):
            put(w2, e, n, c[e, n])
    # doubled scale on the up rows' block that holds column b for expert 1
    w1_s[1, I:, :] = 128
    inp = dict(workload=inputs.Workload(0, "t", T, E, k, H, I), logits=logits, x=x_bits,
               w1=w1, w1_s=w1_s, w2=w2, w2_s=w2_s)
    ref = oracle.moe_layer(inp, L)
    ids, w = ref["ids"], ref["weights"]
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))
    for t in range(T):
        for n in range(H):
            acc = 0.0
            for j in range(k):
                e = int(ids[t, j])
                i = c[e, n]
                g = min(x[t, a[e, i]], L)
                u = x[t, b[e, i]] * (2.0 if e == 1 else 1.0)
                u = max(-L, min(u, L))
                acc += float(w[t, j]) * g * sig(g) * u
            assert abs(float(ref["y"][t, n]) - acc) <= 1e-6 * max(1.0, abs(acc)), (t, n)


def _layer_y(inp, limit):
    return oracle.moe_layer(inp, limit)["y"]


def test_metamorphic_w2_scale_doubles_output():
    inp = _tiny_inputs(12, 10, 3, 64, 64, 21)
    y0 = _layer_y(inp, 10.0)
    inp2 = dict(inp, w2_s=inp["w2_s"] + 1)
    assert np.array_equal(_layer_y(inp2, 10.0), 2 * y0)


def test_metamorphic_w2_sign_flip_negates_output():
    inp = _tiny_inputs(12, 10, 3, 64, 64, 22)
    y0 = _layer_y(inp, 10.0)
    inp2 = dict(inp, w2=inp["w2"] ^ np.uint8(0x88))
    assert np.array_equal(_layer_y(inp2, 10.0), -y0)


def test_metamorphic_up_half_scale_doubles_output_without_clamp():
    inp = _tiny_inputs(12, 10, 3, 64, 64, 23)
    y0 = _layer_y(inp, None)
    s = inp["w1_s"].copy()
    s[:, 64:, :] += 1                  # up rows only
    assert np.array_equal(_layer_y(dict(inp, w1_s=s), None), 2 * y0)
    s = inp["w1_s"].copy()
    s[:, :64, :] += 1                  # gate rows only: SiLU is not linear
    assert not np.array_equal(_layer_y(dict(inp, w1_s=s), None), 2 * y0)


def test_metamorphic_expert_relabelling():
    inp = _tiny_inputs(12, 10, 3, 64, 64, 24)
    y0 = _layer_y(inp, 10.0)
    perm = np.random.default_rng(1).permutation(10)   # new expert q holds old perm[q]
    inp2 = dict(inp, logits=inp["logits"][:, perm], w1=inp["w1"][perm], w1_s=inp["w1_s"][perm],
                w2=inp["w2"][perm], w2_s=inp["w2_s"][perm])
    assert np.array_equal(_layer_y(inp2, 10.0), y0)


# ---------------------------------------------------------------- inputs

def test_inputs_are_seeded_and_shaped():
    a = inputs.make_inputs(0)
    b = inputs.make_inputs(0)
    for key in ("logits", "x", "w1", "w1_s", "w2", "w2_s"):
        assert np.array_equal(a[key], b[key]), key
    assert a["w1"].shape == (256, 256, 128) and a["w2_s"].shape == (256, 256, 4)
    assert a["w1_s"].min() >= 120 and a["w1_s"].max() <= 126
    c = inputs.make_inputs(0, seed=9)
    assert not np.array_equal(a["logits"], c["logits"])


def test_skewed_workload_has_hot_experts_and_boundary_ties():
    inp = inputs.make_inputs(4, weights=False)
    T, E, k = 8191, 256, 6
    ids, _ = oracle.route(inp["logits"], k)
    counts = np.bincount(ids.ravel(), minlength=E)
    assert counts.max() > 10 * counts.mean()
    # some rows have an exact tie between the k-th chosen and the best unchosen logit
    srt = -np.sort(-inp["logits"], axis=1)
    assert int((srt[:, k - 1] == srt[:, k]).sum()) > 100
