"""Gate for a higher-rate precision path: CPU emulation of candidate activation
formats through the whole layer, measured against the oracle.

The GPU path multiplies bf16 activations by exactly dequantised MXFP4 weights
with fp32 accumulation, and rounds h to bf16 between the two GEMMs.  A faster
path would feed the matrix cores narrower activations: MXFP8 (E4M3 elements with
one E8M0 scale per 32, the f8f6f4 MFMA's operand format) or row-asymmetric INT8
(one scale and zero point per row; the weights are then exact integers, since
2 x E2M1 lies in [-12, 12]).  Each emulation below quantises both GEMMs' inputs
(x for W1, h for W2) and is otherwise exact (float64), so its error is the
format's alone.  The parity tolerance is 2e-2 * max|y| + 1e-3.

Measured (this file's shape, clamp 10): bf16 h ~0.1 %, INT8 row-asymmetric
~1.8 %, MXFP8 ~7 %.  Larger shapes (H = 4096, I = 2048) put INT8 at 1.4-2.7 %:
no margin against the tolerance, so no INT8 or f8f6f4 kernel is built.
"""
from __future__ import annotations

import numpy as np

import oracle
from mxfp4_routed_expert_route_amd import inputs
from oracle.mx import dequant_mxfp4

TOL = 2e-2


def _rows_i8_asym(x):
    """Per row: scale s = (max - min) / 255, zero point z, q = clip(round(x/s) + z)."""
    lo = x.min(axis=1, keepdims=True)
    hi = x.max(axis=1, keepdims=True)
    s = np.where(hi > lo, (hi - lo) / 255.0, 1.0)
    z = np.round(-lo / s) - 128.0
    q = np.clip(np.round(x / s) + z, -128, 127)
    return s * (q - z)


def _e4m3(v):
    """Nearest E4M3 value (3 mantissa bits, subnormal below 2^-6, saturating at 448)."""
    a = np.abs(v)
    e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6.0)
    step = 2.0 ** (e - 3)
    return np.sign(v) * np.minimum(np.round(a / step) * step, 448.0)


def _blocks_mxfp8(x):
    """Per 32 consecutive elements: E8M0 scale 2^(floor(log2 amax) - 8), E4M3 elements."""
    R, K = x.shape
    xb = x.reshape(R, K // 32, 32)
    amax = np.abs(xb).max(axis=2, keepdims=True)
    sc = 2.0 ** (np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8.0)
    return (_e4m3(xb / sc) * sc).reshape(R, K)


def _bf16(x):
    bits = inputs.f32_to_bf16_bits(x.astype(np.float32))
    return oracle.bf16_to_f32(bits).astype(np.float64)


def _layer(inp, limit, qx, qh):
    """The layer with qx applied to W1's input and qh to W2's (float64 otherwise)."""
    wl = inp["workload"]
    T, k = inp["logits"].shape[0], wl.k
    ids, w = oracle.route(inp["logits"], k)
    _, offsets, gather, scatter = oracle.expert_offsets(ids, wl.E)
    x = oracle.bf16_to_f32(inp["x"]).astype(np.float64)
    ys = np.zeros((T * k, wl.H))
    for e in range(wl.E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        w1 = dequant_mxfp4(inp["w1"][e], inp["w1_s"][e]).astype(np.float64)
        w2 = dequant_mxfp4(inp["w2"][e], inp["w2_s"][e]).astype(np.float64)
        gu = qx(x[np.asarray(gather[a:b]) // k]) @ w1.T
        g, u = np.minimum(gu[:, :wl.I], limit), np.clip(gu[:, wl.I:], -limit, limit)
        ys[a:b] = qh(g / (1.0 + np.exp(-g)) * u) @ w2.T
    y = np.zeros((T, wl.H))
    for t in range(T):
        for j in range(k):
            y[t] += w[t, j] * ys[scatter[t * k + j]]
    return y


def _inputs(T, E, k, H, I, seed):
    rng = np.random.default_rng(seed)
    return dict(workload=inputs.Workload(0, "emulation", T, E, k, H, I),
                logits=rng.standard_normal((T, E)).astype(np.float32),
                x=inputs.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)),
                w1=rng.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8),
                w1_s=rng.integers(120, 127, (E, 2 * I, H // 32), dtype=np.uint8),
                w2=rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8),
                w2_s=rng.integers(120, 127, (E, H, I // 32), dtype=np.uint8))


def test_activation_formats_against_the_tolerance():
    inp = _inputs(16, 8, 2, 1024, 512, 1)
    ref = oracle.moe_layer(inp, 10.0)["y"].astype(np.float64)
    m = np.abs(ref).max()
    exact = lambda v: v
    cases = {"exact": (exact, exact),                      # the harness itself
             "bf16 h": (exact, _bf16),                     # the GPU path's arithmetic
             "int8 row-asym": (_rows_i8_asym, _rows_i8_asym),
             "mxfp8": (_blocks_mxfp8, _blocks_mxfp8)}
    rel = {name: float(np.abs(_layer(inp, 10.0, qx, qh) - ref).max() / m)
           for name, (qx, qh) in cases.items()}
    print(rel)
    assert rel["exact"] < 1e-5
    assert rel["bf16 h"] < 0.25 * TOL         # wide margin
    assert rel["int8 row-asym"] > 0.25 * TOL  # INT8 activations: no such margin
    assert rel["mxfp8"] > TOL                 # MXFP8 activations fail the tolerance
