"""GPU parity: the HIP library, called through the C ABI, against the CPU oracle.

Routing outputs (ids, bit matrix, counts, offsets, gather, scatter) must match
bit for bit.  Routing weights: |gpu - oracle| <= 1e-6 * oracle (fp32 exponentials
against a float64 softmax).  FFN and combined outputs:
max|gpu - oracle| <= 2e-2 * max|oracle| + 1e-3, the oracle accumulating in fp32
over the dequantised weights.  Full-size workloads are checked on all routing
outputs, on every row of chosen experts and on the rows and outputs of sampled
tokens, with the SwiGLU clamp at 10 and off.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from mxfp4_routed_expert_route_amd import inputs
from tests import invariants

pytestmark = pytest.mark.gpu

REL_TOL, ABS_TOL = 2e-2, 1e-3


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mxfp4_routed_expert_route_amd import binding
    binding.load()          # fails loudly if the library is missing


def _layer():
    from mxfp4_routed_expert_route_amd import layer
    return layer


def run_gpu(inp, limit=10.0, fused=False):
    layer = _layer()
    T = inp["logits"].shape[0]
    wl = inp["workload"]
    dev = layer.to_device(inp)
    b = layer.LayerBuffers.allocate(T, wl.E, wl.k, wl.H, wl.I)
    layer.run_layer(dev, b, 0.0 if limit is None else limit, fused=fused)   # <= 0: no clamp
    torch.cuda.synchronize()
    return b


def ffn_close(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    nan_g, nan_r = np.isnan(gpu), np.isnan(ref)
    assert (nan_g == nan_r).all(), f"NaN positions differ ({nan_g.sum()} vs {nan_r.sum()})"
    ok = ~nan_r
    if not ok.any():
        return 0.0
    err = float(np.abs(gpu[ok] - ref[ok]).max())
    bound = REL_TOL * float(np.abs(ref[ok]).max()) + ABS_TOL
    assert err <= bound, f"max err {err:.4g} > bound {bound:.4g}"
    return err / max(float(np.abs(ref[ok]).max()), 1e-30)


def check_routing(b, ref, E, k):
    ids = b.topk_ids.cpu().numpy()
    assert np.array_equal(ids, ref["ids"]), "topk ids differ"
    w = b.topk_weights.cpu().numpy()
    assert (np.abs(w.astype(np.float64) - ref["weights"]) <= 1e-6 * ref["weights"]).all(), \
        "routing weights differ"
    bm = b.bitmatrix.cpu().numpy().view(np.uint32)
    assert np.array_equal(bm, ref["bitmatrix"]), "bitmatrix differs"
    invariants.check_bitmatrix(bm, ids, E)
    for name in ("counts", "offsets", "gather", "scatter"):
        got = getattr(b, name).cpu().numpy()
        assert np.array_equal(got, ref[name]), f"{name} differs"
    invariants.check_offsets(b.counts.cpu().numpy(), b.offsets.cpu().numpy(),
                             b.gather.cpu().numpy(), b.scatter.cpu().numpy(), ids, E, bm=bm)


def oracle_routing(logits, E, k):
    ids, w = oracle.route(logits, k)
    counts, offsets, gather, scatter = oracle.expert_offsets(ids, E)
    return dict(ids=ids, weights=w, bitmatrix=oracle.bitmatrix(ids, E), counts=counts,
                offsets=offsets, gather=gather, scatter=scatter)


# ------------------------------------------------------------ small, whole-layer parity

def tiny(T, E, k, H, I, seed, skew=False):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    if skew:
        logits += (2.0 * np.log(1.0 / (rng.permutation(E) + 1))).astype(np.float32)
    return dict(
        workload=inputs.Workload(0, "t", T, E, k, H, I), logits=logits,
        x=inputs.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)),
        w1=rng.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8),
        w1_s=rng.integers(120, 127, (E, 2 * I, H // 32), dtype=np.uint8),
        w2=rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8),
        w2_s=rng.integers(120, 127, (E, H, I // 32), dtype=np.uint8))


def whole_layer_parity(inp, limit, fused=False):
    wl = inp["workload"]
    T = inp["logits"].shape[0]
    _say(f"[parity] T={T} E={wl.E} k={wl.k} H={wl.H} I={wl.I} limit={limit} fused={fused}")
    b = run_gpu(inp, limit, fused)
    ref = oracle.moe_layer(inp, limit)
    check_routing(b, ref, wl.E, wl.k)
    r1 = ffn_close(b.y_sorted.float().cpu().numpy(), ref["y_sorted"])
    r2 = ffn_close(b.y.float().cpu().numpy(), ref["y"])
    return r1, r2


@pytest.mark.parametrize("limit", [10.0, 0.0])
def test_workload0_whole_layer(limit):
    whole_layer_parity(inputs.make_inputs(0), limit)


@pytest.mark.parametrize("T,E,k,H,I,seed", [
    (1, 256, 6, 256, 128, 1),        # one token
    (7, 256, 6, 256, 128, 2),
    (11, 64, 6, 128, 256, 3),        # rows span two bitmatrix wavefronts
    (70, 32, 6, 384, 128, 4),        # ragged row tiles (>64 rows for some experts)
    (300, 16, 2, 256, 384, 5),       # many rows per expert: 80-row tiles
    (1030, 48, 8, 128, 128, 6),      # crosses a 1024-token offsets block
    (33, 1024, 8, 128, 128, 7),      # maximum E and k
    (40, 8, 1, 128, 128, 8),         # k = 1
    (400, 16, 4, 768, 512, 14),      # 128-row tiles (100 rows per expert): W1 6 chunks, W2 4
    (260, 8, 3, 512, 768, 15),       # 128-row tiles (97 rows per expert): W1 4 chunks, W2 6,
                                     # ragged tiles
    (300, 8, 2, 1536, 1024, 16),     # 80-row tiles (75 rows per expert, some experts in two
                                     # tiles): W1 12 chunks, W2 8
    (290, 8, 2, 256, 256, 19),       # 80-row tiles, experts of ~60-85 rows: 4 and 5 subtiles
    (100, 8, 2, 8192, 256, 18),      # 80-row tiles, W1 K = 8192: E8M0 scales come with the
                                     # weights (they do not fit in LDS beside the activations)
    (200, 4, 2, 8192, 256, 20),      # 128-row tiles, W1 K = 8192: the same fallback there
    (300, 8, 3, 384, 640, 17),       # 128-row tiles (112 rows per expert): W1 3 chunks, 20
                                     # wavefronts per tile (last workgroup part-idle); W2 5
                                     # chunks, 6 wavefronts per tile
    (300, 16, 3, 640, 896, 21),      # 80-row tiles: W1 5 chunks, W2 7 (the weight pairs' loop
                                     # of four chunks, then one or three more)
    (250, 8, 2, 768, 128, 22),       # 80-row tiles: W1 6 chunks (loop, then two), W2 1 chunk
])
@pytest.mark.parametrize("limit", [10.0, None])
def test_ragged_shapes_whole_layer(T, E, k, H, I, seed, limit):
    whole_layer_parity(tiny(T, E, k, H, I, seed), limit)


@pytest.mark.parametrize("T,E,k,seed", [
    (1, 256, 6, 31), (8, 256, 6, 32), (16, 256, 6, 33), (63, 256, 6, 34), (64, 256, 6, 35),
    (65, 256, 6, 36),                # past the one-launch limit: the routing kernel writes
                                     # the bit matrix, then the offsets kernels
    (300, 40, 5, 56),                # E = 40: a partial last bit-matrix word
    (130, 1024, 8, 57),              # 32 bit-matrix words per row
    (513, 96, 3, 58),                # past one offsets block
    (64, 1024, 8, 37), (20, 40, 3, 38), (10, 64, 1, 39),
])
def test_fused_front_end(T, E, k, seed):
    whole_layer_parity(tiny(T, E, k, 128, 128, seed), 10.0, fused=True)


def test_fused_front_end_ties():
    inp = tiny(50, 64, 6, 128, 128, 40)
    inp["logits"][:] = 0.0
    inp["logits"][1::2, 9] = -0.0
    whole_layer_parity(inp, 10.0, fused=True)


def test_skewed_small_whole_layer():
    whole_layer_parity(tiny(500, 64, 6, 256, 128, 9, skew=True), 10.0)


@pytest.mark.parametrize("limit", [10.0, None])
def test_skewed_128_row_tiles(limit):
    # 131 rows per expert on average -> 128-row tiles; the skew leaves hot experts
    # with several full tiles and the rest with tails that run 2, 4 or 8 subtiles
    whole_layer_parity(tiny(700, 32, 6, 384, 256, 27, skew=True), limit)


def test_all_tied_logits_route_to_lowest_ids():
    inp = tiny(130, 40, 6, 128, 128, 10)
    inp["logits"][:] = 0.0
    inp["logits"][::3, 7] = -0.0
    whole_layer_parity(inp, 10.0)


def test_one_expert_takes_every_token():
    inp = tiny(200, 32, 4, 128, 128, 11)
    inp["logits"][:, 5] += 100.0
    whole_layer_parity(inp, None)


def test_streaming_path_expert_spanning_several_tiles():
    # 3.1 rows per expert on average -> 16-row streaming tiles; expert 5 takes every
    # token (100 rows = six tiles of 16 and one of 4)
    inp = tiny(100, 64, 2, 256, 128, 17)
    inp["logits"][:, 5] += 100.0
    whole_layer_parity(inp, 10.0)


def test_streaming_path_32_row_tiles():
    # 18.75 rows per expert on average -> 32-row streaming tiles (two 16-row subtiles)
    whole_layer_parity(tiny(120, 32, 5, 256, 128, 21), 10.0)


@pytest.mark.parametrize("T,E,k,H,I,seed", [
    # 8 rows per expert on average, skewed: 16-row tiles of 1 to 16 rows.  W1
    # (K = 3072) keeps tiles of <= 4 rows in LDS for all of K and stages larger
    # ones chunk by chunk through the LDS ring; W2 (K = 2048) keeps <= 9 rows.
    (64, 16, 2, 3072, 2048, 22),
    # W1 at K = 4096 keeps <= 2 rows (the decode setting); W2 at K = 1024 keeps
    # every 16-row tile
    (40, 32, 6, 4096, 1024, 23),
    # 12 rows per expert on average (the burst setting): 32-row tiles through the
    # LDS ring, W1 at K = 4096
    (96, 16, 2, 4096, 1024, 26),
    # H = 1152: 18 W2 wavefronts per tile, so a workgroup straddles tiles and W2
    # loads its activations per wavefront (no LDS rows, no ring)
    (64, 8, 2, 1152, 512, 24),
    # 20 rows per expert on average: 32-row tiles (two 16-row subtiles) with the
    # deep pipeline on both GEMMs (activations per wavefront)
    (128, 32, 5, 1024, 512, 25),
])
@pytest.mark.parametrize("limit", [10.0, None])
def test_streaming_activation_paths(T, E, k, H, I, seed, limit):
    whole_layer_parity(tiny(T, E, k, H, I, seed, skew=True), limit)


@pytest.mark.parametrize("T,E,k,H,I,seed", [
    # 150 rows per expert on average, skewed (6 to 580 rows): 128-row tiles with 8
    # subtiles (operand-layout loads) next to tiles with 2 and 4 subtiles (weight
    # transit); W1 5 chunks (one loop of four, then one), W2 3 chunks
    (600, 8, 2, 640, 384, 27),
    # the same routing, W1 8 chunks (two loops), W2 6 chunks (one loop, then two)
    (600, 8, 2, 1024, 768, 27),
])
@pytest.mark.parametrize("limit", [10.0, None])
def test_tiled_subtile_paths(T, E, k, H, I, seed, limit):
    whole_layer_parity(tiny(T, E, k, H, I, seed, skew=True), limit)


@pytest.mark.parametrize("T,E,k,H,I,seed,hot", [
    (7, 16, 2, 2048, 2048, 41, None),   # K = 2048 for both GEMMs: one 1 KB slice per row
    (2, 16, 4, 4096, 2048, 42, None),   # W1 two slices per row, W2 one
    (3, 16, 3, 2048, 4096, 43, None),   # W1 one slice, W2 two
    (7, 16, 2, 2048, 2048, 44, 5),      # expert 5 takes every token: 7 one-row tiles
    (1, 8, 2, 4096, 4096, 45, None),    # one token
])
@pytest.mark.parametrize("limit", [10.0, None])
def test_gemv_decode_path(T, E, k, H, I, seed, hot, limit):
    # fewer rows than experts (T k < E) and K of 2048 or 4096: the one-row tiles of
    # the GEMV kernels, through the separate calls and the one-call layer
    inp = tiny(T, E, k, H, I, seed)
    if hot is not None:
        inp["logits"][:, hot] += 100.0
    _say(f"[parity] gemv T={T} E={E} k={k} H={H} I={I} limit={limit}")
    ref = oracle.moe_layer(inp, limit)
    for fused in (False, True):
        b = run_gpu(inp, limit, fused)
        check_routing(b, ref, E, k)
        ffn_close(b.y_sorted.float().cpu().numpy(), ref["y_sorted"])
        ffn_close(b.y.float().cpu().numpy(), ref["y"])


def test_gemv_nan_and_extreme_scales():
    inp = tiny(6, 16, 2, 2048, 2048, 46)
    ids, _ = oracle.route(inp["logits"], 2)
    e1, e2 = int(ids[0, 0]), int(ids[1, 1])
    w1_s = inp["w1_s"].copy()
    w2_s = inp["w2_s"].copy()
    w1_s[e1, 3, 10] = 255     # NaN block in gate row 3 (h column 3) of a touched expert
    w1_s[e2, :, 0] = 0        # 2^-127 blocks
    w2_s[e2, 17, 5] = 255     # NaN block in output row 17
    inp = dict(inp, w1_s=w1_s, w2_s=w2_s)
    whole_layer_parity(inp, 10.0)


def test_single_expert():
    # E = 1, k = 1: every token routes to expert 0 with weight 1
    whole_layer_parity(tiny(50, 1, 1, 128, 128, 18), 10.0)


def test_every_token_picks_every_expert():
    # k = E: the selection is a full sort of each row
    whole_layer_parity(tiny(20, 4, 4, 128, 128, 19), 10.0, fused=True)


@pytest.mark.parametrize("fused", [False, True])
def test_empty_batch(fused):
    # T = 0: every call returns OK; counts and offsets come back zero, nothing else
    # is written
    layer = _layer()
    E, k, H, I = 64, 6, 256, 128
    inp = tiny(0, E, k, H, I, 20)
    dev = layer.to_device(inp)
    b = layer.LayerBuffers.allocate(0, E, k, H, I)
    b.counts.fill_(-7)
    b.offsets.fill_(-7)
    layer.run_layer(dev, b, 10.0, fused=fused)
    torch.cuda.synchronize()
    assert (b.counts.cpu().numpy() == 0).all()
    assert (b.offsets.cpu().numpy() == 0).all()


def test_nan_and_extreme_scales():
    inp = tiny(24, 16, 3, 128, 128, 12)
    w1_s = inp["w1_s"].copy()
    w2_s = inp["w2_s"].copy()
    w1_s[3, 5, 1] = 255       # NaN block in gate row 5 of expert 3
    w1_s[4, :, 0] = 0         # 2^-127 blocks: contribute ~0, must not misbehave
    w2_s[6, 9, 2] = 255       # NaN block in output row 9 of expert 6
    inp = dict(inp, w1_s=w1_s, w2_s=w2_s)
    whole_layer_parity(inp, 10.0)


def test_repeat_runs_are_bit_identical():
    inp = inputs.make_inputs(0)
    b1 = run_gpu(inp)
    y1 = b1.y.view(torch.int16).cpu().numpy().copy()
    ys1 = b1.y_sorted.view(torch.int16).cpu().numpy().copy()
    b2 = run_gpu(inp)
    assert np.array_equal(y1, b2.y.view(torch.int16).cpu().numpy())
    assert np.array_equal(ys1, b2.y_sorted.view(torch.int16).cpu().numpy())


def test_outputs_leave_guard_bytes_untouched():
    from mxfp4_routed_expert_route_amd import binding
    inp = tiny(37, 64, 6, 256, 128, 13)
    layer = _layer()
    dev = layer.to_device(inp)
    T, E, k, H, I = 37, 64, 6, 256, 128
    pad = 4096
    def guarded(n, dtype):
        nbytes = n * torch.tensor([], dtype=dtype).element_size()
        t = torch.full((nbytes + pad,), 0x5A, dtype=torch.uint8, device="cuda")
        return t, t[:nbytes].view(dtype)
    bufs = {}
    shapes = dict(ids=(T * k, torch.int32), w=(T * k, torch.float32), bm=(T * 2, torch.int32),
                  counts=(E, torch.int32), offsets=(E + 1, torch.int32), gather=(T * k, torch.int32),
                  scatter=(T * k, torch.int32), ys=(T * k * H, torch.bfloat16), y=(T * H, torch.bfloat16))
    for name, (n, dt) in shapes.items():
        bufs[name] = guarded(n, dt)
    ws_n = binding.moe_workspace_bytes(T, E, k, H, I)
    ws_raw, ws = guarded(ws_n, torch.uint8)
    v = {n: t[1] for n, t in bufs.items()}
    binding.moe_route(dev["logits"], k, v["ids"].view(T, k), v["w"].view(T, k))
    binding.moe_build_bitmatrix(v["ids"].view(T, k), E, v["bm"].view(T, 2))
    binding.moe_expert_offsets(v["bm"].view(T, 2), v["ids"].view(T, k), E, v["counts"], v["offsets"],
                               v["gather"], v["scatter"], ws)
    binding.moe_grouped_ffn_mxfp4(dev["x"], k, dev["w1"], dev["w1_s"], dev["w2"], dev["w2_s"],
                                  v["counts"], v["offsets"], v["gather"], 10.0,
                                  v["ys"].view(T * k, H), ws)
    binding.moe_combine(v["ys"].view(T * k, H), v["w"].view(T, k), v["scatter"], v["y"].view(T, H))
    torch.cuda.synchronize()
    for name, (raw, view) in list(bufs.items()) + [("ws", (ws_raw, ws))]:
        tail = raw[view.numel() * view.element_size():].cpu().numpy()
        assert (tail == 0x5A).all(), f"{name}: bytes past the end were written"


# ------------------------------------------------------------ full-size workloads
#
# Each full-size workload runs through moe_forward_mxfp4 (the launch configuration
# bench.py times) with the clamp at 10 and with the clamp off: at H = 4096 the gate
# and up values have a standard deviation of about 41, so with the clamp most of
# them saturate and W1 errors would be hidden.  Routing outputs are compared in
# full.  FFN rows: every row of four experts (the hottest, the second hottest, the
# median and the smallest), and the k rows and the output of sampled tokens (among
# them tokens routed to the hottest and to the smallest expert), each against the
# oracle restricted to those rows.

_FULL_CACHE = {}


def _full_inputs(index):
    if index not in _FULL_CACHE:
        _FULL_CACHE.clear()
        torch.cuda.empty_cache()
        wl = inputs.workload(index)
        _say(f"[full] workload {index} ({wl.name}) T={wl.T}: generating inputs")
        inp = inputs.make_inputs(index)
        ref = oracle_routing(inp["logits"], wl.E, wl.k)
        _FULL_CACHE[index] = (inp, _layer().to_device(inp), ref)
    return _FULL_CACHE[index]


def _check_experts(counts):
    touched = np.nonzero(counts)[0]
    by_count = touched[np.argsort(-counts[touched], kind="stable")]
    picks = [by_count[0], by_count[min(1, len(by_count) - 1)],
             by_count[len(by_count) // 2], by_count[-1]]
    return list(dict.fromkeys(int(e) for e in picks))   # hottest first, smallest last


def _sample_tokens(T, ids, experts, n=6):
    picks = {0, T - 1, T // 2}
    for e in experts:   # one token routed to each checked expert
        picks.add(int(np.nonzero((ids == e).any(axis=1))[0][-1]))
    rng = np.random.default_rng(T)
    while len(picks) < min(n + len(experts), T):
        picks.add(int(rng.integers(0, T)))
    return sorted(picks)


@pytest.mark.parametrize("index,limit", [(1, 10.0), (1, None), (2, 10.0), (2, None),
                                         (3, 10.0), (3, None), (4, 10.0), (4, None)])
def test_full_size_workload(index, limit):
    from tests import oracle_rows
    layer = _layer()
    wl = inputs.workload(index)
    inp, dev, ref = _full_inputs(index)
    b = layer.LayerBuffers.allocate(wl.T, wl.E, wl.k, wl.H, wl.I)
    _say(f"[full] workload {index}: moe_forward_mxfp4, limit={limit}")
    layer.run_forward(dev, b, 0.0 if limit is None else limit)
    torch.cuda.synchronize()
    check_routing(b, ref, wl.E, wl.k)
    ys = b.y_sorted.float().cpu().numpy()
    y = b.y.float().cpu().numpy()
    del b
    counts, offsets = ref["counts"], ref["offsets"]
    experts = _check_experts(counts)
    if index == 1:
        experts = [int(e) for e in np.nonzero(counts)[0]]   # every row of the verify step
    positions = np.concatenate([np.arange(offsets[e], offsets[e + 1]) for e in sorted(experts)])
    _say(f"[full] workload {index}: oracle on every row of experts "
         f"{[(e, int(counts[e])) for e in experts][:8]} ({len(positions)} rows)")
    ffn_close(ys[positions], oracle_rows.sorted_rows(inp, ref["gather"], offsets, wl.k,
                                                     positions, limit))
    S = _sample_tokens(wl.T, ref["ids"], experts[:1] + experts[-1:])
    _say(f"[full] workload {index}: oracle on tokens {S}")
    y_ref, ys_ref, pos = oracle_rows.token_outputs(inp, ref, wl.k, S, limit)
    ffn_close(ys[pos], ys_ref)
    ffn_close(y[S], y_ref)


def _random_shapes(seed, n):
    """Shapes drawn from a fixed generator: experts, k, rows per expert (every tile
    class), widths that are any multiple of 128 up to 1152, skewed routing or not,
    clamp on or off, separate calls or the one-call layer."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([4, 8, 16, 32, 64, 256]))
        k = int(rng.integers(1, min(8, E) + 1))
        rows = int(rng.choice([2, 6, 12, 20, 30, 50, 70, 100, 150]))
        T = int(max(1, min(1200, rows * E // k + int(rng.integers(-5, 6)))))
        H, I = 128 * int(rng.integers(1, 10)), 128 * int(rng.integers(1, 10))
        out.append((T, E, k, H, I, int(rng.integers(0, 10**6)), bool(rng.random() < 0.4),
                    [10.0, None][i % 2], i % 3 == 0))
    return out


@pytest.mark.parametrize("T,E,k,H,I,seed,skew,limit,fused", _random_shapes(2024, 24))
def test_random_shapes(T, E, k, H, I, seed, skew, limit, fused):
    whole_layer_parity(tiny(T, E, k, H, I, seed, skew=skew), limit, fused)
