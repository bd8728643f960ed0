"""Properties that routing outputs must have at any size, whoever produced them.

These checks hold for any correct implementation: each token has exactly k
distinct experts in [0, E); the bit matrix has exactly those bits and no
padding bit; counts sum to T*k and equal the bit matrix column sums; gather and
scatter are inverse permutations and gather is ordered by (expert, token).
Each function raises AssertionError with a message naming the broken property.
"""
from __future__ import annotations

import numpy as np


def popcount32(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a, dtype=np.uint64)
    c = np.zeros(a.shape, dtype=np.int64)
    for b in range(32):
        c += ((a >> np.uint64(b)) & np.uint64(1)).astype(np.int64)
    return c


def check_ids(ids, E: int, k: int):
    ids = np.asarray(ids)
    assert ids.ndim == 2 and ids.shape[1] == k, "ids shape"
    assert ((ids >= 0) & (ids < E)).all(), "expert id out of range"
    s = np.sort(ids, axis=1)
    assert (np.diff(s, axis=1) > 0).all(), "a token has a repeated expert"


def check_bitmatrix(bm, ids, E: int):
    bm = np.asarray(bm, dtype=np.uint32)
    ids = np.asarray(ids)
    T, k = ids.shape
    W = (E + 31) // 32
    assert bm.shape == (T, W), "bitmatrix shape"
    assert (popcount32(bm).sum(axis=1) == k).all(), "a row does not have exactly k bits"
    for j in range(k):
        e = ids[:, j].astype(np.int64)
        word = bm[np.arange(T), e >> 5]
        assert (((word >> (e & 31).astype(np.uint32)) & 1) == 1).all(), "bit of a chosen expert missing"
    if E % 32:
        pad_mask = np.uint32((0xFFFFFFFF << (E % 32)) & 0xFFFFFFFF)
        assert (bm[:, W - 1] & pad_mask == 0).all(), "padding bit set past E"


def bitmatrix_column_counts(bm, E: int) -> np.ndarray:
    bm = np.asarray(bm, dtype=np.uint64)
    cols = np.zeros(E, dtype=np.int64)
    for e in range(E):
        cols[e] = ((bm[:, e >> 5] >> np.uint64(e & 31)) & np.uint64(1)).sum()
    return cols


def check_offsets(counts, offsets, gather, scatter, ids, E: int, bm=None):
    ids = np.asarray(ids)
    T, k = ids.shape
    n = T * k
    counts = np.asarray(counts, dtype=np.int64)
    offsets = np.asarray(offsets, dtype=np.int64)
    gather = np.asarray(gather, dtype=np.int64)
    scatter = np.asarray(scatter, dtype=np.int64)
    assert counts.sum() == n, "counts do not sum to T*k"
    assert offsets[0] == 0 and offsets[-1] == n, "offsets ends"
    assert (np.diff(offsets) == counts).all(), "offsets are not the exclusive sum of counts"
    if bm is not None:
        assert (bitmatrix_column_counts(bm, E) == counts).all(), "counts differ from bitmatrix columns"
    assert np.array_equal(np.sort(gather), np.arange(n)), "gather is not a permutation"
    assert (scatter[gather] == np.arange(n)).all(), "scatter is not the inverse of gather"
    flat = ids.reshape(-1)
    experts = flat[gather]
    tokens = gather // k
    key = experts * (T + 1) + tokens
    assert (np.diff(key) > 0).all(), "gather not ordered by (expert, token)"
    for e in range(E):
        seg = experts[offsets[e]:offsets[e + 1]]
        assert (seg == e).all(), "gather segment holds another expert"
