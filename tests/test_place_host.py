"""pi_place_neurons (host only, no GPU): the placement of neurons over the 64-neuron tiles.

PowerInfer, "Neuron Placement and Management": neurons are laid out by how often they fire
and a neuron table maps each one back.  Pins: the result is a permutation; inside a tile the
neurons keep descending counts; the first T ranks open tiles 0..T-1 in order and the next T
close them in reverse (serpentine); with all counts equal the ranks are the original ids, so
the layout is known exactly; the tiles' count sums differ by at most the largest count; bad
arguments leave perm untouched.
"""
import ctypes

import numpy as np
import pytest

from activation_sparse_pi_amd import _lib as L


def place(counts):
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    perm = np.full(counts.size, -7, dtype=np.int32)
    st = L.pi_place_neurons(counts.ctypes.data, counts.size, perm.ctypes.data)
    return st, perm


def ranks(counts):
    return np.lexsort((np.arange(counts.size), -counts.astype(np.int64)))


@pytest.mark.parametrize("F", [1, 8, 63, 64, 65, 130, 1000, 11008])
def test_permutation_and_order_inside_tiles(F):
    rng = np.random.default_rng(F)
    counts = rng.zipf(1.3, F).clip(max=10_000).astype(np.int32)
    st, perm = place(counts)
    assert st == L.PI_OK
    assert np.array_equal(np.sort(perm), np.arange(F))
    for t0 in range(0, F, 64):
        c = counts[perm[t0:t0 + 64]]
        assert np.all(np.diff(c.astype(np.int64)) <= 0)


def test_serpentine_rounds():
    F, T = 64 * 10, 10
    counts = np.arange(F, 0, -1, dtype=np.int32)          # rank k = neuron k
    st, perm = place(counts)
    assert st == L.PI_OK
    for t in range(T):
        assert perm[t * 64] == t                          # pass 0, left to right
        assert perm[t * 64 + 1] == 2 * T - 1 - t          # pass 1, right to left
        assert perm[t * 64 + 2] == 2 * T + t              # pass 2, left to right


def test_equal_counts_give_the_original_ids_dealt():
    F, T = 256, 4
    st, perm = place(np.zeros(F, np.int32))
    assert st == L.PI_OK
    r = np.arange(64)
    for t in range(T):
        want = np.where(r % 2 == 0, r * T + t, r * T + (T - 1 - t))
        assert np.array_equal(perm[t * 64:(t + 1) * 64], want)


def test_tile_sums_balanced():
    F = 11008
    rng = np.random.default_rng(3)
    counts = (rng.pareto(1.2, F) * 20).clip(max=256).astype(np.int32)
    st, perm = place(counts)
    assert st == L.PI_OK
    sums = counts[perm].astype(np.int64).reshape(-1, 64).sum(1)
    assert sums.max() - sums.min() <= counts.max()
    # an unplaced layout of the same counts sorted by count is far from balanced
    s0 = np.sort(counts)[::-1].astype(np.int64).reshape(-1, 64).sum(1)
    assert s0.max() - s0.min() > 10 * (sums.max() - sums.min())


def test_last_tile_short():
    F = 64 * 3 + 5
    counts = np.arange(F, 0, -1, dtype=np.int32)
    st, perm = place(counts)
    assert st == L.PI_OK and np.array_equal(np.sort(perm), np.arange(F))
    assert np.array_equal(perm[192:], np.sort(perm[192:]))    # 5 entries, descending counts


def test_bad_arguments_leave_perm_untouched():
    counts = np.ones(10, np.int32)
    perm = np.full(10, -7, np.int32)
    assert L.pi_place_neurons(None, 10, perm.ctypes.data) == L.PI_ERR_NULL
    assert L.pi_place_neurons(counts.ctypes.data, 10, None) == L.PI_ERR_NULL
    assert L.pi_place_neurons(counts.ctypes.data, 0, perm.ctypes.data) == L.PI_ERR_SHAPE
    bad = counts.copy(); bad[3] = -1
    assert L.pi_place_neurons(bad.ctypes.data, 10, perm.ctypes.data) == L.PI_ERR_SHAPE
    assert "negative" in L.pi_last_error()
    assert np.all(perm == -7)


# ----------------------------------------------------------------------------- hot block layout
def place_hot(counts, ntok, rate):
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    perm = np.full(counts.size, -7, dtype=np.int32)
    nh = ctypes.c_int32(-1)
    st = L.pi_place_neurons_hot(counts.ctypes.data, counts.size, ntok, rate, perm.ctypes.data, nh)
    return st, perm, nh.value


@pytest.mark.parametrize("F", [8, 100, 1000, 11008])
def test_hot_block_first_then_cold_dealt(F):
    """Neurons at or above the rate lead, hottest first (ties by index); the rest is a
    serpentine deal over the free positions; the result is a permutation."""
    rng = np.random.default_rng(F + 5)
    ntok = 256
    counts = np.minimum(rng.zipf(1.4, F), ntok).astype(np.int32)
    counts[rng.permutation(F)[:F // 10]] = ntok - rng.integers(0, 20, F // 10)   # a hot set
    st, perm, nh = place_hot(counts, ntok, 0.9)
    assert st == L.PI_OK
    assert np.array_equal(np.sort(perm), np.arange(F))
    hot = np.flatnonzero(counts >= 0.9 * ntok)
    T = (F + 63) // 64
    assert nh == min(hot.size, 8 * T)
    r = ranks(counts)
    assert np.array_equal(perm[:nh], r[:nh])                       # hottest first, ties by id
    assert np.all(counts[perm[nh:]] < 0.9 * ntok) or nh == 8 * T
    # cold positions: within each tile, descending counts (a serpentine deal keeps rank order)
    for t0 in range(0, F, 64):
        lo = max(t0, nh)
        c = counts[perm[lo:t0 + 64]].astype(np.int64)
        assert np.all(np.diff(c) <= 0)


def test_hot_block_cap_and_exact_deal():
    """Every neuron hot: the block is capped at 8 per tile (32 of 256 here, ids 0..31 by the
    tie rule); the cold rest, all of equal count, is dealt serpentine over the positions
    32..255 -- tile 0's 32 free slots and tiles 1..3's 64."""
    F, T = 64 * 4, 4
    counts = np.full(F, 10, np.int32)
    st, perm, nh = place_hot(counts, 10, 0.5)
    assert st == L.PI_OK and nh == 8 * T
    assert np.array_equal(perm[:32], np.arange(32))
    assert np.array_equal(np.sort(perm), np.arange(F))
    # the deal: ranks 32, 33, ... go to tiles 0, 1, 2, 3, 3, 2, 1, 0, 0, 1, ...
    assert perm[32] == 32 and perm[64] == 33 and perm[128] == 34 and perm[192] == 35
    assert perm[193] == 36 and perm[129] == 37 and perm[65] == 38 and perm[33] == 39


def test_hot_block_bad_arguments():
    counts = np.ones(10, np.int32)
    perm = np.full(10, -7, np.int32)
    nh = ctypes.c_int32(-1)
    assert L.pi_place_neurons_hot(counts.ctypes.data, 10, 0, 0.5, perm.ctypes.data, nh) == L.PI_ERR_SHAPE
    assert L.pi_place_neurons_hot(counts.ctypes.data, 10, 5, 0.0, perm.ctypes.data, nh) == L.PI_ERR_SHAPE
    assert L.pi_place_neurons_hot(counts.ctypes.data, 10, 5, 1.5, perm.ctypes.data, nh) == L.PI_ERR_SHAPE
    big = counts.copy(); big[2] = 6
    assert L.pi_place_neurons_hot(big.ctypes.data, 10, 5, 0.5, perm.ctypes.data, nh) == L.PI_ERR_SHAPE
    assert np.all(perm == -7) and nh.value == -1
