"""Pins of the oracle's window geometry and mean pooling.

Anchors independent of the oracle's own code: torch's avg_pool1d (the pages'
own consistency check for the pooling kernel: NOSA-1B source analysis part 3,
consistency-check section), closed forms (constant and ramp inputs), a
hand-derived geometry fixture, and packing invariance."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


@pytest.mark.parametrize("L", [0, 1, 31, 32, 33, 47, 48, 49, 64, 100, 4096, 4097, 4111, 4112])
def test_full_window_count_matches_avg_pool1d(L):
    got = oracle.n_windows(L, 32, 16)
    if L < 32:
        assert got == 0
        return
    x = torch.zeros(1, 1, L, dtype=torch.float64)
    assert got == torch.nn.functional.avg_pool1d(x, 32, 16).shape[-1]


def test_geometry_fixture():
    with open(os.path.join(GOLDEN, "window_geometry.json")) as f:
        fx = json.load(f)
    k, s, blk = fx["kernel"], fx["stride"], fx["block"]
    for L, full, tail in fx["window_counts"]:
        assert oracle.n_windows(L, k, s) == full, L
        assert oracle.n_windows(L, k, s, tail=True) == tail, L
    for b, wins in fx["block_windows"]:
        got = [c for c in range(0, 64) if oracle.window_block_overlap(c, b, k, s, blk)]
        assert got == wins, b


def test_full_windows_equal_avg_pool1d_varlen():
    rng = np.random.default_rng(1)
    lengths = [32, 77, 500, 1024, 33]
    x = rng.standard_normal((sum(lengths), 3, 5))
    cu = _cu(lengths)
    nc = [oracle.n_windows(L, 32, 16) for L in lengths]
    cuc = _cu(nc)
    got = oracle.mean_pool_varlen(x, cu, cuc, 32, 16)
    for b, L in enumerate(lengths):
        seq = torch.from_numpy(x[cu[b]:cu[b + 1]])                 # [L, 3, 5]
        ref = torch.nn.functional.avg_pool1d(seq.reshape(L, 15).T.unsqueeze(0), 32, 16)
        ref = ref[0].T.reshape(-1, 3, 5).numpy()
        np.testing.assert_allclose(got[cuc[b]:cuc[b + 1]], ref, rtol=1e-13, atol=1e-13)


def test_constant_and_ramp_closed_forms():
    lengths = [40, 100, 257]
    cu = _cu(lengths)
    for tail in (False, True):
        nc = [oracle.n_windows(L, 32, 16, tail) for L in lengths]
        cuc = _cu(nc)
        const = np.full((sum(lengths), 2), 3.25)
        np.testing.assert_allclose(oracle.mean_pool_varlen(const, cu, cuc, 32, 16), 3.25)
        ramp = np.concatenate([np.arange(L, dtype=np.float64) for L in lengths])[:, None]
        got = oracle.mean_pool_varlen(ramp, cu, cuc, 32, 16)[:, 0]
        for b, L in enumerate(lengths):
            for c in range(nc[b]):
                lo, hi = 16 * c, min(16 * c + 32, L)       # valid tokens lo..hi-1
                assert got[cuc[b] + c] == pytest.approx((lo + hi - 1) / 2.0, abs=1e-12)


def test_packing_invariance_and_empty_windows():
    rng = np.random.default_rng(2)
    lengths = [50, 0, 130, 17]
    x = rng.standard_normal((sum(lengths), 4))
    cu = _cu(lengths)
    # ask for two windows more than the covering count: the extra ones are empty -> 0
    nc = [oracle.n_windows(L, 32, 16, tail=True) + 2 for L in lengths]
    cuc = _cu(nc)
    packed = oracle.mean_pool_varlen(x, cu, cuc, 32, 16)
    assert np.all(np.isfinite(packed))
    for b, L in enumerate(lengths):
        alone = oracle.mean_pool_varlen(x[cu[b]:cu[b + 1]], np.array([0, L]), np.array([0, nc[b]]), 32, 16)
        np.testing.assert_array_equal(packed[cuc[b]:cuc[b + 1]], alone)
        for c in range(nc[b]):
            if 16 * c >= L:                                    # no valid token
                assert np.all(packed[cuc[b] + c] == 0.0)
            else:
                assert np.any(packed[cuc[b] + c] != 0.0)


def test_tail_window_is_valid_suffix_mean():
    L = 57
    x = np.arange(L, dtype=np.float64)[:, None] ** 2
    n = oracle.n_windows(L, 32, 16, tail=True)
    assert n == 3                                              # windows at 0, 16, 32
    got = oracle.mean_pool_varlen(x, np.array([0, L]), np.array([0, n]), 32, 16)[:, 0]
    assert got[2] == pytest.approx(np.mean([j * j for j in range(32, 57)]))
