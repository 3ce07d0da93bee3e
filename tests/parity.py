"""Shared helpers of the GPU parity tests: host copies, tolerance checks and the
index-set agreement rule.

Gates (the stated tolerances of the method's outputs, and derived ones where none is stated):
* pooled means in float32: |gpu - ref| <= 1e-5 * max(|ref|, mean |x| of the
  window), i.e. 1e-5 relative to the magnitude of the summands;
* attention outputs: 2e-2 absolute for bf16 inputs (fp32 accumulation); 1e-4
  absolute for fp32 inputs;
* block indices: identical when both sides select from identical scores; when
  each side selects from its own scores the sets must be equal unless the
  oracle's k-th and (k+1)-th free scores lie within 1e-3, and then every
  mismatched block must score within 1e-3 of the oracle's k-th free score.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import torch


BAND = 1e-3


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def report(*a):
    """A line that must survive pytest's output capture (agreement rates, band
    populations): written to the process's real stderr, and appended to the file
    named by NSA_PARITY_REPORT when that variable is set."""
    line = " ".join(str(x) for x in a)
    print(line, file=sys.__stderr__, flush=True)
    path = os.environ.get("NSA_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def cu(lengths, device="cuda") -> torch.Tensor:
    out = [0]
    for L in lengths:
        out.append(out[-1] + int(L))
    return torch.tensor(out, dtype=torch.int32, device=device)


def assert_close(name, got, ref, atol, rtol=0.0):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    err = np.abs(got - ref)
    lim = atol + rtol * np.abs(ref)
    bad = err > lim
    worst = float(err.max()) if err.size else 0.0
    log(f"[{name}] max abs err {worst:.3e} over {err.size} values")
    if bad.any():
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError(f"{name}: {int(bad.sum())} values out of tolerance; worst at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r} (atol {atol}, rtol {rtol})")
    return worst


def free_scores_sorted(scores, t, nb, n_init, n_local, block=64):
    n_elig = min(nb, t // block + 1)
    forced = set(range(min(n_init, n_elig))) | set(range(max(0, n_elig - n_local), n_elig))
    free = [(float(scores[b]), b) for b in range(n_elig) if b not in forced]
    free.sort(key=lambda x: (-x[0], x[1]))
    return free, forced


def check_index_sets(name, gpu_idx, ref_idx, ref_scores, t, nb, k, n_init, n_local, block=64):
    """Apply the agreement rule to one (row, kv head); returns (exact, band_population)."""
    g = sorted(int(x) for x in gpu_idx if x >= 0)
    r = sorted(int(x) for x in ref_idx if x >= 0)
    assert list(gpu_idx[len(g):]) == [-1] * (len(gpu_idx) - len(g)), f"{name}: bad padding {gpu_idx}"
    assert list(gpu_idx[:len(g)]) == g, f"{name}: not ascending {gpu_idx}"
    free, forced = free_scores_sorted(ref_scores, t, nb, n_init, n_local, block)
    kf = max(0, min(k - len(forced), len(free)))
    band_pop = 0
    if 0 < kf < len(free):
        kth = free[kf - 1][0]
        band_pop = sum(1 for s, _ in free if abs(s - kth) <= BAND)
    if g == r:
        return True, band_pop
    assert len(g) == len(r), f"{name}: {len(g)} ids vs {len(r)}"
    assert forced <= set(g), f"{name}: forced blocks missing"
    assert 0 < kf < len(free), f"{name}: sets differ with nothing to choose: {g} vs {r}"
    kth, nxt = free[kf - 1][0], free[kf][0]
    assert kth - nxt <= BAND, (f"{name}: index sets differ but the oracle's k-th/(k+1)-th free "
                               f"scores are {kth - nxt:.3e} apart (> {BAND})")
    for b in set(g) ^ set(r):
        assert abs(float(ref_scores[b]) - kth) <= BAND, f"{name}: block {b} outside the tie band"
    return False, band_pop


def check_two_stage_sets(name, gpu_idx, ref_idx, s_qk, s_cis, t, nb, k, n_init, n_local, n_cand,
                         block=64):
    """The agreement rule for the two-stage choice on one (row, kv head): the
    sets must be equal unless the oracle's stage-1 boundary (n_cand-th against
    (n_cand+1)-th free attention score) or its stage-2 boundary (the last kept
    against the first dropped candidate CIS score) lies within the band; the
    GPU set must be well formed in any case.  Returns whether they are equal."""
    g = sorted(int(x) for x in gpu_idx if x >= 0)
    r = sorted(int(x) for x in ref_idx if x >= 0)
    assert list(gpu_idx[len(g):]) == [-1] * (len(gpu_idx) - len(g)), f"{name}: bad padding {gpu_idx}"
    assert list(gpu_idx[:len(g)]) == g, f"{name}: not ascending {gpu_idx}"
    if g == r:
        return True
    free, forced = free_scores_sorted(s_qk, t, nb, n_init, n_local, block)
    assert len(g) == len(r), f"{name}: {len(g)} ids vs {len(r)}"
    assert forced <= set(g), f"{name}: forced blocks missing"
    c1 = min(n_cand, len(free))
    near1 = 0 < c1 < len(free) and free[c1 - 1][0] - free[c1][0] <= BAND
    cand = sorted((float(s_cis[b]), b) for _, b in free[:c1])
    cand.sort(key=lambda x: (-x[0], x[1]))
    kf = min(k - len(forced), c1)
    near2 = 0 < kf < c1 and cand[kf - 1][0] - cand[kf][0] <= BAND
    assert near1 or near2, (f"{name}: index sets differ with both stage boundaries outside the "
                            f"band: {g} vs {r}")
    return False
