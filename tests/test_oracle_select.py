"""Pins of the oracle's compressed scores, window->block pooling and selection.

Anchors: probability invariants (sums to the group size, uniform for equal keys,
one planted key takes the mass), visibility boundaries, token-range overlap by
Python sets, exhaustive subset search for top-k on tiny inputs, tie and
planted-score cases."""
import itertools
import math

import numpy as np
import pytest

import oracle


def _kc(rng, n_c, H_kv=2, D=16):
    return rng.standard_normal((n_c, H_kv, D))


def test_group_probs_sum_to_group_size_and_visibility():
    rng = np.random.default_rng(3)
    H, H_kv, D = 8, 2, 16
    q = rng.standard_normal((H, D))
    kc = _kc(rng, 20, H_kv, D)
    for t in (0, 30, 31, 32, 46, 47, 48, 200, 400):
        pg = oracle.group_window_probs(q, kc, t, 32, 16, 0.25)
        n_vis = sum(1 for c in range(20) if 16 * c + 31 <= t)
        if n_vis == 0:
            assert np.all(pg == 0)
            continue
        np.testing.assert_allclose(pg.sum(axis=1), H // H_kv, rtol=1e-13)
        assert np.all(pg[:, n_vis:] == 0)
        assert np.all(pg[:, :n_vis] > 0)
    # window c becomes visible exactly at t = 16c + 31
    assert oracle.group_window_probs(q, kc, 30, 32, 16, 0.25).sum() == 0
    assert oracle.group_window_probs(q, kc, 31, 32, 16, 0.25)[:, 0].tolist() == [4.0, 4.0]


def test_equal_keys_give_uniform_and_planted_key_takes_mass():
    rng = np.random.default_rng(4)
    H, H_kv, D = 8, 2, 16
    q = rng.standard_normal((H, D))
    kc = np.tile(rng.standard_normal((1, H_kv, D)), (12, 1, 1))
    pg = oracle.group_window_probs(q, kc, 10_000, 32, 16, 0.1)
    np.testing.assert_allclose(pg, 4.0 / 12, rtol=1e-13)
    # plant: window 5 of KV head 1 aligned with every query head of group 1
    kc = _kc(rng, 12, H_kv, D) * 0.01
    kc[5, 1] = q[4:8].sum(axis=0) * 50.0
    pg = oracle.group_window_probs(q, kc, 10_000, 32, 16, 1.0)
    assert pg[1, 5] == pytest.approx(4.0, rel=1e-6)
    assert pg[0].argmax() != 5 or pg[0, 5] < 3.0


def test_group_probs_match_per_head_softmax_of_a_hand_case():
    # two windows, one head per group, D=1: logits q*k*scale = [0, ln 3] -> P = [1/4, 3/4]
    q = np.array([[1.0], [2.0]])
    kc = np.array([[[0.0], [0.0]], [[math.log(3.0)], [math.log(3.0) / 2]]])
    pg = oracle.group_window_probs(q, kc, 1000, 32, 16, 1.0)
    np.testing.assert_allclose(pg, [[0.25, 0.75], [0.25, 0.75]], rtol=1e-14)


def _token_sets_overlap(c, b):
    return bool(set(range(16 * c, 16 * c + 32)) & set(range(64 * b, 64 * b + 64)))


def test_block_max_against_token_set_overlap():
    rng = np.random.default_rng(5)
    n_c, n_b = 40, 12
    w = rng.random((3, n_c))
    got = oracle.block_max(w, n_b, 32, 16, 64)
    for b in range(n_b):
        cs = [c for c in range(n_c) if _token_sets_overlap(c, b)]
        want = w[:, cs].max(axis=1) if cs else np.zeros(3)
        np.testing.assert_array_equal(got[:, b], want)
    # 32/16/64: windows 4b-1 .. 4b+3
    for b in range(1, 9):
        assert [c for c in range(n_c) if _token_sets_overlap(c, b)] == list(range(4 * b - 1, 4 * b + 4))
    # block 10 only overlaps window 39 of the 40; block 11 overlaps none and scores 0
    assert np.all(got[:, 10] == w[:, 39])
    assert np.all(got[:, 11] == 0.0)


def _brute_select(score, t, n_blk, k, n_init, n_local):
    n_elig = min(n_blk, t // 64 + 1)
    forced = set(range(min(n_init, n_elig))) | set(range(max(0, n_elig - n_local), n_elig))
    free = [b for b in range(n_elig) if b not in forced]
    m = min(len(free), k - len(forced))
    best, best_key = None, None
    for comb in itertools.combinations(free, m):
        key = (sum(score[b] for b in comb), [-b for b in comb])
        # maximise the score sum; among equal sums prefer lower ids (lexicographic)
        if best_key is None or key[0] > best_key[0] + 1e-12 or (
                abs(key[0] - best_key[0]) <= 1e-12 and sorted(comb) < sorted(best)):
            best, best_key = comb, key
    return sorted(forced | set(best))


@pytest.mark.parametrize("seed", range(12))
def test_select_equals_exhaustive_subset_search(seed):
    rng = np.random.default_rng(100 + seed)
    n_blk = int(rng.integers(3, 11))
    k = int(rng.integers(2, 8))
    n_init = int(rng.integers(0, 2))
    n_local = int(rng.integers(0, 3))
    if n_init + n_local > k:
        n_local = k - n_init
    t = int(rng.integers(0, 64 * n_blk))
    score = rng.random(n_blk)
    got = oracle.select_blocks(score, t, n_blk, k, n_init, n_local, 64)
    want = _brute_select(score, t, n_blk, k, n_init, n_local)
    assert got[:len(want)].tolist() == want
    assert np.all(got[len(want):] == -1)


def test_select_ties_planted_and_structure():
    n_blk, k = 64, 16
    # constant scores: forced {0, 62, 63} plus the lowest free ids
    got = oracle.select_blocks(np.zeros(n_blk), 4095, n_blk, k, 1, 2, 64)
    assert got.tolist() == list(range(0, 14)) + [62, 63]
    # planted high scores must appear
    s = np.zeros(n_blk)
    s[[7, 20, 33, 41]] = [5.0, 4.0, 3.0, 2.0]
    got = oracle.select_blocks(s, 4095, n_blk, 5, 1, 0, 64)
    assert got.tolist() == [0, 7, 20, 33, 41]
    # eligibility: start <= t only; fewer eligible than k -> -1 padding
    got = oracle.select_blocks(np.arange(n_blk, dtype=float), 200, n_blk, 8, 0, 0, 64)
    assert got.tolist() == [0, 1, 2, 3, -1, -1, -1, -1]
    # decode at L=4096: forced init and local, k counts them
    rng = np.random.default_rng(9)
    got = oracle.select_blocks(rng.random(n_blk), 4095, n_blk, 16, 1, 2, 64)
    assert {0, 62, 63} <= set(got.tolist()) and len(set(got.tolist())) == 16
    assert np.all(np.diff(got) > 0)


def test_decode_fusion_with_planted_cis():
    # q = 0 makes every compressed probability equal, so the pooled CIS alone
    # orders the blocks: CIS 0.9 on the tokens of block 7 and 0.1 elsewhere gives
    # block 7 the pooled max 0.9 and blocks 6 and 8 (their windows 27 and 31 are
    # half inside block 7) the max 0.5; every other block has 0.1.
    L, H, H_kv, D = 1024, 8, 2, 16
    rng = np.random.default_rng(15)
    k = rng.standard_normal((L, H_kv, D))
    cis = np.full((L, H_kv), 0.1)
    cis[448:512] = 0.9
    q = np.zeros((1, H, D))
    cu = np.array([0, L])
    res = oracle.decode_step(q, k, k, cu, topk=4, n_init=1, n_local=2, cis=cis, cis_select=True)
    assert res["indices"][0, 0].tolist() == [0, 7, 14, 15]
    res = oracle.decode_step(q, k, k, cu, topk=6, n_init=1, n_local=2, cis=cis, cis_select=True)
    assert res["indices"][0, 1].tolist() == [0, 6, 7, 8, 14, 15]
    sc = res["block_scores"][0, 0]
    n_c = oracle.n_windows(L, 32, 16)
    np.testing.assert_allclose(sc[7] - sc[6], 0.4, rtol=1e-12)
    np.testing.assert_allclose(sc[6] - sc[3], 0.4, rtol=1e-12)
    np.testing.assert_allclose(sc[3], 4.0 / n_c + 0.1, rtol=1e-12)


# ----------------------------------------------------------------------------- two-stage selection

def _brute_two_stage(s_qk, s_cis, t, n_blk, k, n_init, n_local, n_cand):
    """The two-stage rule by counting instead of sorting: a free block is a
    candidate when fewer than n_cand free blocks beat it on (score_qk desc, id
    asc), and it is chosen when fewer than k - |forced| candidates beat it on
    (score_cis desc, id asc)."""
    n_elig = min(n_blk, t // 64 + 1)
    forced = set(range(min(n_init, n_elig))) | set(range(max(0, n_elig - n_local), n_elig))
    free = [b for b in range(n_elig) if b not in forced]

    def beats(s, a, b):  # a ranks above b
        return s[a] > s[b] or (s[a] == s[b] and a < b)

    cand = [b for b in free if sum(beats(s_qk, a, b) for a in free if a != b) < n_cand]
    chosen = [b for b in cand
              if sum(beats(s_cis, a, b) for a in cand if a != b) < k - len(forced)]
    return sorted(forced | set(chosen))


@pytest.mark.parametrize("seed", range(16))
def test_two_stage_equals_counting_definition(seed):
    rng = np.random.default_rng(300 + seed)
    n_blk = int(rng.integers(3, 14))
    k = int(rng.integers(2, 9))
    n_init = int(rng.integers(0, 2))
    n_local = int(rng.integers(0, 3))
    if n_init + n_local > k:
        n_local = k - n_init
    n_cand = int(rng.integers(0, n_blk + 2))
    t = int(rng.integers(0, 64 * n_blk))
    # few distinct values, so ties occur in both stages
    s_qk = rng.integers(0, 4, n_blk).astype(float)
    s_cis = rng.integers(0, 3, n_blk).astype(float)
    got = oracle.select_blocks_two_stage(s_qk, s_cis, t, n_blk, k, n_init, n_local, 64, n_cand)
    want = _brute_two_stage(s_qk, s_cis, t, n_blk, k, n_init, n_local, n_cand)
    assert got[:len(want)].tolist() == want
    assert np.all(got[len(want):] == -1)


def test_two_stage_special_cases_reduce_to_one_stage():
    rng = np.random.default_rng(31)
    n_blk, k, t = 40, 12, 40 * 64 - 1
    s_qk, s_cis = rng.random(n_blk), rng.random(n_blk)
    n_free = n_blk - 1 - 3
    # every free block a candidate: the CIS scores alone rank them
    for n_cand in (n_free, n_free + 5):
        got = oracle.select_blocks_two_stage(s_qk, s_cis, t, n_blk, k, 1, 3, 64, n_cand)
        assert got.tolist() == oracle.select_blocks(s_cis, t, n_blk, k, 1, 3, 64).tolist()
    # as many candidates as free places: stage 2 keeps them all
    got = oracle.select_blocks_two_stage(s_qk, s_cis, t, n_blk, k, 1, 3, 64, k - 4)
    assert got.tolist() == oracle.select_blocks(s_qk, t, n_blk, k, 1, 3, 64).tolist()
    # fewer candidates than free places: only forced + candidates, -1 padded
    got = oracle.select_blocks_two_stage(s_qk, s_cis, t, n_blk, k, 1, 3, 64, 2)
    best2 = sorted(range(1, n_blk - 3), key=lambda b: (-s_qk[b], b))[:2]
    assert got.tolist() == sorted([0, 37, 38, 39] + best2) + [-1] * (k - 6)


def test_two_stage_planted():
    # blocks 5, 9 lead on the attention score but have the lowest CIS; block 30
    # has the best CIS but misses the candidate cut; among the candidates
    # {5, 9, 12, 20} the CIS keeps 12 and 20.
    n_blk = 40
    s_qk = np.zeros(n_blk)
    s_qk[[5, 9, 12, 20]] = [4.0, 3.0, 2.0, 1.0]
    s_cis = np.full(n_blk, 0.5)
    s_cis[[5, 9]] = 0.1
    s_cis[[12, 20]] = [0.8, 0.7]
    s_cis[30] = 0.99
    got = oracle.select_blocks_two_stage(s_qk, s_cis, 64 * n_blk - 1, n_blk, 3, 1, 0, 64, 4)
    assert got.tolist() == [0, 12, 20]


def test_two_stage_decode_with_uniform_attention_and_planted_cis():
    # q = 0: every block has the same compressed-attention score, so stage 1 takes
    # the lowest free ids; with CIS 0.9 on block 7 (0.5 on blocks 6 and 8 through
    # their half-covered windows, 0.1 elsewhere) stage 2 then decides.
    L, H, H_kv, D = 1024, 8, 2, 16
    rng = np.random.default_rng(16)
    k = rng.standard_normal((L, H_kv, D))
    cis = np.full((L, H_kv), 0.1)
    cis[448:512] = 0.9
    q = np.zeros((1, H, D))
    cu = np.array([0, L])
    kw = dict(topk=5, n_init=1, n_local=2, cis=cis, cis_select=True)
    res = oracle.decode_step(q, k, k, cu, n_cand=5, **kw)
    assert res["indices"][0, 0].tolist() == [0, 1, 2, 14, 15]
    res = oracle.decode_step(q, k, k, cu, n_cand=13, **kw)
    assert res["indices"][0, 1].tolist() == [0, 6, 7, 14, 15]
    np.testing.assert_allclose(res["cis_block_scores"][0, 0, [5, 6, 7, 8]], [0.1, 0.5, 0.9, 0.5],
                               rtol=1e-12)
    assert np.ptp(res["block_scores"][0, 0, :16]) == 0.0
