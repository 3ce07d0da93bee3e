"""Pins of the oracle's attention steps and composed paths.

Anchor: torch's scaled_dot_product_attention in float64 on the CPU (a library
routine) with explicit boolean or additive masks, plus special cases (constant
values, a single visible key, constant CIS)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _sdpa(q, k, v, mask, scale):
    """q [H, D]; k, v [L, H, D] (already expanded per query head); mask [H, L]."""
    qt = torch.from_numpy(q)[:, None, :]                      # [H, 1, D]
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))   # [H, L, D]
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))
    m = torch.from_numpy(mask)[:, None, :]
    return F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)[:, 0].numpy()


def _expand(x, G):
    return np.repeat(x, G, axis=1)


def _case(rng, L, H=8, H_kv=2, D=32):
    q = rng.standard_normal((H, D))
    k = rng.standard_normal((L, H_kv, D))
    v = rng.standard_normal((L, H_kv, D))
    return q, k, v


@pytest.mark.parametrize("L,t", [(1, 0), (64, 63), (200, 150), (777, 776), (1024, 1000)])
def test_all_blocks_selected_equals_dense_causal(L, t):
    rng = np.random.default_rng(L)
    q, k, v = _case(rng, L)
    nb = -(-L // 64)
    idx = np.tile(np.arange(nb, dtype=np.int32), (2, 1))
    scale = 1 / math.sqrt(q.shape[1])
    got = oracle.selected_attention_row(q, k, v, idx, t, 64, scale)
    mask = np.zeros((8, L), dtype=bool)
    mask[:, :t + 1] = True
    want = _sdpa(q, _expand(k, 4), _expand(v, 4), mask, scale)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_selected_equals_masked_sdpa_with_skips():
    rng = np.random.default_rng(7)
    L, t = 700, 650
    q, k, v = _case(rng, L)
    # group 0: blocks 0, 3, 10 (its causal part) and an out-of-range id; group 1: -1 padded
    idx = np.array([[0, 3, 10, 11], [2, 5, -1, -1]], dtype=np.int32)
    scale = 0.17
    got = oracle.selected_attention_row(q, k, v, idx, t, 64, scale)
    mask = np.zeros((8, L), dtype=bool)
    for h in range(8):
        g = h // 4
        for blk in idx[g]:
            if blk < 0 or 64 * blk > t:
                continue
            mask[h, 64 * blk:min(64 * blk + 64, t + 1)] = True
    want = _sdpa(q, _expand(k, 4), _expand(v, 4), mask, scale)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    # block 10 starts at 640 <= 650: only tokens 640..650 count
    assert oracle.selected_keys(idx[0], t, L, 64)[-11:] == list(range(640, 651))


def test_constant_values_and_single_key():
    rng = np.random.default_rng(8)
    q, k, v = _case(rng, 300)
    v[:] = 2.5
    idx = np.array([[0, 2], [1, 4]], dtype=np.int32)
    got = oracle.selected_attention_row(q, k, v, idx, 299, 64, 0.3)
    np.testing.assert_allclose(got, 2.5, rtol=1e-14)
    q, k, v = _case(rng, 300)
    got = oracle.selected_attention_row(q, k, v, np.array([[0], [0]]), 0, 64, 0.3)
    np.testing.assert_allclose(got, _expand(v[0:1], 4)[0], rtol=1e-14)
    # nothing visible -> zeros
    got = oracle.selected_attention_row(q, k, v, np.array([[-1], [3]]), 100, 64, 0.3)
    assert np.all(got == 0)


def test_cis_mode_is_softmax_with_log_cis_bias():
    rng = np.random.default_rng(9)
    L, t = 500, 499
    q, k, v = _case(rng, L)
    cis = 1.0 / (1.0 + np.exp(-rng.standard_normal((L, 2))))
    idx = np.array([[0, 1, 4, 7], [0, 2, 5, 6]], dtype=np.int32)
    scale = 0.2
    got = oracle.selected_attention_row(q, k, v, idx, t, 64, scale, cis)
    bias = np.full((8, L), -np.inf)
    for h in range(8):
        g = h // 4
        for blk in idx[g]:
            sl = slice(64 * blk, min(64 * blk + 64, t + 1))
            bias[h, sl] = np.log(cis[sl, g])
    want = _sdpa(q, _expand(k, 4), _expand(v, 4), bias, scale)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    # constant CIS reduces to plain selected attention
    plain = oracle.selected_attention_row(q, k, v, idx, t, 64, scale)
    const = oracle.selected_attention_row(q, k, v, idx, t, 64, scale, np.full((L, 2), 0.37))
    np.testing.assert_allclose(const, plain, rtol=1e-13, atol=1e-14)


def test_window_branch_equals_banded_sdpa():
    rng = np.random.default_rng(10)
    L = 900
    q, k, v = _case(rng, L)
    for t in (0, 100, 511, 512, 899):
        got = oracle.window_attention_row(q, k, v, t, 512, 0.2)
        mask = np.zeros((8, L), dtype=bool)
        mask[:, max(0, t - 511):t + 1] = True
        want = _sdpa(q, _expand(k, 4), _expand(v, 4), mask, 0.2)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_compressed_branch_equals_sdpa_over_pooled_kv():
    rng = np.random.default_rng(11)
    L = 400
    q, k, v = _case(rng, L)
    nc = oracle.n_windows(L, 32, 16)
    kc = torch.nn.functional.avg_pool1d(torch.from_numpy(k.reshape(L, -1).T[None]), 32, 16)[0].T
    vc = torch.nn.functional.avg_pool1d(torch.from_numpy(v.reshape(L, -1).T[None]), 32, 16)[0].T
    kc = kc.numpy().reshape(nc, 2, -1)
    vc = vc.numpy().reshape(nc, 2, -1)
    for t in (31, 32, 47, 200, 399):
        got = oracle.compressed_attention_row(q, kc, vc, t, 32, 16, 0.2)
        mask = np.zeros((8, nc), dtype=bool)
        mask[:, :(t - 31) // 16 + 1] = True
        want = _sdpa(q, _expand(kc, 4), _expand(vc, 4), mask, 0.2)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    assert np.all(oracle.compressed_attention_row(q, kc, vc, 30, 32, 16, 0.2) == 0)


def test_decode_step_with_full_coverage_equals_dense():
    rng = np.random.default_rng(12)
    lengths = [70, 256, 300]
    H, H_kv, D = 8, 2, 16
    N = sum(lengths)
    q = rng.standard_normal((3, H, D))
    k = rng.standard_normal((N, H_kv, D))
    v = rng.standard_normal((N, H_kv, D))
    cis = 1.0 / (1.0 + np.exp(-rng.standard_normal((N, H_kv))))
    cu = oracle.cu_from_lengths(lengths)
    scale = 1 / math.sqrt(D)
    for cis_values in (False, True):
        res = oracle.decode_step(q, k, v, cu, topk=8, n_init=1, n_local=2, cis=cis,
                                 cis_select=True, cis_values=cis_values)
        for b, L in enumerate(lengths):
            ks, vs = k[cu[b]:cu[b + 1]], v[cu[b]:cu[b + 1]]
            bias = np.zeros((H, L))
            if cis_values:
                bias = np.log(_expand(cis[cu[b]:cu[b + 1]][:, :, None], 4)[:, :, 0].T)
            want = _sdpa(q[b], _expand(ks, 4), _expand(vs, 4), bias, scale)
            np.testing.assert_allclose(res["out"][b], want, rtol=1e-12, atol=1e-12)
            assert np.all(res["indices"][b][:, :-(-L // 64)] >= 0)


def test_decode_step_pooled_caches_equal_avg_pool1d():
    rng = np.random.default_rng(13)
    lengths = [100, 64]
    N = sum(lengths)
    k = rng.standard_normal((N, 2, 8))
    cis = rng.random((N, 2))
    res = oracle.decode_step(rng.standard_normal((2, 4, 8)), k, k, oracle.cu_from_lengths(lengths),
                             topk=2, n_init=1, n_local=1, cis=cis, cis_select=True)
    cuc = res["cu_seqlens_c"]
    for b, s0 in ((0, 0), (1, 100)):
        L = lengths[b]
        kk = torch.nn.functional.avg_pool1d(torch.from_numpy(k[s0:s0 + L].reshape(L, -1).T[None]), 32, 16)
        np.testing.assert_allclose(res["kc"][cuc[b]:cuc[b + 1]].reshape(-1, 16), kk[0].T.numpy(), rtol=1e-13)
        cc = torch.nn.functional.avg_pool1d(torch.from_numpy(cis[s0:s0 + L].T[None]), 32, 16)
        np.testing.assert_allclose(res["cis_pooled"][cuc[b]:cuc[b + 1]], cc[0].T.numpy(), rtol=1e-13)


def test_three_branch_gates_and_dense_equivalence():
    rng = np.random.default_rng(14)
    L, H, H_kv, D = 1100, 8, 2, 16
    q = rng.standard_normal((L, H, D))
    k = rng.standard_normal((L, H_kv, D))
    v = rng.standard_normal((L, H_kv, D))
    rows = [0, 40, 511, 700, 1023, 1099]
    for one in range(3):
        g = np.zeros((L, H, 3))
        g[:, :, one] = 1.0
        res = oracle.nsa_prefill_rows(q, k, v, g, rows, topk=16, window=512)
        branch = ("o_cmp", "o_sel", "o_win")[one]
        np.testing.assert_array_equal(res["out"], res[branch])
    g = rng.random((L, H, 3))
    res = oracle.nsa_prefill_rows(q, k, v, g, rows, topk=16, window=512)
    scale = 1 / math.sqrt(D)
    for i, t in enumerate(rows):
        mask = np.zeros((H, L), dtype=bool)
        mask[:, :t + 1] = True
        dense = _sdpa(q[t], _expand(k, 4), _expand(v, 4), mask, scale)
        if t < 1024:        # 16 blocks of 64 cover every causal block
            np.testing.assert_allclose(res["o_sel"][i], dense, rtol=1e-12, atol=1e-12)
        if t < 512:         # the window covers the whole prefix
            np.testing.assert_allclose(res["o_win"][i], dense, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(
            res["out"][i],
            g[t][:, 0:1] * res["o_cmp"][i] + g[t][:, 1:2] * res["o_sel"][i] + g[t][:, 2:3] * res["o_win"][i],
            rtol=1e-14)


# ----------------------------------------------------------------------------- block-mask attention

def _sdpa_masked(q, k, v, allowed):
    """torch's SDPA in float64 with a boolean [T, L] mask per head; rows with no
    allowed key are set to 0 (SDPA would give NaN)."""
    import torch
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]      # [1, H, T, D]
    kt = torch.from_numpy(k).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2)[None]
    m = torch.from_numpy(allowed)[None]                  # [1, H, T, L]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)
    o = torch.nan_to_num(o, nan=0.0)
    o = torch.where(m.any(-1, keepdim=True), o, torch.zeros_like(o))
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("density", [1.0, 0.5, 0.0])
def test_blockmask_attention_matches_masked_sdpa(causal, density):
    rng = np.random.default_rng(41)
    L, H, D, blk = 200, 3, 16, 64
    nb = -(-L // blk)
    q = rng.standard_normal((L, H, D))
    k = rng.standard_normal((L, H, D))
    v = rng.standard_normal((L, H, D))
    mask = (rng.random((H, nb, nb)) < density).astype(np.uint8)
    scale = 1 / math.sqrt(D)
    # the token-level mask written out from the blocks, independently of the oracle
    allowed = np.zeros((H, L, L), dtype=bool)
    for h in range(H):
        for t in range(L):
            for j in range(L):
                allowed[h, t, j] = bool(mask[h, t // blk, j // blk]) and (not causal or j <= t)
    ref = _sdpa_masked(q, k, v, allowed)
    got = np.stack([oracle.blockmask_attention_row(q[t], k, v, mask, t, blk, scale, causal)
                    for t in range(L)])
    np.testing.assert_allclose(got, ref, atol=1e-12)
    if density == 1.0 and not causal:
        # every block on: plain dense attention
        import torch
        dense = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(k).permute(1, 0, 2),
            torch.from_numpy(v).permute(1, 0, 2)).permute(1, 0, 2).numpy()
        np.testing.assert_allclose(got, dense, atol=1e-12)
    if density == 0.0:
        assert np.all(got == 0.0)


# ----------------------------------------------------------------------------- three-branch selection, planted

def _planted_three_branch_case():
    """Rows t >= 1024 of a sequence in which, for each KV group g, a run of 16
    consecutive blocks (the past run) holds keys with a large component along
    the group's own axis e_g, and every query head of the group has a large
    component along e_g too.  The compressed windows inside the run then take
    almost all of the group's compressed-attention mass (logit gap about 11
    against noise of about 0.3), the half-overlapping windows at the run's two
    ends lie about e^-5.6 below them, and the rest sit at noise level, so the
    top-16 blocks of the group are exactly the run.  A second, stronger run lies
    after the query rows (in the future): it is invisible to every checked row,
    and a selection that scored invisible windows would pick it instead."""
    rng = np.random.default_rng(20260)
    L, H, H_kv, D = 3000, 8, 2, 32
    G = H // H_kv
    a = b = 8.0
    q = rng.standard_normal((L, H, D))
    k = rng.standard_normal((L, H_kv, D))
    v = rng.standard_normal((L, H_kv, D))
    runs = {0: 2, 1: 0}              # first block of each group's past run (ends by token 1151)
    future = {0: 39, 1: 39}          # first block of the future run (tokens 2496 ..)
    for g in range(H_kv):
        q[:, g * G:(g + 1) * G, g] += a
        p0 = 64 * runs[g]
        k[p0:p0 + 16 * 64, g, g] += b
        f0 = 64 * future[g]
        k[f0:f0 + 6 * 64, g, g] += 2 * b
    rows = [1151, 1500, 2047, 2367, 2368, 2400, 2495]   # every past-run window visible
    expect = {g: list(range(runs[g], runs[g] + 16)) for g in range(H_kv)}
    return q, k, v, rows, expect, G


def _planted_pin_holds(prefill_rows):
    q, k, v, rows, expect, G = _planted_three_branch_case()
    L, H, D = q.shape
    g1 = np.zeros((L, H, 3))
    g1[:, :, 1] = 1.0
    res = prefill_rows(q, k, v, g1, rows, topk=16, window=512)
    scale = 1 / math.sqrt(D)
    for i, t in enumerate(rows):
        for g in expect:
            if res["indices"][i, g].tolist() != expect[g]:
                return False
        # o_sel against torch SDPA with the token mask written out from the runs
        mask = np.zeros((H, L), dtype=bool)
        for h in range(H):
            for blk in expect[h // G]:
                lo, hi = 64 * blk, min(64 * blk + 64, t + 1)
                mask[h, lo:hi] = True
        dense = _sdpa(q[t], _expand(k, G), _expand(v, G), mask, scale)
        if not np.allclose(res["o_sel"][i], dense, rtol=1e-12, atol=1e-12):
            return False
        if not np.array_equal(res["out"][i], res["o_sel"][i]):
            return False
    return True


def test_three_branch_selection_planted_rows_past_1024():
    """Rows t >= 1024, where 16 blocks no longer cover every causal block: the
    selection inside the three-branch oracle must return exactly the planted run
    of each KV group, and the selected branch must equal SDPA over those blocks
    (DeepSeek NSA with Triton, section 1.1: the selected branch ranks blocks by
    the group's compressed-attention probabilities; no forced blocks)."""
    assert _planted_pin_holds(oracle.nsa_prefill_rows)


@pytest.mark.parametrize("mutation", ["n_local_16", "n_init_1", "topk_15", "invisible_windows"])
def test_three_branch_planted_pin_catches_mutations(mutation, monkeypatch):
    """Plausible mistakes planted in a patched copy of the oracle's selection or
    scoring must make the planted pin fail."""
    import oracle.nsa as onsa
    real_select = onsa.select_blocks
    if mutation == "n_local_16":
        monkeypatch.setattr(onsa, "select_blocks",
                            lambda s, t, nb, k, ni, nl, blk: real_select(s, t, nb, k, ni, 16, blk))
    elif mutation == "n_init_1":
        monkeypatch.setattr(onsa, "select_blocks",
                            lambda s, t, nb, k, ni, nl, blk: real_select(s, t, nb, k, 1, nl, blk))
    elif mutation == "topk_15":
        def sel15(s, t, nb, k, ni, nl, blk):
            out = real_select(s, t, nb, k - 1, ni, nl, blk)
            return np.concatenate([out, [-1]]).astype(np.int32)
        monkeypatch.setattr(onsa, "select_blocks", sel15)
    else:  # invisible windows scored
        monkeypatch.setattr(onsa, "window_visible", lambda c, t, kernel, stride: True)
    assert not _planted_pin_holds(onsa.nsa_prefill_rows)
