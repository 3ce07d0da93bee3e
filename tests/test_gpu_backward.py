"""Selected-attention backward (nsa_selected_attn_bwd) on the GPU against the
float64 oracle's gradient.

Gate: the inputs are exactly the bf16 tensors the oracle widens, so the GPU's
differences come from fp32 accumulation, the forward's fp32 log-normaliser,
delta = dO . O taken from the bf16-rounded forward output (2^-9 relative per
element of O, about 1e-3 of the typical ds) and, for dK and dV, p and ds
entering the matrix-core contractions rounded to bf16 (2^-9 relative per term).
Each gradient must agree within 1e-2 of its largest oracle magnitude, dV
(which does not use delta) within 2^-8.  At full size, sampled dq rows are compared with the oracle and two
identities are checked over all keys: summed over the keys of a KV head, dK is
0 (per row and head the ds sum to 0), and dV equals the summed dO of the
group's heads over every row that sees a key (the p sum to 1).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_compress_amd as nsa
from gen import workloads as W
from parity import cu, log, np64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
F32 = torch.float32


def _inputs(w, q_lengths=None):
    """Inputs of a selected-prefill recipe; with q_lengths, the query rows of
    sequence b are its last q_lengths[b] positions."""
    q_all = W.prefill_query(w, DEV)
    k, v = W.keys_values(w, DEV)
    idx_all = W.given_block_indices(w, DEV)
    do_all = W.prefill_out_grad(w, DEV)
    if q_lengths is None:
        q_lengths = list(w.lengths)
    keep = []
    start = 0
    for L, Lq in zip(w.lengths, q_lengths):
        keep.extend(range(start + L - Lq, start + L))
        start += L
    keep = torch.tensor(keep, dtype=torch.int64, device=DEV)
    return dict(q=q_all[keep].contiguous(), k=k, v=v, idx=idx_all[keep].contiguous(),
                d_out=do_all[keep].contiguous(), cu_q=cu(q_lengths), cu_k=cu(w.lengths),
                max_len=max(w.lengths), q_lengths=list(q_lengths))


def _run(d, path="blocks"):
    """Forward, then the backward with dq key-block stationary ("blocks": the
    binding allocates the full queried workspace) or one workgroup per (row, KV
    head) ("rows": the smallest workspace)."""
    rows, H, D = d["q"].shape
    out = torch.empty_like(d["q"])
    lse = torch.empty((rows, H), dtype=F32, device=DEV)
    nsa.nsa_selected_attn_fwd(d["q"], d["k"], d["v"], d["idx"], d["cu_k"], d["max_len"], out,
                              lse=lse, cu_seqlens_q=d["cu_q"])
    dq = torch.full((rows, H, D), float("nan"), dtype=F32, device=DEV)
    dk = torch.full(d["k"].shape, float("nan"), dtype=F32, device=DEV)
    dv = torch.full(d["v"].shape, float("nan"), dtype=F32, device=DEV)
    ws = None
    if path == "rows":
        n = len(d["q_lengths"])
        ws = torch.empty(nsa.selected_attn_bwd_workspace_size_min(n, rows, d["max_len"], H,
                                                                  d["k"].shape[1], d["idx"].shape[2]),
                         dtype=torch.uint8, device=DEV)
    nsa.nsa_selected_attn_bwd(d["q"], d["k"], d["v"], out, d["d_out"], lse, d["idx"], d["cu_q"],
                              d["cu_k"], d["max_len"], dq, dk, dv, workspace=ws)
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


def _gate(name, got, ref, rel):
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    scale = max(np.abs(ref).max(), 1e-30)
    err = np.abs(got - ref).max()
    log(f"[{name}] max |gpu - oracle| = {err:.3e} (max |oracle| {scale:.3e})")
    assert err <= rel * scale, f"{name}: {err} > {rel} * {scale}"


def _compare(d, dq, dk, dv, tag):
    scale = 1.0 / np.sqrt(128.0)
    rq, rk, rv = oracle.selected_attention_bwd(
        np64(d["q"]), np64(d["k"]), np64(d["v"]), d["idx"].cpu().numpy(), np64(d["d_out"]),
        d["cu_q"].cpu().numpy(), d["cu_k"].cpu().numpy(), 64, scale)
    _gate(tag + ".dq", np64(dq), rq, 1e-2)
    _gate(tag + ".dk", np64(dk), rk, 1e-2)
    _gate(tag + ".dv", np64(dv), rv, 2.0 ** -8)


@pytest.mark.parametrize("H,H_kv,lengths", [(16, 2, [500, 900]), (16, 1, [300, 420]),
                                            (4, 4, [700, 90]), (8, 4, [500, 900]),
                                            (8, 2, [300, 420]), (8, 2, [1500, 700])])
@pytest.mark.parametrize("path", ["blocks", "rows"])
def test_selected_bwd_matches_oracle(H, H_kv, lengths, path):
    """Every row of a ragged batch (several 64-token blocks and a ragged tail;
    rows early in a sequence list fewer than k blocks), GQA groups of 8, 16, 1,
    2 and 4 query heads (the last two: chunks of 2*G*16 rows that are not a
    multiple of 256, and head counts below one 8-head pass)."""
    w = dataclasses.replace(W.scaled(W.selected_prefill(), lengths), heads=H, kv_heads=H_kv)
    d = _inputs(w)
    log(f"selected bwd H={H} H_kv={H_kv} lengths={lengths} dq path={path}")
    _, _, dq, dk, dv = _run(d, path)
    _compare(d, dq, dk, dv, f"bwd_g{H // H_kv}_{path}")


def test_selected_bwd_per_place_lists():
    """The block lists built one place at a time (the path for sequences of more
    than 8192 blocks; every other test builds them per chunk of rows): the same
    ragged batch with max_seqlen_k raised to 600000 tokens (9375 blocks); the
    forward runs row by row, the key-block grid being too large for it."""
    w = dataclasses.replace(W.scaled(W.selected_prefill(), [500, 900]), heads=8, kv_heads=2)
    d = _inputs(w)
    big = 600000
    rows, H, D = d["q"].shape
    log(f"selected bwd, per-place lists: max_seqlen_k={big}")
    out = torch.empty_like(d["q"])
    lse = torch.empty((rows, H), dtype=F32, device=DEV)
    nsa.nsa_selected_attn_fwd(d["q"], d["k"], d["v"], d["idx"], d["cu_k"], big, out, lse=lse,
                              cu_seqlens_q=d["cu_q"],
                              workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
    dq = torch.full((rows, H, D), float("nan"), dtype=F32, device=DEV)
    dk = torch.full(d["k"].shape, float("nan"), dtype=F32, device=DEV)
    dv = torch.full(d["v"].shape, float("nan"), dtype=F32, device=DEV)
    nsa.nsa_selected_attn_bwd(d["q"], d["k"], d["v"], out, d["d_out"], lse, d["idx"], d["cu_q"],
                              d["cu_k"], big, dq, dk, dv)
    torch.cuda.synchronize()
    _compare(d, dq, dk, dv, "bwd_per_place_lists")


@pytest.mark.parametrize("path", ["blocks", "rows"])
def test_selected_bwd_query_tails_and_empty_sequence(path):
    """Query rows that are only the last positions of their sequences (t offset
    by L - Lq), and a sequence with keys but no query rows: its dk and dv are 0."""
    w = W.scaled(W.selected_prefill(), [600, 200, 333])
    d = _inputs(w, q_lengths=[100, 0, 333])
    log("selected bwd query tails and a sequence without query rows")
    _, _, dq, dk, dv = _run(d, path)
    _compare(d, dq, dk, dv, f"bwd_tails_{path}")
    assert torch.count_nonzero(dk[600:800]) == 0 and torch.count_nonzero(dv[600:800]) == 0


@pytest.mark.parametrize("path", ["blocks", "rows"])
def test_selected_bwd_full_size_samples_and_identities(path):
    """The 8 x 16384-token selected-prefill recipe: sampled dq rows against the
    oracle, and the two key-sum identities over every key."""
    w = W.selected_prefill()
    d = _inputs(w)
    log("selected bwd full size 8 x 16384")
    out, lse, dq, dk, dv = _run(d, path)
    scale = 1.0 / np.sqrt(128.0)
    rows = d["q"].shape[0]
    H, H_kv, G = w.heads, w.kv_heads, w.group
    k64, v64 = np64(d["k"]), np64(d["v"])
    cu_np = d["cu_k"].cpu().numpy()
    rng = np.random.default_rng(5)
    for r in sorted(rng.choice(rows, size=12, replace=False).tolist()):
        b = int(np.searchsorted(cu_np, r, side="right") - 1)
        k0, k1 = int(cu_np[b]), int(cu_np[b + 1])
        t = r - k0
        dk_scratch = np.zeros(k64[k0:k1].shape)
        dv_scratch = np.zeros(v64[k0:k1].shape)
        ref = oracle.selected_attention_row_grad(np64(d["q"][r]), k64[k0:k1], v64[k0:k1],
                                                 d["idx"][r].cpu().numpy(), t, 64, scale,
                                                 np64(d["d_out"][r]), dk_scratch, dv_scratch)
        _gate(f"full.dq[{r}]", np64(dq[r]), ref, 1e-2)
    # identities, per sequence and KV head, summed over keys (float64 on the host)
    dk_np, dv_np, do_np = np64(dk), np64(dv), np64(d["d_out"])
    for b in range(w.batch):
        k0, k1 = int(cu_np[b]), int(cu_np[b + 1])
        for g in range(H_kv):
            s_dk = dk_np[k0:k1, g].sum(axis=0)
            s_dv = dv_np[k0:k1, g].sum(axis=0)
            want_dv = do_np[k0:k1, g * G:(g + 1) * G].sum(axis=(0, 1))
            mag_k = np.abs(dk_np[k0:k1, g]).sum(axis=0).max()
            mag_v = np.abs(want_dv).max() + np.abs(do_np[k0:k1, g * G:(g + 1) * G]).sum(axis=(0, 1)).max() * 1e-6
            # ds enters the dK contraction rounded to bf16 (2^-9 relative per term),
            # so the key sum of dK is zero only up to that share of its magnitude; a
            # dropped or doubled row or key would leave an O(1) share
            assert np.abs(s_dk).max() <= 2.0 ** -9 * mag_k, (b, g, np.abs(s_dk).max(), mag_k)
            assert np.abs(s_dv - want_dv).max() <= 1e-3 * mag_v + 1e-3, (b, g)
    log("full-size identities hold")
