"""Backward of the compressed and sliding-window branches and of the window mean
on the GPU against the float64 oracle, and the whole three-branch gradient
composed from the branch entry points.  Calls go through the C ABI.

Gates (as for the selected-attention backward): the inputs are the exact bf16
tensors the oracle widens; the GPU differs by fp32 accumulation, by
delta = dO . O taken from the bf16-rounded branch output (2^-9 relative), and
by p and ds entering the matrix-core contractions rounded to bf16 (2^-9
relative per term), so dq and the key gradients must agree within 1e-2 of
their largest oracle magnitude and the value gradients (no delta term) within
2^-8 (twice the per-term rounding).  The composed gradient feeds
each branch gate * dO rounded to bf16 (nsa_gates_bwd; 2^-9 relative again), so
every part of it is gated at 1e-2.  The window-mean transpose is plain fp32 arithmetic:
1e-6 relative.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import gen
import oracle
import sparse_attention_compress_amd as nsa
from gen import workloads as W
from parity import check_index_sets, cu, log, np64

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
BF16, F32 = torch.bfloat16, torch.float32
SEED = 0x5EED0B00
DV_GATE = 2.0 ** -8


def _gate(name, got, ref, rel):
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    scale = max(np.abs(ref).max(), 1e-30)
    err = np.abs(got - ref).max()
    log(f"[{name}] max |gpu - oracle| = {err:.3e} (max |oracle| {scale:.3e})")
    assert err <= rel * scale, f"{name}: {err} > {rel} * {scale}"


@pytest.mark.parametrize("tail", [False, True])
@pytest.mark.parametrize("accumulate", [False, True])
def test_compress_bwd_matches_oracle(tail, accumulate):
    lengths = [0, 5, 31, 32, 33, 100, 1000, 4097]
    nc = [oracle.n_windows(L, 32, 16, tail) for L in lengths]
    cu_k, cu_c = cu(lengths), cu(nc)
    dxc = gen.normal(SEED + 1, 1, (max(1, sum(nc)), 2, 128), DEV)
    init = gen.normal(SEED + 1, 2, (sum(lengths), 2, 128), DEV)
    dx = init.clone() if accumulate else torch.full_like(init, float("nan"))
    log(f"compress bwd tail={tail} accumulate={accumulate}")
    nsa.nsa_compress_bwd(dxc, dx, cu_k, cu_c, max(lengths), accumulate=accumulate)
    torch.cuda.synchronize()
    ref = oracle.mean_pool_varlen_bwd(np64(dxc)[:sum(nc)], cu_k.cpu().numpy(), cu_c.cpu().numpy(),
                                      32, 16, sum(lengths))
    if accumulate:
        ref = ref + np64(init)
    got = np64(dx)
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-6)


def _window_case(lengths, q_lengths, H, H_kv, seed):
    w = dataclasses.replace(W.scaled(W.nsa_prefill(), lengths), heads=H, kv_heads=H_kv)
    q_all = W.prefill_query(w, DEV)
    k, v = W.keys_values(w, DEV)
    do_all = gen.normal(seed, 9, q_all.shape, DEV, BF16)
    keep, start = [], 0
    for L, Lq in zip(lengths, q_lengths):
        keep.extend(range(start + L - Lq, start + L))
        start += L
    keep = torch.tensor(keep, dtype=torch.int64, device=DEV)
    return dict(q=q_all[keep].contiguous(), k=k, v=v, d_out=do_all[keep].contiguous(),
                cu_q=cu(q_lengths), cu_k=cu(lengths), lengths=lengths, q_lengths=q_lengths,
                H=H, H_kv=H_kv)


def _row_positions(lengths, q_lengths):
    out = []
    for b, (L, n) in enumerate(zip(lengths, q_lengths)):
        out += [(b, L - n + i) for i in range(n)]
    return out


@pytest.mark.parametrize("H,H_kv,window", [(16, 2, 512), (16, 1, 64), (8, 8, 100)])
def test_window_bwd_matches_oracle(H, H_kv, window):
    """Ragged batch with query tails and a sequence without query rows; windows
    of 512, 64 and 100 keys; GQA groups of 8, 16 and 1."""
    lengths, q_lengths = [700, 300, 90, 1200], [700, 0, 40, 333]
    d = _window_case(lengths, q_lengths, H, H_kv, SEED + 2)
    rows = d["q"].shape[0]
    out = torch.empty_like(d["q"])
    lse = torch.empty((rows, H), dtype=F32, device=DEV)
    nsa.nsa_window_attn_fwd(d["q"], d["k"], d["v"], d["cu_q"], d["cu_k"], max(lengths), out,
                            window=window, lse=lse)
    dq = torch.full((rows, H, 128), float("nan"), dtype=F32, device=DEV)
    dk = torch.full(d["k"].shape, float("nan"), dtype=F32, device=DEV)
    dv = torch.full(d["v"].shape, float("nan"), dtype=F32, device=DEV)
    log(f"window bwd H={H} H_kv={H_kv} W={window}")
    nsa.nsa_window_attn_bwd(d["q"], d["k"], d["v"], out, d["d_out"], lse, d["cu_q"], d["cu_k"],
                            max(lengths), dq, dk, dv, window=window)
    torch.cuda.synchronize()
    q, k, v, do = np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["d_out"])
    cu_k = d["cu_k"].cpu().numpy()
    rdq = np.zeros(q.shape)
    rdk, rdv = np.zeros(k.shape), np.zeros(v.shape)
    scale = 1 / math.sqrt(128)
    for r, (b, t) in enumerate(_row_positions(lengths, q_lengths)):
        k0, k1 = cu_k[b], cu_k[b + 1]
        rdq[r] = oracle.window_attention_row_grad(q[r], k[k0:k1], v[k0:k1], t, window, scale, do[r],
                                                  rdk[k0:k1], rdv[k0:k1])
    _gate("window.dq", np64(dq), rdq, 1e-2)
    _gate("window.dk", np64(dk), rdk, 1e-2)
    _gate("window.dv", np64(dv), rdv, DV_GATE)
    assert torch.count_nonzero(dk[700:1000]) == 0 and torch.count_nonzero(dv[700:1000]) == 0


def _compressed_inputs(lengths, H, H_kv, seed):
    w = dataclasses.replace(W.scaled(W.nsa_prefill(), lengths), heads=H, kv_heads=H_kv)
    q = W.prefill_query(w, DEV)
    k, v = W.keys_values(w, DEV)
    nc = [oracle.n_windows(L, 32, 16) for L in lengths]
    cu_k, cu_c = cu(lengths), cu(nc)
    kc = torch.empty((max(1, sum(nc)), H_kv, 128), dtype=BF16, device=DEV)
    vc = torch.empty_like(kc)
    nsa.nsa_compress_k(k, kc, cu_k, cu_c, max(nc))
    nsa.nsa_compress_k(v, vc, cu_k, cu_c, max(nc))
    d_out = gen.normal(seed, 9, q.shape, DEV, BF16)
    return dict(w=w, q=q, k=k, v=v, kc=kc, vc=vc, nc=nc, cu_k=cu_k, cu_c=cu_c, d_out=d_out)


@pytest.mark.parametrize("H,H_kv,lengths", [(16, 2, [20, 700, 1500]), (32, 2, [300, 4100]),
                                            (4, 4, [33, 900])])
def test_compressed_bwd_matches_oracle(H, H_kv, lengths):
    """Every row of a ragged batch (one sequence shorter than a window: no row
    sees any window); dk_c, dv_c against the oracle, then through the window-mean
    transpose dk, dv."""
    d = _compressed_inputs(lengths, H, H_kv, SEED + 3)
    rows = d["q"].shape[0]
    o = torch.empty_like(d["q"])
    lse = torch.empty((rows, H), dtype=F32, device=DEV)
    nsa.nsa_compressed_attn_fwd(d["q"], d["kc"], d["vc"], d["cu_k"], d["cu_k"], d["cu_c"],
                                max(lengths), o, lse=lse)
    dq = torch.full((rows, H, 128), float("nan"), dtype=F32, device=DEV)
    dkc = torch.full(d["kc"].shape, float("nan"), dtype=F32, device=DEV)
    dvc = torch.full(d["vc"].shape, float("nan"), dtype=F32, device=DEV)
    log(f"compressed bwd H={H} H_kv={H_kv} lengths={lengths}")
    nsa.nsa_compressed_attn_bwd(d["q"], d["kc"], d["vc"], o, d["d_out"], lse, d["cu_k"], d["cu_k"],
                                d["cu_c"], max(lengths), dq, dkc, dvc)
    dk = torch.full(d["k"].shape, float("nan"), dtype=F32, device=DEV)
    dv = torch.full(d["v"].shape, float("nan"), dtype=F32, device=DEV)
    nsa.nsa_compress_bwd(dkc, dk, d["cu_k"], d["cu_c"], max(lengths))
    nsa.nsa_compress_bwd(dvc, dv, d["cu_k"], d["cu_c"], max(lengths))
    torch.cuda.synchronize()
    q, kc, vc, do = np64(d["q"]), np64(d["kc"]), np64(d["vc"]), np64(d["d_out"])
    cu_k, cu_c = d["cu_k"].cpu().numpy(), d["cu_c"].cpu().numpy()
    scale = 1 / math.sqrt(128)
    rdq = np.zeros(q.shape)
    rdkc, rdvc = np.zeros(kc.shape), np.zeros(vc.shape)
    for b, L in enumerate(lengths):
        c0, c1 = cu_c[b], cu_c[b + 1]
        for t in range(L):
            r = cu_k[b] + t
            rdq[r] = oracle.compressed_attention_row_grad(q[r], kc[c0:c1], vc[c0:c1], t, 32, 16,
                                                          scale, do[r], rdkc[c0:c1], rdvc[c0:c1])
    nct = int(cu_c[-1])
    _gate("compressed.dq", np64(dq), rdq, 1e-2)
    _gate("compressed.dk_c", np64(dkc)[:nct], rdkc[:nct], 1e-2)
    _gate("compressed.dv_c", np64(dvc)[:nct], rdvc[:nct], DV_GATE)
    rdk = oracle.mean_pool_varlen_bwd(rdkc[:nct], cu_k, cu_c, 32, 16, int(cu_k[-1]))
    rdv = oracle.mean_pool_varlen_bwd(rdvc[:nct], cu_k, cu_c, 32, 16, int(cu_k[-1]))
    _gate("compressed.dk", np64(dk), rdk, 1e-2)
    _gate("compressed.dv", np64(dv), rdv, DV_GATE)


def _three_branch_grads(d, g, topk, window):
    """The three-branch gradient from the branch entry points: forward of each
    branch with its normaliser, then selected (write), window (add) and
    compressed (add to dq; dk_c, dv_c through the window-mean transpose, added
    to dk, dv).  Each branch gets gate_b * dO, rounded to bf16."""
    w = d["w"]
    L = max(w.lengths)
    rows, H = d["q"].shape[0], w.heads
    H_kv = w.kv_heads
    nb_max = -(-L // 64)
    cu_k, cu_c = d["cu_k"], d["cu_c"]
    o_cmp = torch.empty_like(d["q"])
    lse_c = torch.empty((rows, H), dtype=F32, device=DEV)
    bs = torch.empty((rows, H_kv, nb_max), dtype=F32, device=DEV)
    nsa.nsa_compressed_attn_fwd(d["q"], d["kc"], d["vc"], cu_k, cu_k, cu_c, L, o_cmp, lse=lse_c,
                                block_scores=bs)
    idx = torch.empty((rows, H_kv, topk), dtype=torch.int32, device=DEV)
    nsa.nsa_select_topk(bs, idx, cu_k, L, topk, 0, 0, cu_seqlens_q=cu_k)
    o_sel = torch.empty_like(d["q"])
    lse_s = torch.empty((rows, H), dtype=F32, device=DEV)
    nsa.nsa_selected_attn_fwd(d["q"], d["k"], d["v"], idx, cu_k, L, o_sel, lse=lse_s,
                              cu_seqlens_q=cu_k)
    o_win = torch.empty_like(d["q"])
    lse_w = torch.empty((rows, H), dtype=F32, device=DEV)
    nsa.nsa_window_attn_fwd(d["q"], d["k"], d["v"], cu_k, cu_k, L, o_win, window=window, lse=lse_w)
    do_b = [torch.empty_like(d["d_out"]) for _ in range(3)]
    d_gates = torch.empty((rows, H, 3), dtype=F32, device=DEV)
    nsa.nsa_gates_bwd(d["d_out"], o_cmp, o_sel, o_win, g, do_b[0], do_b[1], do_b[2], d_gates)
    # the gate gradient and the per-branch output gradients: exact products of
    # the same bf16 values (the branch gradients rounded once to bf16)
    torch.cuda.synchronize()
    for j, o_b in enumerate((o_cmp, o_sel, o_win)):
        want = (g[:, :, j:j + 1].float() * d["d_out"].float()).to(BF16)
        assert torch.equal(do_b[j], want), f"gate-scaled gradient of branch {j}"
        ref_g = (d["d_out"].double() * o_b.double()).sum(-1)
        assert torch.allclose(d_gates[:, :, j].double(), ref_g, rtol=1e-5, atol=1e-5), j
    dq = torch.empty(d["q"].shape, dtype=F32, device=DEV)
    dk = torch.empty(d["k"].shape, dtype=F32, device=DEV)
    dv = torch.empty(d["v"].shape, dtype=F32, device=DEV)
    nsa.nsa_selected_attn_bwd(d["q"], d["k"], d["v"], o_sel, do_b[1], lse_s, idx, cu_k, cu_k, L,
                              dq, dk, dv)
    nsa.nsa_window_attn_bwd(d["q"], d["k"], d["v"], o_win, do_b[2], lse_w, cu_k, cu_k, L, dq, dk,
                            dv, window=window, accumulate=True)
    # accumulate bit 0 only: dq carries the other branches, dk_c and dv_c are written
    dkc = torch.full(d["kc"].shape, float("nan"), dtype=F32, device=DEV)
    dvc = torch.full(d["vc"].shape, float("nan"), dtype=F32, device=DEV)
    nsa.nsa_compressed_attn_bwd(d["q"], d["kc"], d["vc"], o_cmp, do_b[0], lse_c, cu_k, cu_k, cu_c,
                                L, dq, dkc, dvc, accumulate=1)
    nsa.nsa_compress_bwd(dkc, dk, cu_k, cu_c, L, accumulate=True)
    nsa.nsa_compress_bwd(dvc, dv, cu_k, cu_c, L, accumulate=True)
    torch.cuda.synchronize()
    return dq, dk, dv, idx


@pytest.mark.parametrize("L", [1000, 2048])
def test_three_branch_bwd_composed(L):
    """The whole three-branch gradient (compressed, selected and window
    branches, gates sigmoid(N(0,1)), 16 heads over 2 KV heads, window 512,
    top-16) on every row.  At 1000 tokens every causal block is selected; at
    2048 the GPU's block choice must satisfy the index-set rule against the
    oracle's on sampled rows.  The reference gradient is the oracle's per-branch
    gradients summed over all rows with the GPU's block choice (the choice
    itself passes no gradient)."""
    d = _compressed_inputs([L], 16, 2, SEED + 4)
    w = d["w"]
    g = W.gates(w, DEV)
    log(f"three-branch bwd L={L}")
    dq, dk, dv, idx = _three_branch_grads(d, g, 16, 512)
    q, k, v, do, gn = np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["d_out"]), np64(g)
    gi = idx.cpu().numpy()
    sampled = list(range(0, L, 9)) + [L - 1]
    ref = oracle.nsa_prefill_rows(q, k, v, gn, sampled, topk=16, window=512)
    nb = -(-L // 64)
    for i, t in enumerate(sampled):
        for kv in range(w.kv_heads):
            check_index_sets(f"t={t} kv={kv}", gi[t, kv], ref["indices"][i, kv],
                             ref["block_scores"][i, kv], t, nb, 16, 0, 0)
    if L <= 1024:
        assert all(gi[t].tolist() == ref["indices"][i].tolist() for i, t in enumerate(sampled))
    scale = 1 / math.sqrt(128)
    nc = d["nc"][0]
    kc = oracle.mean_pool_varlen(k, [0, L], [0, nc], 32, 16)
    vc = oracle.mean_pool_varlen(v, [0, L], [0, nc], 32, 16)
    rdq = np.zeros(q.shape)
    rdk, rdv = np.zeros(k.shape), np.zeros(v.shape)
    rdkc, rdvc = np.zeros(kc.shape), np.zeros(vc.shape)
    for t in range(L):
        rdq[t] = oracle.compressed_attention_row_grad(q[t], kc, vc, t, 32, 16, scale,
                                                      gn[t][:, 0:1] * do[t], rdkc, rdvc)
        rdq[t] += oracle.selected_attention_row_grad(q[t], k, v, gi[t], t, 64, scale,
                                                     gn[t][:, 1:2] * do[t], rdk, rdv)
        rdq[t] += oracle.window_attention_row_grad(q[t], k, v, t, 512, scale,
                                                   gn[t][:, 2:3] * do[t], rdk, rdv)
    rdk += oracle.mean_pool_varlen_bwd(rdkc, [0, L], [0, nc], 32, 16, L)
    rdv += oracle.mean_pool_varlen_bwd(rdvc, [0, L], [0, nc], 32, 16, L)
    _gate("three_branch.dq", np64(dq), rdq, 1e-2)
    _gate("three_branch.dk", np64(dk), rdk, 1e-2)
    _gate("three_branch.dv", np64(dv), rdv, 1e-2)
