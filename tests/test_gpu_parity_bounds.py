"""GPU parity at the variant bounds and input forms the other parity files do not
reach: prefill selection over 1024- and 4096-block rows (the 16- and 64-slot
one-wave variants), decode at exactly 512 and 1024 blocks per row (the bounds of
the single-kernel select-and-attend variants), index rows in the form the
block-index attention is specified for (unique ids in any order, -1 entries
anywhere, ids past the query's position), and single-head groups through the
float32 attention kernel.  All calls go through the C ABI."""
import math

import numpy as np
import pytest
import torch

import gen
import oracle
import sparse_attention_compress_amd as nsa
from gen import workloads as W
from parity import assert_close, check_index_sets, cu, log, np64, report

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16, F32 = torch.bfloat16, torch.float32
SEED = 0x5EED0900


def _cu_np(t):
    return t.cpu().numpy().astype(np.int64)


def _row_positions(lk, lq):
    """(row, sequence, position) of packed query rows that are the last lq[b]
    tokens of each sequence."""
    out, r = [], 0
    for b, (L, n) in enumerate(zip(lk, lq)):
        for i in range(n):
            out.append((r, b, L - n + i))
            r += 1
    return out


# ------------------------------------------------------------------ prefill selection bounds

@pytest.mark.parametrize("max_len", [65536, 262144])
@pytest.mark.parametrize("k,n_init,n_local", [(16, 0, 0), (64, 1, 16), (16, 2, 3)])
def test_select_topk_prefill_bit_exact_long_rows(max_len, k, n_init, n_local):
    """Prefill rows of sequences up to 1024 and 4096 blocks (the 16- and 64-slot
    variants of the one-wave selection) on scores with many exact ties, with and
    without forced blocks: the ids must equal the oracle's bit for bit.  The rows
    are the last tokens of each sequence plus every row of a 2000-token one."""
    lk = [1, 63, 64, 65, 1000, 2000, 4096, 30000, max_len - 1000, max_len - 63, max_len]
    lq = [min(L, 5) for L in lk]
    lq[5] = 2000
    rows_total = sum(lq)
    nb_max = -(-max_len // 64)
    z = gen.normal(SEED + 1, 1, (rows_total, 2, nb_max), DEV)
    scores = (torch.floor(z * 4.0) / 4.0).contiguous()
    idx = torch.full((rows_total, 2, k), -7, dtype=torch.int32, device=DEV)
    log(f"select prefill long rows max_len={max_len} k={k} init={n_init} local={n_local}")
    nsa.nsa_select_topk(scores, idx, cu(lk), max_len, k, n_init, n_local, cu_seqlens_q=cu(lq))
    torch.cuda.synchronize()
    s = np64(scores)
    got = idx.cpu().numpy()
    for r, b, t in _row_positions(lk, lq):
        nb = -(-lk[b] // 64)
        for g in range(2):
            ref = oracle.select_blocks(s[r, g, :nb], t, nb, k, n_init, n_local, 64)
            assert got[r, g].tolist() == ref.tolist(), (r, b, t, g)


# ------------------------------------------------------------------ decode variant bounds

def _decode_inputs(lengths, seed, H=16, H_kv=2, dtype=BF16, kc_dtype=F32):
    N = sum(lengths)
    B = len(lengths)
    q = gen.normal(seed, 1, (B, H, 128), DEV, dtype)
    k = gen.normal(seed, 2, (N, H_kv, 128), DEV, dtype)
    v = gen.normal(seed, 3, (N, H_kv, 128), DEV, dtype)
    cis = gen.sigmoid_normal(seed, 4, (N, H_kv), DEV)
    nc = [nsa.window_count(L) for L in lengths]
    cu_k, cu_c = cu(lengths), cu(nc)
    kc = torch.zeros((max(1, sum(nc)), H_kv, 128), dtype=kc_dtype, device=DEV)
    cp = torch.zeros((max(1, sum(nc)), H_kv), dtype=F32, device=DEV)
    nsa.nsa_compress_k(k, kc, cu_k, cu_c, max(nc))
    nsa.nsa_cis_mean_pool_varlen(cis, cp, cu_k, cu_c, max(nc))
    return dict(q=q, k=k, v=v, cis=cis, kc=kc, cp=cp, cu_k=cu_k, cu_c=cu_c, nc=nc,
                lengths=list(lengths), H=H, H_kv=H_kv)


def _decode_and_check(name, d, topk, n_init, n_local, cis_select, cis_values, atol):
    B, H, H_kv = len(d["lengths"]), d["H"], d["H_kv"]
    max_len = max(d["lengths"])
    nb_max = -(-max_len // 64)
    out = torch.full((B, H, 128), float("nan"), dtype=d["q"].dtype, device=DEV)
    bs = torch.full((B, H_kv, nb_max), float("nan"), device=DEV)
    idx = torch.full((B, H_kv, topk), -7, dtype=torch.int32, device=DEV)
    p = nsa.decode_params(d["q"], d["k"], d["v"], d["kc"], d["cu_k"], d["cu_c"], max_len, out,
                          topk=topk, n_init=n_init, n_local=n_local, cis=d["cis"],
                          cis_pooled=d["cp"] if cis_select else None, cis_weight=1.0,
                          cis_values=cis_values, append_window=True, block_scores=bs, indices=idx)
    nsa.nsa_decode_step(p, device=DEV)
    torch.cuda.synchronize()
    q, k, v, cis = np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["cis"])
    res = oracle.decode_step(q, k, v, _cu_np(d["cu_k"]), topk=topk, n_init=n_init,
                             n_local=n_local, cis=cis, cis_select=cis_select,
                             cis_values=cis_values)
    bs_g, idx_g, out_g = np64(bs), idx.cpu().numpy(), np64(out)
    assert_close(name + ".block_scores", bs_g, res["block_scores"][:, :, :nb_max], atol=1e-9,
                 rtol=1e-4)
    G = H // H_kv
    exact, bands = 0, []
    for b, L in enumerate(d["lengths"]):
        nb = -(-L // 64)
        for g in range(H_kv):
            ok, band = check_index_sets(f"{name}[{b},{g}]", idx_g[b, g], res["indices"][b, g],
                                        res["block_scores"][b, g], L - 1, nb, topk, n_init, n_local)
            bands.append(band)
            if ok:
                exact += 1
                assert_close(f"{name}.out[{b},{g}]", out_g[b, g * G:(g + 1) * G],
                             res["out"][b, g * G:(g + 1) * G], atol=atol)
    report(f"[{name}] index sets identical for {exact}/{len(bands)} (row, kv); "
           f"tie-band population per row: {bands}")
    return exact, len(bands)


def test_decode_step_nosa1b_32k_pinned():
    """The batched decode recipe with every context at 32768 tokens: 512 blocks per
    row, exactly the bound of the lightest single-kernel variant (two id slabs per
    thread); every (sequence, KV head) is checked."""
    w = W.nosa1b_decode(pinned_32k=True)
    d = _decode_inputs(w.lengths, w.seed)
    log(f"decode step {w.name}")
    exact, n = _decode_and_check("pinned32k", d, w.topk, w.n_init, w.n_local, True, False, 2e-2)
    assert exact >= 1


def test_decode_step_exactly_1024_blocks():
    """Rows of exactly 1024 blocks (65536 tokens, and 65473, one token into the
    last block) next to a shorter row: the bound of the four-slab variant."""
    d = _decode_inputs([65536, 65473, 30000], SEED + 2)
    log("decode step at exactly 1024 blocks")
    exact, n = _decode_and_check("blocks1024", d, 64, 1, 16, True, False, 2e-2)
    assert exact >= 1


@pytest.mark.parametrize("cis_values", [False, True])
def test_decode_step_fp32_single_head_groups(cis_values):
    """float32 decode with as many query heads as KV heads (groups of one) through
    the separate selection and the float32 attention kernel, whose merge then
    covers 128 output values per workgroup of 256 threads."""
    d = _decode_inputs([700, 3000, 9000], SEED + 3, H=4, H_kv=4, dtype=F32)
    log(f"decode step fp32 H=H_kv=4 cis_values={cis_values}")
    exact, n = _decode_and_check("fp32_g1", d, 16, 1, 2, True, cis_values, 1e-4)
    assert exact >= 1


# ------------------------------------------------------------- index rows in the pages' form

def _pages_style_rows(rng, n_rows, nb_of_row, k):
    """Per row: up to k unique ids drawn uniformly from [0, nb_of_row(r) + 3)
    (ids past the query's own block, and past the sequence, included), in random
    order, with -1 entries scattered among them."""
    idx = np.full((n_rows, 2, k), -1, dtype=np.int32)
    for r in range(n_rows):
        hi = nb_of_row(r) + 3
        for g in range(2):
            n_ids = int(rng.integers(0, min(k, hi) + 1))
            ids = rng.permutation(hi)[:n_ids]
            slots = rng.permutation(k)[:n_ids]
            idx[r, g, slots] = ids
    return idx


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("cis_mode", [False, True])
def test_selected_attn_decode_pages_style_indices(dtype, cis_mode):
    """Decode rows whose index lists are unsorted, hold -1 in the middle and ids
    at or past the sequence's block count (skipped: their start lies beyond the
    query position, TileLang NSA section 2)."""
    lengths = [1, 64, 65, 700, 4096, 9000]
    d = _decode_inputs(lengths, SEED + 4, dtype=dtype)
    rng = np.random.default_rng(11)
    idx = _pages_style_rows(rng, len(lengths), lambda r: -(-lengths[r] // 64), 16)
    out = torch.full((len(lengths), 16, 128), float("nan"), dtype=dtype, device=DEV)
    log(f"selected attn decode, pages-style ids {dtype} cis={cis_mode}")
    nsa.nsa_selected_attn_fwd(d["q"], d["k"], d["v"], torch.from_numpy(idx).to(DEV), d["cu_k"],
                              max(lengths), out, cis=d["cis"] if cis_mode else None)
    torch.cuda.synchronize()
    q, k, v, cis = np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["cis"])
    cu_k = _cu_np(d["cu_k"])
    ref = np.stack([oracle.selected_attention_row(q[b], k[cu_k[b]:cu_k[b] + L],
                                                  v[cu_k[b]:cu_k[b] + L], idx[b], L - 1, 64,
                                                  1 / math.sqrt(128),
                                                  cis[cu_k[b]:cu_k[b] + L] if cis_mode else None)
                    for b, L in enumerate(lengths)])
    assert_close("decode_pages_ids", np64(out), ref, atol=2e-2 if dtype == BF16 else 1e-4)


@pytest.mark.parametrize("dtype,path", [(F32, "rows"), (BF16, "rows"), (BF16, "blocks")])
def test_selected_attn_prefill_pages_style_indices(dtype, path):
    """Prefill rows with ids drawn uniformly over the whole sequence's blocks (the
    pages' correctness check draws them with randint; here without repeats), so
    most rows list blocks past their own position, which must be skipped; -1
    entries and unsorted order as above."""
    lengths = [700, 1300]
    N = sum(lengths)
    q = gen.normal(SEED + 5, 1, (N, 16, 128), DEV, dtype)
    k = gen.normal(SEED + 5, 2, (N, 2, 128), DEV, dtype)
    v = gen.normal(SEED + 5, 3, (N, 2, 128), DEV, dtype)
    rng = np.random.default_rng(12)
    seq_of = np.repeat(np.arange(len(lengths)), lengths)
    idx = _pages_style_rows(rng, N, lambda r: -(-lengths[seq_of[r]] // 64), 16)
    cu_k = cu(lengths)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((N, 16), float("nan"), device=DEV)
    log(f"selected attn prefill, pages-style ids {dtype} path={path}")
    ws = None if path == "blocks" else torch.empty(0, dtype=torch.uint8, device=DEV)
    nsa.nsa_selected_attn_fwd(q, k, v, torch.from_numpy(idx).to(DEV), cu_k, max(lengths), out,
                              lse=lse, cu_seqlens_q=cu_k, workspace=ws)
    torch.cuda.synchronize()
    qn, kn, vn, got, lse_g = np64(q), np64(k), np64(v), np64(out), np64(lse)
    s0, r = 0, 0
    ref = np.zeros_like(got)
    ref_lse = np.full((N, 16), -np.inf)
    scale = 1 / math.sqrt(128)
    for L in lengths:
        for t in range(L):
            ref[r] = oracle.selected_attention_row(qn[r], kn[s0:s0 + L], vn[s0:s0 + L], idx[r], t,
                                                   64, scale)
            for h in (0, 9):
                J = oracle.selected_keys(idx[r, h // 8], t, L, 64)
                if J:
                    s = kn[s0 + np.array(J), h // 8] @ qn[r, h] * scale
                    ref_lse[r, h] = s.max() + math.log(np.exp(s - s.max()).sum())
            r += 1
        s0 += L
    assert_close("prefill_pages_ids", got, ref, atol=2e-2 if dtype == BF16 else 1e-4)
    for h in (0, 9):
        fin = np.isfinite(ref_lse[:, h])
        assert np.array_equal(np.isfinite(lse_g[:, h]), fin), "lse -inf pattern"
        assert_close(f"prefill_pages_lse[h={h}]", lse_g[fin, h], ref_lse[fin, h], atol=1e-3)


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_selected_attn_single_head_groups(dtype):
    """Groups of one query head (heads == kv_heads) through nsa_selected_attn_fwd,
    decode rows and prefill rows."""
    lengths = [90, 1000, 2500]
    N = sum(lengths)
    H = 4
    q = gen.normal(SEED + 6, 1, (N, H, 128), DEV, dtype)
    k = gen.normal(SEED + 6, 2, (N, H, 128), DEV, dtype)
    v = gen.normal(SEED + 6, 3, (N, H, 128), DEV, dtype)
    rng = np.random.default_rng(13)
    seq_of = np.repeat(np.arange(len(lengths)), lengths)
    pos = np.concatenate([np.arange(L) for L in lengths])
    idx = np.full((N, H, 16), -1, dtype=np.int32)
    for r in range(N):
        nb = pos[r] // 64 + 1
        for g in range(H):
            ids = np.sort(rng.permutation(nb)[:16])
            idx[r, g, :len(ids)] = ids
    cu_k = cu(lengths)
    out = torch.full_like(q, float("nan"))
    log(f"selected attn prefill, single-head groups {dtype}")
    nsa.nsa_selected_attn_fwd(q, k, v, torch.from_numpy(idx).to(DEV), cu_k, max(lengths), out,
                              cu_seqlens_q=cu_k)
    torch.cuda.synchronize()
    qn, kn, vn = np64(q), np64(k), np64(v)
    scale = 1 / math.sqrt(128)
    cu_np = _cu_np(cu_k)
    rows = list(range(0, N, 7)) + [N - 1]
    ref = np.stack([oracle.selected_attention_row(qn[r], kn[cu_np[seq_of[r]]:cu_np[seq_of[r] + 1]],
                                                  vn[cu_np[seq_of[r]]:cu_np[seq_of[r] + 1]], idx[r],
                                                  int(pos[r]), 64, scale) for r in rows])
    atol = 2e-2 if dtype == BF16 else 1e-4
    assert_close("prefill_g1", np64(out)[rows], ref, atol=atol)
    # decode rows: the newest token of each sequence
    last = cu_np[1:] - 1
    qd = q[torch.from_numpy(last).to(DEV)].contiguous()
    idx_d = torch.from_numpy(idx[last]).to(DEV)
    out_d = torch.full_like(qd, float("nan"))
    nsa.nsa_selected_attn_fwd(qd, k, v, idx_d, cu_k, max(lengths), out_d)
    torch.cuda.synchronize()
    ref_d = np.stack([oracle.selected_attention_row(qn[last[b]], kn[cu_np[b]:cu_np[b + 1]],
                                                    vn[cu_np[b]:cu_np[b + 1]], idx[last[b]], L - 1,
                                                    64, scale) for b, L in enumerate(lengths)])
    assert_close("decode_g1", np64(out_d), ref_d, atol=atol)
