"""The key-block-stationary selected attention over prefill rows
(nsa_selected_attn_fwd given a workspace) against the oracle, and beside it the
row-by-row kernel (no workspace) on the same inputs.

Cases: every group size the library builds (1, 2, 4, 8, 16 query heads per KV
head), 16, 20 and 64 places per index row, CIS mode, ragged batches whose query
rows are the tails of their sequences (a sequence without query rows, one
shorter than a block, one spanning three 1024-row scan chunks), index rows with
ids in any order, -1 anywhere, ids past the row's own block and rows with no
valid id (output 0, lse -inf).  The normaliser lse is checked on every head.
All calls go through the C ABI."""
import math

import numpy as np
import pytest
import torch

import gen
import oracle
import sparse_attention_compress_amd as nsa
from parity import assert_close, cu, log, np64, report

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16 = torch.bfloat16
SEED = 0x5EED0D00
SCALE = 1 / math.sqrt(128)


def _rows_ws(path):
    """Workspace argument selecting the path: None lets the binding allocate the
    queried size (key-block path); an empty buffer selects the row-by-row path."""
    return None if path == "blocks" else torch.empty(0, dtype=torch.uint8, device=DEV)


def _index_rows(rng, pos, kv_heads, k):
    """Per (row, KV head): unique ids drawn from the row's causal blocks plus two
    past them, in random order, at random places, the rest -1; about one row in
    forty lists nothing valid."""
    n = len(pos)
    idx = np.full((n, kv_heads, k), -1, dtype=np.int32)
    for r in range(n):
        hi = int(pos[r]) // 64 + 3
        for g in range(kv_heads):
            if rng.random() < 0.025:
                idx[r, g, rng.integers(0, k)] = hi - 1  # only a block past the row
                continue
            n_ids = max(0, min(k, hi) - int(rng.integers(0, 3)))
            ids = rng.permutation(hi)[:n_ids]
            idx[r, g, rng.permutation(k)[:n_ids]] = ids
    return idx


def _inputs(lk, lq, H, H_kv, k, seed):
    Nk, Nq = sum(lk), sum(lq)
    q = gen.normal(seed, 1, (Nq, H, 128), DEV, BF16)
    kk = gen.normal(seed, 2, (Nk, H_kv, 128), DEV, BF16)
    v = gen.normal(seed, 3, (Nk, H_kv, 128), DEV, BF16)
    cis = gen.sigmoid_normal(seed, 4, (Nk, H_kv), DEV)
    pos = np.concatenate([np.arange(L - n, L) for L, n in zip(lk, lq)]).astype(np.int64)
    seq = np.repeat(np.arange(len(lk)), lq)
    idx = _index_rows(np.random.default_rng(seed & 0xFFFF), pos, H_kv, k)
    return dict(q=q, k=kk, v=v, cis=cis, pos=pos, seq=seq, idx=idx,
                idx_t=torch.from_numpy(idx).to(DEV), cu_k=cu(lk), cu_q=cu(lq), max_len=max(lk))


def _run(d, path, cis_mode):
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full(d["q"].shape[:2], float("nan"), device=DEV)
    nsa.nsa_selected_attn_fwd(d["q"], d["k"], d["v"], d["idx_t"], d["cu_k"], d["max_len"], out,
                              cis=d["cis"] if cis_mode else None, lse=lse,
                              cu_seqlens_q=d["cu_q"], workspace=_rows_ws(path))
    torch.cuda.synchronize()
    return np64(out), np64(lse)


def _reference(d, rows, cis_mode):
    qn, kn, vn, cn = np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["cis"])
    cu_k = d["cu_k"].cpu().numpy().astype(np.int64)
    H, G = qn.shape[1], qn.shape[1] // kn.shape[1]
    ref = np.zeros((len(rows), H, 128))
    ref_lse = np.full((len(rows), H), -np.inf)
    for i, r in enumerate(rows):
        b, t = int(d["seq"][r]), int(d["pos"][r])
        s0, L = cu_k[b], cu_k[b + 1] - cu_k[b]
        ks, vs, cs = kn[s0:s0 + L], vn[s0:s0 + L], cn[s0:s0 + L]
        ref[i] = oracle.selected_attention_row(qn[r], ks, vs, d["idx"][r], t, 64, SCALE,
                                               cs if cis_mode else None)
        for h in range(H):
            J = oracle.selected_keys(d["idx"][r, h // G], t, L, 64)
            if not J:
                continue
            s = ks[J, h // G] @ qn[r, h] * SCALE
            w = cs[J, h // G] if cis_mode else np.ones(len(J))
            tot = (np.exp(s - s.max()) * w).sum()
            if tot > 0:
                ref_lse[i, h] = s.max() + math.log(tot)
    return ref, ref_lse


def _check(name, d, rows, got, lse, cis_mode):
    ref, ref_lse = _reference(d, rows, cis_mode)
    assert_close(name, got[rows], ref, atol=2e-2)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse[rows]), fin), f"{name}: lse -inf pattern"
    assert np.isfinite(got[rows]).all()
    empty = ~fin
    assert (got[rows][empty] == 0).all(), f"{name}: rows without keys must be 0"
    assert_close(name + "_lse", lse[rows][fin], ref_lse[fin], atol=1e-3)


def _sample(lq, chunk_edges=(0, 1, 63, 64, 1023, 1024, 1025, 2047, 2048, 2049)):
    rows, r0 = [], 0
    for n in lq:
        pick = set(range(min(n, 12))) | set(range(max(0, n - 6), n))
        pick |= {e for e in chunk_edges if e < n}
        pick |= set(np.linspace(0, max(n - 1, 0), 60).astype(int).tolist()) if n else set()
        rows += [r0 + i for i in sorted(pick)]
        r0 += n
    return rows


LK = [1, 63, 1500, 2600, 64, 700]
LQ = [1, 63, 1100, 2600, 0, 13]


@pytest.mark.parametrize("H,H_kv", [(16, 16), (8, 4), (8, 2), (16, 2), (32, 2)])
def test_block_path_group_sizes(H, H_kv):
    d = _inputs(LK, LQ, H, H_kv, 16, SEED + H * 7 + H_kv)
    log(f"block path H={H} H_kv={H_kv}")
    got, lse = _run(d, "blocks", False)
    rows = _sample(LQ)
    _check(f"blocks_g{H // H_kv}", d, rows, got, lse, False)
    rg, rl = _run(d, "rows", False)
    _check(f"rows_g{H // H_kv}", d, rows, rg, rl, False)
    report(f"block vs row path, G={H // H_kv}: max |diff| {np.abs(got - rg).max():.3g} over all rows")


@pytest.mark.parametrize("k_sel", [20, 64])
@pytest.mark.parametrize("cis_mode", [False, True])
def test_block_path_places_and_cis(k_sel, cis_mode):
    d = _inputs(LK, LQ, 16, 2, k_sel, SEED + k_sel + 100 * cis_mode)
    log(f"block path k_sel={k_sel} cis={cis_mode}")
    got, lse = _run(d, "blocks", cis_mode)
    _check(f"blocks_k{k_sel}_cis{int(cis_mode)}", d, _sample(LQ), got, lse, cis_mode)


def test_block_path_every_row_and_deterministic():
    """Every row of a batch with three scan chunks; two calls give the same bits."""
    lk, lq = [2300, 90, 1030], [2300, 90, 1030]
    d = _inputs(lk, lq, 16, 2, 16, SEED + 5)
    log("block path, every row")
    got, lse = _run(d, "blocks", False)
    _check("blocks_all_rows", d, list(range(sum(lq))), got, lse, False)
    got2, lse2 = _run(d, "blocks", False)
    assert np.array_equal(got, got2) and np.array_equal(lse, lse2), "not deterministic"


def test_block_path_workspace_too_small():
    d = _inputs([200], [200], 16, 2, 16, SEED + 6)
    need = nsa.selected_attn_workspace_size(200, 16, 2, 128, 16, False)
    # partial states (264 B per (row, head, place)) and block lists (10 B per (row, KV head, place))
    assert need == 200 * 16 * 16 * (256 + 8) + 200 * 2 * 16 * 10
    ws = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    out = torch.zeros_like(d["q"])
    with pytest.raises(nsa.NsaError) as e:
        nsa.nsa_selected_attn_fwd(d["q"], d["k"], d["v"], d["idx_t"], d["cu_k"], 200, out,
                                  cu_seqlens_q=d["cu_q"], workspace=ws)
    assert e.value.status == 3


@pytest.mark.parametrize("k_sel", [16, 64])
def test_block_path_every_place_listed(k_sel):
    """Single-row chunks whose k_sel ids are all distinct valid blocks: every
    place of the chunk is listed under its own block, so the chunk's list has
    no room for an end marker and the last listed block ends at the list's
    end."""
    lk, lq = [2048, 5000, 70], [1, 1, 1]
    d = _inputs(lk, lq, 16, 2, k_sel, SEED + 7 + k_sel)
    rng = np.random.default_rng(k_sel)
    idx = np.full((3, 2, k_sel), -1, dtype=np.int32)
    for r, t in enumerate([2047, 4999, 69]):
        n_blk = t // 64 + 1
        for g in range(2):
            ids = rng.permutation(n_blk)[:k_sel]
            idx[r, g, :len(ids)] = ids
    d["idx"], d["idx_t"] = idx, torch.from_numpy(idx).to(DEV)
    log(f"block path, every place listed, k_sel={k_sel}")
    got, lse = _run(d, "blocks", False)
    _check(f"blocks_full_list_k{k_sel}", d, [0, 1, 2], got, lse, False)
