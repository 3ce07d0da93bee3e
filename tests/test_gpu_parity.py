"""GPU parity of every step of the hot path against the float64 CPU oracle, on
seeded inputs at sizes the oracle finishes in seconds that still span several
workgroup tiles and ragged tails.  All calls go through the C ABI (ctypes)."""
import math

import numpy as np
import pytest
import torch

import gen
import oracle
import sparse_attention_compress_amd as nsa
from gen import workloads as W
from parity import assert_close, check_index_sets, check_two_stage_sets, cu, log, np64, report

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16, F32 = torch.bfloat16, torch.float32
SEED = 0x5EED0100


def _cu_np(t):
    return t.cpu().numpy().astype(np.int64)


# ------------------------------------------------------------------------------ pooling

@pytest.mark.parametrize("tail", [False, True])
def test_cis_mean_pool_varlen(tail):
    lengths = [0, 1, 31, 32, 33, 100, 4097, 20000]
    N = sum(lengths)
    cis = gen.sigmoid_normal(SEED, 4, (N, 2), device=DEV)
    # tail mode: covering windows plus one more (possibly without any valid token)
    nc = [oracle.n_windows(L, 32, 16, tail) + (1 if tail else 0) for L in lengths]
    cu_k, cu_c = cu(lengths), cu(nc)
    out = torch.full((sum(nc), 2), float("nan"), device=DEV)
    log(f"cis pool tail={tail} lengths={lengths}")
    nsa.nsa_cis_mean_pool_varlen(cis, out, cu_k, cu_c, max(nc))
    torch.cuda.synchronize()
    x = np64(cis)
    ref = oracle.mean_pool_varlen(x, _cu_np(cu_k), _cu_np(cu_c), 32, 16)
    scale = oracle.mean_pool_varlen(np.abs(x), _cu_np(cu_k), _cu_np(cu_c), 32, 16)
    assert_close("cis_pool", np64(out), ref, atol=1e-5 * np.maximum(np.abs(ref), scale))


@pytest.mark.parametrize("src,dst", [(BF16, F32), (BF16, BF16), (F32, F32)])
def test_compress_k(src, dst):
    lengths = [31, 32, 100, 4097, 9000]
    N = sum(lengths)
    x = gen.normal(SEED, 2, (N, 2, 128), DEV, src)
    nc = [oracle.n_windows(L, 32, 16) for L in lengths]
    cu_k, cu_c = cu(lengths), cu(nc)
    x_c = torch.full((sum(nc), 2, 128), float("nan"), dtype=dst, device=DEV)
    log(f"compress_k {src}->{dst}")
    nsa.nsa_compress_k(x, x_c, cu_k, cu_c, max(nc))
    torch.cuda.synchronize()
    xx = np64(x)
    ref = oracle.mean_pool_varlen(xx, _cu_np(cu_k), _cu_np(cu_c), 32, 16)
    scale = oracle.mean_pool_varlen(np.abs(xx), _cu_np(cu_k), _cu_np(cu_c), 32, 16)
    rtol = 0.0 if dst == F32 else 2.0 ** -7       # one bf16 ulp of the rounded mean
    assert_close("compress_k", np64(x_c), ref, atol=1e-5 * scale, rtol=rtol)


# ------------------------------------------------------------------------------ scoring

def _decode_inputs(lengths, seed, H=16, H_kv=2, dtype=BF16, kc_dtype=F32):
    N = sum(lengths)
    B = len(lengths)
    q = gen.normal(seed, 1, (B, H, 128), DEV, dtype)
    k = gen.normal(seed, 2, (N, H_kv, 128), DEV, dtype)
    v = gen.normal(seed, 3, (N, H_kv, 128), DEV, dtype)
    cis = gen.sigmoid_normal(seed, 4, (N, H_kv), DEV)
    nc = [oracle.n_windows(L, 32, 16) for L in lengths]
    cu_k, cu_c = cu(lengths), cu(nc)
    kc = torch.zeros((max(1, sum(nc)), H_kv, 128), dtype=kc_dtype, device=DEV)
    cp = torch.zeros((max(1, sum(nc)), H_kv), dtype=F32, device=DEV)
    nsa.nsa_compress_k(k, kc, cu_k, cu_c, max(nc))
    nsa.nsa_cis_mean_pool_varlen(cis, cp, cu_k, cu_c, max(nc))
    return dict(q=q, k=k, v=v, cis=cis, kc=kc, cp=cp, cu_k=cu_k, cu_c=cu_c, nc=nc,
                lengths=list(lengths), H=H, H_kv=H_kv)


@pytest.mark.parametrize("kc_dtype", [F32, BF16])
@pytest.mark.parametrize("with_cis", [False, True])
def test_compressed_scores_decode(kc_dtype, with_cis):
    lengths = [31, 40, 1000, 5000, 17000]
    d = _decode_inputs(lengths, SEED + 1, kc_dtype=kc_dtype)
    B, H_kv = len(lengths), d["H_kv"]
    max_len = max(lengths)
    nb_max = -(-max_len // 64)
    nc_max = oracle.n_windows(max_len, 32, 16)
    bs = torch.full((B, H_kv, nb_max), float("nan"), device=DEV)
    wp = torch.full((B, H_kv, nc_max), float("nan"), device=DEV)
    log(f"compressed scores kc={kc_dtype} cis={with_cis}")
    nsa.nsa_compressed_scores(d["q"], d["kc"], d["cu_k"], d["cu_c"], max_len, bs, wp,
                              cis_pooled=d["cp"] if with_cis else None, cis_weight=1.0)
    torch.cuda.synchronize()
    q, k, cis = np64(d["q"]), np64(d["k"]), np64(d["cis"])
    cu_k = _cu_np(d["cu_k"])
    scale = 1 / math.sqrt(128)
    rtol = 1e-4 if kc_dtype == F32 else 3e-3
    ref_wp = np.zeros((B, H_kv, nc_max))
    ref_bs = np.zeros((B, H_kv, nb_max))
    for b, L in enumerate(lengths):
        s0 = cu_k[b]
        nc = d["nc"][b]
        kc_b = oracle.mean_pool_varlen(k[s0:s0 + L], [0, L], [0, nc], 32, 16)
        cp_b = oracle.mean_pool_varlen(cis[s0:s0 + L], [0, L], [0, nc], 32, 16)
        nb = -(-L // 64)
        ref_wp[b, :, :nc] = oracle.group_window_probs(q[b], kc_b, L - 1, 32, 16, scale)
        ref_bs[b, :, :nb] = oracle.decode_block_scores(q[b], kc_b, L - 1, nb, 32, 16, 64, scale,
                                                       cp_b if with_cis else None, 1.0)
    assert_close("window_probs", np64(wp), ref_wp, atol=1e-9, rtol=rtol)
    assert_close("block_scores", np64(bs), ref_bs, atol=1e-9, rtol=rtol)


# ----------------------------------------------------------------------------- selection

@pytest.mark.parametrize("k,n_init,n_local", [(64, 1, 16), (16, 1, 2), (16, 0, 0)])
def test_select_topk_decode_bit_exact(k, n_init, n_local):
    lengths = [1, 64, 65, 1000, 4096, 33000, 131072]
    B = len(lengths)
    nb_max = -(-max(lengths) // 64)
    z = gen.normal(SEED + 2, 1, (B, 2, nb_max), DEV)
    scores = (torch.floor(z * 8.0) / 8.0).contiguous()     # many exact ties
    idx = torch.full((B, 2, k), -7, dtype=torch.int32, device=DEV)
    cu_k = cu(lengths)
    log(f"select decode k={k} init={n_init} local={n_local}")
    nsa.nsa_select_topk(scores, idx, cu_k, max(lengths), k, n_init, n_local)
    torch.cuda.synchronize()
    s = np64(scores)
    got = idx.cpu().numpy()
    for b, L in enumerate(lengths):
        nb = -(-L // 64)
        for g in range(2):
            ref = oracle.select_blocks(s[b, g, :nb], L - 1, nb, k, n_init, n_local, 64)
            assert got[b, g].tolist() == ref.tolist(), (b, g)


@pytest.mark.parametrize("dist", ["tiny_wide_range", "with_infinities", "all_equal", "two_values"])
def test_select_topk_edge_distributions(dist):
    """Score sets that stress the histogram selection: distinct values spread over
    many binades (deep refinement), +/-inf (no finite range), all equal and two
    values (pure ties, decided by the lower id)."""
    lengths = [4096, 65536, 131072, 20000]
    B = len(lengths)
    nb_max = -(-max(lengths) // 64)
    z = np64(gen.normal(SEED + 12, 1, (B, 2, nb_max)))
    if dist == "tiny_wide_range":
        # exponents spread over most of float32's normal range, 2^-120 .. 2^120
        sc = np.exp2(np.clip(np.floor(z * 40.0), -120, 120)) * (1.0 + 0.5 * np.tanh(z))
        sc = sc.astype(np.float32)
        assert np.isfinite(sc).all() and (sc > 0).all()
    elif dist == "with_infinities":
        sc = z.astype(np.float32)
        sc[:, :, ::97] = np.inf
        sc[:, :, 5::89] = -np.inf
    elif dist == "all_equal":
        sc = np.full(z.shape, 0.25, dtype=np.float32)
    else:
        sc = np.where(z > 0.3, 1.0, 0.5).astype(np.float32)
    scores = torch.from_numpy(sc).to(DEV)
    idx = torch.full((B, 2, 64), -7, dtype=torch.int32, device=DEV)
    cu_k = cu(lengths)
    log(f"select edge distribution {dist}")
    nsa.nsa_select_topk(scores, idx, cu_k, max(lengths), 64, 1, 16)
    torch.cuda.synchronize()
    s64 = sc.astype(np.float64)
    got = idx.cpu().numpy()
    for b, L in enumerate(lengths):
        nb = -(-L // 64)
        for g in range(2):
            ref = oracle.select_blocks(s64[b, g, :nb], L - 1, nb, 64, 1, 16, 64)
            assert got[b, g].tolist() == ref.tolist(), (dist, b, g)


def test_select_topk_prefill_bit_exact():
    lengths = [100, 3000]
    rows = sum(lengths)
    nb_max = -(-max(lengths) // 64)
    z = gen.normal(SEED + 3, 1, (rows, 2, nb_max), DEV)
    scores = (torch.floor(z * 4.0) / 4.0).contiguous()
    idx = torch.full((rows, 2, 16), -7, dtype=torch.int32, device=DEV)
    cu_k = cu(lengths)
    log("select prefill")
    nsa.nsa_select_topk(scores, idx, cu_k, max(lengths), 16, 0, 0, cu_seqlens_q=cu_k)
    torch.cuda.synchronize()
    s = np64(scores)
    got = idx.cpu().numpy()
    r = 0
    for L in lengths:
        nb = -(-L // 64)
        for t in range(L):
            for g in range(2):
                ref = oracle.select_blocks(s[r, g, :nb], t, nb, 16, 0, 0, 64)
                assert got[r, g].tolist() == ref.tolist(), (r, t, g)
            r += 1


# ----------------------------------------------------------------------------- attention

def _oracle_indices(lengths, k, n_init, n_local, seed):
    """Block lists from the oracle's selection on seeded random scores."""
    out = []
    for b, L in enumerate(lengths):
        nb = -(-L // 64)
        sc = np64(gen.normal(seed, 9 + b, (2, nb)))
        out.append(np.stack([oracle.select_blocks(sc[g], L - 1, nb, k, n_init, n_local, 64)
                             for g in range(2)]))
    return np.stack(out).astype(np.int32)


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("cis_mode", [False, True])
def test_selected_attn_decode(dtype, cis_mode):
    lengths = [1, 63, 64, 65, 700, 4096, 9000]
    d = _decode_inputs(lengths, SEED + 4, dtype=dtype)
    B, H = len(lengths), d["H"]
    idx = _oracle_indices(lengths, 16, 1, 2, SEED + 5)
    idx_t = torch.from_numpy(idx).to(DEV)
    out = torch.full((B, H, 128), float("nan"), dtype=dtype, device=DEV)
    log(f"selected attn decode {dtype} cis={cis_mode}")
    nsa.nsa_selected_attn_fwd(d["q"], d["k"], d["v"], idx_t, d["cu_k"], max(lengths), out,
                              cis=d["cis"] if cis_mode else None)
    torch.cuda.synchronize()
    q, k, v, cis = np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["cis"])
    cu_k = _cu_np(d["cu_k"])
    ref = np.zeros((B, H, 128))
    for b, L in enumerate(lengths):
        s0 = cu_k[b]
        ref[b] = oracle.selected_attention_row(q[b], k[s0:s0 + L], v[s0:s0 + L], idx[b], L - 1, 64,
                                               1 / math.sqrt(128),
                                               cis[s0:s0 + L] if cis_mode else None)
    assert_close("selected_attn", np64(out), ref, atol=2e-2 if dtype == BF16 else 1e-4)


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_selected_attn_block_mass_probe(dtype):
    """V_j = one-hot(block(j) mod 128): each output coordinate is the attention mass
    of one block, so a dropped or doubled block shows at O(1/k) scale."""
    lengths = [4096, 9000, 3000]
    d = _decode_inputs(lengths, SEED + 6, dtype=dtype)
    N = sum(lengths)
    pos = torch.cat([torch.arange(L) for L in lengths])
    onehot = torch.zeros((N, 2, 128), dtype=dtype)
    onehot[torch.arange(N), :, (pos // 64) % 128] = 1.0
    v = onehot.to(DEV)
    idx = _oracle_indices(lengths, 16, 1, 2, SEED + 7)
    out = torch.full((len(lengths), 16, 128), float("nan"), dtype=dtype, device=DEV)
    log(f"block-mass probe {dtype}")
    nsa.nsa_selected_attn_fwd(d["q"], d["k"], v, torch.from_numpy(idx).to(DEV), d["cu_k"],
                              max(lengths), out)
    torch.cuda.synchronize()
    q, k, vv = np64(d["q"]), np64(d["k"]), np64(v)
    cu_k = _cu_np(d["cu_k"])
    ref = np.stack([oracle.selected_attention_row(q[b], k[cu_k[b]:cu_k[b] + L], vv[cu_k[b]:cu_k[b] + L],
                                                  idx[b], L - 1, 64, 1 / math.sqrt(128))
                    for b, L in enumerate(lengths)])
    assert_close("block_mass", np64(out), ref, atol=2e-3)


def _path_ws(path):
    """None: the binding allocates the queried workspace (key-block path for
    bf16 prefill rows); an empty buffer: the row-by-row path."""
    return None if path == "blocks" else torch.empty(0, dtype=torch.uint8, device=DEV)


def _sample_rows(lengths, extra=40):
    rows, r0 = [], 0
    for L in lengths:
        pick = set(range(min(L, 20))) | set(range(max(0, L - 10), L))
        pick |= {t for t in (63, 64, 65, 127, 128, 511, 512, 1023, 1024, 1025) if t < L}
        pick |= set(np.linspace(0, L - 1, extra).astype(int).tolist())
        rows += [(r0 + t, t) for t in sorted(pick)]
        r0 += L
    return rows


@pytest.mark.parametrize("path", ["blocks", "rows"])
@pytest.mark.parametrize("cis_mode", [False, True])
def test_selected_attn_prefill_given_indices(cis_mode, path):
    w = W.scaled(W.selected_prefill(), [1500, 2100])
    q = W.prefill_query(w, DEV)
    k, v = W.keys_values(w, DEV)
    cis = W.cis_scores(w, DEV)
    idx = W.given_block_indices(w, DEV)
    cu_k = cu(w.lengths)
    out = torch.full_like(q, float("nan"))
    log(f"prefill selected attn cis={cis_mode} path={path}")
    nsa.nsa_selected_attn_fwd(q, k, v, idx, cu_k, max(w.lengths), out,
                              cis=cis if cis_mode else None, cu_seqlens_q=cu_k,
                              workspace=_path_ws(path))
    torch.cuda.synchronize()
    rows = _sample_rows(w.lengths)
    qn, kn, vn, cn, idxn = np64(q), np64(k), np64(v), np64(cis), idx.cpu().numpy()
    got = np64(out)
    cu_np = _cu_np(cu_k)
    ref = np.zeros((len(rows), 16, 128))
    gsel = np.zeros_like(ref)
    for i, (r, t) in enumerate(rows):
        b = int(np.searchsorted(cu_np, r, side="right") - 1)
        s0, L = cu_np[b], cu_np[b + 1] - cu_np[b]
        ref[i] = oracle.selected_attention_row(qn[r], kn[s0:s0 + L], vn[s0:s0 + L], idxn[r], t, 64,
                                               1 / math.sqrt(128), cn[s0:s0 + L] if cis_mode else None)
        gsel[i] = got[r]
    assert_close("prefill_selected", gsel, ref, atol=2e-2)


# ----------------------------------------------------------------------------- whole path

def _run_decode_step(d, topk, n_init, n_local, cis_select, cis_values, append=False):
    B, H = len(d["lengths"]), d["H"]
    max_len = max(d["lengths"])
    nb_max = -(-max_len // 64)
    out = torch.full((B, H, 128), float("nan"), dtype=d["q"].dtype, device=DEV)
    bs = torch.full((B, d["H_kv"], nb_max), float("nan"), device=DEV)
    idx = torch.full((B, d["H_kv"], topk), -7, dtype=torch.int32, device=DEV)
    p = nsa.decode_params(d["q"], d["k"], d["v"], d["kc"], d["cu_k"], d["cu_c"], max_len, out,
                          topk=topk, n_init=n_init, n_local=n_local, cis=d["cis"],
                          cis_pooled=d["cp"] if cis_select else None, cis_weight=1.0,
                          cis_values=cis_values, append_window=append, block_scores=bs, indices=idx)
    nsa.nsa_decode_step(p, device=DEV)
    torch.cuda.synchronize()
    return out, bs, idx


def _check_decode(name, d, out, bs, idx, topk, n_init, n_local, cis_select, cis_values, atol):
    q, k, v, cis = np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["cis"])
    cu_k = _cu_np(d["cu_k"])
    res = oracle.decode_step(q, k, v, cu_k, topk=topk, n_init=n_init, n_local=n_local, cis=cis,
                             cis_select=cis_select, cis_values=cis_values)
    bs_g, idx_g, out_g = np64(bs), idx.cpu().numpy(), np64(out)
    nb_max = bs_g.shape[2]
    assert_close(name + ".block_scores", bs_g, res["block_scores"][:, :, :nb_max], atol=1e-9, rtol=1e-4)
    exact_rows, bands = 0, []
    for b, L in enumerate(d["lengths"]):
        nb = -(-L // 64)
        for g in range(d["H_kv"]):
            ok, band = check_index_sets(f"{name}[{b},{g}]", idx_g[b, g], res["indices"][b, g],
                                        res["block_scores"][b, g], L - 1, nb, topk, n_init, n_local)
            bands.append(band)
            if ok:
                G = d["H"] // d["H_kv"]
                assert_close(f"{name}.out[{b},{g}]", out_g[b, g * G:(g + 1) * G],
                             res["out"][b, g * G:(g + 1) * G], atol=atol)
                exact_rows += 1
    report(f"[{name}] index sets identical for {exact_rows}/{len(bands)} (row, kv); "
           f"tie-band population per row: {bands}")
    return res


def test_decode_step_tiny_fp32_full_size():
    w = W.tiny_decode()
    d = _decode_inputs(w.lengths, w.seed, dtype=F32)
    log("decode step: tiny fp32 L=4096")
    out, bs, idx = _run_decode_step(d, 16, 1, 2, False, False)
    _check_decode("tiny", d, out, bs, idx, 16, 1, 2, False, False, atol=1e-4)


def test_decode_step_nosa_small():
    d = _decode_inputs([300, 2000, 5000, 9000], SEED + 8)
    log("decode step: nosa-shaped small batch")
    out, bs, idx = _run_decode_step(d, 64, 1, 16, True, False)
    _check_decode("nosa_small", d, out, bs, idx, 64, 1, 16, True, False, atol=2e-2)


def test_decode_step_cis_values_small():
    d = _decode_inputs([5000, 8192], SEED + 9)
    log("decode step: CIS-valued small batch")
    out, bs, idx = _run_decode_step(d, 64, 1, 16, True, True)
    _check_decode("cis_small", d, out, bs, idx, 64, 1, 16, True, True, atol=2e-2)


@pytest.mark.parametrize("topk,n_local", [(16, 2), (64, 16)])
def test_decode_step_edge_lengths(topk, n_local):
    """Degenerate sequences in one decode batch: empty, shorter than one window,
    exactly one window, one and two blocks, and a ragged tail; with the newest
    window refreshed.  The empty sequence's output is 0."""
    lengths = [0, 1, 31, 32, 33, 64, 65, 1000, 4097]
    d = _decode_inputs(lengths, SEED + 12)
    log(f"decode step edge lengths {lengths} topk={topk} n_local={n_local}")
    out, bs, idx = _run_decode_step(d, topk, 1, n_local, True, False, append=True)
    assert torch.equal(out[0].float(), torch.zeros_like(out[0].float()))
    assert (idx[0] == -1).all()
    _check_decode("edge", d, out, bs, idx, topk, 1, n_local, True, False, atol=2e-2)


@pytest.mark.parametrize("lengths", [[1000, 60000, 33000], [513 * 64, 200], [1025 * 64 - 5, 3000],
                                     [100000, 2048 * 64]])
def test_decode_step_long_rows(lengths):
    """Rows of more than 512 blocks in the single-kernel decode path, which then
    keeps four (up to 1024 blocks) or eight (up to 2048) id slabs per thread
    instead of two; the second and third batches sit just past the lighter
    variants' bounds, the last one at the 2048-block limit."""
    d = _decode_inputs(lengths, SEED + 14)
    log(f"decode step long rows {lengths}")
    out, bs, idx = _run_decode_step(d, 64, 1, 16, True, False)
    _check_decode("long_rows", d, out, bs, idx, 64, 1, 16, True, False, atol=2e-2)


@pytest.mark.parametrize("cis_values", [False, True])
def test_decode_step_beyond_fused_limit(cis_values):
    """A row of more than 2048 blocks sends the bf16 decode step through the
    separate selection kernel and the split attention kernel instead."""
    d = _decode_inputs([2049 * 64 + 17, 5000], SEED + 15)
    log(f"decode step beyond the single-kernel limit cis_values={cis_values}")
    out, bs, idx = _run_decode_step(d, 64, 1, 16, True, cis_values, append=True)
    _check_decode("beyond_fused", d, out, bs, idx, 64, 1, 16, True, cis_values, atol=2e-2)


def _run_two_stage(d, topk, n_init, n_local, n_cand, append=False):
    B, H = len(d["lengths"]), d["H"]
    max_len = max(d["lengths"])
    nb_max = -(-max_len // 64)
    out = torch.full((B, H, 128), float("nan"), dtype=d["q"].dtype, device=DEV)
    bs = torch.full((B, d["H_kv"], nb_max), float("nan"), device=DEV)
    idx = torch.full((B, d["H_kv"], topk), -7, dtype=torch.int32, device=DEV)
    p = nsa.decode_params(d["q"], d["k"], d["v"], d["kc"], d["cu_k"], d["cu_c"], max_len, out,
                          topk=topk, n_init=n_init, n_local=n_local, cis=d["cis"],
                          cis_pooled=d["cp"], append_window=append, block_scores=bs, indices=idx,
                          n_cand=n_cand)
    nsa.nsa_decode_step(p, device=DEV)
    torch.cuda.synchronize()
    return out, bs, idx


@pytest.mark.parametrize("dtype,lengths", [
    (BF16, [0, 40, 1000, 4097, 20000, 33000]),       # single-kernel path
    (F32, [40, 3000, 9000]),                         # separate selection kernel
    (BF16, [2049 * 64 + 17, 700]),                   # beyond the single-kernel bound
])
def test_decode_step_two_stage_uniform_attention(dtype, lengths):
    """Two-stage choice with zero queries: every attention block score is exactly
    tied on both sides, so stage 1 keeps the lowest free ids and stage 2 ranks
    them by the pooled CIS alone; index sets must be identical."""
    d = _decode_inputs(lengths, SEED + 16, dtype=dtype)
    d["q"].zero_()
    topk, n_init, n_local, n_cand = 32, 1, 8, 48
    log(f"decode step two-stage uniform attention {lengths} dtype={dtype}")
    out, bs, idx = _run_two_stage(d, topk, n_init, n_local, n_cand, append=True)
    q, k, v, cis = np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["cis"])
    res = oracle.decode_step(q, k, v, _cu_np(d["cu_k"]), topk=topk, n_init=n_init,
                             n_local=n_local, cis=cis, cis_select=True, n_cand=n_cand)
    idx_g = idx.cpu().numpy()
    assert (idx_g == res["indices"]).all(), "two-stage index sets differ"
    assert_close("two_stage_uniform.block_scores", np64(bs), res["block_scores"][:, :, :bs.shape[2]],
                 atol=1e-9, rtol=1e-4)
    atol = 1e-4 if dtype == F32 else 2e-2
    assert_close("two_stage_uniform.out", np64(out), res["out"], atol=atol)


@pytest.mark.parametrize("n_cand", [16, 64, 100, 5000])
def test_decode_step_two_stage(n_cand):
    """Two-stage choice on N(0,1) queries through the single-kernel path: the
    sets agree unless one of the oracle's stage boundaries is inside the band;
    outputs are compared where they agree.  n_cand 16 keeps fewer than the free
    places; 5000 makes every free block a candidate."""
    lengths = [3000, 9000, 20000, 31000]
    d = _decode_inputs(lengths, SEED + 17)
    topk, n_init, n_local = 64, 1, 16
    log(f"decode step two-stage n_cand={n_cand}")
    out, bs, idx = _run_two_stage(d, topk, n_init, n_local, n_cand)
    q, k, v, cis = np64(d["q"]), np64(d["k"]), np64(d["v"]), np64(d["cis"])
    res = oracle.decode_step(q, k, v, _cu_np(d["cu_k"]), topk=topk, n_init=n_init,
                             n_local=n_local, cis=cis, cis_select=True, n_cand=n_cand)
    assert_close("two_stage.block_scores", np64(bs), res["block_scores"][:, :, :bs.shape[2]],
                 atol=1e-9, rtol=1e-4)
    idx_g, out_g = idx.cpu().numpy(), np64(out)
    exact = 0
    for b, L in enumerate(lengths):
        nb = -(-L // 64)
        for g in range(2):
            ok = check_two_stage_sets(f"two_stage[{b},{g}]", idx_g[b, g], res["indices"][b, g],
                                      res["block_scores"][b, g], res["cis_block_scores"][b, g],
                                      L - 1, nb, topk, n_init, n_local, n_cand)
            if ok:
                exact += 1
                assert_close(f"two_stage.out[{b},{g}]", out_g[b, g * 8:(g + 1) * 8],
                             res["out"][b, g * 8:(g + 1) * 8], atol=2e-2)
    report(f"[two_stage n_cand={n_cand}] identical index sets for {exact}/{2 * len(lengths)}")
    assert exact >= 1


def test_decode_step_large_batch():
    """Twenty sequences with two KV heads: 40 (sequence, KV head) units already
    fill 256 workgroups at 8 selected blocks per workgroup, so each split of the
    single-kernel decode attends to 8 blocks, not the 4 of smaller batches."""
    lengths = gen.uniform_ints(SEED + 18, 1, 20, 1000, 9000)
    d = _decode_inputs(lengths, SEED + 18)
    log(f"decode step large batch {lengths}")
    out, bs, idx = _run_decode_step(d, 64, 1, 16, True, False, append=True)
    _check_decode("large_batch", d, out, bs, idx, 64, 1, 16, True, False, atol=2e-2)


def test_decode_step_grids_not_multiple_of_eight():
    """Three sequences, one KV head, top-20: 60 select-and-attend workgroups (one
    block each) and 27 logits workgroups, so the XCD-grouped order of both grids
    has a ragged last round; a workgroup the mapping skipped or repeated would
    leave a partial state or a chunk of window logits unwritten."""
    lengths = [9000, 700, 5000]
    d = _decode_inputs(lengths, SEED + 19, H=8, H_kv=1)
    log(f"decode step ragged grids {lengths}")
    out, bs, idx = _run_decode_step(d, 20, 1, 4, True, False)
    _check_decode("ragged_grids", d, out, bs, idx, 20, 1, 4, True, False, atol=2e-2)


@pytest.mark.parametrize("H,H_kv", [(32, 2), (8, 2), (4, 4)])
def test_decode_step_group_sizes(H, H_kv):
    """GQA groups of 16, 4 and 1 query heads through the single-kernel decode path."""
    d = _decode_inputs([3000, 7000, 12345], SEED + 13, H=H, H_kv=H_kv)
    log(f"decode step H={H} H_kv={H_kv}")
    out, bs, idx = _run_decode_step(d, 64, 1, 16, True, False)
    _check_decode(f"groups{H}_{H_kv}", d, out, bs, idx, 64, 1, 16, True, False, atol=2e-2)


def test_decode_step_planted_blocks_select_exactly():
    """Keys of blocks 5, 9, 17 and 30 equal half the sum of their group's query
    heads (logits ~ 5.7 against ~ 0 elsewhere), so their windows, and at a lower
    level the half-overlapping windows of the neighbouring blocks, dominate the
    compressed attention by margins far above the 1e-3 tie band: the index sets
    must be identical."""
    lengths = [4096, 3000]
    d = _decode_inputs(lengths, SEED + 10)
    k = d["k"].clone()
    cu_np = _cu_np(d["cu_k"])
    for b in range(len(lengths)):
        for g in range(2):
            for blk in (5, 9, 17, 30):
                s = cu_np[b] + 64 * blk
                k[s:s + 64, g] = (0.5 * d["q"][b, g * 8:(g + 1) * 8].float().sum(0)).to(k.dtype)
    d["k"] = k
    nsa.nsa_compress_k(k, d["kc"], d["cu_k"], d["cu_c"], max(d["nc"]))
    topk = 3 + 12  # init + 2 local + 4 planted + 8 half-overlapping neighbours
    out, bs, idx = _run_decode_step(d, topk, 1, 2, False, False)
    q, kk, v = np64(d["q"]), np64(k), np64(d["v"])
    res = oracle.decode_step(q, kk, v, cu_np, topk=topk, n_init=1, n_local=2)
    got = idx.cpu().numpy()
    for b in range(len(lengths)):
        for g in range(2):
            assert got[b, g].tolist() == res["indices"][b, g].tolist(), (b, g)
            assert {5, 9, 17, 30} <= set(got[b, g].tolist())
    assert_close("planted.out", np64(out), res["out"], atol=2e-2)


def test_decode_step_append_refreshes_last_window():
    d = _decode_inputs([1000, 2047, 4096], SEED + 11)
    cu_c = _cu_np(d["cu_c"])
    last = torch.tensor(cu_c[1:] - 1, device=DEV)
    good_kc = d["kc"][last].clone()
    good_cp = d["cp"][last].clone()
    d["kc"][last] = 0.0
    d["cp"][last] = 0.0
    log("decode step with window refresh")
    out, bs, idx = _run_decode_step(d, 16, 1, 2, True, False, append=True)
    assert torch.equal(d["kc"][last], good_kc)
    assert torch.equal(d["cp"][last], good_cp)
    _check_decode("append", d, out, bs, idx, 16, 1, 2, True, False, atol=2e-2)


# ----------------------------------------------------------------------------- full sizes

def _workload_decode_inputs(w, kc_dtype):
    q = W.decode_query(w, DEV)
    k, v = W.keys_values(w, DEV)
    cis = W.cis_scores(w, DEV)
    nc = [oracle.n_windows(L, 32, 16) for L in w.lengths]
    cu_k, cu_c = cu(w.lengths), cu(nc)
    kc = torch.zeros((sum(nc), w.kv_heads, 128), dtype=kc_dtype, device=DEV)
    cp = torch.zeros((sum(nc), w.kv_heads), dtype=F32, device=DEV)
    nsa.nsa_compress_k(k, kc, cu_k, cu_c, max(nc))
    nsa.nsa_cis_mean_pool_varlen(cis, cp, cu_k, cu_c, max(nc))
    return dict(q=q, k=k, v=v, cis=cis, kc=kc, cp=cp, cu_k=cu_k, cu_c=cu_c, nc=nc,
                lengths=list(w.lengths), H=w.heads, H_kv=w.kv_heads)


@pytest.mark.parametrize("kc_dtype", [F32, BF16])
def test_decode_step_nosa1b_full_size(kc_dtype):
    """The batched decode workload at full size (8 sequences of 8K-32K tokens, CIS
    fused into the block scores, top-64 with 1 init and 16 local blocks), through
    the same single-kernel select-and-attend path the throughput run times; every
    (sequence, kv head) is checked."""
    w = W.nosa1b_decode()
    d = _workload_decode_inputs(w, kc_dtype)
    log(f"decode step full size {w.name} kc={kc_dtype}")
    out, bs, idx = _run_decode_step(d, w.topk, w.n_init, w.n_local, True, False, append=True)
    _check_decode("nosa1b_full", d, out, bs, idx, w.topk, w.n_init, w.n_local, True, False,
                  atol=2e-2)


def test_decode_step_cis_values_full_size():
    """The long-context CIS-valued decode at full size: 4 sequences of 131072 tokens
    (2048 blocks each, the single-kernel path's largest variant)."""
    w = W.cis_decode()
    d = _workload_decode_inputs(w, F32)
    log(f"decode step full size {w.name}")
    out, bs, idx = _run_decode_step(d, w.topk, w.n_init, w.n_local, True, True, append=True)
    _check_decode("cis_full", d, out, bs, idx, w.topk, w.n_init, w.n_local, True, True,
                  atol=2e-2)


@pytest.mark.parametrize("path", ["blocks", "rows"])
def test_selected_attn_prefill_full_size_sampled_rows(path):
    """Given-index selected attention at full size (8 x 16384 rows), sampled rows,
    on the key-block path (the launch the benchmark times) and the row path."""
    w = W.selected_prefill()
    q = W.prefill_query(w, DEV)
    k, v = W.keys_values(w, DEV)
    idx = W.given_block_indices(w, DEV)
    cu_k = cu(w.lengths)
    out = torch.full_like(q, float("nan"))
    log(f"prefill selected attn full size {w.name} path={path}")
    nsa.nsa_selected_attn_fwd(q, k, v, idx, cu_k, max(w.lengths), out, cu_seqlens_q=cu_k,
                              workspace=_path_ws(path))
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    cu_np = _cu_np(cu_k)
    picks = [(0, 0), (0, 63), (0, 64), (1, 1000), (3, 8191), (5, 16320), (7, 16383)]
    picks += [(b, int(t)) for b in range(8) for t in np.linspace(100, 16380, 5).round()]
    rows = [(int(cu_np[b]) + t, t) for b, t in picks]
    ref = np.zeros((len(rows), w.heads, 128))
    got = np.zeros_like(ref)
    idxn = idx.cpu().numpy()
    for i, (r, t) in enumerate(rows):
        b = int(np.searchsorted(cu_np, r, side="right") - 1)
        s0, L = cu_np[b], cu_np[b + 1] - cu_np[b]
        ref[i] = oracle.selected_attention_row(np64(q[r]), np64(k[s0:s0 + L]), np64(v[s0:s0 + L]),
                                               idxn[r], t, 64, 1 / math.sqrt(128))
        got[i] = np64(out[r])
    assert_close("prefill_selected_full", got, ref, atol=2e-2)
