"""Plain float64 CPU oracle of the native-sparse-attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only the
tests, the smoke check and the benchmark's CPU-baseline leg may call it.  It
shares no code, table or helper with the HIP path.

Every function is the plain definition of one step, written out with numpy in
float64, one sequence / row / head at a time, with no blocking or fusion.
Inputs are the exact tensors the GPU receives (bf16- or fp32-rounded), widened
to float64.  Sources ("the pages") and the section each step follows:

* NOSA-1B source analysis part 3 (the Triton CIS pooling kernel): sections on
  the 3-D grid, the block load and sum, the variable-length mask and valid
  count, the avg_pool1d consistency check, and "beyond the kernel" (the
  32/16 windows, the max-pooled block scores fused with the pooled CIS, init and
  local blocks kept, -inf elsewhere, top-k, indices sorted).
* NOSA-1B core components: component 1 (Key compressor: mean of 32-token
  windows, stride 16; block_size 64, window_size 1024), component 2 (CIS
  pooling with the same windows), component 3 (top-k 64 blocks), and the
  decode-stage section (values scaled by CIS, sparse attention over the
  selected blocks, a second attention with all-ones values as normaliser).
* DeepSeek NSA with Triton, section 1.1: three branches (compressed, selected,
  sliding window of the last 512 tokens) summed with gates; selection reuses the
  compressed-attention scores.
* TileLang NSA, section 2 (native sparse attention): per query token t the
  block list BlockIndices[b, t, h, :], block start i*64, a block is used only
  when 0 <= start <= t; KV heads shared by a group of query heads.

Readings of points the pages leave open (each also listed in the design notes):
R1 full windows only by default (avg_pool1d, no padding, floor mode); a caller
   may ask for more windows, each the mean over its valid tokens, 0 if none.
R2 a window is visible to query position t when its last token is <= t.
R3 compressed-attention probabilities are summed over the query heads of a
   GQA group.
R4 window -> block pooling is the max over all windows that overlap the block
   (for 32/16/64: windows 4b-1 .. 4b+3); no overlapping window gives 0.
R5 CIS fusion is additive: S = S_qk + w * max over the same windows of the
   pooled CIS.
R6 selection: blocks with start <= t are eligible; forced = first n_init and
   last n_local eligible blocks; k counts the forced blocks; the rest are the
   best eligible blocks by score, ties to the lower index; output ascending,
   -1 padded.
R7 token-level causality inside the diagonal block (keys j <= t).
R8 CIS mode: o = sum p*cis*v / sum p*cis (the ones-value pass carries the same
   CIS scaling).
R9 sliding window: keys max(0, t-W+1) .. t (W keys including the query's own).
R16 backward of the selected attention (no CIS): the exact gradient of the
   forward above with respect to q, k and v for a given upstream gradient of the
   output; the pages describe the method as trainable end to end (DeepSeek NSA
   with Triton, introduction and section 2.3, the kernels wrapped as a
   trainable module) but print no backward, so the gradient is the plain one.
   Keys reached through no row get zero gradient.
R17 backward of the compressed and sliding-window branches: the exact gradient
   of each branch's output for a given upstream gradient; the compressed
   branch's key and value gradients reach K and V through the transpose of the
   window mean (each window's gradient spread over its valid tokens divided by
   their count).  The selection is a discrete choice and passes no gradient; the
   gates receive dO . o_branch.
R5b two-stage selection (optional): the n_cand best free blocks by the
   compressed-attention block score are the candidates; the k - |forced| best
   candidates by the pooled-CIS block score are chosen (ties to the lower index
   in both stages).  The pages leave n_cand open; callers pass it.
"""
from __future__ import annotations

import math

import numpy as np

# ----------------------------------------------------------------------------- geometry


def n_windows(length: int, kernel: int, stride: int, tail: bool = False) -> int:
    """Number of compressed windows of a sequence of ``length`` tokens.

    Full windows (R1): floor((L - kernel) / stride) + 1, 0 when L < kernel.
    ``tail=True``: enough windows to cover every token (the masked variant of the
    pooling kernel), i.e. the smallest n with stride*(n-1) + kernel >= L."""
    if length <= 0:
        return 0
    if not tail:
        return 0 if length < kernel else (length - kernel) // stride + 1
    if length <= kernel:
        return 1
    return -(-(length - kernel) // stride) + 1


def n_blocks(length: int, block: int) -> int:
    return -(-length // block)


def cu_from_lengths(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int64)


# ----------------------------------------------------------------------------- pooling


def mean_pool_varlen(x, cu_seqlens, cu_seqlens_c, kernel: int, stride: int) -> np.ndarray:
    """Sliding-window mean over packed variable-length sequences.

    Window c of sequence b covers the tokens stride*c .. stride*c + kernel - 1 of
    that sequence that exist; the sum is divided by the number of such tokens
    (the valid count), and a window with none is 0.  ``x`` is [N, ...]; the
    number of windows of sequence b is cu_seqlens_c[b+1] - cu_seqlens_c[b].
    (NOSA part 3: grid/mask/valid-count sections; NOSA core components 1, 2.)"""
    x = np.asarray(x, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    cuc = np.asarray(cu_seqlens_c, dtype=np.int64)
    out = np.zeros((int(cuc[-1]),) + x.shape[1:], dtype=np.float64)
    for b in range(len(cu) - 1):
        start, length = int(cu[b]), int(cu[b + 1] - cu[b])
        for c in range(int(cuc[b + 1] - cuc[b])):
            lo = stride * c
            hi = min(lo + kernel, length)
            if hi > lo:
                out[cuc[b] + c] = x[start + lo:start + hi].sum(axis=0) / (hi - lo)
    return out


# ----------------------------------------------------------------------------- scoring


def window_visible(c: int, t: int, kernel: int, stride: int) -> bool:
    """R2: window c is visible to query position t when it lies wholly in the past."""
    return stride * c + kernel - 1 <= t


def softmax(s: np.ndarray) -> np.ndarray:
    s = np.asarray(s, dtype=np.float64)
    if s.size == 0:
        return s
    e = np.exp(s - s.max())
    return e / e.sum()


def group_window_probs(q, kc_seq, t: int, kernel: int, stride: int, scale: float) -> np.ndarray:
    """Compressed-attention probabilities summed per GQA group (R3).

    q: [H, D] query of position t; kc_seq: [n_c, H_kv, D] compressed keys of the
    query's sequence.  For head h (group h // G) the logits q_h . Kc[c] * scale
    over visible windows go through a softmax; invisible windows get 0.
    Returns [H_kv, n_c].  (NOSA core components 3: stage-1 attention of the query
    against the compressed keys; NSA section 1.1: selection reuses these.)"""
    q = np.asarray(q, dtype=np.float64)
    kc_seq = np.asarray(kc_seq, dtype=np.float64)
    H = q.shape[0]
    n_c, H_kv = kc_seq.shape[0], kc_seq.shape[1]
    G = H // H_kv
    vis = [c for c in range(n_c) if window_visible(c, t, kernel, stride)]
    pg = np.zeros((H_kv, n_c), dtype=np.float64)
    if not vis:
        return pg
    for h in range(H):
        g = h // G
        logits = kc_seq[vis, g] @ q[h] * scale
        pg[g, vis] += softmax(logits)
    return pg


def window_block_overlap(c: int, b: int, kernel: int, stride: int, block: int) -> bool:
    """Window c (tokens [stride*c, stride*c+kernel)) overlaps block b
    (tokens [block*b, block*(b+1)))."""
    return stride * c < block * (b + 1) and stride * c + kernel > block * b


def block_max(wscore, n_blk: int, kernel: int, stride: int, block: int) -> np.ndarray:
    """R4: per block, the max of a per-window score over the windows that
    overlap the block; 0 when no window overlaps.  wscore: [..., n_c].
    (NOSA part 3, "beyond the kernel": max-pooled block scores.)"""
    wscore = np.asarray(wscore, dtype=np.float64)
    n_c = wscore.shape[-1]
    out = np.zeros(wscore.shape[:-1] + (n_blk,), dtype=np.float64)
    for b in range(n_blk):
        # candidates bracket the overlap range; the predicate decides
        c_lo = max(0, (block * b - kernel) // stride)
        c_hi = min(n_c - 1, (block * (b + 1)) // stride)
        cs = [c for c in range(c_lo, c_hi + 1) if window_block_overlap(c, b, kernel, stride, block)]
        if cs:
            out[..., b] = wscore[..., cs].max(axis=-1)
    return out


# ----------------------------------------------------------------------------- selection


def select_blocks(score, t: int, n_blk: int, k: int, n_init: int, n_local: int,
                  block: int) -> np.ndarray:
    """R6: top-k block selection for one (query position, KV head).

    Eligible: blocks b < n_blk with block*b <= t.  Forced: the first n_init and
    the last n_local eligible blocks (init and local blocks, NOSA part 3 "beyond
    the kernel"; NOSA core components 1 and 3).  The remaining k - |forced|
    places go to the highest-scoring other eligible blocks, ties to the lower
    index.  Returns k int32 ids, ascending, -1 padded."""
    score = np.asarray(score, dtype=np.float64)
    n_elig = min(n_blk, t // block + 1) if t >= 0 else 0
    forced = set(range(min(n_init, n_elig)))
    forced |= set(range(max(0, n_elig - n_local), n_elig))
    rest = [b for b in range(n_elig) if b not in forced]
    rest.sort(key=lambda b: (-score[b], b))
    assert len(forced) <= k, "forced blocks must fit in k"
    chosen = sorted(forced | set(rest[:k - len(forced)]))
    out = np.full(k, -1, dtype=np.int32)
    out[:len(chosen)] = chosen
    return out


def select_blocks_two_stage(score_qk, score_cis, t: int, n_blk: int, k: int, n_init: int,
                            n_local: int, block: int, n_cand: int) -> np.ndarray:
    """R5b: two-stage top-k for one (query position, KV head) (NOSA-1B core
    components, component 3: a coarse pick of candidate blocks by the
    compressed-attention block score, then a re-rank by the block score of the
    pooled CIS down to the top-k).

    Eligible and forced blocks as in select_blocks.  Stage 1: the n_cand best
    other eligible blocks by score_qk are the candidates.  Stage 2: the
    k - |forced| best candidates by score_cis are chosen.  Ties go to the lower
    index in both stages.  Returns k int32 ids, ascending, -1 padded."""
    score_qk = np.asarray(score_qk, dtype=np.float64)
    score_cis = np.asarray(score_cis, dtype=np.float64)
    n_elig = min(n_blk, t // block + 1) if t >= 0 else 0
    forced = set(range(min(n_init, n_elig)))
    forced |= set(range(max(0, n_elig - n_local), n_elig))
    assert len(forced) <= k, "forced blocks must fit in k"
    rest = [b for b in range(n_elig) if b not in forced]
    rest.sort(key=lambda b: (-score_qk[b], b))
    cand = rest[:max(0, n_cand)]
    cand.sort(key=lambda b: (-score_cis[b], b))
    chosen = sorted(forced | set(cand[:k - len(forced)]))
    out = np.full(k, -1, dtype=np.int32)
    out[:len(chosen)] = chosen
    return out


# ----------------------------------------------------------------------------- attention


def selected_keys(idx_row, t: int, length: int, block: int) -> list:
    """Token positions attended by query position t through one index list (R7):
    every token j of every listed block with 0 <= id, block*id <= t, j <= t, j < L.
    (TileLang NSA section 2: blocks with a start beyond t or a negative id are
    skipped.)  Ids must be unique."""
    ids = [int(i) for i in idx_row if int(i) >= 0 and block * int(i) <= t]
    assert len(ids) == len(set(ids)), "block ids of one row must be unique"
    keys = []
    for i in sorted(ids):
        keys.extend(j for j in range(block * i, block * (i + 1)) if j <= t and j < length)
    return keys


def attend(q_h, k_rows, v_rows, scale: float, weight=None) -> np.ndarray:
    """softmax(q.k * scale) . v over the given key rows; with ``weight`` (R8) the
    softmax weights are multiplied by it and renormalised.  Empty -> zeros."""
    q_h = np.asarray(q_h, dtype=np.float64)
    k_rows = np.asarray(k_rows, dtype=np.float64)
    v_rows = np.asarray(v_rows, dtype=np.float64)
    if k_rows.shape[0] == 0:
        return np.zeros(q_h.shape[-1])
    p = softmax(k_rows @ q_h * scale)
    if weight is not None:
        p = p * np.asarray(weight, dtype=np.float64)
        den = p.sum()
        return (p @ v_rows) / den if den > 0 else np.zeros(v_rows.shape[-1])
    return p @ v_rows


def selected_attention_row(q, k_seq, v_seq, idx, t: int, block: int, scale: float,
                           cis_seq=None) -> np.ndarray:
    """Attention of the H query heads of position t over the selected blocks.

    q: [H, D]; k_seq, v_seq: [L, H_kv, D]; idx: [H_kv, k] block ids; cis_seq:
    optional [L, H_kv] importance scores (CIS mode, R8).  Returns [H, D].
    (NOSA core components, decode stage; TileLang NSA section 2.)"""
    q = np.asarray(q, dtype=np.float64)
    H, D = q.shape
    L, H_kv = k_seq.shape[0], k_seq.shape[1]
    G = H // H_kv
    out = np.zeros((H, D), dtype=np.float64)
    for h in range(H):
        g = h // G
        J = selected_keys(idx[g], t, L, block)
        w = None if cis_seq is None else np.asarray(cis_seq, dtype=np.float64)[J, g]
        out[h] = attend(q[h], np.asarray(k_seq)[J, g], np.asarray(v_seq)[J, g], scale, w)
    return out


def selected_attention_row_grad(q, k_seq, v_seq, idx, t: int, block: int, scale: float,
                                d_out, dk, dv) -> np.ndarray:
    """Gradient of selected_attention_row (no CIS, R16) for query position t.

    d_out: [H, D] upstream gradient of the row's output.  Adds the row's
    contributions to dk, dv ([L, H_kv, D] float64, in place) and returns dq
    [H, D].  Per head, over the selected keys J: p = softmax(scale * K_J q),
    o = p V_J; dV_J += p d_out^T; dp = V_J d_out; ds = p * (dp - d_out . o);
    dq = scale * ds K_J; dK_J += scale * ds q^T."""
    q = np.asarray(q, dtype=np.float64)
    d_out = np.asarray(d_out, dtype=np.float64)
    k_seq = np.asarray(k_seq, dtype=np.float64)
    v_seq = np.asarray(v_seq, dtype=np.float64)
    H, D = q.shape
    L, H_kv = k_seq.shape[0], k_seq.shape[1]
    G = H // H_kv
    dq = np.zeros((H, D))
    for h in range(H):
        g = h // G
        J = selected_keys(idx[g], t, L, block)
        if not J:
            continue
        K, V = k_seq[J, g], v_seq[J, g]
        p = softmax(K @ q[h] * scale)
        o = p @ V
        ds = p * (V @ d_out[h] - d_out[h] @ o)
        dq[h] = scale * (ds @ K)
        dk[J, g] += scale * np.outer(ds, q[h])
        dv[J, g] += np.outer(p, d_out[h])
    return dq


def selected_attention_bwd(q, k, v, idx, d_out, cu_q, cu_k, block: int, scale: float):
    """Gradients of the selected attention over packed prefill rows (R16).

    q, d_out: [rows, H, D]; k, v: [N_k, H_kv, D]; idx: [rows, H_kv, k];
    cu_q, cu_k: sequence offsets.  Row r of sequence b sits at position
    t = (r - cu_q[b]) + (L_b - Lq_b).  Returns dq [rows, H, D], dk and dv
    [N_k, H_kv, D]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        shift = (k1 - k0) - (q1 - q0)
        for r in range(q0, q1):
            dq[r] = selected_attention_row_grad(q[r], k[k0:k1], v[k0:k1], idx[r], r - q0 + shift,
                                                block, scale, d_out[r], dk[k0:k1], dv[k0:k1])
    return dq, dk, dv


def _attend_grad(q_h, K, V, scale: float, d_out_h):
    """Gradient of softmax(scale K q) V with respect to q, K and V for the upstream
    gradient d_out_h: returns (dq, dK, dV); empty key sets give zeros."""
    if K.shape[0] == 0:
        return np.zeros_like(q_h), np.zeros_like(K), np.zeros_like(V)
    p = softmax(K @ q_h * scale)
    o = p @ V
    ds = p * (V @ d_out_h - d_out_h @ o)
    return scale * (ds @ K), scale * np.outer(ds, q_h), np.outer(p, d_out_h)


def compressed_attention_row_grad(q, kc_seq, vc_seq, t: int, kernel: int, stride: int,
                                  scale: float, d_out, dkc, dvc) -> np.ndarray:
    """Gradient of compressed_attention_row (R17) for query position t: adds the
    row's contributions to dkc, dvc ([n_c, H_kv, D] float64, in place) and
    returns dq [H, D].  The keys are the windows visible to t (R2)."""
    q = np.asarray(q, dtype=np.float64)
    d_out = np.asarray(d_out, dtype=np.float64)
    kc_seq = np.asarray(kc_seq, dtype=np.float64)
    vc_seq = np.asarray(vc_seq, dtype=np.float64)
    H = q.shape[0]
    n_c, H_kv = kc_seq.shape[0], kc_seq.shape[1]
    G = H // H_kv
    vis = [c for c in range(n_c) if window_visible(c, t, kernel, stride)]
    dq = np.zeros(q.shape)
    for h in range(H):
        g = h // G
        dq[h], dk_, dv_ = _attend_grad(q[h], kc_seq[vis, g], vc_seq[vis, g], scale, d_out[h])
        dkc[vis, g] += dk_
        dvc[vis, g] += dv_
    return dq


def window_attention_row_grad(q, k_seq, v_seq, t: int, window: int, scale: float, d_out, dk,
                              dv) -> np.ndarray:
    """Gradient of window_attention_row (R9, R17) for query position t: keys
    max(0, t-window+1) .. t; adds to dk, dv in place and returns dq [H, D]."""
    q = np.asarray(q, dtype=np.float64)
    d_out = np.asarray(d_out, dtype=np.float64)
    k_seq = np.asarray(k_seq, dtype=np.float64)
    v_seq = np.asarray(v_seq, dtype=np.float64)
    H = q.shape[0]
    G = H // k_seq.shape[1]
    J = list(range(max(0, t - window + 1), t + 1))
    dq = np.zeros(q.shape)
    for h in range(H):
        g = h // G
        dq[h], dk_, dv_ = _attend_grad(q[h], k_seq[J, g], v_seq[J, g], scale, d_out[h])
        dk[J, g] += dk_
        dv[J, g] += dv_
    return dq


def mean_pool_varlen_bwd(dxc, cu_seqlens, cu_seqlens_c, kernel: int, stride: int,
                         n_tokens: int) -> np.ndarray:
    """Transpose of mean_pool_varlen (R17): window c's gradient, divided by its
    count of valid tokens, added to each of those tokens.  dxc [N_c, ...] ->
    [n_tokens, ...]."""
    dxc = np.asarray(dxc, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    cuc = np.asarray(cu_seqlens_c, dtype=np.int64)
    dx = np.zeros((n_tokens,) + dxc.shape[1:])
    for b in range(len(cu) - 1):
        start, length = int(cu[b]), int(cu[b + 1] - cu[b])
        for c in range(int(cuc[b + 1] - cuc[b])):
            lo = stride * c
            hi = min(lo + kernel, length)
            if hi > lo:
                dx[start + lo:start + hi] += dxc[cuc[b] + c] / (hi - lo)
    return dx


def blockmask_attention_row(q, k_seq, v_seq, mask_rows, t: int, block: int, scale: float,
                            causal: bool = False) -> np.ndarray:
    """Block-mask attention of query position t of one sequence (TileLang NSA,
    section 1: the attention matrix in block x block tiles, a block mask marking
    the computed ones, the lower triangle only when causal).

    q: [H, D] (the query's heads); k_seq, v_seq: [L, H, D] (multi-head, one K/V
    head per query head); mask_rows: [H, nb, nb].  Head h attends to the keys j
    with mask_rows[h, t // block, j // block] != 0 (and j <= t when causal);
    a query with no key gets 0."""
    q = np.asarray(q, dtype=np.float64)
    k_seq = np.asarray(k_seq, dtype=np.float64)
    v_seq = np.asarray(v_seq, dtype=np.float64)
    H, D = q.shape
    L = k_seq.shape[0]
    j = np.arange(L)
    out = np.zeros((H, D))
    for h in range(H):
        on = np.asarray(mask_rows[h, t // block])[j // block] != 0
        if causal:
            on &= j <= t
        out[h] = attend(q[h], k_seq[on, h], v_seq[on, h], scale)
    return out


def window_attention_row(q, k_seq, v_seq, t: int, window: int, scale: float) -> np.ndarray:
    """Sliding-window branch (R9): keys max(0, t-window+1) .. t.  (NSA section 1.1.)"""
    q = np.asarray(q, dtype=np.float64)
    H, D = q.shape
    H_kv = k_seq.shape[1]
    G = H // H_kv
    J = list(range(max(0, t - window + 1), t + 1))
    out = np.zeros((H, D), dtype=np.float64)
    for h in range(H):
        out[h] = attend(q[h], np.asarray(k_seq)[J, h // G], np.asarray(v_seq)[J, h // G], scale)
    return out


def compressed_attention_row(q, kc_seq, vc_seq, t: int, kernel: int, stride: int,
                             scale: float) -> np.ndarray:
    """Compressed branch: softmax over the visible windows of q.Kc * scale, times Vc;
    zeros when no window is visible.  (NSA section 1.1, compressed attention with a
    plain mean as the compression.)"""
    q = np.asarray(q, dtype=np.float64)
    H, D = q.shape
    n_c, H_kv = kc_seq.shape[0], kc_seq.shape[1]
    G = H // H_kv
    vis = [c for c in range(n_c) if window_visible(c, t, kernel, stride)]
    out = np.zeros((H, D), dtype=np.float64)
    for h in range(H):
        out[h] = attend(q[h], np.asarray(kc_seq)[vis, h // G], np.asarray(vc_seq)[vis, h // G], scale)
    return out


# ----------------------------------------------------------------------------- composed paths


def decode_block_scores(q, kc_seq, t: int, n_blk: int, kernel: int, stride: int, block: int,
                        scale: float, cis_pooled_seq=None, cis_weight: float = 1.0) -> np.ndarray:
    """Fused block scores of one decode query (R3-R5): [H_kv, n_blk]."""
    pg = group_window_probs(q, kc_seq, t, kernel, stride, scale)
    s = block_max(pg, n_blk, kernel, stride, block)
    if cis_pooled_seq is not None and cis_weight != 0.0:
        cp = np.asarray(cis_pooled_seq, dtype=np.float64).T          # [H_kv, n_c]
        s = s + cis_weight * block_max(cp, n_blk, kernel, stride, block)
    return s


def decode_step(q, k, v, cu_seqlens, *, kernel=32, stride=16, block=64, topk=64, n_init=1,
                n_local=16, scale=None, cis=None, cis_select=False, cis_values=False,
                cis_weight=1.0, seqs=None, n_cand=0):
    """One decode step over a packed batch: the newest token (t = L_b - 1) of each
    sequence attends to its selected blocks.

    q: [B, H, D]; k, v: [N, H_kv, D]; cis: [N, H_kv] or None.  Returns a dict with
    kc, cis_pooled (all full windows), block_scores [B, H_kv, n_blk_max] (0 beyond a
    sequence's blocks), indices [B, H_kv, topk] and out [B, H, D].  ``seqs`` limits
    the work to some sequences (others stay zero / -1).  With n_cand > 0 (and
    cis_select) the selection is the two-stage one (R5b): block_scores then holds
    the compressed-attention scores alone and cis_block_scores the pooled-CIS
    block scores."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    B, H, D = q.shape
    H_kv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    lengths = [int(cu[b + 1] - cu[b]) for b in range(B)]
    ncs = [n_windows(L, kernel, stride) for L in lengths]
    cuc = cu_from_lengths(ncs)
    seqs = list(range(B)) if seqs is None else list(seqs)
    nb_max = max(n_blocks(L, block) for L in lengths)
    kc = np.zeros((int(cuc[-1]), H_kv, D))
    cp = np.zeros((int(cuc[-1]), H_kv)) if cis is not None else None
    scores = np.zeros((B, H_kv, nb_max))
    cis_scores = np.zeros((B, H_kv, nb_max))
    two_stage = n_cand > 0
    if two_stage:
        assert cis is not None and cis_select, "the two-stage selection needs the pooled CIS"
    idx = np.full((B, H_kv, topk), -1, dtype=np.int32)
    out = np.zeros((B, H, D))
    for b in seqs:
        s0, L = int(cu[b]), lengths[b]
        one = np.array([0, L])
        onec = np.array([0, ncs[b]])
        kc_b = mean_pool_varlen(k[s0:s0 + L], one, onec, kernel, stride)
        kc[cuc[b]:cuc[b + 1]] = kc_b
        cp_b = None
        if cis is not None:
            cp_b = mean_pool_varlen(np.asarray(cis, dtype=np.float64)[s0:s0 + L], one, onec,
                                    kernel, stride)
            cp[cuc[b]:cuc[b + 1]] = cp_b
        t = L - 1
        nb = n_blocks(L, block)
        if two_stage:
            sc = decode_block_scores(q[b], kc_b, t, nb, kernel, stride, block, scale)
            scc = block_max(np.asarray(cp_b, dtype=np.float64).T, nb, kernel, stride, block)
            cis_scores[b, :, :nb] = scc
            for g in range(H_kv):
                idx[b, g] = select_blocks_two_stage(sc[g], scc[g], t, nb, topk, n_init, n_local,
                                                    block, n_cand)
        else:
            sc = decode_block_scores(q[b], kc_b, t, nb, kernel, stride, block, scale,
                                     cp_b if cis_select else None, cis_weight)
            for g in range(H_kv):
                idx[b, g] = select_blocks(sc[g], t, nb, topk, n_init, n_local, block)
        scores[b, :, :nb] = sc
        cis_seq = np.asarray(cis, dtype=np.float64)[s0:s0 + L] if cis_values else None
        out[b] = selected_attention_row(q[b], k[s0:s0 + L], v[s0:s0 + L], idx[b], t, block,
                                        scale, cis_seq)
    return dict(kc=kc, cis_pooled=cp, block_scores=scores, cis_block_scores=cis_scores,
                indices=idx, out=out, cu_seqlens_c=cuc, lengths=lengths)


def nsa_prefill_rows(q_seq, k_seq, v_seq, gates_seq, rows, *, kernel=32, stride=16, block=64,
                     topk=16, window=512, scale=None):
    """Three-branch NSA output for some query positions of one sequence.

    q_seq [L, H, D], k_seq/v_seq [L, H_kv, D], gates_seq [L, H, 3].  For each row t:
    compressed branch over mean-pooled K/V, selected branch over the top-k blocks
    scored from the compressed probabilities summed per group (no forced blocks),
    sliding window of ``window`` keys, combined as g0*o_cmp + g1*o_sel + g2*o_win
    (NSA section 1.1).  Returns dict of per-row arrays."""
    q_seq = np.asarray(q_seq, dtype=np.float64)
    k_seq = np.asarray(k_seq, dtype=np.float64)
    v_seq = np.asarray(v_seq, dtype=np.float64)
    L, H, D = q_seq.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    nc = n_windows(L, kernel, stride)
    one, onec = np.array([0, L]), np.array([0, nc])
    kc = mean_pool_varlen(k_seq, one, onec, kernel, stride)
    vc = mean_pool_varlen(v_seq, one, onec, kernel, stride)
    nb = n_blocks(L, block)
    res = {"out": [], "o_cmp": [], "o_sel": [], "o_win": [], "indices": [], "block_scores": []}
    for t in rows:
        o_cmp = compressed_attention_row(q_seq[t], kc, vc, t, kernel, stride, scale)
        pg = group_window_probs(q_seq[t], kc, t, kernel, stride, scale)
        sc = block_max(pg, nb, kernel, stride, block)
        idx = np.stack([select_blocks(sc[g], t, nb, topk, 0, 0, block) for g in range(sc.shape[0])])
        o_sel = selected_attention_row(q_seq[t], k_seq, v_seq, idx, t, block, scale)
        o_win = window_attention_row(q_seq[t], k_seq, v_seq, t, window, scale)
        g = np.asarray(gates_seq[t], dtype=np.float64)
        out = g[:, 0:1] * o_cmp + g[:, 1:2] * o_sel + g[:, 2:3] * o_win
        for key, val in (("out", out), ("o_cmp", o_cmp), ("o_sel", o_sel), ("o_win", o_win),
                         ("indices", idx), ("block_scores", sc)):
            res[key].append(val)
    return {key: np.stack(val) for key, val in res.items()}


def nsa_prefill_rows_grad(q_seq, k_seq, v_seq, gates_seq, d_out_seq, rows, *, kernel=32,
                          stride=16, block=64, topk=16, window=512, scale=None):
    """Gradient of the three-branch output of some query positions of one
    sequence (R17), for the upstream gradient d_out_seq [L, H, D] of those rows
    (other rows contribute nothing).  The block choice of each row is the
    forward's (nsa_prefill_rows) and passes no gradient.  Per branch b the
    output gradient is gate_b * dO; the gate gradient is dO . o_b.  Returns a
    dict: dq [len(rows), H, D], dk, dv [L, H_kv, D] and dgates [len(rows), H, 3],
    plus the forward's indices."""
    q_seq = np.asarray(q_seq, dtype=np.float64)
    k_seq = np.asarray(k_seq, dtype=np.float64)
    v_seq = np.asarray(v_seq, dtype=np.float64)
    d_out_seq = np.asarray(d_out_seq, dtype=np.float64)
    L, H, D = q_seq.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    fwd = nsa_prefill_rows(q_seq, k_seq, v_seq, gates_seq, rows, kernel=kernel, stride=stride,
                           block=block, topk=topk, window=window, scale=scale)
    nc = n_windows(L, kernel, stride)
    one, onec = np.array([0, L]), np.array([0, nc])
    kc = mean_pool_varlen(k_seq, one, onec, kernel, stride)
    vc = mean_pool_varlen(v_seq, one, onec, kernel, stride)
    dk = np.zeros(k_seq.shape)
    dv = np.zeros(v_seq.shape)
    dkc = np.zeros(kc.shape)
    dvc = np.zeros(vc.shape)
    dq = np.zeros((len(rows), H, D))
    dg = np.zeros((len(rows), H, 3))
    for i, t in enumerate(rows):
        g = np.asarray(gates_seq[t], dtype=np.float64)
        do = d_out_seq[t]
        for j, key in enumerate(("o_cmp", "o_sel", "o_win")):
            dg[i, :, j] = (do * fwd[key][i]).sum(axis=1)
        dq[i] += compressed_attention_row_grad(q_seq[t], kc, vc, t, kernel, stride, scale,
                                               g[:, 0:1] * do, dkc, dvc)
        dq[i] += selected_attention_row_grad(q_seq[t], k_seq, v_seq, fwd["indices"][i], t, block,
                                             scale, g[:, 1:2] * do, dk, dv)
        dq[i] += window_attention_row_grad(q_seq[t], k_seq, v_seq, t, window, scale,
                                           g[:, 2:3] * do, dk, dv)
    dk += mean_pool_varlen_bwd(dkc, one, onec, kernel, stride, L)
    dv += mean_pool_varlen_bwd(dvc, one, onec, kernel, stride, L)
    return {"dq": dq, "dk": dk, "dv": dv, "dgates": dg, "indices": fwd["indices"]}
