"""Pins of the oracle's selected-attention backward (R16).

Anchors independent of the gradient formulas: central finite differences of the
forward oracle (itself pinned against torch's attention), torch autograd of
dense causal attention in float64 on the CPU when every causal block is
selected (a library routine), and closed forms (a row whose only key is its
own position has dq = 0 and passes d_out straight to dv)."""
import numpy as np
import torch
import torch.nn.functional as F

import oracle


def _forward(q, k, v, idx, cu_q, cu_k, block, scale):
    out = np.zeros(q.shape)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        shift = (k1 - k0) - (q1 - q0)
        for r in range(q0, q1):
            out[r] = oracle.selected_attention_row(q[r], k[k0:k1], v[k0:k1], idx[r],
                                                   r - q0 + shift, block, scale)
    return out


def _random_case(rng, lengths_k, lengths_q, H, H_kv, D, block, k_sel):
    cu_k = oracle.cu_from_lengths(lengths_k)
    cu_q = oracle.cu_from_lengths(lengths_q)
    rows = int(cu_q[-1])
    q = rng.standard_normal((rows, H, D))
    k = rng.standard_normal((int(cu_k[-1]), H_kv, D))
    v = rng.standard_normal((int(cu_k[-1]), H_kv, D))
    idx = -np.ones((rows, H_kv, k_sel), dtype=np.int64)
    for b in range(len(lengths_k)):
        shift = lengths_k[b] - lengths_q[b]
        for r in range(int(cu_q[b]), int(cu_q[b + 1])):
            t = r - int(cu_q[b]) + shift
            n_elig = t // block + 1
            for g in range(H_kv):
                ids = rng.permutation(n_elig)[:k_sel]
                idx[r, g, :len(ids)] = np.sort(ids)
    return q, k, v, idx, cu_q, cu_k


def test_backward_matches_finite_differences():
    rng = np.random.default_rng(11)
    block, scale, H, H_kv, D = 8, 0.3, 4, 2, 6
    q, k, v, idx, cu_q, cu_k = _random_case(rng, [29, 20], [7, 20], H, H_kv, D, block, 2)
    d_out = rng.standard_normal(q.shape)
    dq, dk, dv = oracle.selected_attention_bwd(q, k, v, idx, d_out, cu_q, cu_k, block, scale)

    def loss(q_, k_, v_):
        return float((_forward(q_, k_, v_, idx, cu_q, cu_k, block, scale) * d_out).sum())

    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        flat = x.reshape(-1)
        picks = rng.choice(flat.size, size=min(flat.size, 60), replace=False)
        for i in picks:
            old = flat[i]
            flat[i] = old + eps
            lp = loss(q, k, v)
            flat[i] = old - eps
            lm = loss(q, k, v)
            flat[i] = old
            num = (lp - lm) / (2 * eps)
            assert abs(num - g.reshape(-1)[i]) < 1e-6 * max(1.0, abs(num)), (name, i, num,
                                                                           g.reshape(-1)[i])


def test_backward_all_blocks_equals_dense_autograd():
    """k covering every causal block: the selected attention is dense causal
    attention, so its gradient is torch autograd's of the dense form."""
    rng = np.random.default_rng(12)
    block, scale, H, H_kv, D, L = 16, 0.25, 4, 2, 8, 50
    n_blk = -(-L // block)
    cu = oracle.cu_from_lengths([L])
    q = rng.standard_normal((L, H, D))
    k = rng.standard_normal((L, H_kv, D))
    v = rng.standard_normal((L, H_kv, D))
    idx = np.tile(np.arange(n_blk), (L, H_kv, 1))
    d_out = rng.standard_normal((L, H, D))
    dq, dk, dv = oracle.selected_attention_bwd(q, k, v, idx, d_out, cu, cu, block, scale)

    G = H // H_kv
    qt = torch.tensor(q.transpose(1, 0, 2), requires_grad=True)            # [H, L, D]
    kt = torch.tensor(k.transpose(1, 0, 2), requires_grad=True)            # [H_kv, L, D]
    vt = torch.tensor(v.transpose(1, 0, 2), requires_grad=True)
    ke = kt.repeat_interleave(G, dim=0)
    ve = vt.repeat_interleave(G, dim=0)
    out = F.scaled_dot_product_attention(qt, ke, ve, is_causal=True, scale=scale)
    out.backward(torch.tensor(d_out.transpose(1, 0, 2)))
    np.testing.assert_allclose(dq, qt.grad.numpy().transpose(1, 0, 2), atol=1e-10)
    np.testing.assert_allclose(dk, kt.grad.numpy().transpose(1, 0, 2), atol=1e-10)
    np.testing.assert_allclose(dv, vt.grad.numpy().transpose(1, 0, 2), atol=1e-10)


def test_backward_single_key_and_unreached_keys():
    """Position 0 sees only key 0: softmax over one key has no gradient, so
    dq = 0 and dv[0] gets the sum of its group's d_out.  Keys in blocks no row
    lists get zero gradient."""
    rng = np.random.default_rng(13)
    block, scale, H, H_kv, D = 4, 0.5, 4, 2, 5
    q = rng.standard_normal((1, H, D))
    k = rng.standard_normal((12, H_kv, D))
    v = rng.standard_normal((12, H_kv, D))
    idx = np.array([[[0, -1], [0, -1]]])
    d_out = rng.standard_normal((1, H, D))
    cu_q, cu_k = np.array([0, 1]), np.array([0, 12])
    # a single query row of a 12-token sequence sits at t = 11; use a 1-token
    # sequence view instead so that t = 0
    dq, dk, dv = oracle.selected_attention_bwd(q, k[:1], v[:1], idx, d_out, cu_q,
                                               np.array([0, 1]), block, scale)
    assert np.all(dq == 0)
    assert np.allclose(dv[0, 0], d_out[0, 0] + d_out[0, 1])
    assert np.allclose(dv[0, 1], d_out[0, 2] + d_out[0, 3])
    assert np.allclose(dk, 0)
    # t = 11 with only block 1 listed: keys 0-3 and 8-11 get nothing
    dq, dk, dv = oracle.selected_attention_bwd(q, k, v, np.array([[[1, -1], [1, -1]]]), d_out,
                                               cu_q, cu_k, block, scale)
    assert np.all(dk[:4] == 0) and np.all(dk[8:] == 0) and np.all(dv[8:] == 0)
    assert np.abs(dv[4:8]).sum() > 0


# ----------------------------------------------------------------- compressed and window branches (R17)

def test_pool_bwd_is_the_adjoint_of_the_pooling():
    """<pool(x), y> = <x, pool_bwd(y)> for every window geometry, with tail
    windows (fewer valid tokens, and one with none) and varlen packing; and the
    full-window case equals torch autograd of avg_pool1d."""
    rng = np.random.default_rng(21)
    lengths = [0, 5, 31, 32, 33, 100, 257]
    for kernel, stride, tail in ((32, 16, False), (32, 16, True), (5, 3, True), (4, 4, False)):
        nc = [oracle.n_windows(L, kernel, stride, tail) + (1 if tail else 0) for L in lengths]
        cu, cuc = oracle.cu_from_lengths(lengths), oracle.cu_from_lengths(nc)
        x = rng.standard_normal((int(cu[-1]), 3))
        y = rng.standard_normal((int(cuc[-1]), 3))
        lhs = (oracle.mean_pool_varlen(x, cu, cuc, kernel, stride) * y).sum()
        rhs = (x * oracle.mean_pool_varlen_bwd(y, cu, cuc, kernel, stride, int(cu[-1]))).sum()
        assert abs(lhs - rhs) < 1e-12 * max(1.0, abs(lhs)), (kernel, stride, tail)
    L = 300
    x = torch.tensor(rng.standard_normal((1, 4, L)), requires_grad=True)
    pooled = F.avg_pool1d(x, 32, 16)
    gy = rng.standard_normal(tuple(pooled.shape))
    pooled.backward(torch.tensor(gy))
    nc = oracle.n_windows(L, 32, 16)
    got = oracle.mean_pool_varlen_bwd(gy[0].T, [0, L], [0, nc], 32, 16, L)
    np.testing.assert_allclose(got, x.grad[0].numpy().T, atol=1e-13)


def _sdpa_grads(q, kk, vv, mask, d_out, scale, G):
    """torch autograd of masked SDPA in float64: q [T, H, D], kk, vv [L, H_kv, D]
    tensors that may carry grad (already leaves or functions of leaves), mask
    [T, L] bool (rows with no key are excluded by the caller)."""
    qt = torch.tensor(q.transpose(1, 0, 2), requires_grad=True)
    ke = kk.permute(1, 0, 2).repeat_interleave(G, dim=0)
    ve = vv.permute(1, 0, 2).repeat_interleave(G, dim=0)
    out = F.scaled_dot_product_attention(qt, ke, ve, attn_mask=torch.from_numpy(mask)[None],
                                         scale=scale)
    out.backward(torch.tensor(d_out.transpose(1, 0, 2)))
    return qt.grad.numpy().transpose(1, 0, 2)


def test_compressed_branch_grad_equals_autograd_of_pooled_sdpa():
    """The compressed branch is SDPA over avg_pool1d(32, 16)-pooled K and V with
    the window-visibility mask; torch autograd of that composition gives dq and,
    through the pooling, dK and dV."""
    rng = np.random.default_rng(22)
    L, H, H_kv, D = 260, 4, 2, 8
    G, scale = H // H_kv, 0.3
    q = rng.standard_normal((L, H, D))
    k = rng.standard_normal((L, H_kv, D))
    v = rng.standard_normal((L, H_kv, D))
    d_out = rng.standard_normal((L, H, D))
    nc = oracle.n_windows(L, 32, 16)
    rows = [t for t in range(L) if t >= 31]            # rows that see a window
    kl = torch.tensor(k, requires_grad=True)
    vl = torch.tensor(v, requires_grad=True)
    kc_t = F.avg_pool1d(kl.permute(1, 2, 0).reshape(1, H_kv * D, L), 32, 16)
    kc_t = kc_t.reshape(H_kv, D, nc).permute(2, 0, 1)                 # [nc, H_kv, D]
    vc_t = F.avg_pool1d(vl.permute(1, 2, 0).reshape(1, H_kv * D, L), 32, 16)
    vc_t = vc_t.reshape(H_kv, D, nc).permute(2, 0, 1)
    mask = np.array([[oracle.window_visible(c, t, 32, 16) for c in range(nc)] for t in rows])
    dq_ref = _sdpa_grads(q[rows], kc_t, vc_t, mask, d_out[rows], scale, G)
    kc = oracle.mean_pool_varlen(k, [0, L], [0, nc], 32, 16)
    vc = oracle.mean_pool_varlen(v, [0, L], [0, nc], 32, 16)
    dkc, dvc = np.zeros(kc.shape), np.zeros(vc.shape)
    dq = np.stack([oracle.compressed_attention_row_grad(q[t], kc, vc, t, 32, 16, scale, d_out[t],
                                                        dkc, dvc) for t in rows])
    np.testing.assert_allclose(dq, dq_ref, atol=1e-11)
    dk = oracle.mean_pool_varlen_bwd(dkc, [0, L], [0, nc], 32, 16, L)
    dv = oracle.mean_pool_varlen_bwd(dvc, [0, L], [0, nc], 32, 16, L)
    np.testing.assert_allclose(dk, kl.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, vl.grad.numpy(), atol=1e-11)
    # a row that sees no window contributes nothing
    dkc0 = np.zeros(kc.shape)
    assert np.all(oracle.compressed_attention_row_grad(q[30], kc, vc, 30, 32, 16, scale, d_out[30],
                                                       dkc0, dkc0.copy()) == 0)
    assert np.all(dkc0 == 0)


def test_window_branch_grad_equals_autograd_of_banded_sdpa():
    rng = np.random.default_rng(23)
    L, H, H_kv, D, W = 150, 4, 1, 8, 40
    G, scale = H // H_kv, 0.25
    q = rng.standard_normal((L, H, D))
    k = rng.standard_normal((L, H_kv, D))
    v = rng.standard_normal((L, H_kv, D))
    d_out = rng.standard_normal((L, H, D))
    kl = torch.tensor(k, requires_grad=True)
    vl = torch.tensor(v, requires_grad=True)
    t = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    mask = (j <= t) & (j > t - W)
    dq_ref = _sdpa_grads(q, kl, vl, mask, d_out, scale, G)
    dk, dv = np.zeros(k.shape), np.zeros(v.shape)
    dq = np.stack([oracle.window_attention_row_grad(q[r], k, v, r, W, scale, d_out[r], dk, dv)
                   for r in range(L)])
    np.testing.assert_allclose(dq, dq_ref, atol=1e-11)
    np.testing.assert_allclose(dk, kl.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, vl.grad.numpy(), atol=1e-11)


def test_three_branch_grad_matches_finite_differences():
    """The whole three-branch gradient (dq, dk, dv and the gates) against central
    differences of the forward oracle, on rows past 1024 where the selection
    matters; the block choice is checked to stay put under the perturbations."""
    rng = np.random.default_rng(24)
    L, H, H_kv, D = 1300, 4, 2, 8
    q = rng.standard_normal((L, H, D))
    k = rng.standard_normal((L, H_kv, D))
    v = rng.standard_normal((L, H_kv, D))
    gates = 1 / (1 + np.exp(-rng.standard_normal((L, H, 3))))
    d_out = rng.standard_normal((L, H, D))
    rows = [40, 700, 1100, 1299]
    kw = dict(topk=16, window=64)
    res = oracle.nsa_prefill_rows_grad(q, k, v, gates, d_out, rows, **kw)

    def loss():
        f = oracle.nsa_prefill_rows(q, k, v, gates, rows, **kw)
        assert np.array_equal(f["indices"], res["indices"])
        return float((f["out"] * d_out[rows]).sum())

    eps = 1e-6
    checks = [("q", q, None), ("k", k, res["dk"]), ("v", v, res["dv"]), ("gates", gates, None)]
    for name, x, g in checks:
        for _ in range(12):
            if name in ("q", "gates"):
                i = int(rng.integers(len(rows)))
                idx = (rows[i], int(rng.integers(H)), int(rng.integers(x.shape[2])))
                want = (res["dq"] if name == "q" else res["dgates"])[(i,) + idx[1:]]
            else:
                idx = (int(rng.integers(L)), int(rng.integers(H_kv)), int(rng.integers(D)))
                want = g[idx]
            old = x[idx]
            x[idx] = old + eps
            lp = loss()
            x[idx] = old - eps
            lm = loss()
            x[idx] = old
            num = (lp - lm) / (2 * eps)
            assert abs(num - want) < 1e-6 * max(1.0, abs(num)), (name, idx, num, want)
