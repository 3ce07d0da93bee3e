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
