"""Block-mask attention (nsa_blockmask_attn_fwd) against the float64 oracle."""
import math

import numpy as np
import pytest
import torch

import gen
import oracle
import sparse_attention_compress_amd as nsa
from gen import workloads as W
from parity import assert_close, cu, log, np64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
BF16 = torch.bfloat16
SEED = 0x5EED0800


def _run(lengths, H, density, causal, seed):
    N = sum(lengths)
    q = gen.normal(seed, 1, (N, H, 128), DEV, BF16)
    k = gen.normal(seed, 2, (N, H, 128), DEV, BF16)
    v = gen.normal(seed, 3, (N, H, 128), DEV, BF16)
    nb = -(-max(lengths) // 64)
    keys = gen.random_keys(seed, 8, (len(lengths), H, nb, nb), DEV)
    mask = (keys < int(density * 2 ** 63)).to(torch.uint8)
    cu_k = cu(lengths)
    out = torch.full_like(q, float("nan"))
    nsa.nsa_blockmask_attn_fwd(q, k, v, mask, cu_k, max(lengths), out, causal=causal)
    torch.cuda.synchronize()
    return q, k, v, mask, out


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("density", [0.5, 1.0, 0.1])
def test_blockmask_small_all_rows(causal, density):
    """Every row of a ragged batch (lengths not multiples of 64, one shorter than
    a block) against the oracle."""
    lengths = [1000, 300, 50]
    H = 4
    log(f"blockmask small causal={causal} density={density}")
    q, k, v, mask, out = _run(lengths, H, density, causal, SEED + int(10 * density) + int(causal))
    assert torch.isfinite(out.float()).all()
    qn, kn, vn, mn, on = np64(q), np64(k), np64(v), mask.cpu().numpy(), np64(out)
    cu_np = np.cumsum([0] + lengths)
    ref = np.zeros_like(on)
    for b, L in enumerate(lengths):
        s0 = cu_np[b]
        for t in range(L):
            ref[s0 + t] = oracle.blockmask_attention_row(qn[s0 + t], kn[s0:s0 + L], vn[s0:s0 + L],
                                                         mn[b], t, 64, 1 / math.sqrt(128), causal)
    assert_close(f"blockmask_small[c={causal},d={density}]", on, ref, atol=2e-2)


@pytest.mark.parametrize("seq", [1024, 4096])
def test_blockmask_benchmark_shape_sampled_rows(seq):
    """The pages' benchmark shape (batch 8, 16 heads, 50% of 64 x 64 blocks) at
    1024 and 4096 tokens, on sampled rows of every sequence."""
    w = W.blockmask_prefill(seq)
    q = W.prefill_query(w, DEV)
    k, v = W.keys_values(w, DEV)
    mask = W.block_mask(w, DEV)
    cu_k = cu(w.lengths)
    out = torch.full_like(q, float("nan"))
    log(f"blockmask {w.name}")
    nsa.nsa_blockmask_attn_fwd(q, k, v, mask, cu_k, seq, out)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    mn = mask.cpu().numpy()
    ts = [0, 63, 64, seq // 2 + 17, seq - 1]
    for b in range(w.batch):
        s0 = b * seq
        kn, vn = np64(k[s0:s0 + seq]), np64(v[s0:s0 + seq])
        for t in ts:
            ref = oracle.blockmask_attention_row(np64(q[s0 + t]), kn, vn, mn[b], t, 64,
                                                 1 / math.sqrt(128))
            assert_close(f"blockmask[{b},{t}]", np64(out[s0 + t]), ref, atol=2e-2)


@pytest.mark.parametrize("causal", [False, True])
def test_blockmask_benchmark_shape_16k_sampled_rows(causal):
    """The pages' largest benchmark shape, 8 x 16384 tokens (256 blocks per mask
    row, so the mask-row scan runs over four 64-block chunks), on sampled rows
    of every sequence, including rows at the chunk edges."""
    seq = 16384
    w = W.blockmask_prefill(seq)
    q = W.prefill_query(w, DEV)
    k, v = W.keys_values(w, DEV)
    mask = W.block_mask(w, DEV)
    cu_k = cu(w.lengths)
    out = torch.full_like(q, float("nan"))
    log(f"blockmask {w.name} causal={causal}")
    nsa.nsa_blockmask_attn_fwd(q, k, v, mask, cu_k, seq, out, causal=causal)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    mn = mask.cpu().numpy()
    ts = [0, 63, 64, 4095, 4096, 4097, 8191, 8192, 8209, 12345, 16320, 16383]
    for b in range(w.batch):
        s0 = b * seq
        kn, vn = np64(k[s0:s0 + seq]), np64(v[s0:s0 + seq])
        for t in ts[b % 3::3] + [ts[(5 * b) % len(ts)]]:
            ref = oracle.blockmask_attention_row(np64(q[s0 + t]), kn, vn, mn[b], t, 64,
                                                 1 / math.sqrt(128), causal)
            assert_close(f"blockmask16k[{b},{t},c={int(causal)}]", np64(out[s0 + t]), ref,
                         atol=2e-2)
