"""nsa_decode_step_noalloc (the decode step over the library's fixed scratch)
against nsa_decode_step with a caller workspace: two calls in a row on one GPU,
the second with a smaller batch and shorter contexts, must give bit-identical
outputs, block scores and indices; a step whose workspace exceeds the scratch is
refused before launching.  Calls go through the C ABI."""
import pytest
import torch

import gen
import sparse_attention_compress_amd as nsa
from parity import cu, log

pytestmark = pytest.mark.gpu
DEV = "cuda"
SEED = 0x5EED0A00


def _case(lengths, seed, H=16, H_kv=2, topk=64, n_local=16, cis_values=False):
    N, B = sum(lengths), len(lengths)
    q = gen.normal(seed, 1, (B, H, 128), DEV, torch.bfloat16)
    k = gen.normal(seed, 2, (N, H_kv, 128), DEV, torch.bfloat16)
    v = gen.normal(seed, 3, (N, H_kv, 128), DEV, torch.bfloat16)
    cis = gen.sigmoid_normal(seed, 4, (N, H_kv), DEV)
    nc = [nsa.window_count(L) for L in lengths]
    cu_k, cu_c = cu(lengths), cu(nc)
    kc = torch.zeros((max(1, sum(nc)), H_kv, 128), dtype=torch.float32, device=DEV)
    cp = torch.zeros((max(1, sum(nc)), H_kv), dtype=torch.float32, device=DEV)
    nsa.nsa_compress_k(k, kc, cu_k, cu_c, max(nc))
    nsa.nsa_cis_mean_pool_varlen(cis, cp, cu_k, cu_c, max(nc))
    nb_max = -(-max(lengths) // 64)
    outs = []
    params = []
    for _ in range(2):
        o = dict(out=torch.full((B, H, 128), float("nan"), dtype=torch.bfloat16, device=DEV),
                 bs=torch.full((B, H_kv, nb_max), float("nan"), device=DEV),
                 idx=torch.full((B, H_kv, topk), -7, dtype=torch.int32, device=DEV))
        params.append(nsa.decode_params(q, k, v, kc, cu_k, cu_c, max(lengths), o["out"], topk=topk,
                                        n_init=1, n_local=n_local, cis=cis, cis_pooled=cp,
                                        cis_weight=1.0, cis_values=cis_values, append_window=True,
                                        block_scores=o["bs"], indices=o["idx"]))
        outs.append(o)
    keep = (q, k, v, cis, kc, cp, cu_k, cu_c)
    return params, outs, keep


def _same(a, b, name):
    for key in ("out", "bs", "idx"):
        x, y = a[key], b[key]
        assert torch.equal(x, y) or (x.is_floating_point() and torch.equal(x.nan_to_num(0.5),
                                                                              y.nan_to_num(0.5))), \
            f"{name}.{key} differs"


def test_noalloc_decode_matches_workspace_decode_twice():
    cases = [([31994, 8612, 30991, 19970, 9628, 14163, 9370, 12020], SEED + 1, False),
             ([5000, 700, 40], SEED + 2, True)]              # second call: smaller input
    for lengths, seed, cis_values in cases:
        params, outs, keep = _case(lengths, seed, cis_values=cis_values)
        log(f"no-alloc decode lengths={lengths} cis_values={cis_values}")
        nsa.nsa_decode_step(params[0], device=DEV)
        nsa.nsa_decode_step_noalloc(params[1])
        torch.cuda.synchronize()
        assert torch.isfinite(outs[1]["out"].float()).all()
        _same(outs[0], outs[1], f"noalloc[{len(lengths)}]")


def test_noalloc_decode_refuses_oversized_step():
    big = 40000
    lengths = [32768] * big
    B = len(lengths)
    p = nsa.DecodeParams()
    # sizes only: the check runs on the host before anything is read
    fake = 0x1000
    p.q = p.k = p.v = p.k_c = p.cu_seqlens_k = p.cu_seqlens_c = p.out = fake
    p.dtype, p.kc_dtype = nsa.NSA_BF16, nsa.NSA_F32
    p.batch, p.max_seqlen_k, p.heads, p.kv_heads, p.head_dim = B, 32768, 16, 2, 128
    p.kernel, p.stride, p.block_size = 32, 16, 64
    p.topk, p.n_init, p.n_local = 64, 1, 16
    p.cis_weight = 0.0
    assert nsa.decode_workspace_size(p) > nsa.decode_noalloc_scratch_bytes()
    with pytest.raises(nsa.NsaError) as e:
        nsa.nsa_decode_step_noalloc(p)
    assert e.value.status == 3 and "scratch" in str(e.value)
