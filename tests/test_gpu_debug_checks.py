"""Debug mode (nsa_set_debug_checks): the device checks pass valid calls through
unchanged and turn broken preconditions into NSA_ERR_INVALID_ARG before any
work is launched.  Every broken input used here is one the work kernels would
also survive (they clamp what they read), so the checks are what is tested,
not the kernels' behaviour on bad input."""
import numpy as np
import pytest
import torch

import gen
import oracle
import sparse_attention_compress_amd as nsa
from parity import cu, log

pytestmark = pytest.mark.gpu
DEV = "cuda"
SEED = 0x5EED0C00


@pytest.fixture
def checks_on():
    prev = nsa.set_debug_checks(True)
    assert nsa.set_debug_checks(True) is True    # now on
    yield
    nsa.set_debug_checks(prev)


def _expect_invalid(fn, what):
    with pytest.raises(nsa.NsaError) as e:
        fn()
    assert e.value.status == 1, e.value
    assert what in str(e.value), str(e.value)
    log(f"refused as expected: {e.value}")


def test_valid_calls_unchanged(checks_on):
    """A decode step, a selection and the three-branch prefill with checks on
    give the same bits as with checks off."""
    lengths = [700, 3000, 9000]
    N = sum(lengths)
    q = gen.normal(SEED, 1, (3, 16, 128), DEV, torch.bfloat16)
    k = gen.normal(SEED, 2, (N, 2, 128), DEV, torch.bfloat16)
    v = gen.normal(SEED, 3, (N, 2, 128), DEV, torch.bfloat16)
    cis = gen.sigmoid_normal(SEED, 4, (N, 2), DEV)
    nc = [nsa.window_count(L) for L in lengths]
    cu_k, cu_c = cu(lengths), cu(nc)
    kc = torch.zeros((sum(nc), 2, 128), device=DEV)
    cp = torch.zeros((sum(nc), 2), device=DEV)
    nsa.nsa_compress_k(k, kc, cu_k, cu_c, max(nc))
    nsa.nsa_cis_mean_pool_varlen(cis, cp, cu_k, cu_c, max(nc))
    outs = []
    for on in (True, False):
        nsa.set_debug_checks(on)
        out = torch.zeros((3, 16, 128), dtype=torch.bfloat16, device=DEV)
        idx = torch.zeros((3, 2, 64), dtype=torch.int32, device=DEV)
        p = nsa.decode_params(q, k, v, kc, cu_k, cu_c, max(lengths), out, cis=cis, cis_pooled=cp,
                              indices=idx)
        nsa.nsa_decode_step(p, device=DEV)
        torch.cuda.synchronize()
        outs.append((out.clone(), idx.clone()))
    nsa.set_debug_checks(True)
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    # the selected attention over those ids, prefill form, with checks on
    qp = gen.normal(SEED, 5, (N, 16, 128), DEV, torch.bfloat16)
    nb = -(-max(lengths) // 64)
    scores = gen.normal(SEED, 6, (N, 2, nb), DEV)
    ids = torch.zeros((N, 2, 16), dtype=torch.int32, device=DEV)
    nsa.nsa_select_topk(scores, ids, cu_k, max(lengths), 16, cu_seqlens_q=cu_k)
    o = torch.zeros_like(qp)
    nsa.nsa_selected_attn_fwd(qp, k, v, ids, cu_k, max(lengths), o, cu_seqlens_q=cu_k)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()


def test_broken_offsets_are_refused(checks_on):
    """cu_seqlens_k decreasing, not starting at 0, or holding a sequence longer
    than max_seqlen_k; cu_seqlens_q with more rows than keys."""
    nb = 64
    scores = gen.normal(SEED, 7, (4, 2, nb), DEV)
    idx = torch.full((4, 2, 16), -7, dtype=torch.int32, device=DEV)
    for bad, what in (([0, 100, 50, 4000, 4096], "cu_seqlens_k"),
                      ([5, 100, 200, 300, 400], "cu_seqlens_k"),
                      ([0, 100, 5000, 5100, 5200], "cu_seqlens_k")):
        cu_bad = torch.tensor(bad, dtype=torch.int32, device=DEV)
        _expect_invalid(lambda: nsa.nsa_select_topk(scores, idx, cu_bad, 4096, 16, 1, 2), what)
    assert (idx == -7).all(), "work was launched"
    cu_k = torch.tensor([0, 1, 2], dtype=torch.int32, device=DEV)
    cu_q = torch.tensor([0, 2, 4], dtype=torch.int32, device=DEV)
    _expect_invalid(lambda: nsa.nsa_select_topk(scores, idx, cu_k, 64, 16, cu_seqlens_q=cu_q),
                    "more query rows than keys")
    assert (idx == -7).all(), "work was launched"


def test_too_many_windows_refused(checks_on):
    lengths = [100, 40]
    x = gen.normal(SEED, 8, (sum(lengths), 2, 128), DEV)
    # 100 tokens are covered by 6 windows of 32 at stride 16; ask for 7
    cu_k, cu_c = cu(lengths), cu([7, 1])
    xc = torch.full((8, 2, 128), 3.0, device=DEV)
    _expect_invalid(lambda: nsa.nsa_compress_k(x, xc, cu_k, cu_c, 7), "more windows")
    assert (xc == 3.0).all(), "work was launched"
    assert oracle.n_windows(100, 32, 16, True) == 6


def test_duplicate_ids_and_nan_scores_refused(checks_on):
    lengths = [4096, 2000]
    N = sum(lengths)
    q = gen.normal(SEED, 9, (2, 16, 128), DEV, torch.bfloat16)
    k = gen.normal(SEED, 10, (N, 2, 128), DEV, torch.bfloat16)
    idx = torch.tensor(np.array([[[0, 5, 9, 5], [1, 2, 3, -1]], [[0, 1, -1, -1], [4, 4, -1, -1]]]),
                       dtype=torch.int32, device=DEV)
    out = torch.full((2, 16, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    _expect_invalid(lambda: nsa.nsa_selected_attn_fwd(q, k, k, idx, cu(lengths), 4096, out),
                    "same block id twice")
    assert (out.float() == 7.0).all(), "work was launched"
    scores = gen.normal(SEED, 11, (2, 2, 64), DEV)
    scores[1, 0, 17] = float("nan")
    ids = torch.full((2, 2, 16), -7, dtype=torch.int32, device=DEV)
    _expect_invalid(lambda: nsa.nsa_select_topk(scores, ids, cu(lengths), 4096, 16, 1, 2), "NaN")
    assert (ids == -7).all(), "work was launched"
