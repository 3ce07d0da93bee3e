"""KV offload decode (nsa_decode_step_offload) on the GPU.

The offloaded step reads K/V from pinned host memory through a device block pool.
It must give the resident decode step's indices and outputs bit for bit (the same
selection, and the same attention code over the same values in the same order),
and the float64 oracle's output within the bf16 gate.  The pool bookkeeping is
integer work and is checked exactly against a host model of its rule: listed
blocks already held are kept; every other listed block takes the next free slot
(empty slots first, then slots holding a block the step does not list, each in
ascending order), misses in list order.
"""
import pytest
import torch

import gen
import oracle
import sparse_attention_compress_amd as nsa
from parity import assert_close, cu, log, np64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
BF16 = torch.bfloat16
F32 = torch.float32
SEED = 0x5EED0700


class PoolModel:
    """Host model of the slot tables of one (sequence, KV head)."""

    def __init__(self, slots, nb_cap):
        self.block_of = [-1] * slots
        self.slot_of = [-1] * nb_cap

    def step(self, ids):
        listed = [int(i) for i in ids if i >= 0]
        keep = set(listed)
        free = ([s for s, b in enumerate(self.block_of) if b < 0]
                + [s for s, b in enumerate(self.block_of) if b >= 0 and b not in keep])
        fetched = 0
        for i in listed:
            if self.slot_of[i] < 0:
                s = free[fetched]
                old = self.block_of[s]
                if old >= 0:
                    self.slot_of[old] = -1
                self.slot_of[i] = s
                self.block_of[s] = i
                fetched += 1
        return fetched


def _inputs(lengths, seed, H=16, H_kv=2):
    N = sum(lengths)
    k = gen.normal(seed, 2, (N, H_kv, 128), DEV, BF16)
    v = gen.normal(seed, 3, (N, H_kv, 128), DEV, BF16)
    cis = gen.sigmoid_normal(seed, 4, (N, H_kv), DEV)
    nc = [oracle.n_windows(L, 32, 16) for L in lengths]
    cu_k, cu_c = cu(lengths), cu(nc)
    kc = torch.zeros((max(1, sum(nc)), H_kv, 128), dtype=F32, device=DEV)
    cp = torch.zeros((max(1, sum(nc)), H_kv), dtype=F32, device=DEV)
    nsa.nsa_compress_k(k, kc, cu_k, cu_c, max(nc))
    nsa.nsa_cis_mean_pool_varlen(cis, cp, cu_k, cu_c, max(nc))
    k_host = torch.empty(k.shape, dtype=BF16, pin_memory=True)
    v_host = torch.empty(v.shape, dtype=BF16, pin_memory=True)
    k_host.copy_(k)
    v_host.copy_(v)
    torch.cuda.synchronize()
    return dict(k=k, v=v, k_host=k_host, v_host=v_host, cis=cis, kc=kc, cp=cp, cu_k=cu_k,
                cu_c=cu_c, lengths=list(lengths), H=H, H_kv=H_kv)


def _params(d, q, out, idx, k, v, topk, n_init, n_local, cis_values, n_cand):
    return nsa.decode_params(q, k, v, d["kc"], d["cu_k"], d["cu_c"], max(d["lengths"]), out,
                             topk=topk, n_init=n_init, n_local=n_local, cis=d["cis"],
                             cis_pooled=d["cp"], cis_weight=1.0, cis_values=cis_values,
                             indices=idx, n_cand=n_cand)


@pytest.mark.parametrize("slots,cis_values,n_cand", [(128, False, 0), (64, True, 0), (96, False, 96)])
def test_offload_steps_match_resident_step(slots, cis_values, n_cand):
    """Four decode steps with different queries over the same offloaded cache."""
    lengths = [3000, 9000, 20000, 700, 40]
    d = _inputs(lengths, SEED + 1)
    B, H, H_kv, topk = len(lengths), d["H"], d["H_kv"], 64
    nb_cap = -(-max(lengths) // 64) + 3
    st, keep = nsa.offload_state(B, H_kv, slots, nb_cap, DEV)
    models = [PoolModel(slots, nb_cap) for _ in range(B * H_kv)]
    log(f"offload steps slots={slots} cis_values={cis_values} n_cand={n_cand}")
    for step in range(4):
        # steps 0 and 2 share their queries, so step 2 fetches nothing new
        q = gen.normal(SEED + 1, 10 + (step % 2 if step < 3 else step), (B, H, 128), DEV, BF16)
        out_r = torch.full((B, H, 128), float("nan"), dtype=BF16, device=DEV)
        out_o = torch.full_like(out_r, float("nan"))
        idx_r = torch.full((B, H_kv, topk), -7, dtype=torch.int32, device=DEV)
        idx_o = torch.full_like(idx_r, -7)
        nsa.nsa_decode_step(_params(d, q, out_r, idx_r, d["k"], d["v"], topk, 1, 16, cis_values,
                                    n_cand), device=DEV)
        nsa.nsa_decode_step_offload(_params(d, q, out_o, idx_o, d["k_host"], d["v_host"], topk, 1,
                                            16, cis_values, n_cand), st, device=DEV)
        torch.cuda.synchronize()
        assert torch.equal(idx_o, idx_r), f"step {step}: offloaded selection differs"
        assert torch.equal(out_o, out_r), (f"step {step}: offloaded output differs, max "
                                           f"{(out_o.float() - out_r.float()).abs().max().item()}")
        idx_np = idx_o.cpu().numpy().reshape(B * H_kv, topk)
        want = [m.step(idx_np[u]) for u, m in enumerate(models)]
        got = keep["fetched"].cpu().numpy().tolist()
        assert got == want, f"step {step}: fetched {got} vs model {want}"
        so, bo = keep["slot_of"].cpu().numpy(), keep["block_of"].cpu().numpy()
        for u, m in enumerate(models):
            assert bo[u].tolist() == m.block_of, f"step {step} unit {u}: block_of differs"
            assert so[u].tolist() == m.slot_of, f"step {step} unit {u}: slot_of differs"
        log(f"  step {step}: fetched {sum(got)} blocks ({sum(got) * 32768} bytes)")
        if step == 2 and slots >= 2 * topk:
            assert sum(got) == 0, "a repeated selection must be fully resident"
        if step == 0:
            res = oracle.decode_step(np64(q), np64(d["k"]), np64(d["v"]), np64(d["cu_k"]).astype(int),
                                     topk=topk, n_init=1, n_local=16, cis=np64(d["cis"]),
                                     cis_select=True, cis_values=cis_values, n_cand=n_cand)
            same = [(b, g) for b in range(B) for g in range(H_kv)
                    if (idx_o[b, g].cpu().numpy() == res["indices"][b, g]).all()]
            assert len(same) >= 1
            for b, g in same:
                G = H // H_kv
                assert_close(f"offload.out[{b},{g}]", np64(out_o[b, g * G:(g + 1) * G]),
                             res["out"][b, g * G:(g + 1) * G], atol=2e-2)


def test_offload_pool_exactly_topk_and_degenerate_rows():
    """A pool of exactly topk slots (every block not listed is evicted at once),
    with an empty sequence and sequences shorter than one block or window."""
    lengths = [0, 1, 31, 65, 5000]
    d = _inputs(lengths, SEED + 2)
    B, H, H_kv, topk = len(lengths), d["H"], d["H_kv"], 16
    nb_cap = -(-max(lengths) // 64)
    st, keep = nsa.offload_state(B, H_kv, topk, nb_cap, DEV)
    models = [PoolModel(topk, nb_cap) for _ in range(B * H_kv)]
    for step in range(3):
        q = gen.normal(SEED + 2, 20 + step, (B, H, 128), DEV, BF16)
        out_r = torch.full((B, H, 128), float("nan"), dtype=BF16, device=DEV)
        out_o = torch.full_like(out_r, float("nan"))
        idx_r = torch.full((B, H_kv, topk), -7, dtype=torch.int32, device=DEV)
        idx_o = torch.full_like(idx_r, -7)
        nsa.nsa_decode_step(_params(d, q, out_r, idx_r, d["k"], d["v"], topk, 1, 2, False, 0),
                            device=DEV)
        nsa.nsa_decode_step_offload(_params(d, q, out_o, idx_o, d["k_host"], d["v_host"], topk, 1,
                                            2, False, 0), st, device=DEV)
        torch.cuda.synchronize()
        assert torch.equal(idx_o, idx_r)
        assert torch.equal(out_o, out_r)
        assert torch.equal(out_o[0].float(), torch.zeros_like(out_o[0].float()))
        idx_np = idx_o.cpu().numpy().reshape(B * H_kv, topk)
        want = [m.step(idx_np[u]) for u, m in enumerate(models)]
        assert keep["fetched"].cpu().numpy().tolist() == want
        assert keep["block_of"].cpu().numpy().tolist() == [m.block_of for m in models]


def test_offload_ragged_grid():
    """Three sequences, one KV head, top-20: the pool attention runs 60
    workgroups, not a multiple of the XCD count, in XCD-grouped order."""
    lengths = [9000, 700, 5000]
    d = _inputs(lengths, SEED + 3, H=8, H_kv=1)
    B, H, H_kv, topk, slots = len(lengths), d["H"], d["H_kv"], 20, 40
    nb_cap = -(-max(lengths) // 64)
    st, keep = nsa.offload_state(B, H_kv, slots, nb_cap, DEV)
    models = [PoolModel(slots, nb_cap) for _ in range(B * H_kv)]
    log("offload ragged grid")
    for step in range(2):
        q = gen.normal(SEED + 3, 30 + step, (B, H, 128), DEV, BF16)
        out_r = torch.full((B, H, 128), float("nan"), dtype=BF16, device=DEV)
        out_o = torch.full_like(out_r, float("nan"))
        idx_r = torch.full((B, H_kv, topk), -7, dtype=torch.int32, device=DEV)
        idx_o = torch.full_like(idx_r, -7)
        nsa.nsa_decode_step(_params(d, q, out_r, idx_r, d["k"], d["v"], topk, 1, 4, False, 0),
                            device=DEV)
        nsa.nsa_decode_step_offload(_params(d, q, out_o, idx_o, d["k_host"], d["v_host"], topk, 1,
                                            4, False, 0), st, device=DEV)
        torch.cuda.synchronize()
        assert torch.equal(idx_o, idx_r)
        assert torch.equal(out_o, out_r)
        assert not torch.isnan(out_o.float()).any()
        idx_np = idx_o.cpu().numpy().reshape(B * H_kv, topk)
        want = [m.step(idx_np[u]) for u, m in enumerate(models)]
        assert keep["fetched"].cpu().numpy().tolist() == want
