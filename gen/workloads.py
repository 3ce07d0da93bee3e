"""The five synthetic workloads (shapes, value distributions, seeds).

Shapes follow the pages: the NOSA-1B attention layer (16 query heads, 2 KV heads,
head_dim 128, 28 layers; "NOSA-1B core components", reproduction section), the
TileLang NSA benchmark shape (batch 8, heads 16, dim 128; "TileLang NSA",
performance table) and NSA at 64k tokens ("DeepSeek NSA with Triton",
introduction).  No dataset stands behind any of them: every tensor is drawn from
the seeded generators in :mod:`gen`.

Nothing here computes any step of the method; the workloads only fix sizes and
draw tensors.  Seeds: workload n uses ``0x5EED0000 + n``; each tensor has its own
stream id, and decode layer ``l`` of a multi-layer benchmark adds ``16 * l`` to
the stream ids of its K/V/CIS tensors.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import _lsr, normal, random_keys, sigmoid_normal, u64_at, uniform_ints

S_Q, S_K, S_V, S_CIS, S_GATE, S_LEN, S_IDX, S_MASK, S_DOUT = 1, 2, 3, 4, 5, 6, 7, 8, 9


@dataclass
class Workload:
    name: str
    seed: int
    kind: str                 # "decode" | "prefill_given" | "prefill_nsa"
    batch: int
    lengths: list
    heads: int
    kv_heads: int
    head_dim: int
    dtype: torch.dtype
    kernel: int = 32          # compression window
    stride: int = 16          # compression stride
    block: int = 64           # selection block
    topk: int = 16            # selected blocks per (row, kv head), forced ones included
    n_init: int = 0           # forced leading blocks
    n_local: int = 0          # forced most-recent blocks
    cis_select: bool = False  # pooled CIS added to the block scores
    cis_values: bool = False  # values scaled by CIS, ones-value normaliser
    cis_weight: float = 1.0
    window: int = 0           # sliding-window branch width (three-branch prefill)
    extra: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.heads // self.kv_heads

    @property
    def total_tokens(self) -> int:
        return int(sum(self.lengths))

    def cu_seqlens(self) -> list:
        out = [0]
        for L in self.lengths:
            out.append(out[-1] + int(L))
        return out


def tiny_decode() -> Workload:
    return Workload("tiny_decode_fp32_L4096", 0x5EED0001, "decode", 1, [4096], 16, 2, 128,
                    torch.float32, topk=16, n_init=1, n_local=2)


def nosa1b_decode(pinned_32k: bool = False, batch: int = 8) -> Workload:
    """Batched decode; other batch sizes draw more lengths from the same stream
    (the first 8 are the batch-8 lengths)."""
    seed = 0x5EED0002
    lengths = [32768] * batch if pinned_32k else uniform_ints(seed, S_LEN, batch, 8192, 32768)
    span = "L32768" if pinned_32k else "L8k-32k"
    name = f"nosa1b_decode_b{batch}_{span}"
    return Workload(name, seed, "decode", batch, lengths, 16, 2, 128, torch.bfloat16,
                    topk=64, n_init=1, n_local=1024 // 64, cis_select=True)


def selected_prefill() -> Workload:
    return Workload("selected_prefill_b8_T16384", 0x5EED0003, "prefill_given", 8, [16384] * 8,
                    16, 2, 128, torch.bfloat16, topk=16)


def nsa_prefill() -> Workload:
    return Workload("nsa_three_branch_prefill_T65536", 0x5EED0004, "prefill_nsa", 1, [65536],
                    64, 4, 128, torch.bfloat16, topk=16, window=512)


def cis_decode() -> Workload:
    return Workload("cis_decode_b4_L131072", 0x5EED0005, "decode", 4, [131072] * 4, 16, 2, 128,
                    torch.bfloat16, topk=64, n_init=1, n_local=1024 // 64,
                    cis_select=True, cis_values=True)


def blockmask_prefill(seq: int = 16384, causal: bool = False) -> Workload:
    """The pages' block-sparse benchmark shape (TileLang NSA, performance table):
    batch 8, 16 heads, head_dim 128, 64 x 64 blocks at 50% density."""
    return Workload(f"blockmask_b8_h16_T{seq}" + ("_causal" if causal else ""), 0x5EED0006,
                    "prefill_blockmask", 8, [seq] * 8, 16, 16, 128, torch.bfloat16,
                    extra={"density": 0.5, "causal": causal})


def block_mask(w: Workload, device="cpu", density: float = None) -> torch.Tensor:
    """uint8 [B, H, nb, nb] (nb = ceil(max length / 64)): block (b, h, i, j) is on
    when the top 63 bits of its counter's splitmix64 output fall below
    density * 2**63 (an integer comparison)."""
    if density is None:
        density = w.extra.get("density", 0.5)
    nb = (max(w.lengths) + w.block - 1) // w.block
    keys = random_keys(w.seed, S_MASK, (w.batch, w.heads, nb, nb), device)
    return (keys < int(density * 2 ** 63)).to(torch.uint8)


ALL = {
    1: tiny_decode,
    2: nosa1b_decode,
    3: selected_prefill,
    4: nsa_prefill,
    5: cis_decode,
}


def scaled(w: Workload, lengths: list, name_suffix: str = "_small") -> Workload:
    """Same recipe at other sequence lengths (small cases the oracle finishes quickly)."""
    import dataclasses
    return dataclasses.replace(w, lengths=list(lengths), batch=len(lengths), name=w.name + name_suffix)


# ----------------------------------------------------------------------------- tensors

def decode_query(w: Workload, device="cpu", layer: int = 0) -> torch.Tensor:
    """[B, H, D] query of the newest token of every sequence."""
    return normal(w.seed, S_Q + 16 * layer, (w.batch, w.heads, w.head_dim), device, w.dtype)


def prefill_query(w: Workload, device="cpu") -> torch.Tensor:
    """[N, H, D] packed queries, one per token."""
    return normal(w.seed, S_Q, (w.total_tokens, w.heads, w.head_dim), device, w.dtype)


def prefill_out_grad(w: Workload, device="cpu") -> torch.Tensor:
    """[N, H, D] upstream gradient of the attention output, N(0,1), one per token."""
    return normal(w.seed, S_DOUT, (w.total_tokens, w.heads, w.head_dim), device, w.dtype)


def keys_values(w: Workload, device="cpu", layer: int = 0):
    """Packed K and V, each [N, H_kv, D]."""
    shape = (w.total_tokens, w.kv_heads, w.head_dim)
    k = normal(w.seed, S_K + 16 * layer, shape, device, w.dtype)
    v = normal(w.seed, S_V + 16 * layer, shape, device, w.dtype)
    return k, v


def cis_scores(w: Workload, device="cpu", layer: int = 0) -> torch.Tensor:
    """Per-token, per-KV-head importance scores, sigmoid(N(0,1)), float32 [N, H_kv]."""
    return sigmoid_normal(w.seed, S_CIS + 16 * layer, (w.total_tokens, w.kv_heads), device)


def gates(w: Workload, device="cpu") -> torch.Tensor:
    """Branch gates sigmoid(N(0,1)), float32 [N, H, 3]."""
    return sigmoid_normal(w.seed, S_GATE, (w.total_tokens, w.heads, 3), device)


def given_block_indices(w: Workload, device="cpu", row_chunk: int = 1 << 16) -> torch.Tensor:
    """int32 [N, H_kv, topk]: for the query at position t of its sequence, a
    uniform random subset (without replacement) of min(topk, t//block + 1) of the
    blocks whose start is <= t, sorted ascending, padded with -1.

    The subset is the ``topk`` smallest random keys among the causal blocks; key
    of (row r, slot s) is counter ``r * n_slots + s`` of the index stream, with
    row r = token * H_kv + kv head."""
    n_tok = w.total_tokens
    max_len = max(w.lengths)
    n_slots = (max_len + w.block - 1) // w.block
    pos = torch.cat([torch.arange(L, dtype=torch.int64) for L in w.lengths]).to(device)
    rows_total = n_tok * w.kv_heads
    out = torch.empty(rows_total, w.topk, dtype=torch.int32, device=device)
    big = torch.iinfo(torch.int64).max
    slot = torch.arange(n_slots, dtype=torch.int64, device=device)
    for r0 in range(0, rows_total, row_chunk):
        r1 = min(rows_total, r0 + row_chunk)
        rows = torch.arange(r0, r1, dtype=torch.int64, device=device)
        counters = rows[:, None] * n_slots + slot[None, :]
        keys = _lsr(u64_at(w.seed, S_IDX, counters), 1)
        n_avail = pos[rows // w.kv_heads] // w.block + 1
        keys = torch.where(slot[None, :] < n_avail[:, None], keys, torch.full_like(keys, big))
        kk = min(w.topk, n_slots)
        sel = torch.topk(keys, kk, dim=1, largest=False).indices
        sel = torch.where(sel < n_avail[:, None], sel, torch.full_like(sel, n_slots + 1))
        sel = torch.sort(sel, dim=1).values
        sel = torch.where(sel > n_slots, torch.full_like(sel, -1), sel)
        if kk < w.topk:
            pad = torch.full((r1 - r0, w.topk - kk), -1, dtype=sel.dtype, device=device)
            sel = torch.cat([sel, pad], dim=1)
        out[r0:r1] = sel.to(torch.int32)
    return out.reshape(n_tok, w.kv_heads, w.topk)
