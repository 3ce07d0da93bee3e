"""The C ABI: the built library loads, exports every function include/nsa.h
declares, and rejects bad arguments on the host (before any launch), so these
run without a GPU."""
import ctypes
import os
import re

import pytest

import sparse_attention_compress_amd as nsa

pytestmark = pytest.mark.skipif(not os.path.exists(nsa.LIB_PATH), reason="libnsa.so not built")


def _declared():
    text = open(nsa.HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nsa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_hot_path():
    names = _declared()
    for n in ("nsa_compress_k", "nsa_compressed_scores", "nsa_cis_mean_pool_varlen",
              "nsa_select_topk", "nsa_selected_attn_fwd", "nsa_decode_step"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(nsa.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(L, n)]
    assert not missing, missing
    assert nsa.lib().nsa_version() >= 100


def test_binding_covers_every_declared_entry_point():
    for n in _declared():
        assert n in nsa._SIGS, n


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def test_unsupported_geometry_is_rejected():
    L = nsa.lib()
    st = L.nsa_compressed_scores(FAKE, 1, FAKE, 0, None, 1.0, FAKE, None, FAKE, FAKE, 2, 4096, 16, 2,
                                 64, 32, 16, 64, 0.0, FAKE, 1 << 20, None)
    assert st == 2 and "head_dim" in nsa.last_error()
    st = L.nsa_compressed_scores(FAKE, 1, FAKE, 0, None, 1.0, FAKE, None, FAKE, FAKE, 2, 4096, 16, 2,
                                 128, 64, 32, 64, 0.0, FAKE, 1 << 20, None)
    assert st == 2 and "window" in nsa.last_error()
    st = L.nsa_compressed_scores(FAKE, 1, FAKE, 0, None, 1.0, FAKE, None, FAKE, FAKE, 2, 4096, 16, 3,
                                 128, 32, 16, 64, 0.0, FAKE, 1 << 20, None)
    assert st == 2


def test_workspace_too_small_and_nulls():
    L = nsa.lib()
    need = L.nsa_compressed_scores_workspace_size(2, 4096, 16, 2, 32, 16)
    assert need > 0
    st = L.nsa_compressed_scores(FAKE, 1, FAKE, 0, None, 1.0, FAKE, None, FAKE, FAKE, 2, 4096, 16, 2,
                                 128, 32, 16, 64, 0.0, FAKE, need - 1, None)
    assert st == 3
    st = L.nsa_compressed_scores(None, 1, FAKE, 0, None, 1.0, FAKE, None, FAKE, FAKE, 2, 4096, 16, 2,
                                 128, 32, 16, 64, 0.0, FAKE, need, None)
    assert st == 1


def test_select_argument_checks():
    L = nsa.lib()
    # forced blocks larger than k
    assert L.nsa_select_topk(FAKE, FAKE, None, FAKE, 1, 1, 4096, 2, 64, 4, 2, 3, 64, None) == 1
    # n_blocks_max too small for max_seqlen_k
    assert L.nsa_select_topk(FAKE, FAKE, None, FAKE, 1, 1, 4096, 2, 63, 16, 1, 2, 64, None) == 1
    # too many blocks per row for the in-LDS sort
    assert L.nsa_select_topk(FAKE, FAKE, None, FAKE, 1, 1, 1 << 20, 2, 1 << 14, 16, 1, 2, 64, None) == 2
    # decode needs rows == batch
    assert L.nsa_select_topk(FAKE, FAKE, None, FAKE, 2, 3, 4096, 2, 64, 16, 1, 2, 64, None) == 1
    # empty batch is a no-op
    assert L.nsa_select_topk(None, None, None, None, 0, 0, 0, 2, 0, 16, 1, 2, 64, None) == 0


def test_attention_and_pool_checks():
    L = nsa.lib()
    st = L.nsa_selected_attn_fwd(FAKE, FAKE, FAKE, 1, FAKE, 16, None, FAKE, None, None, FAKE, 2, 2, 4096,
                                 16, 2, 96, 64, 0.0, FAKE, 1 << 20, None)
    assert st == 2
    st = L.nsa_selected_attn_fwd(FAKE, FAKE, FAKE, 7, FAKE, 16, None, FAKE, None, None, FAKE, 2, 2, 4096,
                                 16, 2, 128, 64, 0.0, FAKE, 1 << 20, None)
    assert st == 2
    misaligned = ctypes.c_void_p(0x1008)
    st = L.nsa_selected_attn_fwd(misaligned, FAKE, FAKE, 1, FAKE, 16, None, FAKE, None, None, FAKE, 2, 2,
                                 4096, 16, 2, 128, 64, 0.0, FAKE, 1 << 20, None)
    assert st == 1 and "aligned" in nsa.last_error()
    assert L.nsa_compress_k(FAKE, 1, FAKE, 0, FAKE, FAKE, 1, 10, 2, 128, 0, 16, None) == 1
    assert L.nsa_cis_mean_pool_varlen(None, FAKE, FAKE, FAKE, 1, 10, 2, 32, 16, None) == 1
    assert L.nsa_cis_mean_pool_varlen(None, None, None, None, 0, 0, 2, 32, 16, None) == 0


def test_decode_step_checks():
    import torch
    p = nsa.DecodeParams()
    p.batch, p.max_seqlen_k, p.heads, p.kv_heads, p.head_dim = 2, 4096, 16, 2, 128
    p.kernel, p.stride, p.block_size = 32, 16, 64
    p.topk, p.n_init, p.n_local = 16, 1, 2
    p.dtype, p.kc_dtype = nsa.NSA_BF16, nsa.NSA_F32
    # all pointers null -> invalid argument, and no workspace size
    assert nsa.decode_workspace_size(p) == 0
    assert nsa.lib().nsa_decode_step(ctypes.byref(p), None, 0, None) == 1
    for f in ("q", "k", "v", "k_c", "cu_seqlens_k", "cu_seqlens_c", "out"):
        setattr(p, f, 0x1000)
    need = nsa.decode_workspace_size(p)
    assert need > 0
    assert nsa.lib().nsa_decode_step(ctypes.byref(p), ctypes.c_void_p(0x1000), need - 1, None) == 3
    p.cis_values = 1   # CIS values without cis
    assert nsa.lib().nsa_decode_step(ctypes.byref(p), ctypes.c_void_p(0x1000), need, None) == 1
    p.cis_values = 0
    p.n_local = 16     # forced blocks exceed topk
    assert nsa.lib().nsa_decode_step(ctypes.byref(p), ctypes.c_void_p(0x1000), need, None) == 1
    assert torch is not None


def test_prefill_branch_checks():
    L = nsa.lib()
    need = L.nsa_compressed_attn_workspace_size(1, 100, 100, 64, 4, 32, 16)
    assert need >= 100 * 64 * 4 + 4 * 128 * 64 * 2
    args = [FAKE, FAKE, FAKE, nsa.NSA_BF16, FAKE, nsa.NSA_F32, None, None, 0, FAKE, FAKE, FAKE,
            1, 100, 100, 64, 4, 128, 32, 16, 64, 0.0, FAKE, need, None]
    bad = list(args)
    bad[3] = nsa.NSA_F32          # fp32 inputs: the tiles are bf16
    assert L.nsa_compressed_attn_fwd(*bad) == 2
    bad = list(args)
    bad[9] = None                 # prefill rows need cu_seqlens_q
    assert L.nsa_compressed_attn_fwd(*bad) == 1
    bad = list(args)
    bad[7], bad[8] = FAKE, 1      # n_blocks_max below ceil(max_seqlen_k / 64)
    assert L.nsa_compressed_attn_fwd(*bad) == 1
    bad = list(args)
    bad[23] = need - 1            # workspace too small
    assert L.nsa_compressed_attn_fwd(*bad) == 3
    bad = list(args)
    bad[15] = 3                   # 64 heads / 3 kv heads
    assert L.nsa_compressed_attn_fwd(*bad) == 2
    wneed = L.nsa_window_attn_workspace_size(1, 100, 4)
    assert wneed >= 4 * 128 * 128 * 2
    wargs = [FAKE, FAKE, FAKE, nsa.NSA_BF16, FAKE, nsa.NSA_BF16, None, FAKE, FAKE, 1, 100, 100, 64,
             4, 128, 512, 0.0, FAKE, wneed, None]
    bad = list(wargs)
    bad[18] = wneed - 1           # workspace too small
    assert L.nsa_window_attn_fwd(*bad) == 3
    bad = list(wargs)
    bad[15] = 0                   # empty window
    assert L.nsa_window_attn_fwd(*bad) == 1
    bad = list(wargs)
    bad[7] = None
    assert L.nsa_window_attn_fwd(*bad) == 1
    bad = list(wargs)
    bad[0] = ctypes.c_void_p(0x1008)
    assert L.nsa_window_attn_fwd(*bad) == 1 and "aligned" in nsa.last_error()


def test_prefill_step_checks():
    p = nsa.PrefillParams()
    p.batch, p.rows_total, p.max_seqlen_k, p.heads, p.kv_heads, p.head_dim = 1, 1000, 1000, 64, 4, 128
    p.kernel, p.stride, p.block_size = 32, 16, 64
    p.topk, p.n_init, p.n_local, p.window = 16, 0, 0, 512
    p.dtype = nsa.NSA_BF16
    assert nsa.prefill_workspace_size(p) == 0           # null pointers
    assert nsa.lib().nsa_prefill_step(ctypes.byref(p), None, 0, None) == 1
    for f in ("q", "k", "v", "k_c", "v_c", "gates", "cu_seqlens_q", "cu_seqlens_k",
              "cu_seqlens_c", "out"):
        setattr(p, f, 0x1000)
    need, least = nsa.prefill_workspace_size(p), nsa.prefill_workspace_size_min(p)
    # lse (fp32) + o_cmp and o_sel (bf16 rows) + block scores + indices
    assert least >= 1000 * 64 * 4 + 2 * 1000 * 64 * 128 * 2 + 1000 * 4 * 16 * 4 + 1000 * 4 * 16 * 4
    # the key-block selected branch adds its partial states (256 B of bf16 output
    # and 8 B of (max, sum) per (row, head, place)), its float32 rows and its
    # block lists (2 B of row code and 8 B of list head per (row, KV head, place))
    assert need - least == 1000 * 64 * 16 * 264 + 1000 * 64 * 128 * 4 + 1000 * 4 * 16 * 10
    assert nsa.lib().nsa_prefill_step(ctypes.byref(p), ctypes.c_void_p(0x1000), least - 1, None) == 3
    p.topk = 65                                          # above the per-row staging limit
    assert nsa.lib().nsa_prefill_step(ctypes.byref(p), ctypes.c_void_p(0x1000), need, None) == 2
    p.topk = 16
    p.dtype = nsa.NSA_F32
    assert nsa.lib().nsa_prefill_step(ctypes.byref(p), ctypes.c_void_p(0x1000), need, None) == 2


def test_missing_library_fails_loudly(tmp_path):
    """Without libnsa.so the binding raises ImportError on first use: there is no
    fallback path of any kind."""
    import shutil
    import subprocess
    import sys
    pkg = tmp_path / "sparse_attention_compress_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(os.path.dirname(nsa.__file__), "__init__.py"), pkg / "__init__.py")
    code = (
        "import sys\n"
        f"sys.path.insert(0, {str(tmp_path)!r})\n"
        "import torch\n"
        "import sparse_attention_compress_amd as m\n"
        "assert m.__file__.startswith(sys.path[0])\n"
        "try:\n"
        "    m.lib()\n"
        "except ImportError as e:\n"
        "    print('IMPORT_ERROR', e)\n"
        "try:\n"
        "    x = torch.zeros(64, 2, 128, dtype=torch.bfloat16)\n"
        "    xc = torch.zeros(3, 2, 128, dtype=torch.float32)\n"
        "    cu = torch.tensor([0, 64], dtype=torch.int32)\n"
        "    m.nsa_compress_k(x, xc, cu, torch.tensor([0, 3], dtype=torch.int32), 3)\n"
        "except ImportError as e:\n"
        "    print('ENTRY_IMPORT_ERROR', e)\n")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert "IMPORT_ERROR" in res.stdout, res.stdout + res.stderr
    assert "ENTRY_IMPORT_ERROR" in res.stdout, res.stdout + res.stderr


def test_two_stage_and_offload_checks():
    p = nsa.DecodeParams()
    p.batch, p.max_seqlen_k, p.heads, p.kv_heads, p.head_dim = 2, 4096, 16, 2, 128
    p.kernel, p.stride, p.block_size = 32, 16, 64
    p.topk, p.n_init, p.n_local = 16, 1, 2
    p.dtype, p.kc_dtype = nsa.NSA_BF16, nsa.NSA_F32
    for f in ("q", "k", "v", "k_c", "cu_seqlens_k", "cu_seqlens_c", "out"):
        setattr(p, f, 0x1000)
    need = nsa.decode_workspace_size(p)
    ws = ctypes.c_void_p(0x1000)
    p.n_cand = 32      # two stages need the pooled CIS
    assert nsa.lib().nsa_decode_step(ctypes.byref(p), ws, need, None) == 1
    p.n_cand = -1
    assert nsa.lib().nsa_decode_step(ctypes.byref(p), ws, need, None) == 1
    p.n_cand = 0
    o = nsa.OffloadState()
    o.k_pool = o.v_pool = o.slot_of = o.block_of = 0x1000
    o.pool_slots, o.nb_cap = 64, 64
    need_o = nsa.decode_offload_workspace_size(p, o)
    assert need_o > need
    step = nsa.lib().nsa_decode_step_offload
    assert step(ctypes.byref(p), ctypes.byref(o), ws, need_o - 1, None) == 3   # workspace
    o.pool_slots = 8   # fewer slots than topk
    assert step(ctypes.byref(p), ctypes.byref(o), ws, need_o, None) == 1
    o.pool_slots = 2048  # above the pool limit
    assert step(ctypes.byref(p), ctypes.byref(o), ws, need_o, None) == 2
    o.pool_slots, o.nb_cap = 64, 32  # 64 blocks per sequence above nb_cap
    assert step(ctypes.byref(p), ctypes.byref(o), ws, need_o, None) == 1
    o.nb_cap = 64
    p.dtype = nsa.NSA_F32  # bfloat16 K/V only
    assert step(ctypes.byref(p), ctypes.byref(o), ws, need_o, None) == 2
    p.dtype = nsa.NSA_BF16
    o.k_pool = 0
    assert step(ctypes.byref(p), ctypes.byref(o), ws, need_o, None) == 1
    assert nsa.lib().nsa_offload_reset(ctypes.byref(o), 2, 2, None) == 1
    assert nsa.lib().nsa_offload_pool_bytes(2, 2, 64, 128, nsa.NSA_BF16) == 2 * 2 * 64 * 64 * 128 * 2


def test_selected_bwd_checks():
    """Argument checks of the selected-attention backward, all taken on the host
    before any launch (fake device addresses are never dereferenced)."""
    f = nsa.lib().nsa_selected_attn_bwd
    P = 0x1000
    full = nsa.selected_attn_bwd_workspace_size(2, 100, 4096, 16, 2, 16)
    need = nsa.selected_attn_bwd_workspace_size_min(2, 100, 4096, 16, 2, 16)
    assert 0 < need < full
    # the key-block dq adds its partial states: 256 B of bf16 per (row, head, place)
    # the key-block dq's partial states (bf16) and its block lists
    assert full - ((need + 255) // 256 * 256) == 100 * 16 * 16 * 256 + 100 * 2 * 16 * 10
    assert nsa.selected_attn_bwd_workspace_size(0, 100, 4096, 16, 2, 16) == 0
    assert nsa.selected_attn_bwd_workspace_size_min(0, 100, 4096, 16, 2, 16) == 0

    def call(dtype=nsa.NSA_BF16, k_sel=16, cu_q=P, heads=16, kv=2, hd=128, block=64, ws=P,
             nbytes=None, dk=P):
        return f(P, P, P, P, P, P, dtype, P, k_sel, cu_q, P, 2, 100, 4096, heads, kv, hd, block,
                 0.0, P, dk, P, ws, need if nbytes is None else nbytes, None)
    assert call(dtype=nsa.NSA_F32) == 2          # bfloat16 only
    assert call(k_sel=65) == 2                   # above the prefill top-k limit
    assert call(k_sel=0) == 2
    assert call(cu_q=None) == 1                  # prefill rows only
    assert call(heads=12, kv=5) == 2             # group size
    assert call(hd=64) == 2
    assert call(block=32) == 2
    assert call(nbytes=need - 1) == 3            # workspace below the smallest size
    assert call(ws=None) == 3
    assert call(dk=P + 4) == 1                   # gradients must be 16-byte aligned
    assert call(dk=None) == 1
    assert call(ws=P + 8) == 1                   # workspace must be 16-byte aligned


def test_window_count_export():
    """nsa_window_count against the hand-derived window counts of the geometry
    fixture, and against the oracle's count over a sweep of lengths and window
    shapes, in both tail modes; invalid arguments give -1."""
    import json

    import oracle
    L = nsa.lib()
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "window_geometry.json")))
    for length, full, tail in fx["window_counts"]:
        assert L.nsa_window_count(length, 32, 16, 0) == full, length
        assert L.nsa_window_count(length, 32, 16, 1) == tail, length
        assert nsa.window_count(length) == full
        assert nsa.window_count(length, tail=True) == tail
    for kernel, stride in ((32, 16), (8, 8), (5, 3), (1, 1), (64, 1)):
        for length in list(range(0, 200)) + [4095, 4096, 4097, 65536, 131072]:
            for tail in (0, 1):
                assert L.nsa_window_count(length, kernel, stride, tail) == \
                    oracle.n_windows(length, kernel, stride, bool(tail)), (length, kernel, stride, tail)
    for args in ((-1, 32, 16, 0), (10, 0, 16, 0), (10, 32, 0, 0), (10, 32, 16, 2)):
        assert L.nsa_window_count(*args) == -1
