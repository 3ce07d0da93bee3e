"""Python binding of libnsa (the gfx950 native-sparse-attention hot path).

Argument marshalling only: every function takes torch tensors that already live
on the GPU, passes their device pointers and sizes to the C ABI declared in
``include/nsa.h`` and enqueues the work on torch's current HIP stream.  All
computation happens in the HIP kernels of ``libnsa.so``; if the library is not
built this module raises instead of falling back to anything else.

Workspaces: functions that need one accept ``workspace=`` (a uint8 CUDA tensor
of at least the queried size; no initialisation needed).  When it is omitted the
binding keeps one buffer per (device, size) and reuses it, which is safe for
calls on one stream.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnsa.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "nsa.h")

NSA_F32, NSA_BF16 = 0, 1
STATUS = {0: "NSA_OK", 1: "NSA_ERR_INVALID_ARG", 2: "NSA_ERR_UNSUPPORTED", 3: "NSA_ERR_WORKSPACE",
          4: "NSA_ERR_HIP"}

_lib = None


class NsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


c_i32, c_f32, c_sz, c_vp = ctypes.c_int32, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


class DecodeParams(ctypes.Structure):
    """Mirror of ``nsa_decode_params``."""
    _fields_ = [
        ("q", c_vp), ("k", c_vp), ("v", c_vp), ("k_c", c_vp), ("cis", c_vp), ("cis_pooled", c_vp),
        ("cu_seqlens_k", c_vp), ("cu_seqlens_c", c_vp), ("out", c_vp), ("block_scores", c_vp),
        ("indices", c_vp), ("dtype", ctypes.c_int), ("kc_dtype", ctypes.c_int),
        ("batch", c_i32), ("max_seqlen_k", c_i32), ("heads", c_i32), ("kv_heads", c_i32),
        ("head_dim", c_i32), ("kernel", c_i32), ("stride", c_i32), ("block_size", c_i32),
        ("topk", c_i32), ("n_init", c_i32), ("n_local", c_i32), ("cis_weight", c_f32),
        ("cis_values", c_i32), ("append_window", c_i32), ("softmax_scale", c_f32),
        ("n_cand", c_i32),
    ]


class OffloadState(ctypes.Structure):
    """Mirror of ``nsa_offload_state``."""
    _fields_ = [
        ("k_pool", c_vp), ("v_pool", c_vp), ("slot_of", c_vp), ("block_of", c_vp),
        ("fetched", c_vp), ("pool_slots", c_i32), ("nb_cap", c_i32),
    ]


class PrefillParams(ctypes.Structure):
    """Mirror of ``nsa_prefill_params``."""
    _fields_ = [
        ("q", c_vp), ("k", c_vp), ("v", c_vp), ("k_c", c_vp), ("v_c", c_vp), ("gates", c_vp),
        ("cu_seqlens_q", c_vp), ("cu_seqlens_k", c_vp), ("cu_seqlens_c", c_vp), ("out", c_vp),
        ("block_scores", c_vp), ("indices", c_vp), ("dtype", ctypes.c_int),
        ("batch", c_i32), ("rows_total", c_i32), ("max_seqlen_k", c_i32), ("heads", c_i32),
        ("kv_heads", c_i32), ("head_dim", c_i32), ("kernel", c_i32), ("stride", c_i32),
        ("block_size", c_i32), ("topk", c_i32), ("n_init", c_i32), ("n_local", c_i32),
        ("window", c_i32), ("softmax_scale", c_f32),
    ]


_SIGS = {
    "nsa_last_error": (ctypes.c_char_p, []),
    "nsa_version": (c_i32, []),
    "nsa_window_count": (c_i32, [c_i32, c_i32, c_i32, c_i32]),
    "nsa_set_debug_checks": (c_i32, [c_i32]),
    "nsa_profile_next_launch": (ctypes.c_int, [c_i32, c_vp, c_vp]),
    "nsa_compress_k": (ctypes.c_int, [c_vp, ctypes.c_int, c_vp, ctypes.c_int, c_vp, c_vp, c_i32,
                                      c_i32, c_i32, c_i32, c_i32, c_i32, c_vp]),
    "nsa_cis_mean_pool_varlen": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                                                c_i32, c_vp]),
    "nsa_compressed_scores_workspace_size": (c_sz, [c_i32] * 6),
    "nsa_compressed_scores": (ctypes.c_int, [c_vp, ctypes.c_int, c_vp, ctypes.c_int, c_vp, c_f32,
                                             c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                                             c_i32, c_i32, c_i32, c_i32, c_f32, c_vp, c_sz, c_vp]),
    "nsa_select_topk": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32,
                                       c_i32, c_i32, c_i32, c_i32, c_vp]),
    "nsa_selected_attn_workspace_size": (c_sz, [c_i32] * 6),
    "nsa_selected_attn_fwd": (ctypes.c_int, [c_vp, c_vp, c_vp, ctypes.c_int, c_vp, c_i32, c_vp,
                                             c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                                             c_i32, c_i32, c_i32, c_f32, c_vp, c_sz, c_vp]),
    "nsa_selected_attn_bwd_workspace_size": (c_sz, [c_i32] * 6),
    "nsa_selected_attn_bwd_workspace_size_min": (c_sz, [c_i32] * 6),
    "nsa_selected_attn_bwd": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.c_int,
                                             c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                                             c_i32, c_i32, c_i32, c_f32, c_vp, c_vp, c_vp, c_vp,
                                             c_sz, c_vp]),
    "nsa_branch_attn_bwd_workspace_size": (c_sz, [c_i32, c_i32]),
    "nsa_compressed_attn_bwd": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.c_int,
                                               c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32,
                                               c_i32, c_i32, c_i32, c_f32, c_i32, c_vp, c_vp, c_vp,
                                               c_vp, c_sz, c_vp]),
    "nsa_window_attn_bwd": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.c_int, c_vp,
                                           c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                           c_f32, c_i32, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "nsa_compress_bwd": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32,
                                        c_i32, c_i32, c_vp]),
    "nsa_gates_bwd": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, ctypes.c_int, c_vp, c_i32, c_i32,
                                     c_i32, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "nsa_decode_workspace_size": (c_sz, [ctypes.POINTER(DecodeParams)]),
    "nsa_decode_step": (ctypes.c_int, [ctypes.POINTER(DecodeParams), c_vp, c_sz, c_vp]),
    "nsa_decode_noalloc_scratch_bytes": (c_sz, []),
    "nsa_decode_step_noalloc": (ctypes.c_int, [ctypes.POINTER(DecodeParams), c_vp]),
    "nsa_offload_pool_bytes": (c_sz, [c_i32, c_i32, c_i32, c_i32, ctypes.c_int]),
    "nsa_offload_reset": (ctypes.c_int, [ctypes.POINTER(OffloadState), c_i32, c_i32, c_vp]),
    "nsa_decode_offload_workspace_size": (c_sz, [ctypes.POINTER(DecodeParams),
                                                 ctypes.POINTER(OffloadState)]),
    "nsa_decode_step_offload": (ctypes.c_int, [ctypes.POINTER(DecodeParams),
                                               ctypes.POINTER(OffloadState), c_vp, c_sz, c_vp]),
    "nsa_compressed_attn_workspace_size": (c_sz, [c_i32] * 7),
    "nsa_window_attn_workspace_size": (c_sz, [c_i32] * 3),
    "nsa_blockmask_attn_workspace_size": (c_sz, [c_i32] * 3),
    "nsa_blockmask_attn_fwd": (ctypes.c_int, [c_vp, c_vp, c_vp, ctypes.c_int, c_vp, c_i32, c_vp,
                                              c_vp, c_i32, c_i32, c_i32, c_i32, c_f32, c_vp, c_sz,
                                              c_vp]),
    "nsa_compressed_attn_fwd": (ctypes.c_int, [c_vp, c_vp, c_vp, ctypes.c_int, c_vp, ctypes.c_int,
                                               c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_i32, c_i32,
                                               c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                               c_f32, c_vp, c_sz, c_vp]),
    "nsa_window_attn_fwd": (ctypes.c_int, [c_vp, c_vp, c_vp, ctypes.c_int, c_vp, ctypes.c_int,
                                           c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32,
                                           c_i32, c_i32, c_f32, c_vp, c_sz, c_vp]),
    "nsa_prefill_workspace_size": (c_sz, [ctypes.POINTER(PrefillParams)]),
    "nsa_prefill_workspace_size_min": (c_sz, [ctypes.POINTER(PrefillParams)]),
    "nsa_prefill_step": (ctypes.c_int, [ctypes.POINTER(PrefillParams), c_vp, c_sz, c_vp]),
}


def lib():
    """The loaded libnsa (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m sparse_attention_compress_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().nsa_last_error().decode()


def _check(status: int):
    if status != 0:
        raise NsaError(status, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dt(t) -> int:
    if t.dtype == torch.bfloat16:
        return NSA_BF16
    if t.dtype == torch.float32:
        return NSA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


_ws_cache: dict = {}


def _workspace(nbytes: int, device, workspace=None):
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        return workspace, workspace.numel() * workspace.element_size()
    key = (str(device), nbytes)
    buf = _ws_cache.get(key)
    if buf is None:
        buf = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf, nbytes


# ----------------------------------------------------------------------------- host helpers


def window_count(length: int, kernel: int = 32, stride: int = 16, tail: bool = False) -> int:
    """Window count of one sequence (nsa_window_count): full windows, or with
    ``tail`` the windows that cover every token."""
    n = lib().nsa_window_count(int(length), int(kernel), int(stride), int(bool(tail)))
    if n < 0:
        raise NsaError(1, f"nsa_window_count: invalid arguments ({length}, {kernel}, {stride})")
    return n


def set_debug_checks(on: bool) -> bool:
    """Debug mode (nsa_set_debug_checks): device checks of the preconditions
    before every call, which then synchronises.  Returns the previous setting."""
    return bool(lib().nsa_set_debug_checks(int(bool(on))))


def cu_seqlens_of(lengths, device) -> torch.Tensor:
    out = [0]
    for L in lengths:
        out.append(out[-1] + int(L))
    return torch.tensor(out, dtype=torch.int32, device=device)


# ----------------------------------------------------------------------------- entry points


def nsa_compress_k(x, x_c, cu_seqlens, cu_seqlens_c, max_windows, kernel=32, stride=16, stream=None):
    """x [N, heads, D] -> x_c [N_c, heads, D] (window means)."""
    heads, head_dim = x.shape[1], x.shape[2]
    _check(lib().nsa_compress_k(_ptr(x), _dt(x), _ptr(x_c), _dt(x_c), _ptr(cu_seqlens),
                                _ptr(cu_seqlens_c), cu_seqlens.numel() - 1, int(max_windows), heads,
                                head_dim, kernel, stride, _stream(stream)))
    return x_c


def nsa_cis_mean_pool_varlen(cis, cis_pooled, cu_seqlens, cu_seqlens_c, max_windows, kernel=32,
                             stride=16, stream=None):
    """cis [N, heads] float32 -> cis_pooled [N_c, heads] float32."""
    heads = cis.shape[1] if cis.dim() == 2 else 1
    _check(lib().nsa_cis_mean_pool_varlen(_ptr(cis), _ptr(cis_pooled), _ptr(cu_seqlens),
                                          _ptr(cu_seqlens_c), cu_seqlens.numel() - 1,
                                          int(max_windows), heads, kernel, stride, _stream(stream)))
    return cis_pooled


def compressed_scores_workspace_size(batch, max_seqlen_k, heads, kv_heads, kernel=32, stride=16):
    return lib().nsa_compressed_scores_workspace_size(batch, max_seqlen_k, heads, kv_heads, kernel,
                                                      stride)


def nsa_compressed_scores(q, k_c, cu_seqlens_k, cu_seqlens_c, max_seqlen_k, block_scores,
                          window_probs=None, cis_pooled=None, cis_weight=1.0, softmax_scale=0.0,
                          kernel=32, stride=16, block_size=64, workspace=None, stream=None):
    """Decode queries q [B, H, D] against k_c [N_c, H_kv, D] -> block_scores [B, H_kv, nb_max]."""
    B, H, D = q.shape
    H_kv = k_c.shape[1]
    need = compressed_scores_workspace_size(B, max_seqlen_k, H, H_kv, kernel, stride)
    ws, nbytes = _workspace(need, q.device, workspace)
    _check(lib().nsa_compressed_scores(_ptr(q), _dt(q), _ptr(k_c), _dt(k_c), _ptr(cis_pooled),
                                       float(cis_weight), _ptr(block_scores), _ptr(window_probs),
                                       _ptr(cu_seqlens_k), _ptr(cu_seqlens_c), B, int(max_seqlen_k),
                                       H, H_kv, D, kernel, stride, block_size, float(softmax_scale),
                                       _ptr(ws), nbytes, _stream(stream)))
    return block_scores


def nsa_select_topk(block_scores, indices, cu_seqlens_k, max_seqlen_k, k, n_init=0, n_local=0,
                    cu_seqlens_q=None, block_size=64, stream=None):
    """block_scores [rows, H_kv, nb_max] -> indices [rows, H_kv, k] (ascending, -1 padded)."""
    rows, H_kv, nb_max = block_scores.shape
    batch = cu_seqlens_k.numel() - 1
    _check(lib().nsa_select_topk(_ptr(block_scores), _ptr(indices), _ptr(cu_seqlens_q),
                                 _ptr(cu_seqlens_k), batch, rows, int(max_seqlen_k), H_kv, nb_max,
                                 int(k), int(n_init), int(n_local), block_size, _stream(stream)))
    return indices


def selected_attn_workspace_size(rows, heads, kv_heads, head_dim, k_sel, decode):
    return lib().nsa_selected_attn_workspace_size(rows, heads, kv_heads, head_dim, k_sel, int(decode))


def nsa_selected_attn_fwd(q, k, v, indices, cu_seqlens_k, max_seqlen_k, out, cis=None, lse=None,
                          cu_seqlens_q=None, softmax_scale=0.0, block_size=64, workspace=None,
                          stream=None):
    """q [rows, H, D]; k, v [N_k, H_kv, D]; indices [rows, H_kv, k_sel] -> out [rows, H, D]."""
    rows, H, D = q.shape
    H_kv = k.shape[1]
    k_sel = indices.shape[2]
    batch = cu_seqlens_k.numel() - 1
    decode = cu_seqlens_q is None
    need = selected_attn_workspace_size(rows, H, H_kv, D, k_sel, decode)
    ws, nbytes = _workspace(need, q.device, workspace)
    _check(lib().nsa_selected_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _dt(q), _ptr(indices), k_sel,
                                       _ptr(cis), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
                                       _ptr(cu_seqlens_k), batch, rows, int(max_seqlen_k), H, H_kv,
                                       D, block_size, float(softmax_scale), _ptr(ws), nbytes,
                                       _stream(stream)))
    return out


def selected_attn_bwd_workspace_size(batch, rows, max_seqlen_k, heads, kv_heads, k_sel):
    """Workspace bytes of the selected backward with the key-block dq."""
    return lib().nsa_selected_attn_bwd_workspace_size(int(batch), int(rows), int(max_seqlen_k),
                                                      int(heads), int(kv_heads), int(k_sel))


def selected_attn_bwd_workspace_size_min(batch, rows, max_seqlen_k, heads, kv_heads, k_sel):
    """Smallest workspace of the selected backward (dq one workgroup per (row, KV head))."""
    return lib().nsa_selected_attn_bwd_workspace_size_min(int(batch), int(rows), int(max_seqlen_k),
                                                          int(heads), int(kv_heads), int(k_sel))


def nsa_selected_attn_bwd(q, k, v, out, d_out, lse, indices, cu_seqlens_q, cu_seqlens_k,
                          max_seqlen_k, dq, dk, dv, softmax_scale=0.0, block_size=64,
                          workspace=None, stream=None):
    """Gradient of nsa_selected_attn_fwd (no CIS) over prefill rows: q, out, d_out
    [rows, H, D] bf16, k, v [N_k, H_kv, D] bf16, lse [rows, H] float32 from the
    forward -> dq [rows, H, D], dk, dv [N_k, H_kv, D] float32."""
    rows, H, D = q.shape
    H_kv = k.shape[1]
    k_sel = indices.shape[2]
    batch = cu_seqlens_k.numel() - 1
    need = selected_attn_bwd_workspace_size(batch, rows, max_seqlen_k, H, H_kv, k_sel)
    ws, nbytes = _workspace(need, q.device, workspace)
    _check(lib().nsa_selected_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(d_out),
                                       _ptr(lse), _dt(q), _ptr(indices), k_sel,
                                       _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), batch, rows,
                                       int(max_seqlen_k), H, H_kv, D, block_size,
                                       float(softmax_scale), _ptr(dq), _ptr(dk), _ptr(dv),
                                       _ptr(ws), nbytes, _stream(stream)))
    return dq, dk, dv


def branch_attn_bwd_workspace_size(rows, heads):
    return lib().nsa_branch_attn_bwd_workspace_size(int(rows), int(heads))


def _acc_bits(accumulate):
    """accumulate: False/True (both bits), or an int (bit 0: dq, bit 1: key and
    value gradients)."""
    if isinstance(accumulate, bool):
        return 3 if accumulate else 0
    return int(accumulate)


def nsa_gates_bwd(d_out, o_cmp, o_sel, o_win, gates, do_cmp, do_sel, do_win, d_gates,
                  stream=None):
    """Gradients of the gated three-branch sum: per-branch output gradients
    g_b * d_out (bf16) and d_gates = d_out . o_b (float32 [rows, H, 3])."""
    rows, H, D = d_out.shape
    _check(lib().nsa_gates_bwd(_ptr(d_out), _ptr(o_cmp), _ptr(o_sel), _ptr(o_win), _dt(d_out),
                               _ptr(gates), rows, H, D, _ptr(do_cmp), _ptr(do_sel), _ptr(do_win),
                               _ptr(d_gates), _stream(stream)))
    return do_cmp, do_sel, do_win, d_gates


def nsa_compressed_attn_bwd(q, k_c, v_c, o_cmp, d_out, lse, cu_seqlens_q, cu_seqlens_k,
                            cu_seqlens_c, max_seqlen_k, dq, dk_c, dv_c, accumulate=False,
                            softmax_scale=0.0, kernel=32, stride=16, workspace=None, stream=None):
    """Gradient of nsa_compressed_attn_fwd: q, o_cmp, d_out [rows, H, D] bf16, k_c,
    v_c [N_c, H_kv, D] bf16, lse [rows, H] -> dq [rows, H, D], dk_c, dv_c
    [N_c, H_kv, D] float32 (written, or added to with accumulate)."""
    rows, H, D = q.shape
    H_kv = k_c.shape[1]
    batch = cu_seqlens_k.numel() - 1
    ws, nbytes = _workspace(branch_attn_bwd_workspace_size(rows, H), q.device, workspace)
    _check(lib().nsa_compressed_attn_bwd(_ptr(q), _ptr(k_c), _ptr(v_c), _ptr(o_cmp), _ptr(d_out),
                                         _ptr(lse), _dt(q), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                                         _ptr(cu_seqlens_c), batch, rows, int(max_seqlen_k), H,
                                         H_kv, D, kernel, stride, float(softmax_scale),
                                         _acc_bits(accumulate), _ptr(dq), _ptr(dk_c), _ptr(dv_c),
                                         _ptr(ws), nbytes, _stream(stream)))
    return dq, dk_c, dv_c


def nsa_window_attn_bwd(q, k, v, out, d_out, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_k, dq,
                        dk, dv, window=512, accumulate=False, softmax_scale=0.0, workspace=None,
                        stream=None):
    """Gradient of nsa_window_attn_fwd -> dq [rows, H, D], dk, dv [N_k, H_kv, D] float32."""
    rows, H, D = q.shape
    H_kv = k.shape[1]
    batch = cu_seqlens_k.numel() - 1
    ws, nbytes = _workspace(branch_attn_bwd_workspace_size(rows, H), q.device, workspace)
    _check(lib().nsa_window_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(d_out), _ptr(lse),
                                     _dt(q), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), batch, rows,
                                     int(max_seqlen_k), H, H_kv, D, int(window),
                                     float(softmax_scale), _acc_bits(accumulate), _ptr(dq),
                                     _ptr(dk), _ptr(dv), _ptr(ws), nbytes, _stream(stream)))
    return dq, dk, dv


def nsa_compress_bwd(dx_c, dx, cu_seqlens, cu_seqlens_c, max_seqlen, accumulate=False, kernel=32,
                     stride=16, stream=None):
    """Transpose of nsa_compress_k (float32): dx_c [N_c, heads, D] -> dx [N, heads, D]."""
    heads, head_dim = dx.shape[1], dx.shape[2]
    _check(lib().nsa_compress_bwd(_ptr(dx_c), _ptr(dx), _ptr(cu_seqlens), _ptr(cu_seqlens_c),
                                  cu_seqlens.numel() - 1, int(max_seqlen), heads, head_dim, kernel,
                                  stride, int(bool(accumulate)), _stream(stream)))
    return dx


def decode_params(q, k, v, k_c, cu_seqlens_k, cu_seqlens_c, max_seqlen_k, out, topk=64, n_init=1,
                  n_local=16, cis=None, cis_pooled=None, cis_weight=1.0, cis_values=False,
                  append_window=False, block_scores=None, indices=None, softmax_scale=0.0,
                  kernel=32, stride=16, block_size=64, n_cand=0) -> DecodeParams:
    B, H, D = q.shape
    p = DecodeParams()
    p.q, p.k, p.v, p.k_c = q.data_ptr(), k.data_ptr(), v.data_ptr(), k_c.data_ptr()
    p.cis = cis.data_ptr() if cis is not None else None
    p.cis_pooled = cis_pooled.data_ptr() if cis_pooled is not None else None
    p.cu_seqlens_k, p.cu_seqlens_c = cu_seqlens_k.data_ptr(), cu_seqlens_c.data_ptr()
    p.out = out.data_ptr()
    p.block_scores = block_scores.data_ptr() if block_scores is not None else None
    p.indices = indices.data_ptr() if indices is not None else None
    p.dtype, p.kc_dtype = _dt(q), _dt(k_c)
    p.batch, p.max_seqlen_k, p.heads, p.kv_heads, p.head_dim = B, int(max_seqlen_k), H, k.shape[1], D
    p.kernel, p.stride, p.block_size = kernel, stride, block_size
    p.topk, p.n_init, p.n_local = int(topk), int(n_init), int(n_local)
    p.cis_weight = float(cis_weight)
    p.cis_values = int(bool(cis_values))
    p.append_window = int(bool(append_window))
    p.softmax_scale = float(softmax_scale)
    p.n_cand = int(n_cand)
    return p


def decode_workspace_size(params: DecodeParams) -> int:
    return lib().nsa_decode_workspace_size(ctypes.byref(params))


def nsa_decode_step(params: DecodeParams, workspace=None, device=None, stream=None):
    """Enqueue one decode step described by ``params`` (see :func:`decode_params`)."""
    need = decode_workspace_size(params)
    ws, nbytes = _workspace(need, device or torch.device("cuda"), workspace)
    _check(lib().nsa_decode_step(ctypes.byref(params), _ptr(ws), nbytes, _stream(stream)))


def decode_noalloc_scratch_bytes() -> int:
    return lib().nsa_decode_noalloc_scratch_bytes()


def nsa_decode_step_noalloc(params: DecodeParams, stream=None):
    """Enqueue one decode step whose workspace is the library's fixed per-GPU
    scratch (no allocation by the library or by this binding)."""
    _check(lib().nsa_decode_step_noalloc(ctypes.byref(params), _stream(stream)))


def offload_state(batch, kv_heads, pool_slots, nb_cap, device, head_dim=128, dtype=torch.bfloat16,
                  with_fetched=True):
    """Allocate (with torch) the device pools and tables of ``nsa_offload_state`` and
    reset them; returns (state, tensors) where tensors keeps the allocations alive."""
    units = batch * kv_heads
    t = dict(k_pool=torch.empty((units, pool_slots, 64, head_dim), dtype=dtype, device=device),
             v_pool=torch.empty((units, pool_slots, 64, head_dim), dtype=dtype, device=device),
             slot_of=torch.empty((units, nb_cap), dtype=torch.int32, device=device),
             block_of=torch.empty((units, pool_slots), dtype=torch.int32, device=device))
    if with_fetched:
        t["fetched"] = torch.zeros(units, dtype=torch.int32, device=device)
    st = OffloadState()
    st.k_pool, st.v_pool = t["k_pool"].data_ptr(), t["v_pool"].data_ptr()
    st.slot_of, st.block_of = t["slot_of"].data_ptr(), t["block_of"].data_ptr()
    st.fetched = t["fetched"].data_ptr() if with_fetched else None
    st.pool_slots, st.nb_cap = int(pool_slots), int(nb_cap)
    nsa_offload_reset(st, batch, kv_heads)
    return st, t


def nsa_offload_reset(state: OffloadState, batch, kv_heads, stream=None):
    _check(lib().nsa_offload_reset(ctypes.byref(state), int(batch), int(kv_heads), _stream(stream)))


def decode_offload_workspace_size(params: DecodeParams, state: OffloadState) -> int:
    return lib().nsa_decode_offload_workspace_size(ctypes.byref(params), ctypes.byref(state))


def nsa_decode_step_offload(params: DecodeParams, state: OffloadState, workspace=None, device=None,
                            stream=None):
    """Enqueue one decode step whose K/V (params.k, params.v) live in pinned host memory."""
    need = decode_offload_workspace_size(params, state)
    ws, nbytes = _workspace(need, device or torch.device("cuda"), workspace)
    _check(lib().nsa_decode_step_offload(ctypes.byref(params), ctypes.byref(state), _ptr(ws),
                                         nbytes, _stream(stream)))


KERNEL_POOL, KERNEL_LOGITS, KERNEL_BLOCK_SCORES, KERNEL_SELECTED_ATTN, KERNEL_COMBINE = 0, 1, 2, 3, 4
KERNEL_COMPRESSED_LSE, KERNEL_COMPRESSED_ATTN, KERNEL_WINDOW_ATTN, KERNEL_FETCH = 5, 6, 7, 8
KERNEL_BLOCKMASK_ATTN = 9
KERNEL_SELECTED_BWD_DQ, KERNEL_SELECTED_BWD_DKDV, KERNEL_SELECTED_BWD_LISTS = 10, 11, 12
KERNEL_SELECTED_BWD_DQ_SUM = 13
KERNEL_BLOCK_LISTS = 14


def blockmask_attn_workspace_size(batch, max_seqlen, heads):
    return lib().nsa_blockmask_attn_workspace_size(int(batch), int(max_seqlen), int(heads))


def nsa_blockmask_attn_fwd(q, k, v, mask, cu_seqlens, max_seqlen, out, causal=False,
                           softmax_scale=0.0, workspace=None, stream=None):
    """q, k, v, out [N, H, 128] bf16; mask [B, H, nb, nb] uint8, nb = ceil(max_seqlen / 64)."""
    N, H, D = q.shape
    batch = cu_seqlens.numel() - 1
    need = blockmask_attn_workspace_size(batch, max_seqlen, H)
    ws, nbytes = _workspace(need, q.device, workspace)
    _check(lib().nsa_blockmask_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _dt(q), _ptr(mask),
                                        int(bool(causal)), _ptr(out), _ptr(cu_seqlens), batch,
                                        int(max_seqlen), H, D, float(softmax_scale), _ptr(ws),
                                        nbytes, _stream(stream)))
    return out


def compressed_attn_workspace_size(batch, rows, max_seqlen_k, heads, kv_heads, kernel=32, stride=16):
    return lib().nsa_compressed_attn_workspace_size(int(batch), int(rows), int(max_seqlen_k),
                                                    int(heads), int(kv_heads), kernel, stride)


def window_attn_workspace_size(batch, max_seqlen_k, kv_heads):
    return lib().nsa_window_attn_workspace_size(int(batch), int(max_seqlen_k), int(kv_heads))


def nsa_compressed_attn_fwd(q, k_c, v_c, cu_seqlens_q, cu_seqlens_k, cu_seqlens_c, max_seqlen_k,
                            o_cmp, lse=None, block_scores=None, softmax_scale=0.0, kernel=32,
                            stride=16, block_size=64, workspace=None, stream=None):
    """Compressed-branch attention of prefill rows: q [rows, H, D] bf16, k_c/v_c
    [N_c, H_kv, D] bf16 -> o_cmp [rows, H, D] (bf16 or fp32); optional lse
    [rows, H] and block_scores [rows, H_kv, n_blocks_max]."""
    rows, H, D = q.shape
    H_kv = k_c.shape[1]
    batch = cu_seqlens_k.numel() - 1
    nb_max = block_scores.shape[2] if block_scores is not None else 0
    need = compressed_attn_workspace_size(batch, rows, max_seqlen_k, H, H_kv, kernel, stride)
    ws, nbytes = _workspace(need, q.device, workspace)
    _check(lib().nsa_compressed_attn_fwd(_ptr(q), _ptr(k_c), _ptr(v_c), _dt(q), _ptr(o_cmp),
                                         _dt(o_cmp), _ptr(lse), _ptr(block_scores), nb_max,
                                         _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(cu_seqlens_c),
                                         batch, rows, int(max_seqlen_k), H, H_kv, D, kernel,
                                         stride, block_size, float(softmax_scale), _ptr(ws),
                                         nbytes, _stream(stream)))
    return o_cmp


def nsa_window_attn_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_k, out, window=512,
                        lse=None, softmax_scale=0.0, workspace=None, stream=None):
    """Sliding-window attention of prefill rows over keys t-window+1 .. t."""
    rows, H, D = q.shape
    H_kv = k.shape[1]
    batch = cu_seqlens_k.numel() - 1
    ws, nbytes = _workspace(window_attn_workspace_size(batch, max_seqlen_k, H_kv), q.device, workspace)
    _check(lib().nsa_window_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _dt(q), _ptr(out), _dt(out),
                                     _ptr(lse), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), batch, rows,
                                     int(max_seqlen_k), H, H_kv, D, int(window),
                                     float(softmax_scale), _ptr(ws), nbytes, _stream(stream)))
    return out


def prefill_params(q, k, v, k_c, v_c, gates, cu_seqlens_q, cu_seqlens_k, cu_seqlens_c,
                   max_seqlen_k, out, topk=16, n_init=0, n_local=0, window=512,
                   block_scores=None, indices=None, softmax_scale=0.0, kernel=32, stride=16,
                   block_size=64) -> PrefillParams:
    rows, H, D = q.shape
    p = PrefillParams()
    p.q, p.k, p.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    p.k_c, p.v_c, p.gates = k_c.data_ptr(), v_c.data_ptr(), gates.data_ptr()
    p.cu_seqlens_q, p.cu_seqlens_k = cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr()
    p.cu_seqlens_c, p.out = cu_seqlens_c.data_ptr(), out.data_ptr()
    p.block_scores = block_scores.data_ptr() if block_scores is not None else None
    p.indices = indices.data_ptr() if indices is not None else None
    p.dtype = _dt(q)
    p.batch, p.rows_total, p.max_seqlen_k = cu_seqlens_k.numel() - 1, rows, int(max_seqlen_k)
    p.heads, p.kv_heads, p.head_dim = H, k.shape[1], D
    p.kernel, p.stride, p.block_size = kernel, stride, block_size
    p.topk, p.n_init, p.n_local, p.window = int(topk), int(n_init), int(n_local), int(window)
    p.softmax_scale = float(softmax_scale)
    return p


def prefill_workspace_size(params: PrefillParams) -> int:
    """Workspace bytes of the prefill step with the key-block selected branch."""
    return lib().nsa_prefill_workspace_size(ctypes.byref(params))


def prefill_workspace_size_min(params: PrefillParams) -> int:
    """Smallest workspace of the prefill step (row-by-row selected branch)."""
    return lib().nsa_prefill_workspace_size_min(ctypes.byref(params))


def nsa_prefill_step(params: PrefillParams, workspace=None, device=None, stream=None):
    """Enqueue the three-branch prefill described by ``params`` (see :func:`prefill_params`)."""
    need = prefill_workspace_size(params)
    ws, nbytes = _workspace(need, device or torch.device("cuda"), workspace)
    _check(lib().nsa_prefill_step(ctypes.byref(params), _ptr(ws), nbytes, _stream(stream)))


def nsa_profile_next_launch(kind: int, start: torch.cuda.Event, stop: torch.cuda.Event):
    """Arm the next launch of one kernel kind to record the two (timing) events at
    the kernel's own start and end.  The events must already exist (recorded once)."""
    _check(lib().nsa_profile_next_launch(int(kind), ctypes.c_void_p(start.cuda_event),
                                         ctypes.c_void_p(stop.cuda_event)))


def softmax_scale_default(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
