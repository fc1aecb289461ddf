"""Thin ctypes binding of ``libev.so`` (the C ABI in include/ev.h).

Argument marshalling only: every step of the verification path runs in the library's HIP
kernels.  The ``ev_*`` functions mirror the C entry points one to one (integer device
addresses, sizes, a HIP stream handle).  The lower-case helpers accept torch tensors that
live on a ROCm device, check shapes/dtypes/contiguity, allocate outputs and workspaces with
torch and call the matching ``ev_*`` function on the current torch stream.

There is no fallback: if the library is missing, importing the helpers raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libev.so")

EV_BF16, EV_F32 = 0, 1
EV_OK = 0
STATUS = {0: "EV_OK", 1: "EV_ERR_NULL", 2: "EV_ERR_SHAPE", 3: "EV_ERR_DTYPE", 4: "EV_ERR_ALIGN",
          5: "EV_ERR_WORKSPACE", 6: "EV_ERR_DEVICE", 7: "EV_ERR_HIP"}
DATA_BAD_PARENT, DATA_BAD_NODES, DATA_BAD_TOKEN, DATA_BAD_SLOTS, DATA_BAD_PATH = 1, 2, 4, 8, 16
MAX_NODES = 64
MAX_BATCH = 2048

EXPORTS = ("ev_status_string", "ev_tree_attention_workspace_size", "ev_tree_attention",
           "ev_tree_attention_window", "ev_tree_attention_paged", "ev_node_argmax_workspace_size",
           "ev_node_argmax", "ev_node_sample", "ev_greedy_accept", "ev_sampled_accept", "ev_compact_kv",
           "ev_compact_kv_paged",
           "ev_select_workspace_size", "ev_select_accept_compact", "ev_select_accept_compact_paged",
           "ev_stream_read", "ev_tree_attention_noalloc", "ev_tree_attention_strided",
           "ev_verify_step_workspace_size", "ev_verify_step")

_lib = None
_P, _I32, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class EvError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}")
        self.status = status


def load(path: str = LIB_PATH):
    """Load libev.so (built by draft_tree_verification_amd.build); raise if it is absent."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m draft_tree_verification_amd.build` "
                           "(there is no non-HIP fallback)")
    # torch first (when installed): loaded the other way round, the library binds a second copy of
    # the HIP runtime and every call reports EV_ERR_DEVICE on the GPU
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    lib.ev_status_string.restype = ctypes.c_char_p
    lib.ev_status_string.argtypes = [ctypes.c_int]
    lib.ev_tree_attention_workspace_size.restype = _SZ
    lib.ev_tree_attention_workspace_size.argtypes = [_I32, _I32, _I32, _I32, _I32]
    lib.ev_tree_attention.restype = ctypes.c_int
    lib.ev_tree_attention.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32, _I32,
                                      _I32, ctypes.c_int, _F, _P, _SZ, _P, _P]
    lib.ev_tree_attention_window.restype = ctypes.c_int
    lib.ev_tree_attention_window.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32,
                                             _I32, _I32, ctypes.c_int, _F, _I32, _P, _SZ, _P, _P]
    lib.ev_tree_attention_paged.restype = ctypes.c_int
    lib.ev_tree_attention_paged.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _P, _I32, _I32, _I32, _I32,
                                            _I32, _I32, _I32, ctypes.c_int, _F, _I32, _P, _SZ, _P, _P]
    lib.ev_node_argmax_workspace_size.restype = _SZ
    lib.ev_node_argmax_workspace_size.argtypes = [_I32, _I32]
    lib.ev_node_argmax.restype = ctypes.c_int
    lib.ev_node_argmax.argtypes = [_P, ctypes.c_int, _I64, _I32, _I32, _P, _P, _P, _SZ, _P]
    lib.ev_node_sample.restype = ctypes.c_int
    lib.ev_node_sample.argtypes = [_P, ctypes.c_int, _I64, _I32, _I32, _F, ctypes.c_uint64, ctypes.c_uint64, _P, _P,
                                   _SZ, _P]
    lib.ev_greedy_accept.restype = ctypes.c_int
    lib.ev_greedy_accept.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P]
    lib.ev_sampled_accept.restype = ctypes.c_int
    lib.ev_sampled_accept.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P]
    lib.ev_compact_kv.restype = ctypes.c_int
    lib.ev_compact_kv.argtypes = [_P, _P, _I32, _I32, _I64, _P, _P, _P, _P, _I32, _I32, _I64, _I32, _I32, _P,
                                  _P, _P]
    lib.ev_compact_kv_paged.restype = ctypes.c_int
    lib.ev_compact_kv_paged.argtypes = [_P, _P, _I32, _I32, _I64, _P, _I32, _I32, _P, _P, _P, _I32, _I32, _I32, _I32,
                                        _I32, _P, _P, _P]
    _U64 = ctypes.c_uint64
    lib.ev_select_workspace_size.restype = _SZ
    lib.ev_select_workspace_size.argtypes = [_I32, _I32]
    lib.ev_select_accept_compact.restype = ctypes.c_int
    lib.ev_select_accept_compact.argtypes = [_P, ctypes.c_int, _I64, _I32, _F, _U64, _U64, _P, _P, _P, _I32, _I32,
                                             _I32, _P, _P, _I32, _I32, _I64, _P, _P, _I64, _I32, _I32, _P, _P, _P,
                                             _P, _P, _P, _P, _SZ, _P, _P]
    lib.ev_select_accept_compact_paged.restype = ctypes.c_int
    lib.ev_select_accept_compact_paged.argtypes = [_P, ctypes.c_int, _I64, _I32, _F, _U64, _U64, _P, _P, _P, _I32,
                                                   _I32, _I32, _P, _P, _I32, _I32, _I64, _P, _I32, _I32, _P, _I32,
                                                   _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _P]
    lib.ev_tree_attention_strided.restype = ctypes.c_int
    lib.ev_tree_attention_strided.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32,
                                              _I32, _I32, _I64, _I64, ctypes.c_int, _F, _P, _SZ, _P, _P]
    lib.ev_tree_attention_noalloc.restype = ctypes.c_int
    lib.ev_tree_attention_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32,
                                              _I32, _I32, ctypes.c_int, _F, _P, _P]
    lib.ev_stream_read.restype = ctypes.c_int
    lib.ev_stream_read.argtypes = [_P, _SZ, _P, _P]
    lib.ev_verify_step_workspace_size.restype = _SZ
    lib.ev_verify_step_workspace_size.argtypes = [_I32, _I32, _I32, _I32, _I32, _I32, _I32]
    lib.ev_verify_step.restype = ctypes.c_int
    lib.ev_verify_step.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32, _I32, _I32,
                                   _I64, _I64, ctypes.c_int, _F, _P, ctypes.c_int, _I64, _I32, _F, _U64, _U64, _P,
                                   _I32, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _P]
    if path == LIB_PATH:
        _lib = lib
    return lib


# ------------------------------------------------------------------------------ raw C entry points
def ev_status_string(status: int) -> str:
    return load().ev_status_string(status).decode()


def ev_tree_attention_workspace_size(batch, max_nodes, num_q_heads, num_kv_heads, head_dim) -> int:
    return int(load().ev_tree_attention_workspace_size(batch, max_nodes, num_q_heads, num_kv_heads, head_dim))


def ev_tree_attention(q, k_cache, v_cache, out, lse, node_start, parent, kv_start, prefix_len, batch, total_nodes,
                      max_nodes, total_slots, num_q_heads, num_kv_heads, head_dim, dtype, sm_scale, workspace,
                      workspace_bytes, err_flag, stream) -> int:
    return load().ev_tree_attention(q, k_cache, v_cache, out, lse, node_start, parent, kv_start, prefix_len, batch,
                                    total_nodes, max_nodes, total_slots, num_q_heads, num_kv_heads, head_dim, dtype,
                                    sm_scale, workspace, workspace_bytes, err_flag, stream)


def ev_tree_attention_noalloc(q, k_cache, v_cache, out, lse, node_start, parent, kv_start, prefix_len, batch,
                              total_nodes, max_nodes, total_slots, num_q_heads, num_kv_heads, head_dim, dtype,
                              sm_scale, err_flag, stream) -> int:
    return load().ev_tree_attention_noalloc(q, k_cache, v_cache, out, lse, node_start, parent, kv_start, prefix_len,
                                            batch, total_nodes, max_nodes, total_slots, num_q_heads, num_kv_heads,
                                            head_dim, dtype, sm_scale, err_flag, stream)


def ev_tree_attention_strided(q, k_cache, v_cache, out, lse, node_start, parent, kv_start, prefix_len, batch,
                              total_nodes, max_nodes, total_slots, num_q_heads, num_kv_heads, head_dim, kv_slot_stride,
                              kv_head_stride, dtype, sm_scale, workspace, workspace_bytes, err_flag, stream) -> int:
    return load().ev_tree_attention_strided(q, k_cache, v_cache, out, lse, node_start, parent, kv_start, prefix_len,
                                            batch, total_nodes, max_nodes, total_slots, num_q_heads, num_kv_heads,
                                            head_dim, kv_slot_stride, kv_head_stride, dtype, sm_scale, workspace,
                                            workspace_bytes, err_flag, stream)


def ev_tree_attention_window(q, k_cache, v_cache, out, lse, node_start, parent, kv_start, prefix_len, batch,
                             total_nodes, max_nodes, total_slots, num_q_heads, num_kv_heads, head_dim, dtype,
                             sm_scale, window, workspace, workspace_bytes, err_flag, stream) -> int:
    return load().ev_tree_attention_window(q, k_cache, v_cache, out, lse, node_start, parent, kv_start, prefix_len,
                                           batch, total_nodes, max_nodes, total_slots, num_q_heads, num_kv_heads,
                                           head_dim, dtype, sm_scale, window, workspace, workspace_bytes, err_flag,
                                           stream)


def ev_tree_attention_paged(q, k_pages, v_pages, out, lse, node_start, parent, block_table, bt_stride, page_size,
                            prefix_len, batch, total_nodes, max_nodes, num_pages, num_q_heads, num_kv_heads, head_dim,
                            dtype, sm_scale, window, workspace, workspace_bytes, err_flag, stream) -> int:
    return load().ev_tree_attention_paged(q, k_pages, v_pages, out, lse, node_start, parent, block_table, bt_stride,
                                          page_size, prefix_len, batch, total_nodes, max_nodes, num_pages,
                                          num_q_heads, num_kv_heads, head_dim, dtype, sm_scale, window, workspace,
                                          workspace_bytes, err_flag, stream)


def ev_compact_kv_paged(k_pages, v_pages, elem_bytes, num_layers, layer_stride_bytes, block_table, bt_stride,
                        page_size, prefix_len, accept_len, accept_path, batch, max_nodes, num_pages, num_kv_heads,
                        head_dim, new_len, err_flag, stream) -> int:
    return load().ev_compact_kv_paged(k_pages, v_pages, elem_bytes, num_layers, layer_stride_bytes, block_table,
                                      bt_stride, page_size, prefix_len, accept_len, accept_path, batch, max_nodes,
                                      num_pages, num_kv_heads, head_dim, new_len, err_flag, stream)


def ev_node_argmax_workspace_size(num_rows, vocab) -> int:
    return int(load().ev_node_argmax_workspace_size(num_rows, vocab))


def ev_node_argmax(logits, dtype, row_stride, num_rows, vocab, target_token, max_value, workspace, workspace_bytes,
                   stream) -> int:
    return load().ev_node_argmax(logits, dtype, row_stride, num_rows, vocab, target_token, max_value, workspace,
                                 workspace_bytes, stream)


def ev_node_sample(logits, dtype, row_stride, num_rows, vocab, temperature, seed, offset, target_token, workspace,
                   workspace_bytes, stream) -> int:
    return load().ev_node_sample(logits, dtype, row_stride, num_rows, vocab, temperature, seed, offset, target_token,
                                 workspace, workspace_bytes, stream)


def ev_greedy_accept(node_start, parent, draft_token, target_token, batch, total_nodes, max_nodes, vocab, accept_len,
                     accept_path, bonus_token, out_tokens, err_flag, stream) -> int:
    return load().ev_greedy_accept(node_start, parent, draft_token, target_token, batch, total_nodes, max_nodes,
                                   vocab, accept_len, accept_path, bonus_token, out_tokens, err_flag, stream)


def ev_sampled_accept(node_start, parent, draft_token, target_token, batch, total_nodes, max_nodes, vocab, accept_len,
                     accept_path, bonus_token, out_tokens, err_flag, stream) -> int:
    return load().ev_sampled_accept(node_start, parent, draft_token, target_token, batch, total_nodes, max_nodes,
                                   vocab, accept_len, accept_path, bonus_token, out_tokens, err_flag, stream)


def ev_compact_kv(k_cache, v_cache, elem_bytes, num_layers, layer_stride_bytes, kv_start, prefix_len, accept_len,
                  accept_path, batch, max_nodes, total_slots, num_kv_heads, head_dim, new_len, err_flag,
                  stream) -> int:
    return load().ev_compact_kv(k_cache, v_cache, elem_bytes, num_layers, layer_stride_bytes, kv_start, prefix_len,
                                accept_len, accept_path, batch, max_nodes, total_slots, num_kv_heads, head_dim,
                                new_len, err_flag, stream)


def ev_select_workspace_size(num_rows, vocab) -> int:
    return int(load().ev_select_workspace_size(num_rows, vocab))


def ev_select_accept_compact(logits, dtype, row_stride, vocab, temperature, seed, offset, node_start, parent,
                             draft_token, batch, total_nodes, max_nodes, k_cache, v_cache, elem_bytes, num_layers,
                             layer_stride_bytes, kv_start, prefix_len, total_slots, num_kv_heads, head_dim,
                             target_token, accept_len, accept_path, bonus_token, out_tokens, new_len, workspace,
                             workspace_bytes, err_flag, stream) -> int:
    return load().ev_select_accept_compact(logits, dtype, row_stride, vocab, temperature, seed, offset, node_start,
                                           parent, draft_token, batch, total_nodes, max_nodes, k_cache, v_cache,
                                           elem_bytes, num_layers, layer_stride_bytes, kv_start, prefix_len,
                                           total_slots, num_kv_heads, head_dim, target_token, accept_len,
                                           accept_path, bonus_token, out_tokens, new_len, workspace,
                                           workspace_bytes, err_flag, stream)


def ev_select_accept_compact_paged(logits, dtype, row_stride, vocab, temperature, seed, offset, node_start, parent,
                                   draft_token, batch, total_nodes, max_nodes, k_pages, v_pages, elem_bytes,
                                   num_layers, layer_stride_bytes, block_table, bt_stride, page_size, prefix_len,
                                   num_pages, num_kv_heads, head_dim, target_token, accept_len, accept_path,
                                   bonus_token, out_tokens, new_len, workspace, workspace_bytes, err_flag,
                                   stream) -> int:
    return load().ev_select_accept_compact_paged(logits, dtype, row_stride, vocab, temperature, seed, offset,
                                                 node_start, parent, draft_token, batch, total_nodes, max_nodes,
                                                 k_pages, v_pages, elem_bytes, num_layers, layer_stride_bytes,
                                                 block_table, bt_stride, page_size, prefix_len, num_pages,
                                                 num_kv_heads, head_dim, target_token, accept_len, accept_path,
                                                 bonus_token, out_tokens, new_len, workspace, workspace_bytes,
                                                 err_flag, stream)


def ev_stream_read(src, nbytes, sink, stream) -> int:
    return load().ev_stream_read(src, nbytes, sink, stream)


def ev_verify_step_workspace_size(batch, total_nodes, max_nodes, num_q_heads, num_kv_heads, head_dim, vocab) -> int:
    return int(load().ev_verify_step_workspace_size(batch, total_nodes, max_nodes, num_q_heads, num_kv_heads,
                                                    head_dim, vocab))


def ev_verify_step(q, k_cache, v_cache, out, lse, node_start, parent, kv_start, prefix_len, batch, total_nodes,
                   max_nodes, total_slots, num_q_heads, num_kv_heads, head_dim, kv_slot_stride, kv_head_stride, dtype,
                   sm_scale, logits, logits_dtype, row_stride, vocab, temperature, seed, offset, draft_token,
                   num_layers, layer_stride_bytes, compact_kv_heads, compact_head_dim, target_token, accept_len,
                   accept_path, bonus_token, out_tokens, new_len, workspace, workspace_bytes, err_flag,
                   stream) -> int:
    return load().ev_verify_step(q, k_cache, v_cache, out, lse, node_start, parent, kv_start, prefix_len, batch,
                                 total_nodes, max_nodes, total_slots, num_q_heads, num_kv_heads, head_dim,
                                 kv_slot_stride, kv_head_stride, dtype, sm_scale, logits, logits_dtype, row_stride,
                                 vocab, temperature, seed, offset, draft_token, num_layers, layer_stride_bytes,
                                 compact_kv_heads, compact_head_dim, target_token, accept_len, accept_path,
                                 bonus_token, out_tokens, new_len, workspace, workspace_bytes, err_flag, stream)


# ------------------------------------------------------------------------------ torch helpers
def _torch():
    import torch
    return torch


def _addr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    torch = _torch()
    return (stream if stream is not None else torch.cuda.current_stream()).cuda_stream


def _check(status: int, where: str):
    if status != EV_OK:
        raise EvError(status, where)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return EV_BF16
    if t.dtype == torch.float32:
        return EV_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _need(t, name, dtype=None, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}; the library launches on the current device "
                         f"cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _need_out(t, name, dtype, shape):
    """A caller-supplied output: contiguous, on the current device, of exactly this dtype and shape
    (the kernels write every element of that shape)."""
    _need(t, name, dtype)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _need_flag(err_flag):
    """The optional device error flag: int32 with at least one element (the first is used)."""
    if err_flag is not None:
        _need(err_flag, "err_flag", _torch().int32)
        if err_flag.numel() < 1:
            raise ValueError("err_flag must hold at least one int32")


def _need_accept(out, B, max_nodes):
    torch = _torch()
    if not isinstance(out, dict):
        raise TypeError("out must be a dict with accept_len, accept_path, bonus and out_tokens")
    for key, shape in (("accept_len", (B,)), ("accept_path", (B, max_nodes)), ("bonus", (B,)),
                       ("out_tokens", (B, max_nodes))):
        if key not in out:
            raise ValueError(f"out lacks {key}")
        _need_out(out[key], key, torch.int32, shape)


class Workspace:
    """A device byte buffer zeroed once at creation and reused across calls on one stream."""

    def __init__(self, nbytes: int, device):
        torch = _torch()
        self.nbytes = int(nbytes)
        self.buf = torch.zeros(max(self.nbytes, 256), dtype=torch.uint8, device=device)

    @property
    def ptr(self):
        return self.buf.data_ptr()


def tree_attention(q, k_cache, v_cache, node_start, parent, kv_start, prefix_len, *, max_nodes: int,
                   sm_scale: float, window: int = None, out=None, lse=None, workspace: Workspace = None,
                   err_flag=None, stream=None, head_major: bool = False):
    """Tree-masked GQA attention (ev_tree_attention; ev_tree_attention_window when `window` is given:
    only the last `window` prefix tokens are visible; ev_tree_attention_strided for head-major
    caches).  q [T, Hq, D]; caches [slots, Hkv, D], or [Hkv, slots, D] with head_major; metadata
    int32.  Returns (out, lse, workspace)."""
    torch = _torch()
    _need(q, "q", ndim=3)
    _need(k_cache, "k_cache", q.dtype, 3)
    _need(v_cache, "v_cache", q.dtype, 3)
    for name, t in (("node_start", node_start), ("parent", parent), ("kv_start", kv_start),
                    ("prefix_len", prefix_len)):
        _need(t, name, torch.int32, 1)
    if head_major and window is not None:
        raise ValueError("the sliding window reads [slots, Hkv, D] caches only")
    T, Hq, D = q.shape
    if head_major:
        Hkv, slots, Dk = k_cache.shape
    else:
        slots, Hkv, Dk = k_cache.shape
    if Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q / k_cache / v_cache shapes disagree")
    B = prefix_len.shape[0]
    if node_start.shape[0] != B + 1 or kv_start.shape[0] != B or parent.shape[0] != T:
        raise ValueError("metadata lengths disagree with batch / total nodes")
    if out is None:
        out = torch.empty_like(q)
    else:
        _need_out(out, "out", q.dtype, q.shape)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    else:
        _need_out(lse, "lse", torch.float32, (T, Hq))
    _need_flag(err_flag)
    need = ev_tree_attention_workspace_size(B, max_nodes, Hq, Hkv, D)
    if workspace is None or workspace.nbytes < need:
        workspace = Workspace(need, q.device)
    ptrs = (_addr(q), _addr(k_cache), _addr(v_cache), _addr(out), _addr(lse), _addr(node_start), _addr(parent),
            _addr(kv_start), _addr(prefix_len), B, T, max_nodes, slots, Hq, Hkv, D, _dtype_code(q), float(sm_scale))
    tail = (workspace.ptr, workspace.nbytes, _addr(err_flag), _stream(stream))
    if head_major:
        _check(ev_tree_attention_strided(*ptrs[:16], D, slots * D, *ptrs[16:], *tail), "ev_tree_attention_strided")
    elif window is None:
        _check(ev_tree_attention(*ptrs, *tail), "ev_tree_attention")
    else:
        _check(ev_tree_attention_window(*ptrs, int(window), *tail), "ev_tree_attention_window")
    return out, lse, workspace


def tree_attention_paged(q, k_pages, v_pages, node_start, parent, block_table, prefix_len, *, max_nodes: int,
                         sm_scale: float, window: int = 0, out=None, lse=None, workspace: Workspace = None,
                         err_flag=None, stream=None):
    """Tree-masked GQA attention over a paged pool (ev_tree_attention_paged).  q [T, Hq, D] bf16;
    pools [pages, page_size, Hkv, D] bf16; block_table [B, stride] int32.  Returns (out, lse, ws)."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, 3)
    _need(k_pages, "k_pages", torch.bfloat16, 4)
    _need(v_pages, "v_pages", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    for name, t in (("node_start", node_start), ("parent", parent), ("prefix_len", prefix_len)):
        _need(t, name, torch.int32, 1)
    T, Hq, D = q.shape
    pages, page_size, Hkv, Dk = k_pages.shape
    if Dk != D or tuple(v_pages.shape) != tuple(k_pages.shape):
        raise ValueError("q / k_pages / v_pages shapes disagree")
    B = prefix_len.shape[0]
    if node_start.shape[0] != B + 1 or block_table.shape[0] != B or parent.shape[0] != T:
        raise ValueError("metadata lengths disagree with batch / total nodes")
    if out is None:
        out = torch.empty_like(q)
    else:
        _need_out(out, "out", q.dtype, q.shape)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    else:
        _need_out(lse, "lse", torch.float32, (T, Hq))
    _need_flag(err_flag)
    need = ev_tree_attention_workspace_size(B, max_nodes, Hq, Hkv, D)
    if workspace is None or workspace.nbytes < need:
        workspace = Workspace(need, q.device)
    st = ev_tree_attention_paged(_addr(q), _addr(k_pages), _addr(v_pages), _addr(out), _addr(lse), _addr(node_start),
                                 _addr(parent), _addr(block_table), block_table.shape[1], page_size,
                                 _addr(prefix_len), B, T, max_nodes, pages, Hq, Hkv, D, EV_BF16, float(sm_scale),
                                 int(window), workspace.ptr, workspace.nbytes, _addr(err_flag), _stream(stream))
    _check(st, "ev_tree_attention_paged")
    return out, lse, workspace


def node_argmax(logits, *, vocab: int = None, target=None, max_value=None, workspace: Workspace = None,
                stream=None):
    """Greedy token per row (ev_node_argmax).  logits [R, stride] bf16/fp32.  Returns (target, max_value, ws)."""
    torch = _torch()
    _need(logits, "logits", ndim=2)
    R, stride = logits.shape
    vocab = stride if vocab is None else vocab
    if target is None:
        target = torch.empty(R, dtype=torch.int32, device=logits.device)
    else:
        _need_out(target, "target", torch.int32, (R,))
    if max_value is None:
        max_value = torch.empty(R, dtype=torch.float32, device=logits.device)
    else:
        _need_out(max_value, "max_value", torch.float32, (R,))
    need = ev_node_argmax_workspace_size(R, vocab)
    if need and (workspace is None or workspace.nbytes < need):
        workspace = Workspace(need, logits.device)
    st = ev_node_argmax(_addr(logits), _dtype_code(logits), stride, R, vocab, _addr(target), _addr(max_value),
                        workspace.ptr if workspace is not None else None,
                        workspace.nbytes if workspace is not None else 0, _stream(stream))
    _check(st, "ev_node_argmax")
    return target, max_value, workspace


def node_sample(logits, *, temperature: float, seed: int, offset: int, vocab: int = None, target=None,
                workspace: Workspace = None, stream=None):
    """Sampled token per row at temperature > 0 (ev_node_sample).  logits [R, stride] bf16/fp32.
    Returns (target, workspace)."""
    torch = _torch()
    _need(logits, "logits", ndim=2)
    R, stride = logits.shape
    vocab = stride if vocab is None else vocab
    if target is None:
        target = torch.empty(R, dtype=torch.int32, device=logits.device)
    else:
        _need_out(target, "target", torch.int32, (R,))
    need = ev_node_argmax_workspace_size(R, vocab)
    if need and (workspace is None or workspace.nbytes < need):
        workspace = Workspace(need, logits.device)
    st = ev_node_sample(_addr(logits), _dtype_code(logits), stride, R, vocab, float(temperature),
                        int(seed) & 0xFFFFFFFFFFFFFFFF, int(offset) & 0xFFFFFFFFFFFFFFFF, _addr(target),
                        workspace.ptr if workspace is not None else None,
                        workspace.nbytes if workspace is not None else 0, _stream(stream))
    _check(st, "ev_node_sample")
    return target, workspace


def greedy_accept(node_start, parent, draft_token, target_token, *, max_nodes: int, vocab: int, out=None,
                  err_flag=None, stream=None):
    """Longest accepted path per sequence (ev_greedy_accept).
    Returns dict(accept_len [B], accept_path [B, max_nodes], bonus [B], out_tokens [B, max_nodes])."""
    return _accept(ev_greedy_accept, "ev_greedy_accept", node_start, parent, draft_token, target_token, max_nodes,
                   vocab, out, err_flag, stream)


def sampled_accept(node_start, parent, draft_token, target_token, *, max_nodes: int, vocab: int, out=None,
                   err_flag=None, stream=None):
    """Sampled-verification acceptance from per-node draws (ev_sampled_accept): the walk into the
    lowest-index child holding each node's draw.  Returns what greedy_accept returns."""
    return _accept(ev_sampled_accept, "ev_sampled_accept", node_start, parent, draft_token, target_token, max_nodes,
                   vocab, out, err_flag, stream)


def _accept(fn, name, node_start, parent, draft_token, target_token, max_nodes, vocab, out, err_flag, stream):
    torch = _torch()
    for name, t in (("node_start", node_start), ("parent", parent), ("draft_token", draft_token),
                    ("target_token", target_token)):
        _need(t, name, torch.int32, 1)
    B = node_start.shape[0] - 1
    T = parent.shape[0]
    if draft_token.shape[0] != T or target_token.shape[0] != T:
        raise ValueError("parent / draft_token / target_token lengths disagree")
    out = _accept_outputs(B, max_nodes, parent.device, out)
    _need_flag(err_flag)
    st = fn(_addr(node_start), _addr(parent), _addr(draft_token), _addr(target_token), B, T, max_nodes, vocab,
            _addr(out["accept_len"]), _addr(out["accept_path"]), _addr(out["bonus"]), _addr(out["out_tokens"]),
            _addr(err_flag), _stream(stream))
    _check(st, name)
    return out


def compact_kv(k_cache, v_cache, kv_start, prefix_len, accept_len, accept_path, *, new_len=None, err_flag=None,
               stream=None):
    """In-place KV compaction (ev_compact_kv).  Caches [slots, Hkv, D] or [layers, slots, Hkv, D]."""
    torch = _torch()
    _need(k_cache, "k_cache")
    _need(v_cache, "v_cache", k_cache.dtype)
    if k_cache.dim() == 3:
        layers, (slots, Hkv, D) = 1, k_cache.shape
    elif k_cache.dim() == 4:
        layers, slots, Hkv, D = k_cache.shape
    else:
        raise ValueError("caches must be [slots, Hkv, D] or [layers, slots, Hkv, D]")
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache / v_cache shapes disagree")
    B, max_nodes = _compact_meta(prefix_len, accept_len, accept_path, kv_start=kv_start)
    if new_len is None:
        new_len = torch.empty(B, dtype=torch.int32, device=k_cache.device)
    else:
        _need_out(new_len, "new_len", torch.int32, (B,))
    _need_flag(err_flag)
    esz = k_cache.element_size()
    st = ev_compact_kv(_addr(k_cache), _addr(v_cache), esz, layers, slots * Hkv * D * esz, _addr(kv_start),
                       _addr(prefix_len), _addr(accept_len), _addr(accept_path), B, max_nodes, slots, Hkv, D,
                       _addr(new_len), _addr(err_flag), _stream(stream))
    _check(st, "ev_compact_kv")
    return new_len


def compact_kv_paged(k_pages, v_pages, block_table, prefix_len, accept_len, accept_path, *, new_len=None,
                     err_flag=None, stream=None):
    """In-place KV compaction through a block table (ev_compact_kv_paged).  Pools
    [pages, page_size, Hkv, D] or [layers, pages, page_size, Hkv, D]; block_table [B, stride] int32."""
    torch = _torch()
    _need(k_pages, "k_pages")
    _need(v_pages, "v_pages", k_pages.dtype)
    _need(block_table, "block_table", torch.int32, 2)
    if k_pages.dim() == 4:
        layers, (pages, page_size, Hkv, D) = 1, k_pages.shape
    elif k_pages.dim() == 5:
        layers, pages, page_size, Hkv, D = k_pages.shape
    else:
        raise ValueError("pools must be [pages, page_size, Hkv, D] or [layers, pages, page_size, Hkv, D]")
    if tuple(v_pages.shape) != tuple(k_pages.shape):
        raise ValueError("k_pages / v_pages shapes disagree")
    B, max_nodes = _compact_meta(prefix_len, accept_len, accept_path)
    if block_table.shape[0] != B:
        raise ValueError("block_table rows disagree with the batch")
    if new_len is None:
        new_len = torch.empty(B, dtype=torch.int32, device=k_pages.device)
    else:
        _need_out(new_len, "new_len", torch.int32, (B,))
    _need_flag(err_flag)
    esz = k_pages.element_size()
    st = ev_compact_kv_paged(_addr(k_pages), _addr(v_pages), esz, layers, pages * page_size * Hkv * D * esz,
                             _addr(block_table), block_table.shape[1], page_size, _addr(prefix_len),
                             _addr(accept_len), _addr(accept_path), B, max_nodes, pages, Hkv, D, _addr(new_len),
                             _addr(err_flag), _stream(stream))
    _check(st, "ev_compact_kv_paged")
    return new_len


def _accept_outputs(B, max_nodes, dev, out):
    torch = _torch()
    if out is None:
        out = {"accept_len": torch.empty(B, dtype=torch.int32, device=dev),
               "accept_path": torch.empty((B, max_nodes), dtype=torch.int32, device=dev),
               "bonus": torch.empty(B, dtype=torch.int32, device=dev),
               "out_tokens": torch.empty((B, max_nodes), dtype=torch.int32, device=dev)}
    else:
        _need_accept(out, B, max_nodes)
    return out


def _compact_meta(prefix_len, accept_len, accept_path, kv_start=None):
    """Checks the compaction's per-sequence inputs; returns (batch, max_nodes)."""
    torch = _torch()
    _need(prefix_len, "prefix_len", torch.int32, 1)
    _need(accept_len, "accept_len", torch.int32, 1)
    _need(accept_path, "accept_path", torch.int32, 2)
    B = prefix_len.shape[0]
    if kv_start is not None:
        _need(kv_start, "kv_start", torch.int32, 1)
        if kv_start.shape[0] != B:
            raise ValueError("kv_start / prefix_len lengths disagree")
    if accept_len.shape[0] != B or accept_path.shape[0] != B:
        raise ValueError("accept_len / accept_path rows disagree with the batch")
    return B, accept_path.shape[1]


def select_accept_compact(logits, node_start, parent, draft_token, k_cache, v_cache, kv_start, prefix_len, *,
                          max_nodes: int, temperature: float = 0.0, seed: int = 0, offset: int = 0, vocab: int = None,
                          target=None, out=None, new_len=None, workspace: Workspace = None, err_flag=None,
                          stream=None, block_table=None):
    """Per-node token (argmax at temperature 0, else the sampled draw), acceptance and in-place KV
    compaction in one call (ev_select_accept_compact; with block_table, the paged form and caches
    are pools [pages, page_size, Hkv, D] or [layers, pages, page_size, Hkv, D]).
    Returns (target [R], accept dict as greedy_accept's, new_len [B], workspace)."""
    torch = _torch()
    _need(logits, "logits", ndim=2)
    for name, t in (("node_start", node_start), ("parent", parent), ("draft_token", draft_token)):
        _need(t, name, torch.int32, 1)
    _need(k_cache, "k_cache")
    _need(v_cache, "v_cache", k_cache.dtype)
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache / v_cache shapes disagree")
    R, stride = logits.shape
    vocab = stride if vocab is None else vocab
    B = node_start.shape[0] - 1
    T = parent.shape[0]
    if R != T or draft_token.shape[0] != T:
        raise ValueError("logits rows / parent / draft_token lengths disagree")
    _need(prefix_len, "prefix_len", torch.int32, 1)
    if prefix_len.shape[0] != B:
        raise ValueError("prefix_len length disagrees with the batch")
    dev = parent.device
    paged = block_table is not None
    if paged:
        _need(block_table, "block_table", torch.int32, 2)
        if block_table.shape[0] != B:
            raise ValueError("block_table rows disagree with the batch")
    else:
        _need(kv_start, "kv_start", torch.int32, 1)
        if kv_start.shape[0] != B:
            raise ValueError("kv_start length disagrees with the batch")
    base = 4 if paged else 3
    if k_cache.dim() == base:
        layers, dims = 1, tuple(k_cache.shape)
    elif k_cache.dim() == base + 1:
        layers, dims = k_cache.shape[0], tuple(k_cache.shape[1:])
    else:
        raise ValueError("caches must be [slots, Hkv, D] / [pages, page_size, Hkv, D], optionally with a layer axis")
    Hkv, D = dims[-2], dims[-1]
    rows_per_layer = 1
    for x in dims[:-2]:
        rows_per_layer *= int(x)
    if target is None:
        target = torch.empty(R, dtype=torch.int32, device=dev)
    else:
        _need_out(target, "target", torch.int32, (R,))
    out = _accept_outputs(B, max_nodes, dev, out)
    if new_len is None:
        new_len = torch.empty(B, dtype=torch.int32, device=dev)
    else:
        _need_out(new_len, "new_len", torch.int32, (B,))
    _need_flag(err_flag)
    need = ev_select_workspace_size(T, vocab)
    if need and (workspace is None or workspace.nbytes < need):
        workspace = Workspace(need, dev)
    esz = k_cache.element_size()
    common = (_addr(logits), _dtype_code(logits), stride, vocab, float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF,
              int(offset) & 0xFFFFFFFFFFFFFFFF, _addr(node_start), _addr(parent), _addr(draft_token), B, T, max_nodes,
              _addr(k_cache), _addr(v_cache), esz, layers, rows_per_layer * Hkv * D * esz)
    tail = (Hkv, D, _addr(target), _addr(out["accept_len"]), _addr(out["accept_path"]), _addr(out["bonus"]),
            _addr(out["out_tokens"]), _addr(new_len), workspace.ptr if workspace is not None else None,
            workspace.nbytes if workspace is not None else 0, _addr(err_flag), _stream(stream))
    if paged:
        st = ev_select_accept_compact_paged(*common, _addr(block_table), block_table.shape[1], dims[1],
                                            _addr(prefix_len), dims[0], *tail)
        _check(st, "ev_select_accept_compact_paged")
    else:
        st = ev_select_accept_compact(*common, _addr(kv_start), _addr(prefix_len), dims[0], *tail)
        _check(st, "ev_select_accept_compact")
    return target, out, new_len, workspace


def verify_step(q, k_cache, v_cache, logits, node_start, parent, kv_start, prefix_len, draft_token, *,
                max_nodes: int, sm_scale: float, temperature: float = 0.0, seed: int = 0, offset: int = 0,
                state: dict = None, stream=None, head_major: bool = False, vocab: int = None):
    """One whole verification step (ev_verify_step, one stream): attention, its split merge with
    the per-node token pass in the same launch (argmax at temperature 0, else the sampled draw
    keyed by (seed, offset)), then acceptance and compaction.  Caches [slots, Hkv, D], or [Hkv, slots, D] with head_major.  ``state`` carries
    reusable outputs and the workspace between calls; returns it, with out, lse, target, accept
    (as greedy_accept's dict), new_len and err."""
    torch = _torch()
    state = {} if state is None else state
    _need(q, "q", ndim=3)
    _need(k_cache, "k_cache", q.dtype, 3)
    _need(v_cache, "v_cache", q.dtype, 3)
    _need(logits, "logits", ndim=2)
    for name, t in (("node_start", node_start), ("parent", parent), ("kv_start", kv_start),
                    ("prefix_len", prefix_len), ("draft_token", draft_token)):
        _need(t, name, torch.int32, 1)
    T, Hq, D = q.shape
    if head_major:
        Hkv, slots, Dk = k_cache.shape
    else:
        slots, Hkv, Dk = k_cache.shape
    if Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q / k_cache / v_cache shapes disagree")
    B = prefix_len.shape[0]
    if node_start.shape[0] != B + 1 or kv_start.shape[0] != B or parent.shape[0] != T or draft_token.shape[0] != T:
        raise ValueError("metadata lengths disagree with batch / total nodes")
    R, stride = logits.shape
    if R != T:
        raise ValueError("logits rows disagree with total nodes")
    vocab = stride if vocab is None else vocab
    dev = q.device
    if "err" not in state:
        state["err"] = torch.zeros(1, dtype=torch.int32, device=dev)
    if state.get("out") is None or tuple(state["out"].shape) != tuple(q.shape) or state["out"].dtype != q.dtype:
        state["out"] = torch.empty_like(q)
    if state.get("lse") is None or tuple(state["lse"].shape) != (T, Hq):
        state["lse"] = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    if state.get("target") is None or state["target"].shape[0] != T:
        state["target"] = torch.empty(T, dtype=torch.int32, device=dev)
    state["accept"] = _accept_outputs(B, max_nodes, dev, state.get("accept"))
    if state.get("new_len") is None or state["new_len"].shape[0] != B:
        state["new_len"] = torch.empty(B, dtype=torch.int32, device=dev)
    need = ev_verify_step_workspace_size(B, T, max_nodes, Hq, Hkv, D, vocab)
    if not need:
        raise EvError(2, "ev_verify_step_workspace_size")
    ws = state.get("step_ws")
    if ws is None or ws.nbytes < need:
        ws = Workspace(need, dev)
        state["step_ws"] = ws
    esz = k_cache.element_size()
    if head_major:  # [Hkv][slots][D]: compacted as Hkv one-head layers
        strides, comp = (D, slots * D), (Hkv, slots * D * esz, 1, D)
    else:
        strides, comp = (Hkv * D, D), (1, slots * Hkv * D * esz, Hkv, D)
    acc = state["accept"]
    st = ev_verify_step(_addr(q), _addr(k_cache), _addr(v_cache), _addr(state["out"]), _addr(state["lse"]),
                        _addr(node_start), _addr(parent), _addr(kv_start), _addr(prefix_len), B, T, max_nodes, slots,
                        Hq, Hkv, D, *strides, _dtype_code(q), float(sm_scale), _addr(logits), _dtype_code(logits),
                        stride, vocab, float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF,
                        int(offset) & 0xFFFFFFFFFFFFFFFF, _addr(draft_token), *comp, _addr(state["target"]),
                        _addr(acc["accept_len"]), _addr(acc["accept_path"]), _addr(acc["bonus"]),
                        _addr(acc["out_tokens"]), _addr(state["new_len"]), ws.ptr, ws.nbytes, _addr(state["err"]),
                        _stream(stream))
    _check(st, "ev_verify_step")
    return state
