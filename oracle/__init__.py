"""CPU oracle of the draft-tree verification step -- TEST INFRASTRUCTURE ONLY.

Plain C loops in double precision (``ev_oracle.c``), built with gcc and called through
ctypes.  Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package; the GPU library and its Python binding never do, and the two share
no code.  All arguments are host numpy arrays; bf16 data is passed as raw uint16 bits and
widened exactly inside the C code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ev_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "libev_oracle.so")
_lib = None

BF16 = 0
F32 = 1
MAX_NODES = 1024


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (OpenMP across independent rows/sequences)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-std=c11", "-Wall",
           "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def load(path: str = None):
    """Load the oracle library, building it first if it is missing or older than its source."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_D = ctypes.c_double


def _bind(lib):
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_tree_errors.restype = _I32
    lib.oracle_tree_errors.argtypes = [_P, _I32, _I32]
    lib.oracle_ancestor_path.restype = _I32
    lib.oracle_ancestor_path.argtypes = [_P, _I32, _P]
    lib.oracle_tree_attention.restype = None
    lib.oracle_tree_attention.argtypes = [_P, _P, _P, _I32, _P, _P, _P, _P, _I32, _I32, _I64, _I32, _I32,
                                          _I32, _D, _P, _P, _P]
    lib.oracle_tree_attention_rows.restype = None
    lib.oracle_tree_attention_rows.argtypes = [_P, _P, _P, _I32, _P, _P, _P, _P, _I32, _I32, _I64, _I32,
                                               _I32, _I32, _D, _P, _I64, _P, _P]
    lib.oracle_tree_attention_ex.restype = None
    lib.oracle_tree_attention_ex.argtypes = [_P, _P, _P, _I32, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                             _I64, _I32, _I32, _I32, _D, _P, _P, _P]
    lib.oracle_tree_attention_rows_ex.restype = None
    lib.oracle_tree_attention_rows_ex.argtypes = [_P, _P, _P, _I32, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32,
                                                  _I32, _I64, _I32, _I32, _I32, _D, _P, _I64, _P, _P]
    lib.oracle_compact_kv_paged.restype = None
    lib.oracle_compact_kv_paged.argtypes = [_P, _P, _P, _P, _I32, _I32, _I64, _P, _I32, _I32, _P, _P, _P, _I32,
                                            _I32, _I64, _I32, _I32, _P, _P]
    lib.oracle_node_argmax.restype = None
    lib.oracle_node_argmax.argtypes = [_P, _I32, _I64, _I32, _I32, _P, _P]
    lib.oracle_philox4x32_10.restype = None
    lib.oracle_philox4x32_10.argtypes = [_P, _P, _P]
    lib.oracle_sample_uniform.restype = ctypes.c_float
    lib.oracle_sample_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint64, _I64, _I64]
    lib.oracle_sample_score.restype = ctypes.c_float
    lib.oracle_sample_score.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64, _I64, _I64]
    lib.oracle_node_sample.restype = None
    lib.oracle_node_sample.argtypes = [_P, _I32, _I64, _I32, _I32, ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64,
                                       _P, _P]
    lib.oracle_greedy_accept.restype = None
    lib.oracle_greedy_accept.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P, _P]
    lib.oracle_sampled_accept.restype = None
    lib.oracle_sampled_accept.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P, _P]
    lib.oracle_compact_kv.restype = None
    lib.oracle_compact_kv.argtypes = [_P, _P, _P, _P, _I32, _I32, _I64, _P, _P, _P, _P, _I32, _I32, _I64,
                                      _I32, _I32, _P, _P]
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arguments must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _dtype_of(x: np.ndarray) -> int:
    if x.dtype == np.uint16:
        return BF16
    if x.dtype == np.float32:
        return F32
    raise TypeError(f"oracle expects bf16 bits (uint16) or float32, got {x.dtype}")


def num_threads(lib=None) -> int:
    return int((lib or load()).oracle_num_threads())


def tree_errors(parent, max_nodes: int, lib=None) -> int:
    parent = _i32(parent)
    return int((lib or load()).oracle_tree_errors(_ptr(parent), len(parent), max_nodes))


def ancestor_path(parent, i: int, lib=None) -> np.ndarray:
    """Ancestors of node i, itself included, root first; empty when the chain is malformed or i is
    beyond the oracle's work arrays."""
    parent = _i32(parent)
    out = np.zeros(max(len(parent), MAX_NODES, 1), dtype=np.int32)
    n = (lib or load()).oracle_ancestor_path(_ptr(parent), int(i), _ptr(out))
    return out[:max(n, 0)].copy()


def _layout(kv_start, block_table, page_size):
    """(kv_start, block_table, bt_stride, page_size) arguments of the C oracle."""
    if block_table is None:
        return _i32(kv_start), None, 0, 0
    bt = _i32(block_table)
    assert bt.ndim == 2 and page_size >= 1
    ks = _i32(kv_start) if kv_start is not None else np.zeros(bt.shape[0], np.int32)
    return ks, bt, bt.shape[1], int(page_size)


def tree_attention(q, k, v, node_start, parent, kv_start, prefix_len, *, num_q_heads: int,
                   num_kv_heads: int, head_dim: int, sm_scale: float, total_slots: int,
                   max_nodes: int = None, window: int = 0, block_table=None, page_size: int = 0, lib=None):
    """Every row.  Returns (out [T, Hq, D] float64, lse [T, Hq] float64, seq_err [B] int32).
    Rows of sequences with data errors hold NaN.  window > 0: only the last `window` prefix tokens
    are visible.  block_table [B, pages] with page_size: paged caches ([rows, Hkv, D], token t of
    sequence b at row block_table[b, t // page_size] * page_size + t % page_size; kv_start unused)."""
    lib = lib or load()
    q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
    dt = _dtype_of(q)
    assert _dtype_of(k) == dt and _dtype_of(v) == dt
    node_start, parent, prefix_len = map(_i32, (node_start, parent, prefix_len))
    kv_start, bt, bts, pgs = _layout(kv_start, block_table, page_size)
    B = len(prefix_len)
    T = int(node_start[-1]) if len(node_start) else 0
    if max_nodes is None:
        max_nodes = int(np.diff(node_start).max()) if B else 1
    assert max_nodes <= MAX_NODES
    out = np.full((T, num_q_heads, head_dim), np.nan)
    lse = np.full((T, num_q_heads), np.nan)
    err = np.zeros(max(B, 1), dtype=np.int32)
    lib.oracle_tree_attention_ex(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(node_start), _ptr(parent), _ptr(kv_start),
                                 _ptr(prefix_len), _ptr(bt) if bt is not None else None, bts, pgs, int(window), B,
                                 max_nodes, int(total_slots), num_q_heads, num_kv_heads, head_dim, float(sm_scale),
                                 _ptr(out), _ptr(lse), _ptr(err))
    return out, lse, err[:B]


def tree_attention_rows(q, k, v, node_start, parent, kv_start, prefix_len, rows, *, num_q_heads: int,
                        num_kv_heads: int, head_dim: int, sm_scale: float, total_slots: int,
                        max_nodes: int = None, window: int = 0, block_table=None, page_size: int = 0, lib=None):
    """Selected rows only: ``rows`` is an int array [R, 2] of (global node, q head).
    Returns (out [R, D] float64, lse [R] float64)."""
    lib = lib or load()
    q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
    dt = _dtype_of(q)
    node_start, parent, prefix_len = map(_i32, (node_start, parent, prefix_len))
    kv_start, bt, bts, pgs = _layout(kv_start, block_table, page_size)
    rows = _i32(rows).reshape(-1, 2)
    B = len(prefix_len)
    if max_nodes is None:
        max_nodes = int(np.diff(node_start).max()) if B else 1
    R = rows.shape[0]
    out = np.full((R, head_dim), np.nan)
    lse = np.full(R, np.nan)
    lib.oracle_tree_attention_rows_ex(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(node_start), _ptr(parent),
                                      _ptr(kv_start), _ptr(prefix_len), _ptr(bt) if bt is not None else None, bts,
                                      pgs, int(window), B, max_nodes, int(total_slots), num_q_heads, num_kv_heads,
                                      head_dim, float(sm_scale), _ptr(rows), R, _ptr(out), _ptr(lse))
    return out, lse


def node_argmax(logits, vocab: int = None, row_stride: int = None, lib=None):
    """Returns (target [R] int32, max_value [R] float64)."""
    lib = lib or load()
    logits = np.ascontiguousarray(logits)
    dt = _dtype_of(logits)
    R = logits.shape[0]
    if vocab is None:
        vocab = logits.shape[1]
    if row_stride is None:
        row_stride = logits.shape[1]
    tgt = np.zeros(max(R, 1), dtype=np.int32)
    mx = np.zeros(max(R, 1))
    lib.oracle_node_argmax(_ptr(logits), dt, int(row_stride), R, int(vocab), _ptr(tgt), _ptr(mx))
    return tgt[:R], mx[:R]


def philox4x32_10(ctr, key, lib=None) -> np.ndarray:
    """Philox4x32-10 of a 128-bit counter (4 words) under a 64-bit key (2 words)."""
    lib = lib or load()
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib.oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sample_uniform(seed: int, offset: int, row: int, v: int, lib=None) -> float:
    """The uniform in (0, 1) that the sampled draw uses for element v of row `row`."""
    return float((lib or load()).oracle_sample_uniform(seed, offset, row, v))


def sample_score(z: float, temperature: float, seed: int, offset: int, row: int, v: int, lib=None) -> float:
    """The fp32 score the draw maximises for element v of row `row` with logit z."""
    return float((lib or load()).oracle_sample_score(z, temperature, seed, offset, row, v))


def node_sample(logits, temperature: float, seed: int, offset: int, vocab: int = None, row_stride: int = None,
                lib=None):
    """Sampled target token per row (Gumbel-max draw from softmax(logits / T) with Philox noise).
    Returns (token [R] int32, score [R] float32: the winning base-2 score)."""
    lib = lib or load()
    logits = np.ascontiguousarray(logits)
    dt = _dtype_of(logits)
    R = logits.shape[0]
    vocab = logits.shape[1] if vocab is None else vocab
    row_stride = logits.shape[1] if row_stride is None else row_stride
    tok = np.zeros(max(R, 1), dtype=np.int32)
    sc = np.zeros(max(R, 1), dtype=np.float32)
    lib.oracle_node_sample(_ptr(logits), dt, int(row_stride), R, int(vocab), float(temperature), int(seed),
                           int(offset), _ptr(tok), _ptr(sc))
    return tok[:R], sc[:R]


def greedy_accept(node_start, parent, draft, target, max_nodes: int, vocab: int, lib=None):
    """Greedy (temperature 0) acceptance: the deepest accepted node, lowest index on equal depth.
    Returns dict of accept_len [B], accept_path [B, max_nodes], bonus [B], out_tokens [B, max_nodes],
    seq_err [B]."""
    return _accept("oracle_greedy_accept", node_start, parent, draft, target, max_nodes, vocab, lib)


def sampled_accept(node_start, parent, draft, target, max_nodes: int, vocab: int, lib=None):
    """Sampled (temperature > 0) acceptance, ``target`` holding each node's draw: the walk from the
    root into the lowest-index child holding the current node's draw.  Same returns as
    greedy_accept."""
    return _accept("oracle_sampled_accept", node_start, parent, draft, target, max_nodes, vocab, lib)


def _accept(fn, node_start, parent, draft, target, max_nodes, vocab, lib):
    lib = lib or load()
    node_start, parent, draft, target = map(_i32, (node_start, parent, draft, target))
    B = len(node_start) - 1
    assert max_nodes <= MAX_NODES
    acc = np.zeros(max(B, 1), np.int32)
    path = np.zeros((max(B, 1), max_nodes), np.int32)
    bonus = np.zeros(max(B, 1), np.int32)
    outt = np.zeros((max(B, 1), max_nodes), np.int32)
    err = np.zeros(max(B, 1), np.int32)
    getattr(lib, fn)(_ptr(node_start), _ptr(parent), _ptr(draft), _ptr(target), B, max_nodes, int(vocab),
                     _ptr(acc), _ptr(path), _ptr(bonus), _ptr(outt), _ptr(err))
    return {"accept_len": acc[:B], "accept_path": path[:B], "bonus": bonus[:B], "out_tokens": outt[:B],
            "seq_err": err[:B]}


def compact_kv(k, v, kv_start, prefix_len, accept_len, accept_path, *, num_layers: int, total_slots: int,
               num_kv_heads: int, head_dim: int, lib=None):
    """Out-of-place compaction of caches shaped [layers, total_slots, Hkv, D] (any element type).
    Returns (k_out, v_out, new_len [B], seq_err [B])."""
    lib = lib or load()
    k, v = np.ascontiguousarray(k), np.ascontiguousarray(v)
    kv_start, prefix_len, accept_len = map(_i32, (kv_start, prefix_len, accept_len))
    accept_path = _i32(accept_path)
    B = len(prefix_len)
    max_nodes = accept_path.shape[1] if accept_path.ndim == 2 else 1
    elem = k.dtype.itemsize
    layer_stride = total_slots * num_kv_heads * head_dim * elem
    assert k.nbytes == num_layers * layer_stride and v.nbytes == k.nbytes
    k_out, v_out = np.empty_like(k), np.empty_like(v)
    new_len = np.zeros(max(B, 1), np.int32)
    err = np.zeros(max(B, 1), np.int32)
    lib.oracle_compact_kv(_ptr(k), _ptr(v), _ptr(k_out), _ptr(v_out), elem, num_layers, layer_stride,
                          _ptr(kv_start), _ptr(prefix_len), _ptr(accept_len), _ptr(accept_path), B, max_nodes,
                          int(total_slots), num_kv_heads, head_dim, _ptr(new_len), _ptr(err))
    return k_out, v_out, new_len[:B], err[:B]


def compact_kv_paged(k, v, block_table, page_size: int, prefix_len, accept_len, accept_path, *, num_layers: int,
                     total_rows: int, num_kv_heads: int, head_dim: int, lib=None):
    """Out-of-place compaction of paged caches shaped [layers, total_rows, Hkv, D]: token t of sequence
    b sits at row block_table[b, t // page_size] * page_size + t % page_size.
    Returns (k_out, v_out, new_len [B], seq_err [B])."""
    lib = lib or load()
    k, v = np.ascontiguousarray(k), np.ascontiguousarray(v)
    bt = _i32(block_table)
    prefix_len, accept_len = map(_i32, (prefix_len, accept_len))
    accept_path = _i32(accept_path)
    B = len(prefix_len)
    max_nodes = accept_path.shape[1] if accept_path.ndim == 2 else 1
    elem = k.dtype.itemsize
    layer_stride = total_rows * num_kv_heads * head_dim * elem
    assert k.nbytes == num_layers * layer_stride and v.nbytes == k.nbytes
    k_out, v_out = np.empty_like(k), np.empty_like(v)
    new_len = np.zeros(max(B, 1), np.int32)
    err = np.zeros(max(B, 1), np.int32)
    lib.oracle_compact_kv_paged(_ptr(k), _ptr(v), _ptr(k_out), _ptr(v_out), elem, num_layers, layer_stride, _ptr(bt),
                                bt.shape[1], int(page_size), _ptr(prefix_len), _ptr(accept_len), _ptr(accept_path), B,
                                max_nodes, int(total_rows), num_kv_heads, head_dim, _ptr(new_len), _ptr(err))
    return k_out, v_out, new_len[:B], err[:B]
