"""Seeded synthetic inputs for the draft-tree verification step.

This module is the only code shared by the HIP path's tests/benchmark and by the
CPU oracle's tests.  It draws random numbers and lays them out; it computes none
of the verification step itself.  The one exception is the planting of draft
tokens: the workloads ask for draft tokens that equal the target's greedy choice
with a stated probability, so the generator calls ``numpy.argmax`` (documented to
return the first occurrence of the maximum) on the parent's logits row to decide
what to plant.  Neither the oracle nor the kernels read that value; both compute
their own argmax from the logits.

Workloads (sizes follow the verification-step shapes used throughout):
  tiny    1 seq, Hq 8 / Hkv 2, D 64, fp32, prefix 256, chain of 4 nodes, vocab 1024
  c1x4k   1 seq, Hq 40 / Hkv 8, D 128, bf16, prefix 4096, 16-node tree, vocab 151936
  c8      8 seqs, prefix ~U[1024, 8192], 16-node trees
  c512    512 seqs, prefix ~U[512, 4096], 4-node trees, acceptance prob 0.5
  c128k   1 seq, prefix 131072, 16-node tree

Random trees: node 0 is the root; for i >= 1 the parent is uniform over the
shallower nodes j < i whose depth is below the depth limit (6), so every tree is
in topological order (parent index < child index).
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional, Sequence

import numpy as np

BF16 = 0
F32 = 1

_CHUNK = 1 << 24  # values drawn per chunk for large tensors (bounds temporary memory)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return raw uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of raw bfloat16 bits to float32."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, n: int, scale: float, dtype: int) -> np.ndarray:
    """n draws of N(0, scale^2), produced in chunks; bf16 results are raw uint16 bits."""
    out = np.empty(n, dtype=np.uint16 if dtype == BF16 else np.float32)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[lo:hi] = f32_to_bf16_bits(x) if dtype == BF16 else x
    return out


def random_tree(rng: np.random.Generator, n: int, max_depth: int = 6) -> np.ndarray:
    """Parent array (local indices, root parent -1) of an n-node tree of depth <= max_depth."""
    parent = np.full(n, -1, dtype=np.int32)
    depth = np.zeros(n, dtype=np.int32)
    for i in range(1, n):
        cand = np.nonzero(depth[:i] < max_depth)[0]
        p = int(cand[rng.integers(0, len(cand))])
        parent[i] = p
        depth[i] = depth[p] + 1
    return parent


def chain_tree(n: int) -> np.ndarray:
    return np.arange(-1, n - 1, dtype=np.int32)


@dataclasses.dataclass
class Workload:
    """Host-side inputs of one verification step (all arrays contiguous numpy)."""
    name: str
    dtype: int                 # BF16 (q/k/v/logits are uint16 bit patterns) or F32
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    vocab: int
    sm_scale: float
    node_start: np.ndarray     # int32 [B+1]
    parent: np.ndarray         # int32 [sum N], local parent indices
    kv_start: np.ndarray       # int32 [B]
    prefix_len: np.ndarray     # int32 [B]
    total_slots: int
    q: np.ndarray              # [sum N, Hq, D]
    k: np.ndarray              # [total_slots, Hkv, D]
    v: np.ndarray              # [total_slots, Hkv, D]
    logits: np.ndarray         # [sum N, vocab]
    draft: np.ndarray          # int32 [sum N]; the root's token is never compared
    accept_prob: float

    @property
    def batch(self) -> int:
        return len(self.prefix_len)

    @property
    def total_nodes(self) -> int:
        return int(self.node_start[-1])

    @property
    def nodes_per_seq(self) -> np.ndarray:
        return np.diff(self.node_start).astype(np.int32)

    @property
    def max_nodes(self) -> int:
        return int(self.nodes_per_seq.max()) if self.batch else 0

    @property
    def max_prefix_len(self) -> int:
        return int(self.prefix_len.max()) if self.batch else 0

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == BF16 else 4

    def kv_bytes(self) -> int:
        """K+V bytes of every visible slot (prefix and tree), read once per (sequence, KV head)."""
        slots = int(self.prefix_len.sum()) + self.total_nodes
        return 2 * slots * self.num_kv_heads * self.head_dim * self.elem_bytes

    def digest(self) -> str:
        h = hashlib.sha256()
        for a in (self.node_start, self.parent, self.kv_start, self.prefix_len, self.q, self.k,
                  self.v, self.logits, self.draft):
            h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()[:16]


def make_workload(name: str, seed: int, *, prefix_lens: Sequence[int], trees: Optional[Sequence] = None,
                  nodes: Optional[Sequence[int]] = None, num_q_heads: int = 40, num_kv_heads: int = 8,
                  head_dim: int = 128, dtype: int = BF16, vocab: int = 151936, q_scale: float = None,
                  kv_scale: float = 1.0, logit_scale: float = 2.0, accept_prob: float = 0.7,
                  max_depth: int = 6, sm_scale: float = None, slot_gap: int = 0,
                  distinct_siblings: bool = False, rng: Optional[np.random.Generator] = None) -> Workload:
    """Draw one verification step.

    Draw order: prefix lengths (given) -> parents -> Q -> K -> V -> logits -> planted tokens.
    ``trees`` gives explicit parent arrays; otherwise ``nodes`` gives node counts of random trees.
    ``slot_gap`` leaves unused cache slots between sequences (exercises kv_start).
    """
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    B = len(prefix_lens)
    if trees is None:
        trees = [chain_tree(1) if n == 1 else random_tree(rng, int(n), max_depth) for n in nodes]
    trees = [np.asarray(t, dtype=np.int32) for t in trees]
    assert len(trees) == B
    ns = np.array([len(t) for t in trees], dtype=np.int32)
    node_start = np.zeros(B + 1, dtype=np.int32)
    node_start[1:] = np.cumsum(ns)
    parent = np.concatenate(trees).astype(np.int32) if B else np.zeros(0, np.int32)
    prefix_len = np.asarray(prefix_lens, dtype=np.int32)
    kv_start = np.zeros(B, dtype=np.int32)
    off = 0
    for b in range(B):
        kv_start[b] = off
        off += int(prefix_len[b]) + int(ns[b]) + slot_gap
    total_slots = off
    T = int(node_start[-1])
    if q_scale is None:
        q_scale = 1.0 if dtype == F32 else 1.0 / math.sqrt(head_dim)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(head_dim)
    q = _normal(rng, T * num_q_heads * head_dim, q_scale, dtype).reshape(T, num_q_heads, head_dim)
    k = _normal(rng, total_slots * num_kv_heads * head_dim, kv_scale, dtype).reshape(
        total_slots, num_kv_heads, head_dim)
    v = _normal(rng, total_slots * num_kv_heads * head_dim, kv_scale, dtype).reshape(
        total_slots, num_kv_heads, head_dim)
    logits = _normal(rng, T * vocab, logit_scale, dtype).reshape(T, vocab)
    draft = plant_tokens(rng, logits, dtype, node_start, parent, accept_prob, distinct_siblings)
    return Workload(name=name, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                    head_dim=head_dim, vocab=vocab, sm_scale=float(sm_scale), node_start=node_start,
                    parent=parent, kv_start=kv_start, prefix_len=prefix_len, total_slots=total_slots,
                    q=q, k=k, v=v, logits=logits, draft=draft, accept_prob=accept_prob)


def plant_tokens(rng, logits, dtype, node_start, parent, p, distinct_siblings=False) -> np.ndarray:
    """Draft tokens: for each non-root node, with probability p the parent's greedy token,
    otherwise a token drawn uniformly from the rest of the vocabulary.  Root tokens are uniform."""
    T, V = logits.shape
    B = len(node_start) - 1
    rows = bf16_bits_to_f32(logits) if dtype == BF16 else logits
    greedy = np.array([int(np.argmax(rows[r])) for r in range(T)], dtype=np.int64) if T else np.zeros(0)
    u = rng.random(T)
    alt = rng.integers(0, max(V - 1, 1), T)
    root_tok = rng.integers(0, V, max(B, 1))
    draft = np.zeros(T, dtype=np.int32)
    for b in range(B):
        s, e = int(node_start[b]), int(node_start[b + 1])
        draft[s] = root_tok[b]
        taken = set()  # parents one of whose children already carries the greedy token
        for i in range(1, e - s):
            par = int(parent[s + i])
            g = int(greedy[s + par])
            if u[s + i] < p and not (distinct_siblings and par in taken):
                tok = g
                taken.add(par)
            else:
                tok = int(alt[s + i])
                tok = tok + 1 if tok >= g else tok
            draft[s + i] = tok
    return draft


# ---------------------------------------------------------------------------------------------
# The five workloads of the verification step.

WORKLOADS = ("tiny", "c1x4k", "c8", "c512", "c128k")
SEEDS = {"tiny": 1001, "c1x4k": 1002, "c8": 1003, "c512": 1004, "c128k": 1005}


def make_config(name: str, seed: Optional[int] = None) -> Workload:
    seed = SEEDS[name] if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    if name == "tiny":
        return make_workload(name, seed, prefix_lens=[256], trees=[chain_tree(4)], num_q_heads=8,
                             num_kv_heads=2, head_dim=64, dtype=F32, vocab=1024, q_scale=1.0,
                             logit_scale=1.0, accept_prob=0.7, rng=rng)
    if name == "c1x4k":
        return make_workload(name, seed, prefix_lens=[4096], nodes=[16], rng=rng)
    if name == "c8":
        lens = rng.integers(1024, 8192 + 1, 8)
        return make_workload(name, seed, prefix_lens=lens, nodes=[16] * 8, rng=rng)
    if name == "c512":
        lens = rng.integers(512, 4096 + 1, 512)
        return make_workload(name, seed, prefix_lens=lens, nodes=[4] * 512, accept_prob=0.5, rng=rng)
    if name == "c128k":
        return make_workload(name, seed, prefix_lens=[131072], nodes=[16], rng=rng)
    raise KeyError(name)


def paged_layout(w: Workload, page_size: int, seed: int, spare_pages: int = 3):
    """The workload's caches scattered over randomly placed pages of a pool: returns (k_pool,
    v_pool, block_table [B, width] int32).  Sequence b's token t (prefix, then tree node t - L)
    is copied to pool row block_table[b, t // page_size] * page_size + t % page_size; every page
    is used by one sequence at most, unused pool rows and table entries hold garbage."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ntok = [int(w.prefix_len[b]) + int(w.node_start[b + 1] - w.node_start[b]) for b in range(w.batch)]
    need = [(n + page_size - 1) // page_size for n in ntok]
    total = sum(need) + spare_pages
    order = rng.permutation(total).astype(np.int32)
    width = max(need) + 1
    bt = np.full((w.batch, width), -7, np.int32)
    shape = (total * page_size,) + w.k.shape[1:]
    if w.k.dtype == np.uint16:
        pool_k = rng.integers(0, 1 << 14, shape, dtype=np.uint16)
        pool_v = rng.integers(0, 1 << 14, shape, dtype=np.uint16)
    else:
        pool_k = rng.integers(0, 1 << 14, shape).astype(w.k.dtype)
        pool_v = rng.integers(0, 1 << 14, shape).astype(w.v.dtype)
    nxt = 0
    for b in range(w.batch):
        bt[b, :need[b]] = order[nxt:nxt + need[b]]
        nxt += need[b]
        t = np.arange(ntok[b], dtype=np.int64)
        rows = bt[b, t // page_size].astype(np.int64) * page_size + t % page_size
        pool_k[rows] = w.k[int(w.kv_start[b]) + t]
        pool_v[rows] = w.v[int(w.kv_start[b]) + t]
    return pool_k, pool_v, bt


def describe(w: Workload) -> dict:
    return {"workload": w.name, "batch": w.batch, "tree_nodes": w.total_nodes,
            "prefix_tokens": int(w.prefix_len.sum()), "q_heads": w.num_q_heads,
            "kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "vocab": w.vocab,
            "kv_dtype": "bf16" if w.dtype == BF16 else "f32"}
