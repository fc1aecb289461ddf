"""Independent formulations used to pin the oracle (test infrastructure).

Nothing here calls the oracle or the GPU library.  Each function computes the same quantity
as an oracle function by a different route:
  - the ancestor relation as the reflexive-transitive closure of the child->parent edge matrix
    (repeated boolean matrix products), instead of walking parent pointers;
  - attention as dense textbook softmax over gathered rows, and through torch's
    scaled_dot_product_attention with an explicit boolean mask;
  - acceptance by enumerating every root-to-node path, instead of a forward pass over nodes.
"""
from __future__ import annotations

import numpy as np

from draft_tree_verification_amd.synth import BF16, bf16_bits_to_f32


def as_f64(x: np.ndarray, dtype: int) -> np.ndarray:
    return (bf16_bits_to_f32(x) if dtype == BF16 else np.asarray(x, np.float32)).astype(np.float64)


def ancestor_closure(parent) -> np.ndarray:
    """M[i, j] is True iff j is i or an ancestor of i."""
    parent = np.asarray(parent)
    n = len(parent)
    A = np.zeros((n, n), dtype=np.int64)
    for i in range(1, n):
        A[i, parent[i]] = 1
    M = np.eye(n, dtype=bool)
    P = np.eye(n, dtype=np.int64)
    for _ in range(n):
        P = (P @ A > 0).astype(np.int64)
        if not P.any():
            break
        M |= P.astype(bool)
    return M


def depths(parent) -> np.ndarray:
    return ancestor_closure(parent).sum(axis=1) - 1


def visible_mask(parent, prefix_len: int) -> np.ndarray:
    """Boolean [N, L + N]: which cache positions (relative to the sequence start) each node sees."""
    M = ancestor_closure(parent)
    n = len(parent)
    return np.concatenate([np.ones((n, prefix_len), dtype=bool), M], axis=1)


def attention_seq(w, b: int, sm_scale: float = None, heads=None):
    """Dense textbook attention for every node of sequence b: out [N, Hq, D], lse [N, Hq] (fp64)."""
    sm_scale = w.sm_scale if sm_scale is None else sm_scale
    s, e = int(w.node_start[b]), int(w.node_start[b + 1])
    L, s0 = int(w.prefix_len[b]), int(w.kv_start[b])
    n = e - s
    mask = visible_mask(w.parent[s:e], L)
    K = as_f64(w.k[s0:s0 + L + n], w.dtype)
    V = as_f64(w.v[s0:s0 + L + n], w.dtype)
    Q = as_f64(w.q[s:e], w.dtype)
    G = w.num_q_heads // w.num_kv_heads
    heads = range(w.num_q_heads) if heads is None else heads
    out = np.full((n, w.num_q_heads, w.head_dim), np.nan)
    lse = np.full((n, w.num_q_heads), np.nan)
    for h in heads:
        g = h // G
        S = (Q[:, h, :] @ K[:, g, :].T) * sm_scale          # [N, L+N]
        S = np.where(mask, S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        P = np.exp(S - m)
        Z = P.sum(axis=1, keepdims=True)
        out[:, h, :] = (P @ V[:, g, :]) / Z
        lse[:, h] = (m + np.log(Z))[:, 0]
    return out, lse


def attention_seq_sdpa(w, b: int, sm_scale: float = None, mask: np.ndarray = None):
    """The same rows through torch.nn.functional.scaled_dot_product_attention (CPU, float64)."""
    import torch
    import torch.nn.functional as F
    sm_scale = w.sm_scale if sm_scale is None else sm_scale
    s, e = int(w.node_start[b]), int(w.node_start[b + 1])
    L, s0 = int(w.prefix_len[b]), int(w.kv_start[b])
    n = e - s
    if mask is None:
        mask = visible_mask(w.parent[s:e], L)
    G = w.num_q_heads // w.num_kv_heads
    q = torch.from_numpy(as_f64(w.q[s:e], w.dtype)).permute(1, 0, 2).unsqueeze(0)       # [1,Hq,N,D]
    k = torch.from_numpy(as_f64(w.k[s0:s0 + L + n], w.dtype)).permute(1, 0, 2)            # [Hkv,L+N,D]
    v = torch.from_numpy(as_f64(w.v[s0:s0 + L + n], w.dtype)).permute(1, 0, 2)
    k = k.repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
    v = v.repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=torch.from_numpy(mask), scale=sm_scale)
    return o[0].permute(1, 0, 2).numpy()


def accept_paths(parent, draft, target):
    """Enumerate every root-to-node path whose edges all agree (draft[child] == target[parent]);
    return the one maximising (length, -last node) as (len, path, bonus, out_tokens)."""
    parent = [int(x) for x in parent]
    n = len(parent)
    children = {i: [] for i in range(n)}
    for i in range(1, n):
        children[parent[i]].append(i)
    best = [0]
    stack = [[0]]
    while stack:
        path = stack.pop()
        if (len(path), -path[-1]) > (len(best), -best[-1]):
            best = path
        u = path[-1]
        for c in children[u]:
            if int(draft[c]) == int(target[u]):
                stack.append(path + [c])
    bonus = int(target[best[-1]])
    out = [int(draft[j]) for j in best[1:]] + [bonus]
    return len(best), best, bonus, out


def sampled_accept_paths(parent, draft, target):
    """Sampled acceptance from the set of accepted nodes (not a walk): node c is accepted when its
    parent p is, draft[c] == target[p], and no sibling j < c holds the same drafted token.  The
    accepted nodes then form one root path (checked); its last node ends the round.
    Returns (len, path, bonus, out_tokens)."""
    parent = [int(x) for x in parent]
    n = len(parent)
    acc = [False] * n
    acc[0] = True
    for c in range(1, n):
        p = parent[c]
        first = all(not (parent[j] == p and int(draft[j]) == int(draft[c])) for j in range(1, c))
        acc[c] = acc[p] and int(draft[c]) == int(target[p]) and first
    nodes = [i for i in range(n) if acc[i]]
    for c in nodes[1:]:
        assert acc[parent[c]], "accepted set is not closed under parents"
    kids = [sum(1 for c in nodes if c > 0 and parent[c] == u) for u in range(n)]
    assert max(kids) <= 1, "more than one accepted child of a node"
    last = max(nodes)
    path = []
    j = last
    while j >= 0:
        path.append(j)
        j = parent[j]
    path = path[::-1]
    assert path == sorted(nodes), "accepted nodes are not one root path"
    bonus = int(target[last])
    out = [int(draft[j]) for j in path[1:]] + [bonus]
    return len(path), path, bonus, out


def load_cases(path: str):
    """Parse a ';'-separated golden file into lists of int lists (first column kept as text)."""
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            cols = [c.strip() for c in line.split(";")]
            rows.append([cols[0]] + [[int(x) for x in c.split()] for c in cols[1:]])
    return rows
