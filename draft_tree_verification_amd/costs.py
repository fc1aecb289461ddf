"""Measured verification cost of the draft-tree step on this GPU.

EAGLE-4's tree is hardware-aware: a harness measures, on the hardware it runs on, what drafting
and verification cost, and sizes the tree (how many tokens, how many branches) for each batch
size from those measurements (aiposthub.com analysis, section "EAGLE-4 是什麼？先看推測解碼為什麼能變快";
arex-research.com release note, section "投机树多大，由实测成本决定", whose packaged schedule narrows
the verification width from 16 to 4 once the batch reaches 20).  This module measures the
verification half with this library's kernels: one whole verify step (ev_verify_step: tree
attention, its split merge together with the per-node argmax, then acceptance and KV compaction, on
one stream) for every (batch, tree
nodes, prefix length) of a grid, on synthetic inputs already in HBM, captured in a HIP graph and
timed with device events around its replays (device time, no host launch overhead).  Draft tokens
are random, so nearly every sequence accepts only its root and compaction moves little.
It needs no model weights.  Tree sizing from the table needs the drafter's cost as well, which
the caller supplies (choose_nodes).

    python -m draft_tree_verification_amd.costs [--batches 1,8,64] [--nodes 4,16] [--prefix 4096]
                                                [--out table.json] [--markdown table.md]

cost_profiles/mi355x.json holds the default grid measured on one MI355X (40 q heads, 8 KV heads,
head_dim 128, bf16, vocab 151936); VerifyCostTable.packaged() loads it.
"""
from __future__ import annotations

import argparse
import bisect
import json
import math
import os
import sys
from dataclasses import asdict, dataclass
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import synth

MALL_BYTES = 256 << 20


@dataclass
class CostRow:
    batch: int
    nodes: int
    prefix: int
    step_us: float        # whole verify step, median of the trials
    attention_us: float   # tree attention (incl. its split merge) alone
    kv_bytes: int         # K/V bytes the attention reads

    @property
    def tree_tokens_per_s(self) -> float:
        return self.batch * self.nodes / (self.step_us * 1e-6)


class VerifyCostTable:
    """Measured verify-step costs, with interpolation between grid points: piecewise linear in
    log(prefix length) for each measured (batch, nodes), then piecewise linear in batch; exact at
    grid points, clamped to the nearest measured value outside the grid."""

    def __init__(self, rows: Sequence[CostRow]):
        self.rows = list(rows)
        self._by: Dict[Tuple[int, int], List[Tuple[int, float]]] = {}
        for r in self.rows:
            self._by.setdefault((r.nodes, r.batch), []).append((r.prefix, r.step_us))
        for v in self._by.values():
            v.sort()

    @staticmethod
    def _interp(xs: Sequence[float], ys: Sequence[float], x: float) -> float:
        if x <= xs[0]:
            return ys[0]
        if x >= xs[-1]:
            return ys[-1]
        i = bisect.bisect_right(xs, x)
        t = (x - xs[i - 1]) / (xs[i] - xs[i - 1])
        return ys[i - 1] + t * (ys[i] - ys[i - 1])

    def nodes_measured(self) -> List[int]:
        return sorted({n for n, _ in self._by})

    def cost_us(self, batch: int, nodes: int, prefix: int) -> float:
        """Verify-step time for `batch` sequences of `nodes` tree nodes over `prefix` tokens."""
        batches = sorted(b for n, b in self._by if n == nodes)
        if not batches:
            raise KeyError(f"no measurements with {nodes} tree nodes")
        per_batch = []
        for b in batches:
            pts = self._by[(nodes, b)]
            per_batch.append(self._interp([math.log(max(p, 1)) for p, _ in pts], [c for _, c in pts],
                                          math.log(max(prefix, 1))))
        return self._interp([float(b) for b in batches], per_batch, float(batch))

    def to_json(self) -> str:
        return json.dumps([asdict(r) for r in self.rows], indent=1)

    @classmethod
    def from_json(cls, text: str) -> "VerifyCostTable":
        return cls([CostRow(**d) for d in json.loads(text)])

    @classmethod
    def packaged(cls, device: str = "mi355x") -> "VerifyCostTable":
        """The table measured with this library on one GPU of the named kind and shipped with it
        (the release note has MI355X pick a packaged cost profile by itself)."""
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "cost_profiles", f"{device}.json")
        with open(path) as f:
            return cls.from_json(f.read())

    def markdown(self) -> str:
        lines = ["| batch | tree nodes | prefix | step us | attention us | tree tokens/s | KV GB/s |",
                 "|---:|---:|---:|---:|---:|---:|---:|"]
        for r in sorted(self.rows, key=lambda r: (r.prefix, r.nodes, r.batch)):
            lines.append(f"| {r.batch} | {r.nodes} | {r.prefix} | {r.step_us:.1f} | {r.attention_us:.1f} | "
                         f"{r.tree_tokens_per_s:.3g} | {r.kv_bytes / (r.attention_us * 1e3):.0f} |")
        return "\n".join(lines)


def choose_nodes(table: VerifyCostTable, batch: int, prefix: int, expected_accept: Callable[[int], float],
                 draft_us: Callable[[int, int], float], candidates: Optional[Sequence[int]] = None) -> int:
    """The tree size with the most accepted tokens per unit of time:
    argmax_N expected_accept(N) / (draft_us(batch, N) + verify cost(batch, N, prefix)).
    expected_accept(N) is the mean tokens a step emits with an N-node tree (root and bonus
    included) and draft_us the drafter's time for it, both from the caller's own measurements."""
    best, best_rate = None, -1.0
    for n in candidates or table.nodes_measured():
        rate = expected_accept(n) / (draft_us(batch, n) + table.cost_us(batch, n, prefix))
        if rate > best_rate:
            best, best_rate = n, rate
    return best


# ------------------------------------------------------------------------------------------ GPU
def _inputs(batch: int, nodes: int, prefix: int, *, sets: int, hq: int, hkv: int, d: int, vocab: int, seed: int):
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    rng = np.random.Generator(np.random.PCG64(seed))
    parents = np.concatenate([synth.random_tree(rng, nodes, 6) for _ in range(batch)]).astype(np.int32)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    slots = batch * (prefix + nodes)
    meta = dict(node_start=i32(np.arange(batch + 1) * nodes), parent=i32(parents),
                kv_start=i32(np.arange(batch) * (prefix + nodes)), prefix_len=i32(np.full(batch, prefix)),
                draft=i32(rng.integers(0, vocab, batch * nodes)))
    T = batch * nodes
    data = []
    for _ in range(sets):
        data.append(dict(
            q=(torch.randn((T, hq, d), generator=g, device="cuda") / math.sqrt(d)).to(torch.bfloat16),
            k=torch.randn((slots, hkv, d), generator=g, device="cuda").to(torch.bfloat16),
            v=torch.randn((slots, hkv, d), generator=g, device="cuda").to(torch.bfloat16),
            logits=(2 * torch.randn((T, vocab), generator=g, device="cuda")).to(torch.bfloat16)))
    return meta, data


def _time(fn, sets: int, iters: int, warmup: int, trials: int) -> float:
    """Device time per call of fn(set index): the calls are captured into one HIP graph (every set,
    repeated) and the graph is replayed, so host launch overhead does not enter the figure."""
    import torch
    for i in range(max(warmup, sets)):  # eager calls first: they allocate every output and workspace
        fn(i % sets)
    torch.cuda.synchronize()
    reps = max(1, iters // sets)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            for i in range(sets):
                fn(i)
    g.replay()
    torch.cuda.synchronize()
    res = []
    for _ in range(trials):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(4):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) * 1e3 / (4 * reps * sets))
    del g
    return float(np.median(res))


def measure(batch: int, nodes: int, prefix: int, *, hq: int = 40, hkv: int = 8, d: int = 128, vocab: int = 151936,
            iters: int = 20, warmup: int = 5, trials: int = 3, seed: int = 0) -> CostRow:
    """Time one (batch, nodes, prefix) point: the whole verify step and the attention alone."""
    import torch
    from . import ev
    kv_bytes = 2 * batch * (prefix + nodes) * hkv * d * 2
    per_set = kv_bytes + batch * nodes * vocab * 2
    sets = max(1, min(8, math.ceil(2 * MALL_BYTES / per_set)))
    meta, data = _inputs(batch, nodes, prefix, sets=sets, hq=hq, hkv=hkv, d=d, vocab=vocab, seed=seed)
    state = [dict() for _ in range(sets)]
    scale = 1.0 / math.sqrt(d)

    def step(i):
        x = data[i]
        ev.verify_step(x["q"], x["k"], x["v"], x["logits"], meta["node_start"], meta["parent"], meta["kv_start"],
                       meta["prefix_len"], meta["draft"], max_nodes=nodes, sm_scale=scale, state=state[i])

    def attention(i):
        x = data[i]
        st = state[i]
        # (the workspace is kept: a new one per call would add its zero-fill to the timed work)
        _, _, st["attn_ws"] = ev.tree_attention(x["q"], x["k"], x["v"], meta["node_start"], meta["parent"],
                                                meta["kv_start"], meta["prefix_len"], max_nodes=nodes,
                                                sm_scale=scale, out=st.get("out"), lse=st.get("lse"),
                                                workspace=st.get("attn_ws"))

    step_us = _time(step, sets, iters, warmup, trials)
    attn_us = _time(attention, sets, iters, warmup, trials)
    err = int(state[0]["err"].item())
    if err:
        raise RuntimeError(f"data error flag {err} at batch={batch} nodes={nodes} prefix={prefix}")
    del data, state
    torch.cuda.empty_cache()
    return CostRow(batch, nodes, prefix, step_us, attn_us, kv_bytes)


def sweep(batches: Sequence[int], nodes: Sequence[int], prefixes: Sequence[int], *, max_kv_tokens: int = 2_200_000,
          max_tree_tokens: int = 8192, log=print, **kw) -> VerifyCostTable:
    """Measure every grid point whose batch * prefix and batch * nodes stay within the caps."""
    rows = []
    for L in prefixes:
        for n in nodes:
            for b in batches:
                if b * (L + n) > max_kv_tokens or b * n > max_tree_tokens:
                    continue
                r = measure(b, n, L, **kw)
                rows.append(r)
                log(f"batch {b:4d} nodes {n:3d} prefix {L:6d}: step {r.step_us:8.1f} us  "
                    f"attention {r.attention_us:8.1f} us  {r.tree_tokens_per_s:.3g} tree tokens/s")
    return VerifyCostTable(rows)


def _ints(s: str) -> List[int]:
    return [int(x) for x in s.split(",") if x]


def main(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--batches", default="1,2,4,8,16,32,64,128,256,512")
    p.add_argument("--nodes", default="4,8,16,32,64")
    p.add_argument("--prefix", default="1024,4096,16384")
    p.add_argument("--iters", type=int, default=20)
    p.add_argument("--out", default=None, help="write the table as JSON")
    p.add_argument("--markdown", default=None, help="write the table as a markdown table")
    a = p.parse_args(argv)
    t = sweep(_ints(a.batches), _ints(a.nodes), _ints(a.prefix), iters=a.iters,
              log=lambda s: print(s, flush=True))
    if a.out:
        with open(a.out, "w") as f:
            f.write(t.to_json())
    if a.markdown:
        with open(a.markdown, "w") as f:
            f.write(t.markdown() + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
