"""The whole verification step (ev_verify_step, one stream) against the oracle on every workload,
in the launch configuration the benchmark times; and the sampled step (temperature > 0)."""
import numpy as np
import pytest

import oracle

from . import gpu_util as gu

pytestmark = pytest.mark.gpu


def _tree_rows(w, cache: np.ndarray) -> np.ndarray:
    """The tree-slot rows of every sequence, concatenated: [sum N, Hkv, D]."""
    idx = np.concatenate([np.arange(w.kv_start[b] + w.prefix_len[b],
                                    w.kv_start[b] + w.prefix_len[b] + w.nodes_per_seq[b]) for b in range(w.batch)])
    return cache[idx]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny", "c1x4k", "c8", "c512", "c128k"])
def test_verify_step(name):
    import torch
    from draft_tree_verification_amd import ev
    gu.log(f"[case] verify step {name}")
    w = gu.cached_config(name)
    d = gu.dev_workload(w)
    k0, v0 = d["k"].clone(), d["v"].clone()
    st = ev.verify_step(d["q"], d["k"], d["v"], d["logits"], d["node_start"], d["parent"], d["kv_start"],
                        d["prefix_len"], d["draft"], max_nodes=w.max_nodes, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    assert int(st["err"].item()) == 0

    # 1. attention: every row (the large workloads' oracle rows are computed once per process)
    ref, ref_lse = gu.oracle_full(name)
    gu.check_attention(gu.to_host(st["out"]), ref, gu.to_host(st["lse"]), ref_lse,
                       vmax=float(np.abs(gu.widen(w.v)).max()), what=f"step {name}", tight=w.dtype == 0)

    # 2. argmax, 3. acceptance: bit-exact
    tgt, _ = oracle.node_argmax(w.logits)
    assert np.array_equal(st["target"].cpu().numpy(), tgt)
    r = oracle.greedy_accept(w.node_start, w.parent, w.draft, tgt, w.max_nodes, w.vocab)
    for key in ("accept_len", "accept_path", "bonus", "out_tokens"):
        assert np.array_equal(st["accept"][key].cpu().numpy(), r[key]), key
    gu.log(f"[step] {name}: mean accept_len {r['accept_len'].mean():.3f}")

    # 4. compaction: bit-exact.  Prefix rows must be untouched (compared on the device against the
    # pre-call copy); the tree-slot rows are compared with the oracle's out-of-place compaction of
    # the same rows, each sequence's tree slots taken on their own (prefix length 0).
    assert np.array_equal(st["new_len"].cpu().numpy(), w.prefix_len + r["accept_len"])
    tree_mask = torch.zeros(w.total_slots, dtype=torch.bool, device="cuda")
    for b in range(w.batch):
        lo = int(w.kv_start[b] + w.prefix_len[b])
        tree_mask[lo:lo + int(w.nodes_per_seq[b])] = True
    for cur, orig in ((d["k"], k0), (d["v"], v0)):
        assert torch.equal(cur[~tree_mask], orig[~tree_mask]), "compaction touched non-tree slots"
    n = w.nodes_per_seq
    starts = np.concatenate([[0], np.cumsum(n)])[:-1].astype(np.int32)
    for cur, src in ((d["k"], w.k), (d["v"], w.v)):
        tree_src = _tree_rows(w, src)
        exp, _, nl, err = oracle.compact_kv(tree_src[None], tree_src[None], starts, np.zeros(w.batch, np.int32),
                                            r["accept_len"], r["accept_path"], num_layers=1,
                                            total_slots=tree_src.shape[0], num_kv_heads=w.num_kv_heads,
                                            head_dim=w.head_dim)
        got = _tree_rows(w, gu.to_host(cur))
        assert (err == 0).all() and np.array_equal(got, exp[0]), "compacted tree rows differ"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("T", [1.0, 0.6])
def test_verify_step_sampled(T):
    """Sampled step on the 8-sequence workload: the draws match the oracle's (up to near ties of
    the hardware log2), and acceptance and compaction are bit-exact against the oracle on the
    GPU's own draws."""
    import torch
    from draft_tree_verification_amd import ev
    gu.log(f"[case] verify step c8 sampled T={T}")
    w = gu.cached_config("c8")
    d = gu.dev_workload(w)
    st = ev.verify_step(d["q"], d["k"], d["v"], d["logits"], d["node_start"], d["parent"], d["kv_start"],
                        d["prefix_len"], d["draft"], max_nodes=w.max_nodes, sm_scale=w.sm_scale, temperature=T,
                        seed=31, offset=4)
    torch.cuda.synchronize()
    assert int(st["err"].item()) == 0
    draws = st["target"].cpu().numpy()
    ref, ref_score = oracle.node_sample(w.logits, T, 31, 4)
    bad = np.nonzero(draws != ref)[0]
    z = gu.widen(w.logits)
    for r in bad:
        s_g = oracle.sample_score(float(z[r, draws[r]]), T, 31, 4, int(r), int(draws[r]))
        assert s_g >= float(ref_score[r]) - 1e-5 - 8 * np.spacing(np.float32(max(1.0, abs(float(ref_score[r]))))), r
    assert len(bad) <= 1
    r = oracle.sampled_accept(w.node_start, w.parent, w.draft, draws, w.max_nodes, w.vocab)
    for key in ("accept_len", "accept_path", "bonus", "out_tokens"):
        assert np.array_equal(st["accept"][key].cpu().numpy(), r[key]), key
    kx, vx, nl, err = oracle.compact_kv(w.k[None], w.v[None], w.kv_start, w.prefix_len, r["accept_len"],
                                        r["accept_path"], num_layers=1, total_slots=w.total_slots,
                                        num_kv_heads=w.num_kv_heads, head_dim=w.head_dim)
    assert (err == 0).all() and np.array_equal(st["new_len"].cpu().numpy(), nl)
    assert np.array_equal(gu.to_host(d["k"]), kx[0]) and np.array_equal(gu.to_host(d["v"]), vx[0])
    gu.log(f"[step] sampled T={T}: mean accept_len {r['accept_len'].mean():.3f}")
