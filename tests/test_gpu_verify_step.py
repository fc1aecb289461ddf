"""The whole-step call (ev_verify_step: attention, selection, acceptance and compaction in one
call) against the two separate calls it replaces (ev_tree_attention[_strided] +
ev_select_accept_compact) on the same inputs: every output bit-identical, over workloads with and
without split units, greedy and sampled, both cache layouts, and repeated calls on one workspace
with different shapes."""
import numpy as np
import pytest

import oracle

from . import gpu_util as gu

pytestmark = pytest.mark.gpu


def _inputs(w, head_major):
    d = gu.dev_workload(w)
    if head_major:
        d["k"] = d["k"].permute(1, 0, 2).contiguous()
        d["v"] = d["v"].permute(1, 0, 2).contiguous()
    return d


def _separate(w, d, T, seed, offset, head_major):
    import torch
    from draft_tree_verification_amd import ev
    k, v = d["k"].clone(), d["v"].clone()
    out, lse, _ = ev.tree_attention(d["q"], k, v, d["node_start"], d["parent"], d["kv_start"], d["prefix_len"],
                                    max_nodes=w.max_nodes, sm_scale=w.sm_scale, head_major=head_major)
    if head_major:  # compaction of [Hkv][slots][D] as Hkv one-head layers
        kc, vc = k.unsqueeze(2), v.unsqueeze(2)
    else:
        kc, vc = k, v
    tgt, acc, nl, _ = ev.select_accept_compact(d["logits"], d["node_start"], d["parent"], d["draft"], kc, vc,
                                               d["kv_start"], d["prefix_len"], max_nodes=w.max_nodes,
                                               temperature=T, seed=seed, offset=offset)
    torch.cuda.synchronize()
    return out, lse, tgt, acc, nl, k, v


def _whole(w, d, T, seed, offset, head_major, state=None):
    import torch
    from draft_tree_verification_amd import ev
    k, v = d["k"].clone(), d["v"].clone()
    st = ev.verify_step(d["q"], k, v, d["logits"], d["node_start"], d["parent"], d["kv_start"], d["prefix_len"],
                        d["draft"], max_nodes=w.max_nodes, sm_scale=w.sm_scale, temperature=T, seed=seed,
                        offset=offset, head_major=head_major, state=state)
    torch.cuda.synchronize()
    return st, k, v


def _compare(sep, st, k, v, what):
    import torch
    out, lse, tgt, acc, nl, ks, vs = sep
    assert int(st["err"].item()) == 0, what
    assert torch.equal(st["out"], out) and torch.equal(st["lse"], lse), f"{what}: attention differs"
    assert torch.equal(st["target"], tgt), f"{what}: tokens differ"
    for key in ("accept_len", "accept_path", "bonus", "out_tokens"):
        assert torch.equal(st["accept"][key], acc[key]), f"{what}: {key} differs"
    assert torch.equal(st["new_len"], nl), f"{what}: new_len differs"
    assert torch.equal(k, ks) and torch.equal(v, vs), f"{what}: compacted caches differ"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,T,head_major", [("c8", 0.0, False), ("c8", 1.0, False), ("c8", 0.0, True),
                                               ("c1x4k", 0.6, False), ("c128k", 0.0, True), ("c512", 0.0, False),
                                               ("tiny", 0.0, False), ("tiny", 1.0, False)])
def test_whole_step_equals_separate_calls(name, T, head_major):
    gu.log(f"[case] whole step {name} T={T} head_major={head_major}")
    w = gu.cached_config(name)
    d = _inputs(w, head_major)
    sep = _separate(w, d, T, 77, 5, head_major)
    st, k, v = _whole(w, d, T, 77, 5, head_major)
    _compare(sep, st, k, v, name)
    # and the tokens against the oracle's (greedy: exact; sampled: checked by the draw tests)
    if T == 0.0:
        ref, _ = oracle.node_argmax(w.logits)
        assert np.array_equal(st["target"].cpu().numpy(), ref)


@pytest.mark.timeout(600)
def test_repeated_calls_on_one_workspace():
    """Several calls on one workspace, alternating workloads and temperatures: each equals its
    separate calls (nothing a call leaves in the workspace reaches the next)."""
    gu.log("[case] whole step repeated calls")
    state = {}
    for i, (name, T) in enumerate((("c8", 0.0), ("c8", 1.0), ("c1x4k", 0.0), ("c8", 0.0))):
        w = gu.cached_config(name)
        d = _inputs(w, False)
        sep = _separate(w, d, T, 3, i, False)
        if state.get("out") is not None and tuple(state["out"].shape) != tuple(d["q"].shape):
            state = {"step_ws": state["step_ws"]}  # other shapes: keep only the workspace
        st, k, v = _whole(w, d, T, 3, i, False, state=state)
        _compare(sep, st, k, v, f"call {i} {name}")
