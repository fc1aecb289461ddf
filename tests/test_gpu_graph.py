"""The whole verification step captured in a HIP graph: every replay, with eager work and
synchronizations between replays, reproduces the eager step bit for bit (outputs, tokens,
acceptance, compacted caches).  The library records no memset and allocates nothing inside a
call, so the captured kernels are the whole step."""
import pytest

from . import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,T", [("c1x4k", 0.0), ("c8", 0.0), ("c8", 0.8)])
def test_verify_step_graph_replays(name, T):
    import torch
    from draft_tree_verification_amd import ev
    gu.log(f"[case] graph replay {name} T={T}")
    w = gu.cached_config(name)
    d = gu.dev_workload(w)
    k0, v0 = d["k"].clone(), d["v"].clone()
    state = {}

    def step():
        ev.verify_step(d["q"], d["k"], d["v"], d["logits"], d["node_start"], d["parent"], d["kv_start"],
                       d["prefix_len"], d["draft"], max_nodes=w.max_nodes, sm_scale=w.sm_scale, temperature=T,
                       seed=9, offset=3, state=state)

    step()  # eager: allocates every output and workspace
    torch.cuda.synchronize()
    assert int(state["err"].item()) == 0
    ref = {"out": state["out"].clone(), "lse": state["lse"].clone(), "target": state["target"].clone(),
           "new_len": state["new_len"].clone(), "k": d["k"].clone(), "v": d["v"].clone()}
    ref.update({key: t.clone() for key, t in state["accept"].items()})

    d["k"].copy_(k0)
    d["v"].copy_(v0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        # eager work between replays: restore the caches (compaction is in place), poison outputs
        d["k"].copy_(k0)
        d["v"].copy_(v0)
        state["out"].fill_(7.0)
        state["lse"].fill_(-3.0)
        state["target"].fill_(-9)
        state["new_len"].fill_(-9)
        for t in state["accept"].values():
            t.fill_(-9)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(state["err"].item()) == 0
        for key in ("out", "lse", "target", "new_len"):
            assert torch.equal(state[key], ref[key]), f"replay {r}: {key}"
        for key, t in state["accept"].items():
            assert torch.equal(t, ref[key]), f"replay {r}: {key}"
        assert torch.equal(d["k"], ref["k"]) and torch.equal(d["v"], ref["v"]), f"replay {r}: caches"
    gu.log(f"[graph] {name} T={T}: 3 replays bit-identical to the eager step")
