"""The Python binding refuses caller-supplied outputs of the wrong shape, dtype or layout (and
metadata of inconsistent lengths) with an exception, before anything is launched: a kernel
would otherwise write past the end of a short buffer."""
import pytest

from draft_tree_verification_amd import synth

from . import gpu_util as gu

pytestmark = pytest.mark.gpu


def _tiny():
    w = synth.make_workload("bind", 97, prefix_lens=[20, 9], nodes=[4, 3], vocab=64)
    return w, gu.dev_workload(w)


def test_attention_outputs_checked():
    import torch
    from draft_tree_verification_amd import ev
    gu.log("[case] binding checks: attention")
    w, d = _tiny()
    T, Hq, D = d["q"].shape
    args = (d["q"], d["k"], d["v"], d["node_start"], d["parent"], d["kv_start"], d["prefix_len"])
    kw = dict(max_nodes=4, sm_scale=w.sm_scale)
    bad = [dict(out=torch.empty((T - 1, Hq, D), dtype=d["q"].dtype, device="cuda")),
           dict(out=torch.empty((T, Hq, D), dtype=torch.float32, device="cuda")),
           dict(out=torch.empty((T, D, Hq), dtype=d["q"].dtype, device="cuda").transpose(1, 2)),
           dict(lse=torch.empty((T, Hq - 1), dtype=torch.float32, device="cuda")),
           dict(err_flag=torch.zeros(1, dtype=torch.int64, device="cuda")),
           dict(out=torch.empty((T, Hq, D), dtype=d["q"].dtype))]          # host memory
    for extra in bad:
        with pytest.raises((ValueError, TypeError)):
            ev.tree_attention(*args, **kw, **extra)
    out, lse, _ = ev.tree_attention(*args, **kw, out=torch.empty_like(d["q"]),
                                    lse=torch.empty((T, Hq), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all()


def test_selection_outputs_checked():
    import torch
    from draft_tree_verification_amd import ev
    gu.log("[case] binding checks: selection, acceptance, compaction")
    w, d = _tiny()
    T, B = d["parent"].shape[0], d["prefix_len"].shape[0]
    i32 = dict(dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        ev.node_argmax(d["logits"], target=torch.empty(T + 1, **i32))
    with pytest.raises(ValueError):
        ev.node_sample(d["logits"], temperature=1.0, seed=1, offset=0, target=torch.empty(T - 1, **i32))
    tgt, _, _ = ev.node_argmax(d["logits"])
    with pytest.raises(ValueError):
        ev.greedy_accept(d["node_start"], d["parent"], d["draft"], tgt, max_nodes=4, vocab=w.vocab,
                         out={"accept_len": torch.empty(B, **i32), "accept_path": torch.empty((B, 3), **i32),
                              "bonus": torch.empty(B, **i32), "out_tokens": torch.empty((B, 4), **i32)})
    with pytest.raises(ValueError):
        ev.greedy_accept(d["node_start"], d["parent"], d["draft"][:-1].contiguous(), tgt, max_nodes=4,
                         vocab=w.vocab)
    acc = ev.greedy_accept(d["node_start"], d["parent"], d["draft"], tgt, max_nodes=4, vocab=w.vocab)
    with pytest.raises(ValueError):
        ev.compact_kv(d["k"], d["v"], d["kv_start"], d["prefix_len"], acc["accept_len"], acc["accept_path"],
                      new_len=torch.empty(B - 1, **i32))
    with pytest.raises(ValueError):
        ev.compact_kv(d["k"], d["v"], d["kv_start"][:1].contiguous(), d["prefix_len"], acc["accept_len"],
                      acc["accept_path"])
    common = (d["logits"], d["node_start"], d["parent"], d["draft"], d["k"], d["v"], d["kv_start"], d["prefix_len"])
    with pytest.raises(ValueError):
        ev.select_accept_compact(*common, max_nodes=4, new_len=torch.empty(B + 1, **i32))
    with pytest.raises(ValueError):
        ev.select_accept_compact(d["logits"][:-1].contiguous(), *common[1:], max_nodes=4)
    with pytest.raises((ValueError, TypeError)):
        ev.select_accept_compact(*common, max_nodes=4, err_flag=torch.zeros(0, **i32))
    torch.cuda.synchronize()
