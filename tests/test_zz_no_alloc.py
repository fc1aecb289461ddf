"""The allocation-free attention entry point (ev_tree_attention_noalloc, workspace in a static
device array) against ev_tree_attention with a caller workspace, through the C ABI: two calls in a
row on one GPU -- a large batch, then a smaller input that leaves stale partials of the first call
in the shared array -- each bit-identical to the workspace call and within the attention bar of
the oracle."""
import numpy as np
import pytest

from draft_tree_verification_amd import synth

from . import gpu_util as gu

pytestmark = pytest.mark.gpu


def _raw_attention(w, d, noalloc):
    """One call through the C ABI; out/lse start as NaN so unwritten rows show."""
    import torch
    from draft_tree_verification_amd import ev
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full((w.total_nodes, w.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    p = lambda t: t.data_ptr()
    stream = torch.cuda.current_stream().cuda_stream
    dt = 0 if w.dtype == synth.BF16 else 1
    common = (p(d["q"]), p(d["k"]), p(d["v"]), p(out), p(lse), p(d["node_start"]), p(d["parent"]), p(d["kv_start"]),
              p(d["prefix_len"]), w.batch, w.total_nodes, max(w.max_nodes, 1), w.total_slots, w.num_q_heads,
              w.num_kv_heads, w.head_dim, dt, w.sm_scale)
    if noalloc:
        st = ev.ev_tree_attention_noalloc(*common, p(err), stream)
    else:
        nbytes = ev.ev_tree_attention_workspace_size(w.batch, max(w.max_nodes, 1), w.num_q_heads, w.num_kv_heads,
                                                     w.head_dim)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        st = ev.ev_tree_attention(*common, p(ws), nbytes, p(err), stream)
    assert st == 0, ev.ev_status_string(st)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return gu.to_host(out), lse.cpu().numpy()


def test_noalloc_two_calls_match_workspace_call():
    big = gu.cached_config("c8")
    small = synth.make_workload("noalloc_small", 5, prefix_lens=[0, 3, 700, 129, 2049], nodes=[16, 1, 9, 16, 4],
                                vocab=64, slot_gap=2)
    assert small.total_nodes < big.total_nodes
    for w, name in ((big, "c8"), (small, "small ragged batch")):
        gu.log(f"[case] noalloc attention {name} (B={w.batch}, T={w.total_nodes})")
        d = gu.dev_workload(w)
        o_na, l_na = _raw_attention(w, d, noalloc=True)
        o_ws, l_ws = _raw_attention(w, d, noalloc=False)
        assert o_na.tobytes() == o_ws.tobytes(), f"{name}: outputs differ from the workspace call"
        assert l_na.tobytes() == l_ws.tobytes(), f"{name}: lse differs from the workspace call"
        ref, ref_lse, err = gu.oracle_attention(w)
        assert (err == 0).all()
        gu.check_attention(o_na, ref, l_na, ref_lse, vmax=float(np.abs(gu.widen(w.v)).max()),
                           what=f"noalloc {name}")
