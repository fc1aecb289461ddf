"""GPU parity of ev_select_accept_compact (per-node token, acceptance and KV compaction in one call)
against the three separate calls it replaces, bit for bit, and through them against the oracle.
Drafts are planted to agree with the target along random paths, so acceptance reaches deep
nodes and the compaction really moves rows."""
from types import SimpleNamespace

import numpy as np
import pytest

import oracle
from draft_tree_verification_amd import synth
from draft_tree_verification_amd.synth import BF16, F32

from . import gpu_util as gu

pytestmark = pytest.mark.gpu


def _planted(rng, trees, target, vocab, p_agree):
    """Draft tokens: node i copies its parent's target token with probability p_agree."""
    starts = np.concatenate([[0], np.cumsum([len(t) for t in trees])])
    draft = rng.integers(0, vocab, int(starts[-1])).astype(np.int32)
    for b, par in enumerate(trees):
        s0 = starts[b]
        for i in range(1, len(par)):
            if rng.random() < p_agree:
                draft[s0 + i] = target[s0 + par[i]]
    return draft


def _case(seed, B, max_n, vocab, stride, logit_dtype, layers, H, D, cache_dtype, max_prefix=60):
    rng = np.random.default_rng(seed)
    trees = [synth.random_tree(rng, int(rng.integers(1, max_n + 1)), int(rng.integers(1, 8))) for _ in range(B)]
    n = np.array([len(t) for t in trees])
    T = int(n.sum())
    x = rng.normal(0, 2, (T, stride)).astype(np.float32)
    logits = synth.f32_to_bf16_bits(x) if logit_dtype == BF16 else x
    L = rng.integers(0, max_prefix + 1, B).astype(np.int32)
    kv_start = np.concatenate([[0], np.cumsum(L + n)])[:-1].astype(np.int32)
    slots = int((L + n).sum())
    k = rng.integers(0, 1 << 14, (layers, slots, H, D)).astype(cache_dtype)
    v = rng.integers(0, 1 << 14, (layers, slots, H, D)).astype(cache_dtype)
    return dict(trees=trees, node_start=np.concatenate([[0], np.cumsum(n)]).astype(np.int32),
                parent=np.concatenate(trees).astype(np.int32), logits=logits, vocab=vocab, max_nodes=max_n,
                prefix_len=L, kv_start=kv_start, k=k, v=v, rng=rng)


def _dev(c, draft):
    import torch
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    return dict(logits=gu.to_dev(c["logits"]), node_start=i32(c["node_start"]), parent=i32(c["parent"]),
                draft=i32(draft), kv_start=i32(c["kv_start"]), prefix_len=i32(c["prefix_len"]))


def _separate(d, k, v, c, temperature, seed, offset, block_table=None):
    import torch
    from draft_tree_verification_amd import ev
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    if temperature > 0:
        tgt, _ = ev.node_sample(d["logits"], temperature=temperature, seed=seed, offset=offset, vocab=c["vocab"])
    else:
        tgt, _, _ = ev.node_argmax(d["logits"], vocab=c["vocab"])
    accept = ev.sampled_accept if temperature > 0 else ev.greedy_accept
    acc = accept(d["node_start"], d["parent"], d["draft"], tgt, max_nodes=c["max_nodes"], vocab=c["vocab"],
                 err_flag=err)
    if block_table is None:
        nl = ev.compact_kv(k, v, d["kv_start"], d["prefix_len"], acc["accept_len"], acc["accept_path"], err_flag=err)
    else:
        nl = ev.compact_kv_paged(k, v, block_table, d["prefix_len"], acc["accept_len"], acc["accept_path"],
                                 err_flag=err)
    return tgt, acc, nl, err


def _fused(d, k, v, c, temperature, seed, offset, block_table=None, workspace=None):
    import torch
    from draft_tree_verification_amd import ev
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    tgt, acc, nl, ws = ev.select_accept_compact(d["logits"], d["node_start"], d["parent"], d["draft"], k, v,
                                                d["kv_start"], d["prefix_len"], max_nodes=c["max_nodes"],
                                                temperature=temperature, seed=seed, offset=offset, vocab=c["vocab"],
                                                workspace=workspace, err_flag=err, block_table=block_table)
    return tgt, acc, nl, err, ws


def _compare(a, b, what):
    import torch
    ta, acca, nla, erra = a[:4]
    tb, accb, nlb, errb = b[:4]
    torch.cuda.synchronize()
    assert torch.equal(ta, tb), f"{what}: target tokens"
    for key in ("accept_len", "accept_path", "bonus", "out_tokens"):
        assert torch.equal(acca[key], accb[key]), f"{what}: {key}"
    assert torch.equal(nla, nlb), f"{what}: new_len"
    assert int(erra.item()) == int(errb.item()), f"{what}: error flags {int(erra.item())} vs {int(errb.item())}"


def _run(c, temperature=0.0, seed=0, offset=0, p_agree=0.8, what=""):
    """Fused vs separate on the same inputs (caches copied), then the separate path's acceptance and
    compaction against the oracle on the GPU's own tokens.  Returns the mean accepted length."""
    if temperature > 0:
        tref, _ = oracle.node_sample(c["logits"], temperature, seed, offset, vocab=c["vocab"],
                                     row_stride=c["logits"].shape[1])
    else:
        tref, _ = oracle.node_argmax(c["logits"], vocab=c["vocab"], row_stride=c["logits"].shape[1])
    draft = _planted(c["rng"], c["trees"], tref, c["vocab"], p_agree)
    d = _dev(c, draft)
    k1, v1 = gu.to_dev(c["k"]), gu.to_dev(c["v"])
    k2, v2 = k1.clone(), v1.clone()
    sep = _separate(d, k1, v1, c, temperature, seed, offset)
    fus = _fused(d, k2, v2, c, temperature, seed, offset)
    _compare(sep, fus, what)
    assert gu.to_host(k1).tobytes() == gu.to_host(k2).tobytes(), f"{what}: K caches"
    assert gu.to_host(v1).tobytes() == gu.to_host(v2).tobytes(), f"{what}: V caches"
    tgt = fus[0].cpu().numpy()
    accept = oracle.sampled_accept if temperature > 0 else oracle.greedy_accept
    r = accept(c["node_start"], c["parent"], draft, tgt, c["max_nodes"], c["vocab"])
    for key in ("accept_len", "accept_path", "bonus", "out_tokens"):
        assert np.array_equal(fus[1][key].cpu().numpy(), r[key]), f"{what}: oracle {key}"
    layers, slots, H, D = c["k"].shape
    rk, rv, rnl, rerr = oracle.compact_kv(c["k"], c["v"], c["kv_start"], c["prefix_len"], r["accept_len"],
                                          r["accept_path"], num_layers=layers, total_slots=slots, num_kv_heads=H,
                                          head_dim=D)
    assert (rerr == 0).all() and np.array_equal(fus[2].cpu().numpy(), rnl)
    assert np.array_equal(gu.to_host(k2), rk) and np.array_equal(gu.to_host(v2), rv), f"{what}: oracle compaction"
    mean_len = float(r["accept_len"].mean())
    gu.log(f"[fused] {what}: {len(c['trees'])} sequences, mean accept_len {mean_len:.2f}, bit-exact")
    return mean_len


def test_special_logits_full_rounds():
    """Rows long enough for whole rounds of loads, with repeated maxima, NaNs of either sign,
    signed zeros and infinities at random positions: the fused call's tokens (the maximum over a
    row's per-piece words) equal the oracle's argmax, and the step matches the separate calls."""
    gu.log("[case] fused special logits, full rounds")
    c = _case(77, B=6, max_n=16, vocab=151936, stride=151936, logit_dtype=BF16, layers=1, H=2, D=64,
              cache_dtype=np.uint16)
    rng = np.random.default_rng(78)
    T, V = c["logits"].shape
    x = rng.standard_normal((T, V)).astype(np.float32)
    for r in range(T):
        pos = rng.choice(V, size=3, replace=False)
        kind = r % 5
        if kind == 0:
            x[r, pos] = 8.0
        elif kind == 1:
            x[r, pos[0]] = np.float32("nan")
            x[r, pos[1]] = -np.float32("nan")
        elif kind == 2:
            x[r] = -np.abs(x[r]) - 1.0
            x[r, pos[0]] = -0.0
            x[r, pos[1]] = 0.0
        elif kind == 3:
            x[r, pos[:2]] = np.float32("inf")
        else:
            x[r] = -2.5
    c["logits"] = synth.f32_to_bf16_bits(x)
    tref, _ = oracle.node_argmax(c["logits"], vocab=V, row_stride=V)
    draft = _planted(c["rng"], c["trees"], tref, V, 0.8)
    d = _dev(c, draft)
    k1, v1 = gu.to_dev(c["k"]), gu.to_dev(c["v"])
    k2, v2 = k1.clone(), v1.clone()
    sep = _separate(d, k1, v1, c, 0.0, 0, 0)
    fus = _fused(d, k2, v2, c, 0.0, 0, 0)
    _compare(sep, fus, "special logits")
    assert np.array_equal(fus[0].cpu().numpy(), tref), "fused tokens differ from the oracle argmax"
    assert gu.to_host(k1).tobytes() == gu.to_host(k2).tobytes()


@pytest.mark.parametrize("cache_dtype", [np.uint16, np.float32])
def test_greedy_layers(cache_dtype):
    gu.log(f"[case] fused greedy 3 layers {cache_dtype}")
    c = _case(1, 37, 64, 32000, 32000, BF16, 3, 8, 128, cache_dtype)
    assert _run(c, what="greedy bf16 3 layers") > 2


def test_greedy_f32_ragged_vocab():
    gu.log("[case] fused greedy f32 logits, ragged vocabulary")
    c = _case(2, 23, 16, 1001, 1008, F32, 1, 2, 64, np.float32)
    _run(c, what="greedy f32 1001/1008")


def test_many_rows_unsplit():
    """4096 rows: one piece per row (no split), the pieces array is one word per row."""
    gu.log("[case] fused greedy 4096 rows")
    c = _case(3, 120, 64, 512, 512, BF16, 1, 1, 64, np.uint16)
    assert sum(len(t) for t in c["trees"]) >= 2048
    _run(c, what="greedy many rows")


@pytest.mark.parametrize("T", [0.7, 1.0])
def test_sampled(T):
    gu.log(f"[case] fused sampled T={T}")
    c = _case(4, 29, 32, 50000, 50000, BF16, 2, 4, 128, np.uint16)
    _run(c, temperature=T, seed=77, offset=5, what=f"sampled T={T}")


def test_workload_c8():
    gu.log("[case] fused c8 workload, planted drafts")
    w = gu.cached_config("c8")
    c = dict(trees=[w.parent[w.node_start[b]:w.node_start[b + 1]] for b in range(w.batch)],
             node_start=w.node_start, parent=w.parent, logits=w.logits, vocab=w.vocab, max_nodes=w.max_nodes,
             prefix_len=w.prefix_len, kv_start=w.kv_start, k=w.k[None], v=w.v[None], rng=np.random.default_rng(8))
    assert _run(c, p_agree=0.9, what="c8") > 2


def test_paged():
    import torch
    from draft_tree_verification_amd import ev
    gu.log("[case] fused paged")
    c = _case(5, 19, 40, 20000, 20000, BF16, 1, 8, 128, np.uint16, max_prefix=300)
    tref, _ = oracle.node_argmax(c["logits"], vocab=c["vocab"], row_stride=c["logits"].shape[1])
    draft = _planted(c["rng"], c["trees"], tref, c["vocab"], 0.85)
    w = SimpleNamespace(batch=len(c["trees"]), prefix_len=c["prefix_len"], node_start=c["node_start"],
                        kv_start=c["kv_start"], k=c["k"][0], v=c["v"][0])
    P = 16
    pk, pv, bt = synth.paged_layout(w, P, 31)
    shape = (pk.shape[0] // P, P) + pk.shape[1:]
    d = _dev(c, draft)
    btd = torch.from_numpy(bt).cuda()
    k1, v1 = gu.to_dev(pk).view(shape), gu.to_dev(pv).view(shape)
    k2, v2 = k1.clone(), v1.clone()
    sep = _separate(d, k1, v1, c, 0.0, 0, 0, block_table=btd)
    fus = _fused(d, k2, v2, c, 0.0, 0, 0, block_table=btd)
    _compare(sep, fus, "paged")
    assert torch.equal(k1, k2) and torch.equal(v1, v2), "paged pools"
    assert float(fus[1]["accept_len"].float().mean().item()) > 2
    assert int(fus[3].item()) == 0


def test_workspace_reuse():
    """Two calls in a row on one workspace (never zeroed), the second with other logits and fewer
    rows: each equals the separate calls."""
    gu.log("[case] fused workspace reuse")
    from draft_tree_verification_amd import ev
    ws = ev.Workspace(ev.ev_select_workspace_size(4096, 40000), "cuda")
    for seed, B in ((6, 31), (7, 9)):
        c = _case(seed, B, 48, 40000, 40000, BF16, 1, 2, 64, np.uint16)
        tref, _ = oracle.node_argmax(c["logits"])
        draft = _planted(c["rng"], c["trees"], tref, c["vocab"], 0.8)
        d = _dev(c, draft)
        k1, v1 = gu.to_dev(c["k"]), gu.to_dev(c["v"])
        k2, v2 = k1.clone(), v1.clone()
        _compare(_separate(d, k1, v1, c, 0.0, 0, 0), _fused(d, k2, v2, c, 0.0, 0, 0, workspace=ws),
                 f"reuse B={B}")
        assert gu.to_host(k1).tobytes() == gu.to_host(k2).tobytes()


def test_data_errors():
    """A root with a parent, a draft token outside the vocabulary, and an empty node range (whose
    nodes then fall into the previous sequence, rooted twice): the same outputs and error bits as
    the separate calls, and only the good sequences' rows move."""
    import torch
    gu.log("[case] fused data errors")
    rng = np.random.default_rng(9)
    trees = [np.array([-1, 0, 0, 1, 2, 3][:m], np.int32) for m in (6, 4, 5, 3, 6, 2)]
    n = np.array([len(t) for t in trees])
    T = int(n.sum())
    L = rng.integers(0, 61, len(trees)).astype(np.int32)
    slots = int((L + n).sum())
    c = dict(trees=trees, node_start=np.concatenate([[0], np.cumsum(n)]).astype(np.int32),
             parent=np.concatenate(trees).astype(np.int32),
             logits=synth.f32_to_bf16_bits(rng.normal(0, 2, (T, 304)).astype(np.float32)), vocab=300, max_nodes=8,
             prefix_len=L, kv_start=np.concatenate([[0], np.cumsum(L + n)])[:-1].astype(np.int32),
             k=rng.integers(0, 1 << 14, (1, slots, 1, 64)).astype(np.uint16),
             v=rng.integers(0, 1 << 14, (1, slots, 1, 64)).astype(np.uint16), rng=rng)
    tref, _ = oracle.node_argmax(c["logits"], vocab=300, row_stride=304)
    draft = _planted(rng, trees, tref, 300, 1.0)
    ns = c["node_start"].copy()
    c["parent"][ns[1]] = 0             # sequence 1: its root has a parent
    draft[ns[3] + 2] = 300             # sequence 3: a draft token outside the vocabulary
    c["node_start"][5] = ns[6]         # sequence 5 empty; sequence 4 now holds two roots
    d = _dev(c, draft)
    k1, v1 = gu.to_dev(c["k"]), gu.to_dev(c["v"])
    k2, v2 = k1.clone(), v1.clone()
    sep = _separate(d, k1, v1, c, 0.0, 0, 0)
    fus = _fused(d, k2, v2, c, 0.0, 0, 0)
    _compare(sep, fus, "data errors")
    e = int(fus[3].item())
    assert e & 1 and e & 2 and e & 4, f"error bits {e}"
    lens = fus[1]["accept_len"].cpu().numpy()
    assert list(lens[[1, 3, 4, 5]]) == [0, 0, 0, 0] and lens[0] > 1 and lens[2] > 1, lens
    assert torch.equal(k1, k2) and torch.equal(v1, v2)


def test_argument_errors():
    import torch
    from draft_tree_verification_amd import ev
    gu.log("[case] fused argument errors")
    c = _case(10, 3, 4, 100, 104, BF16, 1, 1, 64, np.uint16)
    d = _dev(c, np.zeros(int(c["node_start"][-1]), np.int32))
    k, v = gu.to_dev(c["k"]), gu.to_dev(c["v"])
    for T in (-1.0, float("nan"), float("inf"), 1e-45):
        with pytest.raises(ev.EvError) as e:
            _fused(d, k, v, c, T, 1, 1)
        assert e.value.status == 2, T
    i32 = lambda n: torch.zeros(n, dtype=torch.int32, device="cuda")
    st = ev.ev_select_accept_compact(None, ev.EV_BF16, 104, 100, 0.0, 0, 0, d["node_start"].data_ptr(),
                                     d["parent"].data_ptr(), d["draft"].data_ptr(), 3, int(c["node_start"][-1]), 4,
                                     k.data_ptr(), v.data_ptr(), 2, 1, k.numel() * 2, d["kv_start"].data_ptr(),
                                     d["prefix_len"].data_ptr(), k.shape[1], 1, 64, i32(16).data_ptr(),
                                     i32(3).data_ptr(), i32(12).data_ptr(), i32(3).data_ptr(), i32(12).data_ptr(),
                                     i32(3).data_ptr(), None, 0, None, torch.cuda.current_stream().cuda_stream)
    assert st == 1
    # a workspace below ev_select_workspace_size: EV_ERR_WORKSPACE, nothing launched
    need = ev.ev_select_workspace_size(int(c["node_start"][-1]), 100)
    ws = ev.Workspace(need, "cuda")
    st = ev.ev_select_accept_compact(d["logits"].data_ptr(), ev.EV_BF16, 104, 100, 0.0, 0, 0,
                                     d["node_start"].data_ptr(), d["parent"].data_ptr(), d["draft"].data_ptr(), 3,
                                     int(c["node_start"][-1]), 4, k.data_ptr(), v.data_ptr(), 2, 1, k.numel() * 2,
                                     d["kv_start"].data_ptr(), d["prefix_len"].data_ptr(), k.shape[1], 1, 64,
                                     i32(16).data_ptr(), i32(3).data_ptr(), i32(12).data_ptr(), i32(3).data_ptr(),
                                     i32(12).data_ptr(), i32(3).data_ptr(), ws.ptr, need - 8, None,
                                     torch.cuda.current_stream().cuda_stream)
    assert need > 8 and st == 5
    # batch 0: nothing launched, EV_OK
    st = ev.ev_select_accept_compact(d["logits"].data_ptr(), ev.EV_BF16, 104, 100, 0.0, 0, 0,
                                     d["node_start"].data_ptr(), d["parent"].data_ptr(), d["draft"].data_ptr(), 0, 0,
                                     4, k.data_ptr(), v.data_ptr(), 2, 1, k.numel() * 2, d["kv_start"].data_ptr(),
                                     d["prefix_len"].data_ptr(), k.shape[1], 1, 64, i32(16).data_ptr(),
                                     i32(3).data_ptr(), i32(12).data_ptr(), i32(3).data_ptr(), i32(12).data_ptr(),
                                     i32(3).data_ptr(), None, 0, None, torch.cuda.current_stream().cuda_stream)
    assert st == 0


def test_randomized_against_separate_calls():
    """Forty random configurations (batch 1-70, trees of 1-64 nodes, vocabularies 1-70,000 with
    padded strides, bf16/fp32 logits, temperature 0 or 0.2-3, 1-2 layers, bf16/fp32 caches):
    the fused call equals the three separate calls bit for bit every time."""
    import torch
    gu.log("[case] fused randomized")
    rng = np.random.default_rng(2024)
    for it in range(40):
        B = int(rng.integers(1, 71))
        max_n = int(rng.choice([1, 4, 16, 64]))
        vocab = int(rng.choice([1, 7, 300, 4096, 70000]))
        stride = vocab + int(rng.integers(0, 3)) * 8
        ldt = BF16 if rng.random() < 0.7 else F32
        if ldt == BF16 and stride % 8:
            stride += 8 - stride % 8
        if ldt == F32 and stride % 4:
            stride += 4 - stride % 4
        T = 0.0 if rng.random() < 0.5 else float(rng.uniform(0.2, 3.0))
        layers = int(rng.integers(1, 3))
        cdt = np.uint16 if rng.random() < 0.7 else np.float32
        c = _case(int(rng.integers(1 << 30)), B, max_n, vocab, stride, ldt, layers, 2, 64, cdt, max_prefix=30)
        if T > 0:
            tref, _ = oracle.node_sample(c["logits"], T, 5, it, vocab=vocab, row_stride=stride)
        else:
            tref, _ = oracle.node_argmax(c["logits"], vocab=vocab, row_stride=stride)
        draft = _planted(c["rng"], c["trees"], tref, vocab, float(rng.uniform(0.3, 1.0)))
        d = _dev(c, draft)
        k1, v1 = gu.to_dev(c["k"]), gu.to_dev(c["v"])
        k2, v2 = k1.clone(), v1.clone()
        what = f"random #{it}: B={B} max_n={max_n} vocab={vocab}/{stride} T={T:.2f} layers={layers}"
        _compare(_separate(d, k1, v1, c, T, 5, it), _fused(d, k2, v2, c, T, 5, it), what)
        assert gu.to_host(k1).tobytes() == gu.to_host(k2).tobytes(), what
        assert gu.to_host(v1).tobytes() == gu.to_host(v2).tobytes(), what
    gu.log("[fused] 40 random configurations bit-exact")


def test_head_major_compaction_as_per_head_layers():
    """Head-major caches [layers][Hkv][slots][D] are compacted by the fused call with one 'layer' per
    (layer, KV head) and one head per layer: the result, read back as [layers][slots][Hkv][D], equals
    the slot-major compaction of the same values, and the acceptance outputs agree."""
    import torch
    gu.log("[case] fused head-major compaction")
    c = _case(123, 6, 16, 5000, 5000, BF16, 2, 4, 64, np.uint16, max_prefix=40)
    tref, _ = oracle.node_argmax(c["logits"], vocab=c["vocab"], row_stride=c["logits"].shape[1])
    draft = _planted(c["rng"], c["trees"], tref, c["vocab"], 0.9)
    d = _dev(c, draft)
    layers, slots, H, D = c["k"].shape
    k1, v1 = gu.to_dev(c["k"]), gu.to_dev(c["v"])
    sm = _fused(d, k1, v1, c, 0.0, 0, 0)
    hm = lambda a: np.ascontiguousarray(a.transpose(0, 2, 1, 3))            # [layers][H][slots][D]
    k2, v2 = gu.to_dev(hm(c["k"]).reshape(layers * H, slots, 1, D)), gu.to_dev(hm(c["v"]).reshape(layers * H, slots, 1, D))
    c2 = dict(c, k=hm(c["k"]).reshape(layers * H, slots, 1, D))
    hd = _fused(d, k2, v2, c2, 0.0, 0, 0)
    _compare(sm, hd, "head-major compaction")
    back = lambda t: gu.to_host(t).reshape(layers, H, slots, D).transpose(0, 2, 1, 3)
    assert np.array_equal(back(k2), gu.to_host(k1)) and np.array_equal(back(v2), gu.to_host(v1))
    assert hd[1]["accept_len"].float().mean().item() > 1.0
