"""Host concurrency: several host threads, each with its own stream, inputs, outputs and
workspace, run whole verification steps at the same time; every result equals the one the same
step gives alone.  (The library keeps no per-call global state; its per-device cache is filled
once under a mutex.)"""
import threading

import pytest

from . import gpu_util as gu

pytestmark = pytest.mark.gpu


def _step(ev, w, d, k, v, state, stream, T):
    return ev.verify_step(d["q"], k, v, d["logits"], d["node_start"], d["parent"], d["kv_start"], d["prefix_len"],
                          d["draft"], max_nodes=w.max_nodes, sm_scale=w.sm_scale, temperature=T, seed=5, offset=9,
                          state=state, stream=stream)


def _snapshot(st, k, v):
    snap = {key: st[key].clone() for key in ("out", "lse", "target", "new_len")}
    snap.update({"acc_" + key: t.clone() for key, t in st["accept"].items()})
    snap["k"], snap["v"] = k.clone(), v.clone()
    return snap


@pytest.mark.timeout(300)
def test_threads_with_their_own_streams():
    import torch
    from draft_tree_verification_amd import ev
    gu.log("[case] four host threads, four streams, whole steps")
    cases = [("c1x4k", 0.0), ("tiny", 1.0), ("c1x4k", 0.7), ("tiny", 0.0)]
    inputs, refs = [], []
    for name, T in cases:
        w = gu.cached_config(name)
        d = gu.dev_workload(w)
        k0, v0 = d["k"].clone(), d["v"].clone()
        k, v = k0.clone(), v0.clone()
        st = _step(ev, w, d, k, v, {}, None, T)
        torch.cuda.synchronize()
        assert int(st["err"].item()) == 0
        refs.append(_snapshot(st, k, v))
        inputs.append((w, d, k0, v0, T))
    torch.cuda.synchronize()
    failures = []

    def worker(i):
        try:
            w, d, k0, v0, T = inputs[i]
            s = torch.cuda.Stream()
            state = {}
            with torch.cuda.stream(s):
                k, v = k0.clone(), v0.clone()
                for it in range(12):
                    k.copy_(k0)
                    v.copy_(v0)
                    st = _step(ev, w, d, k, v, state, s, T)
                    if it % 4 == 3:
                        s.synchronize()
                        got = _snapshot(st, k, v)
                        for key, ref in refs[i].items():
                            if not torch.equal(got[key], ref):
                                failures.append(f"thread {i} ({cases[i]}) iteration {it}: {key} differs")
                                return
                        if int(st["err"].item()) != 0:
                            failures.append(f"thread {i}: error flag {int(st['err'].item())}")
                            return
        except Exception as e:  # reported below, with the thread it came from
            failures.append(f"thread {i}: {type(e).__name__}: {e}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=240)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    torch.cuda.synchronize()
    assert not failures, "; ".join(failures)
    gu.log("[threads] every thread's steps equal the single-threaded results")
