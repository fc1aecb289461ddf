"""Benchmark of the draft-tree verification step on one MI355X.

One step = the whole hot path over one batch: tree-masked GQA attention, the per-node argmax (or
sampled draw), greedy acceptance and in-place KV compaction, as one ev_verify_step call: three
launches on one stream (the attention kernel; the merge of split units together with the
selection pass; acceptance and compaction).  --two-call runs ev_tree_attention then
ev_select_accept_compact (four launches; the paged and window layouts always run this form);
--separate calls the four separate entry points.  The
attention call's own time (ev_tree_attention, for the roofline) is measured on its own.  Inputs
are seeded synthetic data already resident in HBM; several identical input sets sit at different
addresses and the steps rotate over them, so the 256 MB Infinity Cache cannot serve one step's
reads from the previous step's.  Prints ONE JSON line.

  python bench.py [--steps K] [--warmup W] [--trials R] [--workload c8|c128k|c512|c1x4k|tiny]
                  [--also WORKLOAD|''] [--no-cpu] [--kv contiguous|paged|window] [--page-size P]
                  [--window W] [--sample T] [--two-call | --separate]
  python bench.py --copy-calibration     (a plain device copy of known size, for counter scaling)

The default workload is the 8-sequence batch (prefix lengths uniform in [1024, 8192], 16-node
trees, 40 q heads / 8 KV heads, head_dim 128, bf16 KV, vocab 151936); the 128K-context sequence
(same heads, 16-node tree) is measured after it the same way and reported under "also"; both are
measured again over head-major caches [Hkv][slots][D] and reported under "head_major".
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MALL_BYTES = 256 << 20
HBM_PEAK_GBPS = 8000.0
BF16_DENSE_PEAK = 2.5e15  # MI355X dense bf16 matrix-core peak, FLOP/s
METRIC = "verified tree-tokens/s + accepted tokens/s; KV-read HBM GB/s as % of peak"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="c8")
    p.add_argument("--also", default="c128k",
                   help="a second workload measured the same way and reported as a sub-record ('' for none)")
    p.add_argument("--trials", type=int, default=5, help="timed runs the K steps are split into (median)")
    p.add_argument("--no-head-major", dest="head_major_too", action="store_false",
                   help="skip the extra measurement of the same workloads over head-major caches")
    p.add_argument("--sets", type=int, default=0, help="input sets to rotate over (0: enough to defeat the MALL)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--copy-calibration", action="store_true")
    p.add_argument("--kv", default="contiguous", choices=("contiguous", "headmajor", "paged", "window"),
                   help="K/V layout of the step: contiguous [slots][Hkv][D] (default), head-major [Hkv][slots][D] "
                        "(ev_tree_attention_strided; compaction per head), a paged pool through a block table "
                        "(--page-size), or a sliding window over the prefix (--window)")
    p.add_argument("--page-size", type=int, default=16)
    p.add_argument("--window", type=int, default=4096)
    p.add_argument("--separate", action="store_true",
                   help="run the step as four calls (attention, token, acceptance, compaction)")
    p.add_argument("--two-call", action="store_true",
                   help="run the step as attention + the fused token/acceptance/compaction call (the paged and "
                        "window layouts always do) instead of the whole-step call")
    p.add_argument("--sample", type=float, default=0.0,
                   help="temperature > 0: sampled verification (per-node draw instead of the argmax)")
    return p.parse_args()


def copy_calibration():
    """A device-to-device copy of exactly 1 GiB, repeated 5 times: the reference for counter scaling."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)


def lscpu_model() -> str:
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True).stdout
        m = re.search(r"Model name:\s*(.+)", out)
        return m.group(1).strip() if m else platform.processor()
    except OSError:
        return platform.processor()


def cpu_baseline(w, target_seconds: float, temperature: float = 0.0):
    """The oracle (plain C, OpenMP over rows) on the host cores, on a bounded sample of the workload:
    whole steps over the first sequences, repeated until about target_seconds of CPU time."""
    import numpy as np
    import oracle
    lib = oracle.load()
    threads = oracle.num_threads(lib)
    # sample: the first sequences whose oracle attention fits one pass in about a quarter of the budget
    flops_per_s = 1.0e9 * threads  # rough fp64 plain-loop rate, only used to size the sample
    B = w.batch
    per_seq = [4.0 * (int(w.prefix_len[b]) + int(w.nodes_per_seq[b])) * w.head_dim * w.num_q_heads *
               int(w.nodes_per_seq[b]) for b in range(B)]
    nb, acc = 0, 0.0
    while nb < B and (acc + per_seq[nb]) / flops_per_s < target_seconds / 4:
        acc += per_seq[nb]
        nb += 1
    nb = max(nb, 1)
    s_end = int(w.node_start[nb])
    slot_end = int(w.kv_start[nb - 1] + w.prefix_len[nb - 1] + w.nodes_per_seq[nb - 1])
    q, k, v = w.q[:s_end], w.k[:slot_end], w.v[:slot_end]
    ns, par, ks, pl = w.node_start[:nb + 1], w.parent[:s_end], w.kv_start[:nb], w.prefix_len[:nb]
    logits, draft = w.logits[:s_end], w.draft[:s_end]
    reps, tokens, t0 = 0, 0, time.perf_counter()
    while True:
        oracle.tree_attention(q, k, v, ns, par, ks, pl, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                              head_dim=w.head_dim, sm_scale=w.sm_scale, total_slots=slot_end,
                              max_nodes=w.max_nodes, lib=lib)
        if temperature > 0:
            tgt, _ = oracle.node_sample(logits, temperature, 0x5EED, reps, lib=lib)
        else:
            tgt, _ = oracle.node_argmax(logits, lib=lib)
        accept = oracle.sampled_accept if temperature > 0 else oracle.greedy_accept
        acc_r = accept(ns, par, draft, tgt, w.max_nodes, w.vocab, lib=lib)
        oracle.compact_kv(k[None], v[None], ks, pl, acc_r["accept_len"], acc_r["accept_path"], num_layers=1,
                          total_slots=slot_end, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, lib=lib)
        reps += 1
        tokens += s_end
        el = time.perf_counter() - t0
        if el >= target_seconds or reps >= 1000:
            break
    return {"value": tokens / el, "unit": "tree-tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{nb} of {B} sequences ({s_end} tree nodes), whole step x{reps} in {el:.1f} s",
            "cpu_model": lscpu_model()}


def counters_value(kernel_src: str, workload: str, suffix: str, key: str):
    """A figure from a committed counter summary profiles/tree_attention_<workload>_<suffix>.txt, used
    only if that summary was taken on the current kernel source (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"tree_attention_{workload}_{suffix}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        m = re.match(r"\s*([a-z_]+)\s*[:=]\s*(\S+)", line)
        if m:
            vals[m.group(1)] = m.group(2)
    sha = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()[:16]
    if vals.get("kernel_source_sha") != sha or key not in vals:
        return None
    return float(vals[key])


def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def measure(args, workload: str, with_cpu: bool) -> dict:
    """One workload: warmup, then exactly args.steps timed steps split into `trials` equal runs (the
    step time is the median of the runs' means), the attention call timed the same way, per-kernel
    times, the read ceilings, and the oracle on the host cores."""
    import numpy as np
    import torch

    from draft_tree_verification_amd import ev, synth

    w = synth.make_config(workload)
    print(f"[bench] workload {workload}: {synth.describe(w)}", file=sys.stderr, flush=True)
    kv_bytes = w.kv_bytes()
    set_bytes = kv_bytes + w.logits.nbytes + w.q.nbytes
    nsets = args.sets or max(1, math.ceil(2 * MALL_BYTES / set_bytes))

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    meta = {n: dev(getattr(w, n).astype(np.int32)) for n in ("node_start", "parent", "kv_start", "prefix_len",
                                                             "draft")}
    host = {n: dev(getattr(w, n)) for n in ("q", "logits")}
    if args.kv == "paged":
        if w.dtype != synth.BF16:
            raise SystemExit("paged K/V pools hold bf16")
        pk, pv, bt = synth.paged_layout(w, args.page_size, 77)
        host["k"], host["v"] = dev(pk), dev(pv)
        meta["block_table"] = dev(bt)
        num_pages = pk.shape[0] // args.page_size
        del pk, pv
    elif args.kv == "headmajor":  # [Hkv][slots][D]: each KV head's rows contiguous
        host["k"], host["v"] = dev(w.k.transpose(1, 0, 2)), dev(w.v.transpose(1, 0, 2))
    else:
        host["k"], host["v"] = dev(w.k), dev(w.v)
    sets = [host] + [{n: t.clone() for n, t in host.items()} for _ in range(nsets - 1)]
    print(f"[bench] {nsets} input sets of {set_bytes / 1e6:.1f} MB", file=sys.stderr, flush=True)

    B, T, maxn = w.batch, w.total_nodes, w.max_nodes
    Hq, Hkv, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    dt = ev.EV_BF16 if w.dtype == synth.BF16 else ev.EV_F32
    esz = w.elem_bytes
    i32 = lambda n: torch.empty(n, dtype=torch.int32, device="cuda")
    out = [torch.empty_like(s["q"]) for s in sets]
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    target, maxv = i32(T), torch.empty(T, dtype=torch.float32, device="cuda")
    acc_len, bonus, new_len = i32(B), i32(B), i32(B)
    acc_path, out_tok = i32((B, maxn)), i32((B, maxn))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    aws = ev.Workspace(ev.ev_tree_attention_workspace_size(B, maxn, Hq, Hkv, D), "cuda")
    gws = ev.Workspace(max(ev.ev_node_argmax_workspace_size(T, w.vocab), 256), "cuda")
    sws = ev.Workspace(max(ev.ev_select_workspace_size(T, w.vocab), 256), "cuda")
    whole = not args.separate and not args.two_call and args.kv in ("contiguous", "headmajor")
    vws = ev.Workspace(ev.ev_verify_step_workspace_size(B, T, maxn, Hq, Hkv, D, w.vocab), "cuda") if whole else None
    stream = torch.cuda.current_stream().cuda_stream
    lib = ev.load()
    p = lambda t: t.data_ptr()
    m = {n: p(t) for n, t in meta.items()}
    calls = []
    for i, s in enumerate(sets):
        if args.kv == "paged":
            bts = meta["block_table"].shape[1]
            attn = (p(s["q"]), p(s["k"]), p(s["v"]), p(out[i]), p(lse), m["node_start"], m["parent"],
                    m["block_table"], bts, args.page_size, m["prefix_len"], B, T, maxn, num_pages, Hq, Hkv, D, dt,
                    w.sm_scale, 0, aws.ptr, aws.nbytes, p(err), stream)
            cmp = (p(s["k"]), p(s["v"]), esz, 1, num_pages * args.page_size * Hkv * D * esz, m["block_table"], bts,
                   args.page_size, m["prefix_len"], p(acc_len), p(acc_path), B, maxn, num_pages, Hkv, D,
                   p(new_len), p(err), stream)
        elif args.kv == "headmajor":  # compaction sees Hkv one-head layers of [slots][D]
            attn = (p(s["q"]), p(s["k"]), p(s["v"]), p(out[i]), p(lse), m["node_start"], m["parent"],
                    m["kv_start"], m["prefix_len"], B, T, maxn, w.total_slots, Hq, Hkv, D, D, w.total_slots * D, dt,
                    w.sm_scale, aws.ptr, aws.nbytes, p(err), stream)
            cmp = (p(s["k"]), p(s["v"]), esz, Hkv, w.total_slots * D * esz, m["kv_start"], m["prefix_len"],
                   p(acc_len), p(acc_path), B, maxn, w.total_slots, 1, D, p(new_len), p(err), stream)
        else:
            attn = (p(s["q"]), p(s["k"]), p(s["v"]), p(out[i]), p(lse), m["node_start"], m["parent"],
                    m["kv_start"], m["prefix_len"], B, T, maxn, w.total_slots, Hq, Hkv, D, dt, w.sm_scale) + \
                   ((args.window,) if args.kv == "window" else ()) + (aws.ptr, aws.nbytes, p(err), stream)
            cmp = (p(s["k"]), p(s["v"]), esz, 1, w.total_slots * Hkv * D * esz, m["kv_start"], m["prefix_len"],
                   p(acc_len), p(acc_path), B, maxn, w.total_slots, Hkv, D, p(new_len), p(err), stream)
        if not args.separate:  # token, acceptance and compaction in one call (noise offset = the set's index)
            hm = args.kv == "headmajor"
            head = (p(s["logits"]), dt, w.vocab, w.vocab, args.sample, 0x5EED, i, m["node_start"], m["parent"],
                    m["draft"], B, T, maxn, p(s["k"]), p(s["v"]), esz, Hkv if hm else 1)
            out_args = (p(target), p(acc_len), p(acc_path), p(bonus), p(out_tok), p(new_len), sws.ptr, sws.nbytes,
                        p(err), stream)
            if args.kv == "paged":
                fused = head + (num_pages * args.page_size * Hkv * D * esz, m["block_table"],
                                meta["block_table"].shape[1], args.page_size, m["prefix_len"], num_pages, Hkv, D)
            elif hm:
                fused = head + (w.total_slots * D * esz, m["kv_start"], m["prefix_len"], w.total_slots, 1, D)
            else:
                fused = head + (w.total_slots * Hkv * D * esz, m["kv_start"], m["prefix_len"], w.total_slots, Hkv, D)
            if whole:  # the whole step in one call: the attention's arguments with its strides, then the rest
                strides = (D, w.total_slots * D) if hm else (Hkv * D, D)
                comp = (Hkv, w.total_slots * D * esz, 1, D) if hm else (1, w.total_slots * Hkv * D * esz, Hkv, D)
                one = (p(s["q"]), p(s["k"]), p(s["v"]), p(out[i]), p(lse), m["node_start"], m["parent"],
                       m["kv_start"], m["prefix_len"], B, T, maxn, w.total_slots, Hq, Hkv, D) + strides + \
                      (dt, w.sm_scale, p(s["logits"]), dt, w.vocab, w.vocab, args.sample, 0x5EED, i, m["draft"]) + \
                      comp + (p(target), p(acc_len), p(acc_path), p(bonus), p(out_tok), p(new_len), vws.ptr,
                              vws.nbytes, p(err), stream)
                calls.append((attn, one))
                continue
            calls.append((attn, fused + out_args))
            continue
        if args.sample > 0:  # noise offset = the input set's index
            sel = (p(s["logits"]), dt, w.vocab, T, w.vocab, args.sample, 0x5EED, i, p(target), gws.ptr, gws.nbytes,
                   stream)
        else:
            sel = (p(s["logits"]), dt, w.vocab, T, w.vocab, p(target), p(maxv), gws.ptr, gws.nbytes, stream)
        calls.append((
            attn,
            sel,
            (m["node_start"], m["parent"], m["draft"], p(target), B, T, maxn, w.vocab, p(acc_len), p(acc_path),
             p(bonus), p(out_tok), p(err), stream),
            cmp))
    f_attn = {"contiguous": lib.ev_tree_attention, "headmajor": lib.ev_tree_attention_strided,
              "paged": lib.ev_tree_attention_paged, "window": lib.ev_tree_attention_window}[args.kv]
    # the step: (function, index of its argument tuple in a call entry) pairs; entry 0 always holds the
    # attention call's arguments (the attention-only timing below uses it)
    if args.separate:
        f_arg = lib.ev_node_sample if args.sample > 0 else lib.ev_node_argmax
        f_acc = lib.ev_sampled_accept if args.sample > 0 else lib.ev_greedy_accept
        f_cmp = lib.ev_compact_kv_paged if args.kv == "paged" else lib.ev_compact_kv
        plan = ((f_attn, 0), (f_arg, 1), (f_acc, 2), (f_cmp, 3))
        names = ("tree_attention", "node_sample" if args.sample > 0 else "node_argmax",
                 "sampled_accept" if args.sample > 0 else "greedy_accept", "compact_kv")
    elif whole:
        plan = ((lib.ev_verify_step, 1),)
        names = ("verify_step",)
    else:
        plan = ((f_attn, 0),
                (lib.ev_select_accept_compact_paged if args.kv == "paged" else lib.ev_select_accept_compact, 1))
        names = ("tree_attention", "select_accept_compact")

    def step(c):
        r = 0
        for f, j in plan:
            r |= f(*c[j])
        return r

    for i in range(args.warmup):
        if step(calls[i % nsets]):
            raise RuntimeError("a launch failed during warmup")
    torch.cuda.synchronize()
    if int(err.item()):
        raise RuntimeError(f"data error flag {int(err.item())}")

    # exactly K timed steps, in `trials` runs of equal length between event pairs (no marker inside
    # a run); the step time is the median of the runs' means
    K = args.steps
    trials = max(1, min(args.trials, K))
    bounds = [K * j // trials for j in range(trials + 1)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(trials + 1)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    rc = 0
    for j in range(trials):
        evs[j].record()
        for i in range(bounds[j], bounds[j + 1]):
            rc |= step(calls[i % nsets])
    evs[trials].record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    if rc:
        raise RuntimeError("a launch failed in the timed region")
    trial_ms = [evs[j].elapsed_time(evs[j + 1]) / (bounds[j + 1] - bounds[j]) for j in range(trials)]
    ms_step = _median(trial_ms)
    acc_sum = int(acc_len.sum().item())  # the last step's acceptance (every set holds the same inputs)

    # The attention call's launch duration: K attention calls back to back on the same stream
    # (rotating over the input sets like the steps), in `trials` runs between event pairs; the median
    # of the runs' means.  A call is every launch of ev_tree_attention; the mean includes the gaps
    # between launches.  (An event marker costs stream time of its own, ~3 us here, so no run has
    # one between calls.)
    for i in range(min(K, 3)):
        rc |= f_attn(*calls[i % nsets][0])
    torch.cuda.synchronize()
    aevs = [torch.cuda.Event(enable_timing=True) for _ in range(trials + 1)]
    for j in range(trials):
        aevs[j].record()
        for i in range(bounds[j], bounds[j + 1]):
            rc |= f_attn(*calls[i % nsets][0])
    aevs[trials].record()
    torch.cuda.synchronize()
    if rc:
        raise RuntimeError("a launch failed in the attention timing region")
    attn_trials = [aevs[j].elapsed_time(aevs[j + 1]) / (bounds[j + 1] - bounds[j]) for j in range(trials)]
    attn_ms = _median(attn_trials)

    # per-call breakdown (separate pass, an event pair around every call; not part of the timed region)
    nf = len(plan)
    kev = [[torch.cuda.Event(enable_timing=True) for _ in range(nf + 1)] for _ in range(K)]
    for i in range(K):
        c = calls[i % nsets]
        for j, (f, a) in enumerate(plan):
            kev[i][j].record()
            f(*c[a])
        kev[i][nf].record()
    torch.cuda.synchronize()
    kernel_ms = {n: _median([kev[i][j].elapsed_time(kev[i][j + 1]) for i in range(K)]) for j, n in enumerate(names)}

    # streaming-read ceiling of this GPU: ev_stream_read over 2 GiB (8x the Infinity Cache)
    rbuf = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        rc |= lib.ev_stream_read(p(rbuf), rbuf.numel(), p(sink), stream)
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record()
    for _ in range(10):
        rc |= lib.ev_stream_read(p(rbuf), rbuf.numel(), p(sink), stream)
    r1.record()
    torch.cuda.synchronize()
    if rc:
        raise RuntimeError("the streaming-read measurement failed")
    read_ceiling = 10 * rbuf.numel() / (r0.elapsed_time(r1) * 1e-3) / 1e9
    del rbuf
    # the same read over buffers the size of this workload's K/V (ramp-up and drain included),
    # rotated past the Infinity Cache: the time no kernel reading these bytes once can beat
    nsz = (kv_bytes + 15) // 16 * 16
    nbuf = max(2, math.ceil(2 * MALL_BYTES / nsz))
    sbufs = [torch.empty(nsz, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
    for i in range(nbuf):
        rc |= lib.ev_stream_read(p(sbufs[i]), nsz, p(sink), stream)
    r0.record()
    for i in range(20):
        rc |= lib.ev_stream_read(p(sbufs[i % nbuf]), nsz, p(sink), stream)
    r1.record()
    torch.cuda.synchronize()
    if rc:
        raise RuntimeError("the same-size read measurement failed")
    same_size_read_ms = r0.elapsed_time(r1) / 20
    del sbufs

    vis_keys = [int(w.prefix_len[b]) for b in range(B)]
    if args.kv == "window":  # only the last `window` prefix tokens (and the tree) are read
        vis_keys = [min(v, args.window) for v in vis_keys]
        kv_bytes = 2 * sum(v + int(w.nodes_per_seq[b]) for b, v in enumerate(vis_keys)) * Hkv * D * esz
    tree_tps = T / (ms_step / 1e3)
    # Algorithmic bytes of one attention call: every K/V row of every (sequence, KV head) once (the
    # roofline's bytes).  Q read once and the output and log-sum-exp written once are reported beside.
    qo_bytes = 2 * w.q.nbytes + T * Hq * 4
    achieved = kv_bytes / (attn_ms * 1e-3) / 1e9
    # matrix-core work of the call: every row of a (sequence, KV head) unit against every key the unit
    # streams (prefix + tree, masked keys included), 2 products of 2*D flops per (row, key)
    rows_per_unit = [int(w.nodes_per_seq[b]) * (Hq // Hkv) for b in range(B)]
    mfma_flops = sum(4 * D * r * (vis_keys[b] + int(w.nodes_per_seq[b])) * Hkv for b, r in enumerate(rows_per_unit))
    src = os.path.join(ROOT, "draft_tree_verification_amd", "csrc", "ev_attention.hip")
    tag = {"contiguous": workload, "headmajor": f"{workload}_headmajor"}.get(args.kv)
    traffic = counters_value(src, tag, "counters", "traffic_bytes_per_launch") if tag else None
    mfma_busy = counters_value(src, tag, "mfma", "mfma_busy_frac") if tag else None
    rec = {
        "metric": METRIC,
        "value": round(tree_tps, 1),
        "unit": "tree-tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == synth.BF16 else "f32",
        "data": "synthetic (seeded; shapes of the workload, no dataset or weights)",
        "config": dict(synth.describe(w), input_sets=nsets, kv_bytes=kv_bytes,
                       kv_layout={"contiguous": "contiguous [slots][Hkv][D]", "headmajor": "head-major [Hkv][slots][D]",
                                  "paged": f"paged{args.page_size}", "window": f"window{args.window}"}[args.kv],
                       verification=f"sampled T={args.sample}" if args.sample > 0 else "greedy T=0",
                       step_calls=" + ".join(names)),
        "trials": trials,
        "trial_ms_per_step": [round(x, 5) for x in trial_ms],
        "accepted_tokens_per_s": round(acc_sum / (ms_step / 1e3), 1),
        "accept_len_mean": acc_sum / B,
        "kv_read_gbps": round(achieved, 1),
        "kv_read_pct_of_peak": round(100 * achieved / HBM_PEAK_GBPS, 2),
        "read_ceiling_gbps": round(read_ceiling, 1),
        "kv_read_pct_of_ceiling": round(100 * achieved / read_ceiling, 2),
        "kv_sized_read_ms": round(same_size_read_ms, 5),
        "kernel_ms": {k: round(v, 5) for k, v in kernel_ms.items()},
        "selection": ("separate calls" if args.separate else "whole step (ev_verify_step)" if whole
                      else "fused (ev_select_accept_compact)"),
        "wall_s_timed": round(t_wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": "tree_attention", "attention_ms": round(attn_ms, 5),
                     "attention_trial_ms": [round(x, 5) for x in attn_trials],
                     "algorithmic_bytes_per_launch": kv_bytes, "q_o_lse_bytes_per_launch": qo_bytes,
                     "mfma_tflops": round(mfma_flops / (attn_ms * 1e-3) / 1e12, 1),
                     "mfma_frac_of_bf16_dense_peak": round(mfma_flops / (attn_ms * 1e-3) / BF16_DENSE_PEAK, 4),
                     "mfma_busy_frac": mfma_busy},
        "cpu_baseline": None,
    }
    if with_cpu:
        del sets, out
        torch.cuda.empty_cache()
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, args.sample)
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (the verification step "
              "would shard by sequence or by KV head, with no exchange; only the one-GPU path is built)",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch

    torch.cuda.set_device(0)
    rec = measure(args, args.workload, not args.no_cpu)
    # the 128K-context configuration (the other configuration the bandwidth target names) as a
    # sub-record of the same line, measured the same way
    keep = ("value", "unit", "ms_per_step", "trials", "trial_ms_per_step", "accepted_tokens_per_s",
            "accept_len_mean", "config", "kv_read_gbps", "kv_read_pct_of_peak", "read_ceiling_gbps",
            "kv_read_pct_of_ceiling", "kv_sized_read_ms", "kernel_ms", "roofline", "cpu_baseline")
    if args.also and args.also != args.workload:
        torch.cuda.empty_cache()
        sub = measure(args, args.also, not args.no_cpu)
        rec["also"] = {args.also: {k: sub[k] for k in keep}}
    # the same workloads over head-major caches [Hkv][slots][D] (ev_tree_attention_strided): the
    # layout whose rows stream fastest; same values, same step, the oracle leg not repeated
    if args.kv == "contiguous" and args.head_major_too:
        hm_args = argparse.Namespace(**dict(vars(args), kv="headmajor"))
        rec["head_major"] = {}
        for wl in [args.workload] + ([args.also] if args.also and args.also != args.workload else []):
            torch.cuda.empty_cache()
            sub = measure(hm_args, wl, False)
            rec["head_major"][wl] = {k: sub[k] for k in keep if k != "cpu_baseline"}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
