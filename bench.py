#!/usr/bin/env python3
"""Benchmark of the speculative-decoding hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input:

  n-gram propose   64 contexts x 8192 Zipf(1.1) ids, planted copies, n 5..2, K 8
  rejection verify B 64, K 5, V 128256, bf16 target N(0,2) / draft +N(0,0.5), T 1
  greedy verify    B 256, K 8, V 151936, bf16 N(0,2), planted acceptance 0.6
  tree verify      B 32, 64-node trees, V 128256, bf16 N(0,2)

Inputs are resident in HBM before the timed region; the four inputs together
(about 1.4 GB) exceed the 256 MB last-level cache, so every step reads its
logits from HBM.  `value` is verified positions per second over the whole
step (384 + 2304 + 2048 = 4736 positions per step), timed over K steps with
nothing recorded between the calls.  A second pass of K steps brackets each
call with HIP events on the stream the kernels run on; the dominant
kernel's average gives the roofline figure.  The CPU oracle runs the same step on the
host cores beside it (cpu_baseline).  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified positions/s + HBM GB/s (% of peak) at V=128k; n-gram proposals/s"
PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
# What one timed launch of each call runs, in stream order.
LAUNCH_KERNELS = {
    "greedy": "sv_verify_greedy: k_row_argmax<bf16> (2304 rows) + k_greedy_scan",
    "tree": "sv_verify_tree: k_row_argmax<bf16> (2048 rows) + k_tree_scan",
    "rejection": "sv_verify_rejection: k_rej_stats + k_rej_final + k_rej_select",
}

KERNEL_SOURCES = {
    "greedy": ["proposal_sv_verify_amd/csrc/argmax_verify.hip",
               "proposal_sv_verify_amd/csrc/sv_device.hpp",
               "proposal_sv_verify_amd/csrc/sv_kernels.hpp"],
}


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def make_inputs():
    from proposal_sv_verify_amd import workloads as W
    t0 = time.time()
    ng = W.ngram_workload(64, 8192, seed=W.seed_for(2))
    rj = W.rejection_workload(**W.REJECTION, seed=W.seed_for(3))
    gr = W.greedy_workload(256, 8, 151936, "bf16", 2.0, (0.6,), seed=W.seed_for(4))
    tr = W.tree_workload(**W.TREE, seed=W.seed_for(5))
    log("inputs generated in %.1f s" % (time.time() - t0))
    return ng, rj, gr, tr


def ngram_bytes(out, lengths, n_max):
    """Positions the backward scan must examine: from the end of the context
    down to the start of the most recent full-length match, or to the start
    of the context when there is none (4 bytes per position)."""
    mn, mp = out["match_n"], out["match_pos"]
    stop = np.where(mn == n_max, mp, 0)
    return int(4 * (lengths.astype(np.int64) - stop).sum())


def run_gpu(args, ng, rj, gr, tr):
    import torch
    import proposal_sv_verify_amd as sv

    dev = torch.device("cuda:0")

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    d = dict(
        ng_tok=to_dev(ng["tokens"]), ng_len=to_dev(ng["lengths"]),
        rj_t=to_dev(rj["target"]), rj_d=to_dev(rj["draft_logits"]), rj_x=to_dev(rj["draft"]),
        rj_u=to_dev(rj["uniforms"]),
        gr_l=to_dev(gr["logits"]), gr_x=to_dev(gr["drafts"][0.6]),
        tr_l=to_dev(tr["logits"]), tr_p=to_dev(tr["parent"]), tr_t=to_dev(tr["token"]),
    )
    torch.cuda.synchronize()
    calls = [
        ("ngram", sv.prepare_ngram(d["ng_tok"], d["ng_len"], 2, 5, 8)),
        ("rejection", sv.prepare_rejection(d["rj_t"], d["rj_d"], d["rj_x"], d["rj_u"], 1.0)),
        ("greedy", sv.prepare_greedy(d["gr_l"], d["gr_x"])),
        ("tree", sv.prepare_tree(d["tr_l"], d["tr_p"], d["tr_t"])),
    ]
    for _ in range(args.warmup):
        for _, c in calls:
            c()
    torch.cuda.synchronize()
    K = args.steps
    # the timed steps: the calls alone, nothing recorded between them
    t0 = time.perf_counter()
    for s in range(K):
        for _, c in calls:
            c()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the same K steps again with a HIP event after every call, for the
    # per-call figures (event records add a few microseconds per call, so
    # they stay out of the timed steps above)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    for s in range(K):
        e = ev[s]
        e[0].record()
        for j, (_, c) in enumerate(calls):
            c()
            e[j + 1].record()
    torch.cuda.synchronize()
    samples = {name: np.array([ev[s][j].elapsed_time(ev[s][j + 1]) for s in range(K)]) * 1e3
               for j, (name, _) in enumerate(calls)}
    outs = {name: {k: v.cpu().numpy() for k, v in c.out.items()} for name, c in calls}
    return wall, samples, outs, d


def concurrent_step(d, outs, steps, positions):
    """The step's four calls are independent (four different batches), so a
    server could run them at once: each on its own stream, forked from and
    joined back to the main stream by events every step, so that steps do
    not overlap.  The latency-bound tails of one call then overlap another
    call's streaming.  Outputs must equal the sequential step's."""
    import torch
    import proposal_sv_verify_amd as sv

    streams = [torch.cuda.Stream() for _ in range(4)]
    preps = [lambda: sv.prepare_ngram(d["ng_tok"], d["ng_len"], 2, 5, 8),
             lambda: sv.prepare_rejection(d["rj_t"], d["rj_d"], d["rj_x"], d["rj_u"], 1.0),
             lambda: sv.prepare_greedy(d["gr_l"], d["gr_x"]),
             lambda: sv.prepare_tree(d["tr_l"], d["tr_p"], d["tr_t"])]
    calls = []
    for st, prep in zip(streams, preps):
        with torch.cuda.stream(st):
            calls.append(prep())
    main = torch.cuda.current_stream()
    fork = [torch.cuda.Event() for _ in range(steps + 3)]
    joins = [[torch.cuda.Event() for _ in range(4)] for _ in range(steps + 3)]

    def step(i):
        fork[i].record(main)
        for j, (st, c) in enumerate(zip(streams, calls)):
            st.wait_event(fork[i])
            c()
            joins[i][j].record(st)
        for j in range(4):
            main.wait_event(joins[i][j])

    for i in range(3):
        step(steps + i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(main)
    for i in range(steps):
        step(i)
    e1.record(main)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    names = ("ngram", "rejection", "greedy", "tree")
    same = all(np.array_equal(v.cpu().numpy(), outs[n][k]) for n, c in zip(names, calls)
               for k, v in c.out.items())
    return dict(streams=4, us_per_step=round(us, 2), positions_per_s=round(positions / us * 1e6, 1),
                same_outputs_as_sequential=bool(same))


def ngram_bandwidth_mode(args):
    """The n-gram generator at 16384 contexts (512 MiB) in one call."""
    import torch
    import proposal_sv_verify_amd as sv
    from proposal_sv_verify_amd import workloads as W

    wl = W.ngram_workload(16384, 8192, seed=W.seed_for(2, salt=1))
    dev = torch.device("cuda:0")
    tok = torch.from_numpy(wl["tokens"]).to(dev)
    lens = torch.from_numpy(wl["lengths"]).to(dev)
    call = sv.prepare_ngram(tok, lens, 2, 5, 8)
    for _ in range(3):
        call()
    reps = 20
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for r in range(reps):
        call()
        ev[r + 1].record()
    torch.cuda.synchronize()
    us = float(np.mean([ev[r].elapsed_time(ev[r + 1]) for r in range(reps)])) * 1e3
    out = {k: v.cpu().numpy() for k, v in call.out.items()}
    nbytes = ngram_bytes(out, wl["lengths"], 5)
    gbs = nbytes / us / 1e3
    return dict(contexts=16384, context_len=8192, us_per_call=round(us, 2),
                proposals_per_s=round(16384 / us * 1e6, 1), algorithmic_bytes=nbytes,
                gb_per_s=round(gbs, 1), frac_of_peak=round(gbs / PEAK_HBM_GBS, 4))


def _timed(fns, reps):
    """HIP-event mean of one pass over fns, over reps passes (after 3)."""
    import torch
    for _ in range(3):
        for f in fns:
            f()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(reps):
        for f in fns:
            f()
    ev[1].record()
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) * 1e3 / reps


def suffix_proposer(reps=30):
    """Suffix-decoding proposals for the 64 n-gram contexts (8192 tokens)
    against a shared 262144-token history: HIP-event mean per call.  The
    texts hold 4 * (64 * 8192 + 262144) bytes; each sequence scans the
    history itself (64 reads of it, mostly from cache)."""
    import torch
    import proposal_sv_verify_amd as sv
    from proposal_sv_verify_amd import workloads as W

    c = W.SUFFIX
    wl = W.suffix_workload(c["B"], c["L"], c["H"], seed=W.seed_for(2, salt=7))
    dev = torch.device("cuda:0")
    tok = torch.from_numpy(wl["tokens"]).to(dev)
    lens = torch.from_numpy(wl["lengths"]).to(dev)
    hist = torch.from_numpy(wl["history"]).to(dev)
    call = sv.prepare_suffix(tok, lens, hist, c["m_min"], c["m_max"], c["K"], c["min_prob"])
    us = _timed([call], reps)
    out = {k: v.cpu().numpy() for k, v in call().items()}
    text_bytes = 4 * (c["B"] * c["L"] + c["H"])
    return dict(contexts=c["B"], context_len=c["L"], history=c["H"], m_max=c["m_max"], K=c["K"],
                min_prob=c["min_prob"], us_per_call=round(us, 2),
                proposals_per_s=round(c["B"] / us * 1e6, 1), text_bytes=text_bytes,
                gb_per_s_text=round(text_bytes / us / 1e3, 1),
                mean_proposal_len=round(float(out["proposal_len"].mean()), 3),
                from_history=int((out["source"] == 1).sum()))


def greedy_small(reps=200):
    """The small greedy workload (B 4, K 4, V 32000, fp32 logits N(0, 1),
    planted acceptance 0.7): 20 rows, 2.56 MB, so the call is bound by
    launch and memory latency, not bandwidth.  HIP-event mean per call."""
    import torch
    import proposal_sv_verify_amd as sv
    from proposal_sv_verify_amd import workloads as W

    c = W.GREEDY_SMALL
    wl = W.greedy_workload(c["B"], c["K"], c["V"], c["dtype"], c["sigma"], c["alphas"],
                           seed=W.seed_for(1))
    dev = torch.device("cuda:0")
    call = sv.prepare_greedy(torch.from_numpy(wl["logits"]).to(dev),
                             torch.from_numpy(wl["drafts"][c["alphas"][0]]).to(dev))
    us = _timed([call], reps)
    positions = c["B"] * (c["K"] + 1)
    nbytes = positions * c["V"] * 4
    return dict(B=c["B"], K=c["K"], V=c["V"], dtype=c["dtype"], us_per_call=round(us, 2),
                positions_per_s=round(positions / us * 1e6, 1), algorithmic_bytes=nbytes,
                gb_per_s=round(nbytes / us / 1e3, 1))


def greedy_alphas(gr, reps=30):
    """The large greedy workload's three planted acceptance rates on the same
    logits (drafts planted from the numpy argmax of each row): HIP-event mean
    per call, and the measured tokens per step beside the closed form
    (1 - a^(K+1)) / (1 - a).  The call reads every row whatever the drafts,
    so its time does not depend on the rate."""
    import torch
    import proposal_sv_verify_amd as sv
    from proposal_sv_verify_amd import workloads as W

    dev = torch.device("cuda:0")
    lg_np = gr["logits"]
    B, K1, V = lg_np.shape
    K = K1 - 1
    top = W._row_argmax(lg_np[:, :K, :]).reshape(B, K)
    lg = torch.from_numpy(lg_np.view(np.int16)).to(dev).view(torch.bfloat16)
    res = {}
    for a in (0.3, 0.6, 0.9):
        dr = W.planted_acceptance_drafts(top, V, a, seed=W.seed_for(4, salt=int(a * 10)))
        call = sv.prepare_greedy(lg, torch.from_numpy(dr.astype(np.int32)).to(dev))
        us = _timed([call], reps)
        acc = call()["accepted"].cpu().numpy()
        res["alpha_%.1f" % a] = dict(us_per_call=round(us, 2),
                                     gb_per_s=round(B * K1 * V * 2 / us / 1e3, 1),
                                     tokens_per_step=round(float(acc.mean()) + 1.0, 4),
                                     tokens_per_step_closed_form=round((1 - a ** K1) / (1 - a), 4))
    return res


def graph_steps(d, reps=100):
    """The step's four calls captured once in a HIP graph and replayed,
    beside the same calls launched one by one on the same stream; and a
    small-batch decode step (n-gram proposals for 4 contexts of 2048 tokens,
    then greedy verification of B 4, K 4, V 32000 fp32) where launching
    dominates.  HIP-event means per step with the host running ahead, and
    the host-observed median per step when the host waits for each step
    (launch, then synchronise), as a decode loop does."""
    import torch
    import proposal_sv_verify_amd as sv
    from proposal_sv_verify_amd import workloads as W

    dev = torch.device("cuda:0")
    s = torch.cuda.Stream(device=dev)

    def measure(make):
        with torch.cuda.stream(s):
            calls = make()
            for c in calls:
                c()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for c in calls:
                c()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            eager = _timed(calls, reps)
            graph = _timed([g.replay], reps)

        def waited(fns):
            # host-observed latency: launch, then wait for the stream, per step
            for f in fns:
                f()
            s.synchronize()
            t = []
            for _ in range(reps):
                t0 = time.perf_counter()
                for f in fns:
                    f()
                s.synchronize()
                t.append(time.perf_counter() - t0)
            return float(np.median(t)) * 1e6

        with torch.cuda.stream(s):
            eager_w = waited(calls)
            graph_w = waited([g.replay])
        return eager, graph, eager_w, graph_w

    def main_step():
        return [sv.prepare_ngram(d["ng_tok"], d["ng_len"], 2, 5, 8),
                sv.prepare_rejection(d["rj_t"], d["rj_d"], d["rj_x"], d["rj_u"], 1.0),
                sv.prepare_greedy(d["gr_l"], d["gr_x"]),
                sv.prepare_tree(d["tr_l"], d["tr_p"], d["tr_t"])]

    ng = W.ngram_workload(4, 2048, seed=W.seed_for(2, salt=3))
    c1 = W.GREEDY_SMALL
    g1 = W.greedy_workload(c1["B"], c1["K"], c1["V"], c1["dtype"], c1["sigma"], c1["alphas"],
                           seed=W.seed_for(1))
    small_in = [torch.from_numpy(a).to(dev) for a in
                (ng["tokens"], ng["lengths"], g1["logits"], g1["drafts"][c1["alphas"][0]])]

    def small_step():
        return [sv.prepare_ngram(small_in[0], small_in[1], 2, 5, 8),
                sv.prepare_greedy(small_in[2], small_in[3])]

    e_main, g_main, ew_main, gw_main = measure(main_step)
    e_small, g_small, ew_small, gw_small = measure(small_step)
    positions = 64 * 6 + 256 * 9 + 32 * 64
    return dict(step_us_eager=round(e_main, 2), step_us_graph=round(g_main, 2),
                positions_per_s_graph=round(positions / g_main * 1e6, 1),
                step_us_eager_waited=round(ew_main, 1), step_us_graph_waited=round(gw_main, 1),
                small_step=dict(workload="ngram B4 L2048 + greedy B4 K4 V32000 f32",
                                us_eager=round(e_small, 2), us_graph=round(g_small, 2),
                                us_eager_waited=round(ew_small, 1), us_graph_waited=round(gw_small, 1)))


def rejection_shards(d, shards=8, reps=30):
    """The rejection workload in the eight 16032-column vocabulary shards
    of an 8-way tensor-parallel output layer: per-shard statistics, the
    accept test on the partials, per-shard sample masses and the owner
    shard's sample, beside the unsharded call.  HIP-event means."""
    import torch
    import proposal_sv_verify_amd as sv

    tg, dg, x, u = d["rj_t"], d["rj_d"], d["rj_x"], d["rj_u"]
    B, K1, V = tg.shape
    K = K1 - 1
    dev = tg.device
    cuts = [(i * V // shards, (i + 1) * V // shards) for i in range(shards)]
    parts = torch.empty(shards, B * (2 * K + 1), 2, dtype=torch.float64, device=dev)
    stats_calls = [sv.prepare_rejection_shard_stats(tg[..., a:b], dg[..., a:b], x, a, 1.0,
                                                    out=parts[p]) for p, (a, b) in enumerate(cuts)]
    for c in stats_calls:
        c()
    decide = sv.prepare_rejection_partials(parts, x, u, V, 1.0)
    state = decide()["state"]
    masses = torch.empty(shards, B, 2, dtype=torch.float64, device=dev)
    mass_calls = [sv.prepare_rejection_shard_mass(tg[..., a:b], dg[..., a:b], state, 1.0,
                                                  out=masses[p]) for p, (a, b) in enumerate(cuts)]
    emitted = torch.full((B, K1), -1, dtype=torch.int32, device=dev)
    sample_calls = [sv.prepare_rejection_shard_sample(tg[..., a:b], dg[..., a:b], x, u, state, masses,
                                                      p, a, mass_calls[p].out["workspace"], emitted,
                                                      1.0) for p, (a, b) in enumerate(cuts)]
    whole = sv.prepare_rejection(tg, dg, x, u, 1.0)
    t_stats = _timed(stats_calls, reps)
    t_decide = _timed([decide], reps)
    t_mass = _timed(mass_calls, reps)
    t_sample = _timed(sample_calls, reps)
    t_all = _timed(stats_calls + [decide] + mass_calls + sample_calls, reps)
    t_whole = _timed([whole], reps)
    ref = whole()
    same_acc = int((decide()["accepted"] == ref["accepted"]).sum())
    same_emi = int((emitted == ref["emitted"]).all(dim=1).sum())
    nbytes = B * (2 * K + 1) * V * 2
    return dict(shards=shards, us_stats_calls=round(t_stats, 2), us_accept=round(t_decide, 2),
                us_mass_calls=round(t_mass, 2), us_sample_calls=round(t_sample, 2),
                us_all_steps=round(t_all, 2), us_unsharded=round(t_whole, 2),
                gb_per_s_stats_calls=round(nbytes / t_stats / 1e3, 1),
                sequences_same_accepted=same_acc, sequences_same_emitted=same_emi, sequences=B)


def greedy_shards(gr, shards=8, reps=30):
    """The large greedy workload as an 8-way vocabulary-sharded output layer
    would hold it: sv_argmax_shard on each 18992-column slice, then
    sv_verify_greedy_partials, beside the unsharded call on the same
    logits.  Times are HIP-event means over `reps` repetitions."""
    import torch
    import proposal_sv_verify_amd as sv

    dev = torch.device("cuda:0")
    lg = torch.from_numpy(gr["logits"].view(np.int16)).to(dev).view(torch.bfloat16)
    dr = torch.from_numpy(gr["drafts"][0.6]).to(dev)
    V = lg.shape[-1]
    rows = lg.shape[0] * lg.shape[1]
    cuts = [(i * V // shards, (i + 1) * V // shards) for i in range(shards)]
    parts = torch.empty(shards, rows, dtype=torch.int64, device=dev)
    shard_calls = [sv.prepare_argmax_shard(lg[..., a:b], a, out=parts[p]) for p, (a, b) in enumerate(cuts)]
    combine = sv.prepare_greedy_partials(parts, dr, V)
    whole = sv.prepare_greedy(lg, dr)

    t_shards = _timed(shard_calls, reps)
    t_combine = _timed([combine], reps)
    t_whole = _timed([whole], reps)
    same = all(torch.equal(combine()[k], whole()[k]) for k in ("accepted", "emitted", "argmax"))
    nbytes = rows * V * 2
    return dict(shards=shards, us_shard_calls=round(t_shards, 2), us_combine=round(t_combine, 2),
                us_unsharded=round(t_whole, 2),
                gb_per_s_shard_calls=round(nbytes / t_shards / 1e3, 1), same_result=bool(same))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(ng, rj, gr, tr, seconds, gpu_outs, step_bytes):
    """The oracle, as it stands, on the host cores: whole steps (all four
    calls, every sequence), sequences spread over a thread pool, for at
    least `seconds` of wall time, then one step on a single thread.  Also
    reports whether it agrees with the GPU step's outputs."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    threads = len(os.sched_getaffinity(0))
    pool = ThreadPoolExecutor(threads)

    def split(B):
        n = min(B, threads * 4)
        edges = np.linspace(0, B, n + 1).astype(int)
        return [(a, b) for a, b in zip(edges[:-1], edges[1:]) if b > a]

    def merge(parts):
        return {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}

    def step():
        o = {}
        o["ngram"] = merge(list(pool.map(lambda ab: oracle.ngram_propose(
            ng["tokens"][ab[0]:ab[1]], ng["lengths"][ab[0]:ab[1]], 2, 5, 8), split(64))))
        o["rejection"] = merge(list(pool.map(lambda ab: oracle.verify_rejection(
            rj["target"][ab[0]:ab[1]], rj["draft_logits"][ab[0]:ab[1]], rj["draft"][ab[0]:ab[1]],
            rj["uniforms"][ab[0]:ab[1]], 1.0), split(64))))
        o["greedy"] = merge(list(pool.map(lambda ab: oracle.verify_greedy(
            gr["logits"][ab[0]:ab[1]], gr["drafts"][0.6][ab[0]:ab[1]]), split(256))))
        o["tree"] = merge(list(pool.map(lambda ab: oracle.verify_tree(
            tr["logits"][ab[0]:ab[1]], tr["parent"][ab[0]:ab[1]], tr["token"][ab[0]:ab[1]]),
            split(32))))
        return o

    t0 = time.perf_counter()
    n = 0
    ref = None
    while True:
        ref = step()
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    pool.shutdown()
    pool = ThreadPoolExecutor(1)
    t1 = time.perf_counter()
    step()
    el1 = time.perf_counter() - t1
    pool.shutdown()
    parity = None
    if gpu_outs is not None:
        g = gpu_outs
        ok = all(np.array_equal(g["greedy"][k], ref["greedy"][k]) for k in ("accepted", "emitted"))
        ok &= all(np.array_equal(g["tree"][k], ref["tree"][k]) for k in ("accepted", "path", "emitted"))
        ok &= all(np.array_equal(g["ngram"][k], ref["ngram"][k])
                  for k in ("proposal", "proposal_len", "match_n", "match_pos"))
        r = ref["rejection"]
        same = (g["rejection"]["accepted"] == r["accepted"]) & \
               (g["rejection"]["emitted"] == r["emitted"]).all(axis=1)
        tie = r["accept_tie"] | r["sample_tie"]
        ok &= bool((same | tie).all())
        parity = dict(all_match=bool(ok), rejection_flagged_ties=int(tie.sum()),
                      rejection_mismatches=int((~same).sum()))
    return dict(value=round(4736 * n / el, 1), unit="verified positions/s", cores=threads,
                kind="oracle", cpu_model=cpu_model(),
                gb_per_s=round(step_bytes * n / el / 1e9, 2),
                value_1thread=round(4736 / el1, 1),
                sample="%d full step(s): all four calls over every sequence (%.1f s); "
                       "then one step on one thread (%.1f s)" % (n, el, el1)), parity


def stream_ceiling(reps=10):
    """The measured streaming-read rate of this GPU: sv_read_probe (the
    verifiers' 16-byte loads, nothing else) over 2 GiB, well above the
    256 MiB last-level cache; HIP-event mean over reps after a warm-up."""
    import torch
    import proposal_sv_verify_amd as sv
    dev = torch.device("cuda:0")
    nbytes = 2 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    call = sv.prepare_read_probe(buf)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    call()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    gbs = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf
    torch.cuda.empty_cache()
    return dict(read_gb_per_s=round(gbs, 1), bytes=nbytes, kernel="sv_read_probe")


def calibrate_copy():
    """A plain device copy of 256 MiB (reads 256 MiB, writes 256 MiB), three
    times: the reference launch for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.empty(64 * 1024 * 1024, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def load_traffic(name, per_launch_us_unused=None):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if the
    kernel's sources are unchanged since they were taken."""
    path = os.path.join(PROFILES, "%s_counters.json" % name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("source_hash") != source_hash(KERNEL_SOURCES[name]):
        return None
    return c.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-bandwidth-mode", action="store_true",
                    help="skip the 16384-context n-gram measurement")
    ap.add_argument("--no-shards", action="store_true",
                    help="skip the vocabulary-sharded greedy and rejection measurements")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the measured copy / read ceiling")
    ap.add_argument("--no-suffix", action="store_true",
                    help="skip the suffix-decoding proposer measurement")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the alternative step executions: HIP-graph replay (of the step and of a small-batch step) and the four-stream step")
    ap.add_argument("--no-greedy-extra", action="store_true",
                    help="skip the small greedy workload and the acceptance-rate sweep")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the steps, copy a 256 MiB device buffer three times (a "
                         "kernel of known traffic for scaling the rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    ng, rj, gr, tr = make_inputs()
    wall, samples, outs, dev_inputs = run_gpu(args, ng, rj, gr, tr)
    per = {name: float(np.mean(v)) for name, v in samples.items()}
    if args.calibrate_copy:
        calibrate_copy()
    K = args.steps
    ms_step = wall / K * 1e3
    positions = 64 * 6 + 256 * 9 + 32 * 64

    algo = {
        "rejection": 64 * 6 * 128256 * 2 + 64 * 5 * 128256 * 2,
        "greedy": 256 * 9 * 151936 * 2,
        "tree": 32 * 64 * 128256 * 2,
        "ngram": ngram_bytes(outs["ngram"], ng["lengths"], 5),
    }
    units = {"rejection": 384, "greedy": 2304, "tree": 2048, "ngram": 64}
    kernels = {}
    for name, us in per.items():
        gbs = algo[name] / us / 1e3
        p10, p50, p90 = np.percentile(samples[name], [10, 50, 90])
        kernels[name] = dict(us_per_call=round(us, 2), us_p10_p50_p90=[round(float(p10), 2),
                                                                     round(float(p50), 2),
                                                                     round(float(p90), 2)],
                             algorithmic_bytes=algo[name],
                             gb_per_s=round(gbs, 1), frac_of_peak=round(gbs / PEAK_HBM_GBS, 4),
                             units_per_s=round(units[name] / us * 1e6, 1),
                             unit="proposals" if name == "ngram" else "positions")
    dom = max(("rejection", "greedy", "tree"), key=lambda k: per[k])
    achieved = algo[dom] / per[dom] / 1e3
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(achieved / PEAK_HBM_GBS, 4),
                    traffic=load_traffic(dom) if dom in KERNEL_SOURCES else None,
                    kernel=dom, launch=LAUNCH_KERNELS[dom],
                    algorithmic_bytes_per_launch=algo[dom], avg_launch_us=round(per[dom], 2))

    result = dict(metric=METRIC, value=round(positions * K / wall, 1), unit="verified positions/s",
                  n_gpus=1, steps=K, warmup=args.warmup, ms_per_step=round(ms_step, 4),
                  higher_is_better=True, scaling="weak", vs_baseline=None,
                  dtype="bf16 logits (argmax compares in f32); rejection f32 exp and 16-byte-vector sums, "
                        "f64 across vectors and after", data="synthetic",
                  config=dict(workload="one verify+propose pass: ngram B64 L8192 n5..2 K8; "
                                       "rejection B64 K5 V128256 bf16 T1; greedy B256 K8 V151936 "
                                       "bf16 alpha0.6; tree B32 N64 V128256 bf16",
                              positions_per_step=positions, proposals_per_step=64),
                  roofline=roofline, kernels=kernels)
    if not args.no_ceiling:
        ceil = stream_ceiling()
        result["stream_ceiling"] = ceil
        for k in kernels.values():
            k["frac_of_measured_ceiling"] = round(k["gb_per_s"] / ceil["read_gb_per_s"], 4)
        roofline["frac_of_measured_ceiling"] = round(achieved / ceil["read_gb_per_s"], 4)
    if not args.no_bandwidth_mode:
        result["ngram_bandwidth_mode"] = ngram_bandwidth_mode(args)
    if not args.no_suffix:
        result["suffix_proposer"] = suffix_proposer()
    if not args.no_graph:
        result["graph_step"] = graph_steps(dev_inputs)
        result["step_concurrent"] = concurrent_step(dev_inputs, outs, K, positions)
    if not args.no_greedy_extra:
        result["greedy_small"] = greedy_small()
        result["greedy_alphas"] = greedy_alphas(gr)
    if not args.no_shards:
        result["greedy_vocab_shards"] = greedy_shards(gr)
        result["rejection_vocab_shards"] = rejection_shards(dev_inputs)
    if not args.no_cpu:
        cb, parity = cpu_baseline(ng, rj, gr, tr, args.cpu_seconds, outs,
                                  algo["rejection"] + algo["greedy"] + algo["tree"] + algo["ngram"])
        result["cpu_baseline"] = cb
        result["parity"] = parity
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
