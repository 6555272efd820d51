#!/usr/bin/env python3
"""MoG decode-attention throughput on one MI355X.

Prints ONE JSON line: MoG (Iceberg) decode-attention steps/s at N=1M (the
`value`, GQA 40q/8kv, d=128, bf16) and at N=128K (batch 4, 32 MHA heads),
achieved HBM GB/s, the fraction of the KV cache read, the speedup over the
in-library dense decode, approximation errors against dense attention, the
roofline of the exact-attention kernel (timed live with HIP events recorded
around it on its stream), and the CPU oracle timed on a bounded sample.

A step is one full decode pass (cluster scoring, top-c, subcluster scoring
and top-s, exact attention, residual, merge) over one batch of queries; the
KV cache and its cluster layout are resident in HBM when timing starts,
queries rotate through pre-generated sets so selections change every step,
and consecutive steps run on three copies of the cache and layout in other
memory, so the last-level cache cannot serve a step the bytes of the one
before.  Reported per workload: the mean over the timed steps (the value),
the p10 / p50 / p90 of per-step times, the time per step of a replayed HIP
graph of the same steps, and the exact and dense kernels alone, timed by the
events their own dispatches set.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoG decode-attention steps/s at N=128K and 1M + achieved HBM GB/s"
HBM_PEAK_GBPS = 8000.0


class HipEvents:
    """Raw hipEvent_t handles (the library records them on its stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.owned = []

    def create(self):
        ev = ctypes.c_void_p()
        rc = self.hip.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        self.owned.append(ev)
        return ev

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def close(self):
        for ev in self.owned:
            self.hip.hipEventDestroy(ev)
        self.owned.clear()


def selection_volume(wl, lay, sel_c, sel_s, offs):
    """Rows and bytes a step must move, from the selections (per step)."""
    G, d = wl.group, wl.head_dim
    e = 2 if wl.dtype == "bf16" else 4
    rows_union = rows_head = 0
    stat_bytes = 0
    rest_bytes = 0  # the residual of the clusters left out: mean values, scores and head masks read
    n_tokens = 0
    for s in range(wl.n_seq):
        N = wl.seq_lens[s]
        for h in range(wl.n_kv_heads):
            u = s * wl.n_kv_heads + h
            U = lay.unit(u)
            C, S = U.C, U.S
            off = offs[u]
            n_tokens += N
            chosen_sets = []
            subs_union = set()
            sub_vbar_needed = set()
            for g in range(G):
                hq = h * G + g
                cs = set()
                for r, j in enumerate(sel_c[s, hq]):
                    if j < 0:
                        continue
                    cs.add(int(j))
                    picks = {int(i) for i in sel_s[s, hq, r] if i >= 0}
                    for i in range(S):
                        gg = int(j) * S + i
                        if off[gg + 1] == off[gg]:
                            continue
                        if i in picks:
                            subs_union.add(gg)
                            rows_head += off[gg + 1] - off[gg]
                        else:
                            sub_vbar_needed.add(gg)
                chosen_sets.append(cs)
            union_c = set().union(*chosen_sets) if chosen_sets else set()
            inter_c = set.intersection(*chosen_sets) if chosen_sets else set()
            rows_u = sum(off[g + 1] - off[g] for g in subs_union) + wl.n_sink + wl.n_recent
            rows_union += rows_u
            rows_head += G * (wl.n_sink + wl.n_recent)
            # group statistics are read in bf16 (2 bytes an element), counts
            # as int32 offsets
            stat_bytes += C * (2 * d * 2 + 4)              # cluster mean, variance, count
            stat_bytes += (C - len(inter_c)) * d * 2       # cluster mean values left out
            rest_bytes += (C - len(inter_c)) * d * 2 + C * (G + 1) * 4
            stat_bytes += len(union_c) * S * (2 * d * 2 + 4)
            stat_bytes += len(sub_vbar_needed) * d * 2
            stat_bytes += G * d * 4 * 2                    # queries in, outputs out
    kv_rows_bytes = rows_union * d * 2 * e
    return dict(rows_union=rows_union, rows_per_head=rows_head / G, n_tokens=n_tokens,
                kv_row_bytes=kv_rows_bytes, rest_bytes=rest_bytes, step_bytes=kv_rows_bytes + stat_bytes)


def replicate(wl, b, kv0, lay0, replicas):
    """Copies of the cache in other device memory, each with its own layout
    (the build is deterministic, so selections and results are the same):
    a step on copy i % R never re-reads what the step before it touched, so
    the 256 MB last-level cache cannot serve repeated bytes."""
    import torch

    from long_context_sparse_mog_amd import ops

    reps = [(kv0, lay0)]
    for _ in range(1, replicas):
        if wl.paged:
            kv = ops.KVCache(b.pool_K.clone(), b.pool_V.clone(), wl.seq_lens, b.block_table)
        else:
            kv = ops.KVCache(b.K.clone(), b.V.clone(), wl.seq_lens)
        lay = ops.mog_build(kv, wl.n_sink, wl.n_recent, kmeans_iters=wl.kmeans_iters, seed=1)
        reps.append((kv, lay))
    torch.cuda.synchronize()
    return reps


def time_steps(step, k, w):
    """W untimed warmup steps, then exactly K timed steps (torch events around
    them): ms per step.  Then K more steps with an event after each: the
    p10 / p50 / p90 of the per-step times."""
    import numpy as np
    import torch

    for i in range(w):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(k):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    mean = e0.elapsed_time(e1) / k
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(k + 1)]
    evs[0].record()
    for i in range(k):
        step(i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(k)])
    return mean, dict(p10=float(np.percentile(per, 10)), p50=float(np.percentile(per, 50)),
                      p90=float(np.percentile(per, 90)))


def time_graph(step, n_inner, k, check):
    """n_inner steps captured in one HIP graph, replayed until at least K
    steps ran (after one untimed replay): ms per step.  ``check()`` then
    compares the graph's last outputs with an eager run; None if they
    differ."""
    import torch

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(0)  # (warm the allocator and the library on the capture stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(n_inner):
            step(i)
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, -(-k // n_inner))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * n_inner)
    ok = check()
    del g
    return ms if ok else None


def kernel_event_ms(run, n, ev):
    """Mean duration of the exact (or dense) kernel over n single launches,
    from the events its own dispatch sets (one pair per step)."""
    import torch

    pairs = []
    for i in range(n):
        a, z = ev.create(), ev.create()
        run(i, a, z)
        pairs.append((a, z))
    torch.cuda.synchronize()
    return sum(ev.elapsed_ms(a, z) for a, z in pairs) / n


def bench_workload(idx, steps, warmup, n_qsets, ev, with_errors=True, shared_too=False, replicas=3,
                   graph=True):
    import numpy as np
    import torch

    from long_context_sparse_mog_amd import capi, ops, synth

    wl = synth.config(idx)
    t0 = time.time()
    b = synth.generate(wl, device="cuda", n_qsets=n_qsets, keep_contiguous=not wl.paged)
    kv = ops.KVCache.from_batch(b)
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    torch.cuda.synchronize()
    t0 = time.time()
    lay = ops.mog_build(kv, wl.n_sink, wl.n_recent, kmeans_iters=wl.kmeans_iters, seed=1)
    torch.cuda.synchronize()
    build_s = time.time() - t0
    reps = replicate(wl, b, kv, lay, replicas)
    R = len(reps)
    qs = [b.Q[i].contiguous() for i in range(n_qsets)]
    out = torch.empty_like(qs[0])
    lse = torch.empty(qs[0].shape[:2], device="cuda")

    p0 = ops.decode_params(wl.n_q_heads, list(wl.top_c), list(wl.top_s))
    ws = ops.workspace(ops.mog_workspace_size(capi.MOG_OP_DECODE, layout=lay, params=p0))
    pd0 = ops.decode_params(wl.n_q_heads, 1, 1)
    wsd = ops.workspace(ops.mog_workspace_size(capi.MOG_OP_DENSE, kv=kv, params=pd0))

    def mog_step(p):
        return lambda i: ops.mog_decode(reps[i % R][1], reps[i % R][0], qs[i % n_qsets], p, out=out, lse=lse, ws=ws)

    def dense_step(i):
        ops.mog_dense_decode(reps[i % R][0], qs[i % n_qsets], pd0, out=out, lse=lse, ws=wsd)

    def with_events(p_kw, i, a, z, dense=False):
        p = ops.decode_params(wl.n_q_heads, *( (1, 1) if dense else (list(wl.top_c), list(wl.top_s)) ), **p_kw)
        p.exact_begin, p.exact_end = a, z
        if dense:
            ops.mog_dense_decode(reps[i % R][0], qs[i % n_qsets], p, out=out, lse=lse, ws=wsd)
        else:
            ops.mog_decode(reps[i % R][1], reps[i % R][0], qs[i % n_qsets], p, out=out, lse=lse, ws=ws)

    n_ev = min(steps, 64)
    mog_ms, mog_pct = time_steps(mog_step(p0), steps, warmup)
    exact_ms = kernel_event_ms(lambda i, a, z: with_events({}, i, a, z), n_ev, ev)
    graph_ms = None
    if graph:
        n_inner = R * n_qsets // math.gcd(R, n_qsets)

        def check():
            ref = torch.empty_like(out)
            last = n_inner - 1
            got = out.clone()
            ops.mog_decode(reps[last % R][1], reps[last % R][0], qs[last % n_qsets], p0, out=ref, ws=ws)
            torch.cuda.synchronize()
            return torch.equal(got, ref)

        graph_ms = time_graph(mog_step(p0), n_inner, steps, check)
    dsteps = max(10, steps // 4)
    dense_ms, dense_pct = time_steps(dense_step, dsteps, max(2, warmup // 2))
    dense_kern_ms = kernel_event_ms(lambda i, a, z: with_events({}, i, a, z, dense=True), min(dsteps, 16), ev)

    # selections and errors (outside the timed region)
    offs = [lay.export_unit(u)["sub_off"] for u in range(lay.n_units)]
    vols = []
    err_res, err_top = [], []
    pt = ops.decode_params(wl.n_q_heads, list(wl.top_c), list(wl.top_s), residual=False)
    # (the volumes over every query set the timed steps cycle through; the
    # errors against dense on the first four)
    for t in range(n_qsets):
        o, _, sc, ss = ops.mog_decode(lay, kv, qs[t], p0, want_sel=True)
        vols.append(selection_volume(wl, lay, sc.cpu().numpy(), ss.cpu().numpy(), offs))
        if with_errors and t < 4:
            od, _ = ops.mog_dense_decode(kv, qs[t], pd0)
            ot = ops.mog_decode(lay, kv, qs[t], pt)[0]
            err_res.append((torch.linalg.norm(o - od, dim=-1) / torch.linalg.norm(od, dim=-1)).flatten())
            err_top.append((torch.linalg.norm(ot - od, dim=-1) / torch.linalg.norm(od, dim=-1)).flatten())
    mean = lambda k: float(np.mean([v[k] for v in vols]))
    e = 2 if wl.dtype == "bf16" else 4
    dense_bytes = wl.kv_bytes()
    # a whole-cluster budget (top_s >= S everywhere; the timed steps ask for
    # no subcluster output) skips the subcluster kernel; with either budget
    # the residual of the clusters left out runs in the exact kernel's launch,
    # after its exact blocks, so its bytes count there
    whole = all(wl.top_s[s] >= lay.unit(s * wl.n_kv_heads).S for s in range(wl.n_seq))
    exact_bytes = mean("kv_row_bytes") + mean("rest_bytes")
    res = dict(
        workload=wl.name, n_seq=wl.n_seq, seq_lens=wl.seq_lens if wl.n_seq <= 4 else "ragged",
        n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim, dtype=wl.dtype,
        top_c=wl.top_c[0] if len(set(wl.top_c)) == 1 else "per-seq", top_s=wl.top_s[0] if len(set(wl.top_s)) == 1 else "per-seq",
        replicas=R,
        steps_per_s=1000.0 / mog_ms, ms_per_step=mog_ms,
        ms_p10=mog_pct["p10"], ms_p50=mog_pct["p50"], ms_p90=mog_pct["p90"],
        graph_ms_per_step=graph_ms,
        exact_kernel_ms=exact_ms,
        whole_cluster_path=whole,
        step_bytes=mean("step_bytes"), exact_kernel_bytes=exact_bytes, exact_row_bytes=mean("kv_row_bytes"),
        hbm_GBps=mean("step_bytes") / (mog_ms * 1e-3) / 1e9,
        exact_kernel_GBps=exact_bytes / (exact_ms * 1e-3) / 1e9,
        frac_kv_read_union=mean("rows_union") / mean("n_tokens"),
        frac_kv_read_per_head=mean("rows_per_head") / mean("n_tokens"),
        dense_ms_per_step=dense_ms, dense_ms_p50=dense_pct["p50"], dense_kernel_ms=dense_kern_ms,
        dense_GBps=dense_bytes / (dense_kern_ms * 1e-3) / 1e9,
        speedup_vs_dense=dense_ms / mog_ms,
        build_s=build_s, gen_s=gen_s,
    )
    if with_errors:
        er, et = torch.cat(err_res), torch.cat(err_top)
        res.update(err_vs_dense_residual_mean=float(er.mean()), err_vs_dense_residual_max=float(er.max()),
                   err_vs_dense_toponly_mean=float(et.mean()), err_vs_dense_toponly_max=float(et.max()))
    if shared_too:
        # the same step with one selection per KV head (the heads' summed
        # mass fractions): steps/s, exact kernel, rows read, error vs dense
        p0s = ops.decode_params(wl.n_q_heads, list(wl.top_c), list(wl.top_s), shared=True)
        ms_s, pct_s = time_steps(mog_step(p0s), steps, warmup)
        ex_s = kernel_event_ms(lambda i, a, z: with_events({"shared": True}, i, a, z), n_ev, ev)
        vols_s, err_s = [], []
        for t in range(n_qsets):
            o, _, sc, ss = ops.mog_decode(lay, kv, qs[t], p0s, want_sel=True)
            vols_s.append(selection_volume(wl, lay, sc.cpu().numpy(), ss.cpu().numpy(), offs))
            if with_errors and t < 4:
                od, _ = ops.mog_dense_decode(kv, qs[t], pd0)
                err_s.append((torch.linalg.norm(o - od, dim=-1) / torch.linalg.norm(od, dim=-1)).flatten())
        mean_s = lambda k: float(np.mean([v[k] for v in vols_s]))
        res["shared_selection"] = dict(
            steps_per_s=1000.0 / ms_s, ms_per_step=ms_s, ms_p50=pct_s["p50"], exact_kernel_ms=ex_s,
            exact_kernel_bytes=mean_s("kv_row_bytes") + mean_s("rest_bytes"),
            exact_kernel_GBps=(mean_s("kv_row_bytes") + mean_s("rest_bytes")) / (ex_s * 1e-3) / 1e9,
            frac_kv_read_union=mean_s("rows_union") / mean_s("n_tokens"),
            speedup_vs_dense=dense_ms / ms_s,
            err_vs_dense_residual_mean=float(torch.cat(err_s).mean()) if err_s else None,
            err_vs_dense_residual_max=float(torch.cat(err_s).max()) if err_s else None)
    del reps[1:]
    torch.cuda.empty_cache()
    state = dict(wl=wl, b=b, lay=lay, qs=qs, e=e)
    return res, state


def incremental_bench(state, steps, warmup):
    """Incremental decode on the same workload: the layout is built on the
    first N - 2T tokens (T = warmup + steps) with a fold area of 2T rows, then
    (A) T single-token appends alone, (B) T steps of one single-token append
    (mog_append) plus one decode (mog_decode) on the grown cache, (C) decode
    alone on the final cache.  Timed with torch events around the K timed
    calls of each phase (after W untimed ones)."""
    import torch

    from long_context_sparse_mog_amd import capi, ops

    wl, b, qs = state["wl"], state["b"], state["qs"]
    nq = len(qs)
    T = steps + warmup
    kv_full = ops.KVCache.from_batch(b)
    n0 = [L - 2 * T for L in wl.seq_lens]
    kvs = [kv_full.with_lens([x + i for x in n0]) for i in range(2 * T + 1)]
    lay = ops.mog_build(kvs[0], wl.n_sink, wl.n_recent, kmeans_iters=wl.kmeans_iters, seed=1, fold_capacity=2 * T)
    p0 = ops.decode_params(wl.n_q_heads, list(wl.top_c), list(wl.top_s))
    ws = ops.workspace(ops.mog_workspace_size(capi.MOG_OP_DECODE, layout=lay, params=p0))
    out = torch.empty_like(qs[0])
    lse = torch.empty(qs[0].shape[:2], device="cuda")
    torch.cuda.synchronize()

    def burst(fn, lo):
        for i in range(lo, lo + warmup):
            fn(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(lo + warmup, lo + T):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    append_ms = burst(lambda i: ops.mog_append(lay, kvs[i + 1]), 0)

    def step(i):
        ops.mog_append(lay, kvs[i + 1])
        ops.mog_decode(lay, kvs[i + 1], qs[i % nq], p0, out=out, lse=lse, ws=ws)

    step_ms = burst(step, T)
    decode_ms = burst(lambda i: ops.mog_decode(lay, kvs[2 * T], qs[i % nq], p0, out=out, lse=lse, ws=ws), 0)
    # approximation error at the final length, folded layout vs dense
    pd = ops.decode_params(wl.n_q_heads, 1, 1)
    errs = []
    for t in range(min(4, nq)):
        o = ops.mog_decode(lay, kvs[2 * T], qs[t], p0)[0]
        od, _ = ops.mog_dense_decode(kvs[2 * T], qs[t], pd)
        errs.append((torch.linalg.norm(o - od, dim=-1) / torch.linalg.norm(od, dim=-1)).flatten())
    er = torch.cat(errs)
    res = dict(steps_per_s=1000.0 / step_ms, ms_per_step=step_ms, append_ms=append_ms,
               decode_only_ms=decode_ms, folded_tokens_at_end=2 * T, seq_len_at_build=n0[0],
               err_vs_dense_residual_mean=float(er.mean()), err_vs_dense_residual_max=float(er.max()))
    del lay, ws, kvs
    torch.cuda.empty_cache()
    return res


def feature_residual_comparison(steps, warmup, n_qsets, m=128):
    """The ragged paged workload (KV heads 0-3 mixture keys, 4-7 isotropic
    keys with near-uniform attention) built with feature-map summaries (m
    features): the Gaussian residual against the feature-map residual, error
    against dense per head class (mean per-head relative L2 over the query
    sets) and steps/s of each."""
    import torch

    from long_context_sparse_mog_amd import capi, ops, synth

    wl = synth.config(4)
    b = synth.generate(wl, device="cuda", n_qsets=n_qsets, keep_contiguous=False)
    kv = ops.KVCache.from_batch(b)
    W = synth.feature_map_w(m, wl.head_dim, device="cuda")
    torch.cuda.synchronize()
    t0 = time.time()
    lay = ops.mog_build(kv, wl.n_sink, wl.n_recent, kmeans_iters=wl.kmeans_iters, seed=1, fm_w=W)
    torch.cuda.synchronize()
    build_s = time.time() - t0
    qs = [b.Q[i].contiguous() for i in range(n_qsets)]
    out = torch.empty_like(qs[0])
    lse = torch.empty(qs[0].shape[:2], device="cuda")
    pd = ops.decode_params(wl.n_q_heads, 1, 1)
    res = dict(workload=wl.name, fm_dim=m, build_s_with_summaries=build_s)
    G = wl.group
    he = set(wl.high_entropy_heads)
    for name, mode in (("gaussian", True), ("feature_map", "fm"), ("top_only", False)):
        p = ops.decode_params(wl.n_q_heads, list(wl.top_c), list(wl.top_s), residual=mode)
        ws = ops.workspace(ops.mog_workspace_size(capi.MOG_OP_DECODE, layout=lay, params=p))
        for i in range(warmup):
            ops.mog_decode(lay, kv, qs[i % n_qsets], p, out=out, lse=lse, ws=ws)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            ops.mog_decode(lay, kv, qs[i % n_qsets], p, out=out, lse=lse, ws=ws)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        err_mix, err_he = [], []
        for t in range(min(4, n_qsets)):
            o = ops.mog_decode(lay, kv, qs[t], p)[0]
            od, _ = ops.mog_dense_decode(kv, qs[t], pd)
            e = (torch.linalg.norm(o - od, dim=-1) / torch.linalg.norm(od, dim=-1)).cpu()
            for hq in range(wl.n_q_heads):
                (err_he if hq // G in he else err_mix).append(e[:, hq])
        res[name] = dict(steps_per_s=1000.0 / ms, ms_per_step=ms,
                         err_vs_dense_mixture_heads=float(torch.cat(err_mix).mean()),
                         err_vs_dense_high_entropy_heads=float(torch.cat(err_he).mean()))
    del lay, kv, b
    torch.cuda.empty_cache()
    return res


def offload_bench(state, steps, ev, n_dense=4):
    """The same workload with the layout's reordered K/V rows in pinned host
    memory (anchors and statistics stay in HBM): MoG decode steps/s, the
    exact kernel's time and achieved host-link rate on the rows it reads
    (the same selections as the HBM-resident run, so the same algorithmic
    bytes), and the dense baseline reading a pinned host copy of the whole
    cache."""
    import torch

    from long_context_sparse_mog_amd import capi, ops

    wl, b, qs = state["wl"], state["b"], state["qs"]
    nq = len(qs)
    kv = ops.KVCache.from_batch(b)
    t0 = time.time()
    lay = ops.mog_build(kv, wl.n_sink, wl.n_recent, kmeans_iters=wl.kmeans_iters, seed=1, rows_host=True)
    torch.cuda.synchronize()
    build_s = time.time() - t0
    p0 = ops.decode_params(wl.n_q_heads, list(wl.top_c), list(wl.top_s))
    ws = ops.workspace(ops.mog_workspace_size(capi.MOG_OP_DECODE, layout=lay, params=p0))
    out = torch.empty_like(qs[0])
    lse = torch.empty(qs[0].shape[:2], device="cuda")
    for i in range(2):
        ops.mog_decode(lay, kv, qs[i % nq], p0, out=out, lse=lse, ws=ws)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        ops.mog_decode(lay, kv, qs[i % nq], p0, out=out, lse=lse, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    kern = []
    for i in range(min(steps, 8)):
        p = ops.decode_params(wl.n_q_heads, list(wl.top_c), list(wl.top_s))
        a, z = ev.create(), ev.create()
        p.exact_begin, p.exact_end = a, z
        ops.mog_decode(lay, kv, qs[i % nq], p, out=out, lse=lse, ws=ws)
        torch.cuda.synchronize()
        kern.append(ev.elapsed_ms(a, z))
    exact_ms = sum(kern) / len(kern)
    del lay, ws
    torch.cuda.empty_cache()
    # dense over a pinned host copy of the cache
    kh = torch.empty(b.K.shape, dtype=b.K.dtype, pin_memory=True)
    vh = torch.empty(b.V.shape, dtype=b.V.dtype, pin_memory=True)
    kh.copy_(b.K)
    vh.copy_(b.V)
    kvh = ops.KVCache(kh, vh, wl.seq_lens)
    pd = ops.decode_params(wl.n_q_heads, 1, 1)
    ops.mog_dense_decode(kvh, qs[0], pd, out=out, lse=lse)
    torch.cuda.synchronize()
    e0.record()
    for i in range(n_dense):
        ops.mog_dense_decode(kvh, qs[i % nq], pd, out=out, lse=lse)
    e1.record()
    torch.cuda.synchronize()
    dense_ms = e0.elapsed_time(e1) / n_dense
    del kh, vh, kvh
    return dict(rows_in="pinned host memory", steps_per_s=1000.0 / ms, ms_per_step=ms, exact_kernel_ms=exact_ms,
                build_s=build_s, dense_from_host_ms_per_step=dense_ms, dense_from_host_GBps=wl.kv_bytes() / (dense_ms * 1e-3) / 1e9,
                speedup_vs_dense_from_host=dense_ms / ms)


def build_timing(reps=3):
    """mog_build (10 k-means rounds, subclusters, reorder, stats) of the
    single-head 128K-key workload: median wall time over reps."""
    import numpy as np
    import torch

    from long_context_sparse_mog_amd import ops, synth

    wl = synth.build_workload()
    b = synth.generate(wl, device="cuda", n_qsets=1)
    kv = ops.KVCache.from_batch(b)
    ops.mog_build(kv, wl.n_sink, wl.n_recent, kmeans_iters=wl.kmeans_iters, seed=1)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        t0 = time.time()
        ops.mog_build(kv, wl.n_sink, wl.n_recent, kmeans_iters=wl.kmeans_iters, seed=1)
        torch.cuda.synchronize()
        ts.append(time.time() - t0)
    return dict(workload=wl.name, n_keys=wl.seq_lens[0], kmeans_iters=wl.kmeans_iters,
                seconds=float(np.median(ts)))


def cpu_baseline(state, budget_s):
    """The CPU oracle (as it stands) decoding units of the same step on the
    host cores, given the GPU-built layout; extrapolated to a whole step."""
    import numpy as np

    import oracle as O

    wl, b, lay, qs = state["wl"], state["b"], state["lay"], state["qs"]
    G = wl.group
    times = []
    units_done = 0
    qsets_used = set()
    # (seq, KV head) units of the step, query set after query set, until
    # about budget_s seconds of oracle work have been timed
    for t in range(len(qs)):
        for u in range(lay.n_units):
            s, h = divmod(u, wl.n_kv_heads)
            ex = lay.export_unit(u)
            L = O.UnitLayout(N=ex["N"], n_sink=wl.n_sink, n_recent=wl.n_recent, C=ex["C"], S=ex["S"],
                             perm=ex["perm"], sub_off=ex["sub_off"], cl_mu=ex["cl_mu"], cl_var=ex["cl_var"],
                             cl_vbar=ex["cl_vbar"], sub_mu=ex["sub_mu"], sub_var=ex["sub_var"],
                             sub_vbar=ex["sub_vbar"])
            K, V = b.unit_kv(s, h)
            Q = qs[t][s, h * G:(h + 1) * G].cpu().numpy().astype(np.float64)
            t0 = time.time()
            O.decode_unit(L, K, V, Q, wl.top_c[s], wl.top_s[s])
            times.append(time.time() - t0)
            units_done += 1
            qsets_used.add(t)
            del K, V
            if sum(times) > budget_s:
                break
        if sum(times) > budget_s:
            break
    per_unit = float(np.mean(times))
    step_s = per_unit * lay.n_units
    try:
        import threadpoolctl
        blas = [p.get("num_threads") for p in threadpoolctl.threadpool_info()]
        threads = max([t for t in blas if t] or [1])
    except Exception:  # pragma: no cover
        threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    return dict(value=1.0 / step_s, unit="steps/s", cores=threads, kind="oracle",
                sample=f"oracle.decode_unit on {units_done} (seq, KV head) unit decodes ({lay.n_units} per step) "
                       f"of '{wl.name}' over {len(qsets_used)} query set(s), GPU-built layout, "
                       f"{sum(times):.1f} s of CPU work, mean per unit scaled to one step; "
                       f"host cores available {len(os.sched_getaffinity(0))}")


PROFILE_1M = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                          "k_exact_gqa-40q8kv-d128-1M-bf16.md")
KERNEL_SOURCES = ["decode.hip", "attn_tile.h", "mog_internal.h"]


def kernel_sources_sha256():
    """Hash of the sources the exact kernel is compiled from."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "long_context_sparse_mog_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled_traffic():
    """HBM bytes per exact-kernel launch from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy), or None when
    the summary is missing or the kernel sources changed since it was taken."""
    try:
        with open(PROFILE_1M) as f:
            text = f.read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        line = line.strip().strip("`")
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip().lstrip("- ").strip("`")] = v.strip().strip("`")
    if fields.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(n_bytes=1 << 30, reps=10):
    """A plain copy of known size: each dispatch reads and writes n_bytes."""
    import torch

    a = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"copy_bytes_read": n_bytes, "copy_bytes_written": n_bytes, "ms": ms,
                      "GBps_read_plus_write": 2 * n_bytes / (ms * 1e-3) / 1e9}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--qsets", type=int, default=16)
    ap.add_argument("--no-128k", action="store_true", help="skip the N=128K workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the 4K, 32K and ragged workloads and the build timing")
    ap.add_argument("--no-shared", action="store_true",
                    help="skip the 1M step with one selection per KV head")
    ap.add_argument("--no-incremental", action="store_true",
                    help="skip the 1M incremental-decode steps (append one token + decode)")
    ap.add_argument("--no-offload", action="store_true",
                    help="skip the 1M step with the layout rows in pinned host memory")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 10 times (the reference kernel that "
                         "scales rocprofv3 FETCH_SIZE/WRITE_SIZE to bytes) and print its rate")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calib:
        copy_calibration()
        return
    from long_context_sparse_mog_amd import capi

    capi.lib()  # fail loudly when the HIP library is missing
    ev = HipEvents()
    r1m, st1m = bench_workload(3, args.steps, args.warmup, args.qsets, ev, shared_too=not args.no_shared)
    if not args.no_incremental:
        r1m["incremental"] = incremental_bench(st1m, args.steps, args.warmup)
    if not args.no_offload:
        off = offload_bench(st1m, 20, ev)
        # the exact kernel reads the same rows as in HBM, now over the host
        # link (the residual blocks' statistics stay in HBM)
        off["exact_kernel_GBps_host_link"] = r1m["exact_row_bytes"] / (off["exact_kernel_ms"] * 1e-3) / 1e9
        r1m["offload"] = off
    r128 = None
    if not args.no_128k:
        r128, _ = bench_workload(2, args.steps, args.warmup, args.qsets, ev)
    others = {}
    if not args.no_others:
        keep = ("replicas", "steps_per_s", "ms_per_step", "ms_p10", "ms_p50", "ms_p90", "graph_ms_per_step",
                "exact_kernel_ms", "exact_kernel_GBps", "step_bytes", "hbm_GBps", "frac_kv_read_per_head",
                "frac_kv_read_union", "dense_ms_per_step", "speedup_vs_dense", "err_vs_dense_residual_mean",
                "err_vs_dense_toponly_mean")
        for idx in (0, 1, 4):
            r, _ = bench_workload(idx, min(args.steps, 100), min(args.warmup, 10), args.qsets, ev)
            others[r["workload"]] = {k: r[k] for k in keep}
        others["build"] = build_timing()
        others["feature_map_residual"] = feature_residual_comparison(min(args.steps, 100), min(args.warmup, 10),
                                                                     args.qsets)
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(st1m, args.cpu_seconds)
    ev.close()
    ach = r1m["exact_kernel_GBps"]
    line = {
        "metric": METRIC,
        "value": r1m["steps_per_s"],
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r1m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian-mixture keys, N(0,1) values, planted queries)",
        "config": {"workload": r1m["workload"], "batch": r1m["n_seq"], "seq_len": 1048576,
                   "q_heads": r1m["n_q_heads"], "kv_heads": r1m["n_kv_heads"], "head_dim": r1m["head_dim"],
                   "top_c": r1m["top_c"], "top_s": r1m["top_s"]},
        "hbm_GBps": r1m["hbm_GBps"],
        "roofline": {"bound": "hbm", "kernel": "k_exact only (exact split-K attention, MFMA bf16, then the "
                                                "residual blocks of the clusters left out; the dominant kernel, "
                                                "timed by its own dispatch events over single launches)",
                     "achieved": ach, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS,
                     "traffic": profiled_traffic()},
        "step_roofline": {"bound": "hbm", "what": "the whole decode step: algorithmic step bytes / ms_per_step",
                          "bytes": r1m["step_bytes"], "achieved": r1m["hbm_GBps"], "peak": HBM_PEAK_GBPS,
                          "unit": "GB/s", "frac": r1m["hbm_GBps"] / HBM_PEAK_GBPS},
        "cpu_baseline": cpu,
        "at_1m": r1m,
        "at_128k": r128,
        "other_workloads": others or None,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
