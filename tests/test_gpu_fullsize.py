"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (automatic block count), on sampled units.

The library builds the layout (its k-means is tested separately); the
layout is downloaded and handed to the oracle, which decodes the sampled
(sequence, KV head) units from it.  Selections must agree except at near
ties and outputs must be within 2e-3 per-head relative L2 (bf16 K/V).
"""

import sys
from dataclasses import replace

import numpy as np
import pytest
import torch

from long_context_sparse_mog_amd import ops, synth
from parity import compare_unit, oracle_layout_from_export

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_fullsize(wl, units, qset=0, shared=False, check_build=(), sels=None):
    """``check_build``: units whose built layout is also checked (a valid
    partition in (cluster, subcluster, position) order, and every statistic
    equal to the oracle's statistic of that partition).  ``sels``: the
    selection outputs asked for, one decode each on the same layout: "c"
    (the chosen clusters; with a whole-cluster budget this is the path the
    benchmark times, no subcluster kernel) or True (clusters and
    subclusters: the subcluster kernel always runs).  Default: "c" for a
    whole-cluster budget, else True."""
    say(f"[full] {wl.name} n_seq={wl.n_seq} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} "
        f"max_len={wl.max_len} units={units} build-checked={list(check_build)} sels={sels}")
    b = synth.generate(wl, device="cuda", n_qsets=qset + 1)
    kv = ops.KVCache.from_batch(b)
    lay = ops.mog_build(kv, wl.n_sink, wl.n_recent, kmeans_iters=wl.kmeans_iters, seed=1)
    params = ops.decode_params(wl.n_q_heads, list(wl.top_c), list(wl.top_s), shared=shared)
    if sels is None:
        whole = all(wl.top_s[s] >= lay.unit(s * wl.n_kv_heads).S for s in range(wl.n_seq))
        sels = ("c",) if whole else (True,)
    q = b.Q[qset].contiguous()
    runs = []
    for sel in sels:
        out, lse, sel_c, sel_s = ops.mog_decode(lay, kv, q, params, want_sel=sel)
        torch.cuda.synchronize()
        runs.append((sel, out.cpu().numpy(), lse.cpu().numpy(), sel_c.cpu().numpy(),
                     None if sel_s is None else sel_s.cpu().numpy()))
    G = wl.group
    for u in units:
        s, h = divmod(u, wl.n_kv_heads)
        ex = lay.export_unit(u)
        L = oracle_layout_from_export(ex, wl.n_sink, wl.n_recent)
        K, V = b.unit_kv(s, h)
        if u in check_build:
            from test_gpu_build import check_built_unit
            check_built_unit(ex, K, V, wl)
            say(f"  unit {u}: built layout and statistics match the oracle's for its partition")
        Q = q[s, h * G:(h + 1) * G].cpu().numpy().astype(np.float64)
        hs = slice(h * G, (h + 1) * G)
        for sel, out, lse, sel_c, sel_s in runs:
            r = compare_unit(L, K, V, Q, wl.top_c[s], wl.top_s[s], out[s, hs], lse[s, hs], sel_c[s, hs],
                             None if sel_s is None else sel_s[s, hs], 2e-3, shared=shared)
            assert r["lse_err"] < 1e-3 * max(1.0, float(np.abs(lse[s, hs]).max()))
            say(f"  unit {u} (seq {s}, len {wl.seq_lens[s]}, kv head {h}, sel {sel}): worst rel L2 "
                f"{r['max_rel']:.2e}, near ties {r['ties']}")
        del K, V
    del b, kv, lay
    torch.cuda.empty_cache()


def test_fullsize_gqa_32k_all_units():
    run_fullsize(synth.config(1), list(range(8)))


def test_fullsize_gqa_1m_shared_selection_sampled():
    run_fullsize(synth.config(3), [2, 5], qset=1, shared=True, sels=(True,))


def test_fullsize_mha_128k_sampled():
    run_fullsize(synth.config(2), [0, 45, 127], check_build=(45,))


def test_fullsize_one_head_many_clusters():
    """One query head per KV head and more than 512 clusters (N = 600K, C =
    775, s = 2): top-c and the subclusters in one launch, with 16 cluster
    slots per lane."""
    wl = synth.config(2, n_q_heads=2, n_kv_heads=2, seq_lens=[600000], name="mha-2h-d128-600K-bf16")
    assert wl.top_s[0] < 20
    run_fullsize(wl, [0, 1])


def test_fullsize_gqa_1m_sampled():
    run_fullsize(synth.config(3), [0, 3, 7], check_build=(3,))


def test_fullsize_dense_1m_sampled():
    """mog_dense_decode over the whole 1M-token cache, in the launch
    configuration the benchmark times (automatic split count), against the
    oracle's dense attention on two KV heads (all 5 query heads of each)."""
    import oracle as O
    wl = synth.config(3)
    say(f"[full dense] {wl.name}")
    b = synth.generate(wl, device="cuda")
    kv = ops.KVCache.from_batch(b)
    q = b.Q[0].contiguous()
    out, lse = ops.mog_dense_decode(kv, q, ops.decode_params(wl.n_q_heads, 1, 1))
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    G = wl.group
    for h in (1, 6):
        K, V = b.unit_kv(0, h)
        Q = q[0, h * G:(h + 1) * G].cpu().numpy().astype(np.float64)
        ref_o, ref_l = O.dense_attention(K, V, Q)
        errs = [float(np.linalg.norm(out[0, h * G + g] - ref_o[g]) / np.linalg.norm(ref_o[g])) for g in range(G)]
        lerr = float(np.max(np.abs(lse[0, h * G:(h + 1) * G] - ref_l)))
        say(f"  kv head {h}: worst rel L2 {max(errs):.2e}, lse err {lerr:.2e}")
        assert max(errs) <= 2e-3
        assert lerr <= 1e-3 * max(1.0, float(np.abs(ref_l).max()))
        del K, V
    del b, kv
    torch.cuda.empty_cache()


def test_fullsize_ragged_paged_sampled():
    wl = synth.config(4)
    longest = int(np.argmax(wl.seq_lens))
    shortest = int(np.argmin(wl.seq_lens))
    # a mixture head of the longest sequence, a high-entropy head of the
    # shortest one, and a high-entropy head of the longest one
    run_fullsize(wl, [longest * 8 + 1, shortest * 8 + 6, longest * 8 + 7])


def test_maximum_length_single_head():
    """N = 2^22 (the longest sequence the library takes): C = 2048 clusters
    of S = 22 subclusters, the largest partition the kernels size for."""
    L = 1 << 22
    wl = synth.config(3, n_q_heads=4, n_kv_heads=1, seq_lens=[L], n_components=2048,
                      name="gqa-4q1kv-d128-4M-bf16", budget_kappa=34 / 203)
    run_fullsize(wl, [0], sels=("c", True))


def test_fullsize_gqa_1m_incremental_sampled():
    """The 1M workload's cache, the layout built on its first N - 300 tokens,
    then 300 tokens appended (one, one, then 298 at once); fold state and one
    decode step checked on two units."""
    from test_gpu_append import run_append_case
    wl = synth.config(3)
    grow = 300
    wb = replace(wl, seq_lens=[wl.seq_lens[0] - grow])
    run_append_case(wb, [grow], chunks=[[1], [1], [grow - 2]], units=[0, 5], grown_wl=wl)
    torch.cuda.empty_cache()


def test_fullsize_gqa_1m_feature_residual_sampled():
    """The 1M workload built with feature-map summaries (m = 128): summaries
    of two units against the oracle's sums over the same members, and one
    decode step with the feature-map residual on them, on both paths: the
    subcluster kernel (subcluster output asked for) and the whole-cluster
    step the benchmark times (clusters only: the exact launch's residual
    blocks estimate the clusters left out)."""
    from test_gpu_fm import check_summaries
    wl = synth.config(3)
    say(f"[full fm] {wl.name}")
    b = synth.generate(wl, device="cuda")
    kv = ops.KVCache.from_batch(b)
    W = synth.feature_map_w(128, wl.head_dim, device="cuda")
    lay = ops.mog_build(kv, wl.n_sink, wl.n_recent, kmeans_iters=wl.kmeans_iters, seed=1, fm_w=W)
    params = ops.decode_params(wl.n_q_heads, list(wl.top_c), list(wl.top_s), residual="fm")
    q = b.Q[0].contiguous()
    runs = []
    for sel in (True, "c"):
        out, lse, sel_c, sel_s = ops.mog_decode(lay, kv, q, params, want_sel=sel)
        torch.cuda.synchronize()
        runs.append((sel, out.cpu().numpy(), lse.cpu().numpy(), sel_c.cpu().numpy(),
                     None if sel_s is None else sel_s.cpu().numpy()))
    G = wl.group
    for u in (1, 6):
        ex = lay.export_unit(u)
        K, V = b.unit_kv(0, u)
        check_summaries(ex, K, wl, W.cpu().numpy())
        L = oracle_layout_from_export(ex, wl.n_sink, wl.n_recent)
        Q = q[0, u * G:(u + 1) * G].cpu().numpy().astype(np.float64)
        hs = slice(u * G, (u + 1) * G)
        for sel, out, lse, sel_c, sel_s in runs:
            r = compare_unit(L, K, V, Q, wl.top_c[0], wl.top_s[0], out[0, hs], lse[0, hs], sel_c[0, hs],
                             None if sel_s is None else sel_s[0, hs], 2e-3, residual="fm")
            say(f"  unit {u} (sel {sel}): worst rel L2 {r['max_rel']:.2e}, near ties {r['ties']}")
        del K, V
    del b, kv, lay
    torch.cuda.empty_cache()


def test_fullsize_gqa_1m_offloaded_rows():
    """The 1M workload with the layout's rows in pinned host memory: the
    decode step is bit-identical to the HBM-resident one (same kernels, rows
    read over the host link)."""
    wl = synth.config(3)
    say(f"[full offload] {wl.name}")
    b = synth.generate(wl, device="cuda")
    kv = ops.KVCache.from_batch(b)
    dev = ops.mog_build(kv, wl.n_sink, wl.n_recent, kmeans_iters=wl.kmeans_iters, seed=1)
    host = ops.mog_build(kv, wl.n_sink, wl.n_recent, kmeans_iters=wl.kmeans_iters, seed=1, rows_host=True)
    params = ops.decode_params(wl.n_q_heads, list(wl.top_c), list(wl.top_s))
    q = b.Q[0].contiguous()
    a = ops.mog_decode(dev, kv, q, params, want_sel=True)
    h = ops.mog_decode(host, kv, q, params, want_sel=True)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, h))
    del b, kv, dev, host
    torch.cuda.empty_cache()


def test_maximum_length_incremental():
    """N = 2^22 - 64 built, then 64 tokens appended in two calls: C = 2048
    clusters, so the append's cluster scan is spread over its largest block
    count (16 per unit); fold state and a decode step against the oracle."""
    from test_gpu_append import run_append_case
    L = 1 << 22
    wl = synth.config(3, n_q_heads=4, n_kv_heads=1, seq_lens=[L], n_components=2048,
                      name="gqa-4q1kv-d128-4M-bf16", budget_kappa=34 / 203)
    wb = replace(wl, seq_lens=[L - 64])
    run_append_case(wb, [64], chunks=[[1], [63]], grown_wl=wl)
    torch.cuda.empty_cache()
