"""GPU parity of the feature-map residual (residual = 2) against the CPU
oracle.

* Summaries: the library builds the layout with a seeded projection W; the
  layout is downloaded and the oracle recomputes every group's feature sum
  from the same members, keys and W (float64): within 1e-4 relative (the
  library sums float32 exponentials).
* Decode: on a layout built by the oracle (summaries included) and imported,
  selections must agree except at near ties and outputs are within 2e-3
  (bf16 K/V) or 1e-5 (float32 K/V) per-head relative L2 of the oracle's
  decode with the feature-map residual.
* Incremental decode: folded tokens add their features to both groups' sums
  (within 1e-4 relative of the oracle's fold), then one decode step.
"""

import sys
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle as O
from long_context_sparse_mog_amd import capi, ops, synth
from parity import build_oracle_layouts, compare_unit, oracle_layout_from_export, unit_layout_arrays

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_summaries(ex, K, wl, W, scale=None):
    L = oracle_layout_from_export(ex, wl.n_sink, wl.n_recent)
    R = O.with_feature_summaries(L, K, W, scale=scale)
    for name in ("cl_z", "sub_z"):
        got, ref = ex[name].astype(np.float64), getattr(R, name).astype(np.float64)
        tol = 1e-4 * np.maximum(np.abs(ref), 1e-30 + 1e-6 * np.abs(ref).max())
        assert (np.abs(got - ref) <= tol).all(), (name, float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30))))


def run_fm_build_case(wl, m=128, units=None):
    say(f"[fm build] {wl.name} lens={wl.seq_lens} D={wl.head_dim} {wl.dtype} m={m}")
    b = synth.generate(wl, device="cuda")
    kv = ops.KVCache.from_batch(b)
    W = synth.feature_map_w(m, wl.head_dim, device="cuda")
    lay = ops.mog_build(kv, wl.n_sink, wl.n_recent, kmeans_iters=wl.kmeans_iters, seed=5, fm_w=W)
    torch.cuda.synchronize()
    Wn = W.cpu().numpy()
    for u in units if units is not None else range(lay.n_units):
        s, h = divmod(u, wl.n_kv_heads)
        ex = lay.export_unit(u)
        assert np.array_equal(ex["fm_w"], Wn)
        K, _ = b.unit_kv(s, h)
        check_summaries(ex, K, wl, Wn)
    return b, kv, lay


def run_fm_decode_case(wl, m=128, shared=False, top=None, sel=True):
    # sel: True asks for the chosen clusters and subclusters (the subcluster
    # kernel runs), "c" for the clusters only (a whole-cluster budget then
    # skips it: the exact kernel's residual blocks take the feature-map
    # residual)
    tc = list(top[0]) if top else list(wl.top_c)
    ts = list(top[1]) if top else list(wl.top_s)
    say(f"[fm decode] {wl.name} lens={wl.seq_lens} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} D={wl.head_dim} "
        f"{wl.dtype} m={m} c={tc} s={ts} shared={shared} sel={sel}")
    b = synth.generate(wl, device="cuda")
    kv = ops.KVCache.from_batch(b)
    W = synth.feature_map_w(m, wl.head_dim).numpy()
    lays = build_oracle_layouts(b)
    for u in lays:
        s, h = divmod(u, wl.n_kv_heads)
        K, _ = b.unit_kv(s, h)
        lays[u] = O.with_feature_summaries(lays[u], K, W)
    lay = ops.import_layout(kv, wl.n_sink, wl.n_recent, [unit_layout_arrays(lays[u]) for u in range(len(lays))])
    params = ops.decode_params(wl.n_q_heads, tc, ts, residual="fm", shared=shared)
    q = b.Q[0].contiguous()
    out, lse, sel_c, sel_s = ops.mog_decode(lay, kv, q, params, want_sel=sel)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    sel_c = sel_c.cpu().numpy()
    sel_s = sel_s.cpu().numpy() if sel_s is not None else None
    tol = 1e-5 if wl.dtype == "fp32" else 2e-3
    G = wl.group
    worst = 0.0
    for u in sorted(lays):
        s, h = divmod(u, wl.n_kv_heads)
        K, V = b.unit_kv(s, h)
        Q = q[s, h * G:(h + 1) * G].cpu().numpy().astype(np.float64)
        hs = slice(h * G, (h + 1) * G)
        r = compare_unit(lays[u], K, V, Q, tc[s], ts[s], out[s, hs], lse[s, hs], sel_c[s, hs],
                         None if sel_s is None else sel_s[s, hs], tol, residual="fm", shared=shared)
        assert r["lse_err"] < (1e-5 if wl.dtype == "fp32" else 1e-3) * max(1.0, float(np.abs(lse[s, hs]).max()))
        worst = max(worst, r["max_rel"])
    say(f"  worst per-head rel L2 = {worst:.3e}")
    return out


def test_fm_summaries_config0_m64():
    run_fm_build_case(synth.config(0), m=64)


def test_fm_summaries_gqa_bf16_m128():
    run_fm_build_case(synth.config(1, seq_lens=[8192], n_components=64))


def test_fm_summaries_ragged_paged_m256():
    wl = synth.config(4, seq_lens=[3000, 9000, 5000])
    run_fm_build_case(wl, m=256, units=[0, 5, 12, 23])


def test_fm_decode_config0():
    run_fm_decode_case(synth.config(0), m=64)


def test_fm_decode_gqa_bf16():
    run_fm_decode_case(synth.config(1, seq_lens=[8192], n_components=64))


def test_fm_decode_ragged_paged_high_entropy_heads():
    # KV heads 4-7 hold isotropic keys (near-uniform attention)
    run_fm_decode_case(synth.config(4, seq_lens=[4000, 7000]), m=128)


def test_fm_decode_shared_selection_g5():
    run_fm_decode_case(synth.config(3, seq_lens=[6000], n_components=64), shared=True)


def test_fm_decode_no_clusters_chosen():
    # every middle token estimated from the feature sums
    wl = synth.config(0, seq_lens=[3000])
    run_fm_decode_case(wl, m=256, top=([0], [0]))


# whole-cluster budgets (top_s >= S) without the subcluster output: no
# subcluster kernel runs and the exact kernel's residual blocks estimate the
# clusters left out from their feature sums
@pytest.mark.parametrize("name", ["gqa", "ragged-paged", "fp32-g8", "d64-g1"])
def test_fm_decode_whole_cluster(name):
    wl = {
        "gqa": lambda: synth.config(1, seq_lens=[8192], n_kv_heads=2, n_q_heads=8, n_components=64, top_c=[6],
                                    top_s=[13]),
        "ragged-paged": lambda: synth.config(4, seq_lens=[3000, 9000, 1000], n_kv_heads=2, n_q_heads=8,
                                             high_entropy_heads=(1,), n_components=64, top_c=[3, 5, 2],
                                             top_s=[12, 14, 10]),
        "fp32-g8": lambda: synth.config(1, seq_lens=[5000], n_kv_heads=1, n_q_heads=8, n_components=32,
                                        dtype="fp32"),
        "d64-g1": lambda: synth.config(1, seq_lens=[4000], n_kv_heads=2, n_q_heads=2, head_dim=64, n_components=32),
    }[name]()
    run_fm_decode_case(wl, m=128 if name != "ragged-paged" else 256, sel="c")


def test_fm_decode_whole_cluster_edges():
    # no cluster chosen (every middle token estimated), shared selection, and
    # more clusters than one residual block holds (C = 300)
    run_fm_decode_case(synth.config(0, seq_lens=[3000]), m=64, top=([0], [12]), sel="c")
    run_fm_decode_case(synth.config(3, seq_lens=[6000], n_components=64), shared=True, sel="c")
    wl = synth.config(1, seq_lens=[20000], n_kv_heads=1, n_q_heads=4, n_components=300, top_c=[40], top_s=[16])
    run_fm_decode_case(wl, m=128, sel="c")


def test_fm_whole_and_subcluster_paths_agree():
    """On one built layout with feature summaries, the whole-cluster step and
    the subcluster path read the same exact tiles in the same order and sum
    the same feature-map residual terms in another order."""
    wl = synth.config(4, seq_lens=[3000, 9000, 1000], n_kv_heads=2, n_q_heads=8, high_entropy_heads=(1,),
                      n_components=64, top_c=[3, 5, 2], top_s=[12, 14, 10])
    say(f"[fm paths] {wl.name} lens={wl.seq_lens}")
    b = synth.generate(wl, device="cuda")
    kv = ops.KVCache.from_batch(b)
    W = synth.feature_map_w(128, wl.head_dim, device="cuda")
    lay = ops.mog_build(kv, wl.n_sink, wl.n_recent, kmeans_iters=wl.kmeans_iters, seed=1, fm_w=W)
    params = ops.decode_params(wl.n_q_heads, list(wl.top_c), list(wl.top_s), residual="fm")
    q = b.Q[0].contiguous()
    ow, lw, cw, _ = ops.mog_decode(lay, kv, q, params, want_sel="c")
    os_, ls_, cs, _ = ops.mog_decode(lay, kv, q, params, want_sel=True)
    torch.cuda.synchronize()
    assert torch.equal(cw, cs)
    d = ((ow - os_).norm(dim=-1) / os_.norm(dim=-1)).max().item()
    say(f"  max per-head rel difference {d:.2e}, lse {(lw - ls_).abs().max().item():.2e}")
    assert d < 1e-5
    assert torch.allclose(lw, ls_, rtol=0, atol=1e-5 * max(1.0, ls_.abs().max().item()))


@pytest.mark.parametrize("hq,budget", [(8, None), (2, ([4], [3]))])
def test_fm_incremental(hq, budget):
    # (2, c = 4, s = 3): one query head per KV head and some subclusters of
    # each chosen cluster, so the fused top-c and subcluster kernel weights
    # left-out subclusters, folded rows among them, from their feature sums
    from test_gpu_append import run_append_case  # noqa: F401 (fold checks without summaries)
    extra = {} if budget is None else dict(top_c=budget[0], top_s=budget[1])
    wl = synth.config(1, seq_lens=[6000], n_kv_heads=2, n_q_heads=hq, n_components=32, **extra)
    grow, m = 120, 128
    wg = replace(wl, seq_lens=[6000 + grow])
    b = synth.generate(wg, device="cuda")
    kv = ops.KVCache.from_batch(b)
    W = synth.feature_map_w(m, wl.head_dim, device="cuda")
    Wn = W.cpu().numpy()
    lay = ops.mog_build(kv.with_lens([6000]), wl.n_sink, wl.n_recent, fold_capacity=grow, fm_w=W)
    ex0 = [lay.export_unit(u) for u in range(2)]
    ops.mog_append(lay, kv.with_lens([6001]))
    ops.mog_append(lay, kv)
    torch.cuda.synchronize()
    params = ops.decode_params(wl.n_q_heads, wl.top_c, wl.top_s, residual="fm")
    q = b.Q[0].contiguous()
    out, lse, sel_c, sel_s = ops.mog_decode(lay, kv, q, params, want_sel=True)
    torch.cuda.synchronize()
    out, lse, sel_c, sel_s = out.cpu().numpy(), lse.cpu().numpy(), sel_c.cpu().numpy(), sel_s.cpu().numpy()
    G = wl.group
    for u in range(2):
        K, V = b.unit_kv(0, u)
        F = O.fold_tokens(oracle_layout_from_export(ex0[u], wl.n_sink, wl.n_recent), K, V, grow)
        ex = lay.export_unit(u)
        assert [int(x) for x in ex["fold_sub"]] == F.fold_sub
        for name in ("cl_z", "sub_z"):
            got, ref = ex[name].astype(np.float64), getattr(F, name).astype(np.float64)
            assert np.allclose(got, ref, rtol=1e-4, atol=1e-6 * np.abs(ref).max()), name
        # and they equal the sums recomputed over the grown groups
        check_summaries(ex, K, wl, Wn)
        Q = q[0, u * G:(u + 1) * G].cpu().numpy().astype(np.float64)
        hs = slice(u * G, (u + 1) * G)
        compare_unit(F, K, V, Q, wl.top_c[0], wl.top_s[0], out[0, hs], lse[0, hs], sel_c[0, hs], sel_s[0, hs], 2e-3,
                     residual="fm")
