"""GPU parity of mog_decode and mog_dense_decode against the CPU oracle.

mog_decode runs on a layout built by the oracle and imported into the
library, so both sides see the same partition; selections must agree except
at near ties, outputs within the stated tolerance (per-head relative L2:
1e-5 for float32 K/V, 2e-3 for bf16 K/V).
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle as O
from long_context_sparse_mog_amd import ops, synth
from parity import build_oracle_layouts, compare_unit, rel_l2, unit_layout_arrays

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def tol_of(wl):
    return 1e-5 if wl.dtype == "fp32" else 2e-3


def run_decode_case(wl, residual=True, top_c=None, top_s=None, qset=0, n_qsets=1, splits=0, shared=False,
                    sel=True, zero_q=False):
    # sel: True asks for the chosen clusters and subclusters (the subcluster
    # kernel runs), "c" for the clusters only (a whole-cluster budget then
    # skips it)
    say(f"[case] {wl.name} lens={wl.seq_lens} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} "
        f"D={wl.head_dim} {wl.dtype} c={top_c or wl.top_c} s={top_s or wl.top_s} res={residual} shared={shared} "
        f"sel={sel}")
    b = synth.generate(wl, device="cuda", n_qsets=n_qsets)
    kv = ops.KVCache.from_batch(b)
    lays = build_oracle_layouts(b)
    lay = ops.import_layout(kv, wl.n_sink, wl.n_recent,
                            [unit_layout_arrays(lays[u]) for u in range(wl.n_seq * wl.n_kv_heads)])
    tc = top_c if top_c is not None else wl.top_c
    ts = top_s if top_s is not None else wl.top_s
    params = ops.decode_params(wl.n_q_heads, list(tc), list(ts), residual=residual, splits=splits, shared=shared)
    q = b.Q[qset].contiguous()
    if zero_q:
        q.zero_()
    out, lse, sel_c, sel_s = ops.mog_decode(lay, kv, q, params, want_sel=sel)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    sel_c = sel_c.cpu().numpy()
    sel_s = sel_s.cpu().numpy() if sel_s is not None else None
    G = wl.group
    worst = 0.0
    for s in range(wl.n_seq):
        for h in range(wl.n_kv_heads):
            u = s * wl.n_kv_heads + h
            K, V = b.unit_kv(s, h)
            Q = q[s, h * G:(h + 1) * G].cpu().numpy().astype(np.float64)
            hs = slice(h * G, (h + 1) * G)
            r = compare_unit(lays[u], K, V, Q, tc[s], ts[s], out[s, hs], lse[s, hs], sel_c[s, hs],
                             None if sel_s is None else sel_s[s, hs], tol_of(wl), residual=residual,
                             shared=shared)
            assert r["lse_err"] < (1e-5 if wl.dtype == "fp32" else 1e-3) * max(1.0, float(np.abs(lse[s, hs]).max()))
            worst = max(worst, r["max_rel"])
    say(f"  worst per-head rel L2 = {worst:.3e}")
    return b, kv, lays, out


def test_config0_full():
    run_decode_case(synth.config(0))


def test_config0_top_only():
    run_decode_case(synth.config(0), residual=False)


def test_config0_all_clusters_is_dense():
    wl = synth.config(0)
    b, kv, lays, out = run_decode_case(wl, top_c=[64], top_s=[12])
    K, V = b.unit_kv(0, 0)
    o, _ = O.dense_attention(K, V, b.Q[0, 0].cpu().numpy())
    assert rel_l2(out[0], o) < 1e-5


def test_config0_no_clusters():
    run_decode_case(synth.config(0), top_c=[0], top_s=[3])


def test_config1_gqa_reduced():
    run_decode_case(synth.config(1, seq_lens=[8192], n_kv_heads=2, n_q_heads=8, n_components=64))


def test_config2_mha_needles_reduced():
    run_decode_case(synth.config(2, seq_lens=[6000, 6000], n_kv_heads=2, n_q_heads=2,
                                 n_components=64))


def test_config3_gqa5_reduced():
    run_decode_case(synth.config(3, seq_lens=[12000], n_kv_heads=2, n_q_heads=10, n_components=128))


def test_config4_ragged_paged_reduced():
    run_decode_case(synth.config(4, seq_lens=[3000, 9000, 1000], n_kv_heads=2, n_q_heads=8,
                                 high_entropy_heads=(1,), n_components=64))


@pytest.mark.parametrize("G", [2, 3, 6, 7, 8])
def test_other_group_sizes(G):
    # the score kernels' reduce-scatter takes 4G and 6G values per wave:
    # from 8 up to 48, padded to a power of two, over five or six exchanges
    run_decode_case(synth.config(1, seq_lens=[3000], n_kv_heads=1, n_q_heads=G, n_components=32))


def test_fp32_d128_and_splits():
    wl = synth.config(1, seq_lens=[5000], n_kv_heads=1, n_q_heads=4, n_components=32, dtype="fp32")
    run_decode_case(wl, splits=1)
    run_decode_case(wl, splits=37)


def test_bf16_d64():
    run_decode_case(synth.config(1, seq_lens=[4000], n_kv_heads=2, n_q_heads=4, head_dim=64,
                                 n_components=32))


@pytest.mark.parametrize("lens", [[3000] * 5, [2000, 2600, 3100, 1500, 2900]])
def test_many_units_half_block_shares(lens):
    # more than 16 units: the exact blocks take unit shares per half block
    # (the last block's second half is idle when the share count is odd)
    wl = synth.config(1, seq_lens=lens, n_kv_heads=4, n_q_heads=8, n_components=32)
    run_decode_case(wl)
    run_decode_case(wl, sel="c")


def test_more_than_256_units():
    # 272 units: the exact shares take the fixed scale (the units' row counts
    # are read 64 at a time instead of held in registers), per half block;
    # one query head per KV head, with and without the subcluster output
    wl = synth.config(1, seq_lens=[1000 + 37 * i for i in range(34)], n_kv_heads=8, n_q_heads=8,
                      n_components=16)
    run_decode_case(wl, top_c=[2] * 34, top_s=[3] * 34)
    run_decode_case(wl, sel="c")


@pytest.mark.parametrize("residual", [True, False])
def test_subcluster_budgets_mixed(residual):
    # per-sequence subcluster budgets below S, zero and above S in one batch;
    # checked against the oracle with the selection outputs, and the same
    # step without them must give the same bits
    wl = synth.config(4, seq_lens=[3000, 9000, 1000], n_kv_heads=2, n_q_heads=8, high_entropy_heads=(1,),
                      n_components=64)
    tc, ts = [6, 4, 3], [2, 0, 40]
    b, kv, lays, out = run_decode_case(wl, residual=residual, top_c=tc, top_s=ts)
    lay = ops.import_layout(kv, wl.n_sink, wl.n_recent,
                            [unit_layout_arrays(lays[u]) for u in range(wl.n_seq * wl.n_kv_heads)])
    params = ops.decode_params(wl.n_q_heads, tc, ts, residual=residual)
    q = b.Q[0].contiguous()
    o1, l1, _, _ = ops.mog_decode(lay, kv, q, params, want_sel=True)
    o2, l2, _, _ = ops.mog_decode(lay, kv, q, params, want_sel=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert np.array_equal(o1.cpu().numpy(), out)


@pytest.mark.parametrize("ns,nr,L", [(0, 16, 700), (16, 0, 700), (0, 0, 500), (2, 3, 6), (4, 4, 9)])
def test_anchor_edges(ns, nr, L):
    wl = synth.config(1, seq_lens=[L], n_kv_heads=1, n_q_heads=2, n_components=8, n_sink=ns,
                      n_recent=nr, top_c=[2], top_s=[2])
    run_decode_case(wl)


def test_budget_larger_than_partition():
    wl = synth.config(1, seq_lens=[1500], n_kv_heads=1, n_q_heads=2, n_components=16,
                      top_c=[500], top_s=[100])
    b, kv, lays, out = run_decode_case(wl)
    K, V = b.unit_kv(0, 0)
    o, _ = O.dense_attention(K, V, b.Q[0, 0].cpu().numpy())
    assert rel_l2(out[0], o) < 2e-3


@pytest.mark.parametrize("hq", [2, 1])
@pytest.mark.parametrize("c", [3, 17, 40, 64, 65, 120])
def test_exact_ties_go_to_lower_index(c, hq):
    """A zero query makes every group's score its log count, so groups of
    equal size tie exactly in any precision: the chosen clusters and
    subclusters must be exactly the oracle's (ties to the lower index), for
    budgets from a few clusters to most of them."""
    # (hq = 1: one query head per KV head, top-c inside the subcluster launch)
    wl = synth.config(1, seq_lens=[20000], n_kv_heads=1, n_q_heads=hq, n_components=64, top_c=[c],
                      top_s=[3])
    say(f"[case] zero query, {wl.seq_lens} keys, c={c}, G={hq}")
    b = synth.generate(wl, device="cuda", n_qsets=1)
    kv = ops.KVCache.from_batch(b)
    lays = build_oracle_layouts(b)
    lay = ops.import_layout(kv, wl.n_sink, wl.n_recent, [unit_layout_arrays(lays[0])])
    params = ops.decode_params(wl.n_q_heads, [c], [3])
    q = torch.zeros_like(b.Q[0]).contiguous()
    out, lse, sel_c, sel_s = ops.mog_decode(lay, kv, q, params, want_sel=True)
    torch.cuda.synchronize()
    sel_c, sel_s = sel_c.cpu().numpy(), sel_s.cpu().numpy()
    K, V = b.unit_kv(0, 0)
    G, D = wl.group, wl.head_dim
    counts = lays[0].cl_count
    assert len(set(counts[counts > 0].tolist())) < int((counts > 0).sum()), "no equal-size clusters"
    ref = O.decode_unit(lays[0], K, V, np.zeros((G, D)), c, 3, scale=1.0 / math.sqrt(D))
    for h in range(G):
        gc = [int(x) for x in sel_c[0, h] if x >= 0]
        assert gc == [int(x) for x in ref["sel_c"][h]], (h, gc, ref["sel_c"][h])
        for r in range(len(gc)):
            gs = [int(x) for x in sel_s[0, h, r] if x >= 0]
            assert gs == [int(x) for x in ref["sel_s"][h][r]], (h, r, gs, ref["sel_s"][h][r])
    o, _ = O.dense_attention(K, V, np.zeros((G, D)))
    say(f"  {len(gc)} clusters chosen; rel L2 vs dense {rel_l2(out[0].cpu().numpy(), o):.2e}")


# ---------------------------------------------------------------------------
# whole-cluster budgets (top_s >= S) without the subcluster output: the top-c
# kernel lists the chosen clusters' tiles, the residual of the clusters left
# out runs in blocks after the exact ones, and no subcluster kernel runs
# ---------------------------------------------------------------------------
WHOLE = {
    "cfg1r": lambda: synth.config(1, seq_lens=[8192], n_kv_heads=2, n_q_heads=8, n_components=64),
    "cfg3r": lambda: synth.config(3, seq_lens=[12000], n_kv_heads=2, n_q_heads=10, n_components=128),
    "cfg4r-paged": lambda: synth.config(4, seq_lens=[3000, 9000, 1000], n_kv_heads=2, n_q_heads=8,
                                        high_entropy_heads=(1,), n_components=64),
    "fp32": lambda: synth.config(1, seq_lens=[5000], n_kv_heads=1, n_q_heads=4, n_components=32, dtype="fp32"),
    "d64": lambda: synth.config(1, seq_lens=[4000], n_kv_heads=2, n_q_heads=4, head_dim=64, n_components=32),
}


@pytest.mark.parametrize("name", list(WHOLE))
def test_whole_cluster_path(name):
    wl = WHOLE[name]()
    assert all(s >= math.ceil(math.log2(L)) for s, L in zip(wl.top_s, wl.seq_lens))
    run_decode_case(wl, sel="c")


@pytest.mark.parametrize("G", [1, 2, 3, 6, 7, 8])
def test_whole_cluster_group_sizes(G):
    run_decode_case(synth.config(1, seq_lens=[3000], n_kv_heads=1, n_q_heads=G, n_components=32), sel="c")


def test_whole_cluster_top_only_and_shared():
    run_decode_case(WHOLE["cfg1r"](), residual=False, sel="c")
    run_decode_case(WHOLE["cfg3r"](), shared=True, sel="c")


def test_whole_cluster_splits():
    run_decode_case(WHOLE["fp32"](), splits=1, sel="c")
    run_decode_case(WHOLE["fp32"](), splits=37, sel="c")


def test_whole_cluster_edges():
    # no cluster chosen (only anchors and the residual), and a budget above
    # the partition (every cluster whole: dense attention)
    run_decode_case(synth.config(0), top_c=[0], top_s=[12], sel="c")
    wl = synth.config(1, seq_lens=[1500], n_kv_heads=1, n_q_heads=2, n_components=16, top_c=[500], top_s=[100])
    b, kv, lays, out = run_decode_case(wl, sel="c")
    K, V = b.unit_kv(0, 0)
    o, _ = O.dense_attention(K, V, b.Q[0, 0].cpu().numpy())
    assert rel_l2(out[0], o) < 2e-3


def test_whole_cluster_zero_query_ties():
    # every score is a log count: equal-size clusters tie exactly
    wl = synth.config(1, seq_lens=[20000], n_kv_heads=1, n_q_heads=2, n_components=64, top_c=[40], top_s=[15])
    run_decode_case(wl, sel="c", zero_q=True)


@pytest.mark.parametrize("name", ["cfg3r", "cfg4r-paged"])
def test_whole_and_subcluster_paths_agree(name):
    """The two paths list the same exact tiles in the same order (bit-equal
    exact records) and sum the same residual terms in another order."""
    wl = WHOLE[name]()
    b = synth.generate(wl, device="cuda")
    kv = ops.KVCache.from_batch(b)
    lay = ops.mog_build(kv, wl.n_sink, wl.n_recent, kmeans_iters=wl.kmeans_iters, seed=1)
    params = ops.decode_params(wl.n_q_heads, list(wl.top_c), list(wl.top_s))
    q = b.Q[0].contiguous()
    ow, lw, cw, _ = ops.mog_decode(lay, kv, q, params, want_sel="c")
    os_, ls_, cs, ss = ops.mog_decode(lay, kv, q, params, want_sel=True)
    torch.cuda.synchronize()
    assert torch.equal(cw, cs)
    d = ((ow - os_).norm(dim=-1) / os_.norm(dim=-1)).max().item()
    say(f"[paths] {name}: max per-head rel difference {d:.2e}, lse {(lw - ls_).abs().max().item():.2e}")
    assert d < 1e-5
    assert torch.allclose(lw, ls_, rtol=0, atol=1e-5 * max(1.0, ls_.abs().max().item()))


# ---------------------------------------------------------------------------
# dense baseline
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("wl", [
    synth.config(0),
    synth.config(1, seq_lens=[8192], n_kv_heads=2, n_q_heads=8, n_components=64),
    synth.config(4, seq_lens=[3000, 9000, 1000], n_kv_heads=2, n_q_heads=8,
                 high_entropy_heads=(1,), n_components=64),
    synth.config(3, seq_lens=[7001], n_kv_heads=1, n_q_heads=5, n_components=64),
], ids=["cfg0", "cfg1r", "cfg4r-paged", "cfg3r"])
def test_dense_matches_oracle(wl):
    say(f"[dense] {wl.name} {wl.seq_lens}")
    b = synth.generate(wl, device="cuda")
    kv = ops.KVCache.from_batch(b)
    q = b.Q[0].contiguous()
    params = ops.decode_params(wl.n_q_heads, 1, 1)
    out, lse = ops.mog_dense_decode(kv, q, params)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    G = wl.group
    for s in range(wl.n_seq):
        for h in range(wl.n_kv_heads):
            K, V = b.unit_kv(s, h)
            o, l = O.dense_attention(K, V, q[s, h * G:(h + 1) * G].cpu().numpy())
            for g in range(G):
                assert rel_l2(out[s, h * G + g], o[g]) < (1e-5 if wl.dtype == "fp32" else 1e-4)
            np.testing.assert_allclose(lse[s, h * G:(h + 1) * G], l, rtol=1e-5, atol=1e-4)


# one selection per KV head (oracle reading R14)
def test_shared_selection_gqa5_reduced():
    run_decode_case(synth.config(3, seq_lens=[12000], n_kv_heads=2, n_q_heads=10, n_components=128), shared=True)


def test_shared_selection_ragged_paged_reduced():
    run_decode_case(synth.config(4, seq_lens=[3000, 9000, 1000], n_kv_heads=2, n_q_heads=8,
                                 high_entropy_heads=(1,), n_components=64), shared=True)


@pytest.mark.parametrize("G", [1, 8])
def test_shared_selection_group_sizes(G):
    run_decode_case(synth.config(1, seq_lens=[3000], n_kv_heads=1, n_q_heads=G, n_components=32), shared=True)


def test_shared_selection_fp32_top_only():
    wl = synth.config(1, seq_lens=[5000], n_kv_heads=1, n_q_heads=4, n_components=32, dtype="fp32")
    run_decode_case(wl, residual=False, shared=True)


def test_decode_is_deterministic():
    wl = synth.config(1, seq_lens=[8192], n_kv_heads=2, n_q_heads=8, n_components=64)
    b = synth.generate(wl, device="cuda")
    kv = ops.KVCache.from_batch(b)
    lays = build_oracle_layouts(b)
    lay = ops.import_layout(kv, wl.n_sink, wl.n_recent, [unit_layout_arrays(lays[u]) for u in range(2)])
    params = ops.decode_params(wl.n_q_heads, wl.top_c, wl.top_s)
    q = b.Q[0].contiguous()
    o1 = ops.mog_decode(lay, kv, q, params)[0].clone()
    o2 = ops.mog_decode(lay, kv, q, params)[0].clone()
    assert torch.equal(o1, o2)
    # the timing aid relaunches the exact kernel on the same inputs: same bits
    params.exact_repeat = 3
    o3 = ops.mog_decode(lay, kv, q, params)[0].clone()
    assert torch.equal(o1, o3)
