"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a published
test vector, a closed form, an invariant the method must have, a textbook
special case, or brute force on a tiny input.  None of them needs a GPU.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(np.asarray(b)))


def mixture_keys(rng, n, d, m, spread=0.5, sep=1.0):
    cent = rng.normal(0, sep, (m, d))
    comp = rng.integers(0, m, n)
    return cent[comp] + spread * rng.normal(0, 1, (n, d))


# ---------------------------------------------------------------------------
# PRNG and Forgy draws
# ---------------------------------------------------------------------------


def test_splitmix64_published_vector():
    g = json.load(open(os.path.join(GOLDEN, "splitmix64.json")))
    s = g["state"]
    for want in g["outputs_hex"]:
        s, out = O.splitmix64(s)
        assert out == int(want, 16)


def _fisher_yates_array(n, k, state):
    # textbook in-place Fisher-Yates on an explicit array, stopped after k steps
    a = list(range(n))
    for i in range(k):
        state, r = O.splitmix64(state)
        j = i + r % (n - i)
        a[i], a[j] = a[j], a[i]
    return a[:k]


@pytest.mark.parametrize("n,k,seed", [(10, 10, 1), (1000, 37, 7), (5, 0, 3), (4028, 64, 99)])
def test_forgy_ids_match_explicit_shuffle(n, k, seed):
    st = O.unit_state(seed, 0, 0, 1)
    ids = O.forgy_ids(n, k, st)
    assert ids == _fisher_yates_array(n, k, st)
    assert len(set(ids)) == k and all(0 <= i < n for i in ids)


def test_forgy_full_shuffle_is_uniform():
    # every permutation of 3 items appears with frequency near 1/6
    counts = {}
    for seed in range(6000):
        p = tuple(O.forgy_ids(3, 3, O.unit_state(seed, 0, 0, 1)))
        counts[p] = counts.get(p, 0) + 1
    assert len(counts) == 6
    for c in counts.values():
        assert abs(c - 1000) < 5 * math.sqrt(1000 * 5 / 6)


def test_streams_differ():
    a = O.unit_state(5, 0, 0, 8)
    assert len({a, O.unit_state(5, 0, 1, 8), O.unit_state(5, 1, 0, 8)}) == 3
    assert len({O.sub_state(a, j) for j in range(100)}) == 100


# ---------------------------------------------------------------------------
# Sizes
# ---------------------------------------------------------------------------


def test_partition_sizes_of_the_workloads():
    # sqrt / log2 partition sizes quoted for the five workloads
    assert O.unit_dims(4096, 4, 64)[1:] == (64, 12)
    assert O.unit_dims(32768, 64, 256)[1:] == (182, 15)
    assert O.unit_dims(131072, 64, 256)[1:] == (363, 17)
    assert O.unit_dims(1048576, 64, 256)[1:] == (1024, 20)


def test_ceil_sqrt_log2_brute():
    for n in range(1, 5000):
        assert O.ceil_sqrt(n) == min(r for r in range(n + 2) if r * r >= n)
        assert O.ceil_log2(n) == min(e for e in range(64) if 2 ** e >= n)
    with pytest.raises(ValueError):
        O.unit_dims(10, 5, 5)
    # C never exceeds the middle region
    assert O.unit_dims(12, 4, 4) == (4, 4, 4)


# ---------------------------------------------------------------------------
# Score / residual: the Gaussian moment generating function
# ---------------------------------------------------------------------------


def test_group_log_mass_is_gaussian_mgf_montecarlo():
    rng = np.random.default_rng(0)
    d, n_draw, tau = 8, 1_000_000, 0.7
    mu = rng.normal(0, 0.5, d)
    var = rng.uniform(0.2, 1.5, d)
    q = rng.normal(0, 1.0, d)
    k = mu + np.sqrt(var) * rng.normal(0, 1, (n_draw, d))
    x = np.exp(tau * (k @ q))
    n_group = 37
    est = math.log(n_group * x.mean())
    se = x.std() / math.sqrt(n_draw) / x.mean()  # std error of the log estimate
    got = O.group_log_mass(q, np.array([n_group]), mu[None], var[None], tau)[0]
    assert abs(got - est) < 6 * se
    # the variance term is large compared with the MC error, so a dropped
    # 1/2, a missing tau^2 or a dropped q_i^2 would all fail the bound above
    var_term = 0.5 * tau * tau * float(var @ (q * q))
    assert var_term > 100 * se
    assert abs(var_term * 2 - var_term) > 6 * se
    assert abs(0.5 * tau * float(var @ (q * q)) - var_term) > 6 * se


def test_group_log_mass_two_point_closed_form():
    # two keys mu +/- a: true mass 2 e^{tau q.mu} cosh(tau q.a); the Gaussian
    # estimate 2 e^{tau q.mu + tau^2 (q.a)^2/2} differs only at 4th order.
    tau = 0.125
    mu = np.array([0.3, -0.2, 0.1])
    a = np.array([0.4, 0.0, 0.0])
    q = np.array([2.0, 1.0, -1.0])
    K = np.stack([mu + a, mu - a])
    n, m, s, _ = O.group_stats(K, K)
    assert np.allclose(s, a * a) and np.allclose(m, mu)
    got = O.group_log_mass(q, np.array([n]), m[None], s[None], tau)[0]
    x = tau * float(q @ a)
    true = math.log(2 * math.exp(tau * float(q @ mu)) * math.cosh(x))
    assert abs(got - true) == pytest.approx(x ** 4 / 12, rel=0.05)


def test_group_log_mass_empty_is_minus_inf():
    sc = O.group_log_mass(np.ones(2), np.array([0, 3]), np.zeros((2, 2)), np.zeros((2, 2)), 1.0)
    assert sc[0] == -np.inf and sc[1] == pytest.approx(math.log(3))


# ---------------------------------------------------------------------------
# Selection
# ---------------------------------------------------------------------------


def test_top_by_score_ties_and_empties():
    s = np.array([1.0, 3.0, 3.0, 2.0, 3.0, -np.inf])
    valid = np.array([True, True, True, True, True, False])
    assert list(O.top_by_score(s, 2, valid)) == [1, 2]
    assert list(O.top_by_score(s, 3, valid)) == [1, 2, 4]
    assert list(O.top_by_score(s, 10, valid)) == [0, 1, 2, 3, 4]
    assert list(O.top_by_score(s, 0, valid)) == []
    v2 = valid.copy()
    v2[1] = False
    assert list(O.top_by_score(s, 2, v2)) == [2, 4]


# ---------------------------------------------------------------------------
# k-means
# ---------------------------------------------------------------------------


def test_lloyd_monotone_and_fixed_point():
    rng = np.random.default_rng(1)
    X = mixture_keys(rng, 600, 6, 5)
    st = O.unit_state(11, 0, 0, 1)
    init = O.forgy_ids(600, 7, st)
    a, mu, trace = O.lloyd(X, X[init], 10)
    assert all(trace[i + 1] <= trace[i] * (1 + 1e-12) for i in range(len(trace) - 1))
    # the final assignment is nearest-centroid by direct distances
    d2 = ((X[:, None, :] - mu[None, :, :]) ** 2).sum(-1)
    assert np.array_equal(a, np.argmin(d2, axis=1))


def test_nearest_centroid_ties_to_lower_id():
    X = np.array([[0.0, 0.0], [1.0, 1.0]])
    mu = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 0.0]])
    assert list(O.nearest_centroid(X, mu)) == [0, 0]


def test_empty_cluster_keeps_its_centroid():
    # duplicate init centroids: the tie goes to the lower id, the other one
    # gets no member and must keep its position through the update
    X = np.array([[10.0, 0.0], [10.0, 0.0], [10.3, 0.0], [1.0, 1.0], [1.2, 1.0]])
    a, mu, _ = O.lloyd(X, X[[0, 1, 3]], 1)
    np.testing.assert_array_equal(mu[1], [10.0, 0.0])
    np.testing.assert_allclose(mu[0], X[:3].mean(0))
    np.testing.assert_allclose(mu[2], X[3:].mean(0))


def _all_partitions(n, k):
    # assignments with labels in [0,k) up to relabelling, every label used
    for lab in itertools.product(range(k), repeat=n):
        if lab[0] != 0 or len(set(lab)) != k:
            continue
        seen = []
        ok = True
        for x in lab:
            if x not in seen:
                if x != len(seen):
                    ok = False
                    break
                seen.append(x)
        if ok:
            yield np.array(lab)


def test_partition_sse_hand_example():
    # groups {0, 2} (mean 1), {5, 7} (mean 6), {100}: 1 + 1 + 1 + 1 + 0 = 4;
    # rows out of label order and label values not 0..k-1
    X = np.array([[5.0], [0.0], [100.0], [7.0], [2.0]])
    lab = np.array([9, 4, 1, 9, 4])
    assert O.partition_sse(X, lab) == 4.0
    # one group of everything: sum of squared deviations from the grand mean
    assert O.partition_sse(X, np.zeros(5, int)) == pytest.approx(float(((X - X.mean()) ** 2).sum()), rel=1e-15)
    # singletons have no deviation; an empty input has none either
    assert O.partition_sse(X, np.arange(5)) == 0.0
    assert O.partition_sse(np.zeros((0, 3)), np.zeros(0, int)) == 0.0


@pytest.mark.parametrize("seed", range(4))
def test_partition_sse_brute_force_and_identities(seed):
    rng = np.random.default_rng(seed)
    n, d, k = 40, 5, 6
    X = rng.normal(0, 2, (n, d)) + 3.0
    lab = rng.integers(0, k, n) * 7 + 3
    # the definition with plain Python loops
    ref = 0.0
    for g in set(lab.tolist()):
        rows = [i for i in range(n) if lab[i] == g]
        mean = [sum(X[i][e] for i in rows) / len(rows) for e in range(d)]
        ref += sum((X[i][e] - mean[e]) ** 2 for i in rows for e in range(d))
    got = O.partition_sse(X, lab)
    assert got == pytest.approx(ref, rel=1e-12)
    # Koenig-Huygens: sum |x|^2 - sum_g n_g |mu_g|^2
    kh = float((X * X).sum())
    for g in np.unique(lab):
        m = X[lab == g]
        kh -= m.shape[0] * float((m.mean(0) ** 2).sum())
    assert got == pytest.approx(kh, rel=1e-9)
    # relabelling, reordering rows and translating leave it unchanged
    perm = rng.permutation(n)
    relab = {int(g): int(i) for i, g in enumerate(rng.permutation(np.unique(lab)))}
    lab2 = np.array([relab[int(x)] for x in lab])
    assert O.partition_sse(X[perm], lab2[perm]) == pytest.approx(got, rel=1e-12)
    assert O.partition_sse(X - 11.0, lab) == pytest.approx(got, rel=1e-9)
    # moving one point to another group changes it by the textbook amount:
    # removing x from a group of n with mean mu lowers the SSE by
    # n/(n-1) |x - mu|^2, adding it to a group of m with mean nu raises it
    # by m/(m+1) |x - nu|^2
    i = int(np.argmax(np.bincount(lab)))  # a point whose group has >= 2 members
    src = lab == lab[i]
    i = int(np.flatnonzero(src)[0])
    dst_g = next(g for g in np.unique(lab) if g != lab[i])
    dst = lab == dst_g
    nn, mm = src.sum(), dst.sum()
    mu, nu = X[src].mean(0), X[dst].mean(0)
    moved = lab.copy()
    moved[i] = dst_g
    delta = -nn / (nn - 1) * float(((X[i] - mu) ** 2).sum()) + mm / (mm + 1) * float(((X[i] - nu) ** 2).sum())
    assert O.partition_sse(X, moved) == pytest.approx(got + delta, rel=1e-9)


def test_subkmeans_converges_to_a_lloyd_fixed_point_per_cluster():
    # with many rounds the sub-k-means of every cluster stops at a Lloyd
    # fixed point: each member is nearest (squared distance) the mean of its
    # own subcluster among the cluster's nonempty subclusters, and a cluster
    # of n members uses at most min(S, n) subclusters
    rng = np.random.default_rng(11)
    K = mixture_keys(rng, 1200, 6, 10, spread=0.6)
    V = rng.normal(0, 1, K.shape)
    L = O.build_unit(K, V, 0, 0, 60, O.unit_state(2, 0, 0, 1))
    lab_c, lab_s = L.cluster_labels(), L.subcluster_labels()
    Xm = K[:L.n_mid]
    multi = 0
    for j in range(L.C):
        rows = np.flatnonzero(lab_c == j)
        if rows.size == 0:
            continue
        subs = np.unique(lab_s[rows])
        assert subs.size <= min(L.S, rows.size)
        # k = min(S, n) distinct members started the cluster's sub-k-means
        init = L.sub_init_ids[j]
        assert len(init) == min(L.S, rows.size) and len(set(init)) == len(init)
        assert set(init) <= set(rows.tolist())
        assert np.all(subs // L.S == j)
        means = np.stack([Xm[lab_s == g].mean(0) for g in subs])
        d2 = ((Xm[rows][:, None, :] - means[None]) ** 2).sum(-1)
        own = np.searchsorted(subs, lab_s[rows])
        assert np.all(d2[np.arange(rows.size), own] <= d2.min(1) * (1 + 1e-9) + 1e-12), j
        multi += subs.size > 1
    assert multi > L.C // 2  # most clusters were really split


def test_kmeans_brute_force_optimum_tiny():
    rng = np.random.default_rng(2)
    # three well separated blobs of three points: Lloyd from any Forgy init
    # that hits each blob reaches the global optimum of the enumeration
    cent = np.array([[0.0, 0.0], [10.0, 0.0], [0.0, 10.0]])
    X = np.concatenate([c + 0.3 * rng.normal(0, 1, (3, 2)) for c in cent])
    best = min(O.partition_sse(X, lab) for lab in _all_partitions(9, 3))
    a, _, _ = O.lloyd(X, X[[0, 3, 6]], 10)
    assert O.partition_sse(X, a) == pytest.approx(best, rel=1e-12)
    # from any Forgy init Lloyd's objective is at least the optimum
    for seed in range(20):
        ids = O.forgy_ids(9, 3, O.unit_state(seed, 0, 0, 1))
        a, _, _ = O.lloyd(X, X[ids], 10)
        assert O.partition_sse(X, a) >= best * (1 - 1e-12)


# ---------------------------------------------------------------------------
# Build: stats and layout
# ---------------------------------------------------------------------------


def _small_unit(seed=3, N=700, d=8, m=12, fp=np.float64):
    rng = np.random.default_rng(seed)
    K = mixture_keys(rng, N, d, m)
    V = rng.normal(0, 1, (N, d))
    return K, V


def test_stats_match_direct_numpy():
    K, V = _small_unit()
    L = O.build_unit(K, V, 4, 16, 10, O.unit_state(5, 0, 0, 1))
    lab_c = L.cluster_labels()
    lab_s = L.subcluster_labels()
    Km, Vm = K[4:-16], V[4:-16]
    for j in range(L.C):
        m = lab_c == j
        if m.any():
            np.testing.assert_allclose(L.cl_mu[j], Km[m].mean(0), rtol=1e-6, atol=1e-6)
            np.testing.assert_allclose(L.cl_var[j], Km[m].var(0), rtol=1e-5, atol=1e-6)
            np.testing.assert_allclose(L.cl_vbar[j], Vm[m].mean(0), rtol=1e-6, atol=1e-6)
    for g in range(L.C * L.S):
        m = lab_s == g
        assert m.sum() == L.sub_count[g]
        if m.any():
            np.testing.assert_allclose(L.sub_mu[g], Km[m].mean(0), rtol=1e-6, atol=1e-6)
            np.testing.assert_allclose(L.sub_var[g], Km[m].var(0), rtol=1e-5, atol=1e-6)
            np.testing.assert_allclose(L.sub_vbar[g], Vm[m].mean(0), rtol=1e-6, atol=1e-6)
    # rows ordered by (cluster, subcluster, position); perm is a permutation
    assert sorted(L.perm.tolist()) == list(range(4, 700 - 16))
    key = [(lab_s[p - 4], p) for p in L.perm]
    assert key == sorted(key)
    # subclusters stay inside their cluster
    assert np.array_equal(lab_s // L.S, lab_c)
    # sub-k-means used at most min(S, n_j) subclusters per cluster
    for j in range(L.C):
        used = np.count_nonzero(L.sub_count[j * L.S:(j + 1) * L.S])
        assert used <= min(L.S, L.cl_count[j])


def test_build_reaches_a_lloyd_partition():
    K, V = _small_unit(seed=4)
    L = O.build_unit(K, V, 4, 16, 10, O.unit_state(6, 0, 0, 1))
    tr = L.sse_trace
    assert all(tr[i + 1] <= tr[i] * (1 + 1e-12) for i in range(len(tr) - 1))
    # init centroids were the seeded Forgy draw
    assert L.init_ids == O.forgy_ids(L.n_mid, L.C, O.unit_state(6, 0, 0, 1))


# ---------------------------------------------------------------------------
# Decode: invariants the method must have
# ---------------------------------------------------------------------------


def test_all_selected_is_dense():
    K, V = _small_unit(seed=5)
    L = O.build_unit(K, V, 4, 16, 10, O.unit_state(7, 0, 0, 1))
    rng = np.random.default_rng(9)
    Q = rng.normal(0, 1, (3, K.shape[1])) * 1.5
    r = O.decode_unit(L, K, V, Q, L.C, L.S)
    o, lse = O.dense_attention(K, V, Q)
    assert rel(r["out"], o) < 1e-12
    assert rel(r["out_top"], o) < 1e-12
    np.testing.assert_allclose(r["lse"], lse, rtol=1e-12)
    assert (r["n_exact"] == K.shape[0]).all()


@pytest.mark.parametrize("c,s", [(0, 0), (1, 1), (3, 2), (2, 5), (40, 1)])
def test_singleton_groups_make_residual_exact(c, s):
    rng = np.random.default_rng(10)
    N, d, ns, nr = 40, 5, 2, 3
    K = rng.normal(0, 1, (N, d))
    V = rng.normal(0, 1, (N, d))
    n_mid = N - ns - nr
    Q = rng.normal(0, 1, (2, d))
    o, lse = O.dense_attention(K, V, Q)
    # (a) every cluster and every subcluster a single key: exact for any c, s
    C, S = n_mid, 3
    L = O.layout_from_assignment(K, V, ns, nr, C, S, np.arange(n_mid), np.zeros(n_mid, int))
    assert (L.cl_count == 1).all() and (L.cl_var == 0).all()
    r = O.decode_unit(L, K, V, Q, c, s)
    assert rel(r["out"], o) < 1e-6       # stats are stored in float32
    np.testing.assert_allclose(r["lse"], lse, atol=1e-6)
    if c < C:
        assert rel(r["out_top"], o) > 1e-3
    # (b) multi-key clusters, single-key subclusters, every cluster chosen:
    # the estimated part is made of singletons only, so exact for any s
    C, S = 5, 7
    L = O.layout_from_assignment(K, V, ns, nr, C, S, np.arange(n_mid) % C, np.arange(n_mid) // C)
    assert (L.sub_count <= 1).all() and (L.sub_var == 0).all() and (L.cl_count > 1).all()
    r = O.decode_unit(L, K, V, Q, C, s)
    assert rel(r["out"], o) < 1e-6


def test_singletons_from_kmeans_tiny():
    # N_mid <= S: every cluster has at most S members, so each sub-k-means
    # has k = n and every subcluster is a single key
    rng = np.random.default_rng(11)
    N, d = 10, 4
    K = rng.normal(0, 1, (N, d))
    V = rng.normal(0, 1, (N, d))
    L = O.build_unit(K, V, 3, 3, 10, O.unit_state(1, 0, 0, 1))
    assert L.n_mid == 4 and (L.sub_count <= 1).all()
    Q = rng.normal(0, 1, (2, d))
    o, _ = O.dense_attention(K, V, Q)
    for c, s in [(0, 0), (1, 1), (2, 4)]:
        assert rel(O.decode_unit(L, K, V, Q, c, s)["out"], o) < 1e-6


def test_key_permutation_invariance():
    rng = np.random.default_rng(12)
    N, d, ns, nr = 500, 6, 4, 12
    K = mixture_keys(rng, N, d, 9, spread=0.3, sep=2.0)
    V = rng.normal(0, 1, (N, d))
    L1 = O.build_unit(K, V, ns, nr, 10, O.unit_state(3, 0, 0, 1))
    n_mid = L1.n_mid
    pi = rng.permutation(n_mid)          # new middle slot m holds old slot pi[m]
    inv = np.empty_like(pi)
    inv[pi] = np.arange(n_mid)
    K2, V2 = K.copy(), V.copy()
    K2[ns:N - nr] = K[ns:N - nr][pi]
    V2[ns:N - nr] = V[ns:N - nr][pi]
    init2 = [int(inv[i]) for i in L1.init_ids]
    sub2 = {j: [int(inv[i]) for i in ids] for j, ids in L1.sub_init_ids.items()}
    L2 = O.build_unit(K2, V2, ns, nr, 10, O.unit_state(3, 0, 0, 1), init_ids=init2,
                      sub_init_ids=sub2)
    # identical partitions as sets of (key, value) pairs
    c1, c2 = L1.subcluster_labels(), L2.subcluster_labels()
    assert np.array_equal(c2, c1[pi])
    Q = rng.normal(0, 1, (3, d)) * 2
    for c, s in [(2, 2), (4, 3), (1, 6)]:
        r1 = O.decode_unit(L1, K, V, Q, c, s)
        r2 = O.decode_unit(L2, K2, V2, Q, c, s)
        assert rel(r2["out"], r1["out"]) < 1e-12
        assert rel(r2["out_top"], r1["out_top"]) < 1e-12


def _brute_force(L, K, V, q, c, s, scale):
    """Selection by sorting every group, output by the literal unshifted
    quotient of sums over every token and every estimated group."""
    N, C, S = L.N, L.C, L.S
    cnt_c = L.cl_count
    cnt_s = L.sub_count
    lab_s = L.subcluster_labels()
    f64 = lambda a: np.asarray(a, dtype=np.float64)

    def score(n, mu, var):
        return math.log(n) + scale * float(q @ mu) + 0.5 * scale ** 2 * float((q * q) @ var)

    cl_scores = [(score(cnt_c[j], L.cl_mu[j], L.cl_var[j]), j) for j in range(C) if cnt_c[j]]
    chosen = sorted(cl_scores, key=lambda t: (-t[0], t[1]))[:c]
    chosen = {j for _, j in chosen}
    chosen_sub = set()
    for j in chosen:
        subs = [(score(cnt_s[g], L.sub_mu[g], L.sub_var[g]), g) for g in range(j * S, j * S + S) if cnt_s[g]]
        chosen_sub |= {g for _, g in sorted(subs, key=lambda t: (-t[0], t[1]))[:s]}
    num = np.zeros(K.shape[1])
    den = 0.0
    for t in range(N):
        mid = L.n_sink <= t < N - L.n_recent
        if not mid or lab_s[t - L.n_sink] in chosen_sub:
            w = math.exp(scale * float(q @ K[t]))
            num += w * V[t]
            den += w
    for j in range(C):
        if cnt_c[j] and j not in chosen:
            w = math.exp(score(cnt_c[j], L.cl_mu[j], L.cl_var[j]))
            num += w * f64(L.cl_vbar[j])
            den += w
    for g in range(C * S):
        if cnt_s[g] and g // S in chosen and g not in chosen_sub:
            w = math.exp(score(cnt_s[g], L.sub_mu[g], L.sub_var[g]))
            num += w * f64(L.sub_vbar[g])
            den += w
    return num / den, sorted(chosen), sorted(chosen_sub)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_brute_force_tiny(seed):
    rng = np.random.default_rng(100 + seed)
    N, d = 90, 4
    K = mixture_keys(rng, N, d, 6)
    V = rng.normal(0, 1, (N, d))
    L = O.build_unit(K, V, 3, 5, 10, O.unit_state(seed, 0, 0, 1))
    Q = rng.normal(0, 1, (2, d)) * 1.5
    scale = 0.5
    for c, s in [(0, 0), (1, 1), (2, 3), (5, 2), (L.C, L.S)]:
        r = O.decode_unit(L, K, V, Q, c, s, scale=scale)
        for h in range(2):
            out, ch, chs = _brute_force(L, K, V, Q[h], c, s, scale)
            assert rel(r["out"][h], out) < 1e-12
            assert list(r["sel_c"][h]) == ch
            got_subs = sorted(int(j) * L.S + int(i) for j, picks in zip(r["sel_c"][h], r["sel_s"][h]) for i in picks)
            assert got_subs == chs


def test_translation_invariance():
    rng = np.random.default_rng(13)
    N, d = 400, 6
    K = mixture_keys(rng, N, d, 8, spread=0.3, sep=2.0)
    V = rng.normal(0, 1, (N, d))
    Q = rng.normal(0, 1, (2, d))
    st = O.unit_state(4, 0, 0, 1)
    L = O.build_unit(K, V, 4, 8, 10, st)
    r = O.decode_unit(L, K, V, Q, 3, 2)
    b_k = rng.normal(0, 1, d)
    Lk = O.build_unit(K + b_k, V, 4, 8, 10, st)
    assert np.array_equal(Lk.subcluster_labels(), L.subcluster_labels())
    rk = O.decode_unit(Lk, K + b_k, V, Q, 3, 2)
    assert rel(rk["out"], r["out"]) < 1e-6  # float32-stored means shift
    b_v = rng.normal(0, 1, d)
    Lv = O.build_unit(K, V + b_v, 4, 8, 10, st)
    rv = O.decode_unit(Lv, K, V + b_v, Q, 3, 2)
    assert rel(rv["out"], r["out"] + b_v) < 1e-6


def test_selection_override_and_top_only():
    K, V = _small_unit(seed=6)
    L = O.build_unit(K, V, 4, 16, 10, O.unit_state(8, 0, 0, 1))
    Q = np.random.default_rng(1).normal(0, 1, (2, K.shape[1]))
    r = O.decode_unit(L, K, V, Q, 3, 2)
    r2 = O.decode_unit(L, K, V, Q, 3, 2, sel_override=(r["sel_c"], r["sel_s"]))
    assert rel(r2["out"], r["out"]) == 0.0
    # top-only = softmax restricted to the exact rows (textbook)
    for h in range(2):
        rows = list(range(4)) + list(range(K.shape[0] - 16, K.shape[0]))
        for j, picks in zip(r["sel_c"][h], r["sel_s"][h]):
            for i in picks:
                g = j * L.S + i
                rows += list(L.perm[L.sub_off[g]:L.sub_off[g + 1]])
        o, _ = O.dense_attention(K[rows], V[rows], Q[h])
        assert rel(r["out_top"][h], o[0]) < 1e-12
    # residual off returns the top-only output
    r3 = O.decode_unit(L, K, V, Q, 3, 2, residual=False)
    assert rel(r3["out"], r["out_top"]) == 0.0


# ---------------------------------------------------------------------------
# Shared selection per KV head (reading R14)
# ---------------------------------------------------------------------------


def _brute_force_shared(L, K, V, Q, c, s, scale):
    """Shared selection from plain per-group exponentials: each head's
    estimated masses exp(score) divided by the head's total over the
    nonempty clusters, summed over the heads; then every head's output by
    the literal quotient of sums (selection shared)."""
    N, C, S = L.N, L.C, L.S
    cnt_c, cnt_s = L.cl_count, L.sub_count
    lab_s = L.subcluster_labels()
    f64 = lambda a: np.asarray(a, dtype=np.float64)

    def mass(q, n, mu, var):
        return n * math.exp(scale * float(q @ mu) + 0.5 * scale ** 2 * float((q * q) @ var))

    G = Q.shape[0]
    tot = [sum(mass(Q[h], cnt_c[j], L.cl_mu[j], L.cl_var[j]) for j in range(C) if cnt_c[j]) for h in range(G)]
    gsc = [(sum(mass(Q[h], cnt_c[j], L.cl_mu[j], L.cl_var[j]) / tot[h] for h in range(G)), j)
           for j in range(C) if cnt_c[j]]
    chosen = {j for _, j in sorted(gsc, key=lambda t: (-t[0], t[1]))[:c]}
    chosen_sub = set()
    for j in chosen:
        gss = [(sum(mass(Q[h], cnt_s[g], L.sub_mu[g], L.sub_var[g]) / tot[h] for h in range(G)), g)
               for g in range(j * S, j * S + S) if cnt_s[g]]
        chosen_sub |= {g for _, g in sorted(gss, key=lambda t: (-t[0], t[1]))[:s]}
    outs = []
    for h in range(G):
        q = Q[h]
        num, den = np.zeros(K.shape[1]), 0.0
        for t in range(N):
            if not (L.n_sink <= t < N - L.n_recent) or lab_s[t - L.n_sink] in chosen_sub:
                w = math.exp(scale * float(q @ K[t]))
                num += w * V[t]
                den += w
        for j in range(C):
            if cnt_c[j] and j not in chosen:
                w = mass(q, cnt_c[j], L.cl_mu[j], L.cl_var[j])
                num += w * f64(L.cl_vbar[j])
                den += w
        for g in range(C * S):
            if cnt_s[g] and g // S in chosen and g not in chosen_sub:
                w = mass(q, cnt_s[g], L.sub_mu[g], L.sub_var[g])
                num += w * f64(L.sub_vbar[g])
                den += w
        outs.append(num / den)
    return np.array(outs), sorted(chosen), sorted(chosen_sub)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_shared_selection_matches_brute_force_tiny(seed):
    rng = np.random.default_rng(300 + seed)
    N, d = 120, 4
    K = mixture_keys(rng, N, d, 6)
    V = rng.normal(0, 1, (N, d))
    L = O.build_unit(K, V, 3, 5, 10, O.unit_state(seed, 0, 0, 1))
    # heads of very different logit scales: the per-head normalisation is
    # what keeps one of them from deciding alone
    Q = rng.normal(0, 1, (3, d)) * np.array([[0.3], [1.5], [4.0]])
    scale = 0.5
    for c, s in [(1, 1), (2, 2), (4, 3), (L.C, L.S)]:
        r = O.decode_unit(L, K, V, Q, c, s, scale=scale, shared=True)
        out, ch, chs = _brute_force_shared(L, K, V, Q, c, s, scale)
        assert rel(r["out"], out) < 1e-11
        for h in range(3):
            assert list(r["sel_c"][h]) == ch
            got = sorted(int(j) * L.S + int(i) for j, p in zip(r["sel_c"][h], r["sel_s"][h]) for i in p)
            assert got == chs


def test_shared_selection_single_head_is_per_head():
    K, V = _small_unit(seed=9)
    L = O.build_unit(K, V, 4, 16, 10, O.unit_state(2, 0, 0, 1))
    q = np.random.default_rng(4).normal(0, 1, (1, K.shape[1]))
    a = O.decode_unit(L, K, V, q, 3, 2)
    b = O.decode_unit(L, K, V, q, 3, 2, shared=True)
    assert list(a["sel_c"][0]) == list(b["sel_c"][0])
    assert all(list(x) == list(y) for x, y in zip(a["sel_s"][0], b["sel_s"][0]))
    assert rel(b["out"], a["out"]) == 0.0


def test_shared_selection_identical_heads_is_per_head():
    K, V = _small_unit(seed=10)
    L = O.build_unit(K, V, 4, 16, 10, O.unit_state(3, 0, 0, 1))
    q = np.random.default_rng(5).normal(0, 1, K.shape[1])
    Q = np.stack([q, q, q, q])
    a = O.decode_unit(L, K, V, Q, 3, 2)
    b = O.decode_unit(L, K, V, Q, 3, 2, shared=True)
    for h in range(4):
        assert list(a["sel_c"][h]) == list(b["sel_c"][h])
    assert rel(b["out"], a["out"]) < 1e-15


def test_shared_selection_caps_the_union():
    K, V = _small_unit(seed=11, N=1500, m=20)
    L = O.build_unit(K, V, 4, 16, 10, O.unit_state(6, 0, 0, 1))
    Q = np.random.default_rng(6).normal(0, 1, (5, K.shape[1])) * 2.0
    c, s = 4, 2
    per = O.decode_unit(L, K, V, Q, c, s)
    sh = O.decode_unit(L, K, V, Q, c, s, shared=True)
    union_c = set().union(*[set(int(j) for j in x) for x in sh["sel_c"]])
    assert len(union_c) == min(c, int((L.cl_count > 0).sum()))
    assert all(len(p) <= s for p in sh["sel_s"][0])
    # subclusters read once for the KV head: at most one head's budget c s
    # shared; the per-head selections read their union
    subs = lambda r: set().union(*[set(int(j) * L.S + int(i) for j, p in zip(r["sel_c"][h], r["sel_s"][h]) for i in p)
                                   for h in range(5)])
    assert len(subs(sh)) <= c * s
    assert len(subs(per)) >= max(len(set(int(j) * L.S + int(i) for j, p in zip(per["sel_c"][h], per["sel_s"][h])
                                         for i in p)) for h in range(5))


# ---------------------------------------------------------------------------
# Incremental decode: folding the tokens that leave the recent window (R15)
# ---------------------------------------------------------------------------


def _grown_unit(seed, N=600, grow=40, d=6, n_sink=4, n_recent=16):
    rng = np.random.default_rng(seed)
    K = mixture_keys(rng, N + grow, d, 10)
    V = rng.normal(0, 1, (N + grow, d))
    L = O.build_unit(K[:N], V[:N], n_sink, n_recent, 10, O.unit_state(seed, 0, 0, 1))
    return K, V, L


def test_fold_stats_equal_direct_group_stats():
    """Welford's running updates reach the two-pass statistics of the grown
    groups (closed form), and every folded token went to its nearest group."""
    K, V, L = _grown_unit(21)
    F = O.fold_tokens(L, K, V, 40)
    S = L.S
    members = {}
    for g in range(L.C * S):
        members[g] = list(F.group_rows(g))
    for j in range(L.C):
        rows = np.concatenate([members[j * S + i] for i in range(S)])
        if rows.size:
            _, mu, s, vb = O.group_stats(K[rows], V[rows])
            np.testing.assert_allclose(F.cl_mu[j], mu, rtol=1e-5, atol=1e-5)
            np.testing.assert_allclose(F.cl_var[j], s, rtol=1e-4, atol=1e-5)
            np.testing.assert_allclose(F.cl_vbar[j], vb, rtol=1e-5, atol=1e-5)
    for g, rows in members.items():
        if len(rows):
            _, mu, s, vb = O.group_stats(K[rows], V[rows])
            np.testing.assert_allclose(F.sub_mu[g], mu, rtol=1e-5, atol=1e-5)
            np.testing.assert_allclose(F.sub_var[g], s, rtol=1e-4, atol=1e-5)
    # nearest cluster at the time of the fold: replay the folds one by one
    cur = L
    for step, t in enumerate(F.fold_pos):
        d2 = ((cur.cl_mu.astype(np.float64) - K[t]) ** 2).sum(axis=1)
        d2[cur.cl_count == 0] = np.inf
        assert F.fold_sub[step] // S == int(np.flatnonzero(d2 == d2.min())[0])
        g = F.fold_sub[step]
        ds = ((cur.sub_mu[g - g % S:g - g % S + S].astype(np.float64) - K[t]) ** 2).sum(axis=1)
        ds[cur.sub_count[g - g % S:g - g % S + S] == 0] = np.inf
        assert g % S == int(np.flatnonzero(ds == ds.min())[0])
        cur = O.fold_tokens(cur, K[:cur.N + 1], V[:cur.N + 1], 1)
    assert cur.fold_sub == F.fold_sub


def test_fold_all_selected_is_dense_on_the_grown_sequence():
    K, V, L = _grown_unit(22)
    F = O.fold_tokens(L, K, V, 40)
    assert F.N == K.shape[0] and len(F.fold_pos) == 40
    Q = np.random.default_rng(3).normal(0, 1, (2, K.shape[1]))
    r = O.decode_unit(F, K, V, Q, F.C, F.S)
    o, l = O.dense_attention(K, V, Q)
    assert rel(r["out"], o) < 1e-12
    np.testing.assert_allclose(r["lse"], l, rtol=1e-12)


def test_fold_zero_tokens_and_one_at_a_time():
    K, V, L = _grown_unit(23, grow=12)
    F0 = O.fold_tokens(L, K, V, 0)
    assert F0.N == L.N and F0.fold_pos == [] and np.array_equal(F0.cl_mu, L.cl_mu)
    Fa = O.fold_tokens(L, K, V, 12)
    Fb = L
    for k in range(12):
        Fb = O.fold_tokens(Fb, K[:L.N + k + 1], V[:L.N + k + 1], 1)
    assert Fa.fold_sub == Fb.fold_sub and Fa.fold_pos == Fb.fold_pos
    assert np.array_equal(Fa.sub_mu, Fb.sub_mu) and np.array_equal(Fa.cl_var, Fb.cl_var)


def test_fold_skips_empty_clusters_and_lands_near_its_key():
    """A key placed on a nonempty cluster's mean joins that cluster; a key at
    the zero placeholder mean of an empty cluster joins a nonempty one, and
    the empty cluster stays empty."""
    rng = np.random.default_rng(7)
    d, N, n_sink, n_recent = 4, 200, 2, 8
    K = mixture_keys(rng, N + 2, d, 4) + 5.0
    V = rng.normal(0, 1, (N + 2, d))
    n_mid = N - n_sink - n_recent
    C, S = 4, 3
    # clusters 0..2 by the first coordinate's tercile, cluster 3 empty
    x = K[n_sink:N - n_recent, 0]
    cl = np.digitize(x, np.quantile(x, [1 / 3, 2 / 3]))
    sub = np.arange(n_mid) % S
    L = O.layout_from_assignment(K[:N], V[:N], n_sink, n_recent, C, S, cl, sub)
    assert L.cl_count[3] == 0 and not L.cl_mu[3].any()
    j = int(np.argmax(L.cl_count))
    K[N - n_recent] = L.cl_mu[j].astype(np.float64) + 1e-3
    K[N - n_recent + 1] = 0.0  # nearer to the placeholder than to any mean
    F = O.fold_tokens(L, K, V, 2)
    assert F.fold_sub[0] // S == j
    assert F.sub_count[F.fold_sub[0]] == L.sub_count[F.fold_sub[0]] + 1
    assert F.fold_sub[1] // S != 3 and F.cl_count[3] == 0
    assert F.cl_count.sum() == L.cl_count.sum() + 2


# ---------------------------------------------------------------------------
# Dense attention: textbook special cases
# ---------------------------------------------------------------------------


def test_dense_special_cases():
    rng = np.random.default_rng(14)
    V = rng.normal(0, 1, (7, 3))
    # equal keys: plain mean of the values
    K = np.ones((7, 3))
    o, lse = O.dense_attention(K, V, np.array([0.3, 0.1, -2.0]), scale=1.0)
    np.testing.assert_allclose(o[0], V.mean(0), rtol=1e-13)
    assert lse[0] == pytest.approx(math.log(7) + (0.3 + 0.1 - 2.0), rel=1e-13)
    # one key far ahead: its value
    K = rng.normal(0, 1, (7, 3))
    K[4] = [100.0, 0, 0]
    o, _ = O.dense_attention(K, V, np.array([1.0, 0, 0]), scale=1.0)
    np.testing.assert_allclose(o[0], V[4], atol=1e-30 + 1e-12)
    # lse against a library logsumexp
    q = rng.normal(0, 1, 3)
    _, lse = O.dense_attention(K, V, q, scale=0.7)
    assert lse[0] == pytest.approx(logsumexp(0.7 * K @ q), rel=1e-13)


# ---------------------------------------------------------------------------
# Feature-map residual (R16)
# ---------------------------------------------------------------------------


def test_positive_features_estimate_the_softmax_kernel():
    """E[phi(x).phi(y)] = exp(x.y): with w ~ N(0, I) each feature product is
    exp(w.(x+y) - |x|^2/2 - |y|^2/2), whose mean is exp(|x+y|^2/2 - |x|^2/2 -
    |y|^2/2) = exp(x.y) (the Gaussian moment generating function).  A
    million features land within a few standard errors of it."""
    rng = np.random.default_rng(31)
    d, m = 4, 1_000_000
    x = rng.normal(0, 0.4, d)
    y = rng.normal(0, 0.4, d)
    W = rng.normal(0, 1, (m, d))
    est = float(O.positive_features(x, W)[0] @ O.positive_features(y, W)[0])
    exact = math.exp(x @ y)
    var = math.exp(2 * (x + y) @ (x + y) - x @ x - y @ y) - exact ** 2
    assert abs(est - exact) < 5 * math.sqrt(var / m)
    # every feature is positive, and their squared norm estimates exp(|x|^2)
    f = O.positive_features(x, W)[0]
    assert (f > 0).all()
    assert abs(f @ f - math.exp(x @ x)) < 0.02 * math.exp(x @ x)


def test_feature_residual_with_zero_projection_is_a_closed_form():
    """With W = 0 every feature is exp(-|x|^2/2)/sqrt(m), so a group's
    estimated mass is exp(-s|q|^2/2) sum_t exp(-s|k_t|^2/2) exactly; with no
    cluster chosen, the decode output is the merge of the anchors with these
    masses times the mean values."""
    rng = np.random.default_rng(32)
    d, N, ns, nr = 3, 120, 2, 6
    K = mixture_keys(rng, N, d, 3)
    V = rng.normal(0, 1, (N, d))
    L = O.build_unit(K, V, ns, nr, 10, O.unit_state(2, 0, 0, 1))
    W = np.zeros((5, d), np.float32)
    s = 0.7
    F = O.with_feature_summaries(L, K, W, scale=s)
    q = rng.normal(0, 1, d)
    r = O.decode_unit(F, K, V, q[None], 0, 0, scale=s, feature_residual=True)
    anchors = np.r_[0:ns, N - nr:N]
    num = (np.exp(s * K[anchors] @ q)[:, None] * V[anchors]).sum(0)
    den = np.exp(s * K[anchors] @ q).sum()
    for j in range(L.C):
        rows = np.concatenate([L.group_rows(j * L.S + i) for i in range(L.S)])
        if rows.size:
            w = math.exp(-s * (q @ q) / 2) * np.exp(-s * (K[rows] ** 2).sum(1) / 2).sum()
            num = num + w * F.cl_vbar[j].astype(np.float64)
            den += w
    np.testing.assert_allclose(r["out"][0], num / den, rtol=1e-6)


def test_feature_residual_recovers_dense_attention_with_many_features():
    """No cluster chosen: anchors exact, the whole middle region estimated
    from feature sums.  With groups of near-equal values the mean-value model
    is close, and with 200k features the estimate of the mass is close: the
    output approaches dense attention (and the lse the dense lse)."""
    rng = np.random.default_rng(33)
    d, N = 4, 200
    K = 0.3 * rng.normal(0, 1, (N, d))
    V = rng.normal(0, 1, (N, d))
    L = O.build_unit(K, V, 2, 6, 10, O.unit_state(3, 0, 0, 1))
    # every subcluster a singleton group: mean value = the token's value
    lab = L.cluster_labels()
    sub = np.empty(L.n_mid, np.int64)
    for j in range(L.C):
        members = np.flatnonzero(lab == j)
        sub[members] = np.arange(members.size)
    S = int(sub.max()) + 1
    L2 = O.layout_from_assignment(K, V, 2, 6, L.C, S, lab, sub)
    W = rng.normal(0, 1, (200_000, d)).astype(np.float32)
    F = O.with_feature_summaries(L2, K, W, scale=1.0)
    Q = rng.normal(0, 0.3, (2, d))
    r = O.decode_unit(F, K, V, Q, F.C, 0, scale=1.0, feature_residual=True)
    o, lse = O.dense_attention(K, V, Q, scale=1.0)
    # per-group relative standard deviation sqrt((e^{|x|^2+|y|^2} - 1) / m)
    # is about 2e-3 here
    assert rel(r["out"], o) < 1e-2
    np.testing.assert_allclose(r["lse"], lse, atol=5e-3)
    # the Gaussian residual on the same singletons is exact (s = 0) up to
    # the float32 storage of the statistics
    g = O.decode_unit(F, K, V, Q, F.C, 0, scale=1.0)
    assert rel(g["out"], o) < 1e-6
    # the selection does not depend on the residual mode
    g = O.decode_unit(F, K, V, Q, 2, 1, scale=1.0)
    f = O.decode_unit(F, K, V, Q, 2, 1, scale=1.0, feature_residual=True)
    assert all(np.array_equal(a, b) for a, b in zip(g["sel_c"], f["sel_c"]))


def test_feature_sums_follow_the_folds():
    """Folding adds each token's features to its two groups: the running
    sums equal the sums recomputed over the grown groups' members."""
    K, V, L = _grown_unit(24, grow=30)
    W = np.random.default_rng(5).normal(0, 1, (16, K.shape[1])).astype(np.float32)
    F0 = O.with_feature_summaries(L, K, W)
    F = O.fold_tokens(F0, K, V, 30)
    R = O.with_feature_summaries(F, K, W)
    np.testing.assert_allclose(F.cl_z, R.cl_z, rtol=1e-5)
    np.testing.assert_allclose(F.sub_z, R.sub_z, rtol=1e-5)


def test_feature_numerator_with_zero_projection_is_a_closed_form():
    """With W = 0 every feature is exp(-|x|^2/2)/sqrt(m), so a left-out
    group's numerator estimate is exp(-s|q|^2/2) sum_t exp(-s|k_t|^2/2) v_t
    and its denominator estimate the same sum without v_t, exactly: the
    output is the merge of the anchors with these terms."""
    rng = np.random.default_rng(34)
    d, N, ns, nr = 3, 120, 2, 6
    K = mixture_keys(rng, N, d, 3)
    V = rng.normal(0, 1, (N, d))
    L = O.build_unit(K, V, ns, nr, 10, O.unit_state(4, 0, 0, 1))
    W = np.zeros((5, d), np.float32)
    s = 0.7
    F = O.with_feature_summaries(L, K, W, scale=s, V=V)
    q = rng.normal(0, 1, d)
    r = O.decode_unit(F, K, V, q[None], 0, 0, scale=s, feature_residual=True, feature_numerator=True)
    anchors = np.r_[0:ns, N - nr:N]
    num = (np.exp(s * K[anchors] @ q)[:, None] * V[anchors]).sum(0)
    den = np.exp(s * K[anchors] @ q).sum()
    mid = np.arange(ns, N - nr)
    w = math.exp(-s * (q @ q) / 2) * np.exp(-s * (K[mid] ** 2).sum(1) / 2)
    num = num + (w[:, None] * V[mid]).sum(0)
    den += w.sum()
    np.testing.assert_allclose(r["out"][0], num / den, rtol=1e-5)


def test_feature_numerator_recovers_dense_attention_for_any_groups():
    """No cluster chosen, ordinary k-means groups (not singletons): with the
    value summaries both the numerator and the denominator of every group
    converge to the exact sums as the features grow, so the output
    approaches dense attention; the mean-value model does not (its error is
    a property of the groups, not of the features)."""
    rng = np.random.default_rng(35)
    d, N = 4, 240
    K = 0.3 * rng.normal(0, 1, (N, d))
    # values that follow the keys: inside a group the attention-weighted mean
    # value differs from the plain mean
    V = 3.0 * K + 0.1 * rng.normal(0, 1, (N, d))
    L = O.build_unit(K, V, 2, 6, 10, O.unit_state(5, 0, 0, 1))
    assert L.sub_count.max() > 1
    W = rng.normal(0, 1, (200_000, d)).astype(np.float32)
    F = O.with_feature_summaries(L, K, W, scale=1.0, V=V)
    # |q|^2 + |k|^2 stays near 1, so each group's estimates have a relative
    # standard deviation of about sqrt((e - 1) / m) = 3e-3
    Q = rng.normal(0, 0.4, (2, d))
    o, lse = O.dense_attention(K, V, Q, scale=1.0)
    full = O.decode_unit(F, K, V, Q, 0, 0, scale=1.0, feature_residual=True, feature_numerator=True)
    mean_value = O.decode_unit(F, K, V, Q, 0, 0, scale=1.0, feature_residual=True)
    assert rel(full["out"], o) < 2e-2
    np.testing.assert_allclose(full["lse"], lse, atol=1e-2)
    assert rel(mean_value["out"], o) > 5 * rel(full["out"], o)
    # the denominators (and so the lse) of the two models are the same
    np.testing.assert_allclose(full["lse"], mean_value["lse"], rtol=1e-12)


def test_feature_value_sums_follow_the_folds():
    K, V, L = _grown_unit(25, grow=20)
    W = np.random.default_rng(6).normal(0, 1, (8, K.shape[1])).astype(np.float32)
    F0 = O.with_feature_summaries(L, K, W, V=V)
    F = O.fold_tokens(F0, K, V, 20)
    R = O.with_feature_summaries(F, K, W, V=V)
    np.testing.assert_allclose(F.cl_zv, R.cl_zv, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(F.sub_zv, R.sub_zv, rtol=1e-5, atol=1e-6)


# ---------------------------------------------------------------------------
# Reading R18: the decode's statistics in bfloat16
# ---------------------------------------------------------------------------
def test_bf16_round_matches_torch_conversion():
    # torch's float32 -> bfloat16 conversion rounds to nearest, ties to even
    import torch
    rng = np.random.default_rng(18)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.standard_normal(2000), np.array([0.0, -0.0, 1e-40, -1e-40, 3.4e38, -3.4e38])])
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_round(x32)
    assert np.array_equal(got, ref, equal_nan=True)


def test_bf16_round_worked_values():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: the even neighbour (1)
    # wins; 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 (odd last bit) and
    # 1 + 2^-6: the latter wins; anything past halfway rounds up
    cases = {1.0: 1.0, 1 + 2 ** -8: 1.0, 1 + 3 * 2 ** -8: 1 + 2 ** -6, 1 + 2 ** -8 + 2 ** -20: 1 + 2 ** -7,
             -(1 + 2 ** -8 + 2 ** -20): -(1 + 2 ** -7), 1 + 2 ** -9: 1.0, 3.0: 3.0, 0.1: 0.10009765625,
             -0.0: -0.0, 2.0 ** -130: 2.0 ** -130}
    for x, want in cases.items():
        assert O.bf16_round(x) == want, (x, float(O.bf16_round(x)), want)
    big = float(np.finfo(np.float32).max)
    assert O.bf16_round(big) == np.inf and O.bf16_round(-big) == -np.inf
    assert np.isnan(O.bf16_round(np.nan)) and O.bf16_round(np.inf) == np.inf
    # 8 significant bits: every value is within half a unit in the 8th bit
    x = np.random.default_rng(3).uniform(-1e3, 1e3, 10000)
    r = O.bf16_round(x)
    assert np.all(np.abs(r - x.astype(np.float32)) <= np.abs(x) * 2.0 ** -8)
    # and rounding is idempotent
    assert np.array_equal(O.bf16_round(r), r)


def test_decode_statistics_rounds_only_the_statistics():
    rng = np.random.default_rng(5)
    K = rng.standard_normal((700, 16))
    V = rng.standard_normal((700, 16))
    L = O.build_unit(K, V, 4, 16, 3, O.unit_state(1, 0, 0, 1))
    R = O.decode_statistics(L)
    for name in ("cl_mu", "cl_var", "cl_vbar", "sub_mu", "sub_var", "sub_vbar"):
        assert np.array_equal(getattr(R, name), O.bf16_round(getattr(L, name))), name
        assert not np.array_equal(getattr(R, name), getattr(L, name)), name
    assert np.array_equal(R.perm, L.perm) and np.array_equal(R.sub_off, L.sub_off)
    assert np.array_equal(R.cl_count, L.cl_count) and np.array_equal(R.sub_count, L.sub_count)
    # every group chosen whole: no statistic is used, the decode is dense
    Q = rng.standard_normal((2, 16))
    a = O.decode_unit(R, K, V, Q, R.C, R.S)
    o, _ = O.dense_attention(K, V, Q)
    assert np.max(np.abs(a["out"] - o)) < 1e-12
