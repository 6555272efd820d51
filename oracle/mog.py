"""Plain float64 NumPy oracle of Mixture-of-Gaussians (Iceberg) decode attention.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. It shares
no code with the HIP library and imports nothing from it.

What the pages fix
------------------
* "Iceberg Attention: Sublinear Long-Context Decoding with Mixture-of-Gaussians"
  (page 1, abstract): after prefill the keys of each head are partitioned
  hierarchically into O(sqrt N) clusters and O(log N) subclusters per
  cluster; each group is represented by a Gaussian; at decode the query is
  scored against these summaries, the most relevant clusters and
  subclusters are attended exactly, and the rest of the cache is estimated
  from the groups' means and variances.
* Retrieval-completion attention page (page 4, abstract and summary): exact
  attention also covers fixed sink/tail anchor tokens; the exact part and
  the estimated remainder are added as unnormalised numerator and
  denominator, and a single normalisation follows.
* DuoAttention review (page 2, "Method"): 64 sink plus 256 recent tokens is
  the anchor size used on long-context workloads.

Readings taken where the pages leave a step open (each one is also listed
in the design notes of the repository):
  R1  C = ceil(sqrt(N)) clusters and S = ceil(log2(N)) subclusters per
      cluster, N the total sequence length; C is capped at the number of
      middle-region keys.
  R2  Only the middle region [n_sink, N - n_recent) is clustered; anchors are
      always exact.
  R3  The partitioner is Lloyd k-means with squared Euclidean distance,
      Forgy initialisation by a partial Fisher-Yates shuffle driven by
      SplitMix64, T iterations of (assign, update), then one final assign.
      Ties go to the lower centroid id; an empty cluster keeps its centroid.
  R4  A cluster is split by a second k-means over its members with
      k = min(S, n_members), same rules, its own PRNG stream.
  R5  Group Gaussian = diagonal: mean mu and population variance s (divide
      by n), plus count n and mean value vbar.
  R6  Group score = log of the estimated unnormalised attention mass of the
      group: ln n + tau q.mu + tau^2/2 sum_i q_i^2 s_i, which is
      ln(n E[exp(tau q.k)]) for k ~ N(mu, diag s) (Gaussian moment
      generating function).  The residual uses the same quantity:
      denominator term exp(score), numerator term exp(score) * vbar.
  R7  Top-c clusters per query head, then top-s subclusters inside each
      chosen cluster; a chosen cluster is represented by its subclusters
      (chosen ones exact, the others by their own Gaussian).  Ties go to the
      lower id; empty groups are never chosen; with fewer nonempty groups
      than the budget all nonempty ones are chosen.
  R8  Every query head makes its own selection (GQA heads sharing a KV head
      are independent instances).
  R14 Optional shared selection for the G query heads of a KV head (the
      DuoAttention review, page 2, "Limitations" and its closing
      discussion: query heads that share a KV head couple their needs).
      Each head's group scores are turned into estimated fractions of its
      attention mass, exp(score - LSE_h) with LSE_h the log-sum-exp of the
      head's nonempty cluster scores; a cluster's group score is the sum of
      these fractions over the heads, the subclusters of a chosen cluster
      are scored the same way (same LSE_h), and every head then uses the one
      top-c / top-s selection.  The exact read per KV head is then capped at
      one head's budget.
  R15 Incremental decode: the cache grows by appended tokens, and the tokens
      that leave the recent window (oldest first) join the middle region.
      Each goes to the nonempty cluster whose mean key is nearest (squared
      distance, ties to the lower id; an empty cluster has no Gaussian, its
      stored statistics are placeholders), then to the nearest nonempty
      subcluster of that cluster; both groups' count, mean key, population
      variance and mean value are updated by Welford's running formulas, and
      the token's rows are kept in a fold area and read exactly whenever its
      subcluster is chosen.  C, S and the rest of the partition stay until
      the next build.
  R16 Feature-map residual (the retrieval-completion page's abstract: the
      mid-region numerator and denominator left out of the exact part are
      estimated from a fixed-size feature-map summary computed at prefill).
      The feature map is the positive random-feature map of the softmax
      kernel, phi(x) = exp(W x - |x|^2 / 2) / sqrt(m) with the m rows of W
      drawn from N(0, I_d) (an input), so that E[phi(x).phi(y)] = exp(x.y);
      with x = sqrt(scale) q and y = sqrt(scale) k this estimates
      exp(scale q.k).  Every cluster and subcluster g keeps the fixed-size
      sum Z_g = sum over its members of phi(sqrt(scale) k) (m numbers), and
      in this mode an unchosen group's estimated mass is phi(sqrt(scale) q).Z_g
      instead of the Gaussian exp(score); its value estimate stays the mean
      value, and the merge is the same.  Selection is unchanged.  Folded
      tokens add their features to both groups' sums.
      The page estimates the left-out numerator from the summary as well:
      with the per-group value summary Z^v_g = sum over the members of
      phi(sqrt(scale) k) v^T (m x d numbers), a left-out group adds
      phi(sqrt(scale) q).Z^v_g to the numerator and phi(sqrt(scale) q).Z_g to
      the denominator (``feature_numerator``).  The oracle implements both
      numerator models; the library implements the mean-value one (a value
      summary holds m*d floats per group, more than the group's rows at the
      workloads' group sizes).
  R18 Storage precision of the group statistics at decode time (not fixed
      by the pages): the decode reads every group's mean key, variance and
      mean value rounded to bfloat16 (``decode_statistics``: float32, then
      round to nearest, ties to even, at 8 significant bits), the precision
      the cache's own keys and values are stored in.  Selections and
      residual terms are computed from those values; the build and the
      incremental updates (R15) keep the statistics at full precision.
      ``decode_unit`` itself takes whatever statistics the layout holds, so
      every property of the method is checked on exact statistics; the GPU
      parity tests hand it ``decode_statistics(L)``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

# ---------------------------------------------------------------------------
# SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
# generators", OOPSLA 2014; the stand-alone 64-bit generator as published by
# Vigna).  Written from its definition: add the golden gamma to the state,
# then a three-step xor-shift-multiply finaliser.
# ---------------------------------------------------------------------------

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15
_MIX1 = 0xBF58476D1CE4E5B9
_MIX2 = 0x94D049BB133111EB
# Multiplier that separates the per-cluster subcluster streams (an odd
# 64-bit constant; any odd constant would do, this one is fixed so the two
# implementations agree).
SUB_STREAM_MUL = 0xD1B54A32D192ED03


def splitmix64(state: int) -> tuple[int, int]:
    """Advance a SplitMix64 state once; return (new_state, 64-bit output)."""
    state = (state + GOLDEN_GAMMA) & MASK64
    z = state
    z = ((z ^ (z >> 30)) * _MIX1) & MASK64
    z = ((z ^ (z >> 27)) * _MIX2) & MASK64
    return state, z ^ (z >> 31)


def unit_state(seed: int, seq: int, kv_head: int, n_kv_heads: int) -> int:
    """PRNG state of one (sequence, KV head) unit (reading R3)."""
    return (seed ^ ((GOLDEN_GAMMA * (1 + seq * n_kv_heads + kv_head)) & MASK64)) & MASK64


def sub_state(ustate: int, cluster: int) -> int:
    """PRNG state of the subcluster k-means of one cluster (reading R4)."""
    return (ustate ^ ((SUB_STREAM_MUL * (cluster + 1)) & MASK64)) & MASK64


def forgy_ids(n: int, k: int, state: int) -> list[int]:
    """First k entries of a Fisher-Yates shuffle of [0, n) (Forgy init, R3).

    Step i draws r from SplitMix64, picks j = i + (r mod (n - i)) and swaps
    positions i and j; the value that lands in position i is the i-th id.
    """
    if not 0 <= k <= n:
        raise ValueError("need 0 <= k <= n")
    moved: dict[int, int] = {}
    out = []
    for i in range(k):
        state, r = splitmix64(state)
        j = i + r % (n - i)
        vi = moved.get(i, i)
        vj = moved.get(j, j)
        moved[i] = vj
        moved[j] = vi
        out.append(vj)
    return out


# ---------------------------------------------------------------------------
# Sizes (reading R1)
# ---------------------------------------------------------------------------


def ceil_sqrt(n: int) -> int:
    """Smallest integer r with r*r >= n."""
    r = math.isqrt(n)
    return r if r * r == n else r + 1


def ceil_log2(n: int) -> int:
    """Smallest integer e with 2**e >= n."""
    return (n - 1).bit_length() if n > 1 else 0


def unit_dims(N: int, n_sink: int, n_recent: int) -> tuple[int, int, int]:
    """(N_mid, C, S) for one sequence of total length N."""
    n_mid = N - n_sink - n_recent
    if n_mid < 1:
        raise ValueError("the middle region must hold at least one key")
    C = min(ceil_sqrt(N), n_mid)
    S = max(1, ceil_log2(N))
    return n_mid, C, S


# ---------------------------------------------------------------------------
# Lloyd k-means (readings R3, R4)
# ---------------------------------------------------------------------------


def nearest_centroid(X: np.ndarray, mu: np.ndarray, chunk: int = 32768) -> np.ndarray:
    """argmin_j ||x - mu_j||^2 per row; the lowest j wins a tie.

    ||x - mu_j||^2 = ||x||^2 - 2 x.mu_j + ||mu_j||^2 and the first term does
    not depend on j, so the argmin is taken over ||mu_j||^2 - 2 x.mu_j.
    np.argmin returns the first minimum, i.e. the lowest j.
    """
    mu2 = np.einsum("jd,jd->j", mu, mu)
    out = np.empty(X.shape[0], dtype=np.int64)
    for r0 in range(0, X.shape[0], chunk):
        d = mu2[None, :] - 2.0 * (X[r0:r0 + chunk] @ mu.T)
        out[r0:r0 + chunk] = np.argmin(d, axis=1)
    return out


def centroid_sse(X: np.ndarray, mu: np.ndarray, a: np.ndarray) -> float:
    """sum_x ||x - mu_{a(x)}||^2."""
    diff = X - mu[a]
    return float(np.einsum("nd,nd->", diff, diff))


def partition_sse(X: np.ndarray, labels: np.ndarray) -> float:
    """k-means objective of a partition: sum over groups of the squared
    distances of the members to their group mean.

    The rows are sorted by label so that each group is one contiguous block;
    a block's mean is its sum divided by its size, and every member's
    deviation from it is squared and added up.
    """
    X = np.asarray(X, dtype=np.float64)
    labels = np.asarray(labels)
    if labels.size == 0:
        return 0.0
    order = np.argsort(labels, kind="stable")
    lab = labels[order]
    Xs = X[order]
    starts = np.flatnonzero(np.r_[True, lab[1:] != lab[:-1]])
    counts = np.diff(np.r_[starts, lab.size])
    means = np.add.reduceat(Xs, starts, axis=0) / counts[:, None]
    dev = Xs - np.repeat(means, counts, axis=0)
    return float(np.einsum("nd,nd->", dev, dev))


def _recenter(X: np.ndarray, a: np.ndarray, mu_old: np.ndarray) -> np.ndarray:
    """New centroid = mean of its members; an empty cluster keeps its old one."""
    k, d = mu_old.shape
    counts = np.bincount(a, minlength=k)
    sums = np.empty((k, d))
    for i in range(d):
        sums[:, i] = np.bincount(a, weights=X[:, i], minlength=k)
    mu = mu_old.copy()
    nz = counts > 0
    mu[nz] = sums[nz] / counts[nz, None]
    return mu


def lloyd(X: np.ndarray, mu0: np.ndarray, iters: int):
    """T rounds of (assign, update), then one final assign.

    Returns (final assignment, centroids used by the final assign, objective
    trace).  The trace holds, per round, J(a_t, mu_t) and J(a_t, mu_{t+1}),
    then J(a_final, mu_T); for Lloyd's method it never increases.
    """
    mu = np.array(mu0, dtype=np.float64, copy=True)
    trace = []
    for _ in range(iters):
        a = nearest_centroid(X, mu)
        trace.append(centroid_sse(X, mu, a))
        mu = _recenter(X, a, mu)
        trace.append(centroid_sse(X, mu, a))
    a = nearest_centroid(X, mu)
    trace.append(centroid_sse(X, mu, a))
    return a, mu, trace


# ---------------------------------------------------------------------------
# Gaussian summaries (reading R5) and the layout
# ---------------------------------------------------------------------------


def group_stats(Kg: np.ndarray, Vg: np.ndarray):
    """(n, mu, s, vbar) of one group: mean key, population diagonal variance
    (two passes: mean first, then mean squared deviation), mean value."""
    n = Kg.shape[0]
    mu = Kg.mean(axis=0)
    s = ((Kg - mu) ** 2).mean(axis=0)
    vbar = Vg.mean(axis=0)
    return n, mu, s, vbar


@dataclass
class UnitLayout:
    """Cluster layout of one (sequence, KV head).

    Rows of the middle region are ordered by (cluster, subcluster, original
    position).  ``perm[r]`` is the original token position of row r;
    subcluster i of cluster j owns rows [sub_off[j*S+i], sub_off[j*S+i+1]).
    Statistics are stored in float32, as the device keeps them.
    """

    N: int
    n_sink: int
    n_recent: int
    C: int
    S: int
    perm: np.ndarray
    sub_off: np.ndarray
    cl_mu: np.ndarray
    cl_var: np.ndarray
    cl_vbar: np.ndarray
    sub_mu: np.ndarray
    sub_var: np.ndarray
    sub_vbar: np.ndarray
    init_ids: list = field(default_factory=list)
    sub_init_ids: dict = field(default_factory=dict)
    sse_trace: list = field(default_factory=list)
    # tokens folded into the middle region after the build (reading R15):
    # their positions and global subcluster ids, oldest first
    fold_pos: list = field(default_factory=list)
    fold_sub: list = field(default_factory=list)
    # feature-map summaries (reading R16), float32: the map's W [m][d], its
    # scale, and per group the feature sums [C][m] and [C*S][m]; None if absent
    fm_w: np.ndarray = None
    fm_scale: float = None
    cl_z: np.ndarray = None
    sub_z: np.ndarray = None
    # value summaries of the feature-map numerator, float32 [C][m][d] and
    # [C*S][m][d] (sums of phi(sqrt(scale) k) v^T); None if absent
    cl_zv: np.ndarray = None
    sub_zv: np.ndarray = None

    @property
    def n_mid(self) -> int:
        return self.N - self.n_sink - self.n_recent

    @property
    def sub_count(self) -> np.ndarray:
        cnt = np.diff(self.sub_off)
        if self.fold_sub:
            cnt = cnt + np.bincount(np.asarray(self.fold_sub, np.int64), minlength=self.C * self.S)
        return cnt

    @property
    def cl_count(self) -> np.ndarray:
        sc = self.sub_count
        return np.add.reduceat(sc, np.arange(0, self.C * self.S, self.S))

    def group_rows(self, g: int) -> np.ndarray:
        """Token positions of subcluster g: its reordered rows, then the
        tokens folded into it."""
        rows = self.perm[self.sub_off[g]:self.sub_off[g + 1]]
        if self.fold_sub:
            extra = [p for p, q in zip(self.fold_pos, self.fold_sub) if q == g]
            if extra:
                rows = np.concatenate([rows, np.asarray(extra, dtype=rows.dtype)])
        return rows

    def cluster_labels(self) -> np.ndarray:
        """Cluster id of each middle-region key, indexed by position - n_sink."""
        lab = np.empty(self.n_mid, dtype=np.int64)
        for j in range(self.C):
            rows = self.perm[self.sub_off[j * self.S]:self.sub_off[(j + 1) * self.S]]
            lab[rows - self.n_sink] = j
        return lab

    def subcluster_labels(self) -> np.ndarray:
        """Global subcluster id (j*S+i) of each middle-region key."""
        lab = np.empty(self.n_mid, dtype=np.int64)
        for g in range(self.C * self.S):
            rows = self.perm[self.sub_off[g]:self.sub_off[g + 1]]
            lab[rows - self.n_sink] = g
        return lab


def layout_from_assignment(K, V, n_sink, n_recent, C, S, cl_assign, sub_assign):
    """Order the middle region by (cluster, subcluster, position) and compute
    the Gaussian summaries of every cluster and subcluster (reading R5).

    ``cl_assign`` / ``sub_assign`` are indexed by middle-local position
    (token position minus n_sink); ``sub_assign`` holds ids in [0, S).
    """
    N, d = K.shape
    n_mid = N - n_sink - n_recent
    cl_assign = np.asarray(cl_assign, dtype=np.int64)
    sub_assign = np.asarray(sub_assign, dtype=np.int64)
    assert cl_assign.shape == (n_mid,) and sub_assign.shape == (n_mid,)
    assert cl_assign.min(initial=0) >= 0 and cl_assign.max(initial=0) < C
    assert sub_assign.min(initial=0) >= 0 and sub_assign.max(initial=0) < S
    local = np.arange(n_mid)
    order = np.lexsort((local, sub_assign, cl_assign))
    perm = (order + n_sink).astype(np.int64)
    group = cl_assign * S + sub_assign
    counts = np.bincount(group, minlength=C * S)
    sub_off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)

    Km = K[n_sink:N - n_recent]
    Vm = V[n_sink:N - n_recent]
    cl = [np.zeros((C, d), np.float32) for _ in range(3)]
    sb = [np.zeros((C * S, d), np.float32) for _ in range(3)]
    for j in range(C):
        idx = cl_assign == j
        if idx.any():
            _, mu, s, vb = group_stats(Km[idx], Vm[idx])
            cl[0][j], cl[1][j], cl[2][j] = mu, s, vb
    for g in range(C * S):
        if counts[g]:
            rows = order[sub_off[g]:sub_off[g + 1]]
            _, mu, s, vb = group_stats(Km[rows], Vm[rows])
            sb[0][g], sb[1][g], sb[2][g] = mu, s, vb
    return UnitLayout(N=N, n_sink=n_sink, n_recent=n_recent, C=C, S=S,
                      perm=perm, sub_off=sub_off,
                      cl_mu=cl[0], cl_var=cl[1], cl_vbar=cl[2],
                      sub_mu=sb[0], sub_var=sb[1], sub_vbar=sb[2])


def build_unit(K, V, n_sink, n_recent, iters, state, init_ids=None, sub_init_ids=None):
    """Prefill-side build of one (sequence, KV head) (page 1, abstract:
    hierarchical partition of the keys, one Gaussian per group).

    K, V: float64 [N][d], the whole sequence.  ``init_ids`` (middle-local
    positions) and ``sub_init_ids`` ({cluster: middle-local positions})
    override the seeded Forgy draws; the ones actually used are returned in
    the layout so a test can replay them.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    N = K.shape[0]
    n_mid, C, S = unit_dims(N, n_sink, n_recent)
    X = K[n_sink:N - n_recent]
    if init_ids is None:
        init_ids = forgy_ids(n_mid, C, state)
    init_ids = [int(i) for i in init_ids]
    cl_assign, _, trace = lloyd(X, X[init_ids], iters)

    sub_assign = np.zeros(n_mid, dtype=np.int64)
    used_sub_init = {}
    for j in range(C):
        members = np.nonzero(cl_assign == j)[0]  # ascending position
        n_j = members.size
        if n_j == 0:
            continue
        k_j = min(S, n_j)
        if sub_init_ids is not None and j in sub_init_ids:
            where = {int(m): p for p, m in enumerate(members)}
            local = [where[int(m)] for m in sub_init_ids[j]]
        else:
            local = forgy_ids(n_j, k_j, sub_state(state, j))
        used_sub_init[j] = [int(members[p]) for p in local]
        Xj = X[members]
        sa, _, _ = lloyd(Xj, Xj[local], iters)
        sub_assign[members] = sa
    lay = layout_from_assignment(K, V, n_sink, n_recent, C, S, cl_assign, sub_assign)
    lay.init_ids = init_ids
    lay.sub_init_ids = used_sub_init
    lay.sse_trace = trace
    return lay


# ---------------------------------------------------------------------------
# Incremental decode (reading R15)
# ---------------------------------------------------------------------------


def _welford_add(n, mu, var, vbar, k, v):
    """Running update of (mean key, population variance, mean value) of a
    group of n members by one more member (k, v): Welford's formulas,
    computed in float64 from the stored float32 values, stored float32."""
    n1 = n + 1
    mu = np.asarray(mu, np.float64)
    delta = k - mu
    mu1 = mu + delta / n1
    var1 = (n * np.asarray(var, np.float64) + delta * (k - mu1)) / n1
    vbar1 = np.asarray(vbar, np.float64) + (v - np.asarray(vbar, np.float64)) / n1
    return mu1.astype(np.float32), var1.astype(np.float32), vbar1.astype(np.float32)


def fold_tokens(L: UnitLayout, K, V, n_new: int) -> UnitLayout:
    """The layout after the sequence grew by n_new tokens (K, V: float64
    [N + n_new][d] of the grown sequence): the n_new tokens that leave the
    recent window join the middle region as in reading R15.  Returns a new
    layout; ``L`` is unchanged."""
    import copy
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    out = copy.deepcopy(L)
    C, S = out.C, out.S
    for t in range(L.N - L.n_recent, L.N - L.n_recent + n_new):
        k, v = K[t], V[t]
        d2 = ((out.cl_mu.astype(np.float64) - k) ** 2).sum(axis=1)
        d2 = np.where(out.cl_count > 0, d2, np.inf)
        j = int(np.argmin(d2))  # first minimum: ties to the lower id
        cnt = out.sub_count[j * S:(j + 1) * S]
        ds = ((out.sub_mu[j * S:(j + 1) * S].astype(np.float64) - k) ** 2).sum(axis=1)
        i = int(np.argmin(np.where(cnt > 0, ds, np.inf)))
        g = j * S + i
        ncl, nsub = int(out.cl_count[j]), int(cnt[i])
        out.cl_mu[j], out.cl_var[j], out.cl_vbar[j] = _welford_add(ncl, out.cl_mu[j], out.cl_var[j], out.cl_vbar[j], k, v)
        out.sub_mu[g], out.sub_var[g], out.sub_vbar[g] = _welford_add(nsub, out.sub_mu[g], out.sub_var[g],
                                                                      out.sub_vbar[g], k, v)
        if out.cl_z is not None:
            ph = positive_features(math.sqrt(out.fm_scale) * k, out.fm_w)[0]
            out.cl_z[j] = (out.cl_z[j].astype(np.float64) + ph).astype(np.float32)
            out.sub_z[g] = (out.sub_z[g].astype(np.float64) + ph).astype(np.float32)
            if out.cl_zv is not None:
                pv = np.outer(ph, v)
                out.cl_zv[j] = (out.cl_zv[j].astype(np.float64) + pv).astype(np.float32)
                out.sub_zv[g] = (out.sub_zv[g].astype(np.float64) + pv).astype(np.float32)
        out.fold_pos.append(t)
        out.fold_sub.append(g)
    out.N = L.N + n_new
    return out


# ---------------------------------------------------------------------------
# Feature-map summaries (reading R16)
# ---------------------------------------------------------------------------


def positive_features(X, W):
    """phi(x) = exp(W x - |x|^2 / 2) / sqrt(m) for every row x of X: the
    positive random features of the softmax kernel (for rows of W drawn from
    N(0, I), E[phi(x).phi(y)] = exp(x.y))."""
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    W = np.asarray(W, dtype=np.float64)
    m = W.shape[0]
    return np.exp(X @ W.T - 0.5 * (X * X).sum(axis=1, keepdims=True)) / math.sqrt(m)


def with_feature_summaries(L: UnitLayout, K, W, scale=None, V=None) -> UnitLayout:
    """A copy of ``L`` holding, for every cluster and subcluster, the sum of
    phi(sqrt(scale) k) over its members (reordered rows and folded tokens),
    computed in float64 and stored float32; with the values V also the value
    summaries, the sums of phi(sqrt(scale) k) v^T."""
    import copy
    K = np.asarray(K, dtype=np.float64)
    W = np.asarray(W, dtype=np.float32)
    d = K.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = copy.deepcopy(L)
    m = W.shape[0]
    with_v = V is not None
    if with_v:
        V = np.asarray(V, dtype=np.float64)
    sub_z = np.zeros((L.C * L.S, m))
    sub_zv = np.zeros((L.C * L.S, m, V.shape[1]), np.float32) if with_v else None
    for g in range(L.C * L.S):
        rows = L.group_rows(g)
        if rows.size:
            ph = positive_features(math.sqrt(scale) * K[rows], W)
            sub_z[g] = ph.sum(axis=0)
            if with_v:
                sub_zv[g] = ph.T @ V[rows]
    cl_z = np.zeros((L.C, m))
    cl_zv = np.zeros((L.C, m, V.shape[1]), np.float32) if with_v else None
    for j in range(L.C):
        rows = np.concatenate([L.group_rows(j * L.S + i) for i in range(L.S)])
        if rows.size:
            ph = positive_features(math.sqrt(scale) * K[rows], W)
            cl_z[j] = ph.sum(axis=0)
            if with_v:
                cl_zv[j] = ph.T @ V[rows]
    out.fm_w, out.fm_scale = W, float(scale)
    out.cl_z, out.sub_z = cl_z.astype(np.float32), sub_z.astype(np.float32)
    out.cl_zv, out.sub_zv = cl_zv, sub_zv
    return out


def fm_log_mass(q, Z, W, scale):
    """ln(phi(sqrt(scale) q).Z_g) for every row Z_g of Z (-inf where the
    estimate is 0): the feature-map estimate of sum exp(scale q.k) over the
    group's members."""
    ph = positive_features(math.sqrt(scale) * np.asarray(q, np.float64), W)[0]
    mass = np.asarray(Z, np.float64) @ ph
    with np.errstate(divide="ignore"):
        return np.where(mass > 0, np.log(np.maximum(mass, 1e-300)), -np.inf)


# ---------------------------------------------------------------------------
# Decode (readings R6-R8; merge rule from page 4's abstract)
# ---------------------------------------------------------------------------


def bf16_round(x) -> np.ndarray:
    """x rounded to bfloat16, returned as float64 (reading R18).  bfloat16
    keeps float32's sign and 8 exponent bits and the top 7 of its 23
    fraction bits, so the value is first stored as float32 and the float32
    bit pattern is then rounded at bit 16: add half of that unit minus one,
    plus the kept lowest bit (round half to even), and clear the low 16
    bits.  A carry out of the fraction steps the exponent, which also sends
    values past the largest bfloat16 to infinity; NaN stays NaN."""
    f = np.atleast_1d(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    r = (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32)
    out = r.view(np.float32).astype(np.float64)
    out[np.isnan(f)] = np.nan
    return out.reshape(np.shape(x))


def decode_statistics(L: UnitLayout) -> UnitLayout:
    """The layout as the decode reads it (reading R18): cluster and
    subcluster mean keys, variances and mean values rounded to bfloat16.
    Counts, offsets, folded-token bookkeeping and feature sums are kept."""
    return replace(L, cl_mu=bf16_round(L.cl_mu), cl_var=bf16_round(L.cl_var), cl_vbar=bf16_round(L.cl_vbar),
                   sub_mu=bf16_round(L.sub_mu), sub_var=bf16_round(L.sub_var), sub_vbar=bf16_round(L.sub_vbar))


def group_log_mass(q, count, mu, var, scale):
    """Score of each group: ln n + scale q.mu + scale^2/2 sum_i q_i^2 var_i.

    exp(score) = n * E[exp(scale q.k)] for k ~ N(mu, diag var): the estimated
    unnormalised softmax mass of the group (reading R6).  Empty groups score
    -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    count = np.asarray(count)
    mu = np.asarray(mu, dtype=np.float64)
    var = np.asarray(var, dtype=np.float64)
    with np.errstate(divide="ignore"):
        lnn = np.where(count > 0, np.log(np.maximum(count, 1)), -np.inf)
    return lnn + scale * (mu @ q) + 0.5 * scale * scale * (var @ (q * q))


def top_by_score(scores, k, valid):
    """The k highest-scoring valid entries, ties to the lower index, returned
    in ascending index order (reading R7)."""
    idx = np.nonzero(valid)[0]
    if k <= 0 or idx.size == 0:
        return np.zeros(0, dtype=np.int64)
    order = idx[np.lexsort((idx, -np.asarray(scores)[idx]))]
    return np.sort(order[:k])


def _softmax_merge(logw, vals):
    """Single normalisation of unnormalised terms exp(logw_i) * vals_i, with a
    max shift (mathematically the same as the plain quotient)."""
    m = np.max(logw)
    w = np.exp(logw - m)
    den = w.sum()
    return (w @ vals) / den, m + np.log(den)


def shared_selection(L: UnitLayout, Q, top_c, top_s, scale=None):
    """One selection for all query heads of a KV head (reading R14): returns
    (chosen cluster ids ascending, [chosen subcluster ids ascending per chosen
    cluster]) and the per-cluster group scores."""
    Q = np.atleast_2d(np.asarray(Q, dtype=np.float64))
    G, d = Q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    C, S = L.C, L.S
    cl_cnt, sub_cnt = L.cl_count, L.sub_count
    valid = cl_cnt > 0
    sc = np.stack([group_log_mass(Q[h], cl_cnt, L.cl_mu, L.cl_var, scale) for h in range(G)])
    lse = np.array([np.logaddexp.reduce(sc[h][valid]) for h in range(G)])
    gs = np.where(valid, np.exp(sc - lse[:, None]).sum(axis=0), 0.0)
    chosen = top_by_score(gs, top_c, valid)
    picks = []
    for j in chosen:
        g0 = j * S
        sv = sub_cnt[g0:g0 + S] > 0
        ss = np.stack([group_log_mass(Q[h], sub_cnt[g0:g0 + S], L.sub_mu[g0:g0 + S], L.sub_var[g0:g0 + S], scale)
                       for h in range(G)])
        gss = np.where(sv, np.exp(ss - lse[:, None]).sum(axis=0), 0.0)
        picks.append(top_by_score(gss, top_s, sv))
    return chosen, picks, gs


def decode_unit(L: UnitLayout, K, V, Q, top_c, top_s, scale=None, residual=True,
                sel_override=None, shared=False, feature_residual=False, feature_numerator=False):
    """One decode step for the query heads that share one KV head.

    K, V: float64 [N][d] of the sequence (anchors are read from here, the
    middle rows through ``L.perm``).  Q: [G][d].  Returns a dict with
    ``out``/``lse`` (exact + residual, one normalisation), ``out_top`` /
    ``lse_top`` (exact part only, renormalised), ``sel_c`` (per head, chosen
    cluster ids ascending), ``sel_s`` (per head, per chosen cluster, chosen
    subcluster ids ascending) and ``n_exact`` (rows attended exactly per head).
    ``sel_override`` = (sel_c, sel_s) replaces the selection; ``shared``
    takes the one selection of reading R14 for every head;
    ``feature_residual`` estimates the left-out groups' masses from the
    layout's feature-map summaries (reading R16) instead of exp(score);
    ``feature_numerator`` (with it) also takes their numerators from the
    value summaries, phi(sqrt(scale) q).Z^v_g, instead of mass times the mean
    value.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Q = np.atleast_2d(np.asarray(Q, dtype=np.float64))
    G, d = Q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    N, C, S = L.N, L.C, L.S
    anchors = np.concatenate([np.arange(L.n_sink), np.arange(N - L.n_recent, N)])
    cl_cnt = L.cl_count
    sub_cnt = L.sub_count

    res = dict(out=np.zeros((G, d)), lse=np.zeros(G), out_top=np.zeros((G, d)),
               lse_top=np.zeros(G), sel_c=[], sel_s=[], n_exact=np.zeros(G, np.int64))
    if shared and sel_override is None:
        ch, pk, _ = shared_selection(L, Q, top_c, top_s, scale)
        sel_override = ([ch] * G, [pk] * G)
    if feature_residual and (L.cl_z is None or not np.isclose(L.fm_scale, scale)):
        raise ValueError("feature-map residual needs summaries built with the decode scale")
    if feature_numerator and (not feature_residual or L.cl_zv is None):
        raise ValueError("the feature-map numerator needs feature_residual and value summaries")
    for h in range(G):
        q = Q[h]
        sc = group_log_mass(q, cl_cnt, L.cl_mu, L.cl_var, scale)
        # the residual's log-mass of every cluster / subcluster, and the value
        # estimate of a left-out group: its mean value, or (feature-map
        # numerator) phi.Z^v_g / phi.Z_g, so that mass * value = phi.Z^v_g
        r_cl = fm_log_mass(q, L.cl_z, L.fm_w, scale) if feature_residual else sc
        if feature_numerator:
            ph_q = positive_features(math.sqrt(scale) * q, L.fm_w)[0]

            def group_value(zv, z):
                return (ph_q @ zv.astype(np.float64)) / float(ph_q @ z.astype(np.float64))
        if sel_override is not None:
            chosen = np.asarray(sel_override[0][h], dtype=np.int64)
        else:
            chosen = top_by_score(sc, top_c, cl_cnt > 0)
        exact_rows = [anchors]
        r_logw, r_vals = [], []
        chosen_set = set(int(j) for j in chosen)
        for j in range(C):
            if cl_cnt[j] > 0 and j not in chosen_set:
                r_logw.append(r_cl[j])
                r_vals.append(group_value(L.cl_zv[j], L.cl_z[j]) if feature_numerator
                              else L.cl_vbar[j].astype(np.float64))
        sel_s_h = []
        for jj, j in enumerate(chosen):
            g0 = j * S
            ss = group_log_mass(q, sub_cnt[g0:g0 + S], L.sub_mu[g0:g0 + S],
                                L.sub_var[g0:g0 + S], scale)
            if sel_override is not None:
                picks = np.asarray(sel_override[1][h][jj], dtype=np.int64)
            else:
                picks = top_by_score(ss, top_s, sub_cnt[g0:g0 + S] > 0)
            sel_s_h.append(picks)
            pick_set = set(int(i) for i in picks)
            r_sub = fm_log_mass(q, L.sub_z[g0:g0 + S], L.fm_w, scale) if feature_residual else ss
            for i in range(S):
                g = g0 + i
                if sub_cnt[g] == 0:
                    continue
                if i in pick_set:
                    exact_rows.append(L.group_rows(g))
                else:
                    r_logw.append(r_sub[i])
                    r_vals.append(group_value(L.sub_zv[g], L.sub_z[g]) if feature_numerator
                                  else L.sub_vbar[g].astype(np.float64))
        rows = np.concatenate(exact_rows)
        e_logw = scale * (K[rows] @ q)
        e_vals = V[rows]
        res["out_top"][h], res["lse_top"][h] = _softmax_merge(e_logw, e_vals)
        if residual and r_logw:
            logw = np.concatenate([e_logw, np.asarray(r_logw)])
            vals = np.concatenate([e_vals, np.asarray(r_vals)])
            res["out"][h], res["lse"][h] = _softmax_merge(logw, vals)
        else:
            res["out"][h], res["lse"][h] = res["out_top"][h], res["lse_top"][h]
        res["sel_c"].append(np.asarray(chosen, dtype=np.int64))
        res["sel_s"].append(sel_s_h)
        res["n_exact"][h] = rows.size
    return res


def dense_attention(K, V, Q, scale=None):
    """Exact softmax attention of each query row over all N keys:
    out = softmax(scale K q)^T V.  Returns (out [G][d], lse [G])."""
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Q = np.atleast_2d(np.asarray(Q, dtype=np.float64))
    if scale is None:
        scale = 1.0 / math.sqrt(Q.shape[1])
    logits = scale * (Q @ K.T)
    m = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - m)
    den = w.sum(axis=1)
    return (w @ V) / den[:, None], m[:, 0] + np.log(den)


# ---------------------------------------------------------------------------
# Batched drivers: [n_seq][H][N][d] arrays, one layout per (seq, KV head)
# ---------------------------------------------------------------------------


def decode_batch(layouts, K, V, Q, n_kv_heads, top_c, top_s, scale=None,
                 residual=True, units=None, shared=False):
    """Decode every (or the listed) (seq, KV head) unit.

    ``layouts[u]`` with u = seq * n_kv_heads + kv_head; ``K[seq][kvh]`` and
    ``V[seq][kvh]`` are [N_seq][d]; ``Q[seq]`` is [Hq][d]; ``top_c`` /
    ``top_s`` are per-sequence sequences of ints.  Query head h reads KV head
    h // G.  Returns {u: decode_unit result}.
    """
    out = {}
    n_seq = len(Q)
    for seq in range(n_seq):
        Hq = Q[seq].shape[0]
        G = Hq // n_kv_heads
        for kvh in range(n_kv_heads):
            u = seq * n_kv_heads + kvh
            if units is not None and u not in units:
                continue
            out[u] = decode_unit(layouts[u], K[seq][kvh], V[seq][kvh],
                                 Q[seq][kvh * G:(kvh + 1) * G], top_c[seq], top_s[seq],
                                 scale=scale, residual=residual, shared=shared)
    return out


def dense_batch(K, V, Q, n_kv_heads, scale=None):
    """Dense attention for every sequence and query head; returns lists of
    (out [Hq][d], lse [Hq]) per sequence."""
    res = []
    for seq in range(len(Q)):
        Hq = Q[seq].shape[0]
        G = Hq // n_kv_heads
        outs, lses = [], []
        for kvh in range(n_kv_heads):
            o, l = dense_attention(K[seq][kvh], V[seq][kvh], Q[seq][kvh * G:(kvh + 1) * G], scale)
            outs.append(o)
            lses.append(l)
        res.append((np.concatenate(outs), np.concatenate(lses)))
    return res
