"""Seeded synthetic workloads for MoG decode attention.

This module only draws inputs: keys, values, queries, sequence lengths, page
tables and the per-sequence exact budgets of each workload.  It holds none of
the method's arithmetic and is the one piece of code that both the HIP path
(through ``bench.py`` and the GPU tests) and the CPU oracle (through the
tests) consume.  Draws use ``torch.Generator`` on the requested device, so a
workload generated on the GPU and its host copy are the same numbers.

The workloads stand in for the long-context benchmarks run on Qwen3-4B,
Olmo3-7B and Qwen3-14B that page 1 ("Iceberg Attention", abstract) reports;
those datasets and weights are not available, so each workload takes the
decode-layer shape of such a model and fills it with Gaussian-mixture keys.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

BASE_SEED = 20261202


def _isqrt_ceil(n: int) -> int:
    r = math.isqrt(n)
    return r if r * r == n else r + 1


def budget_for_length(L: int, n_sink: int, n_recent: int, frac: float = 0.05, kappa: float = 1.0,
                      split=None):
    """Per-query-head exact budget (top_c, top_s) for a length-L sequence.

    Average-size rule: s subclusters per chosen cluster (``split``: None for
    ceil(S/4), "whole" for all S, i.e. whole clusters, or a number) and c
    the largest count whose expected exact rows (anchors plus c*s
    average-sized subclusters) stay within frac*L.  The groups the log-mass
    score picks are larger than average (their score carries ln n), so a
    workload scales c by ``kappa``, chosen by decoding the workload's query
    sets on the GPU and reading the mean share of the sequence a query head
    attends exactly, so that it stays within frac.  The split of each
    workload is the one with the lowest error against dense attention at
    that read (measured on the GPU over the workload's query sets)."""
    C = _isqrt_ceil(L)
    S = max(1, (L - 1).bit_length())
    s = S if split == "whole" else (-(-S // 4) if split is None else min(int(split), S))
    n_mid = L - n_sink - n_recent
    per_sub = n_mid / (C * S)
    c = int(math.floor((frac * L - (n_sink + n_recent)) / (s * per_sub)))
    return max(int(math.floor(kappa * max(c, 1))), 1), s


@dataclass
class Workload:
    name: str
    n_seq: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seq_lens: list
    dtype: str                      # "fp32" or "bf16"
    n_sink: int
    n_recent: int
    top_c: list
    top_s: list
    n_components: int = 512
    uniform_weights: bool = False
    outlier_dims: int = 0
    needles: int = 0
    high_entropy_heads: tuple = ()  # KV heads with isotropic keys
    paged: bool = False
    page_size: int = 16
    plant_uniform: bool = False     # plant on a uniform middle token, not a component
    seed: int = BASE_SEED
    kmeans_iters: int = 10
    budget_kappa: float = 1.0       # scale of the average-size budget rule
    budget_split: object = None     # subclusters per chosen cluster: None (S/4), "whole" or a number
    notes: str = ""

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def max_len(self) -> int:
        return max(self.seq_lens)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    def kv_bytes(self) -> int:
        e = 4 if self.dtype == "fp32" else 2
        return 2 * e * self.head_dim * self.n_kv_heads * sum(self.seq_lens)


def config(i: int, **override) -> Workload:
    """The five workloads, by index; keyword overrides shrink them for tests."""
    if i == 0:
        wl = Workload(name="single-head-4K-fp32", n_seq=1, n_q_heads=1, n_kv_heads=1,
                      head_dim=64, seq_lens=[4096], dtype="fp32", n_sink=4, n_recent=64,
                      top_c=[4], top_s=[3], n_components=64, uniform_weights=True,
                      plant_uniform=True, seed=BASE_SEED + 0)
    elif i == 1:
        wl = Workload(name="gqa-32q8kv-d128-32K-bf16", n_seq=1, n_q_heads=32, n_kv_heads=8,
                      head_dim=128, seq_lens=[32768], dtype="bf16", n_sink=64, n_recent=256,
                      top_c=[4], top_s=[15], n_components=512, outlier_dims=2,
                      budget_kappa=4 / 7, budget_split="whole", seed=BASE_SEED + 1)
    elif i == 2:
        wl = Workload(name="mha-4x32h-d128-128K-bf16", n_seq=4, n_q_heads=32, n_kv_heads=32,
                      head_dim=128, seq_lens=[131072] * 4, dtype="bf16", n_sink=64,
                      n_recent=256, top_c=[38] * 4, top_s=[2] * 4, n_components=512,
                      outlier_dims=2, needles=16, budget_kappa=38 / 147, budget_split=2,
                      seed=BASE_SEED + 2)
    elif i == 3:
        wl = Workload(name="gqa-40q8kv-d128-1M-bf16", n_seq=1, n_q_heads=40, n_kv_heads=8,
                      head_dim=128, seq_lens=[1048576], dtype="bf16", n_sink=64, n_recent=256,
                      top_c=[17], top_s=[20], n_components=2048, outlier_dims=2,
                      budget_kappa=17 / 50, budget_split="whole", seed=BASE_SEED + 3)
    elif i == 4:
        rng = np.random.default_rng(BASE_SEED + 4)
        lens = [int(math.floor(math.exp(rng.uniform(math.log(8192), math.log(262144)))))
                for _ in range(16)]
        bud = [budget_for_length(L, 64, 256, kappa=0.7, split="whole") for L in lens]
        wl = Workload(name="ragged-16seq-8K-256K-paged-bf16", n_seq=16, n_q_heads=32,
                      n_kv_heads=8, head_dim=128, seq_lens=lens, dtype="bf16", n_sink=64,
                      n_recent=256, top_c=[b[0] for b in bud], top_s=[b[1] for b in bud],
                      n_components=512, outlier_dims=2, high_entropy_heads=(4, 5, 6, 7),
                      paged=True, page_size=16, budget_kappa=0.7, budget_split="whole",
                      seed=BASE_SEED + 4)
    else:
        raise ValueError(f"no workload {i}")
    if "seq_lens" in override:
        override.setdefault("n_seq", len(override["seq_lens"]))
        if "top_c" not in override:
            bud = [budget_for_length(L, override.get("n_sink", wl.n_sink),
                                     override.get("n_recent", wl.n_recent),
                                     kappa=override.get("budget_kappa", wl.budget_kappa),
                                     split=override.get("budget_split", wl.budget_split))
                   for L in override["seq_lens"]]
            override["top_c"] = [b[0] for b in bud]
            override["top_s"] = [b[1] for b in bud]
    return replace(wl, **override)


def build_workload():
    """The 128K-key single-head partition whose build time is reported:
    mixture keys as in the 32K GQA workload, d=128, bf16, 10 iterations."""
    return config(1, n_q_heads=1, n_kv_heads=1, seq_lens=[131072], top_c=[18], top_s=[5],
                  name="build-1head-128K-bf16", seed=BASE_SEED + 40)


# ---------------------------------------------------------------------------
# Drawing
# ---------------------------------------------------------------------------


def _unit_seed(base: int, seq: int, kvh: int) -> int:
    return (base * 1_000_003 + seq * 10_007 + kvh * 101 + 17) % (2 ** 62)


def _unit_draw(wl: Workload, seq: int, kvh: int, n_qsets: int, device):
    """Keys/values [L][d] (float32) and queries [n_qsets][G][d] of one unit."""
    L, d, G = wl.seq_lens[seq], wl.head_dim, wl.group
    g = torch.Generator(device=device)
    g.manual_seed(_unit_seed(wl.seed, seq, kvh))
    V = torch.randn(L, d, generator=g, device=device)
    lo, hi = wl.n_sink, L - wl.n_recent
    if kvh in wl.high_entropy_heads:
        K = torch.randn(L, d, generator=g, device=device)
        Q = 0.25 * torch.randn(n_qsets, G, d, generator=g, device=device)
        return K, V, Q
    m = wl.n_components
    cent = torch.randn(m, d, generator=g, device=device)
    if wl.uniform_weights:
        w = torch.full((m,), 1.0 / m, device=device)
    else:
        w = torch.exp(torch.randn(m, generator=g, device=device))
        w = w / w.sum()
    comp = torch.multinomial(w, L, replacement=True, generator=g)
    K = cent[comp] + 0.5 * torch.randn(L, d, generator=g, device=device)
    Q = torch.empty(n_qsets, G, d, device=device)
    if wl.needles:
        # needle keys k_i = r (0.8 u + 0.6 w_i), w_i a unit vector orthogonal
        # to u, r the median key norm; the query sqrt(d) u has cosine 0.8
        # with every needle.
        u = torch.randn(d, generator=g, device=device)
        u = u / u.norm()
        pos = lo + torch.randperm(hi - lo, generator=g, device=device)[:wl.needles]
        if wl.outlier_dims:
            dims = torch.randperm(d, generator=g, device=device)[:wl.outlier_dims]
            K[:, dims] *= 8.0
        r = K.norm(dim=1).median()
        wv = torch.randn(wl.needles, d, generator=g, device=device)
        wv = wv - (wv @ u)[:, None] * u[None, :]
        wv = wv / wv.norm(dim=1, keepdim=True)
        K[pos] = r * (0.8 * u[None, :] + 0.6 * wv)
        for t in range(n_qsets):
            if t == 0:
                qd = u
            else:  # other query sets: a small random tilt of u
                z = torch.randn(d, generator=g, device=device) * (0.15 / math.sqrt(d))
                qd = (u + z) / (u + z).norm()
            Q[t] = math.sqrt(d) * qd[None, :].expand(G, d)
        return K, V, Q
    # planted queries: each query head copies one middle-region key (before
    # the outlier scaling) and adds N(0, 0.1^2) noise.
    comp_mid = comp[lo:hi]
    for t in range(n_qsets):
        if wl.plant_uniform:
            toks = lo + torch.randint(0, hi - lo, (G,), generator=g, device=device)
        else:
            j = torch.multinomial(w, 1, generator=g)
            cand = torch.nonzero(comp_mid == j).flatten()
            if cand.numel() == 0:
                cand = torch.arange(hi - lo, device=device)
            pick = torch.randint(0, cand.numel(), (G,), generator=g, device=device)
            toks = lo + cand[pick]
        Q[t] = K[toks] + 0.1 * torch.randn(G, d, generator=g, device=device)
    if wl.outlier_dims:
        dims = torch.randperm(d, generator=g, device=device)[:wl.outlier_dims]
        K[:, dims] *= 8.0
    return K, V, Q


@dataclass
class Batch:
    wl: Workload
    K: torch.Tensor            # [n_seq][Hkv][max_len][d] storage dtype (rows >= len are zero)
    V: torch.Tensor
    Q: torch.Tensor            # [n_qsets][n_seq][Hq][d] float32
    pool_K: torch.Tensor = None   # paged: [n_pages][Hkv][page][d]
    pool_V: torch.Tensor = None
    block_table: torch.Tensor = None  # paged: [n_seq][max_blocks] int32
    extra: dict = field(default_factory=dict)

    def unit_kv(self, seq: int, kvh: int):
        """float64 NumPy copies of one unit's keys and values (as stored)."""
        L = self.wl.seq_lens[seq]
        k = self.K[seq, kvh, :L].float().cpu().numpy().astype(np.float64)
        v = self.V[seq, kvh, :L].float().cpu().numpy().astype(np.float64)
        return k, v


def generate(wl: Workload, device="cpu", n_qsets: int = 1, keep_contiguous: bool = True) -> Batch:
    """Draw the whole workload.  K/V are drawn in float32 and rounded to
    nearest-even bf16 for bf16 workloads."""
    d = wl.head_dim
    K = torch.zeros(wl.n_seq, wl.n_kv_heads, wl.max_len, d, dtype=wl.torch_dtype, device=device)
    V = torch.zeros_like(K)
    Q = torch.empty(n_qsets, wl.n_seq, wl.n_q_heads, d, dtype=torch.float32, device=device)
    G = wl.group
    for s in range(wl.n_seq):
        L = wl.seq_lens[s]
        for h in range(wl.n_kv_heads):
            k, v, q = _unit_draw(wl, s, h, n_qsets, device)
            K[s, h, :L] = k.to(wl.torch_dtype)
            V[s, h, :L] = v.to(wl.torch_dtype)
            Q[:, s, h * G:(h + 1) * G] = q
            del k, v
    b = Batch(wl=wl, K=K, V=V, Q=Q)
    if wl.paged:
        to_paged(b)
        if not keep_contiguous:
            b.K = b.V = None
    return b


def to_paged(b: Batch):
    """Scatter the contiguous cache into a page pool [n_pages][Hkv][page][d]
    whose physical page order is a seeded shuffle, plus the block table."""
    wl, P = b.wl, b.wl.page_size
    pages_per = [-(-L // P) for L in wl.seq_lens]
    n_pages = sum(pages_per)
    max_blocks = max(pages_per)
    rng = np.random.default_rng(wl.seed + 7)
    phys = rng.permutation(n_pages)
    bt = np.full((wl.n_seq, max_blocks), -1, dtype=np.int32)
    dev = b.K.device
    pool_K = torch.zeros(n_pages, wl.n_kv_heads, P, wl.head_dim, dtype=b.K.dtype, device=dev)
    pool_V = torch.zeros_like(pool_K)
    nxt = 0
    for s in range(wl.n_seq):
        n = pages_per[s]
        ids = phys[nxt:nxt + n]
        nxt += n
        bt[s, :n] = ids
        Lpad = n * P
        src_k = torch.zeros(wl.n_kv_heads, Lpad, wl.head_dim, dtype=b.K.dtype, device=dev)
        src_v = torch.zeros_like(src_k)
        L = wl.seq_lens[s]
        src_k[:, :L] = b.K[s, :, :L]
        src_v[:, :L] = b.V[s, :, :L]
        idx = torch.as_tensor(ids, device=dev, dtype=torch.long)
        pool_K[idx] = src_k.view(wl.n_kv_heads, n, P, wl.head_dim).transpose(0, 1)
        pool_V[idx] = src_v.view(wl.n_kv_heads, n, P, wl.head_dim).transpose(0, 1)
    b.pool_K, b.pool_V = pool_K, pool_V
    b.block_table = torch.as_tensor(bt, device=dev)
    return b


def feature_map_w(m: int, d: int, seed: int = BASE_SEED + 99, device="cpu") -> torch.Tensor:
    """A seeded float32 [m][d] projection with N(0, 1) entries (the random
    draws of the feature-map summaries; both the library and the oracle take
    it as an input)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randn(m, d, generator=g).to(device)
