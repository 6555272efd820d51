"""CPU study (oracle only): where the approximation error against dense
attention comes from, and how the exact budget is best split between
clusters (c) and subclusters per cluster (s).

For each workload, each s from S (whole clusters) down to 1 takes the
largest c whose mean per-head exact read stays within 5% of the sequence
(selection only), then decodes with the oracle and reports, per query head
(mean over heads and query sets):
  * err_res / err_top: relative L2 error against dense attention with the
    Gaussian residual / with the exact part only;
  * missed: the share of the true attention mass (denominator) outside the
    exactly attended rows;
  * est/true: the residual's estimate of that left-out mass over its true
    value (1 is exact).

    python tests/studies/budget_split.py [workload ...]   (1, 2, 3, 4h, 4m)
"""

import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
from long_context_sparse_mog_amd import synth  # noqa: E402

WORKLOADS = {
    # name: (config, overrides, KV heads studied)
    "1": (1, {}, (0, 1)),
    "2": (2, {"n_seq": 1, "seq_lens": [131072], "top_c": [18], "top_s": [5]}, (0,)),
    "3": (3, {}, (0,)),
    "4m": (4, {"seq_lens": [65536]}, (0,)),
    "4h": (4, {"seq_lens": [65536]}, (4,)),
}


def exact_rows(L, chosen, picks):
    anchors = np.concatenate([np.arange(L.n_sink), np.arange(L.N - L.n_recent, L.N)])
    parts = [anchors]
    for j, pk in zip(chosen, picks):
        for i in pk:
            parts.append(L.group_rows(j * L.S + int(i)))
    return np.concatenate(parts)


def selection(L, q, c, s, scale):
    sc = O.group_log_mass(q, L.cl_count, L.cl_mu, L.cl_var, scale)
    chosen = O.top_by_score(sc, c, L.cl_count > 0)
    picks = []
    for j in chosen:
        g0 = j * L.S
        ss = O.group_log_mass(q, L.sub_count[g0:g0 + L.S], L.sub_mu[g0:g0 + L.S], L.sub_var[g0:g0 + L.S], scale)
        picks.append(O.top_by_score(ss, s, L.sub_count[g0:g0 + L.S] > 0))
    return chosen, picks


def main():
    names = sys.argv[1:] or list(WORKLOADS)
    n_q = 4
    print("| workload | s | c | read per head | err_res | err_top | missed | est/true |")
    print("|---|---|---|---|---|---|---|---|")
    for name in names:
        cfg, over, heads = WORKLOADS[name]
        wl = synth.config(cfg, **over)
        b = synth.generate(wl, device="cpu", n_qsets=n_q)
        N, G, d = wl.seq_lens[0], wl.group, wl.head_dim
        scale = 1.0 / math.sqrt(d)
        t0 = time.time()
        units = []
        for h in heads:
            K, V = b.unit_kv(0, h)
            L = O.build_unit(K, V, wl.n_sink, wl.n_recent, wl.kmeans_iters, O.unit_state(1, 0, h, wl.n_kv_heads))
            Qs = [b.Q[t, 0, h * G:(h + 1) * G].numpy().astype(np.float64) for t in range(n_q)]
            units.append((K, V, L, Qs))
        print(f"<!-- {wl.name}: built {len(units)} unit(s) in {time.time() - t0:.0f} s; "
              f"C = {L.C}, S = {L.S}, configured c = {wl.top_c[0]}, s = {wl.top_s[0]} -->", flush=True)
        S = units[0][2].S
        for s in sorted({S, max(1, S // 2), -(-S // 4), 2, 1}, reverse=True):
            # the largest c (geometric scan, then a bisection) whose mean
            # per-head read is within 5%
            def read(c):
                tot = 0.0
                n = 0
                for K, V, L, Qs in units:
                    for Q in Qs:
                        for q in Q:
                            ch, pk = selection(L, q, c, s, scale)
                            tot += exact_rows(L, ch, pk).size / L.N
                            n += 1
                return tot / n
            lo, hi = 0, 1
            while hi <= units[0][2].C and read(hi) <= 0.05:
                lo, hi = hi, 2 * hi
            hi = min(hi, units[0][2].C + 1)
            while hi - lo > 1:
                mid = (lo + hi) // 2
                if read(mid) <= 0.05:
                    lo = mid
                else:
                    hi = mid
            c = max(lo, 1)
            rows = []
            for K, V, L, Qs in units:
                for Q in Qs:
                    r = O.decode_unit(L, K, V, Q, c, s, scale=scale)
                    o, lse_all = O.dense_attention(K, V, Q, scale)
                    for g in range(G):
                        ch, pk = r["sel_c"][g], r["sel_s"][g]
                        E = exact_rows(L, ch, pk)
                        lse_e = float(np.logaddexp.reduce(scale * (K[E] @ Q[g])))
                        missed = 1.0 - math.exp(lse_e - lse_all[g])
                        true_r = math.exp(lse_all[g]) - math.exp(lse_e)
                        est_r = math.exp(r["lse"][g]) - math.exp(r["lse_top"][g])
                        rows.append((E.size / L.N,
                                     np.linalg.norm(r["out"][g] - o[g]) / np.linalg.norm(o[g]),
                                     np.linalg.norm(r["out_top"][g] - o[g]) / np.linalg.norm(o[g]),
                                     missed, est_r / true_r if true_r > 0 else float("nan")))
            a = np.array(rows)
            print(f"| {wl.name} | {s} | {c} | {a[:, 0].mean():.4f} | {a[:, 1].mean():.3f} | {a[:, 2].mean():.3f} | "
                  f"{a[:, 3].mean():.3f} | {np.median(a[:, 4]):.2f} |", flush=True)


if __name__ == "__main__":
    main()
