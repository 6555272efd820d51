"""CPU study (oracle only): how the left-out part of the cache is estimated.

On the ragged workload's two kinds of KV heads (mixture keys, and isotropic
keys with near-uniform attention), at one sequence length, the per-head
relative L2 error against dense attention of the decode output with
  * the Gaussian residual (mass exp(score), value the mean value),
  * the feature-map mass with the mean value,
  * the feature-map mass and the feature-map numerator (value summaries),
  * no residual (the exact part only, renormalised),
for m positive random features.  Also the memory of each summary per head.

    python tests/studies/residual_models.py [length] [m ...]
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


def rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def main():
    L = int(sys.argv[1]) if len(sys.argv) > 1 else 8192
    ms = [int(x) for x in sys.argv[2:]] or [128, 1024]
    wl = synth.config(4, seq_lens=[L])
    b = synth.generate(wl, device="cpu", n_qsets=4)
    c, s = wl.top_c[0], wl.top_s[0]
    G, d = wl.group, wl.head_dim
    scale = 1.0 / math.sqrt(d)
    print(f"length {L}, {G} query heads per KV head, top_c {c}, top_s {s}, d {d}")
    rows = []
    for h, kind in ((0, "mixture"), (1, "mixture"), (4, "isotropic"), (5, "isotropic")):
        K, V = b.unit_kv(0, h)
        t0 = time.time()
        lay = O.build_unit(K, V, wl.n_sink, wl.n_recent, wl.kmeans_iters, O.unit_state(1, 0, h, wl.n_kv_heads))
        for m in ms:
            W = synth.feature_map_w(m, d).numpy()
            F = O.with_feature_summaries(lay, K, W, scale=scale, V=V)
            for t in range(b.Q.shape[0]):
                Q = b.Q[t, 0, h * G:(h + 1) * G].numpy().astype(np.float64)
                o, _ = O.dense_attention(K, V, Q, scale)
                gauss = O.decode_unit(F, K, V, Q, c, s, scale=scale)
                fm_mean = O.decode_unit(F, K, V, Q, c, s, scale=scale, feature_residual=True)
                fm_full = O.decode_unit(F, K, V, Q, c, s, scale=scale, feature_residual=True, feature_numerator=True)
                for g in range(G):
                    rows.append((kind, m, rel(gauss["out"][g], o[g]), rel(fm_mean["out"][g], o[g]),
                                 rel(fm_full["out"][g], o[g]), rel(gauss["out_top"][g], o[g])))
        print(f"  KV head {h} ({kind}): {time.time() - t0:.1f} s", flush=True)
    print()
    print("| heads | m | Gaussian | feature mass, mean value | feature mass and numerator | exact part only |")
    print("|---|---|---|---|---|---|")
    for kind in ("mixture", "isotropic"):
        for m in ms:
            sel = np.array([r[2:] for r in rows if r[0] == kind and r[1] == m])
            print(f"| {kind} | {m} | " + " | ".join(f"{x:.3f}" for x in sel.mean(0)) + " |")
    C, S = lay.C, lay.S
    print()
    print(f"summary floats per head at this length (C = {C}, S = {S}, d = {d}):")
    print(f"  Gaussian (mu, s, vbar per group): {(C + C * S) * 3 * d}")
    for m in ms:
        print(f"  feature sums Z (m = {m}): {(C + C * S) * m};  value sums Z^v: {(C + C * S) * m * d}")
    print(f"  the cache itself (K and V rows): {2 * L * d}")


if __name__ == "__main__":
    main()
