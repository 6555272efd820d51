"""The seeded workload generator: shapes, determinism and the budgets."""

import numpy as np
import torch

from long_context_sparse_mog_amd import synth


def test_budgets_of_the_workloads():
    assert synth.budget_for_length(32768, 64, 256) == (27, 4)
    assert synth.budget_for_length(131072, 64, 256) == (58, 5)
    assert synth.budget_for_length(1048576, 64, 256) == (203, 5)
    assert synth.budget_for_length(8192, 64, 256) == (3, 4)
    assert synth.budget_for_length(262144, 64, 256) == (90, 5)
    wl = synth.config(4)
    assert wl.n_seq == 16 and all(8192 <= L <= 262144 for L in wl.seq_lens)
    # measured budgets of the workloads (mean per-head read share <= 5%),
    # with the split of the lowest error against dense attention
    assert (synth.config(1).top_c, synth.config(1).top_s) == ([4], [15])
    assert (synth.config(3).top_c, synth.config(3).top_s) == ([17], [20])
    assert (synth.config(2).top_c, synth.config(2).top_s) == ([38] * 4, [2] * 4)
    assert synth.budget_for_length(262144, 64, 256, kappa=0.35) == (31, 5)
    # whole clusters: s = S; a fixed split is capped at S
    assert synth.budget_for_length(262144, 64, 256, split="whole") == (25, 18)
    assert synth.budget_for_length(4096, 4, 64, split=40)[1] == 12


def test_generate_deterministic_and_shaped():
    wl = synth.config(1, seq_lens=[2048], n_kv_heads=2, n_q_heads=8, n_components=16)
    a = synth.generate(wl, n_qsets=2)
    b = synth.generate(wl, n_qsets=2)
    assert a.K.shape == (1, 2, 2048, 128) and a.K.dtype == torch.bfloat16
    assert a.Q.shape == (2, 1, 8, 128)
    assert torch.equal(a.K, b.K) and torch.equal(a.Q, b.Q)
    # outlier dims: two channels with much larger spread
    sd = a.K[0, 0].float().std(0)
    assert (sd > 4 * sd.median()).sum() == 2


def test_paged_pool_round_trip():
    wl = synth.config(4, seq_lens=[100, 37, 300], n_kv_heads=2, n_q_heads=4,
                      high_entropy_heads=(1,), n_components=8, n_sink=4, n_recent=8)
    b = synth.generate(wl)
    P = wl.page_size
    for s, L in enumerate(wl.seq_lens):
        for t in [0, 5, L - 1]:
            page = int(b.block_table[s, t // P])
            assert torch.equal(b.pool_K[page, :, t % P], b.K[s, :, t])
            assert torch.equal(b.pool_V[page, :, t % P], b.V[s, :, t])
    used = b.block_table[b.block_table >= 0].numpy()
    assert len(np.unique(used)) == len(used) == b.pool_K.shape[0]


def test_needles_have_cosine_point_eight():
    wl = synth.config(2, n_seq=1, seq_lens=[4096], n_q_heads=1, n_kv_heads=1, n_components=16)
    b = synth.generate(wl)
    q = b.Q[0, 0, 0]
    k = b.K[0, 0].float()
    cos = (k @ q) / (k.norm(dim=1) * q.norm())
    top = torch.topk(cos, 16).values
    assert torch.allclose(top, torch.full_like(top, 0.8), atol=0.01)
