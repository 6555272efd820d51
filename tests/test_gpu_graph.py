"""The decode step under HIP graph capture: no allocation, no host copy and
no memset on the path, so torch can capture mog_decode (and the dense
baseline) on its stream.  The graph is replayed several times with new
queries written into its input between replays, with eager work and
synchronisations in between, and every replay must equal the eager result
bit for bit."""

import sys

import pytest
import torch

from long_context_sparse_mog_amd import capi, ops, synth

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("residual", [True, False])
def test_decode_graph_replays_match_eager(residual):
    wl = synth.config(1, seq_lens=[8192], n_components=64)
    say(f"[graph] {wl.name} residual={residual}")
    b = synth.generate(wl, device="cuda", n_qsets=4)
    kv = ops.KVCache.from_batch(b)
    lay = ops.mog_build(kv, wl.n_sink, wl.n_recent, seed=2)
    p = ops.decode_params(wl.n_q_heads, wl.top_c, wl.top_s, residual=residual)
    ws = ops.workspace(ops.mog_workspace_size(capi.MOG_OP_DECODE, layout=lay, params=p))
    q_static = b.Q[0].clone()
    out = torch.empty_like(q_static)
    lse = torch.empty(q_static.shape[:2], device="cuda")
    eager = []
    for t in range(4):
        o, l, _, _ = ops.mog_decode(lay, kv, b.Q[t].contiguous(), p, ws=ws)
        eager.append((o.clone(), l.clone()))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ops.mog_decode(lay, kv, q_static, p, out=out, lse=lse, ws=ws)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.mog_decode(lay, kv, q_static, p, out=out, lse=lse, ws=ws)
    for rep in range(3):
        for t in (2, 0, 3, 1):
            q_static.copy_(b.Q[t])
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager[t][0]) and torch.equal(lse, eager[t][1]), (rep, t)
            # eager work between replays
            ops.mog_decode(lay, kv, b.Q[(t + 1) % 4].contiguous(), p)
            torch.cuda.synchronize()


def test_dense_graph_replays_match_eager():
    wl = synth.config(1, seq_lens=[8192], n_kv_heads=2, n_q_heads=8)
    b = synth.generate(wl, device="cuda", n_qsets=2)
    kv = ops.KVCache.from_batch(b)
    p = ops.decode_params(wl.n_q_heads, 1, 1)
    ws = ops.workspace(ops.mog_workspace_size(capi.MOG_OP_DENSE, kv=kv, params=p))
    q_static = b.Q[0].clone()
    out = torch.empty_like(q_static)
    lse = torch.empty(q_static.shape[:2], device="cuda")
    ref = [ops.mog_dense_decode(kv, b.Q[t].contiguous(), p, ws=ws) for t in range(2)]
    ref = [(o.clone(), l.clone()) for o, l in ref]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ops.mog_dense_decode(kv, q_static, p, out=out, lse=lse, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.mog_dense_decode(kv, q_static, p, out=out, lse=lse, ws=ws)
    for rep in range(3):
        for t in (1, 0):
            q_static.copy_(b.Q[t])
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref[t][0]) and torch.equal(lse, ref[t][1]), (rep, t)
