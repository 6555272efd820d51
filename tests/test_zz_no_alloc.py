"""mog_decode_noalloc (the decode step on the library's static device
scratch, for callers that cannot allocate) against mog_decode with a caller
workspace: two calls in a row, the second on a smaller input, then the first
input again; results must be bit-identical (same kernels, same inputs), and
one unit is also checked against the oracle.  A step that needs more scratch
than the static array holds is refused with nothing enqueued."""

import ctypes as C
import sys

import numpy as np
import pytest
import torch

from long_context_sparse_mog_amd import capi, ops, synth
from parity import compare_unit, oracle_layout_from_export

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(wl, seed=3):
    b = synth.generate(wl, device="cuda")
    kv = ops.KVCache.from_batch(b)
    lay = ops.mog_build(kv, wl.n_sink, wl.n_recent, kmeans_iters=wl.kmeans_iters, seed=seed)
    p = ops.decode_params(wl.n_q_heads, list(wl.top_c), list(wl.top_s))
    return b, kv, lay, p


def _run_both(wl, b, kv, lay, p):
    q = b.Q[0].contiguous()
    ref = ops.mog_decode(lay, kv, q, p, want_sel=True)
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:2], float("nan"), device="cuda")
    sel_c = torch.full_like(ref[2], -7)
    sel_s = torch.full_like(ref[3], -7)
    got = ops.mog_decode_noalloc(lay, kv, q, p, out, lse, sel_c, sel_s)
    torch.cuda.synchronize()
    for name, x, y in zip(("out", "lse", "sel_c", "sel_s"), got, ref):
        assert torch.equal(x, y), name
    return q, got


def test_noalloc_matches_workspace_decode_twice_then_smaller():
    wa = synth.config(1, seq_lens=[12000], n_kv_heads=2, n_q_heads=8, n_components=64)
    wb = synth.config(4, seq_lens=[3000, 5000], n_kv_heads=2, n_q_heads=4, high_entropy_heads=(1,),
                      n_components=32)
    ca = _case(wa)
    cb = _case(wb)
    for wl, case in ((wa, ca), (wb, cb), (wa, ca)):
        need = ops.mog_workspace_size(capi.MOG_OP_DECODE, layout=case[2], params=case[3])
        say(f"[noalloc] {wl.name} lens={wl.seq_lens} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} "
            f"paged={wl.paged} scratch needed {need} of {capi.MOG_DECODE_NOALLOC_MAX_WS}")
        q, got = _run_both(wl, *case)
    # the first workload's unit 1 against the oracle as well
    b, kv, lay, p = ca
    q = b.Q[0].contiguous()
    out, lse, sel_c, sel_s = (t.cpu().numpy() for t in _run_both(wa, *ca)[1])
    G = wa.group
    K, V = b.unit_kv(0, 1)
    L = oracle_layout_from_export(lay.export_unit(1), wa.n_sink, wa.n_recent)
    Q = q[0, G:2 * G].cpu().numpy().astype(np.float64)
    r = compare_unit(L, K, V, Q, wa.top_c[0], wa.top_s[0], out[0, G:2 * G], lse[0, G:2 * G], sel_c[0, G:2 * G],
                     sel_s[0, G:2 * G], 2e-3)
    say(f"  oracle: worst rel L2 {r['max_rel']:.2e}, near ties {r['ties']}")


def test_noalloc_refuses_a_step_beyond_the_static_scratch():
    # 16 sequences of 1M tokens, 8 query heads per KV head, top_c = 128:
    # the step's records alone exceed the static scratch.  The layout's rows
    # are external (never read: the call is refused before anything is
    # enqueued) and the paged cache has a single page.
    n_seq, L, Hkv, D = 16, 1 << 20, 1, 128
    lens = [L] * n_seq
    dims, _keep = ops._dims(n_seq, Hkv, D, capi.MOG_BF16, 64, 256, lens, rows_external=1)
    nbytes = C.c_size_t()
    capi.check(capi.lib().mog_layout_size(C.byref(dims), C.byref(nbytes)), "mog_layout_size")
    mem = torch.empty(nbytes.value, dtype=torch.uint8, device="cuda")
    lay_c = capi.mog_layout()
    capi.check(capi.lib().mog_layout_init(C.byref(dims), C.c_void_p(mem.data_ptr()), nbytes.value, C.byref(lay_c),
                                          ops._stream()), "mog_layout_init")
    rows = torch.empty(64, dtype=torch.uint8, device="cuda")
    lay_c.k_mid = rows.data_ptr()
    lay_c.v_mid = rows.data_ptr()
    lay = ops.Layout(lay_c, mem)
    page = 256
    pool = torch.empty(1, Hkv, page, D, dtype=torch.bfloat16, device="cuda")
    table = torch.zeros(n_seq, L // page, dtype=torch.int32, device="cuda")
    kv = ops.KVCache(pool, pool, lens, table)
    p = ops.decode_params(8 * Hkv, 128, 5)
    need = ops.mog_workspace_size(capi.MOG_OP_DECODE, layout=lay, params=p)
    assert need > capi.MOG_DECODE_NOALLOC_MAX_WS
    q = torch.zeros(n_seq, 8 * Hkv, D, device="cuda")
    out = torch.zeros_like(q)
    torch.cuda.synchronize()
    with pytest.raises(capi.MogError) as err:
        ops.mog_decode_noalloc(lay, kv, q, p, out)
    assert err.value.status == capi.MOG_ERR_WORKSPACE
    assert "static scratch" in str(err.value)
    torch.cuda.synchronize()
    assert not out.any()  # nothing was written
    say(f"[noalloc] refused a step needing {need} bytes of scratch")
