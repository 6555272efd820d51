"""The decode's bf16 copies of the group statistics (reading R18): after a
build, after appends and after an import, every copy equals its float32
statistic rounded to nearest, ties to even (torch's own float32 -> bfloat16
conversion on the host), bit for bit."""

import sys

import numpy as np
import pytest
import torch

from long_context_sparse_mog_amd import ops, synth
from parity import build_oracle_layouts, unit_layout_arrays

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_copies(lay, what):
    a = lay.arrays()
    n = 0
    for name in ("cl_ms", "cl_vbar", "sub_ms", "sub_vbar"):
        f32 = a[name].cpu()
        want = f32.to(torch.bfloat16).view(torch.int16)
        got = a[name + "16"].cpu()
        assert torch.equal(got, want), (what, name, int((got != want).sum()))
        n += f32.numel()
    say(f"  {what}: {n} statistics, bf16 copies bit-exact")


def test_copies_after_build_and_appends():
    wl = synth.config(1, seq_lens=[6000, 3000], n_kv_heads=2, n_q_heads=8, n_components=48)
    grow = [40, 7]
    from dataclasses import replace
    wg = replace(wl, seq_lens=[L + g for L, g in zip(wl.seq_lens, grow)])
    say(f"[stats16] build {wl.seq_lens}, then append {grow}")
    b = synth.generate(wg, device="cuda")
    kv = ops.KVCache.from_batch(b)
    lay = ops.mog_build(kv.with_lens(wl.seq_lens), wl.n_sink, wl.n_recent, fold_capacity=64)
    torch.cuda.synchronize()
    check_copies(lay, "build")
    ops.mog_append(lay, kv.with_lens([wl.seq_lens[0] + 1, wl.seq_lens[1]]))
    ops.mog_append(lay, kv)
    torch.cuda.synchronize()
    check_copies(lay, "appends")


def test_copies_after_import_fp32_d64():
    wl = synth.config(0, seq_lens=[3000, 5000], n_kv_heads=2, n_q_heads=2)
    say(f"[stats16] import {wl.name} {wl.seq_lens}")
    b = synth.generate(wl, device="cuda")
    kv = ops.KVCache.from_batch(b)
    lays = build_oracle_layouts(b)
    lay = ops.import_layout(kv, wl.n_sink, wl.n_recent, [unit_layout_arrays(lays[u]) for u in range(len(lays))])
    torch.cuda.synchronize()
    check_copies(lay, "import")
