"""Host logic of the Python binding without a GPU: parameter marshalling,
the feature-map projection's draw, and the refusal of host tensors that the
GPU cannot address (no compute call is made)."""

import ctypes as C

import pytest
import torch

from long_context_sparse_mog_amd import capi, ops, synth


def test_decode_params_residual_modes():
    assert ops.decode_params(8, 4, 2).residual == 1
    assert ops.decode_params(8, 4, 2, residual=False).residual == 0
    assert ops.decode_params(8, 4, 2, residual="fm").residual == 2
    assert ops.decode_params(8, 4, 2, residual=2).residual == 2
    p = ops.decode_params(8, [4, 5], [2, 3], shared=True)
    assert p.shared_selection == 1 and p.top_c == 4
    assert [p.top_c_per_seq[i] for i in range(2)] == [4, 5]
    assert [p.top_s_per_seq[i] for i in range(2)] == [2, 3]


def test_feature_map_projection_is_seeded_and_standard_normal():
    a = synth.feature_map_w(256, 128)
    b = synth.feature_map_w(256, 128)
    assert a.dtype == torch.float32 and a.shape == (256, 128) and torch.equal(a, b)
    assert not torch.equal(a, synth.feature_map_w(256, 128, seed=1))
    assert abs(float(a.mean())) < 0.02 and abs(float(a.std()) - 1.0) < 0.02


def test_kv_cache_refuses_pageable_host_tensors():
    k = torch.zeros(1, 1, 64, 64)
    with pytest.raises(ValueError):
        ops.KVCache(k, k.clone(), [64])


def test_build_params_mirror_feature_map_and_external_rows():
    bp = capi.mog_build_params(10, 4, 64, 32, 7, 128, 0.5, 0x1000, 0x2000, 0x3000)
    assert (bp.kmeans_iters, bp.n_sink, bp.n_recent, bp.fold_capacity, bp.seed) == (10, 4, 64, 32, 7)
    assert (bp.fm_dim, bp.fm_scale, bp.fm_w, bp.rows_k, bp.rows_v) == (128, 0.5, 0x1000, 0x2000, 0x3000)
    d, keep = ops._dims(2, 8, 128, capi.MOG_BF16, 64, 256, [5000, 6000], fold_capacity=16, fm_dim=64,
                        rows_external=1)
    assert (d.fold_capacity, d.fm_dim, d.rows_external) == (16, 64, 1)
    assert [d.seq_lens[i] for i in range(2)] == [5000, 6000]
    rows = C.c_int64()
    assert capi.lib().mog_layout_rows(C.byref(d), C.byref(rows)) == capi.MOG_OK
    assert rows.value == 8 * (5000 - 320) + 8 * (6000 - 320) + 16 * 16
