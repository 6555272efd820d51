"""The C ABI without a GPU: the library loads, exports every function that
include/mog.h declares, the ctypes structs match the C layout, sizes are
computed on the host, and invalid arguments are rejected before anything
is enqueued."""

import ctypes as C
import os
import re
import subprocess

import pytest

from long_context_sparse_mog_amd import build_lib, capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mog.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(capi.LIB_PATH):
        build_lib.build(force=False)
    return capi.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mog_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) == 13, names
    out = subprocess.run(["nm", "-D", "--defined-only", capi.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (mog_\w+)", out))
    assert set(names) == exported, (set(names) ^ exported)
    for n in names:
        assert hasattr(L, n)
    assert set(names) == set(capi.SIGNATURES)


def test_struct_layout_matches_c(tmp_path):
    fields = {
        "mog_kv": capi.mog_kv, "mog_dims": capi.mog_dims, "mog_unit": capi.mog_unit,
        "mog_layout": capi.mog_layout, "mog_build_params": capi.mog_build_params,
        "mog_decode_params": capi.mog_decode_params,
    }
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "mog.h"', 'int main(void){']
    for name, cls in fields.items():
        lines.append(f'printf("{name} %zu\\n", sizeof({name}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{name}.{f} %zu\\n", offsetof({name}, {f}));')
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                       check=True).stdout.splitlines())
    for name, cls in fields.items():
        assert int(got[name]) == C.sizeof(cls), name
        for f, _ in cls._fields_:
            assert int(got[f"{name}.{f}"]) == getattr(cls, f).offset, f"{name}.{f}"


def _dims(lens, n_sink=64, n_recent=256, hkv=8, d=128, dtype=capi.MOG_BF16, fold_capacity=0, fm_dim=0):
    arr = capi.int_array(lens)
    return capi.mog_dims(len(lens), hkv, d, dtype, n_sink, n_recent, fold_capacity, fm_dim, 0,
                         C.cast(arr, C.POINTER(capi.i32))), arr


def test_layout_size_matches_geometry(L):
    d, keep = _dims([1048576])
    out = C.c_size_t()
    assert L.mog_layout_size(C.byref(d), C.byref(out)) == capi.MOG_OK
    n_mid, Cc, S, D = 1048576 - 320, 1024, 20, 128
    # rows, perm, offsets, group statistics (float32, and the decode's bf16
    # copies), per-group fold counts
    expect = 8 * (2 * n_mid * D * 2 + n_mid * 4 + (Cc * S + 1) * 4 + (Cc + Cc * S) * 3 * D * (4 + 2)
                  + (Cc + Cc * S) * 4)
    assert expect <= out.value <= expect + 20 * 256
    # a fold area: K/V rows, their subcluster and position, per unit
    cap = 1000
    d2, keep2 = _dims([1048576], fold_capacity=cap)
    out2 = C.c_size_t()
    assert L.mog_layout_size(C.byref(d2), C.byref(out2)) == capi.MOG_OK
    grow = 8 * cap * (2 * D * 2 + 2 * 4)
    assert grow <= out2.value - out.value <= grow + 8 * 256
    # feature-map summaries: the projection and m floats per group
    d3, keep3 = _dims([1048576], fm_dim=128)
    out3 = C.c_size_t()
    assert L.mog_layout_size(C.byref(d3), C.byref(out3)) == capi.MOG_OK
    grow = 128 * D * 4 + 8 * (Cc + Cc * S) * 128 * 4
    assert grow <= out3.value - out.value <= grow + 4 * 256
    # external rows: none in the buffer; mog_layout_rows counts them
    d4, keep4 = _dims([1048576], fold_capacity=cap)
    d4.rows_external = 1
    out4 = C.c_size_t()
    assert L.mog_layout_size(C.byref(d4), C.byref(out4)) == capi.MOG_OK
    assert out2.value - out4.value >= 2 * (8 * (n_mid + cap)) * D * 2
    rows = C.c_int64()
    assert L.mog_layout_rows(C.byref(d4), C.byref(rows)) == capi.MOG_OK
    assert rows.value == 8 * (n_mid + cap)


def test_layout_unit_geometry(L):
    lens = [4096, 20000, 777]
    d, keep = _dims(lens, n_sink=4, n_recent=64, hkv=2, d=64, dtype=capi.MOG_F32)
    lay = capi.mog_layout()
    lay.n_seq, lay.n_kv_heads, lay.head_dim, lay.n_sink, lay.n_recent = 3, 2, 64, 4, 64
    lay.n_units = 6
    for i, x in enumerate(lens):
        lay.seq_lens[i] = x
    row = cl = sub = off = 0
    import oracle as O
    for u in range(6):
        U = capi.mog_unit()
        assert L.mog_layout_unit(C.byref(lay), u, C.byref(U)) == capi.MOG_OK
        n_mid, Cc, S = O.unit_dims(lens[u // 2], 4, 64)
        assert (U.seq, U.kv_head, U.N, U.n_mid, U.C, U.S) == (u // 2, u % 2, lens[u // 2], n_mid, Cc, S)
        assert (U.row_base, U.cl_base, U.sub_base, U.off_base) == (row, cl, sub, off)
        row += n_mid
        cl += Cc
        sub += Cc * S
        off += Cc * S + 1
    assert L.mog_layout_unit(C.byref(lay), 6, C.byref(U)) == capi.MOG_ERR_INVALID_ARG
    # after folding: the geometry follows the lengths at the build, N the
    # current length
    lay.fold_capacity = 100
    lay.seq_lens[0] = lens[0] + 37
    lay.fold_count[0] = 37
    row = 0
    for u in range(6):
        U = capi.mog_unit()
        assert L.mog_layout_unit(C.byref(lay), u, C.byref(U)) == capi.MOG_OK
        n_mid, Cc, S = O.unit_dims(lens[u // 2], 4, 64)
        assert (U.N, U.n_mid, U.C, U.S, U.row_base) == (lens[u // 2] + (37 if u < 2 else 0), n_mid, Cc, S, row)
        assert U.n_fold == (37 if u < 2 else 0)
        row += n_mid


@pytest.mark.parametrize("bad, status", [
    (dict(lens=[300]), capi.MOG_ERR_INVALID_ARG),              # no middle region after 64+256
    (dict(lens=[5000], d=96), capi.MOG_ERR_UNSUPPORTED),
    (dict(lens=[(1 << 22) + 1]), capi.MOG_ERR_UNSUPPORTED),
    (dict(lens=[5000], n_sink=-1), capi.MOG_ERR_INVALID_ARG),
    (dict(lens=[5000], dtype=7), capi.MOG_ERR_UNSUPPORTED),
    (dict(lens=[]), capi.MOG_ERR_INVALID_ARG),
    (dict(lens=[5000], fold_capacity=-1), capi.MOG_ERR_INVALID_ARG),
    (dict(lens=[5000], fold_capacity=capi.MOG_MAX_FOLD + 1), capi.MOG_ERR_INVALID_ARG),
    (dict(lens=[5000], fm_dim=100), capi.MOG_ERR_UNSUPPORTED),
])
def test_layout_size_rejects(L, bad, status):
    lens = bad.pop("lens")
    d, keep = _dims(lens if lens else [1], **bad)
    if not lens:
        d.n_seq = 0
    out = C.c_size_t()
    assert L.mog_layout_size(C.byref(d), C.byref(out)) == status
    assert L.mog_last_error().decode() != ""


def _kv(lens, **kw):
    arr = capi.int_array(lens)
    kv = capi.mog_kv()
    kv.format, kv.dtype, kv.n_seq, kv.n_kv_heads, kv.head_dim = 0, capi.MOG_BF16, len(lens), 8, 128
    kv.max_len = max(lens)
    kv.seq_lens = C.cast(arr, C.POINTER(capi.i32))
    kv.k, kv.v = 0x100000, 0x200000   # never dereferenced: validation fails first or no launch
    for k, v in kw.items():
        setattr(kv, k, v)
    return kv, arr


def test_decode_and_dense_validation(L):
    kv, keep = _kv([5000])
    p = capi.mog_decode_params(n_q_heads=12, top_c=4, top_s=2, residual=1, scale=0.0, splits=0)
    out = C.c_size_t()
    # 12 query heads on 8 KV heads
    assert L.mog_workspace_size(capi.MOG_OP_DENSE, C.byref(kv), None, None, C.byref(p), C.byref(out)) == capi.MOG_ERR_INVALID_ARG
    p.n_q_heads = 8 * 9   # G = 9 > 8
    assert L.mog_workspace_size(capi.MOG_OP_DENSE, C.byref(kv), None, None, C.byref(p), C.byref(out)) == capi.MOG_ERR_UNSUPPORTED
    p.n_q_heads = 32
    assert L.mog_workspace_size(capi.MOG_OP_DENSE, C.byref(kv), None, None, C.byref(p), C.byref(out)) == capi.MOG_OK
    assert out.value > 0
    p.top_c = -1
    assert L.mog_workspace_size(capi.MOG_OP_DENSE, C.byref(kv), None, None, C.byref(p), C.byref(out)) == capi.MOG_ERR_INVALID_ARG
    p.top_c = 4
    for bad in (-1, 65):   # timing aid: 0..64 launches
        p.exact_repeat = bad
        assert L.mog_workspace_size(capi.MOG_OP_DENSE, C.byref(kv), None, None, C.byref(p), C.byref(out)) == capi.MOG_ERR_INVALID_ARG
    p.exact_repeat = 64
    assert L.mog_workspace_size(capi.MOG_OP_DENSE, C.byref(kv), None, None, C.byref(p), C.byref(out)) == capi.MOG_OK
    p.exact_repeat = 0
    # dense with a NULL q / NULL workspace
    assert L.mog_dense_decode(C.byref(kv), None, C.byref(p), C.c_void_p(0x1000), None, C.c_void_p(0x1000), 1 << 30, None) == capi.MOG_ERR_INVALID_ARG
    assert L.mog_dense_decode(C.byref(kv), C.c_void_p(0x1000), C.byref(p), C.c_void_p(0x1000), None, None, 1 << 30, None) == capi.MOG_ERR_INVALID_ARG
    # workspace too small
    assert L.mog_dense_decode(C.byref(kv), C.c_void_p(0x1000), C.byref(p), C.c_void_p(0x1000), None, C.c_void_p(0x1000), 16, None) == capi.MOG_ERR_WORKSPACE
    # misaligned k
    kv2, keep2 = _kv([5000], k=0x100004)
    assert L.mog_dense_decode(C.byref(kv2), C.c_void_p(0x1000), C.byref(p), C.c_void_p(0x1000), None, C.c_void_p(0x1000), 1 << 30, None) == capi.MOG_ERR_INVALID_ARG
    # paged without a block table
    kv3, keep3 = _kv([5000], format=1, page_size=16, n_pages=400, max_blocks=313)
    assert L.mog_workspace_size(capi.MOG_OP_DENSE, C.byref(kv3), None, None, C.byref(p), C.byref(out)) == capi.MOG_ERR_INVALID_ARG
    kv4, keep4 = _kv([5000], format=1, page_size=12, n_pages=400, max_blocks=313, block_table=0x3000)
    assert L.mog_workspace_size(capi.MOG_OP_DENSE, C.byref(kv4), None, None, C.byref(p), C.byref(out)) == capi.MOG_ERR_INVALID_ARG
    # decode with no layout
    assert L.mog_decode(None, C.byref(kv), C.c_void_p(0x1000), C.byref(p), C.c_void_p(0x1000), None, None, None, C.c_void_p(0x1000), 1 << 30, None) == capi.MOG_ERR_INVALID_ARG
    # layout that does not match the cache
    lay = capi.mog_layout()
    lay.n_seq, lay.n_kv_heads, lay.head_dim, lay.dtype = 1, 4, 128, capi.MOG_BF16
    assert L.mog_decode(C.byref(lay), C.byref(kv), C.c_void_p(0x1000), C.byref(p), C.c_void_p(0x1000), None, None, None, C.c_void_p(0x1000), 1 << 30, None) == capi.MOG_ERR_INVALID_ARG
    assert "does not match" in L.mog_last_error().decode()


def test_build_validation(L):
    kv, keep = _kv([5000])
    bp = capi.mog_build_params(10, 64, 256, 0, 7)
    out = C.c_size_t()
    assert L.mog_workspace_size(capi.MOG_OP_BUILD, C.byref(kv), None, C.byref(bp), None, C.byref(out)) == capi.MOG_OK
    bp.kmeans_iters = -1
    assert L.mog_workspace_size(capi.MOG_OP_BUILD, C.byref(kv), None, C.byref(bp), None, C.byref(out)) == capi.MOG_ERR_INVALID_ARG
    bp.kmeans_iters = 10
    bp.n_recent = 5000
    assert L.mog_workspace_size(capi.MOG_OP_BUILD, C.byref(kv), None, C.byref(bp), None, C.byref(out)) == capi.MOG_ERR_INVALID_ARG
    bp.n_recent = 256
    lay = capi.mog_layout()
    # misaligned layout memory
    assert L.mog_build(C.byref(kv), C.byref(bp), C.c_void_p(0x1001), 1 << 40, C.c_void_p(0x1000), 1 << 40, C.byref(lay), None) == capi.MOG_ERR_INVALID_ARG
    # layout memory too small
    assert L.mog_build(C.byref(kv), C.byref(bp), C.c_void_p(0x1000), 64, C.c_void_p(0x1000), 1 << 40, C.byref(lay), None) == capi.MOG_ERR_WORKSPACE
    # feature-map summaries without a projection, with an odd size, a negative scale
    bp.fm_dim = 128
    assert L.mog_workspace_size(capi.MOG_OP_BUILD, C.byref(kv), None, C.byref(bp), None, C.byref(out)) == capi.MOG_ERR_INVALID_ARG
    bp.fm_w = 0x4000
    assert L.mog_workspace_size(capi.MOG_OP_BUILD, C.byref(kv), None, C.byref(bp), None, C.byref(out)) == capi.MOG_OK
    bp.fm_scale = -1.0
    assert L.mog_workspace_size(capi.MOG_OP_BUILD, C.byref(kv), None, C.byref(bp), None, C.byref(out)) == capi.MOG_ERR_INVALID_ARG
    bp.fm_scale, bp.fm_dim = 0.0, 96
    assert L.mog_workspace_size(capi.MOG_OP_BUILD, C.byref(kv), None, C.byref(bp), None, C.byref(out)) == capi.MOG_ERR_UNSUPPORTED
    bp.fm_dim = 0
    # external rows: both arrays or neither, 16-byte aligned
    bp.rows_k = 0x50000
    assert L.mog_workspace_size(capi.MOG_OP_BUILD, C.byref(kv), None, C.byref(bp), None, C.byref(out)) == capi.MOG_ERR_INVALID_ARG
    bp.rows_v = 0x60008
    assert L.mog_workspace_size(capi.MOG_OP_BUILD, C.byref(kv), None, C.byref(bp), None, C.byref(out)) == capi.MOG_ERR_INVALID_ARG
    bp.rows_v = 0x60000
    assert L.mog_workspace_size(capi.MOG_OP_BUILD, C.byref(kv), None, C.byref(bp), None, C.byref(out)) == capi.MOG_OK


def test_feature_residual_validation(L):
    kv, keep = _kv([5000])
    lay = _host_layout([5000], cap=0, folded=[0])
    p = capi.mog_decode_params(n_q_heads=32, top_c=4, top_s=2, residual=2, scale=0.0, splits=0)
    args = (C.c_void_p(0x1000), C.byref(p), C.c_void_p(0x1000), None, None, None, C.c_void_p(0x1000), 1 << 40, None)
    # residual=2 on a layout without summaries
    assert L.mog_decode(C.byref(lay), C.byref(kv), *args) == capi.MOG_ERR_INVALID_ARG
    assert "fm_dim" in L.mog_last_error().decode()
    # summaries built with another scale
    lay.fm_dim, lay.fm_scale = 128, 0.5
    for name in ("fm_w", "cl_fz", "sub_fz"):
        setattr(lay, name, 0x20000)
    assert L.mog_decode(C.byref(lay), C.byref(kv), *args) == capi.MOG_ERR_INVALID_ARG
    assert "scale" in L.mog_last_error().decode()
    p.residual = 3
    assert L.mog_decode(C.byref(lay), C.byref(kv), *args) == capi.MOG_ERR_INVALID_ARG


def _host_layout(lens, cap, folded):
    """A layout descriptor whose arrays are never dereferenced (validation
    fails first, or there is nothing to enqueue)."""
    lay = capi.mog_layout()
    lay.n_seq, lay.n_kv_heads, lay.head_dim, lay.dtype = len(lens), 8, 128, capi.MOG_BF16
    lay.n_sink, lay.n_recent, lay.n_units, lay.fold_capacity = 64, 256, 8 * len(lens), cap
    for i, (x, f) in enumerate(zip(lens, folded)):
        lay.seq_lens[i] = x
        lay.fold_count[i] = f
    for name in ("units", "k_mid", "v_mid", "perm", "sub_off", "cl_ms", "cl_vbar", "sub_ms", "sub_vbar",
                 "cl_ms16", "cl_vbar16", "sub_ms16", "sub_vbar16", "fold_sub", "fold_pos", "cl_fold", "sub_fold",
                 "append_scratch"):
        setattr(lay, name, 0x10000)
    return lay


def test_append_validation(L):
    lay = _host_layout([5000, 6000], cap=10, folded=[3, 0])
    # nothing grew: nothing to enqueue, layout unchanged
    kv, keep = _kv([5000, 6000])
    assert L.mog_append(C.byref(kv), C.byref(lay), None) == capi.MOG_OK
    assert list(lay.seq_lens[:2]) == [5000, 6000] and list(lay.fold_count[:2]) == [3, 0]
    # a sequence shorter than the layout's
    kv, keep = _kv([4999, 6000])
    assert L.mog_append(C.byref(kv), C.byref(lay), None) == capi.MOG_ERR_INVALID_ARG
    # 3 folded + 8 new > 10: build again; nothing changed
    kv, keep = _kv([5008, 6001])
    assert L.mog_append(C.byref(kv), C.byref(lay), None) == capi.MOG_ERR_CAPACITY
    assert "capacity" in L.mog_last_error().decode()
    assert list(lay.seq_lens[:2]) == [5000, 6000] and list(lay.fold_count[:2]) == [3, 0]
    # a layout without a fold area cannot grow at all
    lay0 = _host_layout([5000], cap=0, folded=[0])
    kv, keep = _kv([5001])
    assert L.mog_append(C.byref(kv), C.byref(lay0), None) == capi.MOG_ERR_CAPACITY
    # shape mismatch, and a fold count beyond the capacity
    kv, keep = _kv([5000])
    assert L.mog_append(C.byref(kv), C.byref(lay), None) == capi.MOG_ERR_INVALID_ARG
    bad = _host_layout([5000], cap=4, folded=[5])
    assert L.mog_append(C.byref(kv), C.byref(bad), None) == capi.MOG_ERR_INVALID_ARG
    assert L.mog_append(C.byref(kv), None, None) == capi.MOG_ERR_INVALID_ARG


def test_status_strings(L):
    for s in range(6):
        assert L.mog_status_string(s).decode()
    assert L.mog_status_string(99).decode() == "unknown status"


def test_sync_stats_validation(L):
    # rejected before anything is enqueued: no layout, a layout with NULL
    # arrays, and a complete descriptor with an unsupported head dimension
    assert L.mog_layout_sync_stats(None, None) == capi.MOG_ERR_INVALID_ARG
    empty = capi.mog_layout()
    assert L.mog_layout_sync_stats(C.byref(empty), None) == capi.MOG_ERR_INVALID_ARG
    assert b"NULL arrays" in L.mog_last_error()
    lay = _host_layout([5000], cap=0, folded=[0])
    lay.head_dim = 96
    assert L.mog_layout_sync_stats(C.byref(lay), None) == capi.MOG_ERR_INVALID_ARG
    assert b"head_dim" in L.mog_last_error()
