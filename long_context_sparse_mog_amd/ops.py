"""Torch-facing wrappers of the libmog C ABI.

Tensors supply device memory and the stream; every computation runs in the
library's HIP kernels.  Nothing here falls back to a CPU path: without a GPU
or without the built library every call raises.
"""

from __future__ import annotations

import ctypes as C
import math

import numpy as np
import torch

from . import capi
from .capi import check, lib

_DTYPES = {torch.float32: capi.MOG_F32, torch.bfloat16: capi.MOG_BF16}


def _vp(t):
    return C.c_void_p(t.data_ptr()) if t is not None else None


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libmog works on device tensors only")


def _require_gpu_addressable(*ts):
    """Device tensors, or pinned host tensors (which the GPU reads over the
    host link)."""
    for t in ts:
        if t is not None and not (t.is_cuda or t.is_pinned()):
            raise ValueError("libmog reads device tensors or pinned host tensors only")


class KVCache:
    """A batch of KV caches as the library sees it.

    Contiguous: ``k``/``v`` are [n_seq][Hkv][max_len][D].  Paged: ``k``/``v``
    are page pools [n_pages][Hkv][page][D] and ``block_table`` is
    [n_seq][max_blocks] int32.  ``seq_lens`` is a host list.
    """

    def __init__(self, k, v, seq_lens, block_table=None):
        # (k and v may be pinned host memory: the offloaded-cache setting)
        _require_gpu_addressable(k, v)
        _require_cuda(block_table)
        if k.dtype not in _DTYPES or v.dtype != k.dtype:
            raise ValueError("k/v must both be float32 or bfloat16")
        if not (k.is_contiguous() and v.is_contiguous()):
            raise ValueError("k/v must be contiguous")
        self.k, self.v, self.block_table = k, v, block_table
        self.seq_lens = [int(x) for x in seq_lens]
        self._lens = capi.int_array(self.seq_lens)
        c = capi.mog_kv()
        c.dtype = _DTYPES[k.dtype]
        c.n_seq = len(self.seq_lens)
        c.n_kv_heads = k.shape[1]
        c.head_dim = k.shape[3]
        c.seq_lens = C.cast(self._lens, C.POINTER(capi.i32))
        c.k = k.data_ptr()
        c.v = v.data_ptr()
        if block_table is None:
            c.format = capi.MOG_KV_CONTIGUOUS
            c.max_len = k.shape[2]
        else:
            if block_table.dtype != torch.int32 or not block_table.is_contiguous():
                raise ValueError("block_table must be contiguous int32")
            c.format = capi.MOG_KV_PAGED
            c.page_size = k.shape[2]
            c.n_pages = k.shape[0]
            c.max_blocks = block_table.shape[1]
            c.block_table = block_table.data_ptr()
        self.c = c

    @property
    def n_kv_heads(self):
        return self.c.n_kv_heads

    @property
    def head_dim(self):
        return self.c.head_dim

    def with_lens(self, seq_lens):
        """The same cache tensors with other sequence lengths (a grown cache)."""
        return KVCache(self.k, self.v, seq_lens, self.block_table)

    @classmethod
    def from_batch(cls, b, paged=None):
        """From a ``synth.Batch``; paged follows the workload unless given."""
        paged = b.wl.paged if paged is None else paged
        if paged:
            return cls(b.pool_K, b.pool_V, b.wl.seq_lens, b.block_table)
        return cls(b.K, b.V, b.wl.seq_lens)


class Layout:
    """A cluster layout living in ``mem`` (a uint8 device tensor); with
    external rows, k_mid / v_mid live in the tensors ``rows`` (e.g. pinned
    host memory)."""

    def __init__(self, c_layout, mem, rows=None):
        self.c = c_layout
        self.mem = mem
        self.rows = rows

    @property
    def n_units(self):
        return self.c.n_units

    def unit(self, u: int) -> capi.mog_unit:
        out = capi.mog_unit()
        check(lib().mog_layout_unit(C.byref(self.c), u, C.byref(out)), "mog_layout_unit")
        return out

    def _view(self, ptr, count, dtype):
        off = ptr - self.mem.data_ptr()
        nbytes = count * torch.empty((), dtype=dtype).element_size()
        return self.mem[off:off + nbytes].view(dtype)

    def arrays(self):
        """Typed device views of every layout array (all units).  ``k_mid`` /
        ``v_mid`` include the fold area after the reordered rows."""
        c, D = self.c, self.c.head_dim
        kd = torch.bfloat16 if c.dtype == capi.MOG_BF16 else torch.float32
        rows = c.total_mid + c.n_units * c.fold_capacity
        cap = c.n_units * c.fold_capacity
        if self.rows is not None:
            kr, vr = (t.view(kd).view(-1, D)[:rows] for t in self.rows)
        else:
            kr = self._view(c.k_mid, rows * D, kd).view(-1, D)
            vr = self._view(c.v_mid, rows * D, kd).view(-1, D)
        fold = {}
        if cap:
            fold = dict(fold_sub=self._view(c.fold_sub, cap, torch.int32).view(c.n_units, -1),
                        fold_pos=self._view(c.fold_pos, cap, torch.int32).view(c.n_units, -1))
        if c.fm_dim:
            m = c.fm_dim
            fold.update(fm_w=self._view(c.fm_w, m * D, torch.float32).view(m, D),
                        cl_fz=self._view(c.cl_fz, c.total_cl * m, torch.float32).view(-1, m),
                        sub_fz=self._view(c.sub_fz, c.total_sub * m, torch.float32).view(-1, m))
        return dict(
            **fold,
            cl_fold=self._view(c.cl_fold, c.total_cl, torch.int32),
            sub_fold=self._view(c.sub_fold, c.total_sub, torch.int32),
            k_mid=kr,
            v_mid=vr,
            perm=self._view(c.perm, c.total_mid, torch.int32),
            sub_off=self._view(c.sub_off, c.total_off, torch.int32),
            cl_ms=self._view(c.cl_ms, c.total_cl * 2 * D, torch.float32).view(-1, 2 * D),
            cl_vbar=self._view(c.cl_vbar, c.total_cl * D, torch.float32).view(-1, D),
            sub_ms=self._view(c.sub_ms, c.total_sub * 2 * D, torch.float32).view(-1, 2 * D),
            sub_vbar=self._view(c.sub_vbar, c.total_sub * D, torch.float32).view(-1, D),
            # the decode's bf16 copies of the four above (the bits, as int16)
            cl_ms16=self._view(c.cl_ms16, c.total_cl * 2 * D, torch.int16).view(-1, 2 * D),
            cl_vbar16=self._view(c.cl_vbar16, c.total_cl * D, torch.int16).view(-1, D),
            sub_ms16=self._view(c.sub_ms16, c.total_sub * 2 * D, torch.int16).view(-1, 2 * D),
            sub_vbar16=self._view(c.sub_vbar16, c.total_sub * D, torch.int16).view(-1, D),
        )

    def export_unit(self, u: int) -> dict:
        """Host (NumPy) copy of one unit's layout."""
        U = self.unit(u)
        a = self.arrays()
        D = self.c.head_dim
        C_, S = U.C, U.S
        rows = slice(U.row_base, U.row_base + U.n_mid)
        cl = slice(U.cl_base, U.cl_base + C_)
        sb = slice(U.sub_base, U.sub_base + C_ * S)
        ms_c = a["cl_ms"][cl].cpu().numpy()
        ms_s = a["sub_ms"][sb].cpu().numpy()
        nf = U.n_fold
        fold = dict(fold_sub=np.zeros(0, np.int64), fold_pos=np.zeros(0, np.int64), fold_k=None, fold_v=None)
        if nf:
            f0 = self.c.total_mid + u * self.c.fold_capacity
            fold = dict(fold_sub=a["fold_sub"][u, :nf].cpu().numpy().astype(np.int64),
                        fold_pos=a["fold_pos"][u, :nf].cpu().numpy().astype(np.int64),
                        fold_k=a["k_mid"][f0:f0 + nf].float().cpu().numpy(),
                        fold_v=a["v_mid"][f0:f0 + nf].float().cpu().numpy())
        if self.c.fm_dim:
            fold.update(fm_w=a["fm_w"].cpu().numpy(), fm_scale=float(self.c.fm_scale),
                        cl_z=a["cl_fz"][cl].cpu().numpy(), sub_z=a["sub_fz"][sb].cpu().numpy())
        return dict(
            **fold,
            cl_fold=a["cl_fold"][cl].cpu().numpy().astype(np.int64),
            sub_fold=a["sub_fold"][sb].cpu().numpy().astype(np.int64),
            N=U.N, C=C_, S=S, n_mid=U.n_mid, n_fold=nf, seq=U.seq, kv_head=U.kv_head,
            perm=a["perm"][rows].cpu().numpy().astype(np.int64),
            sub_off=a["sub_off"][U.off_base:U.off_base + C_ * S + 1].cpu().numpy().astype(np.int64),
            cl_mu=ms_c[:, :D], cl_var=ms_c[:, D:], cl_vbar=a["cl_vbar"][cl].cpu().numpy(),
            sub_mu=ms_s[:, :D], sub_var=ms_s[:, D:], sub_vbar=a["sub_vbar"][sb].cpu().numpy(),
        )


def _dims(n_seq, n_kv_heads, head_dim, dtype, n_sink, n_recent, seq_lens, fold_capacity=0, fm_dim=0,
          rows_external=0):
    lens = capi.int_array(seq_lens)
    d = capi.mog_dims(n_seq, n_kv_heads, head_dim, dtype, n_sink, n_recent, fold_capacity, fm_dim, rows_external,
                      C.cast(lens, C.POINTER(capi.i32)))
    return d, lens


def mog_layout_size(n_kv_heads, head_dim, dtype, n_sink, n_recent, seq_lens, fold_capacity=0, fm_dim=0) -> int:
    d, _keep = _dims(len(seq_lens), n_kv_heads, head_dim, dtype, n_sink, n_recent, seq_lens, fold_capacity,
                     fm_dim)
    out = C.c_size_t()
    check(lib().mog_layout_size(C.byref(d), C.byref(out)), "mog_layout_size")
    return out.value


def mog_layout_init(kv: KVCache, n_sink, n_recent, device="cuda", stream=None, fold_capacity=0,
                    fm_dim=0) -> Layout:
    """Allocate and carve an empty layout for ``kv`` (for importing arrays)."""
    d, _keep = _dims(kv.c.n_seq, kv.c.n_kv_heads, kv.c.head_dim, kv.c.dtype, n_sink, n_recent,
                     kv.seq_lens, fold_capacity, fm_dim)
    nbytes = C.c_size_t()
    check(lib().mog_layout_size(C.byref(d), C.byref(nbytes)), "mog_layout_size")
    mem = torch.zeros(nbytes.value, dtype=torch.uint8, device=device)
    L = capi.mog_layout()
    check(lib().mog_layout_init(C.byref(d), _vp(mem), nbytes.value, C.byref(L), _stream(stream)),
          "mog_layout_init")
    return Layout(L, mem)


def decode_params(n_q_heads, top_c, top_s, residual=True, scale=0.0, splits=0, shared=False):
    """mog_decode_params; ``top_c``/``top_s`` are ints or per-sequence lists;
    ``residual``: False/0 none, True/1 Gaussian, 2 or "fm" feature map;
    ``shared``: one selection per KV head instead of one per query head."""
    p = capi.mog_decode_params()
    p.n_q_heads = n_q_heads
    p.residual = 2 if residual in (2, "fm") else (1 if residual else 0)
    p.scale = float(scale)
    p.splits = int(splits)
    p.shared_selection = 1 if shared else 0
    keep = []
    if isinstance(top_c, (list, tuple)):
        arr = capi.int_array(top_c)
        keep.append(arr)
        p.top_c_per_seq = C.cast(arr, C.POINTER(capi.i32))
        p.top_c = int(top_c[0])
    else:
        p.top_c = int(top_c)
    if isinstance(top_s, (list, tuple)):
        arr = capi.int_array(top_s)
        keep.append(arr)
        p.top_s_per_seq = C.cast(arr, C.POINTER(capi.i32))
        p.top_s = int(top_s[0])
    else:
        p.top_s = int(top_s)
    p._keep = keep
    return p


def mog_workspace_size(op, kv: KVCache = None, layout: Layout = None, build_params=None,
                       params=None) -> int:
    out = C.c_size_t()
    check(lib().mog_workspace_size(
        op, C.byref(kv.c) if kv is not None else None,
        C.byref(layout.c) if layout is not None else None,
        C.byref(build_params) if build_params is not None else None,
        C.byref(params) if params is not None else None, C.byref(out)), "mog_workspace_size")
    return out.value


def workspace(nbytes, device="cuda"):
    """A zero-filled workspace (mog_decode needs its first 256 bytes zero)."""
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)


def mog_build(kv: KVCache, n_sink, n_recent, kmeans_iters=10, seed=0, ws=None, stream=None,
              fold_capacity=0, fm_w=None, fm_scale=0.0, rows_host=False) -> Layout:
    """Prefill-side build; allocates the layout (and the workspace unless given).
    ``fold_capacity``: rows per unit kept for mog_append; ``fm_w``: a device
    float32 [m][head_dim] projection for feature-map summaries (m = 64, 128
    or 256), ``fm_scale`` their logit scale (0: 1/sqrt(head_dim));
    ``rows_host``: keep the reordered K/V rows in pinned host memory (the
    GPU reads the chosen ones over the host link)."""
    fm_dim = 0
    if fm_w is not None:
        _require_cuda(fm_w)
        if fm_w.dtype != torch.float32 or not fm_w.is_contiguous() or fm_w.dim() != 2:
            raise ValueError("fm_w must be a contiguous float32 [m][head_dim] tensor")
        fm_dim = fm_w.shape[0]
    d, _keep = _dims(kv.c.n_seq, kv.c.n_kv_heads, kv.c.head_dim, kv.c.dtype, n_sink, n_recent,
                     kv.seq_lens, fold_capacity, fm_dim, 1 if rows_host else 0)
    rows = None
    if rows_host:
        n = C.c_int64()
        check(lib().mog_layout_rows(C.byref(d), C.byref(n)), "mog_layout_rows")
        nbytes_rows = n.value * kv.head_dim * kv.k.element_size()
        rows = tuple(torch.empty(max(nbytes_rows, 16), dtype=torch.uint8, pin_memory=True) for _ in range(2))
    bp = capi.mog_build_params(kmeans_iters, n_sink, n_recent, fold_capacity, seed, fm_dim, float(fm_scale),
                               _vp(fm_w), rows[0].data_ptr() if rows else None,
                               rows[1].data_ptr() if rows else None)
    nbytes = C.c_size_t()
    check(lib().mog_layout_size(C.byref(d), C.byref(nbytes)), "mog_layout_size")
    mem = torch.empty(nbytes.value, dtype=torch.uint8, device=kv.k.device)
    need = mog_workspace_size(capi.MOG_OP_BUILD, kv=kv, build_params=bp)
    if ws is None or ws.numel() < need:
        ws = workspace(need, kv.k.device)
    L = capi.mog_layout()
    check(lib().mog_build(C.byref(kv.c), C.byref(bp), _vp(mem), nbytes.value, _vp(ws), ws.numel(),
                          C.byref(L), _stream(stream)), "mog_build")
    lay = Layout(L, mem, rows)
    lay._build_ws = ws
    return lay


def mog_append(layout: Layout, kv: KVCache, stream=None) -> None:
    """Fold the tokens that left the recent window since the layout was
    built (``kv`` holds the grown sequences); updates ``layout`` in place."""
    check(lib().mog_append(C.byref(kv.c), C.byref(layout.c), _stream(stream)), "mog_append")


def mog_decode(layout: Layout, kv: KVCache, q, params, out=None, lse=None, want_sel=False,
               ws=None, stream=None):
    """One decode step.  Returns (out, lse, sel_c, sel_s).

    ``want_sel``: False (no selection output), True (chosen clusters and
    subclusters) or ``"c"`` (chosen clusters only).  Asking for the
    subclusters always runs the subcluster kernel; without them a budget of
    whole clusters (top_s >= S everywhere) skips it."""
    _require_cuda(q)
    if q.dtype != torch.float32 or not q.is_contiguous():
        raise ValueError("q must be contiguous float32 [n_seq][Hq][D]")
    n_seq, Hq, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(n_seq, Hq, dtype=torch.float32, device=q.device)
    sel_c = sel_s = None
    if want_sel:
        cs = [params.top_c_per_seq[i] for i in range(n_seq)] if params.top_c_per_seq else [params.top_c]
        ss = [params.top_s_per_seq[i] for i in range(n_seq)] if params.top_s_per_seq else [params.top_s]
        cmax, smax = max(cs), max(ss)
        sel_c = torch.full((n_seq, Hq, max(cmax, 1)), -1, dtype=torch.int32, device=q.device)
        if want_sel != "c":
            sel_s = torch.full((n_seq, Hq, max(cmax, 1), max(smax, 1)), -1, dtype=torch.int32,
                               device=q.device)
    need = mog_workspace_size(capi.MOG_OP_DECODE, layout=layout, params=params)
    if ws is None or ws.numel() < need:
        ws = workspace(need, q.device)
    check(lib().mog_decode(C.byref(layout.c), C.byref(kv.c), _vp(q), C.byref(params), _vp(out),
                           _vp(lse), _vp(sel_c), _vp(sel_s), _vp(ws), ws.numel(), _stream(stream)),
          "mog_decode")
    return out, lse, sel_c, sel_s


def mog_decode_noalloc(layout: Layout, kv: KVCache, q, params, out, lse=None, sel_c=None, sel_s=None,
                       stream=None):
    """One decode step on the library's static device scratch (no workspace
    argument; the library allocates nothing).  ``out`` (and ``lse``,
    ``sel_c``, ``sel_s`` if given) are caller tensors, as in mog_decode."""
    _require_cuda(q, out, lse, sel_c, sel_s)
    if q.dtype != torch.float32 or not q.is_contiguous():
        raise ValueError("q must be contiguous float32 [n_seq][Hq][D]")
    check(lib().mog_decode_noalloc(C.byref(layout.c), C.byref(kv.c), _vp(q), C.byref(params), _vp(out),
                                   _vp(lse), _vp(sel_c), _vp(sel_s), _stream(stream)), "mog_decode_noalloc")
    return out, lse, sel_c, sel_s


def mog_dense_decode(kv: KVCache, q, params, out=None, lse=None, ws=None, stream=None):
    """Dense exact decode attention (the in-library baseline).  Returns (out, lse)."""
    _require_cuda(q)
    if q.dtype != torch.float32 or not q.is_contiguous():
        raise ValueError("q must be contiguous float32 [n_seq][Hq][D]")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
    need = mog_workspace_size(capi.MOG_OP_DENSE, kv=kv, params=params)
    if ws is None or ws.numel() < need:
        ws = workspace(need, q.device)
    check(lib().mog_dense_decode(C.byref(kv.c), _vp(q), C.byref(params), _vp(out), _vp(lse),
                                 _vp(ws), ws.numel(), _stream(stream)), "mog_dense_decode")
    return out, lse


def import_layout(kv: KVCache, n_sink, n_recent, units, k_rows=None, v_rows=None,
                  stream=None, fold_capacity=0) -> Layout:
    """Place a layout computed elsewhere into a fresh library layout.

    ``units[u]`` is a dict with ``perm`` (token position of every reordered
    row), ``sub_off`` (C*S+1 row offsets) and float32 ``cl_mu``, ``cl_var``,
    ``cl_vbar``, ``sub_mu``, ``sub_var``, ``sub_vbar``.  The reordered K/V
    rows are gathered from ``kv`` on the device; the decode's bf16 copies of
    the statistics are then rewritten by the library
    (``mog_layout_sync_stats``).
    """
    fm = units[0].get("cl_z") if units else None
    fm_dim = 0 if fm is None else int(np.asarray(fm).shape[1])
    lay = mog_layout_init(kv, n_sink, n_recent, device=kv.k.device, stream=stream, fold_capacity=fold_capacity,
                          fm_dim=fm_dim)
    a = lay.arrays()
    dev = kv.k.device
    D = kv.head_dim
    Hkv = kv.n_kv_heads
    for u, src in enumerate(units):
        U = lay.unit(u)
        C_, S = U.C, U.S
        perm = torch.as_tensor(np.asarray(src["perm"], dtype=np.int64), device=dev)
        sub_off = np.asarray(src["sub_off"], dtype=np.int64)
        if perm.numel() != U.n_mid or sub_off.size != C_ * S + 1:
            raise ValueError(f"unit {u}: layout arrays do not match the unit geometry")
        seq, kvh = U.seq, U.kv_head
        rows = slice(U.row_base, U.row_base + U.n_mid)
        if kv.block_table is None:
            a["k_mid"][rows] = kv.k[seq, kvh, perm]
            a["v_mid"][rows] = kv.v[seq, kvh, perm]
        else:
            P = kv.k.shape[2]
            page = kv.block_table[seq].long()[perm // P]
            a["k_mid"][rows] = kv.k[page, kvh, perm % P]
            a["v_mid"][rows] = kv.v[page, kvh, perm % P]
        a["perm"][rows] = perm.to(torch.int32)
        a["sub_off"][U.off_base:U.off_base + C_ * S + 1] = torch.as_tensor(sub_off, dtype=torch.int32, device=dev)
        cl = slice(U.cl_base, U.cl_base + C_)
        sb = slice(U.sub_base, U.sub_base + C_ * S)
        f32 = lambda x: torch.as_tensor(np.asarray(x, dtype=np.float32), device=dev)
        a["cl_ms"][cl, :D] = f32(src["cl_mu"])
        a["cl_ms"][cl, D:] = f32(src["cl_var"])
        a["cl_vbar"][cl] = f32(src["cl_vbar"])
        a["sub_ms"][sb, :D] = f32(src["sub_mu"])
        a["sub_ms"][sb, D:] = f32(src["sub_var"])
        a["sub_vbar"][sb] = f32(src["sub_vbar"])
        if fm_dim:
            a["cl_fz"][cl] = f32(src["cl_z"])
            a["sub_fz"][sb] = f32(src["sub_z"])
    # the decode's bf16 copies of the statistics just written
    check(lib().mog_layout_sync_stats(C.byref(lay.c), _stream(stream)), "mog_layout_sync_stats")
    if fm_dim:
        a["fm_w"][:] = torch.as_tensor(np.asarray(units[0]["fm_w"], np.float32), device=dev)
        sc = float(units[0]["fm_scale"])
        # (the carved default is the library's own 1/sqrt(head_dim), the
        # value a decode with scale 0 compares against)
        if abs(sc * math.sqrt(D) - 1.0) > 1e-6:
            lay.c.fm_scale = sc
    return lay
