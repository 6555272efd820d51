"""Helpers shared by the GPU parity tests: conversion of oracle layouts to the
arrays the library imports, oracle runs on downloaded layouts, and the
selection comparison with its near-tie rule."""

from __future__ import annotations

import math

import numpy as np

import oracle as O

NEAR_TIE = 1e-5  # absolute, on float64 oracle scores (natural log)
NEAR_TIE_SHARED = 1e-4  # relative, on the shared group scores (sums of mass fractions)


def unit_layout_arrays(L: "O.UnitLayout") -> dict:
    out = dict(perm=L.perm, sub_off=L.sub_off, cl_mu=L.cl_mu, cl_var=L.cl_var, cl_vbar=L.cl_vbar,
               sub_mu=L.sub_mu, sub_var=L.sub_var, sub_vbar=L.sub_vbar)
    if L.cl_z is not None:
        out.update(cl_z=L.cl_z, sub_z=L.sub_z, fm_w=L.fm_w, fm_scale=L.fm_scale)
    return out


def oracle_layout_from_export(ex: dict, n_sink: int, n_recent: int) -> "O.UnitLayout":
    """An oracle UnitLayout holding a layout downloaded from the device
    (with the tokens folded into it, if any)."""
    return O.UnitLayout(N=ex["N"], n_sink=n_sink, n_recent=n_recent, C=ex["C"], S=ex["S"],
                        perm=ex["perm"], sub_off=ex["sub_off"], cl_mu=ex["cl_mu"],
                        cl_var=ex["cl_var"], cl_vbar=ex["cl_vbar"], sub_mu=ex["sub_mu"],
                        sub_var=ex["sub_var"], sub_vbar=ex["sub_vbar"],
                        fold_pos=[int(x) for x in ex.get("fold_pos", [])],
                        fold_sub=[int(x) for x in ex.get("fold_sub", [])],
                        fm_w=ex.get("fm_w"), fm_scale=ex.get("fm_scale"), cl_z=ex.get("cl_z"),
                        sub_z=ex.get("sub_z"))


def build_oracle_layouts(batch, iters=10, seed=0, units=None):
    wl = batch.wl
    out = {}
    for s in range(wl.n_seq):
        for h in range(wl.n_kv_heads):
            u = s * wl.n_kv_heads + h
            if units is not None and u not in units:
                continue
            k, v = batch.unit_kv(s, h)
            out[u] = O.build_unit(k, v, wl.n_sink, wl.n_recent, iters,
                                  O.unit_state(seed, s, h, wl.n_kv_heads))
    return out


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _cutoff_ok(scores, valid, chosen_gpu, chosen_ora, k, rel_tol=None):
    """Selections may differ only where oracle scores are within NEAR_TIE of
    the k-th best score (or within rel_tol of it, relative)."""
    if set(chosen_gpu) == set(chosen_ora):
        return True
    idx = np.nonzero(valid)[0]
    kk = min(k, idx.size)
    if kk == 0:
        return False
    cut = np.sort(scores[idx])[::-1][kk - 1]
    diff = set(chosen_gpu) ^ set(chosen_ora)
    tol = NEAR_TIE if rel_tol is None else rel_tol * abs(cut)
    return all(abs(scores[i] - cut) <= tol for i in diff) and len(chosen_gpu) == len(chosen_ora)


def _shared_scores(L, Q, scale):
    """Group scores of the shared selection (oracle reading R14): clusters,
    and a function giving a chosen cluster's subcluster group scores."""
    G = Q.shape[0]
    valid = L.cl_count > 0
    sc = np.stack([O.group_log_mass(Q[h], L.cl_count, L.cl_mu, L.cl_var, scale) for h in range(G)])
    lse = np.array([np.logaddexp.reduce(sc[h][valid]) for h in range(G)])
    gs = np.where(valid, np.exp(sc - lse[:, None]).sum(axis=0), 0.0)

    def sub(j):
        g0 = j * L.S
        sv = L.sub_count[g0:g0 + L.S] > 0
        ss = np.stack([O.group_log_mass(Q[h], L.sub_count[g0:g0 + L.S], L.sub_mu[g0:g0 + L.S],
                                        L.sub_var[g0:g0 + L.S], scale) for h in range(G)])
        return np.where(sv, np.exp(ss - lse[:, None]).sum(axis=0), 0.0)

    return gs, sub


def compare_unit(L, K, V, Q, c, s, gpu_out, gpu_lse, gpu_sel_c, gpu_sel_s, tol, residual=True,
                 scale=None, shared=False):
    # residual: False, True (Gaussian) or "fm" (feature map)
    """Compare one unit's GPU results with the oracle's.  Returns a dict of
    the errors; raises AssertionError on a selection mismatch that is not a
    near tie.  ``shared``: one selection per KV head (oracle reading R14).
    ``gpu_sel_s`` None: a budget of whole clusters (s >= S), whose chosen
    subclusters are every nonempty one of each chosen cluster."""
    G, d = Q.shape
    # the statistics as the library's decode reads them (reading R18)
    L = O.decode_statistics(L)
    if gpu_sel_s is None:
        assert s >= L.S, (s, L.S)
        gpu_sel_s = [[np.flatnonzero(L.sub_count[int(j) * L.S:(int(j) + 1) * L.S] > 0) if j >= 0 else []
                      for j in gpu_sel_c[h]] for h in range(G)]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    fmr = residual == "fm"
    ref = O.decode_unit(L, K, V, Q, c, s, scale=scale, residual=bool(residual), shared=shared,
                        feature_residual=fmr)
    if shared:
        gs, gs_sub = _shared_scores(L, Q, scale)
    sel_c_gpu, sel_s_gpu = [], []
    ties = 0
    for h in range(G):
        gc = [int(x) for x in gpu_sel_c[h] if x >= 0]
        sel_c_gpu.append(np.asarray(gc, np.int64))
        subs = []
        for r, j in enumerate(gc):
            subs.append(np.asarray([int(x) for x in gpu_sel_s[h][r] if x >= 0], np.int64))
        sel_s_gpu.append(subs)
        oc = [int(x) for x in ref["sel_c"][h]]
        if gc != oc:
            if shared:
                assert _cutoff_ok(gs, L.cl_count > 0, gc, oc, c, NEAR_TIE_SHARED), (h, gc, oc)
            else:
                sc = O.group_log_mass(Q[h], L.cl_count, L.cl_mu, L.cl_var, scale)
                assert _cutoff_ok(sc, L.cl_count > 0, gc, oc, c), (h, gc, oc)
            ties += 1
        for r, j in enumerate(gc):
            if j in oc:
                osub = [int(x) for x in ref["sel_s"][h][oc.index(j)]]
                gsub = [int(x) for x in subs[r]]
                if gsub != osub:
                    g0 = j * L.S
                    if shared:
                        assert _cutoff_ok(gs_sub(j), L.sub_count[g0:g0 + L.S] > 0, gsub, osub, s,
                                          NEAR_TIE_SHARED), (h, j, gsub, osub)
                    else:
                        ss = O.group_log_mass(Q[h], L.sub_count[g0:g0 + L.S], L.sub_mu[g0:g0 + L.S],
                                              L.sub_var[g0:g0 + L.S], scale)
                        assert _cutoff_ok(ss, L.sub_count[g0:g0 + L.S] > 0, gsub, osub, s), (h, j, gsub, osub)
                    ties += 1
    if ties:
        ref = O.decode_unit(L, K, V, Q, c, s, scale=scale, residual=bool(residual),
                            sel_override=(sel_c_gpu, sel_s_gpu), feature_residual=fmr)
    errs = [rel_l2(gpu_out[h], ref["out"][h]) for h in range(G)]
    lse_err = float(np.max(np.abs(np.asarray(gpu_lse, np.float64) - ref["lse"])))
    assert max(errs) <= tol, (errs, tol)
    return dict(max_rel=max(errs), lse_err=lse_err, ties=ties, ref=ref)
