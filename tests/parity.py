"""Parity helpers: compare the GPU top-k rows with the CPU oracle.

The acceptance rule (scores within tol of the oracle's; index sets equal
except for keys whose oracle score lies within tol of the k-th oracle score)
is applied row by row.  tol = rel * max|I| with rel = 1e-2 for f16/bf16
inputs and 1e-5 for f32 inputs, where max|I| is the oracle's largest
|head-reduced score| over the visible pairs it scored.
"""
from __future__ import annotations

import numpy as np

import oracle

REL_TOL = {"f16": 1e-2, "bf16": 1e-2, "f32": 1e-5}


def check_rows(g_idx, g_sc, o_idx, o_sc, v_rows, tol, rows=None, exact=False):
    """Check GPU rows against oracle rows.

    g_idx/g_sc, o_idx/o_sc: [n, k_top] arrays; v_rows: [n, n_kv] oracle masked
    scores of the same rows (f32, -inf = not visible).  exact=True demands
    identical idx and score arrays.  Returns the number of rows whose index
    set equals the oracle's exactly."""
    n, k_top = o_idx.shape
    exact_rows = 0
    for r in range(n):
        name = rows[r] if rows is not None else r
        gi, gs, oi, os_, v = g_idx[r], g_sc[r], o_idx[r], o_sc[r], v_rows[r]
        if exact:
            assert np.array_equal(gi, oi), f"row {name}: idx differs\n{gi[:16]}\n{oi[:16]}"
            assert np.array_equal(gs, os_), f"row {name}: scores differ"
            exact_rows += 1
            continue
        m = int((oi >= 0).sum())
        gm = int((gi >= 0).sum())
        assert gm == m, f"row {name}: {gm} keys returned, oracle has {m}"
        assert np.all(gi[m:] == -1) and np.all(gs[m:] == -np.inf), f"row {name}: bad padding"
        assert np.all(oi[:m] >= 0)
        gv = gi[:m]
        assert len(np.unique(gv)) == m, f"row {name}: duplicate indices"
        assert np.all((gv >= 0) & (gv < v.shape[0])), f"row {name}: index out of range"
        assert np.all(v[gv] != -np.inf), f"row {name}: a masked key was returned"
        # GPU scores agree with the oracle's score of the same key
        err = np.abs(gs[:m].astype(np.float64) - v[gv].astype(np.float64))
        assert err.max(initial=0) <= tol, f"row {name}: score error {err.max()} > tol {tol}"
        # GPU rows are ordered by (score desc, index asc)
        d = np.diff(gs[:m])
        assert np.all(d <= 0), f"row {name}: scores not descending"
        ties = np.nonzero(d == 0)[0]
        assert np.all(gv[ties] < gv[ties + 1]), f"row {name}: equal scores not in index order"
        og, oo = set(gv.tolist()), set(oi[:m].tolist())
        if og == oo:
            exact_rows += 1
            continue
        assert m == k_top, f"row {name}: fewer than k_top visible keys, but the sets differ"
        tau = float(os_[m - 1])
        for s in og ^ oo:
            assert abs(float(v[s]) - tau) <= tol, (
                f"row {name}: key {s} (oracle score {v[s]}) differs from the oracle set "
                f"but is not within {tol} of the k-th score {tau}")
    return exact_rows


def oracle_rows(q, k, w, mask, ranges, k_top, rows, qk_dtype=None, threads=0):
    """Oracle top-k and full masked score rows for a subset of queries."""
    o_idx, o_sc, maxabs = oracle.topk(q, k, w, mask=mask, kv_range=ranges, k_top=k_top, rows=rows,
                                      qk_dtype=qk_dtype, threads=threads)
    v = oracle.scores(q, k, w, mask=mask, kv_range=ranges, rows=rows, qk_dtype=qk_dtype, threads=threads)
    return o_idx, o_sc, maxabs, v
