"""Comparison rules between the HIP path and the CPU oracle.

Selection: top-k block ids must equal the oracle's bit for bit, except on
near-tie rows (the oracle's k-th and (k+1)-th block scores differ by at most
1e-3 relative).  There the GPU set may differ from the oracle's only by blocks
whose oracle score lies inside that band around the k-th score; it must still
hold exactly min(k, E) distinct eligible ids in ascending order.

Attention: bf16 outputs must satisfy |gpu - ref| <= 2e-3 + 1e-2 * |ref|
element-wise (bf16 inputs, float32 accumulation on both sides).
"""
from __future__ import annotations

import numpy as np

ATOL = 2e-3
RTOL = 1e-2
BAND = 1e-3


def check_selection_invariants(ids, E, k):
    """ids [k] of one (row, group): min(k, E) distinct ascending eligible ids, then -1."""
    m = min(k, E)
    sel = ids[:m]
    assert (ids[m:] == -1).all(), ids
    assert (sel >= 0).all() and (sel < E).all(), ids
    assert (np.diff(sel) > 0).all(), ids


def selection_report(oracle, inp, rows, gpu_ids, ref_ids, kth, tie):
    """The same rule as compare_ids, counted instead of asserted: rows, (row, group) pairs, near ties,
    in-band flips (pairs that differ only inside the near-tie band), and exact mismatches (pairs that
    differ outside it, or break the selection invariants)."""
    wl = inp.wl
    B, k, h = wl.block_size, wl.top_k, wl.num_kv_heads
    report = dict(rows=len(rows), pairs=len(rows) * h, near_tie=int(tie.sum()), exact_mismatch=0,
                  band_flips=0)
    seq_of = np.searchsorted(inp.cu_seqlens_q, rows, side="right") - 1
    for i, row in enumerate(rows):
        s = seq_of[i]
        lq = inp.cu_seqlens_q[s + 1] - inp.cu_seqlens_q[s]
        lk = inp.cu_seqlens_k[s + 1] - inp.cu_seqlens_k[s]
        E = (lk - lq + (row - inp.cu_seqlens_q[s])) // B + 1
        for g in range(h):
            gi, ri = gpu_ids[i, g], ref_ids[i, g]
            try:
                check_selection_invariants(gi, E, k)
            except AssertionError:
                report["exact_mismatch"] += 1
                continue
            if np.array_equal(gi, ri):
                continue
            if not tie[i, g]:
                report["exact_mismatch"] += 1
                continue
            S = oracle.block_scores(inp, int(row), g)
            a, b = float(kth[i, g, 0]), float(kth[i, g, 1])
            tol = BAND * max(abs(a), abs(b))
            diff = set(gi[gi >= 0].tolist()) ^ set(ri[ri >= 0].tolist())
            if all(abs(float(S[j]) - a) <= tol for j in diff):
                report["band_flips"] += 1
            else:
                report["exact_mismatch"] += 1
    return report


def compare_ids(oracle, inp, rows, gpu_ids, ref_ids, kth, tie):
    """Returns a report dict; raises AssertionError on a violation."""
    wl = inp.wl
    B, k, h = wl.block_size, wl.top_k, wl.num_kv_heads
    report = dict(rows=len(rows), pairs=len(rows) * h, near_tie=int(tie.sum()), exact_mismatch=0,
                  band_flips=0)
    seq_of = np.searchsorted(inp.cu_seqlens_q, rows, side="right") - 1
    for i, row in enumerate(rows):
        s = seq_of[i]
        lq = inp.cu_seqlens_q[s + 1] - inp.cu_seqlens_q[s]
        lk = inp.cu_seqlens_k[s + 1] - inp.cu_seqlens_k[s]
        p = lk - lq + (row - inp.cu_seqlens_q[s])
        E = p // B + 1
        for g in range(h):
            gi, ri = gpu_ids[i, g], ref_ids[i, g]
            check_selection_invariants(gi, E, k)
            if np.array_equal(gi, ri):
                continue
            if not tie[i, g]:
                report["exact_mismatch"] += 1
                raise AssertionError(f"row {row} group {g}: ids differ on a row that is not a near tie\n"
                                     f"gpu {gi}\nref {ri}\nkth {kth[i, g]}")
            S = oracle.block_scores(inp, int(row), g)
            a, b = float(kth[i, g, 0]), float(kth[i, g, 1])
            tol = BAND * max(abs(a), abs(b))
            diff = set(gi[gi >= 0].tolist()) ^ set(ri[ri >= 0].tolist())
            for j in diff:
                assert abs(float(S[j]) - a) <= tol, \
                    f"row {row} group {g}: block {j} (score {S[j]}) is outside the near-tie band of {a}"
            report["band_flips"] += 1
    return report


def assert_close(gpu, ref, what=""):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    with np.errstate(invalid="ignore"):
        err = np.abs(gpu - ref)
        bound = ATOL + RTOL * np.abs(ref)
        # equal values (infinities included) match; a NaN anywhere else is a mismatch
        bad = ~((gpu == ref) | (err <= bound))
    err = np.where(gpu == ref, 0.0, err)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance; "
                             f"max err {err.max():.3g}; first bad {idx.tolist()} gpu "
                             f"{gpu[tuple(idx[0])]:.6g} ref {ref[tuple(idx[0])]:.6g}")
    return float(np.nanmax(err)) if err.size else 0.0
