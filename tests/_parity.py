"""Shared helpers for the GPU-vs-oracle parity tests.

Routing: indices must be bit-exact except on tokens whose oracle fp32 score
gap at a selection boundary is below 1e-5 (the group boundary: TG-th vs
(TG+1)-th group score; the expert boundary: k-th vs (k+1)-th candidate score).
Such tokens are "exempt": their GPU choice must still be valid and as good as
the oracle's within 1e-5, and their outputs are compared against the oracle
run with the GPU's routing.  Outputs: max |err| <= 2e-2 * RMS(oracle out).
"""
from __future__ import annotations

import numpy as np

GAP = 1e-5
OUT_TOL = 2e-2
W_TOL = 1e-5


def boundary_gaps(scores, gscores, E, G, TG, k):
    """Per token: (group-boundary gap, expert-boundary gap) from the oracle's
    fp32 scores [T,E] and group scores [T,G].  inf where there is no
    boundary."""
    T = scores.shape[0]
    gsz = E // G
    g_gap = np.full(T, np.inf)
    e_gap = np.full(T, np.inf)
    gs_sorted = -np.sort(-gscores.astype(np.float64), axis=1)
    if TG < G:
        g_gap = gs_sorted[:, TG - 1] - gs_sorted[:, TG]
    order = np.lexsort((np.arange(G)[None, :].repeat(T, 0), -gscores), axis=1)
    kept = order[:, :TG]
    for t in range(T):
        cand = np.concatenate([scores[t, g * gsz:(g + 1) * gsz] for g in kept[t]])
        if k < cand.size:
            c = -np.sort(-cand.astype(np.float64))
            e_gap[t] = c[k - 1] - c[k]
    return g_gap, e_gap


def compare_routing(gpu_ids, gpu_w, ora_ids, ora_w, scores, gscores, E, G, TG, k):
    """Asserts the routing contract; returns (exempt mask, stats dict)."""
    T = gpu_ids.shape[0]
    g_gap, e_gap = boundary_gaps(scores, gscores, E, G, TG, k)
    exempt = (g_gap < GAP) | (e_gap < GAP)
    gsz = E // G
    bad = []
    for t in range(T):
        gi, oi = gpu_ids[t], ora_ids[t]
        # always: valid selection, weights sum to one
        assert len(set(gi.tolist())) == k, f"token {t}: duplicate ids {gi}"
        assert np.all((gi >= 0) & (gi < E)), f"token {t}: id out of range {gi}"
        assert len({int(e) // gsz for e in gi}) <= TG, f"token {t}: more than TG groups"
        assert abs(float(gpu_w[t].astype(np.float64).sum()) - 1.0) <= 1e-5
        if exempt[t]:
            sg = float(scores[t, gi].astype(np.float64).sum())
            so = float(scores[t, oi].astype(np.float64).sum())
            assert sg >= so - 1e-5 * k, f"token {t}: exempt choice worse than oracle"
            continue
        if set(gi.tolist()) != set(oi.tolist()):
            bad.append(t)
            continue
        # order: identical wherever the oracle's adjacent scores differ by >= GAP
        so = scores[t, oi].astype(np.float64)
        for j in range(k):
            if gi[j] != oi[j]:
                lo = j - 1 >= 0 and so[j - 1] - so[j] < GAP
                hi = j + 1 < k and so[j] - so[j + 1] < GAP
                assert lo or hi, f"token {t}: order differs at {j}: {gi} vs {oi}"
        # weights per expert
        wg = dict(zip(gi.tolist(), gpu_w[t].tolist()))
        for e, w in zip(oi.tolist(), ora_w[t].tolist()):
            assert abs(wg[e] - w) <= W_TOL, f"token {t}: weight of {e}: {wg[e]} vs {w}"
    assert not bad, f"routing differs on non-exempt tokens {bad[:10]} (of {len(bad)})"
    return exempt, dict(tokens=T, exempt=int(exempt.sum()))


def out_error(gpu_out, ref_out):
    ref = ref_out.astype(np.float64)
    err = np.abs(gpu_out.astype(np.float64) - ref)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(err.max()) / rms if rms > 0 else float(err.max()), rms
