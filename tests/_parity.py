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


def valid_near_tie(gi, s, gs, E, G, TG, k):
    """For a token with a near tie (gap < GAP) at a selection boundary: is the
    GPU's id set gi one the method gives under some resolution of the ties?
    Every group whose oracle score is more than GAP above the TG-th best is
    kept; the groups within GAP of it fill the remaining places in any
    combination; for each such kept set the top-k experts of its groups
    (oracle fp32 scores) must equal gi, or gi must lie in those groups with a
    score sum no lower than the top-k's minus k * GAP (a near tie at the
    expert boundary)."""
    from itertools import combinations

    gsz = E // G
    gs = gs.astype(np.float64)
    s = s.astype(np.float64)
    thr = np.sort(gs)[::-1][TG - 1]
    sure = [g for g in range(G) if gs[g] > thr + GAP]
    tied = [g for g in range(G) if abs(gs[g] - thr) <= GAP and g not in sure]
    want = set(int(e) for e in gi)
    for combo in combinations(tied, TG - len(sure)):
        kept = sorted(sure + list(combo))
        cand = np.concatenate([np.arange(g * gsz, (g + 1) * gsz) for g in kept])
        top = cand[np.lexsort((cand, -s[cand]))][:k]
        if want == set(top.tolist()):
            return True
        if want <= set(cand.tolist()) and s[list(want)].sum() >= s[top].sum() - k * GAP:
            return True
    return False


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
            assert valid_near_tie(gi, scores[t], gscores[t], E, G, TG, k), \
                f"token {t}: near-tie choice {gi} is not one the method allows (oracle {oi})"
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


def h_error(gpu_h, ref_h):
    """The SwiGLU product h is rounded to bf16 on both sides from fp32 values
    that differ by the accumulation order, so an element may land one bf16
    step (at most 2^-7 of its magnitude) away, plus fp32-level noise.  Returns
    max |gpu - ref| / (2^-7 |ref| + 1e-3 RMS(ref)); <= 1 passes."""
    ref = np.asarray(ref_h, np.float64)
    err = np.abs(np.asarray(gpu_h, np.float64) - ref)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float((err / (2.0 ** -7 * np.abs(ref) + 1e-3 * rms + 1e-30)).max())


def out_error(gpu_out, ref_out):
    ref = ref_out.astype(np.float64)
    err = np.abs(gpu_out.astype(np.float64) - ref)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(err.max()) / rms if rms > 0 else float(err.max()), rms


# ---- unwritten-output detection ----------------------------------------
#
# Every output buffer is prefilled with a value no call writes (NaN for
# floating-point outputs, -1 for indices, 0xFF bytes -- a bf16 NaN -- for the
# workspace), so a tile, row or token that a kernel skips shows up as a
# surviving sentinel instead of a stale correct value left by an earlier call.

def fill_sentinels(bufs):
    """Fill every tensor of a buffer dict (moe.alloc_buffers) in place."""
    import torch
    for v in bufs.values():
        if v.dtype in (torch.float32, torch.bfloat16):
            v.fill_(float("nan"))
        elif v.dtype == torch.int32:
            v.fill_(-1)
        elif v.dtype == torch.uint8:
            v.fill_(0xFF)
        else:
            raise TypeError(v.dtype)
    return bufs


def sentinel_buffers(moe, p, out_dtype=None):
    """moe.alloc_buffers(p) with every buffer holding its sentinel."""
    import torch
    b = moe.alloc_buffers(p, out_dtype=out_dtype or torch.float32)
    return fill_sentinels(b)


def all_finite(t, rows_per_chunk=1 << 16):
    """True if every element of a (possibly many-GB) GPU tensor is finite;
    checked on the GPU in row chunks."""
    import torch
    for c in torch.split(t, rows_per_chunk):
        if not bool(torch.isfinite(c).all()):
            return False
    return True


def assert_forward_written(b, P, E, out=True, y=True):
    """After a forward pass with every pair kept: no sentinel survives in
    out, y (all P rows), topk_ids (all in [0, E)) or topk_weights."""
    import torch
    ids = b["topk_ids"]
    assert int(ids.min()) >= 0 and int(ids.max()) < E, "unwritten or invalid expert id"
    assert bool(torch.isfinite(b["topk_weights"]).all()), "unwritten routing weight"
    if y:
        assert all_finite(b["y"][:P]), "unwritten row of y"
    if out:
        assert all_finite(b["out"]), "unwritten element of out"


def edge_rows(off, n_extra_per_split=(191, 192, 255, 256), big=512):
    """Sorted positions at the edges of the expert GEMMs' row tiles, for
    sampling: the first and last row of every expert; for experts with more
    than 256 rows (split into several row tiles) the rows on either side of
    the 192- and 256-row marks; for experts with more than `big` rows every
    256-row boundary.  Returns a sorted array of positions."""
    off = np.asarray(off, np.int64)
    q = []
    for e in range(off.size - 1):
        a, n = int(off[e]), int(off[e + 1] - off[e])
        if n == 0:
            continue
        q += [a, a + n - 1]
        if n > 256:
            q += [a + m for m in n_extra_per_split if m < n]
        if n > big:
            q += [a + m for m in range(255, n, 256)] + [a + m for m in range(256, n, 256)]
    return np.unique(np.asarray(q, np.int64))


def stratified_tokens(off, sorted_pairs, k, T, n, rng, always=()):
    """About n distinct tokens: those whose pairs sit at the row-tile edges
    (edge_rows; at most n/2 of them, a seeded choice if there are more), the
    tokens in `always`, and seeded random tokens for the rest."""
    edge_tok = np.unique(np.asarray(sorted_pairs, np.int64)[edge_rows(off)] // k)
    if edge_tok.size > n // 2:
        edge_tok = np.sort(rng.choice(edge_tok, n // 2, replace=False))
    chosen = set(edge_tok.tolist()) | {int(t) for t in always}
    rest = np.setdiff1d(np.arange(T), np.fromiter(chosen, np.int64, len(chosen)))
    need = max(0, n - len(chosen))
    if need and rest.size:
        chosen |= set(rng.choice(rest, min(need, rest.size), replace=False).tolist())
    return np.array(sorted(chosen), np.int64)
