"""Keep routing decisions clear of floating-point ties in test inputs.

TEST INFRASTRUCTURE ONLY (see ``oracle/moe_oracle.py``).

Routing turns floating point into integers (which experts a token picks, which
pairs token rounding drops or adds).  The GPU decides on float32 logits, the
oracle on float64 ones; the two agree whenever no decision sits within rounding
error of a tie.  These helpers redraw the input rows of tokens whose decisions
sit closer than a margin to a tie, until none does:

* top-k: every gap between adjacent values among a token's k+1 largest logits
  must be at least ``delta_z`` (absolute);
* token rounding: for every expert whose count moves, the probabilities on both
  sides of the cut (last dropped / first kept, or last added / first not added)
  must differ by at least ``delta_p`` relative.

The caller passes ``redraw(x, rows, attempt) -> new x``; the replacement values
come from the seeded input generator, so the result stays a pure function of
the seed.
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import router_logits, topk_softmax


def topk_tie_tokens(z, k, delta_z):
    z = np.asarray(z, np.float64)
    E = z.shape[1]
    m = min(k + 1, E)
    if m < 2:
        return np.zeros(0, np.int64)
    zs = -np.sort(-z, axis=1)[:, :m]
    gaps = zs[:, :-1] - zs[:, 1:]
    return np.nonzero((gaps < delta_z).any(axis=1))[0]


def rounding_tie_tokens(idx, P, E, tile, delta_p):
    """Tokens on either side of a rounding cut whose P values are too close."""
    T, k = idx.shape
    sel = np.zeros((T, E), bool)
    sel[np.repeat(np.arange(T), k), idx.ravel()] = True
    bad = []
    for e in range(E):
        n = int(sel[:, e].sum())
        target = ((n + tile // 2) // tile) * tile
        if target > T:
            target = (n // tile) * tile
        if target < n:
            cand = np.nonzero(sel[:, e])[0]
            order = np.lexsort((-cand, P[cand, e]))
            c = n - target
            if c < n:
                a, b = cand[order[c - 1]], cand[order[c]]
                pa, pb = P[a, e], P[b, e]
                if abs(pa - pb) < delta_p * max(pa, pb):
                    bad += [a, b]
        elif target > n:
            cand = np.nonzero(~sel[:, e])[0]
            order = np.lexsort((cand, -P[cand, e]))
            c = target - n
            if c < cand.size:
                a, b = cand[order[c - 1]], cand[order[c]]
                pa, pb = P[a, e], P[b, e]
                if abs(pa - pb) < delta_p * max(pa, pb):
                    bad += [a, b]
    return np.unique(np.asarray(bad, np.int64))


def clear_ties(x, w_gate, bias, k, redraw, round_tile=0, delta_z=1e-3, delta_p=1e-4,
               max_iter=200, noise=None):
    """Redraw rows of ``x`` until routing has no near-tie.  Returns (x, redraws).
    ``noise`` [T,E] (noisy routing) is added to the logits the decisions use."""
    to_np = (lambda t: t.float().numpy()) if hasattr(x, "float") else (lambda t: np.asarray(t))
    wg = to_np(w_gate)
    b = None if bias is None else to_np(bias)
    nz = None if noise is None else to_np(noise).astype(np.float64)
    redrawn = 0
    for attempt in range(max_iter):
        z = router_logits(to_np(x), wg, b)
        if nz is not None:
            z = z + nz
        bad = topk_tie_tokens(z, k, delta_z)
        if bad.size == 0 and round_tile:
            idx, _, P = topk_softmax(z, k)
            bad = rounding_tie_tokens(idx, P, wg.shape[0], round_tile, delta_p)
        if bad.size == 0:
            return x, redrawn
        redrawn += int(bad.size)
        x = redraw(x, bad, attempt)
    raise RuntimeError("tie clearance did not converge")
