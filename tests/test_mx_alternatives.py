"""CPU checks of the boundary-decision alternatives used by the MXFP8 parity
tests: a result that took the other side of a boundary decision is accepted,
and a result with a genuine mistake is still rejected."""
import numpy as np
import pytest

import mx_alternatives as mxa
from helpers import MX_MAX_BLOCK_FRACTION, close
from oracle import mx


def _operands(seed=0, n=64, kdim=256, width=96):
    r = np.random.default_rng(seed)
    a = r.standard_normal((n, kdim))
    b = r.standard_normal((kdim, width)) / 16
    # put one block of row 5 right under a power of two: its exponent decision is on the boundary
    blk = a[5, 32:64]
    blk *= (4.0 * (1 - 2.0 ** -9)) / np.abs(blk).max()
    return a, b


def test_boundary_flip_is_accepted():
    a, b = _operands()
    ref = mx.mx_roundtrip(a, axis=1) @ b
    # the "GPU" took the exponent one up for that block: amax 3.99.. -> 4.0 side
    flipped = mx.mx_roundtrip(a, axis=1)
    X = mx.block_exponent(np.abs(a[5, 32:64]).max())
    flipped[5, 32:64] = mx.roundtrip_at(a[5, 32:64], X + 1)
    got = flipped @ b
    assert not close(got, ref, 1e-6, 1e-6)[0]
    adj = ref.copy()
    for r, D, _ in mxa.operand_deltas(a, 1, b):
        adj[r] = mxa._select(got[r], adj[r], D)[0]
    ok, mabs, rf = close(got, adj, 1e-9, 1e-9)
    assert ok, (mabs, rf)


def test_genuine_errors_are_rejected():
    a, b = _operands(1)
    q = mx.mx_roundtrip(a, axis=1)
    ref = q @ b
    # a wrong scale on a block far from any boundary (factor 2 on all its values)
    bad = q.copy()
    amax = np.abs(a[9].reshape(-1, 32)).max(axis=1)
    frac = np.abs(np.log2(amax) - np.round(np.log2(amax)))
    j = int(np.argmax(frac))                 # the block farthest from a power of two
    bad[9, 32 * j:32 * j + 32] *= 2.0
    # a dropped term: one whole K block missing from another row
    bad[20, 64:96] = 0.0
    # a transposed operand in a third row (the wrong row's values)
    bad[30] = q[31]
    got = bad @ b
    adj = ref.copy()
    for r, D, _ in mxa.operand_deltas(a, 1, b):
        adj[r] = mxa._select(got[r], adj[r], D)[0]
    for row in (9, 20, 30):
        assert not close(got[row], adj[row], 6e-2, 3e-2)[0], row


def test_candidates_cover_element_midpoints():
    # a value exactly between two E4M3 codes after scaling: both codes are candidates
    blk = np.zeros((32, 1))
    blk[0, 0] = 256.0          # exponent 0
    blk[1, 0] = 17.0           # midpoint of 16 and 18
    recs = mxa.block_candidates(blk)
    moved = {(j, i) for j, i, d in recs if i >= 0}
    assert (0, 1) in moved


def _swiglu_operand(seed, n=96, kdim=256):
    """Values shaped like the SwiGLU output A = silu(h_g) * h_u with h ~ N(0, 1)."""
    r = np.random.default_rng(seed)
    hg, hu = r.standard_normal((n, kdim)), r.standard_normal((n, kdim))
    return hg / (1.0 + np.exp(-hg)) * hu


def _truncating_roundtrip(a):
    """MX round trip with the element codes truncated toward zero instead of
    rounded to nearest even (a planted mistake, same block exponents)."""
    codes = np.unique(np.abs(mx.e4m3_round(np.linspace(0, 448, 200001))))
    blk = a.reshape(a.shape[0], -1, 32)
    X = mx.block_exponent(np.abs(blk).max(axis=2))
    s = np.abs(blk) / np.ldexp(1.0, X)[..., None]
    t = codes[np.searchsorted(codes, np.minimum(s, 448.0), side="right") - 1]
    return (np.sign(blk) * t * np.ldexp(1.0, X)[..., None]).reshape(a.shape)


def _adjusted(a, b, got, atol):
    ref = mx.mx_roundtrip(a, axis=1) @ b
    adj = ref.copy()
    tally = mxa.Tally(a.size)
    for r, D, ids in mxa.operand_deltas(a, 1, b):
        adj[r], taken = mxa._select(got[r], adj[r], D, atol)
        tally.add(ids, taken)
    return ref, adj, tally


@pytest.mark.parametrize("mistake", ["silu_gain_5pct", "e4m3_truncation"])
def test_subtle_mistakes_in_the_computed_operand_are_rejected(mistake):
    """Mistakes in how the computed operand is formed, sized just past the MXFP8
    tolerance (6e-2 / 3e-2): the adjusted reference must not absorb them.  (A 1%
    error in SiLU moves Y by about 1%, inside the 3e-2 relative tolerance itself,
    so no comparison at that tolerance can see it, adjusted or not.)"""
    a = _swiglu_operand(3)
    b = np.random.default_rng(4).standard_normal((a.shape[1], 128)) / np.sqrt(a.shape[1])
    if mistake == "silu_gain_5pct":
        got = mx.mx_roundtrip(1.05 * a, axis=1) @ b
    else:
        got = _truncating_roundtrip(a) @ b
    ref, adj, tally = _adjusted(a, b, got, atol=6e-2)
    assert not close(got, ref, 6e-2, 3e-2)[0]                 # visible without the adjustment
    ok_adj = close(got, adj, 6e-2, 3e-2)[0]
    frac = tally.as_dict()["mx_block_fraction"]
    assert not ok_adj or frac > MX_MAX_BLOCK_FRACTION, (frac, close(got, adj, 6e-2, 3e-2))
    # and the adjustment removed little of the error
    assert np.linalg.norm(got - adj) >= 0.8 * np.linalg.norm(got - ref)


def test_small_deltas_are_not_candidates():
    """A flip whose effect on every output element is below atol / 2 is never taken,
    whatever the residual looks like."""
    a = _swiglu_operand(5)
    b = np.random.default_rng(6).standard_normal((a.shape[1], 64)) / 64.0    # small effects
    ref = mx.mx_roundtrip(a, axis=1) @ b
    noise = np.random.default_rng(7).standard_normal(ref.shape) * 1e-2
    _, adj, tally = _adjusted(a, b, ref + noise, atol=6e-2)
    assert tally.as_dict()["mx_deltas_taken"] == 0
    np.testing.assert_array_equal(adj, ref)
