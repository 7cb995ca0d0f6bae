"""CPU checks of the boundary-decision alternatives used by the MXFP8 parity
tests: a result that took the other side of a boundary decision is accepted,
and a result with a genuine mistake is still rejected."""
import numpy as np

import mx_alternatives as mxa
from helpers import close
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
    for r, D in mxa.operand_deltas(a, 1, b):
        adj[r] = mxa._select(got[r], adj[r], D)
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
    for r, D in mxa.operand_deltas(a, 1, b):
        adj[r] = mxa._select(got[r], adj[r], D)
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
