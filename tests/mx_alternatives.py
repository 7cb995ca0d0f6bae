"""Both outcomes of MXFP8 quantisation decisions taken on values at a boundary.

An MX operand is decided twice: the block's shared exponent floor(log2 amax) - 8,
then each element's nearest-even E4M3 code.  When the operand is a value the
layer computes (A from the saved H, dH, gA), the GPU's fp32 accumulation and the
oracle's fp64 one can store it in bf16 one or two ulps apart; a decision whose
input sits that close to its boundary (amax at a power of two, an element at the
midpoint of two E4M3 values) then goes either way, and both outcomes are correct
results of the MX contract.  They are visibly different: the amax element may
saturate at 448 on one side only, and the E4M3 step is 1/8 of the value at the
top of a binade.

Each decision is therefore re-taken with its input moved by +-WINDOW (relative).
Where the outcome changes, the changed dequantised values minus the oracle's
give a delta that enters the GEMM output linearly.  Only deltas that move some
element of the output vector by at least half the max-abs tolerance are
candidates: a smaller one cannot decide a comparison by itself, and admitting
every small delta would let the selection fit the residual's noise (a delta
smaller than the noise passes the test below by chance about half the time).
The reference a GPU output vector is compared with is the oracle's vector plus
those candidates that bring it closer to the GPU's (best first, each taken delta
reducing the squared residual by at least half its own squared norm).  Every
delta is computed by the oracle from the oracle's own values; the GPU output
only selects among them.  Inputs of the layer (x, dout, the weights) are never
decided this way: both sides quantise the same bf16 values.
"""
from __future__ import annotations

import numpy as np

from oracle import mx

BLOCK = 32
# bf16 ulps are 2^-8..2^-7 of a value; the computed values that decide a block
# exponent or an element code differ by up to a few ulps between the two sides
# (gA = g * A inherits A's difference, A inherits H's)
WINDOW = 2.0 ** -6
WINDOW_ELEM = 2.0 ** -6


def block_candidates(blk):
    """Decisions of the blocks in ``blk`` [b, M] (one block per column, along
    axis 0) that may go either way, as records (column j, i, delta): i = -1 for
    the block exponent (delta: the block's value change, length b), else the
    element at position i (delta: its value change, a scalar)."""
    blk = np.asarray(blk, np.float64)
    amax = np.abs(blk).max(axis=0)
    X = mx.block_exponent(amax)
    out = []
    q = None
    for f in (1.0 + WINDOW, 1.0 - WINDOW):
        Xa = mx.block_exponent(amax * f)
        for j in np.nonzero((Xa != X) & (amax > 0))[0]:
            if q is None:
                q = mx.mx_roundtrip(blk, axis=0)
            out.append((int(j), -1, mx.roundtrip_at(blk[:, j], Xa[j]) - q[:, j]))
    scale = np.ldexp(1.0, X)[None, :]
    s = np.abs(blk) / scale
    base = mx.e4m3_round(s)
    sign = np.where(np.signbit(blk), -1.0, 1.0)
    for f in (1.0 + WINDOW_ELEM, 1.0 - WINDOW_ELEM):
        alt = mx.e4m3_round(s * f)
        ii, jj = np.nonzero(alt != base)
        vals = sign[ii, jj] * (alt[ii, jj] - base[ii, jj]) * scale[0, jj]
        out.extend(zip(jj.tolist(), ii.tolist(), vals.tolist()))
    return out


def _select(got, ref, D, atol=0.0):
    """ref plus a subset of the deltas (rows of D) chosen best first: repeatedly
    take the delta that most reduces |got - ref|^2, while the reduction is at
    least half of that delta's own |d|^2 (a delta that only fits noise, or one
    that overlaps deltas already taken, is left out).  Deltas whose largest
    element is below atol / 2 are not candidates.  Returns (adjusted ref,
    indices of the deltas taken)."""
    if len(D) == 0:
        return ref, []
    D = np.asarray(D)
    big = np.abs(D).max(axis=1) >= 0.5 * atol
    r = np.asarray(got, np.float64) - ref
    n2 = np.einsum("ij,ij->i", D, D)
    c = D @ r
    out = ref.copy()
    free = (n2 > 0) & big
    taken = []
    for _ in range(len(D)):
        gain = np.where(free, 2.0 * c - n2, -np.inf)
        i = int(np.argmax(gain))
        if not free[i] or gain[i] < 0.5 * n2[i]:
            break
        out = out + D[i]
        c = c - D @ D[i]
        free[i] = False
        taken.append(i)
    return out, taken


class Tally:
    """What the adjustment did for one output tensor: decisions that could go
    either way (candidates), deltas taken, and the distinct 32-value blocks of the
    computed operand those deltas lie in, out of all its blocks."""

    def __init__(self, operand_elements):
        self.candidates = 0
        self.significant = 0
        self.taken = 0
        self.blocks = set()
        self.total_blocks = -(-int(operand_elements) // BLOCK)

    def add(self, ids, taken, significant=None):
        self.candidates += len(ids)
        self.significant += len(ids) if significant is None else int(significant)
        self.taken += len(taken)
        self.blocks.update(ids[i] for i in taken)

    def as_dict(self):
        return {"mx_candidates": self.candidates, "mx_significant": self.significant, "mx_deltas_taken": self.taken,
                "mx_blocks_touched": len(self.blocks), "mx_blocks_total": self.total_blocks,
                "mx_block_fraction": len(self.blocks) / max(1, self.total_blocks)}


def operand_deltas(v, axis, other):
    """Yields (index j along the non-block axis, output deltas [m, width], block id
    of each delta) for the computed operand ``v`` (2-D) quantised in blocks of 32
    along ``axis`` (from 0): its block at positions sl multiplies ``other[sl, :]``.
    A block id is (j, first position of the block)."""
    v = np.asarray(v, np.float64)
    vt = v if axis == 0 else v.T
    by = {}
    for lo in range(0, vt.shape[0], BLOCK):
        sl = slice(lo, min(lo + BLOCK, vt.shape[0]))
        for j, i, d in block_candidates(vt[sl, :]):
            by.setdefault(j, []).append((lo, i, d))
    for j, recs in by.items():
        D = np.empty((len(recs), other.shape[1]))
        for n, (lo, i, d) in enumerate(recs):
            if i < 0:
                D[n] = d @ other[lo:lo + len(d), :]
            else:
                D[n] = d * other[lo + i, :]
        yield j, D, [(j, lo) for lo, _, _ in recs]


# ---------------------------------------------------------------- per output


def _nsig(D, atol):
    return int((np.abs(np.asarray(D)).max(axis=1) >= 0.5 * atol).sum()) if len(D) else 0


def adjust_forward(plan, y_gpu, o_gpu, Y, O, A, w2_mx, atol=0.0):
    """Y rows = A rows (quantised along f) times W2_e^T (w2_mx(e): oracle MX round
    trip of W2_e [d, f]); O sums the gated rows of each token.  Returns
    (Y reference, O reference, Tally)."""
    Yadj = np.array(Y, np.float64, copy=True)
    tally = Tally(np.asarray(A).size)
    for e in range(plan.E):
        a, b = int(plan.offsets[e]), int(plan.offsets[e + 1])
        if a == b:
            continue
        for r, D, ids in operand_deltas(A[a:b], 1, w2_mx(e).T):
            Yadj[a + r], taken = _select(np.asarray(y_gpu[a + r], np.float64), Yadj[a + r], D, atol)
            tally.add([(a + r, lo) for _, lo in ids], taken, _nsig(D, atol))
    Oadj = np.array(O, np.float64, copy=True)
    g = plan.gate_of_row
    for t in range(plan.T):
        for r in plan.tok_rows[plan.tok_ptr[t]:plan.tok_ptr[t + 1]]:
            Oadj[t] += g[r] * (Yadj[r] - Y[r])
    return Yadj, Oadj, tally


def adjust_dx(plan, dx_gpu, dx_ref, dH, w1_mx_k, atol=0.0):
    """dx_perm rows = dH rows (quantised along 2f) times W1_e (w1_mx_k(e): oracle
    MX round trip of W1_e [2f, d] along 2f); dx sums the rows of each token.
    Returns (dx reference, Tally)."""
    per_row = {}
    tally = Tally(np.asarray(dH).size)
    for e in range(plan.E):
        a, b = int(plan.offsets[e]), int(plan.offsets[e + 1])
        if a == b:
            continue
        for r, D, ids in operand_deltas(dH[a:b], 1, w1_mx_k(e)):
            per_row[a + r] = (D, [(a + r, lo) for _, lo in ids])
    adj = np.array(dx_ref, np.float64, copy=True)
    for t in range(plan.T):
        rows = [int(r) for r in plan.tok_rows[plan.tok_ptr[t]:plan.tok_ptr[t + 1]] if int(r) in per_row]
        if rows:
            D = np.concatenate([per_row[r][0] for r in rows])
            ids = [i for r in rows for i in per_row[r][1]]
            adj[t], taken = _select(np.asarray(dx_gpu[t], np.float64), adj[t], D, atol)
            tally.add(ids, taken, _nsig(D, atol))
    return adj, tally


def adjust_wgrad(computed, other, got, ref, rows, atol=0.0):
    """Weight gradient of one expert, both operands quantised along its tokens.

    dW1_e = dH_e^T X_e: computed = dH_e [n, 2f], other = X_e [n, d]; column c of
    dH_e moves row c of dW1_e (rows=True).  dW2_e = dO_e^T gA_e: computed = gA_e
    [n, f], other = dO_e [n, d]; column j of gA_e moves column j of dW2_e.
    Returns (reference, Tally)."""
    oq = mx.mx_roundtrip(other, axis=0)
    adj = np.array(ref, np.float64, copy=True)
    tally = Tally(np.asarray(computed).size)
    for j, D, ids in operand_deltas(computed, 0, oq):
        if rows:
            adj[j], taken = _select(np.asarray(got[j], np.float64), adj[j], D, atol)
        else:
            adj[:, j], taken = _select(np.asarray(got[:, j], np.float64), adj[:, j], D, atol)
        tally.add(ids, taken, _nsig(D, atol))
    return adj, tally
