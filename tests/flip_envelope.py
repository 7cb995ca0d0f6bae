"""How far one bf16 storage step of an intermediate can move an output element.

The oracle and the GPU store the same intermediates in bf16 (H, A from H, Y,
dH, gA, dX_perm), but they round values computed in float64 and float32
respectively.  Where such a value lies within float32 rounding error of the
midpoint between two bf16 neighbours, the two sides store neighbouring bf16
values: a one-step difference of 2^-8..2^-7 of the value, in a small fraction of
the elements.  Downstream, an output element that sums many terms moves by that
step times the term's other factor.  For elements of large magnitude, or with
large terms that cancel, that exceeds an absolute 2e-2 although both results
are correct to the stored precision.

For each compared output this module gives, per element, m = the magnitude of
the largest single term through which such a step can enter (the oracle's own
values, never the GPU's).  An element that misses the literal bar is accepted
when its error is within FLIP * m more, FLIP = 2^-6 (a few one-step
differences of that largest term).  Sensitivities of A to its stored inputs:
A = silu(hg) hu, so a step in hu moves A by up to 2^-7 |silu(hg) hu| and a step
in hg by up to 2^-7 |hg silu'(hg) hu|; the scale used is
|hu| (|silu(hg)| + |hg silu'(hg)|), and likewise for dH through silu''.
"""
from __future__ import annotations

import numpy as np

from oracle import moe_oracle as mo

FLIP = 2.0 ** -6


def _d2silu(x):
    s = 1.0 / (1.0 + np.exp(-x))
    return s * (1.0 - s) * (2.0 + x * (1.0 - 2.0 * s))


class Envelope:
    """Largest-term magnitudes of the layer's outputs for one plan (or sub-plan).

    ``fw``/``bw`` are the oracle's forward/backward results on ``plan``; ``w1``,
    ``w2`` index per expert (arrays or LazyExperts).  Every method takes flat
    indices into the compared array and returns m at those elements."""

    def __init__(self, plan, x, w_gate, w1, w2, fw, bw=None, dout=None, dense_dz=False):
        self.plan, self.x, self.wg = plan, np.asarray(x, np.float64), np.asarray(w_gate, np.float64)
        self.w1, self.w2, self.fw, self.bw = w1, w2, fw, bw
        self.dout = None if dout is None else np.asarray(dout, np.float64)
        self.dense = dense_dz
        H = fw["H"]
        f = H.shape[1] // 2
        self.f = f
        hg, hu = H[:, :f], H[:, f:]
        self.ascale = np.abs(hu) * (np.abs(mo.silu(hg)) + np.abs(hg * mo.dsilu(hg)))
        g = plan.gate_of_row
        self.rows_of = [plan.tok_rows[plan.tok_ptr[t]:plan.tok_ptr[t + 1]] for t in range(plan.T)]
        if bw is not None:
            dA = g[:, None] * bw["dAp"]
            self.dhscale = np.concatenate(
                [np.abs(dA) * np.abs(hu) * (np.abs(mo.dsilu(hg)) + np.abs(hg * _d2silu(hg))),
                 np.abs(dA) * (np.abs(mo.silu(hg)) + np.abs(hg * mo.dsilu(hg)))], axis=1)
            self.m_ds = (np.abs(bw["dAp"]) * self.ascale).max(axis=1) if f else np.zeros(plan.N)
            self.m_dl = np.zeros(plan.T)
            np.add.at(self.m_dl, plan.token_of_row, g * self.m_ds)

    # ------------------------------------------------------------ forward
    def Y(self, idx):
        r, i = np.unravel_index(idx, (self.plan.N, self.x.shape[1]))
        e = self.plan.expert_of_row[r]
        return np.array([(self.ascale[rr] * np.abs(np.asarray(self.w2[ee])[ii])).max()
                         for rr, ii, ee in zip(r, i, e)])

    def O(self, idx):
        t, i = np.unravel_index(idx, (self.plan.T, self.x.shape[1]))
        g, Y = self.plan.gate_of_row, self.fw["Y"]
        out = []
        for tt, ii in zip(t, i):
            rows = self.rows_of[tt]
            my = self.Y(np.asarray(rows) * self.x.shape[1] + ii) if len(rows) else np.zeros(0)
            out.append(float((g[rows] * (np.abs(Y[rows, ii]) + my)).sum()))
        return np.array(out)

    # ------------------------------------------------------------ backward
    def dS(self, idx):
        return self.m_ds[idx]

    def dlogits(self, idx):
        t, _ = np.unravel_index(idx, (self.plan.T, self.plan.E))
        return self.m_dl[t]

    def _dz_experts(self, t):
        if self.dense:
            return np.arange(self.plan.E)
        p = self.plan
        return np.union1d(p.expert_of_row[self.rows_of[t]], p.topk_idx[t])

    def dx(self, idx):
        t, j = np.unravel_index(idx, (self.plan.T, self.x.shape[1]))
        p, dxp = self.plan, self.bw["dx_perm"]
        out = []
        for tt, jj in zip(t, j):
            m = 0.0
            for r in self.rows_of[tt]:
                w1c = np.abs(np.asarray(self.w1[p.expert_of_row[r]])[:, jj])
                m += abs(dxp[r, jj]) + float((self.dhscale[r] * w1c).max())
            m += self.m_dl[tt] * float(np.abs(self.wg[self._dz_experts(tt), jj]).sum())
            out.append(m)
        return np.array(out)

    def _expert_rows(self, e):
        return slice(int(self.plan.offsets[e]), int(self.plan.offsets[e + 1]))

    def dw1(self, e, idx):
        sl = self._expert_rows(e)
        i, j = np.unravel_index(idx, (2 * self.f, self.x.shape[1]))
        dh = self.dhscale[sl]
        xp = np.abs(self.x[self.plan.token_of_row[sl]])
        return np.array([(dh[:, ii] * xp[:, jj]).max() if dh.shape[0] else 0.0 for ii, jj in zip(i, j)])

    def dw2(self, e, idx):
        sl = self._expert_rows(e)
        i, j = np.unravel_index(idx, (self.x.shape[1], self.f))
        do = np.abs(self.dout[self.plan.token_of_row[sl]])
        ga = np.abs(self.plan.gate_of_row[sl])[:, None] * self.ascale[sl]
        return np.array([(do[:, ii] * ga[:, jj]).max() if do.shape[0] else 0.0 for ii, jj in zip(i, j)])

    def dw_gate(self, idx, experts=None):
        """experts: the rows compared (default all E), in the compared order."""
        experts = np.arange(self.plan.E) if experts is None else np.asarray(experts)
        e_i, j = np.unravel_index(idx, (len(experts), self.x.shape[1]))
        p = self.plan
        out = []
        for ei, jj in zip(e_i, j):
            e = experts[ei]
            if self.dense:
                toks = np.arange(p.T)
            else:
                toks = np.union1d(p.token_of_row[self._expert_rows(e)],
                                  np.nonzero((p.topk_idx == e).any(axis=1))[0])
            out.append(float((self.m_dl[toks] * np.abs(self.x[toks, jj])).max()) if len(toks) else 0.0)
        return np.array(out)
