"""CPU oracle for the token-choice top-k MoE FFN layer (forward and backward).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP library.

Plain, slow, obviously-correct numpy in float64.  Every function names the
passage of the source pages that defines what it computes:

* "Beam" blog (hncyxsy.com), section 2.2: the MoE layer replaces the FFN; the
  router is a d_model x N matrix, top-k experts are chosen from its scores and
  the output is the gate-weighted sum of the chosen experts' outputs.
* "Beam" blog, section 5.3: the reference MoELayer -- gate = Linear without bias,
  top-k over the logits, softmax over the k selected values, output accumulated
  over the k slots (the extraction lost the "+=").
* "Trinity Large" commentary (ai-stack.site), code example 1: top-k over the gate
  logits, then softmax over the k selected weights; example 2: per-expert counts
  by bincount; example 3: dispatch into per-expert lists and combine by token.
* SonicMoE article (techwalker.com), section 1: the router-score gradient is
  written as the inner product of dA' and A instead of dO and Y, so the expert
  outputs Y are never stored and A is recomputed.
* SonicMoE article, section 3: token rounding -- each expert's token count is
  moved to the nearest multiple of the GEMM tile (its example: 145 -> 128, not 256).
* Olmo-core 3 article (pwwt.cn), "three splits" section: tokens are written
  straight into per-expert input buffers (row-wise layout); grouped GEMM; an
  MXFP8 switch for the expert GEMMs.

Where the pages are silent the oracle takes these readings (each listed again in
the design notes):

* Expert = SwiGLU FFN without biases: a = silu(x W_g^T) * (x W_u^T), y = a W_2^T,
  with W1 = [W_g; W_u] stored gate rows first ([2f, d]) and W2 as [d, f].
* Top-k ties go to the lower expert index; top-k is stored in descending-logit order.
* Rows of one expert are ordered by ascending token index.
* The router bias (when present) is added to the logits before top-k and softmax
  and receives no gradient.
* Token rounding: count n -> tile * floor((n + tile/2) / tile) (half rounds up);
  if that exceeds T it rounds down instead.  Dropping removes the selected pairs
  with the smallest full-softmax probability P (ties: larger token first);
  padding adds the unselected tokens with the largest P (ties: smaller token
  first) with gate P_te / sum_{j in topk(t)} P_tj; kept pairs keep their gates.
* Precision "contract": the values the GPU path stores in bf16 (H, A, Y, dH,
  gA, dX_perm) are rounded to bf16 (round-to-nearest-even) at the same points
  here; everything else is fp64.  The router gradient dz enters the input- and
  router-weight gradients unrounded: the GPU carries it into those GEMMs as an
  unevaluated sum of two bf16 values (16 significant bits), whose residual is
  far below the fp32 outputs' tolerance.
* MXFP8 (OCP Microscaling v1.0, E4M3 elements, one E8M0 scale per 32 along K,
  shared exponent floor(log2 amax) - 8, saturating): see ``oracle/mx.py``.
* Routing variants (``RouteOpts``; Beam blog sections 2.2, 2.3 and 3.3,
  distributed-MoE article challenge 1, Trinity Large example 2):
  - gate "all": the gates are the full softmax over all E experts at the
    selected experts, not renormalised (section 2.2's formula); "topk" (the
    default) renormalises over the k selected (section 5.3, Trinity example 1).
    Pairs added by token rounding get P_te under "all".
  - noisy routing: a noise array [T,E] given by the caller is added to the
    logits before top-k and the gates (no learned noise scale: the page only
    says noise is added to the router scores); it gets no gradient.
  - capacity factor cf > 0: each expert keeps its first ceil(cf*T*k/E) pairs in
    token order, the rest are dropped (their tokens skip that expert); the
    kept gates are unchanged.  Not combined with token rounding.
  - load-balance loss lb = lb_coef * CV(Pbar)^2, Pbar = the batch mean of the
    per-token routing distributions P_t, CV = population standard deviation
    over the E entries divided by their mean (distributed-MoE article,
    challenge 1 formula); z-loss = z_coef * mean_t (log sum_e exp z_te)^2 (the
    page only names it; this is the usual definition).  Both are added to the
    training loss, so their gradients add to dlogits.
  - count_mse = mean_e (c_e - mean c)^2 over the per-expert counts of the
    selected pairs (Trinity Large example 2): a monitor, no gradient.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

from . import mx as _mx

# ----------------------------------------------------------------------------
# precision helpers


def bf16(a: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even).

    bfloat16 keeps 8 significant bits and float32's exponent range (normal down
    to 2^-126, subnormal quantum 2^-133).  Returns float64 holding bf16 values."""
    a = np.asarray(a, dtype=np.float64)
    out = np.zeros_like(a)
    fin = np.isfinite(a) & (a != 0)
    v = a[fin]
    _, ex = np.frexp(v)                       # v = m * 2^ex, 0.5 <= |m| < 1
    q_exp = np.maximum(ex - 8, -133)          # quantum of an 8-significant-bit value
    q = np.ldexp(1.0, q_exp)
    r = np.round(v / q) * q                   # numpy rounds half to even
    r[np.abs(r) > 3.3895313892515355e38] = np.inf * np.sign(r[np.abs(r) > 3.3895313892515355e38])
    out[fin] = r
    out[~fin] = a[~fin]
    # keep the sign of zero
    out[(a == 0)] = a[(a == 0)]
    return out


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    """silu(x) = x * sigmoid(x) (the SiLU of the Beam blog's MoELayer, section 5.3)."""
    return x * _sigmoid(x)


def dsilu(x):
    """d/dx silu(x) = s(x) * (1 + x * (1 - s(x)))."""
    s = _sigmoid(x)
    return s * (1.0 + x * (1.0 - s))


@dataclasses.dataclass(frozen=True)
class Precision:
    """Where the oracle rounds.

    ``store``: "bf16" rounds at the GPU's bf16 storage points; None keeps fp64.
    ``mx``:    quantise every expert-GEMM operand to MXFP8 along that GEMM's K."""
    store: Optional[str] = "bf16"
    mx: bool = False

    def st(self, a):
        return bf16(a) if self.store == "bf16" else np.asarray(a, dtype=np.float64)


CONTRACT = Precision("bf16", False)
TRUTH = Precision(None, False)
MX_CONTRACT = Precision("bf16", True)

# ----------------------------------------------------------------------------
# routing: F1-F3


@dataclasses.dataclass(frozen=True)
class RouteOpts:
    """Routing variants (see the module notes).  The defaults are the base layer."""
    gate: str = "topk"            # "topk": softmax over the k selected; "all": full softmax, no renormalisation
    capacity_factor: float = 0.0  # 0: no cap
    lb_coef: float = 0.0
    z_coef: float = 0.0

    @property
    def dense_dz(self) -> bool:
        """True when dlogits is nonzero beyond each token's selected experts."""
        return self.gate == "all" or self.lb_coef != 0.0 or self.z_coef != 0.0


BASE = RouteOpts()


def router_logits(x, w_gate, bias=None):
    """z[t, e] = <w_gate[e], x[t]> + b[e].

    Beam blog section 2.2 (router of shape d_model x N) and section 5.3 (gate is an
    nn.Linear(d_model, n_experts) -- stored [E, d])."""
    z = np.asarray(x, np.float64) @ np.asarray(w_gate, np.float64).T
    if bias is not None:
        z = z + np.asarray(bias, np.float64)[None, :]
    return z


def topk_softmax(z, k):
    """Top-k experts per token, then a softmax over the k selected logits.

    Trinity Large commentary, code example 1 (topk then softmax over the k
    weights); Beam blog section 5.3 (same order).  Ties go to the lower expert
    index; the k experts are listed in descending-logit order.
    Returns (topk_idx [T,k] int32, S [T,k] float64, P [T,E] float64) where P is
    the full softmax over all experts (needed by token rounding)."""
    z = np.asarray(z, np.float64)
    T, E = z.shape
    # stable argsort of -z: equal logits keep ascending expert order
    order = np.argsort(-z, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    zk = np.take_along_axis(z, idx.astype(np.int64), axis=1)
    m = zk.max(axis=1, keepdims=True)
    ek = np.exp(zk - m)
    S = ek / ek.sum(axis=1, keepdims=True)
    mz = z.max(axis=1, keepdims=True)
    ez = np.exp(z - mz)
    P = ez / ez.sum(axis=1, keepdims=True)
    return idx, S, P


# ----------------------------------------------------------------------------
# the routing plan: F4


@dataclasses.dataclass
class Plan:
    T: int
    E: int
    k: int
    topk_idx: np.ndarray       # [T,k] int32
    topk_gate: np.ndarray      # [T,k] float64 (softmax over the selected logits)
    probs: np.ndarray          # [T,E] float64 (full softmax)
    counts_raw: np.ndarray     # [E] int32, before rounding
    counts: np.ndarray         # [E] int32
    offsets: np.ndarray        # [E+1] int32
    token_of_row: np.ndarray   # [N] int32
    expert_of_row: np.ndarray  # [N] int32
    gate_of_row: np.ndarray    # [N] float64
    row_of_slot: np.ndarray    # [T,k] int32 (-1 when rounding dropped the pair)
    tok_ptr: np.ndarray        # [T+1] int32
    tok_rows: np.ndarray       # [N] int32, rows of token t in ascending row order

    @property
    def N(self) -> int:
        return int(self.offsets[-1])


def _assemble(T, E, k, topk_idx, S, P, pair_t, pair_e, pair_g):
    """Rows = token-expert pairs grouped by expert, ascending token inside a group.

    Olmo-core 3 article ("three splits" section): tokens go straight into
    contiguous per-expert input buffers; Trinity Large example 2: counts by
    bincount; example 3: dispatch per expert, then combine by token."""
    pair_t = np.asarray(pair_t, np.int64)
    pair_e = np.asarray(pair_e, np.int64)
    pair_g = np.asarray(pair_g, np.float64)
    order = np.lexsort((pair_t, pair_e))          # by expert, then token
    token_of_row = pair_t[order].astype(np.int32)
    expert_of_row = pair_e[order].astype(np.int32)
    gate_of_row = pair_g[order]
    counts = np.bincount(pair_e, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    counts_raw = np.bincount(np.asarray(topk_idx, np.int64).ravel(), minlength=E).astype(np.int32)
    # slot -> row
    row_of_slot = np.full((T, k), -1, np.int32)
    pos = {(int(t), int(e)): r for r, (t, e) in enumerate(zip(token_of_row, expert_of_row))}
    for t in range(T):
        for j in range(k):
            row_of_slot[t, j] = pos.get((t, int(topk_idx[t, j])), -1)
    # token -> rows (CSR), rows ascending
    tok_order = np.lexsort((np.arange(token_of_row.size), token_of_row))
    tok_rows = tok_order.astype(np.int32)
    tok_cnt = np.bincount(token_of_row.astype(np.int64), minlength=T)
    tok_ptr = np.zeros(T + 1, np.int32)
    tok_ptr[1:] = np.cumsum(tok_cnt)
    return Plan(T, E, k, np.asarray(topk_idx, np.int32), np.asarray(S, np.float64),
                np.asarray(P, np.float64), counts_raw, counts, offsets, token_of_row,
                expert_of_row, gate_of_row, row_of_slot, tok_ptr, tok_rows)


def plan_from_topk(topk_idx, S, P, E):
    """Plan without rounding: every (token, selected expert) pair is a row."""
    T, k = topk_idx.shape
    pair_t = np.repeat(np.arange(T), k)
    pair_e = np.asarray(topk_idx).ravel()
    pair_g = np.asarray(S).ravel()
    return _assemble(T, E, k, topk_idx, S, P, pair_t, pair_e, pair_g)


def round_tokens(topk_idx, S, P, E, tile, gate_all=False):
    """Token rounding to a multiple of the GEMM tile (SonicMoE article, section 3).

    For every expert e with n selected pairs, the target is the nearest multiple
    of ``tile`` (half rounds up; if that exceeds T, round down).  Fewer rows:
    drop the selected pairs with the smallest P (ties: larger token dropped
    first).  More rows: add the unselected tokens with the largest P (ties:
    smaller token first), with gate P_te / sum_{j in topk(t)} P_tj (P_te itself
    when the gates are not renormalised, ``gate_all``).  Kept pairs keep their
    gates."""
    topk_idx = np.asarray(topk_idx)
    T, k = topk_idx.shape
    sel = np.zeros((T, E), bool)
    sel[np.repeat(np.arange(T), k), topk_idx.ravel()] = True
    gate = np.zeros((T, E))
    gate[np.repeat(np.arange(T), k), topk_idx.ravel()] = np.asarray(S).ravel()
    ptop = np.take_along_axis(P, topk_idx.astype(np.int64), axis=1).sum(axis=1)
    keep = sel.copy()
    for e in range(E):
        n = int(sel[:, e].sum())
        target = ((n + tile // 2) // tile) * tile
        if target > T:
            target = (n // tile) * tile
        if target < n:
            cand = np.nonzero(sel[:, e])[0]
            # smallest P first; among equal P the larger token goes first
            order = np.lexsort((-cand, P[cand, e]))
            keep[cand[order[: n - target]], e] = False
        elif target > n:
            cand = np.nonzero(~sel[:, e])[0]
            # largest P first; among equal P the smaller token goes first
            order = np.lexsort((cand, -P[cand, e]))
            add = cand[order[: target - n]]
            keep[add, e] = True
            gate[add, e] = P[add, e] if gate_all else P[add, e] / ptop[add]
    pt, pe = np.nonzero(keep)
    return _assemble(T, E, k, topk_idx, S, P, pt, pe, gate[pt, pe])


def apply_capacity(plan: Plan, capacity_factor):
    """Capacity factor (Beam blog section 2.3; distributed-MoE article, challenge
    1): expert e keeps its first C = ceil(cf * T * k / E) pairs in token order and
    drops the others; kept pairs keep their gates."""
    C = int(math.ceil(capacity_factor * plan.T * plan.k / plan.E))
    rank = np.arange(plan.N) - plan.offsets[plan.expert_of_row]
    keep = rank < C
    return _assemble(plan.T, plan.E, plan.k, plan.topk_idx, plan.topk_gate, plan.probs,
                     plan.token_of_row[keep], plan.expert_of_row[keep], plan.gate_of_row[keep])


def route(x, w_gate, bias, k, round_tile=0, opts: RouteOpts = BASE, noise=None):
    """F1-F5: logits (+ the caller's noise), top-k, gates, optional token rounding
    or capacity cap, plan."""
    z = router_logits(x, w_gate, bias)
    if noise is not None:
        z = z + np.asarray(noise, np.float64)
    idx, S, P = topk_softmax(z, k)
    if opts.gate == "all":
        S = np.take_along_axis(P, idx.astype(np.int64), axis=1)
    elif opts.gate != "topk":
        raise ValueError(opts.gate)
    E = np.asarray(w_gate).shape[0]
    if round_tile and opts.capacity_factor:
        raise ValueError("token rounding and a capacity factor are not combined")
    if round_tile:
        plan = round_tokens(idx, S, P, E, round_tile, gate_all=(opts.gate == "all"))
    else:
        plan = plan_from_topk(idx, S, P, E)
    if opts.capacity_factor:
        plan = apply_capacity(plan, opts.capacity_factor)
    return z, plan


def _softmax_lse(z):
    z = np.asarray(z, np.float64)
    m = z.max(axis=1, keepdims=True)
    ez = np.exp(z - m)
    s = ez.sum(axis=1, keepdims=True)
    return ez / s, (m + np.log(s))[:, 0]


def router_losses(z, plan: Plan, opts: RouteOpts = BASE):
    """Router loss terms.  lb = lb_coef * CV(Pbar)^2 with Pbar_e = mean_t P_te and
    CV = (population std over e) / (mean over e) -- distributed-MoE article,
    challenge 1; z = z_coef * mean_t lse_t^2; count_mse = mean_e (c_e - mean c)^2
    of the selected-pair counts (Trinity Large example 2)."""
    P, lse = _softmax_lse(z)
    T, E = P.shape
    pbar = P.sum(axis=0) / T
    m = pbar.sum() / E
    var = ((pbar - m) ** 2).sum() / E
    cv2 = var / (m * m)
    c = plan.counts_raw.astype(np.float64)
    cm = c.sum() / E
    return {"pbar": pbar, "cv2": cv2, "lb": opts.lb_coef * cv2,
            "zloss": opts.z_coef * float((lse ** 2).sum()) / T,
            "count_mse": float(((c - cm) ** 2).sum()) / E}


# ----------------------------------------------------------------------------
# expert FFN forward: F6-F7


def _wexp(w, e):
    """Expert e's weight matrix in float64.  ``w`` is an array [E, ...] or any
    object whose ``w[e]`` converts to one (lets full-size checks avoid
    materialising every expert in float64)."""
    return np.asarray(w[e], dtype=np.float64)


def sub_plan(plan: Plan, tokens=None, experts=None) -> Plan:
    """The plan restricted to the rows of the given tokens and/or experts.

    Same routing decisions, fewer rows: used to evaluate the layer's outputs
    for a sample of tokens (or all rows of a sample of experts) one by one."""
    keep = np.ones(plan.N, bool)
    if tokens is not None:
        keep &= np.isin(plan.token_of_row, np.asarray(tokens))
    if experts is not None:
        keep &= np.isin(plan.expert_of_row, np.asarray(experts))
    return _assemble(plan.T, plan.E, plan.k, plan.topk_idx, plan.topk_gate, plan.probs,
                     plan.token_of_row[keep], plan.expert_of_row[keep], plan.gate_of_row[keep])


def _segments(plan):
    for e in range(plan.E):
        a, b = int(plan.offsets[e]), int(plan.offsets[e + 1])
        yield e, a, b


def _mxk(v, prec, axis):
    """Dequantised MXFP8 value of ``v`` with blocks of 32 along ``axis`` (identity if not MX)."""
    if not prec.mx:
        return v
    return _mx.mx_roundtrip(v, axis=axis)


def forward(x, w1, w2, plan: Plan, prec: Precision = CONTRACT) -> Dict[str, np.ndarray]:
    """Expert FFN on every row, then the gate-weighted combine.

    Row r = (t, e):  h = W1_e x_t (2f), a = silu(h_gate) * h_up, y = W2_e a.
    O_t = sum over the rows of t of gate_r * y_r (Beam blog sections 2.2 and 5.3;
    Trinity Large example 3 for the per-expert dispatch and combine by token).
    Under ``prec`` the stored H, A and Y are rounded to bf16; A is computed from
    the stored H."""
    x = np.asarray(x, np.float64)
    N = plan.N
    T, d = x.shape
    f = w2.shape[2]
    x_perm = x[plan.token_of_row]
    H = np.zeros((N, 2 * f))
    Y = np.zeros((N, d))
    for e, a, b in _segments(plan):
        if a == b:
            continue
        xe = _mxk(x_perm[a:b], prec, 1)
        w1e = _mxk(_wexp(w1, e), prec, 1)
        H[a:b] = xe @ w1e.T
    H = prec.st(H)
    A = prec.st(silu(H[:, :f]) * H[:, f:])
    for e, a, b in _segments(plan):
        if a == b:
            continue
        ae = _mxk(A[a:b], prec, 1)
        w2e = _mxk(_wexp(w2, e), prec, 1)
        Y[a:b] = ae @ w2e.T
    Y = prec.st(Y)
    O = np.zeros((T, d))
    g = plan.gate_of_row
    for t in range(T):
        for r in plan.tok_rows[plan.tok_ptr[t]:plan.tok_ptr[t + 1]]:
            O[t] += g[r] * Y[r]
    return {"x_perm": x_perm, "H": H, "A": A, "Y": Y, "O": O}


# ----------------------------------------------------------------------------
# backward: G1-G5


def router_backward(plan: Plan, dS, z=None, opts: RouteOpts = BASE):
    """Gradient of the loss w.r.t. the logits from the per-row gate gradients.

    Let K_t be the top-k experts of token t (softmax set, gates S) and A_t the
    experts holding a row of t after rounding.  Every gate has the form
    exp(z_te) / sum_{j in K_t} exp(z_tj), so
      dz_te = [e in A_t] g_te dS_te - [e in K_t] S_te * sum_{e' in A_t} g_te' dS_te'.
    Without rounding A_t = K_t and this is the softmax backward S*(dS - <S,dS>)
    of the top-k softmax (Trinity Large example 1; Beam blog section 5.3).

    With gate "all" every gate is P_te = exp(z_te) / sum_{all j} exp(z_tj), so
      dz_tj = [j in A_t] g_tj dS_tj - P_tj * sum_{e' in A_t} g_te' dS_te'.
    The load-balance loss adds P_t * (h - <h, P_t>) with h_e = (1/T) dlb/dPbar_e,
      dlb/dPbar_e = lb_coef * (2 (Pbar_e - m) / (E m^2) - 2 var / (E m^3)),
    and the z-loss adds (2 z_coef / T) lse_t P_t (``router_losses`` defines both)."""
    T, E = plan.T, plan.E
    dz = np.zeros((T, E))
    P = lse = None
    if opts.dense_dz:
        P, lse = _softmax_lse(z)
    for t in range(T):
        rows = plan.tok_rows[plan.tok_ptr[t]:plan.tok_ptr[t + 1]]
        acc = 0.0
        for r in rows:
            e = plan.expert_of_row[r]
            gds = plan.gate_of_row[r] * dS[r]
            dz[t, e] += gds
            acc += gds
        if opts.gate == "all":
            dz[t] -= P[t] * acc
        else:
            for j in range(plan.k):
                e = plan.topk_idx[t, j]
                dz[t, e] -= plan.topk_gate[t, j] * acc
    if opts.lb_coef:
        pbar = P.sum(axis=0) / T
        m = pbar.sum() / E
        var = ((pbar - m) ** 2).sum() / E
        h = opts.lb_coef * (2.0 * (pbar - m) / (E * m * m) - 2.0 * var / (E * m ** 3)) / T
        dz += P * (h[None, :] - (P @ h)[:, None])
    if opts.z_coef:
        dz += (2.0 * opts.z_coef / T) * lse[:, None] * P
    return dz


def backward(x, w_gate, w1, w2, plan: Plan, H, dout, prec: Precision = CONTRACT,
             weight_grads=True, logits=None, opts: RouteOpts = BASE) -> Dict[str, np.ndarray]:
    """Backward of the layer for the loss sum_t <O_t, dout_t>.

    SonicMoE article section 1: the router-score gradient of row r is
    dS_r = <dA'_r, A_r> with dA'_r = W2_e^T dO_t, which equals <dO_t, Y_r> since
    y = W2_e a -- so Y is neither stored nor recomputed; A is recomputed from the
    saved H.  The rest is the chain rule through SwiGLU and the two expert GEMMs,
    the router softmax (``router_backward``; with routing variants it also takes
    the router loss terms, which need the logits) and the router GEMM."""
    x = np.asarray(x, np.float64)
    w_gate = np.asarray(w_gate, np.float64)
    H = np.asarray(H, np.float64)
    dout = np.asarray(dout, np.float64)
    N = plan.N
    T, d = x.shape
    E = plan.E
    f = w2.shape[2]
    g = plan.gate_of_row
    x_perm = x[plan.token_of_row]
    do_perm = dout[plan.token_of_row]
    hg, hu = H[:, :f], H[:, f:]
    A = prec.st(silu(hg) * hu)                      # recomputed from the stored H
    dAp = np.zeros((N, f))
    for e, a, b in _segments(plan):
        if a == b:
            continue
        dAp[a:b] = _mxk(do_perm[a:b], prec, 1) @ _mxk(_wexp(w2, e), prec, 0)
    dS = np.einsum("rj,rj->r", dAp, A)
    dA = g[:, None] * dAp
    dH = prec.st(np.concatenate([dA * hu * dsilu(hg), dA * silu(hg)], axis=1))
    gA = prec.st(g[:, None] * A)
    dx_perm = np.zeros((N, d))
    # weight gradients: True -> full [E, ...] arrays; a collection of experts ->
    # dicts for those experts only; False -> not computed
    if weight_grads is True:
        dw1 = np.zeros((E, 2 * f, d))
        dw2 = np.zeros((E, d, f))
        wanted = range(E)
    elif weight_grads is False:
        dw1 = dw2 = None
        wanted = ()
    else:
        wanted = list(weight_grads)
        dw1 = {e: np.zeros((2 * f, d)) for e in wanted}
        dw2 = {e: np.zeros((d, f)) for e in wanted}
    for e, a, b in _segments(plan):
        if a == b:
            continue
        dx_perm[a:b] = _mxk(dH[a:b], prec, 1) @ _mxk(_wexp(w1, e), prec, 0)
        if e in wanted:
            dw1[e] = _mxk(dH[a:b], prec, 0).T @ _mxk(x_perm[a:b], prec, 0)
            dw2[e] = _mxk(do_perm[a:b], prec, 0).T @ _mxk(gA[a:b], prec, 0)
    dx_perm = prec.st(dx_perm)
    dz = router_backward(plan, dS, logits, opts)
    dx = np.zeros((T, d))
    for t in range(T):
        for r in plan.tok_rows[plan.tok_ptr[t]:plan.tok_ptr[t + 1]]:
            dx[t] += dx_perm[r]
    dx += dz @ w_gate
    dw_gate = dz.T @ x
    return {"dS": dS, "dH": dH, "gA": gA, "dx_perm": dx_perm, "dlogits": dz,
            "dx": dx, "dw_gate": dw_gate, "dw1": dw1, "dw2": dw2, "A": A, "dAp": dAp}


def layer(x, w_gate, bias, w1, w2, k, dout=None, round_tile=0, prec: Precision = CONTRACT,
          opts: RouteOpts = BASE, noise=None):
    """Route, forward and (when ``dout`` is given) backward in one call.  The
    training loss is sum_t <O_t, dout_t> + lb + zloss."""
    z, plan = route(x, w_gate, bias, k, round_tile, opts, noise)
    fw = forward(x, w1, w2, plan, prec)
    out = {"logits": z, "plan": plan, **fw, **router_losses(z, plan, opts)}
    if dout is not None:
        out.update(backward(x, w_gate, w1, w2, plan, fw["H"], dout, prec, logits=z, opts=opts))
    return out
