"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test fixes one part of the oracle to something independent: a library
routine (torch CPU in float64, torch's bf16 / float8 conversions), a closed form,
a brute-force enumeration on tiny inputs, the worked example printed on the
pages, or finite differences of the loss.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as mo
from oracle import mx
from oracle.tie_clearance import clear_ties, topk_tie_tokens
from helpers import tokens_reaching

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


def _tiny_layer(T=8, d=4, E=4, k=2, f=6, seed=1, bias=False):
    r = _rng(seed)
    x = r.standard_normal((T, d))
    wg = r.standard_normal((E, d))
    b = r.standard_normal(E) * 0.5 if bias else None
    w1 = r.standard_normal((E, 2 * f, d)) / math.sqrt(d)
    w2 = r.standard_normal((E, d, f)) / math.sqrt(f)
    dout = r.standard_normal((T, d))

    def redraw(xx, rows, attempt):
        rr = np.random.default_rng([seed, 7, attempt])
        xx = xx.copy()
        xx[rows] = rr.standard_normal((len(rows), d))
        return xx

    return x, wg, b, w1, w2, dout, redraw


# ---------------------------------------------------------------- precision


def test_bf16_rounding_matches_torch():
    r = _rng(3)
    v = (r.standard_normal(200000) * np.exp(r.uniform(-30, 30, 200000))).astype(np.float32)
    # exact halfway cases between neighbouring bf16 values
    base = torch.from_numpy(r.standard_normal(5000).astype(np.float32)).to(torch.bfloat16).float().numpy()
    ulp = np.abs(base) * 2.0 ** -8
    half = (base.astype(np.float64) + np.ldexp(1.0, np.frexp(base)[1] - 9)).astype(np.float32)
    v = np.concatenate([v, half, np.float32([0.0, -0.0, 1e-40, -3e-39])])
    ref = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
    got = mo.bf16(v.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    assert np.all(ulp >= 0)


# ---------------------------------------------------------------- routing


def test_topk_softmax_brute_force():
    r = _rng(4)
    T, E, k = 30, 7, 3
    z = np.round(r.standard_normal((T, E)), 1)       # coarse values: many exact ties
    idx, S, P = mo.topk_softmax(z, k)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-z[t, e], e))[:k]
        assert list(idx[t]) == order
        den = sum(math.exp(z[t, e]) for e in order)
        for j, e in enumerate(order):
            assert abs(S[t, j] - math.exp(z[t, e]) / den) < 1e-14
        den_all = sum(math.exp(z[t, e]) for e in range(E))
        for e in range(E):
            assert abs(P[t, e] - math.exp(z[t, e]) / den_all) < 1e-14


def test_duplicate_gate_rows_lower_index_wins():
    r = _rng(5)
    d, E = 16, 6
    x = np.abs(r.standard_normal((4, d)))
    wg = r.standard_normal((E, d)) * 0.01
    wg[2] = wg[5] = np.ones(d)           # identical rows, largest logits
    idx, S, _ = mo.topk_softmax(mo.router_logits(x, wg), 2)
    assert (idx[:, 0] == 2).all() and (idx[:, 1] == 5).all()
    np.testing.assert_allclose(S, 0.5, rtol=0, atol=1e-15)


def test_gate_invariants_and_special_cases():
    r = _rng(6)
    z = r.standard_normal((50, 9))
    _, S, P = mo.topk_softmax(z, 4)
    np.testing.assert_allclose(S.sum(1), 1.0, atol=1e-14)
    assert (S > 0).all() and (S <= 1).all()
    assert (np.diff(S, axis=1) <= 0).all()
    # k = E: the gates are the full softmax, in sorted order
    idx, S, P = mo.topk_softmax(z, 9)
    np.testing.assert_allclose(S, np.take_along_axis(P, idx.astype(np.int64), 1), atol=1e-15)
    np.testing.assert_allclose(P, torch.softmax(torch.from_numpy(z), -1).numpy(), atol=1e-15)
    # E = 1, k = 1: every gate is 1
    _, S1, _ = mo.topk_softmax(r.standard_normal((10, 1)), 1)
    assert (S1 == 1.0).all()


# ---------------------------------------------------------------- plan


def _check_plan_brute(plan, idx, S):
    T, k = idx.shape
    E = plan.E
    # counts by direct counting
    for e in range(E):
        assert plan.counts[e] == sum(1 for t in range(T) for j in range(k) if idx[t, j] == e)
    assert plan.counts.sum() == T * k and plan.offsets[-1] == T * k
    assert plan.offsets[0] == 0 and (np.diff(plan.offsets) == plan.counts).all()
    # bijection slot <-> row
    rows = plan.row_of_slot.ravel()
    assert sorted(rows.tolist()) == list(range(T * k))
    for t in range(T):
        for j in range(k):
            r = plan.row_of_slot[t, j]
            assert plan.token_of_row[r] == t and plan.expert_of_row[r] == idx[t, j]
            assert plan.gate_of_row[r] == S[t, j]
    for e in range(E):
        seg = plan.token_of_row[plan.offsets[e]:plan.offsets[e + 1]]
        assert (plan.expert_of_row[plan.offsets[e]:plan.offsets[e + 1]] == e).all()
        assert (np.diff(seg) > 0).all()
    # CSR token -> rows, rows ascending
    for t in range(T):
        rr = plan.tok_rows[plan.tok_ptr[t]:plan.tok_ptr[t + 1]]
        assert sorted(rr.tolist()) == rr.tolist()
        assert sorted(rr.tolist()) == sorted(plan.row_of_slot[t].tolist())


def test_plan_brute_force():
    r = _rng(7)
    for T, E, k in [(40, 5, 2), (17, 8, 8), (33, 1, 1), (64, 16, 4)]:
        z = r.standard_normal((T, E))
        idx, S, P = mo.topk_softmax(z, k)
        plan = mo.plan_from_topk(idx, S, P, E)
        _check_plan_brute(plan, idx, S)


# ---------------------------------------------------------------- token rounding


def test_rounding_worked_example_145():
    """SonicMoE article, section 3: 145 tokens on a 128 tile become 128 (17 dropped)."""
    with open(os.path.join(GOLDEN, "token_rounding_145.json")) as fh:
        g = json.load(fh)
    T, tile, n = g["T"], g["tile"], g["n_selected"]
    r = _rng(8)
    # expert 0 is chosen by the first n tokens, expert 1 by the rest (k = 1)
    z = np.zeros((T, 2))
    z[:n, 0] = 1.0 + r.uniform(0, 1, n)
    z[n:, 1] = 1.0 + r.uniform(0, 1, T - n)
    idx, S, P = mo.topk_softmax(z, 1)
    plan = mo.round_tokens(idx, S, P, 2, tile)
    assert plan.counts_raw[0] == n
    assert plan.counts[0] == g["n_rounded"]
    kept = set(plan.token_of_row[plan.offsets[0]:plan.offsets[1]].tolist())
    dropped = sorted(set(range(n)) - kept)
    assert len(dropped) == g["n_selected"] - g["n_rounded"]
    # the dropped ones have the smallest P for expert 0
    pk = sorted(P[list(kept), 0])
    assert max(P[dropped, 0]) < pk[0]


def _brute_round(idx, P, S, E, tile):
    """Per expert: the kept/added sets that maximise the sum of P (unique without ties)."""
    T, k = idx.shape
    sel = np.zeros((T, E), bool)
    sel[np.repeat(np.arange(T), k), idx.ravel()] = True
    pairs = {}
    ptop = np.take_along_axis(P, idx.astype(np.int64), 1).sum(1)
    gsel = {(t, int(idx[t, j])): S[t, j] for t in range(T) for j in range(k)}
    for e in range(E):
        chosen = [t for t in range(T) if sel[t, e]]
        n = len(chosen)
        lo, hi = (n // tile) * tile, (n // tile + 1) * tile
        target = lo if (n - lo) < (hi - n) else hi
        if target > T:
            target = lo
        assert abs(target - n) <= tile // 2 and target % tile == 0
        if target <= n:
            best = max(itertools.combinations(chosen, target), key=lambda c: sum(P[list(c), e]))
            for t in best:
                pairs[(t, e)] = gsel[(t, e)]
        else:
            others = [t for t in range(T) if not sel[t, e]]
            best = max(itertools.combinations(others, target - n), key=lambda c: sum(P[list(c), e]))
            for t in chosen:
                pairs[(t, e)] = gsel[(t, e)]
            for t in best:
                pairs[(t, e)] = P[t, e] / ptop[t]
    return pairs


@pytest.mark.parametrize("seed", range(6))
def test_rounding_brute_force_tile4(seed):
    r = _rng(100 + seed)
    T, E, k, tile = 12, 4, 2, 4
    z = r.standard_normal((T, E)) * 2
    idx, S, P = mo.topk_softmax(z, k)
    plan = mo.round_tokens(idx, S, P, E, tile)
    want = _brute_round(idx, P, S, E, tile)
    got = {(int(t), int(e)): g for t, e, g in zip(plan.token_of_row, plan.expert_of_row, plan.gate_of_row)}
    assert got.keys() == want.keys()
    for key in want:
        assert abs(got[key] - want[key]) < 1e-14
    assert (plan.counts % tile == 0).all()
    assert (np.abs(plan.counts - plan.counts_raw) <= tile // 2).all()
    # CSR and slot maps stay consistent after rounding
    for t in range(T):
        rr = plan.tok_rows[plan.tok_ptr[t]:plan.tok_ptr[t + 1]]
        assert (plan.token_of_row[rr] == t).all() and sorted(rr.tolist()) == rr.tolist()
        for j in range(k):
            r_ = plan.row_of_slot[t, j]
            if r_ >= 0:
                assert plan.token_of_row[r_] == t and plan.expert_of_row[r_] == idx[t, j]
            else:
                assert (t, int(idx[t, j])) not in got


# ---------------------------------------------------------------- forward


def _torch_dense_swiglu(x, w1, w2):
    xt = torch.from_numpy(x)
    h = xt @ torch.from_numpy(w1).T
    f = w2.shape[1]
    a = torch.nn.functional.silu(h[:, :f]) * h[:, f:]
    return (a @ torch.from_numpy(w2).T).numpy()


def test_single_expert_is_dense_swiglu():
    r = _rng(9)
    T, d, f = 20, 8, 12
    x = r.standard_normal((T, d))
    wg = r.standard_normal((1, d))
    w1 = r.standard_normal((1, 2 * f, d))
    w2 = r.standard_normal((1, d, f))
    out = mo.layer(x, wg, None, w1, w2, 1, prec=mo.TRUTH)
    np.testing.assert_allclose(out["O"], _torch_dense_swiglu(x, w1[0], w2[0]), rtol=1e-12, atol=1e-12)


def test_k_equals_E_is_dense_softmax_mixture():
    r = _rng(10)
    T, d, E, f = 16, 6, 4, 5
    x = r.standard_normal((T, d))
    wg = r.standard_normal((E, d))
    b = r.standard_normal(E)
    w1 = r.standard_normal((E, 2 * f, d))
    w2 = r.standard_normal((E, d, f))
    out = mo.layer(x, wg, b, w1, w2, E, prec=mo.TRUTH)
    p = torch.softmax(torch.from_numpy(x) @ torch.from_numpy(wg).T + torch.from_numpy(b), -1).numpy()
    ref = sum(p[:, e:e + 1] * _torch_dense_swiglu(x, w1[e], w2[e]) for e in range(E))
    np.testing.assert_allclose(out["O"], ref, rtol=1e-12, atol=1e-12)


def test_per_token_loop_matches_grouped_oracle():
    x, wg, b, w1, w2, _, _ = _tiny_layer(T=24, d=8, E=6, k=3, f=5, seed=11, bias=True)
    out = mo.layer(x, wg, b, w1, w2, 3, prec=mo.TRUTH)
    f = w2.shape[2]
    for t in range(x.shape[0]):
        z = wg @ x[t] + b
        order = sorted(range(6), key=lambda e: (-z[e], e))[:3]
        ex = [math.exp(z[e]) for e in order]
        acc = np.zeros(x.shape[1])
        for e, w in zip(order, ex):
            h = w1[e] @ x[t]
            a = np.array([h[i] / (1 + math.exp(-h[i])) * h[f + i] for i in range(f)])
            acc += (w / sum(ex)) * (w2[e] @ a)
        np.testing.assert_allclose(out["O"][t], acc, rtol=1e-12, atol=1e-13)


def test_contract_rounds_at_storage_points():
    x, wg, b, w1, w2, dout, _ = _tiny_layer(T=16, d=8, E=4, k=2, f=8, seed=12)
    out = mo.layer(x, wg, b, w1, w2, 2, dout=dout, prec=mo.CONTRACT)
    for key in ("H", "A", "Y", "dH", "gA", "dx_perm"):
        v = out[key]
        np.testing.assert_array_equal(v, torch.from_numpy(v).to(torch.bfloat16).double().numpy())


# ---------------------------------------------------------------- backward


def test_ds_identity_sonicmoe():
    """SonicMoE article, section 1: <dA', A> equals <dO, Y> row by row."""
    x, wg, b, w1, w2, dout, _ = _tiny_layer(T=32, d=16, E=8, k=3, f=12, seed=13, bias=True)
    out = mo.layer(x, wg, b, w1, w2, 3, dout=dout, prec=mo.TRUTH)
    plan = out["plan"]
    dsy = np.einsum("rd,rd->r", dout[plan.token_of_row], out["Y"])
    np.testing.assert_allclose(out["dS"], dsy, rtol=1e-12, atol=1e-12)


def _loss(x, wg, b, w1, w2, dout, k, tile):
    out = mo.layer(x, wg, b, w1, w2, k, round_tile=tile, prec=mo.TRUTH)
    return float((out["O"] * dout).sum()), out["plan"]


@pytest.mark.parametrize("tile", [0, 2])
def test_finite_differences(tile):
    x, wg, b, w1, w2, dout, redraw = _tiny_layer(T=8, d=4, E=4, k=2, f=6, seed=14, bias=True)
    x, _ = clear_ties(x, wg, b, 2, redraw, round_tile=tile, delta_z=1e-2, delta_p=1e-2)
    out = mo.layer(x, wg, b, w1, w2, 2, dout=dout, round_tile=tile, prec=mo.TRUTH)
    base_plan = out["plan"]
    h = 1e-6
    for name, arr, grad in (("x", x, out["dx"]), ("wg", wg, out["dw_gate"]),
                            ("w1", w1, out["dw1"]), ("w2", w2, out["dw2"])):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            args = {"x": x, "wg": wg, "w1": w1, "w2": w2}
            plus = arr.copy(); plus[i] += h
            minus = arr.copy(); minus[i] -= h
            args[name] = plus
            lp, pp = _loss(args["x"], args["wg"], b, args["w1"], args["w2"], dout, 2, tile)
            args[name] = minus
            lm, pm = _loss(args["x"], args["wg"], b, args["w1"], args["w2"], dout, 2, tile)
            assert (pp.token_of_row == base_plan.token_of_row).all()
            assert (pm.token_of_row == base_plan.token_of_row).all()
            num[i] = (lp - lm) / (2 * h)
        err = np.abs(num - grad).max() / max(1.0, np.abs(grad).max())
        assert err < 1e-6, (name, err)


def test_autograd_crosscheck_with_rounding():
    """torch.autograd in float64 through the same routed rows (gates as functions of z)."""
    x, wg, b, w1, w2, dout, redraw = _tiny_layer(T=12, d=6, E=5, k=2, f=4, seed=15, bias=True)
    x, _ = clear_ties(x, wg, b, 2, redraw, round_tile=2, delta_z=1e-2, delta_p=1e-2)
    out = mo.layer(x, wg, b, w1, w2, 2, dout=dout, round_tile=2, prec=mo.TRUTH)
    plan = out["plan"]
    X = torch.tensor(x, requires_grad=True)
    WG = torch.tensor(wg, requires_grad=True)
    W1 = torch.tensor(w1, requires_grad=True)
    W2 = torch.tensor(w2, requires_grad=True)
    z = X @ WG.T + torch.from_numpy(b)
    topk = torch.from_numpy(plan.topk_idx.astype(np.int64))
    den = torch.exp(z).gather(1, topk).sum(1)          # sum over the top-k set
    O = torch.zeros_like(X)
    f = w2.shape[2]
    for r in range(plan.N):
        t, e = int(plan.token_of_row[r]), int(plan.expert_of_row[r])
        g = torch.exp(z[t, e]) / den[t]
        h = W1[e] @ X[t]
        a = torch.nn.functional.silu(h[:f]) * h[f:]
        O = O.index_add(0, torch.tensor([t]), (g * (W2[e] @ a))[None])
    (O * torch.from_numpy(dout)).sum().backward()
    np.testing.assert_allclose(out["O"], O.detach().numpy(), atol=1e-12)
    for mine, ref in ((out["dx"], X.grad), (out["dw_gate"], WG.grad), (out["dw1"], W1.grad),
                      (out["dw2"], W2.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=1e-10, atol=1e-12)
    # kept top-k gates keep their softmax value (they need not sum to 1 any more)
    for r in range(plan.N):
        t, e = int(plan.token_of_row[r]), int(plan.expert_of_row[r])
        zz = z.detach().numpy()
        assert abs(plan.gate_of_row[r] - math.exp(zz[t, e]) / np.exp(zz[t, plan.topk_idx[t]]).sum()) < 1e-12


def test_single_expert_router_gradient_vanishes():
    r = _rng(16)
    T, d, f = 10, 6, 4
    x = r.standard_normal((T, d)); wg = r.standard_normal((1, d))
    w1 = r.standard_normal((1, 2 * f, d)); w2 = r.standard_normal((1, d, f))
    out = mo.layer(x, wg, None, w1, w2, 1, dout=r.standard_normal((T, d)), prec=mo.TRUTH)
    assert np.abs(out["dlogits"]).max() < 1e-12 and np.abs(out["dw_gate"]).max() < 1e-12


# ---------------------------------------------------------------- MXFP8


def test_e4m3_codes_match_torch_float8():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(mx.e4m3_decode(codes), ref)
    mag = np.abs(ref)
    np.testing.assert_array_equal(mx.e4m3_encode(np.signbit(ref).astype(np.int64), mag), codes)
    r = _rng(17)
    v = np.abs(r.standard_normal(100000) * np.exp(r.uniform(-12, 6, 100000)))
    v = v[v < 448]
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(mx.e4m3_round(v.astype(np.float32).astype(np.float64)), ref)


def test_mx_special_cases():
    r = _rng(18)
    # exactly representable block: max 448 * 2^s -> exact round trip, scale s
    vals = mx.e4m3_decode(r.integers(0, 0x7E, 32).astype(np.uint8))
    vals[3] = 448.0
    blk = vals * 2.0 ** -5
    codes, sc, deq = mx.quantize(blk)
    assert sc[0] == 127 - 5
    np.testing.assert_array_equal(deq, blk)
    # power-of-two max: scaled max is exactly 256
    blk = np.full(32, 2.0 ** 5) * np.sign(r.standard_normal(32))
    _, sc, deq = mx.quantize(blk)
    assert sc[0] == 127 + 5 - 8 and (deq == blk).all()
    # saturation: 500 has exponent 8 -> scale 2^0, clipped to 448
    blk = np.zeros(32); blk[0] = 500.0; blk[1] = -470.0; blk[2] = 1.0
    codes, sc, deq = mx.quantize(blk)
    assert sc[0] == 127 and deq[0] == 448.0 and deq[1] == -448.0 and deq[2] == 1.0
    # all-zero block
    codes, sc, deq = mx.quantize(np.zeros(64))
    assert (sc == 0).all() and (codes == 0).all() and (deq == 0).all()
    # partial trailing block and blocks along axis 0
    a = r.standard_normal((70, 3))
    codes, sc, deq = mx.quantize(a, axis=0)
    assert sc.shape == (3, 3) and codes.shape == a.shape
    for c in range(3):
        for bi in range(3):
            blk = a[bi * 32:(bi + 1) * 32, c]
            e = math.floor(math.log2(np.abs(blk).max())) - 8
            assert sc[bi, c] == e + 127
    # error bound: half an E4M3 ulp is at most 2^-4 of the value; saturation of
    # the block maximum (scaled into [256, 512), clipped at 448) loses at most 1/8
    v = r.standard_normal((16, 256))
    deq = mx.mx_roundtrip(v, axis=1)
    blkmax = np.repeat(np.abs(v.reshape(16, 8, 32)).max(-1), 32, axis=1)
    assert (np.abs(deq - v) <= np.maximum(np.abs(v) * 2.0 ** -4, blkmax * 2.0 ** -3) + 1e-300).all()
    unclipped = np.abs(v) / np.ldexp(1.0, np.frexp(blkmax)[1] - 9) < 448
    assert (np.abs(deq - v)[unclipped] <= np.abs(v)[unclipped] * 2.0 ** -4 + 2.0 ** -9 * blkmax[unclipped] / 256).all()


def test_mx_forced_exponent():
    # hand example: amax 3.984375 (just below 4) -> rule exponent -7, scaled 510,
    # saturated to 448 -> 3.5; with the exponent one higher the value is
    # 255 * 2^-6 -> nearest E4M3 is 256 -> 4.0
    b = np.zeros(32); b[0] = 3.984375; b[1] = -1.0; b[2] = 0.3
    assert mx.block_exponent(3.984375) == -7 and mx.block_exponent(4.0) == -6
    assert mx.block_exponent(0.0) == -127
    np.testing.assert_array_equal(mx.roundtrip_at(b, -7)[:2], [3.5, -1.0])
    np.testing.assert_array_equal(mx.roundtrip_at(b, -6)[:2], [4.0, -1.0])
    # 0.3 * 2^6 = 19.2 -> E4M3 step 2 in [16, 32) -> 20 -> 0.3125; at 2^7: 38.4 -> step 4 -> 40 -> 0.3125
    assert mx.roundtrip_at(b, -6)[2] == 0.3125 and mx.roundtrip_at(b, -7)[2] == 0.3125
    # at the rule's exponent it is the quantiser's round trip; scaling by 2 commutes
    r = _rng(23)
    for _ in range(20):
        blk = r.standard_normal(32) * np.exp(r.uniform(-8, 8))
        X = mx.block_exponent(np.abs(blk).max())
        np.testing.assert_array_equal(mx.roundtrip_at(blk, X), mx.mx_roundtrip(blk))
        np.testing.assert_array_equal(mx.roundtrip_at(2 * blk, X + 1), 2 * mx.roundtrip_at(blk, X))
    # array form: the exponents behind the quantiser's scale bytes
    v = r.standard_normal((40, 96)) * np.exp(r.uniform(-40, 40, (40, 1)))
    v[3, :32] = 0.0
    _, sc, _ = mx.quantize(v, axis=1)
    amax = np.abs(v.reshape(40, 3, 32)).max(-1)
    np.testing.assert_array_equal(mx.block_exponent(amax) + 127, sc.astype(np.int64))


def _worst_rel(got, ref):
    """Largest relative Frobenius error over the rows and over the columns."""
    err = got - ref
    rr = np.sqrt((err ** 2).sum(1) / np.maximum((ref ** 2).sum(1), 1e-300))
    cc = np.sqrt((err ** 2).sum(0) / np.maximum((ref ** 2).sum(0), 1e-300))
    return max(rr.max(), cc.max())


def _mx_pair(x, wg, b, w1, w2, dout, k):
    q = mo.layer(x, wg, b, w1, w2, k, dout=dout, prec=mo.Precision(None, True))
    t = mo.layer(x, wg, b, w1, w2, k, dout=dout, prec=mo.TRUTH)
    return q, t


def test_mx_blocks_run_along_each_gemms_k():
    """Operands whose rows or columns differ by up to 2^24 in scale: with blocks along
    each GEMM's K every output element stays close; blocks along the other axis flush
    the small rows/columns and fail.  One run per GEMM operand pair."""
    r = _rng(19)
    T, d, E, k, f = 256, 64, 2, 1, 64
    x = r.standard_normal((T, d)); wg = r.standard_normal((E, d)) * 0.01
    w1 = r.standard_normal((E, 2 * f, d)) / 8; w2 = r.standard_normal((E, d, f)) / 8
    dout = r.standard_normal((T, d))
    # scales in [2^-24, 1]: small enough to be flushed by a block holding a 1,
    # never large, so the SwiGLU nonlinearity sees ordinary magnitudes
    sc = lambda n, s: 2.0 ** (4 * ((np.arange(n) * 5 + s) % 7) - 24)
    one = lambda n: np.ones(n)

    def run(xr=None, xc=None, w1r=None, w1c=None, w2r=None, w2c=None, dr=None, dc=None):
        xr, xc, dr, dc = (v if v is not None else one(n) for v, n in ((xr, T), (xc, d), (dr, T), (dc, d)))
        w1r, w1c = (v if v is not None else one(n) for v, n in ((w1r, 2 * f), (w1c, d)))
        w2r, w2c = (v if v is not None else one(n) for v, n in ((w2r, d), (w2c, f)))
        return _mx_pair(x * np.outer(xr, xc), wg, None, w1 * np.outer(w1r, w1c)[None],
                        w2 * np.outer(w2r, w2c)[None], dout * np.outer(dr, dc), k)

    st, sd, r1, r2 = sc(T, 0), sc(T, 3), sc(2 * f, 1), sc(d, 2)
    cx, cd, q1, p2 = sc(d, 0), sc(d, 3), sc(d, 1), sc(f, 2)
    pp = np.concatenate([p2, p2])
    lim = 0.5       # a flushed row or column has relative error 1
    q, t = run(xr=st, w1r=r1)                                       # GEMM1: x, w1 along d
    assert _worst_rel(q["H"], t["H"]) < lim
    q, t = run(xr=st, w2r=r2)                                       # GEMM2: A, w2 along f
    assert _worst_rel(q["Y"], t["Y"]) < lim
    q, t = run(dr=sd, w2c=p2)                                       # dA': dout, w2 along d
    assert _worst_rel(q["dH"], t["dH"]) < lim
    q, t = run(dr=sd, w1c=q1)                                       # dX_perm: dH, w1 along 2f
    assert _worst_rel(q["dx_perm"], t["dx_perm"]) < lim
    q, t = run(xc=cx, w2c=p2)                                       # dW1: dH, x along tokens
    for e in range(E):
        if t["plan"].counts[e]:
            assert _worst_rel(q["dw1"][e], t["dw1"][e]) < lim
    ru = np.concatenate([one(f), sc(f, 4)])                         # scales A's columns linearly
    q, t = run(dc=cd, w1r=ru)                                       # dW2: dout, gA along tokens
    for e in range(E):
        if t["plan"].counts[e]:
            assert _worst_rel(q["dw2"][e], t["dw2"][e]) < lim


# ---------------------------------------------------------------- tie clearance


def test_tie_clearance_leaves_margin():
    x, wg, b, _, _, _, redraw = _tiny_layer(T=400, d=8, E=16, k=4, f=4, seed=20, bias=True)
    x2, n = clear_ties(x, wg, b, 4, redraw, delta_z=5e-2)
    assert n > 0
    assert topk_tie_tokens(mo.router_logits(x2, wg, b), 4, 5e-2).size == 0


# ---------------------------------------------------------------- more pins


@pytest.mark.parametrize("k", [1, 2])
def test_rounding_rounds_down_when_nearest_multiple_exceeds_T(k):
    """An expert chosen by every token: its nearest multiple of the tile lies past T,
    so it takes the largest multiple that fits.  The target is checked against an
    enumeration of every multiple of the tile in [0, T] (nearest, half up), and the
    kept pairs against the brute-force subset search."""
    T, E, tile = 6, 3, 4
    r = _rng(30 + k)
    z = r.standard_normal((T, E))
    z[:, 0] += 20.0                                   # expert 0 first for every token
    idx, S, P = mo.topk_softmax(z, k)
    plan = mo.round_tokens(idx, S, P, E, tile)
    assert plan.counts_raw[0] == T
    for e in range(E):
        n = int(plan.counts_raw[e])
        fits = [m for m in range(0, T + 1, tile)]
        # nearest multiple that fits; on a tie the larger one
        want = min(fits, key=lambda m: (abs(m - n), -m))
        assert plan.counts[e] == want, (e, n, plan.counts[e], want)
    assert plan.counts[0] == 4                        # 8 would be nearest, but 8 > T = 6
    want = _brute_round(idx, P, S, E, tile)
    got = {(int(t), int(e)): g for t, e, g in zip(plan.token_of_row, plan.expert_of_row, plan.gate_of_row)}
    assert got.keys() == want.keys()


def test_sub_plan_keeps_rows_and_results():
    """A sub-plan holds exactly the rows of the chosen tokens (or experts), in the
    same order, and the layer evaluated on it gives those tokens' outputs and
    gradients, and those experts' weight gradients, as on the full plan.  The
    router-weight gradient row of an expert needs only the tokens with a row there
    or the expert in their top-k (every other logit gradient at it is zero)."""
    x, wg, b, w1, w2, dout, redraw = _tiny_layer(T=40, d=8, E=6, k=2, f=4, seed=31, bias=True)
    x, _ = clear_ties(x, wg, b, 2, redraw, round_tile=4, delta_z=1e-3, delta_p=1e-3)
    for tile in (0, 4):
        full = mo.layer(x, wg, b, w1, w2, 2, dout=dout, round_tile=tile, prec=mo.CONTRACT)
        plan = full["plan"]
        toks = np.array([1, 5, 6, 17, 33])
        sub = mo.sub_plan(plan, tokens=toks)
        keep = np.isin(plan.token_of_row, toks)
        np.testing.assert_array_equal(sub.token_of_row, plan.token_of_row[keep])
        np.testing.assert_array_equal(sub.expert_of_row, plan.expert_of_row[keep])
        np.testing.assert_array_equal(sub.gate_of_row, plan.gate_of_row[keep])
        fw = mo.forward(x, w1, w2, sub, mo.CONTRACT)
        bw = mo.backward(x, wg, w1, w2, sub, fw["H"], dout, mo.CONTRACT, weight_grads=False)
        for key, a_, b_ in (("O", fw["O"], full["O"]), ("dx", bw["dx"], full["dx"]),
                            ("dlogits", bw["dlogits"], full["dlogits"])):
            np.testing.assert_allclose(a_[toks], b_[toks], rtol=1e-12, atol=1e-12, err_msg=key)
        np.testing.assert_allclose(fw["H"], full["H"][keep], rtol=1e-12, atol=1e-12)
        for e in range(plan.E):
            sub_e = mo.sub_plan(plan, experts=[e])
            assert (sub_e.expert_of_row == e).all() and sub_e.N == plan.counts[e]
            fe = mo.forward(x, w1, w2, sub_e, mo.CONTRACT)
            be = mo.backward(x, wg, w1, w2, sub_e, fe["H"], dout, mo.CONTRACT, weight_grads=[e])
            np.testing.assert_allclose(be["dw1"][e], full["dw1"][e], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(be["dw2"][e], full["dw2"][e], rtol=1e-12, atol=1e-12)
            reach = tokens_reaching(plan, e)
            sr = mo.sub_plan(plan, tokens=reach)
            fr = mo.forward(x, w1, w2, sr, mo.CONTRACT)
            br = mo.backward(x, wg, w1, w2, sr, fr["H"], dout, mo.CONTRACT, weight_grads=False)
            np.testing.assert_allclose(br["dw_gate"][e], full["dw_gate"][e], rtol=1e-12, atol=1e-12)


def test_contract_rounding_placement_torch():
    """The contract's bf16 storage points re-derived with torch (float64 arithmetic,
    torch's bf16 conversion, the SiLU derivative from autograd): H rounded after
    the up GEMM; A from the rounded H, then rounded; Y rounded; dS from the
    unrounded dA' and the rounded A; dH and gA rounded; dX_perm rounded; the router
    gradient dz entering dx and dW_g unrounded.  Values must agree to float64
    round-off and the rounded ones bit for bit."""
    x, wg, b, w1, w2, dout, redraw = _tiny_layer(T=24, d=8, E=4, k=2, f=6, seed=32, bias=True)
    x, _ = clear_ties(x, wg, b, 2, redraw)
    out = mo.layer(x, wg, b, w1, w2, 2, dout=dout, prec=mo.CONTRACT)
    plan = out["plan"]
    q = lambda t: t.to(torch.bfloat16).double()
    tor = torch.from_numpy(plan.token_of_row.astype(np.int64))
    X, DO = torch.from_numpy(x), torch.from_numpy(dout)
    g = torch.from_numpy(plan.gate_of_row)
    f = w2.shape[2]
    xp, dop = X[tor], DO[tor]
    ex = torch.from_numpy(plan.expert_of_row.astype(np.int64))
    W1, W2 = torch.from_numpy(w1)[ex], torch.from_numpy(w2)[ex]     # per-row expert weights
    H = q(torch.einsum("rod,rd->ro", W1, xp))
    hg = H[:, :f].clone().requires_grad_(True)
    act = torch.nn.functional.silu(hg)
    (dsilu,) = torch.autograd.grad(act.sum(), hg)
    act = act.detach()
    A = q(act * H[:, f:])
    Y = q(torch.einsum("rdf,rf->rd", W2, A))
    dAp = torch.einsum("rdf,rd->rf", W2, dop)
    dS = (dAp * A).sum(1)
    dA = g[:, None] * dAp
    dH = q(torch.cat([dA * H[:, f:] * dsilu, dA * act], 1))
    gA = q(g[:, None] * A)
    dxp = q(torch.einsum("rod,ro->rd", W1, dH))
    dz = torch.from_numpy(out["dlogits"])
    dx = torch.zeros_like(X).index_add(0, tor, dxp) + dz @ torch.from_numpy(wg)
    dwg = dz.T @ X
    for key, ref, rounded in (("H", H, True), ("A", A, True), ("Y", Y, True), ("dS", dS, False),
                              ("dH", dH, True), ("gA", gA, True), ("dx_perm", dxp, True), ("dx", dx, False),
                              ("dw_gate", dwg, False)):
        if rounded:
            np.testing.assert_array_equal(out[key], ref.numpy(), err_msg=key)
        else:
            np.testing.assert_allclose(out[key], ref.numpy(), rtol=1e-12, atol=1e-12, err_msg=key)
