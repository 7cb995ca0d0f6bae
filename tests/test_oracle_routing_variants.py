"""Pins of the oracle's routing variants (gate normalisation, noisy routing,
capacity factor, load-balance loss, z-loss, count monitor).

Each definition is fixed by something outside the oracle: a closed form worked
by hand, torch's softmax / logsumexp, brute-force enumeration, or finite
differences of the training loss sum <O, dout> + lb + zloss.
"""
import math

import numpy as np
import pytest
import torch

from oracle import moe_oracle as mo
from oracle.tie_clearance import clear_ties


def _tiny(T=8, d=4, E=4, k=2, f=6, seed=1, bias=True):
    r = np.random.default_rng(seed)
    x = r.standard_normal((T, d))
    wg = r.standard_normal((E, d))
    b = r.standard_normal(E) * 0.5 if bias else None
    w1 = r.standard_normal((E, 2 * f, d)) / math.sqrt(d)
    w2 = r.standard_normal((E, d, f)) / math.sqrt(f)
    dout = r.standard_normal((T, d))

    def redraw(xx, rows, attempt):
        rr = np.random.default_rng([seed, 11, attempt])
        xx = xx.copy()
        xx[rows] = rr.standard_normal((len(rows), d))
        return xx

    return x, wg, b, w1, w2, dout, redraw


# ---------------------------------------------------------------- loss values


def test_load_balance_two_experts_closed_form():
    """E = 2, P_t = (p_t, 1 - p_t): Pbar = (q, 1 - q) with q = mean p, mean 1/2,
    population std |q - 1/2|, so CV^2 = (2q - 1)^2 (worked by hand)."""
    p = np.array([0.9, 0.6, 0.2])
    z = np.log(np.stack([p, 1 - p], axis=1))
    plan = mo.plan_from_topk(*mo.topk_softmax(z, 1)[:2], mo.topk_softmax(z, 1)[2], 2)
    out = mo.router_losses(z, plan, mo.RouteOpts(lb_coef=0.25))
    q = p.mean()
    assert abs(out["cv2"] - (2 * q - 1) ** 2) < 1e-12
    assert abs(out["lb"] - 0.25 * (2 * q - 1) ** 2) < 1e-12
    np.testing.assert_allclose(out["pbar"], [q, 1 - q], atol=1e-15)


def test_load_balance_uniform_routing_is_zero():
    z = np.zeros((5, 6))
    idx, S, P = mo.topk_softmax(z, 2)
    out = mo.router_losses(z, mo.plan_from_topk(idx, S, P, 6), mo.RouteOpts(lb_coef=3.0))
    assert out["cv2"] < 1e-28 and out["lb"] < 1e-27


def test_z_loss_closed_form_and_torch():
    """z = c (constant over experts): lse = c + log E.  General z: torch.logsumexp."""
    E, T = 8, 4
    c = np.array([0.0, 1.5, -2.0, 3.0])
    z = np.repeat(c[:, None], E, axis=1)
    idx, S, P = mo.topk_softmax(z, 2)
    out = mo.router_losses(z, mo.plan_from_topk(idx, S, P, E), mo.RouteOpts(z_coef=0.1))
    assert abs(out["zloss"] - 0.1 * np.mean((c + math.log(E)) ** 2)) < 1e-12
    z = np.random.default_rng(3).standard_normal((T, E)) * 4
    idx, S, P = mo.topk_softmax(z, 2)
    out = mo.router_losses(z, mo.plan_from_topk(idx, S, P, E), mo.RouteOpts(z_coef=0.5))
    ref = 0.5 * (torch.logsumexp(torch.from_numpy(z), 1) ** 2).mean().item()
    assert abs(out["zloss"] - ref) < 1e-12


def test_count_mse_trinity_example_2():
    """Counts of the selected experts, then mean squared deviation from their mean:
    counts (3, 1, 0, 0) -> mean 1 -> (4 + 0 + 1 + 1) / 4 = 1.5."""
    idx = np.array([[0], [0], [0], [1]], np.int32)
    S = np.ones((4, 1))
    P = np.full((4, 4), 0.25)
    plan = mo.plan_from_topk(idx, S, P, 4)
    z = np.zeros((4, 4))
    assert mo.router_losses(z, plan)["count_mse"] == 1.5


# ---------------------------------------------------------------- routing


def test_gate_all_is_the_full_softmax():
    x, wg, b, *_ = _tiny(T=9, E=6, seed=2)
    z, plan = mo.route(x, wg, b, 3, opts=mo.RouteOpts(gate="all"))
    P = torch.softmax(torch.from_numpy(z), 1).numpy()
    np.testing.assert_allclose(plan.topk_gate, np.take_along_axis(P, plan.topk_idx.astype(np.int64), 1),
                               rtol=1e-13)
    assert np.all(plan.topk_gate.sum(1) < 1.0)


def test_gate_all_equals_topk_when_k_is_E():
    x, wg, b, w1, w2, dout, _ = _tiny(T=6, E=3, k=3, seed=4)
    a = mo.layer(x, wg, b, w1, w2, 3, dout=dout, prec=mo.TRUTH)
    g = mo.layer(x, wg, b, w1, w2, 3, dout=dout, prec=mo.TRUTH, opts=mo.RouteOpts(gate="all"))
    for key in ("O", "dx", "dw_gate", "dlogits", "dw1"):
        np.testing.assert_allclose(g[key], a[key], rtol=1e-12, atol=1e-13)


def test_noise_shifts_the_selection_and_zero_noise_is_identity():
    x, wg, b, *_ = _tiny(T=7, E=5, seed=5)
    z0, p0 = mo.route(x, wg, b, 2)
    z1, p1 = mo.route(x, wg, b, 2, noise=np.zeros((7, 5)))
    assert (p0.token_of_row == p1.token_of_row).all() and (p0.expert_of_row == p1.expert_of_row).all()
    noise = np.zeros((7, 5))
    noise[0, p0.topk_idx[0, 0]] = -100.0          # push token 0's best expert out
    z2, p2 = mo.route(x, wg, b, 2, noise=noise)
    zz = z0 + noise
    brute = np.argsort(-zz[0], kind="stable")[:2]
    assert list(p2.topk_idx[0]) == list(brute) and p0.topk_idx[0, 0] not in p2.topk_idx[0]
    np.testing.assert_allclose(z2, zz)


@pytest.mark.parametrize("cf", [0.5, 0.75, 1.0, 1.3])
def test_capacity_brute_force(cf):
    """Walk the tokens in order; each expert accepts pairs until it holds C."""
    x, wg, b, *_ = _tiny(T=11, E=3, k=2, seed=6)
    z, base = mo.route(x, wg, b, 2)
    _, plan = mo.route(x, wg, b, 2, opts=mo.RouteOpts(capacity_factor=cf))
    C = math.ceil(cf * 11 * 2 / 3)
    held = [0, 0, 0]
    kept = set()
    for t in range(11):
        for e in base.topk_idx[t]:
            if held[e] < C:
                held[e] += 1
                kept.add((t, int(e)))
    got = set(zip(plan.token_of_row.tolist(), plan.expert_of_row.tolist()))
    assert got == kept
    assert (plan.counts <= C).all() and (plan.counts_raw == base.counts_raw).all()
    for r in range(plan.N):   # kept pairs keep their gates
        t, e = plan.token_of_row[r], plan.expert_of_row[r]
        j = list(base.topk_idx[t]).index(e)
        assert plan.gate_of_row[r] == base.topk_gate[t, j]


def test_capacity_large_factor_is_identity():
    x, wg, b, *_ = _tiny(T=9, E=4, seed=7)
    _, a = mo.route(x, wg, b, 2)
    _, c = mo.route(x, wg, b, 2, opts=mo.RouteOpts(capacity_factor=4.0))
    assert (a.token_of_row == c.token_of_row).all() and (a.gate_of_row == c.gate_of_row).all()


# ---------------------------------------------------------------- gradients


def _total_loss(x, wg, b, w1, w2, dout, k, tile, opts, noise):
    out = mo.layer(x, wg, b, w1, w2, k, round_tile=tile, prec=mo.TRUTH, opts=opts, noise=noise)
    return float((out["O"] * dout).sum()) + out["lb"] + out["zloss"], out["plan"]


VARIANTS = [
    ("all_lb_z_noise", mo.RouteOpts(gate="all", lb_coef=0.7, z_coef=0.05), 0, True),
    ("topk_lb", mo.RouteOpts(lb_coef=1.3), 0, False),
    ("topk_z", mo.RouteOpts(z_coef=0.2), 0, False),
    ("all_round", mo.RouteOpts(gate="all", lb_coef=0.4), 2, False),
    ("capacity", mo.RouteOpts(capacity_factor=0.6, z_coef=0.1), 0, True),
    ("all_capacity", mo.RouteOpts(gate="all", capacity_factor=0.75), 0, False),
]


@pytest.mark.parametrize("name,opts,tile,with_noise", VARIANTS, ids=[v[0] for v in VARIANTS])
def test_finite_differences_with_router_losses(name, opts, tile, with_noise):
    x, wg, b, w1, w2, dout, redraw = _tiny(T=8, d=4, E=4, k=2, f=5, seed=21)
    noise = np.random.default_rng(22).standard_normal((8, 4)) * 0.3 if with_noise else None
    bn = b if noise is None else None
    if noise is not None:
        # ties are cleared on the noisy logits: fold the noise into a per-token bias-free check
        x, _ = clear_ties(x, wg, None, 2, redraw, round_tile=tile, delta_z=1e-2, delta_p=1e-2, noise=noise)
    else:
        x, _ = clear_ties(x, wg, bn, 2, redraw, round_tile=tile, delta_z=1e-2, delta_p=1e-2)
    out = mo.layer(x, wg, bn, w1, w2, 2, dout=dout, round_tile=tile, prec=mo.TRUTH, opts=opts, noise=noise)
    base_plan = out["plan"]
    h = 1e-6
    for pname, arr, grad in (("x", x, out["dx"]), ("wg", wg, out["dw_gate"]), ("w1", w1, out["dw1"]),
                             ("w2", w2, out["dw2"])):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            args = {"x": x, "wg": wg, "w1": w1, "w2": w2}
            plus = arr.copy(); plus[i] += h
            minus = arr.copy(); minus[i] -= h
            args[pname] = plus
            lp, pp = _total_loss(args["x"], args["wg"], bn, args["w1"], args["w2"], dout, 2, tile, opts, noise)
            args[pname] = minus
            lm, pm = _total_loss(args["x"], args["wg"], bn, args["w1"], args["w2"], dout, 2, tile, opts, noise)
            assert (pp.token_of_row == base_plan.token_of_row).all()
            assert (pm.token_of_row == base_plan.token_of_row).all()
            num[i] = (lp - lm) / (2 * h)
        err = np.abs(num - grad).max() / max(1.0, np.abs(grad).max())
        assert err < 1e-6, (name, pname, err)


def test_dense_gradient_matches_torch_autograd():
    """gate "all" + load-balance + z-loss written out in torch float64 from the
    definitions (full softmax gates, CV of the mean distribution with the
    population std, logsumexp), differentiated by autograd."""
    x, wg, b, w1, w2, dout, redraw = _tiny(T=10, d=5, E=5, k=2, f=3, seed=31)
    x, _ = clear_ties(x, wg, b, 2, redraw, delta_z=1e-2, delta_p=1e-2)
    opts = mo.RouteOpts(gate="all", lb_coef=0.9, z_coef=0.07)
    out = mo.layer(x, wg, b, w1, w2, 2, dout=dout, prec=mo.TRUTH, opts=opts)
    plan = out["plan"]
    X = torch.tensor(x, requires_grad=True)
    WG = torch.tensor(wg, requires_grad=True)
    z = X @ WG.T + torch.from_numpy(b)
    P = torch.softmax(z, 1)
    f = w2.shape[2]
    O = torch.zeros_like(X)
    for r in range(plan.N):
        t, e = int(plan.token_of_row[r]), int(plan.expert_of_row[r])
        hh = torch.from_numpy(w1[e]) @ X[t]
        a = torch.nn.functional.silu(hh[:f]) * hh[f:]
        O = O.index_add(0, torch.tensor([t]), (P[t, e] * (torch.from_numpy(w2[e]) @ a))[None])
    pbar = P.mean(0)
    cv = pbar.std(unbiased=False) / pbar.mean()
    loss = (O * torch.from_numpy(dout)).sum() + 0.9 * cv ** 2 + 0.07 * (torch.logsumexp(z, 1) ** 2).mean()
    loss.backward()
    assert abs(out["lb"] - 0.9 * cv.item() ** 2) < 1e-12
    np.testing.assert_allclose(out["dx"], X.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(out["dw_gate"], WG.grad.numpy(), rtol=1e-10, atol=1e-12)
