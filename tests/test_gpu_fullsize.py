"""Parity at the full workload sizes, in the launch configuration bench.py times.

The oracle cannot run the whole layer at these sizes in seconds, so: every
routing integer (top-k, counts, offsets, all plan maps, token rounding) is
compared bit for bit over all tokens; outputs and gradients are compared on a
seeded sample of tokens (all of their rows) and on every element of the
weight gradients of a sample of experts, each computed by the oracle one by
one; dW_g is checked through the identity dW_g = bf16(dlogits)^T X on all tokens."""
import numpy as np
import pytest
import torch

from helpers import LazyExperts, assert_close, make_inputs, precision
from mixture_experts_layer_27_amd import configs
from oracle import moe_oracle as mo

pytestmark = pytest.mark.gpu

FULL = ["fine_e128", "sparse_e256_round", "coarse_e8", "fine_e128_zipf"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    from mixture_experts_layer_27_amd import binding
    cfg = configs.get(name)
    print(f"[fullsize] {name}: generating inputs", flush=True)
    g = make_inputs(cfg)
    run = binding.LayerRun(cfg, g)
    run.forward()
    if run.has_bwd:
        run.backward()
    torch.cuda.synchronize()
    print(f"[fullsize] {name}: GPU done, oracle routing", flush=True)
    f64 = lambda t: None if t is None else t.double().numpy()
    x = f64(g["x"])
    wg = f64(g["w_gate"])
    bias = f64(g.get("bias"))
    z, plan = mo.route(x, wg, bias, cfg.k, cfg.round_tile)
    a = {k: v.cpu() for k, v in run.plan.arrays().items()}
    N = plan.N
    for key in ("topk_idx", "counts_raw", "counts", "offsets", "row_of_slot", "tok_ptr"):
        np.testing.assert_array_equal(a[key].numpy(), getattr(plan, key), err_msg=key)
    for key in ("token_of_row", "expert_of_row", "tok_rows"):
        np.testing.assert_array_equal(a[key][:N].numpy(), getattr(plan, key), err_msg=key)
    np.testing.assert_allclose(a["gate_of_row"][:N].double().numpy(), plan.gate_of_row, rtol=0, atol=2e-6)

    prec = precision(cfg)
    W1, W2 = LazyExperts(g["w1"]), LazyExperts(g["w2"])
    rng = np.random.default_rng(2024)
    toks = np.sort(rng.choice(cfg.T, 32, replace=False))
    sub = mo.sub_plan(plan, tokens=toks)
    print(f"[fullsize] {name}: oracle on {len(toks)} tokens ({sub.N} rows)", flush=True)
    fw = mo.forward(x, W1, W2, sub, prec)
    row_of = {(int(t), int(e)): r for r, (t, e) in enumerate(zip(plan.token_of_row, plan.expert_of_row))}
    rows = np.array([row_of[(int(t), int(e))] for t, e in zip(sub.token_of_row, sub.expert_of_row)])
    assert_close("O", run.out[toks].double().cpu().numpy(), fw["O"][toks])
    assert_close("H", run.h[rows].double().cpu().numpy(), fw["H"])
    if not run.has_bwd:
        return
    dout = f64(g["dout"])
    bw = mo.backward(x, wg, W1, W2, sub, fw["H"], dout, prec, weight_grads=False)
    assert_close("dS", run.ds[rows].double().cpu().numpy(), bw["dS"])
    assert_close("dlogits", run.dlogits[toks].double().cpu().numpy(), bw["dlogits"][toks])
    assert_close("dx", run.dx[toks].double().cpu().numpy(), bw["dx"][toks])
    # every element of the weight gradients of two experts (the busiest and a random one)
    experts = [int(np.argmax(plan.counts)), int(rng.integers(cfg.E))]
    for e in experts:
        sub_e = mo.sub_plan(plan, experts=[e])
        print(f"[fullsize] {name}: oracle weight gradients of expert {e} ({sub_e.N} rows)", flush=True)
        fw_e = mo.forward(x, W1, W2, sub_e, prec)
        bw_e = mo.backward(x, wg, W1, W2, sub_e, fw_e["H"], dout, prec, weight_grads=[e])
        assert_close(f"dw1[{e}]", run.dw1[e].double().cpu().numpy(), bw_e["dw1"][e])
        assert_close(f"dw2[{e}]", run.dw2[e].double().cpu().numpy(), bw_e["dw2"][e])
    # dW_g = bf16(dlogits)^T X over all tokens (the router-weight GEMM on the GPU's own dz)
    dzq = run.dlogits.cpu().to(torch.bfloat16).double().numpy() if cfg.act == "bf16" else f64(run.dlogits.cpu())
    assert_close("dw_gate", run.dw_gate.double().cpu().numpy(), dzq.T @ x)
