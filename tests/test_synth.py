"""The seeded input generator: determinism, shapes, dtypes and moments."""
import math

import numpy as np
import torch

from mixture_experts_layer_27_amd import configs, synth


def test_deterministic_and_shapes():
    c = configs.TINY
    a, b = synth.generate(c), synth.generate(c)
    for k in a:
        assert torch.equal(a[k], b[k])
    assert a["x"].shape == (c.T, c.d) and a["w_gate"].shape == (c.E, c.d)
    assert a["w1"].shape == (c.E, 2 * c.f, c.d) and a["w2"].shape == (c.E, c.d, c.f)
    assert a["dout"].shape == (c.T, c.d) and a["x"].dtype == torch.float32
    assert not torch.equal(synth.generate(c, seed=1)["x"], a["x"])


def test_bf16_moments_and_bias():
    c = configs.FINE_ZIPF.scaled("fz", T=512, d=256, E=16, f=128)
    g = synth.generate(c)
    assert g["x"].dtype == torch.bfloat16 and g["bias"].dtype == torch.float32
    x = g["x"].double()
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1.0) < 0.02
    w1 = g["w1"].double()
    assert abs(w1.std() * math.sqrt(c.d) - 1.0) < 0.02
    w2 = g["w2"].double()
    assert abs(w2.std() * math.sqrt(c.f) - 1.0) < 0.02
    assert abs(g["w_gate"].double().std() * math.sqrt(c.d) - 1.0) < 0.05
    np.testing.assert_allclose(g["bias"].numpy(), -np.log(np.arange(16) + 1.0), rtol=1e-6)


def test_redraw_rows_only_touches_given_rows():
    c = configs.TINY
    g = synth.generate(c)
    y = synth.redraw_rows(c, g["x"], [3, 1], attempt=0)
    diff = (y != g["x"]).any(1).nonzero().flatten().tolist()
    assert diff == [1, 3]
    assert torch.equal(y, synth.redraw_rows(c, g["x"], [1, 3], attempt=0))


def test_micro_batches_differ_and_keep_the_distribution():
    c = configs.FINE.scaled("fm", T=512, d=256, E=16, f=128)
    a, b = synth.micro_batch(c, 0), synth.micro_batch(c, 1)
    assert torch.equal(a["x"], synth.micro_batch(c, 0)["x"])
    assert not torch.equal(a["x"], b["x"]) and not torch.equal(a["dout"], b["dout"])
    assert not torch.equal(a["x"], synth.generate(c)["x"])
    assert a["x"].dtype == torch.bfloat16 and a["x"].shape == (c.T, c.d) and a["dout"].shape == (c.T, c.d)
    assert synth.micro_batch(c, 2, T=100)["x"].shape == (100, c.d)
    x = a["x"].double()
    assert abs(x.mean()) < 0.02 and abs(x.std() - c.x_std) < 0.02
