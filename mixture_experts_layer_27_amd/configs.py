"""Workload table for the token-choice top-k MoE FFN layer.

Shapes only: no arithmetic of the method lives here.  Each entry is one
layer problem: T tokens of width d, E experts with SwiGLU hidden size d_ff,
top-k routing.  Distributions follow the workloads the pages describe:

* ``tiny_fp32``      -- small fp32 layer, forward and backward (oracle-sized).
* ``coarse_e8``      -- 8 experts, top-4, d_ff 4096, forward only: the 8-expert end
                        of the 8->128 expert-count sweep reported for Olmo-core 3
                        ("Key numbers" section of the Olmo-core 3 article).
* ``fine_e128``      -- 128 experts, top-4, d_ff 1024, fwd+bwd, random routing: the
                        "random routing" system benchmark of the same article.
* ``fine_e128_zipf`` -- as above plus a per-expert Zipf(s=1) logit bias (imbalance).
* ``sparse_e256``    -- 256 experts, top-8, d_ff 512, fwd+bwd, with a per-expert bias:
                        the highly sparse case where SonicMoE's token rounding
                        applies (SonicMoE article, section 3).
* ``sparse_e256_round`` -- as above with counts rounded to multiples of 128.
* ``fine_e128_mxfp8`` -- ``fine_e128`` with MXFP8 expert-GEMM operands (Olmo-core 3
                        article, "three splits" section: the MXFP8 switch).
* ``sparse_e256_mxfp8`` -- ``sparse_e256`` with MXFP8 expert-GEMM operands: the
                        switch at the wider d_model, where more tokens share
                        each expert's weight quantisation.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                 # tokens
    d: int                 # model width
    E: int                 # experts
    k: int                 # experts per token
    f: int                 # SwiGLU hidden size per expert (d_ff)
    act: str = "bf16"      # activation / weight storage dtype: "bf16" | "f32"
    gemm: str = "bf16"     # expert GEMM operand format: "bf16" | "f32" | "mxfp8"
    x_std: float = 1.0
    wg_std: float = 0.02
    bias: Optional[str] = None     # None | "normal" | "zipf"
    b_std: float = 0.0
    zipf_s: float = 1.0
    round_tile: int = 0            # 0: no token rounding; else tile multiple
    backward: bool = True
    seed: int = 0
    # routing variants (0 / "topk" = the base layer)
    gate: str = "topk"             # "topk": softmax over the k selected; "all": full softmax, not renormalised
    capacity_factor: float = 0.0   # 0: no cap; else each expert keeps its first ceil(cf*T*k/E) rows
    lb_coef: float = 0.0           # load-balance loss weight (CV(Pbar)^2)
    z_coef: float = 0.0            # z-loss weight (mean lse^2)
    noise_std: float = 0.0         # routing noise ~ N(0, noise_std^2) [T, E] added to the logits

    @property
    def N(self) -> int:
        """Token-expert pairs before rounding."""
        return self.T * self.k

    @property
    def N_max(self) -> int:
        """Upper bound on routed rows (rounding may add up to tile/2 per expert)."""
        return self.T * self.k + (self.E * (self.round_tile // 2) if self.round_tile else 0)

    def scaled(self, name: str, **kw) -> "MoEConfig":
        """A smaller problem with the same distributions (std of weights follows fan-in)."""
        c = dataclasses.replace(self, name=name, **kw)
        if "wg_std" not in kw and self.wg_std != 0.02:
            # routers drawn at 1/sqrt(d) keep that rule at the new width
            c = dataclasses.replace(c, wg_std=1.0 / math.sqrt(c.d))
        return c

    def gemm_flops(self, backward: Optional[bool] = None, rows: Optional[int] = None) -> float:
        """Algorithmic expert-GEMM flops: 2*N*d*2f (GEMM1) + 2*N*f*d (GEMM2), x3 with backward."""
        n = self.N if rows is None else rows
        fwd = 2.0 * n * self.d * 2 * self.f + 2.0 * n * self.f * self.d
        bwd = self.backward if backward is None else backward
        return fwd * 3 if bwd else fwd


TINY = MoEConfig("tiny_fp32", T=256, d=128, E=8, k=2, f=256, act="f32", gemm="f32",
                 wg_std=0.02)
COARSE = MoEConfig("coarse_e8", T=16384, d=2048, E=8, k=4, f=4096, wg_std=0.02,
                   backward=False)
FINE = MoEConfig("fine_e128", T=16384, d=2048, E=128, k=4, f=1024,
                 wg_std=1.0 / math.sqrt(2048))
FINE_ZIPF = dataclasses.replace(FINE, name="fine_e128_zipf", bias="zipf", zipf_s=1.0)
SPARSE = MoEConfig("sparse_e256", T=32768, d=4096, E=256, k=8, f=512,
                   wg_std=1.0 / 64.0, bias="normal", b_std=0.5)
SPARSE_ROUND = dataclasses.replace(SPARSE, name="sparse_e256_round", round_tile=128)
FINE_MX = dataclasses.replace(FINE, name="fine_e128_mxfp8", gemm="mxfp8")
SPARSE_MX = dataclasses.replace(SPARSE, name="sparse_e256_mxfp8", gemm="mxfp8")
# routing variants at the fine_e128 shape: full-softmax gates, noisy top-k and both
# router losses (dense router gradient); a capacity factor on the Zipf-imbalanced routing
FINE_LOSSES = dataclasses.replace(FINE, name="fine_e128_router_losses", gate="all", lb_coef=0.01, z_coef=0.001,
                                  noise_std=1.0)
FINE_CAPACITY = dataclasses.replace(FINE_ZIPF, name="fine_e128_zipf_capacity", capacity_factor=1.25)

CONFIGS = {c.name: c for c in (TINY, COARSE, FINE, FINE_ZIPF, SPARSE, SPARSE_ROUND, FINE_MX, SPARSE_MX,
                               FINE_LOSSES, FINE_CAPACITY)}


def get(name: str) -> MoEConfig:
    return CONFIGS[name]
