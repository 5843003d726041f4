"""Seeded synthetic inputs for the GMA forward mixer.

This module only draws random numbers and casts them; it holds none of the
mixer's arithmetic.  Both the fp64 oracle and the HIP path consume exactly the
tensors returned here (the activations already rounded to their storage dtype),
so any disagreement between the two comes from the computation alone.

The five workload shapes follow the method's statement of the problem
(Gaussian Mixture Attention, arXiv 2606.18283: routing vectors for queries and
keys, values, K diagonal Gaussians with means, softplus variances and softmax
priors; bidirectional and causal variants).  The pages publish no dataset that
the forward mixer is measured on, so these seeded draws stand in for the
long-context classification and language-modelling workloads the pages train on;
K=256 matches the pages' WikiText-103 causal model and K=128 the pages'
128-component responsibility analysis.

Drawing recipe (all in float32 from one ``torch.Generator('cpu')``):
  q, k, v, mu, var_raw, prior_logits in that order, each ``randn * std``;
  the sharp-row workload then draws, for q and then for k, a Bernoulli(0.2)
  row mask, a uniform component index per row and unit normal noise, and
  replaces the masked rows by ``mu[h, c] + 0.1 * noise``.
q, k and v are then cast to the workload dtype (round to nearest even);
the Gaussian parameters stay float32.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" or "bf16": storage type of qr, kr, v, out
    causal: bool
    B: int
    H: int
    N: int
    d_r: int
    d_v: int
    K: int
    seed: int
    eps: float = 1e-6
    var_floor: float = 1e-3
    x_std: float = 1.0        # std of q, k
    v_std: float = 1.0
    mu_std: float = 1.0
    var_raw_std: float = 0.5  # var = softplus(var_raw) + var_floor
    prior_std: float = 1.0
    sharp_frac: float = 0.0   # fraction of q/k rows drawn near a random mean
    sharp_noise: float = 0.1
    N_k: Optional[int] = None  # key/value rows of the cross variant (None: N, self-mixing)

    @property
    def Nk(self) -> int:
        return self.N if self.N_k is None else self.N_k

    @property
    def token_heads(self) -> int:
        return self.B * self.H * self.N

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS: Dict[int, Workload] = {
    1: Workload("tiny-bidir-f32", "f32", False, 1, 1, 256, 16, 16, 8, seed=1001),
    2: Workload("bidir-bf16-K128", "bf16", False, 8, 8, 4096, 64, 64, 128, seed=1002),
    3: Workload("causal-lm-bf16-K256", "bf16", True, 16, 8, 2048, 64, 64, 256, seed=1003),
    4: Workload("long-bidir-bf16-K64-sharp", "bf16", False, 2, 8, 65536, 64, 64, 64,
                seed=1004, var_floor=1e-2, sharp_frac=0.2),
    5: Workload("long-causal-bf16-K256-d128", "bf16", True, 1, 16, 32768, 128, 128, 256,
                seed=1005, mu_std=2.0, var_raw_std=1.0, prior_std=2.0),
    # cross variant: 1024 queries per head read a memory built from 16384 keys
    6: Workload("cross-bf16-K128-q1024-k16384", "bf16", False, 8, 8, 1024, 64, 64, 128, seed=1006,
                N_k=16384),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_inputs(w: Workload) -> Dict[str, torch.Tensor]:
    """Draw the seeded CPU tensors of workload ``w``.

    Returns a dict with ``qr`` [B,H,N,d_r], ``kr`` [B,H,Nk,d_r], ``v`` [B,H,Nk,d_v] in the
    workload dtype (Nk = N unless the workload sets N_k) and ``mu, var_raw`` [H,K,d_r],
    ``prior_logits`` [H,K] in float32.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(int(w.seed))
    B, H, N, dr, dv, K = w.B, w.H, w.N, w.d_r, w.d_v, w.K
    Nk = w.Nk
    f32 = torch.float32
    q = torch.randn((B, H, N, dr), generator=g, dtype=f32) * w.x_std
    k = torch.randn((B, H, Nk, dr), generator=g, dtype=f32) * w.x_std
    v = torch.randn((B, H, Nk, dv), generator=g, dtype=f32) * w.v_std
    mu = torch.randn((H, K, dr), generator=g, dtype=f32) * w.mu_std
    var_raw = torch.randn((H, K, dr), generator=g, dtype=f32) * w.var_raw_std
    prior = torch.randn((H, K), generator=g, dtype=f32) * w.prior_std
    if w.sharp_frac > 0.0:
        for x in (q, k):
            n = x.shape[2]
            hidx = torch.arange(H).view(1, H, 1).expand(B, H, n)
            mask = torch.rand((B, H, n), generator=g) < w.sharp_frac
            comp = torch.randint(0, K, (B, H, n), generator=g)
            noise = torch.randn((B, H, n, dr), generator=g, dtype=f32)
            near = mu[hidx, comp] + w.sharp_noise * noise
            x.copy_(torch.where(mask.unsqueeze(-1), near, x))
    dt = torch_dtype(w.dtype)
    return {
        "qr": q.to(dt).contiguous(),
        "kr": k.to(dt).contiguous(),
        "v": v.to(dt).contiguous(),
        "mu": mu.contiguous(),
        "var_raw": var_raw.contiguous(),
        "prior_logits": prior.contiguous(),
    }
