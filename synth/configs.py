"""The five synthetic workloads of the layer (shapes from the K3 pages; the tiny,
small and D=512 choices are the benchmark's own).

C0  tiny fp32        T=64    d=256   L=128  n=16   k=4  n_s=1 D=64
C1  small bf16       T=4096  d=2048  L=1024 n=128  k=8  n_s=2 D=512, bias ~ N(0, 0.01)
C2  K3 prefill bf16  T=8192  d=7168  L=3584 n=896  k=16 n_s=2 D=512, 0.1% tokens x50
C3  K3 decode bf16   T=64    (C2 weights)
C4  skewed + QB      T=32768 (C2 weights), Zipf(1.1) logit skew, 20 QB steps
"""
from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Config:
    name: str
    T: int
    d: int
    L: int
    n: int
    k: int
    n_shared: int
    D: int
    dtype: str                 # "f32" | "bf16"
    x_seed: int                # seed of the token stream
    w_seed: int                # seed of the weight streams
    bias_std: float = 0.0      # router selection bias ~ N(0, bias_std^2), 0 -> zeros
    outlier_frac: float = 0.0  # fraction of tokens scaled by outlier_mult
    outlier_mult: float = 50.0
    zipf_alpha: float = 0.0    # logit offset alpha * r^-zipf_s (0 -> none)
    zipf_s: float = 1.1
    qb_steps: int = 0
    nbins: int = 1000
    beta1: float = 4.0
    beta2: float = 25.0
    gate: str = "tanh"  # expert caps: "tanh" softcap, or "clip" for the hard-clip ablation
    norm: str = "rms"   # "rms" (the layer's norm); "none" or "both" (an extra norm on z) for ablations
    eps: float = 1e-6

    def flops_per_token(self):
        """Algorithmic FLOPs per token: W_down, router, k routed + n_s shared experts, W_up."""
        dense = 2 * self.d * self.L * 2 + 2 * self.L * self.n
        expert = 2 * 3 * self.L * self.D
        return dense + (self.k + self.n_shared) * expert

    def with_(self, **kw):
        return replace(self, **kw)


CONFIGS = {
    "C0": Config("C0", T=64, d=256, L=128, n=16, k=4, n_shared=1, D=64, dtype="f32", x_seed=0, w_seed=0),
    "C1": Config("C1", T=4096, d=2048, L=1024, n=128, k=8, n_shared=2, D=512, dtype="bf16", x_seed=1,
                 w_seed=1, bias_std=0.1),
    "C2": Config("C2", T=8192, d=7168, L=3584, n=896, k=16, n_shared=2, D=512, dtype="bf16", x_seed=2,
                 w_seed=2, outlier_frac=0.001),
    "C3": Config("C3", T=64, d=7168, L=3584, n=896, k=16, n_shared=2, D=512, dtype="bf16", x_seed=3,
                 w_seed=2),
    "C4": Config("C4", T=32768, d=7168, L=3584, n=896, k=16, n_shared=2, D=512, dtype="bf16", x_seed=4,
                 w_seed=2, zipf_alpha=2.0, qb_steps=20),
}


def get_config(name, **overrides):
    c = CONFIGS[name]
    return c.with_(**overrides) if overrides else c
