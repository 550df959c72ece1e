"""Layer shapes of the Stable LatentMoE forward pass used by tests and the benchmark.

Shapes only: no arithmetic of the method lives here. The K3 dimensions
(d_model 7168, d_latent 3584, 896 routed experts with 16 active, 2 shared
experts) come from vxz.us "苏神复盘 Kimi K3" section 01 and the expert table of
lukebest.github.io "Stable Latent MoE" (section "K3 专家配置"). The routed and
shared inner sizes (512 and 2048) are synthetic choices: the pages give none.
beta1 = 4 and beta2 = 25 are from tahou.com (section "SiTU激活优化"); 1000 bins
from the same page (section "负载均衡优化").
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int                 # tokens in the batch
    d_model: int           # D
    d_latent: int          # L
    n_experts: int         # E routed experts
    top_k: int             # k
    inter: int             # I, routed expert inner size
    n_shared: int          # S always-on shared experts
    inter_shared: int      # I_s, inner size of each shared expert
    n_bins: int            # NB, quantile-balancing histogram bins
    act_dtype: str = "bf16"   # storage type of activations and weights: "bf16" or "f32"
    beta1: float = 4.0
    beta2: float = 25.0
    rms_eps: float = 1e-6
    zipf_s: float = 0.0          # >0: per-expert logit offsets o_e = -zipf_s * ln(r_e)
    outlier_frac: float = 0.0    # fraction of x entries scaled by outlier_scale
    outlier_scale: float = 1.0
    qb_updates: int = 1          # successive batches, each followed by a bias update

    @property
    def pairs(self) -> int:
        return self.T * self.top_k

    def with_tokens(self, T: int) -> "LayerConfig":
        return replace(self, T=T)


TINY_F32 = LayerConfig("tiny_f32", T=64, d_model=256, d_latent=128, n_experts=32, top_k=4,
                       inter=64, n_shared=1, inter_shared=128, n_bins=100, act_dtype="f32")
MID_BF16 = LayerConfig("mid_bf16", T=4096, d_model=2048, d_latent=1024, n_experts=128, top_k=8,
                       inter=256, n_shared=2, inter_shared=1024, n_bins=1000)
K3_PREFILL = LayerConfig("k3_prefill", T=8192, d_model=7168, d_latent=3584, n_experts=896, top_k=16,
                         inter=512, n_shared=2, inter_shared=2048, n_bins=1000)
K3_DECODE = replace(K3_PREFILL, name="k3_decode", T=64)
K3_STRESS = replace(K3_PREFILL, name="k3_stress", T=32768, zipf_s=1.1, outlier_frac=0.001,
                    outlier_scale=50.0, qb_updates=8)

CONFIGS = {c.name: c for c in (TINY_F32, MID_BF16, K3_PREFILL, K3_DECODE, K3_STRESS)}
