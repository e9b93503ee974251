"""The five layer shapes the path is built and measured on.

Notation follows "DeepSeekMoE" (the translated paper page, section 3):
  T   tokens in the batch
  d   hidden size of u_t
  N_r routed fine-grained experts (mN - K_s in eq. 9-10)
  K_s shared experts, always active (section 3.2)
  K'  routed experts chosen per token (mK - K_s in eq. 10)
  I   intermediate width of one routed expert (FFN width / m, section 3.1)
  I_s intermediate width of one shared expert

gate:
  "softmax_topk"  s = Softmax over the N_r routed experts, keep the top K'
                  values unchanged (eq. 10-11; also the Switch-Transformer
                  routing rule on the MoE-survey blog page, section 4)
  "topk_softmax"  Softmax(KeepTopK(H, k)) with the noise term set to zero
                  (noisy top-k gating on the MoE-survey blog page, section 2)
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class LayerConfig:
    name: str
    tokens: int
    d_model: int
    n_routed: int
    n_shared: int
    top_k: int
    d_ff: int
    d_ff_shared: int
    gate: str = "softmax_topk"
    dtype: str = "bf16"        # storage/compute type of x, expert weights, y
    zipf_s: float = 0.0        # > 0: per-expert router bias -s*ln(e+1)
    bias_mode: str = "logits"  # "logits": bias in selection and gates; "selection": selection only
    noisy: bool = False        # noisy top-k gating: inputs gain w_noise [N_r, d] and noise [T, N_r]
    seed: int = 4300
    gap: float = 1e-3          # min logit gap between the K'-th and (K'+1)-th
    ffn: str = "silu"          # "silu": W2 (silu(W1 u) * (W3 u)); "relu": wo ReLU(wi u) (W1, W2)
    capacity: int = 0          # > 0: assignments kept per expert per token group; 0 = dropless
    group_size: int = 0        # tokens per group for the capacity (0 = the whole batch)

    @property
    def assignments(self) -> int:
        return self.tokens * self.top_k

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


CONFIGS = {
    # Tiny fp32 layer: 16 routed fine-grained experts (m = 2 split of 8 base
    # experts) + 1 shared, top-4, width 32.
    "tiny-f32": LayerConfig(
        name="tiny-f32", tokens=64, d_model=64, n_routed=16, n_shared=1,
        top_k=4, d_ff=32, d_ff_shared=32, gate="softmax_topk", dtype="f32",
        seed=4301),
    # DeepSeekMoE 2B-shaped layer: 1 shared + 63 routed, top-7, width 896.
    "2b": LayerConfig(
        name="2b", tokens=8192, d_model=1280, n_routed=63, n_shared=1,
        top_k=7, d_ff=896, d_ff_shared=896, seed=4302),
    # DeepSeekMoE 16B-shaped layer: 2 shared + 64 routed, top-6, width 1408.
    "16b": LayerConfig(
        name="16b", tokens=16384, d_model=2048, n_routed=64, n_shared=2,
        top_k=6, d_ff=1408, d_ff_shared=1408, seed=4303),
    # Same 16B-shaped layer at decode batch size.
    "16b-decode": LayerConfig(
        name="16b-decode", tokens=128, d_model=2048, n_routed=64, n_shared=2,
        top_k=6, d_ff=1408, d_ff_shared=1408, seed=4304),
    # Coarse GShard-style layer: 8 experts, top-2, width 14336, no shared
    # expert, Softmax(KeepTopK) gates, Zipf(1.2) router bias for skew.
    "gshard-zipf": LayerConfig(
        name="gshard-zipf", tokens=8192, d_model=4096, n_routed=8, n_shared=0,
        top_k=2, d_ff=14336, d_ff_shared=14336, gate="topk_softmax",
        zipf_s=1.2, seed=4305),
}


def get_config(name: str) -> LayerConfig:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown layer config {name!r}; known: {sorted(CONFIGS)}")
