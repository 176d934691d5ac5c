"""The five synthetic workloads, by shape.

Shapes follow the models the three pages evaluate on (DeepSeek-V2 and
Mixtral-8x7B in the Speculative MoE notes, Qwen3-30B-A3B in "Speculating
Experts Accelerates Inference for Mixture-of-Experts", and the grouped model of
the Federation of Experts article). No weights of those models exist here;
only their routing shapes enter.
"""

from dataclasses import dataclass, field


@dataclass(frozen=True)
class RouteConfig:
    """Predict -> SRS -> gate -> top-K -> LAR -> permute -> combine workload."""

    name: str
    seed: int
    N: int          # tokens per pass
    d: int          # hidden size
    E: int          # routed experts
    K: int          # experts per token
    P: int          # tensor-parallel partial activations reduced by SRS
    G: int          # destination clusters
    V: int          # vocabulary size (token ids drawn Zipf(1.1) over it)
    lut_mode: str   # "random" or "routing" (argmax cluster of noiseless routing)
    ngram: bool     # confidence + 2-gram cluster fallback enabled
    conf_thr: int = 128   # fall back iff conf byte < conf_thr (128/255 ~ 0.5)
    zipf_s: float = 1.1
    noise: float = 0.3
    kind: str = "route"


@dataclass(frozen=True)
class FoEConfig:
    """Grouped (FoE) workload: reduce H groups -> gate -> grouped top-k/H -> ...."""

    name: str
    seed: int
    N: int
    d: int
    E: int
    H: int
    K: int          # total experts per token (K/H per group)
    G: int
    V: int
    zipf_s: float = 1.1
    noise: float = 0.3
    kind: str = "foe"


@dataclass(frozen=True)
class PredictorConfig:
    """Quasi-hidden-state predictor workload over L layers."""

    name: str
    seed: int
    L: int
    N: int
    d: int
    E: int
    K: int
    hd: int = 512                     # estimator hidden width
    ffn: int = 768                    # expert FFN width: an expert's weights are gate, up
                                      # and down projections, 3 * d * ffn bf16 values
    est_layers: tuple = (0, 1, 2, 3)  # source layers that use the MLP estimator
    dvec_var: float = 0.1
    drift: float = 0.5
    eps: float = 1e-5
    kind: str = "predictor"


CONFIGS = {
    "tiny": RouteConfig("tiny", 1000, N=64, d=128, E=4, K=2, P=2, G=2, V=512,
                        lut_mode="random", ngram=False),
    "mixtral": RouteConfig("mixtral", 1001, N=4096, d=4096, E=8, K=2, P=2, G=4,
                           V=32000, lut_mode="routing", ngram=False),
    "deepseek": RouteConfig("deepseek", 1002, N=16384, d=5120, E=160, K=6, P=2,
                            G=8, V=102400, lut_mode="routing", ngram=True),
    "qwen3": PredictorConfig("qwen3", 1003, L=48, N=8192, d=2048, E=128, K=8),
    "foe": FoEConfig("foe", 1004, N=32768, d=2048, E=64, H=4, K=8, G=8, V=50000),
}


def get_config(name: str):
    try:
        return CONFIGS[name]
    except KeyError as exc:
        raise KeyError(f"unknown config {name!r}; have {sorted(CONFIGS)}") from exc
