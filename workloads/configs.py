"""The five parameter groups the path is measured and checked on.

Each group is a list of (true dim-0 rows T_p, row length K_p) in registration
order, a rank count N = M*L and a contributor count L, plus the value
distribution of the synthetic gradients. Shapes follow the model layers named
on the pages (Llama-3.1 70B, Qwen3-30B-A3B, Wan2.2 14B; page 1 "What do the
results show?"); a 1-D tensor has K_p = 1, and a tensor with more than two dims
would have K_p = the product of its trailing dims.

No data set or trained weights stand behind these shapes: values are seeded
synthetic draws (see values.py).
"""
from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np


@dataclass(frozen=True)
class Config:
    name: str
    shapes: Tuple[Tuple[int, int], ...]
    N: int
    L: int
    sigma: float
    outlier_frac: float = 0.0
    seed: int = 0
    note: str = ""


def _llama70b_layer() -> List[Tuple[int, int]]:
    h, f = 8192, 28672
    return [(h, h), (1024, h), (1024, h), (h, h),  # q k v o
            (f, h), (f, h), (h, f),                  # gate up down
            (h, 1), (h, 1)]                          # two RMSNorm weights


def _qwen3_moe_layer() -> List[Tuple[int, int]]:
    h, e, fe = 2048, 128, 768
    out: List[Tuple[int, int]] = []
    for _ in range(e):
        out += [(fe, h), (fe, h), (h, fe)]           # expert gate up down
    out += [(e, h),                                   # router
            (4096, h), (512, h), (512, h), (h, 4096),  # q k v o
            (h, 1), (h, 1)]                           # two norms
    return out


def _padding_stress(seed: int) -> List[Tuple[int, int]]:
    rng = np.random.default_rng(seed)
    rows = rng.integers(1, 5001, 200)
    ks = rng.choice([1, 64, 4096, 8192], 200)
    return [(int(t), int(k)) for t, k in zip(rows, ks)]


def _wan22_dit_block() -> List[Tuple[int, int]]:
    d, f = 5120, 13824
    return ([(d, d)] * 4 +           # self-attention q k v o
            [(d, d)] * 4 +           # cross-attention q k v o
            [(f, d), (d, f)] +       # FFN in / out
            [(d, 1), (d, 1)] +       # two norms
            [(6, d)])                # modulation, 6 x 5120


CONFIGS = {
    "worked_example": Config(
        "worked_example", ((8, 4), (4, 4), (12, 4)), N=4, L=4, sigma=1.0,
        note="3 params whose per-rank pieces are 2, 1 and 3 rows of K=4"),
    "llama70b_layer": Config(
        "llama70b_layer", tuple(_llama70b_layer()), N=64, L=8, sigma=1e-3),
    "qwen3_moe_layer": Config(
        "qwen3_moe_layer", tuple(_qwen3_moe_layer()), N=64, L=8, sigma=1e-3),
    "padding_stress": Config(
        "padding_stress", tuple(_padding_stress(0)), N=48, L=8, sigma=1.0,
        outlier_frac=0.01, note="rows ~ U{1..5000}, K in {1,64,4096,8192}, seed 0"),
    "wan22_dit_block": Config(
        "wan22_dit_block", tuple(_wan22_dit_block()), N=64, L=8, sigma=1e-3),
}

ORDER = ["worked_example", "llama70b_layer", "qwen3_moe_layer",
         "padding_stress", "wan22_dit_block"]


def config_shapes(name: str) -> List[Tuple[int, int]]:
    return list(CONFIGS[name].shapes)


def padding_stress_shapes(seed: int, count: int = 200, max_rows: int = 5000,
                          ks=(1, 64, 4096, 8192)) -> List[Tuple[int, int]]:
    """The padding-stress shape draw, with its bounds exposed so tests can
    draw smaller groups of the same structure."""
    rng = np.random.default_rng(seed)
    rows = rng.integers(1, max_rows + 1, count)
    kk = rng.choice(list(ks), count)
    return [(int(t), int(k)) for t, k in zip(rows, kk)]
