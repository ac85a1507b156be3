"""Workload shapes for draft-tree construction rounds.

Shapes follow the drafters the pages evaluate (Qwen3-4B / Qwen3-8B hidden
size and vocabulary, a rank-256 correction head) and the tree parameters the
DARTree page sweeps (width W around 8-64, budget B around 64-512, depth
bonus beta <= 0).  No trained weights are involved; see ``inputs.py``.
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int        # seeds the generator; distinct per workload
    d: int             # backbone hidden size (rows of H)
    V: int             # vocabulary size
    e: int             # token-embedding size fed to the GRU
    s: int             # GRU state size
    r: int             # rank of the correction bottleneck
    D: int             # draft depth (block length)
    M: int             # candidates per depth taken from the base logits
    K: int             # children kept per expanded branch
    W: int             # branches kept per depth
    B: int             # node budget of the final tree (root excluded)
    beta: float        # depth bonus, <= 0
    batch: int         # independent requests per round
    wtype: str         # "f32" or "bf16" weight storage

    def with_(self, **kw):
        return replace(self, **kw)


_QWEN4B = dict(d=2560, V=151936, e=2560, s=1024, r=256, D=16, wtype="bf16")
_QWEN8B = dict(d=4096, V=151936, e=4096, s=1024, r=256, D=16, wtype="bf16")

CONFIGS = {
    "tiny": Config("tiny", 0, d=64, V=512, e=32, s=32, r=16, D=4, M=8, K=2,
                   W=4, B=16, beta=-0.1, batch=1, wtype="f32"),
    "qwen3_4b": Config("qwen3_4b", 1, M=32, K=4, W=8, B=64, beta=-0.05,
                       batch=1, **_QWEN4B),
    "wide": Config("wide", 2, M=64, K=8, W=32, B=256, beta=-0.02, batch=1,
                   **_QWEN4B),
    "qwen3_8b_x8": Config("qwen3_8b_x8", 3, M=32, K=4, W=16, B=128,
                          beta=-0.05, batch=8, **_QWEN8B),
    # The stress workload is run at two depth bonuses on the same inputs.
    "stress_b0": Config("stress_b0", 4, M=128, K=8, W=64, B=512, beta=0.0,
                        batch=32, **_QWEN8B),
    "stress_b01": Config("stress_b01", 4, M=128, K=8, W=64, B=512,
                         beta=-0.1, batch=32, **_QWEN8B),
}


def config_by_name(name: str) -> Config:
    return CONFIGS[name]
