"""Named workload presets for the int8-state decode path.

Each preset fixes the head shape, window W, compensator count C, decay form,
token count T, prefill length and input distribution.  The window of 16
tokens and the 4 compensator tokens are the values the LeapQuant news article
('A linear-attention method cuts state storage', paragraphs 3 and 4) reports.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

GDN = 0   # scalar decay per head and token (Gated DeltaNet)
KDA = 1   # per-key-channel decay (Kimi Delta Attention style diagonal gating)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    dk: int
    dv: int
    W: int
    C: int
    T: int
    decay: int = GDN
    prefill: int = 0          # fp32 prefill tokens before decoding (0 = zero state)
    beta_lo: float = 0.1
    beta_hi: float = 0.9
    outliers: bool = False    # 4 key channels x30, 2 value columns x20 per head
    smooth: int = 1
    seed: int = 1000
    w_sweep: tuple = field(default=())

    @property
    def per_key(self) -> bool:
        return self.decay == KDA

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


PRESETS = {
    "tiny_gdn": Workload("tiny_gdn", B=1, H=1, dk=16, dv=16, W=4, C=1, T=64,
                         beta_lo=0.0, beta_hi=1.0, seed=1000),
    "gdn_layer": Workload("gdn_layer", B=1, H=16, dk=128, dv=128, W=16, C=4, T=256,
                          prefill=512, seed=1001),
    "gdn_batched": Workload("gdn_batched", B=64, H=32, dk=128, dv=128, W=16, C=4, T=1024,
                            prefill=512, seed=1002),
    "kda": Workload("kda", B=32, H=32, dk=128, dv=128, W=16, C=4, T=512, decay=KDA,
                    prefill=512, seed=1003),
    "outlier_sweep": Workload("outlier_sweep", B=256, H=32, dk=128, dv=128, W=16, C=4, T=1024,
                              prefill=2048, outliers=True, seed=1004, w_sweep=(8, 16, 32)),
}

ORDER = ["tiny_gdn", "gdn_layer", "gdn_batched", "kda", "outlier_sweep"]
