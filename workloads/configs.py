"""The five verify-step workloads (sizes, dtype, decoding parameters, seed)."""

from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Config:
    name: str
    mode: str  # "sample" or "greedy"
    B: int
    gamma: int
    V: int
    dtype: str  # "f32" or "bf16"
    temperature: float
    top_k: int
    top_p: float
    seed: int
    stats: bool = False  # the workload also asks for acceptance statistics

    @property
    def rows(self) -> int:
        return self.B * (self.gamma + 1)

    @property
    def logit_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    "toy": Config("toy", "sample", 1_000_000, 4, 5, "f32", 1.0, 0, 1.0, 1000),
    "c2": Config("c2", "sample", 64, 4, 32000, "f32", 1.0, 0, 1.0, 1002),
    "c3": Config("c3", "sample", 256, 5, 128256, "bf16", 0.8, 50, 1.0, 1003),
    "c4": Config("c4", "greedy", 512, 8, 152064, "bf16", 1.0, 0, 1.0, 1004),
    "c5": Config("c5", "sample", 1024, 4, 256000, "bf16", 0.7, 0, 0.95, 1005, stats=True),
}
