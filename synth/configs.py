"""The five rank-share workloads, plus reduced copies for fast parity runs.

Each case is one context-parallel rank's share: T tokens split over n_cp
ranks in a layout, h_q query heads and h_kv key/value heads of width d_k.
Sizes follow the long-context stages discussed on the pages (Llama 3 8B-like,
70B and 405B shares after tensor parallelism of 8, and a million-token
striped run).  All inputs are synthetic N(0, 1) draws (Q and K times 2 for the
peaky striped case).
"""

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Case:
    name: str
    T: int
    n_cp: int
    layout: str
    ranks: tuple  # ranks whose share is run (in turn)
    h_q: int
    h_kv: int
    d_k: int
    dtype: str  # "f32" or "bf16"
    seed: int
    q_amp: float = 1.0
    k_amp: float = 1.0
    v_amp: float = 1.0
    causal: bool = True

    @property
    def n(self):
        return self.T // self.n_cp

    def reduced(self, T, n_cp=None, ranks=None, name=None):
        """Same heads, dtype, layout and seed at a smaller sequence."""
        return replace(self, T=T, n_cp=n_cp or self.n_cp, ranks=ranks or self.ranks,
                       name=name or f"{self.name}@T{T}")


CASES = (
    Case("tiny_f32_contiguous", T=1024, n_cp=4, layout="contiguous", ranks=(2,),
         h_q=4, h_kv=4, d_k=64, dtype="f32", seed=1001),
    Case("llama8b_gqa_zigzag", T=32768, n_cp=4, layout="zigzag", ranks=(0, 1, 2, 3),
         h_q=32, h_kv=8, d_k=128, dtype="bf16", seed=1002),
    Case("llama70b_stage_share", T=131072, n_cp=16, layout="zigzag", ranks=(0,),
         h_q=8, h_kv=1, d_k=128, dtype="bf16", seed=1003),
    Case("llama405b_stage_share", T=131072, n_cp=16, layout="zigzag", ranks=(0,),
         h_q=16, h_kv=1, d_k=128, dtype="bf16", seed=1004),
    Case("million_striped_mha", T=524288, n_cp=64, layout="striped", ranks=(0,),
         h_q=8, h_kv=8, d_k=128, dtype="bf16", seed=1005, q_amp=2.0, k_amp=2.0),
)


# Ulysses local shares (heads split across the group, every GPU attends its
# heads over the whole sequence): one block of all T keys, positions 0..T-1.
# 8B-like: 32 q / 8 kv heads over 4 GPUs -> 8 q / 2 kv heads each.
# 405B stage after tensor parallelism: 16 q / 1 kv heads over 16 GPUs -> one
# query head each, the single key/value head replicated.
ULYSSES_CASES = (
    Case("llama8b_ulysses_share", T=32768, n_cp=1, layout="contiguous", ranks=(0,),
         h_q=8, h_kv=2, d_k=128, dtype="bf16", seed=1006),
    Case("llama405b_ulysses_share", T=131072, n_cp=1, layout="contiguous", ranks=(0,),
         h_q=1, h_kv=1, d_k=128, dtype="bf16", seed=1007),
)


def case_by_name(name):
    for c in CASES + ULYSSES_CASES:
        if c.name == name:
            return c
    raise KeyError(name)
