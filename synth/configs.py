"""Workload shapes for the five synthetic decode configurations.

Shapes follow the models the SparDA and SSV reading notes measure on:
Llama-3-8B / MiniCPM-like layers (8 KV heads, head dim 128, GQA group 4),
a 70B-like layer (8 KV heads, group 8), 32K-256K contexts, 64-token blocks
("SparDA: 稀疏解耦注意力" note, prerequisites §3 and eq. (1)-(4); "SSV: 稀疏投机验证"
note, experimental setup).
"""
from dataclasses import dataclass, field

BLOCK = 64


@dataclass(frozen=True)
class Config:
    cid: int                 # 1..5
    name: str
    B: int                   # batch
    H_q: int                 # query heads
    H_kv: int                # KV heads
    d: int                   # head dim
    T: int                   # cached tokens (all sequences the same length)
    n_init: int
    n_local: int
    top_k: int
    NQ: int = 1              # queries per sequence (draft queries in grouped mode)
    group_C: int = 1         # SSV group size
    layers: int = 1          # distinct layers of K/V in the workload
    bias_frac: float = 0.0   # fraction of blocks given a key bias along F (config 2)
    bias_beta: float = 0.0
    gammas: tuple = field(default_factory=tuple)  # target adjacent-query overlaps (config 4)

    @property
    def G(self):
        return self.H_q // self.H_kv

    @property
    def NB(self):
        return -(-self.T // BLOCK)

    @property
    def n_sel(self):
        return min(self.NB, self.n_init + self.n_local + self.top_k)

    @property
    def rows(self):
        """Selection rows: one per (batch, query, KV head)."""
        return self.B * self.NQ * self.H_kv

    def selected_kv_bytes(self):
        """K and V bytes of the selected blocks, one layer, one query per row."""
        return self.rows * self.n_sel * BLOCK * self.d * 2 * 2

    def ktilde_bytes(self):
        """Compressed keys of one layer (bf16): the bytes one scoring pass reads."""
        return self.B * self.H_kv * self.NB * self.d * 2


CONFIGS = {
    1: Config(1, "tiny decode, d=64, T=4K", B=1, H_q=8, H_kv=2, d=64, T=4096,
              n_init=1, n_local=2, top_k=8),
    2: Config(2, "Llama-3-8B-shaped layer, T=32K", B=8, H_q=32, H_kv=8, d=128, T=32768,
              n_init=1, n_local=2, top_k=16, bias_frac=0.05, bias_beta=1.0),
    3: Config(3, "70B-shaped layer at 128K", B=8, H_q=64, H_kv=8, d=128, T=131072,
              n_init=1, n_local=2, top_k=32, layers=2),
    4: Config(4, "SSV grouped verification, T=64K", B=4, H_q=32, H_kv=8, d=128, T=65536,
              n_init=0, n_local=0, top_k=16, NQ=16, group_C=4, gammas=(0.5, 0.75, 0.9)),
    5: Config(5, "offloaded-KV decode, T=256K, 8 layers", B=4, H_q=32, H_kv=8, d=128,
              T=262144, n_init=1, n_local=2, top_k=32, layers=8),
}


def get_config(cid):
    return CONFIGS[int(cid)]
