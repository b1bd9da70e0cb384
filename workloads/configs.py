"""Workload shapes for the verification step.

Each workload fixes the batch, head layout, draft length, context lengths, KV
storage type and the acceptance inputs.  The five named workloads are the
verification-step shapes this project is measured and checked on; the ``mini_*``
and ``edge_*`` workloads are reduced shapes the CPU oracle finishes in seconds
while still spanning several key tiles, several splits and a ragged last block.

Notation (used across the project):
  B      sequences in the batch
  D      draft tokens per sequence; R = D + 1 verified positions
  H_q    query heads, H_kv KV heads, G = H_q / H_kv
  hd     head dimension
  T_b    context length of sequence b before this step; the cache already holds
         the R new positions, so the kernel is given L_b = T_b + R
  V      vocabulary size of the target logits
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

BLOCK_SIZE = 16  # tokens per KV block (the paged-attention default on the pages)

KV_BF16 = "bf16"
KV_FP8 = "fp8_e4m3"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    H_q: int
    H_kv: int
    hd: int
    D: int
    # context length: fixed value, or an inclusive integer range drawn per sequence
    T: Optional[int] = None
    T_range: Optional[Tuple[int, int]] = None
    kv_dtype: str = KV_BF16
    identity_table: bool = False
    # acceptance inputs; V = 0 means the workload is attention only
    V: int = 0
    p_match: Optional[float] = None
    p_range: Optional[Tuple[float, float]] = None
    # spare physical blocks that no sequence uses (they hold poison)
    spare_blocks: int = 0

    @property
    def R(self) -> int:
        return self.D + 1

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def M(self) -> int:
        """Query rows that share one KV head: G * (1 + D)."""
        return self.G * self.R

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.hd)

    @property
    def max_T(self) -> int:
        return self.T if self.T is not None else self.T_range[1]

    @property
    def max_kv_len(self) -> int:
        return self.max_T + self.R

    @property
    def max_blocks_per_seq(self) -> int:
        return -(-self.max_kv_len // BLOCK_SIZE)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five verification-step workloads (seed = 1000 + index).
TINY = Workload("tiny", 1000, B=1, H_q=8, H_kv=2, hd=64, D=3, T=256,
                identity_table=True, V=1024, p_match=0.7)
LLAMA3_8B = Workload("llama3_8b_gqa4_d7", 1001, B=16, H_q=32, H_kv=8, hd=128, D=7,
                     T=8192, V=128256, p_match=0.6)
LLAMA31_70B = Workload("llama31_70b_gqa8_d15", 1002, B=32, H_q=64, H_kv=8, hd=128, D=15,
                       T_range=(2048, 32768), V=128256, p_range=(0.3, 0.9))
FP8_LONG = Workload("fp8_long_gqa8_d15", 1004, B=4, H_q=64, H_kv=8, hd=128, D=15,
                    T=131072, kv_dtype=KV_FP8, V=128256, p_range=(0.3, 0.9))

SWEEP_D = (1, 3, 7, 15, 16, 23, 31)


def tile_sweep(D: int, mqa: bool) -> Workload:
    """Tile-boundary sweep: B=8, H_q=64, H_kv=8 (or 1 for MQA), T=16384, bf16."""
    return Workload(f"tile_sweep_{'mqa' if mqa else 'gqa8'}_d{D}", 1003, B=8, H_q=64,
                    H_kv=1 if mqa else 8, hd=128, D=D, T=16384)


NAMED = {w.name: w for w in (TINY, LLAMA3_8B, LLAMA31_70B, FP8_LONG)}

# Reduced shapes for element-by-element parity against the oracle.
MINI = {
    "mini_gqa4_d7": Workload("mini_gqa4_d7", 2001, B=3, H_q=8, H_kv=2, hd=128, D=7,
                             T_range=(1, 900), V=5000, p_match=0.6, spare_blocks=3),
    "mini_gqa8_d15": Workload("mini_gqa8_d15", 2002, B=3, H_q=16, H_kv=2, hd=128, D=15,
                              T_range=(200, 2500), V=7001, p_range=(0.3, 0.9)),
    "mini_fp8_d15": Workload("mini_fp8_d15", 2003, B=2, H_q=16, H_kv=2, hd=128, D=15,
                             T_range=(300, 3000), kv_dtype=KV_FP8, V=4096,
                             p_range=(0.3, 0.9), spare_blocks=2),
    "mini_mqa_d16": Workload("mini_mqa_d16", 2004, B=2, H_q=64, H_kv=1, hd=128, D=16,
                             T_range=(100, 700)),
    "mini_mqa_d3": Workload("mini_mqa_d3", 2005, B=2, H_q=64, H_kv=1, hd=128, D=3,
                            T_range=(500, 1300)),
    # 1024 rows per KV head: four 256-row units that share the KV head
    "mini_mqa_d15": Workload("mini_mqa_d15", 2008, B=2, H_q=64, H_kv=1, hd=128, D=15,
                             T_range=(100, 700)),
    "mini_hd64_g4": Workload("mini_hd64_g4", 2006, B=4, H_q=8, H_kv=2, hd=64, D=3,
                             T_range=(0, 1000), V=333, p_match=0.7),
    "mini_fp8_hd64": Workload("mini_fp8_hd64", 2007, B=2, H_q=4, H_kv=1, hd=64, D=5,
                              T_range=(1, 600), kv_dtype=KV_FP8),
}

# Degenerate cases the method has.
EDGE = {
    # T_b = 0: the R new positions attend causally among themselves only
    "edge_empty_context": Workload("edge_empty_context", 3001, B=2, H_q=8, H_kv=2, hd=128,
                                   D=7, T=0, V=64, p_match=1.0),
    # D = 0: plain decode, one query position, AL is always 1
    "edge_plain_decode": Workload("edge_plain_decode", 3002, B=3, H_q=8, H_kv=2, hd=128,
                                  D=0, T_range=(1, 300), V=100, p_match=0.5),
    # G = 1: multi-head attention
    "edge_mha": Workload("edge_mha", 3003, B=2, H_q=4, H_kv=4, hd=128, D=3,
                         T_range=(10, 200), V=50, p_match=0.9),
    # one visible key for position 0
    "edge_one_key": Workload("edge_one_key", 3004, B=1, H_q=2, H_kv=1, hd=64, D=0, T=0,
                             V=7, p_match=0.0),
    # largest supported draft length
    "edge_d63": Workload("edge_d63", 3005, B=2, H_q=4, H_kv=2, hd=64, D=63,
                         T_range=(0, 150), V=97, p_range=(0.0, 1.0)),
}


def all_workloads():
    out = dict(NAMED)
    out.update(MINI)
    out.update(EDGE)
    for D in SWEEP_D:
        for mqa in (False, True):
            w = tile_sweep(D, mqa)
            out[w.name] = w
    return out
