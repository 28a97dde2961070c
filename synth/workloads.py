"""The five CSA2 workloads: shapes, dtypes, layer modes and seed streams.

Shapes follow the workload list this implementation is measured on:
  w1  decode, batch 1, one Full layer, 4,096 entries, 1 index head x 64 bf16, k=512
  w2  decode, batch 32, 65,536 entries, group Full/Reindex/Reuse/Reuse, 4x64 bf16, k=2048
  w3  long-context decode, batch 8, 262,144 entries, one Full layer, 4x64 fp8 e4m3, k=2048
  w4  prefill chunk, 4,096 queries against a causal 131,072-entry cache, 4x64 fp8, k=2048
  w5  16-layer decode stack, batch 64, 131,072 entries, (F,Ri,Ru,Ru) x 4, 4x64 bf16, k=2048
  w6  speculative verify: w2 with a draft block of 5 queries per sequence, causal among
      the drafts (query i of the block sees the entries up to its own)
  w7  w2 with FP4 index keys: e2m1 codes with an fp32 scale per 32 elements (the cache
      codec), bf16 index queries
  w8  w2 with hierarchical search: Full keeps a pool of 2,048 blocks of 8 entries
      (16,384 candidates) per query row, Reindex searches only the pool
Every layer: 16 bf16 query heads of dim 128, scale 1/sqrt(128), a 128-row bf16 window,
entries of dim 128 stored as FP4 e2m1 with an fp32 scale per 32 elements.

Stream ids (seed = 0xC5A20000 + 1000*w + stream):
  100*g + 0      cache values of group g        element ((b*N + j)*D + d)
  100*g + 1      index keys of group g          element ((b*N + j)*H_I + h)*d_I + e
  100*g + 10*l + 2  index query of layer l      element ((b*Qs + i)*H_I + h)*d_I + e
  100*g + 10*l + 3  query                       element ((b*Qs + i)*Hq + h)*D + d
  100*g + 10*l + 4  window keys                 element (b*(Qs+W-1) + t)*D + d
  100*g + 10*l + 5  window values               same layout
  100*g + 10*l + 6  new entries (Full layers)   element (b*Qs + i)*D + d
  100*g + 10*l + 7  new index keys (Full)       element ((b*Qs + i)*H_I + h)*d_I + e
"""
from __future__ import annotations

import dataclasses
import math

MODES = ("F", "Ri", "Ru")


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    B: int
    N: int
    H_I: int
    d_I: int
    idx_dtype: str  # 'bf16', 'e4m3' or 'fp4' (keys; fp4 takes bf16 queries)
    k: int
    pattern: tuple  # modes of one sharing group, e.g. ('F','Ri','Ru','Ru')
    groups: int = 1
    Qs: int = 1
    Hq: int = 16
    D: int = 128
    W: int = 128
    pool_blocks: int = 0  # > 0: hierarchical search with a pool of that many 8-entry blocks

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def layers(self) -> int:
        return self.groups * len(self.pattern)

    def seed(self, stream: int) -> int:
        return 0xC5A20000 + 1000 * self.wid + stream

    def stream(self, group: int, layer: int, kind: int) -> int:
        if kind in (0, 1):
            return 100 * group + kind
        return 100 * group + 10 * layer + kind

    def scaled(self, **kw) -> "Workload":
        """Same workload recipe at other sizes (parity cases the oracle finishes quickly)."""
        return dataclasses.replace(self, **kw)


W1 = Workload(1, "decode_b1_n4096_full", B=1, N=4096, H_I=1, d_I=64, idx_dtype="bf16", k=512,
              pattern=("F",))
W2 = Workload(2, "decode_b32_n65536_group_F_Ri_Ru_Ru", B=32, N=65536, H_I=4, d_I=64,
              idx_dtype="bf16", k=2048, pattern=("F", "Ri", "Ru", "Ru"))
W3 = Workload(3, "decode_b8_n262144_full_fp8idx", B=8, N=262144, H_I=4, d_I=64,
              idx_dtype="e4m3", k=2048, pattern=("F",))
W4 = Workload(4, "prefill_q4096_n131072_causal_fp8idx", B=1, N=131072, H_I=4, d_I=64,
              idx_dtype="e4m3", k=2048, pattern=("F",), Qs=4096)
W5 = Workload(5, "decode_b64_n131072_16layer_stack", B=64, N=131072, H_I=4, d_I=64,
              idx_dtype="bf16", k=2048, pattern=("F", "Ri", "Ru", "Ru"), groups=4)

W6 = Workload(6, "verify5_b32_n65536_group_F_Ri_Ru_Ru", B=32, N=65536, H_I=4, d_I=64,
              idx_dtype="bf16", k=2048, pattern=("F", "Ri", "Ru", "Ru"), Qs=5)

W7 = Workload(7, "decode_b32_n65536_group_F_Ri_Ru_Ru_fp4idx", B=32, N=65536, H_I=4, d_I=64,
              idx_dtype="fp4", k=2048, pattern=("F", "Ri", "Ru", "Ru"))

W8 = Workload(8, "decode_b32_n65536_group_F_Ri_Ru_Ru_hier", B=32, N=65536, H_I=4, d_I=64,
              idx_dtype="bf16", k=2048, pattern=("F", "Ri", "Ru", "Ru"), pool_blocks=2048)
ALL = {1: W1, 2: W2, 3: W3, 4: W4, 5: W5, 6: W6, 7: W7, 8: W8}
