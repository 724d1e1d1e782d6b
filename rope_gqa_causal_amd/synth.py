"""Seeded synthetic inputs and the named workload shapes.

This module draws random numbers and names shapes; it holds none of the
attention arithmetic, so the HIP path and the CPU oracle can both be fed from
it.  Everything is drawn on the CPU from ``torch.Generator`` seeded per
workload, as float32 standard normals, then cast to bfloat16 (round to
nearest even) where the workload is bf16.

Workload shapes and where they come from:

* ``tiny``: batch 1, 4 query / 2 KV heads, head dim 32, fp32, RoPE base
  10000, 16 prefill tokens then 8 cached decode steps.  A correctness anchor.
* ``llama125m``: 12 layers each with its own cache, 12 query / 4 KV heads,
  head dim 64 (d_model 768), batch 1, bf16; prefill 512 then 100 decode
  steps, the shape of the cached-generation experiment on the page
  "750美元从零训练3个LLM：一位开发者的实战复盘" (section V3: 100 new tokens
  after a 512-token prompt).
* ``prefill3p8b``: batch 8, 2048 tokens, 24 query / 8 KV heads of dim 128,
  bf16; the head layout of the 3.8B model on the page "训练3.8B LLM至0.384
  CORE，成本998美元 – Hugo Vergnes" (section 设置, model table).
* ``ragged_decode``: 64 sequences with cache lengths uniform on
  {256..2048}, 24 query / 8 KV heads of dim 128, bf16, 32 steps of one new
  token per sequence.
* ``diff``: differential attention, batch 4, 1024 tokens, 16 query / 8 KV
  heads, two maps of dim 64, value dim 64, lambda 0.8, bf16.
* ``varlen``: the 3.8B-shaped prefill's 16384 tokens packed as documents
  whose lengths are uniform on {64..4096} (the last one cut to fit), 24 query
  / 8 KV heads of dim 128, bf16: document-masked packing as on the 3.8B page
  (section 无效的方法).
"""
from dataclasses import dataclass, field

import torch

BASE = 10000.0


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    dtype: torch.dtype
    S: int = 0            # prefill tokens
    steps: int = 0        # decode steps
    layers: int = 1
    len_lo: int = 0       # ragged cache lengths (inclusive) before step 0
    len_hi: int = 0
    Dv: int = 0
    lam: float = 0.0
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def group(self):
        return self.Hq // self.Hkv


WORKLOADS = {
    "tiny": Workload("tiny", B=1, Hq=4, Hkv=2, D=32, dtype=torch.float32, S=16, steps=8, seed=1),
    "llama125m": Workload("llama125m", B=1, Hq=12, Hkv=4, D=64, dtype=torch.bfloat16,
                          S=512, steps=100, layers=12, seed=2),
    "prefill3p8b": Workload("prefill3p8b", B=8, Hq=24, Hkv=8, D=128, dtype=torch.bfloat16,
                            S=2048, seed=3),
    "ragged_decode": Workload("ragged_decode", B=64, Hq=24, Hkv=8, D=128, dtype=torch.bfloat16,
                              steps=32, len_lo=256, len_hi=2048, seed=4),
    "diff": Workload("diff", B=4, Hq=16, Hkv=8, D=64, dtype=torch.bfloat16, S=1024,
                     Dv=64, lam=0.8, seed=5),
    "varlen": Workload("varlen", B=1, Hq=24, Hkv=8, D=128, dtype=torch.bfloat16, S=16384,
                       len_lo=64, len_hi=4096, seed=6),
}


def document_lengths(total: int, lo: int, hi: int, gen: torch.Generator) -> torch.Tensor:
    """Document lengths uniform on {lo..hi} drawn until they cover ``total``
    tokens; the last one is cut so the lengths sum to ``total`` (int32)."""
    out, used = [], 0
    while used < total:
        n = int(torch.randint(lo, hi + 1, (1,), generator=gen).item())
        n = min(n, total - used)
        out.append(n)
        used += n
    return torch.tensor(out, dtype=torch.int32)


def generator(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def normal(shape, gen: torch.Generator, dtype=torch.bfloat16) -> torch.Tensor:
    """Standard normal float32 draws cast to ``dtype`` (CPU tensor)."""
    return torch.randn(tuple(shape), generator=gen, dtype=torch.float32).to(dtype)


def lengths(B: int, lo: int, hi: int, gen: torch.Generator) -> torch.Tensor:
    """B integers uniform on {lo..hi} inclusive (int32, CPU)."""
    return torch.randint(lo, hi + 1, (B,), generator=gen, dtype=torch.int64).to(torch.int32)


def qkv(B, S, Hq, Hkv, D, gen, dtype=torch.bfloat16, Dv=None):
    """Fresh q [B,S,Hq,D], k [B,S,Hkv,D], v [B,S,Hkv,Dv] drawn in that order."""
    q = normal((B, S, Hq, D), gen, dtype)
    k = normal((B, S, Hkv, D), gen, dtype)
    v = normal((B, S, Hkv, Dv or D), gen, dtype)
    return q, k, v


def filled_cache(B, Hkv, S_max, D, gen, dtype=torch.bfloat16):
    """A cache pair [B,Hkv,S_max,D] of normal draws (keys treated as rotated)."""
    k = normal((B, Hkv, S_max, D), gen, dtype)
    v = normal((B, Hkv, S_max, D), gen, dtype)
    return k, v


def nan_cache(B, Hkv, S_max, D, dtype=torch.bfloat16):
    """A cache pair filled with NaN canaries, so a read of an unwritten slot shows."""
    k = torch.full((B, Hkv, S_max, D), float("nan"), dtype=dtype)
    return k, k.clone()
