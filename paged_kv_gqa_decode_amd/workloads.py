"""Seeded synthetic workloads for paged-KV GQA decode attention.

This module only draws inputs: lengths, block tables and N(0, 1) tensors. It
holds none of the attention arithmetic and is the one piece of code that both
the HIP path and the oracle are fed from.

Recipe (fixed generation order, so a seed names one exact input):
  1. cached lengths L_b   (numpy Generator, seed)
  2. block permutation    (same numpy Generator): sequence b takes the next
     ceil(L_b / BS) ids of a random permutation of the physical pool
  3. q, new_k, new_v, k_pool, v_pool: i.i.d. N(0, 1) drawn in float32 with a
     torch Generator seeded with the same seed on the target device, then
     rounded to nearest-even into the I/O dtype
Table entries past a sequence's last page are set to `table_fill` (0 unless a
test asks otherwise); they are never meant to be read.

Workload shapes follow the decode configurations the paged_attention.rs page
(onnxruntime-ep-mlx 0.31.1) is exercised on: a tiny fp32 case, a Llama-3-8B
shaped batch, a long-context split case, a multi-row causal case and a ragged
serving batch.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

DTYPES = {"f32": (torch.float32, 0, 4), "f16": (torch.float16, 1, 2), "bf16": (torch.bfloat16, 2, 2)}


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    B: int
    H: int
    KV: int
    D: int
    BS: int
    NQ: int
    causal: bool
    dtype: str
    lengths: tuple  # ("fixed", L) | ("uniform", lo, hi) | ("lognormal", median, sigma, lo, hi) | ("list", (L0, L1, ...))
    pool: tuple  # ("exact",) | ("oversub", factor) | ("fixed", num_blocks)
    max_blocks: int
    seed: int

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


# The five decode workloads (index = position), seed = 1000 + index.
CONFIGS: Sequence[Spec] = (
    Spec("tiny_fp32", B=1, H=4, KV=2, D=64, BS=16, NQ=1, causal=True, dtype="f32",
         lengths=("fixed", 100), pool=("fixed", 16), max_blocks=7, seed=1000),
    Spec("llama3_8b_decode", B=32, H=32, KV=8, D=128, BS=16, NQ=1, causal=True, dtype="f16",
         lengths=("uniform", 512, 4096), pool=("exact",), max_blocks=256, seed=1001),
    Spec("long_context_splitk", B=4, H=32, KV=8, D=128, BS=16, NQ=1, causal=True, dtype="bf16",
         lengths=("uniform", 32768, 131072), pool=("exact",), max_blocks=8192, seed=1002),
    Spec("multirow_causal", B=16, H=64, KV=8, D=128, BS=16, NQ=8, causal=True, dtype="f16",
         lengths=("uniform", 2048, 8192), pool=("exact",), max_blocks=512, seed=1003),
    Spec("ragged_serving", B=256, H=64, KV=8, D=128, BS=32, NQ=1, causal=True, dtype="bf16",
         lengths=("lognormal", 1024, 1.0, 16, 16384), pool=("oversub", 1.5), max_blocks=512,
         seed=1004),
)


@dataclasses.dataclass
class Workload:
    spec: Spec
    context_lens: np.ndarray  # int32 [B]
    block_table: np.ndarray  # int32 [B, max_blocks]
    num_blocks: int
    q: torch.Tensor  # [B, H, NQ, D]
    k_pool: torch.Tensor  # [num_blocks, BS, KV, D]
    v_pool: torch.Tensor
    new_k: torch.Tensor  # [B, KV, NQ, D]
    new_v: torch.Tensor
    scale: float  # a binary32 value

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0

    @property
    def dtype_code(self) -> int:
        return DTYPES[self.spec.dtype][1]

    @property
    def elem_bytes(self) -> int:
        return DTYPES[self.spec.dtype][2]


def draw_lengths(spec: Spec, rng: np.random.Generator) -> np.ndarray:
    kind = spec.lengths[0]
    if kind == "fixed":
        lens = np.full(spec.B, spec.lengths[1], dtype=np.int64)
    elif kind == "uniform":
        lens = rng.integers(spec.lengths[1], spec.lengths[2], size=spec.B, endpoint=True)
    elif kind == "lognormal":
        median, sigma, lo, hi = spec.lengths[1:]
        z = rng.standard_normal(spec.B)
        lens = np.clip(np.rint(np.exp(math.log(median) + sigma * z)), lo, hi).astype(np.int64)
    elif kind == "list":
        lens = np.asarray(spec.lengths[1], dtype=np.int64)
        assert lens.shape == (spec.B,)
    else:
        raise ValueError(f"unknown length distribution {kind!r}")
    return lens.astype(np.int32)


def _randn(shape, gen: torch.Generator, device, dtype: torch.dtype) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return x.to(dtype) if dtype != torch.float32 else x


def make_workload(spec: Spec, device="cpu", table_fill: int = 0,
                  scale: Optional[float] = None) -> Workload:
    """Draw one workload. Pools are drawn on `device` (use the GPU for large pools)."""
    rng = np.random.default_rng(spec.seed)
    lens = draw_lengths(spec, rng)
    if int(lens.max(initial=0)) > spec.max_blocks * spec.BS:
        raise ValueError("a length exceeds the block-table capacity")
    pages = [(int(L) + spec.BS - 1) // spec.BS for L in lens]
    needed = sum(pages)
    kind = spec.pool[0]
    if kind == "exact":
        nblocks = needed
    elif kind == "oversub":
        nblocks = math.ceil(spec.pool[1] * needed)
    elif kind == "fixed":
        nblocks = spec.pool[1]
    else:
        raise ValueError(f"unknown pool kind {kind!r}")
    nblocks = max(nblocks, 1)
    if nblocks < needed:
        raise ValueError("pool smaller than the pages the sequences need")
    perm = rng.permutation(nblocks).astype(np.int32)
    table = np.full((spec.B, spec.max_blocks), table_fill, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages):
        table[b, :n] = perm[off:off + n]
        off += n

    tdtype = DTYPES[spec.dtype][0]
    gen = torch.Generator(device=device)
    gen.manual_seed(spec.seed)
    q = _randn((spec.B, spec.H, spec.NQ, spec.D), gen, device, tdtype)
    new_k = _randn((spec.B, spec.KV, spec.NQ, spec.D), gen, device, tdtype)
    new_v = _randn((spec.B, spec.KV, spec.NQ, spec.D), gen, device, tdtype)
    k_pool = _randn((nblocks, spec.BS, spec.KV, spec.D), gen, device, tdtype)
    v_pool = _randn((nblocks, spec.BS, spec.KV, spec.D), gen, device, tdtype)
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(spec.D)))
    return Workload(spec, lens, table, nblocks, q, k_pool, v_pool, new_k, new_v,
                    float(np.float32(scale)))


def kv_bytes(w: Workload) -> int:
    """Algorithmic K+V bytes of one decode step: sum_b (L_b + NQ) * KV * D * 2 * s."""
    s = w.spec
    return int(sum(int(L) + s.NQ for L in w.context_lens)) * s.KV * s.D * 2 * w.elem_bytes


def step_bytes(w: Workload) -> int:
    """kv_bytes plus q read, out write, table entries read and the lengths."""
    s = w.spec
    pages = sum((int(L) + s.BS - 1) // s.BS for L in w.context_lens)
    return (kv_bytes(w) + 2 * s.B * s.H * s.NQ * s.D * w.elem_bytes + 4 * pages + 4 * s.B)


def shrink(spec: Spec, B: Optional[int] = None, lengths: Optional[tuple] = None,
           max_blocks: Optional[int] = None, seed: Optional[int] = None) -> Spec:
    """A smaller variant of a workload with the same head geometry and dtype."""
    kw = {}
    if B is not None:
        kw["B"] = B
    if lengths is not None:
        kw["lengths"] = lengths
    if max_blocks is not None:
        kw["max_blocks"] = max_blocks
    if seed is not None:
        kw["seed"] = seed
    return spec.replace(name=spec.name + "_small", **kw)
