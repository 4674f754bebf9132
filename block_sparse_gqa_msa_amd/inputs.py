"""Seeded synthetic inputs for the MSA workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic, so both the HIP path and the fp64 oracle can be fed from
it. The shapes and distributions follow the workloads the MSA pages discuss
(1M-token context, GQA with 4 KV groups, 128-dim heads, an index branch with one
index-query head per group and one shared index key; "MiniMax-M3: MSA 技术报告速读",
section 核心机制 and section 实验数字).

Layouts (all contiguous, row-major):
  q      [B, H_q, n_q, d_h]      main-branch queries
  k, v   [B, H_kv, n_k, d_h]     main-branch keys / values (head-major: one
                                 (group, block) is one contiguous span)
  q_idx  [B, H_kv, n_q, d_idx]   index-branch queries, one head per group
  k_idx  [B, n_k, d_idx]         index-branch key, shared by all groups

Draw order inside one torch.Generator: q, k, v, q_idx, k_idx (each tensor drawn
sequence by sequence), then the needle blocks of each sequence.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" or "bf16": storage type of q, k, v, q_idx, k_idx and o
    batch: int
    n_q: int            # query rows per call
    n_k: int            # visible KV length
    q_start: int        # absolute position of query row 0
    h_q: int
    h_kv: int           # GQA groups = index heads
    d_h: int
    d_idx: int
    block_size: int
    top_k: int          # counts the forced local block
    idx_range: int      # index inputs are integers drawn uniformly from [-idx_range, idx_range]
    qkv_scale: float    # q, k, v ~ qkv_scale * N(0, 1)
    needles: int        # needle blocks per sequence (+2 on every k_idx entry of the block)
    seed: int

    @property
    def n_blocks(self) -> int:
        return -(-self.n_k // self.block_size)

    @property
    def decode(self) -> bool:
        return self.n_q == 1 and self.q_start == self.n_k - 1

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


_COMMON = dict(h_q=32, h_kv=4, d_h=128, d_idx=64, block_size=64, idx_range=4,
               qkv_scale=0.5, dtype="bf16")

WORKLOADS: Dict[str, Workload] = {
    # tiny fp32 causal prefill: 8 query heads in 4 groups, 16 blocks of 32, k=4
    "prefill_512_f32": Workload("prefill_512_f32", "f32", 1, 512, 512, 0, 8, 4, 64, 32,
                                32, 4, 3, 1.0, 0, 1),
    # causal prefill N=8192, 128 blocks, k=16, 8 needle blocks
    "prefill_8k": Workload("prefill_8k", batch=1, n_q=8192, n_k=8192, q_start=0, top_k=16,
                           needles=8, seed=2, **_COMMON),
    # long causal prefill N=131072, 2048 blocks, k=32, 64 needle blocks
    "prefill_128k": Workload("prefill_128k", batch=1, n_q=131072, n_k=131072, q_start=0,
                             top_k=32, needles=64, seed=3, **_COMMON),
    # the same prefill with every index input zero: all block scores tie, so every row
    # takes blocks 0..k-2 plus its local block (the most skewed block popularity)
    "prefill_128k_hot": Workload("prefill_128k_hot", batch=1, n_q=131072, n_k=131072, q_start=0,
                                 top_k=32, needles=0, seed=3,
                                 **dict(_COMMON, idx_range=0)),
    # decode: 32 sequences with 262144 cached tokens each, k=32
    "decode_256k_b32": Workload("decode_256k_b32", batch=32, n_q=1, n_k=262144,
                                q_start=262143, top_k=32, needles=8, seed=4, **_COMMON),
    # chunked prefill: 8192 rows at positions 1040384..1048575 against a 1M-token cache
    "chunk_1m": Workload("chunk_1m", batch=1, n_q=8192, n_k=1048576, q_start=1040384,
                         top_k=32, needles=8, seed=51, **_COMMON),
    # decode: 4 sequences with 1048576 cached tokens each, k=32
    "decode_1m_b4": Workload("decode_1m_b4", batch=4, n_q=1, n_k=1048576, q_start=1048575,
                             top_k=32, needles=8, seed=52, **_COMMON),
}


def torch_dtype(w: Workload) -> torch.dtype:
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def generate(w: Workload, device="cpu", seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Draw the inputs of workload ``w`` on ``device``.

    q, k, v are Gaussian (fp32 draw, scaled, then rounded once to the storage
    type, round-to-nearest-even). q_idx and k_idx are integers, exactly
    representable in both storage types, so index scores are exact in fp32.
    Needle blocks get +2 on every k_idx component of every token in them.
    Returns a dict with q, k, v, q_idx, k_idx and ``needles`` (int64 [B, n]).
    """
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed if seed is None else seed)
    dt = torch_dtype(w)
    B = w.batch

    def gauss(shape_per_seq):
        out = torch.empty((B,) + shape_per_seq, dtype=dt, device=device)
        for b in range(B):
            x = torch.randn(shape_per_seq, generator=gen, device=device, dtype=torch.float32)
            if w.qkv_scale != 1.0:
                x.mul_(w.qkv_scale)
            out[b].copy_(x)
            del x
        return out

    def ints(shape_per_seq):
        out = torch.empty((B,) + shape_per_seq, dtype=dt, device=device)
        for b in range(B):
            x = torch.randint(-w.idx_range, w.idx_range + 1, shape_per_seq, generator=gen,
                              device=device, dtype=torch.int32)
            out[b].copy_(x)
            del x
        return out

    q = gauss((w.h_q, w.n_q, w.d_h))
    k = gauss((w.h_kv, w.n_k, w.d_h))
    v = gauss((w.h_kv, w.n_k, w.d_h))
    q_idx = ints((w.h_kv, w.n_q, w.d_idx))
    k_idx = ints((w.n_k, w.d_idx))
    nb = w.n_blocks
    needles = torch.zeros((B, w.needles), dtype=torch.int64, device=device)
    for b in range(B):
        if w.needles:
            blocks = torch.randperm(nb, generator=gen, device=device)[: w.needles]
            needles[b] = blocks
            for c in blocks.tolist():
                lo, hi = c * w.block_size, min((c + 1) * w.block_size, w.n_k)
                k_idx[b, lo:hi] += 2
    return dict(q=q, k=k, v=v, q_idx=q_idx, k_idx=k_idx, needles=needles)


def generate_dout(w: Workload, device="cpu", seed: Optional[int] = None) -> torch.Tensor:
    """The output gradient for the backward of workload ``w``: [B, H_q, n_q, d_h] Gaussian
    scaled like q (fp32 draw rounded once to the storage type), from its own stream
    (seed + 1 unless ``seed`` is given)."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed((w.seed + 1) if seed is None else seed)
    out = torch.empty((w.batch, w.h_q, w.n_q, w.d_h), dtype=torch_dtype(w), device=device)
    for b in range(w.batch):
        x = torch.randn((w.h_q, w.n_q, w.d_h), generator=gen, device=device, dtype=torch.float32)
        if w.qkv_scale != 1.0:
            x.mul_(w.qkv_scale)
        out[b].copy_(x)
        del x
    return out


def generate_hidden(w: Workload, d_model: int, device="cpu", seed: Optional[int] = None,
                    integer: bool = False) -> Dict[str, torch.Tensor]:
    """Hidden states and the index branch's two projection weights for workload ``w``:
    x [B, n_q, d_model], w_q [h_kv * d_idx, d_model] and w_k [d_idx, d_model] in the
    storage type, from their own stream (seed + 2 unless ``seed`` is given).

    Default: x ~ N(0, 1) and weights ~ N(0, 1 / d_model), so the projections have unit
    scale. ``integer=True``: x in [-2, 2] and weights in [-1, 1], integers, so for
    d_model <= 128 every sum is an integer of magnitude <= 256, exact in fp32 and bf16."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed((w.seed + 2) if seed is None else seed)
    dt = torch_dtype(w)

    def draw(shape, scale, lo, hi):
        if integer:
            v = torch.randint(lo, hi + 1, shape, generator=gen, device=device, dtype=torch.int32)
        else:
            v = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
            if scale != 1.0:
                v.mul_(scale)
        return v.to(dt)

    x = torch.empty((w.batch, w.n_q, d_model), dtype=dt, device=device)
    for b in range(w.batch):
        x[b] = draw((w.n_q, d_model), 1.0, -2, 2)
    w_q = draw((w.h_kv * w.d_idx, d_model), d_model ** -0.5, -1, 1)
    w_k = draw((w.d_idx, d_model), d_model ** -0.5, -1, 1)
    return dict(x=x, w_q=w_q, w_k=w_k)
