"""Seeded synthetic attention inputs, shared by the tests, the oracle side and
the GPU side.

This module holds no step of the attention computation: only workload shapes
and the random-number recipe.  Q, K and V are i.i.d. N(0, 1): the pages'
workloads (BERT-large at length 512, GPT-2 at 1K, Long-Range Arena at 1K-4K,
"FlashAttention (NL)", section "Empirische resultaten") need trained models
and datasets, so dense Gaussian inputs of the shapes below stand in for them.

Recipe: ``numpy.random.default_rng(seed)``; draw q, k, v in that order with
``standard_normal(shape, dtype=float32)``; cast to the workload dtype by
round-to-nearest-even (torch's ``Tensor.to``).  Both sides read these exact
bytes; widening bf16/fp16/fp32 to fp64 for the oracle is exact.  "e4m3"
workloads cast the same draws to torch.float8_e4m3fn (every N(0, 1) draw lies
far inside its range) and are handed over as uint8 codes.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
          "e4m3": torch.float8_e4m3fn}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str      # "f32" | "f16" | "bf16" | "e4m3"
    mask: str       # "none" | "causal" | "sliding"
    window: int     # keys visible to a query under "sliding" (else 0)
    scale: float
    seed: int
    H_kv: int = 0   # key/value heads (0: one per query head)

    @property
    def kv_heads(self) -> int:
        return self.H_kv or self.H


WORKLOADS = [
    Workload("tiny_f32_n128_d64", 1, 1, 128, 64, "f32", "none", 0,
             1.0 / math.sqrt(64), 1000),
    Workload("gpt2s_f16_b16_h12_n1024_d64", 16, 12, 1024, 64, "f16", "none", 0,
             1.0 / 8.0, 1001),
    Workload("prefill_bf16_causal_b4_h16_n2048_d128", 4, 16, 2048, 128, "bf16",
             "causal", 0, 1.0 / math.sqrt(128), 1002),
    Workload("longctx_bf16_causal_b1_h32_n16384_d128", 1, 32, 16384, 128, "bf16",
             "causal", 0, 1.0 / math.sqrt(128), 1003),
    Workload("swa_bf16_w4096_b1_h32_n32768_d128", 1, 32, 32768, 128, "bf16",
             "sliding", 4096, 1.0 / math.sqrt(128), 1004),
]
HEADLINE = WORKLOADS[3]
# The long-context shape with key/value heads shared by groups of query heads
# (4 query heads per key/value head, and one key/value head for all 32).
SHARED_KV_WORKLOADS = [
    Workload("longctx_gqa8_bf16_causal_b1_h32_n16384_d128", 1, 32, 16384, 128, "bf16",
             "causal", 0, 1.0 / math.sqrt(128), 1005, H_kv=8),
    Workload("longctx_mqa_bf16_causal_b1_h32_n16384_d128", 1, 32, 16384, 128, "bf16",
             "causal", 0, 1.0 / math.sqrt(128), 1006, H_kv=1),
]
# Head dim 256: the long-context causal shape with half the heads (the same
# number of FLOPs as the B=1 H=32 N=16384 d=128 workload).
HEAD_DIM_256_WORKLOADS = [
    Workload("longctx_bf16_causal_b1_h16_n16384_d256", 1, 16, 16384, 256, "bf16",
             "causal", 0, 1.0 / math.sqrt(256), 1007),
]
# 8-bit inputs (OCP E4M3): the long-context causal shape, and a batched
# prefill shape.
FP8_WORKLOADS = [
    Workload("longctx_e4m3_causal_b1_h32_n16384_d128", 1, 32, 16384, 128, "e4m3",
             "causal", 0, 1.0 / math.sqrt(128), 1011),
    Workload("prefill_e4m3_causal_b4_h16_n2048_d128", 4, 16, 2048, 128, "e4m3",
             "causal", 0, 1.0 / math.sqrt(128), 1012),
]
BY_NAME = {w.name: w for w in
           WORKLOADS + SHARED_KV_WORKLOADS + HEAD_DIM_256_WORKLOADS + FP8_WORKLOADS}


def make_qkv(B: int, H: int, N: int, d: int, dtype: str, seed: int):
    """q, k, v as contiguous CPU tensors [B, H, N, d] of ``dtype``."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(3):
        x = rng.standard_normal((B, H, N, d), dtype=np.float32)
        out.append(torch.from_numpy(x).to(DTYPES[dtype]).contiguous())
    return tuple(out)


def make_qkv_dout(B: int, H: int, N: int, d: int, dtype: str, seed: int):
    """q, k, v and an output gradient dout, all [B, H, N, d]: the same recipe
    with a fourth draw."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(4):
        x = rng.standard_normal((B, H, N, d), dtype=np.float32)
        out.append(torch.from_numpy(x).to(DTYPES[dtype]).contiguous())
    return tuple(out)


def make_qkv_shared(B: int, H: int, H_kv: int, N: int, d: int, dtype: str, seed: int):
    """q [B, H, N, d] and k, v [B, H_kv, N, d], same recipe and draw order."""
    rng = np.random.default_rng(seed)
    out = []
    for heads in (H, H_kv, H_kv):
        x = rng.standard_normal((B, heads, N, d), dtype=np.float32)
        out.append(torch.from_numpy(x).to(DTYPES[dtype]).contiguous())
    return tuple(out)


def make_qkv_dout_shared(B: int, H: int, H_kv: int, N: int, d: int, dtype: str, seed: int):
    """q [B, H, N, d], k, v [B, H_kv, N, d] and an output gradient dout
    [B, H, N, d]: the same recipe, drawn in that order."""
    rng = np.random.default_rng(seed)
    out = []
    for heads in (H, H_kv, H_kv, H):
        x = rng.standard_normal((B, heads, N, d), dtype=np.float32)
        out.append(torch.from_numpy(x).to(DTYPES[dtype]).contiguous())
    return tuple(out)


def _as_codes(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t


def make_workload(w: Workload):
    """q, k, v of a workload (uint8 E4M3 codes for "e4m3")."""
    if w.dtype == "e4m3":
        return tuple(_as_codes(t) for t in make_qkv_shared(w.B, w.H, w.kv_heads, w.N, w.d,
                                                           w.dtype, w.seed))
    return _make_workload_16(w)


def make_qkv_e4m3(B: int, H: int, H_kv: int, N: int, d: int, seed: int):
    """E4M3 codes (uint8) q [B, H, N, d] and k, v [B, H_kv, N, d]: the
    standard recipe cast to float8_e4m3fn."""
    return tuple(_as_codes(t) for t in make_qkv_shared(B, H, H_kv, N, d, "e4m3", seed))


def make_qkv_e4m3_integer_scores(B: int, H: int, H_kv: int, N: int, d: int, seed: int,
                                 nnz: int = 4):
    """E4M3 codes whose raw scores <q_i, k_j> are integers in [-nnz, nnz]:
    every q row has nnz entries +-1 at random positions (0 elsewhere), every
    k entry is -1, 0 or 1 (uniform), v is the standard N(0, 1) draw.  With
    scale = ln 2 (as a float32) every weight is a power of two times the
    row's normaliser."""
    rng = np.random.default_rng(seed)
    pos = rng.random((B, H, N, d)).argsort(axis=-1)[..., :nnz]
    q = np.zeros((B, H, N, d), dtype=np.float32)
    np.put_along_axis(q, pos, rng.choice(np.array([-1.0, 1.0], dtype=np.float32),
                                         size=pos.shape), axis=-1)
    k = rng.integers(-1, 2, size=(B, H_kv, N, d)).astype(np.float32)
    v = rng.standard_normal((B, H_kv, N, d), dtype=np.float32)
    return tuple(_as_codes(torch.from_numpy(x).to(torch.float8_e4m3fn).contiguous())
                 for x in (q, k, v))


def _make_workload_16(w: Workload):
    if w.kv_heads != w.H:
        return make_qkv_shared(w.B, w.H, w.kv_heads, w.N, w.d, w.dtype, w.seed)
    return make_qkv(w.B, w.H, w.N, w.d, w.dtype, w.seed)


def sha256(t: torch.Tensor) -> str:
    """SHA-256 of a tensor's raw bytes (records exactly what both sides read)."""
    b = t.detach().to("cpu").contiguous().view(torch.uint8).numpy().tobytes()
    return hashlib.sha256(b).hexdigest()
