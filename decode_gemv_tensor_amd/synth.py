"""Seeded synthetic inputs for the tests, the smoke check and the benchmark.

This module only draws random numbers and lays out shapes; it holds none of
the method's arithmetic, so both the HIP path and the oracle can be fed from
it. Weights are float32 normals times sigma, a seeded share of them scaled as
outliers, then rounded to bf16 (torch's round-to-nearest-even). The same seed
on the same device always gives the same bits; the CPU and GPU generators are
different streams, so a test that compares against the oracle hands the
oracle the exact bits it gave the kernel.

Shapes and distributions follow the workloads the pages describe: weight
matrices of LLM linear layers (Llama 3.2 3B and Gemma-class 12B shapes, an
embedding-like tensor for bulk decode, and a 128-expert MoE layer).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class TensorSpec:
    name: str
    rows: int          # N, outputs
    cols: int          # K, inputs
    sigma: float
    seed: int
    outlier_frac: float = 0.0
    outlier_count: int = 0
    outlier_scale: float = 1.0


def normal_bf16(spec: TensorSpec, device="cpu") -> torch.Tensor:
    """bf16 [rows, cols]: N(0, sigma) with seeded outliers."""
    g = torch.Generator(device=device)
    g.manual_seed(spec.seed)
    w = torch.randn(spec.rows, spec.cols, generator=g, device=device,
                    dtype=torch.float32)
    w.mul_(spec.sigma)
    n = spec.rows * spec.cols
    n_out = spec.outlier_count or int(round(spec.outlier_frac * n))
    if n_out and spec.outlier_scale != 1.0:
        pos = torch.randint(0, n, (n_out,), generator=g, device=device)
        pos = torch.unique(pos)
        flat = w.view(-1)
        flat[pos] = flat[pos] * spec.outlier_scale
    return w.to(torch.bfloat16)


def vector_bf16(k: int, seed: int, device="cpu", sigma: float = 1.0,
                count: int | None = None) -> torch.Tensor:
    """bf16 [k] (or [count, k]) of N(0, sigma) activations."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    shape = (k,) if count is None else (count, k)
    v = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    return (v * sigma).to(torch.bfloat16)


def topk_indices(n_tokens: int, top_k: int, n_experts: int, seed: int,
                 device="cpu") -> torch.Tensor:
    """int32 [n_tokens, top_k]: top_k distinct experts per token, uniform
    without replacement."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    keys = torch.rand(n_tokens, n_experts, generator=g, device=device)
    return torch.argsort(keys, dim=1)[:, :top_k].to(torch.int32).contiguous()


def router_weights(n_tokens: int, top_k: int, seed: int, device="cpu") -> torch.Tensor:
    """fp32 [n_tokens, top_k] of positive weights summing to one per token (a
    router's normalised top-k scores), from seeded N(0, 1) logits."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    logits = torch.randn(n_tokens, top_k, generator=g, device=device, dtype=torch.float32)
    return torch.softmax(logits, dim=1).contiguous()


def bits(t: torch.Tensor) -> torch.Tensor:
    """The raw 16-bit patterns of a bf16 tensor, as int16 (same storage)."""
    return t.view(torch.int16)


# ---------------------------------------------------------------- workloads
def single_1024() -> list[TensorSpec]:
    """One 1024x1024 weight, N(0, 0.02), seed 0, 16 outliers x50."""
    return [TensorSpec("w", 1024, 1024, 0.02, 0, outlier_count=16,
                       outlier_scale=50.0)]


LLAMA_3B_LAYERS = 28
LLAMA_3B_SHAPES = [("q", 3072, 3072), ("k", 1024, 3072), ("v", 1024, 3072),
                   ("o", 3072, 3072), ("gate", 8192, 3072),
                   ("up", 8192, 3072), ("down", 3072, 8192)]


def llama32_3b_stack(layers: int = LLAMA_3B_LAYERS) -> list[TensorSpec]:
    """Llama-3.2-3B-shaped linear stack: 7 matrices per layer, N(0, 0.02),
    0.1% outliers x20, seed 1000 + tensor index."""
    out = []
    for layer in range(layers):
        for j, (nm, n, k) in enumerate(LLAMA_3B_SHAPES):
            t = layer * len(LLAMA_3B_SHAPES) + j
            out.append(TensorSpec(f"L{layer}.{nm}", n, k, 0.02, 1000 + t,
                                  outlier_frac=1e-3, outlier_scale=20.0))
    return out


def gemma_12b_ffn() -> list[TensorSpec]:
    """12B-class FFN shapes, hidden 3840 and FFN 15360, N(0, 0.015)."""
    return [TensorSpec("gate", 15360, 3840, 0.015, 2000),
            TensorSpec("up", 15360, 3840, 0.015, 2001),
            TensorSpec("down", 3840, 15360, 0.015, 2002)]


def embedding_64m() -> TensorSpec:
    """Embedding-like 262144x256 tensor (64M weights) for bulk decode."""
    return TensorSpec("embed", 262144, 256, 0.015, 2100)


MOE_EXPERTS = 128
MOE_TOP_K = 8
MOE_TOKENS = 8
MOE_HIDDEN = 2816
MOE_FFN = 704


def moe_layer() -> list[TensorSpec]:
    """Stacked experts as [128*N, K]: gate and up [704, 2816], down
    [2816, 704], N(0, 0.02)."""
    E = MOE_EXPERTS
    return [TensorSpec("gate", E * MOE_FFN, MOE_HIDDEN, 0.02, 3000),
            TensorSpec("up", E * MOE_FFN, MOE_HIDDEN, 0.02, 3001),
            TensorSpec("down", E * MOE_HIDDEN, MOE_FFN, 0.02, 3002)]


GEMM_ROWS = (16, 32, 128, 2048)
