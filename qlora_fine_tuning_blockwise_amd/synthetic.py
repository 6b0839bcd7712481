"""Seeded synthetic inputs for tests, the smoke check and the benchmark.

This module holds random-number recipes and workload shapes only; none of the
quantization or layer arithmetic lives here. Both the CPU oracle's callers and
the GPU path's callers draw their inputs from it, and nothing else is shared
between the two sides.

bf16 tensors on the host travel as ``uint16`` bit patterns. Seeds follow
``1000 * workload + tensor index``.
"""
from __future__ import annotations

import numpy as np
import torch

# --------------------------------------------------------------- workloads
# Shapes of the weights [N, K] (N out-features, K in-features), token counts M,
# LoRA rank r and alpha of the five synthetic workloads.
LINEAR_1024 = dict(name="linear_1024x1024", weights={"w": (1024, 1024)}, M=16, r=16, alpha=32.0,
                   w_std=0.02, w_dtype="f32")
LLAMA7B_DECODE = dict(name="llama7b_decode", weights={"q": (4096, 4096), "up": (11008, 4096)},
                      M=(1, 4, 16), r=16, alpha=32.0, w_std=0.02, w_dtype="bf16")
LLAMA7B_TRAIN = dict(name="llama7b_train", weights={"q": (4096, 4096), "up": (11008, 4096)},
                     M=4096, r=16, alpha=32.0, w_std=0.02, w_dtype="bf16")
LAYER_70B = dict(name="llama70b_layer",
                 weights={"q": (8192, 8192), "k": (1024, 8192), "v": (1024, 8192),
                          "o": (8192, 8192), "gate": (28672, 8192), "up": (28672, 8192),
                          "down": (8192, 28672)},
                 M=2048, r=64, alpha=16.0, w_std=0.015, w_dtype="bf16")
BULK_65B = dict(name="bulk_quantize_65b", tensor=(8192, 28672), n_tensors=277,
                w_dtype="bf16")

# Adapters of every linear layer of a Llama-7B decoder (32 layers; q, k, v, o
# 4096x4096; gate, up 11008x4096; down 4096x11008) at rank 16, laid out
# back to back in one flat arena: A [K, r] then B [r, N] per projection.
LLAMA7B_PROJECTIONS = {"q": (4096, 4096), "k": (4096, 4096), "v": (4096, 4096),
                       "o": (4096, 4096), "gate": (11008, 4096), "up": (11008, 4096),
                       "down": (4096, 11008)}


def adapter_arena_params(projections=LLAMA7B_PROJECTIONS, layers: int = 32, r: int = 16) -> int:
    """Trainable parameters of the adapters: r (K + N) per projection."""
    return layers * sum(r * (K + N) for N, K in projections.values())


def adam_state(n: int, seed: int):
    """A mid-training optimizer state: fp32 master values N(0, 0.02), first
    moments N(0, 1e-3), second moments (N(0, 1e-3))^2."""
    g = np.random.default_rng(seed)
    p = (g.standard_normal(n, dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    m = (g.standard_normal(n, dtype=np.float32) * np.float32(1e-3)).astype(np.float32)
    v = np.square(g.standard_normal(n, dtype=np.float32) * np.float32(1e-3)).astype(np.float32)
    return p, m, v


def adapter_grad_f32(n: int, seed: int) -> np.ndarray:
    """Heavy-tailed adapter gradients: N(0, 1e-2) times a log-normal(0, 1) scale."""
    g = np.random.default_rng(seed)
    z = g.standard_normal(n, dtype=np.float32) * np.float32(1e-2)
    return (z * g.lognormal(0.0, 1.0, n).astype(np.float32)).astype(np.float32)


def seed_of(workload: int, index: int) -> int:
    return 1000 * workload + index


# --------------------------------------------------------------- host (numpy)
def to_bf16_bits(f32: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (torch's round-to-nearest-even) as uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def normal_f32(shape, std: float, seed: int) -> np.ndarray:
    g = np.random.default_rng(seed)
    return (g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def normal_bf16(shape, std: float, seed: int) -> np.ndarray:
    return to_bf16_bits(normal_f32(shape, std, seed))


def bits_to_torch_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def torch_bf16_to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


# --------------------------------------------------------------- device (torch)
def torch_normal_bf16(shape, std: float, seed: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return (t * std).to(torch.bfloat16)


def torch_student_t_outliers_bf16(shape, seed: int, device, nu: int = 4, scale: float = 0.02,
                                  p_outlier: float = 1e-3, outlier_mult: float = 20.0):
    """Heavy-tailed weights: 0.02 x Student-t(4), each value independently an
    outlier (x20) with probability 0.1%. The t variate is z * sqrt(4/chi2_4)
    with chi2_4 = -2 ln(U1 U2)."""
    assert nu == 4
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    u1 = torch.rand(shape, generator=g, device=device, dtype=torch.float32).clamp_min_(1e-30)
    u2 = torch.rand(shape, generator=g, device=device, dtype=torch.float32).clamp_min_(1e-30)
    chi2 = -2.0 * torch.log(u1 * u2)
    t = z * torch.sqrt(4.0 / chi2)
    out = torch.rand(shape, generator=g, device=device, dtype=torch.float32) < p_outlier
    t = torch.where(out, t * outlier_mult, t)
    return (t * scale).to(torch.bfloat16)
