"""Seeded random tensors for the attention workloads.

Values are standard normal, drawn in float32 by torch's generator on the
requested device and, for bf16 runs, rounded to bf16 with round-to-nearest-even
(torch's float32 -> bfloat16 conversion).  Both sides of a comparison receive
the very same tensors; this module never computes anything the method defines.
"""
from __future__ import annotations

import numpy as np
import torch


def _seed(base: int, stream: int) -> int:
    ss = np.random.SeedSequence([int(base), int(stream)])
    return int(ss.generate_state(1, dtype=np.uint32)[0])


def normal(shape, seed: int, stream: int, device="cpu", dtype=torch.float32) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, stream))
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    return x.to(dtype)


def bf16_round(x: torch.Tensor) -> torch.Tensor:
    """Round to bf16 (nearest-even) and return it in the input dtype."""
    return x.to(torch.bfloat16).to(x.dtype)


STREAM_Q, STREAM_K, STREAM_V, STREAM_DO = 1, 2, 3, 4


def attn_inputs(n_tokens: int, hq: int, hkv: int, d: int, seed: int, device="cpu",
                dtype=torch.float32, with_grad: bool = True):
    """q [U,Hq,d], k,v [U,Hkv,d] and the upstream gradient dO [U,Hq,d], token-major."""
    q = normal((n_tokens, hq, d), seed, STREAM_Q, device, dtype)
    k = normal((n_tokens, hkv, d), seed, STREAM_K, device, dtype)
    v = normal((n_tokens, hkv, d), seed, STREAM_V, device, dtype)
    do = normal((n_tokens, hq, d), seed, STREAM_DO, device, dtype) if with_grad else None
    return q, k, v, do
