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


STREAM_GQ, STREAM_GK, STREAM_GV, STREAM_GBETA, STREAM_GALPHA, STREAM_GDO = 11, 12, 13, 14, 15, 16


def gdn_inputs(n_tokens: int, h: int, dk: int, dv: int, seed: int, device="cpu",
               dtype=torch.float32, decay_scale: float = 1.0, with_grad: bool = True):
    """Inputs of one gated-delta-rule layer, token-major.

    q, k [U,H,dk]: standard normal, each head's vector divided by its L2 norm
    (the layer receives normalised queries and keys); v [U,H,dv] standard
    normal; beta [U,H] = sigmoid(N(0,1)); alpha [U,H] = exp(-decay_scale *
    softplus(N(0,1))) (decay_scale < 1 gives slower decay, so that state carries
    across many chunks); dO [U,H,dv] standard normal.  q, k, v, dO are rounded
    to ``dtype`` after normalisation; beta and alpha stay float32.
    """
    def unit(x):
        return x / x.norm(dim=-1, keepdim=True)
    q = unit(normal((n_tokens, h, dk), seed, STREAM_GQ, device)).to(dtype)
    k = unit(normal((n_tokens, h, dk), seed, STREAM_GK, device)).to(dtype)
    v = normal((n_tokens, h, dv), seed, STREAM_GV, device, dtype)
    beta = torch.sigmoid(normal((n_tokens, h), seed, STREAM_GBETA, device))
    alpha = torch.exp(-decay_scale * torch.nn.functional.softplus(normal((n_tokens, h), seed, STREAM_GALPHA,
                                                                          device)))
    do = normal((n_tokens, h, dv), seed, STREAM_GDO, device, dtype) if with_grad else None
    return q, k, v, beta, alpha, do


STREAM_LOGITS, STREAM_LABELS, STREAM_LPGRAD = 21, 22, 23


def logprob_inputs(n_rows: int, vocab: int, n_tokens: int, n_pos: int, seed: int, device="cpu",
                   dtype=torch.float32, spread: float = 2.0, with_grad: bool = True):
    """Inputs of the log-probability step.

    z [n_rows, vocab]: logits, normal with standard deviation ``spread``,
    rounded to ``dtype``; labels [n_tokens]: vocabulary ids uniform over
    [0, vocab), int64; g [n_pos]: upstream gradients of the log-probabilities,
    standard normal float32.
    """
    z = (normal((n_rows, vocab), seed, STREAM_LOGITS, device) * spread).to(dtype)
    gen = torch.Generator(device="cpu")
    gen.manual_seed(_seed(seed, STREAM_LABELS))
    labels = torch.randint(0, vocab, (n_tokens,), generator=gen, dtype=torch.int64)
    g = normal((n_pos,), seed, STREAM_LPGRAD, device) if with_grad else None
    return z, labels, g
