"""Gated delta rule over a rollout tree: the plain token recurrence.

Sources:

* HARTS, Sec. 2.2 (a linear-attention layer carries a recurrent state along
  the token order; a side branch must start from the state at its fork) and
  Sec. 3.4 Eq. 16 (the chunkwise operator maps inputs and an initial state to
  outputs and boundary states) -- the chunked, replayed execution the GPU runs
  reaches exactly (up to rounding order) what this module computes, because a
  child's true initial state is its parent's state at the fork.
* Octopus, Sec. 3 (recurrent layers do not read mounted spans: a read_thread
  edge only changes what full-attention layers see), so the recurrent index of
  a token is its offset along its own root-to-node path, mounts skipped.
* The recurrence itself (the gated delta rule) is not printed on the pages;
  this is the textbook form, cited by both pages:

      S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
      o_t = scale * S_t q_t,                       S_0 = 0 per head,

  with S_t of shape [dv, dk].  **Parity unpinned** for this parameterisation
  and for the output scale (a parameter, default 1): the pages fix neither.

Everything here is float64 NumPy.  The flat form runs the recurrence on each
root-to-leaf trajectory separately; a compact row's output is the same on
every trajectory that holds it, and its upstream gradient dO is placed on its
owning trajectory only (Octopus Sec. 3.4 Eq. 6), so per-trajectory gradients
scatter-added into compact rows give the packed gradient exactly.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from .dag import Dag

CHECKPOINT = 64


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def recurrent_index(spec) -> np.ndarray:
    """Per token: its offset along its own root-to-node path (mounted spans skipped)."""
    dag = Dag(spec)
    idx = np.zeros(dag.n_tokens, np.int64)
    depth = [0] * dag.n
    for u in range(dag.n):                      # parents precede children in the table
        p = dag.parent[u]
        depth[u] = 0 if p < 0 else depth[p] + dag.length[p]
        o = dag.offset[u]
        idx[o:o + dag.length[u]] = depth[u] + np.arange(dag.length[u])
    return idx


def path_ids(dag: Dag, u: int) -> np.ndarray:
    """Token ids of the root-to-u path, own tokens only, in order."""
    parts = [np.arange(dag.offset[a], dag.offset[a] + dag.length[a]) for a in dag.chain(u)]
    return np.concatenate(parts).astype(np.int64) if parts else np.zeros(0, np.int64)


def _step(S, k, v, b, a):
    """One recurrence step for all heads: S [H,dv,dk] -> new S."""
    Sk = np.einsum("hvk,hk->hv", S, k)
    return a[:, None, None] * S + np.einsum("hv,hk->hvk", b[:, None] * v - (a * b)[:, None] * Sk, k)


def recur(ids: np.ndarray, q, k, v, beta, alpha, do=None, scale: float = 1.0,
          heads: Optional[Sequence[int]] = None, S0=None):
    """Run the recurrence along token ids (one sequence).

    q,k [U,H,dk], v [U,H,dv], beta/alpha [U,H] (token-major, float64 or
    convertible); ``do`` [len(ids),H,dv] is the upstream gradient along this
    sequence (None: forward only).  Returns (o [L,H,dv], grads or None) where
    grads holds dq, dk, dv, dbeta, dalpha along the sequence and dS0.
    """
    ids = np.asarray(ids, np.int64)
    hs = slice(None) if heads is None else np.asarray(heads, np.int64)
    Q = _f64(q)[ids][:, hs]
    K = _f64(k)[ids][:, hs]
    V = _f64(v)[ids][:, hs]
    B = _f64(beta)[ids][:, hs]
    A = _f64(alpha)[ids][:, hs]
    L, H, dk = K.shape
    dv = V.shape[-1]
    S = np.zeros((H, dv, dk)) if S0 is None else np.array(S0, np.float64, copy=True)
    o = np.zeros((L, H, dv))
    ckpt = []
    for t in range(L):
        if t % CHECKPOINT == 0:
            ckpt.append(S.copy())
        S = _step(S, K[t], V[t], B[t], A[t])
        o[t] = scale * np.einsum("hvk,hk->hv", S, Q[t])
    if do is None:
        return o, None
    dO = np.asarray(do, np.float64)
    g = {"dq": np.zeros_like(Q), "dk": np.zeros_like(K), "dv": np.zeros_like(V),
         "dbeta": np.zeros_like(B), "dalpha": np.zeros_like(A)}
    G = np.zeros((H, dv, dk))
    for c in range((L + CHECKPOINT - 1) // CHECKPOINT - 1, -1, -1):
        t0, t1 = c * CHECKPOINT, min(L, (c + 1) * CHECKPOINT)
        states = [ckpt[c]]                        # states[j] = S before token t0 + j
        for t in range(t0, t1):
            states.append(_step(states[-1], K[t], V[t], B[t], A[t]))
        for t in range(t1 - 1, t0 - 1, -1):
            S_t, S_p = states[t - t0 + 1], states[t - t0]
            kt, vt, bt, at = K[t], V[t], B[t], A[t]
            G += scale * np.einsum("hv,hk->hvk", dO[t], Q[t])
            g["dq"][t] = scale * np.einsum("hvk,hv->hk", S_t, dO[t])
            Gk = np.einsum("hvk,hk->hv", G, kt)
            Sk = np.einsum("hvk,hk->hv", S_p, kt)
            GkSk = np.einsum("hv,hv->h", Gk, Sk)
            g["dv"][t] = bt[:, None] * Gk
            g["dbeta"][t] = np.einsum("hv,hv->h", vt, Gk) - at * GkSk
            g["dalpha"][t] = np.einsum("hvk,hvk->h", G, S_p) - bt * GkSk
            g["dk"][t] = (bt[:, None] * np.einsum("hvk,hv->hk", G, vt)
                          - (at * bt)[:, None] * (np.einsum("hvk,hv->hk", S_p, Gk)
                                                  + np.einsum("hvk,hv->hk", G, Sk)))
            G = at[:, None, None] * (G - bt[:, None, None] * np.einsum("hv,hk->hvk", Gk, kt))
    g["dS0"] = G
    return o, g


def gdn_flat(spec, q, k, v, beta, alpha, do=None, scale: float = 1.0) -> Dict[str, np.ndarray]:
    """Packed-tree outputs (and gradients) from per-trajectory recurrences.

    Token-major inputs over the DAG's tokens.  Returns {"o"} and, with ``do``,
    {"dq","dk","dv","dbeta","dalpha"}, all float64 and token-major.
    """
    dag = Dag(spec)
    q, k, v, beta, alpha = (_f64(x) for x in (q, k, v, beta, alpha))
    U, H, dk = k.shape
    dv = v.shape[-1]
    o = np.full((U, H, dv), np.nan)
    out = {"o": o}
    if do is not None:
        dO = _f64(do)
        for name, shape in (("dq", q.shape), ("dk", k.shape), ("dv", v.shape),
                            ("dbeta", beta.shape), ("dalpha", alpha.shape)):
            out[name] = np.zeros(shape)
        owner = dag.owner()
    for leaf in dag.leaves_dfs():
        ids = path_ids(dag, leaf)
        if len(ids) == 0:
            continue
        dseq = None
        if do is not None:
            node = np.concatenate([np.full(dag.length[a], a) for a in dag.chain(leaf)])
            mine = np.array([owner[a] == leaf for a in node], bool)
            dseq = np.where(mine[:, None, None], dO[ids], 0.0)
        o_seq, g = recur(ids, q, k, v, beta, alpha, dseq, scale)
        seen = ~np.isnan(o[ids, 0, 0])
        if seen.any():                       # a shared row must come out the same on every trajectory
            assert np.array_equal(o[ids[seen]], o_seq[seen])
        o[ids] = o_seq
        if g is not None:
            for name in ("dq", "dk", "dv", "dbeta", "dalpha"):
                np.add.at(out[name], ids, g[name])
    return out


def gdn_unrolled(ids, q, k, v, beta, alpha, scale: float = 1.0) -> np.ndarray:
    """Outputs along one sequence from the closed form of the recurrence.

    Unrolling S_0 = 0 gives S_t = sum_{i<=t} beta_i v_i k_i^T prod_{j=i+1..t}
    alpha_j (I - beta_j k_j k_j^T): products of explicit [dk,dk] transition
    matrices, O(L^2 dk^3).  Tiny inputs only; used to pin :func:`recur`.
    """
    ids = np.asarray(ids, np.int64)
    Q, K, V, B, A = (_f64(x)[ids] for x in (q, k, v, beta, alpha))
    L, H, dk = K.shape
    dv = V.shape[-1]
    o = np.zeros((L, H, dv))
    for h in range(H):
        trans = [A[j, h] * (np.eye(dk) - B[j, h] * np.outer(K[j, h], K[j, h])) for j in range(L)]
        for t in range(L):
            S = np.zeros((dv, dk))
            for i in range(t + 1):
                M = np.eye(dk)
                for j in range(i + 1, t + 1):
                    M = M @ trans[j]
                S += B[i, h] * np.outer(V[i, h], K[i, h]) @ M
            o[t, h] = scale * S @ Q[t, h]
    return o
