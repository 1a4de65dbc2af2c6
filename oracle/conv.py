"""Short causal convolution of a linear-attention block over a rollout tree.

Sources:

* HARTS, Sec. 4.2 (KDA state reuse and causal convolution): a width-w causal
  convolution may take as history only the true ancestors' most recent w - 1
  projected activations, never an adjacent packed sequence; one result is kept
  per compact token, and when several sequences read one activation, backward
  sums their gradients at its single producer.
* Octopus, Sec. 3 and App. C: recurrent (gated-delta-rule) layers skip mounted
  spans; tree-boundary hooks gather d_conv - 1 = 3 ancestor tokens for the short
  convolutions.
* The operator is not printed on the pages; this is the textbook depthwise
  causal convolution, per channel c along a token sequence x_0, x_1, ...:

      pre_t[c] = sum_{j=0}^{w-1} W[c, j] x_{t-(w-1)+j}[c]     (x_t = 0 for t < 0)
      y_t[c]   = act(pre_t[c]),   act = identity or SiLU(p) = p / (1 + e^-p)

  **Parity unpinned** for the choice of activation (a parameter) and for the
  tap order (W[c, w-1] multiplies the current token; torch's conv1d with
  padding w - 1, cropped to the sequence, uses the same order).

The sequence of a compact token is its own root-to-node path with mounted spans
skipped (``gdn.path_ids``).  The flat form runs the convolution on every
root-to-leaf trajectory; a compact output's upstream gradient lives on its
owning trajectory only (Octopus Sec. 3.4 Eq. 6), so per-trajectory gradients
scatter-added into compact rows give the packed gradient exactly.  Float64
NumPy throughout.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .dag import Dag
from .gdn import path_ids

ACT_NONE, ACT_SILU = 0, 1


def _act(p: np.ndarray, act: int) -> np.ndarray:
    return p / (1.0 + np.exp(-p)) if act == ACT_SILU else p


def _act_grad(p: np.ndarray, act: int) -> np.ndarray:
    if act != ACT_SILU:
        return np.ones_like(p)
    s = 1.0 / (1.0 + np.exp(-p))
    return s * (1.0 + p * (1.0 - s))


def conv_seq(x: np.ndarray, W: np.ndarray, act: int = ACT_NONE):
    """(y, pre) of one sequence x [L, Ch] with taps W [Ch, w]."""
    x = np.asarray(x, np.float64)
    L, _ = x.shape
    w = W.shape[1]
    pre = np.zeros_like(x)
    for t in range(L):
        for j in range(w):
            s = t - (w - 1) + j
            if s >= 0:
                pre[t] += W[:, j] * x[s]
    return _act(pre, act), pre


def conv_seq_grad(x: np.ndarray, W: np.ndarray, dy: np.ndarray, act: int = ACT_NONE):
    """(dx [L, Ch], dW [Ch, w]) of one sequence for the upstream gradient dy [L, Ch]."""
    x = np.asarray(x, np.float64)
    _, pre = conv_seq(x, W, act)
    dpre = np.asarray(dy, np.float64) * _act_grad(pre, act)
    L = x.shape[0]
    w = W.shape[1]
    dx = np.zeros_like(x)
    dW = np.zeros(W.shape)
    for t in range(L):
        for j in range(w):
            s = t - (w - 1) + j
            if s >= 0:
                dx[s] += W[:, j] * dpre[t]
                dW[:, j] += dpre[t] * x[s]
    return dx, dW


def conv_flat(spec, x, W, act: int = ACT_NONE, dy=None) -> Dict[str, np.ndarray]:
    """Compact outputs (and gradients) from per-trajectory convolutions.

    x [U, Ch] token-major over the DAG's tokens, W [Ch, w].  Returns {"y"} and,
    with ``dy`` [U, Ch], {"dx", "dW"}; float64.
    """
    dag = Dag(spec)
    x = np.asarray(x, np.float64)
    W = np.asarray(W, np.float64)
    U, Ch = x.shape
    y = np.full((U, Ch), np.nan)
    out: Dict[str, np.ndarray] = {"y": y}
    if dy is not None:
        dy = np.asarray(dy, np.float64)
        out["dx"] = np.zeros((U, Ch))
        out["dW"] = np.zeros(W.shape)
        owner = dag.owner()
    for leaf in dag.leaves_dfs():
        ids = path_ids(dag, leaf)
        if len(ids) == 0:
            continue
        ys, _ = conv_seq(x[ids], W, act)
        seen = ~np.isnan(y[ids, 0])
        if seen.any():                        # a shared token comes out the same on every trajectory
            assert np.array_equal(y[ids[seen]], ys[seen])
        y[ids] = ys
        if dy is not None:
            node = np.concatenate([np.full(dag.length[a], a) for a in dag.chain(leaf)])
            mine = np.array([owner[a] == leaf for a in node], bool)
            dx, dW = conv_seq_grad(x[ids], W, np.where(mine[:, None], dy[ids], 0.0), act)
            np.add.at(out["dx"], ids, dx)
            out["dW"] += dW
    return out


def conv_paths(spec, x, W, act: int, dy_per_path: Optional[list] = None):
    """Per-trajectory form with an independent upstream gradient for every
    trajectory position (a list of [L_leaf, Ch] arrays, leaves in depth-first
    order): returns the compact (dx, dW) summed over all positions."""
    dag = Dag(spec)
    x = np.asarray(x, np.float64)
    dx = np.zeros_like(x)
    dW = np.zeros(np.shape(W))
    for leaf, g in zip(dag.leaves_dfs(), dy_per_path):
        ids = path_ids(dag, leaf)
        if len(ids) == 0:
            continue
        a, b = conv_seq_grad(x[ids], np.asarray(W, np.float64), g, act)
        np.add.at(dx, ids, a)
        dW += b
    return dx, dW


def path_pred(spec) -> np.ndarray:
    """pred[t]: the token before t on t's own root-to-node path (mounts skipped), -1 at a root's start."""
    dag = Dag(spec)
    pred = np.full(dag.n_tokens, -1, np.int64)
    for u in range(dag.n):
        o, ln = dag.offset[u], dag.length[u]
        if ln == 0:
            continue
        pred[o + 1:o + ln] = np.arange(o, o + ln - 1)
        a = dag.parent[u]
        while a >= 0 and dag.length[a] == 0:
            a = dag.parent[a]
        pred[o] = dag.offset[a] + dag.length[a] - 1 if a >= 0 else -1
    return pred


def conv_compact(spec, x, W, act: int = ACT_NONE, dy=None) -> Dict[str, np.ndarray]:
    """The same results as ``conv_flat`` evaluated once per compact token.

    A token's window is the last w tokens of its own path, the same on every
    trajectory that holds it, so y is a sum over its path predecessors; the input
    gradient scatters each output's dpre back onto the tokens of its window.
    Vectorised one channel at a time (usable on the full workloads for a few
    channels); a missing predecessor reads a zero appended after the last token.
    """
    x = np.asarray(x, np.float64)
    W = np.asarray(W, np.float64)
    U, Ch = x.shape
    w = W.shape[1]
    p1 = np.append(path_pred(spec), -1)
    p1[p1 < 0] = U                               # index U holds the zero
    preds = [np.arange(U)]
    for _ in range(1, w):
        preds.append(p1[preds[-1]])
    y = np.zeros_like(x)
    out = {"y": y}
    if dy is not None:
        dy = np.asarray(dy, np.float64)
        out["dx"] = np.zeros_like(x)
        out["dW"] = np.zeros(W.shape)
    for c in range(Ch):
        xc = np.append(x[:, c], 0.0)
        pre = np.zeros(U)
        for k, q in enumerate(preds):
            pre += W[c, w - 1 - k] * xc[q]
        y[:, c] = _act(pre, act)
        if dy is None:
            continue
        dpre = dy[:, c] * _act_grad(pre, act)
        dxc = np.zeros(U + 1)
        for k, q in enumerate(preds):
            dxc += np.bincount(q, weights=W[c, w - 1 - k] * dpre, minlength=U + 1)
            out["dW"][c, w - 1 - k] = dpre @ xc[q]
        out["dx"][:, c] = dxc[:U]
    return out
