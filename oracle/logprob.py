"""Compact-to-semantic log-probabilities and the gradient of reused logit rows.

Sources:

* HARTS, Sec. 3.5 Eq. 17 -- for every nonterminal semantic position s of the
  original batch, with m(s) its compact logit row and y_s the next token of the
  same trajectory, the log-probability is the target logit minus the log of the
  row's sum of exponentials.  The method computes each compact row's maximum
  and sum-exp once and reads one target logit per position; the plain
  definition written here expands every position to its own full row, which the
  method reaches exactly up to rounding order.
* HARTS, Sec. 3.5 Eq. 19-20 -- a compact row's gradient is the sum, over the
  positions that map to it, of each position's upstream gradient times the
  gradient of its own log-probability.
* Octopus, Sec. 3.4 -- mounted spans carry a zero loss mask: they are context
  of the reader's trajectory, not its own positions.

Reading (where the pages leave a step open):

* The original batch is every root-to-leaf trajectory, leaves in depth-first
  order, each one the flat sequence with mounted spans spliced in
  (``Dag.trajectory``).  Its semantic positions with a log-probability are the
  trajectory's own tokens that have a next token; the target is the flat
  sequence's next token, which may be the first token of a spliced span.
  Spliced positions hold no log-probability: their compact row was computed in
  the producer's context, not the reader's, and their loss mask is zero.
* Vocabulary ids of the tokens (``labels``) are inputs, one per token.

Everything is float64 NumPy; the expanded S x V arrays make this usable on
small inputs only.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .dag import Dag


def semantic_positions(dag: Dag, labels: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(token id m(s), target y_s) for every nonterminal semantic position, in batch order."""
    rows, targets = [], []
    for leaf in dag.leaves_dfs():
        ids, own = dag.trajectory(leaf)
        for j in range(len(ids) - 1):
            if own[j]:
                rows.append(int(ids[j]))
                targets.append(int(labels[ids[j + 1]]))
    return np.asarray(rows, np.int64), np.asarray(targets, np.int64)


def _log_softmax_rows(z: np.ndarray) -> np.ndarray:
    m = z.max(axis=1, keepdims=True)
    return z - (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))


def logprob(z: np.ndarray, pos_row: np.ndarray, pos_target: np.ndarray) -> np.ndarray:
    """lambda_s = log softmax(z[m(s)])[y_s] for every position (HARTS Eq. 17), on expanded rows."""
    z = np.asarray(z, np.float64)
    ze = z[pos_row]                                   # S x V: one full row per position
    return _log_softmax_rows(ze)[np.arange(len(pos_row)), pos_target]


def logprob_grad(z: np.ndarray, pos_row: np.ndarray, pos_target: np.ndarray, g: np.ndarray) -> np.ndarray:
    """dL/dz for upstream gradients g_s = dL/dlambda_s (HARTS Eq. 19-20).

    Each position's gradient with respect to its own expanded row is
    g_s (onehot(y_s) - softmax(row)); the compact row receives the sum over the
    positions that map to it.
    """
    z = np.asarray(z, np.float64)
    g = np.asarray(g, np.float64)
    ze = z[pos_row]
    p = np.exp(_log_softmax_rows(ze))
    ge = -g[:, None] * p
    ge[np.arange(len(pos_row)), pos_target] += g
    dz = np.zeros_like(z)
    np.add.at(dz, pos_row, ge)
    return dz


def row_lse(z: np.ndarray) -> np.ndarray:
    """log sum_v exp z[c, v] per row: the per-row statistic the method keeps."""
    z = np.asarray(z, np.float64)
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))
