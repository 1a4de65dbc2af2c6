"""Attention over a rollout DAG, four independent ways.

What is computed (Octopus Sec. 3.3 Eq. 4 and HARTS Sec. 4.2 Eq. 21-22): every
compact query token t = (u, i) attends, with softmax weights, to the keys of
its visible set V(u, i) -- the node's ancestors, its active mounted spans and
its own tokens up to i -- after rotating q and k at their Eq. 2 positions:

    s_tj = scale * <R(pos_t) q_t,h , R(pos_j) k_j,g>,   g = h // (Hq / Hkv)
    O_t,h = sum_{j in V(t)} softmax_j(s_tj) v_j,g,      lse_t,h = log sum_j exp s_tj

The backward pass is the standard softmax-attention backward chained through
R^T; a key shared by several readers (ancestors, mounted spans) receives the
sum of every reader's contribution (Octopus Sec. 3.4 Eq. 8, HARTS Sec. 3.4).

* :func:`attn_flat` -- the reference: expand every root-to-leaf trajectory with
  its mounted spans spliced in, run dense causal attention on it (positions
  from Eq. 2, not from the sequence index), keep each node's outputs from its
  owning trajectory, and scatter-add the expanded gradients to compact tokens.
  The upstream gradient of a compact token lives on its owner trajectory only
  (Octopus Eq. 6), unless per-trajectory gradients are passed explicitly.
* :func:`attn_brute` -- explicit loops over (query, head, visible key).
* :func:`attn_packed_mask` -- one dense token-by-token mask over the packed tokens.
* :func:`attn_rows` / :func:`attn_key_grads` -- selected outputs and selected
  key gradients, for sampling inputs too large for the other three.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np

from .dag import Dag
from .rope import rotate, rotate_transpose


@dataclass
class AttnParams:
    hq: int
    hkv: int
    scale: Optional[float] = None      # None -> 1/sqrt(d)
    rope_base: float = 10000.0         # 0 -> no rotation

    def scale_for(self, d: int) -> float:
        return (1.0 / np.sqrt(d)) if self.scale is None else float(self.scale)

    def group(self, h: int) -> int:
        return h // (self.hq // self.hkv)


def _np(x):
    """torch tensors become numpy arrays; numpy arrays and other indexable views pass through."""
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        if str(x.dtype) == "torch.bfloat16":
            x = x.float()
        return x.numpy()
    if isinstance(x, (list, tuple)):
        return np.asarray(x)
    return x


def _softmax_rows(s: np.ndarray):
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=-1, keepdims=True)
    return e / z, (m + np.log(z))[..., 0]


# ---------------------------------------------------------------------------
# flat per-trajectory reference
# ---------------------------------------------------------------------------

def attn_flat(spec, q, k, v, do, p: AttnParams, transitive: bool = True,
              dtype=np.float64, traj_do: Optional[Dict[int, np.ndarray]] = None,
              block: int = 1024, with_grad: bool = True, view: str = "mounted"):
    """Returns (o, lse, dq, dk, dv) over compact tokens (token-major, float64 arrays).

    ``traj_do`` maps a leaf to the upstream gradient of its trajectory's rows
    ([len(trajectory), Hq, d]); without it each compact token's ``do`` is placed
    on its owner trajectory and zero elsewhere.  ``view`` selects the table
    pair's view (``oracle.dag.VIEWS``).
    """
    g = Dag(spec, transitive, view)
    q, k, v = _np(q), _np(k), _np(v)
    do = None if do is None else _np(do)
    U, hq, d = q.shape
    scale = p.scale_for(d)
    pos = g.token_positions()
    qr = rotate(q, pos, p.rope_base).astype(dtype)
    kr = rotate(k, pos, p.rope_base).astype(dtype)
    vv = np.asarray(v, np.float64).astype(dtype)
    node_of, _ = g.token_node()
    owner = g.owner()
    o = np.zeros((U, hq, d))
    lse = np.zeros((U, hq))
    dq_r = np.zeros((U, hq, d))
    dk_r = np.zeros((U, p.hkv, d))
    dv = np.zeros((U, p.hkv, d))
    for leaf in g.leaves_dfs():
        seq, own = g.trajectory(leaf)
        L = len(seq)
        if L == 0:
            continue
        mine = own & (np.asarray([owner[node_of[t]] for t in seq]) == leaf)
        Q, K, V = qr[seq], kr[seq], vv[seq]
        if traj_do is not None:
            dO = np.asarray(traj_do.get(leaf, np.zeros((L, hq, d))), np.float64).astype(dtype)
        elif do is not None:
            dO = np.zeros((L, hq, d), dtype)
            dO[mine] = do[seq[mine]]
        else:
            dO = None
        dQ = np.zeros((L, hq, d), dtype)
        dK = np.zeros((L, p.hkv, d), dtype)
        dV = np.zeros((L, p.hkv, d), dtype)
        for h in range(hq):
            gg = p.group(h)
            for r0 in range(0, L, block):
                r1 = min(L, r0 + block)
                s = scale * (Q[r0:r1, h] @ K[:r1, gg].T)
                causal = np.arange(r1)[None, :] > np.arange(r0, r1)[:, None]
                s = np.where(causal, -np.inf, s)
                P, l = _softmax_rows(s)
                O = P @ V[:r1, gg]
                rows = np.nonzero(mine[r0:r1])[0]
                o[seq[r0 + rows], h] = O[rows]
                lse[seq[r0 + rows], h] = l[rows]
                if with_grad and dO is not None:
                    g_o = dO[r0:r1, h]
                    dP = g_o @ V[:r1, gg].T
                    D = (g_o * O).sum(axis=1, keepdims=True)
                    dS = P * (dP - D)
                    dQ[r0:r1, h] += scale * (dS @ K[:r1, gg])
                    dK[:r1, gg] += scale * (dS.T @ Q[r0:r1, h])
                    dV[:r1, gg] += P.T @ g_o
        if with_grad and dO is not None:
            np.add.at(dq_r, seq, dQ.astype(np.float64))
            np.add.at(dk_r, seq, dK.astype(np.float64))
            np.add.at(dv, seq, dV.astype(np.float64))
    if not with_grad or (do is None and traj_do is None):
        return o, lse, None, None, None
    dq = rotate_transpose(dq_r, pos, p.rope_base)
    dk = rotate_transpose(dk_r, pos, p.rope_base)
    return o, lse, dq, dk, dv


# ---------------------------------------------------------------------------
# brute force: explicit loops, float64, tiny inputs only
# ---------------------------------------------------------------------------

def attn_brute(spec, q, k, v, do, p: AttnParams, transitive: bool = True, view: str = "mounted"):
    g = Dag(spec, transitive, view)
    q, k, v, do = (np.asarray(_np(x), np.float64) for x in (q, k, v, do))
    U, hq, d = q.shape
    scale = p.scale_for(d)
    pos = g.token_positions()
    qr, kr = rotate(q, pos, p.rope_base), rotate(k, pos, p.rope_base)
    node_of, off = g.token_node()
    o = np.zeros_like(q)
    lse = np.zeros((U, hq))
    dqr = np.zeros_like(q)
    dkr = np.zeros_like(k)
    dv = np.zeros_like(v)
    for t in range(U):
        keys = g.visible_tokens(int(node_of[t]), int(off[t]))
        for h in range(hq):
            gg = p.group(h)
            s = np.array([scale * float(np.dot(qr[t, h], kr[j, gg])) for j in keys])
            m = max(s)
            w = [np.exp(x - m) for x in s]
            z = sum(w)
            pr = [x / z for x in w]
            lse[t, h] = m + np.log(z)
            for a, j in enumerate(keys):
                o[t, h] += pr[a] * v[j, gg]
            dp = [float(np.dot(do[t, h], v[j, gg])) for j in keys]
            D = float(np.dot(do[t, h], o[t, h]))
            for a, j in enumerate(keys):
                ds = pr[a] * (dp[a] - D)
                dqr[t, h] += scale * ds * kr[j, gg]
                dkr[j, gg] += scale * ds * qr[t, h]
                dv[j, gg] += pr[a] * do[t, h]
    return (o, lse, rotate_transpose(dqr, pos, p.rope_base),
            rotate_transpose(dkr, pos, p.rope_base), dv)


# ---------------------------------------------------------------------------
# dense packed mask over compact tokens, float64
# ---------------------------------------------------------------------------

def visibility_mask(spec, transitive: bool = True) -> np.ndarray:
    g = Dag(spec, transitive)
    node_of, off = g.token_node()
    M = np.zeros((g.n_tokens, g.n_tokens), bool)
    for t in range(g.n_tokens):
        M[t, g.visible_tokens(int(node_of[t]), int(off[t]))] = True
    return M


def attn_packed_mask(spec, q, k, v, do, p: AttnParams, transitive: bool = True):
    g = Dag(spec, transitive)
    q, k, v, do = (np.asarray(_np(x), np.float64) for x in (q, k, v, do))
    U, hq, d = q.shape
    scale = p.scale_for(d)
    pos = g.token_positions()
    qr, kr = rotate(q, pos, p.rope_base), rotate(k, pos, p.rope_base)
    M = visibility_mask(spec, transitive)
    o = np.zeros_like(q)
    lse = np.zeros((U, hq))
    dqr = np.zeros_like(q)
    dkr = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(hq):
        gg = p.group(h)
        s = np.where(M, scale * (qr[:, h] @ kr[:, gg].T), -np.inf)
        P, l = _softmax_rows(s)
        o[:, h] = P @ v[:, gg]
        lse[:, h] = l
        dP = do[:, h] @ v[:, gg].T
        D = (do[:, h] * o[:, h]).sum(axis=1, keepdims=True)
        dS = P * (dP - D)
        dqr[:, h] = scale * (dS @ kr[:, gg])
        dkr[:, gg] += scale * (dS.T @ qr[:, h])
        dv[:, gg] += P.T @ do[:, h]
    return (o, lse, rotate_transpose(dqr, pos, p.rope_base),
            rotate_transpose(dkr, pos, p.rope_base), dv)


# ---------------------------------------------------------------------------
# sampled evaluation for large inputs
# ---------------------------------------------------------------------------

class RowSampler:
    """Per-token evaluation of outputs and key gradients straight from V(t)."""

    def __init__(self, spec, p: AttnParams, transitive: bool = True, view: str = "mounted"):
        self.g = Dag(spec, transitive, view)
        self.p = p
        self.pos = self.g.token_positions()
        self.node_of, self.off = self.g.token_node()

    def _fwd_one(self, t, q, k, v):
        g, p = self.g, self.p
        keys = g.visible_tokens(int(self.node_of[t]), int(self.off[t]))
        d = k.shape[-1]
        scale = p.scale_for(d)
        qt = rotate(np.asarray(q[t:t + 1], np.float64), self.pos[t:t + 1], p.rope_base)[0]
        kk = rotate(np.asarray(k[keys], np.float64), self.pos[keys], p.rope_base)
        vv = np.asarray(v[keys], np.float64)
        out = []
        for h in range(p.hq):
            gg = p.group(h)
            s = scale * (kk[:, gg] @ qt[h])
            P, l = _softmax_rows(s[None, :])
            out.append((keys, P[0], float(l[0]), P[0] @ vv[:, gg], kk[:, gg], qt[h]))
        return out

    def rows(self, tokens: Sequence[int], q, k, v):
        """(o [n,Hq,d], lse [n,Hq]) for the given compact tokens."""
        q, k, v = _np(q), _np(k), _np(v)
        d = k.shape[-1]
        o = np.zeros((len(tokens), self.p.hq, d))
        lse = np.zeros((len(tokens), self.p.hq))
        for a, t in enumerate(tokens):
            for h, (_, _, l, oh, _, _) in enumerate(self._fwd_one(int(t), q, k, v)):
                o[a, h] = oh
                lse[a, h] = l
        return o, lse

    def row_grads(self, tokens: Sequence[int], q, k, v, do, term_size: bool = False):
        """(o [n,Hq,d], lse [n,Hq], dq [n,Hq,d]) for the given compact tokens.

        Each row from its own visible set V(t) alone: P_tj = softmax_j(s_tj),
        D_t = dO_t . O_t, dS_tj = P_tj (dO_t . v_j - D_t) and
        dq_t = R(pos_t)^T scale sum_j dS_tj R(pos_j) k_j, the textbook softmax
        backward for one query row (the row's dO is its compact upstream gradient).
        With ``term_size`` a fourth array [n,Hq,d] bounds the terms behind each dq element:
        scale sum_j P_tj (sum_d |dO_td v_jd| + sum_d |dO_td O_td|) |R(pos_j) k_j| (with
        rotation, the two elements of each rotated pair added, which bounds any rotation of
        them).  dS_tj = P_tj (dP_tj - D_t) cancels two dot products, so summing each of them
        with a relative rounding error e per term moves dq by at most e times this.
        """
        q, k, v, do = _np(q), _np(k), _np(v), _np(do)
        d = k.shape[-1]
        scale = self.p.scale_for(d)
        o = np.zeros((len(tokens), self.p.hq, d))
        lse = np.zeros((len(tokens), self.p.hq))
        dq = np.zeros((len(tokens), self.p.hq, d))
        size = np.zeros((len(tokens), self.p.hq, d))
        for a, t in enumerate(tokens):
            t = int(t)
            for h, (kt, P, l, oh, kk, _) in enumerate(self._fwd_one(t, q, k, v)):
                gg = self.p.group(h)
                g_o = np.asarray(do[t, h], np.float64)
                dp = np.asarray(v[kt, gg], np.float64) @ g_o
                ds = P * (dp - float(g_o @ oh))
                o[a, h], lse[a, h] = oh, l
                dq[a, h] = scale * (ds @ kk)
                if term_size:
                    dp_abs = np.abs(np.asarray(v[kt, gg], np.float64)) @ np.abs(g_o)
                    size[a, h] = scale * ((P * (dp_abs + float(np.abs(g_o) @ np.abs(oh)))) @ np.abs(kk))
            dq[a] = rotate_transpose(dq[a][None], self.pos[t:t + 1], self.p.rope_base)[0]
        if not term_size:
            return o, lse, dq
        if self.p.rope_base != 0:
            half = d // 2
            size = np.concatenate([size[..., :half] + size[..., half:]] * 2, axis=-1)
        return o, lse, dq, size

    def reader_nodes(self, j: int) -> List[int]:
        """Nodes with at least one query token whose visible set contains key token j."""
        g = self.g
        u, jo = int(self.node_of[j]), int(self.off[j])
        out = [u]
        for w in range(g.n):
            if w != u and g.length[w] > 0 and any(b <= jo < e for b, e in g.visible_ranges(w).get(u, [])):
                out.append(w)
        return out

    def key_grads_by_node(self, keys: Sequence[int], q, k, v, do, groups: Sequence[int] = None,
                          block: int = 256):
        """(dk, dv) [n, Hkv, d] for the given key tokens, summed over every reader row;
        only the KV groups in ``groups`` (default all) are filled, the rest stay zero.

        Same sums as :meth:`key_grads`, organised by reader node: the query rows of one
        node w share w's non-self visible set, so they are evaluated together as one
        dense block of rows against [w's non-self keys, w's own keys] with the own part
        causal (key offset <= row offset), each row normalised over its own visible set.
        ``q`` and ``do`` need the rows of every reader node, ``k`` and ``v`` every key.
        """
        g, p = self.g, self.p
        d = k.shape[-1]
        scale = p.scale_for(d)
        groups = list(range(p.hkv)) if groups is None else [int(x) for x in groups]
        heads = [h for h in range(p.hq) if p.group(h) in groups]
        keys = [int(j) for j in keys]
        dk = np.zeros((len(keys), p.hkv, d))
        dv = np.zeros((len(keys), p.hkv, d))
        by_node: Dict[int, List[int]] = {}
        for a, j in enumerate(keys):
            for w in self.reader_nodes(j):
                by_node.setdefault(w, []).append(a)
        for w, idx in sorted(by_node.items()):
            o0, L = g.offset[w], g.length[w]
            nonself = [np.arange(g.offset[s] + b, g.offset[s] + e)
                       for s, rs in sorted(g.visible_ranges(w).items()) for b, e in rs]
            ns = np.concatenate(nonself).astype(np.int64) if nonself else np.zeros(0, np.int64)
            vis = np.concatenate([ns, np.arange(o0, o0 + L)])
            col = {int(t): c for c, t in enumerate(vis)}
            # rows of w that see one of the keys: all of them, unless every key is w's own
            own_min = [int(self.off[keys[a]]) for a in idx if int(self.node_of[keys[a]]) == w]
            r_first = min(own_min) if len(own_min) == len(idx) else 0
            kr = rotate(np.asarray(k[vis], np.float64), self.pos[vis], p.rope_base)
            vv = np.asarray(v[vis], np.float64)
            cols = np.array([col[keys[a]] for a in idx])
            for r0 in range(r_first, L, block):
                r1 = min(L, r0 + block)
                rows = np.arange(o0 + r0, o0 + r1)
                qr = rotate(np.asarray(q[rows], np.float64), self.pos[rows], p.rope_base)
                g_o_all = np.asarray(do[rows], np.float64)
                # own key offset i is visible to own row offset r iff i <= r
                hidden = np.zeros((r1 - r0, len(vis)), bool)
                hidden[:, len(ns):] = np.arange(L)[None, :] > np.arange(r0, r1)[:, None]
                for h in heads:
                    gg = p.group(h)
                    s = np.where(hidden, -np.inf, scale * (qr[:, h] @ kr[:, gg].T))
                    P, _ = _softmax_rows(s)
                    O = P @ vv[:, gg]
                    g_o = g_o_all[:, h]
                    D = (g_o * O).sum(axis=1)
                    Pc = P[:, cols]                                   # [rows, n keys of w]
                    dSc = Pc * (g_o @ vv[cols, gg].T - D[:, None])
                    for c, a in enumerate(idx):
                        dk[a, gg] += scale * (dSc[:, c] @ qr[:, h])
                        dv[a, gg] += Pc[:, c] @ g_o
        for a, j in enumerate(keys):
            dk[a] = rotate_transpose(dk[a][None], self.pos[j:j + 1], p.rope_base)[0]
        return dk, dv

    def readers(self, j: int) -> np.ndarray:
        """Every compact query token whose visible set contains key token j."""
        g = self.g
        u, jo = int(self.node_of[j]), int(self.off[j])
        out = [np.arange(g.offset[u] + jo, g.offset[u] + g.length[u])]
        for w in range(g.n):
            if w == u or g.length[w] == 0:
                continue
            if any(b <= jo < e for b, e in g.visible_ranges(w).get(u, [])):
                out.append(np.arange(g.offset[w], g.offset[w] + g.length[w]))
        return np.concatenate(out)

    def key_grads(self, keys: Sequence[int], q, k, v, do):
        """(dk [n,Hkv,d], dv [n,Hkv,d]) for the given key tokens, summed over all readers."""
        q, k, v, do = _np(q), _np(k), _np(v), _np(do)
        p = self.p
        d = k.shape[-1]
        scale = p.scale_for(d)
        dk = np.zeros((len(keys), p.hkv, d))
        dv = np.zeros((len(keys), p.hkv, d))
        for a, j in enumerate(keys):
            j = int(j)
            for t in self.readers(j):
                t = int(t)
                for h, (kt, P, _, oh, kk, qh) in enumerate(self._fwd_one(t, q, k, v)):
                    gg = p.group(h)
                    g_o = np.asarray(do[t, h], np.float64)
                    idx = int(np.searchsorted(kt, j))
                    dp_all = np.asarray(v[kt, gg], np.float64) @ g_o
                    D = float(g_o @ oh)
                    ds = P[idx] * (dp_all[idx] - D)
                    dk[a, gg] += scale * ds * qh
                    dv[a, gg] += P[idx] * g_o
            dk[a] = rotate_transpose(dk[a][None], self.pos[j:j + 1], p.rope_base)[0]
        return dk, dv
