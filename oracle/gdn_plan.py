"""Minimum-call planning of linear-attention execution over a rollout tree.

Written from HARTS, Sec. 2.2 Eq. 2 (resume anchor a(p) = B floor(p / B)) and
Sec. 3.3 ("Minimum-Call Planning for Linear-Attention Execution": segment
trees, the earliest-legal-start condition Eq. 11, the two minimum call counts
T_pre / T_in of Eq. 12-14, the recovery of Algorithm 1 as its text describes
it, and the mandatory replay R of Eq. 15), with Fig. 2 as the worked example.

Readings where the pages are silent (listed in the design notes):

* the tree is the DAG's parent tree; mounts are ignored (recurrent layers skip
  mounted spans, Octopus Sec. 3);
* zero-length leaves carry no tokens and are pruned before planning, repeatedly;
  what remains is contracted into segments (a node starts a segment iff it is a
  root or its parent has two or more surviving children);
* children are taken in node-table order (the "fixed child order");
* a side branch's initial state is S at a(e_v): in the same-round case that is
  the state the parent's sequence started from (zero for a root), otherwise it
  is exported by the parent's sequence at boundary a(e_v).

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import itertools
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

from .dag import Dag


@dataclass
class Segment:
    nodes: List[int]                 # DAG nodes, in path order
    s: int                           # recurrent index of the first token
    e: int                           # one past the last token (the fork position for an internal segment)
    parent: int = -1                 # parent segment
    children: List[int] = field(default_factory=list)


def segments(spec) -> List[Segment]:
    dag = Dag(spec)
    alive = [False] * dag.n
    for u in range(dag.n - 1, -1, -1):            # children follow their parents in the table
        if dag.length[u] > 0 or any(alive[c] for c in dag.children[u]):
            alive[u] = True
    kids = [[c for c in dag.children[u] if alive[c]] for u in range(dag.n)]
    depth = [0] * dag.n
    for u in range(dag.n):
        p = dag.parent[u]
        depth[u] = 0 if p < 0 else depth[p] + dag.length[p]
    segs: List[Segment] = []
    seg_of: Dict[int, int] = {}

    def start(u: int, par: int) -> None:
        nodes = [u]
        while len(kids[nodes[-1]]) == 1:
            nodes.append(kids[nodes[-1]][0])
        s = depth[u]
        e = depth[nodes[-1]] + dag.length[nodes[-1]]
        segs.append(Segment(nodes, s, e, par))
        me = len(segs) - 1
        seg_of[u] = me
        if par >= 0:
            segs[par].children.append(me)
        for c in kids[nodes[-1]]:
            start(c, me)

    for r in range(dag.n):
        if dag.parent[r] < 0 and alive[r]:
            start(r, -1)
    return segs


def anchor(p: int, B: int) -> int:
    """a(p): the nearest chunk boundary at or before p (HARTS Eq. 2)."""
    return B * (p // B)


def min_calls(segs: List[Segment], B: int) -> Tuple[List[int], List[int]]:
    """T_pre and T_in of every segment (HARTS Eq. 12-14), children before parents."""
    n = len(segs)
    t_pre, t_in = [0] * n, [0] * n
    for v in range(n - 1, -1, -1):                # segments are numbered parents first
        ch = segs[v].children
        if not ch:
            t_pre[v] = t_in[v] = 1
            continue
        best = None
        for o in ch:
            others = [t_pre[u] for u in ch if u != o]
            val = max(t_in[o], 1 + max(others, default=0))
            best = val if best is None else min(best, val)
        t_in[v] = best
        if segs[v].e < anchor(segs[v].s, B) + B:
            t_pre[v] = max(t_pre[u] for u in ch)
        else:
            t_pre[v] = t_in[v]
    return t_pre, t_in


@dataclass
class Sequence:
    round: int
    segs: List[int]
    start: int                       # chunk-aligned recurrent index where the sequence starts
    replay: Tuple[int, int]          # [start, fork) replayed ancestor positions (empty for a root)
    init: Optional[Tuple[int, int]]  # None: zero state; else (producer sequence, boundary index)


def recover(segs: List[Segment], B: int) -> List[Sequence]:
    """Rounds of packed sequences (HARTS Algorithm 1, recovery pass), trees in table order."""
    t_pre, t_in = min_calls(segs, B)
    seqs: List[Sequence] = []

    def rec(v: int, ready: bool, k_round: int, r: int, q: int) -> None:
        seqs[q].segs.append(v)
        ch = segs[v].children
        if not ch:
            return
        sv, ev = segs[v].s, segs[v].e
        same = ready and ev < anchor(sv, B) + B
        delta = 0 if same else 1
        k_side = k_round - delta
        H = {o: (t_pre[o] if same else t_in[o]) for o in ch}
        f = sum(1 for u in ch if t_pre[u] > k_side)
        direct = next(o for o in ch if H[o] <= k_round and f - (1 if t_pre[o] > k_side else 0) == 0)
        rec(direct, same, k_round, r, q)
        b = anchor(ev, B)
        for u in ch:
            if u == direct:
                continue
            init = seqs[q].init if same else (q, b)
            seqs.append(Sequence(r + delta, [], b, (b, ev), init))
            rec(u, True, k_side, r + delta, len(seqs) - 1)

    for root, sg in enumerate(segs):
        if sg.parent >= 0:
            continue
        seqs.append(Sequence(1, [], 0, (0, 0), None))
        rec(root, True, t_pre[root], 1, len(seqs) - 1)
    return seqs


def replay_total(segs: List[Segment], B: int) -> int:
    """R of HARTS Eq. 15: (children - 1) * (e_v mod B) summed over internal segments."""
    return sum((len(s.children) - 1) * (s.e % B) for s in segs if s.children)


def brute_force_calls(segs: List[Segment], B: int) -> int:
    """Fewest rounds over every choice of direct child, by simulating readiness.

    A side child starts a new sequence in the parent's round when the parent
    entered with a ready anchor state and crossed no new chunk boundary
    (e_v < a_v + B, HARTS Eq. 11), otherwise one round later; the direct child
    continues the parent's sequence and inherits readiness only in the first
    case.  Exponential; tiny trees only.
    """
    internal = [v for v, s in enumerate(segs) if s.children]
    best = None
    for pick in itertools.product(*[segs[v].children for v in internal]):
        choice = dict(zip(internal, pick))

        def run(v: int, ready: bool, r: int) -> int:
            ch = segs[v].children
            if not ch:
                return r
            same = ready and segs[v].e < anchor(segs[v].s, B) + B
            out = run(choice[v], same, r)
            for u in ch:
                if u != choice[v]:
                    out = max(out, run(u, True, r if same else r + 1))
            return out

        total = max(run(v, True, 1) for v, s in enumerate(segs) if s.parent < 0)
        best = total if best is None else min(best, total)
    return best or 0
