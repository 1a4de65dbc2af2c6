"""Rollout-DAG semantics, written from the pages' definitions.

Sources (titles of the pages and the places on them):

* Octopus, Sec. 3 (execution DAG with tree edges and read_thread mount edges),
  Sec. 3.2 Eq. 2 (monotonic position continuation and its worked example),
  Sec. 3.3 item 1 (node u = (parent, active mounts incl. transitive, start)),
  Sec. 3.3 Eq. 4 (a node attends to its mounts, its ancestors and itself),
  Sec. 3.4 Eq. 6 (each node belongs to the unique leaf that first generated it).
* HARTS, Sec. 4.2 Eq. 21-22 (a branch's queries see every ancestor key and
  the causal triangle of their own tokens).

Readings where the pages are silent (each one is listed in the design notes):

* a mount is active from the first token of the node that lists it, and stays
  active for every descendant;
* ``pos_end`` of a mount is the position of its last token (the worked example
  of Eq. 2: a read of 1,500-4,000 moves the reader to 4,001);
* a zero-length mount is ignored entirely;
* a direct mount onto the reader's own ancestor chain is rejected; spans that
  reach the chain through transitive closure, and overlapping spans, merge by
  set union (visibility is a set).

Views of one table pair (Octopus App. C: a dense model mounts in a subset of its
layers and gives the others a mount-free view; Octopus Table 5's "unshifted"
regime mounts without the position jump):

* ``mounted``    -- the default: mounted spans visible, positions by Eq. 2;
* ``mount_free`` -- positions by Eq. 2 (they belong to the tokens), mounted
                    spans not visible (reading: the layers that do not mount see
                    their tree ancestors only);
* ``unshifted``  -- mounted spans visible, every node continuing from its
                    parent's next position as if it had no reads.
The tables are validated the same way in every view.
"""
from __future__ import annotations

from typing import Dict, List, Tuple

import numpy as np

INVALID, NOT_TOPO, MOUNT_CYCLE, MOUNT_RANGE, SELF_ANCESTOR_MOUNT = (
    "INVALID", "NOT_TOPO", "MOUNT_CYCLE", "MOUNT_RANGE", "SELF_ANCESTOR_MOUNT")


VIEWS = ("mounted", "mount_free", "unshifted")


class DagError(ValueError):
    def __init__(self, code: str, msg: str):
        super().__init__(f"{code}: {msg}")
        self.code = code


class Dag:
    """Plain-Python view of a node/mount table pair with the derived semantics."""

    def __init__(self, spec, transitive: bool = True, view: str = "mounted"):
        if view not in VIEWS:
            raise ValueError(f"view must be one of {VIEWS}")
        self.view = view
        self.n = int(len(spec.parent))
        self.parent = [int(x) for x in spec.parent]
        self.length = [int(x) for x in spec.length]
        self.transitive = bool(transitive)
        nm = int(len(spec.mount_src))
        self.direct: List[List[Tuple[int, int, int]]] = []
        self._validate_tables(spec, nm)
        self.offset = [0] * self.n                  # first token id of each node
        acc = 0
        for u in range(self.n):
            self.offset[u] = acc
            acc += self.length[u]
        self.n_tokens = acc
        self.children: List[List[int]] = [[] for _ in range(self.n)]
        for u in range(self.n):
            if self.parent[u] >= 0:
                self.children[self.parent[u]].append(u)
        self.ancestors = self._ancestors()
        self._validate_mounts()
        self.order = self._topo_order()
        self.start = self._positions()
        self.active = self._active_spans()

    # -- validation -------------------------------------------------------
    def _validate_tables(self, spec, nm: int) -> None:
        if self.n <= 0:
            raise DagError(INVALID, "a DAG needs at least one node")
        for u in range(self.n):
            p = self.parent[u]
            if p < -1 or p >= self.n:
                raise DagError(INVALID, f"node {u}: parent {p} out of range")
            if p >= u:
                raise DagError(NOT_TOPO, f"node {u}: parent {p} is not earlier")
            if self.length[u] < 0:
                raise DagError(INVALID, f"node {u}: negative length")
        for u in range(self.n):
            f, c = int(spec.mount_first[u]), int(spec.mount_count[u])
            if c < 0 or f < 0 or f + c > nm:
                raise DagError(INVALID, f"node {u}: mount slice out of range")
            ms = []
            for i in range(f, f + c):
                s, b, e = int(spec.mount_src[i]), int(spec.mount_begin[i]), int(spec.mount_end[i])
                if s < 0 or s >= self.n:
                    raise DagError(INVALID, f"node {u}: mount source {s} out of range")
                if not (0 <= b <= e <= self.length[s]):
                    raise DagError(MOUNT_RANGE, f"node {u}: span [{b},{e}) outside source {s}")
                ms.append((s, b, e))
            self.direct.append(ms)

    def _ancestors(self) -> List[set]:
        anc: List[set] = []
        for u in range(self.n):
            p = self.parent[u]
            anc.append(set() if p < 0 else (anc[p] | {p}))
        return anc

    def nonempty_direct(self, u: int) -> List[Tuple[int, int, int]]:
        return [m for m in self.direct[u] if m[2] > m[1]]

    def _validate_mounts(self) -> None:
        for u in range(self.n):
            for s, b, e in self.nonempty_direct(u):
                if s == u or s in self.ancestors[u]:
                    raise DagError(SELF_ANCESTOR_MOUNT, f"node {u} reads its own chain ({s})")

    def _topo_order(self) -> List[int]:
        """Order in which every node follows its parent and its (non-empty) mount sources."""
        deps = [set() for _ in range(self.n)]
        for u in range(self.n):
            if self.parent[u] >= 0:
                deps[u].add(self.parent[u])
            for s, _, _ in self.nonempty_direct(u):
                deps[u].add(s)
        users: List[List[int]] = [[] for _ in range(self.n)]
        indeg = [len(d) for d in deps]
        for u in range(self.n):
            for s in deps[u]:
                users[s].append(u)
        ready = [u for u in range(self.n) if indeg[u] == 0]
        order = []
        while ready:
            ready.sort()
            u = ready.pop(0)
            order.append(u)
            for w in users[u]:
                indeg[w] -= 1
                if indeg[w] == 0:
                    ready.append(w)
        if len(order) != self.n:
            raise DagError(MOUNT_CYCLE, "tree and mount edges form a cycle")
        return order

    # -- Octopus Eq. 2 -----------------------------------------------------
    def _positions(self) -> List[int]:
        """s(u) = max(next position after the parent, max over u's reads of (end position + 1))."""
        start = [0] * self.n
        for u in self.order:
            p = self.parent[u]
            s = 0 if p < 0 else start[p] + self.length[p]
            if self.view != "unshifted":
                for src, b, e in self.nonempty_direct(u):
                    pos_end = start[src] + (e - 1)      # position of the last mounted token
                    s = max(s, pos_end + 1)
            start[u] = s
        return start

    def token_positions(self) -> np.ndarray:
        pos = np.zeros(self.n_tokens, np.int64)
        for u in range(self.n):
            o = self.offset[u]
            pos[o:o + self.length[u]] = self.start[u] + np.arange(self.length[u])
        return pos

    # -- active mounts (Octopus Sec. 3.3 item 1, incl. transitive) ----------
    def _active_spans(self) -> List[List[Tuple[int, int, int]]]:
        act: List[List[Tuple[int, int, int]]] = [[] for _ in range(self.n)]
        for u in self.order:
            p = self.parent[u]
            spans = list(act[p]) if p >= 0 else []
            for m in (self.nonempty_direct(u) if self.view != "mount_free" else []):
                spans.append(m)
                if self.transitive:
                    spans.extend(act[m[0]])
            act[u] = list(dict.fromkeys(spans))          # drop repeats, keep first-seen order
        return act

    # -- visibility -----------------------------------------------------------
    def visible_ranges(self, u: int) -> Dict[int, List[Tuple[int, int]]]:
        """Non-self part of what node u's tokens see: {node: disjoint sorted [lo, hi) ranges}.

        Every strict ancestor entirely, plus the union of the active mounted spans.
        """
        if not hasattr(self, "_vr_cache"):
            self._vr_cache = {}
        if u in self._vr_cache:
            return self._vr_cache[u]
        out: Dict[int, List[Tuple[int, int]]] = {}
        for a in self.ancestors[u]:
            if self.length[a] > 0:
                out[a] = [(0, self.length[a])]
        per_src: Dict[int, List[Tuple[int, int]]] = {}
        for s, b, e in self.active[u]:
            if s in self.ancestors[u]:
                continue                                 # already wholly visible
            per_src.setdefault(s, []).append((b, e))
        for s, rs in per_src.items():
            rs.sort()
            merged: List[List[int]] = []
            for b, e in rs:
                if merged and b <= merged[-1][1]:
                    merged[-1][1] = max(merged[-1][1], e)
                else:
                    merged.append([b, e])
            out[s] = [(b, e) for b, e in merged]
        self._vr_cache[u] = out
        return out

    def _mounted_token_ids(self, u: int) -> np.ndarray:
        """Token ids of the mounted (non-ancestor) part of node u's visible set."""
        parts = [np.arange(self.offset[s] + b, self.offset[s] + e)
                 for s, rs in self.visible_ranges(u).items() if s not in self.ancestors[u]
                 for b, e in rs]
        return np.concatenate(parts) if parts else np.zeros(0, np.int64)

    def visible_tokens(self, u: int, i: int) -> np.ndarray:
        """Sorted token ids visible from token i of node u (the set V(u, i))."""
        ids = [np.arange(self.offset[u], self.offset[u] + i + 1)]
        for s, rs in self.visible_ranges(u).items():
            for b, e in rs:
                ids.append(np.arange(self.offset[s] + b, self.offset[s] + e))
        return np.sort(np.concatenate(ids))

    def token_node(self) -> Tuple[np.ndarray, np.ndarray]:
        node = np.zeros(self.n_tokens, np.int64)
        off = np.zeros(self.n_tokens, np.int64)
        for u in range(self.n):
            o = self.offset[u]
            node[o:o + self.length[u]] = u
            off[o:o + self.length[u]] = np.arange(self.length[u])
        return node, off

    # -- trajectories and owners (Octopus Sec. 3.4 Eq. 6) -----------------------
    def leaves_dfs(self) -> List[int]:
        out = []
        for r in range(self.n):
            if self.parent[r] != -1:
                continue
            stack = [r]
            while stack:
                u = stack.pop()
                if not self.children[u]:
                    out.append(u)
                stack.extend(reversed(self.children[u]))
        return out

    def chain(self, u: int) -> List[int]:
        c = []
        while u >= 0:
            c.append(u)
            u = self.parent[u]
        return c[::-1]

    def trajectory(self, leaf: int) -> Tuple[np.ndarray, np.ndarray]:
        """Token ids of the root-to-leaf sequence with mounted spans spliced in.

        Node by node along the chain: the tokens of the spans that become
        visible at that node (those not already spliced), then the node's own
        tokens.  Returns (token ids, own flag) where own is False for spliced
        tokens.
        """
        seq: List[np.ndarray] = []
        own: List[np.ndarray] = []
        spliced = np.zeros(0, np.int64)
        for a in self.chain(leaf):
            m = self._mounted_token_ids(a)
            new = np.setdiff1d(m, spliced)               # sorted, not yet present
            spliced = np.union1d(spliced, new)
            seq.append(new)
            own.append(np.zeros(len(new), bool))
            seq.append(np.arange(self.offset[a], self.offset[a] + self.length[a]))
            own.append(np.ones(self.length[a], bool))
        return np.concatenate(seq).astype(np.int64), np.concatenate(own)

    def owner(self) -> List[int]:
        """owner[u] = the first leaf in DFS order whose trajectory contains node u."""
        own = [-1] * self.n
        for leaf in self.leaves_dfs():
            for a in self.chain(leaf):
                if own[a] < 0:
                    own[a] = leaf
        return own

    def multiplicity(self) -> np.ndarray:
        """Semantic uses of each token: the number of trajectories that hold it as an own token."""
        q = np.zeros(self.n_tokens, np.int64)
        for leaf in self.leaves_dfs():
            for a in self.chain(leaf):
                q[self.offset[a]:self.offset[a] + self.length[a]] += 1
        return q

    def flat_rows(self) -> int:
        """Rows of the flat expansion: every trajectory's length including spliced spans.

        A leaf's trajectory holds exactly what its last token sees plus that token.
        """
        total = 0
        for leaf in self.leaves_dfs():
            total += self.length[leaf] + sum(e - b for rs in self.visible_ranges(leaf).values()
                                             for b, e in rs)
        return total

    def visible_pairs(self) -> int:
        """P: the number of visible (query, key) pairs over compact query tokens."""
        total = 0
        for u in range(self.n):
            ln = self.length[u]
            if ln == 0:
                continue
            nonself = sum(e - b for rs in self.visible_ranges(u).values() for b, e in rs)
            total += ln * nonself + ln * (ln + 1) // 2
        return total
