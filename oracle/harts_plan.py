"""HARTS's prefix-aware microbatch planning over raw trajectories (plain Python).

Sources (HARTS: Hybrid-Attention RL over Tree Structures):

* Sec. 3.1 Eq. 5 -- the compact work of a set of trajectories is the number of
  unique token nodes of their trie: after a stable lexicographic sort,
  |x_1| + sum_i (|x_i| - LCP(x_{i-1}, x_i)).
* Sec. 3.1 Eq. 6 -- splitting a contiguous interval at t costs exactly L_t, the
  LCP of the two trajectories at the cut; the LCP of two sorted trajectories is
  the minimum adjacent LCP between them.
* Sec. 3.2 -- the objective J(P) (Eq. 4: total work, then summed slot-critical
  work, then the largest replica-cumulative work); the natural partition by
  lowest LCP valleys; K_min and the candidate range of K (Eq. 7-8); exact
  dynamic programming over contiguous partitions for N <= N0 (Eq. 9); sampled K
  with merge / split evolution for N > N0; trie-aware greedy placement with the
  insertion cost of Eq. 10 under four processing orders and two policies;
  sparse repair; boundary refinement of anchors; replica and slot assignment;
  lexicographic selection.

Readings where the pages leave a step open (each one is listed in the design
notes); every tie is broken towards the earliest item in the order stated:

* K_max = max(K_min, min(D ceil(K0 / D), D floor(N / D)));
* natural partition: an interval whose work exceeds T is cut at the lowest
  adjacent LCP, ties by the smaller larger side, then the smaller difference,
  then the leftmost cut; a single trajectory above T makes the input infeasible;
* the exact DP breaks equal (total, max) ties by the leftmost split point;
* sampled K (N > N0, more than 32 candidates): the 16 smallest candidates and 16
  evenly spaced ones over the whole range (both endpoints included);
* merge / split evolution: merge the adjacent pair with the largest saving,
  split at the interior cut with the smallest increase (leftmost on ties);
* greedy: a new microbatch when nothing fits; eliminating small microbatches
  repeatedly dissolves the lightest microbatch if all its members fit elsewhere
  (same policy); K is then raised to a multiple of D by singleton splits of the
  cheapest member; the greedy candidate is the one with the fewest microbatches,
  then the least total work, among the eight;
* replica assignment: microbatches by work descending (index on ties), slots of
  D consecutive ones, each to the replica with the least cumulative work that
  has none in this slot yet (lowest index on ties);
* candidates are compared in generation order: base candidates by K, then the
  greedy candidate, then refined anchors.

Parity unpinned for the heuristic choices above (the pages fix their intent,
not their tie-breaks); Eq. 5, Eq. 6, Eq. 10, the DP's optimality over
contiguous partitions and the plan's feasibility guarantees are pinned.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

N0, Q_MAX, H_NEAR, B_REF = 512, 32, 8, 3


def lcp(x: Sequence[int], y: Sequence[int]) -> int:
    n = 0
    for a, b in zip(x, y):
        if a != b:
            break
        n += 1
    return n


def trie_nodes(trajs: Sequence[Sequence[int]]) -> int:
    """Unique token nodes of the trie of ``trajs`` (every distinct non-empty prefix)."""
    return len({tuple(t[:i]) for t in trajs for i in range(1, len(t) + 1)})


def compact_work(trajs: Sequence[Sequence[int]]) -> int:
    """Eq. 5 over a stable lexicographic sort."""
    xs = sorted((list(t) for t in trajs))
    if not xs:
        return 0
    return len(xs[0]) + sum(len(xs[i]) - lcp(xs[i - 1], xs[i]) for i in range(1, len(xs)))


class PlanError(ValueError):
    pass


@dataclass
class Plan:
    groups: List[List[int]]                 # microbatches as lists of trajectory indices (input numbering)
    work: List[int]
    replica: List[int] = field(default_factory=list)
    slot: List[int] = field(default_factory=list)
    J: Tuple[int, int, int] = (0, 0, 0)
    source: str = ""


class Planner:
    def __init__(self, trajs: Sequence[Sequence[int]], D: int, T: int, n0: int = N0):
        if D < 1 or T < 1:
            raise PlanError("D and T must be positive")
        self.trajs = [list(t) for t in trajs]
        self.N, self.D, self.T, self.n0 = len(self.trajs), D, T, n0
        if self.N < D:
            raise PlanError("fewer trajectories than replicas")
        # global stable lexicographic order and adjacent LCPs
        self.order = sorted(range(self.N), key=lambda i: (self.trajs[i], i))
        self.pos = [0] * self.N
        for p, i in enumerate(self.order):
            self.pos[i] = p
        self.X = [self.trajs[i] for i in self.order]
        self.L = [0] + [lcp(self.X[i - 1], self.X[i]) for i in range(1, self.N)]

    # -- work -------------------------------------------------------------------
    def W(self, a: int, b: int) -> int:
        """Compact work of the contiguous interval X[a..b] (global sorted positions)."""
        return len(self.X[a]) + sum(len(self.X[i]) - self.L[i] for i in range(a + 1, b + 1))

    def C(self, members: Sequence[int]) -> int:
        """Compact work of a set of global positions (any subset)."""
        ps = sorted(members)
        if not ps:
            return 0
        return len(self.X[ps[0]]) + sum(len(self.X[ps[i]]) - lcp(self.X[ps[i - 1]], self.X[ps[i]])
                                        for i in range(1, len(ps)))

    def insert_cost(self, members: Sequence[int], x: int) -> int:
        """Eq. 10: increase of C when global position x joins ``members``."""
        ps = sorted(members)
        p = max((m for m in ps if m < x), default=None)
        q = min((m for m in ps if m > x), default=None)
        d = len(self.X[x])
        if p is not None:
            d -= lcp(self.X[p], self.X[x])
        if q is not None:
            d -= lcp(self.X[x], self.X[q])
        if p is not None and q is not None:
            d += lcp(self.X[p], self.X[q])
        return d

    # -- natural partition and K range ---------------------------------------------
    def natural_partition(self) -> List[Tuple[int, int]]:
        out: List[Tuple[int, int]] = []

        def rec(a: int, b: int):
            if self.W(a, b) <= self.T:
                out.append((a, b))
                return
            if a == b:
                raise PlanError(f"trajectory of {len(self.X[a])} tokens exceeds the capacity {self.T}")
            best = None
            for t in range(a + 1, b + 1):
                l, r = self.W(a, t - 1), self.W(t, b)
                key = (self.L[t], max(l, r), abs(l - r), t)
                if best is None or key < best:
                    best = key
            t = best[3]
            rec(a, t - 1)
            rec(t, b)
        rec(0, self.N - 1)
        return out

    def k_range(self, K0: int) -> List[int]:
        D, T = self.D, self.T
        G = self.W(0, self.N - 1)
        kmin = D * max(1, -(-G // (T * D)))
        kmax = max(kmin, min(D * (-(-K0 // D)), D * (self.N // D)))
        return list(range(kmin, kmax + 1, D))

    # -- exact DP over contiguous partitions (Eq. 9) ----------------------------------
    def exact(self, K: int) -> Optional[List[Tuple[int, int]]]:
        N, INF = self.N, None
        F = [[INF] * (N + 1) for _ in range(K + 1)]
        arg = [[-1] * (N + 1) for _ in range(K + 1)]
        F[0][0] = (0, 0)
        for k in range(1, K + 1):
            for e in range(k, N + 1):
                best = None
                for s in range(k - 1, e):
                    if F[k - 1][s] is None:
                        continue
                    w = self.W(s, e - 1)
                    if w > self.T:
                        continue
                    cand = (F[k - 1][s][0] + w, max(F[k - 1][s][1], w))
                    if best is None or cand < best:
                        best, arg[k][e] = cand, s
                F[k][e] = best
        if F[K][N] is None:
            return None
        parts, e = [], N
        for k in range(K, 0, -1):
            s = arg[k][e]
            parts.append((s, e - 1))
            e = s
        return parts[::-1]

    # -- sampled K and merge / split evolution (N > N0) ---------------------------------
    def sample_k(self, ks: List[int]) -> List[int]:
        if len(ks) <= Q_MAX:
            return ks
        dense = ks[:Q_MAX // 2]
        n_sparse = Q_MAX - len(dense)
        sparse = [ks[round(i * (len(ks) - 1) / (n_sparse - 1))] for i in range(n_sparse)]
        return sorted(set(dense) | set(sparse))

    def evolve(self, P0: List[Tuple[int, int]], K: int) -> Optional[List[Tuple[int, int]]]:
        parts = list(P0)
        while len(parts) > K:
            best = None
            for i in range(len(parts) - 1):
                a, b = parts[i][0], parts[i + 1][1]
                if self.W(a, b) > self.T:
                    continue
                saving = self.L[parts[i + 1][0]]
                if best is None or saving > best[0]:
                    best = (saving, i)
            if best is None:
                return None
            i = best[1]
            parts[i:i + 2] = [(parts[i][0], parts[i + 1][1])]
        while len(parts) < K:
            best = None
            for i, (a, b) in enumerate(parts):
                for t in range(a + 1, b + 1):
                    if best is None or self.L[t] < best[0]:
                        best = (self.L[t], i, t)
            if best is None:
                return None
            _, i, t = best
            a, b = parts[i]
            parts[i:i + 1] = [(a, t - 1), (t, b)]
        return parts

    def refine_boundaries(self, parts: List[Tuple[int, int]]) -> List[Tuple[int, int]]:
        parts = list(parts)
        for _ in range(2):
            changed = False
            for i in range(len(parts) - 1):
                a, b = parts[i][0], parts[i + 1][1]
                t0 = parts[i + 1][0]
                cur = (self.W(a, t0 - 1) + self.W(t0, b), max(self.W(a, t0 - 1), self.W(t0, b)))
                best, bt = cur, t0
                for t in range(max(a + 1, t0 - H_NEAR), min(b, t0 + H_NEAR) + 1):
                    l, r = self.W(a, t - 1), self.W(t, b)
                    if l > self.T or r > self.T:
                        continue
                    key = (l + r, max(l, r))
                    if key < best:
                        best, bt = key, t
                if bt != t0:
                    parts[i], parts[i + 1] = (a, bt - 1), (bt, b)
                    changed = True
            if not changed:
                break
        return parts

    # -- trie-aware greedy (Eq. 10) ---------------------------------------------------
    def _orders(self) -> List[List[int]]:
        N = self.N
        asc = list(range(N))
        desc = asc[::-1]
        by_len = sorted(asc, key=lambda p: (-len(self.X[p]), p))

        def u(p):
            l = self.L[p] if p > 0 else 0
            r = self.L[p + 1] if p + 1 < N else 0
            return len(self.X[p]) - max(l, r)
        by_u = sorted(asc, key=lambda p: (-u(p), p))
        return [asc, desc, by_len, by_u]

    def _place(self, groups: List[List[int]], x: int, policy: str, exclude: int = -1) -> int:
        best, bi = None, -1
        for gi, g in enumerate(groups):
            if gi == exclude or not g:
                continue
            d = self.insert_cost(g, x)
            w = self.C(g) + d
            if w > self.T:
                continue
            key = w if policy == "best_fit" else len(self.X[x]) - d
            if best is None or key > best:
                best, bi = key, gi
        return bi

    def greedy_plan(self, order: List[int], policy: str) -> Optional[List[List[int]]]:
        groups: List[List[int]] = []
        for x in order:
            gi = self._place(groups, x, policy)
            if gi < 0:
                groups.append([x])
            else:
                groups[gi].append(x)
        # eliminate small microbatches
        while len(groups) > 1:
            light = min(range(len(groups)), key=lambda i: (self.C(groups[i]), i))
            trial = [list(g) for g in groups]
            moved = sorted(trial[light])
            trial[light] = []
            ok = True
            for x in moved:
                gi = self._place(trial, x, policy, exclude=light)
                if gi < 0:
                    ok = False
                    break
                trial[gi].append(x)
            if not ok:
                break
            groups = [g for g in trial if g]
        # align K to a multiple of D with singleton splits
        while len(groups) % self.D:
            best = None
            for gi, g in enumerate(groups):
                if len(g) < 2:
                    continue
                for x in sorted(g):
                    rest = [m for m in g if m != x]
                    inc = len(self.X[x]) - self.insert_cost(rest, x)
                    if best is None or inc < best[0]:
                        best = (inc, gi, x)
            if best is None:
                return None
            _, gi, x = best
            groups[gi] = [m for m in groups[gi] if m != x]
            groups.append([x])
        return [sorted(g) for g in groups]

    def sparse_repair(self, groups: List[List[int]], iterations: int = 4) -> List[List[int]]:
        """At most ``iterations`` (the page's four) best strictly improving moves or swaps."""
        groups = [sorted(g) for g in groups]
        for _ in range(iterations):
            where = {x: gi for gi, g in enumerate(groups) for x in g}
            best = None
            for x in range(self.N):
                A = where[x]
                if len(groups[A]) < 2:
                    continue
                cA = self.C(groups[A])
                restA = [m for m in groups[A] if m != x]
                for B, g in enumerate(groups):
                    if B == A or not any(abs(y - x) <= H_NEAR for y in g):
                        continue
                    newB = self.C(g + [x])
                    if newB > self.T:
                        continue
                    gain = cA + self.C(g) - self.C(restA) - newB
                    if gain > 0 and (best is None or gain > best[0]):
                        best = (gain, "move", x, A, B)
            if best is None:
                for x in range(self.N):
                    for y in range(x + 1, min(self.N, x + H_NEAR + 1)):
                        A, B = where[x], where[y]
                        if A == B:
                            continue
                        nA = [m for m in groups[A] if m != x] + [y]
                        nB = [m for m in groups[B] if m != y] + [x]
                        cnA, cnB = self.C(nA), self.C(nB)
                        if cnA > self.T or cnB > self.T:
                            continue
                        gain = self.C(groups[A]) + self.C(groups[B]) - cnA - cnB
                        if gain > 0 and (best is None or gain > best[0]):
                            best = (gain, "swap", x, y)
            if best is None:
                break
            if best[1] == "move":
                _, _, x, A, B = best
                groups[A].remove(x)
                groups[B] = sorted(groups[B] + [x])
            else:
                _, _, x, y = best
                A, B = where[x], where[y]
                groups[A] = sorted([m for m in groups[A] if m != x] + [y])
                groups[B] = sorted([m for m in groups[B] if m != y] + [x])
        return groups

    # -- replica / slot assignment and the objective (Eq. 4) ------------------------------
    def assign(self, groups: List[List[int]], source: str) -> Plan:
        work = [self.C(g) for g in groups]
        K, D = len(groups), self.D
        byw = sorted(range(K), key=lambda i: (-work[i], i))
        replica, slot = [0] * K, [0] * K
        cum = [0] * D
        slot_crit = 0
        for j in range(K // D):
            block = byw[j * D:(j + 1) * D]
            free = list(range(D))
            for i in block:
                d = min(free, key=lambda r: (cum[r], r))
                free.remove(d)
                replica[i], slot[i] = d, j
                cum[d] += work[i]
            slot_crit += max(work[i] for i in block)
        groups_in = [sorted(self.order[p] for p in g) for g in groups]
        return Plan(groups_in, work, replica, slot, (sum(work), slot_crit, max(cum)), source)

    # -- the whole planner --------------------------------------------------------------
    def plan(self) -> Plan:
        P0 = self.natural_partition()
        ks = self.k_range(len(P0))
        cands: List[Plan] = []
        parts_of = {}
        exact = self.N <= self.n0
        for K in (ks if exact else self.sample_k(ks)):
            parts = self.exact(K) if exact else self.evolve(P0, K)
            if parts is None:
                continue
            parts_of[K] = parts
            cands.append(self.assign([list(range(a, b + 1)) for a, b in parts], f"{'exact' if exact else 'evolve'}:{K}"))
        greedy = []
        for oi, order in enumerate(self._orders()):
            for policy in ("best_fit", "max_shared"):
                g = self.greedy_plan(order, policy)
                if g is not None:
                    greedy.append(g)
        gk = None
        if greedy:
            g = min(greedy, key=lambda gr: (len(gr), sum(self.C(m) for m in gr)))
            gk = len(g)
            cands.append(self.assign(self.sparse_repair(g), "greedy"))
        if not exact and parts_of:
            base = [(K, c) for K, c in zip(parts_of.keys(), [c for c in cands if c.source.startswith("evolve")])]
            anchors: List[int] = []
            if gk is not None and gk in parts_of:
                anchors.append(gk)
            low = min(base, key=lambda kc: (kc[1].J[0], kc[0]))[0]
            if low not in anchors:
                anchors.append(low)
            if gk is not None:
                rest = [K for K, _ in base if K not in anchors]
                if rest:
                    anchors.append(min(rest, key=lambda K: (abs(K - gk), K)))
            for K in anchors[:B_REF]:
                r = self.refine_boundaries(parts_of[K])
                cands.append(self.assign([list(range(a, b + 1)) for a, b in r], f"refined:{K}"))
        if not cands:
            raise PlanError("no feasible plan")
        return min(cands, key=lambda c: c.J)          # first among equals: generation order
