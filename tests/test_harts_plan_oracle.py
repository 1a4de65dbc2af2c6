"""Pins for the prefix-aware microbatch planner oracle (HARTS Sec. 3.1-3.2).

Eq. 5 against the trie's node count by brute force; Eq. 6 and the LCP range
minimum; Eq. 10 against the work of the enlarged set; the exact DP against
brute force over every contiguous partition; and every returned plan against
the feasibility guarantees the pages state (exact coverage, nonempty
microbatches within capacity, K mod D = 0, K/D microbatches per replica, one
per slot).
"""
import itertools

import numpy as np
import pytest

from oracle import harts_plan as HP


def _trajs(rng, n, vocab=3, lo=1, hi=9, share=0.7):
    """Random trajectories that share prefixes (some duplicates and strict prefixes)."""
    out = []
    for _ in range(n):
        if out and rng.random() < share:
            base = out[int(rng.integers(0, len(out)))]
            cut = int(rng.integers(0, len(base) + 1))
            t = base[:cut] + [int(v) for v in rng.integers(0, vocab, int(rng.integers(0, hi - lo + 1)))]
        else:
            t = [int(v) for v in rng.integers(0, vocab, int(rng.integers(lo, hi + 1)))]
        out.append(t if t else [0])
    return out


@pytest.mark.parametrize("seed", range(30))
def test_eq5_compact_work_is_the_trie_node_count(seed):
    rng = np.random.default_rng(seed)
    ts = _trajs(rng, int(rng.integers(1, 12)))
    assert HP.compact_work(ts) == HP.trie_nodes(ts)
    p = HP.Planner(ts, 1, 10 ** 6)
    assert p.W(0, p.N - 1) == HP.trie_nodes(ts)
    for a in range(p.N):
        for b in range(a, p.N):
            assert p.W(a, b) == HP.trie_nodes(p.X[a:b + 1])


@pytest.mark.parametrize("seed", range(20))
def test_eq6_split_cost_and_lcp_range_minimum(seed):
    rng = np.random.default_rng(100 + seed)
    p = HP.Planner(_trajs(rng, 10), 1, 10 ** 6)
    for a in range(p.N):
        for t in range(a + 1, p.N):
            for b in range(t, p.N):
                assert p.W(a, t - 1) + p.W(t, b) - p.W(a, b) == p.L[t]
    for i in range(p.N):
        for j in range(i + 1, p.N):
            assert HP.lcp(p.X[i], p.X[j]) == min(p.L[i + 1:j + 1])


@pytest.mark.parametrize("seed", range(20))
def test_eq10_insertion_cost(seed):
    rng = np.random.default_rng(200 + seed)
    p = HP.Planner(_trajs(rng, 10), 1, 10 ** 6)
    for _ in range(30):
        members = sorted(rng.choice(p.N, int(rng.integers(0, p.N)), replace=False).tolist())
        x = int(rng.integers(0, p.N))
        if x in members:
            continue
        assert p.insert_cost(members, x) == p.C(members + [x]) - p.C(members)
        assert p.C(members + [x]) == HP.trie_nodes([p.X[m] for m in members + [x]])


@pytest.mark.parametrize("seed", range(25))
def test_exact_dp_is_optimal_over_contiguous_partitions(seed):
    rng = np.random.default_rng(300 + seed)
    ts = _trajs(rng, int(rng.integers(2, 9)))
    T = max(len(t) for t in ts) + int(rng.integers(0, 12))
    p = HP.Planner(ts, 1, T)
    for K in range(1, p.N + 1):
        best = None
        for cuts in itertools.combinations(range(1, p.N), K - 1):
            bounds = [0, *cuts, p.N]
            ws = [p.W(bounds[i], bounds[i + 1] - 1) for i in range(K)]
            if max(ws) > T:
                continue
            key = (sum(ws), max(ws))
            best = key if best is None or key < best else best
        parts = p.exact(K)
        if best is None:
            assert parts is None
            continue
        ws = [p.W(a, b) for a, b in parts]
        assert (sum(ws), max(ws)) == best


def _check_feasible(p, plan):
    seen = sorted(i for g in plan.groups for i in g)
    assert seen == list(range(p.N))                                   # exact coverage
    assert all(plan.groups) and all(w <= p.T for w in plan.work)
    K = len(plan.groups)
    assert K % p.D == 0
    for d in range(p.D):                                              # K/D per replica, one per slot
        slots = sorted(plan.slot[i] for i in range(K) if plan.replica[i] == d)
        assert slots == list(range(K // p.D))
    for g, w in zip(plan.groups, plan.work):
        assert w == HP.trie_nodes([p.trajs[i] for i in g])
    cum = [sum(plan.work[i] for i in range(K) if plan.replica[i] == d) for d in range(p.D)]
    crit = sum(max(plan.work[i] for i in range(K) if plan.slot[i] == j) for j in range(K // p.D))
    assert plan.J == (sum(plan.work), crit, max(cum))


@pytest.mark.parametrize("seed", range(30))
def test_plans_meet_the_guarantees(seed):
    rng = np.random.default_rng(400 + seed)
    n = int(rng.integers(4, 40))
    ts = _trajs(rng, n, hi=12)
    D = int(rng.integers(1, 5))
    if n < D:
        return
    T = max(len(t) for t in ts) + int(rng.integers(0, 40))
    n0 = 512 if seed % 2 else 6                      # odd seeds: exact search; even: sampled K
    p = HP.Planner(ts, D, T, n0=n0)
    try:
        plan = p.plan()
    except HP.PlanError:
        return
    _check_feasible(p, plan)


def test_natural_partition_cuts_at_the_lowest_valley():
    # two families sharing nothing, each long: the first cut separates them
    a = [[1, 1, 1, 1, 1, 1, i] for i in range(4)]
    b = [[2, 2, 2, 2, 2, 2, i] for i in range(4)]
    p = HP.Planner(a + b, 2, 12)
    parts = p.natural_partition()
    assert all(p.W(x, y) <= 12 for x, y in parts)
    assert (0, 3) in parts and (4, 7) in parts
    plan = p.plan()
    assert sorted(map(sorted, plan.groups)) == [[0, 1, 2, 3], [4, 5, 6, 7]]
    assert plan.J[0] == 2 * (6 + 4)


def test_capacity_below_a_trajectory_is_rejected():
    with pytest.raises(HP.PlanError):
        HP.Planner([[1, 2, 3, 4]], 1, 3).plan()


# ---------------------------------------------------------------- the heuristic steps of Sec. 3.2
# Each step is checked against what the page states it does, with the trie's node count
# (every distinct non-empty prefix, by brute force) as the cost, independent of Eq. 5's
# sorted-LCP evaluation the planner uses.

def _tw(p, members):
    """Compact work of global positions ``members`` by brute force over the trie's prefixes."""
    return HP.trie_nodes([p.X[m] for m in members])


def _planner(seed, n_lo=6, n_hi=24, slack=(0, 30), D=1):
    rng = np.random.default_rng(seed)
    ts = _trajs(rng, int(rng.integers(n_lo, n_hi)), hi=12)
    T = max(len(t) for t in ts) + int(rng.integers(*slack))
    return HP.Planner(ts, D, T), rng


@pytest.mark.parametrize("seed", range(25))
def test_evolve_merges_the_adjacent_pair_with_the_largest_saving(seed):
    """Below K0 every merge joins the capacity-feasible adjacent pair whose union saves the most,
    C(A) + C(B) - C(A u B) (first such pair on ties)."""
    p, _ = _planner(500 + seed, slack=(0, 8))
    P0 = p.natural_partition()
    prev = P0
    for K in range(len(P0) - 1, 0, -1):
        cur = p.evolve(P0, K)
        if cur is None:
            break
        cand = []
        for i in range(len(prev) - 1):
            A, B = list(range(prev[i][0], prev[i][1] + 1)), list(range(prev[i + 1][0], prev[i + 1][1] + 1))
            if _tw(p, A + B) <= p.T:
                cand.append((_tw(p, A) + _tw(p, B) - _tw(p, A + B), -i, i))
        assert cand, "evolve merged an infeasible pair"
        i = max(cand)[2]
        assert cur == prev[:i] + [(prev[i][0], prev[i + 1][1])] + prev[i + 2:]
        prev = cur


@pytest.mark.parametrize("seed", range(25))
def test_evolve_splits_at_the_cut_with_the_smallest_increase(seed):
    """Above K0 every split cuts one microbatch M into contiguous L, R with the smallest
    C(L) + C(R) - C(M) (first such cut on ties)."""
    p, _ = _planner(600 + seed, slack=(10, 60))
    P0 = p.natural_partition()
    prev = P0
    for K in range(len(P0) + 1, min(p.N, len(P0) + 6) + 1):
        cur = p.evolve(P0, K)
        cand = []
        for i, (a, b) in enumerate(prev):
            M = list(range(a, b + 1))
            for t in range(a + 1, b + 1):
                L, R = list(range(a, t)), list(range(t, b + 1))
                cand.append((_tw(p, L) + _tw(p, R) - _tw(p, M), i, t))
        _, i, t = min(cand)
        a, b = prev[i]
        assert cur == prev[:i] + [(a, t - 1), (t, b)] + prev[i + 1:]
        prev = cur


@pytest.mark.parametrize("seed", range(25))
def test_sparse_repair_takes_the_best_strict_improvement_each_iteration(seed):
    """One iteration applies the move of one trajectory (out of a nonsingleton microbatch, into a
    capacity-feasible microbatch holding a trajectory within H = 8 global positions) with the
    largest strict decrease of the two microbatches' total work; only when no move improves, the
    best such swap of two trajectories at most H apart; nothing when neither improves."""
    rng = np.random.default_rng(700 + seed)
    ts = _trajs(rng, int(rng.integers(40, 70)), hi=12)
    q = HP.Planner(ts, 1, 10 ** 6)
    # a random grouping of global positions into about N / 3 microbatches, with a capacity a
    # little above the heaviest so that some moves are infeasible
    K = max(2, q.N // 3)
    lab = np.concatenate([np.arange(K), rng.integers(0, K, q.N - K)])
    rng.shuffle(lab)
    groups = [sorted(int(x) for x in np.nonzero(lab == g)[0]) for g in range(K)]
    T = max(_tw(q, g) for g in groups) + int(rng.integers(0, 6))
    p = HP.Planner(ts, 1, T)
    for _ in range(4):
        where = {x: gi for gi, g in enumerate(groups) for x in g}
        best = None
        for x in range(p.N):
            A = where[x]
            if len(groups[A]) < 2:
                continue
            for B, g in enumerate(groups):
                if B == A or not any(abs(y - x) <= HP.H_NEAR for y in g) or _tw(p, g + [x]) > p.T:
                    continue
                rest = [m for m in groups[A] if m != x]
                gain = _tw(p, groups[A]) + _tw(p, g) - _tw(p, rest) - _tw(p, g + [x])
                if gain > 0 and (best is None or gain > best[0]):
                    best = (gain, x, A, B)
        want = [list(g) for g in groups]
        if best is not None:
            _, x, A, B = best
            want[A].remove(x)
            want[B] = sorted(want[B] + [x])
        else:
            for x in range(p.N):
                for y in range(x + 1, min(p.N, x + HP.H_NEAR + 1)):
                    A, B = where[x], where[y]
                    if A == B:
                        continue
                    nA = [m for m in groups[A] if m != x] + [y]
                    nB = [m for m in groups[B] if m != y] + [x]
                    if _tw(p, nA) > p.T or _tw(p, nB) > p.T:
                        continue
                    gain = _tw(p, groups[A]) + _tw(p, groups[B]) - _tw(p, nA) - _tw(p, nB)
                    if gain > 0 and (best is None or gain > best[0]):
                        best = (gain, x, y)
            if best is not None:
                _, x, y = best
                A, B = where[x], where[y]
                want[A] = sorted([m for m in groups[A] if m != x] + [y])
                want[B] = sorted([m for m in groups[B] if m != y] + [x])
        got = p.sparse_repair(groups, iterations=1)
        assert got == want
        if best is None:
            break
        assert sum(_tw(p, g) for g in got) < sum(_tw(p, g) for g in groups)   # strictly better
        assert all(g and _tw(p, g) <= p.T for g in got) and len(got) == len(groups)
        groups = got


@pytest.mark.parametrize("seed", range(25))
def test_boundary_refinement_never_raises_total_then_max(seed):
    """Refinement moves each cut by at most H = 8 positions within two sweeps, keeps K and
    capacity, and every cut it moves lowers the two neighbours' (total, max) work."""
    p, rng = _planner(800 + seed, n_lo=12, n_hi=40, slack=(5, 40))
    K = int(rng.integers(2, max(3, p.N // 2)))
    parts = p.exact(K)
    if parts is None:
        return
    # perturb the cuts so that refinement has something to do
    cuts = [b for _, b in parts[:-1]]
    cuts = sorted({min(p.N - 2, max(0, c + int(rng.integers(-3, 4)))) for c in cuts})
    bounds = [0] + [c + 1 for c in cuts] + [p.N]
    start = [(bounds[i], bounds[i + 1] - 1) for i in range(len(bounds) - 1)]
    if any(_tw(p, list(range(a, b + 1))) > p.T for a, b in start):
        return
    got = p.refine_boundaries(start)
    assert len(got) == len(start) and got[0][0] == 0 and got[-1][1] == p.N - 1
    assert all(got[i][1] + 1 == got[i + 1][0] for i in range(len(got) - 1))
    assert all(_tw(p, list(range(a, b + 1))) <= p.T for a, b in got)
    assert all(abs(g[0] - s[0]) <= 2 * HP.H_NEAR for g, s in zip(got, start))
    # replay the sweeps cut by cut: each change is a strict (total, max) improvement of its pair
    cur = list(start)
    for _ in range(2):
        changed = False
        for i in range(len(cur) - 1):
            a, b = cur[i][0], cur[i + 1][1]
            t0 = cur[i + 1][0]
            key = lambda t: (_tw(p, list(range(a, t))) + _tw(p, list(range(t, b + 1))),
                             max(_tw(p, list(range(a, t))), _tw(p, list(range(t, b + 1)))))
            opts = [t for t in range(max(a + 1, t0 - HP.H_NEAR), min(b, t0 + HP.H_NEAR) + 1)
                    if _tw(p, list(range(a, t))) <= p.T and _tw(p, list(range(t, b + 1))) <= p.T]
            bt = min(opts + [t0], key=lambda t: (key(t), t != t0, t))
            if key(bt) < key(t0):
                cur[i], cur[i + 1] = (a, bt - 1), (bt, b)
                changed = True
        if not changed:
            break
    assert got == cur
    tot = lambda ps: sum(_tw(p, list(range(a, b + 1))) for a, b in ps)
    assert tot(got) <= tot(start)


@pytest.mark.parametrize("seed", range(30))
def test_replica_assignment_puts_heavier_microbatches_on_lighter_replicas(seed):
    """Microbatches sorted by work descending fill consecutive slots of D; within a slot the
    replicas are distinct, and each microbatch, heaviest first, goes to the replica with the
    least cumulative work among those still free in that slot."""
    rng = np.random.default_rng(900 + seed)
    ts = _trajs(rng, int(rng.integers(8, 40)), hi=12)
    D = int(rng.integers(1, 5))
    p = HP.Planner(ts, D, max(len(t) for t in ts) + 20)
    K = D * int(rng.integers(1, max(2, p.N // D)))
    if K > p.N:
        return
    groups = [list(g) for g in np.array_split(rng.permutation(p.N), K)]
    plan = p.assign(groups, "test")
    work = [_tw(p, g) for g in groups]
    assert plan.work == work
    by_slot = [[i for i in range(K) if plan.slot[i] == j] for j in range(K // D)]
    for j, ms in enumerate(by_slot):
        assert len(ms) == D and sorted(plan.replica[i] for i in ms) == list(range(D))
        if j + 1 < len(by_slot):
            assert min(work[i] for i in ms) >= max(work[i] for i in by_slot[j + 1])
    cum = [0] * D
    for ms in by_slot:
        free = set(range(D))
        for i in sorted(ms, key=lambda i: (-work[i], i)):
            r = plan.replica[i]
            assert r in free and cum[r] == min(cum[f] for f in free)
            free.remove(r)
            cum[r] += work[i]


@pytest.mark.parametrize("seed", range(25))
@pytest.mark.parametrize("policy", ["best_fit", "max_shared"])
def test_greedy_placement_policies(seed, policy):
    """Among capacity-feasible microbatches, best-fit picks the largest work after insertion and
    max-shared the largest shared amount |x| - dC; with none feasible a new microbatch opens."""
    p, rng = _planner(1000 + seed, n_lo=8, n_hi=24, slack=(0, 25))
    groups = []
    for x in rng.permutation(p.N):
        gi = p._place(groups, int(x), policy)
        feas = [(i, _tw(p, g + [int(x)])) for i, g in enumerate(groups) if g and _tw(p, g + [int(x)]) <= p.T]
        if not feas:
            assert gi == -1
            groups.append([int(x)])
            continue
        score = {i: (w if policy == "best_fit" else len(p.X[x]) - (w - _tw(p, groups[i]))) for i, w in feas}
        top = max(score.values())
        assert score[gi] == top and gi == min(i for i in score if score[i] == top)
        groups[gi].append(int(x))


def test_sparse_repair_moves_only_next_to_a_near_trajectory():
    """Sec. 3.2: a move's destination must hold a trajectory within H = 8 global positions.
    Twelve trajectories share a 6-token prefix (global positions 0..11); fifteen unrelated ones
    follow (12..26).  Microbatches: A = {0, 26}, B = {11, 25}, five full ones pairing the family's
    1..10 with unrelated 20..24, and 12..19 alone.  Moving 0 into B (or 11 into A) would save 6
    tokens, but both destinations are more than H away; every other move or swap saves nothing,
    so repair leaves the plan as it is.  With 8 in B's place instead of 11, the move is taken."""
    fam = [[1] * 6 + [k] for k in range(12)]
    other = [[2 + i] * 7 for i in range(15)]
    p = HP.Planner(fam + other, 1, 15)
    assert [list(x) for x in p.X] == fam + other
    pairs = [[1, 2, 20], [3, 4, 21], [5, 6, 22], [7, 8, 23], [9, 10, 24]]
    groups = [[0, 26], [11, 25]] + pairs + [[u] for u in range(12, 20)]
    assert [_tw(p, g) for g in groups[:7]] == [14, 14, 15, 15, 15, 15, 15]
    assert p.sparse_repair(groups) == groups
    near = [[0, 26], [8, 25], [1, 2, 20], [3, 4, 21], [5, 6, 22], [7, 11, 23], [9, 10, 24]] + \
        [[u] for u in range(12, 20)]
    got = p.sparse_repair(near, iterations=1)
    assert got[0] == [26] and got[1] == [0, 8, 25] and got[2:] == near[2:]
