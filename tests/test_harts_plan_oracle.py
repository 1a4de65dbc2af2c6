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
