"""The library's trajectory ingestion and microbatch planner against the oracle.

Host only.  The trie must reproduce every trajectory along its leaf's path, hold
exactly C(X) tokens (Eq. 5) and list its leaves in lexicographic order; the
planner must return the oracle's plan exactly (membership, replica, slot and the
objective) in exact mode and in sampled-K mode, and reject what the oracle rejects.
"""
import numpy as np
import pytest

import dag_packed_attention_amd as dpa
from oracle import harts_plan as HP
from oracle.dag import Dag
from oracle.gdn import path_ids
from tests.test_harts_plan_oracle import _trajs


@pytest.mark.parametrize("seed", range(25))
def test_trie_reproduces_trajectories(seed):
    rng = np.random.default_rng(700 + seed)
    ts = _trajs(rng, int(rng.integers(1, 30)), hi=14)
    if seed % 5 == 0:
        ts = ts + [ts[0], []]                          # a repeat and an empty trajectory
    t = dpa.trie_build(ts)
    assert len(t["node_tokens"]) == HP.compact_work(ts) == HP.trie_nodes(ts)
    dag = Dag(t["spec"])
    assert all(t["parent"][u] < u for u in range(len(t["parent"])))
    toks = t["node_tokens"]
    for i, x in enumerate(ts):
        leaf = int(t["leaf_of_traj"][i])
        assert not dag.children[leaf]
        assert toks[path_ids(dag, leaf)].tolist() == list(x)
    assert len(set(t["leaf_of_traj"].tolist())) == len(ts)           # a leaf of its own each
    order = sorted(range(len(ts)), key=lambda i: (ts[i], i))
    assert dag.leaves_dfs() == [int(t["leaf_of_traj"][i]) for i in order]
    plan = dpa.Plan(t["spec"])                                       # the node table builds
    assert plan.tokens == len(toks)


def _canon_lib(r):
    K = len(r["work"])
    groups = [sorted(np.flatnonzero(r["mb_of_traj"] == m).tolist()) for m in range(K)]
    return sorted((tuple(g), int(r["replica"][m]), int(r["slot"][m]), int(r["work"][m])) for m, g in enumerate(groups))


def _canon_oracle(plan):
    return sorted((tuple(g), plan.replica[m], plan.slot[m], plan.work[m]) for m, g in enumerate(plan.groups))


@pytest.mark.parametrize("seed", range(60))
def test_planner_matches_the_oracle(seed):
    rng = np.random.default_rng(800 + seed)
    n = int(rng.integers(1, 60))
    ts = _trajs(rng, n, vocab=int(rng.integers(2, 5)), hi=int(rng.integers(3, 16)))
    D = int(rng.integers(1, 5))
    T = max(len(t) for t in ts) + int(rng.integers(0, 60))
    n0 = [512, 8, 20][seed % 3]                       # exact search, or sampled K with evolution
    try:
        want = HP.Planner(ts, D, T, n0=n0).plan()
    except HP.PlanError:
        with pytest.raises(dpa.DagError):
            dpa.microbatch_plan(ts, D, T, exact_max=n0)
        return
    got = dpa.microbatch_plan(ts, D, T, exact_max=n0)
    assert _canon_lib(got) == _canon_oracle(want)
    info = got["info"]
    assert (info["total_work"], info["slot_critical_work"], info["max_replica_work"]) == want.J
    assert info["exact"] == int(n <= n0)
    assert info["trie_work"] == HP.compact_work(ts)


@pytest.mark.parametrize("D", [1, 2])
def test_many_candidate_ks_are_sampled(D):
    # no shared first tokens and a tight capacity: a K range wider than 32, sampled
    rng = np.random.default_rng(9)
    ts = [[i] + [int(v) for v in rng.integers(0, 5, int(rng.integers(0, 10)))] for i in range(200 * D)]
    p = HP.Planner(ts, D, 10, n0=10)
    ks = p.k_range(len(p.natural_partition()))
    assert len(ks) > 32 and len(p.sample_k(ks)) < len(ks)
    want = p.plan()
    got = dpa.microbatch_plan(ts, D, 10, exact_max=10)
    assert _canon_lib(got) == _canon_oracle(want)


def test_trie_of_a_workload_recovers_its_tree():
    # raw trajectories of a synthetic rollout forest (own tokens along each chain): the
    # trie holds exactly the forest's unique tokens and its plan's rows match them
    import synth
    spec = synth.dags.config3_structure(5, n_trees=3, seg=(40, 200), depth_hi=3, fan=(2, 4), span=(20, 60))
    tok, off = synth.dags.raw_trajectories(spec, 1)
    t = dpa.trie_build((tok, off))
    assert len(t["node_tokens"]) == int(np.sum(spec.length))
    trajs = [tok[off[i]:off[i + 1]].tolist() for i in range(len(off) - 1)]
    assert len(t["node_tokens"]) == HP.compact_work(trajs)
    mb = dpa.microbatch_plan((tok, off), 2, int(np.diff(off).max()) * 2)
    assert mb["info"]["trie_work"] == len(t["node_tokens"])
    assert sorted(np.unique(mb["mb_of_traj"]).tolist()) == list(range(mb["info"]["microbatches"]))
