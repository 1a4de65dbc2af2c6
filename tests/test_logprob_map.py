"""The library's semantic position map (dag_plan_logprob_map) against the oracle's.

Host logic only: positions, targets and the row grouping must equal what the
oracle derives from the flat trajectories, exactly (integer work), on hand-made
trees, the small configurations and random DAGs with mounts, with and without
page shuffling.
"""
import numpy as np
import pytest

import dag_packed_attention_amd as dpa
import synth.dags as D
from oracle import logprob as LP
from oracle.dag import Dag


def _labels(spec, seed, V=1000):
    return np.random.default_rng(seed).integers(0, V, spec.n_tokens)


def _check(spec, seed=0, **kw):
    plan = dpa.Plan(spec, **kw)
    rot, _ = plan.row_maps()
    lab_tok = _labels(spec, seed)
    lab_rows = np.full(plan.rows, -7, np.int32)          # padding rows: never a target
    lab_rows[rot] = lab_tok
    m = plan.logprob_map(lab_rows)
    tok, tg = LP.semantic_positions(Dag(spec, transitive=plan.info["transitive"] != 0), lab_tok)
    assert np.array_equal(m["pos_row"], rot[tok])
    assert np.array_equal(m["pos_target"], tg)
    rf, rp = m["row_first"], m["row_pos"]
    assert rf[0] == 0 and rf[-1] == len(tok) and np.all(np.diff(rf) >= 0)
    assert sorted(rp.tolist()) == list(range(len(tok)))
    for c in range(plan.rows):
        got = rp[rf[c]:rf[c + 1]]
        assert np.array_equal(got, np.flatnonzero(m["pos_row"] == c)), c
    return m


def test_fork_and_mount_by_hand():
    g = D.DagBuilder()
    r = g.node(-1, 4)
    a = g.node(r, 3)
    b = g.node(r, 2)
    g.mount(b, a, 1, 3)
    m = _check(g.build())
    assert len(m["pos_row"]) == 11


@pytest.mark.parametrize("name", ["config1", "config1_variant"])
def test_small_configurations(name):
    _check(getattr(D, name)())


@pytest.mark.parametrize("seed", range(16))
def test_random_dags(seed):
    rng = np.random.default_rng(2000 + seed)
    spec = D.random_tiny_dag(rng, n_nodes=int(rng.integers(1, 14)), max_len=int(rng.integers(1, 90)),
                             p_mount=0.7, max_mounts=3, n_roots=int(rng.integers(1, 3)))
    _check(spec, seed=seed, transitive=bool(seed % 2))
    _check(spec, seed=seed, transitive=bool(seed % 2), page_shuffle=seed + 1)


def test_negative_label_on_a_target_row_is_rejected():
    g = D.DagBuilder()
    g.node(-1, 3)
    plan = dpa.Plan(g.build())
    lab = np.zeros(plan.rows, np.int32)
    rot, _ = plan.row_maps()
    lab[rot[2]] = -1
    with pytest.raises(dpa.DagError) as e:
        plan.logprob_map(lab)
    assert e.value.code == "INVALID"
    lab[rot[2]] = 5
    lab[rot[0]] = -1                 # the first token is never a target
    assert len(plan.logprob_map(lab)["pos_row"]) == 2
