"""The library's linear-attention schedule against the planning oracle (host only)."""
import json
import os

import numpy as np
import pytest

import dag_packed_attention_amd as dpa
import synth.dags as D
from oracle import gdn_plan

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _expected(spec, B):
    segs = gdn_plan.segments(spec)
    seqs = gdn_plan.recover(segs, B)
    out = []
    for s in seqs:
        out.append({"round": s.round, "first_node": segs[s.segs[0]].nodes[0],
                    "last_node": segs[s.segs[-1]].nodes[-1], "start": s.start,
                    "fork": s.replay[1] if s.init is not None or s.replay != (0, 0) else 0,
                    "own_tokens": sum(int(spec.length[u]) for v in s.segs for u in segs[v].nodes),
                    "init_seq": -1 if s.init is None else s.init[0],
                    "init_boundary": -1 if s.init is None else s.init[1]})
    t_pre, _ = gdn_plan.min_calls(segs, B)
    roots = [i for i, s in enumerate(segs) if s.parent < 0]
    return out, segs, (max(t_pre[r] for r in roots) if roots else 0)


def _check(spec, B, transitive=None):
    plan = dpa.Plan(spec, transitive=transitive, gdn_chunk=B)
    want, segs, calls = _expected(spec, B)
    got = plan.gdn_seqs()
    assert got == want
    info = plan.info
    assert info["gdn_chunk"] == B
    assert info["gdn_rounds"] == calls
    assert info["gdn_replay"] == gdn_plan.replay_total(segs, B)
    assert info["gdn_segments"] == len(segs)
    assert info["gdn_sequences"] == len(want)
    return plan, got


def _golden(name):
    d = json.load(open(os.path.join(GOLDEN, name)))
    g = D.DagBuilder()
    idx = {}
    for s in d["segments"]:
        idx[s["name"]] = g.node(-1 if s["parent"] is None else idx[s["parent"]], s["tokens"])
    return d, g.build(name=name)


@pytest.mark.parametrize("name", ["harts_fig2_plan.json", "harts_case1_plan.json", "harts_case2_plan.json",
                                  "harts_case3_plan.json"])
def test_schedule_on_the_pages_examples(name):
    d, spec = _golden(name)
    plan, got = _check(spec, d["chunk"])
    assert plan.info["gdn_rounds"] == d["calls"]
    assert plan.info["gdn_replay"] == d["replay_total"]


def test_schedule_on_fig3_fork_inside_a_chunk():
    # HARTS Fig. 3(b): B and C start in round 2 from the boundary state after P0 and
    # replay P1 (P0 one chunk, P1 ten tokens of the next; the figure prints no sizes)
    g = D.DagBuilder()
    p = g.node(-1, 74)
    for n in (20, 30, 40):
        g.node(p, n)
    plan = dpa.Plan(g.build(), gdn_chunk=64)
    seqs = plan.gdn_seqs()
    assert plan.info["gdn_rounds"] == 2 and plan.info["gdn_replay"] == 20
    side = [s for s in seqs if s["round"] == 2]
    assert len(side) == 2
    for s in side:
        assert (s["start"], s["fork"], s["init_boundary"]) == (64, 74, 64)
        assert seqs[s["init_seq"]]["round"] == 1


@pytest.mark.parametrize("seed", range(30))
@pytest.mark.parametrize("B", [1, 4, 64])
def test_schedule_matches_oracle_on_random_dags(seed, B):
    rng = np.random.default_rng(seed)
    spec = D.random_tiny_dag(rng, n_nodes=int(rng.integers(1, 14)), max_len=int(rng.integers(1, 90)),
                             n_roots=int(rng.integers(1, 3)))
    _check(spec, B)


def test_schedule_ignores_mounts():
    spec = D.config1()
    bare = D.DagBuilder()
    for p, ln in zip(spec.parent, spec.length):
        bare.node(int(p), int(ln))
    a = dpa.Plan(spec, gdn_chunk=64).gdn_seqs()
    b = dpa.Plan(bare.build(), gdn_chunk=64).gdn_seqs()
    assert a == b


def test_schedule_on_the_sixteen_tree_workload():
    spec = D.config3()
    plan, got = _check(spec, 64)
    info = plan.info
    assert info["gdn_rounds"] >= 2
    # every own token of the tree is in exactly one sequence
    assert sum(s["own_tokens"] for s in got) == info["tokens"]


def test_schedule_bounds():
    with pytest.raises(dpa.DagError):
        dpa.Plan(D.config1(), gdn_chunk=-1)
    with pytest.raises(dpa.DagError):
        dpa.Plan(D.config1()).gdn_seqs()


def test_kept_states_workspace_and_flag():
    plan = dpa.Plan(D.config1(), gdn_chunk=64)
    f0, b0 = dpa.gdn_workspace_bytes(plan, dpa.GdnParams(2))
    fk, bk = dpa.gdn_workspace_bytes(plan, dpa.GdnParams(2, keep_states=True))
    assert f0 < b0 and fk == bk == b0          # the forward fills the backward's state region
    p = dpa.GdnParams(2)
    cp = p.c()
    cp.keep_states = 2
    import ctypes
    f, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert dpa._lib.dag_gdn_workspace(plan._h, ctypes.byref(cp), ctypes.byref(f), ctypes.byref(b)) != 0
