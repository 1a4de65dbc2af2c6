"""Pins for the gated-delta-rule oracle and the minimum-call planning oracle.

The recurrence is checked against its unrolled closed form, against the
delta rule's exact key-value memory property, against finite differences, and
against the per-semantic-position gradient identity; the planner against
HARTS Fig. 2 and Appendix A Case I (tests/golden) and against brute force.
"""
import json
import os

import numpy as np
import pytest
import torch

import synth.dags as D
import synth.tensors as T
from oracle import gdn, gdn_plan
from oracle.dag import Dag

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tree():
    g = D.DagBuilder()
    r = g.node(-1, 5)
    a = g.node(r, 3)
    b = g.node(r, 0)            # zero-length node with children: a fork at the same place
    c = g.node(b, 4)
    d = g.node(b, 2)
    e = g.node(a, 3)
    g.node(a, 2)
    g.mount(c, a, 0, 2)
    g.mount(e, d, 1, 2)
    return g.build(name="gdn_tiny")


def _inputs(spec, h=2, dk=6, dv=5, seed=5, decay=0.2):
    q, k, v, b, a, do = T.gdn_inputs(spec.n_tokens, h, dk, dv, seed, decay_scale=decay)
    return [x.double().numpy() for x in (q, k, v, b, a, do)]


def test_recurrence_matches_unrolled_closed_form():
    q, k, v, b, a, _ = _inputs(D.config1_variant(), h=2, dk=5, dv=4)
    ids = np.arange(14)
    o, _ = gdn.recur(ids, q, k, v, b, a, scale=0.6)
    np.testing.assert_allclose(o, gdn.gdn_unrolled(ids, q, k, v, b, a, scale=0.6), atol=1e-13)


def test_delta_rule_stores_latest_value_per_orthonormal_key():
    # alpha = beta = 1 with orthonormal keys: writing (k_i, v_i) replaces the value
    # stored under k_i, so reading with q = k_j returns the last v written at j.
    rng = np.random.default_rng(0)
    d, L = 6, 20
    basis = np.linalg.qr(rng.standard_normal((d, d)))[0]
    key_of = rng.integers(0, d, L)
    k = basis[key_of][:, None, :]
    q = basis[rng.integers(0, d, L)][:, None, :]
    v = rng.standard_normal((L, 1, 3))
    ones = np.ones((L, 1))
    o, _ = gdn.recur(np.arange(L), q, k, v, ones, ones)
    for t in range(L):
        j = int(np.argmax(np.abs(basis @ q[t, 0])))
        last = [i for i in range(t + 1) if key_of[i] == j]
        want = v[last[-1], 0] if last else np.zeros(3)
        np.testing.assert_allclose(o[t, 0], want, atol=1e-12)


def test_decay_only_scales_the_state():
    # beta = 0 after the first token: the state only decays, o_t = prod(alpha) * o_1-state read.
    rng = np.random.default_rng(1)
    L, d = 7, 4
    q = np.repeat(rng.standard_normal((1, 1, d)), L, 0)
    k = rng.standard_normal((L, 1, d))
    v = rng.standard_normal((L, 1, 3))
    b = np.zeros((L, 1))
    b[0] = 0.7
    a = rng.uniform(0.5, 1.0, (L, 1))
    o, _ = gdn.recur(np.arange(L), q, k, v, b, a)
    s1 = a[0, 0] * 0 + 0.7 * np.outer(v[0, 0], k[0, 0])
    for t in range(L):
        np.testing.assert_allclose(o[t, 0], np.prod(a[1:t + 1, 0]) * s1 @ q[0, 0], atol=1e-13)


def test_finite_differences_on_a_tree():
    spec = _tree()
    q, k, v, b, a, do = _inputs(spec)
    out = gdn.gdn_flat(spec, q, k, v, b, a, do, scale=0.9)
    ins = {"q": q, "k": k, "v": v, "beta": b, "alpha": a}

    def loss(**kw):
        x = dict(ins)
        x.update(kw)
        return float((gdn.gdn_flat(spec, x["q"], x["k"], x["v"], x["beta"], x["alpha"], scale=0.9)["o"]
                      * do).sum())

    rng = np.random.default_rng(2)
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("beta", "dbeta"), ("alpha", "dalpha")):
        for _ in range(6):
            base = ins[name]
            idx = tuple(int(rng.integers(0, s)) for s in base.shape)
            h = 1e-6
            xp, xm = base.copy(), base.copy()
            xp[idx] += h
            xm[idx] -= h
            fd = (loss(**{name: xp}) - loss(**{name: xm})) / (2 * h)
            assert abs(fd - out[key][idx]) < 1e-7 * max(1.0, abs(fd)), (name, idx, fd, out[key][idx])


def test_compact_gradient_is_sum_over_semantic_positions():
    # HARTS Eq. 19-20 for a recurrent layer: each trajectory position s has its own
    # upstream gradient g_s; the compact row's gradient is the sum over its uses.
    spec = _tree()
    q, k, v, b, a, _ = _inputs(spec)
    dag = Dag(spec)
    rng = np.random.default_rng(3)
    dO = np.zeros((spec.n_tokens, 2, 5))
    want = {n: 0.0 for n in ("dq", "dk", "dv", "dbeta", "dalpha")}
    for leaf in dag.leaves_dfs():
        ids = gdn.path_ids(dag, leaf)
        g_s = rng.standard_normal((len(ids), 2, 5))
        np.add.at(dO, ids, g_s)
        _, g = gdn.recur(ids, q, k, v, b, a, g_s)
        for n in want:
            acc = np.zeros_like({"dq": q, "dk": k, "dv": v, "dbeta": b, "dalpha": a}[n])
            np.add.at(acc, ids, g[n])
            want[n] = want[n] + acc
    got = gdn.gdn_flat(spec, q, k, v, b, a, dO)
    for n in want:
        np.testing.assert_allclose(got[n], want[n], atol=1e-12)


def test_mounts_do_not_touch_the_recurrence():
    spec = _tree()
    bare = D.DagBuilder()
    for p, ln in zip(spec.parent, spec.length):
        bare.node(int(p), int(ln))
    q, k, v, b, a, do = _inputs(spec)
    x = gdn.gdn_flat(spec, q, k, v, b, a, do)
    y = gdn.gdn_flat(bare.build(), q, k, v, b, a, do)
    for n in x:
        assert np.array_equal(x[n], y[n])


def test_recurrent_index_skips_mounted_spans():
    spec = D.config1()                  # b2's post-read node starts at Eq. 2 position 96
    idx = gdn.recurrent_index(spec)
    dag = Dag(spec)
    post = 4
    assert dag.start[post] == 96
    assert idx[dag.offset[post]] == 80   # own tokens along root -> pre -> post: 64 + 16
    assert list(idx[:64]) == list(range(64))


# -- planner ---------------------------------------------------------------------

def _golden_plan(name):
    d = json.load(open(os.path.join(GOLDEN, name)))
    g = D.DagBuilder()
    idx = {}
    for s in d["segments"]:
        idx[s["name"]] = g.node(-1 if s["parent"] is None else idx[s["parent"]], s["tokens"])
    return d, g.build(name=name)


@pytest.mark.parametrize("name", ["harts_fig2_plan.json", "harts_case1_plan.json", "harts_case2_plan.json",
                                  "harts_case3_plan.json"])
def test_planner_reproduces_the_pages_examples(name):
    d, spec = _golden_plan(name)
    B = d["chunk"]
    segs = gdn_plan.segments(spec)
    seg_name = {i: d["segments"][s.nodes[0]]["name"] for i, s in enumerate(segs)}
    t_pre, _ = gdn_plan.min_calls(segs, B)
    assert t_pre[0] == d["calls"]
    assert gdn_plan.replay_total(segs, B) == d["replay_total"]
    seqs = gdn_plan.recover(segs, B)
    got = {}
    for s in seqs:
        got.setdefault(str(s.round), []).append(([seg_name[v] for v in s.segs], s.replay[1] - s.replay[0]))
    for call, mem in d["members"].items():
        assert sorted(got[call]) == sorted((m["chain"], m["replay"]) for m in mem), call
    assert set(got) == set(d["members"])
    for s in d["segments"]:
        r = [q.round for q in seqs if any(seg_name[v] == s["name"] for v in q.segs)]
        assert r == [s["call"]], s["name"]


def test_planner_on_fig3_fork_inside_a_chunk():
    # HARTS Fig. 3(a)-(b): the shared path P0-P1 forks into A, B, C after P1, inside a
    # chunk; A continues directly (round 1: P0-P1-A), and B and C run together in
    # round 2, each replaying P1 from the state H0 at the chunk boundary after P0.  The
    # figure prints no sizes: P0 is one chunk and P1 ten tokens of the next.
    B = 64
    g = D.DagBuilder()
    p = g.node(-1, B + 10)
    for n in (20, 30, 40):
        g.node(p, n)
    segs = gdn_plan.segments(g.build())
    t_pre, _ = gdn_plan.min_calls(segs, B)
    assert t_pre[0] == 2
    seqs = gdn_plan.recover(segs, B)
    assert [(s.round, s.segs, s.replay) for s in seqs] == [(1, [0, 1], (0, 0)), (2, [2], (B, B + 10)),
                                                            (2, [3], (B, B + 10))]
    assert seqs[1].init == seqs[2].init == (0, B)       # H0: exported by round 1 at the boundary after P0
    assert gdn_plan.replay_total(segs, B) == 20


def _random_tree(rng, n=9, max_len=9):
    g = D.DagBuilder()
    for u in range(n):
        g.node(-1 if u == 0 else int(rng.integers(0, u)), 0 if rng.random() < 0.1 else int(rng.integers(1, max_len + 1)))
    return g.build()


@pytest.mark.parametrize("seed", range(40))
def test_minimum_calls_equal_brute_force(seed):
    rng = np.random.default_rng(seed)
    spec = _random_tree(rng)
    segs = gdn_plan.segments(spec)
    B = 4
    t_pre, _ = gdn_plan.min_calls(segs, B)
    seqs = gdn_plan.recover(segs, B)
    roots = [i for i, s in enumerate(segs) if s.parent < 0]
    assert max(t_pre[r] for r in roots) == gdn_plan.brute_force_calls(segs, B)
    assert max(s.round for s in seqs) == max(t_pre[r] for r in roots)


@pytest.mark.parametrize("seed", range(40))
def test_recovered_plan_is_valid(seed):
    rng = np.random.default_rng(100 + seed)
    spec = _random_tree(rng, n=12)
    B = 4
    segs = gdn_plan.segments(spec)
    seqs = gdn_plan.recover(segs, B)
    seen = [0] * len(segs)
    for qi, s in enumerate(seqs):
        for x, y in zip(s.segs, s.segs[1:]):
            assert segs[y].parent == x                    # a sequence is a path of direct continuations
        for v in s.segs:
            seen[v] += 1
        first = segs[s.segs[0]]
        if first.parent < 0:
            assert s.init is None and s.replay == (0, 0) and s.round == 1
            continue
        fork = segs[first.parent].e
        assert s.replay == (B * (fork // B), fork)        # fixed replay [a(e_v), e_v)
        assert s.start == B * (fork // B)
        if s.init is not None:
            prod, bnd = s.init
            assert bnd % B == 0
            if bnd == s.start and seqs[prod].round < s.round:
                assert seqs[prod].start < bnd             # exported strictly inside the producer's call
    assert seen == [1] * len(segs)
    assert sum(s.replay[1] - s.replay[0] for s in seqs) == gdn_plan.replay_total(segs, B)


def test_minimum_calls_do_not_depend_on_child_order():
    rng = np.random.default_rng(7)
    for _ in range(10):
        spec = _random_tree(rng, n=10)
        segs = gdn_plan.segments(spec)
        t0 = gdn_plan.min_calls(segs, 4)[0][0]
        # same tree with children stored in reverse table order
        n = spec.n_nodes
        order = [0]
        kids = {u: [c for c in range(n) if spec.parent[c] == u] for u in range(n)}
        stack = [0]
        order = []
        while stack:
            u = stack.pop()
            order.append(u)
            stack.extend(kids[u])                         # pushes in order, pops reversed
        newid = {u: i for i, u in enumerate(order)}
        g = D.DagBuilder()
        for u in order:
            g.node(-1 if spec.parent[u] < 0 else newid[int(spec.parent[u])], int(spec.length[u]))
        segs2 = gdn_plan.segments(g.build())
        assert gdn_plan.min_calls(segs2, 4)[0][0] == t0
        assert gdn_plan.replay_total(segs2, 4) == gdn_plan.replay_total(segs, 4)
