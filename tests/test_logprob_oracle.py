"""Pins for the log-probability oracle (HARTS Sec. 3.5 Eq. 17, 19-20).

The semantic map is checked against hand-written position lists for a fork and
for a mount; the log-probabilities against closed forms, against torch's
log_softmax when the map is the identity, against normalisation over the
vocabulary and against shift invariance; the gradient against finite
differences, against torch autograd run on each flat trajectory separately,
and against the zero row-sum that every log-softmax gradient has.
"""
import numpy as np
import pytest
import torch

import synth.dags as D
import synth.tensors as T
from oracle import logprob as LP
from oracle.dag import Dag


def _fork():
    g = D.DagBuilder()
    r = g.node(-1, 5)
    g.node(r, 3)
    g.node(r, 2)
    return g.build()


def _mount():
    g = D.DagBuilder()
    r = g.node(-1, 4)
    a = g.node(r, 3)
    b = g.node(r, 2)
    g.mount(b, a, 1, 3)
    return g.build()


def _rich():
    g = D.DagBuilder()
    r = g.node(-1, 6)
    a = g.node(r, 4)
    b = g.node(r, 0)             # zero-length fork point
    c = g.node(b, 3)
    d = g.node(b, 5)
    e = g.node(a, 2)
    g.node(a, 0)                 # zero-length leaf: its trajectory ends on a's last token
    g.mount(c, a, 0, 3)
    g.mount(d, e, 1, 2)
    g.mount(e, c, 0, 1)
    return g.build()


def test_fork_positions_by_hand():
    dag = Dag(_fork())
    labels = 100 + np.arange(10)
    rows, tg = LP.semantic_positions(dag, labels)
    # leaf a (tokens 5..7) first: 0..6 predict 1..7; then leaf b (8, 9): 0..4 and 8.
    assert rows.tolist() == [0, 1, 2, 3, 4, 5, 6, 0, 1, 2, 3, 4, 8]
    assert tg.tolist() == [101, 102, 103, 104, 105, 106, 107, 101, 102, 103, 104, 108, 109]
    # the fork row 4 serves two positions with different targets
    assert sorted(tg[rows == 4].tolist()) == [105, 108]


def test_mount_positions_by_hand():
    dag = Dag(_mount())
    labels = 50 + np.arange(9)
    rows, tg = LP.semantic_positions(dag, labels)
    # b's flat trajectory: 0 1 2 3 | 5 6 (a's [1, 3), spliced) | 7 8.  Token 3 predicts the
    # spliced token 5; the spliced tokens hold no position; 7 predicts 8.
    assert rows.tolist() == [0, 1, 2, 3, 4, 5, 0, 1, 2, 3, 7]
    assert tg.tolist() == [51, 52, 53, 54, 55, 56, 51, 52, 53, 55, 58]


def test_positions_per_row_plus_terminal_uses_equal_multiplicity():
    spec = _rich()
    dag = Dag(spec)
    rows, _ = LP.semantic_positions(dag, np.zeros(spec.n_tokens, np.int64))
    per_row = np.bincount(rows, minlength=spec.n_tokens)
    terminal = np.zeros(spec.n_tokens, np.int64)
    for leaf in dag.leaves_dfs():
        ids, own = dag.trajectory(leaf)
        if own[-1]:
            terminal[ids[-1]] += 1
    assert np.array_equal(per_row + terminal, dag.multiplicity())


def test_identity_map_is_log_softmax_gather():
    n, V = 12, 37
    g = D.DagBuilder()
    g.node(-1, n)
    dag = Dag(g.build())
    z, labels, _ = T.logprob_inputs(n, V, n, 0, seed=3, dtype=torch.float64, with_grad=False)
    rows, tg = LP.semantic_positions(dag, labels.numpy())
    assert rows.tolist() == list(range(n - 1))
    want = torch.log_softmax(z, dim=-1)[torch.arange(n - 1), labels[1:]]
    np.testing.assert_allclose(LP.logprob(z.numpy(), rows, tg), want.numpy(), rtol=0, atol=1e-14)


def test_uniform_and_two_level_rows():
    V = 50
    z = np.zeros((3, V))
    z[1, 7] = 4.0
    z[2, 9] = -3.0
    lam = LP.logprob(z, np.array([0, 1, 1, 2]), np.array([5, 7, 8, 9]))
    want = [-np.log(V),
            4.0 - np.log(np.exp(4.0) + V - 1),
            0.0 - np.log(np.exp(4.0) + V - 1),
            -3.0 - np.log(np.exp(-3.0) + V - 1)]
    np.testing.assert_allclose(lam, want, rtol=0, atol=1e-14)


def test_shift_invariance_and_normalisation():
    z, _, _ = T.logprob_inputs(4, 23, 1, 0, seed=4, dtype=torch.float64, with_grad=False)
    z = z.numpy()
    rows = np.repeat(np.arange(4), 23)
    tg = np.tile(np.arange(23), 4)
    lam = LP.logprob(z, rows, tg)
    np.testing.assert_allclose(np.exp(lam).reshape(4, 23).sum(axis=1), 1.0, rtol=0, atol=1e-14)
    shift = np.array([[1e3], [-7.0], [0.5], [300.0]])
    np.testing.assert_allclose(LP.logprob(z + shift, rows, tg), lam, rtol=0, atol=1e-11)
    np.testing.assert_allclose(LP.row_lse(z), np.log(np.exp(z).sum(axis=1)), rtol=0, atol=1e-14)


def _rich_case(V=19, seed=6):
    spec = _rich()
    dag = Dag(spec)
    z, labels, _ = T.logprob_inputs(spec.n_tokens, V, spec.n_tokens, 0, seed=seed, dtype=torch.float64,
                                    with_grad=False)
    rows, tg = LP.semantic_positions(dag, labels.numpy())
    g = T.normal((len(rows),), seed, 99, dtype=torch.float64).numpy()
    return spec, dag, z.numpy(), labels.numpy(), rows, tg, g


def test_gradient_matches_finite_differences():
    _, _, z, _, rows, tg, g = _rich_case()
    dz = LP.logprob_grad(z, rows, tg, g)
    rng = np.random.default_rng(0)
    for _ in range(40):
        c, v = int(rng.integers(0, z.shape[0])), int(rng.integers(0, z.shape[1]))
        h = 1e-6
        zp, zm = z.copy(), z.copy()
        zp[c, v] += h
        zm[c, v] -= h
        fd = (g @ LP.logprob(zp, rows, tg) - g @ LP.logprob(zm, rows, tg)) / (2 * h)
        assert abs(fd - dz[c, v]) < 1e-8 * max(1.0, abs(fd)), (c, v, fd, dz[c, v])


def test_gradient_is_sum_of_independent_trajectory_gradients():
    # Each trajectory evaluated on its own flat rows with torch autograd; the
    # compact gradient must be the sum of what every trajectory sends back.
    _, dag, z, labels, rows, tg, g = _rich_case()
    zt = torch.tensor(z, requires_grad=True)
    loss = torch.zeros((), dtype=torch.float64)
    k = 0
    for leaf in dag.leaves_dfs():
        ids, own = dag.trajectory(leaf)
        flat = zt[torch.as_tensor(ids)]                       # the trajectory's own copy of its rows
        lsm = torch.log_softmax(flat, dim=-1)
        for j in range(len(ids) - 1):
            if own[j]:
                loss = loss + float(g[k]) * lsm[j, int(labels[ids[j + 1]])]
                k += 1
    assert k == len(rows)
    loss.backward()
    np.testing.assert_allclose(LP.logprob_grad(z, rows, tg, g), zt.grad.numpy(), rtol=0, atol=1e-13)


def test_gradient_rows_sum_to_zero_and_unused_rows_are_zero():
    spec, _, z, _, rows, tg, g = _rich_case()
    dz = LP.logprob_grad(z, rows, tg, g)
    np.testing.assert_allclose(dz.sum(axis=1), 0.0, rtol=0, atol=1e-13)
    unused = np.setdiff1d(np.arange(spec.n_tokens), rows)
    assert len(unused) > 0
    assert np.all(dz[unused] == 0)


@pytest.mark.parametrize("name", ["config1", "config1_variant"])
def test_map_on_the_small_configurations(name):
    spec = getattr(D, name)()
    dag = Dag(spec)
    labels = np.arange(spec.n_tokens)
    rows, tg = LP.semantic_positions(dag, labels)
    # an own token predicts the next flat token: its successor on the chain or a spliced span's start
    n_traj = len(dag.leaves_dfs())
    assert len(rows) == int(dag.multiplicity().sum()) - n_traj
    assert np.all(tg != rows)
