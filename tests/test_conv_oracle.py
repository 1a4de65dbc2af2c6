"""Pins for the short causal convolution oracle (HARTS Sec. 4.2; Octopus App. C).

A single chain against torch's grouped conv1d and its autograd; a fork and a
zero-length node worked out by hand with decimal taps, forward and backward;
a pure delay; mount invariance; finite differences on a tree with mounts.
"""
import numpy as np
import pytest
import torch

import synth.dags as D
from oracle import conv as CV


def _torch_conv(x, W, act):
    xt = torch.tensor(x.T[None], requires_grad=True)               # [1, Ch, L]
    Wt = torch.tensor(W[:, None, :], requires_grad=True)            # [Ch, 1, w]
    L, w = x.shape[0], W.shape[1]
    pre = torch.nn.functional.conv1d(xt, Wt, padding=w - 1, groups=x.shape[1])[..., :L]
    y = torch.nn.functional.silu(pre) if act == CV.ACT_SILU else pre
    return xt, Wt, y


@pytest.mark.parametrize("w", [1, 2, 3, 4])
@pytest.mark.parametrize("act", [CV.ACT_NONE, CV.ACT_SILU])
def test_chain_matches_torch_conv1d(w, act):
    rng = np.random.default_rng(w + 10 * act)
    L, Ch = 23, 5
    x = rng.standard_normal((L, Ch))
    W = rng.standard_normal((Ch, w))
    dy = rng.standard_normal((L, Ch))
    xt, Wt, y = _torch_conv(x, W, act)
    (y * torch.tensor(dy.T[None])).sum().backward()
    g = D.DagBuilder()
    g.node(-1, L)
    out = CV.conv_flat(g.build(), x, W, act, dy)
    np.testing.assert_allclose(out["y"], y[0].detach().numpy().T, rtol=0, atol=1e-13)
    np.testing.assert_allclose(out["dx"], xt.grad[0].numpy().T, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out["dW"], Wt.grad[:, 0].numpy(), rtol=0, atol=1e-12)


def _fork():
    g = D.DagBuilder()
    r = g.node(-1, 5)
    g.node(r, 2)                 # a
    b = g.node(r, 0)             # zero-length: its child continues r directly
    g.node(b, 1)                 # c
    return g.build()


def test_fork_and_zero_length_node_by_hand():
    # x = 1..5 on the root, 10, 20 on a, 100 on c; taps 1000, 100, 10, 1 (current last)
    x = np.array([1, 2, 3, 4, 5, 10, 20, 100], np.float64)[:, None]
    W = np.array([[1000.0, 100.0, 10.0, 1.0]])
    out = CV.conv_flat(_fork(), x, W, CV.ACT_NONE, np.ones_like(x))
    assert out["y"][:, 0].tolist() == [1, 12, 123, 1234, 2345, 3460, 4620, 3550]
    # dx[t] = sum over every consumer s (itself and up to 3 tokens later on every
    # branch) of the tap that multiplies x_t in y_s
    want_dx = [1111, 1111, 1 + 10 + 100 + 1000 + 1000,  # root 2: r2, r3, r4, a0 and c0
               1 + 10 + 100 + 1000 + 100,              # root 3: r3, r4, a0, a1, c0
               1 + 10 + 100 + 10,                      # root 4: r4, a0, a1, c0
               11, 1, 1]
    assert out["dx"][:, 0].tolist() == want_dx
    # dW[j] = sum over every compact output of its input at tap j
    taps = np.zeros(4)
    win = {0: [0, 0, 0, 1], 1: [0, 0, 1, 2], 2: [0, 1, 2, 3], 3: [1, 2, 3, 4], 4: [2, 3, 4, 5],
           5: [3, 4, 5, 10], 6: [4, 5, 10, 20], 7: [3, 4, 5, 100]}
    for v in win.values():
        taps += v
    assert out["dW"][0].tolist() == taps.tolist()


def test_pure_delay_reads_ancestors():
    spec = _fork()
    x = np.array([1, 2, 3, 4, 5, 10, 20, 100], np.float64)[:, None]
    y = CV.conv_flat(spec, x, np.array([[1.0, 0, 0, 0]]))["y"][:, 0]
    assert y.tolist() == [0, 0, 0, 1, 2, 3, 4, 3]


def _tree_with_mounts():
    g = D.DagBuilder()
    r = g.node(-1, 6)
    a = g.node(r, 2)
    b = g.node(r, 7)
    c = g.node(a, 1)
    d = g.node(c, 4)
    g.node(a, 0)
    e = g.node(b, 3)
    g.mount(b, a, 0, 2)
    g.mount(d, e, 1, 3)
    return g.build()


@pytest.mark.parametrize("act", [CV.ACT_NONE, CV.ACT_SILU])
def test_mounts_do_not_touch_the_convolution(act):
    spec = _tree_with_mounts()
    bare = D.DagBuilder()
    for p, ln in zip(spec.parent, spec.length):
        bare.node(int(p), int(ln))
    rng = np.random.default_rng(1)
    x = rng.standard_normal((spec.n_tokens, 3))
    W = rng.standard_normal((3, 4))
    dy = rng.standard_normal((spec.n_tokens, 3))
    a, b = CV.conv_flat(spec, x, W, act, dy), CV.conv_flat(bare.build(), x, W, act, dy)
    for k in a:
        assert np.array_equal(a[k], b[k])


@pytest.mark.parametrize("act", [CV.ACT_NONE, CV.ACT_SILU])
def test_finite_differences_on_a_tree(act):
    spec = _tree_with_mounts()
    rng = np.random.default_rng(2)
    x = rng.standard_normal((spec.n_tokens, 3))
    W = rng.standard_normal((3, 4))
    dy = rng.standard_normal((spec.n_tokens, 3))
    out = CV.conv_flat(spec, x, W, act, dy)

    def loss(xx, WW):
        return float((CV.conv_flat(spec, xx, WW, act)["y"] * dy).sum())
    h = 1e-6
    for _ in range(12):
        i, c = int(rng.integers(0, spec.n_tokens)), int(rng.integers(0, 3))
        xp, xm = x.copy(), x.copy()
        xp[i, c] += h
        xm[i, c] -= h
        fd = (loss(xp, W) - loss(xm, W)) / (2 * h)
        assert abs(fd - out["dx"][i, c]) < 1e-7 * max(1.0, abs(fd))
    for c in range(3):
        for j in range(4):
            Wp, Wm = W.copy(), W.copy()
            Wp[c, j] += h
            Wm[c, j] -= h
            fd = (loss(x, Wp) - loss(x, Wm)) / (2 * h)
            assert abs(fd - out["dW"][c, j]) < 1e-7 * max(1.0, abs(fd))


def test_compact_gradient_is_sum_over_semantic_positions():
    # Every trajectory position with its own upstream gradient: the compact
    # gradient is the sum over all positions (HARTS Sec. 4.2, several readers of
    # one activation accumulate at its producer).  With the gradients of shared
    # positions moved onto the owning trajectory, the sums agree.
    from oracle.dag import Dag
    from oracle.gdn import path_ids
    spec = _tree_with_mounts()
    dag = Dag(spec)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((spec.n_tokens, 2))
    W = rng.standard_normal((2, 3))
    per = []
    dy = np.zeros((spec.n_tokens, 2))
    for leaf in dag.leaves_dfs():
        ids = path_ids(dag, leaf)
        g = rng.standard_normal((len(ids), 2))
        per.append(g)
        np.add.at(dy, ids, g)
    dx, dW = CV.conv_paths(spec, x, W, CV.ACT_NONE, per)
    out = CV.conv_flat(spec, x, W, CV.ACT_NONE, dy)
    np.testing.assert_allclose(out["dx"], dx, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out["dW"], dW, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(10))
def test_compact_evaluation_equals_per_trajectory(seed):
    rng = np.random.default_rng(40 + seed)
    spec = D.random_tiny_dag(rng, n_nodes=int(rng.integers(2, 12)), max_len=int(rng.integers(1, 9)),
                             p_mount=0.5, max_mounts=2, n_roots=int(rng.integers(1, 3)))
    w = int(rng.integers(1, 5))
    x = rng.standard_normal((spec.n_tokens, 3))
    W = rng.standard_normal((3, w))
    dy = rng.standard_normal((spec.n_tokens, 3))
    for act in (CV.ACT_NONE, CV.ACT_SILU):
        a, b = CV.conv_flat(spec, x, W, act, dy), CV.conv_compact(spec, x, W, act, dy)
        for k in a:
            np.testing.assert_allclose(b[k], a[k], rtol=0, atol=1e-12)
