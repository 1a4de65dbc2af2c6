"""Pins for the views of one node/mount table pair (Octopus App. C layer groups;
Octopus Table 5's unshifted regime).

The mount-free view must see exactly what the tree without its mounts sees,
at the mounted view's positions; the unshifted view must see exactly what the
mounted view sees, at the positions of the tree without mounts.  Octopus
Sec. 3.2's worked example fixes the unshifted counterfactual: the reader's next
token stays at 2,000 instead of jumping to 4,001.
"""
import json
import os

import numpy as np
import pytest

import synth
from oracle.attention import AttnParams, attn_brute, attn_flat
from oracle.dag import VIEWS, Dag

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bare(spec):
    b = synth.DagBuilder()
    for p, ln in zip(spec.parent, spec.length):
        b.node(int(p), int(ln))
    return b.build()


def test_worked_example_in_every_view():
    g = json.load(open(os.path.join(GOLDEN, "octopus_eq2_example.json")))
    b = synth.DagBuilder()
    root = b.node(-1, g["mounted_first_position"])
    a = b.node(root, g["mounted_last_position"] - g["mounted_first_position"] + 1)
    pre = b.node(root, g["reader_next_position"] - g["mounted_first_position"])
    post = b.node(pre, 10)
    b.mount(post, a, 0, g["mounted_last_position"] - g["mounted_first_position"] + 1)
    spec = b.build()
    assert Dag(spec, view="mounted").start[post] == g["expected_reader_next_position"]
    assert Dag(spec, view="mount_free").start[post] == g["expected_reader_next_position"]
    assert Dag(spec, view="unshifted").start[post] == g["reader_next_position"]
    n_mounted = g["mounted_last_position"] - g["mounted_first_position"] + 1
    d_m, d_f = Dag(spec, view="mounted"), Dag(spec, view="mount_free")
    assert len(d_m.visible_tokens(post, 0)) - len(d_f.visible_tokens(post, 0)) == n_mounted


@pytest.mark.parametrize("seed", range(20))
def test_views_against_the_tree_without_mounts(seed):
    rng = np.random.default_rng(300 + seed)
    spec = synth.random_tiny_dag(rng, n_nodes=int(rng.integers(2, 12)), max_len=9, p_mount=0.8, max_mounts=3,
                                 n_roots=int(rng.integers(1, 3)))
    transitive = bool(seed % 2)
    mounted = Dag(spec, transitive, "mounted")
    free = Dag(spec, transitive, "mount_free")
    unshifted = Dag(spec, transitive, "unshifted")
    bare = Dag(_bare(spec), transitive)
    assert free.start == mounted.start
    assert unshifted.start == bare.start
    for u in range(mounted.n):
        for i in range(mounted.length[u]):
            assert np.array_equal(free.visible_tokens(u, i), bare.visible_tokens(u, i))
            assert np.array_equal(unshifted.visible_tokens(u, i), mounted.visible_tokens(u, i))
    for leaf in mounted.leaves_dfs():
        ids, own = free.trajectory(leaf)
        assert own.all()                              # nothing is spliced in the mount-free view


def test_views_coincide_without_mounts():
    rng = np.random.default_rng(1)
    spec = synth.random_tiny_dag(rng, n_nodes=9, max_len=9, p_mount=0.0)
    d = [Dag(spec, view=v) for v in VIEWS]
    for x in d[1:]:
        assert x.start == d[0].start and x.active == d[0].active


@pytest.mark.parametrize("view", ["mount_free", "unshifted"])
def test_brute_force_equals_flat_in_each_view(view):
    rng = np.random.default_rng(7)
    spec = synth.random_tiny_dag(rng, n_nodes=7, max_len=7, p_mount=0.9, max_mounts=2)
    q, k, v, do = synth.attn_inputs(spec.n_tokens, 2, 1, 8, seed=4)
    p = AttnParams(2, 1)
    a = attn_flat(spec, q.numpy(), k.numpy(), v.numpy(), do.numpy(), p, view=view)
    b = attn_brute(spec, q.numpy(), k.numpy(), v.numpy(), do.numpy(), p, view=view)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-12)
    m = attn_flat(spec, q.numpy(), k.numpy(), v.numpy(), do.numpy(), p, view="mounted")
    assert not np.allclose(a[0], m[0])                # the view changes the result
