"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test ties the oracle to something other than itself: values printed on
the pages (golden fixtures with citations), hand-derived values, closed forms,
a library routine (torch's scaled_dot_product_attention on CPU in float64),
brute force and finite differences.
"""
import json
import os

import numpy as np
import pytest
import torch

import synth
from oracle.attention import AttnParams, attn_brute, attn_flat, attn_packed_mask, RowSampler
from oracle.dag import Dag, DagError
from oracle.rope import inv_freq, rotate, rotate_transpose

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _inputs(spec, hq, hkv, d, seed):
    q, k, v, do = synth.attn_inputs(spec.n_tokens, hq, hkv, d, seed=seed, dtype=torch.float64)
    return q.numpy(), k.numpy(), v.numpy(), do.numpy()


# ---------------------------------------------------------------- positions


def test_eq2_worked_example():
    g = gold("octopus_eq2_example.json")
    b = synth.DagBuilder()
    root = b.node(-1, g["mounted_first_position"])                 # positions 0..1499
    a = b.node(root, g["mounted_last_position"] - g["mounted_first_position"] + 1)
    pre = b.node(root, g["reader_next_position"] - g["mounted_first_position"])
    post = b.node(pre, 10)
    b.mount(post, a, 0, g["mounted_last_position"] - g["mounted_first_position"] + 1)
    dag = Dag(b.build())
    assert dag.start[pre] + dag.length[pre] == g["reader_next_position"]
    assert dag.start[a] == g["mounted_first_position"]
    assert dag.start[a] + dag.length[a] - 1 == g["mounted_last_position"]
    assert dag.start[post] == g["expected_reader_next_position"]
    lo, hi = g["colliding_positions"]
    assert dag.start[pre] == lo and dag.start[pre] + dag.length[pre] - 1 == hi
    # every visible key is strictly in the reader's past (q - k >= 1)
    pos = dag.token_positions()
    for i in range(dag.length[post]):
        t = dag.offset[post] + i
        keys = dag.visible_tokens(post, i)
        assert np.all(pos[keys[keys != t]] < pos[t])


def test_workload1_hand_values():
    g = gold("workload1_tiny.json")
    dag = Dag(synth.config1())
    assert dag.start == g["start_positions"]
    assert len(dag.visible_tokens(4, 0)) == g["visible_count_first_token_of_b2_post"]
    lens, spliced = [], []
    for leaf in dag.leaves_dfs():
        seq, own = dag.trajectory(leaf)
        lens.append(len(seq))
        spliced.append(int((~own).sum()))
    assert lens == g["trajectory_lengths"]
    assert spliced == g["spliced_rows_per_trajectory"]
    assert dag.n_tokens == g["unique_tokens"]
    assert dag.visible_pairs() == g["visible_pairs"]
    assert dag.flat_rows() == sum(g["trajectory_lengths"])


def test_transitive_mount_hand_values():
    g = gold("transitive_mount.json")
    names = g["nodes"]
    b = synth.DagBuilder()
    for p, ln in zip(g["parent"], g["length"]):
        b.node(p, ln)
    for reader, ms in g["mounts"].items():
        for src, lo, hi in ms:
            b.mount(names.index(reader), names.index(src), lo, hi)
    spec = b.build()
    for transitive, key in ((True, "visible_nonself_of_C_transitive"),
                            (False, "visible_nonself_of_C_direct_only")):
        dag = Dag(spec, transitive=transitive)
        assert dag.start == g["start_positions"]
        vr = dag.visible_ranges(names.index("C"))
        want = {names.index(n): [tuple(r) for r in rs] for n, rs in g[key].items()}
        assert vr == want


def test_harts_fig3_bottom_right_mask():
    g = gold("harts_fig3_mask.json")
    b = synth.DagBuilder()
    p = b.node(-1, 2)          # P0, P1
    b.node(p, 2)               # B0, B1
    spec = b.build()
    from oracle.attention import visibility_mask
    M = visibility_mask(spec)
    cols = [0, 1, 2, 3]
    got = M[[2, 3]][:, cols].astype(int).tolist()
    assert got == g["mask"]
    # Eq. 22: query i of a branch with h ancestor keys sees concatenated index j <= h + i
    h = 2
    for i in range(2):
        assert [j for j in range(4) if M[2 + i, j]] == list(range(h + i + 1))


@pytest.mark.parametrize("seed", range(25))
def test_monotonic_positions_random(seed):
    """Every visible pair has pos_j <= pos_t with equality only at j == t; transitive
    spans never raise Eq. 2's maximum (they lie below their source's start)."""
    rng = np.random.default_rng(seed)
    spec = synth.random_tiny_dag(rng, n_nodes=10, p_mount=0.7)
    dag = Dag(spec)
    pos = dag.token_positions()
    for u in range(dag.n):
        for s, b, e in dag.active[u]:
            assert dag.start[s] + e - 1 < dag.start[u]
        for i in range(dag.length[u]):
            t = dag.offset[u] + i
            keys = dag.visible_tokens(u, i)
            assert np.all(pos[keys[keys != t]] < pos[t])
    assert Dag(spec, transitive=False).start == dag.start


# ---------------------------------------------------------------- validation


def _spec(parent, length, mounts):
    b = synth.DagBuilder()
    for p, ln in zip(parent, length):
        b.node(p, ln)
    for r, s, lo, hi in mounts:
        b.mount(r, s, lo, hi)
    return b.build()


@pytest.mark.parametrize("parent,length,mounts,code", [
    ([-1, 2, 0], [4, 4, 4], [], "NOT_TOPO"),
    ([-1, 0], [4, -1], [], "INVALID"),
    ([-1, 0, 0], [4, 4, 4], [(2, 1, 0, 5)], "MOUNT_RANGE"),
    ([-1, 0, 0], [4, 4, 4], [(2, 1, 3, 2)], "MOUNT_RANGE"),
    ([-1, 0, 1], [4, 4, 4], [(2, 0, 0, 2)], "SELF_ANCESTOR_MOUNT"),
    ([-1, 0, 0], [4, 4, 4], [(1, 2, 0, 2), (2, 1, 0, 2)], "MOUNT_CYCLE"),
    ([-1, 0], [4, 4], [(1, 7, 0, 1)], "INVALID"),
])
def test_validation_codes(parent, length, mounts, code):
    with pytest.raises(DagError) as e:
        Dag(_spec(parent, length, mounts))
    assert e.value.code == code


def test_zero_length_mount_is_legal_anywhere_in_range():
    Dag(_spec([-1, 0, 1], [4, 4, 4], [(2, 0, 2, 2)]))      # would be a self-ancestor read otherwise


# ---------------------------------------------------------------- RoPE (Eq. 1)


def test_rope_phase_depends_on_position_difference():
    rng = np.random.default_rng(0)
    d = 16
    q, k = rng.normal(size=(1, 1, d)), rng.normal(size=(1, 1, d))
    th = inv_freq(d, 10000.0)
    for p, pp in [(5, 2), (100, 3), (7, 7), (3, 40)]:
        lhs = float(rotate(q, np.array([p]), 1e4)[0, 0] @ rotate(k, np.array([pp]), 1e4)[0, 0])
        zq = q[0, 0, : d // 2] + 1j * q[0, 0, d // 2:]
        zk = k[0, 0, : d // 2] + 1j * k[0, 0, d // 2:]
        rhs = float(np.real(np.sum(zq * np.conj(zk) * np.exp(1j * (p - pp) * th))))
        assert abs(lhs - rhs) < 1e-12
    x = rng.normal(size=(3, 2, d))
    pos = np.array([0, 9, 123456])
    assert np.allclose(rotate_transpose(rotate(x, pos, 1e4), pos, 1e4), x, atol=1e-12)
    assert np.array_equal(rotate(x, pos, 0), x)


# ---------------------------------------------------------------- textbook reductions


def _sdpa_chain(q, k, v, do, hq, hkv):
    """torch's SDPA on CPU in float64 for one causal sequence, forward and backward."""
    rep = hq // hkv
    Q = torch.tensor(q).permute(1, 0, 2).requires_grad_()
    K = torch.tensor(k).permute(1, 0, 2).requires_grad_()
    V = torch.tensor(v).permute(1, 0, 2).requires_grad_()
    O = torch.nn.functional.scaled_dot_product_attention(
        Q[None], K.repeat_interleave(rep, 0)[None], V.repeat_interleave(rep, 0)[None],
        is_causal=True)[0]
    O.backward(torch.tensor(do).permute(1, 0, 2))
    t = lambda x: x.detach().permute(1, 0, 2).numpy()
    return t(O), Q.grad.permute(1, 0, 2).numpy(), K.grad.permute(1, 0, 2).numpy(), V.grad.permute(1, 0, 2).numpy()


def test_chain_is_plain_causal_attention():
    spec = _spec([-1, 0, 1], [7, 5, 9], [])
    q, k, v, do = _inputs(spec, 4, 2, 16, seed=5)
    p = AttnParams(4, 2, rope_base=0)
    o, lse, dq, dk, dv = attn_flat(spec, q, k, v, do, p)
    O, dQ, dK, dV = _sdpa_chain(q, k, v, do, 4, 2)
    for a, b in ((o, O), (dq, dQ), (dk, dK), (dv, dV)):
        assert np.abs(a - b).max() < 1e-12


def test_tree_rows_match_causal_attention_per_trajectory():
    """Without mounts, a node's outputs equal plain causal attention over any root-to-leaf
    path through it (HARTS Eq. 21-22)."""
    spec = _spec([-1, 0, 0, 1, 1], [6, 4, 5, 3, 2], [])
    q, k, v, do = _inputs(spec, 2, 1, 8, seed=9)
    p = AttnParams(2, 1, rope_base=0)
    o, *_ = attn_flat(spec, q, k, v, do, p, with_grad=False)
    dag = Dag(spec)
    for leaf in dag.leaves_dfs():
        seq, _ = dag.trajectory(leaf)
        O, *_ = _sdpa_chain(q[seq], k[seq], v[seq], do[seq], 2, 1)
        assert np.abs(O - o[seq]).max() < 1e-12


# ---------------------------------------------------------------- invariants I1-I4


@pytest.mark.parametrize("seed", range(12))
def test_flat_equals_packed_mask_equals_brute(seed):
    rng = np.random.default_rng(100 + seed)
    spec = synth.random_tiny_dag(rng, n_nodes=7, max_len=6, p_mount=0.8)
    hq, hkv = (2, 1) if seed % 2 else (2, 2)
    q, k, v, do = _inputs(spec, hq, hkv, 8, seed=seed)
    p = AttnParams(hq, hkv, rope_base=10000.0 if seed % 3 else 0)
    tr = seed % 4 != 0
    F = attn_flat(spec, q, k, v, do, p, transitive=tr)
    M = attn_packed_mask(spec, q, k, v, do, p, transitive=tr)
    B = attn_brute(spec, q, k, v, do, p, transitive=tr)
    for f, m, b in zip(F, M, B):
        assert np.abs(f - m).max() < 1e-11
        assert np.abs(f - b).max() < 1e-11


def test_shared_row_gradient_is_sum_over_trajectories():
    """I2 with per-semantic-position gradients (HARTS Eq. 20): the compact gradient is the sum
    of what every trajectory containing the row contributes."""
    spec = synth.config1()
    dag = Dag(spec)
    q, k, v, _ = _inputs(spec, 2, 1, 16, seed=3)
    p = AttnParams(2, 1)
    rng = np.random.default_rng(7)
    traj_do, packed_do = {}, np.zeros((dag.n_tokens, 2, 16))
    for leaf in dag.leaves_dfs():
        seq, own = dag.trajectory(leaf)
        g = rng.normal(size=(len(seq), 2, 16)) * own[:, None, None]
        traj_do[leaf] = g
        np.add.at(packed_do, seq, g)
    F = attn_flat(spec, q, k, v, None, p, traj_do=traj_do)
    M = attn_packed_mask(spec, q, k, v, packed_do, p)
    for f, m in zip(F[2:], M[2:]):
        assert np.abs(f - m).max() < 1e-11
    # the multiplicities sum to the number of semantic positions
    assert dag.multiplicity().sum() == sum(int(o.sum()) for o in
                                           (dag.trajectory(l)[1] for l in dag.leaves_dfs()))


def test_zero_length_mount_is_bitwise_noop():
    a = synth.config1_variant(16, (16, 16))
    b = synth.config1_variant(16, None)
    q, k, v, do = _inputs(a, 2, 2, 64, seed=1001)
    p = AttnParams(2, 2)
    for x, y in zip(attn_flat(a, q, k, v, do, p), attn_flat(b, q, k, v, do, p)):
        assert np.array_equal(x, y)


def test_finite_differences():
    spec = _spec([-1, 0, 0, 2], [3, 2, 3, 2], [(3, 1, 0, 2)])
    q, k, v, do = _inputs(spec, 2, 1, 4, seed=11)
    p = AttnParams(2, 1, rope_base=100.0)
    _, _, dq, dk, dv = attn_flat(spec, q, k, v, do, p)

    def loss(q_, k_, v_):
        o, *_ = attn_flat(spec, q_, k_, v_, do, p, with_grad=False)
        return float((o * do).sum())

    rng = np.random.default_rng(1)
    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for _ in range(3):
            args = [q, k, v]
            delta = rng.normal(size=args[which].shape)
            plus = list(args); plus[which] = args[which] + h * delta
            minus = list(args); minus[which] = args[which] - h * delta
            fd = (loss(*plus) - loss(*minus)) / (2 * h)
            assert abs(fd - float((grad * delta).sum())) < 1e-6 * max(1.0, abs(fd))


def test_row_sampler_matches_flat():
    rng = np.random.default_rng(4)
    spec = synth.random_tiny_dag(rng, n_nodes=9, max_len=7, p_mount=0.9)
    q, k, v, do = _inputs(spec, 4, 2, 8, seed=2)
    p = AttnParams(4, 2)
    o, lse, dq, dk, dv = attn_flat(spec, q, k, v, do, p)
    rs = RowSampler(spec, p)
    toks = list(range(0, spec.n_tokens, 3))
    ro, rl = rs.rows(toks, q, k, v)
    assert np.abs(ro - o[toks]).max() < 1e-12 and np.abs(rl - lse[toks]).max() < 1e-12
    rk, rv = rs.key_grads(toks, q, k, v, do)
    assert np.abs(rk - dk[toks]).max() < 1e-11 and np.abs(rv - dv[toks]).max() < 1e-11


@pytest.mark.parametrize("seed", [4, 9, 21])
@pytest.mark.parametrize("transitive", [True, False])
def test_row_grads_match_flat_and_brute(seed, transitive):
    """Per-row o, lse and dq from V(t) alone equal the flat reference and brute force."""
    rng = np.random.default_rng(seed)
    spec = synth.random_tiny_dag(rng, n_nodes=10, max_len=9, p_mount=0.9, max_mounts=2)
    q, k, v, do = _inputs(spec, 4, 2, 8, seed=seed)
    p = AttnParams(4, 2)
    o, lse, dq, _, _ = attn_flat(spec, q, k, v, do, p, transitive=transitive)
    bo, bl, bdq, _, _ = attn_brute(spec, q, k, v, do, p, transitive=transitive)
    rs = RowSampler(spec, p, transitive=transitive)
    toks = list(range(spec.n_tokens))
    ro, rl, rdq = rs.row_grads(toks, q, k, v, do)
    for got, a, b in ((ro, o, bo), (rl, lse, bl), (rdq, dq, bdq)):
        assert np.abs(got - a).max() < 1e-11 and np.abs(got - b).max() < 1e-11
    # the term-size bound: |dq| never exceeds the summed size of its terms
    *_, size = rs.row_grads(toks, q, k, v, do, term_size=True)
    assert (np.abs(rdq) <= size + 1e-12).all()


@pytest.mark.parametrize("seed", [4, 9, 21])
@pytest.mark.parametrize("transitive", [True, False])
def test_key_grads_by_node_match_flat(seed, transitive):
    """Reader-node blocks give every key's dK/dV exactly as the flat reference does, for any
    block size (blocks cut nodes), and fill only the requested KV groups."""
    rng = np.random.default_rng(seed)
    spec = synth.random_tiny_dag(rng, n_nodes=10, max_len=9, p_mount=0.9, max_mounts=2)
    q, k, v, do = _inputs(spec, 4, 2, 8, seed=seed + 1)
    p = AttnParams(4, 2)
    _, _, _, dk, dv = attn_flat(spec, q, k, v, do, p, transitive=transitive)
    rs = RowSampler(spec, p, transitive=transitive)
    toks = list(range(spec.n_tokens))
    for block in (3, 256):
        rk, rv = rs.key_grads_by_node(toks, q, k, v, do, block=block)
        assert np.abs(rk - dk).max() < 1e-11 and np.abs(rv - dv).max() < 1e-11
    sel = toks[::2]
    rk, rv = rs.key_grads_by_node(sel, q, k, v, do, groups=[1])
    assert np.abs(rk[:, 1] - dk[sel, 1]).max() < 1e-11 and np.abs(rv[:, 1] - dv[sel, 1]).max() < 1e-11
    assert not rk[:, 0].any() and not rv[:, 0].any()


def test_reader_nodes_cover_every_reader_token():
    rng = np.random.default_rng(17)
    spec = synth.random_tiny_dag(rng, n_nodes=12, max_len=6, p_mount=0.9, max_mounts=2)
    rs = RowSampler(spec, AttnParams(2, 1))
    node_of, _ = rs.g.token_node()
    for j in range(spec.n_tokens):
        assert sorted(set(int(node_of[t]) for t in rs.readers(j))) == sorted(rs.reader_nodes(j))


def test_workload3_seed_record():
    """The recorded structure seed satisfies its selection rule (checked with the oracle)."""
    rec = gold("workload3_seed.json")
    spec = synth.config3()
    assert spec.meta["seed"] == rec["seed"] and spec.meta["transitive"] == bool(rec["transitive"])
    dag = Dag(spec, transitive=bool(rec["transitive"]))
    assert dag.n_tokens == rec["unique_tokens"]
    assert dag.flat_rows() == rec["flat_rows"]
    assert 192_000 <= dag.n_tokens / 16 <= 320_000 and 5.3 <= rec["ratio"] <= 5.9
