"""GPU parity of the compact-to-semantic log-probability kernels against the oracle.

The oracle (float64, expanded rows) and the kernels receive the same logits
(bf16 or fp32) and the same upstream gradients.  Small DAGs with forks, mounts,
zero-length nodes and page shuffling are compared element by element over
every position and every logit; vocabularies cover the 16-byte path, its
remainder loop and the element-wise path (odd V, misaligned base).  Hand-made
maps cover rows with more positions than threads and than the LDS stage, repeated targets on one
row, targets outside the vocabulary and chunked calls.  At the benchmark's
size (65,536 rows of the 16-tree workload's map, V = 131,072) sampled rows are
compared in full.

Tolerances, from the fp32 arithmetic: the vocabulary sum is accumulated per
thread over V / 256 terms and then over a 256-leaf tree, so its relative error
is at most about (V / 256 + 16) 2^-24 plus the exp2 error; lambda is compared
within 8 (V / 256 + 16) 2^-24 + 1e-6 |lambda|.  A gradient entry sums a
softmax term G p (G = the row's sum of g, accumulated in fp32, so its error
scales with sum |g| rather than |G|) and a target term T (the sum of g over
the row's positions with that target): it is compared within
8 (V / 256 + 16) 2^-24 (sum |g|) p + 1e-6 (|value| + sum of |g| in T), plus
2^-8 of its value (half a bf16 ulp) when dz is bf16.
"""
import numpy as np
import pytest
import torch

import synth.dags as D
import synth.tensors as T
from oracle import logprob as LP
from oracle.dag import Dag

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def dpa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dag_packed_attention_amd as m
    return m


def _lam_tol(V, ref):
    return 8 * (V / 256 + 16) * 2.0 ** -24 + 1e-6 * np.abs(ref)


def _dz_tol(V, soft, tabs, ref, bf16):
    t = 8 * (V / 256 + 16) * 2.0 ** -24 * soft + 1e-6 * (np.abs(ref) + tabs) + 1e-30
    return t + (2.0 ** -8 * np.abs(ref) if bf16 else 0.0)


def _check_grad(V, z64, rows, tg, g64, ref, got, bf16):
    # (sum |g| of the row) p[c, v] and the target terms' sum |g|, for the tolerance
    lse = LP.row_lse(z64)
    gabs = np.zeros(z64.shape[0])
    np.add.at(gabs, rows, np.abs(g64))
    soft = gabs[:, None] * np.exp(z64 - lse[:, None])
    tabs = np.zeros_like(z64)
    np.add.at(tabs, (rows, tg), np.abs(g64))
    err = np.abs(got - ref)
    tol = _dz_tol(V, soft, tabs, ref, bf16)
    bad = err > tol
    assert not bad.any(), (int(bad.sum()), float(err.max()), np.argwhere(bad)[:5].tolist())


def _device_map(m):
    return [torch.as_tensor(m[k], device=DEV) for k in ("row_first", "row_pos", "pos_target")]


def _rich():
    g = D.DagBuilder()
    r = g.node(-1, 70)
    a = g.node(r, 40)
    b = g.node(r, 0)
    c = g.node(b, 33)
    d = g.node(b, 65)
    e = g.node(a, 20)
    g.node(a, 0)
    g.node(c, 3)
    g.node(c, 129)
    g.mount(c, a, 0, 30)
    g.mount(d, e, 1, 20)
    g.mount(e, c, 0, 10)
    return g.build(name="lp_rich")


def _dag_case(dpa, spec, V, zdt, gdt, seed, shuffle=0, misalign=False):
    plan = dpa.Plan(spec, page_shuffle=shuffle)
    rot, _ = plan.row_maps()
    C, U = plan.rows, spec.n_tokens
    z_tok, lab, _ = T.logprob_inputs(U, V, U, 0, seed, dtype=zdt, with_grad=False)
    lab_rows = np.full(C, -1, np.int32)
    lab_rows[rot] = lab.numpy()
    m = plan.logprob_map(lab_rows)
    tok, tg = LP.semantic_positions(Dag(spec, transitive=plan.info["transitive"] != 0), lab.numpy())
    assert np.array_equal(m["pos_row"], rot[tok]) and np.array_equal(m["pos_target"], tg)
    n = len(tok)
    g = T.normal((n,), seed, 77)
    # rows with no position (padding, terminal-only rows) hold NaN: they must not be read
    if misalign:
        buf = torch.full((C * V + 1,), float("nan"), dtype=zdt, device=DEV)
        z = buf[1:].view(C, V)
    else:
        z = torch.full((C, V), float("nan"), dtype=zdt, device=DEV)
    used = np.unique(m["pos_row"])
    tok_of_row = np.full(C, -1, np.int64)
    tok_of_row[rot] = np.arange(U)
    z[torch.as_tensor(used, device=DEV)] = z_tok.to(DEV)[torch.as_tensor(tok_of_row[used], device=DEV)]
    rf, rp, pt = _device_map(m)
    lse, lam = dpa.logprob_fwd(z, rf, rp, pt)
    dz = dpa.logprob_bwd(z, lse, rf, rp, pt, g.to(DEV), grad_dtype=gdt)
    torch.cuda.synchronize()
    z64 = z_tok.double().numpy()
    ref_lam = LP.logprob(z64, tok, tg)
    got_lam = lam.cpu().double().numpy()
    assert np.all(np.abs(got_lam - ref_lam) <= _lam_tol(V, ref_lam)), float(np.abs(got_lam - ref_lam).max())
    ref_dz = LP.logprob_grad(z64, tok, tg, g.double().numpy())
    dz_c = dz.double().cpu().numpy()
    _check_grad(V, z64, tok, tg, g.double().numpy(), ref_dz, dz_c[rot], gdt == "bf16")
    unused = np.setdiff1d(np.arange(C), used)
    assert np.all(dz_c[unused] == 0)
    assert np.all(lse.cpu().numpy()[unused] == 0)
    ref_lse = LP.row_lse(z64)[tok_of_row[used]]
    assert np.all(np.abs(lse.cpu().double().numpy()[used] - ref_lse) <= _lam_tol(V, ref_lse))
    return lse, lam, dz


@pytest.mark.parametrize("V,zdt,gdt", [
    (37, torch.bfloat16, "fp32"),        # odd vocabulary: element-wise path
    (64, torch.bfloat16, "bf16"),
    (1000, torch.float32, "fp32"),
    (8200, torch.bfloat16, "bf16"),      # 16-byte path with its remainder loop
    (8192, torch.float32, "bf16"),
])
def test_rich_dag(dpa, V, zdt, gdt):
    print(f"lp rich V={V} z={zdt} dz={gdt}", flush=True)
    _dag_case(dpa, _rich(), V, zdt, gdt, seed=V)


@pytest.mark.parametrize("name", ["config1", "config1_variant"])
def test_small_configurations_with_page_shuffle(dpa, name):
    print(f"lp {name}", flush=True)
    _dag_case(dpa, getattr(D, name)(), 4096, torch.bfloat16, "bf16", seed=11, shuffle=5)


def test_misaligned_logits_take_the_elementwise_path(dpa):
    print("lp misaligned", flush=True)
    _dag_case(dpa, _rich(), 2048, torch.bfloat16, "bf16", seed=12, misalign=True)


def test_random_dags(dpa):
    for seed in range(6):
        rng = np.random.default_rng(500 + seed)
        spec = D.random_tiny_dag(rng, n_nodes=int(rng.integers(2, 12)), max_len=int(rng.integers(1, 120)),
                                 p_mount=0.7, max_mounts=3, n_roots=int(rng.integers(1, 3)))
        print(f"lp random seed={seed}", flush=True)
        _dag_case(dpa, spec, 512 + 8 * seed, torch.bfloat16, "fp32", seed=seed, shuffle=seed)


def _map_from_rows(C, rows, targets):
    rows = np.asarray(rows, np.int32)
    order = np.argsort(rows, kind="stable").astype(np.int32)
    rf = np.zeros(C + 1, np.int32)
    np.add.at(rf, rows + 1, 1)
    return {"row_first": np.cumsum(rf).astype(np.int32), "row_pos": order,
            "pos_target": np.asarray(targets, np.int32)}


def test_crowded_row_repeated_and_invalid_targets(dpa):
    # row 1 holds 700 positions (more than a block's threads) with many repeated
    # targets, row 5 holds 1300 (more than the kernel stages in LDS); two
    # positions target ids outside [0, V).
    print("lp crowded row", flush=True)
    C, V = 6, 3000
    rng = np.random.default_rng(3)
    rows = np.concatenate([np.full(700, 1), [0, 0, 3, 3, 3], [4, 4], np.full(1300, 5)])
    tg = np.concatenate([rng.integers(0, 40, 700), [7, 7, 0, 2999, 0], [V, -3], rng.integers(0, V, 1300)])
    perm = rng.permutation(len(rows))                   # positions in arbitrary batch order
    rows, tg = rows[perm], tg[perm]
    z_cpu, _, _ = T.logprob_inputs(C, V, 1, 0, seed=9, dtype=torch.bfloat16, with_grad=False)
    g = T.normal((len(rows),), 9, 5)
    m = _map_from_rows(C, rows, tg)
    rf, rp, pt = _device_map(m)
    z = z_cpu.to(DEV)
    lse, lam = dpa.logprob_fwd(z, rf, rp, pt)
    dz = dpa.logprob_bwd(z, lse, rf, rp, pt, g.to(DEV), grad_dtype="fp32")
    torch.cuda.synchronize()
    valid = (tg >= 0) & (tg < V)
    z64 = z_cpu.double().numpy()
    lam_c = lam.cpu().double().numpy()
    assert np.all(np.isnan(lam_c[~valid]))
    ref = LP.logprob(z64, rows[valid], tg[valid])
    assert np.all(np.abs(lam_c[valid] - ref) <= _lam_tol(V, ref))
    # an invalid target adds no target term, but its g still weighs the row's softmax term
    ref_dz = LP.logprob_grad(z64, rows[valid], tg[valid], g.double().numpy()[valid])
    lse64 = LP.row_lse(z64)
    for s in np.flatnonzero(~valid):
        ref_dz[rows[s]] -= g.double().numpy()[s] * np.exp(z64[rows[s]] - lse64[rows[s]])
    _check_grad(V, z64, rows, np.where(valid, tg, 0), g.double().numpy(), ref_dz, dz.double().cpu().numpy(), False)
    assert np.all(dz.cpu().numpy()[2] == 0)


def test_chunked_calls_equal_one_call_and_are_deterministic(dpa):
    print("lp chunked", flush=True)
    spec = _rich()
    plan = dpa.Plan(spec)
    C, V = plan.rows, 4096
    lab = np.random.default_rng(1).integers(0, V, C).astype(np.int32)
    m = plan.logprob_map(lab)
    rf, rp, pt = _device_map(m)
    n = len(m["pos_row"])
    z = T.normal((C, V), 3, 1, device=DEV).mul_(3.0).to(torch.bfloat16)
    g = T.normal((n,), 3, 2, device=DEV)
    lse, lam = dpa.logprob_fwd(z, rf, rp, pt)
    dz = dpa.logprob_bwd(z, lse, rf, rp, pt, g)
    lse2, lam2 = dpa.logprob_fwd(z, rf, rp, pt)
    dz2 = dpa.logprob_bwd(z, lse2, rf, rp, pt, g)
    assert torch.equal(lse, lse2) and torch.equal(lam, lam2) and torch.equal(dz, dz2)
    cut = 128
    lse_c = torch.empty_like(lse)
    lam_c = torch.full_like(lam, float("nan"))
    dz_c = torch.empty_like(dz)
    for a, b in ((0, cut), (cut, C)):
        dpa.logprob_fwd(z[a:b], rf[a:b + 1], rp, pt, lse=lse_c[a:b], lam=lam_c)
        dpa.logprob_bwd(z[a:b], lse_c[a:b], rf[a:b + 1], rp, pt, g, dz=dz_c[a:b])
    torch.cuda.synchronize()
    assert torch.equal(lse, lse_c) and torch.equal(lam, lam_c) and torch.equal(dz, dz_c)


def test_benchmark_size_sampled_rows(dpa):
    # The benchmark's launch: the first 65,536 rows of the 16-tree workload's map, V = 131,072.
    print("lp benchmark size", flush=True)
    spec = D.config3()
    plan = dpa.Plan(spec)
    V, CH = 131072, 65536
    lab = np.random.default_rng(21).integers(0, V, plan.rows).astype(np.int32)
    m = plan.logprob_map(lab)
    rf_all, rp, pt = _device_map(m)
    n = len(m["pos_row"])
    rf = rf_all[:CH + 1]
    z = T.normal((CH, V), 21, 1, device=DEV).mul_(2.0).to(torch.bfloat16)
    g = T.normal((n,), 21, 2, device=DEV)
    lse, lam = dpa.logprob_fwd(z, rf, rp, pt)
    dz = dpa.logprob_bwd(z, lse, rf, rp, pt, g)
    torch.cuda.synchronize()
    rfn = m["row_first"]
    counts = np.diff(rfn[:CH + 1])
    rng = np.random.default_rng(4)
    pick = np.concatenate([rng.choice(np.flatnonzero(counts > 0), 40, replace=False),
                           np.flatnonzero(counts == counts.max())[:2], np.flatnonzero(counts == 0)[:2]])
    g_c = g.double().cpu().numpy()
    for c in pick:
        zr = z[c].double().cpu().numpy()[None, :]
        pos = m["row_pos"][rfn[c]:rfn[c + 1]]
        if len(pos) == 0:
            assert lse[c].item() == 0 and torch.all(dz[c] == 0)
            continue
        rows = np.zeros(len(pos), np.int64)
        tg = m["pos_target"][pos].astype(np.int64)
        ref = LP.logprob(zr, rows, tg)
        got = lam[torch.as_tensor(pos, device=DEV)].double().cpu().numpy()
        assert np.all(np.abs(got - ref) <= _lam_tol(V, ref)), (c, float(np.abs(got - ref).max()))
        ref_dz = LP.logprob_grad(zr, rows, tg, g_c[pos])
        _check_grad(V, zr, rows, tg, g_c[pos], ref_dz, dz[c].double().cpu().numpy()[None, :], True)
