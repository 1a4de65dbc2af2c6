"""Host-side checks of the C library: exported symbols, the compactor against the oracle.

Everything here runs without a GPU: dag_build and the plan queries are host code.
Visibility is compared exactly (as integer sets) with the oracle's own construction.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import synth
import dag_packed_attention_amd as dpa
from oracle.dag import Dag, DagError

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "dag_attn.h")).read()
    declared = set(re.findall(r"^\s*(?:dag_status|void|const char\*)\s+(dag_\w+)\s*\(", hdr, re.M))
    assert {"dag_build", "dag_attn_fwd", "dag_attn_bwd", "dag_last_error"} <= declared
    lib = ctypes.CDLL(dpa.LIB_PATH)
    for name in sorted(declared):
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", dpa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (dag_\w+)$", out, re.M))
    assert declared <= exported


def _compare(spec, transitive=True, shuffle=0, view="mounted"):
    plan = dpa.Plan(spec, transitive=transitive, page_shuffle=shuffle, view=view)
    dag = Dag(spec, transitive=transitive, view=view)
    assert list(plan.starts()) == dag.start
    for u in range(dag.n):
        got = plan.node_ranges(u)
        want = sorted((s, b, e) for s, rs in dag.visible_ranges(u).items() for b, e in rs)
        assert sorted(got) == want, u
        # kernel visiting order: mounted spans first, then ancestors from the root down
        kinds = [s in dag.ancestors[u] for s, _, _ in got]
        assert kinds == sorted(kinds)
        anc = [s for s, _, _ in got if s in dag.ancestors[u]]
        assert anc == [a for a in dag.chain(u)[:-1] if dag.length[a] > 0]
    info = plan.info
    assert info["tokens"] == dag.n_tokens
    assert info["visible_pairs"] == dag.visible_pairs()
    assert info["flat_rows"] == dag.flat_rows()
    assert info["n_trajectories"] == len(dag.leaves_dfs())
    # HARTS Sec. 3.5: per-token multiplicity and S = its sum (own tokens of the flat batch)
    mult = dag.multiplicity()
    assert np.array_equal(plan.multiplicity(), mult)
    assert info["semantic_tokens"] == int(mult.sum())
    assert info["rows"] % 64 == 0 and info["rows"] >= dag.n_tokens
    rot, por = plan.row_maps()
    pos = dag.token_positions()
    assert len(set(rot.tolist())) == dag.n_tokens
    assert np.array_equal(por[rot], pos)
    assert (np.delete(por, rot) == -1).all()
    return plan, dag


@pytest.mark.parametrize("variant", [(16, (16, 32)), (24, (16, 32)), (0, (16, 32)), (16, (16, 16)),
                                     (16, None)])
def test_tiny_variants(variant):
    _compare(synth.config1_variant(*variant))


@pytest.mark.parametrize("seed", range(40))
def test_random_dags(seed):
    rng = np.random.default_rng(1000 + seed)
    spec = synth.random_tiny_dag(rng, n_nodes=int(rng.integers(1, 14)), max_len=int(rng.integers(1, 150)),
                                 p_mount=0.7, max_mounts=3, n_roots=int(rng.integers(1, 3)))
    _compare(spec, transitive=bool(seed % 2), shuffle=seed % 3)


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("view", ["mount_free", "unshifted"])
def test_views_match_the_oracle_and_share_the_row_layout(seed, view):
    rng = np.random.default_rng(5000 + seed)
    spec = synth.random_tiny_dag(rng, n_nodes=int(rng.integers(1, 14)), max_len=int(rng.integers(1, 150)),
                                 p_mount=0.7, max_mounts=3, n_roots=int(rng.integers(1, 3)))
    plan, _ = _compare(spec, transitive=bool(seed % 2), shuffle=seed % 3, view=view)
    assert plan.info["view"] == dpa.VIEWS[view]
    base = dpa.Plan(spec, transitive=bool(seed % 2), page_shuffle=seed % 3)
    assert np.array_equal(plan.row_maps()[0], base.row_maps()[0])      # same rows: tensors are shared


def test_transitive_golden():
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "transitive_mount.json")))
    names = g["nodes"]
    b = synth.DagBuilder()
    for p, ln in zip(g["parent"], g["length"]):
        b.node(p, ln)
    for reader, ms in g["mounts"].items():
        for src, lo, hi in ms:
            b.mount(names.index(reader), names.index(src), lo, hi)
    spec = b.build()
    for tr in (True, False):
        _compare(spec, transitive=tr)


@pytest.mark.parametrize("which", ["w2", "w4", "w3", "short"])
def test_workload_plans(which):
    spec = {"w2": synth.config2, "w4": synth.config4, "w3": synth.config3,
            "short": synth.dags.config3_short_segments}[which]()
    plan, dag = _compare(spec, transitive=bool(spec.meta.get("transitive", True)))
    if which == "w4":
        assert plan.info["tokens"] == 1_081_344


def test_page_shuffle_keeps_rows_consistent():
    spec = synth.config1()
    a, b = dpa.Plan(spec), dpa.Plan(spec, page_shuffle=7)
    ra, pa = a.row_maps()
    rb, pb = b.row_maps()
    assert not np.array_equal(ra, rb)
    assert np.array_equal(pa[ra], pb[rb])


CASES = [
    ([-1, 2, 0], [4, 4, 4], [], "NOT_TOPO"),
    ([-1, 0], [4, -1], [], "INVALID"),
    ([-1, 0, 0], [4, 4, 4], [(2, 1, 0, 5)], "MOUNT_RANGE"),
    ([-1, 0, 0], [4, 4, 4], [(2, 1, 3, 2)], "MOUNT_RANGE"),
    ([-1, 0, 1], [4, 4, 4], [(2, 0, 0, 2)], "SELF_ANCESTOR_MOUNT"),
    ([-1, 0, 1], [4, 4, 4], [(2, 2, 0, 2)], "SELF_ANCESTOR_MOUNT"),
    ([-1, 0, 0], [4, 4, 4], [(1, 2, 0, 2), (2, 1, 0, 2)], "MOUNT_CYCLE"),
    ([-1, 0], [4, 4], [(1, 7, 0, 1)], "INVALID"),
    ([-1, 0, 1], [4, 4, 4], [(2, 0, 2, 2)], None),         # zero-length read: legal no-op
]


@pytest.mark.parametrize("parent,length,mounts,code", CASES)
def test_error_codes_match_oracle(parent, length, mounts, code):
    b = synth.DagBuilder()
    for p, ln in zip(parent, length):
        b.node(p, ln)
    for r, s, lo, hi in mounts:
        b.mount(r, s, lo, hi)
    spec = b.build()
    if code is None:
        dpa.Plan(spec)
        Dag(spec)
        return
    with pytest.raises(dpa.DagError) as e:
        dpa.Plan(spec)
    assert e.value.code == code and dpa.last_error()
    with pytest.raises(DagError) as e2:
        Dag(spec)
    assert e2.value.code == code


def test_empty_dag_and_empty_tokens():
    spec = synth.DagBuilder().build()
    with pytest.raises(dpa.DagError) as e:
        dpa.Plan(spec)
    assert e.value.code == "INVALID"
    b = synth.DagBuilder()
    r = b.node(-1, 0)
    b.node(r, 0)
    plan = dpa.Plan(b.build())
    assert plan.info["rows"] == 0 and plan.info["tokens"] == 0 and plan.info["visible_pairs"] == 0


def test_unsupported_page_size_and_params():
    b = synth.DagBuilder()
    b.node(-1, 5)
    spec = b.build()
    plan = dpa.Plan(spec)
    with pytest.raises(dpa.DagError) as e:
        dpa.workspace_bytes(plan, dpa.AttnParams(3, 2, 64))
    assert e.value.code == "UNSUPPORTED"
    with pytest.raises(dpa.DagError):
        dpa.workspace_bytes(plan, dpa.AttnParams(2, 2, 7))
    f, bw = dpa.workspace_bytes(plan, dpa.AttnParams(16, 4, 128))
    assert f > 0 and bw > f


def test_host_compactor_under_sanitizers(tmp_path):
    """Build plan.cpp with a small driver under ASan/UBSan (g++, host only) and run it."""
    exe = tmp_path / "plan_san"
    src = os.path.join(ROOT, "dag_packed_attention_amd", "csrc", "plan.cpp")
    psrc = os.path.join(ROOT, "dag_packed_attention_amd", "csrc", "pack_plan.cpp")
    gsrc = os.path.join(ROOT, "dag_packed_attention_amd", "csrc", "gdn_plan.cpp")
    csrc = os.path.join(ROOT, "dag_packed_attention_amd", "csrc", "conv_plan.cpp")
    drv = os.path.join(ROOT, "tests", "host", "plan_driver.cpp")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           f"-I{os.path.join(ROOT, 'include')}", src, psrc, gsrc, csrc, drv, "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True)
    r = subprocess.run([str(exe), "300"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout


def test_positions_and_rows_beyond_int32_are_rejected():
    # positions: a 2^30-token child of a 2^30-token root ends at position 2^31
    b = synth.DagBuilder()
    r = b.node(-1, 1 << 30)
    b.node(r, 1 << 30)
    with pytest.raises(dpa.DagError) as e:
        dpa.Plan(b.build())
    assert e.value.code == "OVERFLOW"
    # a mount moves the reader's start past int32 even though its own chain is short
    b = synth.DagBuilder()
    a = b.node(-1, (1 << 31) - 2)
    c = b.node(-1, 1)
    b.mount(c, a, (1 << 31) - 3, (1 << 31) - 2)
    with pytest.raises(dpa.DagError) as e:
        dpa.Plan(b.build())
    assert e.value.code == "OVERFLOW"
    # compact rows: 40 roots of 2^26 tokens need 40 * 2^26 > 2^31 - 1 rows
    b = synth.DagBuilder()
    for _ in range(40):
        b.node(-1, 1 << 26)
    with pytest.raises(dpa.DagError) as e:
        dpa.Plan(b.build())
    assert e.value.code == "OVERFLOW"


def _decode_matches_oracle(spec, transitive, view="mounted", pack=False):
    """Every query row's visible rows and every key row's reader rows, decoded from the plan's
    kernel tables (tile ranges, masks, causal rule; dK/dV reader steps), equal Octopus Eq. 4's
    visible sets from the oracle, mapped to rows."""
    from oracle.attention import AttnParams, RowSampler
    plan = dpa.Plan(spec, transitive=transitive, view=view, pack=pack)
    rs = RowSampler(spec, AttnParams(1, 1), transitive=transitive, view=view)
    rot, _ = plan.row_maps()
    dag = rs.g
    node_of, off = dag.token_node()
    for t in range(dag.n_tokens):
        want = np.sort(rot[dag.visible_tokens(int(node_of[t]), int(off[t]))])
        assert np.array_equal(plan.visibility(int(rot[t])), want), ("visibility", t)
        assert np.array_equal(plan.readers(int(rot[t])), np.sort(rot[rs.readers(t)])), ("readers", t)
    pad = np.setdiff1d(np.arange(plan.rows), rot)
    for r in pad[:50]:
        assert len(plan.visibility(int(r))) == 0 and len(plan.readers(int(r))) == 0
    return plan


@pytest.mark.parametrize("pack", [False, True])
@pytest.mark.parametrize("seed", range(16))
def test_kernel_tables_decode_to_visible_sets(seed, pack):
    rng = np.random.default_rng(5000 + seed)
    spec = synth.random_tiny_dag(rng, n_nodes=int(rng.integers(2, 16)), max_len=int(rng.integers(1, 90)),
                                 p_mount=0.7, max_mounts=3, n_roots=int(rng.integers(1, 3)))
    for transitive in (True, False):
        for view in ("mounted", "mount_free", "unshifted"):
            _decode_matches_oracle(spec, transitive, view, pack)


@pytest.mark.parametrize("pack", [False, True])
def test_kernel_tables_decode_on_short_segment_trees(pack):
    # the page-gather diagnostic's shape in small (segments of 1-64 tokens, most pages shared
    # when packed) and a mini commander-worker episode
    spec = synth.dags.config3_structure(7, n_trees=2, seg=(1, 64), depth_hi=3, fan=(2, 4))
    plan = _decode_matches_oracle(spec, bool(spec.meta.get("transitive", True)), pack=pack)
    if pack:
        assert plan.info["pack_pages"] == 1
        assert plan.rows < 0.5 * dpa.Plan(spec).rows          # most padding gone
    spec = synth.config4(n_episodes=1, commander=150, workers=4, budget=520, span=100, first_read=200,
                         read_step=70)
    _decode_matches_oracle(spec, True, pack=pack)


def test_packed_layout_keeps_rows_and_padding_rules():
    """Packed: every node's rows contiguous, every page's valid rows a prefix, padding only at
    the ends of pages that a longer node could not join; positions and multiplicities as
    unpacked."""
    spec = synth.dags.config3_structure(7, n_trees=2, seg=(1, 64), depth_hi=3, fan=(2, 4))
    a, b = dpa.Plan(spec), dpa.Plan(spec, pack=True)
    ra, pa = a.row_maps()
    rb, pb = b.row_maps()
    assert np.array_equal(pa[ra], pb[rb])                     # same position per token
    assert np.array_equal(a.multiplicity(), b.multiplicity())
    dag = Dag(spec, transitive=bool(spec.meta.get("transitive", True)))
    for u in range(dag.n):
        rows = rb[dag.offset[u]: dag.offset[u] + dag.length[u]]
        assert np.array_equal(rows, rows[0] + np.arange(len(rows))) if len(rows) else True
    valid = (pb >= 0).reshape(-1, 64)
    for pg in valid:                                          # a prefix of each page
        k = int(pg.sum())
        assert pg[:k].all() and not pg[k:].any()
    assert b.info["visible_pairs"] == a.info["visible_pairs"]
