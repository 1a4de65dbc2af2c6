"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small inputs are compared element by element with the oracle's flat
per-trajectory attention (float64).  Full-size workloads, in the launch
configuration the benchmark times, are compared on sampled query rows
(outputs and lse) and sampled key rows (dK, dV) that the oracle evaluates one
by one, plus properties that hold at any size.  Padding rows of every input
are filled with NaN to show that they are ignored.

Tolerances: bf16 inputs, max-abs <= 2e-2 and mean-abs <= 2e-3 per tensor;
fp32 mode, max-abs <= 1e-5 on the tiny workload, and 1e-5 * max(1, max|ref|)
on larger DAGs, whose shared rows sum many fp32 terms (|dV| reaches ~11).
"""
import numpy as np
import pytest
import torch

import synth
from oracle.attention import AttnParams as OParams, attn_brute, attn_flat, RowSampler
from oracle.dag import Dag

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, FP32_MAX = 2e-2, 2e-3, 1e-5
DEV = "cuda"


@pytest.fixture(scope="module")
def dpa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dag_packed_attention_amd as m
    return m


def _run(dpa, spec, q, k, v, do, hq, hkv, d, dtype, rope=10000.0, transitive=None, shuffle=0, bwd=True,
         scale=0.0, grad="fp32", view="mounted"):
    """Token-major CPU tensors in, token-major CPU float64 results out (via the row layout).

    Gradients come back in fp32 by default: in these small DAGs a shared row's dK/dV reaches
    magnitudes (~11) where bf16 storage alone is 0.03 away from the exact value.
    """
    plan = dpa.Plan(spec, transitive=transitive, page_shuffle=shuffle, view=view)
    p = dpa.AttnParams(hq, hkv, d, dtype, scale=scale, rope_base=rope, grad_dtype=grad)
    tdt = p.torch_dtype
    rows = lambda x: dpa.to_rows(plan, x.to(DEV, tdt), fill=float("nan"))
    qr, kr, vr = rows(q), rows(k), rows(v)
    o_lo = None
    if dtype == "bf16":
        o, lse, o_lo = dpa.attn_fwd(plan, p, qr, kr, vr, o_lo=True)
    else:
        o, lse = dpa.attn_fwd(plan, p, qr, kr, vr)
    out = {"o": o, "lse": lse}
    if bwd:
        dor = rows(do)
        dq, dk, dv = dpa.attn_bwd(plan, p, qr, kr, vr, o, lse, dor, o_lo=o_lo)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    rot, _ = plan.row_maps()
    pad = np.setdiff1d(np.arange(plan.rows), rot)
    for name, t in out.items():
        if len(pad):
            assert torch.all(t[torch.as_tensor(pad, device=DEV)] == 0), f"{name}: padding rows not zero"
    res = {n: dpa.from_rows(plan, t).double().cpu().numpy() for n, t in out.items()}
    return res, plan


def _ref(spec, q, k, v, do, hq, hkv, rope=10000.0, transitive=True, brute=False, bwd=True, scale=None,
         view="mounted"):
    p = OParams(hq, hkv, scale=scale, rope_base=rope)
    args = [x.double().numpy() for x in (q, k, v)] + [do.double().numpy() if do is not None else None]
    if brute:
        o, lse, dq, dk, dv = attn_brute(spec, *args, p, transitive=transitive, view=view)
    else:
        o, lse, dq, dk, dv = attn_flat(spec, *args, p, transitive=transitive, with_grad=bwd, view=view)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def _assert_close(got, ref, dtype, names=("o", "lse", "dq", "dk", "dv"), tag="", fp32_relative=False):
    for n in names:
        if n not in got:
            continue
        err = np.abs(got[n] - ref[n])
        assert np.isfinite(got[n]).all(), f"{tag} {n}: non-finite"
        if dtype == "fp32":
            bar = FP32_MAX * (max(1.0, float(np.abs(ref[n]).max())) if fp32_relative else 1.0)
            assert err.max() <= bar, f"{tag} {n}: max {err.max():.3g} > {bar:.3g}"
        else:
            assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, \
                f"{tag} {n}: max {err.max():.3g} mean {err.mean():.3g}"


def _inputs(spec, hq, hkv, d, seed, dtype):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v, do = synth.attn_inputs(spec.n_tokens, hq, hkv, d, seed=seed, dtype=tdt)
    return q, k, v, do


# ---------------------------------------------------------------- workload 1: tiny, fp32


@pytest.mark.parametrize("variant", [(16, (16, 32)), (24, (16, 32)), (0, (16, 32)), (16, (16, 16)),
                                     (16, None)])
def test_tiny_fp32_vs_brute(dpa, variant):
    spec = synth.config1_variant(*variant)
    q, k, v, do = _inputs(spec, 2, 2, 64, 1001, "fp32")
    got, _ = _run(dpa, spec, q, k, v, do, 2, 2, 64, "fp32")
    ref = _ref(spec, q, k, v, do, 2, 2, brute=True)
    _assert_close(got, ref, "fp32", tag=f"tiny{variant}")


def test_tiny_zero_length_mount_is_bitwise_noop_on_device(dpa):
    a = synth.config1_variant(16, (16, 16))
    b = synth.config1_variant(16, None)
    q, k, v, do = _inputs(a, 2, 2, 64, 1001, "fp32")
    ga, _ = _run(dpa, a, q, k, v, do, 2, 2, 64, "fp32")
    gb, _ = _run(dpa, b, q, k, v, do, 2, 2, 64, "fp32")
    for n in ga:
        assert np.array_equal(ga[n], gb[n]), n
    q, k, v, do = _inputs(a, 16, 4, 128, 1001, "bf16")
    ga, _ = _run(dpa, a, q, k, v, do, 16, 4, 128, "bf16")
    gb, _ = _run(dpa, b, q, k, v, do, 16, 4, 128, "bf16")
    for n in ga:
        assert np.array_equal(ga[n], gb[n]), n


# ---------------------------------------------------------------- small bf16 cases, full comparison


def _mini_trees2():
    rng = np.random.default_rng(11)
    g = synth.DagBuilder()
    for _ in range(2):
        root = g.node(-1, 200)
        for _ in range(3):
            c = g.node(root, int(rng.integers(60, 200)))
            for _ in range(2):
                g.node(c, int(rng.integers(60, 200)))
    return g.build(name="mini-trees")


def _mini3(seed=5):
    return synth.dags.config3_structure(seed, n_trees=2, seg=(40, 260), depth_hi=3, fan=(2, 3), span=(20, 180))


def _mini4():
    return synth.config4(n_episodes=1, commander=150, workers=4, budget=520, span=100, first_read=200,
                         read_step=70)


def _mini_short():
    # the page-gather diagnostic's shape in small: segments of 1-64 tokens, most pages
    # partly padding, reads clipped to whole sources
    return synth.dags.config3_structure(7, n_trees=2, seg=(1, 64), depth_hi=3, fan=(2, 4))


SMALL = {"mini2": _mini_trees2, "mini3": _mini3, "mini4": _mini4, "tiny": synth.config1,
         "mini_short": _mini_short}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_bf16_mfma_path(dpa, name):
    spec = SMALL[name]()
    tr = bool(spec.meta.get("transitive", True))
    q, k, v, do = _inputs(spec, 16, 4, 128, 2000 + len(name), "bf16")
    got, _ = _run(dpa, spec, q, k, v, do, 16, 4, 128, "bf16", transitive=tr)
    ref = _ref(spec, q, k, v, do, 16, 4, transitive=tr)
    _assert_close(got, ref, "bf16", tag=name)


@pytest.mark.parametrize("view", ["mount_free", "unshifted"])
@pytest.mark.parametrize("name", ["mini3", "mini4"])
def test_layer_group_views_on_device(dpa, name, view):
    # Octopus App. C layer groups and Table 5's unshifted regime: plans of the same
    # tables in another view, run on the same row-layout tensors
    spec = SMALL[name]()
    tr = bool(spec.meta.get("transitive", True))
    print(f"view {view} {name}", flush=True)
    q, k, v, do = _inputs(spec, 16, 4, 128, 3000 + len(name), "bf16")
    got, plan = _run(dpa, spec, q, k, v, do, 16, 4, 128, "bf16", transitive=tr, view=view)
    assert plan.info["view"] == dpa.VIEWS[view]
    ref = _ref(spec, q, k, v, do, 16, 4, transitive=tr, view=view)
    _assert_close(got, ref, "bf16", tag=f"{name}/{view}")


@pytest.mark.parametrize("view", ["mount_free", "unshifted"])
def test_tiny_views_fp32_vs_brute(dpa, view):
    spec = synth.config1()
    q, k, v, do = _inputs(spec, 2, 2, 64, 1001, "fp32")
    got, _ = _run(dpa, spec, q, k, v, do, 2, 2, 64, "fp32", view=view)
    ref = _ref(spec, q, k, v, do, 2, 2, brute=True, view=view)
    _assert_close(got, ref, "fp32", tag=f"tiny/{view}")


@pytest.mark.parametrize("name", ["mini3", "tiny"])
@pytest.mark.parametrize("shape", [(4, 2, 64, "bf16"), (4, 4, 32, "fp32"), (8, 2, 128, "bf16")])
def test_small_generic_path(dpa, name, shape):
    hq, hkv, d, dt = shape
    spec = SMALL[name]()
    tr = bool(spec.meta.get("transitive", True))
    q, k, v, do = _inputs(spec, hq, hkv, d, 31, dt)
    got, _ = _run(dpa, spec, q, k, v, do, hq, hkv, d, dt, transitive=tr)
    ref = _ref(spec, q, k, v, do, hq, hkv, transitive=tr)
    _assert_close(got, ref, dt, tag=f"{name}{shape}", fp32_relative=(name != "tiny"))


def test_bf16_gradients_are_rounded_fp32_gradients(dpa):
    """grad_dtype=bf16 writes exactly the fp32 result rounded to nearest-even bf16."""
    spec = _mini4()
    q, k, v, do = _inputs(spec, 16, 4, 128, 12, "bf16")
    a, _ = _run(dpa, spec, q, k, v, do, 16, 4, 128, "bf16", grad="fp32")
    b, _ = _run(dpa, spec, q, k, v, do, 16, 4, 128, "bf16", grad="bf16")
    for n in ("dq", "dk", "dv"):
        r = torch.tensor(a[n]).float().bfloat16().double().numpy()
        assert np.array_equal(r, b[n]), n
    for n in ("o", "lse"):
        assert np.array_equal(a[n], b[n]), n


def test_transitive_reads_on_device(dpa):
    """A random DAG with chained reads, transitive closure on and off, on the MFMA path."""
    rng = np.random.default_rng(3)
    spec = synth.random_tiny_dag(rng, n_nodes=12, max_len=150, p_mount=0.9, max_mounts=2)
    q, k, v, do = _inputs(spec, 16, 4, 128, 77, "bf16")
    for tr in (True, False):
        got, _ = _run(dpa, spec, q, k, v, do, 16, 4, 128, "bf16", transitive=tr)
        ref = _ref(spec, q, k, v, do, 16, 4, transitive=tr)
        _assert_close(got, ref, "bf16", tag=f"transitive={tr}")


def test_peaky_logits_without_rotation(dpa):
    """q, k scaled x4 (logit std ~16): a dropped or misplaced key moves the outputs visibly."""
    spec = _mini3(seed=8)
    q, k, v, do = _inputs(spec, 16, 4, 128, 5, "bf16")
    q, k = (q.float() * 4).bfloat16(), (k.float() * 4).bfloat16()
    got, _ = _run(dpa, spec, q, k, v, do, 16, 4, 128, "bf16", rope=0.0, transitive=False)
    ref = _ref(spec, q, k, v, do, 16, 4, rope=0.0, transitive=False)
    _assert_close(got, ref, "bf16", tag="peaky")


def test_marker_span_mass(dpa):
    """v = 1 on one mounted span and 0 elsewhere: o equals the attention mass on that span."""
    spec = _mini4()
    dag = Dag(spec)
    q, k, _, do = _inputs(spec, 16, 4, 128, 9, "bf16")
    s, b, e = spec.mounts_of(int(np.nonzero(spec.mount_count)[0][0]))[0]
    v = torch.zeros(spec.n_tokens, 4, 128, dtype=torch.bfloat16)
    v[dag.offset[s] + b: dag.offset[s] + e] = 1
    got, _ = _run(dpa, spec, q, k, v, do, 16, 4, 128, "bf16", bwd=False)
    ref = _ref(spec, q, k, v, do, 16, 4, bwd=False)
    _assert_close(got, ref, "bf16", names=("o", "lse"), tag="marker")
    reader = int(np.nonzero(spec.mount_count)[0][0])
    rows = slice(dag.offset[reader], dag.offset[reader] + dag.length[reader])
    assert (got["o"][rows] > 1e-3).all()          # the span is seen by every reader row


def test_backward_is_deterministic_and_page_order_free(dpa):
    spec = _mini3(seed=12)
    q, k, v, do = _inputs(spec, 16, 4, 128, 41, "bf16")
    a, _ = _run(dpa, spec, q, k, v, do, 16, 4, 128, "bf16")
    b, _ = _run(dpa, spec, q, k, v, do, 16, 4, 128, "bf16")
    c, _ = _run(dpa, spec, q, k, v, do, 16, 4, 128, "bf16", shuffle=99)
    for n in a:
        assert np.array_equal(a[n], b[n]), n
        assert np.array_equal(a[n], c[n]), n


# ---------------------------------------------------------------- full-size workloads, sampled


class _TokenView:
    """Read-only view of selected token rows of a row-layout device tensor, indexed by token id."""

    def __init__(self, x_rows, rot_t, tokens):
        self.idx = {int(t): i for i, t in enumerate(tokens)}
        sel = torch.as_tensor(np.asarray(tokens, np.int64), device=x_rows.device)
        self.data = x_rows[rot_t[sel]].double().cpu().numpy()

    def __getitem__(self, key):
        if isinstance(key, tuple):
            return self.data[self.idx[int(key[0])]][key[1:]]
        if isinstance(key, slice):
            return self.data[[self.idx[t] for t in range(key.start, key.stop)]]
        return self.data[self.idx[int(key)]]


def _full_case(dpa, spec, seed, bwd, n_rows=24, n_keys=6, max_readers=96, view="mounted"):
    tr = bool(spec.meta.get("transitive", True))
    plan = dpa.Plan(spec, transitive=tr, view=view)
    p = dpa.AttnParams(16, 4, 128, "bf16")          # the benchmark's configuration (bf16 gradients)
    C = plan.rows
    q = synth.normal((C, 16, 128), seed, 1, DEV, torch.bfloat16)
    k = synth.normal((C, 4, 128), seed, 2, DEV, torch.bfloat16)
    v = synth.normal((C, 4, 128), seed, 3, DEV, torch.bfloat16)
    o, lse, o_lo = dpa.attn_fwd(plan, p, q, k, v, o_lo=True)
    res = {"o": o, "lse": lse}
    if bwd:
        do = synth.normal((C, 16, 128), seed, 4, DEV, torch.bfloat16)
        res["dq"], res["dk"], res["dv"] = dpa.attn_bwd(plan, p, q, k, v, o, lse, do, o_lo=o_lo)
    torch.cuda.synchronize()
    for n, t in res.items():
        assert torch.isfinite(t).all(), n
    dag = Dag(spec, transitive=tr, view=view)
    rot, _ = plan.row_maps()
    rot_t = torch.as_tensor(rot, dtype=torch.long, device=DEV)
    kh = k[rot_t].float().cpu().numpy()
    vh = v[rot_t].float().cpu().numpy()
    rng = np.random.default_rng(seed)
    # rows: random tokens plus the first and last token of a few nodes (page edges, readers)
    picks = list(rng.choice(dag.n_tokens, n_rows, replace=False))
    for u in rng.choice(dag.n, 6, replace=False):
        if dag.length[u]:
            picks += [dag.offset[u], dag.offset[u] + dag.length[u] - 1]
    picks = np.array(sorted(set(int(x) for x in picks)))
    rs = RowSampler(spec, OParams(16, 4), transitive=tr, view=view)
    o_ref, l_ref = rs.rows(picks, _TokenView(q, rot_t, picks), kh, vh)
    _assert_close({"o": res["o"][rot_t[picks]].double().cpu().numpy(),
                   "lse": res["lse"][rot_t[picks]].double().cpu().numpy()},
                  {"o": o_ref, "lse": l_ref}, "bf16", names=("o", "lse"), tag="sampled rows")
    if bwd:
        # keys with few readers: tail tokens of leaf nodes that no read reaches
        cands = []
        for u in dag.leaves_dfs():
            for j in range(max(0, dag.length[u] - 6), dag.length[u]):
                cands.append(dag.offset[u] + j)
        rng.shuffle(cands)
        keys, readers = [], set()
        for j in cands:
            r = rs.readers(j)
            if len(r) <= max_readers:
                keys.append(j)
                readers.update(int(t) for t in r)
            if len(keys) == n_keys:
                break
        assert keys, "no lightly-read key found"
        keys = np.array(sorted(keys))
        need = np.array(sorted(readers))
        dk_ref, dv_ref = rs.key_grads(keys, _TokenView(q, rot_t, need), kh, vh, _TokenView(do, rot_t, need))
        _assert_close({"dk": res["dk"][rot_t[keys]].double().cpu().numpy(),
                       "dv": res["dv"][rot_t[keys]].double().cpu().numpy()},
                      {"dk": dk_ref, "dv": dv_ref}, "bf16", names=("dk", "dv"), tag="sampled keys")
    return plan, res


@pytest.mark.parametrize("view", ["mount_free", "unshifted"])
def test_full_size_views_sampled(dpa, view):
    # the benchmark's views record: the 16-tree workload in the other two views
    print(f"full-size view {view}", flush=True)
    _full_case(dpa, synth.config3(), seed=1103, bwd=True, view=view)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("which", ["w2", "w4", "w3", "short"])
def test_full_size_sampled(dpa, which):
    spec = {"w2": synth.config2, "w4": synth.config4, "w3": synth.config3,
            "short": synth.dags.config3_short_segments}[which]()
    seed = {"w2": 1002, "w4": 1004, "w3": 1003, "short": 1013}[which]
    _full_case(dpa, spec, seed=seed, bwd=(which != "w2"))
    torch.cuda.empty_cache()
