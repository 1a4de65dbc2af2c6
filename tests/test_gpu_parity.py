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
         scale=0.0, grad="fp32", view="mounted", pack=False):
    """Token-major CPU tensors in, token-major CPU float64 results out (via the row layout).

    Gradients come back in fp32 by default: in these small DAGs a shared row's dK/dV reaches
    magnitudes (~11) where bf16 storage alone is 0.03 away from the exact value.
    """
    plan = dpa.Plan(spec, transitive=transitive, page_shuffle=shuffle, view=view, pack=pack)
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


def test_forward_without_residual_and_backward_that_needs_it(dpa):
    """The bf16 forward writes the same o and lse with or without o_lo; the bf16 backward
    refuses to run without it (rowsum(dO * O) from bf16 O alone is off by more than the
    tolerance where attention is peaked)."""
    spec = _mini4()
    plan = dpa.Plan(spec)
    p = dpa.AttnParams(16, 4, 128, "bf16")
    q, k, v, do = (dpa.to_rows(plan, x.to(DEV)) for x in _inputs(spec, 16, 4, 128, 17, "bf16"))
    o1, l1, lo = dpa.attn_fwd(plan, p, q, k, v, o_lo=True)
    o2, l2 = dpa.attn_fwd(plan, p, q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    with pytest.raises(dpa.DagError) as e:
        dpa.attn_bwd(plan, p, q, k, v, o1, l1, do)
    assert e.value.code == "INVALID"


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


def _outlier_rows(x, rng, n, lo_exp, hi_exp):
    """x with n random token rows rescaled so that each one's largest |element| is 2^e,
    e uniform in [lo_exp, hi_exp) (bf16-exact powers of two times bf16 values)."""
    x = x.float().clone()
    rows = rng.choice(x.shape[0], n, replace=False)
    peak = x[rows].abs().amax(dim=(1, 2), keepdim=True)
    target = torch.tensor(2.0 ** rng.uniform(lo_exp, hi_exp, n), dtype=torch.float32)[:, None, None]
    x[rows] = x[rows] / peak * target
    return x.bfloat16()


@pytest.mark.parametrize("which", ["q", "k", "v", "qv"])
def test_wide_range_operands(dpa, which):
    """bf16 inputs far outside fp16's range: outlier rows of q, k or v (or q and v) whose largest
    element is 2^16..2^17, and dO rows scaled by 2^-u, u uniform in [0, 30].  The MFMA path's
    fp16 operand copies carry per-tensor power-of-two scales, so every output is finite and
    within the bf16 tolerance scaled by max(1, max|ref|) per tensor (the scaling of R13).

    Outlier q or k rows run without rotation: then their fp16 copies are exact, and logits of
    ~3e4 come out to fp32 accumulation accuracy.  With rotation the rotated row is rounded to
    fp16 (2^-12 of its size, ~7 per element here), which puts ~4 of absolute error on such
    logits and can flip near-tied top keys; that is the precision of a half-precision operand,
    not its range.  Outliers in q and k together are left out: their logits reach ~1e9, where
    the fp32 lse that the interface stores is itself only accurate to about +-32."""
    spec = _mini3(seed=21)
    tr = bool(spec.meta.get("transitive", True))
    rope = 0.0 if ("q" in which or "k" in which) else 10000.0
    print(f"wide-range operands: outliers in {which}, rope base {rope}", flush=True)
    q, k, v, do = _inputs(spec, 16, 4, 128, 808, "bf16")
    rng = np.random.default_rng(808)
    if "q" in which:
        q = _outlier_rows(q, rng, 6, 16.0, 17.0)
    if "k" in which:
        k = _outlier_rows(k, rng, 6, 16.0, 17.0)
    if "v" in which:
        v = _outlier_rows(v, rng, 6, 16.0, 17.0)
    do = (do.float() * torch.tensor(2.0 ** -rng.uniform(0.0, 30.0, spec.n_tokens),
                                    dtype=torch.float32)[:, None, None]).bfloat16()
    got, _ = _run(dpa, spec, q, k, v, do, 16, 4, 128, "bf16", transitive=tr, rope=rope)
    ref = _ref(spec, q, k, v, do, 16, 4, transitive=tr, rope=rope)
    # A row whose softmax sits on one key has dS = P (dP - D) = 0 exactly, and the GPU's dP
    # (summed on the matrix cores) and D (summed on the vector units) then agree only to fp32
    # summation accuracy: a 128-term fp32 sum is typically off by about sqrt(128) 2^-24 (about
    # 2^-20.5) of its absolute terms, and with keys of |k| ~ 1e5 that difference, times k, is
    # visible in dq (0.038 at most here, where the exact dq is 0).  The oracle sizes those terms
    # per element (RowSampler.row_grads term_size) and dq may carry 2^-20 of them on top.
    rs = RowSampler(spec, OParams(16, 4, rope_base=rope), transitive=tr)
    *_, dq_terms = rs.row_grads(np.arange(spec.n_tokens), q.double().numpy(), k.double().numpy(),
                                v.double().numpy(), do.double().numpy(), term_size=True)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert np.isfinite(got[n]).all(), f"{which} {n}: non-finite"
        bar = max(1.0, float(np.abs(ref[n]).max()))
        err = np.abs(got[n] - ref[n])
        if n == "dq":
            err = np.maximum(err - 2.0 ** -20 * dq_terms, 0.0)
        assert err.max() <= BF16_MAX * bar and err.mean() <= BF16_MEAN * bar, \
            f"{which} {n}: max {err.max():.3g} mean {err.mean():.3g} (max|ref| {bar:.3g})"


def test_forward_with_huge_logits(dpa):
    """Outlier rows in q and k together (2^16..2^17, no rotation): logits reach ~1e9, past
    where the forward's fused exponent form would overflow; the forward switches to the exact
    form there, and o and lse come out finite and within the scaled bar.  (The backward is
    not compared: the fp32 lse of the interface resolves such logits only to about +-32.)"""
    spec = _mini3(seed=21)
    tr = bool(spec.meta.get("transitive", True))
    q, k, v, do = _inputs(spec, 16, 4, 128, 909, "bf16")
    rng = np.random.default_rng(909)
    q = _outlier_rows(q, rng, 6, 16.0, 17.0)
    k = _outlier_rows(k, rng, 6, 16.0, 17.0)
    got, _ = _run(dpa, spec, q, k, v, do, 16, 4, 128, "bf16", transitive=tr, rope=0.0, bwd=False)
    ref = _ref(spec, q, k, v, do, 16, 4, transitive=tr, rope=0.0, bwd=False)
    assert np.abs(ref["lse"]).max() > 1e8
    for n in ("o", "lse"):
        assert np.isfinite(got[n]).all(), n
        bar = max(1.0, float(np.abs(ref[n]).max()))
        err = np.abs(got[n] - ref[n])
        assert err.max() <= BF16_MAX * bar and err.mean() <= BF16_MEAN * bar, \
            f"{n}: max {err.max():.3g} mean {err.mean():.3g} (max|ref| {bar:.3g})"


def _mid_commander_workers():
    # one commander-worker episode small enough for the flat oracle: a 1,024-token
    # commander, 8 workers of 4,096 own tokens, worker w reading at 1,536 + 256 w the
    # last 1,024 pre-read tokens of workers w +- 1 (33,792 tokens).  A commander page is
    # read by 8 x 4,096 worker rows (about 1,000 reader steps of 32 rows), and every
    # mounted span's dK/dV sums its producer's own rows and two readers' post-read rows.
    return synth.config4(n_episodes=1, commander=1024, workers=8, budget=4096, span=1024, first_read=1536,
                         read_step=256)


def test_mid_commander_workers_elementwise(dpa):
    """All five tensors element by element against the flat oracle on a DAG whose KV pages
    have long reader lists and whose mounted spans route dK/dV to their producers
    (Octopus Sec. 3.4 Eq. 8), in fp32 gradients; bf16 gradients are the same values rounded."""
    spec = _mid_commander_workers()
    print("mid commander-workers: 33,792 tokens, 8/2 heads", flush=True)
    q, k, v, do = _inputs(spec, 8, 2, 128, 4242, "bf16")
    got, _ = _run(dpa, spec, q, k, v, do, 8, 2, 128, "bf16", grad="fp32")
    got16, _ = _run(dpa, spec, q, k, v, do, 8, 2, 128, "bf16", grad="bf16")
    for n in ("dq", "dk", "dv"):
        r = torch.tensor(got[n]).float().bfloat16().double().numpy()
        assert np.array_equal(r, got16[n]), n
    ref = _ref(spec, q, k, v, do, 8, 2)
    _assert_close(got, ref, "bf16", tag="mid-cw")


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
    """Read-only view of selected token rows of a row-layout device tensor, indexed by token id
    (an int, an int array or a slice of token ids)."""

    def __init__(self, x_rows, rot_t, tokens):
        tokens = np.asarray(sorted(set(int(t) for t in tokens)), np.int64)
        self.pos = np.full(int(tokens.max()) + 1 if len(tokens) else 1, -1, np.int64)
        self.pos[tokens] = np.arange(len(tokens))
        sel = torch.as_tensor(tokens, device=x_rows.device)
        self.data = x_rows[rot_t[sel]].double().cpu().numpy()

    def _idx(self, ids):
        i = self.pos[ids]
        assert (i >= 0).all(), "token row not fetched"
        return i

    def __getitem__(self, key):
        if isinstance(key, tuple):
            return self.data[self._idx(int(key[0]))][key[1:]]
        if isinstance(key, slice):
            return self.data[self._idx(np.arange(key.start, key.stop))]
        if isinstance(key, np.ndarray):
            return self.data[self._idx(key.astype(np.int64))]
        return self.data[self._idx(int(key))]


def _n_reader_rows(rs, dag, j):
    """Query rows whose visible set holds key token j (its own node's rows from j on, and
    every row of each other reader node)."""
    u, jo = int(rs.node_of[j]), int(rs.off[j])
    return sum(dag.length[w] for w in rs.reader_nodes(j) if w != u) + dag.length[u] - jo


def _heavy_keys(rs, dag, rng, hi, n_cand=150):
    """Two keys whose dK/dV sums over many readers, each the most-read of a random sample
    of candidates with at most ``hi`` reader rows: one in an inner node whose children are
    all leaves (its later own rows and every child read it), one inside a directly mounted
    span (its producer's later rows and descendants plus the reader's subtree read it)."""
    out = []
    inner = [u for u in range(dag.n)
             if dag.length[u] and dag.children[u] and all(not dag.children[c] for c in dag.children[u])]
    spans = [(s, b, e) for r in range(dag.n) for (s, b, e) in dag.nonempty_direct(r)]
    for kind, pool in (("inner", inner), ("mounted", spans)):
        best = None
        for i in rng.permutation(len(pool))[:n_cand]:
            if kind == "inner":
                u = pool[i]
                j = dag.offset[u] + int(rng.integers(0, dag.length[u]))
            else:
                s_, b_, e_ = pool[i]
                j = dag.offset[s_] + int(rng.integers(b_, e_))
            n = _n_reader_rows(rs, dag, j)
            if n <= hi and (best is None or n > best[0]):
                best = (n, j)
        if best is not None:
            out.append((kind, best[1], best[0]))
    return out


def _full_case(dpa, spec, seed, bwd, n_rows=24, n_keys=6, max_readers=96, view="mounted", heavy_hi=16000,
               transitive=None, pack=False):
    """The workload at full size, in the benchmark's launch configuration (bf16 tensors and
    gradients).  Compared with the oracle: o, lse and dq on sampled query rows (random tokens
    plus the first and last token of a few nodes), and dK/dV on sampled keys -- a few
    lightly read leaf-tail keys (all four KV heads) and, unless ``heavy_hi`` is 0, two
    heavily read keys (an inner node's and a mounted span's, one KV head each) whose
    gradient sums up to ``heavy_hi`` reader rows."""
    tr = bool(spec.meta.get("transitive", True)) if transitive is None else transitive
    plan = dpa.Plan(spec, transitive=tr, view=view, pack=pack)
    p = dpa.AttnParams(16, 4, 128, "bf16")          # the benchmark's configuration (bf16 gradients)
    C = plan.rows
    q = synth.normal((C, 16, 128), seed, 1, DEV, torch.bfloat16)
    k = synth.normal((C, 4, 128), seed, 2, DEV, torch.bfloat16)
    v = synth.normal((C, 4, 128), seed, 3, DEV, torch.bfloat16)
    do = synth.normal((C, 16, 128), seed, 4, DEV, torch.bfloat16)
    o, lse, o_lo = dpa.attn_fwd(plan, p, q, k, v, o_lo=True)
    res = {"o": o, "lse": lse}
    if bwd:
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
    picks = list(rng.choice(dag.n_tokens, n_rows, replace=False))
    for u in rng.choice(dag.n, 6, replace=False):
        if dag.length[u]:
            picks += [dag.offset[u], dag.offset[u] + dag.length[u] - 1]
    picks = np.array(sorted(set(int(x) for x in picks)))
    rs = RowSampler(spec, OParams(16, 4), transitive=tr, view=view)
    got = lambda name, toks: res[name][rot_t[torch.as_tensor(toks, device=DEV)]].double().cpu().numpy()
    if not bwd:
        o_ref, l_ref = rs.rows(picks, _TokenView(q, rot_t, picks), kh, vh)
        _assert_close({"o": got("o", picks), "lse": got("lse", picks)}, {"o": o_ref, "lse": l_ref}, "bf16",
                      names=("o", "lse"), tag="sampled rows")
        return plan, res
    o_ref, l_ref, dq_ref = rs.row_grads(picks, _TokenView(q, rot_t, picks), kh, vh, _TokenView(do, rot_t, picks))
    _assert_close({"o": got("o", picks), "lse": got("lse", picks), "dq": got("dq", picks)},
                  {"o": o_ref, "lse": l_ref, "dq": dq_ref}, "bf16", names=("o", "lse", "dq"), tag="sampled rows")
    # keys with few readers: tail tokens of leaf nodes that no read reaches
    cands = []
    for u in dag.leaves_dfs():
        for j in range(max(0, dag.length[u] - 6), dag.length[u]):
            cands.append(dag.offset[u] + j)
    rng.shuffle(cands)
    keys = []
    for j in cands:
        if _n_reader_rows(rs, dag, j) <= max_readers:
            keys.append(j)
        if len(keys) == n_keys:
            break
    assert keys, "no lightly-read key found"
    sets = [("light", sorted(keys), None)]
    if heavy_hi:
        for i, (kind, j, n) in enumerate(_heavy_keys(rs, dag, rng, heavy_hi)):
            print(f"  heavy key ({kind}): token {j}, {n} reader rows", flush=True)
            sets.append((kind, [j], [i % 4]))
    for kind, ks, groups in sets:
        need = np.unique(np.concatenate([rs.readers(j) for j in ks]))
        dk_ref, dv_ref = rs.key_grads_by_node(ks, _TokenView(q, rot_t, need), kh, vh, _TokenView(do, rot_t, need),
                                              groups=groups)
        sel = slice(None) if groups is None else groups
        _assert_close({"dk": got("dk", ks)[:, sel], "dv": got("dv", ks)[:, sel]},
                      {"dk": dk_ref[:, sel], "dv": dv_ref[:, sel]}, "bf16", names=("dk", "dv"),
                      tag=f"sampled keys ({kind})")
    return plan, res


@pytest.mark.parametrize("view", ["mount_free", "unshifted"])
def test_full_size_views_sampled(dpa, view):
    # the benchmark's views record: the 16-tree workload in the other two views
    print(f"full-size view {view}", flush=True)
    _full_case(dpa, synth.config3(), seed=1103, bwd=True, view=view)
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- packed page layouts


@pytest.mark.parametrize("name", ["mini_short", "mini3", "mini4", "tiny"])
def test_packed_pages_small(dpa, name):
    """Nodes sharing pages (per-tile visibility masks): all five tensors against the flat oracle."""
    spec = SMALL[name]()
    tr = bool(spec.meta.get("transitive", True))
    print(f"packed {name}", flush=True)
    q, k, v, do = _inputs(spec, 16, 4, 128, 6000 + len(name), "bf16")
    got, plan = _run(dpa, spec, q, k, v, do, 16, 4, 128, "bf16", transitive=tr, pack=True)
    assert plan.info["pack_pages"] == 1
    ref = _ref(spec, q, k, v, do, 16, 4, transitive=tr)
    _assert_close(got, ref, "bf16", tag=f"packed {name}")


@pytest.mark.parametrize("seed", [3, 4])
def test_packed_pages_random_reads(dpa, seed):
    """Random DAGs whose reads reach nodes later in depth-first order (a mounted key can then sit
    above its reader in the same page), transitive closure on and off."""
    rng = np.random.default_rng(seed)
    spec = synth.random_tiny_dag(rng, n_nodes=14, max_len=40, p_mount=0.9, max_mounts=2)
    q, k, v, do = _inputs(spec, 16, 4, 128, 70 + seed, "bf16")
    for tr in (True, False):
        got, _ = _run(dpa, spec, q, k, v, do, 16, 4, 128, "bf16", transitive=tr, pack=True)
        ref = _ref(spec, q, k, v, do, 16, 4, transitive=tr)
        _assert_close(got, ref, "bf16", tag=f"packed random {seed} transitive={tr}")


def test_packed_pages_gdn_and_refusals(dpa):
    """The gated delta rule reads rows through the plan's maps: on a packed plan its outputs and
    gradients are bitwise those of the unpacked plan.  The generic attention path and the
    convolution refuse packed plans."""
    spec = SMALL["mini_short"]()
    H = 2
    ins = synth.tensors.gdn_inputs(spec.n_tokens, H, 128, 128, 31, dtype=torch.bfloat16, decay_scale=0.2)
    outs = []
    for pack in (False, True):
        plan = dpa.Plan(spec, gdn_chunk=64, pack=pack)
        p = dpa.GdnParams(H, grad_dtype="fp32")
        rows = lambda x: dpa.to_rows(plan, x.to(DEV), fill=float("nan"))
        qr, kr, vr, br, ar, dr = (rows(x) for x in ins)
        o = dpa.gdn_fwd(plan, p, qr, kr, vr, br, ar)
        g = dpa.gdn_bwd(plan, p, qr, kr, vr, br, ar, dr)
        torch.cuda.synchronize()
        outs.append([dpa.from_rows(plan, t).cpu() for t in (o, *g)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    plan = dpa.Plan(spec, pack=True)
    q, k, v, _ = (dpa.to_rows(plan, x.to(DEV)) for x in _inputs(spec, 4, 2, 64, 5, "bf16"))
    with pytest.raises(dpa.DagError) as e:
        dpa.attn_fwd(plan, dpa.AttnParams(4, 2, 64, "bf16"), q, k, v)
    assert e.value.code == "UNSUPPORTED"
    with pytest.raises(dpa.DagError) as e:
        dpa.conv_workspace_bytes(plan, dpa.ConvParams(64))
    assert e.value.code == "UNSUPPORTED"


@pytest.mark.parametrize("which", ["w2", "w4", "w3", "w3t", "short"])
def test_full_size_sampled(dpa, which):
    # w3t: the 16-tree workload with transitive reads (Octopus Sec. 3.3 item 1), the
    # benchmark's "transitive" record
    spec = {"w2": synth.config2, "w4": synth.config4, "w3": synth.config3, "w3t": synth.config3,
            "short": synth.dags.config3_short_segments}[which]()
    seed = {"w2": 1002, "w4": 1004, "w3": 1003, "w3t": 1023, "short": 1013}[which]
    print(f"full size: {which}", flush=True)
    # the commander-worker episodes' inner keys have 30K-260K reader rows each, beyond what the
    # oracle evaluates in seconds; their reductions are compared element by element on the
    # mid-size episode instead
    _full_case(dpa, spec, seed=seed, bwd=(which != "w2"), heavy_hi=0 if which == "w4" else 16000,
               transitive=True if which == "w3t" else None)
    torch.cuda.empty_cache()


def test_full_size_short_segments_packed(dpa):
    # the page-gather diagnostic in the packed layout, as the benchmark's gather record runs it
    print("full size: short segments, packed pages", flush=True)
    plan, _ = _full_case(dpa, synth.dags.config3_short_segments(), seed=1017, bwd=True, pack=True)
    assert plan.info["pack_pages"] == 1
    torch.cuda.empty_cache()
