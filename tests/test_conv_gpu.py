"""GPU parity of the short causal convolution against the oracle.

Small DAGs (a fork through a zero-length node, a tree with mounts and one-token
nodes, the tiny workload, random DAGs with shuffled physical pages) are
compared element by element with the per-trajectory oracle, for widths 1-4,
both activations, bf16 and fp32 dx, and channel counts that leave a block's
second channel chunk partly empty.  y and dx must be bitwise independent of
the physical page layout and of the run.  On the 16-tree workload at the
benchmark's 6,144 channels (q, k and v of 16 heads x 128), 8 sampled channels
are compared over every row with the oracle's compact evaluation.

Tolerance (bf16 inputs, fp32 arithmetic): y within 2^-8 |y| (half a bf16 ulp)
+ 1e-5 (sum_k |W x|); dx within 1e-5 (sum of |W dpre| over its readers) + 2^-8
|dx| for bf16 dx; dW within 1e-4 of sum_t |dpre x| (fp32 sums over up to 3.3M
rows).
"""
import numpy as np
import pytest
import torch

import synth.dags as D
import synth.tensors as T
from oracle import conv as CV

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def dpa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dag_packed_attention_amd as m
    return m


def _fork():
    g = D.DagBuilder()
    r = g.node(-1, 70)
    a = g.node(r, 2)
    b = g.node(r, 0)
    g.node(b, 1)
    c = g.node(b, 66)
    g.node(a, 130)
    g.node(c, 3)
    g.node(c, 0)
    return g.build(name="conv_fork")


def _mounts():
    g = D.DagBuilder()
    r = g.node(-1, 1)
    a = g.node(r, 2)
    b = g.node(r, 64)
    c = g.node(a, 1)
    d = g.node(c, 65)
    g.node(a, 1)
    g.node(a, 3)
    e = g.node(b, 128)
    g.mount(b, a, 0, 2)
    g.mount(d, e, 1, 30)
    return g.build(name="conv_mounts")


def _inputs(spec, Ch, w, seed):
    x = T.normal((spec.n_tokens, Ch), seed, 31).to(torch.bfloat16)
    W = T.normal((Ch, w), seed, 32) * 0.5
    dy = T.normal((spec.n_tokens, Ch), seed, 33).to(torch.bfloat16)
    return x, W, dy


def _compare(ref, got_y, got_dx, got_dW, x64, W64, act, bf16_dx):
    # bounds from the magnitudes of the terms each result sums
    U = x64.shape[0]
    absy = np.abs(CV.conv_compact(_compare.spec, np.abs(x64), np.abs(W64), CV.ACT_NONE)["y"])
    tol_y = 2.0 ** -8 * np.abs(ref["y"]) + 1e-5 * absy + 1e-6
    assert np.all(np.abs(got_y - ref["y"]) <= tol_y), float(np.abs(got_y - ref["y"]).max())
    absdx = CV.conv_compact(_compare.spec, np.abs(x64), np.abs(W64), CV.ACT_NONE, np.abs(_compare.dpre))["dx"]
    tol_dx = 1e-5 * absdx + 1e-6 + (2.0 ** -8 * np.abs(ref["dx"]) if bf16_dx else 0.0)
    assert np.all(np.abs(got_dx - ref["dx"]) <= tol_dx), float(np.abs(got_dx - ref["dx"]).max())
    absdw = CV.conv_compact(_compare.spec, np.abs(x64), np.ones_like(W64), CV.ACT_NONE, np.abs(_compare.dpre))["dW"]
    assert np.all(np.abs(got_dW - ref["dW"]) <= 1e-4 * absdw + 1e-6), float(np.abs(got_dW - ref["dW"]).max())
    assert U == got_y.shape[0]


def _run(dpa, spec, Ch, w, act, grad, seed, shuffle=0):
    plan = dpa.Plan(spec, page_shuffle=shuffle)
    x, W, dy = _inputs(spec, Ch, w, seed)
    p = dpa.ConvParams(Ch, w, act, grad)
    xr = dpa.to_rows(plan, x.to(DEV), fill=float("nan"))
    dyr = dpa.to_rows(plan, dy.to(DEV), fill=float("nan"))
    Wd = W.to(DEV)
    y = dpa.conv_fwd(plan, p, xr, Wd)
    dx, dW = dpa.conv_bwd(plan, p, xr, Wd, dyr)
    torch.cuda.synchronize()
    rot, _ = plan.row_maps()
    pad = np.setdiff1d(np.arange(plan.rows), rot)
    if len(pad):
        pi = torch.as_tensor(pad, device=DEV)
        assert torch.all(y[pi] == 0) and torch.all(dx[pi] == 0)
    return plan, x, W, dy, y, dx, dW


def _check_small(dpa, spec, Ch, w, act, grad, seed, shuffle=0):
    plan, x, W, dy, y, dx, dW = _run(dpa, spec, Ch, w, act, grad, seed, shuffle)
    a = CV.ACT_SILU if act == "silu" else CV.ACT_NONE
    x64, W64, dy64 = x.double().numpy(), W.double().numpy(), dy.double().numpy()
    ref = CV.conv_flat(spec, x64, W64, a, dy64)
    pre = CV.conv_compact(spec, x64, W64, CV.ACT_NONE)["y"]
    _compare.spec = spec
    _compare.dpre = dy64 * CV._act_grad(pre, a)
    _compare(ref, dpa.from_rows(plan, y).double().cpu().numpy(), dpa.from_rows(plan, dx).double().cpu().numpy(),
             dW.double().cpu().numpy(), x64, W64, a, grad == "bf16")
    return plan, y, dx, dW


@pytest.mark.parametrize("w", [1, 2, 3, 4])
@pytest.mark.parametrize("act", ["none", "silu"])
def test_fork_all_widths(dpa, w, act):
    print(f"conv fork w={w} act={act}", flush=True)
    _check_small(dpa, _fork(), 16, w, act, "fp32", seed=w)


@pytest.mark.parametrize("Ch,grad", [(8, "bf16"), (2056, "fp32"), (64, "bf16")])
def test_mounts_and_channel_chunks(dpa, Ch, grad):
    print(f"conv mounts Ch={Ch} dx={grad}", flush=True)
    _check_small(dpa, _mounts(), Ch, 4, "silu", grad, seed=Ch)


@pytest.mark.parametrize("name", ["config1", "config1_variant"])
def test_small_configurations(dpa, name):
    print(f"conv {name}", flush=True)
    _check_small(dpa, getattr(D, name)(), 24, 4, "silu", "fp32", seed=7, shuffle=3)


def test_random_dags_and_page_layout_independence(dpa):
    for seed in range(5):
        rng = np.random.default_rng(900 + seed)
        spec = D.random_tiny_dag(rng, n_nodes=int(rng.integers(2, 14)), max_len=int(rng.integers(1, 140)),
                                 p_mount=0.6, max_mounts=2, n_roots=int(rng.integers(1, 3)))
        print(f"conv random seed={seed}", flush=True)
        plan0, y0, dx0, _ = _check_small(dpa, spec, 32, 4, "silu", "fp32", seed=seed)
        plan1, y1, dx1, _ = _check_small(dpa, spec, 32, 4, "silu", "fp32", seed=seed, shuffle=seed + 1)
        assert torch.equal(dpa.from_rows(plan0, y0), dpa.from_rows(plan1, y1))
        assert torch.equal(dpa.from_rows(plan0, dx0), dpa.from_rows(plan1, dx1))


def test_deterministic(dpa):
    print("conv determinism", flush=True)
    spec = _mounts()
    _, _, _, _, y, dx, dW = _run(dpa, spec, 2056, 4, "silu", "bf16", seed=3)
    _, _, _, _, y2, dx2, dW2 = _run(dpa, spec, 2056, 4, "silu", "bf16", seed=3)
    assert torch.equal(y, y2) and torch.equal(dx, dx2) and torch.equal(dW, dW2)


def test_benchmark_size_sampled_channels(dpa):
    # 16-tree workload, 6,144 channels, w = 4, SiLU, bf16 dx: the benchmark's launch
    print("conv benchmark size", flush=True)
    spec = D.config3()
    plan = dpa.Plan(spec)
    Ch, w = 6144, 4
    p = dpa.ConvParams(Ch, w, "silu", "bf16")
    C = plan.rows
    gen = torch.Generator(device=DEV)
    gen.manual_seed(41)
    x = torch.empty((C, Ch), dtype=torch.bfloat16, device=DEV).normal_(generator=gen)   # drawn in bf16:
    dy = torch.empty((C, Ch), dtype=torch.bfloat16, device=DEV).normal_(generator=gen)  # no fp32 copy in HBM
    W = (T.normal((Ch, w), 41, 3) * 0.5).to(DEV)
    y = dpa.conv_fwd(plan, p, x, W)
    dx, dW = dpa.conv_bwd(plan, p, x, W, dy)
    torch.cuda.synchronize()
    cols = np.sort(np.random.default_rng(5).choice(Ch, 8, replace=False))
    ci = torch.as_tensor(cols, device=DEV)
    rot, _ = plan.row_maps()
    ri = torch.as_tensor(rot, device=DEV)
    pick = lambda t: t[:, ci][ri].double().cpu().numpy()
    x64, dy64 = pick(x), pick(dy)
    W64 = W[ci].double().cpu().numpy()
    ref = CV.conv_compact(spec, x64, W64, CV.ACT_SILU, dy64)
    pre = CV.conv_compact(spec, x64, W64, CV.ACT_NONE)["y"]
    _compare.spec = spec
    _compare.dpre = dy64 * CV._act_grad(pre, CV.ACT_SILU)
    _compare(ref, pick(y), pick(dx), dW[ci].double().cpu().numpy(), x64, W64, CV.ACT_SILU, True)
