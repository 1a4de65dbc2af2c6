"""Argument checks of the C-ABI entry points that are decided on the host, before any
device call (CPU: the tensor and workspace pointers passed here are never dereferenced).

Each malformed request returns its documented status (include/dag_attn.h) and leaves a
message in dag_last_error(); a well-formed workspace query answers on the host alone.
"""
import ctypes

import numpy as np
import pytest

import dag_packed_attention_amd as dpa
import synth

# Host logic only: on a machine with a visible GPU these are skipped, so that a change in
# the order of the checks can never hand the placeholder pointers to a kernel.
pytestmark = pytest.mark.skipif(__import__("torch").cuda.device_count() > 0,
                                reason="host checks; run where no GPU is visible")

L = dpa._lib
OK, INVALID, WORKSPACE, UNSUPPORTED = 0, 1, 7, 8
FAKE = ctypes.c_void_p(0x1000)  # a pointer value that the checks below never reach
BIG = 1 << 40


@pytest.fixture(scope="module")
def plan():
    return dpa.Plan(synth.config1())


@pytest.fixture(scope="module")
def gdn_plan():
    return dpa.Plan(synth.config1(), gdn_chunk=64)


@pytest.fixture(scope="module")
def packed_plan():
    return dpa.Plan(synth.dags.config3_structure(7, n_trees=2, seg=(1, 64), depth_hi=3, fan=(2, 4)), pack=True)


def _attn(n_q=16, n_kv=4, d=128, dtype=0, grad=0, scale=0.0, rope=10000.0):
    return dpa.DagAttnParams(n_q, n_kv, d, dtype, grad, scale, rope)


def _fwd(plan, cp, q=FAKE, o_lo=None, ws=FAKE, ws_bytes=BIG):
    return L.dag_attn_fwd(plan._h, ctypes.byref(cp), q, FAKE, FAKE, FAKE, FAKE, o_lo, ws, ws_bytes, None)


def _err():
    return (L.dag_last_error() or b"").decode()


@pytest.mark.parametrize("kw,code,word", [
    ({"n_q": 0}, UNSUPPORTED, "n_q_heads"),
    ({"n_kv": 0}, UNSUPPORTED, "n_q_heads"),
    ({"n_q": 6, "n_kv": 4}, UNSUPPORTED, "multiple"),
    ({"d": 0}, UNSUPPORTED, "head_dim"),
    ({"d": 63}, UNSUPPORTED, "head_dim"),
    ({"d": 130}, UNSUPPORTED, "head_dim"),
    ({"dtype": 2}, UNSUPPORTED, "dtype"),
    ({"grad": 5}, UNSUPPORTED, "grad_dtype"),
    ({"dtype": 1, "grad": 0}, UNSUPPORTED, "fp32"),
    ({"rope": 0.5}, INVALID, "rope_base"),
    ({"rope": 1.0}, INVALID, "rope_base"),
    ({"rope": -2.0}, INVALID, "rope_base"),
    ({"rope": float("inf")}, INVALID, "rope_base"),
    ({"rope": float("nan")}, INVALID, "rope_base"),
])
def test_attention_parameters_outside_the_kernels_are_refused(plan, kw, code, word):
    cp = _attn(**kw)
    assert _fwd(plan, cp) == code and word in _err()
    f, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert L.dag_attn_workspace(plan._h, ctypes.byref(cp), ctypes.byref(f), ctypes.byref(b)) == code


def test_attention_workspace_query_and_the_size_check_agree(plan):
    for cp in (_attn(), _attn(2, 2, 64, 1, 1, 0.0, 0.0)):
        f, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
        assert L.dag_attn_workspace(plan._h, ctypes.byref(cp), ctypes.byref(f), ctypes.byref(b)) == OK
        assert f.value > 0 and b.value > 0
        # one byte short, or no workspace at all: refused, naming the size it needs
        assert _fwd(plan, cp, ws_bytes=f.value - 1) == WORKSPACE and str(f.value) in _err()
        assert _fwd(plan, cp, ws=None) == WORKSPACE
        o_lo = FAKE if cp.dtype == 0 else None  # bf16 needs the residual, fp32 takes none
        st = L.dag_attn_bwd(plan._h, ctypes.byref(cp), FAKE, FAKE, FAKE, FAKE, FAKE, o_lo, FAKE, FAKE, FAKE, FAKE,
                            FAKE, b.value - 1, None)
        assert st == WORKSPACE and str(b.value) in _err()


def test_attention_refuses_missing_tensors_and_a_misplaced_residual(plan):
    assert _fwd(plan, _attn(), q=None) == INVALID and "null" in _err()
    assert _fwd(plan, _attn(2, 2, 64, 1, 1), o_lo=FAKE) == INVALID and "o_lo" in _err()
    st = L.dag_attn_bwd(plan._h, ctypes.byref(_attn()), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                        FAKE, BIG, None)
    assert st == INVALID and "null" in _err()
    assert L.dag_attn_fwd(None, ctypes.byref(_attn()), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, BIG, None) == INVALID
    assert L.dag_attn_fwd(plan._h, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, BIG, None) == INVALID


def test_packed_layouts_refuse_the_generic_path(packed_plan):
    # packed pages run on the MFMA kernels only (bf16, head_dim 128, Hq = 4 Hkv)
    for cp in (_attn(2, 2, 64, 1, 1), _attn(8, 4, 128), _attn(16, 4, 64)):
        assert _fwd(packed_plan, cp) == UNSUPPORTED and "packed" in _err()
    assert _fwd(packed_plan, _attn(), ws_bytes=0) == WORKSPACE  # the MFMA shape passes that check


def _gdn(n=16, d=128, dtype=0, grad=0, scale=0.0, keep=0):
    return dpa.DagGdnParams(n, d, dtype, grad, scale, keep)


def _gdn_fwd(plan, cp, q=FAKE, ws=FAKE, ws_bytes=BIG):
    return L.dag_gdn_fwd(plan._h, ctypes.byref(cp), q, FAKE, FAKE, FAKE, FAKE, FAKE, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code,word", [
    ({"n": 0}, UNSUPPORTED, "n_heads"),
    ({"d": 64}, UNSUPPORTED, "head_dim"),
    ({"dtype": 1}, UNSUPPORTED, "dtype"),
    ({"grad": 7}, UNSUPPORTED, "grad_dtype"),
    ({"scale": float("nan")}, INVALID, "scale"),
    ({"scale": float("inf")}, INVALID, "scale"),
    ({"keep": 2}, INVALID, "keep_states"),
])
def test_gdn_parameters_outside_the_kernels_are_refused(gdn_plan, kw, code, word):
    assert _gdn_fwd(gdn_plan, _gdn(**kw)) == code and word in _err()


def test_gdn_needs_a_plan_with_its_schedule_and_enough_workspace(plan, gdn_plan):
    assert _gdn_fwd(plan, _gdn()) == UNSUPPORTED and "gdn_chunk" in _err()
    for keep in (0, 1):
        cp = _gdn(keep=keep)
        f, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
        assert L.dag_gdn_workspace(gdn_plan._h, ctypes.byref(cp), ctypes.byref(f), ctypes.byref(b)) == OK
        assert b.value > 0
        if f.value > 0:
            assert _gdn_fwd(gdn_plan, cp, ws_bytes=f.value - 1) == WORKSPACE and str(f.value) in _err()
        st = L.dag_gdn_bwd(gdn_plan._h, ctypes.byref(cp), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                           FAKE, FAKE, b.value - 1, None)
        assert st == WORKSPACE and str(b.value) in _err()
    assert _gdn_fwd(gdn_plan, _gdn(), q=None) == INVALID and "null" in _err()


def test_plan_queries_check_their_indices(plan):
    n = ctypes.c_int32(0)
    buf = np.zeros(16, np.int32)
    rows = plan.rows
    for r in (-1, rows):
        assert L.dag_plan_readers(plan._h, r, buf.ctypes.data, 16, ctypes.byref(n)) == INVALID and "row" in _err()
    assert L.dag_plan_readers(plan._h, 0, buf.ctypes.data, -1, ctypes.byref(n)) == INVALID
    assert L.dag_plan_readers(plan._h, 0, buf.ctypes.data, 16, None) == INVALID
    assert L.dag_plan_readers(plan._h, 0, buf.ctypes.data, 16, ctypes.byref(n)) == OK and n.value >= 1
    for u in (-1, 1 << 30):
        st = L.dag_plan_node_ranges(plan._h, u, buf.ctypes.data, 16, ctypes.byref(n))
        assert st == INVALID and "node" in _err()
    st = L.dag_plan_gdn_seqs(plan._h, None, 0, ctypes.byref(n))
    assert st == INVALID and "linear-attention" in _err()


@pytest.mark.parametrize("cap", [0, -1, (1 << 20) + 1])
def test_timing_refuses_a_capacity_out_of_range(plan, cap):
    assert L.dag_attn_timing_enable(plan._h, 1, cap) == INVALID and "capacity" in _err()
    assert L.dag_attn_timing_enable(plan._h, 0, cap) == OK  # disabling needs no capacity


@pytest.mark.parametrize("fields,code", [
    ((-1, 0, 10, 0, 0), INVALID), ((1, -1, 10, 0, 0), INVALID), ((1, 0, 0, 0, 0), INVALID),
    ((1, 0, 10, 2, 0), UNSUPPORTED), ((1, 0, 10, 0, 3), UNSUPPORTED), ((1, 1 << 31, 10, 0, 0), 6),
    (((1 << 62), 0, 1 << 20, 0, 0), 6)])
def test_logprob_parameters_are_checked(fields, code):
    p = dpa.DagLogprobParams(*fields)
    st = L.dag_logprob_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == code and _err()


def test_a_plan_without_rows_returns_at_once():
    # every node of length 0: nothing to compute, so no pointer is read (all NULL here)
    b = synth.dags.DagBuilder()
    r = b.node(-1, 0)
    b.node(r, 0)
    for gc in (0, 64):
        empty = dpa.Plan(b.build(), gdn_chunk=gc)
        assert empty.rows == 0
        cp = _attn()
        assert L.dag_attn_fwd(empty._h, ctypes.byref(cp), None, None, None, None, None, None, None, 0, None) == OK
        assert L.dag_attn_bwd(empty._h, ctypes.byref(cp), *([None] * 10), None, 0, None) == OK
        assert _fwd(empty, _attn(n_q=0)) == UNSUPPORTED  # the parameters are still checked
        if gc:
            gp = _gdn()
            assert L.dag_gdn_fwd(empty._h, ctypes.byref(gp), *([None] * 7), 0, None) == OK
            assert L.dag_gdn_bwd(empty._h, ctypes.byref(gp), *([None] * 12), 0, None) == OK
