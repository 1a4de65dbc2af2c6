"""Malformed inputs to the host entry points come back as a status, never a crash."""
import ctypes

import numpy as np
import pytest

import dag_packed_attention_amd as dpa

L = dpa._lib
TOK = np.array([1, 2, 3, 1, 2, 4], np.int32)


def _trie(off, n, tokens=True, counts=True):
    off = np.asarray(off, np.int64)
    nn, nt = ctypes.c_int32(0), ctypes.c_int64(0)
    return L.dag_trie_build(TOK.ctypes.data if tokens else None, off.ctypes.data, n, 0, None, None, 0, None, None,
                            ctypes.byref(nn) if counts else None, ctypes.byref(nt) if counts else None)


@pytest.mark.parametrize("off,n,kw", [
    ([0, 3, 6], -1, {}), ([0], 0, {}), ([1, 3, 6], 2, {}), ([0, 4, 3], 2, {}), ([0, -3, 6], 2, {}),
    ([0, 3, 6], 2, {"tokens": False}), ([0, 3, 6], 2, {"counts": False})])
def test_trie_rejects_malformed_trajectories(off, n, kw):
    assert _trie(off, n, **kw) == 1                      # DAG_E_INVALID
    assert L.dag_last_error()


def test_trie_counts_only_when_outputs_are_short():
    nn, nt = ctypes.c_int32(0), ctypes.c_int64(0)
    off = np.array([0, 3, 6], np.int64)
    assert _trie(off, 2) == 0
    st = L.dag_trie_build(TOK.ctypes.data, off.ctypes.data, 2, 1, (dpa.DagNode * 1)(), np.zeros(2, np.int64).ctypes.data,
                          1, np.zeros(1, np.int32).ctypes.data, np.zeros(2, np.int32).ctypes.data, ctypes.byref(nn),
                          ctypes.byref(nt))
    assert st == 0 and nn.value == 3 and nt.value == 4    # root [1, 2] with leaves [3] and [4]


def _mb(replicas, exact_max, capacity, off=(0, 3, 6), n=2, opts=True):
    off = np.asarray(off, np.int64)
    o = dpa.DagMbOpts(replicas, exact_max, capacity)
    info = dpa.DagMbInfo()
    return L.dag_microbatch_plan(TOK.ctypes.data, off.ctypes.data, n, ctypes.byref(o) if opts else None, None, 0,
                                 None, None, None, ctypes.byref(info))


@pytest.mark.parametrize("args,kw", [
    ((0, 0, 10), {}), ((-1, 0, 10), {}), ((1, 0, 0), {}), ((1, 0, 2), {}), ((1, -5, 10), {}),
    ((1, 0, 10), {"off": (0,), "n": 0}), ((5, 0, 10), {}), ((1, 0, 10), {"off": (0, 4, 3)}),
    ((1, 0, 10), {"opts": False})])
def test_microbatch_plan_rejects_malformed_requests(args, kw):
    assert _mb(*args, **kw) == 1
    assert L.dag_last_error()


def test_microbatch_plan_accepts_a_plain_request():
    assert _mb(1, 0, 10) == 0
    assert _mb(2, 0, 10) == 0


def test_bf16_backward_refuses_a_missing_residual():
    # decided on the host before any device call: the pointers are never dereferenced
    import synth
    plan = dpa.Plan(synth.config1())
    cp = dpa.AttnParams(16, 4, 128, "bf16").c()
    fake = ctypes.c_void_p(0x1000)
    ws = ctypes.c_void_p(0x2000)
    st = L.dag_attn_bwd(plan._h, ctypes.byref(cp), fake, fake, fake, fake, fake, None, fake, fake, fake, fake, ws,
                        1 << 40, None)
    assert st == 1 and "o_lo" in L.dag_last_error().decode()
    cp32 = dpa.AttnParams(2, 2, 64, "fp32").c()
    st = L.dag_attn_bwd(plan._h, ctypes.byref(cp32), fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, ws,
                        1 << 40, None)
    assert st == 1 and "o_lo" in L.dag_last_error().decode()


@pytest.mark.parametrize("scale", [-0.5, float("inf"), float("nan")])
def test_attention_refuses_a_negative_or_non_finite_scale(scale):
    # decided on the host before any device call: the pointers are never dereferenced
    import synth
    plan = dpa.Plan(synth.config1())
    cp = dpa.AttnParams(16, 4, 128, "bf16", scale=scale).c()
    fake = ctypes.c_void_p(0x1000)
    st = L.dag_attn_fwd(plan._h, ctypes.byref(cp), fake, fake, fake, fake, fake, fake, fake, 1 << 40, None)
    assert st == 1 and "scale" in L.dag_last_error().decode()
