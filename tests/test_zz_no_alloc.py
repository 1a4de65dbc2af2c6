"""dag_attn_fwd_noalloc (the forward on the library's static device scratch) against
dag_attn_fwd on the same inputs: two calls in a row, the second on a smaller plan, each
bitwise equal to the allocating entry point; plus its host-side refusals."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def dpa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dag_packed_attention_amd as m
    return m


def _inputs(dpa, plan, p, seed):
    tdt = p.torch_dtype
    C = plan.rows
    q = synth.normal((C, p.n_q_heads, p.head_dim), seed, 1, DEV, tdt)
    k = synth.normal((C, p.n_kv_heads, p.head_dim), seed, 2, DEV, tdt)
    v = synth.normal((C, p.n_kv_heads, p.head_dim), seed, 3, DEV, tdt)
    return q, k, v


def _compare(dpa, spec, p, seed):
    plan = dpa.Plan(spec)
    plan.upload()
    q, k, v = _inputs(dpa, plan, p, seed)
    lo_wanted = p.dtype == "bf16"
    if lo_wanted:
        o_ref, lse_ref, lo_ref = dpa.attn_fwd(plan, p, q, k, v, o_lo=True)
    else:
        o_ref, lse_ref = dpa.attn_fwd(plan, p, q, k, v)
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    lo = torch.full_like(o_ref, float("nan")) if lo_wanted else None
    dpa.attn_fwd_noalloc(plan, p, q, k, v, o, lse, o_lo=lo)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    if lo_wanted:
        assert torch.equal(lo, lo_ref)
    return plan


def test_noalloc_forward_matches_allocating_forward(dpa):
    # a larger plan first (2 trees, ~1.9K tokens, MFMA path), then a smaller one (the tiny
    # workload), so the second call runs on scratch still holding the first call's data
    big = synth.dags.config3_structure(5, n_trees=2, seg=(40, 260), depth_hi=3, fan=(2, 3), span=(20, 180))
    print("noalloc: larger plan, bf16 16/4 heads", flush=True)
    p16 = dpa.AttnParams(16, 4, 128, "bf16")
    _compare(dpa, big, p16, 71)
    print("noalloc: smaller plan, bf16 16/4 heads", flush=True)
    _compare(dpa, synth.config1(), p16, 72)
    print("noalloc: smaller plan, fp32 2/2 heads, d = 64", flush=True)
    _compare(dpa, synth.config1(), dpa.AttnParams(2, 2, 64, "fp32"), 73)


def test_noalloc_refusals(dpa):
    p16 = dpa.AttnParams(16, 4, 128, "bf16")
    # a plan not on the device yet: uploading would allocate
    plan = dpa.Plan(synth.config1())
    q, k, v = _inputs(dpa, plan, p16, 5)
    o = torch.empty_like(q)
    lse = torch.empty((plan.rows, 16), dtype=torch.float32, device=DEV)
    with pytest.raises(dpa.DagError) as e:
        dpa.attn_fwd_noalloc(plan, p16, q, k, v, o, lse)
    assert e.value.code == "INVALID"
    # a plan whose workspace exceeds the static 64 MiB (about 30K rows at 16/4 heads)
    spec = synth.config4(n_episodes=1, commander=1024, workers=8, budget=4096, span=1024, first_read=1536,
                         read_step=256)
    big = dpa.Plan(spec)
    need, _ = dpa.workspace_bytes(big, p16)
    assert need > 64 << 20
    big.upload()
    qb, kb, vb = _inputs(dpa, big, p16, 6)
    ob = torch.empty_like(qb)
    lb = torch.empty((big.rows, 16), dtype=torch.float32, device=DEV)
    with pytest.raises(dpa.DagError) as e:
        dpa.attn_fwd_noalloc(big, p16, qb, kb, vb, ob, lb)
    assert e.value.code == "WORKSPACE"
    torch.cuda.synchronize()
