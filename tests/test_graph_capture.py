"""Graph capture of the device entry points (GPU).

Once a plan is on the device (dag_plan_upload), the attention forward and backward and the
gated-delta-rule layer only launch kernels on the caller's stream: no allocation, no
synchronisation, no memset.  So a HIP graph captured around them replays the same
computation.  Each test captures the calls once, then replays the graph three times; between
replays the outputs are overwritten with NaN by ordinary eager work and the device is
synchronised, and every replay must reproduce the eager call's outputs bit for bit.
"""
import pytest

import dag_packed_attention_amd as dpa
import synth

pytestmark = pytest.mark.gpu


def _mini3():
    return synth.dags.config3_structure(5, n_trees=2, seg=(40, 260), depth_hi=3, fan=(2, 3), span=(20, 180))


def _bits(t):
    import torch
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


def _replay_matches(step, outs):
    import torch
    step()  # eager reference
    torch.cuda.synchronize()
    ref = [_bits(t).clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up off the default stream, as graph capture expects
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(outs, ref)):
            assert torch.equal(_bits(t), r), f"replay {rep}: output {i} differs from the eager call"


@pytest.mark.parametrize("grad_dtype", ["bf16", "fp32"])
def test_attention_forward_and_backward_replay_from_a_graph(grad_dtype):
    import torch
    dev = "cuda:0"
    plan = dpa.Plan(_mini3())
    plan.upload()
    p = dpa.AttnParams(16, 4, 128, "bf16", grad_dtype=grad_dtype)
    C = plan.rows
    g = torch.Generator(device=dev).manual_seed(21)
    mk = lambda h: torch.randn(C, h, 128, device=dev, generator=g).to(torch.bfloat16)  # noqa: E731
    q, k, v, dO = mk(16), mk(4), mk(4), mk(16)
    fw, bw = dpa.workspace_bytes(plan, p)
    ws = torch.empty(max(fw, bw), dtype=torch.uint8, device=dev)
    o, o_lo = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty((C, 16), dtype=torch.float32, device=dev)
    gdt = p.torch_grad_dtype
    dq = torch.empty(q.shape, dtype=gdt, device=dev)
    dk = torch.empty(k.shape, dtype=gdt, device=dev)
    dv = torch.empty(v.shape, dtype=gdt, device=dev)

    def step():
        dpa.attn_fwd(plan, p, q, k, v, o=o, lse=lse, ws=ws, o_lo=o_lo)
        dpa.attn_bwd(plan, p, q, k, v, o, lse, dO, dq=dq, dk=dk, dv=dv, ws=ws, o_lo=o_lo)

    _replay_matches(step, (o, lse, o_lo, dq, dk, dv))


@pytest.mark.parametrize("keep", [False, True])
def test_gated_delta_rule_layer_replays_from_a_graph(keep):
    import torch
    dev = "cuda:0"
    plan = dpa.Plan(_mini3(), gdn_chunk=64)
    plan.upload()
    C, H = plan.rows, 4
    q, k, v, b, a, dO = synth.gdn_inputs(C, H, 128, 128, 31, device=dev, dtype=torch.bfloat16)
    p = dpa.GdnParams(H, grad_dtype="fp32", keep_states=keep)
    fw, bw = dpa.gdn_workspace_bytes(plan, p)
    ws = torch.empty(max(fw, bw, 1), dtype=torch.uint8, device=dev)
    o = torch.empty_like(v)
    grads = (torch.empty(q.shape, dtype=torch.float32, device=dev), torch.empty(k.shape, dtype=torch.float32, device=dev),
             torch.empty(v.shape, dtype=torch.float32, device=dev), torch.empty_like(b), torch.empty_like(a))

    def step():
        dpa.gdn_fwd(plan, p, q, k, v, b, a, o=o, ws=ws)
        dpa.gdn_bwd(plan, p, q, k, v, b, a, dO, ws=ws, out=grads)

    _replay_matches(step, (o,) + grads)
