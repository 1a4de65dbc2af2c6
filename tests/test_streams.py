"""One plan serving several streams at once (GPU).

A built plan is read-only on the device; everything a call writes lives in the caller's
workspace and outputs.  So calls on two streams with their own inputs, workspaces and
outputs may run concurrently: each stream's results must equal, bit for bit, the same
call made alone on the default stream.
"""
import pytest

import dag_packed_attention_amd as dpa
import synth

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


def test_attention_on_two_streams_with_one_plan():
    import torch
    dev = "cuda:0"
    plan = dpa.Plan(synth.dags.config3_structure(5, n_trees=2, seg=(40, 260), depth_hi=3, fan=(2, 3), span=(20, 180)))
    plan.upload()
    p = dpa.AttnParams(16, 4, 128, "bf16", grad_dtype="fp32")
    C = plan.rows
    fw, bw = dpa.workspace_bytes(plan, p)

    def case(seed):
        g = torch.Generator(device=dev).manual_seed(seed)
        mk = lambda h: torch.randn(C, h, 128, device=dev, generator=g).to(torch.bfloat16)  # noqa: E731
        t = {"q": mk(16), "k": mk(4), "v": mk(4), "dO": mk(16)}
        t["ws"] = torch.empty(max(fw, bw), dtype=torch.uint8, device=dev)
        return t

    def run(t, stream=None):
        o, lse, o_lo = dpa.attn_fwd(plan, p, t["q"], t["k"], t["v"], ws=t["ws"], o_lo=True, stream=stream)
        dq, dk, dv = dpa.attn_bwd(plan, p, t["q"], t["k"], t["v"], o, lse, t["dO"], ws=t["ws"], o_lo=o_lo,
                                  stream=stream)
        return o, lse, dq, dk, dv

    cases = [case(41), case(42)]
    alone = []
    for t in cases:
        alone.append([_bits(x).clone() for x in run(t)])
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(2):
        outs = []
        for t, s in zip(cases, streams):  # issued back to back: the two streams overlap
            with torch.cuda.stream(s):
                outs.append(run(t, stream=s))
        torch.cuda.synchronize()
        for i, (res, ref) in enumerate(zip(outs, alone)):
            for j, (x, r) in enumerate(zip(res, ref)):
                assert torch.equal(_bits(x), r), f"repeat {rep}, stream {i}, output {j}"
