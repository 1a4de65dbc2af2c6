"""The device debug build (libdag_attn_debug.so, every source compiled with DAG_DEBUG;
the binding loads it when DAG_ATTN_DEBUG=1).

CPU: it exists beside the release library, exports the same entry points, and
reports itself through dag_debug_build().
GPU: run in a child process (the library is chosen at import), on valid plans in both
page layouts its plan-table checks pass and every output is bitwise the release
build's; with the page limit lowered by dag_debug_limit_pages (page ids are then
redirected to page 0, so every access stays inside its buffer) the forward and the
backward report DAG_E_INVALID naming a failed check, and the next call with the limit
restored passes again.
"""
import ctypes
import json
import os
import re
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "dag_packed_attention_amd")
RELEASE = os.path.join(PKG, "libdag_attn.so")
DEBUG = os.path.join(PKG, "libdag_attn_debug.so")


def _declared():
    text = open(os.path.join(ROOT, "include", "dag_attn.h")).read()
    return sorted(set(re.findall(r"\b(dag_[a-z0-9_]+)\s*\(", text)))


def test_debug_library_exports_the_same_entry_points():
    import dag_packed_attention_amd  # noqa: F401  (builds the release library if missing)
    if not os.path.exists(DEBUG):
        from dag_packed_attention_amd import build_lib
        build_lib.build(debug=True)
    rel, dbg = ctypes.CDLL(RELEASE), ctypes.CDLL(DEBUG)
    for name in _declared():
        assert hasattr(rel, name), f"release build lacks {name}"
        assert hasattr(dbg, name), f"debug build lacks {name}"
    for lib, want in ((rel, 0), (dbg, 1)):
        lib.dag_debug_build.restype = ctypes.c_int32
        assert lib.dag_debug_build() == want
    rel.dag_debug_limit_pages.argtypes = [ctypes.c_int32]
    assert rel.dag_debug_limit_pages(1) == 8  # DAG_E_UNSUPPORTED outside the debug build


CHILD = r"""
import json, sys
import numpy as np, torch
sys.path.insert(0, sys.argv[1])
import dag_packed_attention_amd as dpa
import synth
assert dpa._lib.dag_debug_build() == 1, "not the debug build"
out = sys.argv[2]
res = {}
for name, pack in (("mini3", False), ("mini_short", True)):
    spec = (synth.dags.config3_structure(5, n_trees=2, seg=(40, 260), depth_hi=3, fan=(2, 3), span=(20, 180))
            if name == "mini3" else synth.dags.config3_structure(7, n_trees=2, seg=(1, 64), depth_hi=3, fan=(2, 4)))
    plan = dpa.Plan(spec, pack=pack)
    p = dpa.AttnParams(16, 4, 128, "bf16", grad_dtype="fp32")
    q, k, v, do = synth.attn_inputs(spec.n_tokens, 16, 4, 128, seed=1201, dtype=torch.bfloat16)
    rows = lambda x: dpa.to_rows(plan, x.to("cuda:0"))
    qr, kr, vr, dr = rows(q), rows(k), rows(v), rows(do)
    o, lse, o_lo = dpa.attn_fwd(plan, p, qr, kr, vr, o_lo=True)
    dq, dk, dv = dpa.attn_bwd(plan, p, qr, kr, vr, o, lse, dr, o_lo=o_lo)
    torch.cuda.synchronize()
    np.savez(f"{out}/{name}.npz", **{n: t.float().cpu().numpy() for n, t in
                                       (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))})
    # the checks themselves: page ids >= 1 now fail (and read page 0 instead)
    assert dpa._lib.dag_debug_limit_pages(1) == 0
    for what, call in (("fwd", lambda: dpa.attn_fwd(plan, p, qr, kr, vr, o=o, lse=lse, o_lo=o_lo)),
                       ("bwd", lambda: dpa.attn_bwd(plan, p, qr, kr, vr, o, lse, dr, dq=dq, dk=dk, dv=dv,
                                                    o_lo=o_lo))):
        try:
            call()
            res[f"{name}_{what}_limited"] = "passed"
        except dpa.DagError as e:
            res[f"{name}_{what}_limited"] = str(e)
    assert dpa._lib.dag_debug_limit_pages(0) == 0
    dpa.attn_fwd(plan, p, qr, kr, vr, o=o, lse=lse, o_lo=o_lo)
    torch.cuda.synchronize()
    res[f"{name}_restored"] = "passed"
json.dump(res, open(f"{out}/result.json", "w"))
print("child done", flush=True)
"""


@pytest.mark.gpu
def test_debug_build_on_device(tmp_path):
    import torch

    import dag_packed_attention_amd as dpa
    import synth
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(DEBUG), "build the debug library first (build_lib.build(debug=True))"
    env = dict(os.environ, DAG_ATTN_DEBUG="1")
    print("debug build: child process on mini3 and mini_short", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT, str(tmp_path)], env=env, capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    res = json.load(open(tmp_path / "result.json"))
    for name, pack in (("mini3", False), ("mini_short", True)):
        for what in ("fwd", "bwd"):
            msg = res[f"{name}_{what}_limited"]
            assert msg != "passed", f"{name} {what}: the lowered page limit went unnoticed"
            assert "INVALID" in msg and "device check" in msg, msg
        assert res[f"{name}_restored"] == "passed"
        # the release build on the same inputs: bitwise the same outputs
        spec = (synth.dags.config3_structure(5, n_trees=2, seg=(40, 260), depth_hi=3, fan=(2, 3), span=(20, 180))
                if name == "mini3" else synth.dags.config3_structure(7, n_trees=2, seg=(1, 64), depth_hi=3,
                                                                     fan=(2, 4)))
        plan = dpa.Plan(spec, pack=pack)
        p = dpa.AttnParams(16, 4, 128, "bf16", grad_dtype="fp32")
        q, k, v, do = synth.attn_inputs(spec.n_tokens, 16, 4, 128, seed=1201, dtype=torch.bfloat16)
        rows = lambda x: dpa.to_rows(plan, x.to("cuda:0"))
        qr, kr, vr, dr = rows(q), rows(k), rows(v), rows(do)
        o, lse, o_lo = dpa.attn_fwd(plan, p, qr, kr, vr, o_lo=True)
        dq, dk, dv = dpa.attn_bwd(plan, p, qr, kr, vr, o, lse, dr, o_lo=o_lo)
        torch.cuda.synchronize()
        got = np.load(tmp_path / f"{name}.npz")
        for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
            assert np.array_equal(got[n], t.float().cpu().numpy(), equal_nan=True), f"{name} {n}: differs"
