"""dag_plan_stats_get: the attention kernels' walk and staging volume, from the plan tables
(host only)."""
import pytest

import dag_packed_attention_amd as dpa
import synth

TILE = 64 * 128 * 2             # one fp16 64 x 128 tile
UNIT = 2 * 2 * 32 * 128 * 2 + 2 * 256  # a half-step: two heads' Q and dO rows, their offsets


@pytest.mark.parametrize("name,spec,pack", [
    ("chain", synth.config1(), False),
    ("mini3", synth.dags.config3_structure(5, n_trees=2, seg=(40, 260), depth_hi=3, fan=(2, 3), span=(20, 180)), False),
    ("short", synth.dags.config3_structure(7, n_trees=2, seg=(1, 64), depth_hi=3, fan=(2, 4)), False),
    ("short_packed", synth.dags.config3_structure(7, n_trees=2, seg=(1, 64), depth_hi=3, fan=(2, 4)), True),
])
def test_stats_agree_with_the_plan(name, spec, pack):
    plan = dpa.Plan(spec, pack=pack)
    st = plan.stats()
    # the forward and dQ visit every query page's tile list once
    assert st["fwd_tiles"] == plan.info["fwd_tiles"] > 0
    assert st["fwd_staged_bytes"] == st["dq_staged_bytes"] == st["fwd_tiles"] * 2 * TILE
    # every KV page belongs to exactly one group or pair, which loads its K and V once
    steps = st["dkdv_group_steps"] + st["dkdv_pair_steps"]
    assert steps > 0
    assert st["dkdv_staged_bytes"] == steps * 2 * UNIT + plan.info["pages"] * 2 * TILE
    assert st["dkdv_groups"] + st["dkdv_pairs"] > 0
    if pack:
        assert st["dkdv_groups"] == 0  # packed plans run every page in pairs
    # a step reads at least one page of its group or pair: no more steps than 32-row halves
    # of the reader lists
    assert steps <= 2 * plan.info["bwd_entries"] * 64


def test_groups_for_long_nodes():
    plan = dpa.Plan(synth.dags.config3_structure(5, n_trees=2, seg=(300, 900), depth_hi=2, fan=(2, 3)))
    st = plan.stats()
    assert st["dkdv_groups"] > 0 and st["dkdv_group_steps"] > 0
