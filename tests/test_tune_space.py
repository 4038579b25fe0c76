"""The tuner's search space (no GPU): every knob it moves exists on
ScheduleConfig, and every single-knob candidate lowers to a schedule the
static gate accepts on the full-size 8B shape, so the GPU search never spends
a run on a candidate the engine would refuse."""
import persistent_megakernel_wg_amd as amk
import synth
from persistent_megakernel_wg_amd import tune


def test_space_knobs_exist_and_candidates_are_safe():
    m = amk.ModelConfig.from_workload(synth.get("8b"))
    for knob, values in tune.SPACE:
        assert hasattr(amk.default_schedule_config(m, 256), knob), knob
        for v in values:
            c = tune.apply(amk.default_schedule_config(m, 256), {knob: v})
            s = amk.Schedule.build(m, c)
            assert s.validate() == (0, -1, -1, -1), (knob, v)
            s.close()


def test_apply_sets_array_knobs_elementwise():
    m = amk.ModelConfig.from_workload(synth.get("8b"))
    w = [[1000] * 8, [1000] * 8, [900, 1100] * 4, [1000] * 8, [1000] * 8]
    c = tune.apply(amk.default_schedule_config(m, 256), {"xcd_weight": w, "attn_splits": 24})
    assert [list(r) for r in c.xcd_weight] == w and c.attn_splits == 24
