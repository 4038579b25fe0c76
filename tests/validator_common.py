"""Helpers shared by the safety-gate tests: the library's verdict on a plain
schedule dict, and conversions between the library's schedule view and the
dict form the oracle reads (model as a plain dict)."""
import copy

import persistent_megakernel_wg_amd as amk

MODEL_FIELDS = ("n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "ffn", "vocab", "max_ctx",
                "wfmt")


def model_dict(m):
    return {k: int(getattr(m, k)) for k in MODEL_FIELDS}


def lib_model(d):
    m = amk.ModelConfig()
    for k in MODEL_FIELDS:
        setattr(m, k, int(d[k]))
    m.rms_eps, m.rope_theta = 1e-5, 10000.0
    return m


def lib_verdict(s):
    """(code, task, counter, aux) from amk_validate on a schedule dict."""
    d = dict(s)
    if isinstance(d.get("model"), dict):
        d["model"] = lib_model(d["model"])
    sch = amk.Schedule.from_dict(d)
    try:
        return tuple(sch.validate())
    finally:
        sch.close()


def lowered(model, **cfg):
    """Schedule dict of the library's lowering of `model` (a ModelConfig)."""
    c = amk.default_schedule_config(model, cfg.pop("num_cus", 8))
    for k, v in cfg.items():
        setattr(c, k, v)
    sch = amk.Schedule.build(model, c)
    v = sch.view()
    sch.close()
    v["model"] = model_dict(model)
    del v["config"]
    v["queues"] = [list(map(int, q)) for q in v["queues"]]
    for t in v["tasks"]:
        t["waits"] = [(int(c_), int(th)) for c_, th in t["waits"]]
        t["sigs"] = [int(x) for x in t["sigs"]]
        t["acc"] = [tuple(int(x) for x in a) for a in t["acc"]]
    v["buffers"] = [(int(a), int(b)) for a, b in v["buffers"]]
    return v


def clone(s):
    return copy.deepcopy(s)
