"""Helpers shared by the GPU tests: move the seeded synthetic inputs to the device
and drive the library through its Python binding (which calls the C ABI)."""
import dataclasses

import numpy as np

import synth

WEIGHT_KEYS = ("w_in", "b_in", "w_out", "b_out", "w_mod", "b_mod", "w_qkv", "w_o", "w_gu", "w_d")
LINEARS = ("w_qkv", "w_o", "w_gu", "w_d")


def torch_dtype(d):
    import torch
    return torch.float32 if d.weight_dtype == "f32" else torch.bfloat16


def device_inputs(d, inputs):
    """dict of cuda tensors in the library's element types (int4: linears are
    quantised on the GPU by the library's own quantiser)."""
    import torch
    import flow_matching_action_cached_amd as fm
    el = torch_dtype(d)
    out = {}
    for k in WEIGHT_KEYS + tuple(k for k in ("w_tm1", "b_tm1", "w_tm2", "b_tm2") if k in inputs):
        a = torch.from_numpy(np.ascontiguousarray(inputs[k])).cuda()
        if d.weight_dtype == "int4" and k in LINEARS:
            packed, scales = fm.quantize_int4_g128(a)
            out[k] = packed
            out["s" + k[1:]] = scales
        else:
            out[k] = a.to(el).contiguous()
    out["k_pre"] = torch.from_numpy(inputs["k_pre"]).cuda().to(el).contiguous()
    out["v_pre"] = torch.from_numpy(inputs["v_pre"]).cuda().to(el).contiguous()
    out["noise"] = torch.from_numpy(inputs["noise"]).cuda().contiguous()
    return out


def make_expert(d, dev, t, graph=True, **kw):
    import flow_matching_action_cached_amd as fm
    ex = fm.ActionExpert.from_dims(d, **kw)
    w = {k: dev[k] for k in WEIGHT_KEYS}
    for k in ("s_qkv", "s_o", "s_gu", "s_d", "w_tm1", "b_tm1", "w_tm2", "b_tm2"):
        if k in dev:
            w[k] = dev[k]
    ex.set_weights(w)
    ex.set_prefix_kv(dev["k_pre"], dev["v_pre"])
    ex.set_timestep_tables(t)
    ex.set_graph_mode(graph)
    return ex


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
