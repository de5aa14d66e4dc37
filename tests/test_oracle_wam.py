"""Pins of the joint video/action (WAM) oracle (CPU)."""
import dataclasses

import numpy as np

import synth
from oracle import expert as ex
from oracle import wam

TINY = synth.WAM_CONFIGS["wam_tiny"]
MICRO = dataclasses.replace(TINY, width=256, n_layers=1, latent_tokens=20, action_tokens=6, n_steps=1,
                            mlp_dim=256, weight_std=0.05)


def _inp(d, seed=0):
    return synth.make_wam_inputs(d, seed)


def test_zero_weights_keep_state():
    d = MICRO
    inp = _inp(d)
    for k, v in list(inp.items()):
        if k.startswith(("w_", "b_")):
            inp[k] = np.zeros_like(v)
    zl, za = wam.denoise(inp, d)
    assert np.array_equal(zl, inp["z_lat"].astype(np.float64))
    assert np.array_equal(za, inp["z_act"].astype(np.float64))


def test_guidance_is_affine_with_unconditional_and_conditional_ends():
    """One step: x(gamma) is affine in gamma, x(0) is the unconditional update and x(1)
    the conditional one.  Catches a wrong combination (e.g. v_c + g (v_c - v_u))."""
    d = MICRO
    inp = _inp(d)
    x = {g: np.concatenate([a.ravel() for a in wam.denoise(inp, d, guidance=g)]) for g in (0.0, 1.0, 2.0, 3.0)}
    np.testing.assert_allclose(x[2.0] - 2 * x[1.0] + x[0.0], 0, atol=1e-12)
    np.testing.assert_allclose(x[3.0] - x[0.0], 3 * (x[1.0] - x[0.0]), atol=1e-12)
    # gamma = 0: only the unconditional branch; gamma = 1: only the conditional branch
    t = ex.schedule(d.n_steps)
    dt = ex.step_sizes(t)[0]
    keys = [k for k in inp if k.startswith(("w_", "b_")) and k not in ("w_mod", "b_mod")]
    p = {k: np.asarray(inp[k], np.float64) for k in keys}
    for g, c in ((0.0, inp["c_uncond"]), (1.0, inp["c_cond"])):
        vl, va = wam.velocity(inp["z_lat"].astype(np.float64), inp["z_act"].astype(np.float64),
                              wam.modulation(t[0], c, inp["w_mod"], inp["b_mod"]), p, d)
        ref = np.concatenate([(inp["z_lat"] + dt * vl).ravel(), (inp["z_act"] + dt * va).ravel()])
        np.testing.assert_allclose(x[g], ref, atol=1e-12)
    # the condition matters (the check is not vacuous)
    assert np.abs(x[1.0] - x[0.0]).max() > 1e-6


def test_equal_conditions_make_guidance_irrelevant():
    d = dataclasses.replace(MICRO, n_steps=2)
    inp = _inp(d)
    inp["c_uncond"] = inp["c_cond"].copy()
    a = np.concatenate([v.ravel() for v in wam.denoise(inp, d, guidance=0.0)])
    b = np.concatenate([v.ravel() for v in wam.denoise(inp, d, guidance=7.0)])
    np.testing.assert_allclose(a, b, atol=1e-12)


def test_modulation_reduces_to_expert_tables_and_is_linear_in_the_condition():
    d = MICRO
    inp = _inp(d)
    t = 0.6
    m0 = wam.modulation(t, np.zeros(d.width), inp["w_mod"], inp["b_mod"])
    np.testing.assert_allclose(m0, ex.modulation_tables([t], inp["w_mod"], inp["b_mod"])[0], atol=1e-12)
    mc = wam.modulation(t, inp["c_cond"], inp["w_mod"], inp["b_mod"])
    lin = np.einsum("jod,d->jo", inp["w_mod"].astype(np.float64), inp["c_cond"].astype(np.float64))
    np.testing.assert_allclose((mc - m0).reshape(lin.shape), lin, atol=1e-12)


def test_velocity_without_actions_is_the_expert_velocity_with_an_empty_prefix():
    """With no action tokens and the zero condition, the WAM layer stack is the (pinned)
    action expert with Hq = Hkv, chunk = latent tokens and no cached prefix."""
    d = dataclasses.replace(MICRO, action_tokens=0, n_layers=2)
    inp = _inp(d)
    mods = wam.modulation(0.4, np.zeros(d.width), inp["w_mod"], inp["b_mod"])
    keys = [k for k in inp if k.startswith(("w_", "b_")) and k not in ("w_mod", "b_mod")]
    p = {k: np.asarray(inp[k], np.float64) for k in keys}
    vl, va = wam.velocity(inp["z_lat"].astype(np.float64), np.zeros((0, d.action_dim)), mods, p, d)
    assert va.shape == (0, d.action_dim)
    ed = synth.ExpertDims(d.n_layers, d.width, d.n_heads, d.n_heads, d.head_dim, d.mlp_dim, 0,
                          d.latent_tokens, d.latent_dim, 1, 1, "bf16")
    pe = {"w_in": p["w_in_lat"], "b_in": p["b_in_lat"], "w_out": p["w_out_lat"], "b_out": p["b_out_lat"],
          "w_qkv": p["w_qkv"], "w_o": p["w_o"], "w_gu": p["w_gu"], "w_d": p["w_d"]}
    empty = np.zeros((d.n_layers, 0, d.n_heads, d.head_dim))
    ve = ex.velocity(inp["z_lat"].astype(np.float64), mods, pe, empty, empty, ed)
    np.testing.assert_allclose(vl, ve, rtol=0, atol=1e-12 * np.abs(ve).max())
