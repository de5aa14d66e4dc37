"""GPU parity of the joint video/action denoiser (guided branch pair) through the C ABI.

Reduced shapes against the float64 oracle (bf16 weights and GEMM inputs, fp32
accumulation: max error / max |ref| <= 2e-2), including the full width, heads, MLP and
token count at one layer and one step; the full 28-layer, 8-step shape through properties
that hold at any size (equal branch conditions make the guidance scale irrelevant,
bitwise; graph replay equals eager launches, bitwise; the state stays finite).
"""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import expert as ex
from oracle import wam as owam

from gpu_util import rel_err

pytestmark = pytest.mark.gpu

TINY = synth.WAM_CONFIGS["wam_tiny"]
FULL = synth.WAM_CONFIGS["wam"]
TOL = 2e-2


def _dev(inputs):
    import torch
    out = {}
    for k, v in inputs.items():
        t = torch.from_numpy(np.ascontiguousarray(v)).cuda()
        out[k] = t if k in ("z_lat", "z_act") else t.to(torch.bfloat16).contiguous()
    return out


def _make(d, dev, t, guidance=None, graph=True):
    import flow_matching_action_cached_amd as fm
    jd = fm.JointDenoiser.from_dims(d)
    jd.set_weights(dev)
    jd.set_conditions(dev["c_cond"], dev["c_uncond"], d.guidance if guidance is None else guidance)
    jd.set_timestep_tables(t)
    jd.set_graph_mode(graph)
    return jd


def _run(jd, dev):
    zl, za = jd.denoise(dev["z_lat"], dev["z_act"])
    jd.sync()
    return zl.cpu().numpy(), za.cpu().numpy()


def _check_vs_oracle(d, seed=0):
    inp = synth.make_wam_inputs(d, seed)
    t = ex.schedule(d.n_steps)
    jd = _make(d, _dev(inp), t)
    zl, za = _run(jd, _dev(inp))
    rl, ra = owam.denoise(inp, d, t)
    got = np.concatenate([zl.ravel(), za.ravel()])
    ref = np.concatenate([rl.ravel(), ra.ravel()])
    err = rel_err(got, ref)
    print(f"joint {d.latent_tokens}+{d.action_tokens} tokens L={d.n_layers} N={d.n_steps}: rel err {err:.3e}",
          flush=True)
    assert np.isfinite(got).all()
    assert err <= TOL
    return jd


def test_joint_tiny_matches_oracle():
    _check_vs_oracle(TINY)


@pytest.mark.parametrize("lat,act", [(0, 24), (37, 0), (5, 3)])
def test_joint_ragged_token_mixes_match_oracle(lat, act):
    """Only actions, only latents, and a token count far from a tile multiple."""
    _check_vs_oracle(dataclasses.replace(TINY, latent_tokens=lat, action_tokens=act, n_steps=2))


def test_joint_modulation_tables_match_oracle():
    d = dataclasses.replace(TINY, n_steps=3)
    inp = synth.make_wam_inputs(d, 1)
    t = ex.schedule(d.n_steps)
    jd = _make(d, _dev(inp), t)
    got = jd.get_modulation().cpu().numpy()           # [N][branch][nmod][2][D]
    for k in range(d.n_steps):
        for b, c in enumerate((inp["c_cond"], inp["c_uncond"])):
            ref = owam.modulation(t[k], c, inp["w_mod"], inp["b_mod"])
            np.testing.assert_allclose(got[k, b], ref, rtol=1e-5, atol=1e-5)


def test_joint_graph_equals_eager_and_replays_bitwise():
    d = TINY
    inp = synth.make_wam_inputs(d, 2)
    dev = _dev(inp)
    t = ex.schedule(d.n_steps)
    g = _make(d, dev, t, graph=True)
    a1 = _run(g, dev)
    a2 = _run(g, dev)
    g.set_graph_mode(False)
    e1 = _run(g, dev)
    for x, y in ((a1, a2), (a1, e1)):
        assert np.array_equal(x[0], y[0]) and np.array_equal(x[1], y[1])


def test_joint_guidance_change_recaptures():
    """A new guidance scale is a new launch argument: the loop must follow it."""
    d = dataclasses.replace(TINY, n_steps=2)
    inp = synth.make_wam_inputs(d, 3)
    dev = _dev(inp)
    t = ex.schedule(d.n_steps)
    jd = _make(d, dev, t, guidance=1.0)
    _run(jd, dev)
    jd.set_conditions(dev["c_cond"], dev["c_uncond"], 5.0)
    jd.set_timestep_tables(t)
    zl, za = _run(jd, dev)
    rl, ra = owam.denoise(inp, d, t, guidance=5.0)
    assert rel_err(np.concatenate([zl.ravel(), za.ravel()]), np.concatenate([rl.ravel(), ra.ravel()])) <= TOL


def test_joint_call_order_and_kind_errors():
    import torch
    import flow_matching_action_cached_amd as fm
    d = TINY
    jd = fm.JointDenoiser.from_dims(d)
    z = torch.zeros((d.latent_tokens, d.latent_dim), device="cuda")
    a = torch.zeros((d.action_tokens, d.action_dim), device="cuda")
    with pytest.raises(fm.PhyaiError) as e:
        jd.set_timestep_tables([1.0, 0.5])            # weights not set
    assert e.value.status == 2
    lib = fm.load_library()
    assert lib.phyai_set_prefix_kv(jd._h, z.data_ptr(), z.data_ptr(), 1, 1) == 2
    assert lib.phyai_denoise(jd._h, z.data_ptr(), 1, 1, z.data_ptr()) == 2
    assert lib.phyai_wam_denoise(jd._h, z.data_ptr(), a.data_ptr(), 1, z.data_ptr(), a.data_ptr()) == 2
    inp = _dev(synth.make_wam_inputs(d, 0))
    jd.set_weights(inp)
    with pytest.raises(fm.PhyaiError) as e:
        jd.set_timestep_tables([1.0, 0.5])            # conditions not set
    assert e.value.status == 2
    assert lib.phyai_wam_set_conditions(jd._h, inp["c_cond"].data_ptr(), inp["c_uncond"].data_ptr(),
                                        float("nan")) == 1
    # an action-expert context refuses the joint calls
    e_ctx = fm.ActionExpert.from_dims(synth.CONFIGS["tiny"])
    assert lib.phyai_wam_denoise(e_ctx._h, z.data_ptr(), a.data_ptr(), 1, z.data_ptr(), a.data_ptr()) == 2
    e_ctx.close()
    jd.close()


@pytest.mark.slow
def test_joint_full_width_one_layer_velocity_matches_oracle():
    """Full width, heads, MLP and token count (2048, 16 x 128, 8192, 4096 + 32 tokens) at
    reduced depth: one layer and one step, so the float64 oracle finishes in seconds.
    The velocity v = (z_1 - z_0) / dt is compared (z_0 would otherwise dominate z_1)."""
    d = dataclasses.replace(FULL, n_layers=1, n_steps=1)
    inp = synth.make_wam_inputs(d, 5)
    t = ex.schedule(d.n_steps)
    dt = float(ex.step_sizes(t)[0])
    jd = _make(d, _dev(inp), t)
    zl, za = _run(jd, _dev(inp))
    jd.close()
    rl, ra = owam.denoise(inp, d, t)
    z0 = np.concatenate([inp["z_lat"].ravel(), inp["z_act"].ravel()]).astype(np.float64)
    got = (np.concatenate([zl.ravel(), za.ravel()]) - z0) / dt
    ref = (np.concatenate([rl.ravel(), ra.ravel()]) - z0) / dt
    err = rel_err(got, ref)
    print(f"joint full width, 1 layer: velocity rel err {err:.3e}", flush=True)
    assert err <= TOL


@pytest.mark.slow
def test_joint_full_shape_properties():
    """28 layers, width 2048, 4096 + 32 tokens, 8 steps, device-drawn inputs.  With both
    branches on the same condition the two halves of every GEMM and attention launch see
    identical rows, so v_c == v_u bitwise and the guidance scale must not change one bit."""
    import torch
    d = FULL
    dev = synth.wam_device_inputs(d, 0)
    dev["c_uncond"] = dev["c_cond"].clone()
    t = ex.schedule(d.n_steps)
    jd = _make(d, dev, t, guidance=0.0)
    a = _run(jd, dev)
    jd.set_conditions(dev["c_cond"], dev["c_uncond"], 7.0)
    jd.set_timestep_tables(t)
    b = _run(jd, dev)
    assert np.isfinite(a[0]).all() and np.isfinite(a[1]).all()
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # distinct conditions: guidance now matters, state finite, eager == graph
    c_unc = torch.zeros_like(dev["c_cond"])
    jd.set_conditions(dev["c_cond"], c_unc, 3.0)
    jd.set_timestep_tables(t)
    g = _run(jd, dev)
    jd.set_graph_mode(False)
    e = _run(jd, dev)
    assert np.isfinite(g[0]).all() and np.isfinite(g[1]).all()
    assert not np.array_equal(g[0], a[0])
    assert np.array_equal(g[0], e[0]) and np.array_equal(g[1], e[1])
    jd.close()


# ---------------------------------------------------------------- UniPC solver
def _make_solver(d, dev, t, order, graph=True):
    import flow_matching_action_cached_amd as fm
    jd = fm.JointDenoiser.from_dims(d, solver_order=order)
    jd.set_weights(dev)
    jd.set_conditions(dev["c_cond"], dev["c_uncond"], d.guidance)
    jd.set_timestep_tables(t)
    jd.set_graph_mode(graph)
    return jd


@pytest.mark.parametrize("order,sched", [(1, "uniform"), (2, "uniform"), (2, "below_one")])
def test_joint_unipc_matches_oracle(order, sched):
    """UniPC (corrector on) over 5 steps: from t = 1 (uniform schedule) and from t = 0.9 with
    uneven steps, where every corrector and predictor weight is non-zero; the result is the
    oracle's, more than ten times closer to it than the Euler loop's."""
    d = dataclasses.replace(TINY, n_steps=5)
    inp = synth.make_wam_inputs(d, 2)
    t = ex.schedule(d.n_steps) if sched == "uniform" else np.array([0.9, 0.7, 0.55, 0.3, 0.15], np.float32)
    dev = _dev(inp)
    jd = _make_solver(d, dev, t, order)
    zl, za = _run(jd, dev)
    jd.close()
    rl, ra = owam.denoise(inp, d, t, solver_order=order)
    el, ea = owam.denoise(inp, d, t)
    got = np.concatenate([zl.ravel(), za.ravel()])
    ref = np.concatenate([rl.ravel(), ra.ravel()])
    eul = np.concatenate([el.ravel(), ea.ravel()])
    err = rel_err(got, ref)
    print(f"joint UniPC order {order} ({sched}): rel err {err:.3e}, vs Euler {rel_err(eul, ref):.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err <= TOL
    assert rel_err(eul, ref) > 10 * err              # far closer to UniPC than the Euler loop is


def test_joint_unipc_ragged_mix_and_graph_equals_eager():
    """A token count off the tile grid (5 latent + 3 action tokens), order 2: oracle parity,
    and graph replay equals eager launches bitwise (the state buffers rotate per step)."""
    d = dataclasses.replace(TINY, latent_tokens=5, action_tokens=3, n_steps=4)
    inp = synth.make_wam_inputs(d, 3)
    t = ex.schedule(d.n_steps)
    dev = _dev(inp)
    jg = _make_solver(d, dev, t, 2, graph=True)
    je = _make_solver(d, dev, t, 2, graph=False)
    a = _run(jg, dev)
    b = _run(jg, dev)
    c = _run(je, dev)
    jg.close()
    je.close()
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])
    rl, ra = owam.denoise(inp, d, t, solver_order=2)
    err = rel_err(np.concatenate([a[0].ravel(), a[1].ravel()]), np.concatenate([rl.ravel(), ra.ravel()]))
    print(f"joint UniPC ragged 5+3: rel err {err:.3e}", flush=True)
    assert err <= TOL


def test_joint_unipc_rejects_schedules_it_cannot_take():
    import flow_matching_action_cached_amd as fm
    d = dataclasses.replace(TINY, n_steps=3)
    dev = _dev(synth.make_wam_inputs(d, 0))
    jd = _make_solver(d, dev, ex.schedule(3), 2)
    for bad in ([1.2, 0.5, 0.2], [0.9, 0.9, 0.2], [0.9, 0.5, 0.0], [0.3, 0.5, 0.2]):
        with pytest.raises(fm.PhyaiError):
            jd.set_timestep_tables(np.array(bad, np.float32))
    jd.close()


@pytest.mark.slow
def test_joint_unipc_full_width_one_layer_matches_oracle():
    """Full width, heads, MLP and token count at one layer, UniPC order 2 over three steps
    from t = 0.9 (every predictor and corrector weight non-zero): the displacement z_N - z_0
    is the oracle's, and more than ten times closer to it than the Euler loop's."""
    d = dataclasses.replace(FULL, n_layers=1, n_steps=3)
    inp = synth.make_wam_inputs(d, 6)
    t = np.array([0.9, 0.6, 0.3], np.float32)
    dev = _dev(inp)
    ju = _make_solver(d, dev, t, 2)
    gu = _run(ju, dev)
    ju.close()
    je = _make(d, dev, t)
    ge = _run(je, dev)
    je.close()
    rl, ra = owam.denoise(inp, d, t, solver_order=2)
    z0 = np.concatenate([inp["z_lat"].ravel(), inp["z_act"].ravel()]).astype(np.float64)
    got = np.concatenate([gu[0].ravel(), gu[1].ravel()]) - z0
    eul = np.concatenate([ge[0].ravel(), ge[1].ravel()]) - z0
    ref = np.concatenate([rl.ravel(), ra.ravel()]) - z0
    err = rel_err(got, ref)
    print(f"joint UniPC full width, 1 layer, 3 steps: displacement rel err {err:.3e}, "
          f"Euler {rel_err(eul, ref):.3e}", flush=True)
    assert err <= TOL
    assert rel_err(eul, ref) > 10 * err


@pytest.mark.slow
def test_joint_unipc_single_step_equals_euler_at_full_shape():
    """One step from t = 1 to 0 is first order for both solvers (z_1 = z_0 - v): at the full
    28-layer shape the UniPC context returns the Euler context's result bit for bit."""
    d = dataclasses.replace(FULL, n_steps=1)
    dev = synth.wam_device_inputs(d, 0)
    t = ex.schedule(1)
    je, ju = _make(d, dev, t), _make_solver(d, dev, t, 2)
    a, b = _run(je, dev), _run(ju, dev)
    je.close()
    ju.close()
    assert np.isfinite(a[0]).all() and np.isfinite(a[1]).all()
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.slow
def test_joint_tp4_rank_shard_one_layer_velocity_matches_oracle():
    """The shapes one rank of a 4-way tensor-parallel branch computes (4 of 16 heads, a
    quarter of the MLP: QKV 2048 -> 1536, O 512 -> 2048, gate/up 2048 -> 4096, down
    2048 -> 2048, attention over all 4128 tokens), one layer and one step vs the oracle."""
    d = dataclasses.replace(FULL, n_layers=1, n_steps=1, n_heads=4, mlp_dim=2048)
    inp = synth.make_wam_inputs(d, 7)
    t = ex.schedule(d.n_steps)
    dt = float(ex.step_sizes(t)[0])
    jd = _make(d, _dev(inp), t)
    zl, za = _run(jd, _dev(inp))
    jd.close()
    rl, ra = owam.denoise(inp, d, t)
    z0 = np.concatenate([inp["z_lat"].ravel(), inp["z_act"].ravel()]).astype(np.float64)
    got = (np.concatenate([zl.ravel(), za.ravel()]) - z0) / dt
    ref = (np.concatenate([rl.ravel(), ra.ravel()]) - z0) / dt
    err = rel_err(got, ref)
    print(f"joint TP-4 rank shard, 1 layer: velocity rel err {err:.3e}", flush=True)
    assert err <= TOL
