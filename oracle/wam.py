"""float64 oracle of the joint video/action (WAM) denoiser with classifier-free guidance
(TEST INFRASTRUCTURE).

Page anchors: PhyAI reading ("PhyAI: Real-Time Physical AI at the Edge, Scalable
Rollouts in the Cloud"), Figure 4 and Sec. 5.5 third item: video and action tokens stay
in one generation sequence; the conditional and unconditional branches are combined
with a guidance scale (3.0 in the batch sweep, Sec. 6.2) before every rank advances its
video/action state; skipping the video decode does not remove the joint latent
evolution (Sec. 5.4).  The guidance combination (the reading's Eq. (10)) is described
only in words; the plainest reading is the usual classifier-free guidance
v = v_u + gamma (v_c - v_u).

Readings (the pages give no architecture): per-type linear in/out projections (latent
tokens and action tokens) around the same pre-norm transformer layer as the action
expert (adaptive RMSNorm, QKV, attention, O, GeGLU MLP), here with equal query and KV
heads and full self-attention over all tokens (no cache, no mask); the branch condition
vector is added to the timestep embedding before the modulation map (the unconditional
branch uses the zero vector); the update is first-order Euler with the expert's
schedule.
"""
from __future__ import annotations

import numpy as np

from . import expert as ex

F64 = np.float64


def modulation(t, cond, w_mod, b_mod) -> np.ndarray:
    """[n_mod][2][D] of one step and branch: W_m[j] (e(t) + c) + b_m[j]."""
    w_mod = np.asarray(w_mod, F64)
    n_mod, _, d = w_mod.shape
    e = ex.timestep_embedding(t, d) + np.asarray(cond, F64)
    m = np.einsum("jod,d->jo", w_mod, e) + np.asarray(b_mod, F64)
    return m.reshape(n_mod, 2, d)


def velocity(z_lat, z_act, mods, p, d):
    """Velocity of all latent and action tokens for one branch."""
    hq, dh, f = d.n_heads, d.head_dim, d.mlp_dim
    h = np.concatenate([z_lat @ p["w_in_lat"].T + p["b_in_lat"], z_act @ p["w_in_act"].T + p["b_in_act"]])
    n = h.shape[0]
    for l in range(d.n_layers):
        u = ex.ada_rms(h, mods[2 * l][0], mods[2 * l][1], d.rms_eps)
        qkv = u @ p["w_qkv"][l].T
        q = qkv[:, :hq * dh].reshape(n, hq, dh).transpose(1, 0, 2)
        k = qkv[:, hq * dh:2 * hq * dh].reshape(n, hq, dh).transpose(1, 0, 2)
        v = qkv[:, 2 * hq * dh:].reshape(n, hq, dh).transpose(1, 0, 2)
        o = ex.attention(q, k, v).transpose(1, 0, 2).reshape(n, hq * dh)
        h = h + o @ p["w_o"][l].T
        u = ex.ada_rms(h, mods[2 * l + 1][0], mods[2 * l + 1][1], d.rms_eps)
        gu = u @ p["w_gu"][l].T
        h = h + (ex.gelu_tanh(gu[:, :f]) * gu[:, f:]) @ p["w_d"][l].T
    L = d.n_layers
    u = ex.ada_rms(h, mods[2 * L][0], mods[2 * L][1], d.rms_eps)
    nl = z_lat.shape[0]
    return u[:nl] @ p["w_out_lat"].T + p["b_out_lat"], u[nl:] @ p["w_out_act"].T + p["b_out_act"]


def denoise(inputs, d, t=None, guidance=None):
    """Guided Euler loop; returns (z_lat, z_act) at t = 0 in float64."""
    if t is None:
        t = ex.schedule(d.n_steps)
    g = d.guidance if guidance is None else guidance
    keys = ("w_in_lat", "b_in_lat", "w_in_act", "b_in_act", "w_out_lat", "b_out_lat", "w_out_act", "b_out_act",
            "w_qkv", "w_o", "w_gu", "w_d")
    p = {k: np.asarray(inputs[k], F64) for k in keys}
    zl = np.asarray(inputs["z_lat"], F64).copy()
    za = np.asarray(inputs["z_act"], F64).copy()
    for k, dt in enumerate(ex.step_sizes(t)):
        mc = modulation(t[k], inputs["c_cond"], inputs["w_mod"], inputs["b_mod"])
        mu = modulation(t[k], inputs["c_uncond"], inputs["w_mod"], inputs["b_mod"])
        vcl, vca = velocity(zl, za, mc, p, d)
        vul, vua = velocity(zl, za, mu, p, d)
        zl = zl + dt * (vul + g * (vcl - vul))
        za = za + dt * (vua + g * (vca - vua))
    return zl, za
