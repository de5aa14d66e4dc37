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
schedule, or the UniPC multistep solver that the pages name for the video/action states
(its reading is stated with the code at the end of this module).
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


def denoise(inputs, d, t=None, guidance=None, solver_order=0):
    """Guided Euler loop (solver_order 0) or UniPC with predictor order 1 or 2 (see
    denoise_unipc); returns (z_lat, z_act) at t = 0 in float64."""
    if solver_order:
        return denoise_unipc(inputs, d, solver_order, t, guidance)
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


# ---------------------------------------------------------------- UniPC multistep solver
# The pages name UniPC as the update of the video/action states and print nothing more.
# Reading: the published UniPC predictor-corrector (Zhao et al., 2023) in data-prediction
# form, for the flow of this module (x_t = (1 - t) x_0 + t eps, so alpha_t = 1 - t,
# sigma_t = t; the velocity v = eps - x_0 gives the data prediction m = x - t v).  With
# lambda = log(alpha / sigma) the solution from s to t is
#   x_t = (sigma_t / sigma_s) x_s + sigma_t * integral_{lambda_s}^{lambda_t} e^lambda m dlambda,
# and every update replaces m by the polynomial in lambda through the data predictions it
# uses, integrated exactly.  The predictor of order p (s -> next time) uses the point s and
# the p - 1 points before it; once the model has been evaluated at the predicted point, the
# corrector redoes the same step with that point added (one order higher, no extra model
# evaluation).  Solving for the polynomial exactly is the method's linear system solved
# exactly, so its B(h) factor cancels.  Limits of the formula: a point at t = 1
# (lambda = -inf) enters only as the base of a step (as a neighbour its weight tends to 0),
# and the step to t = 0 (lambda = +inf) is first order with result m_s.


def _als(t):
    """alpha, sigma, lambda of the flow at time t (lambda = -inf at t = 1, +inf at t = 0)."""
    t = float(t)
    a, s = 1.0 - t, t
    with np.errstate(divide="ignore"):
        lam = np.log(a) - np.log(s)
    return a, s, lam


def exp_moments(h, n):
    """J_k(h) = integral_0^h e^{-(h-u)} u^k du for k = 0..n (J_0 = 1 - e^{-h};
    integration by parts gives J_k = h^k - k J_{k-1})."""
    j = [-np.expm1(-h)]
    for k in range(1, n + 1):
        j.append(h ** k - k * j[-1])
    return np.array(j)


def unipc_update(x_s, s, t, m_s, others):
    """One UniPC update from time s to t: base point (s, m_s) plus the (t_j, m_j) in
    ``others``; returns x_t."""
    a_s, sg_s, l_s = _als(s)
    a_t, sg_t, l_t = _als(t)
    if sg_t == 0.0:                      # step to t = 0: first order, x_t = m_s
        assert not others
        return np.array(m_s, F64)
    if a_s == 0.0:                       # base at t = 1: only the new point can join (limit)
        assert len(others) <= 1 and (not others or others[0][0] == t)
        m = others[0][1] if others else m_s
        return (sg_t / sg_s) * x_s + a_t * m
    pts = [(0.0, m_s)] + [(_als(tj)[2] - l_s, mj) for tj, mj in others if _als(tj)[0] > 0.0]
    u = np.array([p[0] for p in pts])
    n = len(pts)
    h = l_t - l_s
    vand = u[:, None] ** np.arange(n)[None, :]          # P(u_i) = sum_k c_k u_i^k = m_i
    wts = np.linalg.solve(vand.T, exp_moments(h, n - 1))  # integral of P against e^{-(h-u)}
    acc = sum(w * np.asarray(mi, F64) for w, (_, mi) in zip(wts, pts))
    return (sg_t / sg_s) * x_s + a_t * acc


def unipc_loop(z, t, order, vel):
    """UniPC from z at t[0] to t = 0 over the times t (predictor order 1 or 2, corrector
    on): vel(z, k) is the velocity at z and t[k]; the model is evaluated at the predicted
    states and the corrector then refines each of them."""
    assert order in (1, 2)
    ts = [float(x) for x in np.asarray(t, F64)] + [0.0]
    z = np.array(z, F64)
    ms, used, x_prev = [], [], None
    for k in range(len(ts) - 1):
        m = z - ts[k] * vel(z, k)
        if k >= 1:                       # corrector of the step k-1 -> k
            z = unipc_update(x_prev, ts[k - 1], ts[k], ms[k - 1], used[k - 1] + [(ts[k], m)])
        ms.append(m)
        nb = [] if ts[k + 1] == 0.0 else [(ts[k - j], ms[k - j]) for j in range(1, order) if k - j >= 0]
        used.append(nb)
        x_prev = z
        z = unipc_update(z, ts[k], ts[k + 1], m, nb)
    return z


def denoise_unipc(inputs, d, order, t=None, guidance=None):
    """Guided UniPC loop of the joint denoiser; returns (z_lat, z_act) at t = 0."""
    if t is None:
        t = ex.schedule(d.n_steps)
    g = d.guidance if guidance is None else guidance
    keys = ("w_in_lat", "b_in_lat", "w_in_act", "b_in_act", "w_out_lat", "b_out_lat", "w_out_act", "b_out_act",
            "w_qkv", "w_o", "w_gu", "w_d")
    p = {k: np.asarray(inputs[k], F64) for k in keys}
    zl0 = np.asarray(inputs["z_lat"], F64)
    za0 = np.asarray(inputs["z_act"], F64)
    nl = zl0.size
    tv = np.asarray(t, F64)

    def vel(z, k):
        zl, za = z[:nl].reshape(zl0.shape), z[nl:].reshape(za0.shape)
        mc = modulation(tv[k], inputs["c_cond"], inputs["w_mod"], inputs["b_mod"])
        mu = modulation(tv[k], inputs["c_uncond"], inputs["w_mod"], inputs["b_mod"])
        vcl, vca = velocity(zl, za, mc, p, d)
        vul, vua = velocity(zl, za, mu, p, d)
        return np.concatenate([(vul + g * (vcl - vul)).ravel(), (vua + g * (vca - vua)).ravel()])

    z = unipc_loop(np.concatenate([zl0.ravel(), za0.ravel()]), t, order, vel)
    return z[:nl].reshape(zl0.shape), z[nl:].reshape(za0.shape)
