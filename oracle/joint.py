"""Recomputed-prefix formulation of the same velocity (TEST INFRASTRUCTURE).

PhyAI reading ("PhyAI: Real-Time Physical AI at the Edge, Scalable Rollouts in
the Cloud"), Sec. 5.1: the vision-language prefix stays fixed while the action
tokens evolve, so its KV can be computed once and reused; Sec. 8.2, check 1,
proposes comparing reference inference with cached-prefix execution.

This module is that reference inference: every Euler step runs ONE joint
sequence [prefix tokens ; chunk tokens] through every layer, with a block mask
under which prefix rows see only prefix rows and chunk rows see everything.
The prefix rows use their own (synthetic) weights and a plain RMSNorm (they do
not depend on t).  ``prefix_kv`` runs the prefix rows alone once and returns
the per-layer K/V that the cached path consumes.  Cached and recomputed
velocities agree because no prefix row ever attends to a chunk row.
"""
from __future__ import annotations

import numpy as np

from . import expert as ex

F64 = np.float64


def _plain_rms(h, eps):
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)


def _masked_attention(q, k, v, allowed):
    """q, k, v: [Heads][S][dh] (k/v already expanded to the query heads);
    allowed[i][j] True where row i may attend to column j."""
    dh = q.shape[-1]
    s = np.einsum("hid,hjd->hij", q, k) / np.sqrt(F64(dh))
    s = np.where(allowed[None], s, -np.inf)
    s = s - s.max(axis=2, keepdims=True)
    p = np.where(allowed[None], np.exp(s), 0.0)
    p /= p.sum(axis=2, keepdims=True)
    return np.einsum("hij,hjd->hid", p, v)


def _split_qkv(x, dims):
    hq, hkv, dh = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    t = x.shape[0]
    q = x[:, : hq * dh].reshape(t, hq, dh).transpose(1, 0, 2)
    k = x[:, hq * dh:(hq + hkv) * dh].reshape(t, hkv, dh).transpose(1, 0, 2)
    v = x[:, (hq + hkv) * dh:].reshape(t, hkv, dh).transpose(1, 0, 2)
    g = hq // hkv
    return q, np.repeat(k, g, axis=0), np.repeat(v, g, axis=0), k, v


def _mlp(u, w_gu, w_d, f):
    gu = u @ w_gu.T
    return (ex.gelu_tanh(gu[:, :f]) * gu[:, f:]) @ w_d.T


def prefix_kv(p_tokens, pp, dims):
    """Run the prefix rows alone (prefix-only attention); return K, V
    [L][P][Hkv][dh] as seen by every layer."""
    hp = np.asarray(p_tokens, F64)
    ks, vs = [], []
    allowed = np.ones((hp.shape[0], hp.shape[0]), dtype=bool)
    for l in range(dims.n_layers):
        up = _plain_rms(hp, dims.rms_eps)
        q, kx, vx, k, v = _split_qkv(up @ pp["w_qkv"][l].T, dims)
        ks.append(k.transpose(1, 0, 2))
        vs.append(v.transpose(1, 0, 2))
        o = _masked_attention(q, kx, vx, allowed)
        hp = hp + o.transpose(1, 0, 2).reshape(hp.shape[0], -1) @ pp["w_o"][l].T
        hp = hp + _mlp(_plain_rms(hp, dims.rms_eps), pp["w_gu"][l], pp["w_d"][l], dims.mlp_dim)
    return np.stack(ks), np.stack(vs)


def joint_velocity(x, mods, p, pp, p_tokens, dims):
    """Velocity of the chunk computed from scratch over the joint sequence."""
    hp = np.asarray(p_tokens, F64)
    hc = x @ p["w_in"].T + p["b_in"]
    n_p, n_c = hp.shape[0], hc.shape[0]
    rows = np.arange(n_p + n_c)
    allowed = (rows[:, None] >= n_p) | (rows[None, :] < n_p)
    for l in range(dims.n_layers):
        sc, sh = mods[2 * l]
        up = _plain_rms(hp, dims.rms_eps)
        uc = ex.ada_rms(hc, sc, sh, dims.rms_eps)
        xx = np.concatenate([up @ pp["w_qkv"][l].T, uc @ p["w_qkv"][l].T])
        q, kx, vx, _, _ = _split_qkv(xx, dims)
        o = _masked_attention(q, kx, vx, allowed).transpose(1, 0, 2).reshape(n_p + n_c, -1)
        hp = hp + o[:n_p] @ pp["w_o"][l].T
        hc = hc + o[n_p:] @ p["w_o"][l].T
        sc, sh = mods[2 * l + 1]
        hp = hp + _mlp(_plain_rms(hp, dims.rms_eps), pp["w_gu"][l], pp["w_d"][l], dims.mlp_dim)
        hc = hc + _mlp(ex.ada_rms(hc, sc, sh, dims.rms_eps), p["w_gu"][l], p["w_d"][l], dims.mlp_dim)
    sc, sh = mods[2 * dims.n_layers]
    return ex.ada_rms(hc, sc, sh, dims.rms_eps) @ p["w_out"].T + p["b_out"]


def denoise_recomputed(inputs, pp, p_tokens, dims, t=None):
    """Euler loop that recomputes the prefix inside every step (batch 1)."""
    if t is None:
        t = ex.schedule(dims.n_steps)
    p = ex.as_f64_params(inputs)
    tables = ex.modulation_tables(t, inputs["w_mod"], inputs["b_mod"])
    return ex.euler(inputs["noise"][0], t,
                    lambda x, k: joint_velocity(x, tables[k], p, pp, p_tokens, dims))
