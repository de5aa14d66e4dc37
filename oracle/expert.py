"""float64 oracle of the pi0.5-style action expert and its Euler denoise loop.

TEST INFRASTRUCTURE: only tests, the smoke check and the benchmark's CPU
baseline call this module.

Page anchors (titles of the three pages; section names as printed there):

* PhyAI reading ("PhyAI: Real-Time Physical AI at the Edge, Scalable Rollouts
  in the Cloud"), Sec. 5.1 (one pi0.5 request): the vision-language prefix is
  fixed over ten Euler steps while the action tokens evolve; its KV and
  attention metadata are cached, timestep/modulation tables are precomputed,
  and a new observation invalidates the prefix.
* Same reading, Sec. 5.5 (implementation flow): fused projections,
  activations and normalisation beneath the layers.
* VLA-HWBench abstract (first page, "FlashRT-PAI: Fast Kernels Are Not Fast
  Pipelines ..."): flow-matching policies generate long action chunks in a
  few steps.

The pages print no architecture.  Readings used here (each one is listed in the
design notes with its reason):

* time runs from t=1 (noise) to t=0; step k evaluates the velocity at t_k and
  advances by dt_k = t_{k+1} - t_k with t_N = 0 (uniform schedule: dt = -1/N);
* sinusoidal embedding with periods log-spaced between 4e-3 and 4.0,
  [sin | cos] halves;
* one linear map per norm turns the embedding into (scale, shift); optionally
  (fidelity variant) the embedding first passes a time MLP W2 swish(W1 e + b1) + b2;
* adaptive RMSNorm  h / sqrt(mean(h^2) + eps) * (1 + scale) + shift, no gain;
* pre-norm layer: attention block then GeGLU MLP block, both residual; with a
  gated residual (fidelity variant) each norm's map also yields a gate and the
  block's output enters the residual as gate * output;
* chunk tokens attend to every prefix key and every chunk key (no mask among
  them, softmax scale 1/sqrt(head_dim)); by default no positional encoding is
  applied to the chunk (the prefix K/V is given already encoded); with a
  rotary base theta > 0 the chunk's queries and keys are rotated at positions
  P + t (rope below);
* grouped-query heads: query head i reads KV head floor(i / (Hq/Hkv));
* GELU in its tanh form; no biases in the expert linears.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64

P_MIN = 4e-3     # shortest embedding period (reading: sinusoid period range)
P_MAX = 4.0      # longest embedding period


def schedule(n_steps: int):
    """Uniform schedule t_k = 1 + k*dt, dt = -1/N (computed in float64, handed
    over as float32).  PhyAI reading Sec. 5.1: a fixed number of Euler steps
    from noise to action."""
    dt = -1.0 / n_steps
    t = np.array([1.0 + k * dt for k in range(n_steps)], dtype=F64)
    return t.astype(np.float32)


def step_sizes(t) -> np.ndarray:
    """dt_k = t_{k+1} - t_k with t_N = 0, evaluated in float64 from the given t."""
    t = np.asarray(t, dtype=F64)
    nxt = np.concatenate([t[1:], [0.0]])
    return nxt - t


def timestep_embedding(t: float, width: int) -> np.ndarray:
    """Sinusoidal embedding e(t) in R^width: e_i = sin(2 pi t / p_i),
    e_{half+i} = cos(2 pi t / p_i), p_i = p_min (p_max/p_min)^(i/(half-1)).
    Feeds the precomputed timestep tables of PhyAI reading Sec. 5.1."""
    half = width // 2
    i = np.arange(half, dtype=F64)
    periods = P_MIN * (P_MAX / P_MIN) ** (i / (half - 1))
    ang = 2.0 * np.pi * F64(t) / periods
    return np.concatenate([np.sin(ang), np.cos(ang)])


def swish(z):
    """swish(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    return z / (1.0 + np.exp(-z))


def time_mlp(e, w1, b1, w2, b2):
    """Time MLP of the fidelity variant: W2 swish(W1 e + b1) + b2 (float64)."""
    u = swish(np.asarray(w1, F64) @ e + np.asarray(b1, F64))
    return np.asarray(w2, F64) @ u + np.asarray(b2, F64)


def modulation_tables(t, w_mod, b_mod, tmlp=None) -> np.ndarray:
    """Per-step (scale, shift[, gate]) of every adaptive norm: m = W_m[j] e(t_k) + b_m[j].

    Returns [N][n_mod][R][D] float64 with R = W_m rows / D (2: scale, shift; 3 with the
    residual gate); index j = 2l (attention norm of layer l), 2l+1 (MLP norm of layer
    l), 2L (final norm).  These are the precomputed timestep/modulation tables of
    PhyAI reading Sec. 5.1 / 5.5.  ``tmlp`` = (W1, b1, W2, b2) runs the embedding through
    the time MLP first.
    """
    w_mod = np.asarray(w_mod, dtype=F64)
    b_mod = np.asarray(b_mod, dtype=F64)
    n_mod, rows, d = w_mod.shape
    out = np.empty((len(t), n_mod, rows // d, d), dtype=F64)
    for k, tk in enumerate(np.asarray(t, dtype=F64)):
        e = timestep_embedding(tk, d)
        if tmlp is not None:
            e = time_mlp(e, *tmlp)
        m = np.einsum("jod,d->jo", w_mod, e) + b_mod
        out[k] = m.reshape(n_mod, rows // d, d)
    return out


def ada_rms(h, scale, shift, eps):
    """Adaptive RMSNorm of each row: h / sqrt(mean(h^2) + eps) * (1 + scale) + shift."""
    r = np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
    return h / r * (1.0 + scale) + shift


def gelu_tanh(z):
    """GELU, tanh form: 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))."""
    return 0.5 * z * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (z + 0.044715 * z ** 3)))


def attention(q, k, v):
    """Softmax attention with grouped KV heads.

    q: [Hq][T][dh]; k, v: [Hkv][S][dh].  Query head i uses KV head
    floor(i / (Hq / Hkv)); scores q k^T / sqrt(dh), row softmax after
    subtracting the row max, then times V.  Returns [Hq][T][dh].
    """
    hq, _, dh = q.shape
    hkv = k.shape[0]
    g = hq // hkv
    out = np.empty_like(q, dtype=F64)
    for i in range(hq):
        r = i // g
        s = q[i] @ k[r].T / np.sqrt(F64(dh))
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[i] = p @ v[r]
    return out


def rope(x, positions, theta):
    """Rotary position embedding on interleaved pairs: for each head row at position
    p, the pair (x_{2i}, x_{2i+1}) is turned by the angle p * theta^(-2i/dh).

    x: [n_heads][T][dh]; positions: [T].  A fidelity variant of the expert (the
    pages stress positional precision, PhyAI reading Sec. 2); the pages print no
    convention, so interleaved pairs and base theta are a reading.
    """
    x = np.asarray(x, F64)
    dh = x.shape[-1]
    freq = F64(theta) ** (-2.0 * np.arange(dh // 2, dtype=F64) / dh)
    ang = np.asarray(positions, F64)[:, None] * freq[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def _heads(x, n_heads, head_dim):
    """[T][n_heads*head_dim] -> [n_heads][T][head_dim]."""
    return x.reshape(x.shape[0], n_heads, head_dim).transpose(1, 0, 2)


def expert_layer(h, l, mods, p, k_pre_l, v_pre_l, dims):
    """One pre-norm expert layer on the chunk's hidden states h [H][D].

    k_pre_l, v_pre_l: cached prefix K/V of this layer, [P][Hkv][dh], used as given
    (PhyAI reading Sec. 5.1: the prefix KV is computed once and reused).
    """
    hq, hkv, dh, f = dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.mlp_dim
    gated = mods.shape[1] == 3  # residual gates: the third row of each norm's map
    sc, sh = mods[2 * l][0], mods[2 * l][1]
    u = ada_rms(h, sc, sh, dims.rms_eps)
    qkv = u @ p["w_qkv"][l].T
    q = _heads(qkv[:, : hq * dh], hq, dh)
    kc = _heads(qkv[:, hq * dh:(hq + hkv) * dh], hkv, dh)
    vc = _heads(qkv[:, (hq + hkv) * dh:], hkv, dh)
    theta = getattr(dims, "rope_theta", 0.0)
    if theta > 0:  # chunk token t sits at position P + t, after the prefix
        pos = np.asarray(k_pre_l).shape[0] + np.arange(h.shape[0])
        q = rope(q, pos, theta)
        kc = rope(kc, pos, theta)
    kk = np.concatenate([np.asarray(k_pre_l, F64).transpose(1, 0, 2), kc], axis=1)
    vv = np.concatenate([np.asarray(v_pre_l, F64).transpose(1, 0, 2), vc], axis=1)
    o = attention(q, kk, vv)                                   # [Hq][H][dh]
    o = o.transpose(1, 0, 2).reshape(h.shape[0], hq * dh)
    blk = o @ p["w_o"][l].T
    h = h + (mods[2 * l][2] * blk if gated else blk)
    sc, sh = mods[2 * l + 1][0], mods[2 * l + 1][1]
    u = ada_rms(h, sc, sh, dims.rms_eps)
    gu = u @ p["w_gu"][l].T
    a = gelu_tanh(gu[:, :f]) * gu[:, f:]
    blk = a @ p["w_d"][l].T
    return h + (mods[2 * l + 1][2] * blk if gated else blk)


def velocity(x, mods, p, k_pre, v_pre, dims):
    """Network velocity v(x, t_k) for one sample.

    x: [H][A]; mods: [n_mod][2][D] of step k; k_pre, v_pre: [L][P][Hkv][dh].
    In-projection, the layer stack, final adaptive norm and out-projection.
    """
    h = x @ p["w_in"].T + p["b_in"]
    for l in range(dims.n_layers):
        h = expert_layer(h, l, mods, p, k_pre[l], v_pre[l], dims)
    sc, sh = mods[2 * dims.n_layers][0], mods[2 * dims.n_layers][1]
    u = ada_rms(h, sc, sh, dims.rms_eps)
    return u @ p["w_out"].T + p["b_out"]


def as_f64_params(inputs: dict, linears: dict | None = None) -> dict:
    """float64 view of the weights.  ``linears`` optionally replaces the four
    expert linears (e.g. by int4-dequantised matrices)."""
    keys = ("w_in", "b_in", "w_out", "b_out", "w_qkv", "w_o", "w_gu", "w_d")
    p = {k: np.asarray(inputs[k], dtype=F64) for k in keys}
    if linears:
        for k, w in linears.items():
            p[k] = np.asarray(w, dtype=F64)
    return p


def euler(x0, t, vel):
    """Explicit Euler from t_0 to 0: x <- x + dt_k v(x, k).  ``vel(x, k)`` is any
    velocity; PhyAI reading Sec. 5.1 (ten Euler steps for pi0.5)."""
    x = np.asarray(x0, dtype=F64).copy()
    for k, dt in enumerate(step_sizes(t)):
        x = x + dt * vel(x, k)
    return x


def denoise(inputs: dict, dims, t=None, linears: dict | None = None, samples=None):
    """Full cached-prefix denoise of every sample: returns x at t=0, [B][H][A] float64.

    Samples never interact (each uses its own prefix K/V and noise).
    """
    if t is None:
        t = schedule(dims.n_steps)
    p = as_f64_params(inputs, linears)
    tmlp = tuple(inputs[k] for k in ("w_tm1", "b_tm1", "w_tm2", "b_tm2")) if getattr(dims, "time_mlp", False) else None
    tables = modulation_tables(t, inputs["w_mod"], inputs["b_mod"], tmlp)
    noise = np.asarray(inputs["noise"], dtype=F64)
    if samples is None:
        samples = range(noise.shape[0])
    out = []
    for b in samples:
        kp = np.asarray(inputs["k_pre"][b], F64)
        vp = np.asarray(inputs["v_pre"][b], F64)
        out.append(euler(noise[b], t, lambda x, k: velocity(x, tables[k], p, kp, vp, dims)))
    return np.stack(out)


def rel_err(got, ref) -> float:
    """Norm-wise max relative error: max|got - ref| / max|ref|."""
    got = np.asarray(got, F64)
    ref = np.asarray(ref, F64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300))
