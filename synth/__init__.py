"""Seeded synthetic inputs for the cached-prefix flow-matching denoise loop.

This module is shared by the CPU oracle, the tests and the benchmark.  It holds
no arithmetic of the method itself: it only draws random tensors with the
shapes and distributions of the workloads and converts them to the storage
types the GPU path consumes (bf16 bit patterns by round-to-nearest-even).

Every tensor has its own PCG64 stream, ``numpy.random.default_rng([seed,
tensor_id])``; per-sample tensors (prefix K/V, noise) add the sample index, so
sample ``b`` of a batch-32 draw equals the batch-1 draw of sample ``b`` at the
same seed.

Workloads (the pages give no expert architecture; the shapes below are the
stated workloads of this implementation, the pi0.5-like figures follow the
PhyAI reading's Section 5.1 / Figure 5 settings: three cameras, 50-action
chunks, ten Euler steps):

* ``tiny``      fp32, 2 layers, width 256, 4q/1kv heads of 64, MLP 1024,
                prefix 64, chunk 16 x 8, 4 steps.
* ``pi05``      bf16, 18 layers, width 1024, 8q/1kv heads of 256, MLP 4096,
                prefix 816 (3 x 256 image + 48 text tokens), chunk 50 x 32,
                10 steps, batch 1.
* ``pi05_b32``  as ``pi05`` at batch 32, each sample with its own prefix.
* ``pi05_int4`` as ``pi05`` with the expert linears stored as group-128 int4.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "ExpertDims", "CONFIGS", "TENSOR_IDS", "normal", "bf16_bits", "bf16_values",
    "make_expert_inputs", "expert_param_shapes", "WamDims", "WAM_CONFIGS", "make_wam_inputs",
    "wam_device_inputs",
]

# one fixed id per tensor; never reorder (changing an id changes every draw)
TENSOR_IDS = {
    "w_in": 1, "b_in": 2, "w_out": 3, "b_out": 4, "w_mod": 5, "b_mod": 6,
    "w_qkv": 7, "w_o": 8, "w_gu": 9, "w_d": 10,
    "k_pre": 11, "v_pre": 12, "noise": 13,
    "w_tm1": 14, "b_tm1": 15, "w_tm2": 16, "b_tm2": 17,
    # prefix network used by the cached-vs-recomputed check
    "p_tokens": 20, "p_w_qkv": 21, "p_w_o": 22, "p_w_gu": 23, "p_w_d": 24,
    # joint video/action (WAM) variant
    "wam_w_in_lat": 40, "wam_b_in_lat": 41, "wam_w_in_act": 42, "wam_b_in_act": 43,
    "wam_w_out_lat": 44, "wam_b_out_lat": 45, "wam_w_out_act": 46, "wam_b_out_act": 47,
    "wam_w_mod": 48, "wam_b_mod": 49, "wam_w_qkv": 50, "wam_w_o": 51, "wam_w_gu": 52,
    "wam_w_d": 53, "wam_z_lat": 54, "wam_z_act": 55, "wam_cond": 56,
}


@dataclasses.dataclass(frozen=True)
class ExpertDims:
    n_layers: int
    width: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    mlp_dim: int
    prefix_len: int
    chunk_len: int
    action_dim: int
    n_steps: int
    batch: int
    weight_dtype: str          # "f32" | "bf16" | "int4"
    rms_eps: float = 1e-6
    weight_std: float = 0.02
    rope_theta: float = 0.0    # > 0: rotary embedding of the chunk's Q/K at positions P + t
    gated_residual: bool = False  # each norm's map also yields a residual gate (3 D rows)
    time_mlp: bool = False     # the timestep embedding passes W2 swish(W1 e + b1) + b2 first

    @property
    def n_mod(self) -> int:    # one (scale, shift) pair per norm: 2 per layer + final
        return 2 * self.n_layers + 1

    @property
    def qkv_dim(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


CONFIGS = {
    "tiny": ExpertDims(2, 256, 4, 1, 64, 1024, 64, 16, 8, 4, 1, "f32"),
    "pi05": ExpertDims(18, 1024, 8, 1, 256, 4096, 816, 50, 32, 10, 1, "bf16"),
    "pi05_b32": ExpertDims(18, 1024, 8, 1, 256, 4096, 816, 50, 32, 10, 32, "bf16"),
    "pi05_int4": ExpertDims(18, 1024, 8, 1, 256, 4096, 816, 50, 32, 10, 1, "int4"),
}


def normal(seed: int, tensor: str, shape, std: float = 1.0, sample: int | None = None) -> np.ndarray:
    """float32 N(0, std^2) draw from the tensor's own PCG64 stream."""
    key = [int(seed), TENSOR_IDS[tensor]] + ([] if sample is None else [int(sample)])
    rng = np.random.default_rng(key)
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_values(a: np.ndarray) -> np.ndarray:
    """float32 array whose values are the bf16 (RNE) roundings of ``a``."""
    return (bf16_bits(a).astype(np.uint32) << np.uint32(16)).view(np.float32)


def expert_param_shapes(d: ExpertDims) -> dict:
    L, D, A, F = d.n_layers, d.width, d.action_dim, d.mlp_dim
    return {
        "w_in": (D, A), "b_in": (D,), "w_out": (A, D), "b_out": (A,),
        "w_mod": (d.n_mod, (3 if getattr(d, "gated_residual", False) else 2) * D, D),
        "b_mod": (d.n_mod, (3 if getattr(d, "gated_residual", False) else 2) * D),
        "w_qkv": (L, d.qkv_dim, D), "w_o": (L, D, d.n_q_heads * d.head_dim),
        "w_gu": (L, 2 * F, D), "w_d": (L, D, F),
        **({"w_tm1": (D, D), "b_tm1": (D,), "w_tm2": (D, D), "b_tm2": (D,)} if getattr(d, "time_mlp", False) else {}),
    }


EXPERT_LINEARS = ("w_qkv", "w_o", "w_gu", "w_d")


def make_prefix_inputs(d: ExpertDims, seed: int = 1, batch: int | None = None) -> dict:
    """Synthetic prefix network (the four linears of its L layers, N(0, weight_std)) and its
    input tokens [B][P][D] (N(0, 1), one stream per sample), float32; bf16 values for the
    bf16 workloads.  Keys: w_qkv, w_o, w_gu, w_d, tokens."""
    B = d.batch if batch is None else batch
    L, D, F = d.n_layers, d.width, d.mlp_dim
    shapes = {"w_qkv": (L, d.qkv_dim, D), "w_o": (L, D, d.n_q_heads * d.head_dim),
              "w_gu": (L, 2 * F, D), "w_d": (L, D, F)}
    rnd = bf16_values if d.weight_dtype == "bf16" else (lambda a: a)
    out = {k: rnd(normal(seed, "p_" + k, shp, d.weight_std)) for k, shp in shapes.items()}
    out["tokens"] = rnd(np.stack([normal(seed, "p_tokens", (d.prefix_len, D), 1.0, sample=s) for s in range(B)]))
    return out


def make_expert_inputs(d: ExpertDims, seed: int = 0, batch: int | None = None,
                       prefix_len: int | None = None, samples=None) -> dict:
    """All inputs of one workload as float32 arrays.

    For ``bf16`` every weight and the prefix K/V hold bf16-representable values
    (RNE of the float32 draw).  For ``int4`` the four expert linears are left as
    the float32 draws (each side quantises them itself); every other weight and
    the prefix K/V are bf16 values.  Noise stays float32.

    ``samples`` selects which per-sample streams to draw (default ``range(batch)``).
    """
    B = d.batch if batch is None else batch
    P = d.prefix_len if prefix_len is None else prefix_len
    if samples is None:
        samples = range(B)
    samples = list(samples)
    out = {}
    for name, shape in expert_param_shapes(d).items():
        w = normal(seed, name, shape, d.weight_std)
        if d.weight_dtype == "bf16" or (d.weight_dtype == "int4" and name not in EXPERT_LINEARS):
            w = bf16_values(w)
        out[name] = w
    kv_shape = (d.n_layers, P, d.n_kv_heads, d.head_dim)
    k = np.stack([normal(seed, "k_pre", kv_shape, 1.0, sample=s) for s in samples])
    v = np.stack([normal(seed, "v_pre", kv_shape, 1.0, sample=s) for s in samples])
    if d.weight_dtype in ("bf16", "int4"):
        k, v = bf16_values(k), bf16_values(v)
    out["k_pre"], out["v_pre"] = k, v
    out["noise"] = np.stack([normal(seed, "noise", (d.chunk_len, d.action_dim), 1.0, sample=s)
                             for s in samples])
    return out


# ---------------------------------------------------------------- joint video/action (WAM)
@dataclasses.dataclass(frozen=True)
class WamDims:
    """Joint video/action denoiser: latent and action tokens evolve together in one
    sequence under full self-attention; a conditional and an unconditional branch are
    combined by classifier-free guidance."""
    n_layers: int
    width: int
    n_heads: int
    head_dim: int
    mlp_dim: int
    latent_tokens: int
    latent_dim: int
    action_tokens: int
    action_dim: int
    n_steps: int
    guidance: float
    rms_eps: float = 1e-6
    weight_std: float = 0.02

    @property
    def tokens(self) -> int:
        return self.latent_tokens + self.action_tokens

    @property
    def n_mod(self) -> int:
        return 2 * self.n_layers + 1


WAM_CONFIGS = {
    # full workload: 28 layers, width 2048, 16 heads of 128, MLP 8192, 4096 latents x 16 + 32 actions x 32
    "wam": WamDims(28, 2048, 16, 128, 8192, 4096, 16, 32, 32, 8, 3.0),
    # reduced shapes the CPU oracle finishes in seconds (several tiles, a ragged last tile)
    "wam_tiny": WamDims(2, 256, 4, 64, 1024, 200, 16, 24, 32, 3, 3.0),
}


def wam_param_shapes(d: WamDims) -> dict:
    L, D, F = d.n_layers, d.width, d.mlp_dim
    hd = d.n_heads * d.head_dim
    return {
        "w_in_lat": (D, d.latent_dim), "b_in_lat": (D,), "w_in_act": (D, d.action_dim), "b_in_act": (D,),
        "w_out_lat": (d.latent_dim, D), "b_out_lat": (d.latent_dim,),
        "w_out_act": (d.action_dim, D), "b_out_act": (d.action_dim,),
        "w_mod": (d.n_mod, (3 if getattr(d, "gated_residual", False) else 2) * D, D),
        "b_mod": (d.n_mod, (3 if getattr(d, "gated_residual", False) else 2) * D),
        "w_qkv": (L, 3 * hd, D), "w_o": (L, D, hd), "w_gu": (L, 2 * F, D), "w_d": (L, D, F),
    }


def make_wam_inputs(d: WamDims, seed: int = 0) -> dict:
    """bf16-valued weights (RNE of float32 N(0, std^2) draws), float32 latents/actions
    N(0, 1), bf16-valued condition vector N(0, 1) (the unconditional branch uses 0)."""
    out = {}
    for name, shape in wam_param_shapes(d).items():
        out[name] = bf16_values(normal(seed, "wam_" + name, shape, d.weight_std))
    out["z_lat"] = normal(seed, "wam_z_lat", (d.latent_tokens, d.latent_dim))
    out["z_act"] = normal(seed, "wam_z_act", (d.action_tokens, d.action_dim))
    out["c_cond"] = bf16_values(normal(seed, "wam_cond", (d.width,)))
    out["c_uncond"] = np.zeros(d.width, np.float32)
    return out


def wam_device_inputs(d: WamDims, seed: int = 0, device: str = "cuda") -> dict:
    """Full-size joint-denoiser inputs drawn directly on the device (1.9 B weights are too
    many to draw on the host in a test): torch's seeded device generator, one stream per
    tensor (seed * 1000 + tensor id), same distributions as ``make_wam_inputs`` (weights
    N(0, std^2) rounded to bf16, latents/actions N(0, 1) fp32, condition N(0, 1) bf16, zero
    unconditional vector).  Not comparable draw-for-draw with ``make_wam_inputs``."""
    import torch
    out = {}

    def draw(name, shape, std, dtype):
        g = torch.Generator(device=device)
        g.manual_seed(int(seed) * 1000 + TENSOR_IDS["wam_" + name if "wam_" + name in TENSOR_IDS else name])
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        return t.to(dtype).contiguous()

    for name, shape in wam_param_shapes(d).items():
        out[name] = draw(name, shape, d.weight_std, torch.bfloat16)
    out["z_lat"] = draw("z_lat", (d.latent_tokens, d.latent_dim), 1.0, torch.float32)
    out["z_act"] = draw("z_act", (d.action_tokens, d.action_dim), 1.0, torch.float32)
    out["c_cond"] = draw("cond", (d.width,), 1.0, torch.bfloat16)
    out["c_uncond"] = torch.zeros(d.width, dtype=torch.bfloat16, device=device)
    return out
