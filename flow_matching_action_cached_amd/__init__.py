"""Thin Python binding of libphyai.so (the MI355X cached-prefix flow-matching denoise loop).

Only argument marshalling lives here: every step of the loop runs in the HIP
kernels behind the C ABI declared in ``include/phyai.h``.  PyTorch supplies device
memory (``tensor.data_ptr()``) and the stream (``torch.cuda.current_stream()``).
The library must be built first (``python -m flow_matching_action_cached_amd.build``);
nothing here falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libphyai.so")

F32, BF16, INT4_G128 = 0, 1, 2
_DTYPES = {"f32": F32, "bf16": BF16, "int4": INT4_G128}
STATUS = {0: "ok", 1: "invalid argument", 2: "bad state", 3: "out of memory", 4: "device error",
          5: "unsupported"}

EXPORTED = (
    "phyai_create", "phyai_set_weights", "phyai_set_prefix_kv", "phyai_set_prefill_weights", "phyai_prefill",
    "phyai_capsule_bytes", "phyai_capsule_save", "phyai_capsule_restore", "phyai_capsule_fork",
    "phyai_unipc_weights",
    "phyai_set_timestep_tables",
    "phyai_denoise", "phyai_denoise_noalloc", "phyai_time_loop_stages", "phyai_set_graph_mode", "phyai_set_persistent", "phyai_loop_form", "phyai_sync", "phyai_last_error", "phyai_status_string",
    "phyai_destroy", "phyai_quantize_int4_g128", "phyai_get_modulation", "phyai_version",
    "phyai_enqueue_kernel_repeat", "phyai_wam_create", "phyai_wam_set_weights", "phyai_wam_set_conditions",
    "phyai_wam_denoise",
)


class PhyaiError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int), ("width", ctypes.c_int), ("n_q_heads", ctypes.c_int),
                ("n_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int), ("mlp_dim", ctypes.c_int),
                ("action_dim", ctypes.c_int), ("chunk_len", ctypes.c_int), ("max_prefix_len", ctypes.c_int),
                ("max_batch", ctypes.c_int), ("weight_dtype", ctypes.c_int), ("rms_eps", ctypes.c_float),
                ("max_arena_bytes", ctypes.c_size_t), ("rope_theta", ctypes.c_float),
                ("gated_residual", ctypes.c_int), ("time_mlp", ctypes.c_int), ("prefill", ctypes.c_int)]


_WFIELDS = ("w_in", "b_in", "w_out", "b_out", "w_mod", "b_mod", "w_qkv", "w_o", "w_gu", "w_d",
            "s_qkv", "s_o", "s_gu", "s_d", "w_tm1", "b_tm1", "w_tm2", "b_tm2")


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _WFIELDS]


class PrefillWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_qkv", "w_o", "w_gu", "w_d")]


class WamConfig(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int), ("width", ctypes.c_int), ("n_heads", ctypes.c_int),
                ("head_dim", ctypes.c_int), ("mlp_dim", ctypes.c_int), ("latent_tokens", ctypes.c_int),
                ("latent_dim", ctypes.c_int), ("action_tokens", ctypes.c_int), ("action_dim", ctypes.c_int),
                ("rms_eps", ctypes.c_float), ("max_arena_bytes", ctypes.c_size_t), ("solver_order", ctypes.c_int)]


_WAM_WFIELDS = ("w_in_lat", "b_in_lat", "w_in_act", "b_in_act", "w_out_lat", "b_out_lat", "w_out_act",
                "b_out_act", "w_mod", "b_mod", "w_qkv", "w_o", "w_gu", "w_d")


class WamWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _WAM_WFIELDS]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libphyai.so (raises if it is not built: there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m flow_matching_action_cached_amd.build`")
    lib = ctypes.CDLL(path)
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.phyai_create.argtypes = [ctypes.POINTER(Config), vp, ctypes.POINTER(vp)]
    lib.phyai_set_weights.argtypes = [vp, ctypes.POINTER(Weights)]
    lib.phyai_set_prefix_kv.argtypes = [vp, vp, vp, ci, ci]
    lib.phyai_set_prefill_weights.argtypes = [vp, ctypes.POINTER(PrefillWeights)]
    lib.phyai_prefill.argtypes = [vp, vp, ci, ci]
    lib.phyai_capsule_bytes.argtypes = [vp]
    lib.phyai_capsule_save.argtypes = [vp, vp, ctypes.c_size_t]
    lib.phyai_capsule_restore.argtypes = [vp, vp, ctypes.c_size_t]
    lib.phyai_capsule_fork.argtypes = [vp, ci, ci]
    lib.phyai_unipc_weights.argtypes = [vp, ci, ci, vp]
    lib.phyai_set_timestep_tables.argtypes = [vp, ctypes.POINTER(cf), ci]
    lib.phyai_denoise.argtypes = [vp, vp, ci, ci, vp]
    lib.phyai_denoise_noalloc.argtypes = [vp, vp, ci, ci, vp]
    lib.phyai_time_loop_stages.argtypes = [vp, vp, ci, ci, vp, vp]
    lib.phyai_set_graph_mode.argtypes = [vp, ci]
    lib.phyai_set_persistent.argtypes = [vp, ci]
    lib.phyai_loop_form.argtypes = [vp, ci]
    lib.phyai_sync.argtypes = [vp]
    lib.phyai_last_error.argtypes = [vp]
    lib.phyai_last_error.restype = ctypes.c_char_p
    lib.phyai_status_string.argtypes = [ci]
    lib.phyai_status_string.restype = ctypes.c_char_p
    lib.phyai_destroy.argtypes = [vp]
    lib.phyai_destroy.restype = None
    lib.phyai_quantize_int4_g128.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, vp, vp, vp]
    lib.phyai_get_modulation.argtypes = [vp, vp]
    lib.phyai_enqueue_kernel_repeat.argtypes = [vp, ci, ci, ci]
    lib.phyai_wam_create.argtypes = [ctypes.POINTER(WamConfig), vp, ctypes.POINTER(vp)]
    lib.phyai_wam_set_weights.argtypes = [vp, ctypes.POINTER(WamWeights)]
    lib.phyai_wam_set_conditions.argtypes = [vp, vp, vp, cf]
    lib.phyai_wam_denoise.argtypes = [vp, vp, vp, ci, vp, vp]
    lib.phyai_version.restype = ctypes.c_char_p
    for name in EXPORTED:
        if name not in ("phyai_last_error", "phyai_status_string", "phyai_destroy", "phyai_version"):
            getattr(lib, name).restype = ci
    lib.phyai_capsule_bytes.restype = ctypes.c_size_t
    _lib = lib
    return lib


def _stream_handle(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


class _Context:
    """Calls shared by both context kinds (see include/phyai.h)."""

    _h = None

    def _check(self, st):
        if st != 0:
            raise PhyaiError(st, self._lib.phyai_last_error(self._h).decode())

    def set_timestep_tables(self, t):
        arr = (ctypes.c_float * len(t))(*[float(x) for x in t])
        self._check(self._lib.phyai_set_timestep_tables(self._h, arr, len(t)))
        self.n_steps = len(t)

    def set_graph_mode(self, use_graph: bool):
        self._check(self._lib.phyai_set_graph_mode(self._h, int(bool(use_graph))))

    def set_persistent(self, enable: bool):
        """Use the persistent one-kernel loop where the shape supports it (see phyai.h)."""
        self._check(self._lib.phyai_set_persistent(self._h, int(bool(enable))))

    def loop_form(self, batch: int) -> int:
        """1: a denoise of `batch` samples runs the persistent kernel; 0: the graph; -1: not runnable."""
        return int(self._lib.phyai_loop_form(self._h, int(batch)))

    def enqueue_kernel_repeat(self, which: int, layer: int, reps: int):
        """One graph replay of `reps` launches of a single loop kernel (see phyai.h)."""
        self._check(self._lib.phyai_enqueue_kernel_repeat(self._h, which, layer, reps))

    def _modulation(self, shape):
        import torch
        out = torch.empty(shape, dtype=torch.float32, device="cuda")
        self._check(self._lib.phyai_get_modulation(self._h, _ptr(out)))
        self.sync()
        return out

    def sync(self):
        self._check(self._lib.phyai_sync(self._h))

    def close(self):
        if getattr(self, "_h", None):
            self._lib.phyai_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class ActionExpert(_Context):
    """One runner context: owns the device arena, the prefix KV cache, the tables
    and the captured denoise graphs (see include/phyai.h)."""

    def __init__(self, *, n_layers, width, n_q_heads, n_kv_heads, head_dim, mlp_dim, action_dim,
                 chunk_len, max_prefix_len, max_batch=1, weight_dtype="bf16", rms_eps=1e-6,
                 max_arena_bytes=0, stream=None, rope_theta=0.0, gated_residual=False, time_mlp=False,
                 prefill=False):
        self._lib = load_library()
        self.weight_dtype = weight_dtype
        cfg = Config(n_layers, width, n_q_heads, n_kv_heads, head_dim, mlp_dim, action_dim, chunk_len,
                     max_prefix_len, max_batch, _DTYPES[weight_dtype], rms_eps, max_arena_bytes, rope_theta,
                     int(bool(gated_residual)), int(bool(time_mlp)), int(bool(prefill)))
        self.cfg = cfg
        self._stream = stream
        h = ctypes.c_void_p()
        st = self._lib.phyai_create(ctypes.byref(cfg), _stream_handle(stream), ctypes.byref(h))
        if st != 0:
            raise PhyaiError(st, "phyai_create failed")
        self._h = h
        self._batch = None

    @classmethod
    def from_dims(cls, d, **kw):
        """Build from a ``synth.ExpertDims``-like object."""
        return cls(n_layers=d.n_layers, width=d.width, n_q_heads=d.n_q_heads, n_kv_heads=d.n_kv_heads,
                   head_dim=d.head_dim, mlp_dim=d.mlp_dim, action_dim=d.action_dim, chunk_len=d.chunk_len,
                   max_prefix_len=kw.pop("max_prefix_len", d.prefix_len), max_batch=kw.pop("max_batch", d.batch),
                   weight_dtype=d.weight_dtype, rms_eps=d.rms_eps, rope_theta=getattr(d, "rope_theta", 0.0),
                   gated_residual=getattr(d, "gated_residual", False), time_mlp=getattr(d, "time_mlp", False),
                   **kw)

    def set_weights(self, w: dict):
        """w: dict of contiguous cuda tensors named as in phyai_weights."""
        for k, t in w.items():
            if t is not None and not t.is_contiguous():
                raise ValueError(f"{k} must be contiguous")
        ws = Weights(*[_ptr(w.get(n)) for n in _WFIELDS])
        self._check(self._lib.phyai_set_weights(self._h, ctypes.byref(ws)))
        self.sync()

    def set_prefill_weights(self, w: dict):
        """w: dict of contiguous cuda tensors w_qkv, w_o, w_gu, w_d of the prefix network."""
        ws = PrefillWeights(*[_ptr(w.get(n)) for n in ("w_qkv", "w_o", "w_gu", "w_d")])
        self._check(self._lib.phyai_set_prefill_weights(self._h, ctypes.byref(ws)))

    def prefill(self, tokens):
        """tokens: cuda [B][P][width] in the weight element type; computes and installs the
        prefix K/V (asynchronous on the stream)."""
        assert tokens.is_contiguous() and tokens.dim() == 3
        self._check(self._lib.phyai_prefill(self._h, _ptr(tokens), int(tokens.shape[0]), int(tokens.shape[1])))
        self._batch = int(tokens.shape[0])

    def capsule_save(self):
        """Snapshot the installed prefix into a new uint8 cuda tensor (the capsule)."""
        import torch
        n = self._lib.phyai_capsule_bytes(self._h)
        if n == 0:
            raise PhyaiError(2, "no prefix installed")
        cap = torch.empty(n, dtype=torch.uint8, device="cuda")
        self._check(self._lib.phyai_capsule_save(self._h, _ptr(cap), n))
        return cap

    def capsule_restore(self, cap):
        """cap: a contiguous uint8 cuda tensor holding a capsule (as capsule_save returns)."""
        import torch
        if cap.dtype != torch.uint8 or not cap.is_contiguous():
            raise ValueError("a capsule is a contiguous uint8 tensor")
        self._check(self._lib.phyai_capsule_restore(self._h, _ptr(cap), cap.numel()))

    def capsule_fork(self, src: int, dst: int):
        self._check(self._lib.phyai_capsule_fork(self._h, int(src), int(dst)))

    def set_prefix_kv(self, k, v):
        """k, v: cuda [B][L][P][Hkv][dh] in the weight element type."""
        assert k.is_contiguous() and v.is_contiguous() and k.shape == v.shape
        self._check(self._lib.phyai_set_prefix_kv(self._h, _ptr(k), _ptr(v), int(k.shape[0]), int(k.shape[2])))
        self._batch = int(k.shape[0])
        self.sync()

    def denoise(self, noise, out=None):
        """noise: cuda float32 [B][H][A]; returns x at t=0 (asynchronous on the stream)."""
        import torch
        assert noise.dtype == torch.float32 and noise.is_contiguous()
        if out is None:
            out = torch.empty_like(noise)
        self._check(self._lib.phyai_denoise(self._h, _ptr(noise), int(noise.shape[0]), self.n_steps, _ptr(out)))
        return out

    def time_loop_stages(self, noise, reps=10):
        """In-loop mean duration (us) of each kernel id of the denoise loop and the mean chunk time
        (ms), from events between the launches of the loop (see phyai_time_loop_stages)."""
        import torch
        assert noise.dtype == torch.float32 and noise.is_contiguous()
        us = (ctypes.c_float * 8)()
        ms = ctypes.c_float()
        self._check(self._lib.phyai_time_loop_stages(self._h, _ptr(noise), int(noise.shape[0]), int(reps),
                                                     ctypes.addressof(us), ctypes.addressof(ms)))
        return list(us), ms.value

    def denoise_noalloc(self, noise, out=None):
        """As denoise, through the allocation-free entry point (static scratch, eager launches)."""
        import torch
        assert noise.dtype == torch.float32 and noise.is_contiguous()
        if out is None:
            out = torch.empty_like(noise)
        self._check(self._lib.phyai_denoise_noalloc(self._h, _ptr(noise), int(noise.shape[0]), self.n_steps,
                                                    _ptr(out)))
        return out

    def get_modulation(self):
        c = self.cfg
        return self._modulation((self.n_steps, 2 * c.n_layers + 1, 2, c.width))


class JointDenoiser(_Context):
    """Joint video/action denoiser context with a guided branch pair (see include/phyai.h)."""

    def __init__(self, *, n_layers, width, n_heads, head_dim, mlp_dim, latent_tokens, latent_dim,
                 action_tokens, action_dim, rms_eps=1e-6, max_arena_bytes=0, stream=None, solver_order=0):
        self._lib = load_library()
        cfg = WamConfig(n_layers, width, n_heads, head_dim, mlp_dim, latent_tokens, latent_dim, action_tokens,
                        action_dim, rms_eps, max_arena_bytes, int(solver_order))
        self.cfg = cfg
        h = ctypes.c_void_p()
        st = self._lib.phyai_wam_create(ctypes.byref(cfg), _stream_handle(stream), ctypes.byref(h))
        if st != 0:
            raise PhyaiError(st, "phyai_wam_create failed")
        self._h = h

    @classmethod
    def from_dims(cls, d, **kw):
        """Build from a ``synth.WamDims``-like object."""
        return cls(n_layers=d.n_layers, width=d.width, n_heads=d.n_heads, head_dim=d.head_dim, mlp_dim=d.mlp_dim,
                   latent_tokens=d.latent_tokens, latent_dim=d.latent_dim, action_tokens=d.action_tokens,
                   action_dim=d.action_dim, rms_eps=d.rms_eps, **kw)

    def set_weights(self, w: dict):
        """w: dict of contiguous bf16 cuda tensors named as in phyai_wam_weights."""
        for k in _WAM_WFIELDS:
            if not w[k].is_contiguous():
                raise ValueError(f"{k} must be contiguous")
        ws = WamWeights(*[_ptr(w[n]) for n in _WAM_WFIELDS])
        self._check(self._lib.phyai_wam_set_weights(self._h, ctypes.byref(ws)))

    def set_conditions(self, c_cond, c_uncond, guidance: float):
        """c_cond, c_uncond: bf16 cuda [D]."""
        assert c_cond.is_contiguous() and c_uncond.is_contiguous()
        self._check(self._lib.phyai_wam_set_conditions(self._h, _ptr(c_cond), _ptr(c_uncond), float(guidance)))

    def denoise(self, z_lat, z_act, out_lat=None, out_act=None):
        """z_lat float32 cuda [Tl][Cl], z_act float32 cuda [Ta][A] -> (z_lat, z_act) at t = 0."""
        import torch
        for z in (z_lat, z_act):
            assert z.dtype == torch.float32 and z.is_contiguous()
        out_lat = torch.empty_like(z_lat) if out_lat is None else out_lat
        out_act = torch.empty_like(z_act) if out_act is None else out_act
        self._check(self._lib.phyai_wam_denoise(self._h, _ptr(z_lat), _ptr(z_act), self.n_steps, _ptr(out_lat),
                                                _ptr(out_act)))
        return out_lat, out_act

    def get_modulation(self):
        c = self.cfg
        return self._modulation((self.n_steps, 2, 2 * c.n_layers + 1, 2, c.width))


def unipc_weights(t, order):
    """UniPC step weights of a schedule (host only, as phyai_unipc_weights): float32 [N][8]."""
    import numpy as np
    lib = load_library()
    tt = np.ascontiguousarray(np.asarray(t, dtype=np.float32))
    out = np.zeros((tt.size, 8), dtype=np.float32)
    st = lib.phyai_unipc_weights(tt.ctypes.data, int(tt.size), int(order), out.ctypes.data)
    if st != 0:
        raise PhyaiError(st, "phyai_unipc_weights: invalid schedule or order")
    return out


def quantize_int4_g128(w, stream=None):
    """Offline int4 quantiser on the GPU: w cuda float32 [..., K] (K % 128 == 0) ->
    (packed uint8 [..., K/2], scales int16 holding bf16 bits [..., K/128])."""
    import torch
    lib = load_library()
    assert w.dtype == torch.float32 and w.is_contiguous() and w.shape[-1] % 128 == 0
    cols = int(w.shape[-1])
    rows = int(w.numel() // cols)
    packed = torch.empty((*w.shape[:-1], cols // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((*w.shape[:-1], cols // 128), dtype=torch.int16, device=w.device)
    st = lib.phyai_quantize_int4_g128(_ptr(w), rows, cols, _ptr(packed), _ptr(scales), _stream_handle(stream))
    if st != 0:
        raise PhyaiError(st, "phyai_quantize_int4_g128 failed")
    return packed, scales
