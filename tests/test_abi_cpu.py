"""C-ABI checks that need no GPU: the library loads, exports every entry point the
public header declares, and rejects bad arguments before touching a device."""
import ctypes
import os
import re

import pytest

import flow_matching_action_cached_amd as fm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "phyai.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(phyai_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fm.LIB_PATH):
        pytest.fail("libphyai.so is not built (run python -m flow_matching_action_cached_amd.build)")
    return fm.load_library()


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("phyai_create", "phyai_set_prefix_kv", "phyai_set_timestep_tables", "phyai_denoise",
              "phyai_set_weights", "phyai_sync", "phyai_destroy", "phyai_last_error"):
        assert n in names
    assert set(names) == set(fm.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for n in _declared():
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    assert lib.phyai_status_string(0) == b"ok"
    assert lib.phyai_status_string(2) == b"bad state"
    assert b"gfx950" in lib.phyai_version()


def _cfg(**kw):
    base = dict(n_layers=2, width=256, n_q_heads=4, n_kv_heads=1, head_dim=64, mlp_dim=1024, action_dim=8,
                chunk_len=16, max_prefix_len=64, max_batch=1, weight_dtype=fm.F32, rms_eps=1e-6,
                max_arena_bytes=0)
    base.update(kw)
    return fm.Config(**base)


def _create(lib, cfg):
    h = ctypes.c_void_p()
    st = lib.phyai_create(ctypes.byref(cfg) if cfg is not None else None, None, ctypes.byref(h))
    return st, h


def test_create_rejects_bad_config_without_a_device(lib):
    assert _create(lib, None)[0] == 1
    assert _create(lib, _cfg(n_layers=0))[0] == 1
    assert _create(lib, _cfg(rms_eps=0.0))[0] == 1
    assert _create(lib, _cfg(weight_dtype=7))[0] == 1
    assert _create(lib, _cfg(width=200))[0] == 5          # not a multiple of 256
    assert _create(lib, _cfg(width=384))[0] == 5
    assert _create(lib, _cfg(action_dim=6))[0] == 5
    assert _create(lib, _cfg(head_dim=48))[0] == 5
    assert _create(lib, _cfg(n_q_heads=3, n_kv_heads=2))[0] == 5
    assert _create(lib, _cfg(chunk_len=50, max_batch=2))[0] == 5   # many rows need bf16 weights
    assert _create(lib, _cfg(rope_theta=0.5))[0] == 1               # rotary base must be 0 or > 1
    assert _create(lib, _cfg(rope_theta=-1e4))[0] == 1
    assert _create(lib, _cfg(rope_theta=float("nan")))[0] == 1
    assert _create(lib, _cfg(gated_residual=2))[0] == 1
    assert _create(lib, _cfg(time_mlp=-1))[0] == 1
    assert _create(lib, _cfg(prefill=2))[0] == 1
    assert _create(lib, _cfg(prefill=1, weight_dtype=fm.INT4_G128))[0] == 5  # no int4 prefix network
    assert _create(lib, _cfg(prefill=1, max_prefix_len=100))[0] == 5        # > 64 prefix rows need bf16
    # weight-streaming GEMMs: every linear's K / 128 must be a power of two <= 64
    for kw in (dict(width=768), dict(width=1280), dict(width=1536), dict(width=1792),
               dict(mlp_dim=384), dict(mlp_dim=640), dict(mlp_dim=1152), dict(mlp_dim=3072),
               dict(mlp_dim=6144), dict(mlp_dim=16384), dict(n_q_heads=6, head_dim=64),
               dict(n_q_heads=3, n_kv_heads=1, head_dim=256)):
        assert _create(lib, _cfg(**kw))[0] == 5, kw
    # ... unless no batch or prefill ever fits 64 rows (then only the tiled GEMMs run)
    assert _create(lib, _cfg(chunk_len=100, mlp_dim=3072, weight_dtype=fm.BF16))[0] != 5
    # the prefix network stores unrotated K/V: no prefill together with rotary positions
    assert _create(lib, _cfg(prefill=1, rope_theta=1e4))[0] == 5
    st, h = _create(lib, _cfg(n_layers=0))
    assert h.value is None


def test_null_context_calls_fail_cleanly(lib):
    assert lib.phyai_set_prefix_kv(None, None, None, 1, 1) == 1
    assert lib.phyai_set_prefill_weights(None, None) == 1
    assert lib.phyai_prefill(None, None, 1, 1) == 1
    assert lib.phyai_capsule_bytes(None) == 0
    assert lib.phyai_capsule_save(None, None, 0) == 1
    assert lib.phyai_capsule_restore(None, None, 0) == 1
    assert lib.phyai_capsule_fork(None, 0, 1) == 1
    assert lib.phyai_denoise(None, None, 1, 1, None) == 1
    assert lib.phyai_sync(None) == 1
    assert lib.phyai_set_weights(None, None) == 1
    assert lib.phyai_set_timestep_tables(None, None, 0) == 1
    assert lib.phyai_set_graph_mode(None, 1) == 1
    assert lib.phyai_get_modulation(None, None) == 1
    assert lib.phyai_denoise_noalloc(None, None, 1, 1, None) == 1
    assert lib.phyai_time_loop_stages(None, None, 1, 1, None, None) == 1
    assert lib.phyai_set_persistent(None, 1) == 1
    assert lib.phyai_loop_form(None, 1) == -1
    assert lib.phyai_enqueue_kernel_repeat(None, 0, 0, 1) == 1
    lib.phyai_destroy(None)


def test_unipc_weights_argument_checks(lib):
    """The host-side UniPC step weights reject what they cannot take, without a device."""
    f = ctypes.c_float
    out = (f * 64)()
    dec = (f * 3)(1.0, 0.6, 0.2)
    assert lib.phyai_unipc_weights(None, 3, 1, out) == 1                       # null schedule
    assert lib.phyai_unipc_weights(dec, 3, 3, out) == 1                        # order 3
    assert lib.phyai_unipc_weights(dec, 0, 1, out) == 1                        # no steps
    assert lib.phyai_unipc_weights((f * 3)(1.0, 0.6, 0.6), 3, 2, out) == 1     # not strictly decreasing
    assert lib.phyai_unipc_weights((f * 3)(1.2, 0.6, 0.2), 3, 2, out) == 1     # starts above 1
    assert lib.phyai_unipc_weights((f * 3)(1.0, 0.6, 0.0), 3, 2, out) == 1     # reaches 0 before the end
    assert lib.phyai_unipc_weights(dec, 3, 2, out) == 0


def test_quantizer_argument_checks(lib):
    assert lib.phyai_quantize_int4_g128(None, 4, 100, None, None, None) == 1   # cols % 128
    assert lib.phyai_quantize_int4_g128(None, -1, 128, None, None, None) == 1
    assert lib.phyai_quantize_int4_g128(None, 0, 128, None, None, None) == 0    # empty: nothing to do
    assert lib.phyai_quantize_int4_g128(None, 4, 128, None, None, None) == 1   # null pointers


def _wcfg(**kw):
    base = dict(n_layers=2, width=256, n_heads=4, head_dim=64, mlp_dim=1024, latent_tokens=200, latent_dim=16,
                action_tokens=24, action_dim=32, rms_eps=1e-6, max_arena_bytes=0)
    base.update(kw)
    return fm.WamConfig(**base)


def _wcreate(lib, cfg):
    h = ctypes.c_void_p()
    return lib.phyai_wam_create(ctypes.byref(cfg) if cfg is not None else None, None, ctypes.byref(h)), h


def test_joint_create_rejects_bad_config_without_a_device(lib):
    assert _wcreate(lib, None)[0] == 1
    assert _wcreate(lib, _wcfg(n_layers=0))[0] == 1
    assert _wcreate(lib, _wcfg(latent_tokens=0, action_tokens=0))[0] == 1   # no tokens at all
    assert _wcreate(lib, _wcfg(latent_tokens=-1))[0] == 1
    assert _wcreate(lib, _wcfg(rms_eps=-1.0))[0] == 1
    assert _wcreate(lib, _wcfg(width=200))[0] == 5
    assert _wcreate(lib, _wcfg(width=4096))[0] == 5
    assert _wcreate(lib, _wcfg(head_dim=48))[0] == 5
    assert _wcreate(lib, _wcfg(n_heads=3))[0] == 5                         # 3 x 64 not a multiple of 128
    assert _wcreate(lib, _wcfg(latent_dim=300))[0] == 5
    assert _wcreate(lib, _wcfg(mlp_dim=1000))[0] == 5
    assert _wcreate(lib, _wcfg(solver_order=3))[0] == 1                    # UniPC orders 1, 2 only
    assert _wcreate(lib, _wcfg(solver_order=-1))[0] == 1
    st, h = _wcreate(lib, _wcfg(n_layers=0))
    assert h.value is None


def test_joint_null_context_calls_fail_cleanly(lib):
    assert lib.phyai_wam_set_weights(None, None) == 1
    assert lib.phyai_wam_set_conditions(None, None, None, 3.0) == 1
    assert lib.phyai_wam_denoise(None, None, None, 1, None, None) == 1
