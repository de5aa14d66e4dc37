"""The action-expert context's call contract on a live device (needs an MI355X):
call order, argument and capacity errors, the arena limit, and batches padded to the
graph bucket.  Every call goes through the C ABI; a rejected call must leave the
context usable and its installed state unchanged.

Pages: PhyAI reading Sec. 5.1 (the cached prefix has a precise boundary: a new
observation invalidates it; tables belong to a fixed schedule) and Sec. 8.1, Appendix D
(local graph batch with padding for incomplete batches)."""
import ctypes
import dataclasses
import sys

import numpy as np
import pytest

import synth
from oracle import expert as ex

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import flow_matching_action_cached_amd as fm  # noqa: E402
from gpu_util import WEIGHT_KEYS, device_inputs, make_expert, rel_err  # noqa: E402

TINY = synth.CONFIGS["tiny"]
TINY_BF16 = dataclasses.replace(TINY, weight_dtype="bf16")
PI05_B32 = synth.CONFIGS["pi05_b32"]

OK, INVALID, BAD_STATE, OOM = 0, 1, 2, 3


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _denoise_raw(e, noise, batch, n_steps, out):
    return e._lib.phyai_denoise(e._h, _ptr(noise), int(batch), int(n_steps), _ptr(out))


def _message(e):
    return e._lib.phyai_last_error(e._h).decode()


def test_expert_call_order_is_enforced():
    """denoise needs weights, a prefix and tables, in that order of availability; tables
    need weights; each refusal is BAD_STATE with a message and leaves the context usable."""
    inp = synth.make_expert_inputs(TINY, 0)
    dev = device_inputs(TINY, inp)
    t = ex.schedule(TINY.n_steps)
    e = fm.ActionExpert.from_dims(TINY)
    out = torch.empty_like(dev["noise"])
    # nothing set yet
    assert _denoise_raw(e, dev["noise"], 1, TINY.n_steps, out) == BAD_STATE
    assert "weights" in _message(e)
    arr = (ctypes.c_float * len(t))(*[float(x) for x in t])
    assert e._lib.phyai_set_timestep_tables(e._h, arr, len(t)) == BAD_STATE   # tables need weights
    e.set_weights({k: dev[k] for k in WEIGHT_KEYS})
    assert _denoise_raw(e, dev["noise"], 1, TINY.n_steps, out) == BAD_STATE
    assert "prefix" in _message(e)
    e.set_prefix_kv(dev["k_pre"], dev["v_pre"])
    assert _denoise_raw(e, dev["noise"], 1, TINY.n_steps, out) == BAD_STATE
    assert "tables" in _message(e)
    e.set_timestep_tables(t)
    got = e.denoise(dev["noise"]).cpu().numpy()
    e.sync()
    assert rel_err(got, ex.denoise(inp, TINY)) <= 1e-4
    # new weights drop the tables (they fold the weights in): denoise refuses until rebuilt
    e.set_weights({k: dev[k] for k in WEIGHT_KEYS})
    assert _denoise_raw(e, dev["noise"], 1, TINY.n_steps, out) == BAD_STATE
    e.set_timestep_tables(t)
    again = e.denoise(dev["noise"]).cpu().numpy()
    e.close()
    assert np.array_equal(again, got)


def test_expert_argument_errors_leave_state_intact():
    """Wrong step count, batches outside [1, installed batch], prefixes and batches beyond
    the context's capacity, null pointers: INVALID_ARG, and the next good call still gives
    the oracle's chunk for the prefix installed before the refused calls."""
    d = dataclasses.replace(TINY, batch=2)
    inp = synth.make_expert_inputs(d, 0)
    dev = device_inputs(d, inp)
    t = ex.schedule(d.n_steps)
    e = make_expert(d, dev, t)                      # max_batch 2, max_prefix_len 64
    out = torch.empty_like(dev["noise"])
    lib, h = e._lib, e._h
    assert _denoise_raw(e, dev["noise"], 2, d.n_steps + 1, out) == INVALID    # tables hold 4 steps
    assert "n_steps" in _message(e)
    assert _denoise_raw(e, dev["noise"], 3, d.n_steps, out) == INVALID        # above the installed batch
    assert _denoise_raw(e, dev["noise"], 0, d.n_steps, out) == INVALID
    assert lib.phyai_denoise(h, None, 2, d.n_steps, _ptr(out)) == INVALID
    assert lib.phyai_denoise(h, _ptr(dev["noise"]), 2, d.n_steps, None) == INVALID
    # prefix beyond the capacity (65 > 64 keys, 3 > 2 samples) and bad sizes
    k_long = torch.zeros((2, d.n_layers, 65, 1, d.head_dim), device="cuda")
    assert lib.phyai_set_prefix_kv(h, _ptr(k_long), _ptr(k_long), 2, 65) == INVALID
    assert lib.phyai_set_prefix_kv(h, _ptr(k_long), _ptr(k_long), 3, 64) == INVALID
    assert lib.phyai_set_prefix_kv(h, _ptr(k_long), _ptr(k_long), 2, 0) == INVALID
    assert lib.phyai_set_prefix_kv(h, None, _ptr(k_long), 2, 64) == INVALID
    assert lib.phyai_set_timestep_tables(h, None, 4) == INVALID
    arr = (ctypes.c_float * 1)(float("nan"))
    assert lib.phyai_set_timestep_tables(h, arr, 1) == INVALID
    # the refused calls changed nothing: same prefix, same tables, same chunk
    got = e.denoise(dev["noise"]).cpu().numpy()
    e.sync()
    e.close()
    assert rel_err(got, ex.denoise(inp, d)) <= 1e-4


def test_expert_smaller_batch_runs_its_first_samples():
    """A call for fewer samples than the installed prefix runs samples 0..b-1 against their
    own prefix rows (batch 1 of a batch-2 prefix = sample 0 alone)."""
    d = dataclasses.replace(TINY, batch=2)
    inp = synth.make_expert_inputs(d, 0)
    dev = device_inputs(d, inp)
    e = make_expert(d, dev, ex.schedule(d.n_steps))
    one = e.denoise(dev["noise"][:1].contiguous()).cpu().numpy()
    e.sync()
    e.close()
    assert one.shape[0] == 1
    assert rel_err(one, ex.denoise(inp, d, samples=[0])) <= 1e-4


def test_expert_arena_limit_is_out_of_memory():
    """max_arena_bytes below what the capacity needs: creation fails with OOM and no
    context; a limit that fits succeeds."""
    cfg = dict(n_layers=TINY.n_layers, width=TINY.width, n_q_heads=TINY.n_q_heads, n_kv_heads=TINY.n_kv_heads,
               head_dim=TINY.head_dim, mlp_dim=TINY.mlp_dim, action_dim=TINY.action_dim,
               chunk_len=TINY.chunk_len, max_prefix_len=TINY.prefix_len, weight_dtype="f32")
    with pytest.raises(fm.PhyaiError) as err:
        fm.ActionExpert(max_arena_bytes=1 << 20, **cfg)             # the fp32 linears alone exceed 1 MiB
    assert err.value.status == OOM
    e = fm.ActionExpert(max_arena_bytes=1 << 30, **cfg)
    e.close()


def _padded_case(d, real, seed, samples):
    """Install `real` samples' prefixes in a context of capacity d.batch and denoise them
    (the bucket pads the rest); then install all d.batch samples whose first `real` are the
    same and denoise all.  Returns (padded run, full run, inputs)."""
    inp = synth.make_expert_inputs(d, seed)
    dev = device_inputs(d, inp)
    t = ex.schedule(d.n_steps)
    e = make_expert(d, dev, t)                      # full prefix installed (capacity batch)
    full = e.denoise(dev["noise"]).cpu().numpy()
    e.set_prefix_kv(dev["k_pre"][:real].contiguous(), dev["v_pre"][:real].contiguous())
    pad = e.denoise(dev["noise"][:real].contiguous()).cpu().numpy()
    e.sync()
    e.close()
    return pad, full, inp


def test_tiny_bf16_27_real_5_padded():
    """27 samples (432 token rows) run in the 32-sample bucket: the 27 real chunks equal
    bit for bit those of the full 32-sample run (same graph shape, samples never
    interact) and match the oracle."""
    d = dataclasses.replace(TINY_BF16, batch=32)
    pad, full, inp = _padded_case(d, 27, 3, None)
    assert pad.shape[0] == 27
    assert np.array_equal(pad, full[:27])
    ref = ex.denoise(inp, d, samples=range(27))
    err = rel_err(pad, ref)
    _say(f"tiny bf16 27 of 32 rel err {err:.3e}")
    assert err <= 2e-2


def test_pi05_batch32_bucket_with_27_real_samples():
    """The pi0.5-shaped batch-32 workload with 27 real samples and 5 pad slots: bitwise equal
    to the real rows of the full run, and sampled samples against the oracle."""
    _say("case: pi05 bf16 27 real + 5 padded")
    pad, full, _ = _padded_case(PI05_B32, 27, 0, None)
    assert np.array_equal(pad, full[:27])
    for b in (0, 26):
        one = synth.make_expert_inputs(PI05_B32, 0, batch=1, samples=[b])
        err = rel_err(pad[b], ex.denoise(one, PI05_B32)[0])
        _say(f"pi05 27/32 sample {b} rel err {err:.3e}")
        assert err <= 2e-2


def test_bucket_graphs_are_bounded():
    """More distinct (batch bucket, prefix length) pairs than the graph cache keeps: every
    call still gives the oracle's chunk (evicted graphs are re-captured)."""
    d = dataclasses.replace(TINY, batch=2)
    inp = synth.make_expert_inputs(d, 0)
    dev = device_inputs(d, inp)
    e = make_expert(d, dev, ex.schedule(d.n_steps))
    first = None
    for rep in range(2):
        for p in range(1, 20):                      # 19 prefix lengths > 16 kept graphs
            e.set_prefix_kv(dev["k_pre"][:, :, :p].contiguous(), dev["v_pre"][:, :, :p].contiguous())
            got = e.denoise(dev["noise"]).cpu().numpy()
            if p == 7:
                if first is None:
                    first = got
                else:
                    assert np.array_equal(got, first)   # re-captured after eviction: same bits
    e.sync()
    e.close()
    sub = dict(inp, k_pre=inp["k_pre"][:, :, :19], v_pre=inp["v_pre"][:, :, :19])
    assert rel_err(got, ex.denoise(sub, dataclasses.replace(d, prefix_len=19))) <= 1e-4
