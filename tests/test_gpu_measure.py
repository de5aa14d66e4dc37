"""The measurement aids of the C ABI on a live device (needs an MI355X):
phyai_time_loop_stages (in-loop duration of each kernel of the denoise loop, as bench.py
uses it for the roofline) and phyai_enqueue_kernel_repeat.  They must measure the same
loop as phyai_denoise without changing its result, reject bad arguments, and report
plausible times: every launched kernel id a positive interval, ids without a launch zero,
and the marked loop no shorter than its parts.

Pages: PhyAI reading Sec. 8.2 check 1 (timing protocol reported explicitly);
"FlashRT-PAI speeds physical AI inference up to 12.66x" (gaps between operations)."""
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
from gpu_util import device_inputs, make_expert  # noqa: E402

SMALL = synth.ExpertDims(2, 256, 8, 1, 128, 1024, 64, 16, 8, 4, 1, "bf16")
INVALID, BAD_STATE = 1, 2


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("d", [dataclasses.replace(SMALL, batch=2), synth.CONFIGS["tiny"]], ids=["bf16-b2", "f32"])
def test_stage_times_measure_the_denoise_loop(d):
    _say(f"case: stage times {d.weight_dtype} batch {d.batch}")
    inp = synth.make_expert_inputs(d, 2)
    dev = device_inputs(d, inp)
    e = make_expert(d, dev, ex.schedule(d.n_steps))
    ref = e.denoise(dev["noise"]).cpu().numpy()
    us, ms = e.time_loop_stages(dev["noise"], reps=3)
    _say(f"  stage us {['%.2f' % u for u in us]}, loop {ms:.4f} ms")
    # every kernel id of the loop launched: 0 QKV, 1 attention, 2 O, 3 gate/up, 4 down,
    # 5 out/Euler/in, 6 first in-projection; 7 the split merge (launched here: several splits)
    for k in range(7):
        assert us[k] > 0.5, k
    L, N = d.n_layers, d.n_steps
    parts_ms = (N * L * sum(us[k] for k in (0, 1, 2, 3, 4, 7)) + N * us[5] + us[6]) / 1000.0
    assert ms >= 0.99 * parts_ms
    # the marked runs leave the state where a denoise leaves it: same result afterwards
    after = e.denoise(dev["noise"]).cpu().numpy()
    e.sync()
    assert np.array_equal(after, ref)
    e.close()


def test_stage_times_and_kernel_repeats_reject_bad_arguments():
    d = SMALL
    inp = synth.make_expert_inputs(d, 0)
    dev = device_inputs(d, inp)
    e = fm.ActionExpert.from_dims(d)
    us = (ctypes.c_float * 8)()
    ms = ctypes.c_float()
    noise_p = ctypes.c_void_p(dev["noise"].data_ptr())
    f = e._lib.phyai_time_loop_stages
    # before weights, prefix and tables
    assert f(e._h, noise_p, 1, 2, ctypes.addressof(us), ctypes.addressof(ms)) == BAD_STATE
    assert e._lib.phyai_enqueue_kernel_repeat(e._h, 0, 0, 1) == BAD_STATE
    e.close()
    e = make_expert(d, dev, ex.schedule(d.n_steps))
    assert f(e._h, noise_p, 1, 0, ctypes.addressof(us), ctypes.addressof(ms)) == INVALID      # reps
    assert f(e._h, noise_p, 1, 1001, ctypes.addressof(us), ctypes.addressof(ms)) == INVALID   # reps
    assert f(e._h, noise_p, 2, 1, ctypes.addressof(us), ctypes.addressof(ms)) == INVALID      # batch
    assert f(e._h, noise_p, 1, 1, None, ctypes.addressof(ms)) == INVALID                       # null
    assert f(e._h, noise_p, 1, 1, ctypes.addressof(us), None) == INVALID
    assert f(e._h, None, 1, 1, ctypes.addressof(us), ctypes.addressof(ms)) == INVALID
    assert e._lib.phyai_enqueue_kernel_repeat(e._h, 8, 0, 1) == INVALID                      # kernel id
    assert e._lib.phyai_enqueue_kernel_repeat(e._h, 0, d.n_layers, 1) == INVALID             # layer
    assert e._lib.phyai_enqueue_kernel_repeat(e._h, 0, 0, 0) == INVALID                      # reps
    assert f(None, noise_p, 1, 1, ctypes.addressof(us), ctypes.addressof(ms)) == INVALID
    # still usable
    out = e.denoise(dev["noise"]).cpu().numpy()
    e.sync()
    assert np.isfinite(out).all()
    e.close()
