"""The library's host-side UniPC step weights (the table phyai_set_timestep_tables uploads
for the joint denoiser) against the oracle's UniPC loop, without a device.

The loop is linear in the data predictions, so applying the weights the way the update
kernel does (corrector A x_{k-1} + w m_k + w m_{k-1} + w m_{k-2}, then predictor
A x_k + w m_k + w m_{k-1}) to a velocity stream that ignores the state must reproduce
oracle.wam.unipc_loop up to the float32 rounding of the weights."""
import numpy as np
import pytest

import flow_matching_action_cached_amd as fm
from oracle import expert as ex
from oracle import wam


def _apply(w, z0, vel):
    z, xp, ms = z0.copy(), None, {}
    for k in range(w.shape[0]):
        m = z - w[k, 0] * vel[k]
        xc = z
        if k >= 1:
            xc = w[k, 1] * xp + w[k, 2] * m + w[k, 3] * ms[k - 1] + w[k, 4] * (ms[k - 2] if k >= 2 else 0.0)
        z = w[k, 5] * xc + w[k, 6] * m + w[k, 7] * (ms[k - 1] if k >= 1 else 0.0)
        xp, ms[k] = xc, m
    return z


@pytest.mark.parametrize("sched", ["uniform6", "below_one", "two_from_one", "single"])
@pytest.mark.parametrize("order", [1, 2])
def test_library_weights_reproduce_the_oracle_loop(order, sched):
    t = {"uniform6": ex.schedule(6), "below_one": np.array([0.9, 0.7, 0.66, 0.4, 0.12], np.float32),
         "two_from_one": np.array([1.0, 0.5], np.float32), "single": np.array([0.8], np.float32)}[sched]
    w = fm.unipc_weights(t, order)
    rng = np.random.default_rng(order * 10 + len(t))
    vel = rng.normal(size=(len(t), 7))
    z0 = rng.normal(size=7)
    ref = wam.unipc_loop(z0, t, order, lambda z, k: vel[k])
    got = _apply(w.astype(np.float64), z0, vel)
    assert np.max(np.abs(got - ref)) <= 1e-6 * max(1.0, np.max(np.abs(ref)))


def test_library_weights_reject_bad_schedules_and_orders():
    for bad in ([1.2, 0.5], [0.5, 0.5], [0.5, 0.0], [0.3, 0.6]):
        with pytest.raises(fm.PhyaiError):
            fm.unipc_weights(np.array(bad, np.float32), 2)
    for order in (0, 3):
        with pytest.raises(fm.PhyaiError):
            fm.unipc_weights(ex.schedule(4), order)
    lib = fm.load_library()
    assert lib.phyai_unipc_weights(None, 1, 2, None) == 1
