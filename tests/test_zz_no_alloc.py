"""The allocation-free denoise (phyai_denoise_noalloc, through the C ABI) against phyai_denoise
on the same context and inputs (needs an MI355X).

Both run the same kernels in the same order, so the bar is bitwise equality.  Each test makes
two calls in a row, the second with a smaller batch: the static scratch keeps the first call's
partials and counters, so the second call shows that it starts from cleared counters and reads
only what it wrote.  A third case checks the documented size limit of the static scratch.
"""
import dataclasses
import sys

import numpy as np
import pytest

import synth
from oracle import expert as ex

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
from gpu_util import device_inputs, make_expert, rel_err  # noqa: E402

PI05 = synth.CONFIGS["pi05"]
SMALL = synth.ExpertDims(2, 256, 8, 1, 128, 1024, 64, 16, 8, 4, 1, "bf16")


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(e, noise):
    ref = e.denoise(noise).cpu().numpy()
    got = e.denoise_noalloc(noise).cpu().numpy()
    e.sync()
    return got, ref


@pytest.mark.parametrize("d, big, small", [
    (dataclasses.replace(SMALL, batch=4), 4, 2),                       # 64 then 32 token rows
    (dataclasses.replace(SMALL, batch=8, prefix_len=100), 8, 3),       # tiled path (128 rows), then streaming
    (dataclasses.replace(synth.CONFIGS["tiny"], batch=2), 2, 1),       # fp32
], ids=["bf16-b4-b2", "bf16-b8-b3", "f32-b2-b1"])
def test_noalloc_matches_denoise_twice(d, big, small):
    _say(f"case: noalloc {d.weight_dtype} L{d.n_layers} D{d.width} batch {big} then {small}")
    inp = synth.make_expert_inputs(d, 3)
    dev = device_inputs(d, inp)
    e = make_expert(d, dev, ex.schedule(d.n_steps))
    got, ref = _both(e, dev["noise"][:big].contiguous())
    assert np.array_equal(got, ref)
    # second call: fewer samples, with noise the first call gave to other samples
    got2, ref2 = _both(e, dev["noise"][big - small:big].contiguous())
    e.close()
    assert np.array_equal(got2, ref2)
    assert not np.array_equal(got2, got[:small])
    err = rel_err(got2, ex.denoise(dict(inp, noise=inp["noise"][big - small:big], k_pre=inp["k_pre"][:small],
                                        v_pre=inp["v_pre"][:small]), dataclasses.replace(d, batch=small)))
    _say(f"  second call vs oracle: {err:.3e}")
    assert err <= (1e-4 if d.weight_dtype == "f32" else 2e-2)


def test_noalloc_pi05_batch1_matches_denoise():
    """The benchmark workload (pi0.5-shaped expert, batch 1, prefix 816), twice."""
    _say("case: noalloc pi05 batch 1")
    inp = synth.make_expert_inputs(PI05, 0)
    dev = device_inputs(PI05, inp)
    e = make_expert(PI05, dev, ex.schedule(PI05.n_steps))
    for _ in range(2):
        got, ref = _both(e, dev["noise"])
        assert np.array_equal(got, ref)
    e.close()


def test_noalloc_rejects_beyond_its_scratch():
    """pi0.5 widths in fp32 (whose attention leaves one partial per 32-key block for a merge
    launch), one layer, 2 samples x 32 tokens over a 990-token prefix (32 key blocks): 32 query
    tiles, each split into 32 one-block splits, need 32 x 32 x 16512 B = 16.9 MB of attention
    partials, above the 16 MiB array.  phyai_denoise still runs it, and one sample (16 query
    tiles, 8.5 MB) fits."""
    import flow_matching_action_cached_amd as fm
    d = dataclasses.replace(PI05, n_layers=1, chunk_len=32, prefix_len=990, batch=2, n_steps=2, weight_dtype="f32")
    _say("case: noalloc limit, pi05 widths fp32, 1 layer, batch 2 x 32, prefix 990")
    inp = synth.make_expert_inputs(d, 5)
    dev = device_inputs(d, inp)
    e = make_expert(d, dev, ex.schedule(d.n_steps))
    with pytest.raises(fm.PhyaiError) as ei:
        e.denoise_noalloc(dev["noise"])
    assert ei.value.status == 1 and "at most 16777216" in str(ei.value)  # INVALID_ARG
    ref = e.denoise(dev["noise"]).cpu().numpy()
    got1, ref1 = _both(e, dev["noise"][:1].contiguous())  # one sample fits
    e.close()
    assert np.array_equal(got1, ref1) and np.isfinite(ref).all()
