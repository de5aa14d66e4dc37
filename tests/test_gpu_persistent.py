"""GPU parity of the persistent Euler loop (one cooperative kernel for the whole chunk) against
the float64 oracle, and against the graph of per-layer launches (needs an MI355X).

The persistent loop runs for bf16 batches of at most 64 token rows on the shapes it implements:
the pi0.5-shaped expert, and a reduced shape with the same head structure (8 query heads, one
KV head) at width 256, head_dim 128, MLP 1024, used here for several batch sizes, ragged chunks
and prefixes.  Tolerance: 2e-2 norm-wise (bf16), as for every bf16 parity test.  Pages: PhyAI
reading Sec. 5.1 (the cached loop); "FlashRT-PAI speeds physical AI inference up to 12.66x"
(deep kernel fusion with launch overlap).
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
# the reduced shape with the persistent loop's head structure
SMALL = synth.ExpertDims(2, 256, 8, 1, 128, 1024, 64, 16, 8, 4, 1, "bf16")


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(d, inputs, persistent=True, reps=1, max_batch=None):
    t = ex.schedule(d.n_steps)
    dev = device_inputs(d, inputs)
    e = make_expert(d, dev, t, max_batch=max_batch or d.batch)
    e.set_persistent(persistent)
    form = e.loop_form(d.batch)
    outs = []
    for _ in range(reps):
        outs.append(e.denoise(dev["noise"]).cpu().numpy())
    e.sync()
    e.close()
    return outs, form


@pytest.mark.parametrize("batch,chunk,prefix", [(1, 16, 64), (2, 16, 64), (4, 16, 100), (1, 50, 64), (3, 20, 1),
                                                (4, 16, 330), (1, 16, 1100)])
def test_small_persistent_matches_oracle(batch, chunk, prefix):
    """Reduced shape: 1-4 samples (16 to 64 token rows: one to four row tiles, ragged), a
    one-token prefix, one-block key splits, and two-block splits with a one-block last split
    (4 x 16 rows over 346 keys: 11 blocks in 6 splits; 16 rows over 1116 keys: 35 blocks in
    18 splits)."""
    d = dataclasses.replace(SMALL, batch=batch, chunk_len=chunk, prefix_len=prefix)
    _say(f"case: persistent small, batch {batch}, chunk {chunk}, prefix {prefix}")
    inp = synth.make_expert_inputs(d, 0)
    (got,), form = _run(d, inp)
    assert form == 1
    ref = ex.denoise(inp, d)
    err = rel_err(got, ref)
    _say(f"persistent small b{batch} H{chunk} P{prefix}: rel err {err:.3e}")
    assert err <= 2e-2
    (graph,), gform = _run(d, inp, persistent=False)
    assert gform == 0
    _say(f"  vs graph path: {rel_err(got, graph):.3e}")
    assert rel_err(got, graph) <= 2e-2


def test_small_persistent_replays_are_bitwise_equal():
    """Every sum of the persistent loop is taken in a fixed order: repeated launches (and the
    epoch flags advancing across them) give the same bits."""
    d = dataclasses.replace(SMALL, batch=2)
    inp = synth.make_expert_inputs(d, 1)
    outs, form = _run(d, inp, reps=4)
    assert form == 1
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_pi05_persistent_matches_oracle():
    _say("case: pi05 bf16 batch 1, persistent loop")
    inp = synth.make_expert_inputs(PI05, 0)
    outs, form = _run(PI05, inp, reps=3)
    assert form == 1
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    err = rel_err(outs[0], ex.denoise(inp, PI05))
    _say(f"pi05 persistent rel err {err:.3e}")
    assert err <= 2e-2


def test_persistent_prefix_invalidation_and_fallback():
    """The loop is off until enabled; a new prefix changes the chunk as the oracle says; shapes
    or modes the persistent loop does not implement (RoPE, a disabled loop) report the graph
    form and still match."""
    d = SMALL
    inp = synth.make_expert_inputs(d, 0)
    t = ex.schedule(d.n_steps)
    dev = device_inputs(d, inp)
    e = make_expert(d, dev, t)
    assert e.loop_form(1) == 0  # off until enabled
    e.set_persistent(True)
    assert e.loop_form(1) == 1
    first = e.denoise(dev["noise"]).cpu().numpy()
    inp2 = synth.make_expert_inputs(d, 7)
    e.set_prefix_kv(torch.from_numpy(inp2["k_pre"]).cuda().to(torch.bfloat16).contiguous(),
                    torch.from_numpy(inp2["v_pre"]).cuda().to(torch.bfloat16).contiguous())
    second = e.denoise(dev["noise"]).cpu().numpy()
    e.set_persistent(False)
    assert e.loop_form(1) == 0
    e.sync()
    e.close()
    ref2 = ex.denoise(dict(inp, k_pre=inp2["k_pre"], v_pre=inp2["v_pre"]), d)
    assert rel_err(second, first) > 1e-2
    assert rel_err(second, ref2) <= 2e-2
    dr = dataclasses.replace(d, rope_theta=1e4)
    er = make_expert(dr, device_inputs(dr, inp), t)
    er.set_persistent(True)
    assert er.loop_form(1) == 0
    er.close()
