"""GPU tests of the execution-state capsules (snapshot, restore and fork of the installed
prefix K/V; page "FlashRT-PAI speeds physical AI inference up to 12.66x", its account of
the three mechanisms).

A restored capsule must reproduce the chunk of the prefix it snapshot bit for bit (the
loop is deterministic: graph replays are bitwise equal), in its own context and in a
second one of the same shape; a fork must give the oracle's chunk for a batch whose
samples share one observation.  Every call goes through the C ABI.
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

TINY = synth.CONFIGS["tiny"]
PI05 = synth.CONFIGS["pi05"]


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _capsule_bytes(d, batch):
    es = 4 if d.weight_dtype == "f32" else 2
    return 256 + 2 * batch * d.n_layers * d.n_kv_heads * d.prefix_len * d.head_dim * es


def test_tiny_capsule_restore_reproduces_the_snapshot():
    """Save prefix A, install prefix B, restore A: the chunk equals A's bitwise (and A's is
    the oracle's to 1e-4); restoring into a second context of the same shape does too."""
    _say("case: tiny fp32 capsule save/restore")
    inp_a = synth.make_expert_inputs(TINY, 0)
    inp_b = synth.make_expert_inputs(TINY, 1)
    t = ex.schedule(TINY.n_steps)
    dev_a = device_inputs(TINY, inp_a)
    dev_b = device_inputs(TINY, inp_b)
    e = make_expert(TINY, dev_a, t)
    a = e.denoise(dev_a["noise"]).cpu().numpy()
    cap = e.capsule_save()
    e.sync()
    assert cap.numel() == _capsule_bytes(TINY, 1)
    # documented payload: K [B][L][Hkv][P][dh], then V^T [B][L][Hkv][dh][P] (prefix K/V are
    # handed over as [B][L][P][Hkv][dh])
    pay = cap[256:].cpu().numpy().view(np.float32)
    half = pay.size // 2
    assert np.array_equal(pay[:half], inp_a["k_pre"].transpose(0, 1, 3, 2, 4).ravel())
    assert np.array_equal(pay[half:], inp_a["v_pre"].transpose(0, 1, 3, 4, 2).ravel())
    e.set_prefix_kv(dev_b["k_pre"], dev_b["v_pre"])
    b = e.denoise(dev_a["noise"]).cpu().numpy()
    assert rel_err(b, a) > 1e-3                      # the other prefix changes the chunk
    e.capsule_restore(cap)
    a2 = e.denoise(dev_a["noise"]).cpu().numpy()
    e.sync()
    assert np.array_equal(a2, a)
    assert rel_err(a, ex.denoise(inp_a, TINY)) <= 1e-4
    # a second context (same weights, prefix B installed, larger prefix capacity) takes it too
    e2 = make_expert(TINY, dict(dev_a, k_pre=dev_b["k_pre"], v_pre=dev_b["v_pre"]), t, max_prefix_len=96)
    e2.capsule_restore(cap)
    a3 = e2.denoise(dev_a["noise"]).cpu().numpy()
    e2.sync()
    assert rel_err(a3, a) <= 1e-5                    # other cache stride: same values, other split
    e.close()
    e2.close()


def test_tiny_capsule_fork_shares_one_observation():
    """Batch 2, fork sample 0's prefix into slot 1: sample 1 is the oracle's chunk of its
    own noise under sample 0's prefix; sample 0 is unchanged."""
    _say("case: tiny fp32 capsule fork, batch 2")
    d = dataclasses.replace(TINY, batch=2)
    inp = synth.make_expert_inputs(d, 0)
    t = ex.schedule(d.n_steps)
    dev = device_inputs(d, inp)
    e = make_expert(d, dev, t)
    before = e.denoise(dev["noise"]).cpu().numpy()
    e.capsule_fork(0, 1)
    after = e.denoise(dev["noise"]).cpu().numpy()
    e.sync()
    ref_inp = dict(inp, k_pre=inp["k_pre"][[0, 0]], v_pre=inp["v_pre"][[0, 0]])
    ref = ex.denoise(ref_inp, d)
    _say(f"fork rel err {rel_err(after, ref):.3e}")
    assert rel_err(after, ref) <= 1e-4
    assert np.array_equal(after[0], before[0])
    assert rel_err(after[1], before[1]) > 1e-3
    e.close()


def test_capsule_argument_errors():
    """No prefix, foreign bytes, a short buffer, a capsule of another shape or a larger batch,
    and sample indices outside the batch are rejected with an error and change nothing."""
    import flow_matching_action_cached_amd as fm
    inp = synth.make_expert_inputs(TINY, 0)
    t = ex.schedule(TINY.n_steps)
    dev = device_inputs(TINY, inp)
    bare = fm.ActionExpert.from_dims(TINY)
    assert bare._lib.phyai_capsule_bytes(bare._h) == 0
    with pytest.raises(fm.PhyaiError):
        bare.capsule_save()
    e = make_expert(TINY, dev, t)
    ref = e.denoise(dev["noise"]).cpu().numpy()
    cap = e.capsule_save()
    e.sync()
    bad = cap.clone()
    bad[0] ^= 1
    with pytest.raises(fm.PhyaiError):
        e.capsule_restore(bad)
    with pytest.raises(fm.PhyaiError):
        e.capsule_restore(cap[: cap.numel() - 4])
    with pytest.raises(fm.PhyaiError):
        e.capsule_fork(0, 1)                         # batch 1: slot 1 does not exist
    other = make_expert(dataclasses.replace(TINY, n_layers=1), device_inputs(
        dataclasses.replace(TINY, n_layers=1), synth.make_expert_inputs(dataclasses.replace(TINY, n_layers=1), 0)), t)
    with pytest.raises(fm.PhyaiError):
        other.capsule_restore(cap)                   # 2-layer capsule into a 1-layer context
    d2 = dataclasses.replace(TINY, batch=2)
    e2 = make_expert(d2, device_inputs(d2, synth.make_expert_inputs(d2, 0)), t)
    cap2 = e2.capsule_save()
    e2.sync()
    with pytest.raises(fm.PhyaiError):
        e.capsule_restore(cap2)                      # batch 2 into a batch-1 context
    got = e.denoise(dev["noise"]).cpu().numpy()      # the failed calls left the prefix alone
    e.sync()
    assert np.array_equal(got, ref)
    for x in (bare, e, other, e2):
        x.close()


def test_pi05_capsule_restore_after_prefix_change():
    """bf16 at the full shape (816 prefix tokens, 18 layers): snapshot, install a random
    prefix, restore: the chunk is bitwise the snapshot's."""
    _say("case: pi05 bf16 capsule save/restore")
    inp = synth.make_expert_inputs(PI05, 0)
    t = ex.schedule(PI05.n_steps)
    dev = device_inputs(PI05, inp)
    e = make_expert(PI05, dev, t)
    a = e.denoise(dev["noise"]).cpu().numpy()
    cap = e.capsule_save()
    e.sync()
    assert cap.numel() == _capsule_bytes(PI05, 1)
    g = torch.Generator(device="cuda").manual_seed(5)
    k = torch.randn(dev["k_pre"].shape, generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn(dev["v_pre"].shape, generator=g, device="cuda").to(torch.bfloat16)
    e.set_prefix_kv(k, v)
    b = e.denoise(dev["noise"]).cpu().numpy()
    e.capsule_restore(cap)
    a2 = e.denoise(dev["noise"]).cpu().numpy()
    e.sync()
    assert rel_err(b, a) > 1e-2
    assert np.array_equal(a2, a)
    e.close()


def test_tiny_capsule_restores_into_a_larger_context_and_self_fork_is_a_no_op():
    """A batch-1 capsule restored into a context with room for 2 samples and 128 prefix
    rows installs batch 1 there (the chunk equals the source context's bit for bit only up
    to the attention split of the other capacity: 1e-5); forking a sample onto itself
    changes nothing."""
    _say("case: tiny fp32 capsule into a larger context")
    inp = synth.make_expert_inputs(TINY, 0)
    t = ex.schedule(TINY.n_steps)
    dev = device_inputs(TINY, inp)
    e = make_expert(TINY, dev, t)
    a = e.denoise(dev["noise"]).cpu().numpy()
    cap = e.capsule_save()
    e.capsule_fork(0, 0)
    a2 = e.denoise(dev["noise"]).cpu().numpy()
    e.sync()
    assert np.array_equal(a2, a)
    d2 = dataclasses.replace(TINY, batch=2)
    dev2 = device_inputs(d2, synth.make_expert_inputs(d2, 1))
    big = make_expert(d2, dict(dev2, **{k: dev[k] for k in dev if k not in ("k_pre", "v_pre", "noise")}), t,
                      max_prefix_len=128)
    big.capsule_restore(cap)
    assert big._lib.phyai_capsule_bytes(big._h) == cap.numel()   # now holds batch 1, 64 rows
    b = big.denoise(dev["noise"]).cpu().numpy()
    big.sync()
    assert rel_err(b, a) <= 1e-5
    assert rel_err(a, ex.denoise(inp, TINY)) <= 1e-4
    e.close()
    big.close()
