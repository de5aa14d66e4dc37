"""GPU parity of the attention kernels on peaked softmaxes (needs an MI355X).

Both attention kernels keep a reference maximum per query row and rescale the running
output and row sum only when a later group of keys raises some row's maximum by more
than 8 in log2 units.  At N(0, 0.02) weights the scores are nearly flat and that branch
never runs, so these cases make it run and check the result against the float64 oracle:

* planted keys: in a key group after the first of every key split, one prefix key is set
  to c * q_hat, q_hat the unit direction of a query row's layer-0, step-0 query, with c
  chosen so that row's score on it beats every other key by 12 (natural units);
* queries scaled by 8 (the query rows of W_qkv times 8, exact in bf16), the stress
  variant of the method's softmax (scores of standard deviation ~6 instead of ~0.7),
  and for the joint denoiser query and key rows x6.

Each test recomputes the layer-0, step-0 scores with the oracle's building blocks and
asserts that some query row really crosses the threshold inside some key split under
the key grouping the kernels use (the launch plan below restates the host's choice).
Tolerances: 1e-4 (fp32), 2e-2 (bf16), norm-wise, as for every parity test.
Pages: PhyAI reading Sec. 5.1 (attention over the cached prefix and the chunk), Sec. 8.2
check 1 (numerical checks on fixed inputs with stated tolerances).
"""
import dataclasses
import math
import sys

import numpy as np
import pytest

import synth
from oracle import expert as ex
from oracle import wam as owam

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
from gpu_util import device_inputs, make_expert, rel_err  # noqa: E402

TINY = synth.CONFIGS["tiny"]
PI05 = synth.CONFIGS["pi05"]
LOG2E = 1.4426950408889634


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _plan(B, hq, hkv, H, T, dh, es):
    """Key grouping of the attention launch for B samples, T keys (restating the host's
    plan): returns (blocks per split, 32-key blocks per staged group, wide kernel?)."""
    nblk = -(-T // 32)
    QT = -(-(hq // hkv) * H // 16)
    QG = -(-QT // 4)
    S = min(max(1, 256 // (B * hkv * QG)), 32, nblk)
    wide = es == 2 and B * hkv * QT >= 64
    if wide:
        tpw, nbg = (16 if dh <= 128 else 8), (4 if dh <= 64 else 2)
        wbase = B * hkv * -(-QT // tpw)
        S = 1
        for c in range(2, min(4, -(-nblk // nbg)) + 1):
            if -(-wbase * c // 256) * S < -(-wbase * S // 256) * c:
                S = c
        return -(-nblk // S), nbg, True
    bps = -(-nblk // S)
    nb = 1 if bps == 1 else (2 if (bps <= 2 or dh * es > 512) else 4)
    return bps, nb, False


def _crossings(s2, bps, nb):
    """(row, split) pairs whose max over a later key group of the split exceeds the max
    over the split's first group by more than 8; s2: [rows][T] scores in log2 units."""
    T = s2.shape[1]
    nblk = -(-T // 32)
    n = 0
    for b0 in range(0, nblk, bps):
        b1 = min(nblk, b0 + bps)
        first = s2[:, b0 * 32:min(T, min(b1, b0 + nb) * 32)].max(axis=1)
        for g0 in range(b0 + nb, b1, nb):
            later = s2[:, g0 * 32:min(T, min(b1, g0 + nb) * 32)].max(axis=1)
            n += int(np.sum(later > first + 8.0))
    return n


def _layer0_q(inp, d, b):
    """Layer-0, step-0 queries of sample b, [Hq][H][dh] (float64, the oracle's blocks)."""
    t = ex.schedule(d.n_steps)
    mods = ex.modulation_tables(t, inp["w_mod"], inp["b_mod"])[0]
    h = np.asarray(inp["noise"][b], np.float64) @ np.asarray(inp["w_in"], np.float64).T + inp["b_in"]
    u = ex.ada_rms(h, mods[0][0], mods[0][1], d.rms_eps)
    q = u @ np.asarray(inp["w_qkv"][0][:d.n_q_heads * d.head_dim], np.float64).T
    return q.reshape(d.chunk_len, d.n_q_heads, d.head_dim).transpose(1, 0, 2)


def _layer0_scores_log2(inp, d, b):
    """Scores of every query row (head-major, then token) over the prefix keys of layer 0,
    in log2 units: q k / sqrt(dh) * log2(e).  The chunk's own keys are left out; they sit
    in the split's last block and only add keys."""
    q = _layer0_q(inp, d, b)                                     # Hkv = 1 in these cases
    k = np.asarray(inp["k_pre"][b][0][:, 0], np.float64)          # [P][dh]
    s = np.einsum("htd,pd->htp", q, k).reshape(-1, k.shape[0])
    return s / math.sqrt(d.head_dim) * LOG2E


def _boost_queries(inp, d, factor):
    w = inp["w_qkv"].copy()
    w[:, :d.n_q_heads * d.head_dim] *= np.float32(factor)         # power of two: exact in bf16
    return dict(inp, w_qkv=w)


def _plant(inp, d, bps, nb, margin=12.0):
    """Plant one key per split in the split's second key group: for sample b, every planted
    row of layer 0's prefix K is c q_hat (q_hat: head 0, token 0's query direction), c giving
    that row a score `margin` above its best unplanted key."""
    rnd = synth.bf16_values if d.weight_dtype == "bf16" else (lambda a: a)
    k_pre = inp["k_pre"].copy()
    P = d.prefix_len
    nblk = -(-(P + d.chunk_len) // 32)
    for b in range(k_pre.shape[0]):
        q0 = _layer0_q(inp, d, b)[0, 0]
        s_best = float(np.max(np.asarray(k_pre[b][0][:, 0], np.float64) @ q0)) / math.sqrt(d.head_dim)
        c = (s_best + margin) * math.sqrt(d.head_dim) / float(np.linalg.norm(q0))
        vec = rnd((c * q0 / np.linalg.norm(q0)).astype(np.float32))
        for b0 in range(0, nblk, bps):
            key = (b0 + nb) * 32 + 3                     # first block of the split's second group
            if b0 + nb < min(nblk, b0 + bps) and key < P:
                k_pre[b][0][key][0] = vec
    return dict(inp, k_pre=k_pre)


def _run(d, inp, max_batch=None):
    t = ex.schedule(d.n_steps)
    dev = device_inputs(d, inp)
    e = make_expert(d, dev, t, max_batch=max_batch or d.batch)
    out = e.denoise(dev["noise"]).cpu().numpy()
    e.sync()
    e.close()
    return out


def test_few_row_attention_multi_group_rescale_fp32():
    """Few-row kernel with several staged key groups per split: a 4200-key prefix at batch
    1 gives 27 splits of 5 blocks, staged as 4 + 1.  Queries x8 and a planted key in every
    split's second group; fp32 parity 1e-4."""
    d = dataclasses.replace(TINY, prefix_len=4200)
    bps, nb, wide = _plan(1, d.n_q_heads, d.n_kv_heads, d.chunk_len, d.prefix_len + d.chunk_len, d.head_dim, 4)
    assert (bps, nb, wide) == (5, 4, False)
    inp = _plant(_boost_queries(synth.make_expert_inputs(d, 2), d, 8.0), d, bps, nb)
    n = _crossings(_layer0_scores_log2(inp, d, 0), bps, nb)
    _say(f"fp32 4200 keys: {n} (row, split) threshold crossings at layer 0, step 0")
    assert n >= 20
    got = _run(d, inp)
    err = rel_err(got, ex.denoise(inp, d))
    _say(f"fp32 4200 keys peaked rel err {err:.3e}")
    assert err <= 1e-4


def test_wide_attention_planted_keys_rescale_bf16():
    """Many-row kernel (16 samples x 64 query rows, bf16): a 1200-key prefix gives 4 splits
    of 10 blocks staged 4 + 4 + 2; each sample plants a key in every split's second group."""
    d = dataclasses.replace(TINY, weight_dtype="bf16", batch=16, prefix_len=1200)
    bps, nb, wide = _plan(16, d.n_q_heads, d.n_kv_heads, d.chunk_len, d.prefix_len + d.chunk_len, d.head_dim, 2)
    assert (bps, nb, wide) == (10, 4, True)
    inp = _plant(synth.make_expert_inputs(d, 3), d, bps, nb)
    n = sum(_crossings(_layer0_scores_log2(inp, d, b), bps, nb) for b in range(d.batch))
    _say(f"bf16 wide planted: {n} threshold crossings at layer 0, step 0")
    assert n >= 16 * 3
    got = _run(d, inp)
    err = rel_err(got, ex.denoise(inp, d))
    _say(f"bf16 wide planted rel err {err:.3e}")
    assert err <= 2e-2


# The stress variant is ill-conditioned in bf16 itself at the full depth: a float64 simulation
# of the path's bf16 rounding points (GEMM inputs, q/k/v, softmax weights, attention output;
# no kernel involved) lands 1.6e-1 from the exact oracle on the 18-layer, 10-step pi0.5 chunk
# with queries x8 (2.0e-3 at x1, 3.1e-3 at x2, 1.2e-2 at 2 layers x 2 steps, 5.1e-3 at one
# layer and one step).  So x8 is checked where the tolerance measures the kernels: the full
# width, heads, MLP and 816-key prefix at one layer and one step; and x2 at the full depth.
@pytest.mark.parametrize("batch", [1, 3])
def test_pi05_queries_x8_one_layer_one_step(batch):
    """Queries x8 at the pi0.5 width, heads and prefix, one layer, one Euler step.  Batch 1
    runs the few-row kernel (28 one-block splits merged by the split-merge launch: peaked
    partials with very different maxima); batch 3 (75 query tiles) the many-row kernel with
    4 splits of 7 blocks staged in pairs, where the rescale branch runs."""
    _say(f"case: pi05 queries x8, 1 layer, 1 step, batch {batch}")
    d = dataclasses.replace(PI05, batch=batch, n_layers=1, n_steps=1)
    inp = _boost_queries(synth.make_expert_inputs(d, 0), d, 8.0)
    bps, nb, wide = _plan(batch, d.n_q_heads, d.n_kv_heads, d.chunk_len, d.prefix_len + d.chunk_len,
                          d.head_dim, 2)
    assert wide == (batch == 3)
    s2 = _layer0_scores_log2(inp, d, 0)
    _say(f"layer-0 score std {s2.std() / LOG2E:.2f} (natural units)")
    assert s2.std() / LOG2E > 4.0                                  # peaked, not the flat ~0.7
    if wide:
        n = sum(_crossings(_layer0_scores_log2(inp, d, b), bps, nb) for b in range(batch))
        _say(f"pi05 x8 batch {batch}: {n} threshold crossings at layer 0, step 0")
        assert n >= 10
    got = _run(d, inp)
    err = rel_err(got, ex.denoise(inp, d))
    _say(f"pi05 queries x8 batch {batch} rel err {err:.3e}")
    assert err <= 2e-2


def test_pi05_queries_x2_full_depth():
    """Queries x2 through all 18 layers and 10 steps at batch 1 (scores of standard deviation
    ~1.5 instead of ~0.7)."""
    _say("case: pi05 queries x2, batch 1")
    inp = _boost_queries(synth.make_expert_inputs(PI05, 0), PI05, 2.0)
    got = _run(PI05, inp)
    err = rel_err(got, ex.denoise(inp, PI05))
    _say(f"pi05 queries x2 rel err {err:.3e}")
    assert err <= 2e-2


def test_joint_peaked_scores_multi_group():
    """Joint denoiser self-attention with 1000 latent + 24 action tokens (4 splits of 8
    blocks, two staged groups each) and query and key rows of W_qkv x6 (scores of standard
    deviation ~5): the rescale branch of the many-row kernel with no prefix, at one layer
    and one step (the peaked softmax is ill-conditioned in bf16 at depth, see above)."""
    d = dataclasses.replace(synth.WAM_CONFIGS["wam_tiny"], latent_tokens=1000, n_steps=1, n_layers=1)
    inp = synth.make_wam_inputs(d, 0)
    w = inp["w_qkv"].copy()
    w[:, :2 * d.n_heads * d.head_dim] *= np.float32(6.0)
    inp = dict(inp, w_qkv=w)
    T = d.latent_tokens + d.action_tokens
    # two branches run as a batch of two: B = 2, Hq = Hkv = heads, one query head per KV head
    bps, nb, wide = _plan(2, d.n_heads, d.n_heads, T, T, d.head_dim, 2)
    assert (bps, nb, wide) == (8, 4, True)
    t = ex.schedule(d.n_steps)
    p = {k: np.asarray(inp[k], np.float64) for k in ("w_in_lat", "b_in_lat", "w_in_act", "b_in_act", "w_qkv")}
    mods = owam.modulation(t[0], inp["c_cond"], inp["w_mod"], inp["b_mod"])
    h = np.concatenate([np.asarray(inp["z_lat"], np.float64) @ p["w_in_lat"].T + p["b_in_lat"],
                        np.asarray(inp["z_act"], np.float64) @ p["w_in_act"].T + p["b_in_act"]])
    u = ex.ada_rms(h, mods[0][0], mods[0][1], d.rms_eps)
    qkv = u @ p["w_qkv"][0].T
    hd = d.n_heads * d.head_dim
    q = qkv[:, :hd].reshape(T, d.n_heads, d.head_dim).transpose(1, 0, 2)
    k = qkv[:, hd:2 * hd].reshape(T, d.n_heads, d.head_dim).transpose(1, 0, 2)
    n = sum(_crossings(q[i] @ k[i].T / math.sqrt(d.head_dim) * LOG2E, bps, nb) for i in range(d.n_heads))
    _say(f"joint peaked: {n} threshold crossings (conditional branch, layer 0, step 0)")
    assert n >= 10

    import flow_matching_action_cached_amd as fm
    dev = {}
    for key, v in inp.items():
        tt = torch.from_numpy(np.ascontiguousarray(v)).cuda()
        dev[key] = tt if key in ("z_lat", "z_act") else tt.to(torch.bfloat16).contiguous()
    jd = fm.JointDenoiser.from_dims(d)
    jd.set_weights(dev)
    jd.set_conditions(dev["c_cond"], dev["c_uncond"], d.guidance)
    jd.set_timestep_tables(t)
    zl, za = jd.denoise(dev["z_lat"], dev["z_act"])
    jd.sync()
    got = np.concatenate([zl.cpu().numpy().ravel(), za.cpu().numpy().ravel()])
    jd.close()
    rl, ra = owam.denoise(inp, d, t)
    err = rel_err(got, np.concatenate([rl.ravel(), ra.ravel()]))
    _say(f"joint peaked rel err {err:.3e}")
    assert err <= 2e-2
