"""GPU parity of the HIP denoise loop against the float64 oracle (needs an MI355X).

Tolerances (norm-wise max relative error max|gpu - ref| / max|ref|): 1e-4 for the
fp32 workload, 2e-2 for bf16 and int4 (fp32 accumulation), as stated for the
method's parity gate.  Every call goes through the C ABI.
"""
import dataclasses
import sys

import numpy as np
import pytest

import synth
from oracle import expert as ex
from oracle import int4 as q4

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


def _run(d, inputs, graph=True, t=None):
    t = ex.schedule(d.n_steps) if t is None else t
    dev = device_inputs(d, inputs)
    e = make_expert(d, dev, t, graph=graph)
    out = e.denoise(dev["noise"])
    e.sync()
    res = out.cpu().numpy()
    e.close()
    return res


def test_tiny_fp32_matches_oracle():
    _say("case: tiny fp32, seed 0")
    inp = synth.make_expert_inputs(TINY, 0)
    got = _run(TINY, inp)
    ref = ex.denoise(inp, TINY)
    err = rel_err(got, ref)
    _say(f"tiny fp32 rel err {err:.3e}")
    assert err <= 1e-4


def test_tiny_modulation_tables_match_oracle():
    inp = synth.make_expert_inputs(TINY, 0)
    t = ex.schedule(TINY.n_steps)
    dev = device_inputs(TINY, inp)
    e = make_expert(TINY, dev, t)
    got = e.get_modulation().cpu().numpy()
    e.close()
    ref = ex.modulation_tables(t, inp["w_mod"], inp["b_mod"])
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-6 * np.abs(ref).max())


def test_tiny_zero_weights_keep_noise():
    inp = synth.make_expert_inputs(TINY, 0)
    for k in ("w_in", "b_in", "w_out", "b_out", "w_mod", "b_mod", "w_qkv", "w_o", "w_gu", "w_d"):
        inp[k] = np.zeros_like(inp[k])
    got = _run(TINY, inp)
    assert np.array_equal(got, inp["noise"])


def test_tiny_graph_equals_eager_and_replays_are_deterministic():
    inp = synth.make_expert_inputs(TINY, 0)
    t = ex.schedule(TINY.n_steps)
    dev = device_inputs(TINY, inp)
    e = make_expert(TINY, dev, t, graph=False)
    eager = e.denoise(dev["noise"]).clone()
    e.set_graph_mode(True)
    g1 = e.denoise(dev["noise"]).clone()
    g2 = e.denoise(dev["noise"]).clone()
    e.sync()
    e.close()
    assert torch.equal(eager, g1) and torch.equal(g1, g2)


def test_tiny_prefix_invalidation():
    """A new prefix changes the output, and the new output matches the oracle fed the
    new prefix (stale-cache detection)."""
    inp = synth.make_expert_inputs(TINY, 0)
    t = ex.schedule(TINY.n_steps)
    dev = device_inputs(TINY, inp)
    e = make_expert(TINY, dev, t)
    first = e.denoise(dev["noise"]).cpu().numpy()
    inp2 = synth.make_expert_inputs(TINY, 5)
    k2 = torch.from_numpy(inp2["k_pre"]).cuda().contiguous()
    v2 = torch.from_numpy(inp2["v_pre"]).cuda().contiguous()
    e.set_prefix_kv(k2, v2)
    second = e.denoise(dev["noise"]).cpu().numpy()
    e.close()
    inp_new = dict(inp, k_pre=inp2["k_pre"], v_pre=inp2["v_pre"])
    assert rel_err(second, first) > 1e-3
    assert rel_err(second, ex.denoise(inp_new, TINY)) <= 1e-4


@pytest.mark.parametrize("prefix_len", [1, 33, 100])
def test_tiny_ragged_prefix_lengths(prefix_len):
    d = dataclasses.replace(TINY, prefix_len=prefix_len)
    inp = synth.make_expert_inputs(d, 0)
    got = _run(d, inp)
    assert rel_err(got, ex.denoise(inp, d)) <= 1e-4


@pytest.mark.parametrize("prefix_len", [1, 33, 1008, 1009])
def test_tiny_bf16_few_row_attention_key_ranges(prefix_len):
    """bf16 at batch 1 (4 query tiles) across key ranges of the split kernel: 17 keys (one
    block, a single split with no merge launch), 49 (two one-block splits, the second
    ragged), 1024 (32 one-block splits, the merge width) and 1025 (33 blocks: 17 two-block
    splits, the last holding one block)."""
    d = dataclasses.replace(TINY, prefix_len=prefix_len, weight_dtype="bf16")
    _say(f"case: tiny bf16, prefix {prefix_len}")
    inp = synth.make_expert_inputs(d, 4)
    got = _run(d, inp)
    err = rel_err(got, ex.denoise(inp, d))
    _say(f"tiny bf16 prefix {prefix_len} rel err {err:.3e}")
    assert err <= 2e-2


@pytest.mark.parametrize("wd,tol,batch", [("f32", 1e-4, 1), ("bf16", 2e-2, 3)])
def test_wide_action_dim_matches_oracle(wd, tol, batch):
    """Action dim 72 (four and a half 16-column tiles) with 20 chunk tokens: the
    out-projection / Euler / in-projection kernel updates a second element per thread
    (5 x 64 > 256 threads) and runs its in-projection over three 32-wide chunks, beyond the
    operands it loads up front for the first element and the first pass."""
    d = dataclasses.replace(TINY, action_dim=72, chunk_len=20, weight_dtype=wd, batch=batch)
    _say(f"case: action dim 72, {wd}, batch {batch}")
    inp = synth.make_expert_inputs(d, 2)
    got = _run(d, inp)
    err = rel_err(got, ex.denoise(inp, d))
    _say(f"  rel err {err:.3e}")
    assert err <= tol


def test_pi05_bf16_matches_oracle():
    _say("case: pi05 bf16 batch 1, seed 0")
    inp = synth.make_expert_inputs(PI05, 0)
    got = _run(PI05, inp)
    _say("pi05: gpu done, running oracle")
    ref = ex.denoise(inp, PI05)
    err = rel_err(got, ref)
    _say(f"pi05 bf16 rel err {err:.3e}")
    assert err <= 2e-2


def test_pi05_graph_replay_bitwise():
    inp = synth.make_expert_inputs(PI05, 0)
    t = ex.schedule(PI05.n_steps)
    dev = device_inputs(PI05, inp)
    e = make_expert(PI05, dev, t, graph=False)
    eager = e.denoise(dev["noise"]).clone()
    e.set_graph_mode(True)
    outs = [e.denoise(dev["noise"]).clone() for _ in range(3)]
    e.sync()
    e.close()
    assert all(torch.equal(eager, o) for o in outs)


@pytest.mark.parametrize("cfg,tol", [("tiny", 1e-4), ("pi05", 2e-2)])
def test_rope_variant_matches_oracle(cfg, tol):
    """Rotary embedding of the chunk's queries and keys (positions P + t, base 1e4) in the
    QKV epilogue of the weight-streaming GEMM, against the oracle's rotation."""
    d = dataclasses.replace({"tiny": TINY, "pi05": PI05}[cfg], rope_theta=1e4)
    _say(f"case: rope {cfg}")
    inp = synth.make_expert_inputs(d, 0)
    got = _run(d, inp)
    ref = ex.denoise(inp, d)
    err = rel_err(got, ref)
    _say(f"rope {cfg} rel err {err:.3e}")
    assert err <= tol
    assert rel_err(ref, ex.denoise(inp, dataclasses.replace(d, rope_theta=0.0))) > 2 * tol  # the rotation matters


@pytest.mark.parametrize("cfg,tol", [("tiny", 1e-4), ("pi05", 2e-2)])
def test_gated_residual_variant_matches_oracle(cfg, tol):
    """Residual gates from a third row block of each norm's modulation map, applied in the
    residual epilogues of the weight-streaming GEMMs, against the oracle."""
    d = dataclasses.replace({"tiny": TINY, "pi05": PI05}[cfg], gated_residual=True)
    _say(f"case: gated residual {cfg}")
    inp = synth.make_expert_inputs(d, 0)
    got = _run(d, inp)
    err = rel_err(got, ex.denoise(inp, d))
    _say(f"gated {cfg} rel err {err:.3e}")
    assert err <= tol


def test_time_mlp_tables_and_loop_match_oracle():
    """Time MLP before the modulation maps (tables built on the GPU in fp64): the tables and
    the whole tiny fp32 loop against the oracle."""
    d = dataclasses.replace(TINY, time_mlp=True)
    inp = synth.make_expert_inputs(d, 0)
    t = ex.schedule(d.n_steps)
    dev = device_inputs(d, inp)
    e = make_expert(d, dev, t)
    got_tab = e.get_modulation().cpu().numpy()
    got = e.denoise(dev["noise"]).cpu().numpy()
    e.sync()
    e.close()
    tm = tuple(inp[k] for k in ("w_tm1", "b_tm1", "w_tm2", "b_tm2"))
    ref_tab = ex.modulation_tables(t, inp["w_mod"], inp["b_mod"], tm)
    np.testing.assert_allclose(got_tab, ref_tab, rtol=0, atol=1e-6 * np.abs(ref_tab).max())
    err = rel_err(got, ex.denoise(inp, d))
    _say(f"time-mlp tiny rel err {err:.3e}")
    assert err <= 1e-4


def test_pi05_fidelity_variants_combined_match_oracle():
    """RoPE, residual gates and the time MLP together on the pi0.5-shaped bf16 expert."""
    d = dataclasses.replace(PI05, rope_theta=1e4, gated_residual=True, time_mlp=True)
    _say("case: pi05 rope + gated + time MLP")
    inp = synth.make_expert_inputs(d, 0)
    got = _run(d, inp)
    err = rel_err(got, ex.denoise(inp, d))
    _say(f"pi05 fidelity variants rel err {err:.3e}")
    assert err <= 2e-2


@pytest.mark.parametrize("prefix_len", [1200, 2100])
def test_tiny_long_prefix_uses_bounded_splits(prefix_len):
    """Prefixes with more key blocks than the merge width (32 splits): 1200 -> 38 blocks
    in 19 splits of two, 2100 -> 67 blocks in 23 splits of three (four staged blocks)."""
    d = dataclasses.replace(TINY, prefix_len=prefix_len)
    inp = synth.make_expert_inputs(d, 0)
    got = _run(d, inp)
    assert rel_err(got, ex.denoise(inp, d)) <= 1e-4


# ---------------------------------------------------------------- int4 (group-128) variant
PI05_I4 = synth.CONFIGS["pi05_int4"]


def test_int4_quantiser_bit_exact():
    """The library's GPU quantiser produces exactly the oracle's codes and scales
    (integer work: bit-exact), including an all-zero group, a ragged row count and exact
    ties: groups whose scale is a power of two (7 * 2^e as the largest magnitude) holding
    every half-integer multiple (n + 1/2) 2^e, so W / s is an exact tie that round half to
    even must settle, plus the hand-worked golden row (scale 1)."""
    import json
    import os
    import flow_matching_action_cached_amd as fm
    from oracle import int4 as q4
    w = synth.normal(0, "w_qkv", (37, 1024), 0.02)
    w[3, 128:256] = 0.0
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "int4_nibbles.json")))
    w[5, :128] = 0.0
    w[5, :8] = g["row_head"]                                   # scale 1, ties 2.5, 3.5, -2.5, 0.5
    halves = np.array([n + 0.5 for n in range(-7, 7)], np.float32)   # -6.5 .. 6.5: 14 ties
    for row, e in ((6, 0), (7, -7), (8, -9), (9, 3)):
        grp = np.zeros(128, np.float32)
        grp[:14] = halves
        grp[14], grp[15] = 7.0, -7.0                           # largest magnitude 7: s = 2^e exactly
        w[row, 256:384] = grp * np.float32(2.0 ** e)
    packed, scales = fm.quantize_int4_g128(torch.from_numpy(w).cuda())
    ref_p, ref_s = q4.quantize(w)
    got_p, got_s = packed.cpu().numpy(), scales.cpu().numpy().view(np.uint16)
    assert got_s[5, 0] == g["scale_bits"] and got_p[5, :4].tolist() == g["bytes_head"]
    codes = q4.unpack_codes(got_p)
    for row in (6, 7, 8, 9):                                   # half to even: -6.5 -> -6, 0.5 -> 0, ...
        assert codes[row, 256:270].tolist() == [int(2 * round(x / 2)) for x in halves]
    assert np.array_equal(got_p, ref_p)
    assert np.array_equal(got_s, ref_s)


def test_tiny_int4_matches_oracle():
    """int4 path at tiny shapes (bf16 activations, int4 expert linears)."""
    from oracle import int4 as q4
    d = dataclasses.replace(TINY, weight_dtype="int4")
    inp = synth.make_expert_inputs(d, 0)
    got = _run(d, inp)
    deq = {k: q4.dequantize_stack(*q4.quantize_stack(inp[k])) for k in ("w_qkv", "w_o", "w_gu", "w_d")}
    ref = ex.denoise(inp, d, linears=deq)
    err = rel_err(got, ref)
    _say(f"tiny int4 rel err {err:.3e}")
    assert err <= 2e-2


def test_pi05_int4_matches_oracle():
    _say("case: pi05 int4 g128 batch 1, seed 0")
    from oracle import int4 as q4
    inp = synth.make_expert_inputs(PI05_I4, 0)
    got = _run(PI05_I4, inp)
    deq = {k: q4.dequantize_stack(*q4.quantize_stack(inp[k])) for k in ("w_qkv", "w_o", "w_gu", "w_d")}
    ref = ex.denoise(inp, PI05_I4, linears=deq)
    err = rel_err(got, ref)
    _say(f"pi05 int4 rel err {err:.3e}")
    assert err <= 2e-2


def test_int4_lossless_weights_match_bf16_path():
    """When W is exactly q*s, quantisation is lossless, so the int4 path must match
    the bf16 path fed the dequantised weights (same activations, fp32 accumulation)."""
    from oracle import int4 as q4
    d4 = dataclasses.replace(TINY, weight_dtype="int4")
    db = dataclasses.replace(TINY, weight_dtype="bf16")
    inp = synth.make_expert_inputs(d4, 0)
    for k in ("w_qkv", "w_o", "w_gu", "w_d"):
        inp[k] = q4.dequantize_stack(*q4.quantize_stack(inp[k])).astype(np.float32)
    got4 = _run(d4, inp)
    gotb = _run(db, inp)
    # The two paths add their fp32 partial sums in different groupings (dequantised
    # quads with a row-sum correction against plain bf16 products), and every GEMM input
    # activation is rounded to bf16 (spacing 2^-8 = 3.9e-3 relative), so an input may land
    # one bf16 step apart and the difference grows through the layers and steps (1.0e-3 to
    # 1.4e-3 observed).  A mis-decoded nibble, scale or correction gives errors of order 1.
    assert rel_err(got4, gotb) <= 5e-3


# ---------------------------------------------------------------- prefix prefill
def _prefill_case(d, seeds):
    """GPU: prefill from the prefix tokens, then denoise; oracle: the prefix network's K/V
    (joint.prefix_kv, the same network the cached-vs-recomputed pin uses), then the cached
    loop.  Each seed is a new observation (the prefill replaces the previous prefix)."""
    from oracle import joint
    inp = synth.make_expert_inputs(d, 0)
    t = ex.schedule(d.n_steps)
    dev = device_inputs(d, inp)
    el = torch.float32 if d.weight_dtype == "f32" else torch.bfloat16
    e = make_expert(d, dev, t, prefill=True)
    outs = []
    for seed in seeds:
        pre = synth.make_prefix_inputs(d, seed)
        e.set_prefill_weights({k: torch.from_numpy(pre[k]).cuda().to(el).contiguous()
                               for k in ("w_qkv", "w_o", "w_gu", "w_d")})
        e.prefill(torch.from_numpy(pre["tokens"]).cuda().to(el).contiguous())
        got = e.denoise(dev["noise"]).cpu().numpy()
        e.sync()
        pp = {k: np.asarray(pre[k], np.float64) for k in ("w_qkv", "w_o", "w_gu", "w_d")}
        kv = [joint.prefix_kv(pre["tokens"][b], pp, d) for b in range(d.batch)]
        ref_inp = dict(inp, k_pre=np.stack([k for k, _ in kv]), v_pre=np.stack([v for _, v in kv]))
        outs.append((got, ex.denoise(ref_inp, d)))
    e.close()
    return outs


def test_tiny_prefill_then_denoise_matches_oracle():
    """64 prefix tokens through the weight-streaming kernels (fp32): parity 1e-4, and a new
    observation (other prefix network and tokens) changes the chunk accordingly."""
    (g1, r1), (g2, r2) = _prefill_case(TINY, [1, 2])
    _say(f"tiny prefill rel err {rel_err(g1, r1):.3e}, {rel_err(g2, r2):.3e}")
    assert rel_err(g1, r1) <= 1e-4 and rel_err(g2, r2) <= 1e-4
    assert rel_err(r2, r1) > 1e-3


def test_tiny_bf16_batch2_prefill_then_denoise_matches_oracle():
    """Two observations prefilled at once (2 x 64 rows: the tiled GEMMs and many-row
    attention, bf16), each sample's chunk against its own prefix network K/V."""
    _say("case: tiny bf16 prefill, batch 2")
    ((g, r),) = _prefill_case(dataclasses.replace(TINY, weight_dtype="bf16", batch=2), [3])
    err = rel_err(g, r)
    _say(f"tiny bf16 batch-2 prefill rel err {err:.3e}")
    assert err <= 2e-2
    assert rel_err(g[1], g[0]) > 0.1                 # the two samples differ


def test_pi05_prefill_then_denoise_matches_oracle():
    """816 prefix tokens through the tiled GEMMs and many-row attention (bf16)."""
    _say("case: pi05 prefill 816 tokens")
    ((g, r),) = _prefill_case(PI05, [1])
    err = rel_err(g, r)
    _say(f"pi05 prefill rel err {err:.3e}")
    assert err <= 2e-2
