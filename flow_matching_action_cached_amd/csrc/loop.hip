// The Euler loop on the host side: launch plans, the per-layer launch sequence of the
// action expert, the prefix prefill and the joint denoiser, gfx950.
//
// One Euler step (PhyAI reading "PhyAI: Real-Time Physical AI at the Edge,
// Scalable Rollouts in the Cloud", Sec. 5.1 and 5.5) is, per layer,
//   k_gemm<QKV>    adaptive-RMSNorm folded in, fused Q|K|V projection, chunk K/V
//                  written straight into the cache rows after the prefix;
//   k_attn         split-key flash decode over [cached prefix ; chunk] keys,
//                  online softmax, one partial per split;
//   k_attn_merge   log-sum-exp merge of the splits in split order;
//   k_gemm<RESID>  output projection + residual;
//   k_gemm<GEGLU>  adaptive-RMSNorm folded in, gate/up projection, gelu(g)*u;
//   k_gemm<RESID>  down projection + residual;
// and once per step k_out_rows (final norm, out-projection, x += dt v, and the
// next step's in-projection, 16 token rows per workgroup).
//
// Norm folding.  adaRMS(h) W^T = rinv * ((h * (1 + scale)) W^T) + W shift, with
// rinv = 1/sqrt(mean(h^2) + eps) per token row.  The producer of h (residual
// epilogues, in-projection) writes h itself (fp32), hs = h * (1 + scale) in the
// GEMM input type, and per-16-column partial sums of h^2; the consumer GEMM
// multiplies its accumulator by rinv and adds the per-step vector W shift, which
// is precomputed with the timestep tables.  No kernel needs a whole row of h
// before its matrix product, and the norm costs no extra launch.
//
// Files: gemv.hip (weight-streaming GEMMs, <= 64 rows), gemm_tiled.hip (LDS-tiled MFMA
// GEMMs, more rows), attention.hip, update.hip (per-step update and prefill input kernels).
#include "launch.h"

#include <algorithm>

namespace phyai {

// ================================================================== host side
size_t gemm_counters(const Dims& d) {
  size_t n = d.qkv / 16;
  if ((size_t)d.D / 16 > n) n = d.D / 16;
  if ((size_t)d.F / 16 > n) n = d.F / 16;
  if (d.M > 64) n = std::max(n, tiled_split_counters(d));
  return n;
}
size_t gemm_ws_floats(const Dims& d, const Plan& p) {
  const int MT = std::min((d.M + 15) / 16, 4);  // the split scratch serves the streaming path only
  size_t n = 0;
  auto upd = [&](size_t tiles, int S, int NT) {
    if (S > 1) n = std::max(n, tiles * S * NT * MT * 256);
  };
  upd(d.qkv / 16, p.s_qkv, 1);
  upd(d.D / 16, p.s_o, 1);
  upd(d.F / 16, p.s_gu, 2);
  upd(d.D / 16, p.s_d, 1);
  if (d.M > 64) n = std::max(n, tiled_split_ws_floats(d));
  return n;
}

// Splits across workgroups for a linear with K inputs: the fewest (a power of two dividing
// the K/128 quads; int4 waves own whole quads) that keep a split at most 32 k-blocks (8 per
// wave).  More splits would add workgroups, but each split costs a cross-workgroup hand-off
// (agent-scope partials, arrival, reload by the last arrival), which on this chip takes
// longer than streaming twice the weights per workgroup: QKV 7.8 -> 5.2 us at one split.
static int pick_split(int K) {
  const int nq = K / 128;
  int S = 1;
  while (S < 8 && nq % (2 * S) == 0 && nq / S > 8) S *= 2;
  return S;
}


Plan make_plan(const Dims& d, WDtype wt) {
  Plan p;
  p.s_qkv = pick_split(d.D);
  p.s_o = pick_split(d.Hq * d.dh);
  p.s_gu = pick_split(d.D);
  p.s_d = pick_split(d.F);
  // Key splits only as far as needed to give the chip ~256 workgroups (a batch of many
  // samples needs none), at most 32 (the merge width of k_attn_merge).  The splits are
  // merged by a launch of their own over many workgroups, so that a split can be as
  // short as one 32-key block: at batch 1 the time of a split is its load of K/V into one
  // CU, and 28 one-block splits beat 7 four-block splits merged in-kernel (8.54 -> 8.05
  // ms per chunk).
  const int T = d.P + d.H, nblk = (T + 31) / 32;
  const int QT = ((d.Hq / d.Hkv) * d.H + 15) / 16, QG = (QT + 3) / 4;
  const int base = d.B * d.Hkv * QG;
  int S = std::max(1, 256 / base);
  S = std::min(S, std::min(32, nblk));
  // Many query tiles (bf16): the shared-staging kernel, with key splits only up to ~256
  // workgroups and at least one whole key group per split.
  p.attn_wide = wt != W_F32 && d.B * d.Hkv * QT >= 64;
  if (p.attn_wide) {
    // One workgroup per CU at a time: pick the split count (<= 4, at least one key group
    // per split) that minimises the rounds of 256 workgroups per unit of work, e.g. the
    // joint denoiser's 544 query groups run in 9 rounds of quarter sweeps (2.25 full
    // sweeps) instead of 3 rounds of full sweeps.
    const int tpw = attn_wide_tiles(d.dh), nbg = d.dh <= 64 ? 4 : 2;
    const int wbase = d.B * d.Hkv * ((QT + tpw - 1) / tpw);
    const int smax = std::min(4, (nblk + nbg - 1) / nbg);
    S = 1;
    for (int c = 2; c <= smax; ++c) {
      const long rc = (long)((wbase * c + 255) / 256) * S, rs = (long)((wbase * S + 255) / 256) * c;
      if (rc < rs) S = c;  // rounds(c)/c < rounds(S)/S
    }
  }
  int bps = (nblk + S - 1) / S;
  p.attn_bps = bps;
  return p;
}

template <class T> static size_t wbytes_row(int K);
template <> size_t wbytes_row<float>(int K) { return (size_t)K * 4; }
template <> size_t wbytes_row<bf16>(int K) { return (size_t)K * 2; }
template <> size_t wbytes_row<i4>(int K) { return (size_t)K / 2; }

// Weight-streaming layers whose weights stay in the memory-side cache from one step to the
// next.  A step reads every layer's weights once, in layer order; when they exceed the
// MI355X's 256 MB memory-side cache (623 MB per step at the pi0.5 shape in bf16) a
// recency-ordered cache keeps none of them until the next step.  The first layers whose
// weights fit kResidentWeightBytes (room left for the prefix K/V and the activations) are
// read with the normal policy and stay; the later layers' weights are read non-temporally
// and pass through.  Measured at the pi0.5 shape (34.6 MB of weights per layer): 5 / 6 / 7 /
// 9 resident layers 6.76 / 6.74 / 6.74 / 6.89 ms per chunk; all normal 6.95, all
// non-temporal 6.86.  int4 weights (8.7 MB per layer) all fit.
constexpr size_t kResidentWeightBytes = (size_t)208 << 20;
template <class WT>
static int resident_weight_layers(const Dims& d) {
  const size_t per_layer = wbytes_row<WT>(d.D) * (d.qkv + 2 * (size_t)d.F) + wbytes_row<WT>(d.Hq * d.dh) * d.D +
                           wbytes_row<WT>(d.F) * d.D;
  return (int)std::min<size_t>(d.L, kResidentWeightBytes / per_layer);
}

// One launch of kernel `which` for (step k, layer l).  Kinds: 0 QKV, 1 attention,
// 7 merge of the attention's key splits (no launch when there is none), 2 O + residual,
// 3 gate/up GeGLU, 4 down + residual, 5 out-projection/Euler/in-projection (layer
// ignored), 6 in-projection of step 0 (layer ignored).  A layer runs kLayerOrder.
static constexpr int kLayerOrder[6] = {0, 1, 7, 2, 3, 4};
template <class AT, class WT, class IOT>
static hipError_t launch_one(const Dims& d, const Bufs& b, const Plan& p, int which, int k, int l,
                             hipStream_t st) {
  constexpr WDtype wt = __is_same(WT, float) ? W_F32 : __is_same(WT, i4) ? W_INT4 : W_BF16;
  const int qd = d.Hq * d.dh;
  const float* cv = b.cvec + (size_t)k * b.cv_stride;
  GemmLaunch g{};
  g.layer = l;
  g.wnt = l >= resident_weight_layers<WT>(d) ? 1 : 0;
  switch (which) {
    case 0:
      g.A = b.hs; g.lda = d.D; g.K = d.D;
      g.W = static_cast<const char*>(b.w_qkv) + wbytes_row<WT>(d.D) * d.qkv * l;
      g.Ws = b.s_qkv ? b.s_qkv + (size_t)l * d.qkv * (d.D / 128) : nullptr;
      g.S = p.s_qkv; g.cvec = cv + (size_t)l * d.qkv;
      if (d.M > 64) return launch_gemm_tiled(d, b, g, EPI_QKV, d.qkv, st);
      return launch_gemv(d, b, g, wt, EPI_QKV, d.qkv / 16, st);
    case 1:
      return launch_attention(d, b, p, l, 0, sizeof(AT) == 4, st);
    case 7:
      return launch_attention(d, b, p, l, 1, sizeof(AT) == 4, st);
    case 2:  // consumer of h is the MLP norm 2l+1
      g.A = b.o; g.lda = qd; g.K = qd;
      g.W = static_cast<const char*>(b.w_o) + wbytes_row<WT>(qd) * d.D * l;
      g.Ws = b.s_o ? b.s_o + (size_t)l * d.D * (qd / 128) : nullptr;
      g.S = p.s_o; g.scale_next = b.mod + (((size_t)k * d.nmod + 2 * l + 1) * 2) * d.D;
      g.gate = b.gate ? b.gate + ((size_t)k * d.nmod + 2 * l) * d.D : nullptr;  // attention block of layer l
      if (d.M > 64) return launch_gemm_tiled(d, b, g, EPI_RESID, d.D, st);
      return launch_gemv(d, b, g, wt, EPI_RESID, d.D / 16, st);
    case 3:
      g.A = b.hs; g.lda = d.D; g.K = d.D;
      g.W = static_cast<const char*>(b.w_gu) + wbytes_row<WT>(d.D) * 2 * d.F * l;
      g.Ws = b.s_gu ? b.s_gu + (size_t)l * 2 * d.F * (d.D / 128) : nullptr;
      g.n_second = d.F; g.S = p.s_gu; g.cvec = cv + b.cv_gu_off + (size_t)l * 2 * d.F;
      if (d.M > 64) return launch_gemm_tiled(d, b, g, EPI_GEGLU, 2 * d.F, st);
      return launch_gemv(d, b, g, wt, EPI_GEGLU, d.F / 16, st);
    case 4: {  // consumer of h is norm 2(l+1), or the final norm 2L
      g.A = b.act; g.lda = d.F; g.K = d.F;
      g.W = static_cast<const char*>(b.w_d) + wbytes_row<WT>(d.F) * d.D * l;
      g.Ws = b.s_d ? b.s_d + (size_t)l * d.D * (d.F / 128) : nullptr;
      g.S = p.s_d;
      const int jn = (l + 1 < d.L) ? 2 * (l + 1) : 2 * d.L;
      g.scale_next = b.mod + (((size_t)k * d.nmod + jn) * 2) * d.D;
      g.gate = b.gate ? b.gate + ((size_t)k * d.nmod + 2 * l + 1) * d.D : nullptr;  // MLP block of layer l
      if (d.M > 64) return launch_gemm_tiled(d, b, g, EPI_RESID, d.D, st);
      return launch_gemv(d, b, g, wt, EPI_RESID, d.D / 16, st);
    }
    case 5:
      return launch_out_rows(d, b, wt, k, k + 1 < d.N ? k + 1 : -1, st);
    case 6:
      return launch_out_rows(d, b, wt, -1, 0, st);
  }
  return hipErrorInvalidValue;
}

template <class AT, class WT, class IOT>
static hipError_t denoise_impl(const Dims& d, const Bufs& b, const Plan& p, hipStream_t st, LaunchMarks* mk) {
  // with marks: an event before the first launch and after every launch, and its kind
  auto mark = [&](int which) -> hipError_t {
    if (!mk) return hipSuccess;
    if (mk->n >= mk->cap) return hipErrorInvalidValue;
    mk->kind[mk->n] = which;
    return hipEventRecord(mk->ev[mk->n++], st);
  };
  hipError_t e = mark(-1);
  auto one = [&](int which, int k, int l) {
    if (e == hipSuccess) e = launch_one<AT, WT, IOT>(d, b, p, which, k, l, st);
    if (e == hipSuccess) e = mark(which);
  };
  one(6, 0, 0);
  for (int k = 0; k < d.N && e == hipSuccess; ++k) {
    for (int l = 0; l < d.L && e == hipSuccess; ++l)
      for (int i = 0; i < 6 && e == hipSuccess; ++i) one(kLayerOrder[i], k, l);
    one(5, k, 0);
  }
  return e;
}

Dims prefill_dims(const Dims& base, int batch, int prefix_len) {
  Dims d = base;
  d.B = batch;
  d.H = prefix_len;           // the prefix rows take the place of the chunk ...
  d.P = 0;                    // ... with no cached keys before them
  d.M = batch * prefix_len;
  d.Mst = d.M;
  d.N = 1;
  d.rope_theta = 0.f;         // the prefix network: plain layers (its K/V are stored as computed)
  d.gated = 0;
  d.tmlp = 0;
  return d;
}

template <class AT>
static hipError_t prefill_impl(const Dims& d, const Bufs& b, const Plan& p, const void* tokens, hipStream_t st) {
  hipError_t e = launch_prefill_in(d, b, tokens, sizeof(AT) == 4, st);
  // every layer's QKV epilogue writes the prefix rows' K/V into cache rows [0, prefix_len)
  for (int l = 0; l < d.L && e == hipSuccess; ++l)
    for (int i = 0; i < 6 && e == hipSuccess; ++i) e = launch_one<AT, AT, AT>(d, b, p, kLayerOrder[i], 0, l, st);
  return e;
}

hipError_t enqueue_prefill(const Dims& d, const Bufs& b, const Plan& p, WDtype wt, const void* tokens,
                           hipStream_t st) {
  switch (wt) {
    case W_F32: return prefill_impl<float>(d, b, p, tokens, st);
    case W_BF16: return prefill_impl<bf16>(d, b, p, tokens, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t enqueue_one(const Dims& d, const Bufs& b, const Plan& p, WDtype wt, int which, int k, int l,
                       hipStream_t st) {
  switch (wt) {
    case W_F32: return launch_one<float, float, float>(d, b, p, which, k, l, st);
    case W_BF16: return launch_one<bf16, bf16, bf16>(d, b, p, which, k, l, st);
    case W_INT4: return launch_one<bf16, i4, bf16>(d, b, p, which, k, l, st);
  }
  return hipErrorInvalidValue;
}

// Joint denoiser: one launch of kernel `which` (0 QKV, 1 attention, 2 O, 3 gate/up, 4 down,
// 5 guidance/Euler/in-projection, 6 first in-projection) for step k, layer l.  No K/V is
// kept across layers (one cache layer, no prefix); every linear runs on the tiled GEMMs
// with one modulation table per branch.
static hipError_t launch_one_wam(const Dims& d, const Bufs& b, const Plan& p, int which, int k, int l,
                                 hipStream_t st) {
  const int qd = d.Hq * d.dh;
  const float* cv = b.cvec + (size_t)k * d.ntab * b.cv_stride;
  const float* md = b.mod + (size_t)k * d.ntab * d.nmod * 2 * d.D;
  GemmLaunch g{};
  g.layer = 0;  // cache layer
  g.S = 1;
  switch (which) {
    case 0:
      g.A = b.hs; g.K = d.D; g.W = static_cast<const bf16*>(b.w_qkv) + (size_t)l * d.qkv * d.D;
      g.cvec = cv + (size_t)l * d.qkv;
      return launch_gemm_tiled(d, b, g, EPI_QKV, d.qkv, st);
    case 1:
      return launch_attention(d, b, p, 0, 0, false, st);
    case 7:
      return launch_attention(d, b, p, 0, 1, false, st);
    case 2:
      g.A = b.o; g.K = qd; g.W = static_cast<const bf16*>(b.w_o) + (size_t)l * d.D * qd;
      g.scale_next = md + (size_t)(2 * l + 1) * 2 * d.D;
      return launch_gemm_tiled(d, b, g, EPI_RESID, d.D, st);
    case 3:
      g.A = b.hs; g.K = d.D; g.W = static_cast<const bf16*>(b.w_gu) + (size_t)l * 2 * d.F * d.D;
      g.n_second = d.F; g.cvec = cv + b.cv_gu_off + (size_t)l * 2 * d.F;
      return launch_gemm_tiled(d, b, g, EPI_GEGLU, 2 * d.F, st);
    case 4: {
      g.A = b.act; g.K = d.F; g.W = static_cast<const bf16*>(b.w_d) + (size_t)l * d.D * d.F;
      const int jn = (l + 1 < d.L) ? 2 * (l + 1) : 2 * d.L;
      g.scale_next = md + (size_t)jn * 2 * d.D;
      return launch_gemm_tiled(d, b, g, EPI_RESID, d.D, st);
    }
    case 5:
      return launch_wam_rows(d, b, k, k + 1 < d.N ? k + 1 : -1, st);
    case 6:
      return launch_wam_rows(d, b, -1, 0, st);
  }
  return hipErrorInvalidValue;
}

hipError_t enqueue_wam_one(const Dims& d, const Bufs& b, const Plan& p, int which, int k, int l, hipStream_t st) {
  return launch_one_wam(d, b, p, which, k, l, st);
}

hipError_t enqueue_wam_denoise(const Dims& d, const Bufs& b, const Plan& p, hipStream_t st) {
  hipError_t e = launch_one_wam(d, b, p, 6, 0, 0, st);
  for (int k = 0; k < d.N && e == hipSuccess; ++k) {
    for (int l = 0; l < d.L && e == hipSuccess; ++l)
      for (int i = 0; i < 6 && e == hipSuccess; ++i) e = launch_one_wam(d, b, p, kLayerOrder[i], k, l, st);
    if (e == hipSuccess) e = launch_one_wam(d, b, p, 5, k, 0, st);
  }
  return e;
}

hipError_t enqueue_denoise(const Dims& d, const Bufs& b, const Plan& p, WDtype wt, hipStream_t st,
                           LaunchMarks* marks) {
  switch (wt) {
    case W_F32: return denoise_impl<float, float, float>(d, b, p, st, marks);
    case W_BF16: return denoise_impl<bf16, bf16, bf16>(d, b, p, st, marks);
    case W_INT4: return denoise_impl<bf16, i4, bf16>(d, b, p, st, marks);
  }
  return hipErrorInvalidValue;
}

}  // namespace phyai
