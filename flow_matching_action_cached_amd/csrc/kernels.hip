// HIP kernels (gfx950) of the cached-prefix flow-matching denoise loop.
//
// One Euler step (PhyAI reading "PhyAI: Real-Time Physical AI at the Edge,
// Scalable Rollouts in the Cloud", Sec. 5.1 and 5.5) is, per layer,
//   k_gemm<QKV>    adaptive-RMSNorm folded in, fused Q|K|V projection, chunk K/V
//                  written straight into the cache rows after the prefix;
//   k_attn         split-key flash decode over [cached prefix ; chunk] keys,
//                  online softmax, deterministic log-sum-exp merge;
//   k_gemm<RESID>  output projection + residual;
//   k_gemm<GEGLU>  adaptive-RMSNorm folded in, gate/up projection, gelu(g)*u;
//   k_gemm<RESID>  down projection + residual;
// and once per step k_out_euler (final norm, out-projection, x += dt v, and the
// next step's in-projection).
//
// Norm folding.  adaRMS(h) W^T = rinv * ((h * (1 + scale)) W^T) + W shift, with
// rinv = 1/sqrt(mean(h^2) + eps) per token row.  The producer of h (residual
// epilogues, in-projection) writes h itself (fp32), hs = h * (1 + scale) in the
// GEMM input type, and per-16-column partial sums of h^2; the consumer GEMM
// multiplies its accumulator by rinv and adds the per-step vector W shift, which
// is precomputed with the timestep tables.  No kernel needs a whole row of h
// before its matrix product, and the norm costs no extra launch.
//
// Batch-1 linears stream every weight byte exactly once: a workgroup owns 16
// (or 16 gate + 16 up) output columns and a contiguous share of K, its four
// waves interleave over 32-wide k-blocks, and the token rows (<= 64) sit in
// MFMA 16x16 tiles.  Partial sums across waves meet in LDS; partial sums across
// workgroups meet in a scratch buffer and the last workgroup to arrive adds
// them in a fixed order, so results do not depend on arrival order.
#include "common.h"
#include "kernels.h"

#include <math.h>

#include <algorithm>

namespace phyai {

enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_GEGLU = 2 };

struct GemmLaunch {
  const void* A;             // activations [M][K] (row stride lda)
  int lda, K;
  const void* W;             // weights of this layer, [N][K] (int4: repacked codes [N][K/2])
  const uint16_t* Ws;        // int4 scales of this layer [N][K/128]
  int n_second;              // row offset of the second weight tile (gate/up: F)
  int S;                     // k-splits across workgroups
  int layer;
  const float* cvec;         // norm-folded bias of this step/layer (QKV, GEGLU)
  const float* scale_next;   // raw scale of the norm that consumes h (RESID)
};

// ------------------------------------------------------------------ weight fragments
template <class WT> struct WFrag;
template <> struct WFrag<float> { typedef f32x8 type; };
template <> struct WFrag<bf16> { typedef bf16x8 type; };
template <> struct WFrag<i4> { typedef bf16x8 type; };

// Repacked int4 word (8 consecutive inputs k0..k7): the offset-binary code u = q + 8 of
// k_{2j} sits in bits [4j, 4j+4) and that of k_{2j+1} in bits [16+4j, 16+4j+4).  OR-ing a
// pair into 0x4300 (bf16 128.0, where one mantissa step is 1) yields the exact bf16 pair
// (q_{2j} + 136, q_{2j+1} + 136).  The kernels remove the +136 afterwards with the
// per-group row sums of the activations.
__device__ __forceinline__ bf16x8 int4_word_to_bf16x8_biased(uint32_t w) {
  u32x4 r;
  r[0] = (w & 0x000F000Fu) | 0x43004300u;
  r[1] = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
  r[2] = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
  r[3] = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
  return __builtin_bit_cast(bf16x8, r);
}

// ------------------------------------------------------------------ stream GEMM
template <class AT, class WT, int MT, int NT, int EPI>
__global__ __launch_bounds__(256) void k_gemm(Dims d, Bufs bf, GemmLaunch g) {
  constexpr bool NORM = (EPI == EPI_QKV || EPI == EPI_GEGLU);
  constexpr bool INT4 = __is_same(WT, i4);
  __shared__ f32x4 red[4][NT][MT][64];
  __shared__ float rinv_s[64];
  __shared__ unsigned flag;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r16 = lane & 15, grp = lane >> 4;
  const int s = blockIdx.x % g.S, tile = blockIdx.x / g.S;
  int nrow[NT];
  nrow[0] = tile * 16;
  if (NT == 2) nrow[NT - 1] = g.n_second + tile * 16;

  if (NORM && tid < d.M) {
    float ss = 0.f;
    const int ntd = d.D / 16;
    for (int j = 0; j < ntd; ++j) ss += bf.ssq[(size_t)j * d.Mst + tid];
    rinv_s[tid] = 1.0f / sqrtf(ss / (float)d.D + d.eps);
  }

  f32x4 acc[NT][MT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const AT* A = static_cast<const AT*>(g.A);
  const int kblocks = g.K / 32;
  const int kbs = kblocks / g.S;
  const int kb0 = s * kbs, kb1 = kb0 + kbs;

  if constexpr (!INT4) {
    const WT* W = static_cast<const WT*>(g.W);
#pragma unroll 2
    for (int kb = kb0 + w; kb < kb1; kb += 4) {
      const int k = kb * 32 + grp * 8;
      typename WFrag<WT>::type bw[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) bw[nt] = load_frag(W + (size_t)(nrow[nt] + r16) * g.K + k);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + r16;
        typename FragOf<AT>::type a = m < d.M ? load_frag(A + (size_t)m * g.lda + k) : zero_frag<AT>();
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][mt] = mma(a, bw[nt], acc[nt][mt]);
      }
    }
  } else {
    // int4: waves interleave over 128-wide groups (4 k-blocks share one scale).
    const uint32_t* W = static_cast<const uint32_t*>(g.W);  // [N][K/8] words
    const int kw = g.K / 8;
    const int ng = g.K / 128;
    const bf16x8 ones = {(bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f,
                         (bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f};
    for (int gi = kb0 / 4 + w; gi < kb1 / 4; gi += 4) {
      f32x4 part[NT][MT], rs[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        rs[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) part[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      float sc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sc[nt] = bf16_bits_to_f32(g.Ws[(size_t)(nrow[nt] + r16) * ng + gi]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kb = gi * 4 + j;
        const int k = kb * 32 + grp * 8;
        bf16x8 bw[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          bw[nt] = int4_word_to_bf16x8_biased(W[(size_t)(nrow[nt] + r16) * kw + k / 8]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = mt * 16 + r16;
          bf16x8 a = m < d.M ? load_frag(A + (size_t)m * g.lda + k) : zero_frag<bf16>();
          rs[mt] = mma(a, ones, rs[mt]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) part[nt][mt] = mma(a, bw[nt], part[nt][mt]);
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[nt][mt][i] += sc[nt] * (part[nt][mt][i] - 136.0f * rs[mt][i]);
    }
  }

  // ---- cross-wave reduction (fixed order), wave w then owns M-tile w
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[w][nt][mt][lane] = acc[nt][mt];
  __syncthreads();
  const int mt = w;
  f32x4 tot[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    tot[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (mt < MT) {
      f32x4 v = red[0][nt][mt][lane];
      v += red[1][nt][mt][lane];
      v += red[2][nt][mt][lane];
      v += red[3][nt][mt][lane];
      tot[nt] = v;
    }
  }

  // ---- cross-workgroup split-K: last arrival sums the partials in split order
  if (g.S > 1) {
    const size_t part_floats = (size_t)NT * MT * 256;
    f32x4* mine = reinterpret_cast<f32x4*>(bf.gemm_ws + ((size_t)tile * g.S + s) * part_floats);
    if (mt < MT)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) mine[(nt * MT + mt) * 64 + lane] = tot[nt];
    if (!arrive_last<true>(bf.gemm_cnt + tile, (unsigned)g.S, &flag)) return;
    if (mt < MT) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int s2 = 0; s2 < g.S; ++s2) {
          const f32x4* p = reinterpret_cast<const f32x4*>(bf.gemm_ws + ((size_t)tile * g.S + s2) * part_floats);
          sum += (s2 == s) ? tot[nt] : p[(nt * MT + mt) * 64 + lane];
        }
        tot[nt] = sum;
      }
    }
  }
  if (mt >= MT) return;

  // ---- epilogues.  tot[nt][i] is row mt*16 + 4*grp + i, column nrow[nt] + r16.
  if constexpr (EPI == EPI_QKV) {
    const int col = nrow[0] + r16;
    const float c = g.cvec[col];
    const int qd = d.Hq * d.dh, kd = d.Hkv * d.dh;
    AT* q = static_cast<AT*>(bf.q);
    AT* kc = static_cast<AT*>(bf.kc);
    AT* vt = static_cast<AT*>(bf.vt);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + grp * 4 + i;
      if (m >= d.M) continue;
      const float y = rinv_s[m] * tot[0][i] + c;
      const int b = m / d.H, t = m % d.H;
      if (col < qd) {
        q[(size_t)m * qd + col] = to_elem<AT>(y);
      } else if (col < qd + kd) {
        const int r = (col - qd) / d.dh, dd = (col - qd) % d.dh;
        kc[((((size_t)b * d.L + g.layer) * d.Hkv + r) * d.KS + d.P + t) * d.dh + dd] = to_elem<AT>(y);
      } else {
        const int r = (col - qd - kd) / d.dh, dd = (col - qd - kd) % d.dh;
        vt[((((size_t)b * d.L + g.layer) * d.Hkv + r) * d.dh + dd) * d.KS + d.P + t] = to_elem<AT>(y);
      }
    }
  } else if constexpr (EPI == EPI_RESID) {
    const int col = nrow[0] + r16;
    const float sc1 = 1.0f + g.scale_next[col];
    AT* hs = static_cast<AT*>(bf.hs);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + grp * 4 + i;
      float hn = 0.f;
      if (m < d.M) {
        hn = bf.h[(size_t)m * d.D + col] + tot[0][i];
        bf.h[(size_t)m * d.D + col] = hn;
        hs[(size_t)m * d.D + col] = to_elem<AT>(hn * sc1);
      }
      const float sq = sum16(hn * hn);
      if (r16 == 0 && m < d.M) bf.ssq[(size_t)tile * d.Mst + m] = sq;
    }
  } else {  // EPI_GEGLU
    const int f = nrow[0] + r16;
    const float cg = g.cvec[f], cu = g.cvec[d.F + f];
    AT* act = static_cast<AT*>(bf.act);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + grp * 4 + i;
      if (m >= d.M) continue;
      const float yg = rinv_s[m] * tot[0][i] + cg;
      const float yu = rinv_s[m] * tot[NT - 1][i] + cu;
      act[(size_t)m * d.F + f] = to_elem<AT>(gelu_tanh(yg) * yu);
    }
  }
}

// ------------------------------------------------------------------ attention
// Split-key flash decode.  The query rows of one KV head r are the g*H pairs
// (query head r*g + j, chunk token t), row j*H + t, in 16-row tiles; the keys are
// the P cached prefix rows followed by the H chunk rows (no mask among them).
// One wave owns (sample, KV head, 16-row query tile, key split) and walks its
// 32-key blocks: S^T = K q^T and O^T += V^T P^T on MFMA, so that the softmax
// probabilities come out of the first product already laid out as the second
// product's B operand (no LDS round trip).  V is kept transposed in the cache for
// the same reason.  Splits are merged by log-sum-exp weights in split order by
// the last wave to finish.
template <class AT, int DH>
__global__ __launch_bounds__(256) void k_attn(Dims d, Bufs bf, int layer, int S, int bps) {
  typedef typename FragOf<AT>::type Frag;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, r16 = lane & 15, grp = lane >> 4;
  const int gq = d.Hq / d.Hkv;
  const int QT = (gq * d.H + 15) / 16, QG = (QT + 3) / 4;
  int idx = blockIdx.x;
  const int s = idx % S;
  idx /= S;
  const int qg = idx % QG;
  idx /= QG;
  const int r = idx % d.Hkv;
  const int b = idx / d.Hkv;
  const int qt = qg * 4 + w;
  if (qt >= QT) return;
  const int T = d.P + d.H;
  const int nblk = (T + 31) / 32;
  const int blk0 = s * bps, blk1 = min(nblk, blk0 + bps);

  const int qrow = qt * 16 + r16;
  const bool qvalid = qrow < gq * d.H;
  const int head = r * gq + (qvalid ? qrow / d.H : 0);
  const int tok = qvalid ? qrow % d.H : 0;
  const int m = b * d.H + tok;
  const int qd = d.Hq * DH;

  Frag qf[DH / 32];
  {
    const AT* qp = static_cast<const AT*>(bf.q) + (size_t)m * qd + head * DH + grp * 8;
#pragma unroll
    for (int j = 0; j < DH / 32; ++j) qf[j] = qvalid ? load_frag(qp + 32 * j) : zero_frag<AT>();
  }
  const size_t kvbase = ((size_t)b * d.L + layer) * d.Hkv + r;
  const AT* Kc = static_cast<const AT*>(bf.kc) + kvbase * d.KS * DH;
  const AT* Vt = static_cast<const AT*>(bf.vt) + kvbase * DH * d.KS;
  const float sc = 1.4426950408889634f / sqrtf((float)DH);  // log2(e) / sqrt(dh)

  float m_run = -INFINITY, l_part = 0.f;
  f32x4 o[DH / 16];
#pragma unroll
  for (int t = 0; t < DH / 16; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int blk = blk0; blk < blk1; ++blk) {
    const int kb = blk * 32;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    const AT* k0 = Kc + (size_t)(kb + r16) * DH + grp * 8;
#pragma unroll
    for (int j = 0; j < DH / 32; ++j) {
      s0 = mma(load_frag(k0 + 32 * j), qf[j], s0);
      s1 = mma(load_frag(k0 + 16 * DH + 32 * j), qf[j], s1);
    }
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kb + grp * 4 + i;
      v[i] = key < T ? s0[i] * sc : -INFINITY;
      v[4 + i] = key + 16 < T ? s1[i] * sc : -INFINITY;
    }
    float mx = v[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, v[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    float p[8], ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = exp2f(v[e] - m_new);
      ps += p[e];
    }
    l_part = l_part * alpha + ps;
    m_run = m_new;
    Frag pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[e] = to_elem<AT>(p[e]);
#pragma unroll
    for (int t = 0; t < DH / 16; ++t) {
      o[t] *= alpha;
      const AT* vp = Vt + (size_t)(t * 16 + r16) * d.KS + kb + grp * 4;
      o[t] = mma(load_frag_split4(vp, vp + 16), pf, o[t]);
    }
  }
  float l_row = l_part;
  l_row += __shfl_xor(l_row, 16, 64);
  l_row += __shfl_xor(l_row, 32, 64);

  if (S > 1) {
    const size_t item = ((size_t)(b * d.Hkv + r) * QT + qt);
    const size_t stride = (size_t)(DH / 16) * 256 + 32;
    float* mine = bf.attn_ws + (item * S + s) * stride;
    f32x4* mo = reinterpret_cast<f32x4*>(mine);
#pragma unroll
    for (int t = 0; t < DH / 16; ++t) mo[t * 64 + lane] = o[t];
    if (grp == 0) {
      mine[(DH / 16) * 256 + r16] = m_run;
      mine[(DH / 16) * 256 + 16 + r16] = l_row;
    }
    if (!arrive_last<false>(bf.attn_cnt + item, (unsigned)S, nullptr)) return;
    const float* base = bf.attn_ws + item * S * stride;
    float M = -INFINITY;
    for (int s2 = 0; s2 < S; ++s2) M = fmaxf(M, base[s2 * stride + (DH / 16) * 256 + r16]);
    float den = 0.f;
    f32x4 num[DH / 16];
#pragma unroll
    for (int t = 0; t < DH / 16; ++t) num[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s2 = 0; s2 < S; ++s2) {
      const float* ps2 = base + s2 * stride;
      const float wgt = exp2f(ps2[(DH / 16) * 256 + r16] - M);
      den += wgt * ps2[(DH / 16) * 256 + 16 + r16];
      const f32x4* po = reinterpret_cast<const f32x4*>(ps2);
#pragma unroll
      for (int t = 0; t < DH / 16; ++t) num[t] += wgt * (s2 == s ? o[t] : po[t * 64 + lane]);
    }
#pragma unroll
    for (int t = 0; t < DH / 16; ++t) o[t] = num[t];
    l_row = den;
  }
  if (!qvalid) return;
  const float inv = 1.0f / l_row;
  AT* op = static_cast<AT*>(bf.o) + (size_t)m * qd + head * DH + grp * 4;
#pragma unroll
  for (int t = 0; t < DH / 16; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) op[t * 16 + i] = to_elem<AT>(o[t][i] * inv);
}

// ------------------------------------------------------------------ out-projection + Euler + in-projection
// One workgroup per token row.  k_prev >= 0: final adaptive norm of step k_prev,
// v = rinv (hs W_out^T) + W_out shift + b_out, x += dt v.  k_next >= 0: in-projection
// h = x W_in^T + b_in for step k_next, writing h, hs = h * (1 + scale) of that step's
// first norm, and the row's sum-of-squares partials.
template <class AT, class IOT>
__global__ __launch_bounds__(256) void k_out_euler(Dims d, Bufs bf, int k_prev, int k_next) {
  __shared__ float xs[256];
  __shared__ float wred[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int m = blockIdx.x;
  if (k_prev >= 0) {
    float ss = 0.f;
    for (int j = tid; j < d.D / 16; j += 256) ss += bf.ssq[(size_t)j * d.Mst + m];
    ss = wave_sum(ss);
    if (lane == 0) wred[w] = ss;
    __syncthreads();
    const float rinv = 1.0f / sqrtf((((wred[0] + wred[1]) + wred[2]) + wred[3]) / (float)d.D + d.eps);
    const AT* hs = static_cast<const AT*>(bf.hs) + (size_t)m * d.D;
    const IOT* wo = static_cast<const IOT*>(bf.w_out);
    const IOT* bo = static_cast<const IOT*>(bf.b_out);
    const float* cv = bf.cvec + (size_t)k_prev * bf.cv_stride + bf.cv_out_off;
    const float dt = bf.dt[k_prev];
    for (int a = w; a < d.A; a += 4) {
      float acc = 0.f;
      for (int k = lane; k < d.D; k += 64) acc += to_f32(hs[k]) * to_f32(wo[(size_t)a * d.D + k]);
      acc = wave_sum(acc);
      if (lane == 0) {
        const float v = rinv * acc + cv[a] + to_f32(bo[a]);
        const float xn = bf.x[(size_t)m * d.A + a] + dt * v;
        bf.x[(size_t)m * d.A + a] = xn;
        xs[a] = xn;
      }
    }
    __syncthreads();
  } else {
    for (int a = tid; a < d.A; a += 256) xs[a] = bf.x[(size_t)m * d.A + a];
    __syncthreads();
  }
  if (k_next < 0) return;
  const IOT* wi = static_cast<const IOT*>(bf.w_in);
  const IOT* bi = static_cast<const IOT*>(bf.b_in);
  const float* scl = bf.mod + (size_t)k_next * d.nmod * 2 * d.D;  // norm 0, scale row
  AT* hs = static_cast<AT*>(bf.hs);
  for (int n0 = 0; n0 < d.D; n0 += 256) {
    const int n = n0 + tid;
    float hn = 0.f;
    if (n < d.D) {
      hn = to_f32(bi[n]);
      for (int a = 0; a < d.A; ++a) hn += xs[a] * to_f32(wi[(size_t)n * d.A + a]);
      bf.h[(size_t)m * d.D + n] = hn;
      hs[(size_t)m * d.D + n] = to_elem<AT>(hn * (1.0f + scl[n]));
    }
    const float sq = sum16(hn * hn);
    if ((lane & 15) == 0 && n < d.D) bf.ssq[(size_t)(n / 16) * d.Mst + m] = sq;
  }
}

// ------------------------------------------------------------------ timestep / modulation tables
// Embedding e(t_k) in fp64: e_i = sin(2 pi t / p_i), e_{D/2+i} = cos(2 pi t / p_i),
// p_i = 4e-3 * 1000^(i / (D/2 - 1)).
__global__ void k_embed(const float* t, int N, int D, double* e) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= N * D) return;
  const int k = idx / D, c = idx % D, half = D / 2;
  const int i = c % half;
  const double period = 4e-3 * pow(1000.0, (double)i / (double)(half - 1));
  const double ang = 2.0 * M_PI * (double)t[k] / period;
  e[idx] = c < half ? sin(ang) : cos(ang);
}

// One wave per row o of W_mod[j] (j = norm, o in [0, 2D)): m_k = W_mod[j][o] . e(t_k) + b_mod[j][o]
// for every step k, accumulated in fp64.
template <class IOT>
__global__ __launch_bounds__(256) void k_modulation(const IOT* w_mod, const IOT* b_mod, const double* e,
                                                    int N, int nmod, int D, float* mod) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= nmod * 2 * D) return;
  const int j = row / (2 * D), o = row % (2 * D);
  const IOT* wr = w_mod + (size_t)row * D;
  const double bias = (double)to_f32(b_mod[row]);
  for (int k0 = 0; k0 < N; k0 += 8) {
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int c = lane; c < D; c += 64) {
      const double wv = (double)to_f32(wr[c]);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        if (k0 + kk < N) acc[kk] += wv * e[(size_t)(k0 + kk) * D + c];
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const double v = wave_sum(acc[kk]);
      if (lane == 0 && k0 + kk < N)
        mod[(((size_t)(k0 + kk) * nmod + j) * 2 + (o >= D ? 1 : 0)) * D + (o % D)] = (float)(v + bias);
    }
  }
}

// Scalar weight read for the one-off table kernels.
template <class WT> struct WRow {
  const WT* w;
  const uint16_t* s;
  int K;
  __device__ float at(size_t n, int k) const { return to_f32(w[n * K + k]); }
};
template <> struct WRow<i4> {
  const i4* w;
  const uint16_t* s;
  int K;
  __device__ float at(size_t n, int k) const {
    // repacked word of inputs [8c, 8c+8): see int4_word_to_bf16x8_biased
    const uint32_t word = reinterpret_cast<const uint32_t*>(w)[n * (K / 8) + k / 8];
    const int e = k & 7, j = e >> 1;
    const int shift = (e & 1) ? 16 + 4 * j : 4 * j;
    const int q = (int)((word >> shift) & 0xFu) - 8;
    return (float)q * bf16_bits_to_f32(s[n * (K / 128) + k / 128]);
  }
};

// Norm-folded biases: for every step k, c = W shift_j(t_k) for the QKV rows (j = 2l),
// the gate/up rows (j = 2l+1) and the out-projection rows (j = 2L).  One wave per row.
template <class WT, class IOT>
__global__ __launch_bounds__(256) void k_shift_proj(Dims d, Bufs bf, const float* mod, float* cvec) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nq = d.L * d.qkv, ng = d.L * 2 * d.F;
  if (row >= nq + ng + d.A) return;
  int j, off;
  WRow<WT> wq{static_cast<const WT*>(bf.w_qkv), bf.s_qkv, d.D};
  WRow<WT> wg{static_cast<const WT*>(bf.w_gu), bf.s_gu, d.D};
  WRow<IOT> wo{static_cast<const IOT*>(bf.w_out), nullptr, d.D};
  int which;
  size_t n;
  if (row < nq) {
    which = 0; n = row; j = 2 * (row / d.qkv); off = row;
  } else if (row < nq + ng) {
    which = 1; n = row - nq; j = 2 * ((row - nq) / (2 * d.F)) + 1; off = bf.cv_gu_off + (row - nq);
  } else {
    which = 2; n = row - nq - ng; j = 2 * d.L; off = bf.cv_out_off + (row - nq - ng);
  }
  for (int k0 = 0; k0 < d.N; k0 += 8) {
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int c = lane; c < d.D; c += 64) {
      const double wv = which == 0 ? wq.at(n, c) : which == 1 ? wg.at(n, c) : wo.at(n, c);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        if (k0 + kk < d.N) acc[kk] += wv * (double)mod[(((size_t)(k0 + kk) * d.nmod + j) * 2 + 1) * d.D + c];
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const double v = wave_sum(acc[kk]);
      if (lane == 0 && k0 + kk < d.N) cvec[(size_t)(k0 + kk) * bf.cv_stride + off] = (float)v;
    }
  }
}

// ------------------------------------------------------------------ prefix install
// K [B][L][P][Hkv][dh] -> cache [b][l][r][p][dh];  V -> V^T cache [b][l][r][dh][p].
template <class T>
__global__ void k_install_prefix(Dims d, const T* k, const T* v, int B, int P, T* kc, T* vt) {
  const size_t total = (size_t)B * d.L * d.Hkv * d.dh * P;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    // V^T write order: p fastest
    size_t rem = idx;
    const int p = rem % P; rem /= P;
    const int dd = rem % d.dh; rem /= d.dh;
    const int r = rem % d.Hkv; rem /= d.Hkv;
    const int l = rem % d.L;
    const int b = rem / d.L;
    const size_t src = ((((size_t)b * d.L + l) * P + p) * d.Hkv + r) * d.dh + dd;
    const size_t cb = ((size_t)b * d.L + l) * d.Hkv + r;
    vt[(cb * d.dh + dd) * d.KS + p] = v[src];
    // K with dh fastest: reuse the same index space transposed
    const int dd2 = idx % d.dh;
    size_t rem2 = idx / d.dh;
    const int p2 = rem2 % P;
    rem2 /= P;
    const size_t cb2 = rem2;  // (b*L + l)*Hkv + r
    const int r2 = cb2 % d.Hkv;
    const size_t bl2 = cb2 / d.Hkv;
    kc[(cb2 * d.KS + p2) * d.dh + dd2] = k[((bl2 * P + p2) * d.Hkv + r2) * d.dh + dd2];
  }
}

// ------------------------------------------------------------------ int4 quantiser and repack
// One wave per (row, 128-column group); lane i quantises columns 2i, 2i+1 and writes one byte.
__global__ __launch_bounds__(256) void k_quantize_int4(const float* w, int64_t rows, int64_t cols,
                                                       uint8_t* packed, uint16_t* scales) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t ng = cols / 128;
  if (item >= rows * ng) return;
  const int64_t row = item / ng, gi = item % ng;
  const float* src = w + row * cols + gi * 128 + 2 * lane;
  const float a = src[0], b = src[1];
  float mx = fmaxf(fabsf(a), fabsf(b));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  const float s32 = mx / 7.0f;
  // bf16 round to nearest even of s32
  uint32_t u = __builtin_bit_cast(uint32_t, s32);
  u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  const float s = __builtin_bit_cast(float, u << 16);
  int qa = 0, qb = 0;
  if (s > 0.f) {
    qa = (int)fminf(fmaxf(rintf(a / s), -8.f), 7.f);
    qb = (int)fminf(fmaxf(rintf(b / s), -8.f), 7.f);
  }
  packed[row * (cols / 2) + gi * 64 + lane] = (uint8_t)((qa & 0xF) | ((qb & 0xF) << 4));
  if (lane == 0) scales[row * ng + gi] = (uint16_t)u;
}

// ABI nibble order (byte j: input 2j low, 2j+1 high; two's complement) -> internal words
// (see int4_word_to_bf16x8_biased; offset binary).  One thread per 32-bit output word.
__global__ void k_repack_int4(const uint8_t* src, uint32_t* dst, int64_t words) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= words) return;
  const uint8_t* b = src + i * 4;
  uint32_t out = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = (b[j] & 0xFu) ^ 0x8u, hi = ((b[j] >> 4) & 0xFu) ^ 0x8u;
    out |= lo << (4 * j);
    out |= hi << (16 + 4 * j);
  }
  dst[i] = out;
}

// ================================================================== host side
size_t attn_counters(const Dims& d) {
  const int QT = ((d.Hq / d.Hkv) * d.H + 15) / 16;
  return (size_t)d.B * d.Hkv * QT;
}
size_t attn_ws_floats(const Dims& d, const Plan& p) {
  const int T = d.P + d.H, nblk = (T + 31) / 32;
  const int S = (nblk + p.attn_bps - 1) / p.attn_bps;
  return attn_counters(d) * S * ((size_t)(d.dh / 16) * 256 + 32);
}
size_t gemm_counters(const Dims& d) {
  size_t n = d.qkv / 16;
  if ((size_t)d.D / 16 > n) n = d.D / 16;
  if ((size_t)d.F / 16 > n) n = d.F / 16;
  return n;
}
size_t gemm_ws_floats(const Dims& d, const Plan& p) {
  const int MT = (d.M + 15) / 16;
  size_t n = 0;
  auto upd = [&](size_t tiles, int S, int NT) {
    if (S > 1) n = std::max(n, tiles * S * NT * MT * 256);
  };
  upd(d.qkv / 16, p.s_qkv, 1);
  upd(d.D / 16, p.s_o, 1);
  upd(d.F / 16, p.s_gu, 2);
  upd(d.D / 16, p.s_d, 1);
  return n;
}

static int pick_split(int K, int tiles, bool int4) {
  // aim for about 256 workgroups; each split must hold whole 4-wave rounds (int4: whole groups)
  const int unit = int4 ? 128 * 4 : 32 * 4;
  int best = 1;
  for (int S = 1; S <= 8; S *= 2) {
    if (K % (S * unit)) break;
    best = S;
    if (tiles * S >= 256) break;
  }
  return best;
}

Plan make_plan(const Dims& d, WDtype wt) {
  Plan p;
  const bool i4 = wt == W_INT4;
  p.s_qkv = pick_split(d.D, d.qkv / 16, i4);
  p.s_o = pick_split(d.Hq * d.dh, d.D / 16, i4);
  p.s_gu = pick_split(d.D, d.F / 16, i4);
  p.s_d = pick_split(d.F, d.D / 16, i4);
  const int T = d.P + d.H, nblk = (T + 31) / 32;
  const int QT = ((d.Hq / d.Hkv) * d.H + 15) / 16, QG = (QT + 3) / 4;
  // enough splits for ~2 waves per CU overall, at least 2 blocks per split
  int want = 256 / (QG * 4 * d.B * d.Hkv);
  if (want < 1) want = 1;
  int bps = (nblk + want - 1) / want;
  if (bps < 2) bps = 2;
  p.attn_bps = bps;
  return p;
}

template <class AT, class WT, int EPI, int NT>
static hipError_t launch_gemm_mt(const Dims& d, const Bufs& b, const GemmLaunch& g, int tiles, hipStream_t st) {
  const int MT = (d.M + 15) / 16;
  dim3 grid(tiles * g.S), block(256);
  switch (MT) {
    case 1: hipLaunchKernelGGL((k_gemm<AT, WT, 1, NT, EPI>), grid, block, 0, st, d, b, g); break;
    case 2: hipLaunchKernelGGL((k_gemm<AT, WT, 2, NT, EPI>), grid, block, 0, st, d, b, g); break;
    case 3: hipLaunchKernelGGL((k_gemm<AT, WT, 3, NT, EPI>), grid, block, 0, st, d, b, g); break;
    case 4: hipLaunchKernelGGL((k_gemm<AT, WT, 4, NT, EPI>), grid, block, 0, st, d, b, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class AT>
static hipError_t launch_attn(const Dims& d, const Bufs& b, const Plan& p, int layer, hipStream_t st) {
  const int T = d.P + d.H, nblk = (T + 31) / 32;
  const int S = (nblk + p.attn_bps - 1) / p.attn_bps;
  const int QT = ((d.Hq / d.Hkv) * d.H + 15) / 16, QG = (QT + 3) / 4;
  dim3 grid(d.B * d.Hkv * QG * S), block(256);
  switch (d.dh) {
    case 32: hipLaunchKernelGGL((k_attn<AT, 32>), grid, block, 0, st, d, b, layer, S, p.attn_bps); break;
    case 64: hipLaunchKernelGGL((k_attn<AT, 64>), grid, block, 0, st, d, b, layer, S, p.attn_bps); break;
    case 128: hipLaunchKernelGGL((k_attn<AT, 128>), grid, block, 0, st, d, b, layer, S, p.attn_bps); break;
    case 256: hipLaunchKernelGGL((k_attn<AT, 256>), grid, block, 0, st, d, b, layer, S, p.attn_bps); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class T> static size_t wbytes_row(int K);
template <> size_t wbytes_row<float>(int K) { return (size_t)K * 4; }
template <> size_t wbytes_row<bf16>(int K) { return (size_t)K * 2; }
template <> size_t wbytes_row<i4>(int K) { return (size_t)K / 2; }

template <class AT, class WT, class IOT>
static hipError_t denoise_impl(const Dims& d, const Bufs& b, const Plan& p, hipStream_t st) {
#define PHYAI_CHECK(x)            \
  do {                            \
    hipError_t e_ = (x);          \
    if (e_ != hipSuccess) return e_; \
  } while (0)
  const int qd = d.Hq * d.dh;
  const size_t sz_qkv = wbytes_row<WT>(d.D) * d.qkv, sz_o = wbytes_row<WT>(qd) * d.D;
  const size_t sz_gu = wbytes_row<WT>(d.D) * 2 * d.F, sz_d = wbytes_row<WT>(d.F) * d.D;
  const char* wq = static_cast<const char*>(b.w_qkv);
  const char* wo = static_cast<const char*>(b.w_o);
  const char* wg = static_cast<const char*>(b.w_gu);
  const char* wd = static_cast<const char*>(b.w_d);
  hipLaunchKernelGGL((k_out_euler<AT, IOT>), dim3(d.M), dim3(256), 0, st, d, b, -1, 0);
  PHYAI_CHECK(hipGetLastError());
  for (int k = 0; k < d.N; ++k) {
    const float* cv = b.cvec + (size_t)k * b.cv_stride;
    for (int l = 0; l < d.L; ++l) {
      GemmLaunch g{};
      g.layer = l;
      // QKV
      g.A = b.hs; g.lda = d.D; g.K = d.D; g.W = wq + sz_qkv * l;
      g.Ws = b.s_qkv ? b.s_qkv + (size_t)l * d.qkv * (d.D / 128) : nullptr;
      g.S = p.s_qkv; g.cvec = cv + (size_t)l * d.qkv;
      PHYAI_CHECK((launch_gemm_mt<AT, WT, EPI_QKV, 1>(d, b, g, d.qkv / 16, st)));
      PHYAI_CHECK(launch_attn<AT>(d, b, p, l, st));
      // O + residual; consumer is the MLP norm 2l+1
      g = GemmLaunch{};
      g.layer = l; g.A = b.o; g.lda = qd; g.K = qd; g.W = wo + sz_o * l;
      g.Ws = b.s_o ? b.s_o + (size_t)l * d.D * (qd / 128) : nullptr;
      g.S = p.s_o; g.scale_next = b.mod + (((size_t)k * d.nmod + 2 * l + 1) * 2) * d.D;
      PHYAI_CHECK((launch_gemm_mt<AT, WT, EPI_RESID, 1>(d, b, g, d.D / 16, st)));
      // gate/up + GeGLU
      g = GemmLaunch{};
      g.layer = l; g.A = b.hs; g.lda = d.D; g.K = d.D; g.W = wg + sz_gu * l;
      g.Ws = b.s_gu ? b.s_gu + (size_t)l * 2 * d.F * (d.D / 128) : nullptr;
      g.n_second = d.F; g.S = p.s_gu; g.cvec = cv + b.cv_gu_off + (size_t)l * 2 * d.F;
      PHYAI_CHECK((launch_gemm_mt<AT, WT, EPI_GEGLU, 2>(d, b, g, d.F / 16, st)));
      // down + residual; consumer is norm 2(l+1), or the final norm 2L
      g = GemmLaunch{};
      g.layer = l; g.A = b.act; g.lda = d.F; g.K = d.F; g.W = wd + sz_d * l;
      g.Ws = b.s_d ? b.s_d + (size_t)l * d.D * (d.F / 128) : nullptr;
      g.S = p.s_d;
      const int jn = (l + 1 < d.L) ? 2 * (l + 1) : 2 * d.L;
      g.scale_next = b.mod + (((size_t)k * d.nmod + jn) * 2) * d.D;
      PHYAI_CHECK((launch_gemm_mt<AT, WT, EPI_RESID, 1>(d, b, g, d.D / 16, st)));
    }
    hipLaunchKernelGGL((k_out_euler<AT, IOT>), dim3(d.M), dim3(256), 0, st, d, b, k, k + 1 < d.N ? k + 1 : -1);
    PHYAI_CHECK(hipGetLastError());
  }
  return hipSuccess;
#undef PHYAI_CHECK
}

hipError_t enqueue_denoise(const Dims& d, const Bufs& b, const Plan& p, WDtype wt, hipStream_t st) {
  switch (wt) {
    case W_F32: return denoise_impl<float, float, float>(d, b, p, st);
    case W_BF16: return denoise_impl<bf16, bf16, bf16>(d, b, p, st);
    case W_INT4: return denoise_impl<bf16, i4, bf16>(d, b, p, st);
  }
  return hipErrorInvalidValue;
}

template <class WT, class IOT>
static hipError_t tables_impl(const Dims& d, const Bufs& b, const float* t_dev, double* e, float* mod,
                              float* cvec, hipStream_t st) {
  const int ne = d.N * d.D;
  hipLaunchKernelGGL(k_embed, dim3((ne + 255) / 256), dim3(256), 0, st, t_dev, d.N, d.D, e);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int rows = d.nmod * 2 * d.D;
  hipLaunchKernelGGL((k_modulation<IOT>), dim3((rows + 3) / 4), dim3(256), 0, st,
                     static_cast<const IOT*>(b.w_mod), static_cast<const IOT*>(b.b_mod), e, d.N, d.nmod, d.D, mod);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int rows2 = d.L * d.qkv + d.L * 2 * d.F + d.A;
  hipLaunchKernelGGL((k_shift_proj<WT, IOT>), dim3((rows2 + 3) / 4), dim3(256), 0, st, d, b, mod, cvec);
  return hipGetLastError();
}

hipError_t enqueue_tables(const Dims& d, const Bufs& b, WDtype wt, const float* t_dev, double* e,
                          float* mod, float* cvec, hipStream_t st) {
  switch (wt) {
    case W_F32: return tables_impl<float, float>(d, b, t_dev, e, mod, cvec, st);
    case W_BF16: return tables_impl<bf16, bf16>(d, b, t_dev, e, mod, cvec, st);
    case W_INT4: return tables_impl<i4, bf16>(d, b, t_dev, e, mod, cvec, st);
  }
  return hipErrorInvalidValue;
}

hipError_t enqueue_install_prefix(const Dims& d, const void* k, const void* v, int batch, int P, void* kc,
                                  void* vt, size_t es, hipStream_t st) {
  const size_t total = (size_t)batch * d.L * d.Hkv * d.dh * P;
  const int blocks = (int)std::min<size_t>((total + 255) / 256, 65536);
  if (es == 4)
    hipLaunchKernelGGL(k_install_prefix<float>, dim3(blocks), dim3(256), 0, st, d, static_cast<const float*>(k),
                       static_cast<const float*>(v), batch, P, static_cast<float*>(kc), static_cast<float*>(vt));
  else
    hipLaunchKernelGGL(k_install_prefix<uint16_t>, dim3(blocks), dim3(256), 0, st, d,
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), batch, P,
                       static_cast<uint16_t*>(kc), static_cast<uint16_t*>(vt));
  return hipGetLastError();
}

hipError_t enqueue_quantize_int4(const float* w, int64_t rows, int64_t cols, uint8_t* packed, uint16_t* scales,
                                 hipStream_t st) {
  const int64_t items = rows * (cols / 128);
  if (items == 0) return hipSuccess;
  hipLaunchKernelGGL(k_quantize_int4, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, st, w, rows, cols, packed,
                     scales);
  return hipGetLastError();
}

hipError_t enqueue_repack_int4(const uint8_t* src, uint8_t* dst, int64_t rows, int64_t cols, hipStream_t st) {
  const int64_t words = rows * cols / 8;
  if (words == 0) return hipSuccess;
  hipLaunchKernelGGL(k_repack_int4, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, st, src,
                     reinterpret_cast<uint32_t*>(dst), words);
  return hipGetLastError();
}

}  // namespace phyai
