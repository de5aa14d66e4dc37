// Euler-loop kernels for few token rows (batch x chunk <= 64), gfx950.
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
// Weight streaming.  With at most 64 token rows every weight byte is used by
// only 64 rows, so these linears are bound by reading the weights once from
// HBM and by latency.  A workgroup owns 16 (or 16 gate + 16 up) output columns
// and a contiguous share of K; each of its four waves issues every load it will
// need (weights and activations) before its first MFMA, so one memory round
// trip covers the whole kernel.  K is walked in "quads" of 128: inside a quad,
// lane group g (lanes 16g..16g+15) owns k in [32g, 32g+32) -- 64 contiguous bytes
// of a bf16 row -- and MFMA j of the quad takes k in [32g+8j, 32g+8j+8) from both
// operands.  Partial sums across waves meet in LDS; across workgroups they meet
// through agent-scope stores and the last workgroup to arrive adds them in split
// order, so results never depend on arrival order.
#include "epilogue.h"

#include <math.h>

#include <algorithm>
#include <type_traits>

namespace phyai {

#ifdef PHYAI_PHASE_TRACE
__device__ uint64_t g_phase_trace[4096 * 4 * 8];
#endif

// ------------------------------------------------------------------ int4 fragments
// Swizzled int4 word (8 codes of one lane for one k-block, see sw4_word in common.h):
// OR-ing a pair of offset-binary codes into 0x4300 (bf16 128.0, whose mantissa step is 1)
// gives the exact bf16 pair (q + 136, q' + 136); the +136 is removed afterwards with the
// per-group row sums of the activations.
__device__ __forceinline__ bf16x8 int4_frag_biased(uint32_t w) {
  u32x4 r;
  r[0] = (w & 0x000F000Fu) | 0x43004300u;
  r[1] = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
  r[2] = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
  r[3] = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
  return __builtin_bit_cast(bf16x8, r);
}

// ------------------------------------------------------------------ weight-streaming GEMM
// The operands that the weight and activation loads need (W, A, K, splits, second row
// block) lead the argument list as scalars: they are preloaded into SGPRs at wave launch,
// so the loads do not wait for the kernel-argument fetch.
template <class AT, class WT, int MT, int NT, int KBW, int EPI>
__global__ __launch_bounds__(256) void k_gemm(const void* Wp, const void* Ap, int Kp, int Sp, int nsec, Dims d,
                                              Bufs bf, GemmLaunch g) {
  constexpr bool NORM = (EPI == EPI_QKV || EPI == EPI_GEGLU);
  constexpr bool INT4 = __is_same(WT, i4);
  __shared__ f32x4 red[4][NT][MT][64];
  __shared__ float rinv_s[64];
  __shared__ unsigned flag;
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int s = blockIdx.x % Sp, tile = blockIdx.x / Sp;
  int nrow[NT];
  nrow[0] = tile * 16;
  if (NT == 2) nrow[NT - 1] = nsec + tile * 16;

  PHASE_MARK(0);
  // this wave's k-blocks: [kbeg, min(kbeg + KBW, kend)), contiguous
  const int KB = Kp / 32, kbs = KB / Sp;
  const int kbeg = s * kbs + w * KBW, kend = s * kbs + kbs;

  // ---- 1. loads: first the weights (HBM) and activations (L2), whose addresses come from
  // the preloaded arguments alone.
  // A wave owns exactly KBW k-blocks (the host sizes splits so that every wave is full),
  // except int4 splits of fewer than four quads, whose surplus waves are idle: the
  // branch below is uniform and no per-block exit exists that the compiler could sink
  // the loads behind.
  const bool wave_active = kbeg < kend;
  const AT* A = static_cast<const AT*>(Ap);
  typedef typename FragOf<AT>::type AFrag;
  AFrag af[KBW][MT];
  typename FragOf<AT>::type wf[INT4 ? 1 : KBW][INT4 ? 1 : NT];   // fp32 / bf16 weight fragments
  constexpr int NQW = (INT4 && KBW >= 4) ? KBW / 4 : 1;          // int4 quads per wave (KBW >= 4)
  u32x4 wq[NQW][NT];                                               // int4: one 16-byte slot per quad
  float wsc[NQW][NT];
  if (wave_active) {
#pragma unroll
    for (int i = 0; i < KBW; ++i) {
      const int kb = kbeg + i;
      if constexpr (!INT4) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          wf[i][nt] = load_frag(static_cast<const WT*>(Wp) + sw_frag(nrow[nt] >> 4, kb, Kp, lane));
      } else {
        if ((i & 3) == 0) {
          const int q = kb >> 2;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            wq[i >> 2][nt] =
                reinterpret_cast<const u32x4*>(Wp)[((size_t)(nrow[nt] >> 4) * (Kp >> 7) + q) * 64 + lane];
            wsc[i >> 2][nt] = bf16_bits_to_f32(g.Ws[(size_t)(nrow[nt] + r16) * (g.K >> 7) + q]);
          }
        }
      }
#pragma unroll
      for (int mtl = 0; mtl < MT; ++mtl) af[i][mtl] = load_frag(A + sw_frag(mtl, kb, Kp, lane));
    }
  }
  // ---- 1b. then the epilogue operands and norm statistics (L2), which wait for the
  // kernel-argument fetch.  Addresses are clamped to valid rows/quads instead of
  // predicating the loads; rows/quads past the end are masked out afterwards.
  const int mt = w;                            // M-tile this wave finishes in the epilogue
  float epi_h[4] = {0.f, 0.f, 0.f, 0.f};       // residual rows (RESID)
  float epi_c0 = 0.f, epi_c1 = 0.f;            // cvec / scale_next of this lane's column(s)
  if constexpr (EPI == EPI_RESID) {
    const int col = nrow[0] + r16;
    epi_c0 = g.scale_next[col];
    epi_c1 = g.gate ? g.gate[col] : 1.f;   // residual gate (1: plain residual, exact)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = min(mt * 16 + grp * 4 + i, d.M - 1);
      epi_h[i] = bf.h[(size_t)m * d.D + col];
    }
  } else if constexpr (EPI == EPI_QKV) {
    epi_c0 = g.cvec[nrow[0] + r16];
  } else {
    epi_c0 = g.cvec[nrow[0] + r16];
    epi_c1 = g.cvec[g.n_second + nrow[0] + r16];
  }
  // row statistics: 4 threads per token row, each a quarter of the D/16 partials
  f32x4 ssv[8];
  const int srow = min(tid >> 2, d.M - 1), squart = tid & 3;
  const int n4 = d.D / 256;                    // f32x4 per quarter (D % 256 == 0 here)
  if constexpr (NORM) {
    const f32x4* p = reinterpret_cast<const f32x4*>(bf.ssq + (size_t)srow * (d.D / 16) + squart * (d.D / 64));
#pragma unroll
    for (int j = 0; j < 8; ++j) ssv[j] = p[min(j, n4 - 1)];
  }
  // keep every load above in flight together: nothing below may be scheduled before them
  __builtin_amdgcn_sched_barrier(0);
  PHASE_MARK(1);
  // ---- 2. MFMA
  f32x4 acc[NT][MT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (wave_active) {
    if constexpr (!INT4) {
#pragma unroll
      for (int i = 0; i < KBW; ++i)
#pragma unroll
        for (int mtl = 0; mtl < MT; ++mtl)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[nt][mtl] = mma(af[i][mtl], wf[i][nt], acc[nt][mtl]);
    } else {
      // one 128-wide quad = one scale group: sum(x (q + 136)) - 136 sum(x), times the scale
      const bf16x8 ones = {(bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f,
                           (bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f};
#pragma unroll
      for (int qi = 0; qi < (KBW >= 4 ? KBW / 4 : 0); ++qi) {
        f32x4 part[NT][MT], rs[MT];
#pragma unroll
        for (int mtl = 0; mtl < MT; ++mtl) {
          rs[mtl] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) part[nt][mtl] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int mtl = 0; mtl < MT; ++mtl) {
            const bf16x8 a = af[4 * qi + j][mtl];
            rs[mtl] = mma(a, ones, rs[mtl]);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) part[nt][mtl] = mma(a, int4_frag_biased(wq[qi][nt][j]), part[nt][mtl]);
          }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int mtl = 0; mtl < MT; ++mtl)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[nt][mtl][e] += wsc[qi][nt] * (part[nt][mtl][e] - 136.0f * rs[mtl][e]);
      }
    }
  }

  // row norms (needed by the epilogue only): after the products, so that the MFMAs start
  // as soon as the weights and activations have landed
  if constexpr (NORM) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < n4) {
        ss += ssv[j][0];
        ss += ssv[j][1];
        ss += ssv[j][2];
        ss += ssv[j][3];
      }
    // fixed-order combination of the four quarters of a row
    const float s1 = __shfl_xor(ss, 1, 64);
    const float s2 = __shfl_xor(ss, 2, 64);
    const float s3 = __shfl_xor(ss, 3, 64);
    float q0, q1, q2, q3;  // quarter 0..3 of this row
    q0 = squart == 0 ? ss : squart == 1 ? s1 : squart == 2 ? s2 : s3;
    q1 = squart == 1 ? ss : squart == 0 ? s1 : squart == 3 ? s2 : s3;
    q2 = squart == 2 ? ss : squart == 3 ? s1 : squart == 0 ? s2 : s3;
    q3 = squart == 3 ? ss : squart == 2 ? s1 : squart == 1 ? s2 : s3;
    if (squart == 0 && (tid >> 2) < d.M) rinv_s[tid >> 2] = 1.0f / sqrtf((((q0 + q1) + q2) + q3) / (float)d.D + d.eps);
  }

  PHASE_MARK(2);
  // ---- 3. cross-wave reduction in a fixed order; wave w then owns M-tile w
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[w][nt][mt][lane] = acc[nt][mt];
  __syncthreads();
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

  PHASE_MARK(3);
  // ---- 4. cross-workgroup split: the last arrival sums the partials in split order
  if (g.S > 1) {
    const uint32_t part_bytes = (uint32_t)NT * MT * 1024;
    const __amdgpu_buffer_rsrc_t ws = agent_rsrc(bf.gemm_ws + (size_t)tile * g.S * NT * MT * 256, part_bytes * g.S);
    if (mt < MT)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) st_agent16(ws, s * part_bytes + ((nt * MT + mt) * 64 + lane) * 16, tot[nt]);
    PHASE_MARK(4);
    const bool last = split_arrive_wg(bf.gemm_cnt + tile, (unsigned)g.S, &flag);
    PHASE_MARK(5);
    if (!last) return;
    if (mt < MT) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4 parts[8];
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2)
          parts[s2] = ld_agent16(ws, min(s2, g.S - 1) * part_bytes + ((nt * MT + mt) * 64 + lane) * 16);
        f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2)
          if (s2 < g.S) sum += (s2 == s) ? tot[nt] : parts[s2];
        tot[nt] = sum;
      }
    }
  }
  PHASE_MARK(6);
  if (mt >= MT) return;

  // ---- 5. epilogues.  tot[nt][i] is row mt*16 + 4*grp + i, column nrow[nt] + r16.
  if constexpr (EPI == EPI_QKV) {
    const int col = nrow[0] + r16;
    const float c = epi_c0;
    const int qd = d.Hq * d.dh, kd = d.Hkv * d.dh;
    AT* q = static_cast<AT*>(bf.q);
    AT* kc = static_cast<AT*>(bf.kc);
    AT* vt = static_cast<AT*>(bf.vt);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + grp * 4 + i;       // < 64: rinv_s holds every row slot
      float y = rinv_s[m] * tot[0][i] + c;
      if (d.rope_theta > 0.f) y = rope_rotate(d, m, col, y, __shfl_xor(y, 1, 64));  // all lanes shuffle
      if (m >= d.M) continue;
      const int b = m / d.H, t = m % d.H;
      if (col < qd) {
        q[(size_t)m * qd + col] = to_elem<AT>(y);
      } else if (col < qd + kd) {
        const int r = (col - qd) / d.dh, dd = (col - qd) % d.dh;
        kc[((((size_t)b * d.Lc + g.layer) * d.Hkv + r) * d.KS + d.P + t) * d.dh + dd] = to_elem<AT>(y);
      } else {
        const int r = (col - qd - kd) / d.dh, dd = (col - qd - kd) % d.dh;
        vt[((((size_t)b * d.Lc + g.layer) * d.Hkv + r) * d.dh + dd) * d.KS + d.P + t] = to_elem<AT>(y);
      }
    }
  } else if constexpr (EPI == EPI_RESID) {
    const int col = nrow[0] + r16;
    const float sc1 = 1.0f + epi_c0;
    AT* hs = static_cast<AT*>(bf.hs);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + grp * 4 + i;
      float hn = 0.f;
      if (m < d.M) {
        hn = epi_h[i] + epi_c1 * tot[0][i];
        bf.h[(size_t)m * d.D + col] = hn;
        hs[sw_idx(m, col, d.D)] = to_elem<AT>(hn * sc1);
      }
      const float sq = sum16(hn * hn);
      if (r16 == 0 && m < d.M) bf.ssq[(size_t)m * (d.D / 16) + tile] = sq;
    }
  } else {  // EPI_GEGLU
    const int f = nrow[0] + r16;
    const float cg = epi_c0, cu = epi_c1;
    AT* act = static_cast<AT*>(bf.act);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + grp * 4 + i;
      if (m >= d.M) continue;
      const float yg = rinv_s[m] * tot[0][i] + cg;
      const float yu = rinv_s[m] * tot[NT - 1][i] + cu;
      act[sw_idx(m, f, d.F)] = to_elem<AT>(gelu_tanh(yg) * yu);
    }
  }
  PHASE_MARK(7);
}

// ------------------------------------------------------------------ attention
// End of one query tile's attention (one wave): with S > 1 key splits, publish this split's
// partial; then either k_attn_merge combines the splits in a later launch (ext_merge), or
// the last split to arrive merges all S partials in split order with log-sum-exp weights.
// The normalised output goes to o (swizzled [Mpad][Hq*dh], the A operand of the output
// projection).  o holds O^T of the tile (lane: column r16, rows
// 4 grp + i of 16-column tile t), m_run / l_part the running max (log2 units) and this
// lane's part of the row sums.  item indexes the tile's split workspace and counter.
template <class AT, int DH>
__device__ __forceinline__ void attn_finish(const Dims& d, const Bufs& bf, f32x4 (&o)[DH / 16], float m_run,
                                            float l_part, int S, int s, size_t item, bool qvalid, int m, int head,
                                            bool ext_merge) {
  constexpr int ES = sizeof(AT);
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
  const int qd = d.Hq * DH;
  float l_row = l_part;
  l_row += __shfl_xor(l_row, 16, 64);
  l_row += __shfl_xor(l_row, 32, 64);

  if (S > 1) {
    // Partial of this split: (m, l) in fp32 and O / l in the activation type (bf16 halves
    // the hand-off; fp32 workloads keep fp32), as 16-byte lane slots.  Every split, the
    // merging one included, enters the merge through the stored (rounded) value, so the
    // result does not depend on which split finishes last.
    constexpr int PAY = ES == 2 ? DH / 32 : DH / 16;   // 16-byte slots per lane
    constexpr uint32_t STRIDE = PAY * 1024 + 128;      // bytes per split partial
    const __amdgpu_buffer_rsrc_t ws = agent_rsrc(bf.attn_ws + item * S * (STRIDE / 4), STRIDE * S);
    const float inv_l = 1.0f / l_row;
#pragma unroll
    for (int u = 0; u < PAY; ++u) {
      f32x4 v;
      if constexpr (ES == 2) {
        const f32x4 a = o[2 * u] * inv_l, c = o[2 * u + 1] * inv_l;
        const bf16x8 pk = {(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3], (bf16)c[0], (bf16)c[1], (bf16)c[2], (bf16)c[3]};
        v = __builtin_bit_cast(f32x4, pk);
      } else {
        v = o[u] * inv_l;
      }
      st_agent16(ws, s * STRIDE + (u * 64 + lane) * 16, v);
    }
    if (grp == 0) {
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, m_run), ws, s * STRIDE + PAY * 1024 + r16 * 4, 0, 16);
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, l_row), ws, s * STRIDE + PAY * 1024 + 64 + r16 * 4,
                                            0, 16);
    }
    PHASE_MARK(3);
    if (ext_merge) return;                           // k_attn_merge combines the splits
    const bool last = split_arrive_wave(bf.attn_cnt + item, (unsigned)S);
    PHASE_MARK(4);
    if (!last) return;
    // the statistics and the first four payloads in one round trip
    float ms[8], ls[8];
    f32x4 v0[4][PAY];
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) {
      const uint32_t off = min(s2, S - 1) * STRIDE + PAY * 1024;
      ms[s2] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ws, off + r16 * 4, 0, 16));
      ls[s2] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ws, off + 64 + r16 * 4, 0, 16));
    }
#pragma unroll
    for (int u4 = 0; u4 < 4; ++u4)
#pragma unroll
      for (int u = 0; u < PAY; ++u) v0[u4][u] = ld_agent16(ws, min(u4, S - 1) * STRIDE + (u * 64 + lane) * 16);
    float M = -INFINITY;
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2)
      if (s2 < S) M = fmaxf(M, ms[s2]);
    float wgt[8], den = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) {
      wgt[s2] = s2 < S ? exp2f(ms[s2] - M) * ls[s2] : 0.f;
      den += wgt[s2];
    }
#pragma unroll
    for (int t = 0; t < DH / 16; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h2 = 0; h2 < 8; h2 += 4) {
      if (h2 >= S) break;
      f32x4 v[4][PAY];
#pragma unroll
      for (int u4 = 0; u4 < 4; ++u4)
#pragma unroll
        for (int u = 0; u < PAY; ++u)
          v[u4][u] = h2 == 0 ? v0[u4][u] : ld_agent16(ws, min(h2 + u4, S - 1) * STRIDE + (u * 64 + lane) * 16);
#pragma unroll
      for (int u4 = 0; u4 < 4; ++u4)
#pragma unroll
        for (int u = 0; u < PAY; ++u) {
          if constexpr (ES == 2) {
            const bf16x8 pk = __builtin_bit_cast(bf16x8, v[u4][u]);
            o[2 * u] += wgt[h2 + u4] * f32x4{(float)pk[0], (float)pk[1], (float)pk[2], (float)pk[3]};
            o[2 * u + 1] += wgt[h2 + u4] * f32x4{(float)pk[4], (float)pk[5], (float)pk[6], (float)pk[7]};
          } else {
            o[u] += wgt[h2 + u4] * v[u4][u];
          }
        }
    }
    l_row = den;
  }
  if (!qvalid) return;
  const float inv = 1.0f / l_row;
  // o is the A operand of the output projection: swizzled [Mpad][Hq*dh].  The four values
  // of (t, i = 0..3) are consecutive columns inside one 8-wide lane slot.
  AT* op = static_cast<AT*>(bf.o);
#pragma unroll
  for (int t = 0; t < DH / 16; ++t) {
    AT* dst = op + sw_idx(m, head * DH + t * 16 + grp * 4, qd);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = to_elem<AT>(o[t][i] * inv);
  }
}

// Split-key flash decode.  The query rows of one KV head r are the g*H pairs
// (query head r*g + j, chunk token t), row j*H + t, in 16-row tiles; the keys are
// the P cached prefix rows followed by the H chunk rows (no mask among them).
// A workgroup owns (sample, KV head, 4 query tiles, key split).  Its threads stage the
// split's keys -- up to NB blocks of 32 at once -- as K and V^T tiles in LDS with one
// burst of loads; for each query tile one wave (NB = 1) or two waves, one per half of the
// staged blocks, run S^T = K q^T on MFMA, a direct softmax over the staged keys (online
// rescaling only between groups of NB blocks), then O^T += V^T P^T on MFMA, and the two
// halves combine through LDS.  The probabilities come out of the first product already
// laid out as the second product's B operand, which is why V is kept transposed in the
// cache.  Each split leaves a partial (O / l, m, l) for k_attn_merge.
template <class AT, int DH, int NB>
__global__ __launch_bounds__(NB >= 2 ? 512 : 256) void k_attn(Dims d, Bufs bf, int layer, int S, int bps) {
  typedef typename FragOf<AT>::type Frag;
  constexpr int KH = NB >= 2 ? 2 : 1;                 // waves per query tile (key halves of a group)
  constexpr int NT = 64 * 4 * KH;                     // threads
  static_assert(NB == 1 || NB == 2 || (NB == 4 && DH * sizeof(AT) <= 512),
                "32-key blocks staged per group (LDS <= 160 KB)");
  constexpr int NBH = NB / KH;                        // blocks of a group per wave
  constexpr int NK = NB * 32;
  constexpr int ES = sizeof(AT);
  constexpr int KROW = DH + 16 / ES;                 // K row: DH + 16 B pad
  constexpr int VROW = NK + 4;                       // V^T row: NK keys + 4-element pad (bank spread)
  constexpr int KCPR = DH * ES / 16;                 // 16-byte chunks per K row
  constexpr int VCPR = NK * ES / 16;                 // 16-byte chunks per staged V^T row
  constexpr int KCH = NK * KCPR, VCH = DH * VCPR;    // chunks of one group
  constexpr int CPT = (KCH + VCH) / NT;              // chunks per thread
  constexpr int KS_B = NK * KROW * ES, VS_B = DH * VROW * ES;
  constexpr int CMB = DH / 4 + 2;                    // floats per lane handed from half 1 to half 0
  constexpr int CMB_B = 4 * CMB * 64 * 4;
  constexpr int PAIR_B = 8 * (DH / 8 + 2) * 64 * 4;  // both halves hand over half their columns
  constexpr int CMX_B = KH == 1 ? 0 : CMB_B > PAIR_B ? CMB_B : PAIR_B;
  constexpr int LDS_B = KS_B + VS_B > CMX_B ? KS_B + VS_B : CMX_B;
  static_assert((KCH + VCH) % NT == 0 && NB % KH == 0, "group size");
  __shared__ __attribute__((aligned(16))) char lds_raw[LDS_B];
  AT* ks = reinterpret_cast<AT*>(lds_raw);
  AT* vs = reinterpret_cast<AT*>(lds_raw + KS_B);

  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = w & 3, half = w >> 2;               // query tile slot, key half
  const int gq = d.Hq / d.Hkv;
  const int QT = (gq * d.H + 15) / 16, QG = (QT + 3) / 4;
  // Workgroups go to the 8 XCDs round robin: the split index is the workgroup index mod 8
  // (or mod 16 / 32 for more splits), so all query groups of one key split run on one XCD
  // and share its L2 copy of the split's K/V (S <= 32; slots s >= S have no work).
  int idx = blockIdx.x;
  const int sl = S > 16 ? 5 : S > 8 ? 4 : 3;
  const int s = idx & ((1 << sl) - 1);
  if (s >= S) return;
  idx >>= sl;
  const int qg = idx % QG;
  idx /= QG;
  const int r = idx % d.Hkv;
  const int b = idx / d.Hkv;
  const int qt = qg * 4 + wq;
  const bool active = qt < QT;
  const int T = d.P + d.H;
  const int nblk = (T + 31) / 32;
  const int blk0 = s * bps, blk1 = min(nblk, blk0 + bps);
  const int kend = min(T, blk1 * 32);                // keys of this split: [blk0*32, kend)

  const int qrow = qt * 16 + r16;
  const bool qvalid = active && qrow < gq * d.H;
  const int head = r * gq + (qvalid ? qrow / d.H : 0);
  const int tok = qvalid ? qrow % d.H : 0;
  const int m = b * d.H + tok;
  const int qd = d.Hq * DH;

  const size_t kvbase = ((size_t)b * d.Lc + layer) * d.Hkv + r;
  const AT* Kc = static_cast<const AT*>(bf.kc) + kvbase * d.KS * DH;
  const AT* Vt = static_cast<const AT*>(bf.vt) + kvbase * DH * d.KS;

  PHASE_MARK(0);
  Frag qf[DH / 32];
  {
    const AT* qp = static_cast<const AT*>(bf.q) + (size_t)m * qd + head * DH + grp * 8;
#pragma unroll
    for (int j = 0; j < DH / 32; ++j) qf[j] = load_frag(qp + 32 * j);
  }

  const float sc = 1.4426950408889634f / sqrtf((float)DH);  // log2(e) / sqrt(dh)
  float m_run = -INFINITY, l_part = 0.f;
  f32x4 o[DH / 16];
#pragma unroll
  for (int t = 0; t < DH / 16; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int g0 = blk0; g0 < blk1; g0 += NB) {
    const int glast = min(blk1, g0 + NB) - 1;          // last block of this group
    // ---- one burst of loads for the whole group (blocks past the split are clamped to
    // its last block: their keys are masked below), then into LDS
    u32x4 stage[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + NT * i;
      const char* src;
      if (c < KCH) {
        const int row = c / KCPR;                        // staged key row 0..NK-1
        const int blk = min(g0 + row / 32, glast);
        src = reinterpret_cast<const char*>(Kc + (size_t)(blk * 32 + row % 32) * DH) + (c % KCPR) * 16;
      } else {
        const int cv = c - KCH;
        const int row = cv / VCPR;                       // dh row
        const int kofs = (cv % VCPR) * (16 / ES);        // staged key offset 0..NK-1
        const int blk = min(g0 + kofs / 32, glast);
        src = reinterpret_cast<const char*>(Vt + (size_t)row * d.KS + blk * 32 + kofs % 32);
      }
      stage[i] = *reinterpret_cast<const u32x4*>(src);
    }
    __syncthreads();                                     // previous group's LDS reads are done
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + NT * i;
      AT* dst = c < KCH ? ks + (c / KCPR) * KROW + (c % KCPR) * (16 / ES)
                        : vs + ((c - KCH) / VCPR) * VROW + ((c - KCH) % VCPR) * (16 / ES);
      if (ES == 4 || c < KCH) {
        *reinterpret_cast<u32x4*>(dst) = stage[i];
      } else {  // bf16 V^T rows are 8-byte aligned
        reinterpret_cast<u32x2*>(dst)[0] = u32x2{stage[i][0], stage[i][1]};
        reinterpret_cast<u32x2*>(dst)[1] = u32x2{stage[i][2], stage[i][3]};
      }
    }
    __syncthreads();
    if (g0 == blk0) PHASE_MARK(1);
    // this wave's blocks of the group: [g0 + half*NBH, g0 + half*NBH + NBH) up to glast
    const int jb = half * NBH;
    if (!active || g0 + jb > glast) continue;
    // ---- scores of the wave's blocks, masked past the split
    float sv[NBH][8];
    float mx = -INFINITY;
#pragma unroll
    for (int jh = 0; jh < NBH; ++jh) {
      const int j = jb + jh;
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
      if (g0 + j <= glast) {
#pragma unroll
        for (int jj = 0; jj < DH / 32; ++jj) {
          s0 = mma(load_frag(ks + (j * 32 + r16) * KROW + 32 * jj + grp * 8), qf[jj], s0);
          s1 = mma(load_frag(ks + (j * 32 + 16 + r16) * KROW + 32 * jj + grp * 8), qf[jj], s1);
        }
      }
      // raw scores (the scale is applied inside the exponential), masked past the split
      // only in a block that straddles its end
      const int kb = (g0 + j) * 32 + grp * 4;
      const bool full = (g0 + j) * 32 + 32 <= kend;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[jh][i] = full || kb + i < kend ? s0[i] : -INFINITY;
        sv[jh][4 + i] = full || kb + 16 + i < kend ? s1[i] : -INFINITY;
        mx = fmaxf(mx, fmaxf(sv[jh][i], sv[jh][4 + i]));
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // Reference max in scaled (log2) units.  It is raised (and O, l rescaled) only when a
    // row's max exceeds it by more than 8: until then the weights stay below 2^8.
    const float m_cand = fmaxf(m_run, mx * sc);
    if (g0 == blk0) {
      m_run = m_cand;
    } else if (__any(m_cand > m_run + 8.f)) {
      const float alpha = fast_exp2(m_run - m_cand);
      l_part *= alpha;
#pragma unroll
      for (int t = 0; t < DH / 16; ++t) o[t] *= alpha;
      m_run = m_cand;
    }
    const float m_new = m_run;
#pragma unroll
    for (int jh = 0; jh < NBH; ++jh) {
      const int j = jb + jh;
      if (g0 + j > glast) break;
      Frag pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = fast_exp2(fmaf(sv[jh][e], sc, -m_new));
        l_part += p;
        pf[e] = to_elem<AT>(p);
      }
#pragma unroll
      for (int t = 0; t < DH / 16; ++t) {
        const AT* vp = vs + (t * 16 + r16) * VROW + j * 32 + grp * 4;
        o[t] = mma(load_frag_split4(vp, vp + 16), pf, o[t]);
      }
    }
  }
  PHASE_MARK(2);
  // ---- combine the two key halves of each query tile through LDS (the staging buffers
  // are free once every wave is past its last group).  Half 0 always holds the split's
  // first key, so its running max is finite.
  constexpr int PAY = ES == 2 ? DH / 32 : DH / 16;    // 16-byte partial slots per lane
  constexpr int PAYH = PAY / 2;                        // slots finished by each half
  constexpr bool PAIR = PAYH >= 1 && PAYH <= 4;        // both halves finish the tile
  if constexpr (KH == 1) {                             // one wave per tile: nothing to combine
    if (!active) return;
    attn_finish<AT, DH>(d, bf, o, m_run, l_part, S, s, ((size_t)(b * d.Hkv + r) * QT + qt), qvalid, m, head, true);
  } else if constexpr (!PAIR) {
    float* cmb = reinterpret_cast<float*>(lds_raw) + wq * CMB * 64;
    __syncthreads();
    if (half == 1 && active) {
      cmb[lane] = m_run;
      cmb[64 + lane] = l_part;
#pragma unroll
      for (int t = 0; t < DH / 16; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) cmb[(2 + 4 * t + i) * 64 + lane] = o[t][i];
    }
    __syncthreads();
    if (half == 1 || !active) return;
    {
      const float m1 = cmb[lane], l1 = cmb[64 + lane];
      const float M = fmaxf(m_run, m1);
      const float a0 = exp2f(m_run - M), a1 = exp2f(m1 - M);
      l_part = l_part * a0 + l1 * a1;
      m_run = M;
#pragma unroll
      for (int t = 0; t < DH / 16; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[t][i] = o[t][i] * a0 + cmb[(2 + 4 * t + i) * 64 + lane] * a1;
    }
    attn_finish<AT, DH>(d, bf, o, m_run, l_part, S, s, ((size_t)(b * d.Hkv + r) * QT + qt), qvalid, m, head, true);
  } else {
    // Both halves finish the tile, each its own half of the output columns (16-column
    // tiles [half*T2, half*T2 + T2)): each hands the other (m, l) and the other's columns
    // of its O^T, and both form the combination in the same order (half 0's part first).
    // The half index is made a compile-time constant (H) so that the register arrays are
    // indexed with constants (a run-time index would move them to scratch memory).
    constexpr int T2 = DH / 32;
    constexpr int CM2 = 4 * T2 + 2;                    // floats per lane handed over
    auto finish = [&](auto hc) {
    constexpr int H = decltype(hc)::value;
    float* mine = reinterpret_cast<float*>(lds_raw) + (wq * 2 + H) * CM2 * 64;
    const float* other = reinterpret_cast<const float*>(lds_raw) + (wq * 2 + (H ^ 1)) * CM2 * 64;
    __syncthreads();
    if (active) {
      mine[lane] = m_run;
      mine[64 + lane] = l_part;
#pragma unroll
      for (int t2 = 0; t2 < T2; ++t2)
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[(2 + 4 * t2 + i) * 64 + lane] = o[(H ^ 1) * T2 + t2][i];
    }
    __syncthreads();
    f32x4 oh[T2];                                      // this half's output tiles
    if (active) {
      const float mo = other[lane], lo = other[64 + lane];
      const float m0 = H ? mo : m_run, m1 = H ? m_run : mo;
      const float l0 = H ? lo : l_part, l1 = H ? l_part : lo;
      const float M = fmaxf(m0, m1);
      const float a0 = exp2f(m0 - M), a1 = exp2f(m1 - M);
      l_part = l0 * a0 + l1 * a1;
      m_run = M;
#pragma unroll
      for (int t2 = 0; t2 < T2; ++t2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float own = o[H * T2 + t2][i], oth = other[(2 + 4 * t2 + i) * 64 + lane];
          oh[t2][i] = H ? oth * a0 + own * a1 : own * a0 + oth * a1;
        }
    }
    float l_row = l_part;
    l_row += __shfl_xor(l_row, 16, 64);
    l_row += __shfl_xor(l_row, 32, 64);
    AT* op = static_cast<AT*>(bf.o);
    auto write_out = [&](const f32x4 (&v)[T2], float inv) {
#pragma unroll
      for (int t2 = 0; t2 < T2; ++t2) {
        AT* dst = op + sw_idx(m, head * DH + (H * T2 + t2) * 16 + grp * 4, qd);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = to_elem<AT>(v[t2][i] * inv);
      }
    };
    if (S == 1) {
      if (active && qvalid) write_out(oh, 1.0f / l_row);
      return;
    }
    // Split partial (O / l in the activation type, 16-byte slots, each half its own; (m, l)
    // in fp32 by half 0); k_attn_merge combines the splits in the next launch.
    constexpr uint32_t STRIDE = PAY * 1024 + 128;       // bytes per split partial
    const size_t item = (size_t)(b * d.Hkv + r) * QT + qt;
    const __amdgpu_buffer_rsrc_t ws = agent_rsrc(bf.attn_ws + item * S * (STRIDE / 4), STRIDE * S);
    if (active) {
      const float inv_l = 1.0f / l_row;
#pragma unroll
      for (int uh = 0; uh < PAYH; ++uh) {
        const int u = H * PAYH + uh;
        f32x4 v;
        if constexpr (ES == 2) {
          const f32x4 a = oh[2 * uh] * inv_l, c = oh[2 * uh + 1] * inv_l;
          const bf16x8 pk = {(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3],
                             (bf16)c[0], (bf16)c[1], (bf16)c[2], (bf16)c[3]};
          v = __builtin_bit_cast(f32x4, pk);
        } else {
          v = oh[uh] * inv_l;
        }
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ws, s * STRIDE + (u * 64 + lane) * 16, 0, 0);
      }
      if (H == 0 && grp == 0) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, m_run), ws, s * STRIDE + PAY * 1024 + r16 * 4, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, l_row), ws,
                                              s * STRIDE + PAY * 1024 + 64 + r16 * 4, 0, 0);
      }
    }
    PHASE_MARK(3);
    };
    if (half) finish(std::integral_constant<int, 1>{});
    else finish(std::integral_constant<int, 0>{});
  }
  PHASE_MARK(7);
}

// Merge of the key splits of the few-row attention, one launch after it: a one-wave
// workgroup per (query tile, 16-byte slot); each lane reads its slot and its row's (m, l)
// from every split,
// weights split s by 2^(m_s - M) l_s (M the largest m_s) and writes the normalised output
// columns of the slot to o.  Slot u of a lane holds output columns 32u + 4 grp + i and
// 32u + 16 + 4 grp + i (bf16 partials) or 16u + 4 grp + i (fp32), row r16 of the tile.
template <class AT, int DH, int SM>
__global__ __launch_bounds__(64) void k_attn_merge(Dims d, Bufs bf, int S) {
  constexpr int ES = sizeof(AT);
  constexpr int PAY = ES == 2 ? DH / 32 : DH / 16;
  constexpr uint32_t STRIDE = PAY * 1024 + 128;
  const int gq = d.Hq / d.Hkv, QT = (gq * d.H + 15) / 16;
  const int lane = threadIdx.x, r16 = lane & 15, grp = lane >> 4;
  const int u = blockIdx.x % PAY, item = blockIdx.x / PAY;  // one wave per (query tile, slot)
  if (item >= d.B * d.Hkv * QT) return;
  const int qt = item % QT, r = (item / QT) % d.Hkv, b = item / QT / d.Hkv;
  const int qrow = qt * 16 + r16;
  if (qrow >= gq * d.H) return;
  const int head = r * gq + qrow / d.H, m = b * d.H + qrow % d.H;
  const char* ws = reinterpret_cast<const char*>(bf.attn_ws) + (size_t)item * S * STRIDE;
  float ms[SM], ls[SM];
  u32x4 pv[SM];
#pragma unroll
  for (int s2 = 0; s2 < SM; ++s2) {
    const char* sp = ws + (size_t)min(s2, S - 1) * STRIDE;
    ms[s2] = *reinterpret_cast<const float*>(sp + PAY * 1024 + r16 * 4);
    ls[s2] = *reinterpret_cast<const float*>(sp + PAY * 1024 + 64 + r16 * 4);
    pv[s2] = *reinterpret_cast<const u32x4*>(sp + (u * 64 + lane) * 16);
  }
  float M = -INFINITY;
#pragma unroll
  for (int s2 = 0; s2 < SM; ++s2)
    if (s2 < S) M = fmaxf(M, ms[s2]);
  float den = 0.f;
  f32x4 acc[ES == 2 ? 2 : 1];
#pragma unroll
  for (int t = 0; t < (ES == 2 ? 2 : 1); ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s2 = 0; s2 < SM; ++s2) {
    const float wgt = s2 < S ? exp2f(ms[s2] - M) * ls[s2] : 0.f;
    den += wgt;
    if constexpr (ES == 2) {
      const bf16x8 pk = __builtin_bit_cast(bf16x8, pv[s2]);
      acc[0] += wgt * f32x4{(float)pk[0], (float)pk[1], (float)pk[2], (float)pk[3]};
      acc[1] += wgt * f32x4{(float)pk[4], (float)pk[5], (float)pk[6], (float)pk[7]};
    } else {
      acc[0] += wgt * __builtin_bit_cast(f32x4, pv[s2]);
    }
  }
  const float inv = 1.0f / den;
  const int qd = d.Hq * DH;
  AT* op = static_cast<AT*>(bf.o);
#pragma unroll
  for (int t = 0; t < (ES == 2 ? 2 : 1); ++t) {
    const int col = (ES == 2 ? 32 * u + 16 * t : 16 * u) + grp * 4;
    AT* dst = op + sw_idx(m, head * DH + col, qd);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = to_elem<AT>(acc[t][i] * inv);
  }
}

// ------------------------------------------------------------------ attention, many query rows
// The same split-key attention for batches and long joint sequences (hundreds to thousands
// of query rows per KV head): NW waves each own QPW query tiles and all of them share the
// staged key groups, so every staged K/V byte feeds NW*QPW tiles, and the group loads are
// spread over NW waves (the load rate of a workgroup grows with its wave count).  Groups
// are double-buffered: the loads of group g+1 are in flight (in registers) while group g
// is used, and land in the other LDS buffer afterwards.  bf16 only.
template <int DH, int NW, int QPW>
__global__ __launch_bounds__(64 * NW) void k_attn_wide(Dims d, Bufs bf, int layer, int S, int bps) {
  typedef bf16 AT;
  typedef typename FragOf<AT>::type Frag;
  constexpr int NB = DH <= 64 ? 4 : 2;   // 32-key blocks per group (registers: 2 waves per SIMD)
  constexpr int NK = NB * 32;
  constexpr int KROW = DH + 8;           // K row: DH + 16 B pad
  // V^T row: NK keys + 8 B pad.  The fragment reads are 8-byte pairs along a row at rows
  // r16 = 0..15; a row stride of 2 mod 32 dwords puts the 16 rows on distinct banks (a
  // 16-byte pad, 4 mod 32, paired rows r and r + 8: 40.5 -> 37.6 us per batch-32 launch).
  constexpr int VROW = NK + 4;
  constexpr int KCPR = DH / 8, VCPR = NK / 8;
  constexpr int KCH = NK * KCPR, VCH = DH * VCPR;
  constexpr int CPT = (KCH + VCH) / (64 * NW);
  static_assert((KCH + VCH) % (64 * NW) == 0, "group chunks split evenly over the threads");
  __shared__ __attribute__((aligned(16))) AT ks[2][NK * KROW];
  __shared__ __attribute__((aligned(16))) AT vs[2][DH * VROW];

  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gq = d.Hq / d.Hkv;
  const int QT = (gq * d.H + 15) / 16, QG = (QT + NW * QPW - 1) / (NW * QPW);
  // Consecutive workgroups go to different XCDs (round robin over 8); with a grid that is a
  // multiple of 8, each XCD takes a contiguous run of the ordinal order instead, so the key
  // splits and query groups of one (sample, KV head) share that XCD's L2 for their K/V.
  int idx = blockIdx.x;
  if ((gridDim.x & 7) == 0) idx = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int s = idx % S;
  idx /= S;
  const int qg = idx % QG;
  idx /= QG;
  const int r = idx % d.Hkv;
  const int b = idx / d.Hkv;
  const int T = d.P + d.H;
  const int nblk = (T + 31) / 32;
  const int blk0 = s * bps, blk1 = min(nblk, blk0 + bps);
  const int kend = min(T, blk1 * 32);
  const int qd = d.Hq * DH;

  const size_t kvbase = ((size_t)b * d.Lc + layer) * d.Hkv + r;
  const AT* Kc = static_cast<const AT*>(bf.kc) + kvbase * d.KS * DH;
  const AT* Vt = static_cast<const AT*>(bf.vt) + kvbase * DH * d.KS;

  int qt[QPW], head[QPW], mrow[QPW];
  bool active[QPW], qvalid[QPW];
  Frag qf[QPW][DH / 32];
#pragma unroll
  for (int p = 0; p < QPW; ++p) {
    qt[p] = (qg * NW + w) * QPW + p;
    active[p] = qt[p] < QT;
    const int qrow = qt[p] * 16 + r16;
    qvalid[p] = active[p] && qrow < gq * d.H;
    head[p] = r * gq + (qvalid[p] ? qrow / d.H : 0);
    const int tok = qvalid[p] ? qrow % d.H : 0;
    mrow[p] = b * d.H + tok;
    const AT* qp = static_cast<const AT*>(bf.q) + (size_t)mrow[p] * qd + head[p] * DH + grp * 8;
#pragma unroll
    for (int j = 0; j < DH / 32; ++j) qf[p][j] = load_frag(qp + 32 * j);
  }

  // group g0.. (blocks past the split are clamped to its last block: masked below)
  auto load_group = [&](int g0, u32x4 (&stage)[CPT]) {
    const int glast = min(blk1, g0 + NB) - 1;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 64 * NW * i;
      const char* src;
      if (c < KCH) {
        const int row = c / KCPR;
        const int blk = min(g0 + row / 32, glast);
        src = reinterpret_cast<const char*>(Kc + (size_t)(blk * 32 + row % 32) * DH) + (c % KCPR) * 16;
      } else {
        const int cv = c - KCH;
        const int row = cv / VCPR;
        const int kofs = (cv % VCPR) * 8;
        const int blk = min(g0 + kofs / 32, glast);
        src = reinterpret_cast<const char*>(Vt + (size_t)row * d.KS + blk * 32 + kofs % 32);
      }
      stage[i] = *reinterpret_cast<const u32x4*>(src);
    }
  };
  auto store_group = [&](const u32x4 (&stage)[CPT], int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 64 * NW * i;
      AT* dst = c < KCH ? ks[buf] + (c / KCPR) * KROW + (c % KCPR) * 8
                        : vs[buf] + ((c - KCH) / VCPR) * VROW + ((c - KCH) % VCPR) * 8;
      if (c < KCH) {
        *reinterpret_cast<u32x4*>(dst) = stage[i];
      } else {  // V^T rows are 8-byte aligned
        reinterpret_cast<u32x2*>(dst)[0] = u32x2{stage[i][0], stage[i][1]};
        reinterpret_cast<u32x2*>(dst)[1] = u32x2{stage[i][2], stage[i][3]};
      }
    }
  };

  const float sc = 1.4426950408889634f / sqrtf((float)DH);  // log2(e) / sqrt(dh)
  float m_run[QPW], l_part[QPW];
  f32x4 o[QPW][DH / 16];
#pragma unroll
  for (int p = 0; p < QPW; ++p) {
    m_run[p] = -INFINITY;
    l_part[p] = 0.f;
#pragma unroll
    for (int t = 0; t < DH / 16; ++t) o[p][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  PHASE_MARK(0);
  u32x4 stage[CPT];
  load_group(blk0, stage);
  store_group(stage, 0);
  __syncthreads();
  PHASE_MARK(1);
  int buf = 0;
  for (int g0 = blk0; g0 < blk1; g0 += NB) {
    const int glast = min(blk1, g0 + NB) - 1;
    const bool has_next = g0 + NB < blk1;
    if (has_next) load_group(g0 + NB, stage);
    const AT* kb_ = ks[buf];
    const AT* vb_ = vs[buf];
    // ---- scores of the group for every tile of the wave (K fragments shared)
    float sv[QPW][NB][8];
    float mx[QPW];
#pragma unroll
    for (int p = 0; p < QPW; ++p) mx[p] = -INFINITY;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      f32x4 s0[QPW], s1[QPW];
#pragma unroll
      for (int p = 0; p < QPW; ++p) s0[p] = s1[p] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (g0 + j <= glast) {
        // all K fragments of the block in flight before the first product, and the dh sum
        // as two interleaved chains per key half (even / odd 32-wide dh slices)
        Frag kf[DH / 32][2];
#pragma unroll
        for (int jj = 0; jj < DH / 32; ++jj) {
          kf[jj][0] = load_frag(kb_ + (j * 32 + r16) * KROW + 32 * jj + grp * 8);
          kf[jj][1] = load_frag(kb_ + (j * 32 + 16 + r16) * KROW + 32 * jj + grp * 8);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < QPW; ++p) {
          f32x4 e0 = {0.f, 0.f, 0.f, 0.f}, e1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int jj = 0; jj < DH / 32; jj += 2) {
            s0[p] = mma(kf[jj][0], qf[p][jj], s0[p]);
            s1[p] = mma(kf[jj][1], qf[p][jj], s1[p]);
            if (jj + 1 < DH / 32) {
              e0 = mma(kf[jj + 1][0], qf[p][jj + 1], e0);
              e1 = mma(kf[jj + 1][1], qf[p][jj + 1], e1);
            }
          }
          s0[p] += e0;
          s1[p] += e1;
        }
      }
      // raw scores (scaled inside the exponential), masked only in a block that straddles
      // the end of the split
      const int kb = (g0 + j) * 32 + grp * 4;
      if ((g0 + j) * 32 + 32 <= kend) {                // uniform: every key of the block valid
#pragma unroll
        for (int p = 0; p < QPW; ++p)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sv[p][j][i] = s0[p][i];
            sv[p][j][4 + i] = s1[p][i];
          }
      } else {
#pragma unroll
        for (int p = 0; p < QPW; ++p)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sv[p][j][i] = kb + i < kend ? s0[p][i] : -INFINITY;
            sv[p][j][4 + i] = kb + 16 + i < kend ? s1[p][i] : -INFINITY;
          }
      }
#pragma unroll
      for (int p = 0; p < QPW; ++p)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx[p] = fmaxf(mx[p], fmaxf(sv[p][j][i], sv[p][j][4 + i]));
    }
#pragma unroll
    for (int p = 0; p < QPW; ++p) {
      mx[p] = fmaxf(mx[p], __shfl_xor(mx[p], 16, 64));
      mx[p] = fmaxf(mx[p], __shfl_xor(mx[p], 32, 64));
      // reference max in log2 units, raised (with a rescale) only when exceeded by more than 8
      const float m_cand = fmaxf(m_run[p], mx[p] * sc);
      if (g0 == blk0) {
        m_run[p] = m_cand;
      } else if (__any(m_cand > m_run[p] + 8.f)) {
        const float alpha = fast_exp2(m_run[p] - m_cand);
        l_part[p] *= alpha;
#pragma unroll
        for (int t = 0; t < DH / 16; ++t) o[p][t] *= alpha;
        m_run[p] = m_cand;
      }
    }
    // ---- per key block: probabilities, then O^T += V^T P^T (V fragments shared)
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (g0 + j > glast) break;
      Frag pf[QPW];
#pragma unroll
      for (int p = 0; p < QPW; ++p)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = fast_exp2(fmaf(sv[p][j][e], sc, -m_run[p]));
          l_part[p] += pv;
          pf[p][e] = to_elem<AT>(pv);
        }
      // V fragments in batches of up to 8 (registers), each batch in flight before its products
      constexpr int VB = DH / 16 < 8 ? DH / 16 : 8;
#pragma unroll
      for (int t0 = 0; t0 < DH / 16; t0 += VB) {
        Frag vf[VB];
#pragma unroll
        for (int t = 0; t < VB; ++t) {
          const AT* vp = vb_ + ((t0 + t) * 16 + r16) * VROW + j * 32 + grp * 4;
          vf[t] = load_frag_split4(vp, vp + 16);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < VB; ++t)
#pragma unroll
          for (int p = 0; p < QPW; ++p) o[p][t0 + t] = mma(vf[t], pf[p], o[p][t0 + t]);
      }
    }
    if (has_next) store_group(stage, buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  PHASE_MARK(2);
#pragma unroll
  for (int p = 0; p < QPW; ++p)
    if (active[p])
      attn_finish<AT, DH>(d, bf, o[p], m_run[p], l_part[p], S, s, (size_t)(b * d.Hkv + r) * QT + qt[p], qvalid[p],
                          mrow[p], head[p], false);
}

// ------------------------------------------------------------------ out-projection + Euler + in-projection
// k_prev >= 0: final adaptive norm of step k_prev, v = rinv (hs W_out^T) + W_out shift +
// b_out, x += dt v.  k_next >= 0: in-projection h = x W_in^T + b_in for step k_next,
// writing h, hs = h * (1 + scale) of that step's first norm, and the rows' sum-of-squares
// partials.  One 16-row tile (the row tile of the swizzled activations) per workgroup, so
// that the io weights are read once per 16 rows.  Out-projection
// on MFMA (the bf16 or fp32 activations and weights, fp32 accumulation): the four waves
// take the k-blocks round robin and their products are added in wave order; the update
// and the in-projection (fp32, x from LDS, one output column per thread and pass) follow.
// With few row tiles the in-projection's columns are split over `cs` workgroups per tile
// (workgroup = tile * cs + c); each recomputes the tile's update (the out-projection is
// small).  The state may be overwritten only once every workgroup of the tile has read it:
// each arrives on the tile's counter after its reads, and the last to arrive writes it.
template <class AT, class IOT>
__global__ __launch_bounds__(256) void k_out_rows(Dims d, Bufs bf, int k_prev, int k_next, int cs) {
  typedef typename FragOf<AT>::type AF;
  typedef typename FragOf<IOT>::type WF;
  __shared__ float xs[16][257];
  __shared__ f32x4 red[4][16][64];
  __shared__ float rinv_s[16];
  __shared__ unsigned last_s;
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rt = blockIdx.x / cs, cpart = blockIdx.x - rt * cs, m0 = rt * 16;
  const int nta = (d.A + 15) / 16;  // 16-column output tiles of the out-projection (A <= 256)
  PHASE_MARK(0);
  if (k_prev >= 0) {
    {  // final-norm statistics of the tile's rows: 16 threads per row
      const int r = tid >> 4, j0 = tid & 15, m = min(m0 + r, d.M - 1), n16 = d.D / 16;
      float ss = 0.f;
      for (int j = j0; j < n16; j += 16) ss += bf.ssq[(size_t)m * n16 + j];
      ss = sum16(ss);
      if (j0 == 0) rinv_s[r] = 1.0f / sqrtf(ss / (float)d.D + d.eps);
    }
    PHASE_MARK(1);
    const AT* hs = static_cast<const AT*>(bf.hs);
    const IOT* wo = static_cast<const IOT*>(bf.w_out);
    const int kbn = d.D / 32;
    for (int nt0 = 0; nt0 < nta; nt0 += 2) {  // two output tiles at a time
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      for (int kb0 = w; kb0 < kbn; kb0 += 32) {  // this wave's k-blocks kb0 + 4 i, all loads in flight
        AF af[8];
        WF wf[2][8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int kb = min(kb0 + 4 * i, kbn - 1);
          af[i] = load_frag(hs + sw_frag(rt, kb, d.D, lane));
#pragma unroll
          for (int j = 0; j < 2; ++j)
            wf[j][i] = load_frag(wo + (size_t)min((nt0 + j) * 16 + r16, d.A - 1) * d.D + kb * 32 + grp * 8);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            if (kb0 + 4 * i < kbn) acc[j] = mma(af[i], (nt0 + j) * 16 + r16 < d.A ? wf[j][i] : zero_frag<IOT>(), acc[j]);
      }
      red[w][nt0][lane] = acc[0];
      if (nt0 + 1 < nta) red[w][nt0 + 1][lane] = acc[1];
    }
    PHASE_MARK(2);
    __syncthreads();
    const IOT* bo = static_cast<const IOT*>(bf.b_out);
    const float* cv = bf.cvec + (size_t)k_prev * bf.cv_stride + bf.cv_out_off;
    const float dt = bf.dt[k_prev];
    for (int e = tid; e < 16 * 256; e += 256) xs[e >> 8][e & 255] = 0.f;  // columns past A stay zero
    __syncthreads();
    for (int e = tid; e < nta * 64; e += 256) {
      const int nt = e >> 6, l = e & 63, a = nt * 16 + (l & 15);
      const f32x4 s = ((red[0][nt][l] + red[1][nt][l]) + red[2][nt][l]) + red[3][nt][l];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * (l >> 4) + i, m = m0 + r;
        if (m < d.M && a < d.A) {
          const float v = rinv_s[r] * s[i] + cv[a] + to_f32(bo[a]);
          const float xn = bf.x[(size_t)m * d.A + a] + dt * v;
          xs[r][a] = xn;
          if (cs == 1) bf.x[(size_t)m * d.A + a] = xn;
        }
      }
    }
    __syncthreads();
  } else {
    for (int e = tid; e < 16 * 256; e += 256) {
      const int r = e >> 8, a = e & 255, m = m0 + r;
      xs[r][a] = (m < d.M && a < d.A) ? bf.x[(size_t)m * d.A + a] : 0.f;
    }
    __syncthreads();
  }
  PHASE_MARK(3);
  const bool split_x = k_prev >= 0 && cs > 1;
  unsigned arrived = 0;
  if (split_x && tid == 0)  // every thread's reads of the state are done (barrier above)
    arrived = __hip_atomic_fetch_add(bf.gemm_cnt + rt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  auto write_state = [&]() {
    if (!split_x) return;
    if (tid == 0) {
      last_s = arrived == (unsigned)cs - 1 ? 1u : 0u;
      if (last_s) __hip_atomic_store(bf.gemm_cnt + rt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last_s) return;
    for (int e = tid; e < 16 * d.A; e += 256) {
      const int r = e / d.A, a = e - r * d.A, m = m0 + r;
      if (m < d.M) bf.x[(size_t)m * d.A + a] = xs[r][a];
    }
  };
  if (k_next < 0) {
    write_state();
    return;
  }
  // in-projection on fp32 MFMA (exact products of the fp32 state and the weights):
  // H = X W_in^T + b_in, one 16 x 16 output tile per MFMA chain, K = A in 32-wide chunks
  // (columns past A are zero in xs and in the weight fragments)
  const IOT* wi = static_cast<const IOT*>(bf.w_in);
  const IOT* bi = static_cast<const IOT*>(bf.b_in);
  const float* scl = bf.mod + (size_t)k_next * d.nmod * 2 * d.D;  // norm 0, scale row
  AT* hsw = static_cast<AT*>(bf.hs);
  const int kc_n = (d.A + 31) / 32, ntn = d.D / 16;
  // this workgroup's column tiles: [ntb, nte), four of a wave's (nt0 + 4 j) at a time
  const int ntb = cpart * (ntn / cs), nte = ntb + ntn / cs;
  for (int nt0 = ntb + w; nt0 < nte; nt0 += 16) {
    f32x4 acc[4];
    float b0[4], sc1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kc = 0; kc < kc_n; ++kc) {
      const int a0 = kc * 32 + grp * 8;
      WF wv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = min(nt0 + 4 * j, nte - 1) * 16 + r16;
        wv[j] = load_frag(wi + (size_t)n * d.A + min(a0, d.A - 8));
        if (kc == 0) {  // the epilogue's bias and scale, with the first weights
          b0[j] = to_f32(bi[n]);
          sc1[j] = 1.0f + scl[n];
        }
      }
      f32x8 xa;
#pragma unroll
      for (int e = 0; e < 8; ++e) xa[e] = xs[r16][a0 + e];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x8 wb;
#pragma unroll
        for (int e = 0; e < 8; ++e) wb[e] = a0 < d.A ? to_f32(wv[j][e]) : 0.f;
        acc[j] = mma(xa, wb, acc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nt = nt0 + 4 * j;
      if (nt >= nte) break;
      const int n = nt * 16 + r16;
      // acc[j][i]: row 4 grp + i, column n
      float hn[4], sq[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hn[i] = acc[j][i] + b0[j];
        sq[i] = sum16(hn[i] * hn[i]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 4 * grp + i;
        if (m < d.M) {
          bf.h[(size_t)m * d.D + n] = hn[i];
          hsw[sw_idx(m, n, d.D)] = to_elem<AT>(hn[i] * sc1[j]);
          if (r16 == 0) bf.ssq[(size_t)m * (d.D / 16) + nt] = sq[i];
        }
      }
    }
  }
  write_state();
  PHASE_MARK(7);
}

// ------------------------------------------------------------------ joint denoiser: guidance + Euler
// Joint video/action denoiser (PhyAI reading, Figure 4: conditional and unconditional
// branches combined by the guidance scale, then every rank advances its video/action
// state).  Rows [0, H) of every activation hold the conditional branch (modulation
// table 0), rows [H, 2H) the unconditional one (table 1); token t < Tl is a latent
// token (Cl channels, latent projections), the rest action tokens (A dims).
// k_prev >= 0: both branches' final norm and out-projection, v = v_u + gamma (v_c - v_u),
// z += dt v (or the UniPC update).  k_next >= 0: in-projection of z (identical for both
// branches), hs of each branch with its own first-norm scale, row statistics.  One 16-token
// tile per workgroup (tokens of one kind: latent tiles first, then action tiles; the last
// tile of a kind may be ragged), so that the io projections are read once per 16 tokens:
// the out-projection of both branches on MFMA (the four waves take the k-blocks round
// robin, products added in wave order), the guided update per element, and the
// in-projection on fp32 MFMA.  Token dims up to 256, four 16-column output tiles per pass
// of the out-projection.
template <class AT, class IOT>
__global__ __launch_bounds__(256) void k_wam_rows(Dims d, Bufs bf, int k_prev, int k_next) {
  typedef typename FragOf<AT>::type AF;
  typedef typename FragOf<IOT>::type WF;
  constexpr int NTC = 4;  // 16-column output tiles per pass (both branches: 8 products)
  __shared__ float xs[16][257];
  __shared__ f32x4 red[4][2 * NTC][64];
  __shared__ float rinv_s[2][16];
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntl = (d.Tl + 15) / 16;
  const bool lat = (int)blockIdx.x < ntl;
  const int t0 = lat ? blockIdx.x * 16 : d.Tl + ((int)blockIdx.x - ntl) * 16;
  const int tend = lat ? d.Tl : d.H;  // end of this kind's tokens
  const int dim = lat ? d.Cl : d.A;
  const int ntd = (dim + 15) / 16;
  const IOT* wo = static_cast<const IOT*>(lat ? bf.w_out : bf.w_out2);
  const IOT* bo = static_cast<const IOT*>(lat ? bf.b_out : bf.b_out2);
  const IOT* wi = static_cast<const IOT*>(lat ? bf.w_in : bf.w_in2);
  const IOT* bi = static_cast<const IOT*>(lat ? bf.b_in : bf.b_in2);
  // state of token t, channel a
  auto zptr = [&](int t) { return lat ? bf.x + (size_t)t * d.Cl : bf.x2 + (size_t)(t - d.Tl) * d.A; };
  for (int e = tid; e < 16 * 256; e += 256) xs[e >> 8][e & 255] = 0.f;  // channels past dim stay zero
  __syncthreads();
  if (k_prev >= 0) {
    {  // final-norm statistics of the 32 rows (2 branches x 16 tokens), 16 threads per row
      const int n16 = d.D / 16;
      for (int rr = tid >> 4; rr < 32; rr += 16) {
        const int br = rr >> 4, t = min(t0 + (rr & 15), tend - 1), m = br * d.H + t;
        float ss = 0.f;
        for (int j = tid & 15; j < n16; j += 16) ss += bf.ssq[(size_t)m * n16 + j];
        ss = sum16(ss);
        if ((tid & 15) == 0) rinv_s[br][rr & 15] = 1.0f / sqrtf(ss / (float)d.D + d.eps);
      }
    }
    const AT* hs = static_cast<const AT*>(bf.hs);
    const int kbn = d.D / 32;
    const int trow = min(t0 + r16, tend - 1);
    for (int nc = 0; nc < ntd; nc += NTC) {  // output tiles [nc, nc + nn) of both branches
      const int nn = min(NTC, ntd - nc);
      for (int bt = 0; bt < 2 * nn; ++bt) {
        const int br = bt / nn, nt = nc + bt - br * nn;
        const int m = br * d.H + trow;
        const int a = min(nt * 16 + r16, dim - 1);
        const bool av = nt * 16 + r16 < dim;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int kb0 = w; kb0 < kbn; kb0 += 32) {
          AF af[8];
          WF wf[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int kb = min(kb0 + 4 * i, kbn - 1);
            af[i] = load_frag(hs + sw_idx(m, kb * 32 + grp * 8, d.D));
            wf[i] = load_frag(wo + (size_t)a * d.D + kb * 32 + grp * 8);
          }
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (kb0 + 4 * i < kbn) acc = mma(af[i], av ? wf[i] : zero_frag<IOT>(), acc);
        }
        red[w][bt][lane] = acc;
      }
      __syncthreads();
      const int ca = min(dim - nc * 16, NTC * 16);  // channels of this pass
      for (int e = tid; e < 16 * ca; e += 256) {
        const int r = e / ca, a = nc * 16 + (e - r * ca), t = t0 + r;
        if (t >= tend) continue;
        const int nt = (a >> 4) - nc, l = (r >> 2) * 16 + (a & 15), i = r & 3;
        const int ooff = bf.cv_out_off + (lat ? 0 : d.Cl) + a;
        float v[2];
#pragma unroll
        for (int br = 0; br < 2; ++br) {
          const int bt = br * nn + nt;
          const float sum = ((red[0][bt][l][i] + red[1][bt][l][i]) + red[2][bt][l][i]) + red[3][bt][l][i];
          const float* cv = bf.cvec + ((size_t)k_prev * d.ntab + br) * bf.cv_stride;
          v[br] = rinv_s[br][r] * sum + cv[ooff] + to_f32(bo[a]);
        }
        const float vg = v[1] + d.gamma * (v[0] - v[1]);
        float* z = zptr(t);
        float zn;
        if (d.solver) {  // UniPC: corrector of the step into k_prev, then the predictor out of it
          const float* cf = bf.uni + (size_t)k_prev * 8;
          const size_t ne = (size_t)d.Tl * d.Cl + (size_t)(d.H - d.Tl) * d.A;
          const size_t el = lat ? (size_t)t * d.Cl + a : (size_t)d.Tl * d.Cl + (size_t)(t - d.Tl) * d.A + a;
          float* xp = bf.ust;                                          // corrected z_{k-1} -> z_k
          float* m_new = bf.ust + ne * (1 + (k_prev & 1));             // holds m_{k-2}, takes m_k
          const float* m_km1 = bf.ust + ne * (1 + ((k_prev + 1) & 1));  // m_{k-1}
          const float zk = z[a];
          const float mm = zk - cf[0] * vg;
          float xc = zk, m1 = 0.f;
          if (k_prev >= 1) {
            m1 = m_km1[el];
            const float m2 = k_prev >= 2 ? m_new[el] : 0.f;
            xc = cf[1] * xp[el] + cf[2] * mm + cf[3] * m1 + cf[4] * m2;
          }
          zn = cf[5] * xc + cf[6] * mm + cf[7] * m1;
          xp[el] = xc;
          m_new[el] = mm;
        } else {
          zn = z[a] + bf.dt[k_prev] * vg;
        }
        z[a] = zn;
        xs[r][a] = zn;
      }
      __syncthreads();  // red is reused by the next pass; xs complete for the in-projection
    }
  } else {
    for (int e = tid; e < 16 * dim; e += 256) {
      const int r = e / dim, a = e - r * dim, t = t0 + r;
      if (t < tend) xs[r][a] = zptr(t)[a];
    }
    __syncthreads();
  }
  if (k_next < 0) return;
  // in-projection (identical for both branches) on fp32 MFMA; hs of each branch with its
  // own first-norm scale; the same row statistics for both rows
  AT* hsw = static_cast<AT*>(bf.hs);
  const size_t stab = (size_t)d.nmod * 2 * d.D;
  const float* scl = bf.mod + (size_t)k_next * d.ntab * stab;  // table 0, norm 0, scale row
  const int kc_n = (dim + 31) / 32, ntn = d.D / 16;
  for (int nt0 = w; nt0 < ntn; nt0 += 16) {
    f32x4 acc[4];
    float b0[4], s0[4], s1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kc = 0; kc < kc_n; ++kc) {
      const int a0 = kc * 32 + grp * 8;
      WF wv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = min(nt0 + 4 * j, ntn - 1) * 16 + r16;
        wv[j] = load_frag(wi + (size_t)n * dim + min(a0, dim - 8));
        if (kc == 0) {
          b0[j] = to_f32(bi[n]);
          s0[j] = 1.0f + scl[n];
          s1[j] = 1.0f + scl[stab + n];
        }
      }
      f32x8 xa;
#pragma unroll
      for (int e = 0; e < 8; ++e) xa[e] = xs[r16][min(a0 + e, 255)];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x8 wb;
#pragma unroll
        for (int e = 0; e < 8; ++e) wb[e] = a0 < dim ? to_f32(wv[j][e]) : 0.f;
        acc[j] = mma(xa, wb, acc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nt = nt0 + 4 * j;
      if (nt >= ntn) break;
      const int n = nt * 16 + r16;
      float hn[4], sq[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hn[i] = acc[j][i] + b0[j];
        sq[i] = sum16(hn[i] * hn[i]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * grp + i;
        if (t >= tend) continue;
#pragma unroll
        for (int br = 0; br < 2; ++br) {
          const int m = br * d.H + t;
          bf.h[(size_t)m * d.D + n] = hn[i];
          hsw[sw_idx(m, n, d.D)] = to_elem<AT>(hn[i] * (br ? s1[j] : s0[j]));
          if (r16 == 0) bf.ssq[(size_t)m * (d.D / 16) + nt] = sq[i];
        }
      }
    }
  }
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

// Query tiles per workgroup of the many-row attention kernel (8 waves x tiles per wave).
static int attn_wide_tiles(int dh) { return dh <= 128 ? 16 : 8; }

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

template <class AT, class WT, int EPI, int NT, int MT>
static hipError_t launch_gemm_q(const Dims& d, const Bufs& b, const GemmLaunch& g, int tiles, hipStream_t st) {
  const int kbs = g.K / 32 / g.S;        // k-blocks per split (a multiple of 4), shared by 4 waves
  // every wave owns exactly kbw k-blocks; int4 waves own whole 128-wide quads (one scale
  // group each), so splits of fewer than four quads leave the surplus waves idle
  const int qps = kbs / 4;
  const int kbw = __is_same(WT, i4) ? (qps >= 4 ? qps : 4) : qps;
  if (__is_same(WT, i4) && qps > 4 && qps % 4) return hipErrorInvalidValue;
  dim3 grid(tiles * g.S), block(256);
  switch (kbw) {
    case 1: hipLaunchKernelGGL((k_gemm<AT, WT, MT, NT, 1, EPI>), grid, block, 0, st, g.W, g.A, g.K, g.S, g.n_second, d, b, g); break;
    case 2: hipLaunchKernelGGL((k_gemm<AT, WT, MT, NT, 2, EPI>), grid, block, 0, st, g.W, g.A, g.K, g.S, g.n_second, d, b, g); break;
    case 4: hipLaunchKernelGGL((k_gemm<AT, WT, MT, NT, 4, EPI>), grid, block, 0, st, g.W, g.A, g.K, g.S, g.n_second, d, b, g); break;
    case 8: hipLaunchKernelGGL((k_gemm<AT, WT, MT, NT, 8, EPI>), grid, block, 0, st, g.W, g.A, g.K, g.S, g.n_second, d, b, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class AT, class WT, int EPI, int NT>
static hipError_t launch_gemm(const Dims& d, const Bufs& b, const GemmLaunch& g, int tiles, hipStream_t st) {
  if constexpr (!__is_same(AT, bf16) || !__is_same(WT, bf16)) {
    if (d.M > 64) return hipErrorInvalidValue;  // many rows: bf16 only (tiled family)
  }
  switch ((d.M + 15) / 16) {
    case 1: return launch_gemm_q<AT, WT, EPI, NT, 1>(d, b, g, tiles, st);
    case 2: return launch_gemm_q<AT, WT, EPI, NT, 2>(d, b, g, tiles, st);
    case 3: return launch_gemm_q<AT, WT, EPI, NT, 3>(d, b, g, tiles, st);
    case 4: return launch_gemm_q<AT, WT, EPI, NT, 4>(d, b, g, tiles, st);
  }
  return hipErrorInvalidValue;
}

template <class AT>
static hipError_t launch_attn_merge(const Dims& d, const Bufs& b, int S, hipStream_t st) {
  const int QT = ((d.Hq / d.Hkv) * d.H + 15) / 16;
  const int pay = sizeof(AT) == 2 ? d.dh / 32 : d.dh / 16;
  dim3 mgrid(d.B * d.Hkv * QT * pay), mblock(64);
#define PHYAI_MERGE(DH)                                                                          \
  if (S > 16) hipLaunchKernelGGL((k_attn_merge<AT, DH, 32>), mgrid, mblock, 0, st, d, b, S);      \
  else hipLaunchKernelGGL((k_attn_merge<AT, DH, 16>), mgrid, mblock, 0, st, d, b, S);
  switch (d.dh) {
    case 32: PHYAI_MERGE(32) break;
    case 64: PHYAI_MERGE(64) break;
    case 128: PHYAI_MERGE(128) break;
    case 256: PHYAI_MERGE(256) break;
    default: return hipErrorInvalidValue;
  }
#undef PHYAI_MERGE
  return hipGetLastError();
}

// part 0: the attention kernel; part 1: the merge of its key splits (a launch only for the
// few-row kernel with more than one split).
template <class AT>
static hipError_t launch_attn_part(const Dims& d, const Bufs& b, const Plan& p, int layer, int part,
                                   hipStream_t st) {
  const int T = d.P + d.H, nblk = (T + 31) / 32;
  const int S = (nblk + p.attn_bps - 1) / p.attn_bps;
  const int QT = ((d.Hq / d.Hkv) * d.H + 15) / 16;
  if constexpr (sizeof(AT) == 2) {
    if (p.attn_wide) {
      if (part) return hipSuccess;                    // merged in-kernel
      const int tpw = attn_wide_tiles(d.dh);
      dim3 grid(d.B * d.Hkv * ((QT + tpw - 1) / tpw) * S), block(512);
      switch (d.dh) {
        case 32: hipLaunchKernelGGL((k_attn_wide<32, 8, 2>), grid, block, 0, st, d, b, layer, S, p.attn_bps); break;
        case 64: hipLaunchKernelGGL((k_attn_wide<64, 8, 2>), grid, block, 0, st, d, b, layer, S, p.attn_bps); break;
        case 128: hipLaunchKernelGGL((k_attn_wide<128, 8, 2>), grid, block, 0, st, d, b, layer, S, p.attn_bps); break;
        case 256: hipLaunchKernelGGL((k_attn_wide<256, 8, 1>), grid, block, 0, st, d, b, layer, S, p.attn_bps); break;
        default: return hipErrorInvalidValue;
      }
      return hipGetLastError();
    }
  }
  if (S > 32) return hipErrorInvalidValue;
  if (part) return S > 1 ? launch_attn_merge<AT>(d, b, S, st) : hipSuccess;
  const int QG = (QT + 3) / 4;
  dim3 grid(d.B * d.Hkv * QG * (S > 16 ? 32 : S > 8 ? 16 : 8));  // 8, 16 or 32 split slots per query group
  // blocks staged per group: one or two when a split has that many (four would not always
  // fit LDS); a single block is run by one wave per query tile
  const int nb = p.attn_bps == 1 ? 1 : (p.attn_bps <= 2 || d.dh * (int)sizeof(AT) > 512) ? 2 : 4;
#define PHYAI_ATTN(DH)                                                                                        \
  if (nb == 1) hipLaunchKernelGGL((k_attn<AT, DH, 1>), grid, dim3(256), 0, st, d, b, layer, S, p.attn_bps);    \
  else if (nb == 2) hipLaunchKernelGGL((k_attn<AT, DH, 2>), grid, dim3(512), 0, st, d, b, layer, S, p.attn_bps); \
  else hipLaunchKernelGGL((k_attn<AT, DH, (DH * sizeof(AT) <= 512 ? 4 : 2)>), grid, dim3(512), 0, st, d, b, layer, \
                          S, p.attn_bps);
  switch (d.dh) {
    case 32: PHYAI_ATTN(32) break;
    case 64: PHYAI_ATTN(64) break;
    case 128: PHYAI_ATTN(128) break;
    case 256: PHYAI_ATTN(256) break;
    default: return hipErrorInvalidValue;
  }
#undef PHYAI_ATTN
  return hipGetLastError();
}

template <class T> static size_t wbytes_row(int K);
template <> size_t wbytes_row<float>(int K) { return (size_t)K * 4; }
template <> size_t wbytes_row<bf16>(int K) { return (size_t)K * 2; }
template <> size_t wbytes_row<i4>(int K) { return (size_t)K / 2; }

// One launch of kernel `which` for (step k, layer l).  Kinds: 0 QKV, 1 attention,
// 7 merge of the attention's key splits (no launch when there is none), 2 O + residual,
// 3 gate/up GeGLU, 4 down + residual, 5 out-projection/Euler/in-projection (layer
// ignored), 6 in-projection of step 0 (layer ignored).  A layer runs kLayerOrder.
static constexpr int kLayerOrder[6] = {0, 1, 7, 2, 3, 4};
template <class AT, class WT, class IOT>
static hipError_t launch_one(const Dims& d, const Bufs& b, const Plan& p, int which, int k, int l,
                             hipStream_t st) {
  const int qd = d.Hq * d.dh;
  const float* cv = b.cvec + (size_t)k * b.cv_stride;
  GemmLaunch g{};
  g.layer = l;
  switch (which) {
    case 0:
      g.A = b.hs; g.lda = d.D; g.K = d.D;
      g.W = static_cast<const char*>(b.w_qkv) + wbytes_row<WT>(d.D) * d.qkv * l;
      g.Ws = b.s_qkv ? b.s_qkv + (size_t)l * d.qkv * (d.D / 128) : nullptr;
      g.S = p.s_qkv; g.cvec = cv + (size_t)l * d.qkv;
      if (d.M > 64) return launch_gemm_tiled(d, b, g, EPI_QKV, d.qkv, st);
      return launch_gemm<AT, WT, EPI_QKV, 1>(d, b, g, d.qkv / 16, st);
    case 1:
      return launch_attn_part<AT>(d, b, p, l, 0, st);
    case 7:
      return launch_attn_part<AT>(d, b, p, l, 1, st);
    case 2:  // consumer of h is the MLP norm 2l+1
      g.A = b.o; g.lda = qd; g.K = qd;
      g.W = static_cast<const char*>(b.w_o) + wbytes_row<WT>(qd) * d.D * l;
      g.Ws = b.s_o ? b.s_o + (size_t)l * d.D * (qd / 128) : nullptr;
      g.S = p.s_o; g.scale_next = b.mod + (((size_t)k * d.nmod + 2 * l + 1) * 2) * d.D;
      g.gate = b.gate ? b.gate + ((size_t)k * d.nmod + 2 * l) * d.D : nullptr;  // attention block of layer l
      if (d.M > 64) return launch_gemm_tiled(d, b, g, EPI_RESID, d.D, st);
      return launch_gemm<AT, WT, EPI_RESID, 1>(d, b, g, d.D / 16, st);
    case 3:
      g.A = b.hs; g.lda = d.D; g.K = d.D;
      g.W = static_cast<const char*>(b.w_gu) + wbytes_row<WT>(d.D) * 2 * d.F * l;
      g.Ws = b.s_gu ? b.s_gu + (size_t)l * 2 * d.F * (d.D / 128) : nullptr;
      g.n_second = d.F; g.S = p.s_gu; g.cvec = cv + b.cv_gu_off + (size_t)l * 2 * d.F;
      if (d.M > 64) return launch_gemm_tiled(d, b, g, EPI_GEGLU, 2 * d.F, st);
      return launch_gemm<AT, WT, EPI_GEGLU, 2>(d, b, g, d.F / 16, st);
    case 4: {  // consumer of h is norm 2(l+1), or the final norm 2L
      g.A = b.act; g.lda = d.F; g.K = d.F;
      g.W = static_cast<const char*>(b.w_d) + wbytes_row<WT>(d.F) * d.D * l;
      g.Ws = b.s_d ? b.s_d + (size_t)l * d.D * (d.F / 128) : nullptr;
      g.S = p.s_d;
      const int jn = (l + 1 < d.L) ? 2 * (l + 1) : 2 * d.L;
      g.scale_next = b.mod + (((size_t)k * d.nmod + jn) * 2) * d.D;
      g.gate = b.gate ? b.gate + ((size_t)k * d.nmod + 2 * l + 1) * d.D : nullptr;  // MLP block of layer l
      if (d.M > 64) return launch_gemm_tiled(d, b, g, EPI_RESID, d.D, st);
      return launch_gemm<AT, WT, EPI_RESID, 1>(d, b, g, d.D / 16, st);
    }
    case 5:
    case 6: {
      // column splits of the in-projection: about 128 workgroups, at least 4 column tiles each
      const int tiles = (d.M + 15) / 16;
      int cs = 1;
      if (b.gemm_cnt && (size_t)tiles <= gemm_counters(d))  // the tiles' arrival counters
        while (tiles * cs * 2 <= 128 && (d.D / 16) % (cs * 2) == 0 && d.D / 16 / (cs * 2) >= 4) cs *= 2;
      if (which == 5)
        hipLaunchKernelGGL((k_out_rows<AT, IOT>), dim3(tiles * cs), dim3(256), 0, st, d, b, k, k + 1 < d.N ? k + 1 : -1,
                           cs);
      else
        hipLaunchKernelGGL((k_out_rows<AT, IOT>), dim3(tiles * cs), dim3(256), 0, st, d, b, -1, 0, cs);
      return hipGetLastError();
    }
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

// ------------------------------------------------------------------ prefix prefill
// The prefix rows enter the layer stack as given (no in-projection): h = tokens, hs = h (the
// prefix network's norm is a plain RMSNorm: zero scale and shift) and the row statistics.
// One workgroup per token row.
template <class AT, class IOT>
__global__ __launch_bounds__(256) void k_prefill_in(Dims d, Bufs bf, const IOT* tokens) {
  const int m = blockIdx.x, tid = threadIdx.x;
  AT* hs = static_cast<AT*>(bf.hs);
  for (int n0 = 0; n0 < d.D; n0 += 256) {
    const int n = n0 + tid;  // D % 256 == 0: every thread has a column
    const float v = to_f32(tokens[(size_t)m * d.D + n]);
    bf.h[(size_t)m * d.D + n] = v;
    hs[sw_idx(m, n, d.D)] = to_elem<AT>(v);
    const float sq = sum16(v * v);
    if ((tid & 15) == 0) bf.ssq[(size_t)m * (d.D / 16) + n / 16] = sq;
  }
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
  hipLaunchKernelGGL((k_prefill_in<AT, AT>), dim3(d.M), dim3(256), 0, st, d, b, static_cast<const AT*>(tokens));
  hipError_t e = hipGetLastError();
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
      return launch_attn_part<bf16>(d, b, p, 0, 0, st);
    case 7:
      return launch_attn_part<bf16>(d, b, p, 0, 1, st);
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
      hipLaunchKernelGGL((k_wam_rows<bf16, bf16>), dim3((d.Tl + 15) / 16 + (d.H - d.Tl + 15) / 16), dim3(256), 0, st, d,
                         b, k, k + 1 < d.N ? k + 1 : -1);
      return hipGetLastError();
    case 6:
      hipLaunchKernelGGL((k_wam_rows<bf16, bf16>), dim3((d.Tl + 15) / 16 + (d.H - d.Tl + 15) / 16), dim3(256), 0, st, d,
                         b, -1, 0);
      return hipGetLastError();
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

#ifdef PHYAI_PHASE_TRACE
// Phase-trace build only: copy the per-wave timestamps out (host dst of 4096*4*8 uint64),
// then clear them.
extern "C" int phyai_phase_trace(void* host_dst) {
  static uint64_t zeros[4096 * 4 * 8];
  if (hipMemcpyFromSymbol(host_dst, HIP_SYMBOL(phyai::g_phase_trace), sizeof(zeros), 0, hipMemcpyDeviceToHost) !=
          hipSuccess ||
      hipMemcpyToSymbol(HIP_SYMBOL(phyai::g_phase_trace), zeros, sizeof(zeros), 0, hipMemcpyHostToDevice) != hipSuccess)
    return 4;
  return 0;
}
#endif
