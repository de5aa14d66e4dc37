// Weight-streaming GEMMs of the Euler loop for few token rows (batch x chunk <= 64), gfx950:
// the QKV (norm folded, chunk K/V into the cache), output-projection + residual, gate/up +
// GeGLU and down-projection + residual linears, bf16, fp32 or int4-g128 weights.
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
#include "launch.h"

#include <math.h>

#include <algorithm>
#include <type_traits>

namespace phyai {

#ifdef PHYAI_PHASE_TRACE
PHYAI_PHASE_TRACE_READER(phyai_phase_trace_gemv)
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

// A weight fragment read with the non-temporal policy (buffer load, nt), through resource r
// over the weights at base: for weights that the caches should not keep (bf16; fp32 weights
// take the plain load).
__device__ __forceinline__ bf16x8 load_frag_nt(__amdgpu_buffer_rsrc_t r, const bf16* base, const bf16* p) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)((p - base) * 2), 0, 2));
}
__device__ __forceinline__ f32x8 load_frag_nt(__amdgpu_buffer_rsrc_t, const float*, const float* p) { return load_frag(p); }

// ------------------------------------------------------------------ weight-streaming GEMM
// The operands that the weight and activation loads need (W, A, K, log2 of the split
// count, second row block, k-blocks per split, non-temporal weights) lead the argument list
// as scalars: they are preloaded into SGPRs at wave launch, so the loads wait neither for
// the kernel-argument fetch nor for an integer division.  wnt: the weights are read with the
// non-temporal policy (this layer's weights are not meant to stay in the memory-side cache
// until the next step; see resident_weight_layers).
template <class AT, class WT, int MT, int NT, int KBW, int EPI>
__global__ __launch_bounds__(256) void k_gemm(const void* Wp, const void* Ap, int Kp, int slog, int nsec, int kbs,
                                              int wnt, Dims d, Bufs bf, GemmLaunch g) {
  constexpr bool NORM = (EPI == EPI_QKV || EPI == EPI_GEGLU);
  constexpr bool INT4 = __is_same(WT, i4);
  __shared__ f32x4 red[4][NT][MT][64];
  __shared__ float rinv_s[64];
  __shared__ unsigned flag;
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int s = blockIdx.x & ((1 << slog) - 1), tile = blockIdx.x >> slog;
  int nrow[NT];
  nrow[0] = tile * 16;
  if (NT == 2) nrow[NT - 1] = nsec + tile * 16;

  PHASE_MARK(0);
  // this wave's k-blocks: [kbeg, min(kbeg + KBW, kend)), contiguous
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
    if constexpr (!INT4) {
      // every weight fragment of the wave, then the activations (one branch per policy, so
      // that each load's cache policy is a constant)
      auto load_w = [&](auto ntc) {
        constexpr bool NTL = decltype(ntc)::value;
        const __amdgpu_buffer_rsrc_t wr =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(Wp), (short)0, 0x7fffffff, 0x00020000);
#pragma unroll
        for (int i = 0; i < KBW; ++i)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const WT* p = static_cast<const WT*>(Wp) + sw_frag(nrow[nt] >> 4, kbeg + i, Kp, lane);
            wf[i][nt] = NTL ? load_frag_nt(wr, static_cast<const WT*>(Wp), p) : load_frag(p);
          }
      };
      if (wnt) load_w(std::true_type{});
      else load_w(std::false_type{});
    }
#pragma unroll
    for (int i = 0; i < KBW; ++i) {
      const int kb = kbeg + i;
      if constexpr (INT4) {
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
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + grp * 4 + i;       // < 64: rinv_s holds every row slot
      float y = rinv_s[m] * tot[0][i] + epi_c0;
      if (d.rope_theta > 0.f) y = rope_rotate(d, m, col, y, __shfl_xor(y, 1, 64));  // all lanes shuffle
      if (m >= d.M) continue;
      qkv_store<AT, true>(d, bf, g.layer, m, col, y);
    }
  } else if constexpr (EPI == EPI_RESID) {
    const int col = nrow[0] + r16;
    const float sc1 = 1.0f + epi_c0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + grp * 4 + i;
      const float hn = m < d.M ? resid_store<AT, true>(d, bf, m, col, epi_h[i], epi_c1 * tot[0][i], sc1) : 0.f;
      const float sq = sum16(hn * hn);
      if (r16 == 0 && m < d.M) st_act<true>(bf.ssq + (size_t)m * (d.D / 16) + tile, sq);
    }
  } else {  // EPI_GEGLU
    const int f = nrow[0] + r16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + grp * 4 + i;
      if (m >= d.M) continue;
      geglu_store<AT, true>(d, bf, m, f, rinv_s[m] * tot[0][i] + epi_c0, rinv_s[m] * tot[NT - 1][i] + epi_c1);
    }
  }
  PHASE_MARK(7);
}

template <class AT, class WT, int EPI, int NT, int MT>
static hipError_t launch_gemm_q(const Dims& d, const Bufs& b, const GemmLaunch& g, int tiles, hipStream_t st) {
  if (g.S <= 0 || (g.S & (g.S - 1))) return hipErrorInvalidValue;   // splits: a power of two
  const int kbs = g.K / 32 / g.S;        // k-blocks per split (a multiple of 4), shared by 4 waves
  const int slog = __builtin_ctz((unsigned)g.S);
  // every wave owns exactly kbw k-blocks; int4 waves own whole 128-wide quads (one scale
  // group each), so splits of fewer than four quads leave the surplus waves idle
  const int qps = kbs / 4;
  const int kbw = __is_same(WT, i4) ? (qps >= 4 ? qps : 4) : qps;
  if (__is_same(WT, i4) && qps > 4 && qps % 4) return hipErrorInvalidValue;
  dim3 grid(tiles * g.S), block(256);
  switch (kbw) {
    case 1: hipLaunchKernelGGL((k_gemm<AT, WT, MT, NT, 1, EPI>), grid, block, 0, st, g.W, g.A, g.K, slog, g.n_second, kbs, g.wnt, d, b, g); break;
    case 2: hipLaunchKernelGGL((k_gemm<AT, WT, MT, NT, 2, EPI>), grid, block, 0, st, g.W, g.A, g.K, slog, g.n_second, kbs, g.wnt, d, b, g); break;
    case 4: hipLaunchKernelGGL((k_gemm<AT, WT, MT, NT, 4, EPI>), grid, block, 0, st, g.W, g.A, g.K, slog, g.n_second, kbs, g.wnt, d, b, g); break;
    case 8: hipLaunchKernelGGL((k_gemm<AT, WT, MT, NT, 8, EPI>), grid, block, 0, st, g.W, g.A, g.K, slog, g.n_second, kbs, g.wnt, d, b, g); break;
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

template <class AT, class WT>
static hipError_t launch_gemv_t(const Dims& d, const Bufs& b, const GemmLaunch& g, int epi, int tiles, hipStream_t st) {
  switch (epi) {
    case EPI_QKV: return launch_gemm<AT, WT, EPI_QKV, 1>(d, b, g, tiles, st);
    case EPI_RESID: return launch_gemm<AT, WT, EPI_RESID, 1>(d, b, g, tiles, st);
    case EPI_GEGLU: return launch_gemm<AT, WT, EPI_GEGLU, 2>(d, b, g, tiles, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv(const Dims& d, const Bufs& b, const GemmLaunch& g, WDtype wt, int epi, int tiles,
                       hipStream_t st) {
  switch (wt) {
    case W_F32: return launch_gemv_t<float, float>(d, b, g, epi, tiles, st);
    case W_BF16: return launch_gemv_t<bf16, bf16>(d, b, g, epi, tiles, st);
    case W_INT4: return launch_gemv_t<bf16, i4>(d, b, g, epi, tiles, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace phyai
