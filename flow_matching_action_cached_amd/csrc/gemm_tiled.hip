// LDS-tiled MFMA GEMMs of the Euler loop for many token rows (batch x chunk > 64),
// gfx950.  Same norm-folded epilogues as the weight-streaming kernels.
//
// With hundreds or thousands of token rows the linears are dense contractions
// (1600 x 1024 x 2560 for the QKV projection of 32 samples of 50 tokens), bound by
// MFMA throughput rather than weight bytes.  A workgroup of four waves computes a
// 16*BMT x 16*BNT output tile; each wave a 16*WMT x 16*WNT sub-tile held in MFMA
// accumulators.  Operands live in HBM in the fragment-native layout (common.h), so a
// stage of the tile -- whole 16 x 32 fragment blocks -- is copied block by block
// straight from global memory into LDS with direct-to-LDS loads (one contiguous
// 1 KB wave access per block, no register staging) and read back by the waves as
// contiguous 16 B/lane fragments (no bank conflicts).  Stages are double-buffered:
// the copy of stage k+1 is in flight while stage k feeds the MFMAs.
#include "epilogue.h"

#include <math.h>

namespace phyai {

#define PHYAI_GLOBAL_AS __attribute__((address_space(1)))
#define PHYAI_LDS_AS __attribute__((address_space(3)))

template <int WMT, int WNT, int EPI>
__global__ __launch_bounds__(256) void k_gemm_tiled(Dims d, Bufs bf, GemmLaunch g, int tilesN) {
  typedef bf16 AT;
  constexpr int BMT = 2 * WMT, BNT = 2 * WNT;  // 16-row / 16-column tiles per workgroup
  constexpr int BKB = 2;                       // 32-wide k-blocks per stage
  constexpr int BM = 16 * BMT;
  constexpr bool NORM = (EPI == EPI_QKV || EPI == EPI_GEGLU);
  static_assert(EPI != EPI_GEGLU || WNT % 2 == 0, "gate/up tiles come in pairs");
  __shared__ __attribute__((aligned(16))) u32x4 lds_a[2][BMT * BKB][64];
  __shared__ __attribute__((aligned(16))) u32x4 lds_b[2][BNT * BKB][64];
  __shared__ float rinv_s[BM];

  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;
  const int tn = blockIdx.x % tilesN, tm = blockIdx.x / tilesN;
  const int nstage = g.K / 32 / BKB;
  const int mtiles = (d.M + 15) / 16;  // 16-row tiles present in the activation buffer
  const AT* A = static_cast<const AT*>(g.A);
  const AT* W = static_cast<const AT*>(g.W);

  // virtual column tile -> weight row tile: for gate/up the virtual order interleaves
  // 16 gate rows and the matching 16 up rows, so a wave owns both halves of its outputs
  auto wtile = [&](int vt) -> int {
    if constexpr (EPI == EPI_GEGLU) return (vt & 1) ? (g.n_second >> 4) + (vt >> 1) : (vt >> 1);
    return vt;
  };
  // one stage: BMT*BKB activation blocks and BNT*BKB weight blocks, wave w copies every 4th
  auto issue = [&](int ks, int buf) {
#pragma unroll
    for (int blk = w; blk < BMT * BKB; blk += 4) {
      const int rt = min(tm * BMT + blk / BKB, mtiles - 1);  // past the last rows: any valid tile
      const AT* src = A + sw_frag(rt, ks * BKB + blk % BKB, g.K, lane);
      __builtin_amdgcn_global_load_lds((const void PHYAI_GLOBAL_AS*)src, (void PHYAI_LDS_AS*)&lds_a[buf][blk][0], 16,
                                       0, 0);
    }
#pragma unroll
    for (int blk = w; blk < BNT * BKB; blk += 4) {
      const AT* src = W + sw_frag(wtile(tn * BNT + blk / BKB), ks * BKB + blk % BKB, g.K, lane);
      __builtin_amdgcn_global_load_lds((const void PHYAI_GLOBAL_AS*)src, (void PHYAI_LDS_AS*)&lds_b[buf][blk][0], 16,
                                       0, 0);
    }
  };
  issue(0, 0);

  if (NORM && tid < BM) {
    // row statistics of this tile's rows: D/16 partial sums per row, in column order
    const int m = min(tm * BM + tid, d.M - 1);
    const f32x4* p = reinterpret_cast<const f32x4*>(bf.ssq + (size_t)m * (d.D / 16));
    float ss = 0.f;
    for (int j = 0; j < d.D / 64; ++j) {
      const f32x4 v = p[j];
      ss += v[0];
      ss += v[1];
      ss += v[2];
      ss += v[3];
    }
    rinv_s[tid] = 1.0f / sqrtf(ss / (float)d.D + d.eps);
  }

  f32x4 acc[WMT][WNT];
#pragma unroll
  for (int i = 0; i < WMT; ++i)
#pragma unroll
    for (int j = 0; j < WNT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int ks = 0; ks < nstage; ++ks) {
    wait_all_mem();   // this wave's copies of stage ks have landed
    __syncthreads();  // ... and everyone's; everyone is also done reading stage ks-1
    if (ks + 1 < nstage) issue(ks + 1, (ks + 1) & 1);
    const int buf = ks & 1;
#pragma unroll
    for (int kb = 0; kb < BKB; ++kb) {
      bf16x8 af[WMT], bw[WNT];
#pragma unroll
      for (int i = 0; i < WMT; ++i) af[i] = __builtin_bit_cast(bf16x8, lds_a[buf][(wm * WMT + i) * BKB + kb][lane]);
#pragma unroll
      for (int j = 0; j < WNT; ++j) bw[j] = __builtin_bit_cast(bf16x8, lds_b[buf][(wn * WNT + j) * BKB + kb][lane]);
#pragma unroll
      for (int i = 0; i < WMT; ++i)
#pragma unroll
        for (int j = 0; j < WNT; ++j) acc[i][j] = mma(af[i], bw[j], acc[i][j]);
    }
  }

  // ---- epilogues: acc[i][j][e] is row rowbase + 16 i + 4 grp + e, virtual column tile vt0 + j.
  // Rows may belong to different modulation tables (a guided pair: one table per branch):
  // the per-step vectors of table tb sit tb * cv_stride (W shift) or tb * nmod * 2 * D
  // (scale) after table 0's.
  const int rowbase = tm * BM + wm * WMT * 16;
  const int vt0 = tn * BNT + wn * WNT;
  const size_t scale_tab = (size_t)d.nmod * 2 * d.D;
#pragma unroll
  for (int i = 0; i < WMT; ++i) {
    const int m0 = rowbase + i * 16 + grp * 4;
    if constexpr (EPI == EPI_QKV) {
#pragma unroll
      for (int j = 0; j < WNT; ++j) {
        const int col = (vt0 + j) * 16 + r16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + e;
          if (m >= d.M) continue;
          const float c = g.cvec[(size_t)(m / d.rows_per_tab) * bf.cv_stride + col];
          qkv_store<AT>(d, bf, g.layer, m, col, rinv_s[m - tm * BM] * acc[i][j][e] + c);
        }
      }
    } else if constexpr (EPI == EPI_RESID) {
#pragma unroll
      for (int j = 0; j < WNT; ++j) {
        const int col = (vt0 + j) * 16 + r16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + e;
          float hn = 0.f;
          if (m < d.M) {
            const float sc1 = 1.0f + g.scale_next[(size_t)(m / d.rows_per_tab) * scale_tab + col];
            hn = resid_store<AT>(d, bf, m, col, bf.h[(size_t)m * d.D + col], acc[i][j][e], sc1);
          }
          const float sq = sum16(hn * hn);
          if (r16 == 0 && m < d.M) bf.ssq[(size_t)m * (d.D / 16) + vt0 + j] = sq;
        }
      }
    } else {  // EPI_GEGLU: virtual tiles (2q, 2q+1) are (gate, up) of feature block vt/2
#pragma unroll
      for (int j = 0; j < WNT; j += 2) {
        const int f = ((vt0 + j) >> 1) * 16 + r16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + e;
          if (m >= d.M) continue;
          const float* cv = g.cvec + (size_t)(m / d.rows_per_tab) * bf.cv_stride;
          const float cg = cv[f], cu = cv[g.n_second + f];
          const float ri = rinv_s[m - tm * BM];
          const float yg = ri * acc[i][j][e] + cg;
          const float yu = ri * acc[i][j + 1][e] + cu;
          static_cast<AT*>(bf.act)[sw_idx(m, f, d.F)] = to_elem<AT>(gelu_tanh(yg) * yu);
        }
      }
    }
  }
}

// Host launch for the tiled family.  n_cols = output columns (gate/up: 2F).  Chooses a
// 128x128 tile, or 64x128 when that leaves fewer than 256 workgroups.
hipError_t launch_gemm_tiled(const Dims& d, const Bufs& b, const GemmLaunch& g, int epi, int n_cols,
                             hipStream_t st) {
  if (n_cols % 128 || g.K % 64) return hipErrorInvalidValue;
  const int tilesN = n_cols / 128;
  const int big = (d.M + 127) / 128 * tilesN;
  const bool small_m = big < 256;
  const int tilesM = small_m ? (d.M + 63) / 64 : (d.M + 127) / 128;
  dim3 grid(tilesM * tilesN), block(256);
#define PHYAI_TILED(WM, E) \
  hipLaunchKernelGGL((k_gemm_tiled<WM, 4, E>), grid, block, 0, st, d, b, g, tilesN)
  switch (epi) {
    case EPI_QKV:
      if (small_m) PHYAI_TILED(2, EPI_QKV); else PHYAI_TILED(4, EPI_QKV);
      break;
    case EPI_RESID:
      if (small_m) PHYAI_TILED(2, EPI_RESID); else PHYAI_TILED(4, EPI_RESID);
      break;
    case EPI_GEGLU:
      if (small_m) PHYAI_TILED(2, EPI_GEGLU); else PHYAI_TILED(4, EPI_GEGLU);
      break;
    default:
      return hipErrorInvalidValue;
  }
#undef PHYAI_TILED
  return hipGetLastError();
}

}  // namespace phyai
