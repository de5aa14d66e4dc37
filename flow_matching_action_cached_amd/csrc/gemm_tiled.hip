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

// Waits of the pipeline: stage ks has landed once at most `after` later stages (LPW loads
// each) are still in flight.
template <int LPW, int NSTG>
__device__ __forceinline__ void wait_stage(int after) {
  if constexpr (NSTG >= 4) {
    if (after >= 2) { wait_vmem_le<2 * LPW>(); return; }
  }
  if constexpr (NSTG >= 3) {
    if (after >= 1) { wait_vmem_le<LPW>(); return; }
  }
  wait_vmem_le<0>();
}

// WGM x WGN waves, each owning a 16*WMT x 16*WNT sub-tile; NSTG stages of 32*BKB
// k-columns in LDS, up to NSTG-1 of them in flight while one feeds the MFMAs.  With
// ksplit > 1 the K range is cut into ksplit equal parts, one workgroup each: every part
// stores its fp32 tile (agent scope) and the last to arrive adds the parts in split order
// before the epilogue.
template <int WMT, int WNT, int WGM, int WGN, int NSTG, int BKB, int EPI>
__global__ __launch_bounds__(64 * WGM * WGN) void k_gemm_tiled(Dims d, Bufs bf, GemmLaunch g, int tilesN,
                                                               int tilesM, int ksplit) {
  typedef bf16 AT;
  constexpr int NW = WGM * WGN;
  constexpr int BMT = WGM * WMT, BNT = WGN * WNT;  // 16-row / 16-column tiles per workgroup
  constexpr int LA = BMT * BKB, LB = BNT * BKB;    // 1 KB fragment blocks per stage
  constexpr int LPW = (LA + LB) / NW;              // direct-to-LDS loads per wave per stage
  constexpr int BM = 16 * BMT;
  constexpr bool NORM = (EPI == EPI_QKV || EPI == EPI_GEGLU);
  static_assert((LA + LB) % NW == 0, "stage loads split evenly over the waves");
  static_assert(NSTG >= 2 && NSTG <= 4, "pipeline depth");
  static_assert(EPI != EPI_GEGLU || WNT % 2 == 0, "gate/up tiles come in pairs");
  static_assert(BM <= 64 * NW, "one thread per tile row for the row statistics");
  // One LDS object per stage: with distinct objects the compiler can tell that the reads of
  // stage ks do not alias the direct-to-LDS copies into the other stages, and does not wait
  // for those copies before the reads (with one array it waits for every copy in flight).
  __shared__ __attribute__((aligned(16))) u32x4 lds0[LA + LB][64];
  __shared__ __attribute__((aligned(16))) u32x4 lds1[LA + LB][64];
  __shared__ __attribute__((aligned(16))) u32x4 lds2[NSTG >= 3 ? LA + LB : 1][64];
  __shared__ __attribute__((aligned(16))) u32x4 lds3[NSTG >= 4 ? LA + LB : 1][64];
  auto stage = [&](int b) -> u32x4 (*)[64] { return b == 0 ? lds0 : b == 1 ? lds1 : b == 2 ? lds2 : lds3; };
  __shared__ float rinv_s[BM];

  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / WGN, wn = w % WGN;
  // Tile order.  Consecutive workgroups go to different XCDs (round robin over 8), so each
  // XCD gets a contiguous run of the ordinal order; the ordinal order walks groups of GM
  // row tiles column by column, so the workgroups resident on one XCD at a time cover a
  // GM x (resident / GM) block and share operand panels in that XCD's L2.
  constexpr int GM = 8;
  const int ntiles = tilesM * tilesN;
  int t = blockIdx.x;
  if ((gridDim.x & 7) == 0) t = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int split = t / ntiles;  // K part (outermost in the ordinal order)
  t -= split * ntiles;
  const int gi = t / (GM * tilesN), rows_g = min(GM, tilesM - gi * GM), within = t - gi * GM * tilesN;
  const int tm = gi * GM + within % rows_g, tn = within / rows_g;
  const int nstage = g.K / 32 / BKB / ksplit;
  const int ks_off = split * nstage;  // first stage of this K part
  const int mtiles = (d.M + 15) / 16;  // 16-row tiles present in the activation buffer
  const AT* A = static_cast<const AT*>(g.A);
  const AT* W = static_cast<const AT*>(g.W);

  // virtual column tile -> weight row tile: for gate/up the virtual order interleaves
  // 16 gate rows and the matching 16 up rows, so a wave owns both halves of its outputs
  auto wtile = [&](int vt) -> int {
    if constexpr (EPI == EPI_GEGLU) return (vt & 1) ? (g.n_second >> 4) + (vt >> 1) : (vt >> 1);
    return vt;
  };
  // one stage: LA activation blocks then LB weight blocks; wave w copies blocks w, w+NW, ...
  auto issue = [&](int ks, int buf) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int blk = w + i * NW;
      const AT* src;
      if (blk < LA) {
        const int rt = min(tm * BMT + blk / BKB, mtiles - 1);  // past the last rows: any valid tile
        src = A + sw_frag(rt, (ks_off + ks) * BKB + blk % BKB, g.K, lane);
      } else {
        const int b2 = blk - LA;
        src = W + sw_frag(wtile(tn * BNT + b2 / BKB), (ks_off + ks) * BKB + b2 % BKB, g.K, lane);
      }
      __builtin_amdgcn_global_load_lds((const void PHYAI_GLOBAL_AS*)src, (void PHYAI_LDS_AS*)&stage(buf)[blk][0], 16,
                                       0, 0);
    }
  };
#pragma unroll
  for (int s = 0; s < NSTG - 1; ++s)
    if (s < nstage) issue(s, s);

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

  // main loop, unrolled by the pipeline depth so every LDS buffer index is a constant
  for (int ks0 = 0; ks0 < nstage; ks0 += NSTG) {
#pragma unroll
    for (int j = 0; j < NSTG; ++j) {
      const int ks = ks0 + j;
      if (ks < nstage) {
        wait_stage<LPW, NSTG>(min(NSTG - 2, nstage - 1 - ks));  // this wave's copies of stage ks landed
        // ... and everyone's; everyone is also done reading stage ks-1.  A bare barrier: the
        // fences of __syncthreads would wait for the later stages' copies as well.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (ks + NSTG - 1 < nstage) issue(ks + NSTG - 1, (j + NSTG - 1) % NSTG);
#pragma unroll
        for (int kb = 0; kb < BKB; ++kb) {
          bf16x8 af[WMT], bw[WNT];
#pragma unroll
          for (int i = 0; i < WMT; ++i) af[i] = __builtin_bit_cast(bf16x8, stage(j)[(wm * WMT + i) * BKB + kb][lane]);
#pragma unroll
          for (int t = 0; t < WNT; ++t)
            bw[t] = __builtin_bit_cast(bf16x8, stage(j)[LA + (wn * WNT + t) * BKB + kb][lane]);
          // every fragment of the k-block read before its products: one LDS round trip per
          // k-block instead of one per fragment
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < WMT; ++i)
#pragma unroll
            for (int t = 0; t < WNT; ++t) acc[i][t] = mma(af[i], bw[t], acc[i][t]);
        }
      }
    }
  }

  if (ksplit > 1) {  // cross-workgroup K split: the last arrival sums the parts in split order
    __shared__ unsigned flag;
    constexpr uint32_t part_bytes = (uint32_t)NW * WMT * WNT * 1024;
    const __amdgpu_buffer_rsrc_t ws =
        agent_rsrc(bf.gemm_ws + (size_t)t * ksplit * (part_bytes / 4), part_bytes * (uint32_t)ksplit);
#pragma unroll
    for (int i = 0; i < WMT; ++i)
#pragma unroll
      for (int j = 0; j < WNT; ++j)
        st_agent16(ws, split * part_bytes + ((w * WMT * WNT + i * WNT + j) * 64 + lane) * 16, acc[i][j]);
    if (!split_arrive_wg(bf.gemm_cnt + t, (unsigned)ksplit, &flag)) return;
#pragma unroll
    for (int i = 0; i < WMT; ++i)
#pragma unroll
      for (int j = 0; j < WNT; ++j) {
        f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int s2 = 0; s2 < ksplit; ++s2)
          sum += (s2 == split) ? acc[i][j]
                               : ld_agent16(ws, s2 * part_bytes + ((w * WMT * WNT + i * WNT + j) * 64 + lane) * 16);
        acc[i][j] = sum;
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
          const int m = m0 + e, mc = min(m, d.M - 1);  // rows past the end: any valid row's tables
          const float c = g.cvec[(size_t)(mc / d.rows_per_tab) * bf.cv_stride + col];
          float y = rinv_s[m - tm * BM] * acc[i][j][e] + c;
          if (d.rope_theta > 0.f) y = rope_rotate(d, m, col, y, __shfl_xor(y, 1, 64));  // all lanes shuffle
          if (m >= d.M) continue;
          qkv_store<AT>(d, bf, g.layer, m, col, y);
        }
      }
    } else if constexpr (EPI == EPI_RESID) {
#pragma unroll
      for (int j = 0; j < WNT; ++j) {
        const int col = (vt0 + j) * 16 + r16;
        const float gt = g.gate ? g.gate[col] : 1.f;  // residual gate (1: plain residual, exact)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + e;
          float hn = 0.f;
          if (m < d.M) {
            const float sc1 = 1.0f + g.scale_next[(size_t)(m / d.rows_per_tab) * scale_tab + col];
            hn = resid_store<AT>(d, bf, m, col, bf.h[(size_t)m * d.D + col], gt * acc[i][j][e], sc1);
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
          geglu_store<AT>(d, bf, m, f, ri * acc[i][j][e] + cg, ri * acc[i][j + 1][e] + cu);
        }
      }
    }
  }
}

// Host launch for the tiled family.  n_cols = output columns (gate/up: 2F).
//
// On gfx950 the load rate of a workgroup grows with its wave count much more than with
// its pipeline depth, so every shape runs 16 waves per workgroup with two LDS stages
// (two workgroups fit a CU), and the tile shape follows the output size:
//   gate/up (2F columns)        256 x 256, each wave 64 x 64
//   QKV, O and down when there are >= 512 tiles of 128 x 128: 128 x 128, waves 32 x 32
//   (O / down: four stages of 32 k-columns, 5 % faster than two of 64 on these shapes)
//   otherwise (few output tiles) QKV: 64 x 128 with 8 waves and three stages; O / down:
//   64 x 128 with 16 waves and 128-wide stages
template <int WMT, int WNT, int WGM, int WGN, int NSTG, int BKB, int EPI>
static hipError_t launch_cfg(const Dims& d, const Bufs& b, const GemmLaunch& g, int n_cols, hipStream_t st,
                             int ksplit = 1) {
  constexpr int BM = 16 * WGM * WMT, BN = 16 * WGN * WNT;
  if (n_cols % BN || g.K % (32 * BKB * ksplit)) return hipErrorInvalidValue;
  const int tilesN = n_cols / BN, tilesM = (d.M + BM - 1) / BM;
  if (ksplit > 1 && (!b.gemm_ws || !b.gemm_cnt)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_gemm_tiled<WMT, WNT, WGM, WGN, NSTG, BKB, EPI>), dim3(tilesM * tilesN * ksplit),
                     dim3(64 * WGM * WGN), 0, st, d, b, g, tilesN, tilesM, ksplit);
  return hipGetLastError();
}

// K split of the residual GEMMs (O and down) when their 64 x 128 output tiles are few.
// That configuration holds 144 KB of LDS, one workgroup per CU, so splitting pays only
// while tiles x splits still fit one round of 256 CUs (e.g. an 816-row prefill: 104 tiles,
// two parts); with more tiles (batch 32: 200) the second round costs more than the split
// saves.  Needs the split scratch (not kept by the joint denoiser, whose shapes take the
// 128 x 128 configuration).
static int resid_ksplit(const Dims& d, int n_cols, int K) {
  const int tiles128 = (d.M + 127) / 128 * (n_cols / 128);
  if (d.joint || tiles128 >= 512) return 1;
  const int tiles = (d.M + 63) / 64 * (n_cols / 128);
  int ks = 1;
  while (ks < 4 && tiles * ks * 2 <= 256 && K % (128 * ks * 2) == 0) ks *= 2;
  return ks;
}

// Scratch for every call of a context: a call may run fewer rows than the capacity d.M, and
// fewer tiles take more parts, but parts x tiles never exceed 256 (one round), each part a
// 64 x 128 fp32 tile.
size_t tiled_split_ws_floats(const Dims& d) {
  if (d.joint || d.M <= 64) return 0;
  return (size_t)256 * 64 * 128;
}

size_t tiled_split_counters(const Dims& d) { return (size_t)((d.M + 63) / 64) * (d.D / 128); }

hipError_t launch_gemm_tiled(const Dims& d, const Bufs& b, const GemmLaunch& g, int epi, int n_cols,
                             hipStream_t st) {
  switch (epi) {
    case EPI_QKV:
      if ((d.M + 127) / 128 * (n_cols / 128) >= 512) return launch_cfg<2, 2, 4, 4, 2, 2, EPI_QKV>(d, b, g, n_cols, st);
      return launch_cfg<2, 2, 2, 4, 3, 2, EPI_QKV>(d, b, g, n_cols, st);
    case EPI_RESID: {
      const int tiles128 = (d.M + 127) / 128 * (n_cols / 128);
      if (tiles128 >= 512) return launch_cfg<2, 2, 4, 4, 4, 1, EPI_RESID>(d, b, g, n_cols, st);
      const int ks = resid_ksplit(d, n_cols, g.K);
      return launch_cfg<1, 2, 4, 4, 3, 4, EPI_RESID>(d, b, g, n_cols, st, ks > 1 && b.gemm_ws ? ks : 1);
    }
    case EPI_GEGLU: {
      // 256 x 256 tiles; 128 x 256 when those would leave half the CUs or more idle and
      // the smaller tiles still fit one round (an 816-row prefill: 128 -> 224 workgroups)
      const int t256 = (d.M + 255) / 256 * (n_cols / 256), t128 = (d.M + 127) / 128 * (n_cols / 256);
      if (t256 <= 128 && t128 <= 256) return launch_cfg<2, 4, 4, 4, 2, 2, EPI_GEGLU>(d, b, g, n_cols, st);
      return launch_cfg<4, 4, 4, 4, 2, 2, EPI_GEGLU>(d, b, g, n_cols, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace phyai
