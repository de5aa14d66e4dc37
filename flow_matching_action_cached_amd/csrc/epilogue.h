// Launch record and per-element epilogues shared by the two GEMM families (the
// weight-streaming kernels for few token rows and the LDS-tiled kernels for many).
//
// Norm folding.  adaRMS(h) W^T = rinv * ((h * (1 + scale)) W^T) + W shift, with
// rinv = 1/sqrt(mean(h^2) + eps) per token row: the GEMM input is hs = h * (1 + scale)
// (written by the producer of h), the accumulator is multiplied by rinv and the per-step
// vector W shift (precomputed with the timestep tables) is added.
#pragma once

#include "common.h"
#include "kernels.h"

namespace phyai {

enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_GEGLU = 2 };

struct GemmLaunch {
  const void* A;             // activations, swizzled [Mpad][K]
  int lda, K;
  const void* W;             // weights of this layer, swizzled [N][K] (int4: swizzled codes)
  const uint16_t* Ws;        // int4 scales of this layer [N][K/128]
  int n_second;              // row offset of the second weight tile (gate/up: F)
  int S;                     // k-splits across workgroups
  int layer;
  const float* cvec;         // norm-folded bias of this step/layer (QKV, GEGLU)
  const float* scale_next;   // raw scale of the norm that consumes h (RESID)
  const float* gate;         // residual gate of the block this GEMM closes (RESID; null: none)
  int wnt;                   // 1: weights read with the non-temporal policy (weight-streaming GEMMs)
};

// Rotary position embedding of the QKV output y at token row m, column col (PhyAI reading
// Sec. 2 stresses positional precision; the pages print no convention): the query and key
// columns of every head form interleaved pairs (2i, 2i+1), turned by the angle
// p * theta^(-2i/dh) at the chunk token's position p = P + (m mod H).  yp is the pair
// partner's value (the neighbouring lane holds column col ^ 1 of the same row); value
// columns are returned unchanged.  Angle in fp32: the position is exact, the frequency is
// rounded once.
__device__ __forceinline__ float rope_rotate(const Dims& d, int m, int col, float y, float yp) {
  if (col >= (d.Hq + d.Hkv) * d.dh) return y;
  const int pair = (col % d.dh) >> 1;
  const float freq = exp2f(-(float)(2 * pair) / (float)d.dh * log2f(d.rope_theta));
  float sn, cs;
  sincosf((float)(d.P + m % d.H) * freq, &sn, &cs);
  return (col & 1) ? fmaf(yp, sn, y * cs) : fmaf(y, cs, -yp * sn);
}

// QKV output y of token row m, column col: q rows go to q [M][Hq*dh]; the chunk's own
// K and V go straight into the cache after the prefix rows (V transposed).  WT: write-through
// stores (st_act), for the weight-streaming GEMMs.
template <class AT, bool WT = false>
__device__ __forceinline__ void qkv_store(const Dims& d, const Bufs& bf, int layer, int m, int col, float y) {
  const int qd = d.Hq * d.dh, kd = d.Hkv * d.dh;
  const int b = m / d.H, t = m % d.H;
  if (col < qd) {
    st_act<WT>(static_cast<AT*>(bf.q) + (size_t)m * qd + col, to_elem<AT>(y));
  } else if (col < qd + kd) {
    const int r = (col - qd) / d.dh, dd = (col - qd) % d.dh;
    st_act<WT>(static_cast<AT*>(bf.kc) + ((((size_t)b * d.Lc + layer) * d.Hkv + r) * d.KS + d.P + t) * d.dh + dd,
          to_elem<AT>(y));
  } else {
    const int r = (col - qd - kd) / d.dh, dd = (col - qd - kd) % d.dh;
    st_act<WT>(static_cast<AT*>(bf.vt) + ((((size_t)b * d.Lc + layer) * d.Hkv + r) * d.dh + dd) * d.KS + d.P + t,
          to_elem<AT>(y));
  }
}

// Residual update of token row m, column col: h += delta; hs = h * (1 + scale of the next
// norm) in the GEMM input type (swizzled).  Returns the new h (for the row statistics).
template <class AT, bool WT = false>
__device__ __forceinline__ float resid_store(const Dims& d, const Bufs& bf, int m, int col, float h_old, float delta,
                                             float sc1) {
  const float hn = h_old + delta;
  st_act<WT>(bf.h + (size_t)m * d.D + col, hn);
  st_act<WT>(static_cast<AT*>(bf.hs) + sw_idx(m, col, d.D), to_elem<AT>(hn * sc1));
  return hn;
}

// GeGLU output of token row m, feature f from the gate and up pre-activations (norm folded
// in): act = gelu_tanh(gate) * up, swizzled [Mpad][F] in the GEMM input type.
template <class AT, bool WT = false>
__device__ __forceinline__ void geglu_store(const Dims& d, const Bufs& bf, int m, int f, float yg, float yu) {
  st_act<WT>(static_cast<AT*>(bf.act) + sw_idx(m, f, d.F), to_elem<AT>(gelu_tanh(yg) * yu));
}

// LDS-tiled GEMM family (gemm_tiled.hip) for more than 64 token rows, bf16 only.
// n_cols: output columns (gate/up: 2F); epi: Epi.
hipError_t launch_gemm_tiled(const Dims& d, const Bufs& b, const GemmLaunch& g, int epi, int n_cols,
                             hipStream_t stream);

}  // namespace phyai
