// Per-step update kernels of the Euler loop, gfx950: the final norm, out-projection, state
// update and next in-projection of the action expert (k_out_rows) and of the joint
// video/action denoiser with its guided branch pair (k_wam_rows), and the input kernel of
// the prefix prefill (k_prefill_in).
#include "launch.h"

#include <math.h>

#include <algorithm>

namespace phyai {

#ifdef PHYAI_PHASE_TRACE
PHYAI_PHASE_TRACE_READER(phyai_phase_trace_update)
#endif

// An io-typed value loaded as a 32-bit word with nothing computed from it yet (bf16: the
// zero-extended bits), widened to fp32 only where it is used: a conversion next to the load
// would make the wave wait for the load there.
template <class T> __device__ __forceinline__ uint32_t ld_bits(const T* p);
template <> __device__ __forceinline__ uint32_t ld_bits<float>(const float* p) {
  return *reinterpret_cast<const uint32_t*>(p);
}
template <> __device__ __forceinline__ uint32_t ld_bits<bf16>(const bf16* p) {
  return *reinterpret_cast<const uint16_t*>(p);
}
template <class T> __device__ __forceinline__ float bits_f32(uint32_t v) {
  return __builtin_bit_cast(float, sizeof(T) == 2 ? v << 16 : v);
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
  // Operands that need nothing computed here are loaded up front, so that their round trips
  // overlap the out-projection's instead of following it: the in-projection weights, bias
  // and scale of this wave's first pass, the final-norm statistics, and the state, W_out
  // shift and bias of this thread's first update element.  The loads are unconditional
  // (indices clamped to valid rows, columns and steps; what a launch does not use is
  // ignored) and nothing is computed from them here, so no wait follows them.
  const IOT* wi = static_cast<const IOT*>(bf.w_in);
  const IOT* bi = static_cast<const IOT*>(bf.b_in);
  const int ntn = d.D / 16, ntb = cpart * (ntn / cs), nte = ntb + ntn / cs;
  WF wv0[4];
  uint32_t b00[4];
  float sc10[4];
  {
    const float* scl = bf.mod + (size_t)max(k_next, 0) * d.nmod * 2 * d.D;  // norm 0, scale row
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = min(ntb + w + 4 * j, nte - 1) * 16 + r16;
      wv0[j] = load_frag(wi + (size_t)n * d.A + min(grp * 8, d.A - 8));
      b00[j] = ld_bits(bi + n);
      sc10[j] = scl[n];
    }
  }
  const int sr = tid >> 4, sj0 = tid & 15, n16 = d.D / 16;   // statistics: 16 threads per row
  float ssv[8];
  float xv0[4], cva0;
  uint32_t boa0;
  {
    const int sm = min(m0 + sr, d.M - 1);
#pragma unroll
    for (int q = 0; q < 8; ++q) ssv[q] = bf.ssq[(size_t)sm * n16 + min(sj0 + 16 * q, n16 - 1)];
    const int l = tid & 63, a = min((tid >> 6) * 16 + (l & 15), d.A - 1);
    cva0 = bf.cvec[(size_t)max(k_prev, 0) * bf.cv_stride + bf.cv_out_off + a];
    boa0 = ld_bits(static_cast<const IOT*>(bf.b_out) + a);
#pragma unroll
    for (int i = 0; i < 4; ++i) xv0[i] = bf.x[(size_t)min(m0 + 4 * (l >> 4) + i, d.M - 1) * d.A + a];
  }
  if (k_prev >= 0) {
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
    {  // final-norm statistics of the tile's rows, summed in column order
      float ss = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) ss += sj0 + 16 * q < n16 ? ssv[q] : 0.f;
      for (int j = sj0 + 128; j < n16; j += 16) ss += bf.ssq[(size_t)min(m0 + sr, d.M - 1) * n16 + j];
      ss = sum16(ss);
      if (sj0 == 0) rinv_s[sr] = 1.0f / sqrtf(ss / (float)d.D + d.eps);
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
      const bool first = e == tid;   // this thread's first element: operands loaded up front
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * (l >> 4) + i, m = m0 + r;
        if (m < d.M && a < d.A) {
          const float v = rinv_s[r] * s[i] + (first ? cva0 : cv[a]) + (first ? bits_f32<IOT>(boa0) : to_f32(bo[a]));
          const float xn = (first ? xv0[i] : bf.x[(size_t)m * d.A + a]) + dt * v;
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
  const float* scl = bf.mod + (size_t)k_next * d.nmod * 2 * d.D;  // norm 0, scale row
  AT* hsw = static_cast<AT*>(bf.hs);
  const int kc_n = (d.A + 31) / 32;
  // this workgroup's column tiles: [ntb, nte), four of a wave's (nt0 + 4 j) at a time
  for (int nt0 = ntb + w; nt0 < nte; nt0 += 16) {
    f32x4 acc[4];
    float b0[4], sc1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kc = 0; kc < kc_n; ++kc) {
      const int a0 = kc * 32 + grp * 8;
      WF wv[4];
      const bool first = nt0 == ntb + w && kc == 0;   // loaded up front
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = min(nt0 + 4 * j, nte - 1) * 16 + r16;
        if (first) {
          wv[j] = wv0[j];
          b0[j] = bits_f32<IOT>(b00[j]);
          sc1[j] = 1.0f + sc10[j];
          continue;
        }
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

// ------------------------------------------------------------------ host side
hipError_t launch_out_rows(const Dims& d, const Bufs& b, WDtype wt, int k_prev, int k_next, hipStream_t st) {
  // column splits of the in-projection: up to 256 workgroups (one per CU), at least 4 column
  // tiles each (batch 32: 100 row tiles x 2; 128 workgroups at most took 17.6 us per step, 256
  // take 14.5)
  const int tiles = (d.M + 15) / 16;
  int cs = 1;
  if (b.gemm_cnt && (size_t)tiles <= gemm_counters(d))  // the tiles' arrival counters
    while (tiles * cs * 2 <= 256 && (d.D / 16) % (cs * 2) == 0 && d.D / 16 / (cs * 2) >= 4) cs *= 2;
  if (wt == W_F32)
    hipLaunchKernelGGL((k_out_rows<float, float>), dim3(tiles * cs), dim3(256), 0, st, d, b, k_prev, k_next, cs);
  else
    hipLaunchKernelGGL((k_out_rows<bf16, bf16>), dim3(tiles * cs), dim3(256), 0, st, d, b, k_prev, k_next, cs);
  return hipGetLastError();
}

hipError_t launch_wam_rows(const Dims& d, const Bufs& b, int k_prev, int k_next, hipStream_t st) {
  hipLaunchKernelGGL((k_wam_rows<bf16, bf16>), dim3((d.Tl + 15) / 16 + (d.H - d.Tl + 15) / 16), dim3(256), 0, st, d, b,
                     k_prev, k_next);
  return hipGetLastError();
}

hipError_t launch_prefill_in(const Dims& d, const Bufs& b, const void* tokens, bool f32, hipStream_t st) {
  if (f32)
    hipLaunchKernelGGL((k_prefill_in<float, float>), dim3(d.M), dim3(256), 0, st, d, b, static_cast<const float*>(tokens));
  else
    hipLaunchKernelGGL((k_prefill_in<bf16, bf16>), dim3(d.M), dim3(256), 0, st, d, b, static_cast<const bf16*>(tokens));
  return hipGetLastError();
}

}  // namespace phyai
