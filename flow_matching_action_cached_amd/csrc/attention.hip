// Attention of the Euler loop over [cached prefix ; chunk] keys, gfx950 (PhyAI reading
// "PhyAI: Real-Time Physical AI at the Edge, Scalable Rollouts in the Cloud", Sec. 5.1: the
// chunk attends to the cached prefix K/V and to itself, no mask among them):
//   k_attn         few query rows: split-key flash decode, online softmax, one partial
//                  per split;
//   k_attn_merge   log-sum-exp merge of those splits in split order (its own launch);
//   k_attn_wide    many query rows (batches, joint sequences): shared K/V staging, splits
//                  merged in-kernel.
#include "launch.h"

#include <math.h>

#include <algorithm>
#include <type_traits>

namespace phyai {

#ifdef PHYAI_PHASE_TRACE
PHYAI_PHASE_TRACE_READER(phyai_phase_trace_attn)
#endif

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
  constexpr int KROW = DH + 32 / ES;                 // K row: DH + 32 B pad (fewer bank conflicts than 16)
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
      if (g0 + j <= glast && !(ES == 4 && DH > 128)) {
        // every K fragment of the block read before the first product (one LDS round trip,
        // not one per product), and the dh sum as two interleaved chains per key half
        // (fp32 fragments of dh > 128 would not fit the registers: read per product below)
        Frag kf[DH / 32][2];
#pragma unroll
        for (int jj = 0; jj < DH / 32; ++jj) {
          kf[jj][0] = load_frag(ks + (j * 32 + r16) * KROW + 32 * jj + grp * 8);
          kf[jj][1] = load_frag(ks + (j * 32 + 16 + r16) * KROW + 32 * jj + grp * 8);
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x4 e0 = {0.f, 0.f, 0.f, 0.f}, e1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jj = 0; jj < DH / 32; jj += 2) {
          s0 = mma(kf[jj][0], qf[jj], s0);
          s1 = mma(kf[jj][1], qf[jj], s1);
          if (jj + 1 < DH / 32) {
            e0 = mma(kf[jj + 1][0], qf[jj + 1], e0);
            e1 = mma(kf[jj + 1][1], qf[jj + 1], e1);
          }
        }
        s0 += e0;
        s1 += e1;
      } else if (g0 + j <= glast) {
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
      // V fragments in batches of up to 8, each batch read before its products
      constexpr int VB = DH / 16 < 8 ? DH / 16 : 8;
#pragma unroll
      for (int t0 = 0; t0 < DH / 16; t0 += VB) {
        Frag vf[VB];
#pragma unroll
        for (int t = 0; t < VB; ++t) {
          const AT* vp = vs + ((t0 + t) * 16 + r16) * VROW + j * 32 + grp * 4;
          vf[t] = load_frag_split4(vp, vp + 16);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < VB; ++t) o[t0 + t] = mma(vf[t], pf, o[t0 + t]);
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

// Merge of the key splits of the few-row attention, one launch after it: a four-wave
// workgroup per (query tile, 16-byte slot).  Wave w takes the splits [w spw, w spw + spw)
// (spw = ceil(S / 4)) and forms their log-sum-exp state: its largest m_s as M_w,
// den_w = sum 2^(m_s - M_w) l_s and acc_w = sum 2^(m_s - M_w) l_s (O_s / l_s); wave 0 then
// combines the four states in wave order with the weights 2^(M_w - M), M the largest M_w,
// and writes acc / den, the normalised output columns of the slot, to o.  Four waves keep
// four times the loads of one in flight on the CU.  Slot u of a lane holds output columns
// 32u + 4 grp + i and 32u + 16 + 4 grp + i (bf16 partials) or 16u + 4 grp + i (fp32), row r16
// of the tile.  The arguments are the scalars the first loads need, in the order the
// kernel-argument preload puts them in SGPRs at wave launch (no wait for the argument
// fetch): the split workspace, the output o, the split count, the (sample, KV head, query
// tile) items, query tiles per KV head, KV heads, query heads per KV head, chunk tokens.
template <class AT, int DH, int SM>
__global__ __launch_bounds__(256) void k_attn_merge(const float* attn_ws, void* o_out, int S, int nitems, int QT,
                                                    int Hkv, int gq, int H) {
  constexpr int ES = sizeof(AT);
  constexpr int PAY = ES == 2 ? DH / 32 : DH / 16;
  constexpr uint32_t STRIDE = PAY * 1024 + 128;
  constexpr int NWV = 4, SPW = SM / NWV;     // waves; split capacity of a wave's registers
  constexpr int NA = ES == 2 ? 2 : 1;        // f32x4 accumulators per lane
  __shared__ f32x4 c_acc[NWV - 1][NA][64];
  __shared__ float c_m[NWV - 1][64], c_den[NWV - 1][64];
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int u = blockIdx.x % PAY, item = blockIdx.x / PAY;  // one workgroup per (query tile, slot)
  if (item >= nitems) return;
  const int spw = (S + NWV - 1) / NWV, s0 = w * spw, ns = max(0, min(S - s0, spw));  // this wave's splits
  // the item's splits through one buffer resource: the split offset is the scalar operand of
  // each load and the lane offsets are the same for every split
  const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(reinterpret_cast<const char*>(attn_ws) + (size_t)item * S * STRIDE), (short)0,
      (int)(S * STRIDE), 0x00020000);
  const uint32_t o_m = PAY * 1024 + r16 * 4, o_p = (u * 64 + lane) * 16;
  float ms[SPW], ls[SPW];
  u32x4 pv[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const uint32_t so = (uint32_t)min(s0 + j, S - 1) * STRIDE;
    ms[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ws, o_m, so, 0));
    ls[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ws, o_m + 64, so, 0));
    pv[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ws, o_p, so, 0));
  }
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < SPW; ++j)
    if (j < ns) M = fmaxf(M, ms[j]);
  float den = 0.f;
  f32x4 acc[NA];
#pragma unroll
  for (int t = 0; t < NA; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const float wgt = j < ns ? exp2f(ms[j] - M) * ls[j] : 0.f;
    den += wgt;
    if constexpr (ES == 2) {
      const bf16x8 pk = __builtin_bit_cast(bf16x8, pv[j]);
      acc[0] += wgt * f32x4{(float)pk[0], (float)pk[1], (float)pk[2], (float)pk[3]};
      acc[1] += wgt * f32x4{(float)pk[4], (float)pk[5], (float)pk[6], (float)pk[7]};
    } else {
      acc[0] += wgt * __builtin_bit_cast(f32x4, pv[j]);
    }
  }
  // the four states, combined by wave 0 in wave order (a wave without splits has den 0 and
  // M = -inf: weight 0)
  if (w > 0) {
    c_m[w - 1][lane] = M;
    c_den[w - 1][lane] = den;
#pragma unroll
    for (int t = 0; t < NA; ++t) c_acc[w - 1][t][lane] = acc[t];
  }
  __syncthreads();
  if (w > 0) return;
  float Mw[NWV];
  Mw[0] = M;
#pragma unroll
  for (int v = 1; v < NWV; ++v) Mw[v] = c_m[v - 1][lane];
  float Mx = Mw[0];
#pragma unroll
  for (int v = 1; v < NWV; ++v) Mx = fmaxf(Mx, Mw[v]);
  {
    const float f0 = exp2f(Mw[0] - Mx);
    den *= f0;
#pragma unroll
    for (int t = 0; t < NA; ++t) acc[t] *= f0;
  }
#pragma unroll
  for (int v = 1; v < NWV; ++v) {
    const float f = Mw[v] == -INFINITY ? 0.f : exp2f(Mw[v] - Mx);
    den += f * c_den[v - 1][lane];
#pragma unroll
    for (int t = 0; t < NA; ++t) acc[t] += f * c_acc[v - 1][t][lane];
  }
  const float inv = 1.0f / den;
  // this lane's row (rows past the last query row of the tile: nothing to write)
  const int qt = item % QT, r = (item / QT) % Hkv, b = item / QT / Hkv;
  const int qrow = qt * 16 + r16;
  if (qrow >= gq * H) return;
  const int head = r * gq + qrow / H, m = b * H + qrow % H;
  const int qd = gq * Hkv * DH;
  AT* op = static_cast<AT*>(o_out);
#pragma unroll
  for (int t = 0; t < NA; ++t) {
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
  // K row: DH + 32 B pad.  V^T row: NK keys + 32 B pad, the keys of each 32-key block
  // permuted so that the eight keys a lane's probability fragment holds (4 grp + i and
  // 16 + 4 grp + i, i < 4) are adjacent: key 16 h + 4 g + i sits at 8 g + 4 h + i, and a V
  // fragment is one 16-byte read.  Measured on gfx950 (SQ_LDS_BANK_CONFLICT, head dim 256
  // and 128): 32-byte pads on both rows leave 13 % of the bank-conflict cycles of 16-byte
  // pads (a 32-byte pad on K alone 50 %, on V^T alone 62 %); batch-32 attention 34.5 ->
  // 29.9 us per launch.
  constexpr int KROW = DH + 16;
  constexpr int VROW = NK + 16;
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
      } else {
        // keys k .. k+7 of a block (k = 0, 8, 16, 24): two runs of four, g = k % 16 / 4 and
        // g + 1, half h = k / 16, to 8 g + 4 h and 8 (g + 1) + 4 h
        const int k32 = (((c - KCH) % VCPR) * 8) % 32, h = k32 >> 4, g = (k32 & 15) >> 2;
        AT* blk = dst - k32;
        *reinterpret_cast<u32x2*>(blk + 8 * g + 4 * h) = u32x2{stage[i][0], stage[i][1]};
        *reinterpret_cast<u32x2*>(blk + 8 * (g + 1) + 4 * h) = u32x2{stage[i][2], stage[i][3]};
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
          vf[t] = load_frag(vb_ + ((t0 + t) * 16 + r16) * VROW + j * 32 + grp * 8);
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

// ------------------------------------------------------------------ host side
size_t attn_counters(const Dims& d) {
  const int QT = ((d.Hq / d.Hkv) * d.H + 15) / 16;
  return (size_t)d.B * d.Hkv * QT;
}
size_t attn_ws_floats(const Dims& d, const Plan& p) {
  const int T = d.P + d.H, nblk = (T + 31) / 32;
  const int S = (nblk + p.attn_bps - 1) / p.attn_bps;
  return attn_counters(d) * S * ((size_t)(d.dh / 16) * 256 + 32);
}
// Query tiles per workgroup of the many-row attention kernel (8 waves x tiles per wave).
int attn_wide_tiles(int dh) { return dh <= 128 ? 16 : 8; }

template <class AT>
static hipError_t launch_attn_merge(const Dims& d, const Bufs& b, int S, hipStream_t st) {
  const int gq = d.Hq / d.Hkv, QT = (gq * d.H + 15) / 16, nitems = d.B * d.Hkv * QT;
  const int pay = sizeof(AT) == 2 ? d.dh / 32 : d.dh / 16;
  dim3 mgrid(nitems * pay), mblock(256);
#define PHYAI_MERGE(DH)                                                                          \
  if (S > 16)                                                                                        \
    hipLaunchKernelGGL((k_attn_merge<AT, DH, 32>), mgrid, mblock, 0, st, b.attn_ws, b.o, S, nitems, QT, d.Hkv, gq, \
                       d.H);                                                                           \
  else                                                                                               \
    hipLaunchKernelGGL((k_attn_merge<AT, DH, 16>), mgrid, mblock, 0, st, b.attn_ws, b.o, S, nitems, QT, d.Hkv, gq, \
                       d.H);
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

hipError_t launch_attention(const Dims& d, const Bufs& b, const Plan& p, int layer, int part, bool f32,
                            hipStream_t st) {
  return f32 ? launch_attn_part<float>(d, b, p, layer, part, st) : launch_attn_part<bf16>(d, b, p, layer, part, st);
}

}  // namespace phyai
