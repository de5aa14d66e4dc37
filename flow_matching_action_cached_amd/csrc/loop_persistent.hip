// Persistent Euler loop for few token rows (batch x chunk <= 64, bf16), gfx950.
//
// The same step as the per-layer launches (PhyAI reading "PhyAI: Real-Time Physical AI at
// the Edge, Scalable Rollouts in the Cloud", Sec. 5.1 and 5.5: QKV with the adaptive norm
// folded in, attention over the cached prefix and the chunk, output projection, GeGLU MLP,
// final norm, out-projection and the Euler update), but the whole N-step loop is one kernel
// of co-resident workgroups, one per compute unit.  Each former launch boundary becomes a
// hand-off between workgroups, and every workgroup issues the next phase's weight loads
// before it waits for that hand-off, so the weight stream leaves the dependency chain (the
// page "FlashRT-PAI speeds physical AI inference up to 12.66x": deep kernel fusion with
// launch overlap removes the gaps between operations).
//
// Placement.  Workgroups go to the 8 XCDs round robin (workgroup w on XCD w mod 8; checked
// at start against HW_REG_XCC_ID).  XCD x owns the query heads [x hpx, (x+1) hpx): it
// computes their queries and, redundantly, the chunk's keys and values, runs their attention
// and split merge, and their slice of the output projection's inputs; it owns the MLP columns
// [x F/8, (x+1) F/8) of gate/up and the same slice of the down projection's inputs.  The two
// residual sums (output projection over the 8 head groups, down projection over the 8 column
// groups) and the out-projection rows are the only hand-offs between XCDs; the others stay
// inside one XCD's L2.  Each residual sum is an all-reduce: every XCD adds the 8 partials of
// its tile pairs itself (in XCD order, so all copies agree bit for bit), keeps the residual
// of its tile pair in registers and writes its own copy of the next norm's input and its
// statistics.
//
// Hand-offs.  A workgroup publishes a monotonic epoch flag when it has finished a phase (all
// its stores performed); a consumer polls exactly the flags of what it reads: its XCD's 32
// workgroups, the (tile pair, XCD) partials of a residual sum, or the token rows of the
// out-projection.  An XCD's 32 flags are contiguous; flags that only that XCD reads are
// stored plainly into its L2 and polled with scalar loads (which do not wait behind the
// weight loads in flight), the others are stored and polled at agent scope.  Every wait is
// bounded: on overrun a sticky abort word is set, every workgroup leaves at its next wait,
// and the host reports a device error.
//
// Visibility.  Data read across XCDs (the out-projection's outputs, residual partials, the
// state, the chunk's own K/V rows) is written with agent-scope stores.  Data that many
// workgroups read (norm inputs, statistics, q, o, act) lives in per-(step, layer) buffers
// that nothing has read before in this launch, so plain loads (served by L1 and L2) cannot
// meet stale lines; data read once (split partials, the out-projection's residual rows, the
// state, the K/V rows) is read with agent-scope loads.
#include "epilogue.h"
#include "persistent.h"

#include <math.h>

#include <algorithm>

namespace phyai {

#ifdef PHYAI_PHASE_TRACE
// Trace build only: per workgroup and phase, the real-time counter (100 MHz) when the wait
// for the phase begins, when it ends, and when the phase's flag is published, then stamps
// inside the phase (kTraceSlots per phase).
constexpr int kTracePhases = 4096;
constexpr int kTraceSlots = 8;
__device__ uint64_t g_ptrace[256 * kTracePhases * kTraceSlots];
__device__ int g_ptrace_phase;  // not used for indexing; the phase index travels in a register
#define PTRACE(phase, slot)                                                                        \
  do {                                                                                             \
    if (threadIdx.x == 0 && (phase) < kTracePhases)                                                \
      g_ptrace[((size_t)blockIdx.x * kTracePhases + (phase)) * kTraceSlots + (slot)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define PTRACE(phase, slot) ((void)0)
#endif

namespace {

constexpr unsigned kSpinMax = 1u << 21;  // polls per wait before the loop gives up (about 1 s)
constexpr int kSC1 = 16;                  // buffer-instruction cache policy: agent scope (sc1)

__device__ __forceinline__ uint64_t ld_flag(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_flag(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_u32_agent(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u32_agent(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Stores: agent scope by default; AUX 0 (plain, into this XCD's L2) for data that only this
// XCD's workgroups read.
template <int AUX = kSC1>
__device__ __forceinline__ void st_bf16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (bf16)v), r, byte_off, 0, AUX);
}
template <int AUX = kSC1>
__device__ __forceinline__ void st_f32(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), r, byte_off, 0, AUX);
}
__device__ __forceinline__ float ld_f32_sc1(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, kSC1));
}
__device__ __forceinline__ u32x4 ld_16_sc1(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kSC1));
}
__device__ __forceinline__ void st_16_sc1(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, kSC1);
}
// 16-byte buffer load: uniform resource and soffset, per-lane voffset (in the fragment-native
// layout the per-lane part of every fragment address is lane * 16, so one VGPR serves all
// loads of a wave).  aux: 0 plain, kNT non-temporal (weights, read once per step), kSC1.
constexpr int kNT = 2;
template <int AUX = 0>
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX));
}
template <int AUX = 0>
__device__ __forceinline__ bf16x8 bload_frag(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(bf16x8, bload16<AUX>(r, voff, soff));
}

// ------------------------------------------------------------------ hand-off waits
// Lanes of wave 0 poll flags base[i * stride] (i < n) until each reaches epoch e; every wave
// then meets at the workgroup barrier.  With stride 0 the flags are those of workgroups
// 0 .. n-1 in the XCD-major flag array (workgroup i at (i mod 8) 32 + i / 8).  False once the
// loop is aborted (by this wait's overrun or by another workgroup): the caller leaves the
// kernel.
__device__ bool wait_flags(const PArgs& a, const uint64_t* base, int stride, int n, uint64_t e, int* lds_ok,
                           int skip = -1) {
  const int tid = threadIdx.x;
  PTRACE((int)(e - a.epoch0) + 1, 0);
  if (tid < 64) {
    int ok = 1;
    for (int i = tid; i < n && ok; i += 64) {
      if (i == skip) continue;
      const uint64_t* f = base + (stride ? (size_t)i * stride : (size_t)((i & 7) * 32 + (i >> 3)));
      unsigned spins = 0;
      while ((int64_t)(ld_flag(f) - e) < 0) {
        ++spins;
        if ((spins & 255) == 0 && ld_u32_agent(a.ctl) != 0) {
          ok = 0;
          break;
        }
        if (spins > kSpinMax) {
          st_u32_agent(a.ctl, 1u);
          st_u32_agent(a.ctl + 1, (unsigned)(e - a.epoch0));
          ok = 0;
          break;
        }
      }
    }
    ok = __all(ok) ? 1 : 0;
    if (tid == 0) *lds_ok = ok;
  }
  __syncthreads();
  PTRACE((int)(e - a.epoch0) + 1, 1);
  return *lds_ok != 0;
}

// 32 contiguous flags (256 B) all at epoch e or later, read with four scalar loads that miss
// the scalar cache (glc) and read this XCD's L2, issued together and waited for once.  Scalar
// loads wait only for scalar and LDS operations, not behind the vector loads in flight (the
// next phase's weights, issued before the wait), which would hold a vector poll's result
// until they have all returned.
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ bool flags32_reached(const uint64_t* f, uint64_t e) {
  u32x16 v0, v1, v2, v3;
  asm volatile(
      "s_load_dwordx16 %0, %4, 0x0 glc\n\t"
      "s_load_dwordx16 %1, %4, 0x40 glc\n\t"
      "s_load_dwordx16 %2, %4, 0x80 glc\n\t"
      "s_load_dwordx16 %3, %4, 0xc0 glc\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(v0), "=&s"(v1), "=&s"(v2), "=&s"(v3)
      : "s"(f)
      : "memory");
  bool ok = true;
  auto chk = [&](const u32x16& v) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint64_t fv = ((uint64_t)v[2 * i + 1] << 32) | v[2 * i];
      ok &= (int64_t)(fv - e) >= 0;
    }
  };
  chk(v0);
  chk(v1);
  chk(v2);
  chk(v3);
  return ok;
}

// wait_flags for the 32 flags of this XCD's workgroups (contiguous, written by workgroups
// that share this XCD's L2): wave 0 polls them with scalar loads.
__device__ bool wait_local(const PArgs& a, const uint64_t* flags32, uint64_t e, int* lds_ok) {
  PTRACE((int)(e - a.epoch0) + 1, 0);
  if (threadIdx.x < 64) {
    int ok = 1;
    unsigned spins = 0;
    for (;;) {
      if (flags32_reached(flags32, e)) break;
      ++spins;
      if ((spins & 255) == 0 && ld_u32_agent(a.ctl) != 0) {
        ok = 0;
        break;
      }
      if (spins > kSpinMax) {
        if (threadIdx.x == 0) {
          st_u32_agent(a.ctl, 1u);
          st_u32_agent(a.ctl + 1, (unsigned)(e - a.epoch0));
        }
        ok = 0;
        break;
      }
    }
    if (threadIdx.x == 0) *lds_ok = ok;
  }
  __syncthreads();
  PTRACE((int)(e - a.epoch0) + 1, 1);
  return *lds_ok != 0;
}

// All of this workgroup's stores are performed; then its flag takes epoch e.
__device__ __forceinline__ void publish(uint64_t* flag, uint64_t e) {
  wait_all_mem();
  __syncthreads();
  if (threadIdx.x == 0) st_flag(flag, e);
}
// The end of a phase.  A flag that only this XCD's workgroups poll (scalar loads of this
// XCD's L2) takes a plain store, which lands in that L2; one that other XCDs poll (agent-scope
// loads) an agent-scope store.
__device__ __forceinline__ void publish_wg(const PArgs& a, uint64_t* flag, uint64_t e, bool cross) {
  wait_all_mem();
  __syncthreads();
  if (threadIdx.x == 0) {
    if (cross)
      st_flag(flag, e);
    else
      __hip_atomic_store(flag, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  PTRACE((int)(e - a.epoch0), 2);
}

// ------------------------------------------------------------------ weight-streaming GEMM unit
// One unit: output column tiles rt0 and rt1 (rt1 < 0: only rt0) over the k-blocks
// [kb0, kb0 + 4 KBW) of the activation A (swizzled [64][K]); wave w owns k-blocks
// kb0 + w KBW + [0, KBW).  The weight fragments are loaded ahead of the hand-off (WFr).
template <int KBW>
struct WFr {
  bf16x8 f[KBW][2];
};

// W: one layer's swizzled [rows][K] matrix.
template <int KBW>
__device__ __forceinline__ void load_w(WFr<KBW>& wr, const bf16* W, int rows, int K, int rt0, int rt1, int kb0) {
  const __amdgpu_buffer_rsrc_t r = rsrc(W, (uint32_t)((size_t)rows * K * 2));
  const uint32_t vo = (threadIdx.x & 63) * 16;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r1 = rt1 < 0 ? rt0 : rt1;
#pragma unroll
  for (int i = 0; i < KBW; ++i) {
    const int kb = kb0 + w * KBW + i;
    wr.f[i][0] = bload_frag<kNT>(r, vo, (uint32_t)(rt0 * (K / 32) + kb) * 1024u);
    wr.f[i][1] = bload_frag<kNT>(r, vo, (uint32_t)(r1 * (K / 32) + kb) * 1024u);
  }
}

// Products of the unit, reduced over the four waves in a fixed order; wave w returns m-tile w
// (tot[nt], nt = 0, 1).  With norm, rinv_s[m] = 1 / sqrt(mean(h_m^2) + eps) from the row
// statistics ssq [64][D/16] is also left in LDS.
template <int MT, int KBW, bool NORM>
__device__ __forceinline__ void gemm_unit(const Dims& d, const WFr<KBW>& wr, const bf16* A, int K, int kb0,
                                          const float* ssq, f32x4 (&tot)[2], char* lds, int tph) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  f32x4(*red)[2][MT][64] = reinterpret_cast<f32x4(*)[2][MT][64]>(lds);
  float* rinv_s = reinterpret_cast<float*>(lds + sizeof(f32x4) * 4 * 2 * MT * 64);
  bf16x8 af[KBW][MT];
  const __amdgpu_buffer_rsrc_t ra = rsrc(A, (uint32_t)(64 * K * 2));
  const uint32_t vo = lane * 16;
#pragma unroll
  for (int i = 0; i < KBW; ++i)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      af[i][mt] = bload_frag(ra, vo, (uint32_t)(mt * (K / 32) + kb0 + w * KBW + i) * 1024u);
  f32x4 ssv[8];
  const int srow = min(tid >> 2, d.M - 1), squart = tid & 3, n4 = d.D / 256;
  if constexpr (NORM) {
    const __amdgpu_buffer_rsrc_t rs = rsrc(ssq, (uint32_t)(64 * (d.D / 16) * 4));
    const uint32_t so = (uint32_t)(srow * (d.D / 16) + squart * (d.D / 64)) * 4;
#pragma unroll
    for (int j = 0; j < 8; ++j) ssv[j] = __builtin_bit_cast(f32x4, bload16(rs, so, (uint32_t)min(j, n4 - 1) * 16u));
  }
  __builtin_amdgcn_sched_barrier(0);
  f32x4 acc[2][MT];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < KBW; ++i)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[nt][mt] = mma(af[i][mt], wr.f[i][nt], acc[nt][mt]);
  PTRACE(tph, 3);
  if constexpr (NORM) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < n4) ss += ((ssv[j][0] + ssv[j][1]) + ssv[j][2]) + ssv[j][3];
    const float s1 = __shfl_xor(ss, 1, 64), s2 = __shfl_xor(ss, 2, 64), s3 = __shfl_xor(ss, 3, 64);
    const float q0 = squart == 0 ? ss : squart == 1 ? s1 : squart == 2 ? s2 : s3;
    const float q1 = squart == 1 ? ss : squart == 0 ? s1 : squart == 3 ? s2 : s3;
    const float q2 = squart == 2 ? ss : squart == 3 ? s1 : squart == 0 ? s2 : s3;
    const float q3 = squart == 3 ? ss : squart == 2 ? s1 : squart == 1 ? s2 : s3;
    if (squart == 0) rinv_s[tid >> 2] = 1.0f / sqrtf((((q0 + q1) + q2) + q3) / (float)d.D + d.eps);
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[w][nt][mt][lane] = acc[nt][mt];
  __syncthreads();
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    tot[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (w < MT) tot[nt] = ((red[0][nt][w][lane] + red[1][nt][w][lane]) + red[2][nt][w][lane]) + red[3][nt][w][lane];
  }
  PTRACE(tph, 4);
}

// ------------------------------------------------------------------ attention unit
// (sample b, query head `head`, key split s): wave j owns the head's query tile j (chunk
// tokens 16 j .. 16 j + 15) and all four share the split's K/V, staged block by block in LDS.
// The first block may come from registers loaded before the hand-off (pre).  Blocks that hold
// chunk rows (written this step) are read with agent-scope loads.  The split leaves a partial
// (O / l in bf16, m and l in fp32) for the merge, or with a single split the output itself.
template <int DH>
struct KVPre {
  static constexpr int CPT = (32 * DH / 8 + DH * 4) / 256;  // 16-byte chunks per thread per block
  u32x4 c[CPT];
};

template <int DH>
__device__ __forceinline__ void kv_load(const PArgs& a, KVPre<DH>& kv, int b, int l, int r, int blk, bool agent) {
  const Dims& d = a.d;
  constexpr int KCPR = DH / 8, KCH = 32 * KCPR, VCPR = 4;
  const size_t kvbase = ((size_t)b * d.Lc + l) * d.Hkv + r;
  const bf16* Kc = static_cast<const bf16*>(a.b.kc) + kvbase * d.KS * DH;
  const bf16* Vt = static_cast<const bf16*>(a.b.vt) + kvbase * DH * d.KS;
  const __amdgpu_buffer_rsrc_t rk = rsrc(Kc, (uint32_t)((size_t)d.KS * DH * 2));
  const __amdgpu_buffer_rsrc_t rv = rsrc(Vt, (uint32_t)((size_t)d.KS * DH * 2));
  // chunk c = tid + 256 i: K rows hold KCPR chunks (256 threads cover 256 / KCPR rows per i),
  // V^T rows VCPR chunks (256 / VCPR rows per i); per lane the offset is fixed, the rest uniform
  const int tid = threadIdx.x;
  const uint32_t vk = (uint32_t)((tid / KCPR) * DH * 2 + (tid % KCPR) * 16);
  const uint32_t vv = (uint32_t)(((tid / VCPR) * d.KS + (tid % VCPR) * 8) * 2);
  const int aux = agent ? kSC1 : 0;
#pragma unroll
  for (int i = 0; i < KVPre<DH>::CPT; ++i) {
    if (256 * i < KCH) {
      const uint32_t so = (uint32_t)((blk * 32 + i * (256 / KCPR)) * DH * 2);
      kv.c[i] = aux ? bload16<kSC1>(rk, vk, so) : bload16(rk, vk, so);
    } else {
      const uint32_t so = (uint32_t)(((i - KCH / 256) * (256 / VCPR) * d.KS + blk * 32) * 2);
      kv.c[i] = aux ? bload16<kSC1>(rv, vv, so) : bload16(rv, vv, so);
    }
  }
}

template <int DH>
__device__ void attn_unit(const PArgs& a, const char* blk_kl, int k, int l, int b, int head, int s,
                          const KVPre<DH>& pre, bool pre_valid, char* lds) {
  const Dims& d = a.d;
  typedef bf16x8 Frag;
  constexpr int KROW = DH + 8, VROW = 32 + 4, KCPR = DH / 8, KCH = 32 * KCPR, VCPR = 4;
  bf16* ks = reinterpret_cast<bf16*>(lds);
  bf16* vs = ks + 32 * KROW;
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
  const int j = __builtin_amdgcn_readfirstlane(tid >> 6);  // query tile of this wave
  const int qd = d.Hq * DH, r = head / (d.Hq / d.Hkv);
  const int T = d.P + d.H, nblk = (T + 31) / 32;
  const int blk0 = s * a.bps, blk1 = min(nblk, blk0 + a.bps);
  const int kend = min(T, blk1 * 32);
  const bool active = j * 16 < d.H;
  const int tok = j * 16 + r16;
  const bool qvalid = tok < d.H;
  const int m = b * d.H + (qvalid ? tok : 0);

  Frag qf[DH / 32];
  {
    const __amdgpu_buffer_rsrc_t rq = rsrc(blk_kl + a.o_q, (uint32_t)(64 * qd * 2));
    const uint32_t vq = (uint32_t)((m * qd + grp * 8) * 2);
#pragma unroll
    for (int jj = 0; jj < DH / 32; ++jj) qf[jj] = bload_frag(rq, vq, (uint32_t)(head * DH + 32 * jj) * 2u);
  }
  const float sc = 1.4426950408889634f / sqrtf((float)DH);
  float m_run = -INFINITY, l_part = 0.f;
  f32x4 o[DH / 16];
#pragma unroll
  for (int t = 0; t < DH / 16; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int g = blk0; g < blk1; ++g) {
    KVPre<DH> kv;
    if (g == blk0 && pre_valid) kv = pre;
    else kv_load<DH>(a, kv, b, l, r, g, (g + 1) * 32 > d.P);
    __syncthreads();  // the previous block's LDS reads are done
#pragma unroll
    for (int i = 0; i < KVPre<DH>::CPT; ++i) {
      const int c = tid + 256 * i;
      if (c < KCH) {
        *reinterpret_cast<u32x4*>(ks + (c / KCPR) * KROW + (c % KCPR) * 8) = kv.c[i];
      } else {
        bf16* dst = vs + ((c - KCH) / VCPR) * VROW + ((c - KCH) % VCPR) * 8;
        reinterpret_cast<u32x2*>(dst)[0] = u32x2{kv.c[i][0], kv.c[i][1]};
        reinterpret_cast<u32x2*>(dst)[1] = u32x2{kv.c[i][2], kv.c[i][3]};
      }
    }
    __syncthreads();
    if (!active) continue;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < DH / 32; ++jj) {
      s0 = mma(load_frag(ks + r16 * KROW + 32 * jj + grp * 8), qf[jj], s0);
      s1 = mma(load_frag(ks + (16 + r16) * KROW + 32 * jj + grp * 8), qf[jj], s1);
    }
    float sv[8];
    float mx = -INFINITY;
    const int kb = g * 32 + grp * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = kb + i < kend ? s0[i] : -INFINITY;
      sv[4 + i] = kb + 16 + i < kend ? s1[i] : -INFINITY;
      mx = fmaxf(mx, fmaxf(sv[i], sv[4 + i]));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_cand = fmaxf(m_run, mx * sc);
    if (g == blk0) {
      m_run = m_cand;
    } else if (__any(m_cand > m_run + 8.f)) {
      const float alpha = fast_exp2(m_run - m_cand);
      l_part *= alpha;
#pragma unroll
      for (int t = 0; t < DH / 16; ++t) o[t] *= alpha;
      m_run = m_cand;
    }
    Frag pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = fast_exp2(fmaf(sv[e], sc, -m_run));
      l_part += p;
      pf[e] = (bf16)p;
    }
#pragma unroll
    for (int t = 0; t < DH / 16; ++t) {
      const bf16* vp = vs + (t * 16 + r16) * VROW + grp * 4;
      o[t] = mma(load_frag_split4(vp, vp + 16), pf, o[t]);
    }
  }
  if (!active) return;
  float l_row = l_part;
  l_row += __shfl_xor(l_row, 16, 64);
  l_row += __shfl_xor(l_row, 32, 64);
  const int QTh = (d.H + 15) / 16;
  const int S = a.S;
  if (S == 1) {  // single split: the normalised output goes straight to o
    if (!qvalid) return;
    const __amdgpu_buffer_rsrc_t ro = rsrc(blk_kl + a.o_o, (uint32_t)(64 * qd * 2));
    const float inv = 1.0f / l_row;
#pragma unroll
    for (int t = 0; t < DH / 16; ++t) {
      const bf16x4 v4 = {(bf16)(o[t][0] * inv), (bf16)(o[t][1] * inv), (bf16)(o[t][2] * inv), (bf16)(o[t][3] * inv)};
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v4), ro,
                                            (uint32_t)(sw_idx(m, head * DH + t * 16 + grp * 4, qd) * 2), 0, kSC1);
    }
    return;
  }
  constexpr int PAY = DH / 32;
  constexpr uint32_t STRIDE = PAY * 1024 + 128;
  const size_t item = ((size_t)b * d.Hq + head) * QTh + j;
  const __amdgpu_buffer_rsrc_t ws = rsrc(a.attn_ws + item * S * (STRIDE / 4), STRIDE * S);
  const float inv_l = 1.0f / l_row;
#pragma unroll
  for (int u = 0; u < PAY; ++u) {
    const f32x4 x0 = o[2 * u] * inv_l, x1 = o[2 * u + 1] * inv_l;
    const bf16x8 pk = {(bf16)x0[0], (bf16)x0[1], (bf16)x0[2], (bf16)x0[3],
                       (bf16)x1[0], (bf16)x1[1], (bf16)x1[2], (bf16)x1[3]};
    st_16_sc1(ws, s * STRIDE + (u * 64 + lane) * 16, __builtin_bit_cast(u32x4, pk));
  }
  if (grp == 0) {
    st_f32(ws, s * STRIDE + PAY * 1024 + r16 * 4, m_run);
    st_f32(ws, s * STRIDE + PAY * 1024 + 64 + r16 * 4, l_row);
  }
}

// Merge of the key splits, one workgroup per (sample, head, query tile, 16-byte slot u):
// wave w merges splits [8 w, 8 w + 8) with weights 2^(m_s - M_w) l_s (few values in flight
// per lane, so every load of a wave is issued before the first is used), then wave 0
// combines the four partial merges with weights 2^(M_w - M).  Output columns
// 32 u + 16 t + 4 grp + i of the head.
template <int DH>
__device__ void merge_wg(const PArgs& a, const char* blk_kl, int b, int head, int jt, int u, char* lds) {
  const Dims& d = a.d;
  constexpr int PAY = DH / 32, SW = 8;
  constexpr uint32_t STRIDE = PAY * 1024 + 128;
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int QTh = (d.H + 15) / 16, S = a.S, qd = d.Hq * DH;
  const int tok = jt * 16 + r16;
  const size_t item = ((size_t)b * d.Hq + head) * QTh + jt;
  const __amdgpu_buffer_rsrc_t ws = rsrc(a.attn_ws + item * S * (STRIDE / 4), STRIDE * S);
  float ms[SW], ls[SW];
  u32x4 pv[SW];
#pragma unroll
  for (int i = 0; i < SW; ++i) {
    const uint32_t sp = (uint32_t)min(w * SW + i, S - 1) * STRIDE;
    ms[i] = ld_f32_sc1(ws, sp + PAY * 1024 + r16 * 4);
    ls[i] = ld_f32_sc1(ws, sp + PAY * 1024 + 64 + r16 * 4);
    pv[i] = ld_16_sc1(ws, sp + (u * 64 + lane) * 16);
  }
  float Mw = -INFINITY;
#pragma unroll
  for (int i = 0; i < SW; ++i)
    if (w * SW + i < S) Mw = fmaxf(Mw, ms[i]);
  float den = 0.f;
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int i = 0; i < SW; ++i) {
    const float wgt = w * SW + i < S ? exp2f(ms[i] - Mw) * ls[i] : 0.f;
    den += wgt;
    const bf16x8 pk = __builtin_bit_cast(bf16x8, pv[i]);
    acc[0] += wgt * f32x4{(float)pk[0], (float)pk[1], (float)pk[2], (float)pk[3]};
    acc[1] += wgt * f32x4{(float)pk[4], (float)pk[5], (float)pk[6], (float)pk[7]};
  }
  // partial merges of waves 1..3 to LDS: [wave][10][64] floats (M_w, den_w, 8 sums)
  float* pm = reinterpret_cast<float*>(lds);
  if (w > 0) {
    float* q = pm + (size_t)(w - 1) * 10 * 64 + lane;
    q[0] = Mw;
    q[64] = den;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) q[(2 + 4 * t + i) * 64] = acc[t][i];
  }
  __syncthreads();
  if (w != 0 || tok >= d.H) return;
  float M = Mw;
#pragma unroll
  for (int v = 1; v < 4; ++v) M = fmaxf(M, pm[(v - 1) * 640 + lane]);
  const float c0 = exp2f(Mw - M);
  den *= c0;
  acc[0] *= c0;
  acc[1] *= c0;
#pragma unroll
  for (int v = 1; v < 4; ++v) {
    const float* q = pm + (v - 1) * 640 + lane;
    const float cv = q[0] == -INFINITY ? 0.f : exp2f(q[0] - M);
    den += cv * q[64];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][i] += cv * q[(2 + 4 * t + i) * 64];
  }
  const int m = b * d.H + tok;
  const float inv = 1.0f / den;
  const __amdgpu_buffer_rsrc_t ro = rsrc(blk_kl + a.o_o, (uint32_t)(64 * qd * 2));
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int col = head * DH + 32 * u + 16 * t + grp * 4;
    const bf16x4 v4 = {(bf16)(acc[t][0] * inv), (bf16)(acc[t][1] * inv), (bf16)(acc[t][2] * inv),
                       (bf16)(acc[t][3] * inv)};
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v4), ro, (uint32_t)(sw_idx(m, col, qd) * 2), 0, kSC1);
  }
}

// ------------------------------------------------------------------ out-projection + Euler + in-projection
// One workgroup per token row m (as the launch-per-kernel form), on XCD x.  k_prev >= 0:
// final norm of step k_prev (its input and statistics from XCD x's copy of that step's final
// buffers), v, x += dt v.  k_next >= 0: h = x W_in^T + b_in, and the first norm's input and
// statistics of step k_next, into every XCD's copy.
__device__ void out_row(const PArgs& a, int m, int x, int k_prev, int k_next, char* lds) {
  const Dims& d = a.d;
  const Bufs& bf = a.b;
  float* xs = reinterpret_cast<float*>(lds);
  float* vres = xs + 256;
  float* wred = vres + 256;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const __amdgpu_buffer_rsrc_t rx = rsrc(bf.x, (uint32_t)(d.M * d.A * 4));
  if (k_prev >= 0) {
    const char* fin = a.fin + (size_t)k_prev * a.k_bytes;
    const float* ssq = reinterpret_cast<const float*>(fin + a.o_ssqf + (size_t)x * a.ssq_cb);
    const bf16* hsr = reinterpret_cast<const bf16*>(fin + a.o_hsf + (size_t)x * a.hs_cb);
    const bf16* wo = static_cast<const bf16*>(bf.w_out);
    const int n16 = d.D / 16;
    float ss = 0.f;
    if (w == 0) {
      const float a0 = ssq[(size_t)m * n16 + min(lane, n16 - 1)];
      const float a1 = ssq[(size_t)m * n16 + min(lane + 64, n16 - 1)];
      ss = (lane < n16 ? a0 : 0.f) + (lane + 64 < n16 ? a1 : 0.f);
    }
    bf16x8 hv[4];
    float hmask[4];
    const __amdgpu_buffer_rsrc_t rhs = rsrc(hsr, (uint32_t)(64 * d.D * 2));
    const __amdgpu_buffer_rsrc_t rwo = rsrc(wo, (uint32_t)(d.A * d.D * 2));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kk = lane * 8 + 512 * j;
      hmask[j] = kk < d.D ? 1.f : 0.f;
      hv[j] = bload_frag(rhs, (uint32_t)(sw_idx(m, min(kk, d.D - 8), d.D) * 2), 0u);
    }
    for (int a0 = w; a0 < d.A; a0 += 8) {  // outputs a0 and a0 + 4 per pass
      bf16x8 wv[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int aa = min(a0 + 4 * u, d.A - 1);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          wv[u][j] = bload_frag(rwo, (uint32_t)min(lane * 8 + 512 * j, d.D - 8) * 2u, (uint32_t)(aa * d.D * 2));
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float part = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) part += (float)hv[j][e] * (float)wv[u][j][e];
          acc += hmask[j] * part;
        }
        acc = wave_sum(acc);
        if (lane == 0 && a0 + 4 * u < d.A) vres[a0 + 4 * u] = acc;
      }
    }
    if (w == 0) {
      ss = wave_sum(ss);
      if (lane == 0) wred[0] = ss;
    }
    __syncthreads();
    const float rinv = 1.0f / sqrtf(wred[0] / (float)d.D + d.eps);
    for (int aa = tid; aa < d.A; aa += 256) {
      const bf16* bo = static_cast<const bf16*>(bf.b_out);
      const float* cv = bf.cvec + (size_t)k_prev * bf.cv_stride + bf.cv_out_off;
      const float v = rinv * vres[aa] + cv[aa] + (float)bo[aa];
      const uint32_t xo = (uint32_t)(((size_t)m * d.A + aa) * 4);
      const float xn = ld_f32_sc1(rx, xo) + bf.dt[k_prev] * v;
      st_f32(rx, xo, xn);
      xs[aa] = xn;
    }
    __syncthreads();
  } else {
    for (int aa = tid; aa < d.A; aa += 256) xs[aa] = ld_f32_sc1(rx, (uint32_t)(((size_t)m * d.A + aa) * 4));
    __syncthreads();
  }
  if (k_next < 0) return;
  const bf16* wi = static_cast<const bf16*>(bf.w_in);
  const bf16* bi = static_cast<const bf16*>(bf.b_in);
  const float* scl = bf.mod + (size_t)k_next * d.nmod * 2 * d.D;  // norm 0, scale row
  char* blk = a.act + (size_t)k_next * d.L * a.kl_bytes;            // (k_next, layer 0)
  const __amdgpu_buffer_rsrc_t rh = rsrc(a.hx, (uint32_t)(64 * d.D * 4));
  const __amdgpu_buffer_rsrc_t rhs = rsrc(blk + a.o_hsa, 8 * a.hs_cb);
  const __amdgpu_buffer_rsrc_t rss = rsrc(blk + a.o_ssqa, 8 * a.ssq_cb);
  const int na = d.A / 8;
  const __amdgpu_buffer_rsrc_t rwi = rsrc(wi, (uint32_t)(d.D * d.A * 2));
  for (int n0 = 0; n0 < d.D; n0 += 256) {
    const int n = n0 + tid;
    float hn = (float)bi[n];
    const float sc1 = 1.0f + scl[n];
    for (int c0 = 0; c0 < na; c0 += 8) {
      bf16x8 wv[8];
#pragma unroll
      for (int c = 0; c < 8; ++c)
        wv[c] = bload_frag(rwi, (uint32_t)(tid * d.A * 2), (uint32_t)((n0 * d.A + 8 * min(c0 + c, na - 1)) * 2));
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (c0 + c < na)
#pragma unroll
          for (int e = 0; e < 8; ++e) hn += xs[8 * (c0 + c) + e] * (float)wv[c][e];
    }
    const uint32_t oh = (uint32_t)(((size_t)m * d.D + n) * 4), ohs = (uint32_t)(sw_idx(m, n, d.D) * 2);
    const float sq = sum16(hn * hn);
    const uint32_t oss = (uint32_t)(((size_t)m * (d.D / 16) + n / 16) * 4);
    st_f32(rh, oh, hn);
#pragma unroll
    for (int xc = 0; xc < 8; ++xc) {
      st_bf16(rhs, xc * a.hs_cb + ohs, hn * sc1);
      if ((tid & 15) == 0) st_f32(rss, xc * a.ssq_cb + oss, sq);
    }
  }
}

// ------------------------------------------------------------------ residual sums across XCDs
// Tile pair p of a residual linear has one partial per XCD (its split of the input columns).
// Workgroup p of every XCD stores its partial in the sum's slot (output projection 0, down
// projection 1) and raises its (pair, XCD) flag, waits for the seven others, and adds the
// eight partials in XCD order: every XCD gets the same sums bit for bit, keeps the residual
// h += sum of its pair in registers and writes its own copy of the next norm's input
// hs = h (1 + scale_next) and of its statistics.  A slot is written again two sums later,
// after its writer has seen every other XCD's flag of the sum in between, raised after that
// XCD's loads of the slot had returned.
struct ResidPre {
  float sc1[2];  // 1 + scale of the norm that consumes h, at this lane's column of tile nt
};

// Loads ahead of the phase's wait: the static scale of both tiles' columns.
__device__ __forceinline__ void resid_pre_static(ResidPre& rp, const float* scale_next, int pair) {
  const int r16 = threadIdx.x & 15;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) rp.sc1[nt] = 1.0f + scale_next[(2 * pair + nt) * 16 + r16];
}
// The residual rows of the pair (this wave's m-tile) as the out-projection rows wrote them at
// the start of the step; the residual sums then keep them in registers.
template <int MT>
__device__ __forceinline__ void load_h0(const PArgs& a, float (&h)[2][4], int pair) {
  const Dims& d = a.d;
  const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const __amdgpu_buffer_rsrc_t rh = rsrc(a.hx, (uint32_t)(64 * d.D * 4));
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = min(w * 16 + grp * 4 + i, d.M - 1);
      h[nt][i] = w < MT ? ld_f32_sc1(rh, (uint32_t)(((size_t)m * d.D + (2 * pair + nt) * 16 + r16) * 4)) : 0.f;
    }
}

// Partial layout: [slot][pair][x][nt][w][64] f32x4.  The partial's stores are performed before
// the flag; a few lanes poll the seven other flags, then the seven partials are loaded in one
// round trip.  hs_next / ssq_next: XCD x's copies.  False if the loop was aborted.
template <int MT>
__device__ bool resid_allreduce(const PArgs& a, int slot, int pair, int x, const f32x4 (&tot)[2], const ResidPre& rp,
                                float (&h)[2][4], char* hs_next, char* ssq_next, uint64_t e, int* lds_ok) {
  const Dims& d = a.d;
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr uint32_t part_bytes = 2 * MT * 1024;
  const size_t pair_floats = (size_t)8 * (part_bytes / 4);
  const __amdgpu_buffer_rsrc_t ws = rsrc(a.part + ((size_t)slot * (d.D / 32) + pair) * pair_floats, part_bytes * 8);
  uint64_t* pflag = a.flag_part + pair * 8;
  if (w < MT)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      st_16_sc1(ws, x * part_bytes + ((nt * MT + w) * 64 + lane) * 16, __builtin_bit_cast(u32x4, tot[nt]));
  publish(pflag + x, e);
  PTRACE((int)(e - a.epoch0), 6);
  if (!wait_flags(a, pflag, 1, 8, e, lds_ok, x)) return false;
  PTRACE((int)(e - a.epoch0), 7);
  if (w < MT) {
    const __amdgpu_buffer_rsrc_t rhs = rsrc(hs_next, (uint32_t)(64 * d.D * 2));
    const __amdgpu_buffer_rsrc_t rss = rsrc(ssq_next, (uint32_t)(64 * (d.D / 16) * 4));
    u32x4 pv[2][8];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int x2 = 0; x2 < 8; ++x2)
        pv[nt][x2] = x2 == x ? __builtin_bit_cast(u32x4, tot[nt])
                             : ld_16_sc1(ws, x2 * part_bytes + ((nt * MT + w) * 64 + lane) * 16);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int x2 = 0; x2 < 8; ++x2) sum += __builtin_bit_cast(f32x4, pv[nt][x2]);
      const int tile = 2 * pair + nt, col = tile * 16 + r16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = w * 16 + grp * 4 + i;
        float hn = 0.f;
        if (m < d.M) {
          hn = h[nt][i] + sum[i];
          h[nt][i] = hn;
          st_bf16<0>(rhs, (uint32_t)(sw_idx(m, col, d.D) * 2), hn * rp.sc1[nt]);
        }
        const float sq = sum16(hn * hn);
        if (r16 == 0 && m < d.M) st_f32<0>(rss, (uint32_t)(((size_t)m * (d.D / 16) + tile) * 4), sq);
      }
    }
  }
  return true;
}

// ------------------------------------------------------------------ the loop
template <int DH, int MT, int KQ, int KO, int KD>
__global__ __launch_bounds__(256) void k_loop_persistent(PArgs a) {
  const Dims& d = a.d;
  const Bufs& bf = a.b;
  __shared__ __attribute__((aligned(16))) char lds[40960];
  __shared__ int lds_ok;
  const int tid = threadIdx.x;
  const int wg = blockIdx.x, x = wg & 7, c = wg >> 3;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (ld_u32_agent(a.ctl) != 0) return;  // an earlier launch aborted: the host must reset first
  // Every hand-off is made at agent scope, so a placement other than round robin costs only
  // L2 locality; it is recorded for the host.
  if (tid == 0 && (int)(__builtin_amdgcn_s_getreg((15 << 11) | 20) & 0xF) != x)
    st_u32_agent(a.ctl + 2, 0x80000000u | (unsigned)wg);
  // lines cached by an earlier launch (same per-step buffers) must not be served
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  const int L = d.L, qd = d.Hq * DH, hpx = a.hpx;
  const int nq_t = hpx * DH / 16, nkv_t = 2 * d.Hkv * DH / 16;   // QKV tiles of this XCD
  const int qkv_pairs = (nq_t + nkv_t + 1) / 2;
  const int npair = d.D / 32;                                      // residual tile pairs
  const int gu_units = d.F / 128;                                  // gate/up tiles per XCD
  const int QTh = (d.H + 15) / 16;
  const int att_units = d.B * hpx * a.S;
  const int mrg_items = d.B * hpx * QTh * (DH / 32);
  const uint64_t e0 = a.epoch0;
  const uint64_t per_step = 6 * (uint64_t)L + 1;
  auto E = [&](int k, int l, int ph) { return e0 + 1 + (uint64_t)k * per_step + 6 * (uint64_t)l + ph; };
  auto E_out = [&](int k) { return e0 + 1 + (uint64_t)k * per_step + 6 * (uint64_t)L; };
  // XCD-major flags: an XCD's 32 flags share two cache lines that no other XCD writes
  uint64_t* myflag = a.flag_wg + x * 32 + c;
  const uint64_t* local_flags = a.flag_wg + x * 32;

  // QKV tile pair pp of this XCD -> global column tiles
  auto qkv_tile = [&](int t) { return t < nq_t ? x * nq_t + t : qd / 16 + (t - nq_t); };
  auto qkv_rts = [&](int pp, int& rt0, int& rt1) {
    rt0 = qkv_tile(2 * pp);
    rt1 = 2 * pp + 1 < nq_t + nkv_t ? qkv_tile(2 * pp + 1) : -1;
  };
  WFr<KQ> wq;   // QKV or gate/up weights of the next unit
  WFr<KO> wo;
  WFr<KD> wd;
  KVPre<DH> kvp;
  bool kvp_valid = false;
  float cq[2];  // norm-folded bias of the QKV unit's two tiles at this lane's column (or gate, up)
  ResidPre ro, rd;
  float hreg[2][4] = {};  // residual rows of tile pair c (this wave's m-tile), kept across the step
  const int r16 = tid & 15;
  // weights and the static epilogue operands of this workgroup's first QKV unit of (k, l)
  auto pre_qkv = [&](int k, int l) {
    if (c < qkv_pairs) {
      int rt0, rt1;
      qkv_rts(c, rt0, rt1);
      load_w<KQ>(wq, static_cast<const bf16*>(bf.w_qkv) + (size_t)l * d.qkv * d.D, d.qkv, d.D, rt0, rt1, 0);
      const float* cv = bf.cvec + (size_t)k * bf.cv_stride + (size_t)l * d.qkv;
      cq[0] = cv[rt0 * 16 + r16];
      cq[1] = cv[(rt1 < 0 ? rt0 : rt1) * 16 + r16];
    }
  };

  // ---- in-projection of step 0
  if (wg < d.M) out_row(a, wg, x, -1, 0, lds);
  publish_wg(a, myflag, e0, true);
  pre_qkv(0, 0);

  for (int k = 0; k < d.N; ++k) {
    for (int l = 0; l < L; ++l) {
      char* blk = a.act + ((size_t)k * L + l) * a.kl_bytes;
      // ---------------- QKV (+ the chunk's K/V into the cache)
      {
        const uint64_t e = E(k, l, 0);
        bool ok = l == 0 ? wait_flags(a, a.flag_wg, 0, d.M, k == 0 ? e0 : E_out(k - 1), &lds_ok)
                         : wait_local(a, local_flags, E(k, l - 1, 5), &lds_ok);
        if (!ok) return;
        const float* cv = bf.cvec + (size_t)k * bf.cv_stride + (size_t)l * d.qkv;
        const bf16* W = static_cast<const bf16*>(bf.w_qkv) + (size_t)l * d.qkv * d.D;
        for (int pp = c; pp < qkv_pairs; pp += 32) {
          int rt[2];
          qkv_rts(pp, rt[0], rt[1]);
          if (pp != c) {
            load_w<KQ>(wq, W, d.qkv, d.D, rt[0], rt[1], 0);
            cq[0] = cv[rt[0] * 16 + r16];
            cq[1] = cv[(rt[1] < 0 ? rt[0] : rt[1]) * 16 + r16];
          }
          f32x4 tot[2];
          gemm_unit<MT, KQ, true>(d, wq, reinterpret_cast<const bf16*>(blk + a.o_hsa + (size_t)x * a.hs_cb), d.D, 0,
                                  reinterpret_cast<const float*>(blk + a.o_ssqa + (size_t)x * a.ssq_cb), tot, lds,
                                  (int)(e - e0));
          const float* rinv_s = reinterpret_cast<const float*>(lds + sizeof(f32x4) * 4 * 2 * MT * 64);
          if (w < MT) {
            const int lane = tid & 63, grp = lane >> 4;
            const int kd = d.Hkv * DH;
            // row m0 + i of this lane: sample b, chunk token t (32-bit offsets: the cache
            // resources are below 4 GB)
            const int m0 = w * 16 + grp * 4;
            int b0 = m0 / d.H;
            const int t0 = m0 - b0 * d.H;
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
              if (rt[nt] < 0) continue;
              const int c0 = rt[nt] * 16;  // the tile lies in one of q, k, v (uniform)
              const int col = c0 + r16;
              __amdgpu_buffer_rsrc_t rdst;
              uint32_t base, rstride, bstride;  // byte offset of (b, t): base + b bstride + t rstride
              if (c0 < qd) {
                rdst = rsrc(blk + a.o_q, (uint32_t)(64 * qd * 2));
                base = (uint32_t)col * 2;
                rstride = (uint32_t)qd * 2;
                bstride = (uint32_t)(d.H * qd * 2);
              } else {
                const uint32_t cache_bytes = (uint32_t)((size_t)d.B * d.Lc * d.Hkv * d.KS * DH * 2);
                const bool isk = c0 < qd + kd;
                const int cc = col - qd - (isk ? 0 : kd), r = cc / DH, dd = cc % DH;
                rdst = rsrc(isk ? bf.kc : bf.vt, cache_bytes);
                const uint32_t head_off = (uint32_t)(((l * d.Hkv + r) * d.KS) * DH) * 2;
                base = head_off + (uint32_t)(isk ? (d.P * DH + dd) : (dd * d.KS + d.P)) * 2;
                rstride = (uint32_t)(isk ? DH : 1) * 2;
                bstride = (uint32_t)(d.Lc * d.Hkv * d.KS * DH) * 2;
              }
              int b = b0, t = t0;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int m = m0 + i;
                if (m < d.M) {
                  const float y = rinv_s[m] * tot[nt][i] + cq[nt];
                  st_bf16(rdst, base + (uint32_t)b * bstride + (uint32_t)t * rstride, y);
                }
                if (++t == d.H) {
                  t = 0;
                  ++b;
                }
              }
            }
          }
          __syncthreads();  // LDS (partials, rinv) reused by the next unit
        }
        PTRACE((int)(e - e0), 5);
        publish_wg(a, myflag, e, false);
        // the first block of this workgroup's attention unit, when it holds prefix rows only
        kvp_valid = false;
        if (c < att_units) {
          const int s = c % a.S, hl = (c / a.S) % hpx, b = c / a.S / hpx;
          const int head = x * hpx + hl;
          if ((s * a.bps + 1) * 32 <= d.P) {
            kv_load<DH>(a, kvp, b, l, head / (d.Hq / d.Hkv), s * a.bps, false);
            kvp_valid = true;
          }
        }
      }
      // ---------------- attention over the cached prefix and the chunk
      {
        const uint64_t e = E(k, l, 1);
        if (!wait_local(a, local_flags, E(k, l, 0), &lds_ok)) return;
        for (int u = c; u < att_units; u += 32) {
          const int s = u % a.S, hl = (u / a.S) % hpx, b = u / a.S / hpx;
          attn_unit<DH>(a, blk, k, l, b, x * hpx + hl, s, kvp, kvp_valid && u == c, lds);
          __syncthreads();
        }
        PTRACE((int)(e - e0), 5);
        publish_wg(a, myflag, e, false);
        // output projection: weights of tile pair c over this XCD's heads, the next norm's scale
        if (c < npair) {
          load_w<KO>(wo, static_cast<const bf16*>(bf.w_o) + (size_t)l * d.D * qd, d.D, qd, 2 * c, 2 * c + 1,
                     x * hpx * DH / 32);
          resid_pre_static(ro, bf.mod + (((size_t)k * d.nmod + 2 * l + 1) * 2) * d.D, c);
        }
      }
      // ---------------- merge of the key splits
      {
        const uint64_t e = E(k, l, 2);
        if (!wait_local(a, local_flags, E(k, l, 1), &lds_ok)) return;
        if (a.S > 1)
          for (int it = c; it < mrg_items; it += 32) {
            const int u = it % (DH / 32), jt = (it / (DH / 32)) % QTh, hl = it / (DH / 32) / QTh % hpx;
            const int b = it / (DH / 32) / QTh / hpx;
            merge_wg<DH>(a, blk, b, x * hpx + hl, jt, u, lds);
            __syncthreads();  // LDS reused by the next item
          }
        PTRACE((int)(e - e0), 5);
        publish_wg(a, myflag, e, false);
      }
      // ---------------- output projection (this XCD's heads) + residual across XCDs
      {
        const uint64_t e = E(k, l, 3);
        if (!wait_local(a, local_flags, E(k, l, 2), &lds_ok)) return;
        if (c < npair) {  // at most 32 pairs: one per workgroup
          if (l == 0) load_h0<MT>(a, hreg, c);
          f32x4 tot[2];
          gemm_unit<MT, KO, false>(d, wo, reinterpret_cast<const bf16*>(blk + a.o_o), qd, x * hpx * DH / 32, nullptr,
                                   tot, lds, (int)(e - e0));
          if (!resid_allreduce<MT>(a, 0, c, x, tot, ro, hreg, blk + a.o_hsm + (size_t)x * a.hs_cb,
                                   blk + a.o_ssqm + (size_t)x * a.ssq_cb, e, &lds_ok))
            return;
          __syncthreads();
        }
        PTRACE((int)(e - e0), 5);
        publish_wg(a, myflag, e, false);
        if (c < gu_units) {
          const int j = x * gu_units + c;  // gate tile j, up tile F/16 + j
          load_w<KQ>(wq, static_cast<const bf16*>(bf.w_gu) + (size_t)l * 2 * d.F * d.D, 2 * d.F, d.D, j, d.F / 16 + j, 0);
          const float* cv = bf.cvec + (size_t)k * bf.cv_stride + bf.cv_gu_off + (size_t)l * 2 * d.F;
          cq[0] = cv[j * 16 + r16];
          cq[1] = cv[d.F + j * 16 + r16];
        }
      }
      // ---------------- gate/up + GeGLU (this XCD's MLP columns)
      {
        const uint64_t e = E(k, l, 4);
        if (!wait_local(a, local_flags, E(k, l, 3), &lds_ok)) return;
        const float* cv = bf.cvec + (size_t)k * bf.cv_stride + bf.cv_gu_off + (size_t)l * 2 * d.F;
        const __amdgpu_buffer_rsrc_t ract = rsrc(blk + a.o_act, (uint32_t)(64 * d.F * 2));
        for (int u = c; u < gu_units; u += 32) {
          const int j = x * gu_units + u;
          if (u != c) {
            load_w<KQ>(wq, static_cast<const bf16*>(bf.w_gu) + (size_t)l * 2 * d.F * d.D, 2 * d.F, d.D, j, d.F / 16 + j,
                       0);
            cq[0] = cv[j * 16 + r16];
            cq[1] = cv[d.F + j * 16 + r16];
          }
          f32x4 tot[2];
          gemm_unit<MT, KQ, true>(d, wq, reinterpret_cast<const bf16*>(blk + a.o_hsm + (size_t)x * a.hs_cb), d.D, 0,
                                  reinterpret_cast<const float*>(blk + a.o_ssqm + (size_t)x * a.ssq_cb), tot, lds,
                                  (int)(e - e0));
          const float* rinv_s = reinterpret_cast<const float*>(lds + sizeof(f32x4) * 4 * 2 * MT * 64);
          if (w < MT) {
            const int grp = (tid & 63) >> 4;
            const int f = j * 16 + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int m = w * 16 + grp * 4 + i;
              if (m >= d.M) continue;
              const float yg = rinv_s[m] * tot[0][i] + cq[0], yu = rinv_s[m] * tot[1][i] + cq[1];
              st_bf16(ract, (uint32_t)(sw_idx(m, f, d.F) * 2), gelu_tanh(yg) * yu);
            }
          }
          __syncthreads();
        }
        PTRACE((int)(e - e0), 5);
        publish_wg(a, myflag, e, false);
        if (c < npair) {
          load_w<KD>(wd, static_cast<const bf16*>(bf.w_d) + (size_t)l * d.D * d.F, d.D, d.F, 2 * c, 2 * c + 1,
                     x * (d.F / 256));
          const int jn = (l + 1 < L) ? 2 * (l + 1) : 2 * L;
          resid_pre_static(rd, bf.mod + (((size_t)k * d.nmod + jn) * 2) * d.D, c);
        }
      }
      // ---------------- down projection (this XCD's MLP columns) + residual across XCDs
      {
        const uint64_t e = E(k, l, 5);
        if (!wait_local(a, local_flags, E(k, l, 4), &lds_ok)) return;
        char* nblk = l + 1 < L ? a.act + ((size_t)k * L + l + 1) * a.kl_bytes : nullptr;
        char* fin = a.fin + (size_t)k * a.k_bytes;
        char* hs_next = (nblk ? nblk + a.o_hsa : fin + a.o_hsf) + (size_t)x * a.hs_cb;
        char* ssq_next = (nblk ? nblk + a.o_ssqa : fin + a.o_ssqf) + (size_t)x * a.ssq_cb;
        if (c < npair) {
          f32x4 tot[2];
          gemm_unit<MT, KD, false>(d, wd, reinterpret_cast<const bf16*>(blk + a.o_act), d.F, x * (d.F / 256), nullptr,
                                   tot, lds, (int)(e - e0));
          if (!resid_allreduce<MT>(a, 1, c, x, tot, rd, hreg, hs_next, ssq_next, e, &lds_ok)) return;
          __syncthreads();
        }
        PTRACE((int)(e - e0), 5);
        publish_wg(a, myflag, e, l + 1 == L);
        if (l + 1 < L) pre_qkv(k, l + 1);
      }
    }
    // ---------------- final norm, out-projection, Euler update, next in-projection
    {
      const uint64_t e = E_out(k);
      // a row's workgroup overwrites every XCD's copy of h: it waits for every workgroup's
      // last residual sum (the others only for their own XCD's)
      const bool ok = wg < d.M ? wait_flags(a, a.flag_wg, 1, kPersistWGs, E(k, L - 1, 5), &lds_ok)
                               : wait_local(a, local_flags, E(k, L - 1, 5), &lds_ok);
      if (!ok) return;
      if (wg < d.M) out_row(a, wg, x, k, k + 1 < d.N ? k + 1 : -1, lds);
      PTRACE((int)(e - e0), 5);
      publish_wg(a, myflag, e, true);
      if (k + 1 < d.N) pre_qkv(k + 1, 0);
    }
  }
}

}  // namespace

// ------------------------------------------------------------------ host side
bool persistent_supported(const Dims& d, WDtype wt) {
  if (wt != W_BF16 || d.joint || d.M > 64 || d.rope_theta > 0.f || d.gated) return false;
  if (d.Hq % 8 || d.Hq % d.Hkv) return false;
  const int hpx = d.Hq / 8;
  // D <= 1024: at most 32 residual tile pairs, one per workgroup of an XCD
  if ((hpx * d.dh) % 128 || d.D % 256 || d.D > 1024 || d.F % 1024 || d.A > 256) return false;
  const int MT = (d.M + 15) / 16;
  const int KQ = d.D / 128, KO = hpx * d.dh / 128, KD = d.F / 1024;
  if (d.dh == 256 && MT == 4 && KQ == 8 && KO == 2 && KD == 4) return true;   // pi0.5-shaped expert
  if (d.dh == 128 && KQ == 2 && KO == 1 && KD == 1) return true;              // small test shapes, any MT
  return false;
}

PersistLayout persistent_layout(const Dims& d) {
  PersistLayout p{};
  auto a256 = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const size_t qd = (size_t)d.Hq * d.dh;
  p.hs_cb = a256(64 * d.D * 2);
  p.ssq_cb = a256(64 * (d.D / 16) * 4);
  size_t off = 0;
  p.o_hsa = off; off += 8 * p.hs_cb;
  p.o_ssqa = off; off += 8 * p.ssq_cb;
  p.o_q = off; off = a256(off + 64 * qd * 2);
  p.o_o = off; off = a256(off + 64 * qd * 2);
  p.o_hsm = off; off += 8 * p.hs_cb;
  p.o_ssqm = off; off += 8 * p.ssq_cb;
  p.o_act = off; off = a256(off + 64 * (size_t)d.F * 2);
  p.kl_bytes = off;
  off = 0;
  p.o_hsf = off; off += 8 * p.hs_cb;
  p.o_ssqf = off; off += 8 * p.ssq_cb;
  p.k_bytes = off;
  return p;
}

// Key splits of the attention (sample, head) units: as many one-block splits as the XCD's
// 32 workgroups hold (a merge of up to 32 partials), else longer splits.
static void attn_split(const Dims& d, int hpx, int& S, int& bps) {
  const int nblk = (d.P + d.H + 31) / 32;
  const int per = std::max(1, 32 / std::max(1, d.B * hpx));
  S = std::min(nblk, std::min(per, 32));
  bps = (nblk + S - 1) / S;
  S = (nblk + bps - 1) / bps;
}

// [slot][pair][x][nt][m-tile (<= 4)][64 lanes] f32x4
size_t persistent_part_floats(const Dims& d) { return (size_t)2 * (d.D / 32) * 8 * 2 * 4 * 64 * 4; }
size_t persistent_hx_floats(const Dims& d) { return (size_t)64 * d.D; }

size_t persistent_attn_floats(const Dims& d) {
  int S, bps;
  attn_split(d, d.Hq / 8, S, bps);
  const size_t items = (size_t)d.B * d.Hq * ((d.H + 15) / 16);
  return items * S * ((size_t)(d.dh / 32) * 256 + 32);
}

hipError_t enqueue_denoise_persistent(const Dims& d, const Bufs& b, const PersistBufs& pb, uint64_t epoch0,
                                      hipStream_t st) {
  if (!persistent_supported(d, W_BF16)) return hipErrorInvalidValue;
  PArgs a{};
  a.d = d;
  a.b = b;
  const PersistLayout lay = persistent_layout(d);
  a.act = pb.act;
  a.kl_bytes = (uint32_t)lay.kl_bytes;
  a.o_hsa = (uint32_t)lay.o_hsa; a.o_ssqa = (uint32_t)lay.o_ssqa; a.o_q = (uint32_t)lay.o_q; a.o_o = (uint32_t)lay.o_o;
  a.o_hsm = (uint32_t)lay.o_hsm; a.o_ssqm = (uint32_t)lay.o_ssqm; a.o_act = (uint32_t)lay.o_act;
  a.fin = pb.fin;
  a.k_bytes = (uint32_t)lay.k_bytes; a.o_hsf = (uint32_t)lay.o_hsf; a.o_ssqf = (uint32_t)lay.o_ssqf;
  a.hs_cb = (uint32_t)lay.hs_cb; a.ssq_cb = (uint32_t)lay.ssq_cb;
  a.flag_wg = pb.flag_wg;
  a.flag_part = pb.flag_part;
  a.hx = pb.hx;
  a.ctl = pb.ctl;
  a.part = pb.part;
  a.attn_ws = pb.attn_ws;
  a.epoch0 = epoch0;
  a.hpx = d.Hq / 8;
  attn_split(d, a.hpx, a.S, a.bps);
  if (a.S > 32) return hipErrorInvalidValue;
  void* args[] = {&a};
  const int MT = (d.M + 15) / 16;
  const void* fn = nullptr;
  if (d.dh == 256) fn = reinterpret_cast<const void*>(&k_loop_persistent<256, 4, 8, 2, 4>);
  else if (MT == 1) fn = reinterpret_cast<const void*>(&k_loop_persistent<128, 1, 2, 1, 1>);
  else if (MT == 2) fn = reinterpret_cast<const void*>(&k_loop_persistent<128, 2, 2, 1, 1>);
  else if (MT == 3) fn = reinterpret_cast<const void*>(&k_loop_persistent<128, 3, 2, 1, 1>);
  else fn = reinterpret_cast<const void*>(&k_loop_persistent<128, 4, 2, 1, 1>);
  return hipLaunchCooperativeKernel(fn, dim3(kPersistWGs), dim3(256), args, 0, st);
}

uint64_t persistent_phases(const Dims& d) { return 1 + (uint64_t)d.N * (6 * (uint64_t)d.L + 1); }

}  // namespace phyai

#ifdef PHYAI_PHASE_TRACE
// Trace build only: copy the persistent loop's phase timestamps out (host dst of
// 256 * 4096 * 8 uint64: per workgroup and phase, wait begin, wait end, publish, products done,
// cross-wave sum done, epilogue issued, residual partial's flag raised, other partials'
// wait ended), then clear.
extern "C" int phyai_persist_trace(void* host_dst) {
  static uint64_t zeros[256 * phyai::kTracePhases * phyai::kTraceSlots];
  if (hipMemcpyFromSymbol(host_dst, HIP_SYMBOL(phyai::g_ptrace), sizeof(zeros), 0, hipMemcpyDeviceToHost) !=
          hipSuccess ||
      hipMemcpyToSymbol(HIP_SYMBOL(phyai::g_ptrace), zeros, sizeof(zeros), 0, hipMemcpyHostToDevice) != hipSuccess)
    return 4;
  return 0;
}
#endif
