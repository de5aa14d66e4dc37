// Device-side building blocks for gfx950 (CDNA4, wave64).
//
// MFMA fragments.  Every matrix product in this library is expressed as a
// sequence of 16x16 output tiles accumulated over "k-blocks" of 32.  For one
// k-block a lane l (r16 = l % 16, grp = l / 16) holds
//   A fragment: 8 elements of row    r16 of A, at the lane group's k-set,
//   B fragment: 8 elements of column r16 of B, at the same k-set,
// and the 16x16 fp32 accumulator holds D[4*grp + i][r16], i = 0..3.
// Because the sum over k does not care how the 32 k indices are dealt to the
// (group, element) slots, any k-set assignment works as long as A and B use
// the same one; kernels pick the assignment that makes their loads contiguous.
//   bf16: one v_mfma_f32_16x16x32_bf16 per k-block;
//   fp32: eight v_mfma_f32_16x16x4_f32, op j taking element j of every group.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace phyai {

// Optional per-phase timestamps (a build with -DPHYAI_PHASE_TRACE only): each wave's lane 0
// stores the 100 MHz real-time counter at numbered points of a kernel into this file's
// g_phase_trace[(workgroup * 8 + wave) * 8 + slot] (workgroups < 2048, waves < 8); each
// kernel file exports a reader (PHYAI_PHASE_TRACE_READER) that copies its array out.
#ifdef PHYAI_PHASE_TRACE
static __device__ uint64_t g_phase_trace[4096 * 4 * 8];
#define PHASE_MARK(slot)                                                                          \
  do {                                                                                            \
    if ((threadIdx.x & 63) == 0 && blockIdx.x < 2048 && (threadIdx.x >> 6) < 8)                   \
      g_phase_trace[((size_t)blockIdx.x * 8 + (threadIdx.x >> 6)) * 8 + (slot)] =                 \
          __builtin_amdgcn_s_memrealtime();                                                       \
  } while (0)
// Copy this file's timestamps out (host dst of 4096*4*8 uint64), then clear them.
#define PHYAI_PHASE_TRACE_READER(fn)                                                                   \
  extern "C" int fn(void* host_dst) {                                                                 \
    static uint64_t zeros[4096 * 4 * 8];                                                               \
    if (hipMemcpyFromSymbol(host_dst, HIP_SYMBOL(g_phase_trace), sizeof(zeros), 0, hipMemcpyDeviceToHost) != \
            hipSuccess ||                                                                              \
        hipMemcpyToSymbol(HIP_SYMBOL(g_phase_trace), zeros, sizeof(zeros), 0, hipMemcpyHostToDevice) !=     \
            hipSuccess)                                                                                \
      return 4;                                                                                        \
    return 0;                                                                                          \
  }
#else
#define PHASE_MARK(slot) ((void)0)
#endif

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Tag type for packed int4 weights (codes + per-128 bf16 scales).
struct i4 {};

template <class T> struct FragOf;
template <> struct FragOf<bf16> { typedef bf16x8 type; };
template <> struct FragOf<float> { typedef f32x8 type; };

__device__ __forceinline__ bf16x8 load_frag(const bf16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ f32x8 load_frag(const float* p) {
  const f32x4* q = reinterpret_cast<const f32x4*>(p);
  f32x4 a = q[0], b = q[1];
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// Fragment from two runs of 4 consecutive elements (elements 0..3 from p, 4..7 from q).
__device__ __forceinline__ bf16x8 load_frag_split4(const bf16* p, const bf16* q) {
  u32x2 a = *reinterpret_cast<const u32x2*>(p), b = *reinterpret_cast<const u32x2*>(q);
  return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}
__device__ __forceinline__ f32x8 load_frag_split4(const float* p, const float* q) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(q);
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
template <class T> __device__ __forceinline__ typename FragOf<T>::type zero_frag() {
  return typename FragOf<T>::type{};
}

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(f32x8 a, f32x8 b, f32x4 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

// ---- fragment-native ("swizzled") matrix layout
// A matrix X [R][K] (R a multiple of 16, K of 32) is stored block by block: the 16 x 32
// block (row tile rt = r / 16, k-block kb = k / 32) occupies 64 lanes x 8 contiguous
// elements, lane = 16 * ((k % 32) / 8) + r % 16 -- exactly the MFMA fragment each lane of
// a wave holds -- so a wave loads one block with a single contiguous 16 B/lane access.
// Blocks are ordered row tile major, k-block minor.  Stacks of matrices whose row count is
// a multiple of 16 are stacks of swizzled matrices.
__host__ __device__ __forceinline__ size_t sw_idx(int r, int k, int K) {
  return ((((size_t)(r >> 4) * (size_t)(K >> 5) + (size_t)(k >> 5)) * 64 + ((k >> 3) & 3) * 16 + (r & 15)) << 3) +
         (size_t)(k & 7);
}
__device__ __forceinline__ size_t sw_frag(int rt, int kb, int K, int lane) {
  return (((size_t)rt * (size_t)(K >> 5) + (size_t)kb) * 64 + lane) << 3;
}
// int4 weights: per (row tile, 128-wide quad) each lane owns one 16-byte slot whose word j
// holds its 8 codes of k-block j of the quad.  Inside a word, the offset-binary code
// (q + 8) of element 2i sits in bits [4i, 4i+4) and that of element 2i+1 in [16+4i, 20+4i).
__host__ __device__ __forceinline__ size_t sw4_word(int r, int k, int K) {
  return ((((size_t)(r >> 4) * (size_t)(K >> 7) + (size_t)(k >> 7)) * 64 + ((k >> 3) & 3) * 16 + (r & 15)) << 2) +
         (size_t)((k >> 5) & 3);
}
__host__ __device__ __forceinline__ int sw4_shift(int k) {
  const int e = k & 7;
  return (e & 1) ? 16 + 4 * (e >> 1) : 4 * (e >> 1);
}

// fp32 -> storage element (bf16: round to nearest even).
// Store of an activation that a later launch reads.  WT: write-through (agent scope), the
// line goes out to memory at once instead of staying dirty in this XCD's L2 until the
// write-back at the end of the kernel -- cheaper for the few kilobytes a weight-streaming
// GEMM's workgroup writes, dearer for the megabytes of a tiled GEMM's.
template <bool WT, class T>
__device__ __forceinline__ void st_act(T* p, T v) {
  if constexpr (!WT) {
    *p = v;
  } else if constexpr (sizeof(T) == 4) {
    __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __builtin_bit_cast(uint32_t, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  } else {
    __hip_atomic_store(reinterpret_cast<uint16_t*>(p), __builtin_bit_cast(uint16_t, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}
template <class T> __device__ __forceinline__ T to_elem(float v);
template <> __device__ __forceinline__ float to_elem<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 to_elem<bf16>(float v) { return (bf16)v; }

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Wave-wide butterfly reductions (wave64).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Value of another lane of the same 16-lane row (DPP, no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// Sum over the 16 lanes of a DPP row (lanes 16 g .. 16 g + 15): lane ^ 1 and lane ^ 2 within
// each quad, then the row rotated by 4 and by 8.  Every lane ends with the row's total (the
// association may differ between lanes in the last bit; callers take one lane's value).
__device__ __forceinline__ float sum16(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_mov<0x124>(v);  // row_ror 4
  v += dpp_mov<0x128>(v);  // row_ror 8
  return v;
}

__device__ __forceinline__ float gelu_tanh(float z) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  return 0.5f * z * (1.0f + tanhf(c * (z + 0.044715f * z * z * z)));
}

// ---- cross-workgroup hand-off inside one kernel
// Partial results that another workgroup reads within the same kernel are written
// and read with relaxed agent-scope atomics (gfx950: global_store/load ... sc1), which
// are coherent across the XCDs' separate L2s.  Before a participant signals arrival it
// waits for its own stores to complete (s_waitcnt 0); the arrival counter is an
// agent-scope atomic.  This avoids the whole-L2 write-back/invalidate that a
// device-scope fence costs on this chip.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st_agent(float* p, f32x4 v) {
  uint64_t* q = reinterpret_cast<uint64_t*>(p);
  __hip_atomic_store(q, __builtin_bit_cast(uint64_t, f32x2{v[0], v[1]}), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, __builtin_bit_cast(uint64_t, f32x2{v[2], v[3]}), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x4 ld_agent4(const float* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  f32x2 a = __builtin_bit_cast(f32x2, __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  f32x2 b = __builtin_bit_cast(f32x2, __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  return f32x4{a[0], a[1], b[0], b[1]};
}
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte agent-scope accesses through a raw buffer resource (buffer_load/store ... sc1):
// same coherence as the atomics above, four times the width of a 64-bit atomic.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t agent_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ f32x4 ld_agent16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 16));
}
__device__ __forceinline__ void st_agent16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, byte_off, 0, 16);
}

// 2^x on the hardware exponential (v_exp_f32) without the range scaling of exp2f for
// results below 2^-126: softmax weights that small count as zero.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_all_mem() { __builtin_amdgcn_s_waitcnt(0); }

// Wait until at most N of this wave's vector-memory operations are outstanding (loads
// complete in issue order), leaving the LDS and export counters alone.  gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Arrival of one workgroup (all threads call it) at a split reduction with n_parts
// participants.  True for exactly the last arrival; that workgroup resets the counter.
__device__ __forceinline__ bool split_arrive_wg(unsigned* counter, unsigned n_parts, unsigned* lds_flag) {
  wait_all_mem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned last = (old == n_parts - 1) ? 1u : 0u;
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *lds_flag = last;
  }
  __syncthreads();
  return *lds_flag != 0;
}
// Same for one wave (all 64 lanes call it).
__device__ __forceinline__ bool split_arrive_wave(unsigned* counter, unsigned n_parts) {
  wait_all_mem();
  unsigned old = 0;
  if ((threadIdx.x & 63) == 0) {
    old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == n_parts - 1) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  old = __shfl(old, 0, 64);
  return old == n_parts - 1;
}

}  // namespace phyai
