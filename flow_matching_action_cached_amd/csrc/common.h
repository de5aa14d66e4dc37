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

// fp32 -> storage element (bf16: round to nearest even).
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
// Sum over the 16 lanes that share a lane group (xor 1..8).
__device__ __forceinline__ float sum16(float v) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float gelu_tanh(float z) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  return 0.5f * z * (1.0f + tanhf(c * (z + 0.044715f * z * z * z)));
}

// Split-reduction arrival: every participant calls this after writing its partial.
// Returns true for exactly one caller (the last to arrive), which may then read all
// partials.  The counter is reset by that caller, so it is 0 again for the next use.
// Must be called by all threads of a workgroup (wg = true) or of one wave (wg = false).
template <bool WG>
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned n_parts, unsigned* lds_flag) {
  __threadfence();  // release this participant's partial stores at device scope
  if (WG) {
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned old = atomicAdd(counter, 1u);
      bool last = (old == n_parts - 1);
      if (last) atomicExch(counter, 0u);
      *lds_flag = last ? 1u : 0u;
    }
    __syncthreads();
    bool last = *lds_flag != 0;
    if (last) __threadfence();  // acquire the other participants' partials
    return last;
  } else {
    unsigned old = 0;
    if ((threadIdx.x & 63) == 0) {
      old = atomicAdd(counter, 1u);
      if (old == n_parts - 1) atomicExch(counter, 0u);
    }
    old = __shfl(old, 0, 64);
    bool last = (old == n_parts - 1);
    if (last) __threadfence();
    return last;
  }
}

}  // namespace phyai
