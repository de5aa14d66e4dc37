// One-off kernels (outside the Euler loop): timestep embedding and modulation
// tables, the norm-folded shift projections, prefix K/V installation, and the
// offline int4 quantiser / repacker.
//
// Tables (PhyAI reading "PhyAI: Real-Time Physical AI at the Edge, Scalable
// Rollouts in the Cloud", Sec. 5.1: timestep/modulation tables over the fixed
// schedule are precomputed once) are computed in fp64 and stored as fp32.
#include "common.h"
#include "kernels.h"

#include <math.h>

#include <algorithm>

namespace phyai {

// Scalar weight read for the table kernels.  Expert linears are stored swizzled (see
// common.h); the in/out projections are plain row-major.
template <class WT, bool SW> struct WRow {
  const WT* w;
  const uint16_t* s;
  int K;
  __device__ float at(size_t n, int k) const {
    return SW ? to_f32(w[sw_idx((int)n, k, K)]) : to_f32(w[n * K + k]);
  }
};
template <bool SW> struct WRow<i4, SW> {
  const i4* w;
  const uint16_t* s;
  int K;
  __device__ float at(size_t n, int k) const {
    const uint32_t word = reinterpret_cast<const uint32_t*>(w)[sw4_word((int)n, k, K)];
    const int q = (int)((word >> sw4_shift(k)) & 0xFu) - 8;
    return (float)q * bf16_bits_to_f32(s[n * (K / 128) + k / 128]);
  }
};

// ------------------------------------------------------------------ timestep / modulation tables
// Embedding e(t_k) in fp64: e_i = sin(2 pi t / p_i), e_{D/2+i} = cos(2 pi t / p_i),
// p_i = 4e-3 * 1000^(i / (D/2 - 1)).
__global__ void k_embed(const float* t, int N, int D, double* e) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= N * D) return;
  const int k = idx / D, c = idx % D, half = D / 2;
  const int i = c % half;
  const double period = 4e-3 * pow(1000.0, (double)i / (double)(half - 1));
  const double ang = 2.0 * M_PI * (double)t[k] / period;
  e[idx] = c < half ? sin(ang) : cos(ang);
}

// Time MLP layer (fidelity variant): out[k][o] = act(W[o] . in[k] + b[o]) for every step k,
// accumulated in fp64; act = swish (z / (1 + exp(-z))) for the first layer, identity for the
// second.  One wave per output row o.
template <class IOT>
__global__ __launch_bounds__(256) void k_time_mlp(const IOT* w, const IOT* bias, const double* in, int N, int D,
                                                  int swish, double* out) {
  const int lane = threadIdx.x & 63;
  const int o = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (o >= D) return;
  const IOT* wr = w + (size_t)o * D;
  const double b = (double)to_f32(bias[o]);
  for (int k0 = 0; k0 < N; k0 += 8) {
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int c = lane; c < D; c += 64) {
      const double wv = (double)to_f32(wr[c]);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        if (k0 + kk < N) acc[kk] += wv * in[(size_t)(k0 + kk) * D + c];
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const double v = wave_sum(acc[kk]) + b;
      if (lane == 0 && k0 + kk < N) out[(size_t)(k0 + kk) * D + o] = swish ? v / (1.0 + exp(-v)) : v;
    }
  }
}

// One wave per (table tb, row o of W_mod[j]) (j = norm, o in [0, R D): scale, shift and,
// with R = 3, the residual gate):
// m_k = W_mod[j][o] . (e(t_k) + cond_tb) + b_mod[j][o] for every step k, accumulated in fp64.
// cond (io [ntab][D]) may be null (no condition: a single table).
template <class IOT>
__global__ __launch_bounds__(256) void k_modulation(const IOT* w_mod, const IOT* b_mod, const IOT* cond,
                                                    const double* e, int N, int nmod, int D, int ntab, int R,
                                                    float* mod, float* gate) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= ntab * nmod * R * D) return;
  const int tb = row / (nmod * R * D), wrow = row % (nmod * R * D);
  const int j = wrow / (R * D), o = wrow % (R * D);
  const IOT* wr = w_mod + (size_t)wrow * D;
  const double bias = (double)to_f32(b_mod[wrow]);
  for (int k0 = 0; k0 < N; k0 += 8) {
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int c = lane; c < D; c += 64) {
      const double wv = (double)to_f32(wr[c]);
      const double cv = cond ? (double)to_f32(cond[(size_t)tb * D + c]) : 0.0;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        if (k0 + kk < N) acc[kk] += wv * (e[(size_t)(k0 + kk) * D + c] + cv);
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const double v = wave_sum(acc[kk]);
      if (lane == 0 && k0 + kk < N) {
        if (o < 2 * D)
          mod[((((size_t)(k0 + kk) * ntab + tb) * nmod + j) * 2 + (o >= D ? 1 : 0)) * D + (o % D)] = (float)(v + bias);
        else
          gate[(((size_t)(k0 + kk) * ntab + tb) * nmod + j) * D + (o - 2 * D)] = (float)(v + bias);
      }
    }
  }
}

// Norm-folded biases: for every step k and table tb, c = W shift_j(t_k) for the QKV rows
// (j = 2l), the gate/up rows (j = 2l+1) and the out-projection rows (j = 2L; the joint
// denoiser has latent then action out-projection rows).  One wave per (table, row).
template <class WT, class IOT>
__global__ __launch_bounds__(256) void k_shift_proj(Dims d, Bufs bf, const float* mod, float* cvec, int n_out1,
                                                    int n_out2) {
  const int lane = threadIdx.x & 63;
  const int nq = d.L * d.qkv, ng = d.L * 2 * d.F;
  const int per_tab = nq + ng + n_out1 + n_out2;
  const int row0 = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row0 >= d.ntab * per_tab) return;
  const int tb = row0 / per_tab, row = row0 % per_tab;
  WRow<WT, true> wq{static_cast<const WT*>(bf.w_qkv), bf.s_qkv, d.D};
  WRow<WT, true> wg{static_cast<const WT*>(bf.w_gu), bf.s_gu, d.D};
  WRow<IOT, false> wo{static_cast<const IOT*>(bf.w_out), nullptr, d.D};
  WRow<IOT, false> wo2{static_cast<const IOT*>(bf.w_out2), nullptr, d.D};
  int which, j, off;
  size_t n;
  if (row < nq) {
    which = 0; n = row; j = 2 * (row / d.qkv); off = row;
  } else if (row < nq + ng) {
    which = 1; n = row - nq; j = 2 * ((row - nq) / (2 * d.F)) + 1; off = bf.cv_gu_off + (row - nq);
  } else if (row < nq + ng + n_out1) {
    which = 2; n = row - nq - ng; j = 2 * d.L; off = bf.cv_out_off + (row - nq - ng);
  } else {
    which = 3; n = row - nq - ng - n_out1; j = 2 * d.L; off = bf.cv_out_off + (row - nq - ng);
  }
  for (int k0 = 0; k0 < d.N; k0 += 8) {
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int c = lane; c < d.D; c += 64) {
      const double wv = which == 0 ? wq.at(n, c) : which == 1 ? wg.at(n, c) : which == 2 ? wo.at(n, c) : wo2.at(n, c);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        if (k0 + kk < d.N)
          acc[kk] += wv * (double)mod[((((size_t)(k0 + kk) * d.ntab + tb) * d.nmod + j) * 2 + 1) * d.D + c];
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const double v = wave_sum(acc[kk]);
      if (lane == 0 && k0 + kk < d.N) cvec[((size_t)(k0 + kk) * d.ntab + tb) * bf.cv_stride + off] = (float)v;
    }
  }
}

// ------------------------------------------------------------------ prefix install
// K [B][L][P][Hkv][dh] -> cache [b][l][r][p][dh];  V -> V^T cache [b][l][r][dh][p].
template <class T>
__global__ void k_install_prefix(Dims d, const T* k, const T* v, int B, int P, T* kc, T* vt) {
  const size_t total = (size_t)B * d.L * d.Hkv * d.dh * P;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    // V^T write order: p fastest
    size_t rem = idx;
    const int p = rem % P; rem /= P;
    const int dd = rem % d.dh; rem /= d.dh;
    const int r = rem % d.Hkv; rem /= d.Hkv;
    const int l = rem % d.L;
    const int b = rem / d.L;
    const size_t src = ((((size_t)b * d.L + l) * P + p) * d.Hkv + r) * d.dh + dd;
    const size_t cb = ((size_t)b * d.L + l) * d.Hkv + r;
    vt[(cb * d.dh + dd) * d.KS + p] = v[src];
    // K with dh fastest: reuse the same index space transposed
    const int dd2 = idx % d.dh;
    size_t rem2 = idx / d.dh;
    const int p2 = rem2 % P;
    rem2 /= P;
    const size_t cb2 = rem2;  // (b*L + l)*Hkv + r
    const int r2 = cb2 % d.Hkv;
    const size_t bl2 = cb2 / d.Hkv;
    kc[(cb2 * d.KS + p2) * d.dh + dd2] = k[((bl2 * P + p2) * d.Hkv + r2) * d.dh + dd2];
  }
}

// ------------------------------------------------------------------ execution-state capsules
// Prefix rows of the caches <-> packed capsule payload (K [B][L][Hkv][P][dh], then V^T
// [B][L][Hkv][dh][P]).  Both halves are pitched row copies: K has B*L*Hkv rows of P*dh
// elements at cache pitch KS*dh, V^T has B*L*Hkv*dh rows of P elements at pitch KS.  The
// copy moves U-sized units (16 bytes when every row, pitch and base allows it), one unit per
// thread per grid-stride pass; blockIdx.y picks the half.
struct RowCopy {
  const char* src;
  char* dst;
  size_t rows, units, spitch, dpitch;  // units per row and pitches in units of U
};

template <class U>
__global__ __launch_bounds__(256) void k_capsule_rows(RowCopy k, RowCopy v) {
  const RowCopy& c = blockIdx.y == 0 ? k : v;
  const U* src = reinterpret_cast<const U*>(c.src);
  U* dst = reinterpret_cast<U*>(c.dst);
  const size_t total = c.rows * c.units;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / c.units, u = i - r * c.units;
    dst[r * c.dpitch + u] = src[r * c.spitch + u];
  }
}

struct CapsuleWords {
  uint32_t w[16];
};
__global__ void k_capsule_header(CapsuleWords h, int n, uint32_t* dst) {
  if ((int)threadIdx.x < n) dst[threadIdx.x] = h.w[threadIdx.x];
}

hipError_t enqueue_capsule_header(const uint32_t* words, int n, void* dst, hipStream_t st) {
  if (n < 1 || n > 16) return hipErrorInvalidValue;
  CapsuleWords h{};
  for (int i = 0; i < n; ++i) h.w[i] = words[i];
  hipLaunchKernelGGL(k_capsule_header, dim3(1), dim3(64), 0, st, h, n, static_cast<uint32_t*>(dst));
  return hipGetLastError();
}

// Zero-fill of a float range (pad slots of a bucketed batch): a kernel rather than a memset,
// so that a caller capturing the denoise call into a graph records no memset node.
__global__ __launch_bounds__(256) void k_zero_f32(float* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0.f;
}

hipError_t enqueue_zero_f32(float* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

// One wave that returns after `ticks` of the 100 MHz real-time counter (a bounded wait:
// measurement code queues work behind it so that the queue runs back to back).
__global__ void k_delay(uint64_t ticks) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (__builtin_amdgcn_s_memrealtime() - t0 < ticks) __builtin_amdgcn_s_sleep(10);
}

hipError_t enqueue_delay_us(unsigned us, hipStream_t st) {
  hipLaunchKernelGGL(k_delay, dim3(1), dim3(64), 0, st, (uint64_t)us * 100u);
  return hipGetLastError();
}

hipError_t enqueue_capsule_copy(const Dims& d, void* kc, void* vt, void* payload, int batch, int prefix_len,
                                size_t es, bool save, hipStream_t st) {
  const size_t heads = (size_t)batch * d.L * d.Hkv;
  if (heads == 0 || prefix_len == 0) return hipSuccess;
  char* pay = static_cast<char*>(payload);
  // byte geometry of the two halves: {rows, row bytes, cache pitch}
  const size_t kb = (size_t)prefix_len * d.dh * es, kp = (size_t)d.KS * d.dh * es;
  const size_t vb = (size_t)prefix_len * es, vp = (size_t)d.KS * es;
  char* pk = pay;
  char* pv = pay + heads * kb;
  size_t unit = 16;
  for (; unit > es; unit /= 2) {
    const size_t m = unit - 1;
    if (!((kb | kp | vb | vp) & m) && !(((uintptr_t)kc | (uintptr_t)vt | (uintptr_t)pk | (uintptr_t)pv) & m)) break;
  }
  auto plan = [&](char* cache, char* packed, size_t rows, size_t rb, size_t pitch) {
    RowCopy r;
    r.rows = rows;
    r.units = rb / unit;
    r.src = save ? cache : packed;
    r.dst = save ? packed : cache;
    r.spitch = (save ? pitch : rb) / unit;
    r.dpitch = (save ? rb : pitch) / unit;
    return r;
  };
  const RowCopy ck = plan(static_cast<char*>(kc), pk, heads, kb, kp);
  const RowCopy cv = plan(static_cast<char*>(vt), pv, heads * d.dh, vb, vp);
  const size_t units = ck.rows * ck.units;  // the same for both halves
  const int blocks = (int)std::min<size_t>((units + 255) / 256, 4096);
  const dim3 grid(blocks, 2);
  switch (unit) {
    case 16: hipLaunchKernelGGL(k_capsule_rows<uint4>, grid, dim3(256), 0, st, ck, cv); break;
    case 8: hipLaunchKernelGGL(k_capsule_rows<uint2>, grid, dim3(256), 0, st, ck, cv); break;
    case 4: hipLaunchKernelGGL(k_capsule_rows<uint32_t>, grid, dim3(256), 0, st, ck, cv); break;
    default: hipLaunchKernelGGL(k_capsule_rows<uint16_t>, grid, dim3(256), 0, st, ck, cv); break;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ int4 quantiser and repack
// One wave per (row, 128-column group); lane i quantises columns 2i, 2i+1 and writes one byte.
__global__ __launch_bounds__(256) void k_quantize_int4(const float* w, int64_t rows, int64_t cols,
                                                       uint8_t* packed, uint16_t* scales) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t ng = cols / 128;
  if (item >= rows * ng) return;
  const int64_t row = item / ng, gi = item % ng;
  const float* src = w + row * cols + gi * 128 + 2 * lane;
  const float a = src[0], b = src[1];
  float mx = fmaxf(fabsf(a), fabsf(b));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  const float s32 = mx / 7.0f;
  // bf16 round to nearest even of s32
  uint32_t u = __builtin_bit_cast(uint32_t, s32);
  u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  const float s = __builtin_bit_cast(float, u << 16);
  int qa = 0, qb = 0;
  if (s > 0.f) {
    qa = (int)fminf(fmaxf(rintf(a / s), -8.f), 7.f);
    qb = (int)fminf(fmaxf(rintf(b / s), -8.f), 7.f);
  }
  packed[row * (cols / 2) + gi * 64 + lane] = (uint8_t)((qa & 0xF) | ((qb & 0xF) << 4));
  if (lane == 0) scales[row * ng + gi] = (uint16_t)u;
}

// Row-major [rows][K] -> swizzled layout (rows a multiple of 16).  One thread per element.
template <class T>
__global__ void k_swizzle(const T* src, T* dst, int64_t rows, int K) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * K) return;
  const int64_t r = i / K;
  const int k = (int)(i % K);
  // rows are handled 16 at a time (r >> 4 < 2^31 for any arena that fits the device)
  dst[(size_t)(r >> 4) * 16 * K + sw_idx((int)(r & 15), k, K)] = src[i];
}

// ABI int4 (byte j of a row: input 2j in the low nibble, 2j+1 in the high nibble, two's
// complement) -> swizzled words (sw4_word / sw4_shift, offset binary).  One thread per word.
__global__ void k_swizzle_int4(const uint8_t* src, uint32_t* dst, int64_t rows, int K) {
  const int64_t words = rows * (K / 8);
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= words) return;
  // decode the word index: [row tile][quad][lane = g*16 + r16][j]
  const int64_t per_tile = (int64_t)(K / 128) * 64 * 4;
  const int64_t rt = i / per_tile;
  int64_t rem = i % per_tile;
  const int q = (int)(rem / 256);
  rem %= 256;
  const int lane = (int)(rem / 4), j = (int)(rem % 4);
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t row = rt * 16 + r16;
  const int k0 = q * 128 + j * 32 + g * 8;
  const uint8_t* b = src + row * (K / 2) + k0 / 2;
  uint32_t out = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t nib = ((e & 1) ? (b[e >> 1] >> 4) : b[e >> 1]) & 0xFu;
    out |= (nib ^ 0x8u) << sw4_shift(k0 + e);
  }
  dst[i] = out;
}

// ================================================================== host side
template <class WT, class IOT>
static hipError_t tables_impl(const Dims& d, const Bufs& b, const float* t_dev, double* e, float* mod,
                              float* cvec, float* gate, hipStream_t st) {
  const int ne = d.N * d.D;
  hipLaunchKernelGGL(k_embed, dim3((ne + 255) / 256), dim3(256), 0, st, t_dev, d.N, d.D, e);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (d.tmlp) {  // e -> swish(W1 e + b1) -> W2 (.) + b2, in the scratch after e
    const double* e0 = e;
    double* e1 = e + (size_t)d.N * d.D;
    double* e2 = e1 + (size_t)d.N * d.D;
    hipLaunchKernelGGL((k_time_mlp<IOT>), dim3((d.D + 3) / 4), dim3(256), 0, st, static_cast<const IOT*>(b.w_tm1),
                       static_cast<const IOT*>(b.b_tm1), e0, d.N, d.D, 1, e1);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL((k_time_mlp<IOT>), dim3((d.D + 3) / 4), dim3(256), 0, st, static_cast<const IOT*>(b.w_tm2),
                       static_cast<const IOT*>(b.b_tm2), e1, d.N, d.D, 0, e2);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    e = e2;
  }
  const int R = d.gated ? 3 : 2;
  if (d.gated && !gate) return hipErrorInvalidValue;
  const int rows = d.ntab * d.nmod * R * d.D;
  hipLaunchKernelGGL((k_modulation<IOT>), dim3((rows + 3) / 4), dim3(256), 0, st, static_cast<const IOT*>(b.w_mod),
                     static_cast<const IOT*>(b.b_mod), static_cast<const IOT*>(b.cond), e, d.N, d.nmod, d.D, d.ntab,
                     R, mod, gate);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  // out-projection rows: the expert has A; the joint denoiser has Cl latent + A action rows
  const int n_out1 = d.joint ? d.Cl : d.A, n_out2 = d.joint ? d.A : 0;
  const int rows2 = d.ntab * (d.L * d.qkv + d.L * 2 * d.F + n_out1 + n_out2);
  hipLaunchKernelGGL((k_shift_proj<WT, IOT>), dim3((rows2 + 3) / 4), dim3(256), 0, st, d, b, mod, cvec, n_out1,
                     n_out2);
  return hipGetLastError();
}

hipError_t enqueue_tables(const Dims& d, const Bufs& b, WDtype wt, const float* t_dev, double* e,
                          float* mod, float* cvec, float* gate, hipStream_t st) {
  switch (wt) {
    case W_F32: return tables_impl<float, float>(d, b, t_dev, e, mod, cvec, gate, st);
    case W_BF16: return tables_impl<bf16, bf16>(d, b, t_dev, e, mod, cvec, gate, st);
    case W_INT4: return tables_impl<i4, bf16>(d, b, t_dev, e, mod, cvec, gate, st);
  }
  return hipErrorInvalidValue;
}

hipError_t enqueue_install_prefix(const Dims& d, const void* k, const void* v, int batch, int P, void* kc,
                                  void* vt, size_t es, hipStream_t st) {
  const size_t total = (size_t)batch * d.L * d.Hkv * d.dh * P;
  const int blocks = (int)std::min<size_t>((total + 255) / 256, 65536);
  if (es == 4)
    hipLaunchKernelGGL(k_install_prefix<float>, dim3(blocks), dim3(256), 0, st, d, static_cast<const float*>(k),
                       static_cast<const float*>(v), batch, P, static_cast<float*>(kc), static_cast<float*>(vt));
  else
    hipLaunchKernelGGL(k_install_prefix<uint16_t>, dim3(blocks), dim3(256), 0, st, d,
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), batch, P,
                       static_cast<uint16_t*>(kc), static_cast<uint16_t*>(vt));
  return hipGetLastError();
}

hipError_t enqueue_quantize_int4(const float* w, int64_t rows, int64_t cols, uint8_t* packed, uint16_t* scales,
                                 hipStream_t st) {
  const int64_t items = rows * (cols / 128);
  if (items == 0) return hipSuccess;
  hipLaunchKernelGGL(k_quantize_int4, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, st, w, rows, cols, packed,
                     scales);
  return hipGetLastError();
}

hipError_t enqueue_swizzle(const void* src, void* dst, int64_t rows, int K, size_t es, hipStream_t st) {
  const int64_t n = rows * K;
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (es == 4)
    hipLaunchKernelGGL(k_swizzle<float>, dim3(blocks), dim3(256), 0, st, static_cast<const float*>(src),
                       static_cast<float*>(dst), rows, K);
  else
    hipLaunchKernelGGL(k_swizzle<uint16_t>, dim3(blocks), dim3(256), 0, st, static_cast<const uint16_t*>(src),
                       static_cast<uint16_t*>(dst), rows, K);
  return hipGetLastError();
}

hipError_t enqueue_swizzle_int4(const uint8_t* src, uint8_t* dst, int64_t rows, int K, hipStream_t st) {
  const int64_t words = rows * (K / 8);
  if (words == 0) return hipSuccess;
  hipLaunchKernelGGL(k_swizzle_int4, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, st, src,
                     reinterpret_cast<uint32_t*>(dst), rows, K);
  return hipGetLastError();
}

}  // namespace phyai
