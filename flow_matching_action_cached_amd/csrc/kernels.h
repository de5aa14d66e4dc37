// Internal interface between the host runtime (runtime.cpp) and the HIP kernels
// (loop.hip, gemv.hip, attention.hip, update.hip, gemm_tiled.hip, tables.hip).  Not part of
// the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace phyai {

enum WDtype { W_F32 = 0, W_BF16 = 1, W_INT4 = 2 };

// Model, batch and schedule dimensions of one denoise launch.
struct Dims {
  int L, D, Hq, Hkv, dh, F, A, H;  // layers, width, heads, head_dim, MLP dim, action dim, chunk
  int B, M, Mst;                   // batch, token rows (B*H), row stride of ssq (>= M)
  int P, KS;                       // prefix length, key stride of the cache (>= P + H)
  int qkv, nmod;                   // (Hq + 2 Hkv) * dh, 2L + 1
  int N;                           // Euler steps
  float eps;
  int Lc;                          // layers held by the KV cache (L; 1 when no cache is kept)
  int ntab, rows_per_tab;          // modulation tables (1; 2 for a guided pair), token rows per table
  int joint;                       // 1: joint video/action denoiser (no prefix, guided branch pair)
  int Tl, Cl;                      // joint denoiser: latent tokens and their channels (0 otherwise)
  float gamma;                     // joint denoiser: guidance scale
  float rope_theta;                // > 0: rotary embedding of the chunk's Q/K at positions P + t
  int gated;                       // 1: each norm's map also yields a residual gate (3 D rows per norm)
  int tmlp;                        // 1: the timestep embedding passes the time MLP first
  int solver;                      // joint denoiser: 0 Euler, 1 or 2 UniPC predictor order
};

// Device pointers of one context.  Element types depend on the weight dtype:
// "io" = fp32 (F32) or bf16 (BF16, INT4); "act" = fp32 (F32) or bf16 (BF16, INT4);
// expert linears: fp32 / bf16 / repacked int4 codes + bf16 scales.
struct Bufs {
  const void *w_in, *b_in, *w_out, *b_out, *w_mod, *b_mod;  // io (joint denoiser: latent projections)
  const void *w_in2, *b_in2, *w_out2, *b_out2;              // joint denoiser: action projections
  const void* cond;                                         // [ntab][D] io: added to the embedding
  const void *w_tm1, *b_tm1, *w_tm2, *b_tm2;                // time MLP (io [D][D], [D]; tmlp only)
  const void *w_qkv, *w_o, *w_gu, *w_d;                     // expert linears
  const uint16_t *s_qkv, *s_o, *s_gu, *s_d;                 // int4 scales (bf16 bits)
  void *kc, *vt;          // K cache [Bmax][L][Hkv][KS][dh], V^T cache [Bmax][L][Hkv][dh][KS] (act)
  const float* mod;       // [N][ntab][nmod][2][D] (scale, shift)
  const float* gate;      // [N][ntab][nmod][D] residual gates (gated variant; null otherwise)
  const float* uni;       // UniPC: [N][8] per step t_k, corrector (A, w_new, w_k-1, w_k-2), predictor (A, w_k, w_k-1)
  float* ust;             // UniPC state: corrected z_{k-1}, then two data-prediction slots (3 x E floats)
  const float* cvec;      // [N][ntab][cv_stride]: W_qkv shift_2l | W_gu shift_2l+1 | W_out shift_2L
  const float* dt;        // [N]
  int cv_stride, cv_gu_off, cv_out_off;
  float *x, *h, *ssq;     // state [M][A], residual [M][D], row sum-of-squares partials [Mst][D/16]
  float* x2;              // joint denoiser: action state [Ta][A] (x holds the latents [Tl][Cl])
  void *hs, *q, *o, *act; // act-typed: hs [Mpad][D], o [Mpad][Hq dh], act [Mpad][F] swizzled; q [M][Hq dh]
  float* attn_ws; unsigned* attn_cnt;
  float* gemm_ws; unsigned* gemm_cnt;
};

// Launch shape of the split reductions (chosen by the host once per context).
struct Plan {
  int s_qkv, s_o, s_gu, s_d;  // k-splits across workgroups per linear
  int attn_bps;               // 32-key blocks per attention split
  int attn_wide;              // 1: many query tiles, shared-staging attention kernel
};

// Scratch sizes the plan needs (floats / counters).
size_t attn_ws_floats(const Dims& d, const Plan& p);
size_t attn_counters(const Dims& d);
size_t gemm_ws_floats(const Dims& d, const Plan& p);
size_t gemm_counters(const Dims& d);
size_t tiled_split_ws_floats(const Dims& d);  // split scratch of the tiled residual GEMMs (floats)
size_t tiled_split_counters(const Dims& d);
Plan make_plan(const Dims& d, WDtype wt);

// Measurement marks: with them, enqueue_denoise records ev[0] before the first launch and
// ev[i] after launch i (kind[i] = its kernel id as in enqueue_one, kind[0] = -1); cap is the
// number of events available (1 + N (6 L + 1) + 1 are needed).
struct LaunchMarks {
  hipEvent_t* ev;
  int* kind;
  int n, cap;
};

// Enqueue the whole Euler loop (N steps) on `stream`.  x must already hold the noise.
hipError_t enqueue_denoise(const Dims& d, const Bufs& b, const Plan& p, WDtype wt, hipStream_t stream,
                           LaunchMarks* marks = nullptr);

// Enqueue one launch of loop kernel `which` (0 QKV, 1 attention, 2 O, 3 gate/up, 4 down,
// 5 out/Euler/in-projection, 6 first in-projection) with the arguments of step k, layer l.
hipError_t enqueue_one(const Dims& d, const Bufs& b, const Plan& p, WDtype wt, int which, int k, int l,
                       hipStream_t stream);

// Prefix prefill: the dims of running the layer stack over batch x prefix_len prefix rows with
// no cached keys (their K/V land in cache rows [0, prefix_len) of every layer), and the
// enqueue of the whole prefill on `stream`: input kernel, then the layers' launches.  b holds
// the prefix network's linears and zero modulation tables (plain RMSNorm).
Dims prefill_dims(const Dims& base, int batch, int prefix_len);
hipError_t enqueue_prefill(const Dims& d, const Bufs& b, const Plan& p, WDtype wt, const void* tokens,
                           hipStream_t stream);

// Execution-state capsule payload: the prefix rows [0, P) of the K and V^T caches of `batch`
// samples, packed as K [batch][L][Hkv][P][dh] then V^T [batch][L][Hkv][dh][P] (elements of
// elem_bytes).  save: cache -> capsule; restore: capsule -> cache.
// Writes a capsule header (n <= 16 32-bit words, passed by value) at dst, stream-ordered.
hipError_t enqueue_capsule_header(const uint32_t* words, int n, void* dst, hipStream_t stream);
hipError_t enqueue_capsule_copy(const Dims& d, void* kc, void* vt, void* payload, int batch, int prefix_len,
                                size_t elem_bytes, bool save, hipStream_t stream);

// Joint video/action denoiser (bf16): whole guided loop, and one launch of a loop kernel.
hipError_t enqueue_wam_denoise(const Dims& d, const Bufs& b, const Plan& p, hipStream_t stream);
hipError_t enqueue_wam_one(const Dims& d, const Bufs& b, const Plan& p, int which, int k, int l,
                           hipStream_t stream);

// Zero n floats at p (stream-ordered kernel; no memset node when a caller captures it).
hipError_t enqueue_zero_f32(float* p, size_t n, hipStream_t stream);
// A one-wave kernel that returns after `us` microseconds (bounded wait for measurements).
hipError_t enqueue_delay_us(unsigned us, hipStream_t stream);

// One-off kernels.  With Dims::tmlp, e_scratch holds 3 N D doubles (embedding, hidden, MLP output).
hipError_t enqueue_tables(const Dims& d, const Bufs& b, WDtype wt, const float* t_dev, double* e_scratch,
                          float* mod_out, float* cvec_out, float* gate_out, hipStream_t stream);
hipError_t enqueue_install_prefix(const Dims& d, const void* k, const void* v, int batch, int prefix_len,
                                  void* kc, void* vt, size_t elem_bytes, hipStream_t stream);
hipError_t enqueue_quantize_int4(const float* w, int64_t rows, int64_t cols, uint8_t* packed,
                                 uint16_t* scales, hipStream_t stream);
// Weight layout conversion at load time (see the swizzled layout in common.h).
hipError_t enqueue_swizzle(const void* src, void* dst, int64_t rows, int K, size_t elem_bytes, hipStream_t stream);
hipError_t enqueue_swizzle_int4(const uint8_t* src, uint8_t* dst, int64_t rows, int K, hipStream_t stream);

}  // namespace phyai
