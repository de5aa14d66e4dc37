// Launchers of the Euler loop's kernel families, for the host side of the loop (loop.hip).
#pragma once

#include "epilogue.h"

namespace phyai {

// Weight-streaming GEMM of one linear (<= 64 token rows): tiles output column tiles of 16
// (gate/up: 16 gate + 16 up columns), epi an Epi, weights of type wt (activations bf16, or
// fp32 with fp32 weights).
hipError_t launch_gemv(const Dims& d, const Bufs& b, const GemmLaunch& g, WDtype wt, int epi, int tiles,
                       hipStream_t st);

// Attention of layer `layer`: part 0 the attention kernel, part 1 the merge of its key splits
// (a launch only for the few-row kernel with more than one split).  f32: fp32 activations.
hipError_t launch_attention(const Dims& d, const Bufs& b, const Plan& p, int layer, int part, bool f32,
                            hipStream_t st);
// Query tiles per workgroup of the many-row attention kernel.
int attn_wide_tiles(int dh);

// Final norm + out-projection + state update of step k_prev (k_prev >= 0) and in-projection
// of step k_next (k_next >= 0) for every token row (action expert).
hipError_t launch_out_rows(const Dims& d, const Bufs& b, WDtype wt, int k_prev, int k_next, hipStream_t st);
// The same for the joint denoiser (guided branch pair, latent and action tokens).
hipError_t launch_wam_rows(const Dims& d, const Bufs& b, int k_prev, int k_next, hipStream_t st);
// Input of the prefix prefill: h = tokens, hs, row statistics.
hipError_t launch_prefill_in(const Dims& d, const Bufs& b, const void* tokens, bool f32, hipStream_t st);

}  // namespace phyai
