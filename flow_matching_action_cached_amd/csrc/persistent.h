// Internal interface of the persistent Euler loop (loop_persistent.hip) for the host runtime.
#pragma once

#include "kernels.h"

namespace phyai {

constexpr int kPersistWGs = 256;  // one workgroup per compute unit (8 XCDs x 32)

// Byte offsets of the per-(step, layer) activation block and of the per-step final block.
// The norm inputs (hs*) and their statistics (ssq*) hold one copy per XCD, hs_cb and
// ssq_cb bytes apart: each XCD's workgroups read only their own copy.
struct PersistLayout {
  size_t o_hsa, o_ssqa, o_q, o_o, o_hsm, o_ssqm, o_act, kl_bytes;  // per (step, layer)
  size_t o_hsf, o_ssqf, k_bytes;                                     // per step (final norm input)
  size_t hs_cb, ssq_cb;                                              // bytes per XCD copy
};

// Device buffers of the persistent loop (owned by the context, allocated with the tables).
struct PersistBufs {
  char* act;            // N * L activation blocks
  char* fin;            // N final blocks
  uint64_t* flag_wg;    // [8][32] last finished phase (epoch) of each workgroup, XCD-major:
                        // workgroup w (XCD w mod 8, index w / 8 there) at (w mod 8) 32 + w / 8
  uint64_t* flag_part;  // [D/32][8] last residual partial (epoch) of each (tile pair, XCD)
  unsigned* ctl;        // [0] abort word (sticky until the host resets it), [1] failing epoch, [2] placement
  float* part;          // residual partials, two slots (output projection, down projection)
  float* hx;            // the residual h, one [64][D] copy per XCD
  float* attn_ws;       // attention split partials
};

// Kernel arguments.
struct PArgs {
  Dims d;
  Bufs b;
  char* act;
  uint32_t kl_bytes, o_hsa, o_ssqa, o_q, o_o, o_hsm, o_ssqm, o_act;
  char* fin;
  uint32_t k_bytes, o_hsf, o_ssqf;
  uint32_t hs_cb, ssq_cb;
  uint64_t* flag_wg;
  uint64_t* flag_part;
  unsigned* ctl;
  float* part;
  float* hx;
  float* attn_ws;
  uint64_t epoch0;  // epoch of this launch's first phase (monotonic across launches)
  int hpx;          // query heads per XCD
  int S, bps;       // attention key splits per (sample, head), 32-key blocks per split
};

// Shapes the persistent loop implements (bf16, <= 64 token rows, heads a multiple of 8, ...).
bool persistent_supported(const Dims& d, WDtype wt);
PersistLayout persistent_layout(const Dims& d);
size_t persistent_part_floats(const Dims& d);
size_t persistent_hx_floats(const Dims& d);
size_t persistent_attn_floats(const Dims& d);
// Phases of one launch (the host advances epoch0 by this much plus one per launch).
uint64_t persistent_phases(const Dims& d);
// One cooperative launch of the whole loop on `stream`; x must hold the noise.
hipError_t enqueue_denoise_persistent(const Dims& d, const Bufs& b, const PersistBufs& pb, uint64_t epoch0,
                                      hipStream_t stream);

}  // namespace phyai
