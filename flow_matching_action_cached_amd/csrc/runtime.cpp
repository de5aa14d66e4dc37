// Host runtime behind include/phyai.h: the runner-like context that owns the
// device arena (weights, prefix KV cache, activations, split scratch), the
// timestep tables and the captured step graphs (PhyAI reading "PhyAI: Real-Time
// Physical AI at the Edge, Scalable Rollouts in the Cloud", Figure 3 and
// Sec. 5.5: stateful runners own KV caches, buffers and graph buckets).
#include "../../include/phyai.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "kernels.h"
#include "persistent.h"

using namespace phyai;

struct phyai_ctx {
  phyai_config cfg{};
  int device = 0;
  hipStream_t stream = nullptr;      // caller's stream: every call is ordered on it
  hipStream_t cap_stream = nullptr;  // private stream used only for graph capture
  std::string err;
  WDtype wt = W_F32;
  size_t es_io = 4, es_act = 4;      // element bytes of io weights / GEMM activations
  // prefix prefill (config prefill): the prefix network's linears and zero modulation tables
  bool prefill = false, have_prefill_weights = false;
  Bufs bp{};                          // c->b with the prefix network's linears and zero tables

  void* arena = nullptr;
  size_t arena_bytes = 0;
  Bufs b{};
  Dims base{};

  // tables (own allocation, grows with n_steps)
  void* tab = nullptr;
  int tab_cap = 0;
  float* t_dev = nullptr;
  double* e_dev = nullptr;

  int joint = 0;                     // 1: joint video/action denoiser context
  bool have_weights = false, have_prefix = false, have_tables = false, have_cond = false;
  int batch = 0, prefix_len = 0, n_steps = 0;
  int use_graph = 1;
  // captured loops per (bucket batch, prefix length, steps), least recently used evicted
  struct GraphEntry {
    hipGraphExec_t exec;
    uint64_t last_use;
  };
  std::map<std::tuple<int, int, int>, GraphEntry> graphs;
  uint64_t graph_clock = 0;
  // persistent loop (<= 64 token rows, bf16; off until enabled): its buffers are sized with
  // the tables
  int persist_enabled = 0;
  // this device's allocation-free scratch (null if its address lookup failed: lookup_err)
  void* noalloc_scratch = nullptr;
  hipError_t noalloc_lookup_err = hipSuccess;
  void* pmem = nullptr;
  PersistBufs pb{};
  int p_steps = 0;                   // steps the buffers hold
  uint64_t p_epoch = 1;              // first epoch of the next launch (monotonic)
  bool p_pending = false;            // a launch ran since the last abort check
  // single-kernel repeat graphs for measurement: (which, layer, reps, batch, prefix, steps)
  std::map<std::tuple<int, int, int, int, int, int>, hipGraphExec_t> kgraphs;
};

namespace {

phyai_status fail(phyai_ctx* c, phyai_status s, const std::string& msg) {
  if (c) c->err = msg;
  return s;
}

#define HIPCHK(c, call)                                                                        \
  do {                                                                                         \
    hipError_t e_ = (call);                                                                    \
    if (e_ != hipSuccess)                                                                      \
      return fail((c), PHYAI_ERR_DEVICE, std::string(#call) + ": " + hipGetErrorString(e_));  \
  } while (0)

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  }
};

size_t wrow_bytes(WDtype wt, int K) { return wt == W_F32 ? (size_t)K * 4 : wt == W_BF16 ? (size_t)K * 2 : (size_t)K / 2; }

constexpr size_t kMaxGraphs = 16;  // captured loops kept per context

void drop_graphs(phyai_ctx* c) {
  for (auto& kv : c->graphs) hipGraphExecDestroy(kv.second.exec);
  c->graphs.clear();
  for (auto& kv : c->kgraphs) hipGraphExecDestroy(kv.second);
  c->kgraphs.clear();
}

Dims launch_dims(const phyai_ctx* c, int batch, int prefix_len, int n_steps) {
  Dims d = c->base;
  if (c->joint) {  // fixed shape: the branch pair over all tokens, no prefix
    d.N = n_steps;
    return d;
  }
  d.B = batch;
  d.M = batch * d.H;
  d.P = prefix_len;
  d.N = n_steps;
  return d;
}

// Enqueue the whole loop on the context stream: one graph launch (captured on first use for
// this (batch, prefix_len, n_steps)) or the same kernels launched eagerly.
phyai_status run_loop(phyai_ctx* c, const Dims& d, const Plan& plan, const char* who) {
  auto enqueue = [&](hipStream_t st) {
    return c->joint ? enqueue_wam_denoise(d, c->b, plan, st) : enqueue_denoise(d, c->b, plan, c->wt, st);
  };
  if (!c->use_graph) {
    HIPCHK(c, enqueue(c->stream));
    return PHYAI_OK;
  }
  auto key = std::make_tuple(d.B, d.P, d.N);
  auto it = c->graphs.find(key);
  if (it == c->graphs.end()) {
    if (c->graphs.size() >= kMaxGraphs) {  // evict the least recently used loop
      auto lru = c->graphs.begin();
      for (auto j = c->graphs.begin(); j != c->graphs.end(); ++j)
        if (j->second.last_use < lru->second.last_use) lru = j;
      HIPCHK(c, hipStreamSynchronize(c->stream));  // a launch of it may still be queued
      hipGraphExecDestroy(lru->second.exec);
      c->graphs.erase(lru);
    }
    hipGraph_t graph = nullptr;
    HIPCHK(c, hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal));
    hipError_t e = enqueue(c->cap_stream);
    hipError_t e2 = hipStreamEndCapture(c->cap_stream, &graph);
    if (e != hipSuccess || e2 != hipSuccess) {
      if (graph) hipGraphDestroy(graph);
      return fail(c, PHYAI_ERR_DEVICE,
                  std::string(who) + ": graph capture failed: " + hipGetErrorString(e != hipSuccess ? e : e2));
    }
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    hipGraphDestroy(graph);
    if (e != hipSuccess)
      return fail(c, PHYAI_ERR_DEVICE, std::string(who) + ": graph instantiate: " + hipGetErrorString(e));
    it = c->graphs.emplace(key, phyai_ctx::GraphEntry{exec, 0}).first;
  }
  it->second.last_use = ++c->graph_clock;
  HIPCHK(c, hipGraphLaunch(it->second.exec, c->stream));
  return PHYAI_OK;
}

// Graph bucket of a batch (PhyAI reading Sec. 8.1, Appendix D: a local graph batch with
// padding for incomplete batches).  Batches on the weight-streaming path (<= 64 token rows)
// run at their own size, since padding them could push them onto the tiled path; larger
// ones round up to a multiple of 8 within the context's capacity.
int graph_bucket(const phyai_ctx* c, int batch) {
  const int H = c->base.H;
  if (batch * H <= 64) return batch;
  return std::min(c->base.B, (batch + 7) / 8 * 8);
}

// Dims of a persistent launch at `batch` (nullopt-like: ok = false when unsupported).
bool persistent_dims(const phyai_ctx* c, int batch, Dims& d) {
  if (c->joint || !c->persist_enabled || !c->pmem || batch * c->base.H > 64) return false;
  d = launch_dims(c, batch, c->prefix_len, c->n_steps);
  return d.N <= c->p_steps && persistent_supported(d, c->wt);
}

void free_persistent(phyai_ctx* c) {
  if (c->pmem) hipFree(c->pmem);
  c->pmem = nullptr;
  c->pb = PersistBufs{};
  c->p_steps = 0;
}

// Buffers of the persistent loop for n_steps (kept when large enough).  Silently absent when
// the shape is not one the persistent kernel implements or the allocation fails: the graph
// path then runs.
void alloc_persistent(phyai_ctx* c, int n_steps) {
  if (!c->persist_enabled || c->joint || c->wt != W_BF16 || c->base.H > 64) return;
  Dims d = launch_dims(c, 1, c->cfg.max_prefix_len, n_steps);
  if (!persistent_supported(d, c->wt)) return;
  if (c->pmem && c->p_steps >= n_steps) return;
  free_persistent(c);
  const PersistLayout lay = persistent_layout(d);
  size_t attn_f = 0;
  for (int b = 1; b <= c->base.B && b * d.H <= 64; ++b) {  // every batch the path may run
    Dims db = launch_dims(c, b, c->cfg.max_prefix_len, n_steps);
    attn_f = std::max(attn_f, persistent_attn_floats(db));
  }
  Layout pl;
  const size_t o_act = pl.take(lay.kl_bytes * (size_t)n_steps * d.L);
  const size_t o_fin = pl.take(lay.k_bytes * (size_t)n_steps);
  const size_t o_fw = pl.take(kPersistWGs * 8), o_fp = pl.take((size_t)(d.D / 32) * 8 * 8);
  const size_t o_ctl = pl.take(16);
  const size_t o_part = pl.take(persistent_part_floats(d) * 4), o_attn = pl.take(attn_f * 4);
  const size_t o_hx = pl.take(persistent_hx_floats(d) * 4);
  if (hipMalloc(&c->pmem, pl.off) != hipSuccess) {
    c->pmem = nullptr;
    return;
  }
  // zero: padding rows of the activation blocks stay zero; flags start below every epoch
  if (hipMemsetAsync(c->pmem, 0, pl.off, c->stream) != hipSuccess || hipStreamSynchronize(c->stream) != hipSuccess) {
    free_persistent(c);
    return;
  }
  char* base = static_cast<char*>(c->pmem);
  c->pb.act = base + o_act;
  c->pb.fin = base + o_fin;
  c->pb.flag_wg = reinterpret_cast<uint64_t*>(base + o_fw);
  c->pb.flag_part = reinterpret_cast<uint64_t*>(base + o_fp);
  c->pb.ctl = reinterpret_cast<unsigned*>(base + o_ctl);
  c->pb.part = reinterpret_cast<float*>(base + o_part);
  c->pb.hx = reinterpret_cast<float*>(base + o_hx);
  c->pb.attn_ws = reinterpret_cast<float*>(base + o_attn);
  c->p_steps = n_steps;
  c->p_epoch = 1;
}

// After the stream has drained: a persistent launch that gave up on a wait left the abort
// word set (and every later launch returned at once).  Report it and reset the flags.
phyai_status check_persistent(phyai_ctx* c) {
  if (!c->pmem || !c->p_pending) return PHYAI_OK;
  c->p_pending = false;
  unsigned ctl[3] = {0, 0, 0};
  HIPCHK(c, hipMemcpy(ctl, c->pb.ctl, sizeof(ctl), hipMemcpyDeviceToHost));
  if (ctl[0] == 0) return PHYAI_OK;
  const Dims d = launch_dims(c, 1, c->cfg.max_prefix_len, c->p_steps);
  HIPCHK(c, hipMemset(c->pb.flag_wg, 0, kPersistWGs * 8));
  HIPCHK(c, hipMemset(c->pb.flag_part, 0, (size_t)(d.D / 32) * 8 * 8));
  HIPCHK(c, hipMemset(c->pb.ctl, 0, 16));
  c->p_epoch = 1;
  char msg[160];
  std::snprintf(msg, sizeof(msg),
                "persistent loop aborted: a hand-off wait exceeded its bound (phase %u of the launch); "
                "its output is invalid",
                ctl[1]);
  return fail(c, PHYAI_ERR_DEVICE, msg);
}

// ---------------------------------------------------------------- UniPC step weights
// Flow x_t = (1 - t) x_0 + t eps: alpha = 1 - t, sigma = t, lambda = log(alpha / sigma).  The
// exact step from s to t is x_t = (sigma_t/sigma_s) x_s + alpha_t int_0^h e^{-(h-u)} m(lambda_s + u) du
// (h = lambda_t - lambda_s).  Writing m at the neighbour points as m_s + sum_k (u_j)^k / k! m^(k)
// and matching the terms k = 1..n against the moments phi_k(h) = (1/k!) int_0^h e^{-(h-u)} u^k du
// (phi_0 = 1 - e^{-h}, phi_k = h^k/k! - phi_{k-1}) gives the n x n system sum_j c_j u_j^k / k! =
// phi_k; the step is x_t = A x_s + w_s m_s + sum_j w_j m_j with A = sigma_t/sigma_s,
// w_j = alpha_t c_j, w_s = alpha_t (phi_0 - sum_j c_j).  Limits: to t = 0 the step is m_s; from
// t = 1 (lambda_s = -inf) it is sigma_t x_s + alpha_t m_new with the new point (or m_s without
// one); a neighbour at t = 1 has weight 0.
struct StepW {
  double A = 0, ws = 0, w[2] = {0, 0};
};

StepW unipc_step(double s, double t, const double* nb, int n) {
  StepW r;
  const double as = 1.0 - s, ss = s, at = 1.0 - t, st = t;
  if (st == 0.0) {  // to t = 0
    r.ws = 1.0;
    return r;
  }
  r.A = st / ss;
  if (as == 0.0) {  // from t = 1: the only neighbour can be the new point t
    if (n == 0) r.ws = at;
    else r.w[0] = at;
    return r;
  }
  const double ls = std::log(as / ss), h = std::log(at / st) - ls;
  double phi[3];
  phi[0] = -std::expm1(-h);
  phi[1] = h - phi[0];
  phi[2] = h * h / 2.0 - phi[1];
  int idx[2], m = 0;
  double u[2];
  for (int j = 0; j < n; ++j)
    if (nb[j] < 1.0) {
      idx[m] = j;
      u[m++] = std::log((1.0 - nb[j]) / nb[j]) - ls;
    }
  double c[2] = {0, 0};
  if (m == 1) {
    c[0] = phi[1] / u[0];
  } else if (m == 2) {  // [u0 u1; u0^2/2 u1^2/2] c = [phi1; phi2]
    const double a11 = u[0], a12 = u[1], a21 = u[0] * u[0] / 2, a22 = u[1] * u[1] / 2;
    const double det = a11 * a22 - a12 * a21;
    c[0] = (phi[1] * a22 - a12 * phi[2]) / det;
    c[1] = (a11 * phi[2] - a21 * phi[1]) / det;
  }
  r.ws = at * (phi[0] - c[0] - c[1]);
  for (int k = 0; k < m; ++k) r.w[idx[k]] = at * c[k];
  return r;
}

// Per step k: {t_k, corrector A, w_new, w_{k-1}, w_{k-2}, predictor A, w_k, w_{k-1}} (float).
std::vector<float> unipc_weights(const float* t_host, int n, int order) {
  std::vector<double> t(t_host, t_host + n);
  t.push_back(0.0);
  std::vector<float> out((size_t)n * 8, 0.f);
  std::vector<int> pred_nb(n, 0);  // 1: the predictor of step k used the point k-1
  for (int k = 0; k < n; ++k) {
    float* o = &out[(size_t)k * 8];
    o[0] = (float)t[k];
    if (k >= 1) {  // corrector of the step k-1 -> k: neighbours (k-2 if used) and the new point k
      double nb[2];
      int nn = 0, slot_km2 = -1;
      if (pred_nb[k - 1]) {
        slot_km2 = nn;
        nb[nn++] = t[k - 2];
      }
      const int slot_new = nn;
      nb[nn++] = t[k];
      const StepW c = unipc_step(t[k - 1], t[k], nb, nn);
      o[1] = (float)c.A;
      o[2] = (float)c.w[slot_new];
      o[3] = (float)c.ws;
      o[4] = slot_km2 >= 0 ? (float)c.w[slot_km2] : 0.f;
    }
    pred_nb[k] = (order >= 2 && k >= 1 && t[k + 1] > 0.0) ? 1 : 0;
    const double nb = k >= 1 ? t[k - 1] : 0.0;
    const StepW p = unipc_step(t[k], t[k + 1], &nb, pred_nb[k]);
    o[5] = (float)p.A;
    o[6] = (float)p.ws;
    o[7] = (float)p.w[0];
  }
  return out;
}

}  // namespace

// ---------------------------------------------------------------- allocation-free scratch
// Split-reduction scratch of phyai_denoise_noalloc (callers that cannot allocate device
// memory): one copy per device, held until the process ends.  In host code `scratch` names
// a host-side stand-in, not device memory: the host uses only the address that
// hipGetSymbolAddress returns for a device, looked up once per device with that device
// current and kept in g_scratch.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

hipError_t scratch_address(int device, void** out) {
  *out = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[device] = p;
  }
  *out = g_scratch[device];
  return hipSuccess;
}

// Argument and state checks shared by the two denoise entry points.
phyai_status check_denoise(phyai_ctx* c, const float* noise, int batch, int n_steps, const float* out,
                           const char* who) {
  const std::string w(who);
  if (c->joint) return fail(c, PHYAI_ERR_BAD_STATE, w + ": joint denoiser context (use phyai_wam_denoise)");
  if (!noise || !out) return fail(c, PHYAI_ERR_INVALID_ARG, w + ": null pointer");
  if (!c->have_weights) return fail(c, PHYAI_ERR_BAD_STATE, w + ": weights not set");
  if (!c->have_prefix) return fail(c, PHYAI_ERR_BAD_STATE, w + ": prefix KV not set");
  if (!c->have_tables) return fail(c, PHYAI_ERR_BAD_STATE, w + ": timestep tables not set");
  if (n_steps != c->n_steps) return fail(c, PHYAI_ERR_INVALID_ARG, w + ": n_steps differs from the tables");
  if (batch < 1 || batch > c->batch)
    return fail(c, PHYAI_ERR_INVALID_ARG, w + ": batch outside [1, batch of the installed prefix]");
  return PHYAI_OK;
}

extern "C" {

const char* phyai_version(void) { return "phyai-mi355x 0.1 (gfx950)"; }

const char* phyai_status_string(phyai_status s) {
  switch (s) {
    case PHYAI_OK: return "ok";
    case PHYAI_ERR_INVALID_ARG: return "invalid argument";
    case PHYAI_ERR_BAD_STATE: return "bad state";
    case PHYAI_ERR_OOM: return "out of memory";
    case PHYAI_ERR_DEVICE: return "device error";
    case PHYAI_ERR_UNSUPPORTED: return "unsupported";
  }
  return "unknown status";
}

const char* phyai_last_error(const phyai_ctx* c) { return c ? c->err.c_str() : "null context"; }

phyai_status phyai_create(const phyai_config* cfg, void* hip_stream, phyai_ctx** out) {
  if (!out) return PHYAI_ERR_INVALID_ARG;
  *out = nullptr;
  if (!cfg) return PHYAI_ERR_INVALID_ARG;
  const phyai_config& g = *cfg;
  if (g.n_layers < 1 || g.width < 1 || g.n_q_heads < 1 || g.n_kv_heads < 1 || g.head_dim < 1 || g.mlp_dim < 1 ||
      g.action_dim < 1 || g.chunk_len < 1 || g.max_prefix_len < 1 || g.max_batch < 1 || !(g.rms_eps > 0.f) ||
      !(g.rope_theta == 0.f || (g.rope_theta > 1.f && g.rope_theta < 1e30f)) ||
      (g.gated_residual != 0 && g.gated_residual != 1) || (g.time_mlp != 0 && g.time_mlp != 1))
    return PHYAI_ERR_INVALID_ARG;
  if (g.weight_dtype != PHYAI_F32 && g.weight_dtype != PHYAI_BF16 && g.weight_dtype != PHYAI_INT4_G128)
    return PHYAI_ERR_INVALID_ARG;
  if (g.width % 256 || g.width > 2048 || g.mlp_dim % 128 || (g.n_q_heads * g.head_dim) % 128 ||
      g.head_dim % 32 || g.head_dim > 256 || g.n_q_heads % g.n_kv_heads || g.action_dim > 256 ||
      g.action_dim % 8)
    return PHYAI_ERR_UNSUPPORTED;
  // more than 64 token rows run on the LDS-tiled MFMA GEMMs: bf16 weights, 128-wide tiles
  if (g.chunk_len * g.max_batch > 64 &&
      (g.weight_dtype != PHYAI_BF16 || ((g.n_q_heads + 2 * g.n_kv_heads) * g.head_dim) % 128))
    return PHYAI_ERR_UNSUPPORTED;
  if (g.head_dim != 32 && g.head_dim != 64 && g.head_dim != 128 && g.head_dim != 256) return PHYAI_ERR_UNSUPPORTED;
  if (g.prefill != 0 && g.prefill != 1) return PHYAI_ERR_INVALID_ARG;
  // The weight-streaming GEMMs (batches of at most 64 token rows; the prefill of a short
  // prefix) deal each wave a power-of-two run of k-blocks: every linear's input count K
  // (width, n_q_heads * head_dim, mlp_dim) needs K / 128 a power of two <= 64.
  auto pow2_quads = [](int K) {
    const int q = K / 128;
    return K % 128 == 0 && q >= 1 && q <= 64 && (q & (q - 1)) == 0;
  };
  if ((g.chunk_len <= 64 || g.prefill) &&
      (!pow2_quads(g.width) || !pow2_quads(g.n_q_heads * g.head_dim) || !pow2_quads(g.mlp_dim)))
    return PHYAI_ERR_UNSUPPORTED;
  // The prefix network stores its K/V without positions (the cached loop's convention for a
  // given prefix); a rotated chunk would then mix encoded and unencoded positions.
  if (g.prefill && g.rope_theta != 0.f) return PHYAI_ERR_UNSUPPORTED;
  // the prefill runs the loop's kernels over batch x prefix rows: no int4 prefix network, and
  // more than 64 rows need the bf16 tiled GEMMs
  if (g.prefill && (g.weight_dtype == PHYAI_INT4_G128 ||
                    (g.max_prefix_len * g.max_batch > 64 &&
                     (g.weight_dtype != PHYAI_BF16 || ((g.n_q_heads + 2 * g.n_kv_heads) * g.head_dim) % 128))))
    return PHYAI_ERR_UNSUPPORTED;

  phyai_ctx* c = new phyai_ctx();
  c->prefill = g.prefill != 0;
  c->cfg = g;
  c->stream = static_cast<hipStream_t>(hip_stream);
  c->wt = g.weight_dtype == PHYAI_F32 ? W_F32 : g.weight_dtype == PHYAI_BF16 ? W_BF16 : W_INT4;
  c->es_io = c->wt == W_F32 ? 4 : 2;
  c->es_act = c->es_io;
  if (hipGetDevice(&c->device) != hipSuccess) {
    delete c;
    return PHYAI_ERR_DEVICE;
  }
  // set-up of the allocation-free path: this device's scratch address (the device is current)
  c->noalloc_lookup_err = scratch_address(c->device, &c->noalloc_scratch);

  Dims& d = c->base;
  d.L = g.n_layers; d.D = g.width; d.Hq = g.n_q_heads; d.Hkv = g.n_kv_heads; d.dh = g.head_dim;
  d.F = g.mlp_dim; d.A = g.action_dim; d.H = g.chunk_len;
  d.B = g.max_batch; d.M = g.max_batch * g.chunk_len; d.Mst = d.M;
  d.P = g.max_prefix_len;
  d.KS = (g.max_prefix_len + g.chunk_len + 31) / 32 * 32;
  d.qkv = (g.n_q_heads + 2 * g.n_kv_heads) * g.head_dim;
  d.nmod = 2 * g.n_layers + 1;
  d.N = 1;
  d.eps = g.rms_eps;
  d.Lc = d.L;
  d.joint = 0;
  d.ntab = 1;
  d.rows_per_tab = 1 << 30;
  d.Tl = 0;
  d.Cl = 0;
  d.gamma = 0.f;
  d.rope_theta = g.rope_theta;
  d.gated = g.gated_residual;
  d.tmlp = g.time_mlp;

  const int L = d.L, D = d.D, F = d.F, A = d.A, qd = d.Hq * d.dh;
  Layout lay;
  const size_t o_w_in = lay.take((size_t)D * A * c->es_io), o_b_in = lay.take((size_t)D * c->es_io);
  const size_t o_w_out = lay.take((size_t)A * D * c->es_io), o_b_out = lay.take((size_t)A * c->es_io);
  const int R = d.gated ? 3 : 2;  // modulation rows per norm: scale, shift (, residual gate)
  const size_t o_w_mod = lay.take((size_t)d.nmod * R * D * D * c->es_io);
  const size_t o_b_mod = lay.take((size_t)d.nmod * R * D * c->es_io);
  const size_t o_w_qkv = lay.take(wrow_bytes(c->wt, D) * d.qkv * L);
  const size_t o_w_o = lay.take(wrow_bytes(c->wt, qd) * D * L);
  const size_t o_w_gu = lay.take(wrow_bytes(c->wt, D) * 2 * F * L);
  const size_t o_w_d = lay.take(wrow_bytes(c->wt, F) * D * L);
  const size_t tm_w = d.tmlp ? (size_t)D * D * c->es_io : 0, tm_b = d.tmlp ? (size_t)D * c->es_io : 0;
  const size_t o_w_tm1 = lay.take(tm_w), o_b_tm1 = lay.take(tm_b), o_w_tm2 = lay.take(tm_w), o_b_tm2 = lay.take(tm_b);
  size_t o_s_qkv = 0, o_s_o = 0, o_s_gu = 0, o_s_d = 0;
  if (c->wt == W_INT4) {
    o_s_qkv = lay.take((size_t)d.qkv * (D / 128) * 2 * L);
    o_s_o = lay.take((size_t)D * (qd / 128) * 2 * L);
    o_s_gu = lay.take((size_t)2 * F * (D / 128) * 2 * L);
    o_s_d = lay.take((size_t)D * (F / 128) * 2 * L);
  }
  const size_t kv_elems = (size_t)d.B * L * d.Hkv * d.KS * d.dh;
  const size_t o_kc = lay.take(kv_elems * c->es_act), o_vt = lay.take(kv_elems * c->es_act);
  const size_t zero_begin = o_kc;
  // the prefill runs the same kernels over batch x prefix rows (no cached keys): its dims
  Dims dp = prefill_dims(d, g.max_batch, g.max_prefix_len);
  const size_t rows = c->prefill ? std::max<size_t>(d.M, dp.M) : (size_t)d.M;  // activation rows
  const size_t o_x = lay.take((size_t)d.M * A * 4), o_h = lay.take(rows * D * 4);
  const size_t o_ssq = lay.take((size_t)(D / 16) * rows * 4);
  const size_t mpad = (rows + 15) / 16 * 16;  // swizzled activations hold whole 16-row tiles
  const size_t o_hs = lay.take(mpad * D * c->es_act), o_q = lay.take(rows * qd * c->es_act);
  const size_t o_o = lay.take(mpad * qd * c->es_act), o_act = lay.take(mpad * F * c->es_act);
  // scratch for split reductions: upper bounds over every batch / prefix length
  const int nblk_max = (d.P + d.H + 31) / 32;
  size_t attn_ws = attn_counters(d) * nblk_max * ((size_t)(d.dh / 16) * 256 + 32);
  size_t attn_cnt_n = attn_counters(d);
  Plan pmax = make_plan(d, c->wt);
  size_t gemm_ws_n = std::max<size_t>(gemm_ws_floats(d, pmax), 1);
  if (c->prefill) {
    const int nblk_p = (dp.H + 31) / 32;
    attn_ws = std::max(attn_ws, attn_counters(dp) * nblk_p * ((size_t)(d.dh / 16) * 256 + 32));
    attn_cnt_n = std::max(attn_cnt_n, attn_counters(dp));
    gemm_ws_n = std::max(gemm_ws_n, gemm_ws_floats(dp, make_plan(dp, c->wt)));
  }
  const size_t o_attn_ws = lay.take(attn_ws * 4);
  const size_t o_attn_cnt = lay.take(attn_cnt_n * 4);
  const size_t o_gemm_ws = lay.take(gemm_ws_n * 4);
  const size_t o_gemm_cnt = lay.take((c->prefill ? std::max(gemm_counters(d), gemm_counters(dp)) : gemm_counters(d)) * 4);
  // prefill: the prefix network's four linears (same shapes as the expert's) and zero tables
  const size_t pw = c->prefill ? 1 : 0;
  const size_t o_pw_qkv = lay.take(pw * wrow_bytes(c->wt, D) * d.qkv * L);
  const size_t o_pw_o = lay.take(pw * wrow_bytes(c->wt, qd) * D * L);
  const size_t o_pw_gu = lay.take(pw * wrow_bytes(c->wt, D) * 2 * F * L);
  const size_t o_pw_d = lay.take(pw * wrow_bytes(c->wt, F) * D * L);
  const size_t zcv = (size_t)d.L * d.qkv + (size_t)d.L * 2 * d.F + d.A;
  const size_t o_zmod = lay.take(pw * (size_t)d.nmod * 2 * D * 4), o_zcv = lay.take(pw * zcv * 4);
  c->arena_bytes = lay.off;
  if (g.max_arena_bytes && c->arena_bytes > g.max_arena_bytes) {
    delete c;
    return PHYAI_ERR_OOM;
  }
  if (hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking) != hipSuccess) {
    delete c;
    return PHYAI_ERR_DEVICE;
  }
  if (hipMalloc(&c->arena, c->arena_bytes) != hipSuccess) {
    hipStreamDestroy(c->cap_stream);
    delete c;
    return PHYAI_ERR_OOM;
  }
  char* base = static_cast<char*>(c->arena);
  Bufs& b = c->b;
  b.w_in = base + o_w_in; b.b_in = base + o_b_in; b.w_out = base + o_w_out; b.b_out = base + o_b_out;
  b.w_mod = base + o_w_mod; b.b_mod = base + o_b_mod;
  b.w_qkv = base + o_w_qkv; b.w_o = base + o_w_o; b.w_gu = base + o_w_gu; b.w_d = base + o_w_d;
  if (d.tmlp) {
    b.w_tm1 = base + o_w_tm1; b.b_tm1 = base + o_b_tm1; b.w_tm2 = base + o_w_tm2; b.b_tm2 = base + o_b_tm2;
  }
  if (c->wt == W_INT4) {
    b.s_qkv = reinterpret_cast<uint16_t*>(base + o_s_qkv);
    b.s_o = reinterpret_cast<uint16_t*>(base + o_s_o);
    b.s_gu = reinterpret_cast<uint16_t*>(base + o_s_gu);
    b.s_d = reinterpret_cast<uint16_t*>(base + o_s_d);
  }
  b.kc = base + o_kc; b.vt = base + o_vt;
  b.x = reinterpret_cast<float*>(base + o_x);
  b.h = reinterpret_cast<float*>(base + o_h);
  b.ssq = reinterpret_cast<float*>(base + o_ssq);
  b.hs = base + o_hs; b.q = base + o_q; b.o = base + o_o; b.act = base + o_act;
  b.attn_ws = reinterpret_cast<float*>(base + o_attn_ws);
  b.attn_cnt = reinterpret_cast<unsigned*>(base + o_attn_cnt);
  b.gemm_ws = reinterpret_cast<float*>(base + o_gemm_ws);
  b.gemm_cnt = reinterpret_cast<unsigned*>(base + o_gemm_cnt);
  if (c->prefill) {  // prefix network: its own linears, plain RMSNorm (zero scale and shift)
    c->bp = b;
    c->bp.w_qkv = base + o_pw_qkv; c->bp.w_o = base + o_pw_o; c->bp.w_gu = base + o_pw_gu;
    c->bp.w_d = base + o_pw_d;
    c->bp.mod = reinterpret_cast<const float*>(base + o_zmod);
    c->bp.cvec = reinterpret_cast<const float*>(base + o_zcv);
    c->bp.cv_stride = (int)zcv;
    c->bp.cv_gu_off = d.L * d.qkv;
    c->bp.cv_out_off = d.L * d.qkv + d.L * 2 * d.F;
    c->bp.gate = nullptr;
  }
  // cache (keys past the live rows must read as finite), activations and counters start at 0
  if (hipMemsetAsync(base + zero_begin, 0, c->arena_bytes - zero_begin, c->stream) != hipSuccess ||
      hipStreamSynchronize(c->stream) != hipSuccess) {
    hipFree(c->arena);
    hipStreamDestroy(c->cap_stream);
    delete c;
    return PHYAI_ERR_DEVICE;
  }
  *out = c;
  return PHYAI_OK;
}

phyai_status phyai_set_weights(phyai_ctx* c, const phyai_weights* w) {
  if (!c) return PHYAI_ERR_INVALID_ARG;
  c->err.clear();
  if (c->joint) return fail(c, PHYAI_ERR_BAD_STATE, "set_weights: joint denoiser context (use phyai_wam_set_weights)");
  if (!w || !w->w_in || !w->b_in || !w->w_out || !w->b_out || !w->w_mod || !w->b_mod || !w->w_qkv || !w->w_o ||
      !w->w_gu || !w->w_d)
    return fail(c, PHYAI_ERR_INVALID_ARG, "set_weights: null weight pointer");
  if (c->wt == W_INT4 && (!w->s_qkv || !w->s_o || !w->s_gu || !w->s_d))
    return fail(c, PHYAI_ERR_INVALID_ARG, "set_weights: int4 weights need the four scale arrays");
  if (c->base.tmlp && (!w->w_tm1 || !w->b_tm1 || !w->w_tm2 || !w->b_tm2))
    return fail(c, PHYAI_ERR_INVALID_ARG, "set_weights: the time MLP needs w_tm1, b_tm1, w_tm2 and b_tm2");
  const Dims& d = c->base;
  const int L = d.L, D = d.D, F = d.F, A = d.A, qd = d.Hq * d.dh;
  const size_t e = c->es_io;
  auto cp = [&](const void* dst, const void* src, size_t bytes) {
    return hipMemcpyAsync(const_cast<void*>(dst), src, bytes, hipMemcpyDeviceToDevice, c->stream);
  };
  HIPCHK(c, cp(c->b.w_in, w->w_in, (size_t)D * A * e));
  HIPCHK(c, cp(c->b.b_in, w->b_in, (size_t)D * e));
  HIPCHK(c, cp(c->b.w_out, w->w_out, (size_t)A * D * e));
  HIPCHK(c, cp(c->b.b_out, w->b_out, (size_t)A * e));
  const int R = d.gated ? 3 : 2;
  HIPCHK(c, cp(c->b.w_mod, w->w_mod, (size_t)d.nmod * R * D * D * e));
  HIPCHK(c, cp(c->b.b_mod, w->b_mod, (size_t)d.nmod * R * D * e));
  if (d.tmlp) {
    HIPCHK(c, cp(c->b.w_tm1, w->w_tm1, (size_t)D * D * e));
    HIPCHK(c, cp(c->b.b_tm1, w->b_tm1, (size_t)D * e));
    HIPCHK(c, cp(c->b.w_tm2, w->w_tm2, (size_t)D * D * e));
    HIPCHK(c, cp(c->b.b_tm2, w->b_tm2, (size_t)D * e));
  }
  // expert linears: re-laid out into the fragment-native (swizzled) layout the kernels stream
  if (c->wt != W_INT4) {
    auto sw = [&](const void* dst, const void* src, int64_t rows, int cols) {
      return enqueue_swizzle(src, const_cast<void*>(dst), rows, cols, e, c->stream);
    };
    HIPCHK(c, sw(c->b.w_qkv, w->w_qkv, (int64_t)L * d.qkv, D));
    HIPCHK(c, sw(c->b.w_o, w->w_o, (int64_t)L * D, qd));
    HIPCHK(c, sw(c->b.w_gu, w->w_gu, (int64_t)L * 2 * F, D));
    HIPCHK(c, sw(c->b.w_d, w->w_d, (int64_t)L * D, F));
  } else {
    auto rp = [&](const void* dst, const void* src, int64_t rows, int cols) {
      return enqueue_swizzle_int4(static_cast<const uint8_t*>(src), static_cast<uint8_t*>(const_cast<void*>(dst)),
                                  rows, cols, c->stream);
    };
    HIPCHK(c, rp(c->b.w_qkv, w->w_qkv, (int64_t)L * d.qkv, D));
    HIPCHK(c, rp(c->b.w_o, w->w_o, (int64_t)L * D, qd));
    HIPCHK(c, rp(c->b.w_gu, w->w_gu, (int64_t)L * 2 * F, D));
    HIPCHK(c, rp(c->b.w_d, w->w_d, (int64_t)L * D, F));
    HIPCHK(c, cp(c->b.s_qkv, w->s_qkv, (size_t)L * d.qkv * (D / 128) * 2));
    HIPCHK(c, cp(c->b.s_o, w->s_o, (size_t)L * D * (qd / 128) * 2));
    HIPCHK(c, cp(c->b.s_gu, w->s_gu, (size_t)L * 2 * F * (D / 128) * 2));
    HIPCHK(c, cp(c->b.s_d, w->s_d, (size_t)L * D * (F / 128) * 2));
  }
  c->have_weights = true;
  c->have_tables = false;  // the tables fold the weights in: they must be rebuilt
  drop_graphs(c);
  return PHYAI_OK;
}

phyai_status phyai_set_prefix_kv(phyai_ctx* c, const void* k, const void* v, int batch, int prefix_len) {
  if (!c) return PHYAI_ERR_INVALID_ARG;
  c->err.clear();
  if (c->joint) return fail(c, PHYAI_ERR_BAD_STATE, "set_prefix_kv: a joint denoiser context has no cached prefix");
  if (!k || !v) return fail(c, PHYAI_ERR_INVALID_ARG, "set_prefix_kv: null pointer");
  if (batch < 1 || batch > c->cfg.max_batch)
    return fail(c, PHYAI_ERR_INVALID_ARG, "set_prefix_kv: batch out of range [1, max_batch]");
  if (prefix_len < 1 || prefix_len > c->cfg.max_prefix_len)
    return fail(c, PHYAI_ERR_INVALID_ARG, "set_prefix_kv: prefix_len out of range [1, max_prefix_len]");
  HIPCHK(c, enqueue_install_prefix(c->base, k, v, batch, prefix_len, c->b.kc, c->b.vt, c->es_act, c->stream));
  c->batch = batch;
  c->prefix_len = prefix_len;
  c->have_prefix = true;
  return PHYAI_OK;
}

phyai_status phyai_set_timestep_tables(phyai_ctx* c, const float* t_host, int n_steps) {
  if (!c) return PHYAI_ERR_INVALID_ARG;
  c->err.clear();
  if (!t_host || n_steps < 1) return fail(c, PHYAI_ERR_INVALID_ARG, "set_timestep_tables: need n_steps >= 1 times");
  if (!c->have_weights) return fail(c, PHYAI_ERR_BAD_STATE, "set_timestep_tables: weights not set");
  if (c->joint && !c->have_cond)
    return fail(c, PHYAI_ERR_BAD_STATE, "set_timestep_tables: branch conditions not set");
  for (int i = 0; i < n_steps; ++i)
    if (!std::isfinite(t_host[i])) return fail(c, PHYAI_ERR_INVALID_ARG, "set_timestep_tables: non-finite time");
  if (c->base.solver) {
    bool ok = t_host[0] <= 1.f && t_host[n_steps - 1] > 0.f;
    for (int i = 1; i < n_steps; ++i) ok = ok && t_host[i] < t_host[i - 1];
    if (!ok) return fail(c, PHYAI_ERR_INVALID_ARG, "set_timestep_tables: UniPC needs 1 >= t_0 > ... > t_{N-1} > 0");
  }
  Dims d = c->base;
  d.N = n_steps;
  const size_t mod_f = (size_t)n_steps * d.ntab * d.nmod * 2 * d.D;
  // per table: W_qkv shifts | W_gu shifts | out-projection shifts (expert A; joint Cl + A)
  const int cv_stride = d.L * d.qkv + d.L * 2 * d.F + (d.joint ? d.Cl + d.A : d.A);
  const size_t cv_f = (size_t)n_steps * d.ntab * cv_stride;
  if (n_steps > c->tab_cap) {
    HIPCHK(c, hipStreamSynchronize(c->stream));
    drop_graphs(c);
    if (c->tab) hipFree(c->tab);
    c->tab = nullptr;
    c->tab_cap = 0;
    const size_t gate_f = d.gated ? (size_t)n_steps * d.ntab * d.nmod * d.D : 0;
    const size_t e_f = (size_t)n_steps * d.D * (d.tmlp ? 3 : 1);  // embedding (+ time-MLP hidden, output)
    const size_t bytes = align256(mod_f * 4) + align256(cv_f * 4) + align256((size_t)n_steps * 4) * 2 +
                         align256(e_f * 8) + align256(gate_f * 4) + align256((size_t)n_steps * 8 * 4);
    if (hipMalloc(&c->tab, bytes) != hipSuccess) return fail(c, PHYAI_ERR_OOM, "set_timestep_tables: hipMalloc");
    c->tab_cap = n_steps;
  }
  // layout for capacity tab_cap (pointers stay fixed for smaller schedules)
  const int cap = c->tab_cap;
  char* p = static_cast<char*>(c->tab);
  float* mod = reinterpret_cast<float*>(p);
  p += align256((size_t)cap * d.ntab * d.nmod * 2 * d.D * 4);
  float* cvec = reinterpret_cast<float*>(p);
  p += align256((size_t)cap * d.ntab * cv_stride * 4);
  float* dt = reinterpret_cast<float*>(p);
  p += align256((size_t)cap * 4);
  c->t_dev = reinterpret_cast<float*>(p);
  p += align256((size_t)cap * 4);
  c->e_dev = reinterpret_cast<double*>(p);
  p += align256((size_t)cap * d.D * (d.tmlp ? 3 : 1) * 8);
  float* gate = d.gated ? reinterpret_cast<float*>(p) : nullptr;  // [cap][ntab][nmod][D]
  p += align256(d.gated ? (size_t)cap * d.ntab * d.nmod * d.D * 4 : 0);
  float* uni = reinterpret_cast<float*>(p);  // [cap][8] UniPC weights
  std::vector<float> unih;
  if (d.solver) unih = unipc_weights(t_host, n_steps, d.solver);
  // step sizes dt_k = t_{k+1} - t_k with t_N = 0
  std::vector<float> dth(n_steps);
  for (int i = 0; i < n_steps; ++i) {
    const double nxt = (i + 1 < n_steps) ? (double)t_host[i + 1] : 0.0;
    dth[i] = (float)(nxt - (double)t_host[i]);
  }
  HIPCHK(c, hipMemcpyAsync(c->t_dev, t_host, (size_t)n_steps * 4, hipMemcpyHostToDevice, c->stream));
  HIPCHK(c, hipMemcpyAsync(dt, dth.data(), (size_t)n_steps * 4, hipMemcpyHostToDevice, c->stream));
  if (d.solver) HIPCHK(c, hipMemcpyAsync(uni, unih.data(), unih.size() * 4, hipMemcpyHostToDevice, c->stream));
  c->b.uni = d.solver ? uni : nullptr;
  c->b.mod = mod;
  c->b.gate = gate;
  c->b.cvec = cvec;
  c->b.dt = dt;
  c->b.cv_stride = cv_stride;
  c->b.cv_gu_off = d.L * d.qkv;
  c->b.cv_out_off = d.L * d.qkv + d.L * 2 * d.F;
  HIPCHK(c, enqueue_tables(d, c->b, c->wt, c->t_dev, c->e_dev, mod, cvec, gate, c->stream));
  // host buffers above must outlive the async copies
  HIPCHK(c, hipStreamSynchronize(c->stream));
  {
    const phyai_status ps = check_persistent(c);  // (buffers are replaced only when the stream is idle)
    if (ps != PHYAI_OK) return ps;
  }
  alloc_persistent(c, n_steps);
  c->n_steps = n_steps;
  c->have_tables = true;
  return PHYAI_OK;
}

phyai_status phyai_set_graph_mode(phyai_ctx* c, int use_graph) {
  if (!c) return PHYAI_ERR_INVALID_ARG;
  c->use_graph = use_graph ? 1 : 0;
  return PHYAI_OK;
}

phyai_status phyai_denoise(phyai_ctx* c, const float* noise, int batch, int n_steps, float* out) {
  if (!c) return PHYAI_ERR_INVALID_ARG;
  c->err.clear();
  {
    const phyai_status st = check_denoise(c, noise, batch, n_steps, out, "denoise");
    if (st != PHYAI_OK) return st;
  }
  // the loop runs at the bucket's batch; pad slots start from x = 0 on their (stale but
  // finite) cache rows, and samples never interact, so the real rows are those of the
  // bucket's run
  const int bucket = graph_bucket(c, batch);
  const Dims d = launch_dims(c, bucket, c->prefix_len, n_steps);
  const Plan plan = make_plan(d, c->wt);
  const size_t xbytes = (size_t)batch * d.H * d.A * 4, xbucket = (size_t)d.M * d.A * 4;
  HIPCHK(c, hipMemcpyAsync(c->b.x, noise, xbytes, hipMemcpyDeviceToDevice, c->stream));
  if (xbucket > xbytes) HIPCHK(c, enqueue_zero_f32(c->b.x + xbytes / 4, (xbucket - xbytes) / 4, c->stream));
  Dims dp;
  if (persistent_dims(c, bucket, dp)) {  // the whole loop as one persistent kernel
    const hipError_t e = enqueue_denoise_persistent(dp, c->b, c->pb, c->p_epoch, c->stream);
    if (e == hipSuccess) {
      c->p_epoch += persistent_phases(dp) + 1;
      c->p_pending = true;
      HIPCHK(c, hipMemcpyAsync(out, c->b.x, xbytes, hipMemcpyDeviceToDevice, c->stream));
      return PHYAI_OK;
    }
    // a cooperative launch that the device cannot hold: use the graph path from now on
    (void)hipGetLastError();
    c->persist_enabled = 0;
  }
  const phyai_status st = run_loop(c, d, plan, "denoise");
  if (st != PHYAI_OK) return st;
  HIPCHK(c, hipMemcpyAsync(out, c->b.x, xbytes, hipMemcpyDeviceToDevice, c->stream));
  return PHYAI_OK;
}

phyai_status phyai_denoise_noalloc(phyai_ctx* c, const float* noise, int batch, int n_steps, float* out) {
  if (!c) return PHYAI_ERR_INVALID_ARG;
  c->err.clear();
  {
    const phyai_status st = check_denoise(c, noise, batch, n_steps, out, "denoise_noalloc");
    if (st != PHYAI_OK) return st;
  }
  if (!c->noalloc_scratch)
    return fail(c, PHYAI_ERR_DEVICE, std::string("denoise_noalloc: no scratch address for this device: ") +
                                         hipGetErrorString(c->noalloc_lookup_err));
  const int bucket = graph_bucket(c, batch);
  const Dims d = launch_dims(c, bucket, c->prefix_len, n_steps);
  const Plan plan = make_plan(d, c->wt);
  // the scratch: arrival counters first (cleared by every call), then the split partials
  Layout sl;
  const size_t o_acnt = sl.take(attn_counters(d) * 4), o_gcnt = sl.take(gemm_counters(d) * 4);
  const size_t cnt_bytes = sl.off;
  const size_t o_aws = sl.take(std::max<size_t>(attn_ws_floats(d, plan), 1) * 4);
  const size_t o_gws = sl.take(std::max<size_t>(gemm_ws_floats(d, plan), 1) * 4);
  if (sl.off > kNoAllocScratchBytes) {
    char msg[200];
    std::snprintf(msg, sizeof(msg),
                  "denoise_noalloc: this batch and prefix need %zu bytes of split scratch; the allocation-free "
                  "path holds at most %zu (use phyai_denoise)",
                  sl.off, kNoAllocScratchBytes);
    return fail(c, PHYAI_ERR_INVALID_ARG, msg);
  }
  char* sp = static_cast<char*>(c->noalloc_scratch);
  Bufs b = c->b;
  b.attn_cnt = reinterpret_cast<unsigned*>(sp + o_acnt);
  b.gemm_cnt = reinterpret_cast<unsigned*>(sp + o_gcnt);
  b.attn_ws = reinterpret_cast<float*>(sp + o_aws);
  b.gemm_ws = reinterpret_cast<float*>(sp + o_gws);
  const size_t xbytes = (size_t)batch * d.H * d.A * 4, xbucket = (size_t)d.M * d.A * 4;
  HIPCHK(c, hipMemcpyAsync(c->b.x, noise, xbytes, hipMemcpyDeviceToDevice, c->stream));
  if (xbucket > xbytes) HIPCHK(c, enqueue_zero_f32(c->b.x + xbytes / 4, (xbucket - xbytes) / 4, c->stream));
  // a fill kernel, not a memset: the counters start at zero whatever the last call left
  HIPCHK(c, enqueue_zero_f32(reinterpret_cast<float*>(sp), cnt_bytes / 4, c->stream));
  HIPCHK(c, enqueue_denoise(d, b, plan, c->wt, c->stream));
  HIPCHK(c, hipMemcpyAsync(out, c->b.x, xbytes, hipMemcpyDeviceToDevice, c->stream));
  return PHYAI_OK;
}

phyai_status phyai_enqueue_kernel_repeat(phyai_ctx* c, int which, int layer, int reps) {
  if (!c) return PHYAI_ERR_INVALID_ARG;
  c->err.clear();
  if (which < 0 || which > 7 || reps < 1 || reps > 100000 || layer < 0 || layer >= c->base.L)
    return fail(c, PHYAI_ERR_INVALID_ARG, "enqueue_kernel_repeat: bad kernel id, layer or reps");
  if (!c->have_weights || !(c->have_prefix || c->joint) || !c->have_tables)
    return fail(c, PHYAI_ERR_BAD_STATE, "enqueue_kernel_repeat: weights, prefix and tables must be set");
  const Dims d = launch_dims(c, c->batch, c->prefix_len, c->n_steps);
  const Plan plan = make_plan(d, c->wt);
  if (which == 7 && !c->joint) {  // the split merge has a launch of its own only on one path
    const int nblk = (d.P + d.H + 31) / 32;
    if (plan.attn_wide || (nblk + plan.attn_bps - 1) / plan.attn_bps == 1) return PHYAI_OK;
  }
  auto key = std::make_tuple(which, layer, reps, c->batch, c->prefix_len, c->n_steps);
  auto it = c->kgraphs.find(key);
  if (it == c->kgraphs.end()) {
    if (c->kgraphs.size() >= kMaxGraphs) {  // measurement graphs: drop them all
      HIPCHK(c, hipStreamSynchronize(c->stream));
      for (auto& kv : c->kgraphs) hipGraphExecDestroy(kv.second);
      c->kgraphs.clear();
    }
    hipGraph_t graph = nullptr;
    HIPCHK(c, hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal));
    hipError_t e = hipSuccess;
    for (int i = 0; i < reps && e == hipSuccess; ++i)
      e = c->joint ? enqueue_wam_one(d, c->b, plan, which, 0, layer, c->cap_stream)
                   : enqueue_one(d, c->b, plan, c->wt, which, 0, layer, c->cap_stream);
    hipError_t e2 = hipStreamEndCapture(c->cap_stream, &graph);
    if (e != hipSuccess || e2 != hipSuccess) {
      if (graph) hipGraphDestroy(graph);
      return fail(c, PHYAI_ERR_DEVICE, std::string("enqueue_kernel_repeat: capture failed: ") +
                                           hipGetErrorString(e != hipSuccess ? e : e2));
    }
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    hipGraphDestroy(graph);
    if (e != hipSuccess) return fail(c, PHYAI_ERR_DEVICE, std::string("enqueue_kernel_repeat: instantiate: ") + hipGetErrorString(e));
    it = c->kgraphs.emplace(key, exec).first;
  }
  HIPCHK(c, hipGraphLaunch(it->second, c->stream));
  return PHYAI_OK;
}

phyai_status phyai_time_loop_stages(phyai_ctx* c, const float* noise, int batch, int reps, float* stage_us,
                                    float* chunk_ms) {
  if (!c) return PHYAI_ERR_INVALID_ARG;
  c->err.clear();
  {
    const phyai_status st = check_denoise(c, noise, batch, c->n_steps, stage_us, "time_loop_stages");
    if (st != PHYAI_OK) return st;
  }
  if (!chunk_ms || reps < 1 || reps > 1000)
    return fail(c, PHYAI_ERR_INVALID_ARG, "time_loop_stages: null output or reps outside [1, 1000]");
  const int bucket = graph_bucket(c, batch);
  const Dims d = launch_dims(c, bucket, c->prefix_len, c->n_steps);
  const Plan plan = make_plan(d, c->wt);
  const int n_ev = 2 + d.N * (6 * d.L + 1);
  std::vector<hipEvent_t> ev(n_ev, nullptr);
  std::vector<int> kind(n_ev, -1);
  auto release = [&]() {
    for (hipEvent_t e : ev)
      if (e) hipEventDestroy(e);
  };
  auto bail = [&](const char* what, hipError_t e) {
    release();
    return fail(c, PHYAI_ERR_DEVICE, std::string("time_loop_stages: ") + what + ": " + hipGetErrorString(e));
  };
  for (int i = 0; i < n_ev; ++i) {
    const hipError_t e = hipEventCreate(&ev[i]);
    if (e != hipSuccess) return bail("event", e);
  }
  double sum[8] = {0}, total = 0.0;
  long cnt[8] = {0};
  const size_t xbytes = (size_t)batch * d.H * d.A * 4, xbucket = (size_t)d.M * d.A * 4;
  hipError_t e = hipSuccess;
  for (int r = 0; r < reps; ++r) {
    // the loop of phyai_denoise with an event after every launch, queued behind a short
    // wait so that it runs back to back (graph capture cannot record timing events here)
    LaunchMarks mk{ev.data(), kind.data(), 0, n_ev};
    if ((e = hipMemcpyAsync(c->b.x, noise, xbytes, hipMemcpyDeviceToDevice, c->stream)) != hipSuccess ||
        (xbucket > xbytes && (e = enqueue_zero_f32(c->b.x + xbytes / 4, (xbucket - xbytes) / 4, c->stream)) != hipSuccess) ||
        (e = enqueue_delay_us(20000, c->stream)) != hipSuccess ||
        (e = enqueue_denoise(d, c->b, plan, c->wt, c->stream, &mk)) != hipSuccess ||
        (e = hipStreamSynchronize(c->stream)) != hipSuccess)
      return bail("replay", e);
    float ms = 0.f;
    for (int i = 1; i < mk.n; ++i) {
      if ((e = hipEventElapsedTime(&ms, ev[i - 1], ev[i])) != hipSuccess) return bail("elapsed time", e);
      if (kind[i] >= 0 && kind[i] < 8) {
        sum[kind[i]] += ms;
        ++cnt[kind[i]];
      }
    }
    if ((e = hipEventElapsedTime(&ms, ev[0], ev[mk.n - 1])) != hipSuccess) return bail("elapsed time", e);
    total += ms;
  }
  release();
  for (int k = 0; k < 8; ++k) stage_us[k] = cnt[k] ? (float)(sum[k] / cnt[k] * 1000.0) : 0.f;
  *chunk_ms = (float)(total / reps);
  return PHYAI_OK;
}

phyai_status phyai_set_prefill_weights(phyai_ctx* c, const phyai_prefill_weights* w) {
  if (!c) return PHYAI_ERR_INVALID_ARG;
  c->err.clear();
  if (!c->prefill) return fail(c, PHYAI_ERR_BAD_STATE, "set_prefill_weights: context created without prefill");
  if (!w || !w->w_qkv || !w->w_o || !w->w_gu || !w->w_d)
    return fail(c, PHYAI_ERR_INVALID_ARG, "set_prefill_weights: null weight pointer");
  const Dims& d = c->base;
  const int L = d.L, D = d.D, F = d.F, qd = d.Hq * d.dh;
  auto sw = [&](const void* dst, const void* src, int64_t rows, int cols) {
    return enqueue_swizzle(src, const_cast<void*>(dst), rows, cols, c->es_io, c->stream);
  };
  HIPCHK(c, sw(c->bp.w_qkv, w->w_qkv, (int64_t)L * d.qkv, D));
  HIPCHK(c, sw(c->bp.w_o, w->w_o, (int64_t)L * D, qd));
  HIPCHK(c, sw(c->bp.w_gu, w->w_gu, (int64_t)L * 2 * F, D));
  HIPCHK(c, sw(c->bp.w_d, w->w_d, (int64_t)L * D, F));
  HIPCHK(c, hipStreamSynchronize(c->stream));
  c->have_prefill_weights = true;
  return PHYAI_OK;
}

phyai_status phyai_prefill(phyai_ctx* c, const void* tokens, int batch, int prefix_len) {
  if (!c) return PHYAI_ERR_INVALID_ARG;
  c->err.clear();
  if (!c->prefill) return fail(c, PHYAI_ERR_BAD_STATE, "prefill: context created without prefill");
  if (!tokens) return fail(c, PHYAI_ERR_INVALID_ARG, "prefill: null tokens");
  if (!c->have_prefill_weights) return fail(c, PHYAI_ERR_BAD_STATE, "prefill: prefix network weights not set");
  if (batch < 1 || batch > c->base.B || prefix_len < 1 || prefix_len > c->cfg.max_prefix_len)
    return fail(c, PHYAI_ERR_INVALID_ARG, "prefill: batch or prefix length outside the context's capacity");
  const Dims d = prefill_dims(c->base, batch, prefix_len);
  const Plan plan = make_plan(d, c->wt);
  HIPCHK(c, enqueue_prefill(d, c->bp, plan, c->wt, tokens, c->stream));
  // the new prefix replaces the old one (the invalidation point); graphs read the cache in place
  c->have_prefix = true;
  c->batch = batch;
  c->prefix_len = prefix_len;
  return PHYAI_OK;
}

// ---------------------------------------------------------------- execution-state capsules
// Page "FlashRT-PAI speeds physical AI inference up to 12.66x", its account of the three
// mechanisms: execution-state capsules snapshot, restore and fork persistent state.
// The persistent state of this runner is the installed prefix (batch, prefix length and the
// cache rows [0, P) of every layer); a capsule is a device buffer: a 256-byte header, then
// the payload of enqueue_capsule_copy.
namespace {
struct CapsuleHeader {
  uint64_t magic;
  int32_t version, batch, prefix_len, L, Hkv, dh, elem_bytes, pad;
};
constexpr uint64_t kCapsuleMagic = 0x5048594149434150ull;  // "PHYAICAP"
constexpr size_t kCapsuleHeader = 256;
size_t capsule_payload(const Dims& d, int batch, int prefix_len, size_t es) {
  return 2 * (size_t)batch * d.L * d.Hkv * prefix_len * d.dh * es;
}
}  // namespace

size_t phyai_capsule_bytes(const phyai_ctx* c) {
  if (!c || c->joint || !c->have_prefix) return 0;
  return kCapsuleHeader + capsule_payload(c->base, c->batch, c->prefix_len, c->es_act);
}

phyai_status phyai_capsule_save(phyai_ctx* c, void* capsule, size_t bytes) {
  if (!c) return PHYAI_ERR_INVALID_ARG;
  c->err.clear();
  if (c->joint) return fail(c, PHYAI_ERR_BAD_STATE, "capsule_save: joint denoiser context");
  if (!c->have_prefix) return fail(c, PHYAI_ERR_BAD_STATE, "capsule_save: no prefix installed");
  if (!capsule || bytes < phyai_capsule_bytes(c))
    return fail(c, PHYAI_ERR_INVALID_ARG, "capsule_save: null capsule or fewer bytes than phyai_capsule_bytes");
  CapsuleHeader h{kCapsuleMagic, 1, c->batch, c->prefix_len, c->base.L, c->base.Hkv, c->base.dh, (int)c->es_act, 0};
  static_assert(sizeof(CapsuleHeader) % 4 == 0 && sizeof(CapsuleHeader) <= 64, "header words");
  uint32_t words[sizeof(CapsuleHeader) / 4];
  std::memcpy(words, &h, sizeof(h));
  HIPCHK(c, enqueue_capsule_header(words, (int)(sizeof(h) / 4), capsule, c->stream));
  HIPCHK(c, enqueue_capsule_copy(c->base, c->b.kc, c->b.vt, static_cast<char*>(capsule) + kCapsuleHeader, c->batch,
                                 c->prefix_len, c->es_act, true, c->stream));
  return PHYAI_OK;
}

phyai_status phyai_capsule_restore(phyai_ctx* c, const void* capsule, size_t bytes) {
  if (!c) return PHYAI_ERR_INVALID_ARG;
  c->err.clear();
  if (c->joint) return fail(c, PHYAI_ERR_BAD_STATE, "capsule_restore: joint denoiser context");
  if (!capsule || bytes < kCapsuleHeader) return fail(c, PHYAI_ERR_INVALID_ARG, "capsule_restore: null or short capsule");
  CapsuleHeader h{};
  HIPCHK(c, hipStreamSynchronize(c->stream));  // the capsule may have been written on this stream
  HIPCHK(c, hipMemcpy(&h, capsule, sizeof(h), hipMemcpyDeviceToHost));
  if (h.magic != kCapsuleMagic || h.version != 1)
    return fail(c, PHYAI_ERR_INVALID_ARG, "capsule_restore: not a capsule of this library");
  if (h.L != c->base.L || h.Hkv != c->base.Hkv || h.dh != c->base.dh || h.elem_bytes != (int)c->es_act ||
      h.batch < 1 || h.batch > c->base.B || h.prefix_len < 1 || h.prefix_len > c->cfg.max_prefix_len)
    return fail(c, PHYAI_ERR_INVALID_ARG, "capsule_restore: capsule shape does not fit this context");
  if (bytes < kCapsuleHeader + capsule_payload(c->base, h.batch, h.prefix_len, c->es_act))
    return fail(c, PHYAI_ERR_INVALID_ARG, "capsule_restore: capsule shorter than its header says");
  HIPCHK(c, enqueue_capsule_copy(c->base, c->b.kc, c->b.vt,
                                 const_cast<char*>(static_cast<const char*>(capsule)) + kCapsuleHeader, h.batch,
                                 h.prefix_len, c->es_act, false, c->stream));
  c->have_prefix = true;  // the restored prefix replaces the installed one (invalidation point)
  c->batch = h.batch;
  c->prefix_len = h.prefix_len;
  return PHYAI_OK;
}

phyai_status phyai_capsule_fork(phyai_ctx* c, int src_sample, int dst_sample) {
  if (!c) return PHYAI_ERR_INVALID_ARG;
  c->err.clear();
  if (c->joint) return fail(c, PHYAI_ERR_BAD_STATE, "capsule_fork: joint denoiser context");
  if (!c->have_prefix) return fail(c, PHYAI_ERR_BAD_STATE, "capsule_fork: no prefix installed");
  if (src_sample < 0 || src_sample >= c->batch || dst_sample < 0 || dst_sample >= c->batch)
    return fail(c, PHYAI_ERR_INVALID_ARG, "capsule_fork: sample index outside the installed batch");
  if (src_sample == dst_sample) return PHYAI_OK;
  const Dims& d = c->base;
  const size_t per = (size_t)d.L * d.Hkv * d.KS * d.dh * c->es_act;  // one sample's K (or V^T) region
  char* kc = static_cast<char*>(c->b.kc);
  char* vt = static_cast<char*>(c->b.vt);
  HIPCHK(c, hipMemcpyAsync(kc + dst_sample * per, kc + src_sample * per, per, hipMemcpyDeviceToDevice, c->stream));
  HIPCHK(c, hipMemcpyAsync(vt + dst_sample * per, vt + src_sample * per, per, hipMemcpyDeviceToDevice, c->stream));
  return PHYAI_OK;
}

phyai_status phyai_unipc_weights(const float* t_host, int n_steps, int order, float* out_host) {
  if (!t_host || !out_host || n_steps < 1 || (order != 1 && order != 2)) return PHYAI_ERR_INVALID_ARG;
  bool ok = t_host[0] <= 1.f && t_host[n_steps - 1] > 0.f;
  for (int i = 1; i < n_steps; ++i) ok = ok && t_host[i] < t_host[i - 1];
  if (!ok) return PHYAI_ERR_INVALID_ARG;
  const std::vector<float> w = unipc_weights(t_host, n_steps, order);
  std::memcpy(out_host, w.data(), w.size() * sizeof(float));
  return PHYAI_OK;
}

phyai_status phyai_sync(phyai_ctx* c) {
  if (!c) return PHYAI_ERR_INVALID_ARG;
  HIPCHK(c, hipStreamSynchronize(c->stream));
  HIPCHK(c, hipGetLastError());
  return check_persistent(c);
}

phyai_status phyai_set_persistent(phyai_ctx* c, int enable) {
  if (!c) return PHYAI_ERR_INVALID_ARG;
  c->err.clear();
  c->persist_enabled = enable ? 1 : 0;
  if (c->persist_enabled && c->have_tables && !c->pmem) {
    // buffers for the installed tables; replaced only once the stream is idle
    HIPCHK(c, hipStreamSynchronize(c->stream));
    alloc_persistent(c, c->n_steps);
  }
  return PHYAI_OK;
}

int phyai_loop_form(const phyai_ctx* c, int batch) {
  if (!c || c->joint || !c->have_prefix || !c->have_tables || batch < 1 || batch > c->batch) return -1;
  Dims d;
  return persistent_dims(c, graph_bucket(c, batch), d) ? 1 : 0;
}

phyai_status phyai_get_modulation(phyai_ctx* c, float* dst) {
  if (!c) return PHYAI_ERR_INVALID_ARG;
  c->err.clear();
  if (!dst) return fail(c, PHYAI_ERR_INVALID_ARG, "get_modulation: null pointer");
  if (!c->have_tables) return fail(c, PHYAI_ERR_BAD_STATE, "get_modulation: tables not set");
  const size_t bytes = (size_t)c->n_steps * c->base.ntab * c->base.nmod * 2 * c->base.D * 4;
  HIPCHK(c, hipMemcpyAsync(dst, c->b.mod, bytes, hipMemcpyDeviceToDevice, c->stream));
  return PHYAI_OK;
}

void phyai_destroy(phyai_ctx* c) {
  if (!c) return;
  hipStreamSynchronize(c->stream);
  drop_graphs(c);
  free_persistent(c);
  if (c->tab) hipFree(c->tab);
  if (c->arena) hipFree(c->arena);
  if (c->cap_stream) hipStreamDestroy(c->cap_stream);
  delete c;
}

// ---------------------------------------------------------------- joint video/action denoiser
// PhyAI reading, Figure 4 and Sec. 5.5 third item: the conditional and unconditional branches
// run as a batch of two over one joint latent/action sequence with full self-attention.
phyai_status phyai_wam_create(const phyai_wam_config* cfg, void* hip_stream, phyai_ctx** out) {
  if (!out) return PHYAI_ERR_INVALID_ARG;
  *out = nullptr;
  if (!cfg) return PHYAI_ERR_INVALID_ARG;
  const phyai_wam_config& g = *cfg;
  if (g.n_layers < 1 || g.width < 1 || g.n_heads < 1 || g.head_dim < 1 || g.mlp_dim < 1 || g.latent_tokens < 0 ||
      g.action_tokens < 0 || g.latent_tokens + g.action_tokens < 1 || g.latent_dim < 1 || g.action_dim < 1 ||
      !(g.rms_eps > 0.f) || g.solver_order < 0 || g.solver_order > 2)
    return PHYAI_ERR_INVALID_ARG;
  if (g.width % 256 || g.width > 2048 || g.mlp_dim % 128 || (g.n_heads * g.head_dim) % 128 ||
      (g.head_dim != 32 && g.head_dim != 64 && g.head_dim != 128 && g.head_dim != 256) || g.latent_dim > 256 ||
      g.action_dim > 256)
    return PHYAI_ERR_UNSUPPORTED;

  phyai_ctx* c = new phyai_ctx();
  c->joint = 1;
  c->stream = static_cast<hipStream_t>(hip_stream);
  c->wt = W_BF16;
  c->es_io = 2;
  c->es_act = 2;
  if (hipGetDevice(&c->device) != hipSuccess) {
    delete c;
    return PHYAI_ERR_DEVICE;
  }
  Dims& d = c->base;
  d.L = g.n_layers; d.D = g.width; d.Hq = g.n_heads; d.Hkv = g.n_heads; d.dh = g.head_dim;
  d.F = g.mlp_dim; d.A = g.action_dim;
  d.H = g.latent_tokens + g.action_tokens;  // tokens of one branch
  d.B = 2; d.M = 2 * d.H; d.Mst = d.M;       // rows [0, H): conditional, [H, 2H): unconditional
  d.P = 0;
  d.KS = (d.H + 31) / 32 * 32;
  d.qkv = 3 * g.n_heads * g.head_dim;
  d.nmod = 2 * g.n_layers + 1;
  d.N = 1;
  d.eps = g.rms_eps;
  d.Lc = 1;                // K/V of the current layer only
  d.joint = 1;
  d.ntab = 2;
  d.rows_per_tab = d.H;
  d.Tl = g.latent_tokens;
  d.Cl = g.latent_dim;
  d.gamma = 0.f;
  d.rope_theta = 0.f;
  d.gated = 0;
  d.tmlp = 0;
  d.solver = g.solver_order;
  // mirror into cfg the fields the shared calls read
  c->cfg.n_layers = g.n_layers; c->cfg.width = g.width; c->cfg.n_q_heads = g.n_heads; c->cfg.n_kv_heads = g.n_heads;
  c->cfg.head_dim = g.head_dim; c->cfg.mlp_dim = g.mlp_dim; c->cfg.action_dim = g.action_dim;
  c->cfg.chunk_len = d.H; c->cfg.max_prefix_len = 0; c->cfg.max_batch = 2; c->cfg.weight_dtype = PHYAI_BF16;
  c->cfg.rms_eps = g.rms_eps; c->cfg.max_arena_bytes = g.max_arena_bytes;

  const int L = d.L, D = d.D, F = d.F, A = d.A, Cl = d.Cl, qd = d.Hq * d.dh;
  Layout lay;
  const size_t o_w_in = lay.take((size_t)D * Cl * 2), o_b_in = lay.take((size_t)D * 2);
  const size_t o_w_in2 = lay.take((size_t)D * A * 2), o_b_in2 = lay.take((size_t)D * 2);
  const size_t o_w_out = lay.take((size_t)Cl * D * 2), o_b_out = lay.take((size_t)Cl * 2);
  const size_t o_w_out2 = lay.take((size_t)A * D * 2), o_b_out2 = lay.take((size_t)A * 2);
  const size_t o_w_mod = lay.take((size_t)d.nmod * 2 * D * D * 2), o_b_mod = lay.take((size_t)d.nmod * 2 * D * 2);
  const size_t o_cond = lay.take((size_t)2 * D * 2);
  const size_t o_w_qkv = lay.take((size_t)L * d.qkv * D * 2), o_w_o = lay.take((size_t)L * D * qd * 2);
  const size_t o_w_gu = lay.take((size_t)L * 2 * F * D * 2), o_w_d = lay.take((size_t)L * D * F * 2);
  const size_t kv_elems = (size_t)d.B * d.Lc * d.Hkv * d.KS * d.dh;
  const size_t o_kc = lay.take(kv_elems * 2), o_vt = lay.take(kv_elems * 2);
  const size_t zero_begin = o_kc;
  const size_t o_x = lay.take(std::max<size_t>((size_t)d.Tl * Cl, 1) * 4);
  const size_t o_x2 = lay.take(std::max<size_t>((size_t)(d.H - d.Tl) * A, 1) * 4);
  const size_t n_state = (size_t)d.Tl * Cl + (size_t)(d.H - d.Tl) * A;  // latent then action elements
  const size_t o_ust = lay.take(d.solver ? 3 * n_state * 4 : 4);
  const size_t o_h = lay.take((size_t)d.M * D * 4), o_ssq = lay.take((size_t)(D / 16) * d.Mst * 4);
  const size_t mpad = (size_t)(d.M + 15) / 16 * 16;
  const size_t o_hs = lay.take(mpad * D * 2), o_q = lay.take((size_t)d.M * qd * 2);
  const size_t o_o = lay.take(mpad * qd * 2), o_act = lay.take(mpad * F * 2);
  const Plan plan = make_plan(d, c->wt);
  const int nblk = (d.H + 31) / 32;
  const size_t attn_ws = (nblk + plan.attn_bps - 1) / plan.attn_bps > 1 ? attn_ws_floats(d, plan) : 1;
  const size_t o_attn_ws = lay.take(attn_ws * 4), o_attn_cnt = lay.take(attn_counters(d) * 4);
  const size_t o_gemm_cnt = lay.take(gemm_counters(d) * 4);
  c->arena_bytes = lay.off;
  if (g.max_arena_bytes && c->arena_bytes > g.max_arena_bytes) {
    delete c;
    return PHYAI_ERR_OOM;
  }
  if (hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking) != hipSuccess) {
    delete c;
    return PHYAI_ERR_DEVICE;
  }
  if (hipMalloc(&c->arena, c->arena_bytes) != hipSuccess) {
    hipStreamDestroy(c->cap_stream);
    delete c;
    return PHYAI_ERR_OOM;
  }
  char* base = static_cast<char*>(c->arena);
  Bufs& b = c->b;
  b.w_in = base + o_w_in; b.b_in = base + o_b_in; b.w_in2 = base + o_w_in2; b.b_in2 = base + o_b_in2;
  b.w_out = base + o_w_out; b.b_out = base + o_b_out; b.w_out2 = base + o_w_out2; b.b_out2 = base + o_b_out2;
  b.w_mod = base + o_w_mod; b.b_mod = base + o_b_mod; b.cond = base + o_cond;
  b.w_qkv = base + o_w_qkv; b.w_o = base + o_w_o; b.w_gu = base + o_w_gu; b.w_d = base + o_w_d;
  b.kc = base + o_kc; b.vt = base + o_vt;
  b.x = reinterpret_cast<float*>(base + o_x);
  b.x2 = reinterpret_cast<float*>(base + o_x2);
  b.ust = d.solver ? reinterpret_cast<float*>(base + o_ust) : nullptr;
  b.h = reinterpret_cast<float*>(base + o_h);
  b.ssq = reinterpret_cast<float*>(base + o_ssq);
  b.hs = base + o_hs; b.q = base + o_q; b.o = base + o_o; b.act = base + o_act;
  b.attn_ws = reinterpret_cast<float*>(base + o_attn_ws);
  b.attn_cnt = reinterpret_cast<unsigned*>(base + o_attn_cnt);
  b.gemm_ws = nullptr;  // the tiled GEMMs reduce inside the workgroup
  b.gemm_cnt = reinterpret_cast<unsigned*>(base + o_gemm_cnt);
  // keys past the live rows must read as finite; activations and counters start at 0
  if (hipMemsetAsync(base + zero_begin, 0, c->arena_bytes - zero_begin, c->stream) != hipSuccess ||
      hipStreamSynchronize(c->stream) != hipSuccess) {
    hipFree(c->arena);
    hipStreamDestroy(c->cap_stream);
    delete c;
    return PHYAI_ERR_DEVICE;
  }
  *out = c;
  return PHYAI_OK;
}

phyai_status phyai_wam_set_weights(phyai_ctx* c, const phyai_wam_weights* w) {
  if (!c) return PHYAI_ERR_INVALID_ARG;
  c->err.clear();
  if (!c->joint) return fail(c, PHYAI_ERR_BAD_STATE, "wam_set_weights: not a joint denoiser context");
  if (!w || !w->w_in_lat || !w->b_in_lat || !w->w_in_act || !w->b_in_act || !w->w_out_lat || !w->b_out_lat ||
      !w->w_out_act || !w->b_out_act || !w->w_mod || !w->b_mod || !w->w_qkv || !w->w_o || !w->w_gu || !w->w_d)
    return fail(c, PHYAI_ERR_INVALID_ARG, "wam_set_weights: null weight pointer");
  const Dims& d = c->base;
  const int L = d.L, D = d.D, F = d.F, A = d.A, Cl = d.Cl, qd = d.Hq * d.dh;
  auto cp = [&](const void* dst, const void* src, size_t bytes) {
    return hipMemcpyAsync(const_cast<void*>(dst), src, bytes, hipMemcpyDeviceToDevice, c->stream);
  };
  auto sw = [&](const void* dst, const void* src, int64_t rows, int cols) {
    return enqueue_swizzle(src, const_cast<void*>(dst), rows, cols, 2, c->stream);
  };
  HIPCHK(c, cp(c->b.w_in, w->w_in_lat, (size_t)D * Cl * 2));
  HIPCHK(c, cp(c->b.b_in, w->b_in_lat, (size_t)D * 2));
  HIPCHK(c, cp(c->b.w_in2, w->w_in_act, (size_t)D * A * 2));
  HIPCHK(c, cp(c->b.b_in2, w->b_in_act, (size_t)D * 2));
  HIPCHK(c, cp(c->b.w_out, w->w_out_lat, (size_t)Cl * D * 2));
  HIPCHK(c, cp(c->b.b_out, w->b_out_lat, (size_t)Cl * 2));
  HIPCHK(c, cp(c->b.w_out2, w->w_out_act, (size_t)A * D * 2));
  HIPCHK(c, cp(c->b.b_out2, w->b_out_act, (size_t)A * 2));
  HIPCHK(c, cp(c->b.w_mod, w->w_mod, (size_t)d.nmod * 2 * D * D * 2));
  HIPCHK(c, cp(c->b.b_mod, w->b_mod, (size_t)d.nmod * 2 * D * 2));
  HIPCHK(c, sw(c->b.w_qkv, w->w_qkv, (int64_t)L * d.qkv, D));
  HIPCHK(c, sw(c->b.w_o, w->w_o, (int64_t)L * D, qd));
  HIPCHK(c, sw(c->b.w_gu, w->w_gu, (int64_t)L * 2 * F, D));
  HIPCHK(c, sw(c->b.w_d, w->w_d, (int64_t)L * D, F));
  HIPCHK(c, hipStreamSynchronize(c->stream));
  c->have_weights = true;
  c->have_tables = false;
  drop_graphs(c);
  return PHYAI_OK;
}

phyai_status phyai_wam_set_conditions(phyai_ctx* c, const void* c_cond, const void* c_uncond, float guidance) {
  if (!c) return PHYAI_ERR_INVALID_ARG;
  c->err.clear();
  if (!c->joint) return fail(c, PHYAI_ERR_BAD_STATE, "wam_set_conditions: not a joint denoiser context");
  if (!c_cond || !c_uncond) return fail(c, PHYAI_ERR_INVALID_ARG, "wam_set_conditions: null pointer");
  if (!std::isfinite(guidance)) return fail(c, PHYAI_ERR_INVALID_ARG, "wam_set_conditions: non-finite guidance");
  const size_t bytes = (size_t)c->base.D * 2;
  char* dst = static_cast<char*>(const_cast<void*>(c->b.cond));
  HIPCHK(c, hipMemcpyAsync(dst, c_cond, bytes, hipMemcpyDeviceToDevice, c->stream));
  HIPCHK(c, hipMemcpyAsync(dst + bytes, c_uncond, bytes, hipMemcpyDeviceToDevice, c->stream));
  HIPCHK(c, hipStreamSynchronize(c->stream));
  c->base.gamma = guidance;
  c->have_cond = true;
  c->have_tables = false;  // the modulation tables fold the conditions in
  drop_graphs(c);          // the guidance scale is a launch argument
  return PHYAI_OK;
}

phyai_status phyai_wam_denoise(phyai_ctx* c, const float* z_lat, const float* z_act, int n_steps, float* z_lat_out,
                               float* z_act_out) {
  if (!c) return PHYAI_ERR_INVALID_ARG;
  c->err.clear();
  if (!c->joint) return fail(c, PHYAI_ERR_BAD_STATE, "wam_denoise: not a joint denoiser context");
  const Dims& bd = c->base;
  const size_t lat_bytes = (size_t)bd.Tl * bd.Cl * 4, act_bytes = (size_t)(bd.H - bd.Tl) * bd.A * 4;
  if ((lat_bytes && (!z_lat || !z_lat_out)) || (act_bytes && (!z_act || !z_act_out)))
    return fail(c, PHYAI_ERR_INVALID_ARG, "wam_denoise: null pointer");
  if (!c->have_weights) return fail(c, PHYAI_ERR_BAD_STATE, "wam_denoise: weights not set");
  if (!c->have_tables) return fail(c, PHYAI_ERR_BAD_STATE, "wam_denoise: timestep tables not set");
  if (n_steps != c->n_steps) return fail(c, PHYAI_ERR_INVALID_ARG, "wam_denoise: n_steps differs from the tables");
  const Dims d = launch_dims(c, 2, 0, n_steps);
  const Plan plan = make_plan(d, c->wt);
  if (lat_bytes) HIPCHK(c, hipMemcpyAsync(c->b.x, z_lat, lat_bytes, hipMemcpyDeviceToDevice, c->stream));
  if (act_bytes) HIPCHK(c, hipMemcpyAsync(c->b.x2, z_act, act_bytes, hipMemcpyDeviceToDevice, c->stream));
  const phyai_status st = run_loop(c, d, plan, "wam_denoise");
  if (st != PHYAI_OK) return st;
  if (lat_bytes) HIPCHK(c, hipMemcpyAsync(z_lat_out, c->b.x, lat_bytes, hipMemcpyDeviceToDevice, c->stream));
  if (act_bytes) HIPCHK(c, hipMemcpyAsync(z_act_out, c->b.x2, act_bytes, hipMemcpyDeviceToDevice, c->stream));
  return PHYAI_OK;
}

phyai_status phyai_quantize_int4_g128(const float* w, int64_t rows, int64_t cols, uint8_t* packed,
                                      uint16_t* scales, void* hip_stream) {
  if (rows < 0 || cols < 0 || cols % 128) return PHYAI_ERR_INVALID_ARG;
  if (rows * cols == 0) return PHYAI_OK;
  if (!w || !packed || !scales) return PHYAI_ERR_INVALID_ARG;
  hipError_t e = enqueue_quantize_int4(w, rows, cols, packed, scales, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? PHYAI_OK : PHYAI_ERR_DEVICE;
}

}  // extern "C"
