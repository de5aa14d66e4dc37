/*
 * phyai.h -- C ABI of the MI355X (gfx950) cached-prefix flow-matching denoise loop.
 *
 * What the library computes (pages: "PhyAI: Real-Time Physical AI at the Edge,
 * Scalable Rollouts in the Cloud", reading Sec. 5.1 and Sec. 5.5; Figure 3):
 * a pi0.5-style action expert integrates a chunk of noisy action tokens with a
 * fixed number of explicit Euler steps of its learned velocity.  The
 * vision-language prefix is fixed during the whole loop, so its per-layer K/V
 * is handed over once ("cached") and reused by every step; the timestep /
 * modulation tables of a fixed schedule are precomputed once; a new
 * observation replaces (invalidates) the prefix before the next prediction.
 * The runner-like context owns the KV cache, the tables, the buffers and the
 * captured step graphs, which gives every cached tensor a defined lifetime
 * (Figure 3 and the Sec. 5.5 "separate request state from computation" item).
 *
 * Network of one step (readings of the pages, which print no architecture):
 *   h  = x W_in^T + b_in
 *   per layer l:  u = adaRMS(h; norm 2l);   [q|k|v] = u W_qkv[l]^T
 *                 K = [K_pre[l]; k], V = [V_pre[l]; v]   (chunk sees prefix + chunk)
 *                 o_i = softmax(q_i K_{i/g}^T / sqrt(dh)) V_{i/g}   (g = Hq/Hkv)
 *                 h += o W_o[l]^T
 *                 u = adaRMS(h; norm 2l+1);  h += (gelu_tanh(u W_g^T) * (u W_u^T)) W_d^T
 *   v  = adaRMS(h; norm 2L) W_out^T + b_out;   x += dt_k v
 *   adaRMS(h; j) = h / sqrt(mean(h^2) + eps) * (1 + scale_j(t_k)) + shift_j(t_k)
 *   [scale_j; shift_j](t) = W_mod[j] e(t) + b_mod[j],  e(t) = [sin(2 pi t/p_i) | cos(2 pi t/p_i)],
 *   p_i = 4e-3 * (4/4e-3)^(i/(D/2-1)).
 *
 * Conventions for every entry point:
 *  - Matrices are row-major, PyTorch Linear layout [out][in]; stacks over layers
 *    are outermost.  "dev" pointers are HIP device memory, "host" pointers are
 *    host memory.
 *  - Every input pointer is borrowed for the duration of the call only: the
 *    library copies what it keeps into its own device arena (stream-ordered on
 *    the context stream), so the caller may reuse its buffers afterwards.
 *  - Argument and state errors are reported synchronously as a status and a
 *    per-context message (phyai_last_error); the library never aborts.  Device
 *    errors of asynchronous work surface at the next call or at phyai_sync().
 *  - A context is not thread-safe; calls on one context must be serialised.
 */
#ifndef PHYAI_H
#define PHYAI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct phyai_ctx phyai_ctx;

typedef enum {
  PHYAI_OK = 0,
  PHYAI_ERR_INVALID_ARG = 1,   /* bad pointer, size or dimension */
  PHYAI_ERR_BAD_STATE = 2,     /* call order violated (e.g. denoise before weights) */
  PHYAI_ERR_OOM = 3,           /* arena larger than max_arena_bytes or hipMalloc failed */
  PHYAI_ERR_DEVICE = 4,        /* a HIP runtime call failed */
  PHYAI_ERR_UNSUPPORTED = 5    /* dimensions the kernels do not implement */
} phyai_status;

typedef enum {
  PHYAI_F32 = 0,        /* weights, prefix K/V and activations fp32 */
  PHYAI_BF16 = 1,       /* weights and prefix K/V bf16; GEMM inputs bf16; fp32 accumulation,
                           residual stream, norm statistics, softmax and state */
  PHYAI_INT4_G128 = 2   /* as BF16, but the four expert linears (QKV, O, gate/up, down) are
                           symmetric int4 with one bf16 scale per 128 consecutive inputs */
} phyai_dtype;

/* Model and capacity.  Constraints (else PHYAI_ERR_UNSUPPORTED): width a multiple of 256
 * and <= 2048; mlp_dim and n_q_heads*head_dim multiples of 128; head_dim 32, 64, 128 or
 * 256; n_q_heads a multiple of n_kv_heads; action_dim a multiple of 8 and <= 256.  Up to
 * 64 token rows (batch x chunk_len) run on weight-streaming kernels (any weight dtype),
 * which deal each wave a power-of-two run of k-blocks: when chunk_len <= 64 or prefill = 1,
 * width / 128, n_q_heads*head_dim / 128 and mlp_dim / 128 must each be a power of two
 * <= 64.  More rows run on LDS-tiled MFMA GEMMs, which need PHYAI_BF16 and
 * (Hq+2Hkv)*head_dim a multiple of 128.  The activation element type follows the weight
 * dtype (fp32 for PHYAI_F32, bf16 otherwise), so no separate activation dtype is taken. */
typedef struct {
  int n_layers, width, n_q_heads, n_kv_heads, head_dim, mlp_dim;
  int action_dim, chunk_len, max_prefix_len, max_batch;
  phyai_dtype weight_dtype;
  float rms_eps;              /* > 0, e.g. 1e-6 */
  size_t max_arena_bytes;     /* 0 = no limit; else creation fails with OOM above it */
  float rope_theta;           /* 0: no positional encoding of the chunk (the prefix K/V comes
                                 encoded); > 1: rotary embedding of the chunk's queries and keys
                                 at positions P + t (chunk token t after a P-token prefix):
                                 interleaved pairs (2i, 2i+1) of every head turned by
                                 (P + t) * rope_theta^(-2i/head_dim) (the pages stress positional
                                 precision, PhyAI reading Sec. 2; the convention is a reading) */
  int gated_residual;         /* 0: plain residual blocks; 1: each norm's modulation map also
                                 yields a gate g (w_mod [2L+1][3D][D], b_mod [2L+1][3D]: rows
                                 0..D-1 scale, D..2D-1 shift, 2D..3D-1 gate) and a block's
                                 output enters the residual as g * output (a reading) */
  int time_mlp;               /* 0: the modulation maps read the timestep embedding e(t); 1: they
                                 read W_tm2 swish(W_tm1 e + b_tm1) + b_tm2 (phyai_weights w_tm*,
                                 swish(z) = z / (1 + exp(-z)); a reading) */
  int prefill;                /* 1: the context also holds a prefix network and can compute the
                                 prefix K/V itself (phyai_prefill); fp32 or bf16 weights, bf16 when
                                 max_batch * max_prefix_len > 64; not with rope_theta > 0 (the
                                 prefix network stores its K/V without positions) */
} phyai_config;

/* Device pointers to the weights.  Element type: fp32 for PHYAI_F32, bf16 otherwise,
 * except the four expert linears under PHYAI_INT4_G128, which are packed codes
 * (uint8 [L][N][K/2]: byte j of a row holds input 2j in its low nibble and 2j+1 in
 * its high nibble, two's complement) with bf16 scales s_* [L][N][K/128]
 * (w = code * scale), as written by phyai_quantize_int4_g128.
 *   w_in [D][A], b_in [D], w_out [A][D], b_out [A]
 *   w_mod [2L+1][2D][D], b_mod [2L+1][2D]   (rows 0..D-1 scale, D..2D-1 shift; norm j:
 *                                           2l attention norm, 2l+1 MLP norm, 2L final;
 *                                           gated_residual: [2L+1][3D][D] and [2L+1][3D],
 *                                           rows 2D..3D-1 the residual gate)
 *   w_qkv [L][(Hq+2Hkv)*dh][D]  (rows: q heads, then k heads, then v heads)
 *   w_o [L][D][Hq*dh], w_gu [L][2F][D] (rows 0..F-1 gate, F..2F-1 up), w_d [L][D][F] */
typedef struct {
  const void *w_in, *b_in, *w_out, *b_out, *w_mod, *b_mod;
  const void *w_qkv, *w_o, *w_gu, *w_d;
  const void *s_qkv, *s_o, *s_gu, *s_d;
  const void *w_tm1, *b_tm1, *w_tm2, *b_tm2;   /* time_mlp only: [D][D], [D], [D][D], [D] (io type) */
} phyai_weights;

/* Create a context on the current HIP device (PhyAI reading, Figure 3 and the Sec. 5.5
 * item on separating request state from computation: a stateful runner owns the KV cache,
 * the buffers and the graph buckets, so cached tensors have a defined lifetime).
 * hip_stream: the hipStream_t every call is ordered on (NULL = the null stream).
 * Allocates the whole device arena (weights, KV cache for max_batch x (max_prefix_len +
 * chunk_len) keys, buffers) at once; nothing on the denoise path allocates afterwards.
 * *out receives the context, or NULL on error (no message is kept then): INVALID_ARG for a
 * null pointer or a non-positive size, UNSUPPORTED for shapes outside the constraints
 * above, OOM when the arena exceeds max_arena_bytes or the allocation fails, DEVICE when
 * no HIP device is usable. */
phyai_status phyai_create(const phyai_config* cfg, void* hip_stream, phyai_ctx** out);

/* Copy the weights (dev pointers, layouts above) into the arena (PhyAI reading Sec. 5.4
 * and Figure 3: weights are prepared offline and loaded once by the runner).  The expert
 * linears are re-laid out for the kernels on the way in.  Must precede
 * phyai_set_timestep_tables (the tables fold the weights' response to the shift) and
 * invalidates any tables and captured graphs.  INVALID_ARG for a null pointer (int4: the
 * four scale arrays too; time_mlp: its four tensors); the pointers are only read. */
phyai_status phyai_set_weights(phyai_ctx* ctx, const phyai_weights* w);

/* Install the cached prefix K/V (PhyAI reading Sec. 5.1: computed once per
 * observation and reused by every Euler step).  k, v: dev [batch][L][prefix_len][Hkv][dh]
 * in the weight element type (fp32 or bf16).  Replaces any previous prefix: this
 * is the cache invalidation point.  1 <= batch <= max_batch,
 * 1 <= prefix_len <= max_prefix_len. */
phyai_status phyai_set_prefix_kv(phyai_ctx* ctx, const void* k, const void* v,
                                 int batch, int prefix_len);

/* Prefix network of a context created with prefill = 1: the four linears of its L layers
 * (dev pointers, fp32 or bf16 as the expert's; shapes and row order as the expert's w_qkv,
 * w_o, w_gu, w_d).  The layer is the expert's with a plain RMSNorm in place of the
 * adaptive one, no positional encoding, and bidirectional attention among the prefix
 * tokens only.  Copied (re-laid out) into the arena. */
typedef struct {
  const void *w_qkv, *w_o, *w_gu, *w_d;
} phyai_prefill_weights;
phyai_status phyai_set_prefill_weights(phyai_ctx* ctx, const phyai_prefill_weights* w);

/* Compute the prefix K/V from the prefix tokens and install it (PhyAI reading Sec. 5.1:
 * the vision-language prefix is computed once per observation; Sec. 8.2 check 1).  tokens:
 * dev [batch][prefix_len][width] in the weight element type (the prefix network's input
 * embeddings).  Runs the prefix network's L layers over the batch x prefix_len rows on the
 * context stream; every layer's K/V lands in the cache rows the cached loop reads, replacing
 * any previous prefix (the invalidation point, as phyai_set_prefix_kv).  Requires
 * phyai_set_prefill_weights; 1 <= batch <= max_batch, 1 <= prefix_len <= max_prefix_len.
 * Overwrites the loop's activation buffers (a denoise call after it starts afresh). */
phyai_status phyai_prefill(phyai_ctx* ctx, const void* tokens, int batch, int prefix_len);

/* Execution-state capsules (page "FlashRT-PAI speeds physical AI inference up to 12.66x",
 * its account of the three mechanisms: capsules snapshot, restore and fork persistent
 * state).  The persistent state of an action-expert context is its installed prefix:
 * batch, prefix length and every layer's cached prefix K/V (each denoise starts from the
 * noise it is given, so nothing else carries over between predictions).
 * A capsule is caller-owned device memory of phyai_capsule_bytes(ctx) bytes (0: no prefix
 * installed, a joint context, or ctx NULL); the library keeps no pointer to it.  Layout:
 * a 256-byte header (uint64 magic, then int32 version, batch, prefix_len, layers, KV heads,
 * head_dim, element bytes), then K [batch][layers][KV heads][prefix_len][head_dim] and
 * V^T [batch][layers][KV heads][head_dim][prefix_len] in the activation element type.
 *   save:    snapshot the installed prefix into the capsule; header and payload are
 *            written by kernels, asynchronous on the stream.  PHYAI_ERR_BAD_STATE without
 *            a prefix, PHYAI_ERR_INVALID_ARG for a NULL or short buffer.
 *   restore: install the prefix a capsule holds, replacing the current one (the
 *            invalidation point, as phyai_set_prefix_kv); the capsule may come from any
 *            context with the same layers, KV heads, head_dim and element type whose
 *            max_batch and max_prefix_len it fits.  Waits for the stream, then reads the
 *            header; a foreign or short buffer or a shape that does not fit is
 *            PHYAI_ERR_INVALID_ARG and leaves the installed prefix unchanged.
 *   fork:    copy sample src's prefix into sample slot dst of the installed batch, so that
 *            several rollouts share one observation (stream-ordered); indices outside
 *            [0, batch) are PHYAI_ERR_INVALID_ARG. */
size_t phyai_capsule_bytes(const phyai_ctx* ctx);
phyai_status phyai_capsule_save(phyai_ctx* ctx, void* capsule, size_t capsule_bytes);
phyai_status phyai_capsule_restore(phyai_ctx* ctx, const void* capsule, size_t capsule_bytes);
phyai_status phyai_capsule_fork(phyai_ctx* ctx, int src_sample, int dst_sample);

/* Precompute the timestep / modulation tables of a schedule (PhyAI reading
 * Sec. 5.1: fixed tables over the fixed schedule).  t_host: host float[n_steps], the
 * times at which the velocity is evaluated; step k advances by dt_k = t_{k+1} - t_k
 * with t_{n_steps} = 0 (uniform: t_k = 1 - k/N, dt = -1/N).  Requires weights. */
phyai_status phyai_set_timestep_tables(phyai_ctx* ctx, const float* t_host, int n_steps);

/* Run the whole Euler loop (PhyAI reading Sec. 5.1: the chunk is denoised by a fixed
 * number of Euler steps over the cached prefix, and the loop is replayed as one captured
 * graph): actions_out = x at t = 0 starting from x = noise at t_0.
 * noise, actions_out: dev float [batch][chunk_len][action_dim] (caller-owned; noise is
 * only read).  1 <= batch <= the batch of the installed prefix: sample b uses prefix
 * sample b, and samples never interact.  A batch that does not fill its graph bucket is
 * padded (PhyAI reading Sec. 8.1, Appendix D: local graph batch and padding): the graph
 * of the bucket runs, the pad slots compute on whatever their cache rows hold, and only
 * the first `batch` samples are written to actions_out.  Buckets: the exact batch while
 * batch x chunk_len <= 64 (the weight-streaming path), else the batch rounded up to a
 * multiple of 8, capped at the installed batch.  n_steps must equal the table length.
 * Asynchronous on the context stream; one hipGraph launch, captured on first use for
 * each (bucket, prefix_len, n_steps); at most 16 graphs are kept (least recently used
 * evicted).  BAD_STATE before weights, prefix or tables; INVALID_ARG for null pointers,
 * a batch outside [1, installed batch] or n_steps different from the tables. */
phyai_status phyai_denoise(phyai_ctx* ctx, const float* noise, int batch, int n_steps,
                           float* actions_out);

/* Allocation-free denoise, for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops or harnesses that forbid hipMalloc).  Same arguments, checks,
 * bucketing and result as phyai_denoise (bitwise: the same kernels in the same order), but
 * the loop is launched eagerly (no graph is captured, the persistent loop is not used) and
 * its split-reduction scratch (partial sums and arrival counters) lives in the library's
 * static device array of 16 MiB per device, held until the process ends, instead of the
 * context's arena.  The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).  Every call on one device shares that array: the counters are cleared
 * at the start of each call, and calls that overlap on one device (other streams or
 * contexts) race and give wrong results.  INVALID_ARG, with the sizes in phyai_last_error,
 * when the batch and prefix need more than 16 MiB of scratch (e.g. pi0.5 at batch 1 and
 * prefix 816 needs about 12.0 MiB); DEVICE if the array's address could not be obtained
 * when the context was created. */
phyai_status phyai_denoise_noalloc(phyai_ctx* ctx, const float* noise, int batch, int n_steps,
                                   float* actions_out);

/* Choose graph replay (1, default) or eager kernel launches (0) for phyai_denoise.
 * Both run the same kernels in the same order and give bitwise identical results. */
phyai_status phyai_set_graph_mode(phyai_ctx* ctx, int use_graph);

/* Persistent loop (page "FlashRT-PAI speeds physical AI inference up to 12.66x": deep kernel
 * fusion with launch overlap).  For batches of at most 64 token rows with bf16 weights and a
 * supported shape (n_q_heads a multiple of 8, (n_q_heads/8)*head_dim a multiple of 128, width
 * a multiple of 256, mlp_dim of 1024, no rotary positions or residual gates; implemented for
 * the pi0.5-shaped expert and head_dim 128 / width 256 / mlp_dim 1024 test shapes), the whole
 * N-step loop runs as one cooperative launch of 256 co-resident workgroups that hand each
 * phase's results to the next through flags in device memory; every other call runs the
 * graph of per-layer launches.  enable = 1 uses it where supported, 0 (default) never.  The
 * persistent launch cannot be captured into a caller's graph: leave it disabled for capture.
 * Its buffers (about 1.3 MB per step and layer for the pi0.5 shape) are allocated with the
 * timestep tables, or by this call when the tables are already set (the call then waits for
 * the context stream); without them the graph path runs.  A wait that exceeds its bound
 * aborts the launch; phyai_sync then reports PHYAI_ERR_DEVICE and resets the loop's flags. */
phyai_status phyai_set_persistent(phyai_ctx* ctx, int enable);

/* Which form a phyai_denoise of `batch` samples would run now: 1 the persistent kernel, 0 the
 * graph (or eager) launches, -1 not runnable (prefix or tables missing, bad batch, NULL). */
int phyai_loop_form(const phyai_ctx* ctx, int batch);

/* Wait for the context stream; reports asynchronous device errors (DEVICE, with the
 * HIP message in phyai_last_error).  The reading of the pages' request life cycle
 * (PhyAI reading Sec. 5.4: a request ends when its action chunk is ready) is this call:
 * after it returns OK, actions_out holds the chunk. */
phyai_status phyai_sync(phyai_ctx* ctx);

/* Message of the last failed call on ctx ("" if none; "null context" for NULL).  Valid
 * until the next call on ctx.  Errors are values, never aborts (PhyAI reading Sec. 8.2
 * check 1 asks failures to be reported; the runner's state survives a rejected call). */
const char* phyai_last_error(const phyai_ctx* ctx);

/* Static name of a status code. */
const char* phyai_status_string(phyai_status s);

/* Free the context, its arena, tables and graphs (synchronises its stream first), which
 * ends the lifetime of every cached tensor the context owned (PhyAI reading Figure 3).
 * NULL is a no-op. */
void phyai_destroy(phyai_ctx* ctx);

/* Offline round-to-nearest int4 quantiser (PhyAI reading Sec. 5.4 and Figure 3:
 * the quantizer prepares low-precision artifacts offline).  w: dev float [rows][cols],
 * cols a multiple of 128.  Per row and group G of 128 columns: s = bf16_rne(max|W_G| / 7)
 * (fp32 division; s = 0 for an all-zero group), code = clamp(round_half_even(W / s), -8, 7)
 * (fp32 division; 0 when s = 0).  Writes packed dev uint8 [rows][cols/2] (nibble order as
 * in phyai_weights) and scales dev uint16 (bf16 bits) [rows][cols/128].  Asynchronous on
 * hip_stream. */
phyai_status phyai_quantize_int4_g128(const float* w, int64_t rows, int64_t cols,
                                      uint8_t* packed, uint16_t* scales, void* hip_stream);

/* Copy the precomputed modulation tables out, for checking: dst dev float
 * [n_steps][2L+1][2][D] holding (scale, shift) of every norm at every step. */
phyai_status phyai_get_modulation(phyai_ctx* ctx, float* dst);

/* Measurement aid: enqueue on the context stream one graph replay of `reps` back-to-back
 * launches of a single kernel of the loop, with the arguments it has at step 0 and layer
 * `layer`.  which: 0 norm-folded QKV (+ chunk K/V into the cache), 1 attention, 7 merge of
 * the attention's key splits (nothing is enqueued where attention merges in-kernel or
 * runs unsplit), 2 O-projection + residual, 3 gate/up + GeGLU, 4 down-projection + residual,
 * 5 out-projection + Euler + in-projection, 6 first in-projection.  Requires weights, prefix and tables.  The caller
 * brackets the call with events on the same stream to time one kernel in isolation.  It
 * overwrites the context's activations, state and chunk K/V rows (re-run phyai_denoise after). */
phyai_status phyai_enqueue_kernel_repeat(phyai_ctx* ctx, int which, int layer, int reps);

/* Measurement aid: the in-loop duration of each kernel of phyai_denoise.  Queues the same
 * loop as phyai_denoise for `batch` (same bucket, launches and order) on the context stream
 * with an event recorded before the first launch and after every launch, behind a 20 ms
 * one-wave wait so that the queued launches run back to back; `reps` times (1..1000) from
 * x = noise, each run synchronised.  Returns in host
 * stage_us[8] the mean time in microseconds between the events around each launch of a
 * kernel id (0 QKV, 1 attention, 2 O + residual, 3 gate/up, 4 down + residual,
 * 5 out-projection/Euler/in-projection, 6 first in-projection, 7 merge of the attention
 * splits; 0 for an id with no launch), and in host *chunk_ms the mean first-to-last event
 * interval of a run.  Synchronous; the events are released before return.  Arguments and
 * state are checked as for phyai_denoise. */
phyai_status phyai_time_loop_stages(phyai_ctx* ctx, const float* noise, int batch, int reps, float* stage_us,
                                    float* chunk_ms);

/* ---------------------------------------------------------------- joint video/action denoiser
 * (PhyAI reading, Figure 4 and Sec. 5.5 third item; Sec. 5.4): latent video tokens and action
 * tokens evolve together in one sequence under full self-attention (no cached prefix, no
 * mask, nothing kept across steps); a conditional and an unconditional branch run as a
 * batch of two and are combined before the update:
 *   h  = [z_lat W_in_lat^T + b_in_lat ; z_act W_in_act^T + b_in_act]      (T = Tl + Ta rows)
 *   per branch b (condition c_b) the layer stack of the action expert with Hq = Hkv heads,
 *   modulation [scale_j; shift_j](t) = W_mod[j] (e(t) + c_b) + b_mod[j], keys = the T tokens;
 *   v_b = adaRMS(h; 2L) W_out_type^T + b_out_type  (latent rows: *_lat, action rows: *_act)
 *   v  = v_u + gamma (v_c - v_u),   z += dt_k v   (or the UniPC update of solver_order 1, 2)
 * The same context calls apply: phyai_set_timestep_tables, phyai_set_graph_mode, phyai_sync,
 * phyai_last_error, phyai_get_modulation ([n_steps][2][2L+1][2][D], branch-major: cond then
 * uncond), phyai_enqueue_kernel_repeat (which 0..4 and 7 as for the expert, 5 out-projections +
 * guidance + Euler + in-projections, 6 first in-projections) and phyai_destroy.
 * phyai_set_prefix_kv and phyai_denoise refuse a joint context (PHYAI_ERR_BAD_STATE), and the
 * phyai_wam_* calls refuse an action-expert context. */

/* bf16 weights, fp32 accumulation, residual stream, statistics, softmax and state.
 * Constraints (else PHYAI_ERR_UNSUPPORTED): width a multiple of 256 and <= 2048; mlp_dim and
 * n_heads*head_dim multiples of 128; head_dim 32, 64, 128 or 256; latent_dim and action_dim
 * in [1, 256]; latent_tokens, action_tokens >= 0 with at least one token. */
typedef struct {
  int n_layers, width, n_heads, head_dim, mlp_dim;
  int latent_tokens, latent_dim, action_tokens, action_dim;
  float rms_eps;              /* > 0 */
  size_t max_arena_bytes;     /* 0 = no limit */
  int solver_order;           /* 0: Euler (z += dt_k v); 1 or 2: UniPC with this predictor order and
                               * its corrector (see phyai_wam_denoise); else PHYAI_ERR_INVALID_ARG */
} phyai_wam_config;

/* bf16 dev pointers, row-major [out][in]:
 *   w_in_lat [D][Cl], b_in_lat [D], w_in_act [D][A], b_in_act [D],
 *   w_out_lat [Cl][D], b_out_lat [Cl], w_out_act [A][D], b_out_act [A],
 *   w_mod [2L+1][2D][D], b_mod [2L+1][2D]  (as in phyai_weights),
 *   w_qkv [L][3 H dh][D] (q heads, k heads, v heads), w_o [L][D][H dh],
 *   w_gu [L][2F][D] (gate rows, then up rows), w_d [L][D][F]. */
typedef struct {
  const void *w_in_lat, *b_in_lat, *w_in_act, *b_in_act;
  const void *w_out_lat, *b_out_lat, *w_out_act, *b_out_act;
  const void *w_mod, *b_mod, *w_qkv, *w_o, *w_gu, *w_d;
} phyai_wam_weights;

/* Create a joint-denoiser context on the current HIP device (arena for the weights, the two
 * branches' activations and one layer of K/V).  Same stream and error rules as phyai_create. */
phyai_status phyai_wam_create(const phyai_wam_config* cfg, void* hip_stream, phyai_ctx** out);

/* Copy the weights (layouts above) into the arena; invalidates tables and graphs. */
phyai_status phyai_wam_set_weights(phyai_ctx* ctx, const phyai_wam_weights* w);

/* Branch conditions and guidance scale: c_cond, c_uncond dev bf16 [D] (added to the timestep
 * embedding of the conditional / unconditional branch), guidance gamma finite.  Must precede
 * phyai_set_timestep_tables (the tables fold the conditions in); invalidates tables and graphs. */
phyai_status phyai_wam_set_conditions(phyai_ctx* ctx, const void* c_cond, const void* c_uncond,
                                      float guidance);

/* UniPC (solver_order 1 or 2; the multistep solver the PhyAI reading names for the
 * video/action states, Figure 4 and its parallelism section, read as the published UniPC
 * predictor-corrector): with alpha_t = 1 - t, sigma_t = t, lambda_t = log(alpha_t / sigma_t)
 * and the data prediction m_k = z_k - t_k v_k of the guided velocity at the evaluated
 * state z_k, a step s -> t sets
 *   z_t = (sigma_t / sigma_s) z_s + alpha_t * sum_j w_j m_j,
 * the weights integrating e^{-(lambda_t - lambda)} against the polynomial in lambda through
 * the data predictions used: the predictor (t_k -> t_{k+1}) uses m_k and, at order 2,
 * m_{k-1}; after the model is evaluated at z_{k+1}, the corrector redoes the step from the
 * corrected z_k with m_{k+1} added.  Points at t = 1 enter only as a step's base, and the
 * step to t = 0 is first order (z_N = m_{N-1}).  The weights are computed in float64 by
 * phyai_set_timestep_tables, which then requires 1 >= t_0 > t_1 > ... > t_{N-1} > 0
 * (else PHYAI_ERR_INVALID_ARG); solver order 0 keeps the Euler update below. */

/* Host helper, no device needed: the UniPC step weights that phyai_set_timestep_tables
 * computes for the schedule t_host[0..n_steps) at predictor order 1 or 2, written to
 * out_host[8 * n_steps] as, per step k: t_k; the corrector of the step into t_k (A on the
 * corrected z_{k-1}, w on m_k, w on m_{k-1}, w on m_{k-2}; zeros at k = 0); the predictor out
 * of t_k (A on the corrected z_k, w on m_k, w on m_{k-1}).  PHYAI_ERR_INVALID_ARG for a null
 * pointer, n_steps < 1, another order, or a schedule not strictly decreasing in (0, 1]. */
phyai_status phyai_unipc_weights(const float* t_host, int n_steps, int order, float* out_host);

/* Run the guided loop from z = (z_lat, z_act) at t_0 to t = 0.  z_lat, z_lat_out: dev
 * float [latent_tokens][latent_dim]; z_act, z_act_out: dev float [action_tokens][action_dim]
 * (a pointer may be NULL when its token count is 0).  n_steps must equal the table length.
 * Asynchronous on the context stream, one hipGraph launch (captured once per n_steps). */
phyai_status phyai_wam_denoise(phyai_ctx* ctx, const float* z_lat, const float* z_act, int n_steps,
                               float* z_lat_out, float* z_act_out);

/* Library version string. */
const char* phyai_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PHYAI_H */
