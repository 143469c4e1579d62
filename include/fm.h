/*
 * fm.h - C ABI of the flow-matching denoise loop of a VLA action head (MI355X / gfx950).
 *
 * What it computes. An action chunk X in R^{B x H x d_a} is integrated by explicit Euler
 * steps X^{k+1} = X^k + (tau_{k+1} - tau_k) v(X^k, tau_k, C) for k = 0..T-1 (vla.cpp: A
 * Unified Inference Runtime for Vision-Language-Action Models, Sec. III-A, Eq. (1)). The
 * velocity v is one pass of a modulated action-expert transformer over the chunk tokens,
 * attending to conditioning C bound once per observation (vla.cpp Sec. III-B, Eq. (2)):
 *   - FM_ARCH_PREFIX_JOINT: pi0.5-shaped expert (pi0.5 Design page: architecture diagram,
 *     sequence diagram, "Component contract", "Attention and the K/V pool"). Per layer:
 *     AdaRMS-modulated norm, Q/K/V with RoPE at positions P + i, attention over the bound
 *     prefix K/V followed by the chunk's own K/V through ONE shared K/V head, gated
 *     residual, AdaRMS norm, gated-GELU MLP, gated residual; final AdaRMS norm and the
 *     velocity projection.
 *   - FM_ARCH_DIT_CROSS: GR00T-style DiT head (GR00T N1.7 page, section "action" and
 *     "Build-time constants"): a state token then the action tokens; even blocks
 *     cross-attend into a context projected to K/V once at bind, odd blocks self-attend;
 *     AdaLN-modulated LayerNorm with a gated attention residual; plain LayerNorm + GELU
 *     feed-forward; AdaLN output norm and the velocity projection.
 * The per-step modulation rows (scale, shift, gate) come from a time embedding passed
 * through a time MLP and one Dense per norm site; they depend only on the schedule and
 * are computed by fm_set_schedule, off the step path (pi0.5 Design: the cond component).
 *
 * Threading and streams. One context per caller thread; a context is not thread-safe.
 * Every call enqueues its device work on the stream given to fm_create and returns
 * without waiting, except where stated. An error returns a status, sets the message read
 * by fm_last_error and never aborts; after FM_ERR_DEVICE the context is poisoned and every
 * later call but fm_destroy / fm_last_error returns FM_ERR_DEVICE.
 *
 * Memory. Pointers documented "device" are HIP device pointers (e.g. torch tensors'
 * data_ptr()); "host" pointers are ordinary host memory. Weights, prefix K/V and context
 * are consumed (copied / projected) into library-owned, address-stable device memory by
 * work enqueued on the context stream: the caller may free or reuse its buffers once that
 * stream has passed the call. The library never retains caller pointers across calls.
 */
#ifndef FM_H_
#define FM_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fm_ctx fm_ctx;

typedef enum {
  FM_OK = 0,
  FM_ERR_INVALID_ARG = 1, /* null pointer, out-of-range count or config field */
  FM_ERR_SHAPE = 2,       /* tensor name/rank/shape/dtype mismatch at load */
  FM_ERR_STATE = 3,       /* call order: weights, schedule or binding missing */
  FM_ERR_SCHEDULE = 4,    /* steps or batch disagree with the schedule / binding */
  FM_ERR_UNSUPPORTED = 5, /* a configuration this build does not implement */
  FM_ERR_OOM = 6,         /* device allocation failed */
  FM_ERR_DEVICE = 7       /* a HIP call failed; the context is poisoned */
} fm_status;

enum { FM_ARCH_PREFIX_JOINT = 0, FM_ARCH_DIT_CROSS = 1 };
enum { FM_F32 = 0, FM_BF16 = 1 };

/* Model and capacity description, fixed for the life of a context.
 *  arch            FM_ARCH_PREFIX_JOINT or FM_ARCH_DIT_CROSS
 *  dtype           FM_F32 or FM_BF16: weights, K/V and GEMM operands; accumulation, the
 *                  residual stream, the modulation table, x and v are always fp32
 *  n_layers        expert layers (DiT: blocks; even 0-based blocks cross-attend)
 *  hidden          D, a multiple of 64
 *  n_heads, head_dim, n_kv_heads
 *                  PREFIX_JOINT requires n_kv_heads == 1 (the pages' pool constraint);
 *                  DIT_CROSS requires n_kv_heads == n_heads; head_dim in {64, 128, 256}
 *  mlp_dim         F; mlp_gated = 1: GELU(gate) * up (PREFIX_JOINT), 0: GELU (DiT)
 *  action_horizon  H tokens per request; action_dim d_a
 *  state_tokens, state_dim   DiT state token(s) prepended to the action tokens (0 otherwise)
 *  ctx_len_max, ctx_dim      DiT context capacity and width (0 otherwise)
 *  max_prefix_len  capacity of the prefix part of the K/V pool (PREFIX_JOINT)
 *  max_batch, max_steps      capacity of a binding and a schedule
 *  rope_base       RoPE base (0 = no RoPE); norm_eps    epsilon of every norm */
typedef struct {
  int32_t arch, dtype, n_layers, hidden, n_heads, head_dim, n_kv_heads, mlp_dim, mlp_gated,
      action_horizon, action_dim, state_tokens, state_dim, ctx_len_max, ctx_dim,
      max_prefix_len, max_batch, max_steps;
  float rope_base, norm_eps;
} fm_config;

/* One named weight tensor: dtype must equal the config dtype, shape in nn.Linear
 * convention [out, in], data a contiguous row-major DEVICE buffer. */
typedef struct {
  const char* name;
  int32_t dtype;
  int32_t ndim;
  int64_t shape[4];
  const void* data;
} fm_tensor;

/* Sizes derived from a config, computed on the host without touching a device. */
typedef struct {
  int32_t n_sites;        /* modulation sites: 2L+1 (PREFIX_JOINT) or L+1 (DIT_CROSS) */
  int32_t pool_capacity;  /* K/V slots per request: max_prefix_len + H rounded up to 256 */
  int32_t n_weights;      /* number of weight tensors fm_load_weights expects */
  int64_t weight_bytes;   /* device bytes of weights after load */
  int64_t pool_bytes;     /* device bytes of the K/V pool / bound context */
} fm_plan_info;

/* Validate a config and report derived sizes. Host only; needs no GPU.
 * Returns FM_ERR_INVALID_ARG / FM_ERR_UNSUPPORTED with a message in msg (may be NULL). */
fm_status fm_query(const fm_config* cfg, fm_plan_info* info, char* msg, int32_t msg_len);

/* Name of the i-th weight tensor expected by fm_load_weights, in a fixed order, and its
 * shape. Host only. Returns FM_ERR_INVALID_ARG for i out of range. */
fm_status fm_weight_spec(const fm_config* cfg, int32_t i, const char** name, int32_t* ndim, int64_t shape[4]);

/* Whether a device can run this library, from its properties alone (host only, no GPU
 * needed): gcn_arch the agent name (hipDeviceProp_t::gcnArchName), num_xcc the XCD count
 * (hipDeviceAttributeNumberOfXccs), num_cus the compute units. The split-K GEMMs and the loop
 * kernel exchange partial results through one XCD's L2 and rely on the whole-GPU dispatch
 * that deals a launch's workgroups round-robin over the XCDs (each residue of the workgroup
 * index mod 8 on one XCD), so a gfx950 with 8 XCDs (a whole MI355X) is required;
 * FM_ERR_UNSUPPORTED with a message in msg (may be NULL) otherwise, and FM_ERR_INVALID_ARG for
 * a NULL gcn_arch. fm_create applies this check to its device, and also launches a probe
 * whose workgroups report their XCD, refusing the device unless the placement is round-robin.
 * The loop kernel verifies it again on every launch (see fm_loop_status). */
fm_status fm_device_supported(const char* gcn_arch, int32_t num_xcc, int32_t num_cus, char* msg, int32_t msg_len);

/* Create a context on the current HIP device (refused with FM_ERR_UNSUPPORTED unless
 * fm_device_supported accepts it). hip_stream: a hipStream_t (NULL = the default stream) on
 * which all of this context's work runs, in order (pi0.5 Design, "Runtime boundary": one
 * caller stream per engine, and a context is not safe to share between threads). Allocates
 * the pool and the activation buffers for max_batch. */
fm_status fm_create(const fm_config* cfg, void* hip_stream, fm_ctx** out);

/* Synchronize the context stream and release every device allocation (GR00T N1.7, "Who
 * runs what": the runner owns execution and the lifetime of its buffers). NULL is a no-op. */
fm_status fm_destroy(fm_ctx* ctx);

/* Message of the last failed call on ctx (or of the last failed fm_create / fm_query /
 * fm_device_supported / kernel-level call when ctx is NULL). Valid until the next call on the
 * same context. What this build does not implement is refused with a status and a message
 * instead of being run (pi0.5 Design, "Runtime boundary": an unimplemented configuration is
 * refused at load rather than run; GR00T N1.7, "Who runs what": a mismatch fails at load).
 * That a device error poisons the context is this library's own rule. */
const char* fm_last_error(const fm_ctx* ctx);

/* Load all weights (fm_weight_spec lists names and shapes). Each tensor is validated
 * (name, dtype, rank, shape: a mismatch names expected vs got and returns FM_ERR_SHAPE)
 * and then copied into the library's layout; nothing is loaded that does not match, and no
 * tensor is silently cast, reshaped or skipped (GR00T N1.7, "Checkpoint": a checkpoint whose
 * tensors do not fit the build is refused at load; pi0.5 Design, "Component contract": the
 * expert's tensor names and shapes are part of the contract). Biases are converted to fp32.
 * Calling it again replaces the weights and invalidates schedule and captured graphs. */
fm_status fm_load_weights(fm_ctx* ctx, const fm_tensor* tensors, int32_t n);

/* Build the per-step modulation table for `steps` Euler steps and `batch` requests
 * (pi0.5 Design: the cond component, evaluated again only when the step count or batch
 * changes). tau_host: steps + 1 HOST floats tau_0..tau_T, or NULL for tau_k = 1 - k/T
 * (t from 1 to 0). The table rows are equal across requests and are stored once per step.
 * 0 <= steps <= max_steps, 1 <= batch <= max_batch, else FM_ERR_INVALID_ARG. Requires
 * loaded weights (FM_ERR_STATE). Synchronizes the context stream before returning. */
fm_status fm_set_schedule(fm_ctx* ctx, int32_t steps, int32_t batch, const float* tau_host);

/* Bind the conditioning of one observation batch, kept for the whole loop and never
 * written by it (vla.cpp Sec. III-B observation reuse).
 * PREFIX_JOINT: k_dev[l], v_dev[l] for l < n_layers are DEVICE buffers [batch, prefix_len,
 *   1, head_dim] in the config dtype: the prefix keys (already rotated by the prefix
 *   tower) and values, copied into pool slots [0, prefix_len) of each request (pi0.5
 *   Design, "Attention and the K/V pool"); the chunk's own K/V is appended at
 *   [prefix_len, prefix_len + H) on every step. ctx_dev / state_dev must be NULL.
 *   0 <= prefix_len <= max_prefix_len.
 * DIT_CROSS: ctx_dev is a DEVICE buffer [batch, prefix_len, ctx_dim] (config dtype), the
 *   VL context, projected here to the cross-attention K/V of every even block; state_dev is
 *   a DEVICE fp32 buffer [batch, state_tokens, state_dim], embedded here to the state
 *   token(s). k_dev / v_dev must be NULL. 1 <= prefix_len <= ctx_len_max.
 * 1 <= batch <= max_batch. Requires loaded weights. Every request sees the whole binding
 * (all prefix_len prefix keys, every context token) until one of the two calls below
 * narrows it. */
fm_status fm_bind_prefix_kv(fm_ctx* ctx, int32_t batch, int32_t prefix_len, const void* const* k_dev,
                            const void* const* v_dev, const void* ctx_dev, const void* state_dev);

/* The step before the path without a copy: a prefix producer (the prefix tower's last
 * projection) writes each layer's K and V straight into the library's pool, and the binding
 * then only records the batch and length (pi0.5 Design, "Attention and the K/V pool": the
 * tower writes its output into the pool instead of having it repacked; here the pool keeps
 * the layout its kernels read, given below).
 *
 * fm_prefix_kv_slot (PREFIX_JOINT): *k_dev, *v_dev = DEVICE addresses of layer `layer`'s K
 *   and V planes; stable for the context's lifetime. With cap = fm_plan_info.pool_capacity,
 *   dh = head_dim and elements of the config dtype, prefix key j of request b goes to
 *     K: k_dev[(b * cap + j) * dh + fm_pool_k_col(d, dh, rope_base > 0)] = k[b, j, d]
 *     V: v_dev[(b * dh + d) * cap + fm_pool_v_slot(j, dtype)]            = v[b, j, d]
 *   for j < prefix_len (the rows and slots past it belong to the chunk; do not write them).
 *   Keys are taken as already rotated, as for fm_bind_prefix_kv. FM_ERR_INVALID_ARG for a
 *   layer out of range or a NULL output.
 * fm_bind_prefix_inplace (PREFIX_JOINT): binds what the pool holds for requests
 *   [0, batch) and keys [0, prefix_len), with the bounds of fm_bind_prefix_kv. It synchronizes
 *   the context stream first: writes enqueued there are complete; writes on another stream
 *   must be complete before the call. Every request sees the whole prefix (see
 *   fm_bind_prefix_lengths). The loop never writes pool rows [0, prefix_len), so a binding
 *   stays valid until the producer writes again. */
fm_status fm_prefix_kv_slot(fm_ctx* ctx, int32_t layer, void** k_dev, void** v_dev);
fm_status fm_bind_prefix_inplace(fm_ctx* ctx, int32_t batch, int32_t prefix_len);
/* Pool column of head-dim index d of a key: RoPE pairs (d, d + dh/2) side by side when the
 * config uses RoPE, else d. */
static inline int32_t fm_pool_k_col(int32_t d, int32_t head_dim, int32_t rope) {
  return !rope ? d : (d < head_dim / 2 ? 2 * d : 2 * (d - head_dim / 2) + 1);
}
/* Slot of key j in a transposed V row: bf16 permutes each 32-key tile so that a lane's
 * MFMA operand is contiguous; fp32 keeps the order. */
static inline int32_t fm_pool_v_slot(int32_t j, int32_t dtype) {
  return dtype != FM_BF16 ? j : ((j & ~31) | (((j >> 2) & 3) << 3) | (((j >> 4) & 1) << 2) | (j & 3));
}

/* Storage of the expert's per-layer matrices (listed below), applied by the next
 * fm_load_weights (vla.cpp Sec. IV-D, Table V: quantized action-head weights; pi0.5 Design
 * names FP8 for the expert).
 *   FM_WEIGHTS_AS_GIVEN  the config dtype (default).
 *   FM_WEIGHTS_FP8_E4M3  each row (output feature) becomes OCP FP8 E4M3 codes times one
 *     power-of-two scale 2^e, e the smallest exponent with max |row| <= 448 2^e; codes round
 *     to nearest, ties to even. The loop kernel and the per-operation graph's weight-streaming
 *     GEMMs (64 rows, or groups of 64 rows over a narrow output) stream the codes (half the
 *     bytes) and turn them into bf16 exactly, scaling each output column's sums by its row's
 *     2^e; the large-M GEMMs use the dequantized bf16 weights. All therefore compute the same function of the
 *     dequantized weights, which is the model. Quantized: the per-layer q / k / v, o and MLP
 *     matrices (PREFIX_JOINT), and every block's q, the self blocks' k and v, o, ff1 and ff2
 *     (DIT_CROSS; the cross blocks' context projections, applied once per binding, stay in
 *     the config dtype). FM_BF16 with mlp_dim, and for DIT_CROSS hidden, a multiple of 64
 *     (FM_ERR_UNSUPPORTED otherwise).
 * FM_ERR_INVALID_ARG for another format. */
enum { FM_WEIGHTS_AS_GIVEN = 0, FM_WEIGHTS_FP8_E4M3 = 1 };
fm_status fm_set_weight_format(fm_ctx* ctx, int32_t format);

/* Per-request key visibility of the bound batch: the additive mask M of Eq. (2) (vla.cpp
 * Sec. III-B: 0 for a visible key, -inf for a hidden one). Both calls copy what they are
 * given into library memory and synchronize the context stream before returning (the host
 * arrays may then be reused); loops already enqueued run with the previous visibility. They
 * may be called any number of times per binding. A batch that sees the whole binding runs
 * attention without the visibility test; a change between the two re-captures the loop's
 * graph on the next fm_denoise. FM_ERR_STATE before a binding; FM_ERR_UNSUPPORTED on the
 * other architecture.
 *
 * fm_bind_prefix_lengths (PREFIX_JOINT): lens_host HOST int32 [batch], request b's compact
 *   prefix length 0 <= P_b <= prefix_len (FM_ERR_INVALID_ARG otherwise), or NULL for
 *   prefix_len everywhere. Request b attends to its first P_b prefix keys and to its chunk's
 *   own keys, and its chunk takes RoPE positions P_b .. P_b + H - 1: its filled length after
 *   the append is P_b + H (pi0.5 Design, "Component contract": attention_sequence_lengths;
 *   the prefix is compact, so a shorter observation is a shorter prefix). Pool rows
 *   [P_b, prefix_len) of the request are kept but not read.
 * fm_bind_context_masks (DIT_CROSS): text_host, image_host HOST bytes [batch, prefix_len]
 *   (the bound context length), nonzero = the context token is visible, or NULL for all
 *   visible. Cross block i (even) reads the text mask when i % 4 == 0 and the image mask
 *   otherwise (GR00T N1.7, section "action": the masks are arbitrary booleans over the
 *   context). FM_ERR_INVALID_ARG when a mask that some cross block reads shows a request no
 *   token (softmax over no key has no value); nothing is changed then. */
fm_status fm_bind_prefix_lengths(fm_ctx* ctx, const int32_t* lens_host);
fm_status fm_bind_context_masks(fm_ctx* ctx, const uint8_t* text_host, const uint8_t* image_host);

/* Run the whole Euler loop: out_dev = X^T for X^0 = x0_dev. Both are DEVICE fp32 buffers
 * [batch, H, d_a] (the bound batch); out_dev may equal x0_dev. steps must equal the
 * scheduled step count (FM_ERR_SCHEDULE otherwise), and the scheduled batch must equal the
 * bound batch; steps == 0 copies x0 to out. Where the loop kernel applies (see
 * fm_set_loop_mode) the T steps run inside ONE cooperative launch of one workgroup per CU;
 * otherwise they replay as one captured hipGraph of per-operation kernels, built on the
 * first call after a schedule, bind or load changed the loop. The first loop-kernel call
 * after a schedule or bind allocates its per-step activation buffers. */
fm_status fm_denoise(fm_ctx* ctx, const float* x0_dev, int32_t steps, float* out_dev);

/* One step's velocity v(X, tau_k) without the Euler update (pi0.5 Design: the action
 * component returns the velocity), for teacher-forced checks: x_dev, v_dev DEVICE fp32
 * [batch, H, d_a]; 0 <= k < scheduled steps. Runs on the context stream with the same
 * implementation fm_denoise uses (one loop-kernel launch of one step, or the per-operation
 * kernels launched eagerly). */
fm_status fm_step_velocity(fm_ctx* ctx, const float* x_dev, int32_t k, float* v_dev);

/* The step after the path: the chunk leaves fm_denoise in normalized model space, and is
 * mapped back to robot units with per-dimension action statistics and cut to the robot's
 * share of it.
 *   FM_UNNORM_QUANTILE_EPS (pi0.5): the inverse of openpi's quantile normalization with its
 *     epsilon, y = (x + 1) / 2 * (q99 - q01 + 1e-6) + q01 (pi0.5 Design, "Embodiment
 *     adapters": quantile normalization follows openpi exactly, epsilon included, inverted
 *     on the way out; the chunk is unnormalized and sliced to the robot's width).
 *   FM_UNNORM_QUANTILE_CLIP (GR00T): y = (clip(x, -1, 1) + 1) / 2 * (q99 - q01) + q01, no
 *     guard for a degenerate group (GR00T N1.7, "Policy contract"; the policy keeps an
 *     action horizon shorter than the model's).
 * fm_set_action_stats: q01_host, q99_host HOST fp32 [robot_dim], copied; 1 <= robot_horizon
 * <= action_horizon, 1 <= robot_dim <= action_dim (FM_ERR_INVALID_ARG otherwise). The
 * statistics are kept until replaced.
 * fm_unnormalize: x_dev DEVICE fp32 [batch, action_horizon, action_dim] (e.g. the output of
 * fm_denoise), out_dev DEVICE fp32 [batch, robot_horizon, robot_dim] holding steps
 * [0, robot_horizon) and dimensions [0, robot_dim); batch is the bound batch.
 * FM_ERR_STATE before fm_set_action_stats or a binding. Enqueued on the context stream. */
enum { FM_UNNORM_QUANTILE_EPS = 0, FM_UNNORM_QUANTILE_CLIP = 1 };
fm_status fm_set_action_stats(fm_ctx* ctx, int32_t kind, int32_t robot_horizon, int32_t robot_dim,
                              const float* q01_host, const float* q99_host);
fm_status fm_unnormalize(fm_ctx* ctx, const float* x_dev, float* out_dev);

/* Like fm_step_velocity, and also copies the fp32 residual stream after the in-projection
 * and after every layer into h_trace_dev: DEVICE fp32 [n_layers + 1, rows, hidden], rows =
 * batch * (state_tokens + H). Intermediate tensors localize a discrepancy (vla.cpp
 * Sec. III-E). */
fm_status fm_step_trace(fm_ctx* ctx, const float* x_dev, int32_t k, float* v_dev, float* h_trace_dev);

/* Launch roles inside one Euler step, for fm_profile_loop. */
enum {
  FM_OP_INPROJ = 0,   /* action (and state) tokens -> residual stream */
  FM_OP_QKV = 1,      /* modulated norm + Q/K/V projection (+ RoPE, K/V append); DiT cross: Q */
  FM_OP_ATTN = 2,     /* attention over bound + own K/V */
  FM_OP_OPROJ = 3,    /* output projection + gated residual */
  FM_OP_MLP_UP = 4,   /* modulated norm + gate/up (or FF1) + GELU */
  FM_OP_MLP_DOWN = 5, /* down (or FF2) projection + residual */
  FM_OP_OUT = 6,      /* final modulated norm + velocity projection + Euler update */
  FM_OP_LOOP = 7      /* the single launch of the loop kernel (all roles of all steps) */
};

/* Implementation of fm_denoise / fm_step_velocity.
 * FM_LOOP_AUTO: the loop kernel wherever it applies, the per-operation graph elsewhere. It
 *   applies to the bf16 pi0.5-family expert (PREFIX_JOINT, one K/V head, gated MLP) with
 *   head_dim 256, 1 to 8 query heads (one per XCD), hidden 512 or 1024, mlp_dim a multiple of
 *   512 up to 4096, action_dim a multiple of 4 up to 32, batch * H <= 64 action rows, at most
 *   64 layers and at most 32 attention key-tile pairs per head (64 key tiles of 32 over the
 *   requests' compact prefixes and chunks), on a device of 256 CUs in 8 XCDs.
 * FM_LOOP_GRAPH: always the captured graph of per-operation kernels.
 * Both compute the same function (reduction orders differ). Default FM_LOOP_AUTO.
 * FM_ERR_INVALID_ARG for another mode. */
enum { FM_LOOP_AUTO = 0, FM_LOOP_GRAPH = 1 };
fm_status fm_set_loop_mode(fm_ctx* ctx, int32_t mode);

/* Synchronize the context stream. *persistent = 1 when the loop kernel serves the current
 * weights, schedule and binding (0 otherwise). *fault: 0, or what went wrong since the last
 * query: 1, 2 or 3 when one of the loop kernel's bounded waits expired (1 an XCD barrier, 2 the
 * wait for a norm operand from every XCD, 3 the wait for the O or down partial sums); 4 when two
 * of its workgroups took one (XCD, rank) slot, i.e. the launch was not dealt round-robin over
 * the XCDs. Results since then are invalid: the context is poisoned and FM_ERR_DEVICE is
 * returned (the word is cleared). A loop-kernel launch that starts with its fault word set
 * writes NaN to its output and does nothing else. Either pointer may be NULL. */
fm_status fm_loop_status(fm_ctx* ctx, int32_t* persistent, uint32_t* fault);

/* Run the same loop as fm_denoise, eagerly, with a hipEvent pair on the context stream
 * around every launch of `role`; returns the summed duration in *ms (milliseconds) and
 * the number of those launches in *launches. Synchronizes the context stream. Arguments
 * and results as fm_denoise (steps must be the scheduled count, >= 1). For measurement.
 * FM_OP_LOOP times the loop kernel's one launch (FM_ERR_UNSUPPORTED when it does not
 * serve the current loop); the per-role values time the per-operation kernels. */
fm_status fm_profile_loop(fm_ctx* ctx, const float* x0_dev, int32_t steps, float* out_dev, int32_t role, float* ms,
                          int32_t* launches);

/* Kernel-level entry points on caller buffers, used to check single kernels.
 * fm_op_linear: out[M, N] = act(A[M, K] W[N, K]^T + bias) with the library GEMM (split-K
 *   and tile choice as the loop would plan them). A, W DEVICE in `dtype`, row-major; bias
 *   DEVICE fp32 [N] or NULL; act 0 none, 1 SiLU, 2 GELU (tanh); out DEVICE, fp32 when
 *   out_f32 else `dtype`. K must be a multiple of 32 (bf16) or 16 (fp32). Allocates and
 *   frees its scratch; synchronizes `hip_stream`.
 * fm_op_attention: o = softmax(q k^T / sqrt(dh)) v per head (vla.cpp Eq. (2), no mask).
 *   q, o DEVICE [B, Tq, n_heads, dh]; k, v DEVICE [B, n_kv, n_keys, dh] with n_kv = 1 or
 *   n_heads; all in `dtype`. Allocates and frees its scratch; synchronizes `hip_stream`. */
fm_status fm_op_linear(int32_t dtype, int32_t M, int32_t N, int32_t K, const void* A, const void* W,
                       const float* bias, int32_t act, void* out, int32_t out_f32, void* hip_stream);
fm_status fm_op_attention(int32_t dtype, int32_t B, int32_t Tq, int32_t n_heads, int32_t n_kv, int32_t n_keys,
                          int32_t dh, const void* q, const void* k, const void* v, void* o, void* hip_stream);
/* fm_op_attention_noalloc: fm_op_attention for callers that cannot allocate device memory
 *   (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 *   Same arguments, kernels and results as fm_op_attention; it calls no hipMalloc / hipFree and
 *   does not synchronize: the work is enqueued on hip_stream. Its scratch (the transposed V
 *   plane, B * n_kv * dh * round_up(n_keys, 64) elements, then the split partials) lives in a
 *   fixed 16 MiB device array per GPU, held until the process ends; a call needing more
 *   returns FM_ERR_INVALID_ARG with the byte counts in fm_last_error(NULL). Every call on one GPU
 *   shares that array: calls that overlap on one GPU (two streams, two threads) race. */
fm_status fm_op_attention_noalloc(int32_t dtype, int32_t B, int32_t Tq, int32_t n_heads, int32_t n_kv,
                                  int32_t n_keys, int32_t dh, const void* q, const void* k, const void* v, void* o,
                                  void* hip_stream);
/* fm_op_quantize_fp8: the FP8 weight quantizer alone (see fm_set_weight_format), for parity.
 *   src DEVICE bf16 [N, K] row-major (K even); codes DEVICE bytes [N, K]; scale DEVICE fp32 [N]
 *   (2^e of each row); deq DEVICE bf16 [N, K] = code value x 2^e (exact). Synchronizes
 *   hip_stream. FM_ERR_INVALID_ARG for a NULL buffer or an odd K. */
fm_status fm_op_quantize_fp8(int32_t N, int32_t K, const void* src, void* codes, float* scale, void* deq,
                             void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* FM_H_ */
