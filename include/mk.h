/*
 * mk.h -- C ABI of the MI355X (gfx950) persistent decode megakernel.
 *
 * One call runs one small-batch decode step, or one speculative-verify block, of a whole hybrid
 * decoder stack as a single kernel launch. The problem statement follows the pages:
 *   - "Kimi K3's TPU megakernel: 92 layers in one Pallas call, and what 709 tokens a second
 *     measures", section "How it maps onto a TPU v7": the whole layer loop runs inside one kernel;
 *     the decode positions and the linear-attention state are the step's scalar inputs; every weight
 *     enters as a raw reference into device memory, loaded by the kernel itself.
 *   - same page, section "What DSpark changes per step": a verify step evaluates an anchor plus seven
 *     drafts as eight rows of one sequence and emits the accepted prefix plus one bonus token.
 *   - page "TPU megakernels for Kimi K3, Qwen3.8-27B, and Muse-Spark-Open": the stacks are a
 *     gated-delta-net + grouped-query-attention hybrid (dense bf16), a Kimi delta attention + latent
 *     attention mixture of experts, and an NVFP4 mixture of experts.
 *
 * Conventions (all entry points):
 *   - Every call returns an mk_status; nothing throws across the ABI. mk_last_error() returns a
 *     thread-local message for the last failing call on this thread.
 *   - Arguments and shapes are checked before anything is enqueued: a rejected call has no side
 *     effects.
 *   - All device memory is owned by the caller (for example torch tensors). The context keeps the raw
 *     device pointers given to mk_bind_buffers until mk_destroy.
 *   - Step calls are asynchronous on the caller's stream. Device faults surface at the caller's
 *     synchronisation; a bounded in-kernel wait that expires is reported by mk_read_device_status
 *     (after which caches and recurrent states are undefined and the next step call resets the
 *     context's inter-workgroup counters).
 *   - One context is not thread-safe; distinct contexts may be used from distinct threads/streams.
 *     Two steps of one context must not overlap in time (they share the bound scratch buffer).
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MK_MAX_LAYERS 128
/* Rows of a decode step. Each activation enters the matrix products as a bf16 high and a bf16 low half
 * (16 significant bits): one matrix-core product per weight fragment covers 8 rows, two cover 9 to 16.
 * Mixture-of-experts configurations run at most 8 rows. */
#define MK_MAX_BATCH 16
#define MK_VERIFY_ROWS 8

typedef enum {
  MK_OK = 0,
  MK_E_ARG = 1,          /* null pointer, bad enum, inconsistent dimension */
  MK_E_SHAPE = 2,        /* a tensor's shape does not match the configuration */
  MK_E_UNSUPPORTED = 3,  /* valid request this build does not implement (or a host-only context) */
  MK_E_CAPACITY = 4,     /* batch > max_batch, position + rows > max_ctx, on-chip budget exceeded */
  MK_E_HIP = 5,          /* a HIP runtime call failed (message in mk_last_error) */
  MK_E_DEVICE_TIMEOUT = 6, /* an in-kernel wait expired (from mk_read_device_status) */
  MK_E_STATE = 7,        /* call out of order (e.g. a step before all buffers/weights are in place) */
  MK_E_INEXACT = 8       /* a weight re-encoding the configuration asks for is not lossless (nothing kept) */
} mk_status;

typedef enum { MK_MIXER_GQA = 0, MK_MIXER_GDN = 1, MK_MIXER_KDA = 2, MK_MIXER_MLA = 3 } mk_mixer;
typedef enum { MK_FFN_DENSE = 0, MK_FFN_MOE = 1 } mk_ffn_kind;
/* Weight element formats. MK_DT_MXFP4 (expert matrices only): FP4 E2M1 codes [rows][cols/2] (element 2i
 * in the low nibble of byte i) with an E8M0 scale per 32 consecutive elements of a row [rows][cols/32]
 * (OCP Microscaling). A configuration whose experts are MXFP4 keeps down in MXFP4 and re-encodes gate and
 * up at load time into FP8 E4M3 with one bf16 scale per 256 elements of a row, checking that the new
 * encoding decodes to the same values bit for bit (page "Kimi K3's TPU megakernel: 92 layers in one Pallas
 * call, and what 709 tokens a second measures", section "How it maps onto a TPU v7"). */
typedef enum { MK_DT_BF16 = 0, MK_DT_NVFP4 = 1, MK_DT_MXFP4 = 2 } mk_dtype;

/* Model configuration. A layer is RMSNorm -> mixer -> residual add -> RMSNorm -> FFN -> residual add.
 * vocab > 0: the step embeds tokens and ends with a final RMSNorm and LM head (logits out).
 * vocab == 0: a slice of a stack: hidden states in, hidden states out. */
typedef struct mk_config {
  int32_t n_layers, hidden, vocab;
  int32_t mixer[MK_MAX_LAYERS];    /* mk_mixer per layer */
  int32_t ffn_kind[MK_MAX_LAYERS]; /* mk_ffn_kind per layer */
  int32_t ffn;                     /* dense SwiGLU width */
  int32_t n_q_heads, n_kv_heads, head_dim;           /* GQA */
  int32_t lin_heads, d_k, d_v;                        /* GDN / KDA (d_k == d_v == 128 supported) */
  int32_t mla_heads, kv_rank, rope_dim, nope_dim, v_dim; /* latent attention */
  int32_t n_experts, top_k, expert_ffn, n_shared, expert_format; /* MoE (mk_dtype for experts) */
  int32_t max_ctx;   /* cache capacity in positions (cached tokens + new rows) */
  int32_t max_batch; /* 1..MK_MAX_BATCH */
  float eps;         /* RMSNorm epsilon */
  float rope_theta;
} mk_config;

typedef struct mk_ctx mk_ctx; /* opaque; host memory only */

/* Byte sizes of the buffers the caller must allocate (device memory, 256-byte aligned). */
typedef struct mk_sizes {
  uint64_t packed_weights; /* all weights in the kernel's tile-major layout */
  uint64_t scratch;        /* activations, partial sums, inter-workgroup counters, verify snapshots */
  uint64_t kv_cache_per_layer;  /* per GQA layer, one of K or V: bf16 [max_batch][n_kv][max_ctx][head_dim] */
  uint64_t lin_state_per_layer; /* per GDN/KDA layer: fp32 [max_batch][lin_heads][d_v][d_k] */
  uint64_t latent_per_layer;    /* per MLA layer: bf16 [max_batch][max_ctx][kv_rank + rope_dim] */
  int32_t n_phases;        /* phases (grid-wide dependency steps) in one decode step */
  int32_t n_workgroups;    /* persistent workgroups the step launches (one per compute unit) */
} mk_sizes;

/* Caller-owned device buffers. Per-layer arrays are indexed by layer; entries of layers without
 * that state are ignored. Layouts are those documented in mk_sizes. */
typedef struct mk_buffers {
  void *packed_weights;
  void *scratch;
  void *k_cache[MK_MAX_LAYERS];
  void *v_cache[MK_MAX_LAYERS];
  void *lin_state[MK_MAX_LAYERS];
  void *latent[MK_MAX_LAYERS];
} mk_buffers;

typedef enum {
  MK_W_EMBED = 0, MK_W_FINAL_NORM, MK_W_LM_HEAD, MK_W_ATTN_NORM, MK_W_FFN_NORM,
  MK_W_Q, MK_W_K, MK_W_V, MK_W_A, MK_W_B, MK_W_O,       /* attention / delta-rule projections */
  MK_W_DKV, MK_W_KR, MK_W_UK, MK_W_UV,                   /* latent attention */
  MK_W_GATE, MK_W_UP, MK_W_DOWN, MK_W_ROUTER             /* FFN / MoE */
} mk_weight_kind;

/* One weight tensor in its natural layout: bf16 [rows][cols] row-major (output rows, reduction
 * columns), or NVFP4: codes uint8 [rows][cols/2] (element 2i in the low nibble), E4M3 scales uint8
 * [rows][cols/16], one fp32 tensor scale. expert: -1 for dense tensors, e >= 0 routed expert e,
 * -2 - s for shared expert s. data/scales are device pointers; they are read by kernels enqueued on
 * the stream passed to mk_load_weights and may be freed once that stream has synchronised. */
typedef struct mk_weight_desc {
  int32_t layer; /* -1 for embed / final_norm / lm_head */
  int32_t kind;  /* mk_weight_kind */
  int32_t expert;
  int32_t dtype; /* mk_dtype */
  int64_t rows, cols;
  const void *data;
  const void *scales;
  float tensor_scale;
} mk_weight_desc;

/* Inputs and outputs of one step: device pointers except positions. Unused fields may be NULL. */
typedef struct mk_step_io {
  const int32_t *tokens;    /* vocab configs: int32 [B] (verify: [8] = anchor + 7 drafts) */
  const float *hidden_in;   /* slice configs: fp32 [B][hidden] */
  const int32_t *positions; /* HOST int32 [B]: position of each sequence's new token (verify: of the
                               anchor). Passed to the kernel as scalars; checked against max_ctx. */
  float *logits;            /* vocab configs: fp32 [B][vocab] (verify: [8][vocab]) */
  float *hidden_out;        /* slice configs: fp32 [B][hidden] */
  int32_t *argmax;          /* optional int32 [B] (verify: [8]): first index of the row maximum */
  int32_t *route_idx;       /* optional int32 [n_moe_layers][B][top_k] */
  float *route_w;           /* optional fp32 [n_moe_layers][B][top_k] */
} mk_step_io;

/* Validates cfg and builds the step schedule. hip_device >= 0 selects a GPU; hip_device == -1 makes a
 * host-only context (schedule and sizes only; step and load calls return MK_E_UNSUPPORTED), used to
 * test the host logic without a GPU. */
mk_status mk_create(const mk_config *cfg, int hip_device, mk_ctx **out);

/* Sizes of the caller-allocated buffers for this configuration. */
mk_status mk_query_sizes(const mk_ctx *ctx, mk_sizes *out);

/* Records the caller's device buffers (sizes as mk_query_sizes reports) and initialises the scratch
 * buffer's tables and counters (enqueued on the null stream and waited for). */
mk_status mk_bind_buffers(mk_ctx *ctx, const mk_buffers *bufs);

/* Copies n weight tensors into the packed buffer, converting each to the kernel's tile-major layout
 * (asynchronous on stream). Every tensor the configuration needs must be loaded once before the first
 * step; loading a tensor again replaces it. MXFP4 gate and up matrices are re-encoded to FP8 E4M3 with a
 * power-of-two bf16 scale per 256 elements of a row; when any of them has an element without an exact
 * E4M3 value at its block's scale, the call waits for the stream and returns MK_E_INEXACT, and those
 * matrices count as not loaded (a step refuses to run until they are loaded again). */
mk_status mk_load_weights(mk_ctx *ctx, const mk_weight_desc *w, int n, void *hip_stream);

/* One decode step for `batch` sequences (1 <= batch <= max_batch) as one persistent kernel launch on
 * hip_stream. Appends the new tokens' K/V (or latents) at positions[b], advances linear-attention
 * states, writes logits (and argmax) or hidden_out, and the MoE routing if requested. */
mk_status mk_decode_step(mk_ctx *ctx, const mk_step_io *io, int batch, void *hip_stream);

/* Most decode steps one mk_decode_loop launch runs. */
#define MK_MAX_LOOP_STEPS 32

/* n_steps greedy decode steps of `batch` sequences in one persistent kernel launch (the pages' on-device
 * loop, page "Kimi K3's TPU megakernel: 92 layers in one Pallas call, and what 709 tokens a second
 * measures", section "What DSpark changes per step": many steps inside one device call, so the host takes
 * part once per call). Step 0 embeds io->tokens at io->positions[b]; step s > 0 embeds, at positions[b] + s,
 * the token step s - 1 emitted: the argmax of its logits (first maximum), chosen and re-embedded inside the
 * kernel with no host round trip. Each step appends its K/V (or latent) rows and advances the linear
 * states exactly as mk_decode_step would. d_tokens_out: device int32 [n_steps][batch], the token each step
 * emitted. io->logits and io->argmax receive the last step's. Needs a vocabulary configuration;
 * 1 <= n_steps <= MK_MAX_LOOP_STEPS and positions[b] + n_steps <= max_ctx (else MK_E_CAPACITY). Calls on
 * one context are ordered on one stream (the expanded phase table lives in the bound workspace). */
mk_status mk_decode_loop(mk_ctx *ctx, const mk_step_io *io, int batch, int n_steps, int32_t *d_tokens_out,
                         void *hip_stream);

/* Size of the library-held device array of mk_decode_step_noalloc, one per GPU (64 MiB). */
#define MK_NOALLOC_SCRATCH_BYTES (64ll << 20)

/* The decode step of mk_decode_step for callers that cannot allocate device memory or hand over a
 * workspace at step time: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. Same arguments, kernel and results as mk_decode_step (bit-identical outputs and state
 * updates). The step's per-call working set (grid-barrier and finalise counters, residual stream,
 * k-split partial sums, attention partials, argmax candidates) lives in a device array inside the
 * library, MK_NOALLOC_SCRATCH_BYTES per GPU, reserved when the library's code is loaded on that GPU
 * and held until the process ends; the call allocates nothing. The context's constant tables (phase
 * table, RoPE tables, cache pointers) and its device status word stay in its bound workspace.
 * Each call clears that GPU's array with a fill kernel on hip_stream, then runs the step there; the
 * array keeps the last call's contents, so calls that overlap on one GPU (any context, any stream)
 * race and must be ordered by the caller. Errors: MK_E_CAPACITY when the working set at this batch
 * exceeds the array, MK_E_STATE when the array's address was not taken at mk_create (device index
 * 64 or above); otherwise those of mk_decode_step. */
mk_status mk_decode_step_noalloc(mk_ctx *ctx, const mk_step_io *io, int batch, void *hip_stream);

/* Speculative verify of one sequence (batch 1): rows j = 0..7 are io->tokens[j] at positions[0] + j.
 * Row j attends to positions 0..positions[0]+j and advances linear states one row at a time. Writes
 * logits [8][vocab] and argmax [8], the accepted draft count a in [0, 7] (longest prefix with
 * tokens[j+1] == argmax[j]) to *d_accepted and the bonus token argmax[a] to *d_bonus (device int32),
 * and commits every linear-attention state to its value after row a. K/V of all 8 rows are written. */
mk_status mk_verify_step(mk_ctx *ctx, const mk_step_io *io, int32_t *d_accepted, int32_t *d_bonus,
                         void *hip_stream);

/* The same decode step as mk_decode_step, run as one kernel launch per phase (no persistent kernel,
 * no cross-phase prefetch): the non-fused baseline whose op boundaries the megakernel removes.
 * use_graph != 0 runs the same launches as one HIP graph: captured (on a stream of the context's own)
 * the first time a row count is called with a given argument block, replayed on hip_stream by later
 * calls with the same block (positions, tokens and output buffers); a call with another block captures
 * again. The graph holds kernel launches only. */
mk_status mk_decode_step_perop(mk_ctx *ctx, const mk_step_io *io, int batch, int use_graph, void *hip_stream);

/* After the caller has synchronised the step's stream: *status is MK_OK or MK_E_DEVICE_TIMEOUT and
 * *phase the phase index whose wait expired (-1 if none). */
mk_status mk_read_device_status(mk_ctx *ctx, int32_t *status, int32_t *phase);

void mk_destroy(mk_ctx *ctx);

/* Launch mode of the persistent step kernel. cooperative != 0 (default): hipLaunchCooperativeKernel,
 * whose runtime check guarantees that all workgroups are co-resident. cooperative == 0: an ordinary
 * launch of the same grid (one workgroup per compute unit; each workgroup's LDS use admits only one per
 * CU), for tools that do not follow cooperative launches; if a workgroup could not become resident,
 * the bounded in-kernel waits expire and the step reports MK_E_DEVICE_TIMEOUT instead of hanging. */
mk_status mk_set_launch_mode(mk_ctx *ctx, int cooperative);

/* Tracing: when device_buffer is not NULL, every later step records, per phase and workgroup, two
 * 64-bit timestamps of the GPU's constant 100 MHz clock (phase start, end of the phase's work before
 * the grid barrier) at [phase][workgroup][2]. bytes must cover the longest schedule
 * (n_phases * n_workgroups * 16). NULL turns tracing off. Adds one workgroup barrier per phase. */
mk_status mk_set_trace(mk_ctx *ctx, void *device_buffer, int64_t bytes);

/* Host-logic introspection (works on host-only contexts): number of phases in the schedule for a row
 * count, and 16 integers describing phase i: type, layer, N, K, tiles, fragments, k-splits, fragments
 * per split, activation kind, output kind, source splits, source row stride, split-KV chunks, chunk
 * length, partial buffer, counter offset. Returns -1 on bad arguments. */
int mk_debug_phase_count(const mk_ctx *ctx, int rows);
int mk_debug_phase(const mk_ctx *ctx, int rows, int i, int32_t *out16);
/* The whole descriptor of phase i (the library's internal layout, for host-side checks of the schedule):
 * copies it to out when bytes is large enough; returns its size in bytes, or -1 on bad arguments. */
int mk_debug_phase_bytes(const mk_ctx *ctx, int rows, int i, void *out, int bytes);
/* Bytes of the packed weight buffer (as mk_query_sizes reports), or -1 for a NULL context. */
int64_t mk_debug_packed_bytes(const mk_ctx *ctx);

const char *mk_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
