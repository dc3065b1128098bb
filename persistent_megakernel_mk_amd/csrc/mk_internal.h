// Shared host/device definitions of the megakernel: the phase table the host builds and the kernel
// interprets, and the argument block of one step launch. Internal to libmk.so.
#pragma once
#include <stdint.h>

namespace mk {

constexpr int kCWaves = 4;                // weight-streaming (compute) waves per workgroup
constexpr int kSyncWave = kCWaves;        // index of the sync wave (reductions, stores, grid barrier)
constexpr int kWavesTotal = kCWaves + 1;
constexpr int kThreads = kWavesTotal * 64;  // threads per workgroup
constexpr int kCThreads = kCWaves * 64;     // threads of the compute waves
constexpr int kRing = 12;                 // weight items in flight per compute wave (12 KiB), bf16 build
constexpr int kRingNvfp4 = 8;            // the same for the build that also streams NVFP4 items
constexpr int kRingWide = 10;             // the same for the build for more than 8 rows
constexpr int kTileRows = 16;             // weight rows per MFMA tile
constexpr int kFragK = 32;                // reduction columns per 1 KiB weight fragment
constexpr int kLdsBytes = 160 * 1024 - 512;  // dynamic LDS per workgroup (gfx950: 160 KiB per CU, minus static)
constexpr int kActLdsBudget = 112 * 1024;     // LDS for the activation fragments of one k-split
constexpr int kActLdsBudgetNarrow = 96 * 1024; // what the k-split choice uses up to kMaxRows rows
constexpr int kMaxRows = 8;               // rows of a verify block; rows whose activations enter products
                                          // as bf16 high and low halves (2 MFMA columns each)
constexpr int kMaxBatch = 16;             // rows of a decode step; above kMaxRows each activation enters
                                          // products as one bf16 column (the 16 columns hold 16 rows)
constexpr int kMaxUnits = 512;            // product units (tile x k-split) per workgroup and phase
constexpr int kMaxTopK = 16;              // routed experts per token
constexpr int kMaxExperts = 1024;         // routed experts per MoE layer
constexpr int kMaxShared = 4;             // shared experts per MoE layer
constexpr int kMaxSeg = kMaxShared + kMaxRows * kMaxTopK;  // expert segments of one MoE product phase
constexpr int kMaxPieces = 4;             // activation pieces (segment x k-split) staged per workgroup
// grid barrier: workgroups arrive at kBarGroups group counters (workgroup i at i mod kBarGroups), the
// last arrival of a group at one top counter that every workgroup polls; counters 128 B apart. Four
// groups of 64 measured faster than 2, 8 or 16 (16 slowest).
constexpr int kBarGroups = 4;
constexpr int kBarBytes = (kBarGroups + 1) * 128;

enum PhaseType : int32_t {
  PH_EMBED = 1,      // residual x <- embedding rows (or hidden_in); per-tile sums of squares
  PH_GEMV = 2,       // weight-streaming matrix-vector product (MFMA, bf16 weights, fp32 accumulation)
  PH_DELTA = 3,      // gated delta rule state update + readout (scalar or per-channel gate)
  PH_ATTN = 4,       // split-KV grouped-query attention partials (+ RoPE and K/V append)
  PH_MERGE = 5,      // log-sum-exp merge of the split-KV partials
  PH_FINAL = 6,      // argmax over LM-head candidates; verify accept + state commit
  PH_HIDDEN_OUT = 7, // slice configs: x -> hidden_out
  PH_MLA = 8,        // split-KV absorbed latent attention partials (+ RoPE and latent append), MFMA
  PH_MLA_MERGE = 9   // log-sum-exp merge of the latent attention partials
};

// Segmented products: the phase's tiles belong to segments with their own activation (and, for
// experts, their own weight block chosen at run time by the router).
enum SegKind : int32_t {
  SEG_NONE = 0,     // one matrix, one activation per k-split
  SEG_HEADS = 1,    // consecutive blocks of seg_T tiles, each with its own activation slice (per head)
  SEG_EXPERT = 2    // expert weight blocks (shared experts, then the batch's routed union), chosen per step
};

enum ActKind : int32_t {
  ACT_NORM = 0,   // y = x * rstd * gain    (rstd from per-tile sums of squares)
  ACT_PART = 1,   // y = sum over S_src partials of the previous product
  ACT_SWIGLU = 2, // y = silu(sum gate partials) * (sum up partials); up rows follow gate rows
  ACT_MIX = 3     // y = mixer output vector
};

enum WeightFmt : int32_t {
  FMT_BF16 = 0,   // [tile][fragment][lane][8] bf16
  FMT_NVFP4 = 1,  // codes [tile][4-fragment group][lane][16 B], then E4M3 scales [tile][group][32][4 B]
  FMT_FP8R = 2,   // FP8 E4M3 [tile][2-fragment item][lane][16 B], then bf16 scales [tile][256 columns][16]
  FMT_MXFP4 = 3   // codes as NVFP4, then E8M0 scales [tile][group][16][4 B]
};
// MFMA fragments (16 rows x 32 columns) per 1 KiB stream item of a format
constexpr int frags_per_item(int fmt) { return fmt == FMT_BF16 ? 1 : (fmt == FMT_FP8R ? 2 : 4); }

enum OutKind : int32_t {
  OUT_PART = 0,   // partial sums per k-split -> part[dst]
  OUT_RESID = 1,  // partial sums, then the last contributor of each tile adds them into x
  OUT_LOGITS = 2  // final values (one k-split) -> logits, plus per-workgroup argmax candidates
};

struct Phase {
  int32_t type;
  int32_t layer;
  // ---- GEMV ----
  int64_t w_off;     // byte offset of the packed matrix in the weight buffer
  int64_t gain_off;  // byte offset of the bf16 RMSNorm gain (ACT_NORM)
  int32_t N, K;      // rows, columns
  int32_t T, KF;     // 16-row tiles, 32-column fragments
  int32_t S, nf;     // k-splits, fragments per split (nf = KF / S, a multiple of kCWaves)
  int32_t act, out;
  int32_t src_part, src_S, src_N, src_off;  // activation partials: buffer, splits, row stride, row offset
  int32_t dst_part;  // partial buffer written
  int32_t cnt_off;   // finalizer counters (OUT_RESID)
  // ---- mixers ----
  int32_t lin_idx;   // index among linear-attention layers (state snapshots)
  int32_t per_channel_gate;  // 1: Kimi delta attention (gate per key channel)
  int32_t n_chunks, chunk;   // split-KV geometry
  int32_t q_off, k_off, v_off, a_off, b_off;  // row offsets inside the fused projection output
  int32_t next_gemv;  // index of the next product phase (-1: none); the weight stream follows it
  // ---- segmented products ----
  int32_t seg;        // SegKind
  int32_t nseg;       // static segments (heads; shared experts)
  int32_t seg_T;      // tiles per segment
  int32_t src_seg;    // activation source offset between consecutive segments (floats)
  int64_t seg_stride; // bytes between consecutive expert blocks (SEG_EXPERT)
  int32_t fmt;        // WeightFmt of the streamed matrix
  int32_t pieces;     // activation pieces per workgroup the schedule guarantees (<= kMaxPieces)
  // ---- mixture of experts ----
  int32_t moe_idx;    // index among MoE layers (routing outputs)
  int32_t route_q;    // SEG_EXPERT: phase index of the layer's expert gate/up product (owner of the routing)
  int32_t n_exp, top_k, n_shared;
  int32_t z_part, z_S, z_N;  // router logits: partial buffer, k-splits, row stride
  int64_t ts_off;     // NVFP4: byte offset of the per-expert tensor scales [E + shared][3] (gate, up, down)
  // ---- latent attention ----
  int32_t rank, rope, nope, qk_stride;  // latent width, rotary width, no-rope query width, q row stride
  int32_t dkv_off, kr_off;              // offsets of the new latent and rotary key in the projection
  int32_t heads, hgroup;                // query heads, heads per unit
  int32_t mla_src;                      // partial buffer of the absorbed queries
  int32_t step;       // decode step of a multi-step launch this phase belongs to (0 in a one-step table)
  int32_t chunk_verify;  // delta rule: state rows per unit in a verify block (chunk: in a decode step)
  // ---- staged activations ----
  // A product's activation fragments (the B operand: bf16 high and low halves of each row's value, in
  // the LDS layout) can be written to a global buffer by the phase that produces its input, so that
  // staging them is one copy of the product's K slice into LDS instead of a gather, sum and conversion
  // in every workgroup.
  int32_t stg_in;        // StgBuf the product copies its activation from (STG_NONE: formed as before)
  int64_t stg_gain_off;  // x writers: byte offset of the bf16 gain of the RMSNorm that reads x next
  int32_t stg_out;       // producer of a staged buffer: x writers (embed, residual products) write x times
                         // that gain, delta / merge phases their output, a dense gate|up product its SwiGLU
  int32_t swi_cnt_off;   // dense gate|up product with stg_out: finaliser counters of its 16-row pairs
};
enum StgBuf : int32_t { STG_NONE = 0, STG_X = 1, STG_MIX = 2, STG_H = 3 };

struct StepArgs {
  const Phase *phases;
  int32_t n_phases;
  int32_t n_barriers;  // grid barriers per step
  uint32_t bar_done;   // grid barriers completed on these counters before this launch (they are monotone)
  int32_t R;           // rows in this step: batch, or 8 for verify
  int32_t verify;
  int32_t phase_begin, phase_end;  // phases run by this launch (all, or one for the per-op baseline)
  int32_t barrier_base;            // barriers completed before phase_begin within this step
  const uint8_t *wbuf;
  // scratch regions
  uint32_t *bar;       // kBarGroups group counters and the top counter, 128 B apart
  uint32_t *fin;       // finalizer counters
  int32_t *status;     // [0] status, [1] phase, [2] abort flag
  float *x;            // residual [R][H]
  float *ss;           // [R][H/16] per-tile sums of squares of x
  float *part[3];      // partial sums [S][R][N]
  float *mix;          // mixer outputs [R][M]
  float *attn;         // split-KV partials [R][nq][n_chunks][hd + 2] (latent: [R][heads][n_chunks][rank + 2])
  const float *rope_mla;  // [max_ctx][rope/2][2] cos, sin for the latent attention's rotary part
  void *const *lat;    // per layer latent caches
  float *cand;         // argmax candidates [G][R][2]
  const float *rope;   // [max_ctx][hd/2][2] cos, sin
  float *snap;         // verify snapshots [lin layers][8][heads][d_v][d_k]
  uint16_t *stg[3];    // staged activations (x times the next gain, mixer output, SwiGLU output), each
                       // [K / 8][C][8] bf16 with C = 2R columns up to 8 rows (high halves, then low),
                       // 32 above (two groups of 8 rows, 16 columns each)
  void *const *kc;     // per layer K cache pointers
  void *const *vc;
  void *const *ls;     // per layer linear states
  void *const *lsl;    // per linear-attention index: state pointers (verify commit)
  // io
  const int32_t *tokens;
  const float *hidden_in;
  int32_t pos[kMaxBatch];  // position of each sequence's new token (verify: of the anchor)
  float *logits;
  float *hidden_out;
  int32_t *argmax;
  int32_t *route_idx;  // optional [n_moe][R][top_k]
  float *route_w;
  int32_t *accepted;
  int32_t *bonus;
  int32_t *loop_tokens;  // multi-step launch: [steps][R] token emitted by each step (its argmax), which the
                         // next step embeds; null for one step
  // config scalars
  int32_t H, V, max_ctx, mix_stride;
  int32_t nq, nkv, hd;
  int32_t lin_heads, dk, dv, n_lin;
  int32_t part_stride;  // floats per partial buffer
  float eps;
  int64_t timeout_ticks;  // bound of every in-kernel wait, in s_memrealtime ticks (100 MHz)
  uint64_t *trace;        // optional [n_phases][G][2] s_memrealtime at phase start / end of work
};

}  // namespace mk
