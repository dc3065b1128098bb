// Host runtime of the persistent decode megakernel: configuration checks, the step schedule (the
// phase table the kernel interprets), buffer layout, weight repacking and the step launches. Everything
// here is plain C++ over the HIP runtime; the C ABI is declared in include/mk.h.
//
// The schedule is the device-side layer/op list of the pages' design ("Kimi K3's TPU megakernel: 92
// layers in one Pallas call, and what 709 tokens a second measures", section "How it maps onto a TPU
// v7": a layer loop whose body branches on the layer kind; per layer norm, mixer, residual, norm, FFN,
// residual). It is built once per row count (1..8) at mk_create and copied to device memory at bind.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "mk.h"
#include "mk_internal.h"

using namespace mk;

extern "C" __global__ void mk_step_kernel(StepArgs a);
extern "C" __global__ void mk_step_kernel_nvfp4(StepArgs a);
extern "C" __global__ void mk_step_kernel_wide(StepArgs a);
extern "C" __global__ void mk_repack_bf16(const uint16_t *src, int64_t rows, int64_t cols, uint4 *dst, int64_t row_off,
                                          int64_t KF);
extern "C" __global__ void mk_repack_nvfp4(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols, uint8_t *dst,
                                           int64_t row_off, int64_t dst_rows);
extern "C" __global__ void mk_store_f32(float *dst, float v);
extern "C" __global__ void mk_repack_mxfp4(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols, uint8_t *dst,
                                           int64_t row_off, int64_t dst_rows);
extern "C" __global__ void mk_reencode_fp8(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols, uint8_t *dst,
                                           int64_t row_off, int64_t dst_rows, uint32_t *inexact);

// ---------------------------------------------------------------------------------------------
// Library-held working memory of mk_decode_step_noalloc: one array per GPU, part of this code object
// (no allocation call is ever made for it; the runtime reserves it when the code object is loaded on
// a device and holds it until the process ends). It holds one step's per-call working set: barrier
// and finalise counters, the residual stream, k-split partial sums, attention partials and argmax
// candidates. On the host the name `scratch` only stands in for the array: it is never passed to a
// kernel or a copy. Its device address is taken once per device, in mk_create with that device
// current, and kept in g_noalloc_ptr.
// ---------------------------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[MK_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int64_t kNoAllocBytes = MK_NOALLOC_SCRATCH_BYTES;
constexpr int kNoAllocDevices = 64;
uint8_t *g_noalloc_ptr[kNoAllocDevices] = {};
std::mutex g_noalloc_mu;
}  // namespace

// Zero n 16-byte words (a fill kernel rather than hipMemsetAsync, so a caller may capture the call).
extern "C" __global__ void mk_zero16(uint4 *p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}
extern "C" __global__ void mk_repack_bf16_headT(const uint16_t *src, int64_t heads, int64_t nope, int64_t rank, uint4 *dst);

namespace {

thread_local std::string g_err;

mk_status fail(mk_status st, const char *fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define HIP_TRY(expr)                                                                           \
  do {                                                                                          \
    hipError_t e_ = (expr);                                                                     \
    if (e_ != hipSuccess) return fail(MK_E_HIP, "%s failed: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

inline int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }
inline int64_t round16(int64_t v) { return align_up(v, 16); }

// One matrix (or vector) inside the packed weight buffer.
struct Slot {
  int64_t off = -1;  // bytes
  int32_t N = 0, K = 0;
  bool packed = false;  // tile-major MFMA fragments (else natural row-major bf16)
  int64_t bytes() const { return (int64_t)N * K * 2; }
};

struct LayerSlots {
  Slot attn_norm, ffn_norm, mix_in, wo, gu, wd;
  // row offsets inside mix_in
  int32_t q_off = 0, k_off = 0, v_off = 0, a_off = 0, b_off = 0;
  // required tensors (kind bitmask) and loaded tensors
  uint32_t need = 0, have = 0;
  // latent attention: absorbed key up-projection (per-head transposed) and value up-projection
  Slot wuk_t, wuv;
  int32_t dkv_off = 0, kr_off = 0;
  // mixture of experts: router, then (routed experts + shared experts) gate|up blocks and down blocks
  Slot router;
  int64_t ex_gu_off = -1, ex_down_off = -1, ex_gu_bytes = 0, ex_down_bytes = 0, ts_off = -1;
  std::vector<uint8_t> ex_have;  // [(E + shared) * 3]: gate, up, down loaded
};

// Bytes of one packed matrix: bf16, or NVFP4 codes (half a byte per weight) plus one E4M3 scale per
// 16 weights.
int64_t matrix_bytes(int64_t rows, int64_t cols, int fmt) {
  switch (fmt) {
    case FMT_NVFP4: return rows * cols / 2 + rows * cols / 16;  // codes + an E4M3 scale per 16
    case FMT_MXFP4: return rows * cols / 2 + rows * cols / 32;  // codes + an E8M0 scale per 32
    case FMT_FP8R: return rows * cols + rows * cols / 128;      // E4M3 + a bf16 scale per 256
    default: return rows * cols * 2;
  }
}

// Stream formats of an expert layer's gate|up and down matrices for the configured expert format.
int gate_up_fmt(const mk_config &f) {
  return f.expert_format == MK_DT_NVFP4 ? FMT_NVFP4 : (f.expert_format == MK_DT_MXFP4 ? FMT_FP8R : FMT_BF16);
}
int down_fmt(const mk_config &f) {
  return f.expert_format == MK_DT_NVFP4 ? FMT_NVFP4 : (f.expert_format == MK_DT_MXFP4 ? FMT_MXFP4 : FMT_BF16);
}

struct Schedule {
  std::vector<Phase> phases;
  int64_t part_floats[3] = {0, 0, 0};
  int32_t n_chunks = 0, chunk = 0;
  int32_t mla_chunks = 0, mla_chunk = 0;  // latent attention split-KV geometry
};

}  // namespace

struct mk_ctx {
  mk_config cfg;
  int device = -1;
  int G = 0;  // workgroups (compute units)
  std::vector<LayerSlots> L;
  Slot embed, final_norm, lm_head;
  uint32_t global_need = 0, global_have = 0;
  int64_t packed_bytes = 0;
  int n_lin = 0, n_resid = 0, n_moe = 0, n_swi = 0, max_rows = 1;  // n_swi: dense FFN layers (SwiGLU finalisers)
  std::vector<int> lin_index;  // per layer: index among linear-attention layers (-1 otherwise)
  int mix_stride = 0;
  Schedule sched[kMaxBatch + 1];  // by row count
  // scratch layout (byte offsets)
  int64_t o_rope_mla = 0, o_loop = 0;
  int64_t o_status = 0, o_bar = 0, o_fin = 0, o_x = 0, o_ss = 0, o_part[3] = {0, 0, 0}, o_mix = 0, o_attn = 0,
          o_cand = 0, o_rope = 0, o_snap = 0, o_ptrs = 0, o_phases[kMaxBatch + 1] = {}, scratch_bytes = 0,
          o_stg[3] = {0, 0, 0};
  int64_t kv_bytes = 0, lin_bytes = 0, latent_bytes = 0;
  // bound buffers
  bool bound = false;
  uint8_t *wbuf = nullptr, *scratch = nullptr;
  mk_buffers bufs;
  uint32_t bar_done = 0;  // grid barriers completed on the bound workspace's counters (they are monotone)
  // multi-step launches: expanded phase tables by (rows, steps), and which one the workspace holds
  std::map<std::pair<int, int>, std::vector<Phase>> loop_tables;
  std::pair<int, int> loop_loaded = {0, 0};
  bool needs_reset = false;
  uint64_t *trace = nullptr;  // optional per-phase timestamps (device buffer)
  bool cooperative = true;    // cooperative launch (co-residency guaranteed by the runtime)
  bool nvfp4 = false;         // the schedule has NVFP4 products: the step kernel build that decodes them
  // per-op baseline graphs: one instantiated graph per row count, with the launch arguments it was
  // captured with (a call whose arguments differ captures again), and the stream it is captured on
  hipGraphExec_t graph[kMaxBatch + 1] = {};
  StepArgs graph_args[kMaxBatch + 1];
  hipStream_t capture_stream = nullptr;
};

namespace {

uint32_t kind_bit(int kind) { return 1u << kind; }

mk_status validate(const mk_config *c) {
  if (!c) return fail(MK_E_ARG, "cfg is NULL");
  if (c->n_layers < 1 || c->n_layers > MK_MAX_LAYERS) return fail(MK_E_ARG, "n_layers %d out of [1, %d]", c->n_layers, MK_MAX_LAYERS);
  if (c->hidden <= 0 || c->hidden % 256) return fail(MK_E_UNSUPPORTED, "hidden %d must be a positive multiple of 256", c->hidden);
  if (c->vocab < 0 || c->vocab % 16) return fail(MK_E_UNSUPPORTED, "vocab %d must be a multiple of 16", c->vocab);
  if (c->max_batch < 1 || c->max_batch > MK_MAX_BATCH) return fail(MK_E_ARG, "max_batch %d out of [1, %d]", c->max_batch, MK_MAX_BATCH);
  if (c->max_ctx < 1) return fail(MK_E_ARG, "max_ctx %d", c->max_ctx);
  if (!(c->eps > 0.0f)) return fail(MK_E_ARG, "eps must be positive");
  bool any_gqa = false, any_lin = false, any_dense = false, any_moe = false, any_mla = false;
  for (int l = 0; l < c->n_layers; ++l) {
    int m = c->mixer[l], f = c->ffn_kind[l];
    if (m < MK_MIXER_GQA || m > MK_MIXER_MLA) return fail(MK_E_ARG, "layer %d: bad mixer %d", l, m);
    if (f != MK_FFN_DENSE && f != MK_FFN_MOE) return fail(MK_E_ARG, "layer %d: bad ffn kind %d", l, f);
    any_mla |= m == MK_MIXER_MLA;
    any_gqa |= m == MK_MIXER_GQA;
    any_lin |= m == MK_MIXER_GDN || m == MK_MIXER_KDA;
    any_dense |= f == MK_FFN_DENSE;
    any_moe |= f == MK_FFN_MOE;
  }
  if (any_dense && (c->ffn <= 0 || c->ffn % 256)) return fail(MK_E_UNSUPPORTED, "ffn %d must be a positive multiple of 256", c->ffn);
  if (any_moe) {
    if (c->max_batch > kMaxRows) return fail(MK_E_UNSUPPORTED, "mixture-of-experts layers run at most %d rows per step", kMaxRows);
    if (c->n_experts < 1 || c->n_experts > kMaxExperts) return fail(MK_E_UNSUPPORTED, "n_experts %d out of [1, %d]", c->n_experts, kMaxExperts);
    if (c->top_k < 1 || c->top_k > kMaxTopK || c->top_k > c->n_experts)
      return fail(MK_E_UNSUPPORTED, "top_k %d out of [1, min(%d, n_experts)]", c->top_k, kMaxTopK);
    if (c->n_shared < 0 || c->n_shared > kMaxShared) return fail(MK_E_UNSUPPORTED, "n_shared %d out of [0, %d]", c->n_shared, kMaxShared);
    if (c->expert_format != MK_DT_BF16 && c->expert_format != MK_DT_NVFP4 && c->expert_format != MK_DT_MXFP4)
      return fail(MK_E_ARG, "bad expert_format %d", c->expert_format);
    const int q = c->expert_format == MK_DT_BF16 ? 256 : 512;
    if (c->expert_ffn <= 0 || c->expert_ffn % q || c->hidden % q)
      return fail(MK_E_UNSUPPORTED, "expert_ffn %d and hidden %d must be positive multiples of %d", c->expert_ffn, c->hidden, q);
  }
  if (any_gqa) {
    if (c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->n_q_heads % c->n_kv_heads)
      return fail(MK_E_ARG, "n_q_heads %d must be a positive multiple of n_kv_heads %d", c->n_q_heads, c->n_kv_heads);
    if (c->head_dim != 64 && c->head_dim != 128) return fail(MK_E_UNSUPPORTED, "head_dim %d (64 or 128 supported)", c->head_dim);
    if ((c->n_q_heads * c->head_dim) % 256) return fail(MK_E_UNSUPPORTED, "n_q_heads * head_dim must be a multiple of 256");
    if (c->n_q_heads / c->n_kv_heads > 8)
      return fail(MK_E_UNSUPPORTED, "query heads per kv head %d exceed 8", c->n_q_heads / c->n_kv_heads);
    if (!(c->rope_theta > 0.0f)) return fail(MK_E_ARG, "rope_theta must be positive");
  }
  if (any_mla) {
    if (c->mla_heads < 1) return fail(MK_E_ARG, "mla_heads %d", c->mla_heads);
    if (c->kv_rank <= 0 || c->kv_rank % 128 || c->kv_rank + c->rope_dim > 576 || (c->kv_rank + c->rope_dim) % 32)
      return fail(MK_E_UNSUPPORTED, "latent rank %d (multiple of 128) + rotary width %d must be a multiple of 32 up to 576",
                  c->kv_rank, c->rope_dim);
    if (c->rope_dim <= 0 || c->rope_dim % 16) return fail(MK_E_UNSUPPORTED, "rope_dim %d must be a positive multiple of 16", c->rope_dim);
    if (c->nope_dim <= 0 || c->nope_dim % 128) return fail(MK_E_UNSUPPORTED, "nope_dim %d must be a positive multiple of 128", c->nope_dim);
    if (c->v_dim <= 0 || c->v_dim % 16 || (c->mla_heads * c->v_dim) % 128)
      return fail(MK_E_UNSUPPORTED, "v_dim %d: a multiple of 16 with heads * v_dim a multiple of 128", c->v_dim);
    if (!(c->rope_theta > 0.0f)) return fail(MK_E_ARG, "rope_theta must be positive");
  }
  if (any_lin) {
    if (c->d_k != 128 || c->d_v != 128) return fail(MK_E_UNSUPPORTED, "d_k = d_v = 128 supported (got %d, %d)", c->d_k, c->d_v);
    if (c->lin_heads <= 0 || (c->lin_heads * c->d_v) % 256)
      return fail(MK_E_UNSUPPORTED, "lin_heads * d_v must be a positive multiple of 256");
  }
  return MK_OK;
}

// Chooses the k-split count of a product: a power of two dividing the workgroup count (each
// workgroup works inside one split), nf = KF / S a multiple of the compute-wave count (of four times
// it for NVFP4, whose stream items hold four fragments; above kMaxRows rows a bf16 split only needs a
// fragment per wave, the waves taking runs one fragment apart), the activation pieces of one workgroup within
// the LDS budget, and the fewest fragment-slots on the busiest workgroup (plus about one fragment's
// time per unit for the cross-wave reduction). A product of nseg segments of segT tiles each gives every
// segment its own activation when per_seg_act (one piece per segment a workgroup's units touch).
int choose_splits(int segT, int nseg, int KF, int R, int G, int max_S, bool per_seg_act = false, int fpi = 1,
                  int *pieces_out = nullptr, bool resid = false, int consumer_rows = 0) {
  int best = -1, best_pieces = 1;
  double best_cost = 1e300;
  const int64_t U = (int64_t)segT * nseg;
  if (fpi != 1 && fpi != 2 && fpi != 4) return -1;
  const int q = fpi * kCWaves;  // fpi: fragments per stream item (1 bf16, 2 FP8, 4 NVFP4 / MXFP4)
  const bool uneven = fpi == 1 && R > kMaxRows;
  for (int S = 1; S <= KF / q && S <= G; S *= 2) {
    if (KF % S || (!uneven && (KF / S) % q) || S > max_S || G % S) continue;
    const int nf = KF / S;
    const int64_t per_split = G / S;                     // workgroups per k-split
    const int64_t per = (U + per_split - 1) / per_split;  // units per workgroup (the cost estimate)
    const int64_t per_max = per;  // the busiest workgroup's units
    if (per_max > kMaxUnits) continue;
    const int np = per_seg_act ? (int)std::min<int64_t>((per_max - 1 + segT - 1) / segT + 1, nseg) : 1;
    if (np > kMaxPieces) continue;
    const int C = R <= kMaxRows ? 2 * R : 32;  // B-operand columns: bf16 high and low halves, 16 per group of 8 rows
    if ((int64_t)np * nf * 64 * C > (R <= kMaxRows ? kActLdsBudgetNarrow : kActLdsBudget)) continue;
    // a residual product split over k also pays, per unit, the acknowledgement of its partials and the
    // tile counter round trip (about five fragment times); with one split the unit adds into the
    // residual directly
    const double fin = (resid && S > 1) ? 5.0 * per : 0.0;
    // a consumer that sums the k-split partials of every value it reads (the mixers read their inputs
    // that way, every workgroup's routing its router logits) pays for each split, per row
    const double cost = (double)per * ((nf + kCWaves - 1) / kCWaves + 1.0) + fin + (double)S * consumer_rows + 0.01 * S;
    if (cost < best_cost) { best_cost = cost; best = S; best_pieces = np; }
  }
  if (pieces_out) *pieces_out = best_pieces;
  return best;
}

Phase gemv_phase(const Slot &w, int act, int out, int R, int G, int max_S, int consumer_rows = 0) {
  const bool resid = out == OUT_RESID;
  Phase p;
  memset(&p, 0, sizeof(p));
  p.type = PH_GEMV;
  p.w_off = w.off;
  p.N = w.N;
  p.K = w.K;
  p.T = w.N / kTileRows;
  p.KF = w.K / kFragK;
  p.S = choose_splits(p.T, 1, p.KF, R, G, max_S, false, 1, nullptr, resid, consumer_rows);
  p.nf = p.S > 0 ? p.KF / p.S : 0;
  p.act = act;
  p.out = out;
  p.nseg = 1;
  p.seg_T = p.T;
  p.pieces = 1;
  return p;
}

mk_status build_schedule(mk_ctx *c, int R, Schedule &sc) {
  const mk_config &f = c->cfg;
  const int G = c->G;
  sc.phases.clear();
  sc.part_floats[0] = sc.part_floats[1] = sc.part_floats[2] = 0;
  // partial buffers: 0 = mixer inputs / router / dense gate-up, 1 = residual products, 2 = expert gate-up
  auto add_gemv = [&](Phase p, int buf) -> mk_status {
    if (p.S <= 0) return fail(MK_E_CAPACITY, "no k-split of a %dx%d product fits the on-chip budget at %d rows", p.N, p.K, R);
    const int64_t units = p.seg == SEG_EXPERT ? (int64_t)p.seg_T * (p.n_shared + std::min(p.n_exp, R * p.top_k)) : p.T;
    if ((units + G / p.S - 1) / (G / p.S) > kMaxUnits)
      return fail(MK_E_CAPACITY, "%dx%d product: too many units per workgroup", p.N, p.K);
    int64_t need = (int64_t)p.S * R * p.N;
    if (p.seg == SEG_EXPERT && p.out == OUT_RESID)  // one partial per (segment, k-split)
      need = (int64_t)(p.n_shared + std::min(p.n_exp, R * p.top_k)) * p.S * R * p.seg_T * kTileRows;
    if (!(p.out == OUT_LOGITS && p.S == 1)) sc.part_floats[buf] = std::max(sc.part_floats[buf], need);
    p.dst_part = buf;
    sc.phases.push_back(p);
    return MK_OK;
  };
  // split-KV chunking: fewest positions on the busiest workgroup
  if (f.n_q_heads > 0) {
    const int nseq_max = R;  // decode: R sequences; verify (R = 8): 1 sequence, 8 query rows
    double best = 1e300;
    for (int cs = 64; cs <= 64 * ((f.max_ctx + 63) / 64); cs += 64) {
      const int nc = (f.max_ctx + cs - 1) / cs;
      const int64_t units = (int64_t)nseq_max * f.n_kv_heads * nc;
      const double cost = (double)((units + G - 1) / G) * (cs + 64) + 1e-3 * nc;
      if ((int64_t)nc * (f.head_dim + 2) * 4 + (nc + 1) * 4 + f.head_dim * 4 > kLdsBytes) continue;  // merge stages
                                                                                                     // all chunks in LDS
      if (cost < best) { best = cost; sc.chunk = cs; sc.n_chunks = nc; }
    }
    if (sc.chunk == 0) return fail(MK_E_CAPACITY, "no split-KV chunking fits max_ctx %d", f.max_ctx);
  }
  // latent attention split-KV: units (row, chunk, 8-head group), chunks a multiple of 64 positions;
  // fewest positions on the busiest workgroup, then the fewest chunks
  bool has_mla = false;
  for (int l = 0; l < f.n_layers; ++l) has_mla |= f.mixer[l] == MK_MIXER_MLA;
  if (has_mla) {
    const int nhg = (f.mla_heads + 7) / 8;
    double best = 1e300;
    for (int cs = 64; cs <= 64 * ((f.max_ctx + 63) / 64); cs += 64) {
      const int nc = (f.max_ctx + cs - 1) / cs;
      const int64_t units = (int64_t)R * nc * nhg;
      if ((int64_t)nc * (f.kv_rank + 2) * 4 + (nc + 1) * 4 > kLdsBytes) continue;  // merge stages all chunks
      const double cost = (double)((units + G - 1) / G) * (cs + 64) + 1e-3 * nc;
      if (cost < best) { best = cost; sc.mla_chunk = cs; sc.mla_chunks = nc; }
    }
    if (sc.mla_chunk == 0) return fail(MK_E_CAPACITY, "no latent split-KV chunking fits max_ctx %d", f.max_ctx);
  }
  Phase e;
  memset(&e, 0, sizeof(e));
  e.type = PH_EMBED;
  e.w_off = c->embed.off;
  sc.phases.push_back(e);
  int resid = 0;
  c->n_moe = 0;
  for (int l = 0; l < f.n_layers; ++l) {
    const LayerSlots &s = c->L[l];
    const int m = f.mixer[l];
    Phase p = gemv_phase(s.mix_in, ACT_NORM, OUT_PART, R, G, 64, R);
    p.layer = l;
    p.gain_off = s.attn_norm.off;
    if (mk_status st = add_gemv(p, 0)) return st;
    Phase mx;
    memset(&mx, 0, sizeof(mx));
    mx.layer = l;
    mx.src_part = 0;
    mx.src_S = p.S;
    mx.src_N = p.N;
    mx.q_off = s.q_off; mx.k_off = s.k_off; mx.v_off = s.v_off; mx.a_off = s.a_off; mx.b_off = s.b_off;
    if (m == MK_MIXER_GQA) {
      mx.type = PH_ATTN;
      mx.chunk = sc.chunk;
      mx.n_chunks = sc.n_chunks;
      sc.phases.push_back(mx);
      Phase mg = mx;
      mg.type = PH_MERGE;
      sc.phases.push_back(mg);
    } else if (m == MK_MIXER_MLA) {
      // latent attention: absorbed queries (one product per head, its slice of the projection as the
      // activation), split-KV attention over the latent cache, merge, value up-projection per head
      const int hq = f.mla_heads, rank = f.kv_rank;
      Phase ak = gemv_phase(s.wuk_t, ACT_PART, OUT_PART, R, G, 1);
      ak.layer = l;
      ak.seg = SEG_HEADS;
      ak.nseg = hq;
      ak.seg_T = rank / kTileRows;
      ak.src_part = 0;
      ak.src_S = p.S;
      ak.src_N = p.N;
      ak.src_off = s.q_off;
      ak.src_seg = f.nope_dim + f.rope_dim;
      ak.S = choose_splits(ak.seg_T, hq, ak.KF, R, G, 1, true, 1, &ak.pieces);
      ak.nf = ak.S > 0 ? ak.KF / ak.S : 0;
      if (mk_status st = add_gemv(ak, 2)) return st;
      mx.type = PH_MLA;
      mx.rank = rank;
      mx.rope = f.rope_dim;
      mx.nope = f.nope_dim;
      mx.qk_stride = f.nope_dim + f.rope_dim;
      mx.dkv_off = s.dkv_off;
      mx.kr_off = s.kr_off;
      mx.heads = hq;
      mx.hgroup = 8;
      mx.mla_src = 2;
      mx.chunk = sc.mla_chunk;
      mx.n_chunks = sc.mla_chunks;
      sc.phases.push_back(mx);
      Phase mg = mx;
      mg.type = PH_MLA_MERGE;
      sc.phases.push_back(mg);
      Phase av = gemv_phase(s.wuv, ACT_MIX, OUT_PART, R, G, 64);
      av.layer = l;
      av.seg = SEG_HEADS;
      av.nseg = hq;
      av.seg_T = f.v_dim / kTileRows;
      av.src_off = 0;
      av.src_seg = rank;
      av.S = choose_splits(av.seg_T, hq, av.KF, R, G, 64, true, 1, &av.pieces);
      av.nf = av.S > 0 ? av.KF / av.S : 0;
      if (mk_status st = add_gemv(av, 0)) return st;
      Phase o = gemv_phase(s.wo, ACT_PART, OUT_RESID, R, G, 68);
      o.layer = l;
      o.src_part = 0;
      o.src_S = av.S;
      o.src_N = av.N;
      o.cnt_off = (resid++) * (f.hidden / kTileRows);
      if (mk_status st = add_gemv(o, 1)) return st;
    } else {
      mx.type = PH_DELTA;
      mx.lin_idx = c->lin_index[l];
      mx.per_channel_gate = m == MK_MIXER_KDA;
      // state rows per unit: the fewest (8, 16, 32, 64) that give at most one unit per workgroup, else
      // 64: a workgroup's units run one after another, each a round trip to memory, while the rows of
      // one unit load together. A verify block (one sequence, 8 token rows applied in order) counts
      // its units separately.
      auto rows_per_unit = [&](int64_t seqs) {
        int rpu = 8;
        while (rpu < 64 && rpu < f.d_v && seqs * f.lin_heads * (f.d_v / rpu) > G) rpu *= 2;
        return rpu;
      };
      mx.chunk = rows_per_unit(R);
      mx.chunk_verify = rows_per_unit(1);
      sc.phases.push_back(mx);
    }
    if (m != MK_MIXER_MLA) {
      Phase o = gemv_phase(s.wo, ACT_MIX, OUT_RESID, R, G, 68);
      o.layer = l;
      o.cnt_off = (resid++) * (f.hidden / kTileRows);
      if (mk_status st = add_gemv(o, 1)) return st;
    }
    if (f.ffn_kind[l] == MK_FFN_DENSE) {
      Phase gu = gemv_phase(s.gu, ACT_NORM, OUT_PART, R, G, 64);
      gu.layer = l;
      gu.gain_off = s.ffn_norm.off;
      if (mk_status st = add_gemv(gu, 0)) return st;
      Phase d = gemv_phase(s.wd, ACT_SWIGLU, OUT_RESID, R, G, 68);
      d.layer = l;
      d.src_part = 0;
      d.src_S = gu.S;
      d.src_N = gu.N;
      d.cnt_off = (resid++) * (f.hidden / kTileRows);
      if (mk_status st = add_gemv(d, 1)) return st;
    } else {
      // mixture of experts: router logits; gate|up of the shared experts and the batch's routed union
      // (every workgroup derives the union from the logits); down of the same segments, each row's
      // activation scaled by its routing weight, summed into the residual
      const int fmt_gu = gate_up_fmt(f), fmt_d = down_fmt(f);
      const int F = f.expert_ffn, H = f.hidden;
      const int nseg_max = f.n_shared + std::min(f.n_experts, R * f.top_k);
      Phase r = gemv_phase(s.router, ACT_NORM, OUT_PART, R, G, 64, R);  // every workgroup sums its splits
      r.layer = l;
      r.gain_off = s.ffn_norm.off;
      if (mk_status st = add_gemv(r, 0)) return st;
      Phase gu;
      memset(&gu, 0, sizeof(gu));
      gu.type = PH_GEMV;
      gu.layer = l;
      gu.seg = SEG_EXPERT;
      gu.fmt = fmt_gu;
      gu.w_off = s.ex_gu_off;
      gu.seg_stride = s.ex_gu_bytes;
      gu.seg_T = 2 * F / kTileRows;
      gu.nseg = f.n_shared;
      gu.N = nseg_max * 2 * F;
      gu.K = H;
      gu.T = gu.N / kTileRows;
      gu.KF = H / kFragK;
      gu.S = choose_splits(gu.seg_T, nseg_max, gu.KF, R, G, 64, false, frags_per_item(fmt_gu), &gu.pieces);
      gu.nf = gu.S > 0 ? gu.KF / gu.S : 0;
      gu.act = ACT_NORM;
      gu.gain_off = s.ffn_norm.off;
      gu.out = OUT_PART;
      gu.moe_idx = c->n_moe;
      gu.n_exp = f.n_experts;
      gu.top_k = f.top_k;
      gu.n_shared = f.n_shared;
      gu.z_part = 0;
      gu.z_S = r.S;
      gu.z_N = r.N;
      gu.ts_off = s.ts_off;
      gu.route_q = (int)sc.phases.size();
      if (mk_status st = add_gemv(gu, 2)) return st;
      Phase d = gu;
      d.w_off = s.ex_down_off;
      d.seg_stride = s.ex_down_bytes;
      d.seg_T = H / kTileRows;
      d.N = H;
      d.K = F;
      d.T = d.seg_T;
      d.KF = F / kFragK;
      d.fmt = fmt_d;
      d.S = choose_splits(d.seg_T, nseg_max, d.KF, R, G, 64, true, frags_per_item(fmt_d), &d.pieces);
      d.nf = d.S > 0 ? d.KF / d.S : 0;
      d.act = ACT_SWIGLU;
      d.gain_off = 0;
      d.src_part = 2;
      d.src_S = gu.S;
      d.src_N = gu.N;
      d.src_off = 0;
      d.src_seg = 2 * F;
      d.out = OUT_RESID;
      d.cnt_off = (resid++) * (H / kTileRows);
      if (mk_status st = add_gemv(d, 1)) return st;
      ++c->n_moe;
    }
  }
  c->n_resid = resid;
  if (f.vocab > 0) {
    Phase lm = gemv_phase(c->lm_head, ACT_NORM, OUT_LOGITS, R, G, 68);
    lm.gain_off = c->final_norm.off;
    lm.cnt_off = resid * (f.hidden / kTileRows);  // finalizer counters after the residual ones
    if (mk_status st = add_gemv(lm, 0)) return st;
    Phase fin;
    memset(&fin, 0, sizeof(fin));
    fin.type = PH_FINAL;
    sc.phases.push_back(fin);
  } else {
    Phase ho;
    memset(&ho, 0, sizeof(ho));
    ho.type = PH_HIDDEN_OUT;
    sc.phases.push_back(ho);
  }
  // staged activations: each product whose activation is the RMSNorm of x, a mixer output (one for
  // all its rows) or a dense SwiGLU copies it from a buffer its producer wrote in the LDS layout
  {
    const int pairs = f.ffn / kTileRows;
    int x_writer = -1, mix_writer = -1, n_swi = 0;
    for (size_t i = 0; i < sc.phases.size(); ++i) {
      Phase &p = sc.phases[i];
      if (p.type == PH_EMBED) {
        x_writer = (int)i;
      } else if (p.type == PH_DELTA || p.type == PH_MERGE) {
        mix_writer = (int)i;
      } else if (p.type == PH_GEMV) {
        const bool shared = p.seg == SEG_NONE || p.act == ACT_NORM;
        if (p.act == ACT_NORM && shared && x_writer >= 0) {
          Phase &w = sc.phases[(size_t)x_writer];
          if (!w.stg_out) {
            w.stg_out = 1;
            w.stg_gain_off = p.gain_off;
          }
          if (w.stg_gain_off == p.gain_off) p.stg_in = STG_X;
        } else if (p.act == ACT_MIX && p.seg == SEG_NONE && p.src_off == 0 && mix_writer >= 0) {
          sc.phases[(size_t)mix_writer].stg_out = 1;
          p.stg_in = STG_MIX;
        } else if (p.act == ACT_SWIGLU && p.seg == SEG_NONE && i > 0) {
          Phase &gu = sc.phases[i - 1];  // the dense gate|up product right before its down product
          if (gu.type == PH_GEMV && gu.seg == SEG_NONE && gu.out == OUT_PART && gu.N == 2 * f.ffn && p.K == f.ffn &&
              p.src_off == 0 && p.src_S == gu.S) {
            gu.stg_out = 1;
            gu.swi_cnt_off = (int32_t)((int64_t)resid * (f.hidden / kTileRows) + f.vocab / kTileRows + (int64_t)n_swi * pairs);
            ++n_swi;
            p.stg_in = STG_H;
          }
        }
        if (p.out == OUT_RESID) x_writer = (int)i;
      }
    }
    c->n_swi = n_swi;
  }
  // the weight stream of the compute waves follows the product phases in order
  int next = -1;
  for (int i = (int)sc.phases.size() - 1; i >= 0; --i) {
    sc.phases[(size_t)i].next_gemv = next;
    if (sc.phases[(size_t)i].type == PH_GEMV) next = i;
  }
  return MK_OK;
}

mk_status layout(mk_ctx *c) {
  const mk_config &f = c->cfg;
  const int H = f.hidden;
  int64_t off = 0;
  auto place = [&](Slot &s, int N, int K, bool packed) {
    s.N = N;
    s.K = K;
    s.packed = packed;
    s.off = off;
    off = align_up(off + s.bytes(), 256);
  };
  c->L.assign(f.n_layers, LayerSlots());
  c->lin_index.assign(f.n_layers, -1);
  c->n_lin = 0;
  int mix_w = 0;
  if (f.vocab > 0) {
    place(c->embed, f.vocab, H, false);
    c->global_need = kind_bit(MK_W_EMBED) | kind_bit(MK_W_FINAL_NORM) | kind_bit(MK_W_LM_HEAD);
  }
  for (int l = 0; l < f.n_layers; ++l) {
    LayerSlots &s = c->L[l];
    place(s.attn_norm, 1, H, false);
    place(s.ffn_norm, 1, H, false);
    const int m = f.mixer[l];
    int rows, inner;
    if (m == MK_MIXER_GQA) {
      s.q_off = 0;
      s.k_off = f.n_q_heads * f.head_dim;
      s.v_off = s.k_off + f.n_kv_heads * f.head_dim;
      rows = s.v_off + f.n_kv_heads * f.head_dim;
      inner = f.n_q_heads * f.head_dim;
      s.need = kind_bit(MK_W_Q) | kind_bit(MK_W_K) | kind_bit(MK_W_V) | kind_bit(MK_W_O);
    } else if (m == MK_MIXER_MLA) {
      const int hq = f.mla_heads, qk = f.nope_dim + f.rope_dim;
      s.q_off = 0;
      s.dkv_off = (int)round16((int64_t)hq * qk);
      s.kr_off = s.dkv_off + f.kv_rank;
      rows = (int)round16(s.kr_off + f.rope_dim);
      inner = hq * f.v_dim;
      mix_w = std::max(mix_w, hq * f.kv_rank);  // merged latent outputs
      s.need = kind_bit(MK_W_Q) | kind_bit(MK_W_DKV) | kind_bit(MK_W_KR) | kind_bit(MK_W_UK) | kind_bit(MK_W_UV) |
               kind_bit(MK_W_O);
    } else {
      const int hk = f.lin_heads * f.d_k;
      s.q_off = 0;
      s.k_off = hk;
      s.v_off = 2 * hk;
      s.a_off = (int)round16(s.v_off + f.lin_heads * f.d_v);
      s.b_off = (int)round16(s.a_off + (m == MK_MIXER_KDA ? hk : f.lin_heads));
      rows = (int)round16(s.b_off + f.lin_heads);
      inner = f.lin_heads * f.d_v;
      s.need = kind_bit(MK_W_Q) | kind_bit(MK_W_K) | kind_bit(MK_W_V) | kind_bit(MK_W_A) | kind_bit(MK_W_B) |
               kind_bit(MK_W_O);
      c->lin_index[l] = c->n_lin++;
    }
    s.need |= kind_bit(MK_W_ATTN_NORM) | kind_bit(MK_W_FFN_NORM);
    mix_w = std::max(mix_w, inner);
    place(s.mix_in, rows, H, true);
    if (m == MK_MIXER_MLA) {
      place(s.wuk_t, f.mla_heads * f.kv_rank, f.nope_dim, true);
      place(s.wuv, f.mla_heads * f.v_dim, f.kv_rank, true);
    }
    place(s.wo, H, inner, true);
    if (f.ffn_kind[l] == MK_FFN_DENSE) {
      s.need |= kind_bit(MK_W_GATE) | kind_bit(MK_W_UP) | kind_bit(MK_W_DOWN);
      place(s.gu, 2 * f.ffn, H, true);
      place(s.wd, H, f.ffn, true);
    } else {
      const int64_t nblk = (int64_t)f.n_experts + f.n_shared;
      s.need |= kind_bit(MK_W_ROUTER);
      place(s.router, (int)round16(f.n_experts), H, true);
      s.ex_gu_bytes = align_up(matrix_bytes(2LL * f.expert_ffn, H, gate_up_fmt(f)), 256);
      s.ex_down_bytes = align_up(matrix_bytes(H, f.expert_ffn, down_fmt(f)), 256);
      s.ex_gu_off = off;
      off += nblk * s.ex_gu_bytes;
      s.ex_down_off = off;
      off += nblk * s.ex_down_bytes;
      s.ts_off = off;  // tensor scales [block][gate, up, down] (NVFP4; 1 for bf16)
      off = align_up(off + nblk * 3 * 4, 256);
      s.ex_have.assign((size_t)nblk * 3, 0);
    }
  }
  if (f.vocab > 0) {
    place(c->final_norm, 1, H, false);
    place(c->lm_head, f.vocab, H, true);
  }
  c->packed_bytes = off;
  c->mix_stride = (int)align_up(mix_w, 64);
  return MK_OK;
}

// Finaliser counters: 16-row tiles of each residual product, of the vocabulary, then the 16-row pairs
// of each dense gate|up product whose SwiGLU is staged.
int64_t fin_counters(const mk_ctx *c) {
  const mk_config &f = c->cfg;
  return (int64_t)c->n_resid * (f.hidden / kTileRows) + f.vocab / kTileRows + (int64_t)c->n_swi * (f.ffn / kTileRows);
}

// Staged activation buffers at R rows: [K / 8][C][8] bf16 each (C columns of the B operand).
int act_columns(int R) { return R <= kMaxRows ? 2 * R : 32; }
void stg_sizes(const mk_ctx *c, int R, int64_t (&bytes)[3]) {
  const mk_config &f = c->cfg;
  const int64_t C = act_columns(R);
  bytes[0] = (int64_t)f.hidden * C * 2;
  bytes[1] = (int64_t)c->mix_stride * C * 2;
  bytes[2] = c->n_swi > 0 ? (int64_t)f.ffn * C * 2 : 0;
}

mk_status scratch_layout(mk_ctx *c) {
  const mk_config &f = c->cfg;
  const int R = c->max_rows, H = f.hidden, G = c->G;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    int64_t o = off;
    off = align_up(off + std::max<int64_t>(bytes, 0), 256);
    return o;
  };
  int64_t part[3] = {0, 0, 0}, attn = 0;
  for (int r = 1; r <= kMaxBatch; ++r) {
    const Schedule &s = c->sched[r];
    if (s.phases.empty()) continue;
    for (int i = 0; i < 3; ++i) part[i] = std::max<int64_t>(part[i], s.part_floats[i]);
    if (f.n_q_heads > 0) attn = std::max<int64_t>(attn, (int64_t)r * f.n_q_heads * s.n_chunks * (f.head_dim + 2));
    if (s.mla_chunks > 0) attn = std::max<int64_t>(attn, (int64_t)r * f.mla_heads * s.mla_chunks * (f.kv_rank + 2));
  }
  c->o_status = take(256);
  c->o_bar = take(kBarBytes);
  c->o_fin = take(fin_counters(c) * 4);
  c->o_x = take((int64_t)R * H * 4);
  {
    int64_t sb[3];
    stg_sizes(c, R, sb);
    for (int i = 0; i < 3; ++i) c->o_stg[i] = take(sb[i]);
  }
  c->o_ss = take((int64_t)R * (H / kTileRows) * 4);
  for (int i = 0; i < 3; ++i) c->o_part[i] = take(part[i] * 4);
  c->o_mix = take((int64_t)R * c->mix_stride * 4);
  c->o_attn = take(attn * 4);
  c->o_cand = take((int64_t)G * R * 2 * 4);
  c->o_rope = take(f.n_q_heads > 0 ? (int64_t)f.max_ctx * (f.head_dim / 2) * 2 * 4 : 0);
  c->o_snap = take(f.vocab > 0 ? (int64_t)c->n_lin * kMaxRows * f.lin_heads * f.d_v * f.d_k * 4 : 0);
  c->o_rope_mla = take(f.mla_heads > 0 ? (int64_t)f.max_ctx * (f.rope_dim / 2) * 2 * 4 : 0);
  c->o_ptrs = take((int64_t)5 * MK_MAX_LAYERS * 8);
  for (int r = 1; r <= kMaxBatch; ++r)
    if (!c->sched[r].phases.empty()) c->o_phases[r] = take((int64_t)c->sched[r].phases.size() * sizeof(Phase));
  int64_t max_phases = 0;
  for (int r = 1; r <= kMaxBatch; ++r) max_phases = std::max<int64_t>(max_phases, (int64_t)c->sched[r].phases.size());
  c->o_loop = take(f.vocab > 0 ? (int64_t)MK_MAX_LOOP_STEPS * max_phases * sizeof(Phase) : 0);  // multi-step tables
  c->scratch_bytes = off;
  c->kv_bytes = (int64_t)f.max_batch * f.n_kv_heads * f.max_ctx * f.head_dim * 2;
  c->lin_bytes = (int64_t)f.max_batch * f.lin_heads * f.d_v * f.d_k * 4;
  c->latent_bytes = (int64_t)f.max_batch * f.max_ctx * (f.kv_rank + f.rope_dim) * 2;
  return MK_OK;
}

// Where a weight descriptor lands: a slot of the packed buffer (dense tensors), or an expert block.
struct Target {
  Slot *slot = nullptr;       // dense tensor
  int64_t off = -1;           // expert matrix: byte offset of the packed matrix (gate|up or down)
  int64_t mrows = 0;          // expert matrix rows (gate|up: 2F)
  int64_t ts_off = -1;        // expert: byte offset of its tensor scale
  uint8_t *have_flag = nullptr;
  int fmt = FMT_BF16;
};

mk_status resolve(mk_ctx *c, const mk_weight_desc &w, Slot **slot, int64_t *row_off, int64_t *rows, int64_t *cols,
                  uint32_t **have, Target *tg) {
  const mk_config &f0 = c->cfg;
  *tg = Target();
  if (w.expert != -1) {  // expert tensor: routed expert e >= 0, shared expert s as -2 - s
    if (w.layer < 0 || w.layer >= f0.n_layers || f0.ffn_kind[w.layer] != MK_FFN_MOE)
      return fail(MK_E_ARG, "expert tensor for layer %d, which has no mixture of experts", w.layer);
    const int blk = w.expert >= 0 ? w.expert : f0.n_experts + (-2 - w.expert);
    if ((w.expert >= 0 && w.expert >= f0.n_experts) || (w.expert < 0 && (-2 - w.expert) >= f0.n_shared))
      return fail(MK_E_ARG, "layer %d: expert index %d out of range", w.layer, w.expert);
    LayerSlots &s = c->L[w.layer];
    const int F = f0.expert_ffn, H = f0.hidden;
    int which;
    switch (w.kind) {
      case MK_W_GATE: which = 0; *rows = F; *cols = H; *row_off = 0; break;
      case MK_W_UP: which = 1; *rows = F; *cols = H; *row_off = F; break;
      case MK_W_DOWN: which = 2; *rows = H; *cols = F; *row_off = 0; break;
      default: return fail(MK_E_ARG, "layer %d: kind %d is not an expert tensor", w.layer, w.kind);
    }
    tg->fmt = which < 2 ? gate_up_fmt(f0) : down_fmt(f0);
    tg->off = which < 2 ? s.ex_gu_off + (int64_t)blk * s.ex_gu_bytes : s.ex_down_off + (int64_t)blk * s.ex_down_bytes;
    tg->mrows = which < 2 ? 2LL * F : H;
    tg->ts_off = s.ts_off + ((int64_t)blk * 3 + which) * 4;
    tg->have_flag = &s.ex_have[(size_t)blk * 3 + which];
    *slot = nullptr;
    *have = nullptr;
    return MK_OK;
  }
  const mk_config &f = c->cfg;
  const int H = f.hidden;
  *row_off = 0;
  if (w.layer == -1) {
    *have = &c->global_have;
    if (f.vocab <= 0) return fail(MK_E_ARG, "global tensor kind %d in a slice configuration", w.kind);
    switch (w.kind) {
      case MK_W_EMBED: *slot = &c->embed; *rows = f.vocab; *cols = H; return MK_OK;
      case MK_W_FINAL_NORM: *slot = &c->final_norm; *rows = 1; *cols = H; return MK_OK;
      case MK_W_LM_HEAD: *slot = &c->lm_head; *rows = f.vocab; *cols = H; return MK_OK;
      default: return fail(MK_E_ARG, "kind %d is not a global tensor", w.kind);
    }
  }
  if (w.layer < 0 || w.layer >= f.n_layers) return fail(MK_E_ARG, "layer %d out of range", w.layer);
  LayerSlots &s = c->L[w.layer];
  *have = &s.have;
  const int m = f.mixer[w.layer];
  const bool lin = m == MK_MIXER_GDN || m == MK_MIXER_KDA;
  switch (w.kind) {
    case MK_W_ATTN_NORM: *slot = &s.attn_norm; *rows = 1; *cols = H; return MK_OK;
    case MK_W_FFN_NORM: *slot = &s.ffn_norm; *rows = 1; *cols = H; return MK_OK;
    case MK_W_Q:
      *slot = &s.mix_in; *row_off = s.q_off; *cols = H;
      *rows = m == MK_MIXER_MLA ? (int64_t)f.mla_heads * (f.nope_dim + f.rope_dim)
                                : lin ? (int64_t)f.lin_heads * f.d_k : (int64_t)f.n_q_heads * f.head_dim;
      return MK_OK;
    case MK_W_DKV:
      if (m != MK_MIXER_MLA) break;
      *slot = &s.mix_in; *row_off = s.dkv_off; *rows = f.kv_rank; *cols = H;
      return MK_OK;
    case MK_W_KR:
      if (m != MK_MIXER_MLA) break;
      *slot = &s.mix_in; *row_off = s.kr_off; *rows = f.rope_dim; *cols = H;
      return MK_OK;
    case MK_W_UK:  // natural [heads * nope][rank]; stored per-head transposed
      if (m != MK_MIXER_MLA) break;
      *slot = &s.wuk_t; *rows = (int64_t)f.mla_heads * f.nope_dim; *cols = f.kv_rank;
      return MK_OK;
    case MK_W_UV:
      if (m != MK_MIXER_MLA) break;
      *slot = &s.wuv; *rows = (int64_t)f.mla_heads * f.v_dim; *cols = f.kv_rank;
      return MK_OK;
    case MK_W_K:
      if (m == MK_MIXER_MLA) break;
      *slot = &s.mix_in; *row_off = s.k_off; *cols = H;
      *rows = lin ? (int64_t)f.lin_heads * f.d_k : (int64_t)f.n_kv_heads * f.head_dim;
      return MK_OK;
    case MK_W_V:
      if (m == MK_MIXER_MLA) break;
      *slot = &s.mix_in; *row_off = s.v_off; *cols = H;
      *rows = lin ? (int64_t)f.lin_heads * f.d_v : (int64_t)f.n_kv_heads * f.head_dim;
      return MK_OK;
    case MK_W_A:
      if (!lin) break;
      *slot = &s.mix_in; *row_off = s.a_off; *cols = H;
      *rows = m == MK_MIXER_KDA ? (int64_t)f.lin_heads * f.d_k : f.lin_heads;
      return MK_OK;
    case MK_W_B:
      if (!lin) break;
      *slot = &s.mix_in; *row_off = s.b_off; *cols = H; *rows = f.lin_heads;
      return MK_OK;
    case MK_W_O: *slot = &s.wo; *rows = H; *cols = s.wo.K; return MK_OK;
    case MK_W_GATE:
      if (f.ffn_kind[w.layer] != MK_FFN_DENSE) break;
      *slot = &s.gu; *rows = f.ffn; *cols = H; return MK_OK;
    case MK_W_UP:
      if (f.ffn_kind[w.layer] != MK_FFN_DENSE) break;
      *slot = &s.gu; *row_off = f.ffn; *rows = f.ffn; *cols = H; return MK_OK;
    case MK_W_DOWN:
      if (f.ffn_kind[w.layer] != MK_FFN_DENSE) break;
      *slot = &s.wd; *rows = H; *cols = f.ffn; return MK_OK;
    case MK_W_ROUTER:
      if (f.ffn_kind[w.layer] != MK_FFN_MOE) break;
      *slot = &s.router; *rows = f.n_experts; *cols = H;
      return MK_OK;
    default: break;
  }
  return fail(MK_E_ARG, "layer %d: weight kind %d does not apply to this layer", w.layer, w.kind);
}

void fill_args(mk_ctx *c, StepArgs &a, int R, int verify, const mk_step_io *io) {
  const mk_config &f = c->cfg;
  memset(&a, 0, sizeof(a));
  const Schedule &sc = c->sched[R];
  a.phases = reinterpret_cast<const Phase *>(c->scratch + c->o_phases[R]);
  a.n_phases = (int)sc.phases.size();
  a.n_barriers = a.n_phases - 1;
  a.bar_done = c->bar_done;
  a.R = R;
  a.verify = verify;
  a.phase_begin = 0;
  a.phase_end = a.n_phases;
  a.wbuf = c->wbuf;
  a.bar = reinterpret_cast<uint32_t *>(c->scratch + c->o_bar);
  a.fin = reinterpret_cast<uint32_t *>(c->scratch + c->o_fin);
  a.status = reinterpret_cast<int32_t *>(c->scratch + c->o_status);
  a.x = reinterpret_cast<float *>(c->scratch + c->o_x);
  a.ss = reinterpret_cast<float *>(c->scratch + c->o_ss);
  for (int i = 0; i < 3; ++i) a.part[i] = reinterpret_cast<float *>(c->scratch + c->o_part[i]);
  a.mix = reinterpret_cast<float *>(c->scratch + c->o_mix);
  a.attn = reinterpret_cast<float *>(c->scratch + c->o_attn);
  a.cand = reinterpret_cast<float *>(c->scratch + c->o_cand);
  a.rope = reinterpret_cast<const float *>(c->scratch + c->o_rope);
  a.snap = reinterpret_cast<float *>(c->scratch + c->o_snap);
  for (int i = 0; i < 3; ++i) a.stg[i] = reinterpret_cast<uint16_t *>(c->scratch + c->o_stg[i]);
  void **ptrs = reinterpret_cast<void **>(c->scratch + c->o_ptrs);
  a.kc = ptrs;
  a.vc = ptrs + MK_MAX_LAYERS;
  a.ls = ptrs + 2 * MK_MAX_LAYERS;
  a.lsl = ptrs + 3 * MK_MAX_LAYERS;
  a.lat = ptrs + 4 * MK_MAX_LAYERS;
  a.rope_mla = reinterpret_cast<const float *>(c->scratch + c->o_rope_mla);
  a.tokens = io->tokens;
  a.hidden_in = io->hidden_in;
  const int nseq = verify ? 1 : R;
  for (int b = 0; b < nseq; ++b) a.pos[b] = io->positions[b];
  a.logits = io->logits;
  a.hidden_out = io->hidden_out;
  a.argmax = io->argmax;
  a.route_idx = io->route_idx;
  a.route_w = io->route_w;
  a.H = f.hidden;
  a.V = f.vocab;
  a.max_ctx = f.max_ctx;
  a.mix_stride = c->mix_stride;
  a.nq = f.n_q_heads;
  a.nkv = f.n_kv_heads;
  a.hd = f.head_dim;
  a.lin_heads = f.lin_heads;
  a.dk = f.d_k;
  a.dv = f.d_v;
  a.n_lin = c->n_lin;
  a.eps = f.eps;
  a.timeout_ticks = 200000000;  // 2 s at 100 MHz
  a.trace = c->trace;
}

mk_status check_step(mk_ctx *c, const mk_step_io *io, int R, int nseq, int nrow) {
  if (!c) return fail(MK_E_ARG, "ctx is NULL");
  if (c->device < 0) return fail(MK_E_UNSUPPORTED, "host-only context");
  if (!c->bound) return fail(MK_E_STATE, "buffers are not bound");
  if (!io) return fail(MK_E_ARG, "io is NULL");
  const mk_config &f = c->cfg;
  if (c->global_have != c->global_need) return fail(MK_E_STATE, "global weights missing (mask %x of %x)", c->global_have, c->global_need);
  for (int l = 0; l < f.n_layers; ++l) {
    if (c->L[l].have != c->L[l].need) return fail(MK_E_STATE, "layer %d weights missing (mask %x of %x)", l, c->L[l].have, c->L[l].need);
    for (size_t i = 0; i < c->L[l].ex_have.size(); ++i)
      if (!c->L[l].ex_have[i]) return fail(MK_E_STATE, "layer %d: expert block %zu matrix %zu missing", l, i / 3, i % 3);
  }
  if (!io->positions) return fail(MK_E_ARG, "positions is NULL");
  if (f.vocab > 0) {
    if (!io->tokens || !io->logits) return fail(MK_E_ARG, "tokens and logits are required");
  } else {
    if (!io->hidden_in || !io->hidden_out) return fail(MK_E_ARG, "hidden_in and hidden_out are required");
  }
  for (int b = 0; b < nseq; ++b) {
    const int p = io->positions[b];
    if (p < 0 || (int64_t)p + nrow > f.max_ctx)
      return fail(MK_E_CAPACITY, "position %d + %d rows exceeds max_ctx %d", p, nrow, f.max_ctx);
  }
  if (c->sched[R].phases.empty()) return fail(MK_E_CAPACITY, "no schedule for %d rows", R);
  return MK_OK;
}

mk_status reset_counters(mk_ctx *c, hipStream_t st) {
  HIP_TRY(hipMemsetAsync(c->scratch + c->o_status, 0, 256, st));
  HIP_TRY(hipMemsetAsync(c->scratch + c->o_bar, 0, kBarBytes, st));
  HIP_TRY(hipMemsetAsync(c->scratch + c->o_fin, 0, (size_t)fin_counters(c) * 4, st));
  c->bar_done = 0;
  c->needs_reset = false;
  return MK_OK;
}

// The step kernel build for a step of R rows: NVFP4 experts (at most 8 rows), bf16 up to 8 rows, or
// bf16 above 8 rows (two row groups per weight fragment).
const void *step_kernel(const mk_ctx *c, int R) {
  if (c->nvfp4) return reinterpret_cast<const void *>(mk_step_kernel_nvfp4);
  return R > kMaxRows ? reinterpret_cast<const void *>(mk_step_kernel_wide) : reinterpret_cast<const void *>(mk_step_kernel);
}

mk_status launch_step(mk_ctx *c, StepArgs &a, hipStream_t st) {
  void *args[] = {&a};
  if (c->cooperative) {
    HIP_TRY(hipLaunchCooperativeKernel(step_kernel(c, a.R), dim3(c->G), dim3(kThreads), args, kLdsBytes, st));
  } else {
    HIP_TRY(hipLaunchKernel(step_kernel(c, a.R), dim3(c->G), dim3(kThreads), args, kLdsBytes, st));
  }
  return MK_OK;
}

// The phase table of a launch that runs n decode steps: n copies of the one-step table, each phase
// tagged with its step; the weight stream's link from a step's last product phase (and the phases after
// it) continues into the next step's first product phase, so the weights of step s + 1 are in flight
// while step s finishes; routing owners are re-indexed into their copy.
std::vector<Phase> loop_table(const Schedule &sc, int n) {
  const int P = (int)sc.phases.size();
  int first_gemv = -1;
  for (int i = 0; i < P && first_gemv < 0; ++i)
    if (sc.phases[(size_t)i].type == PH_GEMV) first_gemv = i;
  std::vector<Phase> out;
  out.reserve((size_t)n * P);
  for (int s = 0; s < n; ++s) {
    for (int i = 0; i < P; ++i) {
      Phase ph = sc.phases[(size_t)i];
      ph.step = s;
      if (ph.next_gemv >= 0) ph.next_gemv += s * P;
      else if (s + 1 < n && first_gemv >= 0) ph.next_gemv = first_gemv + (s + 1) * P;
      if (ph.seg == SEG_EXPERT) ph.route_q += s * P;
      out.push_back(ph);
    }
  }
  return out;
}

// Takes the device address of this device's library-held array (once per device; the device is current).
mk_status noalloc_init(int device) {
  if (device < 0 || device >= kNoAllocDevices) return MK_OK;  // mk_decode_step_noalloc then refuses
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (g_noalloc_ptr[device]) return MK_OK;
  void *p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) return fail(MK_E_HIP, "hipGetSymbolAddress of the library working memory: %s", hipGetErrorString(e));
  g_noalloc_ptr[device] = static_cast<uint8_t *>(p);
  return MK_OK;
}

// Byte offsets of one step's working set at R rows inside the library-held array (the same regions,
// sized for R rather than for the context's largest row count, as the bound workspace holds).
struct NoAllocLayout {
  int64_t bar, fin, x, ss, part[3], mix, attn, cand, stg[3], total;
};

NoAllocLayout noalloc_layout(const mk_ctx *c, int R) {
  const mk_config &f = c->cfg;
  const Schedule &s = c->sched[R];
  const int H = f.hidden;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    int64_t o = off;
    off = align_up(off + std::max<int64_t>(bytes, 0), 256);
    return o;
  };
  int64_t attn = 0;
  if (f.n_q_heads > 0) attn = std::max<int64_t>(attn, (int64_t)R * f.n_q_heads * s.n_chunks * (f.head_dim + 2));
  if (s.mla_chunks > 0) attn = std::max<int64_t>(attn, (int64_t)R * f.mla_heads * s.mla_chunks * (f.kv_rank + 2));
  NoAllocLayout L;
  L.bar = take(kBarBytes);
  L.fin = take(fin_counters(c) * 4);
  L.x = take((int64_t)R * H * 4);
  L.ss = take((int64_t)R * (H / kTileRows) * 4);
  for (int i = 0; i < 3; ++i) L.part[i] = take(s.part_floats[i] * 4);
  L.mix = take((int64_t)R * c->mix_stride * 4);
  L.attn = take(attn * 4);
  L.cand = take((int64_t)c->G * R * 2 * 4);
  {
    int64_t sb[3];
    stg_sizes(c, R, sb);
    for (int i = 0; i < 3; ++i) L.stg[i] = take(sb[i]);
  }
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

const char *mk_last_error(void) { return g_err.c_str(); }

mk_status mk_create(const mk_config *cfg, int hip_device, mk_ctx **out) {
  if (!out) return fail(MK_E_ARG, "out is NULL");
  *out = nullptr;
  if (mk_status st = validate(cfg)) return st;
  mk_ctx *c = new mk_ctx();
  c->cfg = *cfg;
  c->device = hip_device;
  c->max_rows = cfg->vocab > 0 ? std::max(kMaxRows, cfg->max_batch) : cfg->max_batch;  // verify blocks have kMaxRows rows
  for (int l = 0; l < cfg->n_layers; ++l)
    if (cfg->ffn_kind[l] == MK_FFN_MOE && cfg->expert_format != MK_DT_BF16) c->nvfp4 = true;
  if (hip_device >= 0) {
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, hip_device);
    if (e != hipSuccess) { delete c; return fail(MK_E_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e)); }
    if (std::string(prop.gcnArchName).find("gfx950") == std::string::npos) {
      delete c;
      return fail(MK_E_UNSUPPORTED, "device %d is %s; this build targets gfx950", hip_device, prop.gcnArchName);
    }
    c->G = prop.multiProcessorCount;
  } else {
    c->G = 256;  // host-only context: MI355X compute unit count
  }
  memset(&c->bufs, 0, sizeof(c->bufs));
  mk_status st = layout(c);
  for (int r = 1; st == MK_OK && r <= kMaxBatch; ++r) {
    if (r > c->max_rows) break;
    st = build_schedule(c, r, c->sched[r]);
  }
  if (st == MK_OK) st = scratch_layout(c);
  if (st != MK_OK) { delete c; return st; }
  if (hip_device >= 0) {
    hipError_t e = hipSetDevice(hip_device);
    for (int R : {1, c->max_rows}) {  // the builds this context launches
      if (e == hipSuccess)
        e = hipFuncSetAttribute(step_kernel(c, R), hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
      if (e != hipSuccess) { delete c; return fail(MK_E_HIP, "kernel setup: %s", hipGetErrorString(e)); }
      int nb = 0;
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, step_kernel(c, R), kThreads, kLdsBytes);
      if (e != hipSuccess || nb < 1) {
        delete c;
        return fail(MK_E_HIP, "step kernel cannot be resident (%d per CU): %s", nb, hipGetErrorString(e));
      }
    }
    if (mk_status s = noalloc_init(hip_device)) { delete c; return s; }
  }
  *out = c;
  return MK_OK;
}

mk_status mk_query_sizes(const mk_ctx *c, mk_sizes *out) {
  if (!c || !out) return fail(MK_E_ARG, "NULL argument");
  out->packed_weights = (uint64_t)c->packed_bytes;
  out->scratch = (uint64_t)c->scratch_bytes;
  out->kv_cache_per_layer = (uint64_t)c->kv_bytes;
  out->lin_state_per_layer = (uint64_t)c->lin_bytes;
  out->latent_per_layer = (uint64_t)c->latent_bytes;
  out->n_phases = (int32_t)c->sched[1].phases.size();
  out->n_workgroups = c->G;
  return MK_OK;
}

mk_status mk_bind_buffers(mk_ctx *c, const mk_buffers *b) {
  if (!c || !b) return fail(MK_E_ARG, "NULL argument");
  if (c->device < 0) return fail(MK_E_UNSUPPORTED, "host-only context");
  const mk_config &f = c->cfg;
  if (!b->packed_weights || !b->scratch) return fail(MK_E_ARG, "packed_weights and scratch are required");
  if (((uintptr_t)b->packed_weights | (uintptr_t)b->scratch) & 255) return fail(MK_E_ARG, "buffers must be 256-byte aligned");
  for (int l = 0; l < f.n_layers; ++l) {
    const int m = f.mixer[l];
    if (m == MK_MIXER_GQA && (!b->k_cache[l] || !b->v_cache[l])) return fail(MK_E_ARG, "layer %d: K/V cache missing", l);
    if ((m == MK_MIXER_GDN || m == MK_MIXER_KDA) && !b->lin_state[l]) return fail(MK_E_ARG, "layer %d: state missing", l);
    if (m == MK_MIXER_MLA && (!b->latent[l] || ((uintptr_t)b->latent[l] & 15)))
      return fail(MK_E_ARG, "layer %d: latent cache missing or not 16-byte aligned", l);
  }
  HIP_TRY(hipSetDevice(c->device));
  c->bufs = *b;
  c->wbuf = static_cast<uint8_t *>(b->packed_weights);
  c->scratch = static_cast<uint8_t *>(b->scratch);
  c->loop_loaded = {0, 0};
  HIP_TRY(hipMemset(c->wbuf, 0, (size_t)c->packed_bytes));  // padding rows of fused matrices are zero
  HIP_TRY(hipMemset(c->scratch, 0, (size_t)c->scratch_bytes));
  // per-layer state pointers
  std::vector<void *> ptrs(5 * MK_MAX_LAYERS, nullptr);
  for (int l = 0; l < f.n_layers; ++l) {
    ptrs[4 * MK_MAX_LAYERS + l] = b->latent[l];
    ptrs[l] = b->k_cache[l];
    ptrs[MK_MAX_LAYERS + l] = b->v_cache[l];
    ptrs[2 * MK_MAX_LAYERS + l] = b->lin_state[l];
    if (c->lin_index[l] >= 0) ptrs[3 * MK_MAX_LAYERS + c->lin_index[l]] = b->lin_state[l];
  }
  HIP_TRY(hipMemcpy(c->scratch + c->o_ptrs, ptrs.data(), ptrs.size() * 8, hipMemcpyHostToDevice));
  // rotary table: angle p * theta^(-2i/d) in double, cosine and sine rounded to fp32
  if (f.n_q_heads > 0) {
    const int half = f.head_dim / 2;
    std::vector<float> rope((size_t)f.max_ctx * half * 2);
    for (int p = 0; p < f.max_ctx; ++p)
      for (int i = 0; i < half; ++i) {
        const double ang = (double)p * std::pow((double)f.rope_theta, -2.0 * i / (double)f.head_dim);
        rope[((size_t)p * half + i) * 2] = (float)std::cos(ang);
        rope[((size_t)p * half + i) * 2 + 1] = (float)std::sin(ang);
      }
    HIP_TRY(hipMemcpy(c->scratch + c->o_rope, rope.data(), rope.size() * 4, hipMemcpyHostToDevice));
  }
  // rotary table of the latent attention's rotary part (width rope_dim), same convention
  if (f.mla_heads > 0) {
    const int half = f.rope_dim / 2;
    std::vector<float> rope((size_t)f.max_ctx * half * 2);
    for (int p = 0; p < f.max_ctx; ++p)
      for (int i = 0; i < half; ++i) {
        const double ang = (double)p * std::pow((double)f.rope_theta, -2.0 * i / (double)f.rope_dim);
        rope[((size_t)p * half + i) * 2] = (float)std::cos(ang);
        rope[((size_t)p * half + i) * 2 + 1] = (float)std::sin(ang);
      }
    HIP_TRY(hipMemcpy(c->scratch + c->o_rope_mla, rope.data(), rope.size() * 4, hipMemcpyHostToDevice));
  }
  for (int r = 1; r <= kMaxBatch; ++r) {
    const Schedule &s = c->sched[r];
    if (s.phases.empty()) continue;
    HIP_TRY(hipMemcpy(c->scratch + c->o_phases[r], s.phases.data(), s.phases.size() * sizeof(Phase), hipMemcpyHostToDevice));
  }
  c->bar_done = 0;
  c->bound = true;
  c->global_have = 0;
  for (auto &s : c->L) {
    s.have = 0;
    std::fill(s.ex_have.begin(), s.ex_have.end(), 0);
  }
  return MK_OK;
}

mk_status mk_load_weights(mk_ctx *c, const mk_weight_desc *w, int n, void *stream) {
  if (!c || (!w && n > 0) || n < 0) return fail(MK_E_ARG, "bad arguments");
  if (c->device < 0) return fail(MK_E_UNSUPPORTED, "host-only context");
  if (!c->bound) return fail(MK_E_STATE, "buffers are not bound");
  hipStream_t st = static_cast<hipStream_t>(stream);
  // validate all first (a rejected call enqueues nothing)
  for (int i = 0; i < n; ++i) {
    Slot *slot;
    int64_t ro, rows, cols;
    uint32_t *have;
    Target tg;
    if (mk_status s = resolve(c, w[i], &slot, &ro, &rows, &cols, &have, &tg)) return s;
    const int want = tg.off >= 0 ? c->cfg.expert_format : MK_DT_BF16;
    if (w[i].dtype != want)
      return fail(MK_E_UNSUPPORTED, "tensor %d (layer %d kind %d): dtype %d, this configuration stores it as %d", i, w[i].layer,
                  w[i].kind, w[i].dtype, want);
    if (w[i].rows != rows || w[i].cols != cols)
      return fail(MK_E_SHAPE, "tensor %d (layer %d kind %d): shape %lldx%lld, expected %lldx%lld", i, w[i].layer, w[i].kind,
                  (long long)w[i].rows, (long long)w[i].cols, (long long)rows, (long long)cols);
    if (!w[i].data || ((uintptr_t)w[i].data & 15)) return fail(MK_E_ARG, "tensor %d: data must be 16-byte aligned", i);
    if (want == MK_DT_NVFP4) {
      if (!w[i].scales) return fail(MK_E_ARG, "tensor %d: NVFP4 scales are required", i);
      if (!(std::isfinite(w[i].tensor_scale))) return fail(MK_E_ARG, "tensor %d: tensor scale must be finite", i);
    }
    if (want == MK_DT_MXFP4 && (!w[i].scales || ((uintptr_t)w[i].scales & 3)))
      return fail(MK_E_ARG, "tensor %d: MXFP4 scales are required (4-byte aligned)", i);
  }
  HIP_TRY(hipSetDevice(c->device));
  // FP8 re-encodings count their inexact elements in a device word of the workspace's status block
  uint32_t *inexact = reinterpret_cast<uint32_t *>(c->scratch + c->o_status + 64);
  bool reencoded = false;
  std::vector<uint8_t *> reencoded_flags;
  for (int i = 0; i < n; ++i) {
    Slot *slot;
    int64_t ro, rows, cols;
    uint32_t *have;
    Target tg;
    resolve(c, w[i], &slot, &ro, &rows, &cols, &have, &tg);
    if (tg.off >= 0) {  // expert matrix
      if (tg.fmt == FMT_FP8R || tg.fmt == FMT_MXFP4) {
        if (tg.fmt == FMT_FP8R) {
          if (!reencoded) HIP_TRY(hipMemsetAsync(inexact, 0, 4, st));
          reencoded = true;
          const int64_t total = rows * (cols / 256);
          const int blocks = (int)std::min<int64_t>((total + 255) / 256, 65536);
          hipLaunchKernelGGL(mk_reencode_fp8, dim3(blocks), dim3(256), 0, st, static_cast<const uint8_t *>(w[i].data),
                             static_cast<const uint8_t *>(w[i].scales), rows, cols, c->wbuf + tg.off, ro, tg.mrows, inexact);
          reencoded_flags.push_back(tg.have_flag);
        } else {
          const int64_t total = (rows / 16) * (cols / 128) * 64;
          const int blocks = (int)std::min<int64_t>((total + 255) / 256, 65536);
          hipLaunchKernelGGL(mk_repack_mxfp4, dim3(blocks), dim3(256), 0, st, static_cast<const uint8_t *>(w[i].data),
                             static_cast<const uint8_t *>(w[i].scales), rows, cols, c->wbuf + tg.off, ro, tg.mrows);
        }
        HIP_TRY(hipGetLastError());
        hipLaunchKernelGGL(mk_store_f32, dim3(1), dim3(1), 0, st, reinterpret_cast<float *>(c->wbuf + tg.ts_off), 1.0f);
      } else if (tg.fmt == FMT_NVFP4) {
        const int64_t total = (rows / 16) * (cols / 128) * 64;
        const int blocks = (int)std::min<int64_t>((total + 255) / 256, 65536);
        hipLaunchKernelGGL(mk_repack_nvfp4, dim3(blocks), dim3(256), 0, st, static_cast<const uint8_t *>(w[i].data),
                           static_cast<const uint8_t *>(w[i].scales), rows, cols, c->wbuf + tg.off, ro, tg.mrows);
        HIP_TRY(hipGetLastError());
        hipLaunchKernelGGL(mk_store_f32, dim3(1), dim3(1), 0, st, reinterpret_cast<float *>(c->wbuf + tg.ts_off), w[i].tensor_scale);
      } else {
        const int64_t KF = cols / kFragK;
        const int64_t total = ((rows + 15) / 16) * KF * 64;
        const int blocks = (int)std::min<int64_t>((total + 255) / 256, 65536);
        hipLaunchKernelGGL(mk_repack_bf16, dim3(blocks), dim3(256), 0, st, static_cast<const uint16_t *>(w[i].data), rows, cols,
                           reinterpret_cast<uint4 *>(c->wbuf + tg.off), ro, KF);
        HIP_TRY(hipGetLastError());
        hipLaunchKernelGGL(mk_store_f32, dim3(1), dim3(1), 0, st, reinterpret_cast<float *>(c->wbuf + tg.ts_off), 1.0f);
      }
      HIP_TRY(hipGetLastError());
      *tg.have_flag = 1;
      continue;
    }
    if (w[i].kind == MK_W_UK) {
      const mk_config &f = c->cfg;
      const int64_t total = ((int64_t)f.mla_heads * f.kv_rank / 16) * (f.nope_dim / kFragK) * 64;
      const int blocks = (int)std::min<int64_t>((total + 255) / 256, 65536);
      hipLaunchKernelGGL(mk_repack_bf16_headT, dim3(blocks), dim3(256), 0, st, static_cast<const uint16_t *>(w[i].data),
                         (int64_t)f.mla_heads, (int64_t)f.nope_dim, (int64_t)f.kv_rank, reinterpret_cast<uint4 *>(c->wbuf + slot->off));
      HIP_TRY(hipGetLastError());
    } else if (!slot->packed) {
      HIP_TRY(hipMemcpyAsync(c->wbuf + slot->off, w[i].data, (size_t)rows * cols * 2, hipMemcpyDeviceToDevice, st));
    } else {
      const int64_t KF = cols / kFragK;
      const int64_t total = ((rows + 15) / 16) * KF * 64;
      const int blocks = (int)std::min<int64_t>((total + 255) / 256, 65536);
      hipLaunchKernelGGL(mk_repack_bf16, dim3(blocks), dim3(256), 0, st, static_cast<const uint16_t *>(w[i].data), rows, cols,
                         reinterpret_cast<uint4 *>(c->wbuf + slot->off), ro, KF);
      HIP_TRY(hipGetLastError());
    }
    *have |= kind_bit(w[i].kind);
  }
  if (reencoded) {  // the loader's bit-for-bit check of the FP8 re-encodings: wait for it, refuse on failure
    uint32_t bad = 0;
    HIP_TRY(hipMemcpyAsync(&bad, inexact, 4, hipMemcpyDeviceToHost, st));
    HIP_TRY(hipStreamSynchronize(st));
    if (bad) {
      for (uint8_t *flag : reencoded_flags) *flag = 0;  // those matrices count as not loaded
      return fail(MK_E_INEXACT, "FP8 re-encoding of MXFP4 gate/up weights is not lossless: %u elements have no exact "
                                "E4M3 value at their block's bf16 scale", bad);
    }
  }
  return MK_OK;
}

mk_status mk_decode_step(mk_ctx *c, const mk_step_io *io, int batch, void *stream) {
  if (!c) return fail(MK_E_ARG, "ctx is NULL");
  if (batch < 1 || batch > c->cfg.max_batch) return fail(MK_E_CAPACITY, "batch %d out of [1, %d]", batch, c->cfg.max_batch);
  if (mk_status s = check_step(c, io, batch, batch, 1)) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  HIP_TRY(hipSetDevice(c->device));
  if (c->needs_reset) { if (mk_status s = reset_counters(c, st)) return s; }
  StepArgs a;
  fill_args(c, a, batch, 0, io);
  c->bar_done += (uint32_t)a.n_barriers;
  return launch_step(c, a, st);
}

mk_status mk_decode_loop(mk_ctx *c, const mk_step_io *io, int batch, int n_steps, int32_t *d_tokens_out, void *stream) {
  if (!c) return fail(MK_E_ARG, "ctx is NULL");
  if (c->cfg.vocab <= 0) return fail(MK_E_UNSUPPORTED, "a decode loop samples tokens: it needs a vocabulary configuration");
  if (batch < 1 || batch > c->cfg.max_batch) return fail(MK_E_CAPACITY, "batch %d out of [1, %d]", batch, c->cfg.max_batch);
  if (n_steps < 1 || n_steps > MK_MAX_LOOP_STEPS) return fail(MK_E_CAPACITY, "n_steps %d out of [1, %d]", n_steps, MK_MAX_LOOP_STEPS);
  if (!d_tokens_out) return fail(MK_E_ARG, "tokens_out is required");
  if (mk_status s = check_step(c, io, batch, batch, n_steps)) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  HIP_TRY(hipSetDevice(c->device));
  if (c->needs_reset) { if (mk_status s = reset_counters(c, st)) return s; }
  const std::pair<int, int> key(batch, n_steps);
  auto it = c->loop_tables.find(key);
  if (it == c->loop_tables.end()) it = c->loop_tables.emplace(key, loop_table(c->sched[batch], n_steps)).first;
  if (c->loop_loaded != key) {  // ordered on the stream before this launch (and after earlier ones)
    HIP_TRY(hipMemcpyAsync(c->scratch + c->o_loop, it->second.data(), it->second.size() * sizeof(Phase),
                           hipMemcpyHostToDevice, st));
    c->loop_loaded = key;
  }
  StepArgs a;
  fill_args(c, a, batch, 0, io);
  a.phases = reinterpret_cast<const Phase *>(c->scratch + c->o_loop);
  a.n_phases = (int)it->second.size();
  a.n_barriers = a.n_phases - 1;
  a.phase_end = a.n_phases;
  a.loop_tokens = d_tokens_out;
  a.trace = nullptr;  // a trace buffer is sized for one step
  c->bar_done += (uint32_t)a.n_barriers;
  return launch_step(c, a, st);
}

mk_status mk_decode_step_noalloc(mk_ctx *c, const mk_step_io *io, int batch, void *stream) {
  if (!c) return fail(MK_E_ARG, "ctx is NULL");
  if (batch < 1 || batch > c->cfg.max_batch) return fail(MK_E_CAPACITY, "batch %d out of [1, %d]", batch, c->cfg.max_batch);
  if (mk_status s = check_step(c, io, batch, batch, 1)) return s;
  if (c->device >= kNoAllocDevices || !g_noalloc_ptr[c->device])
    return fail(MK_E_STATE, "device %d has no library working memory", c->device);
  const NoAllocLayout L = noalloc_layout(c, batch);
  if (L.total > kNoAllocBytes)
    return fail(MK_E_CAPACITY, "the step's working set at batch %d is %lld bytes; the library holds %lld per GPU", batch,
                (long long)L.total, (long long)kNoAllocBytes);
  hipStream_t st = static_cast<hipStream_t>(stream);
  HIP_TRY(hipSetDevice(c->device));
  if (c->needs_reset) { if (mk_status s = reset_counters(c, st)) return s; }
  uint8_t *base = g_noalloc_ptr[c->device];
  // the previous call on this GPU left its counters and partials here: start from zeros, and count
  // this call's barriers from zero
  const int64_t n16 = L.total / 16;
  hipLaunchKernelGGL(mk_zero16, dim3((unsigned)std::min<int64_t>(1024, (n16 + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<uint4 *>(base), n16);
  HIP_TRY(hipGetLastError());
  StepArgs a;
  fill_args(c, a, batch, 0, io);
  a.bar_done = 0;
  a.bar = reinterpret_cast<uint32_t *>(base + L.bar);
  a.fin = reinterpret_cast<uint32_t *>(base + L.fin);
  a.x = reinterpret_cast<float *>(base + L.x);
  a.ss = reinterpret_cast<float *>(base + L.ss);
  for (int i = 0; i < 3; ++i) a.part[i] = reinterpret_cast<float *>(base + L.part[i]);
  a.mix = reinterpret_cast<float *>(base + L.mix);
  a.attn = reinterpret_cast<float *>(base + L.attn);
  a.cand = reinterpret_cast<float *>(base + L.cand);
  for (int i = 0; i < 3; ++i) a.stg[i] = reinterpret_cast<uint16_t *>(base + L.stg[i]);
  return launch_step(c, a, st);
}

mk_status mk_verify_step(mk_ctx *c, const mk_step_io *io, int32_t *d_accepted, int32_t *d_bonus, void *stream) {
  if (!c) return fail(MK_E_ARG, "ctx is NULL");
  if (c->cfg.vocab <= 0) return fail(MK_E_UNSUPPORTED, "verify needs a vocabulary (logits) configuration");
  if (!d_accepted || !d_bonus) return fail(MK_E_ARG, "accepted and bonus outputs are required");
  if (mk_status s = check_step(c, io, kMaxRows, 1, kMaxRows)) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  HIP_TRY(hipSetDevice(c->device));
  if (c->needs_reset) { if (mk_status s = reset_counters(c, st)) return s; }
  StepArgs a;
  fill_args(c, a, kMaxRows, 1, io);
  c->bar_done += (uint32_t)a.n_barriers;
  a.accepted = d_accepted;
  a.bonus = d_bonus;
  return launch_step(c, a, st);
}

mk_status mk_decode_step_perop(mk_ctx *c, const mk_step_io *io, int batch, int use_graph, void *stream) {
  if (!c) return fail(MK_E_ARG, "ctx is NULL");
  if (batch < 1 || batch > c->cfg.max_batch) return fail(MK_E_CAPACITY, "batch %d out of [1, %d]", batch, c->cfg.max_batch);
  if (mk_status s = check_step(c, io, batch, batch, 1)) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  HIP_TRY(hipSetDevice(c->device));
  if (c->needs_reset) { if (mk_status s = reset_counters(c, st)) return s; }
  // one launch per phase: no grid barrier runs, so the barrier counters (and the count of completed
  // barriers their targets start from) stay as they are for the next persistent step
  StepArgs a;
  fill_args(c, a, batch, 0, io);
  a.bar_done = 0;  // unused by one-phase launches (they wait at no grid barrier); fixed, so graphs are reused
  const int n = a.n_phases;
  auto launch_all = [&](hipStream_t s) -> mk_status {
    for (int p = 0; p < n; ++p) {
      StepArgs ap = a;
      ap.phase_begin = p;
      ap.phase_end = p + 1;
      ap.barrier_base = p;
      void *args[] = {&ap};
      HIP_TRY(hipLaunchKernel(step_kernel(c, ap.R), dim3(c->G), dim3(kThreads), args, kLdsBytes, s));
    }
    return MK_OK;
  };
  if (!use_graph) return launch_all(st);
  // the same launches as one HIP graph: captured on the context's own stream (the caller's may be the
  // null stream, which cannot capture), instantiated once per row count and argument block, replayed
  // on the caller's stream
  if (!c->graph[batch] || memcmp(&c->graph_args[batch], &a, sizeof(StepArgs)) != 0) {
    if (c->graph[batch]) {
      HIP_TRY(hipGraphExecDestroy(c->graph[batch]));
      c->graph[batch] = nullptr;
    }
    if (!c->capture_stream) HIP_TRY(hipStreamCreateWithFlags(&c->capture_stream, hipStreamNonBlocking));
    HIP_TRY(hipStreamBeginCapture(c->capture_stream, hipStreamCaptureModeThreadLocal));
    mk_status s = launch_all(c->capture_stream);
    hipGraph_t g = nullptr;
    const hipError_t e = hipStreamEndCapture(c->capture_stream, &g);
    if (s != MK_OK) { if (g) (void)hipGraphDestroy(g); return s; }
    if (e != hipSuccess) return fail(MK_E_HIP, "graph capture: %s", hipGetErrorString(e));
    const hipError_t e2 = hipGraphInstantiate(&c->graph[batch], g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    if (e2 != hipSuccess) { c->graph[batch] = nullptr; return fail(MK_E_HIP, "graph instantiate: %s", hipGetErrorString(e2)); }
    c->graph_args[batch] = a;
  }
  HIP_TRY(hipGraphLaunch(c->graph[batch], st));
  return MK_OK;
}

mk_status mk_read_device_status(mk_ctx *c, int32_t *status, int32_t *phase) {
  if (!c || !status || !phase) return fail(MK_E_ARG, "NULL argument");
  if (c->device < 0 || !c->bound) return fail(MK_E_STATE, "no bound device context");
  int32_t s[3] = {0, 0, 0};
  HIP_TRY(hipSetDevice(c->device));
  HIP_TRY(hipMemcpy(s, c->scratch + c->o_status, sizeof(s), hipMemcpyDeviceToHost));
  *status = s[0];
  *phase = s[0] ? s[1] : -1;
  if (s[0] != 0) c->needs_reset = true;
  return MK_OK;
}

void mk_destroy(mk_ctx *c) {
  if (!c) return;
  for (auto &g : c->graph)
    if (g) (void)hipGraphExecDestroy(g);
  if (c->capture_stream) (void)hipStreamDestroy(c->capture_stream);
  delete c;
}

mk_status mk_set_launch_mode(mk_ctx *c, int cooperative) {
  if (!c) return fail(MK_E_ARG, "ctx is NULL");
  c->cooperative = cooperative != 0;
  return MK_OK;
}

mk_status mk_set_trace(mk_ctx *c, void *device_buffer, int64_t bytes) {
  if (!c) return fail(MK_E_ARG, "ctx is NULL");
  if (device_buffer) {
    int64_t need = 0;
    for (int r = 1; r <= kMaxBatch; ++r) need = std::max<int64_t>(need, (int64_t)c->sched[r].phases.size() * c->G * 16);
    if (bytes < need) return fail(MK_E_CAPACITY, "trace buffer %lld bytes < %lld", (long long)bytes, (long long)need);
    if ((uintptr_t)device_buffer & 7) return fail(MK_E_ARG, "trace buffer must be 8-byte aligned");
  }
  c->trace = static_cast<uint64_t *>(device_buffer);
  return MK_OK;
}

// Host-logic introspection for tests (no device needed): the phase table for a row count.
int mk_debug_phase_count(const mk_ctx *c, int rows) {
  if (!c || rows < 1 || rows > kMaxBatch) return -1;
  return (int)c->sched[rows].phases.size();
}

int mk_debug_phase(const mk_ctx *c, int rows, int i, int32_t *out16) {
  if (!c || rows < 1 || rows > kMaxBatch || i < 0 || i >= (int)c->sched[rows].phases.size() || !out16) return -1;
  const Phase &p = c->sched[rows].phases[(size_t)i];
  const int32_t v[16] = {p.type, p.layer, p.N, p.K, p.T, p.KF, p.S, p.nf, p.act, p.out, p.src_S, p.src_N, p.n_chunks, p.chunk,
                         p.dst_part, p.cnt_off};
  memcpy(out16, v, sizeof(v));
  return 0;
}

int mk_debug_phase_bytes(const mk_ctx *c, int rows, int i, void *out, int bytes) {
  if (!c || rows < 1 || rows > kMaxBatch || i < 0 || i >= (int)c->sched[rows].phases.size() || !out) return -1;
  if (bytes < (int)sizeof(Phase)) return (int)sizeof(Phase);
  memcpy(out, &c->sched[rows].phases[(size_t)i], sizeof(Phase));
  return (int)sizeof(Phase);
}

int64_t mk_debug_packed_bytes(const mk_ctx *c) { return c ? c->packed_bytes : -1; }

}  // extern "C"
