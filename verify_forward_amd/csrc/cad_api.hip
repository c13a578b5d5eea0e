// Host side of libcad: argument validation, workspace ownership and the
// launch sequence of the splice forward.  Every compute step is one of the
// HIP kernels in k_*.hip; this file only decides what runs, in which order,
// on which buffers.
//
// One splice forward (Copy-as-Decode §2.4; CopyLoop §2) enqueues:
//   embedding gather
//   per cache index (layer, or depth of a looped block):
//     RMSNorm -> QKV projection -> rotary + KV append -> span attention
//     -> O projection (+residual) -> RMSNorm -> gate/up projection (SwiGLU)
//     -> down projection (+residual)
//   final RMSNorm -> LM head (masked-argmax candidates in its epilogue; fp32
//   logits only when the caller asks) -> decision (argmax + acceptance)
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "cad_internal.h"

using namespace cad;

namespace {

thread_local std::string g_err;

cad_status fail(cad_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
cad_status fail(cad_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  try {
    g_err = buf;
  } catch (...) {  // no room for the message: the status still reports the failure
  }
  return s;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define HIP_TRY(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess) return fail(CAD_E_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

}  // namespace

enum ProfFamily {
  PF_EMBED, PF_NORM, PF_QKV, PF_ROPE, PF_ATTN, PF_MERGE, PF_O, PF_GATEUP, PF_DOWN, PF_HEAD,
  PF_DECIDE, PF_LOOP_STATE, PF_COUNT
};
static const char* const kProfNames[PF_COUNT] = {
    "embed", "rmsnorm", "gemm_qkv", "rope_append", "attention", "attn_merge", "gemm_o",
    "gemm_gate_up", "gemm_down", "gemm_lm_head", "decide", "loop_state"};

struct ProfRec {
  int family;
  hipEvent_t a, b;
};

// Per-call device buffers of the splice path (activations, partial sums,
// attention partials, candidates), carved from one block of device memory:
// the model's workspace (allocated at create, sized for max_tokens rows and
// CAD_MAX_SEQS sequences) or, for cad_decode_step_noalloc, the library's
// static scratch array (one row, one sequence).
struct Workspace {
  int64_t rows = 0;          // row capacity T (plane stride of the two-plane buffers)
  float* x = nullptr;        // [T][d] residual stream
  // activations feeding a projection: fp32 [T][n] (fp32 models) or two bf16
  // planes [T][n] each, hi then lo (bf16 models), in the same bytes
  void* hn = nullptr;        // [T][d] normalised activations
  float* qkv = nullptr;      // [T][(hq+2hkv) hd]
  void* q = nullptr;         // [T][hq][hd] rotated queries
  void* attn = nullptr;      // [T][hq hd] attention output
  void* act = nullptr;       // [T][F] SwiGLU activation
  uint32_t* cand = nullptr;  // [max_candidates(V)][T] masked-argmax candidates of the LM head
  float* part_o = nullptr;   // attention partials
  float* part_ml = nullptr;
  int64_t part_cap = 0;      // rows x partitions the partials hold
  int32_t* survivors = nullptr;  // [1] acceptance output when the caller passes none
  f16_t* span_k = nullptr;       // this call's span K/V at half precision (bf16 models)
  f16_t* span_v = nullptr;
  int32_t span_cap = 0;          // rows of the span workspace
  float* split_ws = nullptr;     // split-K partial sums of the projections (bf16 models)
  int64_t split_cap = 0;         // floats in split_ws
  float* norm_ss = nullptr;      // [16][d / 256] slice sums of squares (bf16 models, few rows)
};

struct cad_model {
  cad_config cfg;
  // instrumentation
  uint32_t prof_mask = 0;  // families whose launches are bracketed by events
  std::vector<ProfRec> prof;
  std::vector<hipEvent_t> prof_pool;
  size_t prof_used = 0;
  int esize;  // bytes per weight / cache element
  // weights (caller-owned)
  const void* tok_embed;
  const void* final_norm;
  const void* lm_head;
  std::vector<const void*> attn_norm, w_qkv, w_o, ffn_norm, w_gate_up, w_down;
  // device memory owned by the model (one allocation): the workspace and
  // the rotary frequencies
  void* ws = nullptr;
  size_t ws_bytes = 0;
  Workspace main;
  Workspace* w = &main;      // the workspace the current call runs on
  double* freq = nullptr;    // [hd/2] rotary frequencies
  int x_parts = 0;           // partial planes in split_ws still to be added to x
};

namespace {

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

hipEvent_t prof_event(cad_model* m) {
  if (m->prof_used == m->prof_pool.size()) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    m->prof_pool.push_back(e);
  }
  return m->prof_pool[m->prof_used++];
}

// Launch `fn` (returning hipError_t), bracketed by events when profiling.
template <typename Fn>
hipError_t prof_launch(cad_model* m, int family, hipStream_t s, Fn fn) {
  if (!(m->prof_mask >> family & 1u)) return fn();
  ProfRec r{family, prof_event(m), prof_event(m)};
  if (r.a && r.b) (void)hipEventRecord(r.a, s);
  hipError_t e = fn();
  if (r.a && r.b) {
    (void)hipEventRecord(r.b, s);
    m->prof.push_back(r);
  }
  return e;
}

#define LAUNCH(fam, expr) HIP_TRY(prof_launch(m, fam, s, [&]() { return (expr); }))

cad_status check_config(const cad_config* c) {
  if (!c) return fail(CAD_E_ARG, "cfg is NULL");
  if (c->n_layers < 1 || c->d_model < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 ||
      c->head_dim < 2 || c->ffn_dim < 1 || c->vocab < 1 || c->loop_depth < 1 || c->max_tokens < 1)
    return fail(CAD_E_ARG, "non-positive dimension in cfg");
  if (c->dtype != CAD_F32 && c->dtype != CAD_BF16) return fail(CAD_E_ARG, "bad dtype %d", c->dtype);
  if (c->n_q_heads % c->n_kv_heads) return fail(CAD_E_ARG, "n_q_heads not a multiple of n_kv_heads");
  if (c->loop_depth > 1 && c->n_layers != 1) return fail(CAD_E_ARG, "looped model needs n_layers == 1");
  if (!(c->rope_theta > 0.f) || !(c->rms_eps >= 0.f)) return fail(CAD_E_ARG, "bad rope_theta or rms_eps");
  if (c->head_dim % 2) return fail(CAD_E_UNSUPPORTED, "odd head_dim");
  if (c->d_model % 4 || c->d_model > 8192) return fail(CAD_E_UNSUPPORTED, "d_model must be a multiple of 4, at most 8192");
  if (c->dtype == CAD_F32) {
    if (c->head_dim > 128) return fail(CAD_E_UNSUPPORTED, "fp32 path supports head_dim <= 128");
  } else {
    if (c->head_dim != 64 && c->head_dim != 128)
      return fail(CAD_E_UNSUPPORTED, "bf16 path supports head_dim 64 or 128");
    if (c->d_model % 64 || c->ffn_dim % 64 || (c->n_q_heads * c->head_dim) % 64)
      return fail(CAD_E_UNSUPPORTED, "bf16 path needs d_model, ffn_dim, n_q_heads*head_dim multiples of 64");
  }
  // the rotary kernel stages one row's projection output (every q, k and v
  // head, fp32) in LDS when it takes a whole row per work-group
  if ((int64_t)(c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim * 4 > 65536)
    return fail(CAD_E_UNSUPPORTED, "(n_q_heads + 2 n_kv_heads) * head_dim = %d exceeds 16384",
                (c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim);
  if (c->max_tokens > (1 << 20)) return fail(CAD_E_CAPACITY, "max_tokens too large");
  return CAD_OK;
}

int64_t max_parts_rows(const cad_config& c, int64_t T) {
  // largest n_parts * rows over every row count a call may carry
  int64_t best = 0;
  for (int r = 1; r <= T; ++r) {
    // both tile shapes: one sequence, and r one-row sequences
    const int p1 = attention_parts(r, 1, c.n_q_heads, c.n_kv_heads, (int64_t)1 << 40, r);
    const int p2 = attention_parts(r, r, c.n_q_heads, c.n_kv_heads, (int64_t)1 << 40, 1);
    const int p = p1 > p2 ? p1 : p2;
    if ((int64_t)p * r > best) best = (int64_t)p * r;
  }
  return best;
}

cad_status check_kv(const cad_model* m, const cad_kv* kv) {
  if (!kv) return fail(CAD_E_ARG, "kv is NULL");
  if (!kv->k || !kv->v || !kv->block_table) return fail(CAD_E_ARG, "kv buffers are NULL");
  if (kv->num_blocks < 1 || kv->max_blocks_per_seq < 1) return fail(CAD_E_ARG, "empty kv pool");
  if (m->cfg.dtype == CAD_BF16 && (!aligned16(kv->k) || !aligned16(kv->v)))
    return fail(CAD_E_ARG, "kv pools must be 16-byte aligned");
  return CAD_OK;
}

KVView view_of(const cad_model* m, const cad_kv* kv, int ci) {
  const cad_config& c = m->cfg;
  const int64_t per = kv->num_blocks * c.n_kv_heads * CAD_KV_BLOCK * c.head_dim * m->esize;
  KVView v;
  v.k = (char*)kv->k + per * ci;
  v.v = (char*)kv->v + per * ci;
  v.table = kv->block_table;
  v.num_blocks = kv->num_blocks;
  v.max_blocks = kv->max_blocks_per_seq;
  v.cache_stride = kv->num_blocks * c.n_kv_heads * CAD_KV_BLOCK * c.head_dim;
  v.span_k = m->w->span_k;
  v.span_v = m->w->span_v;
  v.span_cap = m->w->span_cap;
  return v;
}

// lo plane of an activation buffer (bf16 models): after the T x n hi plane
void* lo_plane(const cad_model* m, void* buf, int64_t n) {
  return m->cfg.dtype == CAD_BF16 ? (void*)((bf16_t*)buf + m->w->rows * n) : nullptr;
}

// half remainder plane of q (bf16 models): after the T x hq x hd hi plane
void* q_lo_plane(const cad_model* m) {
  const cad_config& c = m->cfg;
  return c.dtype == CAD_BF16 ? (void*)((f16_t*)m->w->q + m->w->rows * c.n_q_heads * c.head_dim) : nullptr;
}

// Lay out a workspace for T rows of at most `seqs` sequences with
// `split_floats` floats of split-K partial sums, from `base` (nullptr: only
// size it).  Returns the bytes it takes.
size_t layout_workspace(const cad_config& c, int64_t T, int64_t seqs, int64_t split_floats, char* base,
                        Workspace* w) {
  const int64_t d = c.d_model, hq = c.n_q_heads, hkv = c.n_kv_heads, hd = c.head_dim, F = c.ffn_dim, V = c.vocab;
  const bool bf = c.dtype == CAD_BF16;
  const int64_t es = bf ? 2 : 4;
  const int64_t pr = max_parts_rows(c, T);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  const size_t o_x = take(T * d * 4), o_hn = take(T * d * 4), o_qkv = take(T * (hq + 2 * hkv) * hd * 4),
               o_q = take(T * hq * hd * es * (bf ? 2 : 1)), o_attn = take(T * hq * hd * 4), o_act = take(T * F * 4),
               o_cand = take((size_t)max_candidates((int)V) * T * 8), o_po = take(pr * hq * hd * 4),
               o_pml = take(pr * hq * 2 * 4), o_sv = take(4);
  // each sequence's span rows padded to 64 in the span K/V workspace
  const int64_t span_cap = bf ? (T + 64 * seqs + 63) / 64 * 64 : 0;
  const size_t o_spk = take((size_t)span_cap * hkv * hd * 2), o_spv = take((size_t)span_cap * hkv * hd * 2);
  const size_t o_sws = take(bf ? (size_t)split_floats * 4 : 0);
  const size_t o_nss = take(bf ? (size_t)16 * rms_slices((int)d) * 4 : 0);
  if (base) {
    *w = Workspace{};
    w->rows = T;
    w->x = (float*)(base + o_x);
    w->hn = base + o_hn;
    w->qkv = (float*)(base + o_qkv);
    w->q = base + o_q;
    w->attn = base + o_attn;
    w->act = base + o_act;
    w->cand = (uint32_t*)(base + o_cand);
    w->part_o = (float*)(base + o_po);
    w->part_ml = (float*)(base + o_pml);
    w->part_cap = pr;
    w->survivors = (int32_t*)(base + o_sv);
    if (bf) {
      w->span_k = (f16_t*)(base + o_spk);
      w->span_v = (f16_t*)(base + o_spv);
      w->span_cap = (int32_t)span_cap;
      w->split_ws = (float*)(base + o_sws);
      w->split_cap = split_floats;
      w->norm_ss = (float*)(base + o_nss);
    }
  }
  return off;
}

// RMSNorm (with gain `gain`) of the R rows of the residual stream, after
// adding the pending k-split partials, as the activation operand of the
// projection described by g.  A bf16 model with at most
// NORM_IN_PROJ_MAX_ROWS rows leaves the normalisation to the
// weight-streaming projection (launch_rms_slices writes the slice sums of
// squares; g carries the residual and the gain): every work-group of the
// projection then normalises the rows it stages, which beats the one-row-
// per-work-group norm kernel for a few rows (N = 1: 2.2 us saved per norm,
// the projections about even) but not at 16 (each of the 448 gate/up
// work-groups repeats the work for 16 rows).  Otherwise the full kernel
// writes the hi/lo planes.
constexpr int NORM_IN_PROJ_MAX_ROWS = 8;
hipError_t launch_norm(cad_model* m, const void* gain, int R, GemmArgs& g, hipStream_t s) {
  const cad_config& c = m->cfg;
  const int np = m->x_parts;
  m->x_parts = 0;
  g.lda = c.d_model;
  if (c.dtype == CAD_BF16 && R <= NORM_IN_PROJ_MAX_ROWS && aligned16(gain)) {
    g.A = m->w->x;
    g.A_lo = nullptr;
    g.norm_g = gain;
    g.norm_ss = m->w->norm_ss;
    g.norm_slices = rms_slices(c.d_model);
    g.norm_eps = c.rms_eps;
    return launch_rms_slices(m->w->x, m->w->split_ws, np, R, c.d_model, m->w->norm_ss, s);
  }
  g.A = m->w->hn;
  g.A_lo = lo_plane(m, m->w->hn, c.d_model);
  return launch_rmsnorm(c.dtype, m->w->x, m->w->split_ws, np, gain, R, c.d_model, c.rms_eps, m->w->hn,
                        lo_plane(m, m->w->hn, c.d_model), s);
}

// Run cache indices [c0, c1) over the rows already embedded in m->w->x.
cad_status run_blocks(cad_model* m, const cad_kv* kv, const RowMap& rm, int c0, int c1,
                      const int32_t* write_limit, int32_t* dev_status, hipStream_t s) {
  const cad_config& c = m->cfg;
  const int R = rm.total;
  const int d = c.d_model, hq = c.n_q_heads, hkv = c.n_kv_heads, hd = c.head_dim, F = c.ffn_dim;
  const int qkv_rows = (hq + 2 * hkv) * hd;
  int64_t max_L = 0;
  int max_rows = 0;
  for (int b = 0; b < rm.n_seq; ++b) {
    max_L = rm.L[b] > max_L ? rm.L[b] : max_L;
    max_rows = rm.start[b + 1] - rm.start[b] > max_rows ? rm.start[b + 1] - rm.start[b] : max_rows;
  }
  // partitions of each query tile's key axis (cached keys, then the span's own)
  const int n_parts = attention_parts(R, rm.n_seq, hq, hkv, max_L, max_rows);
  if ((int64_t)n_parts * R > m->w->part_cap)
    return fail(CAD_E_CAPACITY, "attention partitions %d x %d rows exceed the workspace", n_parts, R);
  if (c.dtype == CAD_BF16 && rm.pstart[rm.n_seq] > m->w->span_cap)
    return fail(CAD_E_CAPACITY, "span workspace too small for %d padded rows", rm.pstart[rm.n_seq]);
  for (int ci = c0; ci < c1; ++ci) {
    const int li = c.loop_depth > 1 ? 0 : ci;
    const KVView v = view_of(m, kv, ci);
    GemmArgs g{};
    LAUNCH(PF_NORM, launch_norm(m, m->attn_norm[li], R, g, s));
    g.W = m->w_qkv[li]; g.ldw = d;
    g.M = R; g.N = qkv_rows; g.K = d; g.out_f32 = m->w->qkv; g.ldo = qkv_rows;
    g.split_ws = m->w->split_ws; g.split_cap = m->w->split_cap;
    int qkv_parts = 0;
    LAUNCH(PF_QKV, launch_gemm(c.dtype, GEMM_QKV, g, s, &qkv_parts));
    LAUNCH(PF_ROPE, launch_rope_append(c.dtype, m->w->qkv, m->w->split_ws, qkv_parts, R, hq, hkv, hd, m->freq, rm, v,
                                       write_limit, m->w->q, q_lo_plane(m), dev_status, s));
    LAUNCH(PF_ATTN, launch_attention(c.dtype, m->w->q, q_lo_plane(m), R, hq, hkv, hd, rm, v, n_parts, m->w->part_o,
                                     m->w->part_ml, m->w->attn, lo_plane(m, m->w->attn, (int64_t)hq * hd), dev_status, s));
    if (c.dtype == CAD_BF16 && n_parts > 1)
      LAUNCH(PF_MERGE, launch_attention_merge(m->w->part_o, m->w->part_ml, n_parts, R, hq, hd, m->w->attn,
                                              lo_plane(m, m->w->attn, (int64_t)hq * hd), s));
    g = GemmArgs{};
    g.A = m->w->attn; g.A_lo = lo_plane(m, m->w->attn, (int64_t)hq * hd); g.lda = hq * hd;
    g.W = m->w_o[li]; g.ldw = hq * hd;
    g.M = R; g.N = d; g.K = hq * hd; g.out_f32 = m->w->x; g.ldo = d;
    g.split_ws = m->w->split_ws; g.split_cap = m->w->split_cap;
    LAUNCH(PF_O, launch_gemm(c.dtype, GEMM_O, g, s, &m->x_parts));
    g = GemmArgs{};
    LAUNCH(PF_NORM, launch_norm(m, m->ffn_norm[li], R, g, s));
    g.W = m->w_gate_up[li]; g.ldw = d;
    // more than 16 rows (tiled projections): the SwiGLU activation goes to
    // the down projection as one half plane (its input is the one whose
    // rounding the logits tolerate best: 7B, N = 512, 9.4e-3 -> 1.3e-2
    // against 2e-2), which halves that projection's matrix-core work and
    // activation reads; the weight-streaming path keeps the two bf16 planes
    const int act_f16 = c.dtype == CAD_BF16 && R > 16;
    g.M = R; g.N = F; g.K = d; g.up_off = F; g.out_act = m->w->act;
    g.out_act_lo = act_f16 ? nullptr : lo_plane(m, m->w->act, F);
    g.act_f16 = act_f16;
    g.status = dev_status;
    g.split_ws = m->w->split_ws; g.split_cap = m->w->split_cap;
    LAUNCH(PF_GATEUP, launch_gemm(c.dtype, GEMM_GATE_UP, g, s));
    g = GemmArgs{};
    g.A = m->w->act; g.A_lo = act_f16 ? nullptr : lo_plane(m, m->w->act, F); g.lda = F; g.W = m->w_down[li]; g.ldw = F;
    g.act_f16 = act_f16;
    g.M = R; g.N = d; g.K = F; g.out_f32 = m->w->x; g.ldo = d;
    g.split_ws = m->w->split_ws; g.split_cap = m->w->split_cap;
    LAUNCH(PF_DOWN, launch_gemm(c.dtype, GEMM_DOWN, g, s, &m->x_parts));
  }
  return CAD_OK;
}

// final norm + LM head (masked-argmax candidates; fp32 logits only if
// `logits` is set) + the decision step: every row's argmax and the
// acceptance of every sequence (rows at or beyond *limit, when given, get
// argmax -1 and are not examined)
cad_status readout(cad_model* m, const RowMap& rm, float* logits, const uint32_t* mask, const int32_t* span,
                   int mode, const int32_t* limit, int32_t* argmax, int32_t* accepted, int32_t* dev_status,
                   hipStream_t s) {
  const cad_config& c = m->cfg;
  const int R = rm.total;
  GemmArgs g{};
  LAUNCH(PF_NORM, launch_norm(m, m->final_norm, R, g, s));
  g.W = m->lm_head; g.ldw = c.d_model;
  g.M = R; g.N = c.vocab; g.K = c.d_model; g.out_f32 = logits; g.ldo = c.vocab;
  g.split_ws = m->w->split_ws; g.split_cap = m->w->split_cap;
  g.mask = mask;
  g.mask_words = (c.vocab + 31) / 32;
  g.cand = m->w->cand;
  int n_cand = 0;
  g.n_cand = &n_cand;
  LAUNCH(PF_HEAD, launch_gemm(c.dtype, GEMM_LM_HEAD, g, s));
  LAUNCH(PF_DECIDE, launch_decide(m->w->cand, n_cand, R, rm, span, mode, limit, argmax, accepted, dev_status, s));
  return CAD_OK;
}

cad_status check_common(cad_model* m, const cad_kv* kv, const int32_t* span, const int32_t* argmax,
                        const int32_t* accepted, const float* logits, int mode) {
  if (!m) return fail(CAD_E_ARG, "model is NULL");
  cad_status st = check_kv(m, kv);
  if (st != CAD_OK) return st;
  if (!span) return fail(CAD_E_ARG, "span is NULL");
  if (!argmax || !accepted) return fail(CAD_E_ARG, "argmax/accepted is NULL");
  if (mode != CAD_COMMIT && mode != CAD_VERIFY) return fail(CAD_E_ARG, "bad mode %d", mode);
  if (logits && !aligned16(logits)) return fail(CAD_E_ARG, "logits must be 16-byte aligned");
  return CAD_OK;
}

cad_status check_seq(const cad_kv* kv, int64_t L, int64_t N, int max_tokens) {
  if (N < 1) return fail(CAD_E_ARG, "span length %lld < 1", (long long)N);
  if (N > max_tokens) return fail(CAD_E_CAPACITY, "span length %lld > max_tokens %d", (long long)N, max_tokens);
  if (L < 0) return fail(CAD_E_ARG, "negative cache length");
  if (L + N > (int64_t)kv->max_blocks_per_seq * CAD_KV_BLOCK)
    return fail(CAD_E_CAPACITY, "L + N = %lld exceeds the block table (%d blocks of %d)",
                (long long)(L + N), kv->max_blocks_per_seq, CAD_KV_BLOCK);
  return CAD_OK;
}

// ---------------------------------------------------------------------------
// Static scratch for cad_decode_step_noalloc: the one-row workspace of a
// decode step lives here, so that call allocates nothing.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory: its device
// address is resolved per device with hipGetSymbolAddress and only that
// address is passed to kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[CAD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device (nullptr until resolved)

// The device address of `scratch` on the current device, resolved once per
// device (with that device current) and kept.
cad_status scratch_of_current_device(void** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(CAD_E_UNSUPPORTED, "device %d beyond the scratch table", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(CAD_E_HIP, "hipGetSymbolAddress returned no address for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CAD_OK;
}

// Split-K partial floats a one-row call needs: the weight-streaming
// projections that leave partial sums (QKV, O, down) split K into at most one
// piece per 512 k.  With this capacity a one-row call takes the same splits
// as on the model's own workspace.
int64_t one_row_split_floats(const cad_config& c) {
  if (c.dtype != CAD_BF16) return 0;
  auto f = [](int64_t K, int64_t N) { return (K + 511) / 512 * N; };
  const int64_t qkv = (int64_t)(c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  int64_t best = f(c.d_model, qkv);
  best = std::max(best, f((int64_t)c.n_q_heads * c.head_dim, c.d_model));
  best = std::max(best, f(c.ffn_dim, c.d_model));
  return best;
}

}  // namespace

namespace cad {
cad_status set_error(cad_status s, const char* msg) {
  try {
    g_err = msg;
  } catch (...) {  // no room for the message: the status still reports the failure
  }
  return s;
}

cad_status splice_rows(cad_model* m, const cad_kv* kv, int64_t L, const int32_t* span, int N, const uint32_t* mask,
                       int mode, const int32_t* limit, int32_t* argmax, int32_t* accepted, float* logits,
                       int32_t* dev_status, hipStream_t s) {
  cad_status st = check_common(m, kv, span, argmax, accepted, logits, mode);
  if (st != CAD_OK) return st;
  if (m->cfg.loop_depth > 1) return fail(CAD_E_ARG, "looped model: use cad_splice_forward_looped");
  st = check_seq(kv, L, N, m->cfg.max_tokens);
  if (st != CAD_OK) return st;
  RowMap rm{};
  rm.n_seq = 1;
  rm.total = N;
  rm.start[0] = 0;
  rm.start[1] = N;
  rm.L[0] = L;
  rowmap_pad(rm);
  const cad_config& c = m->cfg;
  m->x_parts = 0;
  LAUNCH(PF_EMBED, launch_embed(c.dtype, m->tok_embed, c.vocab, c.d_model, span, N, m->w->x, dev_status, s));
  st = run_blocks(m, kv, rm, 0, c.n_layers, limit, dev_status, s);
  if (st != CAD_OK) return st;
  return readout(m, rm, logits, mask, span, mode, limit, argmax, accepted, dev_status, s);
}
}  // namespace cad

const cad_config* cad_model_config(const cad_model* m) { return &m->cfg; }

extern "C" {

const char* cad_last_error(void) { return g_err.c_str(); }

cad_status cad_model_create(const cad_config* cfg, const cad_weights* w, cad_model** out) try {
  if (!out) return fail(CAD_E_ARG, "out is NULL");
  *out = nullptr;
  cad_status st = check_config(cfg);
  if (st != CAD_OK) return st;
  if (!w || !w->tok_embed || !w->final_norm || !w->lm_head || !w->attn_norm || !w->w_qkv || !w->w_o ||
      !w->ffn_norm || !w->w_gate_up || !w->w_down)
    return fail(CAD_E_ARG, "weights incomplete");
  const cad_config& c = *cfg;
  const bool need_align = c.dtype == CAD_BF16;
  auto ok_ptr = [&](const void* p) { return p && (!need_align || aligned16(p)); };
  if (!ok_ptr(w->tok_embed) || !ok_ptr(w->lm_head)) return fail(CAD_E_ARG, "embedding/head pointer NULL or misaligned");
  for (int i = 0; i < c.n_layers; ++i)
    if (!w->attn_norm[i] || !w->ffn_norm[i] || !ok_ptr(w->w_qkv[i]) || !ok_ptr(w->w_o[i]) ||
        !ok_ptr(w->w_gate_up[i]) || !ok_ptr(w->w_down[i]))
      return fail(CAD_E_ARG, "layer %d weight pointer NULL or misaligned", i);

  // rotary frequencies theta^(-2i / hd), uploaded with the workspace
  const int64_t hd = c.head_dim;
  std::vector<double> fr(hd / 2);
  for (int64_t i = 0; i < hd / 2; ++i) fr[i] = std::pow((double)c.rope_theta, -2.0 * (double)i / (double)hd);

  cad_model* m = new (std::nothrow) cad_model();
  if (!m) return fail(CAD_E_HIP, "host allocation failed");
  m->cfg = c;
  m->esize = c.dtype == CAD_BF16 ? 2 : 4;
  m->tok_embed = w->tok_embed;
  m->final_norm = w->final_norm;
  m->lm_head = w->lm_head;
  try {
    m->attn_norm.assign(w->attn_norm, w->attn_norm + c.n_layers);
    m->w_qkv.assign(w->w_qkv, w->w_qkv + c.n_layers);
    m->w_o.assign(w->w_o, w->w_o + c.n_layers);
    m->ffn_norm.assign(w->ffn_norm, w->ffn_norm + c.n_layers);
    m->w_gate_up.assign(w->w_gate_up, w->w_gate_up + c.n_layers);
    m->w_down.assign(w->w_down, w->w_down + c.n_layers);
  } catch (...) {
    delete m;
    throw;
  }
  const int64_t split_floats = c.dtype == CAD_BF16 ? GEMM_SPLIT_FLOATS : 0;
  const size_t o_freq = layout_workspace(c, c.max_tokens, CAD_MAX_SEQS, split_floats, nullptr, nullptr);
  const size_t bytes = o_freq + align_up(hd / 2 * 8);
  hipError_t e = hipMalloc(&m->ws, bytes);
  if (e != hipSuccess) {
    delete m;
    return fail(CAD_E_HIP, "hipMalloc(%zu): %s", bytes, hipGetErrorString(e));
  }
  m->ws_bytes = bytes;
  layout_workspace(c, c.max_tokens, CAD_MAX_SEQS, split_floats, (char*)m->ws, &m->main);
  // set-up of the allocation-free decode step: the scratch address of this device
  void* scratch_dev = nullptr;
  st = scratch_of_current_device(&scratch_dev);
  if (st != CAD_OK) {
    (void)hipFree(m->ws);
    delete m;
    return st;
  }
  m->freq = (double*)((char*)m->ws + o_freq);
  e = hipMemcpy(m->freq, fr.data(), fr.size() * 8, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    (void)hipFree(m->ws);
    delete m;
    return fail(CAD_E_HIP, "workspace init: %s", hipGetErrorString(e));
  }
  *out = m;
  return CAD_OK;
} catch (...) {
  // host containers and messages are C++: nothing they throw crosses the C ABI
  return cad::set_error(CAD_E_HIP, "host allocation failed");
}

void cad_model_destroy(cad_model* m) {
  if (!m) return;
  (void)hipDeviceSynchronize();
  for (hipEvent_t e : m->prof_pool) (void)hipEventDestroy(e);
  (void)hipFree(m->ws);
  delete m;
}

cad_status cad_splice_forward(cad_model* m, const cad_kv* kv, int64_t L, const int32_t* span,
                              int32_t N, const uint32_t* mask, cad_mode mode, int32_t* argmax,
                              int32_t* accepted, float* logits, int32_t* dev_status,
                              cad_stream stream) try {
  return cad::splice_rows(m, kv, L, span, N, mask, mode, nullptr, argmax, accepted, logits, dev_status,
                          (hipStream_t)stream);
} catch (...) {
  // host containers and messages are C++: nothing they throw crosses the C ABI
  return cad::set_error(CAD_E_HIP, "host allocation failed");
}

cad_status cad_decode_step(cad_model* m, const cad_kv* kv, int64_t L, const int32_t* token,
                           const uint32_t* mask_row, int32_t* argmax, float* logits,
                           int32_t* dev_status, cad_stream stream) try {
  if (!m) return fail(CAD_E_ARG, "model is NULL");
  return cad_splice_forward(m, kv, L, token, 1, mask_row, CAD_COMMIT, argmax, m->w->survivors, logits,
                            dev_status, stream);
} catch (...) {
  // host containers and messages are C++: nothing they throw crosses the C ABI
  return cad::set_error(CAD_E_HIP, "host allocation failed");
}

cad_status cad_decode_step_noalloc(cad_model* m, const cad_kv* kv, int64_t L, const int32_t* token,
                                   const uint32_t* mask_row, int32_t* argmax, float* logits, int32_t* dev_status,
                                   cad_stream stream) try {
  if (!m) return fail(CAD_E_ARG, "model is NULL");
  void* base = nullptr;
  cad_status st = scratch_of_current_device(&base);
  if (st != CAD_OK) return st;
  const int64_t split_floats = one_row_split_floats(m->cfg);
  const size_t need = layout_workspace(m->cfg, 1, 1, split_floats, nullptr, nullptr);
  if (need > (size_t)CAD_NOALLOC_SCRATCH_BYTES)
    return fail(CAD_E_CAPACITY, "a decode step of this model needs %zu bytes of scratch; the maximum is %d", need,
                CAD_NOALLOC_SCRATCH_BYTES);
  Workspace ws;
  layout_workspace(m->cfg, 1, 1, split_floats, (char*)base, &ws);
  // run on the scratch workspace, with no instrumentation (recording would
  // create events)
  const uint32_t prof = m->prof_mask;
  m->prof_mask = 0;
  m->w = &ws;
  st = cad_splice_forward(m, kv, L, token, 1, mask_row, CAD_COMMIT, argmax, ws.survivors, logits, dev_status,
                          stream);
  m->w = &m->main;
  m->prof_mask = prof;
  return st;
} catch (...) {
  // host containers and messages are C++: nothing they throw crosses the C ABI
  return cad::set_error(CAD_E_HIP, "host allocation failed");
}

cad_status cad_splice_forward_batched(cad_model* m, const cad_kv* kv, int32_t n_seq,
                                      const int64_t* seq_L, const int32_t* offsets,
                                      const int32_t* spans, const uint32_t* mask, cad_mode mode,
                                      int32_t* argmax, int32_t* accepted, float* logits,
                                      int32_t* dev_status, cad_stream stream) try {
  cad_status st = check_common(m, kv, spans, argmax, accepted, logits, mode);
  if (st != CAD_OK) return st;
  if (m->cfg.loop_depth > 1) return fail(CAD_E_ARG, "looped model: use cad_splice_forward_looped");
  if (n_seq < 1 || n_seq > CAD_MAX_SEQS) return fail(CAD_E_ARG, "n_seq %d outside [1, %d]", n_seq, CAD_MAX_SEQS);
  if (!seq_L || !offsets) return fail(CAD_E_ARG, "seq_L/offsets is NULL");
  if (offsets[0] != 0) return fail(CAD_E_ARG, "offsets[0] must be 0");
  RowMap rm{};
  rm.n_seq = n_seq;
  for (int b = 0; b < n_seq; ++b) {
    const int64_t n = (int64_t)offsets[b + 1] - offsets[b];
    if (n < 1) return fail(CAD_E_ARG, "sequence %d has no span rows", b);
    st = check_seq(kv, seq_L[b], n, m->cfg.max_tokens);
    if (st != CAD_OK) return st;
    rm.start[b] = offsets[b];
    rm.L[b] = seq_L[b];
  }
  rm.start[n_seq] = offsets[n_seq];
  rm.total = offsets[n_seq];
  rowmap_pad(rm);
  if (rm.total > m->cfg.max_tokens)
    return fail(CAD_E_CAPACITY, "total rows %d > max_tokens %d", rm.total, m->cfg.max_tokens);
  hipStream_t s = (hipStream_t)stream;
  const cad_config& c = m->cfg;
  m->x_parts = 0;
  LAUNCH(PF_EMBED, launch_embed(c.dtype, m->tok_embed, c.vocab, c.d_model, spans, rm.total, m->w->x, dev_status, s));
  st = run_blocks(m, kv, rm, 0, c.n_layers, nullptr, dev_status, s);
  if (st != CAD_OK) return st;
  return readout(m, rm, logits, mask, spans, mode, nullptr, argmax, accepted, dev_status, s);
} catch (...) {
  // host containers and messages are C++: nothing they throw crosses the C ABI
  return cad::set_error(CAD_E_HIP, "host allocation failed");
}

cad_status cad_splice_forward_looped(cad_model* m, const cad_kv* kv, int64_t L,
                                     const int32_t* span, int32_t N, int32_t screen_depth,
                                     const uint32_t* mask, int32_t* screen_argmax,
                                     int32_t* survivors, int32_t* argmax, int32_t* accepted,
                                     float* logits, int32_t* dev_status, cad_stream stream) try {
  cad_status st = check_common(m, kv, span, argmax, accepted, logits, CAD_VERIFY);
  if (st != CAD_OK) return st;
  const cad_config& c = m->cfg;
  if (c.loop_depth < 2) return fail(CAD_E_ARG, "model is not looped (loop_depth < 2)");
  if (screen_depth < 1 || screen_depth > c.loop_depth)
    return fail(CAD_E_ARG, "screen_depth %d outside [1, %d]", screen_depth, c.loop_depth);
  if (!screen_argmax || !survivors) return fail(CAD_E_ARG, "screen_argmax/survivors is NULL");
  st = check_seq(kv, L, N, c.max_tokens);
  if (st != CAD_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  RowMap rm{};
  rm.n_seq = 1;
  rm.total = N;
  rm.start[1] = N;
  rm.L[0] = L;
  rowmap_pad(rm);
  m->x_parts = 0;
  LAUNCH(PF_EMBED, launch_embed(c.dtype, m->tok_embed, c.vocab, c.d_model, span, N, m->w->x, dev_status, s));
  st = run_blocks(m, kv, rm, 0, screen_depth, nullptr, dev_status, s);
  if (st != CAD_OK) return st;
  st = readout(m, rm, nullptr, mask, span, CAD_VERIFY, nullptr, screen_argmax, survivors, dev_status, s);
  if (st != CAD_OK) return st;
  st = run_blocks(m, kv, rm, screen_depth, c.loop_depth, survivors, dev_status, s);
  if (st != CAD_OK) return st;
  return readout(m, rm, logits, mask, span, CAD_VERIFY, survivors, argmax, accepted, dev_status, s);
} catch (...) {
  // host containers and messages are C++: nothing they throw crosses the C ABI
  return cad::set_error(CAD_E_HIP, "host allocation failed");
}

cad_status cad_loop_step(cad_model* m, const cad_kv* kv, int32_t n_groups, const cad_loop_group* groups,
                         const int32_t* tokens, float* state, int32_t state_rows, const uint32_t* mask,
                         int32_t* argmax, int32_t* accepted, float* logits, int32_t* dev_status,
                         cad_stream stream) try {
  if (!m) return fail(CAD_E_ARG, "model is NULL");
  const cad_config& c = m->cfg;
  if (c.loop_depth < 2) return fail(CAD_E_ARG, "model is not looped (loop_depth < 2)");
  cad_status st = check_kv(m, kv);
  if (st != CAD_OK) return st;
  if (n_groups < 1 || n_groups > CAD_MAX_SEQS) return fail(CAD_E_ARG, "n_groups %d outside [1, %d]", n_groups, CAD_MAX_SEQS);
  if (!groups || !tokens || !state) return fail(CAD_E_ARG, "groups/tokens/state is NULL");
  if (state_rows < 1) return fail(CAD_E_ARG, "state_rows %d < 1", state_rows);
  RowMap rm{};
  StateMap sm{};
  rm.n_seq = n_groups;
  bool any_readout = false;
  for (int b = 0; b < n_groups; ++b) {
    const cad_loop_group& g = groups[b];
    if (g.rows < 1) return fail(CAD_E_ARG, "group %d has no rows", b);
    if (g.depth < 0 || g.depth >= c.loop_depth)
      return fail(CAD_E_ARG, "group %d depth %d outside [0, %d)", b, g.depth, c.loop_depth);
    if (g.readout != 0 && g.readout != 1) return fail(CAD_E_ARG, "group %d readout %d is neither 0 nor 1", b, g.readout);
    if (g.table_row < 0) return fail(CAD_E_ARG, "group %d table row %d < 0", b, g.table_row);
    if (g.state < 0 || (int64_t)g.state + g.rows > state_rows)
      return fail(CAD_E_ARG, "group %d state rows [%d, %d) outside [0, %d)", b, g.state, g.state + g.rows, state_rows);
    for (int o = 0; o < b; ++o)
      if (g.state < groups[o].state + groups[o].rows && groups[o].state < g.state + g.rows)
        return fail(CAD_E_ARG, "groups %d and %d share state rows", o, b);
    st = check_seq(kv, g.pos, g.rows, c.max_tokens);
    if (st != CAD_OK) return st;
    rm.start[b + 1] = rm.start[b] + g.rows;
    if (rm.start[b + 1] > c.max_tokens)
      return fail(CAD_E_CAPACITY, "%d rows in the tick exceed max_tokens %d", rm.start[b + 1], c.max_tokens);
    rm.L[b] = g.pos;
    sm.base[b] = g.state;
    any_readout |= g.readout != 0;
  }
  if ((any_readout && (!argmax || !accepted))) return fail(CAD_E_ARG, "argmax/accepted is NULL with a readout");
  if (logits && !aligned16(logits)) return fail(CAD_E_ARG, "logits must be 16-byte aligned");
  rm.total = rm.start[n_groups];
  rowmap_pad(rm);
  for (int b = 0; b < n_groups; ++b) {
    rm.trow[b] = groups[b].table_row;
    rm.cidx[b] = groups[b].depth;  // its depth's cache
  }
  hipStream_t s = (hipStream_t)stream;
  LAUNCH(PF_LOOP_STATE, launch_loop_load(c.dtype, m->tok_embed, c.vocab, c.d_model, tokens, state, rm, sm, m->w->x,
                                         dev_status, s));
  m->x_parts = 0;
  st = run_blocks(m, kv, rm, 0, 1, nullptr, dev_status, s);
  if (st != CAD_OK) return st;
  LAUNCH(PF_LOOP_STATE, launch_loop_store(m->w->x, m->w->split_ws, m->x_parts, c.d_model, state, rm, sm, s));
  m->x_parts = 0;
  if (!any_readout) return CAD_OK;
  return readout(m, rm, logits, mask, tokens, CAD_VERIFY, nullptr, argmax, accepted, dev_status, s);
} catch (...) {
  // host containers and messages are C++: nothing they throw crosses the C ABI
  return cad::set_error(CAD_E_HIP, "host allocation failed");
}

cad_status cad_profile_enable(cad_model* m, int32_t family_mask) try {
  if (!m) return fail(CAD_E_ARG, "model is NULL");
  if (family_mask) {
    HIP_TRY(hipDeviceSynchronize());
    m->prof.clear();
    m->prof_used = 0;
  }
  m->prof_mask = (uint32_t)family_mask & ((1u << PF_COUNT) - 1u);
  return CAD_OK;
} catch (...) {
  // host containers and messages are C++: nothing they throw crosses the C ABI
  return cad::set_error(CAD_E_HIP, "host allocation failed");
}

cad_status cad_profile_read(cad_model* m, const char* family, int64_t* launches, double* total_ms) try {
  if (!m || !family || !launches || !total_ms) return fail(CAD_E_ARG, "NULL argument");
  int f = -1;
  for (int i = 0; i < PF_COUNT; ++i)
    if (!strcmp(family, kProfNames[i])) f = i;
  if (f < 0) return fail(CAD_E_ARG, "unknown kernel family '%s'", family);
  int64_t n = 0;
  double ms = 0.0;
  for (const ProfRec& r : m->prof) {
    if (r.family != f) continue;
    HIP_TRY(hipEventSynchronize(r.b));
    float t = 0.f;
    HIP_TRY(hipEventElapsedTime(&t, r.a, r.b));
    ++n;
    ms += t;
  }
  *launches = n;
  *total_ms = ms;
  return CAD_OK;
} catch (...) {
  // host containers and messages are C++: nothing they throw crosses the C ABI
  return cad::set_error(CAD_E_HIP, "host allocation failed");
}

cad_status cad_propose_suffix_match(const int32_t* tokens, int64_t T, int32_t max_ngram,
                                    int32_t min_ngram, int32_t K, int32_t* out_tokens,
                                    int32_t* out_len, int64_t* out_pos, cad_stream stream) try {
  if (T < 0) return fail(CAD_E_ARG, "negative history length");
  if (T > 0 && !tokens) return fail(CAD_E_ARG, "tokens is NULL");
  if (!out_tokens || !out_len || !out_pos) return fail(CAD_E_ARG, "output pointer is NULL");
  if (min_ngram < 1 || max_ngram < min_ngram || max_ngram > 64)
    return fail(CAD_E_ARG, "need 1 <= min_ngram <= max_ngram <= 64");
  if (K < 1) return fail(CAD_E_ARG, "K must be >= 1");
  HIP_TRY(launch_suffix_match(tokens, T, max_ngram, min_ngram, K, out_tokens, out_len, out_pos,
                              (hipStream_t)stream));
  return CAD_OK;
} catch (...) {
  // host containers and messages are C++: nothing they throw crosses the C ABI
  return cad::set_error(CAD_E_HIP, "host allocation failed");
}

}  // extern "C"
