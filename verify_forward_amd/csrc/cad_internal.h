// Internal declarations shared by the HIP kernels and the host entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cad.h"

namespace cad {

typedef uint16_t bf16_t;  // bfloat16 bits: weights and KV cache of a bf16 model
typedef _Float16 f16_t;   // half: matrix-core operands (activations, q, P) of a bf16 model
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// float -> half, round to nearest even, saturated to the finite range
__device__ __forceinline__ f16_t f2h(float f) { return (f16_t)fminf(fmaxf(f, -65504.f), 65504.f); }

// float -> (hi, lo) bf16 pair: hi = bf16(x), lo = bf16(x - hi), both round
// to nearest even; x - hi is exact in fp32, so hi + lo equals x to about
// 2^-17 relative.  This is how a bf16 model hands activations to a
// projection: two planes, each multiplied with the bf16 weights on the
// matrix cores (two products, fp32 accumulate).
__device__ __forceinline__ void split_bf16(float x, bf16_t& hi, bf16_t& lo) {
  hi = f2bf(x);
  lo = f2bf(x - bf2f(hi));
}

// eight bf16 values (one 16-byte load) -> eight halves.  bf16 -> fp32 is a
// shift; fp32 -> half is exact for every bf16 value in the half normal range
// (half carries three more mantissa bits), truncation only touches values
// below 2^-17 and saturates above 65504.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(v[i] << 16);
    const float hi = __uint_as_float(v[i] & 0xFFFF0000u);
    r[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  }
  return r;
}

__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(a), as_f16x8(b), c, 0, 0, 0);
}

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
// v_mfma_f32_16x16x32_bf16: same fragment layout as the half variant
__device__ __forceinline__ f32x4 mfma16_bf(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, a), __builtin_bit_cast(bf16x8v, b), c,
                                                 0, 0, 0);
}

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t v) { return bf2f(v); }
template <> __device__ __forceinline__ float to_f<f16_t>(f16_t v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float v) { return f2bf(v); }
template <> __device__ __forceinline__ f16_t from_f<f16_t>(float v) { return f2h(v); }

// Which sequence each span row belongs to and at which absolute position it
// sits.  Passed by value to the kernels (fits the kernel-argument segment).
// A "sequence" here is a run of consecutive positions that share a cache: a
// request of a batched call, or a group of positions of a looped decoder at
// one recurrence depth (CopyLoop's concurrent pipeline runs groups at
// several depths in one launch, each on its own depth's cache).
struct RowMap {
  int32_t n_seq;
  int32_t total;
  int32_t start[CAD_MAX_SEQS + 1];   // CSR row offsets
  int32_t pstart[CAD_MAX_SEQS + 1];  // row offsets in the span K/V workspace (each sequence padded to 64 rows)
  int64_t L[CAD_MAX_SEQS];           // cache length before the call (absolute position of the first row)
  int32_t trow[CAD_MAX_SEQS];        // block-table row of the sequence
  int32_t cidx[CAD_MAX_SEQS];        // cache index of the sequence, relative to the KVView's base
};

// fill pstart from start; every sequence reads its own block-table row and
// the KVView's cache (callers with other tables or caches set trow / cidx
// afterwards)
inline void rowmap_pad(RowMap& rm) {
  rm.pstart[0] = 0;
  for (int b = 0; b < rm.n_seq; ++b) {
    rm.pstart[b + 1] = rm.pstart[b] + (rm.start[b + 1] - rm.start[b] + 63) / 64 * 64;
    rm.trow[b] = b;
    rm.cidx[b] = 0;
  }
}

__device__ __forceinline__ int row_seq(const RowMap& rm, int r) {
  int b = 0;
  while (b + 1 < rm.n_seq && rm.start[b + 1] <= r) ++b;
  return b;
}

// KV pool view for one cache index (layer or depth).
struct KVView {
  void* k;               // [num_blocks][Hkv][16][hd]
  void* v;               // [num_blocks][Hkv][hd][16]
  const int32_t* table;  // [rows][max_blocks]
  int64_t num_blocks;
  int32_t max_blocks;
  int64_t cache_stride;  // elements from one cache index to the next (RowMap.cidx)
  // bf16 models: this call's span K (after rotation) and V at half precision,
  // read by attention for keys >= L instead of their bf16 cache copies.
  // span_k [span_cap][Hkv][hd]; span_v [Hkv][hd][span_cap]; rows at RowMap.pstart
  f16_t* span_k;
  f16_t* span_v;
  int32_t span_cap;
};

// EPI_ARGMAX (the LM head): the fp32 logits are stored only if out_f32 is
// set; every row gets one masked-argmax candidate (value, lowest id) per
// column tile in `cand`, which k_decide reduces
enum Epi { EPI_STORE_F32 = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_ARGMAX = 3 };
// projection roles; each fixes its epilogue (qkv: store; lm_head: masked
// argmax candidates; o, down: residual add; gate_up: SwiGLU) and names its
// kernels
enum GemmRole { GEMM_QKV = 0, GEMM_O = 1, GEMM_GATE_UP = 2, GEMM_DOWN = 3, GEMM_LM_HEAD = 4 };

struct GemmArgs {
  // activations [M][lda]: fp32 for fp32 models; for bf16 models two bf16
  // planes, A = hi part, A_lo = the bf16-rounded remainder (hi + lo ~ fp32)
  const void* A;
  const void* A_lo;
  int64_t lda;
  const void* W;   // weight rows [rows][ldw]
  int64_t ldw;
  int M, N, K;     // N = logical output columns (SWIGLU: ffn width)
  int64_t up_off;  // SWIGLU: first row of the "up" half
  float* out_f32;  // STORE_F32 / RESID destination [M][ldo]
  int64_t ldo;
  void* out_act;     // SWIGLU destination [M][N]: fp32 (fp32 models) or the hi plane (bf16 models)
  void* out_act_lo;  // bf16 models: lo plane of the SWIGLU destination
  // split-K scratch (library workspace): fp32 partial sums [split][M][cols],
  // split_cap floats
  float* split_ws;
  int64_t split_cap;
  // bf16 models, at most 16 rows: when norm_ss is set, A is the fp32
  // residual stream [M][lda] and the projection normalises it while staging
  // (RMSNorm with gain norm_g [K], bf16, and the slice sums of squares
  // norm_ss [M][norm_slices] written by launch_rms_slices) into hi/lo planes
  const void* norm_g;
  const float* norm_ss;
  int norm_slices;
  float norm_eps;
  // bf16 models, more than 16 rows: the SWIGLU epilogue writes one half
  // plane (out_act as f16, no lo plane), and the down projection reads it
  // (A is then a single half plane and the weights are widened to half);
  // a value beyond half's range is saturated and sets CAD_DEV_F16_RANGE in
  // *status (when status is set)
  int act_f16;
  int32_t* status;
  // EPI_ARGMAX: per-row vocabulary bitmask [M][mask_words] (bit v % 32 of
  // word v / 32 = id v allowed) or nullptr (all allowed); candidates
  // cand[c][M] as (fp32 value bits, id) pairs, id -1 when tile c allows
  // nothing for that row; the launcher reports the candidate count per row
  // in *n_cand (a host pointer, never read by a kernel)
  const uint32_t* mask;
  int mask_words;
  uint32_t* cand;
  int* n_cand;
};

// most masked-argmax candidates per row any LM-head path produces: one per
// 64 vocabulary ids
inline int max_candidates(int vocab) { return (vocab + 63) / 64; }

// split-K workspace of a model's own workspace: GEMM_SPLIT_FLOATS floats (128 MB)
constexpr int64_t GEMM_SPLIT_FLOATS = (int64_t)32 << 20;

// First row of each sequence's hidden states in a caller's state buffer
// (the looped decoder's pipeline tick carries every row's residual stream
// from one tick to the next).
struct StateMap {
  int32_t base[CAD_MAX_SEQS];
};

// the calling thread's error message (cad_last_error) and the given status
cad_status set_error(cad_status s, const char* msg);

// ---- launchers (stream-ordered, no host sync) ----
hipError_t launch_embed(int dtype, const void* table, int vocab, int d, const int32_t* tokens,
                        int rows, float* x, int32_t* status, hipStream_t s);
// out: fp32 [rows][d] (fp32 models) or bf16 planes out (hi) / out_lo (bf16 models)
// x += the n_part pending k-split partial planes x_part [n_part][rows][d]
// (added in order, x written back), then the norm
hipError_t launch_rmsnorm(int dtype, float* x, const float* x_part, int n_part, const void* gain, int rows, int d,
                          float eps, void* out, void* out_lo, hipStream_t s);
// few rows: x += the n_part partial planes (x written back) and the sums of
// squares of 256-element slices to ss [rows][rms_slices(d)]; the
// weight-streaming projection that follows applies the norm (GemmArgs.norm_*)
hipError_t launch_rms_slices(float* x, const float* x_part, int n_part, int rows, int d, float* ss, hipStream_t s);
// pipeline tick of a looped model: x[r] = the embedding of tokens[r] for rows
// of sequences at cache index 0 (their first application of the block), else
// the row's saved state state[sm.base[b] + j] (fp32 [.][d])
hipError_t launch_loop_load(int dtype, const void* table, int vocab, int d, const int32_t* tokens, const float* state,
                            const RowMap& rm, const StateMap& sm, float* x, int32_t* status, hipStream_t s);
// x += the n_part pending partial planes (written back) and every row saved
// to state[sm.base[b] + j]
hipError_t launch_loop_store(float* x, const float* x_part, int n_part, int d, float* state, const RowMap& rm,
                             const StateMap& sm, hipStream_t s);
int rms_slices(int d);
// partials: see launch_epi; nullptr makes every launch apply its epilogue
hipError_t launch_gemm(int dtype, int role, const GemmArgs& a, hipStream_t s, int* partials = nullptr);
// qkv: [rows][width] fp32, or (n_part > 0) the sum of the partial planes
// qkv_part [n_part][rows][width]
hipError_t launch_rope_append(int dtype, const float* qkv, const float* qkv_part, int n_part, int rows, int hq,
                              int hkv, int hd, const double* freq, const RowMap& rm, KVView kv,
                              const int32_t* write_limit, void* q_out, void* q_lo, int32_t* status,
                              hipStream_t s);
// n_parts = partitions of each query tile's key axis (its cached keys, then
// the call's own keys), equal runs of 64-key tiles each
// q_lo: bf16 models, the half remainder plane of q (nullptr for fp32)
hipError_t launch_attention(int dtype, const void* q, const void* q_lo, int rows, int hq, int hkv, int hd,
                            const RowMap& rm, KVView kv, int n_parts,
                            float* part_o, float* part_ml, void* out, void* out_lo, int32_t* status,
                            hipStream_t s);
// log-sum-exp merge of the key partitions (bf16 models, n_parts > 1), into bf16 planes
hipError_t launch_attention_merge(const float* part_o, const float* part_ml, int n_parts, int rows,
                                  int hq, int hd, void* out, void* out_lo, hipStream_t s);
// Masked argmax of every row from the LM head's candidates (cand[c][rows],
// n_cand per row: larger value wins, then the lower id), then the
// acceptance scan of every sequence (COMMIT: its row count; VERIFY: 1 + the
// leading j >= 1 with argmax[j-1] == span[j]).  `limit` (device, optional,
// single-sequence calls) caps the rows: rows at or beyond max(1, *limit)
// get argmax -1 and are not examined.  Rows that allow nothing get -1 and
// set CAD_DEV_EMPTY_MASK.
hipError_t launch_decide(const uint32_t* cand, int n_cand, int rows, const RowMap& rm, const int32_t* span,
                         int mode, const int32_t* limit, int32_t* argmax, int32_t* accepted, int32_t* status,
                         hipStream_t s);
hipError_t launch_suffix_match(const int32_t* tokens, int64_t T, int max_n, int min_n, int K,
                               int32_t* out_tokens, int32_t* out_len, int64_t* out_pos,
                               hipStream_t s);

// the next block's context-copy proposal straight after a readout: head =
// argmax[*kept - 1] is written to hist[pos + *kept] (and out_head), then the
// suffix match runs over hist[0 .. pos + *kept]
hipError_t launch_propose_next(int32_t* hist, int64_t pos, const int32_t* kept, const int32_t* argmax, int max_n,
                               int min_n, int K, int32_t* out_tokens, int32_t* out_len, int64_t* out_pos,
                               int32_t* out_head, hipStream_t s);

// ---- Copy-as-Decode program automaton (device-resident state) ----
enum FsmStateId { FSM_AWAIT_OP = 0, FSM_AFTER_LT = 1, FSM_NUM_A = 2, FSM_NUM_B = 3, FSM_GEN_BODY = 4, FSM_DONE = 5 };
// what the next forward is: none yet; one chained single step (the feed is
// one token); a splice of feed_n tokens whose last row takes a decision; the
// terminator's splice (no decision follows); nothing more (stream limit,
// error)
enum FsmAction { FSM_ACT_NONE = 0, FSM_ACT_STEP = 1, FSM_ACT_FEED = 2, FSM_ACT_LAST = 3, FSM_ACT_STOP = 4 };
// token ids of the program's structural literals (kw: " lines" or " tokens")
struct FsmTable {
  int32_t lt, lt_slash, gt, copy, gen, program, kw, eq_quote, quote, slash_gt, hyphen;
  int32_t digits[10];
};
struct FsmLimits {
  int32_t units;        // copy ranges lie in [1, units] (lines or tokens of the document)
  int32_t unit_tokens;  // 1: a range counts document tokens, 0: lines (through the line table)
  int32_t max_ops, max_gen, max_stream;
  int32_t vocab_words;  // ceil(vocab / 32)
  int32_t doc_n;        // document tokens at the front of the history
  int32_t hist_cap;     // history capacity (document + stream + one feed + a draft)
  int32_t draft_k;      // draft length inside gen bodies (0: none)
};
// one int32 per field so the host reads it back as a plain array
struct FsmState {
  int32_t state, n_ops, v, nd, a, gen_len, win[3];
  int32_t action, feed_n, chain_ok, stream_n, error;
  int32_t decisions, chained, masked, forced, copies, copied, drafts, draft_tokens, draft_accepted, out_n;
};
// op records [max_ops][5]: kind (0 copy, 1 gen), a, b (copy range), body
// start in the stream and body length (gen)
constexpr int FSM_OP_INTS = 5;

hipError_t launch_fsm_init(FsmState* st, hipStream_t s);
// the current decision's vocabulary mask, replicated to `rows` rows
hipError_t launch_fsm_mask(const FsmState* st, const FsmTable& t, const FsmLimits& lim, uint32_t* mask, int rows,
                           hipStream_t s);
// take the decision argmax[decide_row] (force = 1: after a host-launched
// splice; 0: a chained step, which acts only while chain_ok is set) and build
// the next feed, appended to the stream (hist[doc_n + stream_n ..])
hipError_t launch_fsm_advance(FsmState* st, const FsmTable& t, const FsmLimits& lim, const int32_t* argmax,
                              int decide_row, int force, const int32_t* line_start, int32_t* hist, int32_t* feed,
                              int32_t* ops, hipStream_t s);
// inside a gen body with a pending single-token feed: append up to draft_k
// drafted tokens (suffix match over the history) to the feed, set feed_n to
// the rows that count and write the verify forward's draft_k + 1 mask rows
hipError_t launch_fsm_draft(FsmState* st, const FsmTable& t, const FsmLimits& lim, int32_t* hist, int32_t* feed,
                            uint32_t* mask, int32_t* tmp_len, int64_t* tmp_pos, hipStream_t s);
// after the verify forward: pass the accepted drafts through the automaton,
// then take the decision that follows them
hipError_t launch_fsm_verified(FsmState* st, const FsmTable& t, const FsmLimits& lim, const int32_t* argmax,
                               const int32_t* accepted, const int32_t* line_start, int32_t* hist, int32_t* feed,
                               int32_t* ops, hipStream_t s);
// the program's output: copies expanded from the document, gen bodies from
// the stream, into out[0 .. out_cap) (out_n = the full length)
hipError_t launch_fsm_resolve(FsmState* st, const FsmLimits& lim, const int32_t* line_start, const int32_t* hist,
                              const int32_t* ops, int32_t* out, int out_cap, hipStream_t s);

// cad_splice_forward (models with loop_depth 1, its checks included) with
// an optional device row limit: rows at or beyond *limit write no K/V and
// rows at or beyond max(1, *limit) are not decided
cad_status splice_rows(cad_model* m, const cad_kv* kv, int64_t L, const int32_t* span, int N, const uint32_t* mask,
                       int mode, const int32_t* limit, int32_t* argmax, int32_t* accepted, float* logits,
                       int32_t* dev_status, hipStream_t s);

// attention split: partitions of each query tile's key axis (cached keys up
// to max L, then the span's own) so that small spans still fill the chip
// (max_seq_rows: the most span rows any sequence of the call has)
int attention_parts(int rows, int n_seq, int hq, int hkv, int64_t max_cache_keys, int max_seq_rows);

}  // namespace cad

// shape of a model handle (library-internal accessor)
const cad_config* cad_model_config(const cad_model* m);
