// Copy-as-Decode's token-level grammar automaton on the device (Copy-as-Decode
// §2.1 grammar, §2.2 resolver, §2.3 masked steps and forced-template
// prefills, appendix paragraphs "States.", "Forced prefills." and
// "Token-sequence end-of-gen detector."; §5 "Token-level extension." for
// copies of token ranges and "Composition with speculative decoding." for
// drafts inside gen bodies).
//
// The automaton's state lives in device memory.  k_fsm_mask writes the
// vocabulary bitmask of the decision the state asks for; k_fsm_advance takes
// the decision (the masked argmax the LM head's epilogue produced), moves the
// state and builds the next forward's input: the chosen id alone (a masked or
// free step), a forced template, or the closing quote, "/>" and the copied
// span gathered from the document.  Every feed is appended to the stream
// when it is built and is fed exactly once afterwards.  The state tells the
// host what the next forward is (a single step, a splice of feed_n tokens,
// the terminator, nothing), so chains of single steps need no host round
// trip: the advance after a chained step whose chain has ended does nothing
// (that step's K/V lands past the stream's end, where the next forward
// overwrites it).
//
// History layout: hist[0 .. doc_n) is the document, hist[doc_n + j] the j-th
// program token fed after the prompt (the stream); copies read the front,
// drafts search the whole of it.
#include "cad_internal.h"
#include "suffix_match.h"

namespace cad {

// suffix lengths of the gen-body drafts: four down to one (the same search as
// the context-copy proposals)
constexpr int kDraftMaxN = 4;
constexpr int kDraftMinN = 1;

// some integer in [lo, hi] has `prefix` as its leading decimal digits
__device__ __forceinline__ bool can_extend(int64_t prefix, int64_t lo, int64_t hi) {
  for (int64_t k = 1; prefix * k <= hi; k *= 10)
    if (prefix * k + (k - 1) >= lo) return true;
  return false;
}

// ids allowed at an op boundary after n_ops ops: "<" before the first op,
// "<" or "</" after, only "</" once max_ops ops are done
__device__ __forceinline__ int boundary_ids(int n_ops, const FsmTable& t, const FsmLimits& lim, int32_t* ids) {
  if (n_ops >= lim.max_ops) { ids[0] = t.lt_slash; return 1; }
  ids[0] = t.lt;
  if (n_ops == 0) return 1;
  ids[1] = t.lt_slash;
  return 2;
}

// allowed ids of the current decision as (count, ids); -1: every id (free
// generation inside a gen body)
__device__ int fsm_allowed(const FsmState& s, const FsmTable& t, const FsmLimits& lim, int32_t* ids) {
  switch (s.state) {
    case FSM_AWAIT_OP:
      return boundary_ids(s.n_ops, t, lim, ids);
    case FSM_AFTER_LT:
      ids[0] = t.copy;
      ids[1] = t.gen;
      return 2;
    case FSM_NUM_A:
    case FSM_NUM_B: {
      // no leading zero; the first number in [1, units], the second in [first, units]
      const int64_t lo = s.state == FSM_NUM_A ? 1 : s.a;
      int n = 0;
      for (int d = 0; d < 10; ++d)
        if (!(s.nd == 0 && d == 0) && can_extend((int64_t)s.v * 10 + d, lo, lim.units)) ids[n++] = t.digits[d];
      if (s.nd > 0 && s.v >= lo && s.v <= lim.units) ids[n++] = s.state == FSM_NUM_A ? t.hyphen : t.quote;
      return n;
    }
    case FSM_GEN_BODY:
      return -1;
    default:
      return 0;  // after the program's end nothing is allowed
  }
}

// mask words of an id set (n < 0: every id)
__device__ __forceinline__ uint32_t mask_word(int w, int n, const int32_t* ids) {
  uint32_t bits = n < 0 ? 0xFFFFFFFFu : 0u;
  for (int i = 0; i < n; ++i)
    if (ids[i] >> 5 == w) bits |= 1u << (ids[i] & 31);
  return bits;
}

// One work-group: the mask of the current decision, replicated to `rows`
// rows (a splice's rows before the last are not decisions; replicating keeps
// every row's argmax well defined).  After the program's end (a chained step
// launched past the terminator) no decision follows: every id is allowed, so
// that row is not reported as one that allows nothing.
__global__ void __launch_bounds__(256) k_fsm_mask(const FsmState* __restrict__ st, FsmTable t, FsmLimits lim,
                                                  uint32_t* __restrict__ mask, int rows) {
  __shared__ int32_t ids[16];
  __shared__ int n;
  if (threadIdx.x == 0) n = st->state == FSM_DONE ? -1 : fsm_allowed(*st, t, lim, ids);
  __syncthreads();
  const int words = lim.vocab_words;
  for (int w = threadIdx.x; w < words; w += blockDim.x) {
    const uint32_t bits = mask_word(w, n, ids);
    for (int r = 0; r < rows; ++r) mask[(int64_t)r * words + w] = bits;
  }
}

// What a decision appends to the stream: `fn` template ids already in
// feed[0 .. fn), then span_n document tokens from hist[span_a ..]; all of it
// goes to the stream at hist[out0 ..].
struct Emit {
  int fn, span_a, span_n, out0;
};

__device__ __forceinline__ void close_state(FsmState& s) {
  s.n_ops += 1;
  s.state = FSM_AWAIT_OP;
}

// one id through the gen body: the rolling window over the last three ids
// and the body length; returns 1 if the window now holds the end-of-gen ids,
// 2 if the body reached max_gen ids, else 0 (the op is closed in both cases)
__device__ __forceinline__ int gen_token(FsmState& s, const FsmTable& t, const FsmLimits& lim, int32_t c,
                                         int32_t* ops) {
  s.win[0] = s.win[1];
  s.win[1] = s.win[2];
  s.win[2] = c;
  s.gen_len += 1;
  int32_t* op = ops + FSM_OP_INTS * s.n_ops;
  op[4] = s.gen_len;
  if (s.win[0] == t.lt_slash && s.win[1] == t.gen && s.win[2] == t.gt) {
    op[4] = s.gen_len - 3;  // the body ends before the "</gen>" ids
    close_state(s);
    return 1;
  }
  if (s.gen_len >= lim.max_gen) {
    close_state(s);
    return 2;
  }
  return 0;
}

// sets feed_n, the action and chain_ok for a feed of e.fn + e.span_n ids
// and appends it to the stream (the copy itself is done by emit_copy)
__device__ __forceinline__ void finish(FsmState& s, const FsmLimits& lim, Emit& e) {
  const int n = e.fn + e.span_n;
  e.out0 = lim.doc_n + s.stream_n;
  if (e.out0 + n > lim.hist_cap) {  // cannot happen within the capacities the host checked; refuse
    s.error = 2;
    s.state = FSM_DONE;
    e.fn = e.span_n = 0;
    s.feed_n = 0;
    s.action = FSM_ACT_STOP;
    s.chain_ok = 0;
    return;
  }
  s.feed_n = n;
  s.action = s.state == FSM_DONE ? FSM_ACT_LAST : (n == 1 ? FSM_ACT_STEP : FSM_ACT_FEED);
  s.chain_ok = s.action == FSM_ACT_STEP ? 1 : 0;
  s.stream_n += n;
}

// Thread 0: take decision c in the current state.  A decision once the
// stream holds max_stream ids is not taken (the decoder stops there); a
// decision the state's mask refuses (possible only when the mask allows
// nothing) stops with an error.
__device__ Emit fsm_decide(FsmState& s, const FsmTable& t, const FsmLimits& lim, int32_t c, int32_t* feed,
                           int32_t* ops, const int32_t* line_start) {
  Emit e{0, 0, 0, 0};
  if (s.stream_n >= lim.max_stream || s.state == FSM_DONE) {
    s.action = FSM_ACT_STOP;
    s.feed_n = 0;
    s.chain_ok = 0;
    return e;
  }
  int32_t ids[16];
  const int n_allowed = fsm_allowed(s, t, lim, ids);
  bool legal = n_allowed < 0;
  for (int i = 0; i < n_allowed; ++i) legal |= ids[i] == c;
  if (!legal) {
    s.error = 1;
    s.state = FSM_DONE;
    s.action = FSM_ACT_STOP;
    s.feed_n = 0;
    s.chain_ok = 0;
    return e;
  }
  s.decisions += 1;
  if (n_allowed >= 0) s.masked += 1;
  int fn = 0;
  switch (s.state) {
    case FSM_AWAIT_OP:
      if (c == t.lt) {
        s.state = FSM_AFTER_LT;
        feed[fn++] = c;
      } else {  // "</": the terminator's forced prefill
        s.state = FSM_DONE;
        feed[fn++] = t.lt_slash;
        feed[fn++] = t.program;
        feed[fn++] = t.gt;
        s.forced += 1;
      }
      break;
    case FSM_AFTER_LT:
      if (c == t.copy) {  // copy opener: "copy" " lines" '="'
        s.state = FSM_NUM_A;
        s.v = s.nd = 0;
        feed[fn++] = t.copy;
        feed[fn++] = t.kw;
        feed[fn++] = t.eq_quote;
      } else {  // gen opener: "gen" ">"
        s.state = FSM_GEN_BODY;
        s.gen_len = 0;
        s.win[0] = s.win[1] = s.win[2] = -1;
        int32_t* op = ops + FSM_OP_INTS * s.n_ops;
        op[0] = 1;
        op[1] = op[2] = 0;
        op[3] = s.stream_n + 2;  // the body starts after "gen" ">"
        op[4] = 0;
        feed[fn++] = t.gen;
        feed[fn++] = t.gt;
      }
      s.forced += 1;
      break;
    case FSM_NUM_A:
    case FSM_NUM_B: {
      int d = -1;
      for (int i = 0; i < 10; ++i)
        if (t.digits[i] == c) d = i;
      if (d >= 0) {
        s.v = s.v * 10 + d;
        s.nd += 1;
        feed[fn++] = c;
      } else if (s.state == FSM_NUM_A) {  // hyphen
        s.a = s.v;
        s.v = s.nd = 0;
        s.state = FSM_NUM_B;
        feed[fn++] = c;
      } else {  // closing quote: '"' "/>" and the copied units, one splice
        int32_t* op = ops + FSM_OP_INTS * s.n_ops;
        op[0] = 0;
        op[1] = s.a;
        op[2] = s.v;
        op[3] = op[4] = 0;
        feed[fn++] = t.quote;
        feed[fn++] = t.slash_gt;
        // units a..b, 1-indexed and inclusive: tokens directly, lines through the line table
        e.span_a = lim.unit_tokens ? s.a - 1 : line_start[s.a - 1];
        e.span_n = (lim.unit_tokens ? s.v : line_start[s.v]) - e.span_a;
        s.copies += 1;
        s.copied += e.span_n;
        close_state(s);
      }
      break;
    }
    default: {  // FSM_GEN_BODY: free generation
      feed[fn++] = c;
      if (gen_token(s, t, lim, c, ops) == 2) {  // length cap: "</gen>" force-prefilled after the id
        feed[fn++] = t.lt_slash;
        feed[fn++] = t.gen;
        feed[fn++] = t.gt;
        s.forced += 1;
      }
      break;
    }
  }
  e.fn = fn;
  finish(s, lim, e);
  return e;
}

// All threads: the stream copy of feed[0 .. fn) and the copied span (to the
// feed and the stream).
__device__ __forceinline__ void emit_copy(const Emit& e, int32_t* hist, int32_t* feed) {
  for (int i = threadIdx.x; i < e.span_n; i += blockDim.x) {
    const int32_t v = hist[e.span_a + i];
    feed[e.fn + i] = v;
    hist[e.out0 + e.fn + i] = v;
  }
  for (int i = threadIdx.x; i < e.fn; i += blockDim.x) hist[e.out0 + i] = feed[i];
}

// One work-group.  With force = 1 (the host just fed the current feed in one
// splice) or chain_ok set (a chained single step fed it), takes the decision
// argmax[decide_row] and builds the next feed in feed[0 .. feed_n);
// otherwise (a chained step after its chain ended) it does nothing.
__global__ void __launch_bounds__(256) k_fsm_advance(FsmState* __restrict__ st, FsmTable t, FsmLimits lim,
                                                     const int32_t* __restrict__ argmax, int decide_row, int force,
                                                     const int32_t* __restrict__ line_start,
                                                     int32_t* __restrict__ hist, int32_t* __restrict__ feed,
                                                     int32_t* __restrict__ ops) {
  __shared__ Emit e;
  __shared__ int go;
  if (threadIdx.x == 0) {
    FsmState s = *st;
    go = force || s.chain_ok;
    if (go) {
      if (!force) s.chained += 1;
      e = fsm_decide(s, t, lim, argmax[decide_row], feed, ops, line_start);
      *st = s;
    }
  }
  __syncthreads();
  if (go) emit_copy(e, hist, feed);
}

// One work-group of SUFFIX_THREADS, in a gen body with the pending feed [c]
// (c is the stream's last id): drafts up to draft_k ids continuing the most
// recent earlier match of the history's suffix, into feed[1 ..] and the
// stream positions after c (they stay there only if accepted); feed rows past
// the draft repeat c (valid ids for the fixed-size verify, which neither
// writes nor decides them: feed_n = 1 + the draft length).  Mask rows
// 0 .. draft_k: every id, except the row after the first draft id that
// completes the end-of-gen window (its decision is an op boundary's).
__global__ void __launch_bounds__(SUFFIX_THREADS) k_fsm_draft(FsmState* __restrict__ st, FsmTable t, FsmLimits lim,
                                                              int32_t* __restrict__ hist, int32_t* __restrict__ feed,
                                                              uint32_t* __restrict__ mask,
                                                              int32_t* __restrict__ tmp_len,
                                                              int64_t* __restrict__ tmp_pos) {
  __shared__ int32_t ids[4];
  __shared__ int n_ids, mrow;
  const int64_t T = (int64_t)lim.doc_n + st->stream_n;
  int K = lim.draft_k;
  if (T + K > lim.hist_cap) K = (int)(lim.hist_cap - T);  // never, within the capacities the host checked
  if (K < 0) K = 0;
  suffix_match_body(hist, T, kDraftMaxN, kDraftMinN, K, feed + 1, tmp_len, tmp_pos);
  __syncthreads();
  if (threadIdx.x == 0) {
    FsmState s = *st;
    const int len = *tmp_len;
    for (int j = 1 + len; j <= lim.draft_k; ++j) feed[j] = feed[0];
    for (int j = 1; j <= len; ++j) hist[T + j - 1] = feed[j];
    // the window over the drafted ids, from the state after c
    int32_t w0 = s.win[0], w1 = s.win[1], w2 = s.win[2];
    int g = s.gen_len;
    mrow = -1;
    for (int j = 1; j <= len; ++j) {
      w0 = w1;
      w1 = w2;
      w2 = feed[j];
      g += 1;
      if (w0 == t.lt_slash && w1 == t.gen && w2 == t.gt) {
        mrow = j;
        break;
      }
      if (g >= lim.max_gen) break;  // the body ends by its length: no decision at this row
    }
    n_ids = boundary_ids(s.n_ops + 1, t, lim, ids);
    s.feed_n = 1 + len;
    s.drafts += 1;
    s.draft_tokens += len;
    *st = s;
  }
  __syncthreads();
  const int words = lim.vocab_words;
  for (int i = threadIdx.x; i < (lim.draft_k + 1) * words; i += blockDim.x) {
    const int r = i / words, w = i - r * words;
    mask[i] = r == mrow ? mask_word(w, n_ids, ids) : 0xFFFFFFFFu;
  }
}

// One work-group, after the verify forward of [c, drafts]: the accepted
// drafts (feed[1 .. accepted)) go through the gen body in order, already in
// the stream; the body may end inside them (end-of-gen window: the decision
// is the op boundary's at that row; length cap: "</gen>" is the next feed,
// force-prefilled, no decision).  Otherwise the decision after the last
// accepted id (the correction, or the bonus on a full match) is taken.
__global__ void __launch_bounds__(256) k_fsm_verified(FsmState* __restrict__ st, FsmTable t, FsmLimits lim,
                                                      const int32_t* __restrict__ argmax,
                                                      const int32_t* __restrict__ accepted,
                                                      const int32_t* __restrict__ line_start,
                                                      int32_t* __restrict__ hist, int32_t* __restrict__ feed,
                                                      int32_t* __restrict__ ops) {
  __shared__ Emit e;
  if (threadIdx.x == 0) {
    FsmState s = *st;
    const int acc = *accepted;
    int row = acc - 1, ended = 0;
    for (int j = 1; j < acc; ++j) {
      s.stream_n += 1;
      s.draft_accepted += 1;
      ended = gen_token(s, t, lim, feed[j], ops);
      if (ended) {
        row = j;
        break;
      }
    }
    if (ended == 2) {
      feed[0] = t.lt_slash;
      feed[1] = t.gen;
      feed[2] = t.gt;
      s.forced += 1;
      e = Emit{3, 0, 0, 0};
      finish(s, lim, e);
    } else {
      e = fsm_decide(s, t, lim, argmax[row], feed, ops, line_start);
    }
    *st = s;
  }
  __syncthreads();
  emit_copy(e, hist, feed);
}

// One work-group: the program's output (Copy-as-Decode §2.2's resolver), op
// by op: a copy expands to the document's units a..b, a gen op to its body
// as generated (an unfinished one to the ids so far).
__global__ void __launch_bounds__(256) k_fsm_resolve(FsmState* __restrict__ st, FsmLimits lim,
                                                     const int32_t* __restrict__ line_start,
                                                     const int32_t* __restrict__ hist,
                                                     const int32_t* __restrict__ ops, int32_t* __restrict__ out,
                                                     int out_cap) {
  const FsmState s = *st;
  const int n_rec = s.n_ops + (s.state == FSM_GEN_BODY ? 1 : 0);
  int64_t o = 0;
  for (int i = 0; i < n_rec; ++i) {
    const int32_t* op = ops + FSM_OP_INTS * i;
    int64_t src, n;
    if (op[0] == 0) {
      src = lim.unit_tokens ? op[1] - 1 : line_start[op[1] - 1];
      n = (lim.unit_tokens ? op[2] : line_start[op[2]]) - src;
    } else {
      src = (int64_t)lim.doc_n + op[3];
      n = op[4];
    }
    for (int64_t j = threadIdx.x; j < n; j += blockDim.x)
      if (o + j < out_cap) out[o + j] = hist[src + j];
    o += n;
  }
  __syncthreads();
  if (threadIdx.x == 0) st->out_n = (int32_t)o;
}

__global__ void k_fsm_init(FsmState* st) {
  if (threadIdx.x == 0) {
    FsmState s{};
    s.state = FSM_AWAIT_OP;
    s.action = FSM_ACT_NONE;
    s.win[0] = s.win[1] = s.win[2] = -1;
    *st = s;
  }
}

hipError_t launch_fsm_init(FsmState* st, hipStream_t s) {
  hipLaunchKernelGGL(k_fsm_init, dim3(1), dim3(64), 0, s, st);
  return hipGetLastError();
}

hipError_t launch_fsm_mask(const FsmState* st, const FsmTable& t, const FsmLimits& lim, uint32_t* mask, int rows,
                           hipStream_t s) {
  hipLaunchKernelGGL(k_fsm_mask, dim3(1), dim3(256), 0, s, st, t, lim, mask, rows);
  return hipGetLastError();
}

hipError_t launch_fsm_advance(FsmState* st, const FsmTable& t, const FsmLimits& lim, const int32_t* argmax,
                              int decide_row, int force, const int32_t* line_start, int32_t* hist, int32_t* feed,
                              int32_t* ops, hipStream_t s) {
  hipLaunchKernelGGL(k_fsm_advance, dim3(1), dim3(256), 0, s, st, t, lim, argmax, decide_row, force, line_start,
                     hist, feed, ops);
  return hipGetLastError();
}

hipError_t launch_fsm_draft(FsmState* st, const FsmTable& t, const FsmLimits& lim, int32_t* hist, int32_t* feed,
                            uint32_t* mask, int32_t* tmp_len, int64_t* tmp_pos, hipStream_t s) {
  hipLaunchKernelGGL(k_fsm_draft, dim3(1), dim3(SUFFIX_THREADS), 0, s, st, t, lim, hist, feed, mask, tmp_len,
                     tmp_pos);
  return hipGetLastError();
}

hipError_t launch_fsm_verified(FsmState* st, const FsmTable& t, const FsmLimits& lim, const int32_t* argmax,
                               const int32_t* accepted, const int32_t* line_start, int32_t* hist, int32_t* feed,
                               int32_t* ops, hipStream_t s) {
  hipLaunchKernelGGL(k_fsm_verified, dim3(1), dim3(256), 0, s, st, t, lim, argmax, accepted, line_start, hist, feed,
                     ops);
  return hipGetLastError();
}

hipError_t launch_fsm_resolve(FsmState* st, const FsmLimits& lim, const int32_t* line_start, const int32_t* hist,
                              const int32_t* ops, int32_t* out, int out_cap, hipStream_t s) {
  hipLaunchKernelGGL(k_fsm_resolve, dim3(1), dim3(256), 0, s, st, lim, line_start, hist, ops, out, out_cap);
  return hipGetLastError();
}

}  // namespace cad
