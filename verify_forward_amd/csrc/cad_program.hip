// Copy-as-Decode program decoding: the host driver over the device automaton
// (k_fsm.hip) and the splice forward (Copy-as-Decode §2.3 "the decoder":
// masked steps at decision points, forced-template prefills, copy splices;
// §5 drafts inside gen bodies).
//
// The automaton, its masks, the feeds and the stream live on the device;
// the host only reads the automaton's small state back, and only when the
// next forward's length depends on a decision:
//   * FEED (a template, or a copy: quote, "/>" and the span): one splice of
//     feed_n rows whose last row takes the next decision under its mask;
//   * STEP (one id): single-token steps, chained without a host round trip
//     -- each is mask, forward, advance; the advance acts only while the
//     chain holds, so steps launched after it ended (the decision asked for
//     a longer feed) take no decision.  They write K/V at positions past the
//     stream's end, which the next forward overwrites before any query
//     reads them.  How many steps to launch ahead is predicted from the
//     state: one after "<" (the op type's decision asks for a template), two
//     after a gen body's end, at most the digits a range can still take, at
//     most the ids a gen body can still take, and never more than `chain`;
//   * in a gen body with drafts: one verify forward of [pending id, drafts]
//     with a fixed row count (1 + draft_k; rows past the draft neither write
//     K/V nor decide, so the forward's shape needs no host knowledge);
//   * LAST: the terminator's splice, no decision.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "cad_internal.h"

using namespace cad;

struct cad_program {
  cad_model* m = nullptr;
  cad_config cfg{};
  FsmTable t{};
  cad_program_params p{};
  int64_t max_len = 0;
  int32_t hist_cap = 0, feed_cap = 0, mask_rows = 0, words = 0, out_cap = 0;
  void* dev = nullptr;  // one device allocation
  FsmState* st = nullptr;
  int32_t* hist = nullptr;        // [hist_cap]: document, then the stream
  int32_t* feed = nullptr;        // [feed_cap]
  int32_t* ops = nullptr;         // [max_ops + 1][FSM_OP_INTS]
  int32_t* line_start = nullptr;  // [max_doc + 1]
  int32_t* prompt = nullptr;      // [max_len]
  int32_t* argmax = nullptr;      // [max_tokens]
  int32_t* accepted = nullptr;    // [1]
  int32_t* status = nullptr;      // [1]
  int32_t* tmp_len = nullptr;     // [1]
  int64_t* tmp_pos = nullptr;     // [1]
  int32_t* out = nullptr;         // [out_cap]
  uint32_t* mask = nullptr;       // [mask_rows][words]
  FsmState* h_st = nullptr;       // pinned
};

namespace {

static_assert(sizeof(cad_program_table) == sizeof(FsmTable), "table layouts differ");

cad_status prog_fail(cad_status s, const std::string& msg) { return cad::set_error(s, msg.c_str()); }

std::string fmt(const char* f, long long a, long long b = 0) {
  char buf[256];
  snprintf(buf, sizeof buf, f, a, b);
  return buf;
}

size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

#define PROG_HIP(expr)                                                                                \
  do {                                                                                                \
    hipError_t e_ = (expr);                                                                           \
    if (e_ != hipSuccess) return prog_fail(CAD_E_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

// an internal call that sets its own message
#define PROG_CALL(expr)              \
  do {                               \
    cad_status s_ = (expr);          \
    if (s_ != CAD_OK) return s_;     \
  } while (0)

int decimal_digits(int64_t v) {
  int n = 1;
  while (v >= 10) { v /= 10; ++n; }
  return n;
}

struct Decode {
  cad_program* pr;
  const cad_kv* kv;
  hipStream_t s;
  FsmLimits lim{};
  int64_t L0 = 0;
  int64_t cap = 0;  // positions the block table holds
  int64_t launched_chained = 0;

  // feed_n ids of the feed at absolute position pos, in chunks of at most
  // max_tokens rows; the last row takes the next decision under the
  // state's mask unless `decide` is 0
  cad_status splice_feed(int64_t pos, int n, bool decide) {
    cad_program* P = pr;
    const int T = P->cfg.max_tokens;
    for (int off = 0; off < n; off += T) {
      const int rows = std::min(T, n - off);
      const bool last = off + rows == n;
      if (last && decide) PROG_HIP(launch_fsm_mask(P->st, P->t, lim, P->mask, rows, s));
      PROG_CALL(splice_rows(P->m, kv, pos + off, P->feed + off, rows, last && decide ? P->mask : nullptr, CAD_COMMIT,
                            nullptr, P->argmax, P->accepted, nullptr, P->status, s));
      if (last && decide)
        PROG_HIP(launch_fsm_advance(P->st, P->t, lim, P->argmax, rows - 1, 1, P->line_start, P->hist, P->feed, P->ops,
                                    s));
    }
    return CAD_OK;
  }

  // g single steps at positions pos0 .. pos0 + g - 1, each feeding feed[0]
  cad_status chain(int64_t pos0, int g) {
    cad_program* P = pr;
    if (pos0 + g > cap) return prog_fail(CAD_E_CAPACITY, fmt("a step would reach position %lld of %lld", pos0 + g, cap));
    for (int k = 0; k < g; ++k) {
      PROG_HIP(launch_fsm_mask(P->st, P->t, lim, P->mask, 1, s));
      PROG_CALL(splice_rows(P->m, kv, pos0 + k, P->feed, 1, P->mask, CAD_COMMIT, nullptr, P->argmax, P->accepted,
                            nullptr, P->status, s));
      PROG_HIP(launch_fsm_advance(P->st, P->t, lim, P->argmax, 0, 0, P->line_start, P->hist, P->feed, P->ops, s));
    }
    launched_chained += g;
    return CAD_OK;
  }

  // single steps worth launching ahead (an upper bound on the steps before
  // the next decision that asks for a longer feed): from a state whose
  // pending feed is one id, or (`after_feed`) from the state a template or
  // copy feed leaves, whose first decision that feed's own forward takes
  int predict(const FsmState& h, bool after_feed) const {
    const cad_program_params& p = pr->p;
    const int du = decimal_digits(lim.units);
    int g;
    switch (h.state) {
      case FSM_AFTER_LT: g = 1; break;                    // the op type asks for a template
      case FSM_AWAIT_OP: g = after_feed ? 1 : 2; break;  // "<", then the op type
      case FSM_NUM_A:  // digits left in the first number, "-", the second number, the quote
        g = after_feed ? 2 * du + 1 : 2 * du - h.nd + 2;
        break;
      case FSM_NUM_B: g = du - h.nd + 1; break;
      case FSM_GEN_BODY:  // ids the body can still take before its length cap
        if (p.draft_k > 0) return 0;
        g = after_feed ? p.max_gen - 1 : p.max_gen - h.gen_len;
        break;
      default: g = 0;
    }
    // no decision is taken once the stream holds max_stream ids
    const int64_t room = (int64_t)lim.max_stream - h.stream_n + (after_feed ? 0 : 1);
    return (int)std::max<int64_t>(0, std::min<int64_t>({(int64_t)g, (int64_t)p.chain, room}));
  }
};

}  // namespace

extern "C" {

void cad_program_destroy(cad_program* pr) {
  if (!pr) return;
  (void)hipDeviceSynchronize();
  if (pr->h_st) (void)hipHostFree(pr->h_st);
  if (pr->dev) (void)hipFree(pr->dev);
  delete pr;
}

cad_status cad_program_create(cad_model* m, int64_t max_len, const cad_program_table* t,
                              const cad_program_params* p, cad_program** out) try {
  if (!out) return prog_fail(CAD_E_ARG, "out is NULL");
  *out = nullptr;
  if (!m || !t || !p) return prog_fail(CAD_E_ARG, "model/table/params is NULL");
  const cad_config* c = cad_model_config(m);
  if (c->loop_depth != 1) return prog_fail(CAD_E_ARG, "program decoding needs a model with loop_depth 1");
  if (p->max_doc < 1) return prog_fail(CAD_E_ARG, "max_doc must be >= 1");
  if (p->max_stream < 1) return prog_fail(CAD_E_ARG, "max_stream must be >= 1");
  if (p->max_ops < 1) return prog_fail(CAD_E_ARG, "max_ops must be >= 1");
  if (p->max_gen < 1) return prog_fail(CAD_E_ARG, "max_gen must be >= 1");
  if (p->draft_k < 0 || p->draft_k > 64) return prog_fail(CAD_E_ARG, "draft_k must be in [0, 64]");
  if (p->chain < 1 || p->chain > 64) return prog_fail(CAD_E_ARG, "chain must be in [1, 64]");
  if (p->draft_k + 1 > c->max_tokens) return prog_fail(CAD_E_CAPACITY, "draft_k + 1 exceeds the model's max_tokens");
  if (max_len < 1) return prog_fail(CAD_E_ARG, "max_len must be >= 1");
  const int32_t* ids = &t->lt;
  for (int i = 0; i < (int)(sizeof(cad_program_table) / 4); ++i)
    if (ids[i] < 0 || ids[i] >= c->vocab) return prog_fail(CAD_E_ARG, fmt("table id %lld outside the vocabulary", ids[i]));
  if ((int64_t)p->max_doc * 2 + p->max_stream + 2 * (int64_t)p->draft_k + 64 > INT32_MAX)
    return prog_fail(CAD_E_ARG, "max_doc / max_stream too large");
  cad_program* pr = new (std::nothrow) cad_program();
  if (!pr) return prog_fail(CAD_E_HIP, "host allocation failed");
  pr->m = m;
  pr->cfg = *c;
  memcpy(&pr->t, t, sizeof(FsmTable));
  pr->p = *p;
  pr->max_len = max_len;
  // one feed: a copy (quote, "/>", at most the whole document), a template
  // (at most four ids) or a verify (1 + draft_k)
  pr->feed_cap = std::max(p->max_doc + 2, p->draft_k + 1) + 8;
  // the stream stops at the first decision at or past max_stream: at most
  // one feed and one draft beyond it
  pr->hist_cap = p->max_doc + p->max_stream + pr->feed_cap + 2 * p->draft_k + 8;
  pr->mask_rows = std::max(c->max_tokens, p->draft_k + 1);
  pr->words = (c->vocab + 31) / 32;
  // copies can repeat the document: at most max_ops copies of it, plus the gen bodies
  pr->out_cap = (int32_t)std::min<int64_t>((int64_t)p->max_ops * p->max_doc + p->max_stream + 8, INT32_MAX);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = up256(off + bytes); return o; };
  const size_t o_st = take(sizeof(FsmState)), o_hist = take((size_t)pr->hist_cap * 4),
               o_feed = take((size_t)pr->feed_cap * 4), o_ops = take((size_t)(p->max_ops + 1) * FSM_OP_INTS * 4),
               o_ls = take((size_t)(p->max_doc + 1) * 4), o_pr = take((size_t)max_len * 4),
               o_am = take((size_t)std::max(c->max_tokens, p->draft_k + 1) * 4), o_acc = take(4), o_stat = take(4),
               o_tl = take(4), o_tp = take(8), o_out = take((size_t)pr->out_cap * 4),
               o_mask = take((size_t)pr->mask_rows * pr->words * 4);
  hipError_t e = hipMalloc(&pr->dev, off);
  if (e != hipSuccess) {
    delete pr;
    return prog_fail(CAD_E_HIP, std::string("hipMalloc: ") + hipGetErrorString(e));
  }
  char* b = (char*)pr->dev;
  pr->st = (FsmState*)(b + o_st);
  pr->hist = (int32_t*)(b + o_hist);
  pr->feed = (int32_t*)(b + o_feed);
  pr->ops = (int32_t*)(b + o_ops);
  pr->line_start = (int32_t*)(b + o_ls);
  pr->prompt = (int32_t*)(b + o_pr);
  pr->argmax = (int32_t*)(b + o_am);
  pr->accepted = (int32_t*)(b + o_acc);
  pr->status = (int32_t*)(b + o_stat);
  pr->tmp_len = (int32_t*)(b + o_tl);
  pr->tmp_pos = (int64_t*)(b + o_tp);
  pr->out = (int32_t*)(b + o_out);
  pr->mask = (uint32_t*)(b + o_mask);
  e = hipHostMalloc((void**)&pr->h_st, sizeof(FsmState), hipHostMallocDefault);
  if (e != hipSuccess) {
    pr->h_st = nullptr;
    cad_program_destroy(pr);
    return prog_fail(CAD_E_HIP, std::string("hipHostMalloc: ") + hipGetErrorString(e));
  }
  // every feed id must be valid before its first use (rows past a draft repeat the pending id)
  e = hipMemset(pr->dev, 0, off);
  if (e != hipSuccess) {
    cad_program_destroy(pr);
    return prog_fail(CAD_E_HIP, std::string("hipMemset: ") + hipGetErrorString(e));
  }
  *out = pr;
  return CAD_OK;
} catch (...) {
  // host containers and messages are C++: nothing they throw crosses the C ABI
  return cad::set_error(CAD_E_HIP, "host allocation failed");
}

cad_status cad_program_decode(cad_program* pr, const cad_kv* kv, const int32_t* prompt, int64_t L0,
                              const int32_t* doc, int32_t doc_n, const int32_t* line_start, int32_t n_lines,
                              int32_t unit_tokens, int32_t* stream_out, int32_t stream_cap, int32_t* ops_out,
                              int32_t* out, int32_t out_cap, cad_program_stats* stats, cad_stream stream) try {
  if (!pr || !kv || !prompt || !doc || !stats || !stream_out || !ops_out || !out)
    return prog_fail(CAD_E_ARG, "NULL argument");
  const cad_program_params& p = pr->p;
  if (L0 < 1 || L0 > pr->max_len) return prog_fail(CAD_E_ARG, fmt("prompt length %lld outside [1, %lld]", L0, pr->max_len));
  if (doc_n < 1 || doc_n > p.max_doc) return prog_fail(CAD_E_ARG, fmt("doc_n %lld outside [1, %lld]", doc_n, p.max_doc));
  if (unit_tokens != 0 && unit_tokens != 1) return prog_fail(CAD_E_ARG, "unit_tokens must be 0 or 1");
  if (!unit_tokens) {
    if (!line_start || n_lines < 1 || n_lines > doc_n) return prog_fail(CAD_E_ARG, "line table missing or n_lines outside [1, doc_n]");
    if (line_start[0] != 0 || line_start[n_lines] != doc_n) return prog_fail(CAD_E_ARG, "line_start must run from 0 to doc_n");
    for (int i = 0; i < n_lines; ++i)
      if (line_start[i + 1] < line_start[i]) return prog_fail(CAD_E_ARG, "line_start must be non-decreasing");
  }
  for (int64_t i = 0; i < L0; ++i)
    if (prompt[i] < 0 || prompt[i] >= pr->cfg.vocab) return prog_fail(CAD_E_ARG, fmt("prompt id %lld at %lld outside the vocabulary", prompt[i], i));
  for (int i = 0; i < doc_n; ++i)
    if (doc[i] < 0 || doc[i] >= pr->cfg.vocab) return prog_fail(CAD_E_ARG, fmt("document id %lld at %lld outside the vocabulary", doc[i], i));
  if (!kv->block_table || kv->max_blocks_per_seq < 1) return prog_fail(CAD_E_ARG, "bad KV cache");
  const int64_t need = L0 + p.max_stream + 2 * (int64_t)p.max_doc + 2 * p.draft_k + p.chain + 16;
  const int64_t cap = std::min<int64_t>((int64_t)kv->max_blocks_per_seq * CAD_KV_BLOCK, pr->max_len);
  if (need > cap)
    return prog_fail(CAD_E_CAPACITY, fmt("the decode may reach position %lld; the cache holds %lld", need, cap));
  memset(stats, 0, sizeof *stats);
  Decode d;
  d.pr = pr;
  d.kv = kv;
  d.s = (hipStream_t)stream;
  d.L0 = L0;
  d.cap = cap;
  FsmLimits& lim = d.lim;
  lim.units = unit_tokens ? doc_n : n_lines;
  lim.unit_tokens = unit_tokens;
  lim.max_ops = p.max_ops;
  lim.max_gen = p.max_gen;
  lim.max_stream = p.max_stream;
  lim.vocab_words = pr->words;
  lim.doc_n = doc_n;
  lim.hist_cap = pr->hist_cap;
  lim.draft_k = p.draft_k;
  hipStream_t s = d.s;
  PROG_HIP(hipMemcpyAsync(pr->hist, doc, (size_t)doc_n * 4, hipMemcpyHostToDevice, s));
  if (!unit_tokens)
    PROG_HIP(hipMemcpyAsync(pr->line_start, line_start, (size_t)(n_lines + 1) * 4, hipMemcpyHostToDevice, s));
  PROG_HIP(hipMemcpyAsync(pr->prompt, prompt, (size_t)L0 * 4, hipMemcpyHostToDevice, s));
  PROG_HIP(hipMemsetAsync(pr->status, 0, 4, s));
  PROG_HIP(launch_fsm_init(pr->st, s));
  // the prompt, its last row deciding the first op boundary
  const int T = pr->cfg.max_tokens;
  for (int64_t off = 0; off < L0; off += T) {
    const int rows = (int)std::min<int64_t>(T, L0 - off);
    const bool last = off + rows == L0;
    if (last) PROG_HIP(launch_fsm_mask(pr->st, pr->t, lim, pr->mask, rows, s));
    PROG_CALL(splice_rows(pr->m, kv, off, pr->prompt + off, rows, last ? pr->mask : nullptr, CAD_COMMIT, nullptr,
                          pr->argmax, pr->accepted, nullptr, pr->status, s));
  }
  PROG_HIP(launch_fsm_advance(pr->st, pr->t, lim, pr->argmax, (int)((L0 - 1) % T), 1, pr->line_start, pr->hist,
                              pr->feed, pr->ops, s));
  stats->forwards = 1;
  int64_t feeds = 0;
  // every round trip feeds at least one program id, and the stream stops
  // growing at max_stream plus one feed and one draft
  const int64_t max_trips = (int64_t)pr->hist_cap + 8;
  for (int64_t trip = 0;; ++trip) {
    if (trip > max_trips) return prog_fail(CAD_E_HIP, "the automaton made no progress");
    PROG_HIP(hipMemcpyAsync(pr->h_st, pr->st, sizeof(FsmState), hipMemcpyDeviceToHost, s));
    PROG_HIP(hipStreamSynchronize(s));
    stats->host_syncs += 1;
    const FsmState h = *pr->h_st;
    if (h.action == FSM_ACT_STOP || h.action == FSM_ACT_NONE) break;
    const int64_t S = h.stream_n;
    const int64_t pos = L0 + S - h.feed_n;  // the pending feed's first position
    if (h.action == FSM_ACT_LAST) {
      PROG_CALL(d.splice_feed(pos, h.feed_n, false));
      feeds += 1;
      break;
    }
    if (h.action == FSM_ACT_FEED) {
      PROG_CALL(d.splice_feed(pos, h.feed_n, true));
      feeds += 1;
      // if that forward's decision is a single id, it is fed at L0 + S
      PROG_CALL(d.chain(L0 + S, d.predict(h, true)));
      continue;
    }
    // FSM_ACT_STEP: the pending id sits at L0 + S - 1
    if (h.state == FSM_GEN_BODY && p.draft_k > 0) {
      PROG_HIP(launch_fsm_draft(pr->st, pr->t, lim, pr->hist, pr->feed, pr->mask, pr->tmp_len, pr->tmp_pos, s));
      PROG_CALL(splice_rows(pr->m, kv, pos, pr->feed, p.draft_k + 1, pr->mask, CAD_VERIFY, &pr->st->feed_n,
                            pr->argmax, pr->accepted, nullptr, pr->status, s));
      PROG_HIP(launch_fsm_verified(pr->st, pr->t, lim, pr->argmax, pr->accepted, pr->line_start, pr->hist, pr->feed,
                                   pr->ops, s));
      feeds += 1;
      continue;
    }
    const int g = std::max(1, d.predict(h, false));
    PROG_CALL(d.chain(pos, g));
  }
  PROG_HIP(launch_fsm_resolve(pr->st, lim, pr->line_start, pr->hist, pr->ops, pr->out, pr->out_cap, s));
  PROG_HIP(hipMemcpyAsync(pr->h_st, pr->st, sizeof(FsmState), hipMemcpyDeviceToHost, s));
  int32_t dev_status = 0;
  PROG_HIP(hipMemcpyAsync(&dev_status, pr->status, 4, hipMemcpyDeviceToHost, s));
  PROG_HIP(hipStreamSynchronize(s));
  const FsmState h = *pr->h_st;
  stats->forwards += feeds + h.chained;
  stats->idle_steps = d.launched_chained - h.chained;
  stats->decisions = h.decisions;
  stats->masked_steps = h.masked;
  stats->forced_prefills = h.forced;
  stats->copies = h.copies;
  stats->copied_tokens = h.copied;
  stats->drafts = h.drafts;
  stats->draft_tokens = h.draft_tokens;
  stats->draft_accepted = h.draft_accepted;
  stats->stream_n = h.stream_n;
  stats->n_ops = h.n_ops + (h.state == FSM_GEN_BODY ? 1 : 0);
  stats->out_n = h.out_n;
  stats->fsm_error = h.error;
  stats->dev_status = dev_status;
  const int32_t ns = std::min(h.stream_n, stream_cap), no = std::min(h.out_n, std::min(out_cap, pr->out_cap));
  if (ns > 0) PROG_HIP(hipMemcpy(stream_out, pr->hist + doc_n, (size_t)ns * 4, hipMemcpyDeviceToHost));
  if (stats->n_ops > 0)
    PROG_HIP(hipMemcpy(ops_out, pr->ops, (size_t)stats->n_ops * FSM_OP_INTS * 4, hipMemcpyDeviceToHost));
  if (no > 0) PROG_HIP(hipMemcpy(out, pr->out, (size_t)no * 4, hipMemcpyDeviceToHost));
  if (h.stream_n > stream_cap || h.out_n > out_cap || h.out_n > pr->out_cap)
    return prog_fail(CAD_E_CAPACITY, fmt("results longer than their buffers (stream %lld, output %lld)", h.stream_n,
                                         h.out_n));
  return CAD_OK;
} catch (...) {
  // host containers and messages are C++: nothing they throw crosses the C ABI
  return cad::set_error(CAD_E_HIP, "host allocation failed");
}

}  // extern "C"
