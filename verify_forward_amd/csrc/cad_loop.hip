// CopyLoop's concurrent decode pipeline on a looped model: the host
// scheduler that drives cad_loop_step (CopyLoop §2 "Block Construction",
// "Shallow Screening", "Concurrent Pipeline", "Full-Depth Verification";
// §A.1 "Decoding algorithm": initialisation from the prompt, admission,
// pruning at the screening depth, commitment at full depth, admission
// limit).
//
// Every tick advances every block in flight by one depth in one call of
// cad_loop_step (each block on its own depth's cache); the blocks that reach
// the screening depth or the full depth are read out in the same call, and
// right after it the device makes the context-copy proposal for the block
// that would follow each readout (the screened block's successor, and the
// correction after a full-depth readout), so the host reads decisions and
// proposals back with one synchronisation per tick with a readout.  (A head
// that waits for room gets its proposal when it is admitted, with one more.)
//
// Rules (the plainest reading of the pages where they leave a step open):
//   * the prompt is prefilled at every depth; its last full-depth prediction
//     is the first token, and the first block's head;
//   * a block is [head, tail]: the tail is up to K tokens copied after the
//     longest earlier match of the history's suffix (n-gram lengths
//     max_ngram down to min_ngram, most recent occurrence);
//   * at depth ds the tail is cut to the longest prefix agreeing with the
//     predictions one position earlier (the pruned rows are released), and
//     the last survivor's prediction heads the next block;
//   * at depth D the tail is verified the same way against the full-depth
//     predictions: the first mismatch commits the full-depth token as a
//     correction and discards the rest of the block and every younger block;
//     a fully verified block's last prediction is the next token, which must
//     equal the next block's head (else that block and its descendants are
//     discarded and a correction block takes their place);
//   * the rows in flight never exceed max_rows: a block admitted with r free
//     rows keeps at most r - 1 copied tokens, and a head with no free row
//     waits;
//   * blocks are processed oldest first after each tick.
#include <cstring>
#include <deque>
#include <new>
#include <string>
#include <vector>

#include "cad_internal.h"

namespace {

struct Block {
  int64_t pos = 0;
  std::vector<int32_t> toks;
  int32_t depth = 0;
  int32_t slot = -1;
  bool in_flight = false;
  int32_t ready = -1;  // waiting head: proposal slot already computed on the device this tick (-1: none)
};

constexpr int kPropSlots = 2;  // proposals made after a tick: 0 after screening, 1 after full depth

cad_status loop_fail(cad_status s, const std::string& msg) { return cad::set_error(s, msg.c_str()); }

}  // namespace

struct cad_loop {
  cad_model* m = nullptr;
  cad_config cfg{};
  cad_loop_params p{};
  int64_t max_len = 0;
  int32_t slot_rows = 0, n_slots = 0, tick_rows = 0, prefill_rows = 0;
  void* dev = nullptr;       // one device allocation
  float* state = nullptr;    // [n_slots * slot_rows][d_model]
  int32_t* d_tokens = nullptr;
  int32_t* d_argmax = nullptr;
  int32_t* d_accepted = nullptr;
  int32_t* d_hist = nullptr;
  int32_t* d_prop = nullptr;      // [1 + kPropSlots][65]: tokens[64], then the length
  int64_t* d_prop_pos = nullptr;  // [1 + kPropSlots]
  int32_t* d_prop_head = nullptr; // [kPropSlots]
  int32_t* d_status = nullptr;
  int32_t* d_pf_sargmax = nullptr;
  int32_t* d_pf_argmax = nullptr;
  int32_t* d_pf_misc = nullptr;
  void* host = nullptr;      // one pinned host allocation
  int32_t* h_tokens[2] = {nullptr, nullptr};  // tick tokens, double-buffered
  hipEvent_t tok_copied[2] = {nullptr, nullptr};  // the last copy out of each token buffer
  int32_t* h_argmax = nullptr;
  int32_t* h_accepted = nullptr;
  int32_t* h_hist = nullptr;
  int32_t* h_prop = nullptr;      // [1 + kPropSlots][65]
};

namespace {

size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

#define LOOP_HIP(expr)                                                                               \
  do {                                                                                               \
    hipError_t e_ = (expr);                                                                          \
    if (e_ != hipSuccess) return loop_fail(CAD_E_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

// a C-ABI call inside the scheduler: its error message is kept
#define LOOP_CALL(expr)                                                     \
  do {                                                                      \
    cad_status s_ = (expr);                                                 \
    if (s_ != CAD_OK) return loop_fail(s_, std::string(cad_last_error())); \
  } while (0)

struct Run {
  cad_loop* lp;
  const cad_kv* kv;
  hipStream_t s;
  cad_loop_stats st{};
  std::vector<int32_t> hist;     // tokens at positions 0 .. (prompt, committed, in flight)
  size_t dev_valid = 0;          // leading positions of hist already on the device
  std::vector<int32_t> out;
  std::deque<Block> blocks;      // oldest first; the youngest may wait for admission
  std::vector<int32_t> free_slots;

  int32_t rows_in_flight() const {
    int32_t n = 0;
    for (const Block& b : blocks)
      if (b.in_flight) n += (int32_t)b.toks.size();
    return n;
  }

  void truncate_hist(size_t n) {
    if (hist.size() > n) hist.resize(n);
    if (dev_valid > n) dev_valid = n;
  }

  void release(Block& b) {
    if (b.slot >= 0) free_slots.push_back(b.slot);
    b.slot = -1;
  }

  // drop blocks[i..] (discarded continuations)
  void discard_from(size_t i) {
    for (size_t j = i; j < blocks.size(); ++j)
      if (blocks[j].in_flight) {
        st.discarded += (int64_t)blocks[j].toks.size();
        release(blocks[j]);
      }
    blocks.erase(blocks.begin() + (std::ptrdiff_t)i, blocks.end());
  }

  // the youngest entry, if it waits: admit it with a context-copy tail when
  // a row is free (proposal on the device, one synchronisation)
  // upload the host history's changes to the device copy
  cad_status sync_hist() {
    const size_t n = hist.size() - dev_valid;
    if (n > 0) {
      std::memcpy(lp->h_hist, hist.data() + dev_valid, n * 4);
      LOOP_HIP(hipMemcpyAsync(lp->d_hist + dev_valid, lp->h_hist, n * 4, hipMemcpyHostToDevice, s));
      dev_valid = hist.size();
    }
    return CAD_OK;
  }

  cad_status admit_waiting() {
    if (blocks.empty() || blocks.back().in_flight) return CAD_OK;
    Block& b = blocks.back();
    const int32_t room = lp->p.max_rows - rows_in_flight();
    if (room < 1) {
      b.ready = -1;  // a later admission proposes again
      return CAD_OK;
    }
    truncate_hist((size_t)b.pos);
    hist.push_back(b.toks[0]);
    int32_t n_tail = 0;
    const int32_t* tail = nullptr;
    if (lp->p.max_copy > 0 && room > 1) {
      int slot = b.ready;
      if (slot < 0) {
        // no proposal made on the device after the last tick: make one now
        slot = kPropSlots;
        cad_status r = sync_hist();
        if (r != CAD_OK) return r;
        int32_t* dp = lp->d_prop + slot * 65;
        LOOP_CALL(cad_propose_suffix_match(lp->d_hist, (int64_t)hist.size(), lp->p.max_ngram, lp->p.min_ngram,
                                           lp->p.max_copy, dp, dp + 64, lp->d_prop_pos + slot, s));
        LOOP_HIP(hipMemcpyAsync(lp->h_prop + slot * 65, dp, 65 * 4, hipMemcpyDeviceToHost, s));
        LOOP_HIP(hipStreamSynchronize(s));
        ++st.host_syncs;
      }
      tail = lp->h_prop + slot * 65;
      n_tail = tail[64];
      if (n_tail > room - 1) n_tail = room - 1;
      if (n_tail < 0) n_tail = 0;
    }
    b.ready = -1;
    b.toks.resize(1);
    for (int32_t j = 0; j < n_tail; ++j) b.toks.push_back(tail[j]);
    for (int32_t j = 0; j < n_tail; ++j) hist.push_back(tail[j]);
    // blocks in flight sit at distinct depths, so the loop_depth slots never run out
    if (free_slots.empty()) return loop_fail(CAD_E_ARG, "no free pipeline slot (more blocks in flight than depths)");
    b.slot = free_slots.back();
    free_slots.pop_back();
    b.in_flight = true;
    ++st.blocks;
    st.proposed += n_tail;
    return CAD_OK;
  }

  cad_status prefill(const int32_t* prompt, int64_t L0) {
    // the prompt through every depth (a looped splice screened at the full
    // depth keeps every row), in chunks of at most prefill_rows
    std::memcpy(lp->h_hist, prompt, (size_t)L0 * 4);
    LOOP_HIP(hipMemcpyAsync(lp->d_hist, lp->h_hist, (size_t)L0 * 4, hipMemcpyHostToDevice, s));
    hist.assign(prompt, prompt + L0);
    dev_valid = (size_t)L0;
    const int32_t D = lp->cfg.loop_depth;
    int64_t last = 0;
    for (int64_t c0 = 0; c0 < L0; c0 += lp->prefill_rows) {
      const int32_t n = (int32_t)std::min<int64_t>(lp->prefill_rows, L0 - c0);
      LOOP_CALL(cad_splice_forward_looped(lp->m, kv, c0, lp->d_hist + c0, n, D, nullptr, lp->d_pf_sargmax,
                                          lp->d_pf_misc, lp->d_pf_argmax, lp->d_pf_misc + 1, nullptr,
                                          lp->d_status, s));
      last = n - 1;
    }
    LOOP_HIP(hipMemcpyAsync(lp->h_argmax, lp->d_pf_sargmax + last, 4, hipMemcpyDeviceToHost, s));
    LOOP_HIP(hipStreamSynchronize(s));
    ++st.host_syncs;
    return CAD_OK;
  }

  cad_status decode(const int32_t* prompt, int64_t L0, int32_t n_new, int32_t* out_tokens) {
    const int32_t D = lp->cfg.loop_depth, ds = lp->p.screen_depth;
    for (int32_t i = lp->n_slots - 1; i >= 0; --i) free_slots.push_back(i);
    cad_status r = prefill(prompt, L0);
    if (r != CAD_OK) return r;
    const int32_t first = lp->h_argmax[0];
    out.push_back(first);
    Block b0;
    b0.pos = L0;
    b0.toks.push_back(first);
    blocks.push_back(b0);
    r = admit_waiting();
    if (r != CAD_OK) return r;
    std::vector<cad_loop_group> groups;
    std::vector<size_t> live;  // index in `blocks` of each group
    while ((int32_t)out.size() < n_new) {
      groups.clear();
      live.clear();
      int32_t total = 0;
      // a tick without a readout does not synchronise: the token buffer is
      // reused only once the copy out of it two ticks ago has completed
      int32_t* h_tok = lp->h_tokens[st.ticks & 1];
      LOOP_HIP(hipEventSynchronize(lp->tok_copied[st.ticks & 1]));
      bool any_read = false;
      for (size_t i = 0; i < blocks.size(); ++i) {
        Block& b = blocks[i];
        if (!b.in_flight) continue;
        cad_loop_group g;
        g.pos = b.pos;
        g.rows = (int32_t)b.toks.size();
        g.depth = b.depth;
        g.state = b.slot * lp->slot_rows;
        g.readout = (b.depth + 1 == ds || b.depth + 1 == D) ? 1 : 0;
        any_read |= g.readout != 0;
        for (int32_t t : b.toks) h_tok[total++] = t;
        groups.push_back(g);
        live.push_back(i);
      }
      if (groups.empty()) return loop_fail(CAD_E_ARG, "pipeline empty before the decode finished");
      const bool propose = any_read && lp->p.max_copy > 0;
      if (propose) {
        // the device history must hold every token in flight for the proposals below
        cad_status r2 = sync_hist();
        if (r2 != CAD_OK) return r2;
      }
      LOOP_HIP(hipMemcpyAsync(lp->d_tokens, h_tok, (size_t)total * 4, hipMemcpyHostToDevice, s));
      LOOP_HIP(hipEventRecord(lp->tok_copied[st.ticks & 1], s));
      LOOP_CALL(cad_loop_step(lp->m, kv, (int32_t)groups.size(), groups.data(), lp->d_tokens, lp->state,
                              lp->n_slots * lp->slot_rows, nullptr, lp->d_argmax, lp->d_accepted, nullptr,
                              lp->d_status, s));
      ++st.ticks;
      st.rows_run += total;
      if (any_read) {
        if (propose) {
          // proposals for the successor of the screened block (slot 0) and for
          // the token after the full-depth block (slot 1), screening first: the
          // full-depth one may write a correction into the history
          int32_t o = 0;
          for (int pass = 0; pass < kPropSlots; ++pass) {
            o = 0;
            for (size_t k = 0; k < groups.size(); ++k) {
              const int32_t after = groups[k].depth + 1;
              if (groups[k].readout && ((pass == 0 && after == ds) || (pass == 1 && after == D))) {
                int32_t* dp = lp->d_prop + pass * 65;
                LOOP_HIP(cad::launch_propose_next(lp->d_hist, groups[k].pos, lp->d_accepted + k, lp->d_argmax + o,
                                             lp->p.max_ngram, lp->p.min_ngram, lp->p.max_copy, dp, dp + 64,
                                             lp->d_prop_pos + pass, lp->d_prop_head + pass, s));
              }
              o += groups[k].rows;
            }
          }
          LOOP_HIP(hipMemcpyAsync(lp->h_prop, lp->d_prop, kPropSlots * 65 * 4, hipMemcpyDeviceToHost, s));
        }
        LOOP_HIP(hipMemcpyAsync(lp->h_argmax, lp->d_argmax, (size_t)total * 4, hipMemcpyDeviceToHost, s));
        LOOP_HIP(hipMemcpyAsync(lp->h_accepted, lp->d_accepted, groups.size() * 4, hipMemcpyDeviceToHost, s));
        LOOP_HIP(hipStreamSynchronize(s));
        ++st.host_syncs;
        if (propose) {
          // the device wrote each proposal's head into its history copy; the
          // host history takes those positions over when it admits or corrects
          for (size_t k = 0; k < groups.size(); ++k)
            if (groups[k].readout) {
              const size_t at = (size_t)(groups[k].pos + lp->h_accepted[k]);
              if (dev_valid > at) dev_valid = at;
            }
        }
      }
      // per block of this tick: its readout (row offset in the tick, accepted)
      std::vector<int32_t> row0(blocks.size(), -1), accd(blocks.size(), 0);
      {
        int32_t o = 0;
        for (size_t k = 0; k < live.size(); ++k) {
          if (groups[k].readout) {
            row0[live[k]] = o;
            accd[live[k]] = lp->h_accepted[k];
          }
          o += groups[k].rows;
          blocks[live[k]].depth += 1;
        }
      }
      size_t i = 0;
      while (i < blocks.size()) {
        Block& b = blocks[i];
        if (!b.in_flight || row0[i] < 0) {
          ++i;
          continue;
        }
        const int32_t* a = lp->h_argmax + row0[i];
        const int32_t m = (int32_t)b.toks.size();
        if (b.depth == D) {
          // full-depth verification of the tail (the head is verified already)
          const int32_t acc = accd[i];
          for (int32_t j = 1; j < acc; ++j) out.push_back(b.toks[j]);
          const int32_t nxt = a[acc - 1];
          st.rejected += m - acc;
          const int64_t pos_next = b.pos + acc;
          release(b);
          blocks.erase(blocks.begin() + (std::ptrdiff_t)i);
          row0.erase(row0.begin() + (std::ptrdiff_t)i);
          accd.erase(accd.begin() + (std::ptrdiff_t)i);
          if (i < blocks.size() && acc == m && blocks[i].toks[0] == nxt) {
            out.push_back(nxt);  // the next block's head is the verified token
          } else {
            discard_from(i);
            row0.resize(blocks.size());
            accd.resize(blocks.size());
            truncate_hist((size_t)pos_next);
            out.push_back(nxt);
            Block c;
            c.pos = pos_next;
            c.toks.push_back(nxt);
            c.ready = 1;  // proposed on the device after this tick
            blocks.push_back(c);
            row0.push_back(-1);
            accd.push_back(0);
          }
          continue;
        }
        if (b.depth == ds) {
          // shallow screening: the agreeing prefix survives, the rest is released
          const int32_t keep = accd[i];
          st.screened_out += m - keep;
          b.toks.resize(keep);
          truncate_hist((size_t)(b.pos + keep));
          if (i + 1 == blocks.size()) {
            Block nb;
            nb.pos = b.pos + keep;
            nb.toks.push_back(a[keep - 1]);
            nb.ready = 0;  // proposed on the device after this tick
            blocks.push_back(nb);
            row0.push_back(-1);
            accd.push_back(0);
          }
        }
        ++i;
      }
      r = admit_waiting();
      if (r != CAD_OK) return r;
    }
    st.committed = (int64_t)out.size();
    for (int32_t j = 0; j < n_new; ++j) out_tokens[j] = out[j];
    LOOP_HIP(hipMemcpyAsync(lp->h_accepted, lp->d_status, 4, hipMemcpyDeviceToHost, s));
    LOOP_HIP(hipStreamSynchronize(s));
    ++st.host_syncs;
    st.dev_status = lp->h_accepted[0];
    return CAD_OK;
  }
};

}  // namespace

extern "C" {

cad_status cad_loop_create(cad_model* m, int64_t max_len, const cad_loop_params* p, cad_loop** out) {
  if (!out) return loop_fail(CAD_E_ARG, "out is NULL");
  *out = nullptr;
  if (!m || !p) return loop_fail(CAD_E_ARG, "model/params is NULL");
  const cad_config* c = cad_model_config(m);
  if (c->loop_depth < 2) return loop_fail(CAD_E_ARG, "model is not looped (loop_depth < 2)");
  if (p->screen_depth < 1 || p->screen_depth >= c->loop_depth)
    return loop_fail(CAD_E_ARG, "screen_depth must be in [1, loop_depth)");
  if (p->max_copy < 0 || p->max_copy > 64) return loop_fail(CAD_E_ARG, "max_copy must be in [0, 64]");
  if (p->min_ngram < 1 || p->max_ngram < p->min_ngram || p->max_ngram > 64)
    return loop_fail(CAD_E_ARG, "need 1 <= min_ngram <= max_ngram <= 64");
  if (p->max_rows < 1) return loop_fail(CAD_E_ARG, "max_rows must be >= 1");
  if (max_len < 1) return loop_fail(CAD_E_ARG, "max_len must be >= 1");
  cad_loop* lp = new (std::nothrow) cad_loop();
  if (!lp) return loop_fail(CAD_E_HIP, "host allocation failed");
  lp->m = m;
  lp->cfg = *c;
  lp->p = *p;
  lp->max_len = max_len;
  lp->slot_rows = p->max_copy + 1;
  lp->n_slots = c->loop_depth;  // blocks in flight sit at distinct depths
  lp->tick_rows = std::min(p->max_rows, lp->n_slots * lp->slot_rows);
  lp->prefill_rows = c->max_tokens;
  if (lp->tick_rows > c->max_tokens) {
    delete lp;
    return loop_fail(CAD_E_CAPACITY, "max_rows exceeds the model's max_tokens");
  }
  const int64_t d = c->d_model, srows = (int64_t)lp->n_slots * lp->slot_rows, T = c->max_tokens;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = up256(off + bytes); return o; };
  const size_t o_state = take(srows * d * 4), o_tok = take(srows * 4), o_am = take(srows * 4),
               o_acc = take(CAD_MAX_SEQS * 4), o_hist = take(max_len * 4), o_prop = take((1 + kPropSlots) * 65 * 4),
               o_phead = take(kPropSlots * 4), o_ppos = take((1 + kPropSlots) * 8), o_st = take(4),
               o_pfs = take(T * 4), o_pfa = take(T * 4), o_pfm = take(2 * 4);
  hipError_t e = hipMalloc(&lp->dev, off);
  if (e != hipSuccess) {
    delete lp;
    return loop_fail(CAD_E_HIP, std::string("hipMalloc: ") + hipGetErrorString(e));
  }
  char* b = (char*)lp->dev;
  lp->state = (float*)(b + o_state);
  lp->d_tokens = (int32_t*)(b + o_tok);
  lp->d_argmax = (int32_t*)(b + o_am);
  lp->d_accepted = (int32_t*)(b + o_acc);
  lp->d_hist = (int32_t*)(b + o_hist);
  lp->d_prop = (int32_t*)(b + o_prop);
  lp->d_prop_head = (int32_t*)(b + o_phead);
  lp->d_prop_pos = (int64_t*)(b + o_ppos);
  lp->d_status = (int32_t*)(b + o_st);
  lp->d_pf_sargmax = (int32_t*)(b + o_pfs);
  lp->d_pf_argmax = (int32_t*)(b + o_pfa);
  lp->d_pf_misc = (int32_t*)(b + o_pfm);
  size_t hoff = 0;
  auto htake = [&](size_t bytes) { size_t o = hoff; hoff = up256(hoff + bytes); return o; };
  const size_t h_tok0 = htake(srows * 4), h_tok1 = htake(srows * 4), h_am = htake(std::max<int64_t>(srows, 1) * 4), h_acc = htake(CAD_MAX_SEQS * 4),
               h_hist = htake(max_len * 4), h_prop = htake((1 + kPropSlots) * 65 * 4);
  e = hipHostMalloc(&lp->host, hoff, hipHostMallocDefault);
  if (e != hipSuccess) {
    (void)hipFree(lp->dev);
    delete lp;
    return loop_fail(CAD_E_HIP, std::string("hipHostMalloc: ") + hipGetErrorString(e));
  }
  char* h = (char*)lp->host;
  lp->h_tokens[0] = (int32_t*)(h + h_tok0);
  lp->h_tokens[1] = (int32_t*)(h + h_tok1);
  for (int k = 0; k < 2; ++k) {
    e = hipEventCreateWithFlags(&lp->tok_copied[k], hipEventDisableTiming);
    if (e != hipSuccess) {
      cad_loop_destroy(lp);
      return loop_fail(CAD_E_HIP, std::string("hipEventCreate: ") + hipGetErrorString(e));
    }
  }
  lp->h_argmax = (int32_t*)(h + h_am);
  lp->h_accepted = (int32_t*)(h + h_acc);
  lp->h_hist = (int32_t*)(h + h_hist);
  lp->h_prop = (int32_t*)(h + h_prop);
  *out = lp;
  return CAD_OK;
}

void cad_loop_destroy(cad_loop* lp) {
  if (!lp) return;
  (void)hipDeviceSynchronize();
  for (hipEvent_t e : lp->tok_copied)
    if (e) (void)hipEventDestroy(e);
  (void)hipFree(lp->dev);
  (void)hipHostFree(lp->host);
  delete lp;
}

cad_status cad_loop_decode(cad_loop* lp, const cad_kv* kv, const int32_t* prompt, int64_t L0, int32_t n_new,
                           int32_t* out_tokens, cad_loop_stats* stats, cad_stream stream) {
  if (!lp || !kv || !prompt || !out_tokens) return loop_fail(CAD_E_ARG, "NULL argument");
  if (L0 < 1 || n_new < 1) return loop_fail(CAD_E_ARG, "need a prompt and at least one new token");
  const int64_t need = L0 + n_new + (int64_t)lp->n_slots * lp->slot_rows;
  if (need > lp->max_len) return loop_fail(CAD_E_CAPACITY, "prompt + new tokens + blocks in flight exceed max_len");
  if (need > (int64_t)kv->max_blocks_per_seq * CAD_KV_BLOCK)
    return loop_fail(CAD_E_CAPACITY, "prompt + new tokens + blocks in flight exceed the block table");
  Run run;
  run.lp = lp;
  run.kv = kv;
  run.s = (hipStream_t)stream;
  LOOP_HIP(hipMemsetAsync(lp->d_status, 0, 4, run.s));
  const cad_status r = run.decode(prompt, L0, n_new, out_tokens);
  if (stats) *stats = run.st;
  return r;
}

}  // extern "C"
