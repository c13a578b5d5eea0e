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
//
// Second-readout branching (CopyLoop §A.2, branch_depth = d2 > 0): a block
// read out at d2 whose last surviving row predicts another token than the
// depth-ds prediction that headed its child admits a second child headed by
// the d2 prediction.  The two children and their descendants form two
// lines over the same positions: blocks older than the fork belong to both,
// the first line maps its positions through block-table row 0 and the
// second through row 1 (the caller's row 0 up to the block where the fork
// starts, spare blocks after it), with its own device history.  The slots
// of older positions inside that block are copied to the second line's
// block when the fork is made and after every tick while it is live (older
// blocks keep writing them at their later depths).  At the parent's
// full-depth readout the line whose head is the verified token is kept --
// the second line's K/V are then copied into row 0's blocks and its history
// becomes the history -- or neither (a correction block follows).  At most
// one fork is live; it needs its parent's first child in flight, a free row
// and a free slot.  The second line's screened successors and the second
// child itself are proposed on the device after the tick like the first
// line's (the child's history is copied from its line's, with the depth-d2
// head written after it).
#include <algorithm>
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
  int32_t line = -1;   // -1: older than any live fork (both lines); 0 / 1: the first / second child's line
  int32_t tick_row = 0;  // block-table row of its group in the last tick (its device proposal's history)
  uint64_t id = 0;
};

// proposals made on the device after a tick: the successor of the block
// screened on the first line's history (0), the token after the full-depth
// block (1), the successor of the block screened on the second line's (2),
// and the second child's head of a block read out at the branch depth on
// the first or the second line's history (3, 4); then the slot of a
// proposal made when a head is admitted
constexpr int kPropScreen0 = 0, kPropFull = 1, kPropScreen1 = 2, kPropFork = 3, kPropSlots = 5;
// What the host reads back after a tick, contiguous on the device and in
// pinned memory so that one copy brings it: the groups' acceptance, the
// proposals ([1 + kPropSlots][65]: tokens[64], then the length; padded to
// 16 bytes), then the argmax of every row.
constexpr int kRbProp = CAD_MAX_SEQS, kRbArgmax = kRbProp + ((1 + kPropSlots) * 65 + 3) / 4 * 4;

// Copy cache slots [lo, hi) of block `src` into block `dst` at every cache
// index of a paged pool (a looped model's depths): one work-group per (pair,
// cache index, KV head).  pairs: [n_pairs][4] = src, dst, lo, hi (checked
// by the host: blocks in [0, num_blocks), 0 <= lo < hi <= 16).
template <typename T>
__global__ void __launch_bounds__(256) k_kv_copy(T* __restrict__ k, T* __restrict__ v, int64_t cache_stride, int hd,
                                                 const int32_t* __restrict__ pairs) {
  const int pr = blockIdx.x, h = blockIdx.z, hkv = gridDim.z;
  const int lo = pairs[4 * pr + 2], n = pairs[4 * pr + 3] - lo;
  const int64_t blk = (int64_t)hkv * CAD_KV_BLOCK * hd;
  const int64_t head = (int64_t)blockIdx.y * cache_stride + (int64_t)h * CAD_KV_BLOCK * hd;
  T* ks = k + pairs[4 * pr] * blk + head;
  T* kd = k + pairs[4 * pr + 1] * blk + head;
  T* vs = v + pairs[4 * pr] * blk + head;
  T* vd = v + pairs[4 * pr + 1] * blk + head;
  // K [slot][hd]: slots lo .. lo + n - 1 are contiguous
  for (int i = threadIdx.x; i < n * hd; i += blockDim.x) kd[lo * hd + i] = ks[lo * hd + i];
  // V [hd][slot]: n slots of each dimension
  for (int dd = threadIdx.x; dd < hd; dd += blockDim.x)
    for (int sl = lo; sl < lo + n; ++sl) vd[dd * CAD_KV_BLOCK + sl] = vs[dd * CAD_KV_BLOCK + sl];
}

hipError_t launch_kv_copy(int dtype, void* k, void* v, int64_t cache_stride, int n_cache, int hkv, int hd,
                          const int32_t* pairs, int n_pairs, hipStream_t s) {
  if (n_pairs < 1) return hipSuccess;
  const dim3 grid((unsigned)n_pairs, (unsigned)n_cache, (unsigned)hkv);
  if (dtype == CAD_BF16)
    hipLaunchKernelGGL((k_kv_copy<cad::bf16_t>), grid, dim3(256), 0, s, (cad::bf16_t*)k, (cad::bf16_t*)v, cache_stride,
                       hd, pairs);
  else
    hipLaunchKernelGGL((k_kv_copy<float>), grid, dim3(256), 0, s, (float*)k, (float*)v, cache_stride, hd, pairs);
  return hipGetLastError();
}

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
  int32_t* d_hist = nullptr;      // history of the first line (device)
  int32_t* d_hist2 = nullptr;     // history of the second line (branching)
  int32_t* d_spec[2] = {nullptr, nullptr};  // a possible second child's history, per line (branching)
  int32_t* d_table = nullptr;     // [2][tbl_stride] block-table rows the pipeline runs on
  int32_t* d_pairs = nullptr;     // [max_pairs][4] KV block copies
  int32_t tbl_stride = 0, max_pairs = 0;
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
  hipEvent_t hist_copied = nullptr;               // the last copy out of the history staging buffer
  int32_t* h_argmax = nullptr;
  int32_t* h_accepted = nullptr;
  int32_t* h_hist = nullptr;
  int32_t* h_prop = nullptr;      // [1 + kPropSlots][65]
  int32_t* h_table = nullptr;     // [2][tbl_stride]
  int32_t* h_pairs = nullptr;     // [max_pairs][4]
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
  const cad_kv* user_kv;
  cad_kv kv_run{};               // branching: the caller's pool through the pipeline's own table rows
  const cad_kv* kv = nullptr;    // what the ticks run on
  hipStream_t s;
  cad_loop_stats st{};
  // per line (0: the first line, and every block before a fork; 1: the
  // second line while a fork is live): tokens at positions 0 .. (prompt,
  // committed, in flight), the leading positions already on the device
  std::vector<int32_t> hist[2];
  size_t dev_valid[2] = {0, 0};
  int32_t* d_hist[2] = {nullptr, nullptr};
  int32_t* d_spec[2] = {nullptr, nullptr};  // branching: histories made for a possible second child
  std::vector<int32_t> out;
  std::deque<Block> blocks;      // oldest first; waiting heads are admitted in this order
  std::vector<int32_t> free_slots;
  uint64_t next_id = 1;
  // the live fork
  bool fork_live = false;
  uint64_t fork_parent = 0;
  int64_t fork_pos = 0;          // first position of the two children
  std::vector<int32_t> row0, spare;  // the request's blocks (block-table row 0) and the spare blocks
  int32_t n_spare = 0;
  int64_t cache_stride = 0;

  static int ln(const Block& b) { return b.line == 1 ? 1 : 0; }
  int n_caches() const { return lp->cfg.n_layers * lp->cfg.loop_depth; }

  int32_t rows_in_flight() const {
    int32_t n = 0;
    for (const Block& b : blocks)
      if (b.in_flight) n += (int32_t)b.toks.size();
    return n;
  }

  void truncate_hist(int line, size_t n) {
    if (hist[line].size() > n) hist[line].resize(n);
    if (dev_valid[line] > n) dev_valid[line] = n;
  }

  void release(Block& b) {
    if (b.slot >= 0) free_slots.push_back(b.slot);
    b.slot = -1;
  }

  // remove the blocks matching `pred` (with their per-block readout
  // records); returns the rows they had in flight, counted as discarded
  template <typename Pred>
  int64_t drop(Pred pred, std::vector<int32_t>& row0r, std::vector<int32_t>& accd) {
    int64_t n = 0;
    size_t w = 0;
    for (size_t j = 0; j < blocks.size(); ++j) {
      if (pred(blocks[j], j)) {
        if (blocks[j].in_flight) {
          n += (int64_t)blocks[j].toks.size();
          release(blocks[j]);
        }
        continue;
      }
      if (w != j) {
        blocks[w] = std::move(blocks[j]);
        row0r[w] = row0r[j];
        accd[w] = accd[j];
      }
      ++w;
    }
    blocks.resize(w);
    row0r.resize(w);
    accd.resize(w);
    st.discarded += n;
    return n;
  }

  // upload the host history's changes of a line to its device copy
  cad_status sync_hist(int line) {
    const size_t n = hist[line].size() - dev_valid[line];
    if (n > 0) {
      // the staging buffer is rewritten only once the last copy out of it is done
      LOOP_HIP(hipEventSynchronize(lp->hist_copied));
      std::memcpy(lp->h_hist, hist[line].data() + dev_valid[line], n * 4);
      LOOP_HIP(hipMemcpyAsync(d_hist[line] + dev_valid[line], lp->h_hist, n * 4, hipMemcpyHostToDevice, s));
      LOOP_HIP(hipEventRecord(lp->hist_copied, s));
      dev_valid[line] = hist[line].size();
    }
    return CAD_OK;
  }

  // admit a waiting block with a context-copy tail of at most room - 1
  // tokens (from the device proposal made after the last tick, or a fresh
  // one: one synchronisation)
  cad_status admit(Block& b, int32_t room) {
    const int line = ln(b);
    truncate_hist(line, (size_t)b.pos);
    hist[line].push_back(b.toks[0]);
    int32_t n_tail = 0;
    const int32_t* tail = nullptr;
    if (lp->p.max_copy > 0 && room > 1) {
      int slot = b.ready;
      if (slot < 0) {
        slot = kPropSlots;
        cad_status r = sync_hist(line);
        if (r != CAD_OK) return r;
        int32_t* dp = lp->d_prop + slot * 65;
        LOOP_CALL(cad_propose_suffix_match(d_hist[line], (int64_t)hist[line].size(), lp->p.max_ngram,
                                           lp->p.min_ngram, lp->p.max_copy, dp, dp + 64, lp->d_prop_pos + slot, s));
        LOOP_HIP(hipMemcpyAsync(lp->h_prop + slot * 65, dp, 65 * 4, hipMemcpyDeviceToHost, s));
        LOOP_HIP(hipStreamSynchronize(s));
        ++st.host_syncs;
      }
      tail = lp->h_prop + slot * 65;
      n_tail = tail[64];
      if (n_tail > room - 1) n_tail = room - 1;
      if (line == 1) {  // the second line's positions stay within the spare blocks
        const int64_t end = (fork_pos / CAD_KV_BLOCK + n_spare) * (int64_t)CAD_KV_BLOCK;
        if (b.pos + 1 + n_tail > end) n_tail = (int32_t)std::max<int64_t>(0, end - b.pos - 1);
      }
      if (n_tail < 0) n_tail = 0;
    }
    if (line == 1 && b.pos + 1 > (fork_pos / CAD_KV_BLOCK + n_spare) * (int64_t)CAD_KV_BLOCK)
      return loop_fail(CAD_E_CAPACITY, "the second line outgrew its spare blocks");
    b.ready = -1;
    b.toks.resize(1);
    for (int32_t j = 0; j < n_tail; ++j) b.toks.push_back(tail[j]);
    for (int32_t j = 0; j < n_tail; ++j) hist[line].push_back(tail[j]);
    b.slot = free_slots.back();
    free_slots.pop_back();
    b.in_flight = true;
    ++st.blocks;
    st.proposed += n_tail;
    return CAD_OK;
  }

  // waiting heads in list order, while a row and a slot are free
  cad_status admit_waiting() {
    for (size_t j = 0; j < blocks.size(); ++j) {
      Block& b = blocks[j];
      if (b.in_flight) continue;
      const int32_t room = lp->p.max_rows - rows_in_flight();
      if (room < 1 || free_slots.empty()) {
        for (size_t k = j; k < blocks.size(); ++k)
          if (!blocks[k].in_flight) blocks[k].ready = -1;  // a later admission proposes again
        return CAD_OK;
      }
      cad_status r = admit(b, room);
      if (r != CAD_OK) return r;
    }
    return CAD_OK;
  }

  // copy cache slots between blocks at every depth: pairs staged from slot
  // `first` of the pinned / device pair buffers
  cad_status kv_copy(int first, int n) {
    if (n <= 0) return CAD_OK;
    LOOP_HIP(hipMemcpyAsync(lp->d_pairs + 4 * first, lp->h_pairs + 4 * first, (size_t)n * 16, hipMemcpyHostToDevice, s));
    LOOP_HIP(launch_kv_copy(lp->cfg.dtype, user_kv->k, user_kv->v, cache_stride, n_caches(),
                                 lp->cfg.n_kv_heads, lp->cfg.head_dim, lp->d_pairs + 4 * first, n, s));
    return CAD_OK;
  }

  // the older positions' slots of the block where the fork starts, from
  // row 0's block to the second line's (pair 0, staged at the fork)
  cad_status sync_fork_block() {
    if (!fork_live || fork_pos % CAD_KV_BLOCK == 0) return CAD_OK;
    LOOP_HIP(launch_kv_copy(lp->cfg.dtype, user_kv->k, user_kv->v, cache_stride, n_caches(),
                                 lp->cfg.n_kv_heads, lp->cfg.head_dim, lp->d_pairs, 1, s));
    return CAD_OK;
  }

  // make the fork at block i (read out at d2): the second child, headed by
  // h1; with `proposed`, its history and proposal were made on the device
  // after the tick (in d_spec of the block's table row, proposal slot
  // kPropFork + that row)
  cad_status make_fork(size_t i, int32_t h1, int32_t room, bool proposed, std::vector<int32_t>& row0r,
                       std::vector<int32_t>& accd) {
    const Block& b = blocks[i];
    const int trow = b.tick_row;
    fork_live = true;
    fork_parent = b.id;
    fork_pos = b.pos + (int64_t)b.toks.size();
    for (size_t j = i + 1; j < blocks.size(); ++j) blocks[j].line = 0;
    // block-table row 1: row 0 before the fork's block, spare blocks from it
    const int64_t fb = fork_pos / CAD_KV_BLOCK;
    int32_t* r1 = lp->h_table + lp->tbl_stride;
    for (int64_t j = 0; j < lp->tbl_stride; ++j)
      r1[j] = j < fb ? row0[j] : (j - fb < n_spare ? spare[j - fb] : 0);
    LOOP_HIP(hipMemcpyAsync(lp->d_table + lp->tbl_stride, r1, (size_t)lp->tbl_stride * 4, hipMemcpyHostToDevice, s));
    if (fork_pos % CAD_KV_BLOCK != 0) {
      int32_t* pr = lp->h_pairs;
      pr[0] = row0[fb];
      pr[1] = spare[0];
      pr[2] = 0;
      pr[3] = (int32_t)(fork_pos % CAD_KV_BLOCK);
      cad_status r = kv_copy(0, 1);
      if (r != CAD_OK) return r;
    }
    // the second line's history: the first line's up to the fork
    if (proposed) {
      std::swap(d_hist[1], d_spec[trow]);
    } else {
      cad_status r = sync_hist(0);
      if (r != CAD_OK) return r;
      LOOP_HIP(hipMemcpyAsync(d_hist[1], d_hist[0], (size_t)fork_pos * 4, hipMemcpyDeviceToDevice, s));
    }
    hist[1].assign(hist[0].begin(), hist[0].begin() + fork_pos);
    dev_valid[1] = (size_t)fork_pos;
    Block nb;
    nb.pos = fork_pos;
    nb.toks.push_back(h1);
    nb.line = 1;
    nb.ready = proposed ? kPropFork + trow : -1;
    nb.id = next_id++;
    blocks.push_back(nb);
    row0r.push_back(-1);
    accd.push_back(0);
    ++st.forks;
    return admit(blocks.back(), room);
  }

  // close the live fork keeping line `keep`; with the second line, its K/V
  // go to row 0's blocks and its history becomes the history
  cad_status end_fork(int keep) {
    if (keep == 1) {
      int64_t end = fork_pos;
      for (const Block& b : blocks)
        if (b.line == 1 && b.in_flight) end = std::max<int64_t>(end, b.pos + (int64_t)b.toks.size());
      const int64_t fb = fork_pos / CAD_KV_BLOCK;
      int n = 0;
      for (int64_t j = fb; j * CAD_KV_BLOCK < end; ++j, ++n) {
        int32_t* pr = lp->h_pairs + 4 * (1 + n);
        pr[0] = spare[j - fb];
        pr[1] = row0[j];
        pr[2] = j == fb ? (int32_t)(fork_pos % CAD_KV_BLOCK) : 0;
        pr[3] = CAD_KV_BLOCK;
      }
      cad_status r = kv_copy(1, n);
      if (r != CAD_OK) return r;
      std::swap(d_hist[0], d_hist[1]);
      hist[0].swap(hist[1]);
      dev_valid[0] = dev_valid[1];
    }
    hist[1].clear();
    dev_valid[1] = 0;
    for (Block& b : blocks) b.line = -1;
    fork_live = false;
    return CAD_OK;
  }

  cad_status prefill(const int32_t* prompt, int64_t L0) {
    // the prompt through every depth (a looped splice screened at the full
    // depth keeps every row), in chunks of at most prefill_rows
    LOOP_HIP(hipEventSynchronize(lp->hist_copied));
    std::memcpy(lp->h_hist, prompt, (size_t)L0 * 4);
    LOOP_HIP(hipMemcpyAsync(d_hist[0], lp->h_hist, (size_t)L0 * 4, hipMemcpyHostToDevice, s));
    LOOP_HIP(hipEventRecord(lp->hist_copied, s));
    hist[0].assign(prompt, prompt + L0);
    dev_valid[0] = (size_t)L0;
    const int32_t D = lp->cfg.loop_depth;
    int64_t last = 0;
    for (int64_t c0 = 0; c0 < L0; c0 += lp->prefill_rows) {
      const int32_t n = (int32_t)std::min<int64_t>(lp->prefill_rows, L0 - c0);
      LOOP_CALL(cad_splice_forward_looped(lp->m, kv, c0, d_hist[0] + c0, n, D, nullptr, lp->d_pf_sargmax,
                                          lp->d_pf_misc, lp->d_pf_argmax, lp->d_pf_misc + 1, nullptr,
                                          lp->d_status, s));
      last = n - 1;
    }
    LOOP_HIP(hipMemcpyAsync(lp->h_argmax, lp->d_pf_sargmax + last, 4, hipMemcpyDeviceToHost, s));
    LOOP_HIP(hipStreamSynchronize(s));
    ++st.host_syncs;
    return CAD_OK;
  }

  // the pipeline's table rows from the caller's: row 0 (the request's
  // blocks for `need` positions) and the spare blocks of row 1 (branching);
  // checked against the pool
  cad_status setup_tables(int64_t need) {
    const int64_t nb = (need + CAD_KV_BLOCK - 1) / CAD_KV_BLOCK;
    std::vector<int32_t> tmp((size_t)(2 * user_kv->max_blocks_per_seq));
    LOOP_HIP(hipMemcpyAsync(tmp.data(), user_kv->block_table, tmp.size() * 4, hipMemcpyDeviceToHost, s));
    LOOP_HIP(hipStreamSynchronize(s));
    ++st.host_syncs;
    row0.assign(tmp.begin(), tmp.begin() + nb);
    for (int32_t e : row0)
      if (e < 0 || e >= user_kv->num_blocks) return loop_fail(CAD_E_ARG, "block table row 0 holds a block outside the pool");
    n_spare = lp->max_pairs - 1;
    spare.assign(tmp.begin() + user_kv->max_blocks_per_seq, tmp.begin() + user_kv->max_blocks_per_seq + n_spare);
    std::vector<int32_t> used(row0);
    std::sort(used.begin(), used.end());
    for (int32_t e : spare) {
      if (e < 0 || e >= user_kv->num_blocks) return loop_fail(CAD_E_ARG, "block table row 1 holds a block outside the pool");
      if (std::binary_search(used.begin(), used.end(), e))
        return loop_fail(CAD_E_ARG, "a spare block of row 1 is also in row 0");
    }
    std::vector<int32_t> sp(spare);
    std::sort(sp.begin(), sp.end());
    if (std::adjacent_find(sp.begin(), sp.end()) != sp.end()) return loop_fail(CAD_E_ARG, "row 1 repeats a spare block");
    for (int64_t j = 0; j < 2 * (int64_t)lp->tbl_stride; ++j) lp->h_table[j] = j < nb ? row0[j] : 0;
    LOOP_HIP(hipMemcpyAsync(lp->d_table, lp->h_table, (size_t)lp->tbl_stride * 2 * 4, hipMemcpyHostToDevice, s));
    kv_run = *user_kv;
    kv_run.block_table = lp->d_table;
    kv_run.max_blocks_per_seq = lp->tbl_stride;
    cache_stride = user_kv->num_blocks * (int64_t)lp->cfg.n_kv_heads * CAD_KV_BLOCK * lp->cfg.head_dim;
    return CAD_OK;
  }

  cad_status decode(const int32_t* prompt, int64_t L0, int32_t n_new, int32_t* out_tokens, int64_t need) {
    const int32_t D = lp->cfg.loop_depth, ds = lp->p.screen_depth, d2 = lp->p.branch_depth;
    d_hist[0] = lp->d_hist;
    d_hist[1] = lp->d_hist2;
    d_spec[0] = lp->d_spec[0];
    d_spec[1] = lp->d_spec[1];
    for (int32_t i = lp->n_slots - 1; i >= 0; --i) free_slots.push_back(i);
    kv = user_kv;
    cad_status r = CAD_OK;
    if (d2 > 0) {
      r = setup_tables(need);
      if (r != CAD_OK) return r;
      kv = &kv_run;
    }
    r = prefill(prompt, L0);
    if (r != CAD_OK) return r;
    const int32_t first = lp->h_argmax[0];
    out.push_back(first);
    Block b0;
    b0.pos = L0;
    b0.toks.push_back(first);
    b0.id = next_id++;
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
      // a fork can start this tick where none is live, or where the live
      // one's parent reaches full depth (it is resolved first)
      bool may_fork = !fork_live;
      for (const Block& b : blocks)
        if (fork_live && b.id == fork_parent && b.in_flight && b.depth + 1 == D) may_fork = true;
      for (size_t i = 0; i < blocks.size(); ++i) {
        Block& b = blocks[i];
        if (!b.in_flight) continue;
        cad_loop_group g;
        g.pos = b.pos;
        g.rows = (int32_t)b.toks.size();
        g.depth = b.depth;
        g.state = b.slot * lp->slot_rows;
        // the second readout only where a fork can start
        const bool fork_read = d2 > 0 && b.depth + 1 == d2 && may_fork;
        g.readout = (b.depth + 1 == ds || b.depth + 1 == D || fork_read) ? 1 : 0;
        g.table_row = b.line == 1 ? 1 : 0;
        b.tick_row = g.table_row;
        any_read |= g.readout != 0;
        for (int32_t t : b.toks) h_tok[total++] = t;
        groups.push_back(g);
        live.push_back(i);
      }
      if (groups.empty()) return loop_fail(CAD_E_ARG, "pipeline empty before the decode finished");
      const bool propose = any_read && lp->p.max_copy > 0;
      if (propose) {
        // the device histories must hold every token in flight for the proposals below
        cad_status r2 = sync_hist(0);
        if (r2 == CAD_OK && fork_live) r2 = sync_hist(1);
        if (r2 != CAD_OK) return r2;
      }
      // with branching, each group's row count follows the tokens (the kept
      // rows of a possible second child's proposal)
      int32_t n_up = total;
      if (d2 > 0)
        for (const cad_loop_group& g : groups) h_tok[n_up++] = g.rows;
      LOOP_HIP(hipMemcpyAsync(lp->d_tokens, h_tok, (size_t)n_up * 4, hipMemcpyHostToDevice, s));
      LOOP_HIP(hipEventRecord(lp->tok_copied[st.ticks & 1], s));
      LOOP_CALL(cad_loop_step(lp->m, kv, (int32_t)groups.size(), groups.data(), lp->d_tokens, lp->state,
                              lp->n_slots * lp->slot_rows, nullptr, lp->d_argmax, lp->d_accepted, nullptr,
                              lp->d_status, s));
      ++st.ticks;
      st.rows_run += total;
      if (any_read) {
        if (propose) {
          // For a block read out at the branch depth, the history of a
          // possible second child (its line's up to the child, then the
          // depth-d2 prediction at its last row as the head) and that
          // child's proposal.
          int32_t o = 0;
          for (size_t k = 0; k < groups.size(); ++k) {
            const cad_loop_group& g = groups[k];
            if (g.readout && d2 > 0 && g.depth + 1 == d2) {
              const int r = g.table_row, slot = kPropFork + r;
              LOOP_HIP(hipMemcpyAsync(d_spec[r], d_hist[r], (size_t)(g.pos + g.rows) * 4, hipMemcpyDeviceToDevice, s));
              int32_t* dp = lp->d_prop + slot * 65;
              LOOP_HIP(cad::launch_propose_next(d_spec[r], g.pos, lp->d_tokens + total + k, lp->d_argmax + o,
                                                lp->p.max_ngram, lp->p.min_ngram, lp->p.max_copy, dp, dp + 64,
                                                lp->d_prop_pos + slot, lp->d_prop_head + slot, s));
            }
            o += g.rows;
          }
          // Then the successor of the block screened on each line's history
          // and the token after the full-depth block, screening first: the
          // full-depth one may write a correction into the history.
          const int passes[3][3] = {{kPropScreen0, 0, ds}, {kPropScreen1, 1, ds}, {kPropFull, 0, D}};
          for (const auto& ps : passes) {
            o = 0;
            for (size_t k = 0; k < groups.size(); ++k) {
              const cad_loop_group& g = groups[k];
              if (g.readout && g.table_row == ps[1] && g.depth + 1 == ps[2]) {
                int32_t* dp = lp->d_prop + ps[0] * 65;
                LOOP_HIP(cad::launch_propose_next(d_hist[ps[1]], g.pos, lp->d_accepted + k, lp->d_argmax + o,
                                                  lp->p.max_ngram, lp->p.min_ngram, lp->p.max_copy, dp, dp + 64,
                                                  lp->d_prop_pos + ps[0], lp->d_prop_head + ps[0], s));
              }
              o += g.rows;
            }
          }
        }
        // acceptance, proposals and argmax in one copy
        LOOP_HIP(hipMemcpyAsync(lp->h_accepted, lp->d_accepted, (size_t)(kRbArgmax + total) * 4,
                                hipMemcpyDeviceToHost, s));
        LOOP_HIP(hipStreamSynchronize(s));
        ++st.host_syncs;
        if (propose) {
          // the device wrote the head of each screening or full-depth
          // proposal into its line's history copy; the host history takes
          // those positions over when it admits or corrects
          for (size_t k = 0; k < groups.size(); ++k) {
            const int32_t after = groups[k].depth + 1;
            if (groups[k].readout && (after == ds || after == D)) {
              const int r = groups[k].table_row;
              const size_t at = (size_t)(groups[k].pos + lp->h_accepted[k]);
              if (dev_valid[r] > at) dev_valid[r] = at;
            }
          }
        }
      }
      // per block of this tick: its readout (row offset in the tick, accepted)
      std::vector<int32_t> row0r(blocks.size(), -1), accd(blocks.size(), 0);
      {
        int32_t o = 0;
        for (size_t k = 0; k < live.size(); ++k) {
          if (groups[k].readout) {
            row0r[live[k]] = o;
            accd[live[k]] = lp->h_accepted[k];
          }
          o += groups[k].rows;
          blocks[live[k]].depth += 1;
        }
      }
      size_t i = 0;
      while (i < blocks.size()) {
        Block& b = blocks[i];
        if (!b.in_flight || row0r[i] < 0) {
          ++i;
          continue;
        }
        const int32_t* a = lp->h_argmax + row0r[i];
        const int32_t m = (int32_t)b.toks.size();
        if (b.depth == D) {
          // full-depth verification of the tail (the head is verified already)
          const int32_t acc = accd[i];
          for (int32_t j = 1; j < acc; ++j) out.push_back(b.toks[j]);
          const int32_t nxt = a[acc - 1];
          st.rejected += m - acc;
          const int64_t pos_next = b.pos + acc;
          const bool parent = fork_live && b.id == fork_parent;
          release(b);
          blocks.erase(blocks.begin() + (std::ptrdiff_t)i);
          row0r.erase(row0r.begin() + (std::ptrdiff_t)i);
          accd.erase(accd.begin() + (std::ptrdiff_t)i);
          bool correct = false;
          if (parent) {
            // resolve the fork: keep the line whose head is the verified token
            int keep = -1;
            if (acc == m)
              for (int line = 0; line < 2 && keep < 0; ++line)
                for (const Block& c : blocks)
                  if (c.line == line) {
                    if (c.toks[0] == nxt) keep = line;
                    break;
                  }
            if (keep < 0) {
              drop([](const Block& c, size_t) { return c.line >= 0; }, row0r, accd);
              r = end_fork(0);
              if (r != CAD_OK) return r;
              correct = true;
            } else {
              st.fork_rows_dropped += drop([keep](const Block& c, size_t) { return c.line == 1 - keep; }, row0r, accd);
              if (keep == 1) ++st.forks_kept;
              else ++st.forks_lost;
              r = end_fork(keep);
              if (r != CAD_OK) return r;
              out.push_back(nxt);
            }
          } else if (i < blocks.size() && acc == m && blocks[i].toks[0] == nxt) {
            out.push_back(nxt);  // the next block's head is the verified token
          } else {
            drop([i](const Block&, size_t j) { return j >= i; }, row0r, accd);
            if (fork_live) {
              r = end_fork(0);
              if (r != CAD_OK) return r;
            }
            correct = true;
          }
          if (correct) {
            truncate_hist(0, (size_t)pos_next);
            out.push_back(nxt);
            Block c;
            c.pos = pos_next;
            c.toks.push_back(nxt);
            c.ready = kPropFull;  // proposed on the device after this tick
            c.id = next_id++;
            blocks.push_back(c);
            row0r.push_back(-1);
            accd.push_back(0);
          }
          continue;
        }
        if (d2 > 0 && b.depth == d2) {
          // the second readout: a second child where the prediction at the
          // last surviving row differs from the one that headed the child
          if (!fork_live && b.line < 0 && i + 1 < blocks.size()) {
            const Block& child = blocks[i + 1];
            if (child.in_flight && child.pos == b.pos + m) {
              const int32_t h1 = a[m - 1];
              const int32_t room = lp->p.max_rows - rows_in_flight();
              if (h1 != child.toks[0] && room >= 1 && !free_slots.empty()) {
                r = make_fork(i, h1, room, propose, row0r, accd);
                if (r != CAD_OK) return r;
              }
            }
          }
        } else if (b.depth == ds) {
          // shallow screening: the agreeing prefix survives, the rest is released
          const int32_t keep = accd[i];
          st.screened_out += m - keep;
          b.toks.resize(keep);
          truncate_hist(ln(b), (size_t)(b.pos + keep));
          bool younger = false;
          for (size_t j = i + 1; j < blocks.size() && !younger; ++j) younger = blocks[j].line == b.line;
          if (!younger) {
            Block nb;
            nb.pos = b.pos + keep;
            nb.toks.push_back(a[keep - 1]);
            nb.line = b.line;
            // proposed on the device after this tick, on the history the block ran on
            nb.ready = b.tick_row == 0 ? kPropScreen0 : kPropScreen1;
            nb.id = next_id++;
            // a first-line block goes before the second line's blocks
            size_t at = blocks.size();
            if (b.line == 0)
              for (size_t j = 0; j < blocks.size(); ++j)
                if (blocks[j].line == 1) {
                  at = j;
                  break;
                }
            blocks.insert(blocks.begin() + (std::ptrdiff_t)at, nb);
            row0r.insert(row0r.begin() + (std::ptrdiff_t)at, -1);
            accd.insert(accd.begin() + (std::ptrdiff_t)at, 0);
          }
        }
        ++i;
      }
      r = sync_fork_block();
      if (r != CAD_OK) return r;
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

cad_status cad_loop_create(cad_model* m, int64_t max_len, const cad_loop_params* p, cad_loop** out) try {
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
  if (p->branch_depth != 0 && (p->branch_depth <= p->screen_depth || p->branch_depth >= c->loop_depth))
    return loop_fail(CAD_E_ARG, "branch_depth must be 0 or in (screen_depth, loop_depth)");
  if (max_len < 1) return loop_fail(CAD_E_ARG, "max_len must be >= 1");
  cad_loop* lp = new (std::nothrow) cad_loop();
  if (!lp) return loop_fail(CAD_E_HIP, "host allocation failed");
  lp->m = m;
  lp->cfg = *c;
  lp->p = *p;
  lp->max_len = max_len;
  lp->slot_rows = p->max_copy + 1;
  // blocks in flight sit at distinct depths on each line (two lines with branching)
  const bool branch = p->branch_depth > 0;
  lp->n_slots = (branch ? 2 : 1) * c->loop_depth;
  lp->tbl_stride = branch ? (int32_t)((max_len + CAD_KV_BLOCK - 1) / CAD_KV_BLOCK) : 0;
  // the second line's positions: at most loop_depth blocks of max_copy + 1
  // rows after the fork, which may start anywhere in a block (+ one)
  lp->max_pairs = branch ? 1 + (int32_t)((c->loop_depth * (int64_t)lp->slot_rows + 2 * CAD_KV_BLOCK - 1) / CAD_KV_BLOCK) + 1 : 0;
  lp->tick_rows = std::min(p->max_rows, lp->n_slots * lp->slot_rows);
  lp->prefill_rows = c->max_tokens;
  if (lp->n_slots > CAD_MAX_SEQS) {
    delete lp;
    return loop_fail(CAD_E_CAPACITY, "more blocks in flight than a tick's groups (CAD_MAX_SEQS)");
  }
  if (lp->tick_rows > c->max_tokens) {
    delete lp;
    return loop_fail(CAD_E_CAPACITY, "max_rows exceeds the model's max_tokens");
  }
  const int64_t d = c->d_model, srows = (int64_t)lp->n_slots * lp->slot_rows, T = c->max_tokens;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = up256(off + bytes); return o; };
  const size_t rb_bytes = (size_t)(kRbArgmax + std::max<int64_t>(srows, 1)) * 4;
  const size_t o_state = take(srows * d * 4), o_tok = take((srows + CAD_MAX_SEQS) * 4), o_rb = take(rb_bytes),
               o_hist = take(max_len * 4),
               o_hist2 = take(branch ? max_len * 4 : 0), o_spec0 = take(branch ? max_len * 4 : 0),
               o_spec1 = take(branch ? max_len * 4 : 0), o_tbl = take((size_t)lp->tbl_stride * 2 * 4),
               o_pairs = take((size_t)lp->max_pairs * 16),
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
  lp->d_accepted = (int32_t*)(b + o_rb);
  lp->d_prop = lp->d_accepted + kRbProp;
  lp->d_argmax = lp->d_accepted + kRbArgmax;
  lp->d_hist = (int32_t*)(b + o_hist);
  lp->d_hist2 = branch ? (int32_t*)(b + o_hist2) : nullptr;
  lp->d_spec[0] = branch ? (int32_t*)(b + o_spec0) : nullptr;
  lp->d_spec[1] = branch ? (int32_t*)(b + o_spec1) : nullptr;
  lp->d_table = branch ? (int32_t*)(b + o_tbl) : nullptr;
  lp->d_pairs = branch ? (int32_t*)(b + o_pairs) : nullptr;
  lp->d_prop_head = (int32_t*)(b + o_phead);
  lp->d_prop_pos = (int64_t*)(b + o_ppos);
  lp->d_status = (int32_t*)(b + o_st);
  lp->d_pf_sargmax = (int32_t*)(b + o_pfs);
  lp->d_pf_argmax = (int32_t*)(b + o_pfa);
  lp->d_pf_misc = (int32_t*)(b + o_pfm);
  size_t hoff = 0;
  auto htake = [&](size_t bytes) { size_t o = hoff; hoff = up256(hoff + bytes); return o; };
  const size_t h_tok0 = htake((srows + CAD_MAX_SEQS) * 4), h_tok1 = htake((srows + CAD_MAX_SEQS) * 4), h_rb = htake(rb_bytes),
               h_hist = htake(max_len * 4),
               h_tbl = htake((size_t)lp->tbl_stride * 2 * 4), h_pairs = htake((size_t)lp->max_pairs * 16);
  e = hipHostMalloc(&lp->host, hoff, hipHostMallocDefault);
  if (e != hipSuccess) {
    (void)hipFree(lp->dev);
    delete lp;
    return loop_fail(CAD_E_HIP, std::string("hipHostMalloc: ") + hipGetErrorString(e));
  }
  char* h = (char*)lp->host;
  lp->h_tokens[0] = (int32_t*)(h + h_tok0);
  lp->h_tokens[1] = (int32_t*)(h + h_tok1);
  for (int k = 0; k < 3; ++k) {
    e = hipEventCreateWithFlags(k < 2 ? &lp->tok_copied[k] : &lp->hist_copied, hipEventDisableTiming);
    if (e != hipSuccess) {
      cad_loop_destroy(lp);
      return loop_fail(CAD_E_HIP, std::string("hipEventCreate: ") + hipGetErrorString(e));
    }
  }
  lp->h_accepted = (int32_t*)(h + h_rb);
  lp->h_prop = lp->h_accepted + kRbProp;
  lp->h_argmax = lp->h_accepted + kRbArgmax;
  lp->h_hist = (int32_t*)(h + h_hist);
  lp->h_table = branch ? (int32_t*)(h + h_tbl) : nullptr;
  lp->h_pairs = branch ? (int32_t*)(h + h_pairs) : nullptr;
  *out = lp;
  return CAD_OK;
} catch (...) {
  // host containers and messages are C++: nothing they throw crosses the C ABI
  return cad::set_error(CAD_E_HIP, "host allocation failed");
}

void cad_loop_destroy(cad_loop* lp) {
  if (!lp) return;
  (void)hipDeviceSynchronize();
  for (hipEvent_t e : lp->tok_copied)
    if (e) (void)hipEventDestroy(e);
  if (lp->hist_copied) (void)hipEventDestroy(lp->hist_copied);
  (void)hipFree(lp->dev);
  (void)hipHostFree(lp->host);
  delete lp;
}

cad_status cad_loop_decode(cad_loop* lp, const cad_kv* kv, const int32_t* prompt, int64_t L0, int32_t n_new,
                           int32_t* out_tokens, cad_loop_stats* stats, cad_stream stream) try {
  if (!lp || !kv || !prompt || !out_tokens) return loop_fail(CAD_E_ARG, "NULL argument");
  if (L0 < 1 || n_new < 1) return loop_fail(CAD_E_ARG, "need a prompt and at least one new token");
  const int64_t need = L0 + n_new + (int64_t)lp->cfg.loop_depth * lp->slot_rows;
  if (need > lp->max_len) return loop_fail(CAD_E_CAPACITY, "prompt + new tokens + blocks in flight exceed max_len");
  if (need > (int64_t)kv->max_blocks_per_seq * CAD_KV_BLOCK)
    return loop_fail(CAD_E_CAPACITY, "prompt + new tokens + blocks in flight exceed the block table");
  if (lp->p.branch_depth > 0 && kv->max_blocks_per_seq < lp->max_pairs - 1)
    return loop_fail(CAD_E_CAPACITY, "block-table row 1 cannot hold the second line's spare blocks");
  Run run;
  run.lp = lp;
  run.user_kv = kv;
  run.s = (hipStream_t)stream;
  LOOP_HIP(hipMemsetAsync(lp->d_status, 0, 4, run.s));
  const cad_status r = run.decode(prompt, L0, n_new, out_tokens, need);
  if (stats) *stats = run.st;
  return r;
} catch (...) {
  // host containers and messages are C++: nothing they throw crosses the C ABI
  return cad::set_error(CAD_E_HIP, "host allocation failed");
}

}  // extern "C"
