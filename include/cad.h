/*
 * cad.h -- C ABI of libcad: the copy-span splice forward on AMD MI355X (gfx950).
 *
 * The operation: commit a span of N known tokens to a decoder's KV cache in
 * one parallel forward instead of N autoregressive steps, then take a
 * (grammar-)masked argmax per position and a longest-agreeing-prefix
 * acceptance.  Sources:
 *   - "Copy-as-Decode: Grammar-Constrained Parallel Prefill for LLM Editing",
 *     §2.4 (the splice: one forward over the span with the existing KV
 *     cache), §2.3 (masked argmax at decision points, forced-template
 *     prefills spliced the same way), Fig. 1 (acceptance is 1 inside a copy
 *     op), appendix "Position-encoding correctness" (positions advance by N).
 *   - "CopyLoop: Fast Looped Transformer Decoding via Context Copying and
 *     Shallow Screening", §2 "Block Construction" (suffix-match proposal),
 *     "Shallow Screening", "Concurrent Pipeline", "Full-Depth Verification".
 *
 * Conventions for every entry point:
 *   - Pointers marked "dev" are device (HBM) pointers; "host" are host
 *     pointers read before the call returns.  The caller owns and frees every
 *     buffer it passes; the library owns only the workspace it allocates in
 *     cad_model_create and frees in cad_model_destroy.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and is asynchronous: outputs are valid once the caller synchronises.
 *     Nothing synchronises the host except create and destroy.
 *   - Argument errors are detected on the host, return a non-zero
 *     cad_status and enqueue nothing; cad_last_error() then describes the
 *     failure (thread-local string).  HIP launch failures return CAD_E_HIP,
 *     and so does a failed host allocation ("host allocation failed"): no
 *     C++ exception leaves the library.
 *   - Data-dependent faults found on the device (token id outside the
 *     vocabulary, a mask row that allows nothing, a block-table entry outside
 *     the pool) are OR-ed into the optional `dev_status` word; the kernels
 *     then skip the offending read or write instead of faulting.
 *   - A model handle is not re-entrant: one host thread and one stream at a
 *     time per handle, because calls share its workspace.
 */
#ifndef CAD_H
#define CAD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct cad_model cad_model; /* opaque, library-owned */
typedef void* cad_stream;           /* hipStream_t */

typedef enum { CAD_F32 = 0, CAD_BF16 = 1 } cad_dtype;

/* COMMIT: acceptance is N by construction (a copy op or a forced template).
 * VERIFY: accept the longest prefix on which the model agrees (see below). */
typedef enum { CAD_COMMIT = 0, CAD_VERIFY = 1 } cad_mode;

typedef enum {
  CAD_OK = 0,
  CAD_E_ARG = 1,         /* null pointer, bad size or enum, misaligned pointer */
  CAD_E_CAPACITY = 2,    /* span longer than max_tokens, cache too small */
  CAD_E_UNSUPPORTED = 3, /* shape the kernels do not implement */
  CAD_E_HIP = 4          /* a HIP runtime call failed */
} cad_status;

/* bits of the device status word */
#define CAD_DEV_BAD_TOKEN 1u  /* a span token is outside [0, vocab): its embedding row reads as zeros */
#define CAD_DEV_EMPTY_MASK 2u /* a mask row allows no id: that argmax is -1 */
#define CAD_DEV_BAD_BLOCK 4u  /* a block-table entry is outside [0, num_blocks): that K/V is skipped */
#define CAD_DEV_F16_RANGE 8u  /* a value written at half precision for the matrix cores (q, the span's own
                                 K/V, the down projection's input above 16 rows) exceeded 65504 and was
                                 saturated: the results of that call are not reliable */

#define CAD_KV_BLOCK 16       /* tokens per KV block */
#define CAD_MAX_SEQS 64       /* sequences per batched call */

/* Model shape.  Llama-style decoder: RMSNorm, rotary positions (half-split
 * pairs, base rope_theta), grouped-query attention (query head h reads KV
 * head h / (n_q_heads / n_kv_heads)), SwiGLU FFN, no biases, untied LM head.
 * loop_depth > 1: one shared block (n_layers must be 1) applied loop_depth
 * times, with one KV cache per depth (CopyLoop's looped decoder).
 * max_tokens: the most span rows one call may carry (sizes the workspace).
 * Supported: d_model a multiple of 4, at most 8192; (n_q_heads + 2
 * n_kv_heads) * head_dim at most 16384; dtype CAD_F32 any head_dim <= 128
 * (even); dtype CAD_BF16 head_dim 64 or 128 and d_model, ffn_dim,
 * n_q_heads*head_dim multiples of 64.  Other shapes: CAD_E_UNSUPPORTED. */
typedef struct {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab;
  int32_t loop_depth;
  float rope_theta, rms_eps;
  int32_t dtype; /* cad_dtype */
  int32_t max_tokens;
} cad_config;

/* Weights: dev pointers, element type = cfg.dtype, row-major [out][in]
 * (nn.Linear layout).  Per-layer fields are HOST arrays of n_layers dev
 * pointers; the library copies the arrays, never the weights, and reads the
 * weights on every call, so they must outlive the model.
 *   tok_embed  [vocab][d]            final_norm [d]     lm_head [vocab][d]
 *   attn_norm  [d]                    ffn_norm   [d]
 *   w_qkv      [(Hq + 2 Hkv) hd][d]   rows: all q heads, then k heads, then v heads
 *   w_o        [d][Hq hd]
 *   w_gate_up  [2 F][d]               rows: gate (F rows) then up (F rows)
 *   w_down     [d][F]                                                      */
typedef struct {
  const void* tok_embed;
  const void* final_norm;
  const void* lm_head;
  const void* const* attn_norm;
  const void* const* w_qkv;
  const void* const* w_o;
  const void* const* ffn_norm;
  const void* const* w_gate_up;
  const void* const* w_down;
} cad_weights;

/* Paged KV cache, element type = cfg.dtype, caller-owned (dev):
 *   k: [n_layers * loop_depth][num_blocks][Hkv][16][hd]   keys after rotation
 *   v: [n_layers * loop_depth][num_blocks][Hkv][hd][16]   values, token-minor
 * Token t of a sequence lives in block block_table[seq][t / 16], slot t % 16.
 * block_table: dev int32 [n_seq][max_blocks_per_seq]; a single-sequence call
 * uses row 0 (an identity table gives a contiguous cache).  Blocks of
 * different sequences must not overlap. */
typedef struct {
  void* k;
  void* v;
  int64_t num_blocks;
  const int32_t* block_table;
  int32_t max_blocks_per_seq;
} cad_kv;

/* Create a model handle over caller-owned weights.  Validates the shape,
 * allocates the workspace for cfg->max_tokens rows and synchronises once.
 * Returns CAD_E_UNSUPPORTED for shapes the kernels do not implement. */
cad_status cad_model_create(const cad_config* cfg, const cad_weights* w, cad_model** out);

/* Free the workspace (synchronises the device).  NULL is a no-op. */
void cad_model_destroy(cad_model* m);

/* Message for the last failed call on this thread ("" if none). */
const char* cad_last_error(void);

/* Copy-span splice forward (Copy-as-Decode §2.4; CopyLoop §2 "Full-Depth
 * Verification").
 *   L        valid cache length before the call: span token k sits at absolute
 *            position L + k and attends to positions 0 .. L + k.
 *   span     dev int32 [N]; 1 <= N <= max_tokens; L + N <= 16 * max_blocks_per_seq.
 *   mask     dev uint32 [N][ceil(vocab/32)] or NULL (everything allowed): bit
 *            v % 32 of word v / 32 set = id v allowed at that position.
 *   mode     CAD_COMMIT or CAD_VERIFY.
 *   argmax   dev int32 [N]: masked argmax of each row's logits, lowest id on
 *            ties, -1 for a row that allows nothing.
 *   accepted dev int32 [1]: N (COMMIT) or 1 + the number of leading j >= 1
 *            with argmax[j-1] == span[j] (VERIFY).  The caller's new valid
 *            length is L + accepted and its next token is argmax[accepted-1]
 *            (the correction, or the bonus token on a full match).
 *   logits   dev float [N][vocab] or NULL: the fp32 logits, if wanted (with
 *            NULL no logits reach memory: the mask and the argmax are
 *            applied in the LM head's epilogue).
 *   dev_status dev int32 [1] or NULL: CAD_DEV_* bits are OR-ed in.
 * All N rows' K/V are written to cache slots L .. L+N-1 in place (slots
 * beyond L + accepted are stale afterwards and are overwritten by the next
 * call).  Slots outside L .. L+N-1 are not written. */
cad_status cad_splice_forward(cad_model* m, const cad_kv* kv, int64_t L, const int32_t* span,
                              int32_t N, const uint32_t* mask, cad_mode mode, int32_t* argmax,
                              int32_t* accepted, float* logits, int32_t* dev_status,
                              cad_stream stream);

/* One autoregressive decode step: the splice with N = 1 (Copy-as-Decode §3
 * "Kernel microbenchmark": the comparator is N one-token forwards, each
 * appending to the cache).  token: dev int32 [1]; mask_row: dev uint32
 * [ceil(vocab/32)] or NULL; argmax: dev int32 [1]; logits: dev float [vocab]
 * or NULL. */
cad_status cad_decode_step(cad_model* m, const cad_kv* kv, int64_t L, const int32_t* token,
                           const uint32_t* mask_row, int32_t* argmax, float* logits,
                           int32_t* dev_status, cad_stream stream);

/* The decode step for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, semantics and errors as cad_decode_step; the
 * step's per-call buffers (activations, split-K partial sums, attention
 * partials, argmax candidates) live in a static device array of
 * CAD_NOALLOC_SCRATCH_BYTES bytes that the library holds on each GPU until
 * the process ends (its address is resolved once per device, at
 * cad_model_create or this call's first use on a device), instead of the
 * model's workspace.  The call allocates nothing.  A model whose one-row
 * workspace exceeds the scratch returns CAD_E_CAPACITY.  Every call on one
 * GPU shares that GPU's array, which keeps the last call's contents (nothing
 * in it needs to start at zero): calls that overlap in time on one GPU (two
 * streams, two host threads) race and must be serialised by the caller. */
#define CAD_NOALLOC_SCRATCH_BYTES (4 << 20)
cad_status cad_decode_step_noalloc(cad_model* m, const cad_kv* kv, int64_t L, const int32_t* token,
                                   const uint32_t* mask_row, int32_t* argmax, float* logits,
                                   int32_t* dev_status, cad_stream stream);

/* Context-copy proposal (CopyLoop §2 "Block Construction").  tokens: dev
 * int32 [T], the whole history whose last element is the new head.  For n =
 * min(max_ngram, T-1) down to min_ngram, find the largest p with p + n <= T-1
 * and tokens[p .. p+n-1] == tokens[T-n .. T-1]; the first n that matches
 * gives out_pos = p + n and out_tokens = tokens[p+n .. min(p+n+K, T) - 1]
 * (out_len of them).  No match: out_len = 0, out_pos = -1.
 * 1 <= min_ngram <= max_ngram <= 64, K >= 1, T >= 0.  out_tokens dev int32
 * [K]; out_len dev int32 [1]; out_pos dev int64 [1]. */
cad_status cad_propose_suffix_match(const int32_t* tokens, int64_t T, int32_t max_ngram,
                                    int32_t min_ngram, int32_t K, int32_t* out_tokens,
                                    int32_t* out_len, int64_t* out_pos, cad_stream stream);

/* Batched splice over n_seq independent sequences sharing one paged pool
 * (continuous-batching form of the splice; Copy-as-Decode §7 names paged
 * attention integration as the next step).  seq_L: host int64 [n_seq];
 * offsets: host int32 [n_seq + 1], offsets[0] = 0, sequence b owns span rows
 * offsets[b] .. offsets[b+1]-1 (at least one) of spans (dev int32 [total]),
 * mask (dev uint32 [total][ceil(vocab/32)] or NULL), argmax (dev int32
 * [total]) and logits (dev float [total][vocab] or NULL).  Sequence b uses
 * block-table row b.  accepted: dev int32 [n_seq].  total <= max_tokens,
 * n_seq <= CAD_MAX_SEQS. */
cad_status cad_splice_forward_batched(cad_model* m, const cad_kv* kv, int32_t n_seq,
                                      const int64_t* seq_L, const int32_t* offsets,
                                      const int32_t* spans, const uint32_t* mask, cad_mode mode,
                                      int32_t* argmax, int32_t* accepted, float* logits,
                                      int32_t* dev_status, cad_stream stream);

/* Looped decoder with shallow screening (CopyLoop §2): the block [head,
 * copied tail] (span, N rows) runs through depths 1 .. screen_depth; the
 * readout there gives screen_argmax (dev int32 [N]) and the survivors count
 * (dev int32 [1]) by the VERIFY acceptance rule; only survivors continue to
 * depth loop_depth (rows at or beyond the survivors count write no deeper
 * KV), where the readout gives argmax (dev int32 [N], -1 beyond the
 * survivors) and accepted (dev int32 [1]).  Requires loop_depth > 1 and
 * 1 <= screen_depth <= loop_depth.  mask applies to both readouts. */
cad_status cad_splice_forward_looped(cad_model* m, const cad_kv* kv, int64_t L,
                                     const int32_t* span, int32_t N, int32_t screen_depth,
                                     const uint32_t* mask, int32_t* screen_argmax,
                                     int32_t* survivors, int32_t* argmax, int32_t* accepted,
                                     float* logits, int32_t* dev_status, cad_stream stream);

/* ---- CopyLoop's concurrent pipeline on a looped model (loop_depth D > 1) ----
 * CopyLoop §2 "Concurrent Pipeline": positions at different recurrence
 * depths advance together, each on its own depth's KV states; §2 "Shallow
 * Screening" and "Full-Depth Verification" read them out at depths ds and D.
 *
 * cad_loop_step: one tick.  Every group -- a run of `rows` consecutive
 * positions starting at absolute position `pos`, that has had `depth`
 * applications of the shared block so far -- gets one more application, on
 * cache index `depth` (its rows attend to keys 0 .. pos + j of that depth's
 * cache, and write their own K/V there).  A group's residual streams live in
 * the caller's `state` (dev fp32 [state_rows][d_model], rows state ..
 * state + rows - 1): read at the start of the tick for depth > 0 (depth 0
 * starts from the embedding of the group's tokens), written back at its end.
 * Groups must not share state rows; older (lower-position) groups must be
 * deeper, so that every key a row reads has been written at its depth.
 * tokens: dev int32 [total rows], the groups' tokens in group order.  If any
 * group has readout = 1, the final norm and LM head run after the tick and
 * argmax (dev int32 [total rows]; masked by `mask`, dev uint32 [total
 * rows][ceil(V/32)] or NULL) and accepted (dev int32 [n_groups]; the VERIFY
 * rule applied to each group's tokens) are written for every row and group
 * (the caller uses those of its readout groups), and the fp32 logits of
 * every row to `logits` (dev float [total rows][V]) if it is not NULL;
 * otherwise none of them is touched.  Each group reads and writes its
 * positions through block-table row `table_row` (one request: row 0; two
 * lines of blocks over the same positions, as branching makes, map their
 * own positions to different blocks).
 * 1 <= n_groups <= CAD_MAX_SEQS; total rows <= max_tokens. */
typedef struct {
  int64_t pos;        /* absolute position of the group's first row */
  int32_t rows;       /* >= 1 consecutive positions */
  int32_t depth;      /* applications done before this tick, 0 .. loop_depth - 1 */
  int32_t state;      /* first row of the group in `state` */
  int32_t readout;    /* 1: masked argmax + acceptance after the tick; 0: none */
  int32_t table_row;  /* block-table row its positions map through (>= 0; the caller's table holds it) */
} cad_loop_group;
cad_status cad_loop_step(cad_model* m, const cad_kv* kv, int32_t n_groups, const cad_loop_group* groups,
                         const int32_t* tokens, float* state, int32_t state_rows, const uint32_t* mask,
                         int32_t* argmax, int32_t* accepted, float* logits, int32_t* dev_status,
                         cad_stream stream);

/* cad_loop_decode: CopyLoop decoding of one request on a looped model, the
 * native scheduler over cad_loop_step (CopyLoop §2; §A.1 "Decoding
 * algorithm").  The prompt (host int32 [L0]) is prefilled at every depth and
 * its last full-depth prediction is the first token.  Then every tick
 * advances every block in flight by one depth: a block is a head followed by
 * up to max_copy tokens copied after the longest earlier match of the
 * history's suffix (lengths max_ngram down to min_ngram, the suffix-match
 * kernel); at screen_depth its tail is cut to the prefix agreeing with the
 * predictions one position earlier, the cut rows are released and the last
 * survivor's prediction heads the next block; at the full depth the tail is
 * verified the same way -- the first mismatch commits the full-depth token as
 * a correction and discards the block's rest and every younger block, a full
 * match commits the last prediction as the next token (which the next
 * block's head must equal, or that block and its descendants are discarded
 * the same way).  At most max_rows rows are in flight: a block admitted with
 * r free rows keeps at most r - 1 copied tokens, a head with no free row
 * waits.  The committed tokens (out, host int32 [n_new]) are greedy
 * full-depth decoding's.  With branch_depth = d2 > 0 (CopyLoop §A.2) a
 * block is also read out at depth d2: if the prediction at its last
 * surviving row differs there from the depth-ds one that headed its child,
 * a second child headed by the d2 prediction is admitted (at most one such
 * fork is live; it needs a free row and the first child in flight); the
 * two children's lines keep their own KV states -- the second line maps its
 * positions through block-table row 1, whose first spare entries (at least
 * ceil((loop_depth x (max_copy + 1) + 16) / 16) + 1 blocks not used by row
 * 0) the caller provides, the slots of older positions in the block where
 * the fork starts being copied there as they are written -- until the
 * parent's full-depth readout keeps the line whose head is the verified
 * token (the second line's K/V are then copied into row 0's blocks) or
 * neither (a correction block follows).  The host reads decisions back after every tick
 * that reads a block out (and after each proposal): this call synchronises
 * its stream.  cad_loop_create allocates the pipeline's device buffers (the
 * residual streams of loop_depth x (max_copy + 1) rows -- twice that with
 * branching --, a device history of max_len tokens -- four with branching:
 * the two lines' and a possible second child's per line -- and with
 * branching a two-row block table of ceil(max_len / 16) entries per row)
 * and pinned host staging; the model's max_tokens bounds the rows per tick
 * and the prefill chunk.  max_len and block-table row 0 must hold L0 + n_new
 * + loop_depth x (max_copy + 1) positions; with branching the caller's
 * table has two rows (the first spare entries of row 1 as above, in the
 * pool, distinct and not in row 0's first blocks; checked on the host).  The
 * KV cache is overwritten from position 0 (the spare blocks too). */
typedef struct cad_loop cad_loop;
typedef struct {
  int32_t screen_depth;  /* ds, 1 <= ds < loop_depth */
  int32_t max_copy;      /* K, 0 .. 64 */
  int32_t max_ngram, min_ngram;  /* suffix lengths, 1 <= min <= max <= 64 */
  int32_t max_rows;      /* admission limit: rows in flight, >= 1, <= max_tokens */
  int32_t branch_depth;  /* d2 of second-readout branching, ds < d2 < loop_depth; 0: none */
} cad_loop_params;
typedef struct {
  int64_t ticks;         /* cad_loop_step calls */
  int64_t rows_run;      /* rows advanced by one depth, summed over ticks */
  int64_t blocks;        /* blocks admitted */
  int64_t proposed;      /* copied tokens proposed */
  int64_t screened_out;  /* copied rows released at the screening depth */
  int64_t rejected;      /* copied rows refused at the full depth */
  int64_t discarded;     /* rows of younger blocks dropped with a refusal */
  int64_t committed;     /* tokens committed (may pass n_new by a block) */
  int64_t host_syncs;    /* host synchronisations */
  int64_t forks;         /* second children admitted (branching) */
  int64_t forks_kept;    /* resolutions that kept the second child's line */
  int64_t forks_lost;    /* resolutions that kept the first child's line */
  int64_t fork_rows_dropped;  /* rows in flight of the line removed there (also in discarded) */
  int32_t dev_status;    /* CAD_DEV_* bits seen by the device */
} cad_loop_stats;
cad_status cad_loop_create(cad_model* m, int64_t max_len, const cad_loop_params* p, cad_loop** out);
void cad_loop_destroy(cad_loop* lp);
cad_status cad_loop_decode(cad_loop* lp, const cad_kv* kv, const int32_t* prompt, int64_t L0, int32_t n_new,
                           int32_t* out, cad_loop_stats* stats, cad_stream stream);

/* ---- Copy-as-Decode program decoding (Copy-as-Decode §2) ----
 * cad_program_decode: the model writes a program over a document, one
 * request, with the grammar automaton on the device (§2.1 grammar, §2.3
 * masked steps and forced-template prefills, appendix "States.", "Forced
 * prefills." and "Token-sequence end-of-gen detector."):
 *   program := <program> op* </program>;  op := <copy lines="a-b"/> | <gen> text </gen>
 * The prompt (host int32 [L0], ending with the ids of "<program>") is
 * prefilled; then every decision is the masked argmax of the last fed row:
 * at an op boundary {"<"} (first op) or {"<", "</"} ({"</"} once max_ops
 * ops are done); after "<" {copy, gen}; inside a copy range the digits that
 * keep the number reachable (no leading zero, the first number in [1, U],
 * the second in [first, U]; U = the document's lines, or tokens when
 * unit_tokens = 1, §5 "Token-level extension."), then "-" or the closing
 * quote; inside a gen body every id (free generation) until the rolling
 * window over the last three ids holds the ids of "</gen>", or max_gen ids.
 * What follows a decision is fed in one forward: the chosen id alone; a
 * forced template ("copy" kw '="' after copy, "gen" ">" after gen, "</"
 * "program" ">" for the end, "</gen>" after a length-capped body); after the
 * closing quote, the quote, "/>" and the document's units a..b (the copy
 * splice, §2.4).  Inside a gen body with draft_k > 0, the pending id and up
 * to draft_k ids continuing the most recent earlier match of the suffix of
 * document + stream (lengths 4 down to 1) are verified in one forward (§5
 * "Composition with speculative decoding."; lossless: the stream is the
 * same as without drafts).  Decoding stops after the terminator, or at the
 * first decision once max_stream program ids have been fed.
 * The host synchronises when the next forward's length depends on a
 * decision (a template, a copy, a verify) and otherwise launches up to
 * `chain` single steps ahead; a chained step whose chain has ended (the
 * decision before it asked for a longer feed) writes its K/V past the end of
 * the stream, where the next forward overwrites it, and takes no decision.
 * Results: stream_out (host int32 [stream_cap]) the program ids fed after
 * the prompt; ops_out (host int32 [max_ops][5]) one record per op: kind (0
 * copy, 1 gen), a, b (copy), body start in the stream, body length (gen; an
 * unfinished body at a stop counts its ids so far); out (host int32
 * [out_cap]) the resolved output (§2.2: copies expanded to the document,
 * gen bodies as generated).  A result longer than its buffer is truncated
 * and the call returns CAD_E_CAPACITY (stats are filled either way).
 * doc: host int32 [doc_n], 1 <= doc_n <= max_doc; line_start: host int32
 * [n_lines + 1], line_start[0] = 0, non-decreasing, line_start[n_lines] =
 * doc_n (NULL allowed when unit_tokens = 1).  Needs loop_depth 1,
 * max_tokens >= draft_k + 1 and a block table and max_len holding L0 +
 * max_stream + 2 x max_doc + 2 x draft_k + chain + 16 positions.  The KV
 * cache is overwritten from position 0.  The call synchronises its stream. */
typedef struct cad_program cad_program;
typedef struct {
  int32_t lt, lt_slash, gt;        /* "<", "</", ">" */
  int32_t copy, gen, program;      /* tag names */
  int32_t kw;                      /* " lines" (or " tokens") */
  int32_t eq_quote, quote, slash_gt, hyphen;  /* '="', '"', "/>", "-" */
  int32_t digits[10];              /* "0" .. "9" */
} cad_program_table;
typedef struct {
  int32_t max_doc;     /* most document tokens, >= 1 */
  int32_t max_stream;  /* no decision once this many program ids are fed, >= 1 */
  int32_t max_ops;     /* ops per program, >= 1 */
  int32_t max_gen;     /* ids per gen body, >= 1 */
  int32_t draft_k;     /* drafted ids per verify inside gen bodies, 0 (no drafts) .. 64 */
  int32_t chain;       /* most single steps launched between host synchronisations, 1 .. 64 */
} cad_program_params;
typedef struct {
  int64_t forwards;         /* forwards that fed program ids, plus one for the prompt */
  int64_t idle_steps;       /* chained steps launched after their chain had ended */
  int64_t host_syncs;       /* host synchronisations */
  int32_t decisions;        /* decisions taken */
  int32_t masked_steps;     /* of them under a mask (every decision outside gen bodies) */
  int32_t forced_prefills;  /* template feeds */
  int32_t copies, copied_tokens;
  int32_t drafts, draft_tokens, draft_accepted;  /* verify forwards, drafted ids, accepted ids */
  int32_t stream_n;         /* program ids fed */
  int32_t n_ops;            /* op records (an unfinished gen op included) */
  int32_t out_n;            /* resolved output length */
  int32_t fsm_error;        /* 0; 1: a decision outside its mask (a mask that allowed nothing) */
  int32_t dev_status;       /* CAD_DEV_* bits seen by the device */
} cad_program_stats;
cad_status cad_program_create(cad_model* m, int64_t max_len, const cad_program_table* t,
                              const cad_program_params* p, cad_program** out);
void cad_program_destroy(cad_program* pr);
cad_status cad_program_decode(cad_program* pr, const cad_kv* kv, const int32_t* prompt, int64_t L0,
                              const int32_t* doc, int32_t doc_n, const int32_t* line_start, int32_t n_lines,
                              int32_t unit_tokens, int32_t* stream_out, int32_t stream_cap, int32_t* ops_out,
                              int32_t* out, int32_t out_cap, cad_program_stats* stats, cad_stream stream);

/* ---- instrumentation (measurement only, not part of the method) ----
 * Kernel families, in bit order: 0 "embed", 1 "rmsnorm", 2 "gemm_qkv",
 * 3 "rope_append", 4 "attention" (the partial-attention kernel), 5
 * "attn_merge" (the log-sum-exp merge of key partitions), 6 "gemm_o",
 * 7 "gemm_gate_up", 8 "gemm_down", 9 "gemm_lm_head" (with the mask and the
 * per-tile argmax in its epilogue), 10 "decide" (the argmax over the LM
 * head's tiles and the acceptance scan), 11 "loop_state" (loading and saving
 * the residual streams of a pipeline tick).  Each family is one kernel (one
 * named kernel per path; the LM head after a k split adds its reduce).
 * cad_profile_enable(m, family_mask) starts a fresh collection in which
 * every launch of a family whose bit is set is bracketed by a pair of
 * hipEvents recorded on the launch's stream (synchronises the device once);
 * family_mask 0 stops recording (records are kept until the next start; -1
 * records every family).  cad_profile_read waits for the recorded events of
 * `family` and returns how many launches were recorded and their summed
 * duration in milliseconds.  Unknown family: CAD_E_ARG. */
#define CAD_PROFILE_ALL (-1)
cad_status cad_profile_enable(cad_model* m, int32_t family_mask);
cad_status cad_profile_read(cad_model* m, const char* family, int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif
#endif /* CAD_H */
