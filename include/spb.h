/* spb.h -- C ABI of libspb: the packed forward of one token-budget scoring pass
 * on an AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [PyPI]    "spinf-serve 0.1.1", project page on pypi.org;
 *   [man]     "spinf-serve", man page on linuxcommandlibrary.com;
 *   [article] "Bulk classification and decision inference on one GPU"
 *             (English original on aitujian.cn).
 *
 * The pass: many inputs are packed into one forward pass of at most a token
 * budget (16,384 by default) [PyPI "What it does": Throughput; man PARAMETERS
 * --token-budget].  Each input is a content read once, followed by its
 * questions as branches of that read [PyPI "What it does": Many questions, one
 * read].  A question is a template ending where the answer goes; multi-token
 * options hang under it as a token trie [PyPI "What it does": Scoring; PyPI
 * "Layout": compiler.py].  Every token attends to its own content and the
 * causal prefix of its own branch only.  At the answer slot each option gets a
 * vocab-wide log-probability, p renormalised over the options, the residual
 * mass outside them, and the floor p of the same question on empty content
 * [article, the response example and the paragraph after it].
 *
 * Conventions for every call:
 *   - The caller owns every buffer (host arrays and device memory).  The library
 *     owns only the opaque plan.  No call allocates device memory or
 *     synchronises a stream; work is enqueued on the caller's stream
 *     (a hipStream_t passed as void*, NULL = the null stream).
 *   - All argument and limit checks run on the host before any HIP call, so a
 *     call that returns an error has enqueued nothing.  Kernel faults surface
 *     at the caller's next synchronisation as HIP errors.
 *   - Errors: a negative spb_status; spb_last_error() gives a message
 *     (thread-local, valid until the next spb_* call on that thread).
 *   - Plans are immutable after spb_pack_pass: concurrent readers are safe.
 *   - Results are a function of the logical problem alone: an input's scores
 *     are bit-identical whatever it is packed with, in any order, at any budget
 *     ("batch invariance", [PyPI "What it does"]).
 */
#ifndef SPB_H
#define SPB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t spb_status;
enum {
  SPB_OK = 0,
  SPB_ERR_ARG = -1,   /* null pointer, malformed CSR, token id >= vocab, duplicate option */
  SPB_ERR_LIMIT = -2, /* a request limit or the token budget is exceeded                  */
  SPB_ERR_DTYPE = -3, /* unsupported dtype, head_dim, GQA ratio or hidden size            */
  SPB_ERR_SIZE = -4,  /* caller buffer, metadata or workspace too small                   */
  SPB_ERR_HIP = -5    /* HIP runtime or launch error (no device, bad launch)               */
};

typedef enum { SPB_F32 = 0, SPB_BF16 = 1, SPB_FP8_E4M3 = 2 /* OCP e4m3fn */ } spb_dtype;

/* The message of the last failed spb_* call on the calling thread: what went
 * wrong, with the offending index or size (e.g. "question 3: template of 300
 * tokens exceeds max_query_tokens 256").  The pages name the engine's error
 * envelopes without giving their contents [PyPI "Status": the response and
 * error envelopes]; this string is what such an envelope's message would
 * carry, and the negative spb_status its kind.  Returns "" when the last
 * spb_* call on this thread succeeded (or none was made).  The pointer is
 * library-owned, thread-local and valid until the next spb_* call on the same
 * thread; never NULL. */
const char *spb_last_error(void);
/* Build id, tile constants and numerics-contract version.  Two results are
 * bit-comparable when their fingerprints are equal (PyPI "What it does":
 * system_fingerprint). */
const char *spb_fingerprint(void);

/* ------------------------------------------------------------------ problem
 * The logical problem, in token ids.  Host memory, owned by the caller, read
 * only during spb_pack_pass.
 *   input i: content of content_len[i] tokens; asks the questions
 *            branch_q[branch_off[i] .. branch_off[i+1]).
 *   question q: template of q_len[q] tokens (the last one is the row in front
 *            of the answer slot, whose next-token distribution scores the
 *            options' first tokens); options opt_off[q] .. opt_off[q+1).
 *   option o: tokens tok[tok_off[o] .. tok_off[o+1]).
 * Options of one question must be distinct (SPB_ERR_ARG).  An option that is
 * a prefix of another is accepted; then the residual can be negative.
 *
 * Logical rows (the numbering activations are addressed by): inputs in order,
 * then, with floors, one floor input per distinct asked question in ascending
 * id; inside an input its content rows, then per branch the template rows
 * followed by the option-trie nodes of its question.  Trie nodes are the
 * distinct proper prefixes of the options in first-appearance order (options
 * in order, each option's prefixes by increasing length).
 *
 * Template tries [PyPI "Layout": the engine compiles templates into token
 * tries; "What it does": placeholder values expand one template into many
 * questions]: with tmpl_tok
 * (the template token ids, question after question, q_len[q] each; NULL: none
 * given), the questions of one input share the tokens of every template prefix
 * that at least two of them start with, except that a question's last
 * template token is always its own.  A shared token is one logical row; the
 * shared rows of a branch's template come, in template order, right before
 * its first own template row in the numbering when they have not appeared
 * earlier in that input.  Token ids are only compared, never bounds-checked
 * against the vocabulary. */
typedef struct {
  int32_t n_inputs;
  const int32_t *content_len; /* [n_inputs], >= 0                  */
  const int32_t *branch_off;  /* [n_inputs + 1]                    */
  const int32_t *branch_q;    /* [branch_off[n_inputs]]            */
  int32_t n_questions;
  const int32_t *q_len;       /* [n_questions], >= 1               */
  const int32_t *opt_off;     /* [n_questions + 1]                 */
  const int32_t *tok_off;     /* [opt_off[n_questions] + 1]        */
  const int32_t *tok;         /* [tok_off[n_options]], < vocab     */
  int32_t vocab;
  const int32_t *tmpl_tok;    /* [sum q_len] or NULL (no sharing)  */
} spb_problem;

/* Packing options; request limits default to the man page's [man PARAMETERS]. */
typedef struct {
  int32_t token_budget;          /* packed tokens per pass, default 16384                    */
  int32_t floors;                /* 1: add one empty-content floor branch per asked question */
  int32_t max_content_tokens;    /* default 4096                                             */
  int32_t max_query_tokens;      /* default 256 (template length)                           */
  int32_t max_options;           /* default 1000 (per question)                             */
  int32_t max_option_tokens;     /* default 5                                                */
  int32_t max_prompts_per_input; /* default 10000 (branches per input)                      */
  int64_t max_processed_tokens;  /* default 2000000 (all passes, re-staged content, floors) */
} spb_pack_opts;

/* Fills *opts (caller-owned) with the defaults: a 16,384-token budget [man
 * PARAMETERS --token-budget], floors on [article, the floor paragraph], and the
 * man page's request limits [man PARAMETERS].  A NULL opts is ignored. */
void spb_pack_opts_default(spb_pack_opts *opts);

typedef struct spb_plan spb_plan; /* opaque, library-owned */

typedef struct {
  int32_t n_tokens;       /* packed rows of the pass                          */
  int32_t n_segments;     /* placed contents (a re-staged content counts again) */
  int32_t n_branches;     /* branches placed (content + floor)                */
  int32_t n_options;      /* option slots (lp / p outputs)                    */
  int32_t n_scored_rows;  /* rows fed to the lm head                          */
  int32_t n_targets;      /* distinct (scored row, next token) logits captured */
  int32_t n_tiles;        /* attention tiles (at most 128 rows of one segment) */
  int32_t n_passes;       /* totals only (pass = -1)                          */
  int64_t unmasked_pairs; /* (query row, key row) pairs attended, per head    */
  size_t meta_bytes;      /* device metadata size for spb_plan_upload         */
  int32_t n_content_branches, n_content_options; /* totals only: finalize sizes */
  int32_t n_logical_inputs; /* totals only: inputs, then floor inputs           */
} spb_pass_info;

/* Packs every input (and the floors) into passes of at most token_budget rows.
 * Rule: inputs in order, then floors; an input goes whole into the current
 * pass if it fits, else whole into a new pass; an input larger than the
 * budget spills at branch boundaries, its content re-staged in each pass it
 * continues in.  SPB_ERR_LIMIT when content + one branch exceeds the budget.
 * Cites [PyPI "What it does": Throughput; man PARAMETERS --token-budget,
 * --max-tokens and the request limits; man CAVEATS]. */
spb_status spb_pack_pass(const spb_problem *problem, const spb_pack_opts *opts, spb_plan **out);
/* Releases a plan made by spb_pack_pass (NULL is accepted and ignored).  The
 * pages name no such step: the plan is this library's own handle.  Device
 * memory the caller filled from the plan (uploaded metadata) stays the
 * caller's; after the call the plan must not be used. */
void spb_plan_free(spb_plan *plan);
/* The number of passes the plan packs its inputs into (*n >= 1).  The pages
 * count passes for the news set ("packs the 24 articles into two 16k-token
 * passes" [PyPI "Speed and scale"]) and add packed tokens and engine
 * internals to a response on request [man PARAMETERS --debug]; this is that
 * count.  SPB_ERR_ARG for a NULL plan or n. */
spb_status spb_plan_num_passes(const spb_plan *plan, int32_t *n);
/* Sizes of pass `pass` (0 .. n_passes-1), or with pass = -1 the sums over
 * all passes (meta_bytes then is the largest pass's): the packed tokens and
 * engine internals a debug response shows [man PARAMETERS --debug], and every
 * size a caller needs to allocate the pass's device buffers (n_tokens rows of
 * Q/K/V/O and hidden states, meta_bytes of metadata, n_options and n_branches
 * score outputs).  n_passes, n_content_branches, n_content_options and
 * n_logical_inputs are plan totals in every call.  *out is caller-owned host
 * memory.  SPB_ERR_ARG for a NULL argument or a pass out of range. */
spb_status spb_plan_info(const spb_plan *plan, int32_t pass, spb_pass_info *out);
/* The placement map of one pass [PyPI "Layout": packer.py packs; man
 * PARAMETERS --debug: packed tokens]: logical_row[n_tokens] receives the
 * logical row (numbered as above) placed at each pass row; a re-staged
 * content row appears in every pass that holds it.  scored_row[n_scored_rows]
 * receives the pass rows read by the lm head, in scoring order.  Either
 * pointer may be NULL (that array is skipped).  Host buffers, caller-owned,
 * sized from spb_plan_info.  SPB_ERR_ARG for a NULL plan or a pass out of
 * range; nothing is written then. */
spb_status spb_plan_rows(const spb_plan *plan, int32_t pass, int64_t *logical_row, int32_t *scored_row);
/* Per placed branch of the pass (every question is a branch of its input's
 * read [PyPI "What it does": Many questions, one read]): its logical branch
 * (content branches numbered in input / CSR order, then floor branches in
 * ascending question id) and its first option slot in the pass's lp / p
 * outputs.  Host arrays of n_branches, caller-owned; either pointer may be
 * NULL.  SPB_ERR_ARG for a NULL plan or a pass out of range. */
spb_status spb_plan_branches(const spb_plan *plan, int32_t pass, int32_t *logical_branch, int32_t *opt_first);
/* Logical inputs in row-numbering order (inputs, then floor inputs, one per
 * asked question [article, the floor paragraph]): row_off[n_logical_inputs +
 * 1] is the first logical row of each; floor_question[n_logical_inputs] is the
 * question of a floor input, -1 for a content input.  The numbering is this
 * library's addressing of activations; the pages have none.  Host arrays,
 * caller-owned; either pointer may be NULL.  SPB_ERR_ARG for a NULL plan. */
spb_status spb_plan_inputs(const spb_plan *plan, int64_t *row_off, int32_t *floor_question);
/* Host debugging aid: the pass rows that pass row `row` attends to (its own
 * content and the causal prefix of its own branch [PyPI "What it does": Many
 * questions, one read]), read from the same metadata and visibility rule the
 * kernel uses, in key order.  keys[cap] is caller-owned; *n_keys receives the
 * count.  SPB_ERR_ARG for a NULL argument or a pass or row out of range,
 * SPB_ERR_SIZE when more than cap keys are visible. */
spb_status spb_plan_visible(const spb_plan *plan, int32_t pass, int32_t row, int32_t *keys, int32_t cap,
                            int32_t *n_keys);
/* Enqueues the host-to-device copy of the pass's metadata (meta_bytes bytes:
 * row, tile, work-item, chunk, branch and scoring tables, the layout
 * branch_attention and score_options read) into d_meta on `stream` (a
 * hipStream_t; NULL = the null stream).  The pages name no upload step: it is
 * the host-to-device half of one packed forward [PyPI "Layout": packer.py,
 * scorer.py].  d_meta: device memory of at least `bytes` >= meta_bytes,
 * 256-byte aligned, caller-owned; it must stay untouched until the copy and
 * every kernel reading it have run.  The host side is read from the plan,
 * which must outlive the copy.  Checks run first and enqueue nothing on
 * failure: SPB_ERR_ARG (NULL plan or d_meta, pass out of range, misaligned
 * d_meta), SPB_ERR_SIZE (bytes < meta_bytes); SPB_ERR_HIP if the runtime
 * refuses the copy. */
spb_status spb_plan_upload(const spb_plan *plan, int32_t pass, void *d_meta, size_t bytes, void *stream);
/* Host-to-host copy of the same metadata bytes into caller memory (bytes >=
 * meta_bytes), e.g. pinned memory from which the caller uploads the pass
 * asynchronously on a copy stream, overlapping the previous pass's kernels.
 * The device layout is identical to what spb_plan_upload writes.  No passage
 * of the pages: a staging variant of the upload.  SPB_ERR_ARG (NULL argument,
 * pass out of range), SPB_ERR_SIZE (bytes < meta_bytes); nothing written then. */
spb_status spb_plan_meta_copy(const spb_plan *plan, int32_t pass, void *host_dst, size_t bytes);

/* ------------------------------------------------------------------ attention
 * For every packed row x and query head h:
 *   O[x,h] = sum_{y in path(x)} softmax_y(scale * q[x,h] . k[y,g]) v[y,g],
 *   g = h / (hq / hkv),
 * path(x) = own content (causal for content rows, all of it for branch rows),
 * own template prefix, own option-trie ancestors.  Equals plain causal
 * attention over each content + branch sequence run alone [PyPI "Speed and
 * scale": the same answers as per-question prompts].
 * Layout: q [rows, hq, d], k and v [rows, hkv, d], o [rows, hq, d], token-major,
 * contiguous, device memory, rows >= n_tokens of the pass.  All inputs finite.
 * in_dtype: SPB_F32 (rounded to bf16 on load), SPB_BF16, or SPB_FP8_E4M3 with
 * per-tensor dequantisation scales s_q, s_k, s_v (static "fp8s"-style
 * calibration [man DESCRIPTION: calibrate]; QK^T on fp8 MFMA, P.V on bf16).
 * out_dtype: SPB_F32 or SPB_BF16.  head_dim 64 or 128; hq % hkv == 0 and
 * hq / hkv in {1, 2, 4}.  softmax_scale <= 0 selects 1/sqrt(head_dim).
 * SPB_BF16 passes need n_tokens * hkv * head_dim * 2 < 4 GiB (SPB_ERR_LIMIT).
 * d_meta: the upload of (plan, pass).
 * workspace (SPB_FP8_E4M3 only; ignored otherwise): NULL, or device memory of
 * spb_attention_workspace_bytes, 256-byte aligned, caller-owned, not shared
 * with a call in flight.  With it, V is first widened to bf16 there (exact:
 * every e4m3 value is a bf16 value) and K/V chunks reach LDS by asynchronous
 * copies; without it they pass through registers.  The two give the same
 * bits: same MFMAs in the same order.  SPB_ERR_SIZE if it is too small;
 * SPB_ERR_LIMIT if the widened V (n_tokens * hkv * head_dim * 2) reaches 4 GiB. */
typedef struct {
  const void *q, *k, *v;
  void *o;
  int32_t in_dtype, out_dtype;
  int32_t hq, hkv, head_dim;
  float softmax_scale;
  float s_q, s_k, s_v;
  int64_t rows; /* rows of q/k/v/o buffers, >= n_tokens */
  void *workspace;
  size_t workspace_bytes;
} spb_attn_args;

/* Workspace bytes spb_branch_attention can use for this pass and input
 * dtype: n_tokens * hkv * head_dim * 2 for SPB_FP8_E4M3 (V widened to bf16),
 * 0 otherwise.  SPB_ERR_ARG for a pass out of range or hkv / head_dim < 1. */
spb_status spb_attention_workspace_bytes(const spb_plan *plan, int32_t pass, int32_t in_dtype, int32_t hkv,
                                         int32_t head_dim, size_t *out);

/* Roofline calibration, not part of the scoring path (the pages have no such
 * step): the rate the head's MFMA (32x32x16 bf16, f32 accumulation) sustains
 * alone.  Enqueues work_groups (1 .. 2^20) work groups of four waves, each wave
 * running 16 independent accumulators through 16 x iters MFMAs on operands
 * held in registers -- random bf16 values (random_operands != 0) or small
 * integers -- with no memory traffic in the loop; flops = work_groups * 4 *
 * iters * 16 * 32768.  The caller times it with events on `stream`.  d_out:
 * device memory of work_groups * 256 floats, caller-owned (overwritten with
 * sums that keep the loop from being eliminated).  SPB_ERR_ARG / SPB_ERR_LIMIT
 * for bad sizes before any HIP call. */
spb_status spb_mfma_calibration(float *d_out, int32_t work_groups, int32_t iters, int32_t random_operands,
                                void *stream);

spb_status spb_branch_attention(const spb_plan *plan, int32_t pass, const void *d_meta, const spb_attn_args *args,
                                void *stream);

/* ------------------------------------------------------------------ scoring
 * For every scored row r (each template's last row and each trie node):
 *   z_r = W h_r over the whole vocabulary; LSE_r = log sum exp z_r.
 * The lm head's output kind [man page "spinf-serve", PARAMETERS --lm-head]:
 *   SPB_HEAD_F32OUT (0, default): bf16 W times bf16 h (an f32 hidden row is
 *     rounded to bf16), f32 logits;
 *   SPB_HEAD_BF16 (1): the same product, each logit rounded to bf16 (nearest
 *     even) before the log-sum-exp and the option gather;
 *   SPB_HEAD_FP32 (2): bf16 W (exact in f32) times the f32 hidden row without
 *     rounding it: h is split into three bf16 terms whose sum is h, each
 *     multiplied on the bf16 MFMA with f32 accumulation (three times the
 *     f32out work; for bf16 hidden rows it equals f32out).
 * For option o of a branch with tokens t_1..t_n:
 *   lp_o = sum_k z_{r_{k-1}}[t_k] - LSE_{r_{k-1}}  (r_0 = template's last row,
 *          r_k = trie node of t_1..t_k);
 *   p_o  = exp(lp_o) / sum_{o'} exp(lp_o')        (probability among the options);
 *   residual = 1 - sum_o exp(lp_o)                (mass outside the options)
 * [article, the response example and the paragraph after it].
 * hidden [rows, hidden_dim] (SPB_BF16, or SPB_F32 rounded to bf16 on load),
 * only scored rows are read; lm_head [vocab, hidden_dim] bf16 row-major;
 * hidden_dim % 64 == 0.  Outputs (device, f32): lp and p [n_options],
 * residual [n_branches], in the pass's slot order.  workspace: device memory
 * of spb_score_workspace_bytes for the same lm_head_kind, 256-byte aligned;
 * no state is kept in it between calls.  An lm_head_kind outside 0..2 is
 * SPB_ERR_ARG. */
enum { SPB_HEAD_F32OUT = 0, SPB_HEAD_BF16 = 1, SPB_HEAD_FP32 = 2 };
typedef struct {
  const void *hidden;
  int32_t h_dtype;
  int32_t hidden_dim;
  int64_t rows; /* rows of the hidden buffer, >= n_tokens */
  const void *lm_head;
  int32_t vocab;
  void *workspace;
  size_t workspace_bytes;
  float *lp, *p, *residual;
  /* Optional timing hooks: hipEvent_t handles (created by the caller) recorded
   * on the stream right before and right after the lm-head GEMM kernel, so a
   * caller can time that kernel alone.  NULL: not recorded. */
  void *gemm_event_begin, *gemm_event_end;
  int32_t lm_head_kind; /* SPB_HEAD_*; 0 (f32out) in a zero-initialised struct */
} spb_score_args;

/* Workspace bytes spb_score_options needs for this pass, vocabulary, hidden
 * size and lm-head kind. */
spb_status spb_score_workspace_bytes(const spb_plan *plan, int32_t pass, int32_t vocab, int32_t hidden_dim,
                                     int32_t lm_head_kind, size_t *out);
spb_status spb_score_options(const spb_plan *plan, int32_t pass, const void *d_meta, const spb_score_args *args,
                             void *stream);

/* spb_score_options for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, bit for bit, with the workspace
 * taken from a library-owned device array of 64 MiB per GPU instead of
 * args->workspace (which is ignored, as is workspace_bytes).  The array is
 * in the library's code object: each GPU the library runs on holds its own
 * copy until the process ends; its address is looked up once per device, on
 * the first call with that device current.  The call allocates nothing.
 * Every call on one GPU shares that GPU's array and finds the last call's
 * contents there (the kernels write every byte they read, so nothing needs
 * clearing): calls that overlap on one GPU, on different streams or threads,
 * race and corrupt each other's results; serialise them.  A pass whose
 * workspace (spb_score_workspace_bytes) exceeds 64 MiB is refused with
 * SPB_ERR_SIZE before anything is enqueued: about 4,200 scored rows at
 * vocabulary 262,144 and hidden 3,840 with f32out or bf16 output, 2,100 with
 * fp32.  Otherwise the arguments, checks and errors are spb_score_options'. */
spb_status spb_score_options_noalloc(const spb_plan *plan, int32_t pass, const void *d_meta,
                                     const spb_score_args *args, void *stream);

/* Several passes' scored rows through ONE lm-head stream: W is read once for
 * the whole batch instead of once per pass (for passes whose scored rows alone
 * leave the head HBM-bound, this moves the head toward its MFMA roofline).
 * Every output equals, bit for bit, what spb_score_options gives pass by
 * pass: each logit depends only on its W row and hidden row (fixed K order)
 * and each row's vocabulary-slice merge runs in a fixed order.
 * passes[0..n): distinct passes of the plan (n <= 64); d_metas[i]: the upload
 * of passes[i]; args[i]: hidden, rows, lp, p, residual of passes[i] (all
 * entries must agree on h_dtype, hidden_dim, lm_head, vocab and
 * lm_head_kind; the workspace fields and the timing events are read from
 * args[0] only, the events bracketing the single GEMM launch).  workspace:
 * device memory of spb_score_batch_workspace_bytes, 256-byte aligned. */
spb_status spb_score_batch_workspace_bytes(const spb_plan *plan, int32_t n, const int32_t *passes, int32_t vocab,
                                           int32_t hidden_dim, int32_t lm_head_kind, size_t *out);
spb_status spb_score_options_batch(const spb_plan *plan, int32_t n, const int32_t *passes, const void *const *d_metas,
                                   const spb_score_args *args, void *workspace, size_t workspace_bytes,
                                   void *stream);

/* Host, after all passes: gathers each content branch's results into logical
 * order and joins the floors.  *_per_pass[k] are host copies of pass k's lp,
 * p and residual outputs.  Outputs (host, caller-owned): lp, p, floor_p, lift
 * [n_content_options] and residual [n_content_branches] in logical order
 * (content branches in input / CSR order, options in question order).
 * floor_p = p of the same question's floor branch, lift = p - floor_p
 * [PyPI "What it does": Scoring; article, after the response example]; NaN
 * when the plan has no floors.  Any output pointer may be NULL. */
spb_status spb_score_finalize(const spb_plan *plan, const float *const *lp_per_pass, const float *const *p_per_pass,
                              const float *const *residual_per_pass, float *lp, float *p, float *residual,
                              float *floor_p, float *lift);

/* ------------------------------------------------------------ decoder stack
 * The engine runs a whole decoder model over the packed pass and hands its
 * last hidden states to the head [PyPI "spinf-serve 0.1.1", "Layout": one
 * packed forward; models/ one stack per architecture family].  The pages do
 * not spell out the layer, so these calls build the plain pre-norm decoder
 * layer around spb_branch_attention, on the packed rows:
 *   h = rmsnorm(x) * g_attn;  q, k, v = h [Wq; Wk; Wv]^T, q and k rotated at
 *   each row's position (spb_plan_positions);  x += attention(q, k, v) Wo^T;
 *   h = rmsnorm(x) * g_mlp;  x += (silu(h Wg^T) * h Wu^T) Wd^T;
 * and rmsnorm(x) * g_final feeds spb_score_options.  x, the residual stream,
 * is f32; every other activation is bf16 (rounded to nearest even once, at
 * the end of the op that makes it).  Each row's results depend only on its
 * own root path, as for attention alone.  All calls enqueue on the stream,
 * allocate nothing and validate every argument before any HIP call. */

/* Position of each pass row on its own root path (content token t: t;
 * template token j: C + j; trie node of depth k: C + L - 1 + k), i.e. the
 * position the row has when its question runs as its own prompt.  host_out:
 * [n_tokens] int32, caller-owned. */
spb_status spb_plan_positions(const spb_plan *plan, int32_t pass, int32_t *host_out);

/* Rotary embedding table [n_pos][head_dim / 2][2] = (cos, sin) of
 * p * base^(-2i / head_dim), computed in double and rounded to f32: the
 * rotary position embedding of Su et al. (RoFormer), pairs (2i, 2i+1).
 * host_out: n_pos * head_dim floats, caller-owned; head_dim even. */
spb_status spb_rope_table(float *host_out, int32_t n_pos, int32_t head_dim, double base);

/* out[r] = bf16(x[r] / sqrt(mean(x[r]^2) + eps) * gain) for r < rows.
 * x: f32 [rows][dim]; gain: bf16 [dim]; out: bf16 [rows][dim]; device
 * memory, 16-byte aligned; dim % 4 == 0. */
typedef struct {
  const float *x;
  const void *gain;
  void *out;
  int64_t rows;
  int32_t dim;
  float eps;
} spb_rmsnorm_args;
spb_status spb_rmsnorm(const spb_rmsnorm_args *args, void *stream);

/* Linear layer on MFMA: acc = x W^T in f32 (x: bf16 [m][k], W: bf16 [n][k],
 * both row-major), K summed in a fixed order, so a row's result does not
 * depend on m.  Epilogues (mode):
 *   SPB_LINEAR_BF16:      y[m][n] = bf16(acc);
 *   SPB_LINEAR_RESIDUAL:  resid[m][n] += bf16(acc) (resid f32, in place);
 *   SPB_LINEAR_SILU_GATE: y[m][n/2] = bf16(silu(gate) * up), with W's rows
 *     in blocks of 64: rows 64j .. 64j+31 the gate rows 32j .. 32j+31 and
 *     rows 64j+32 .. 64j+63 the up rows 32j .. 32j+31 (n % 64 == 0);
 *   SPB_LINEAR_F32:       yf[m][n] = acc (f32; the lm head's logits of decoded rows);
 *   SPB_LINEAR_QKV_ROPE:  W = [Wq; Wk; Wv] (n = (hq + 2 hkv) head_dim); the
 *     three column ranges go to q [m][hq*d], k [m][hkv*d], v [m][hkv*d], q
 *     and k rotated by pos[r] with rope_table (spb_rope_table; positions
 *     clamped into [0, n_pos)).
 * k % 64 == 0, n % 8 == 0, m * k * 2 and n * k * 2 below 4 GiB; every
 * tensor is device memory, 16-byte aligned, caller-owned.  gemm_event_begin /
 * gemm_event_end: optional hipEvent_t handles recorded around the kernel. */
enum { SPB_LINEAR_BF16 = 0, SPB_LINEAR_RESIDUAL = 1, SPB_LINEAR_SILU_GATE = 2, SPB_LINEAR_QKV_ROPE = 3,
       SPB_LINEAR_F32 = 4 };
typedef struct {
  const void *x;
  const void *w;
  int64_t m;
  int32_t n, k;
  int32_t mode;
  void *y;
  float *resid;
  float *yf;
  void *q, *k_out, *v;
  int32_t hq, hkv, head_dim;
  const int32_t *pos;
  const float *rope_table;
  int32_t n_pos;
  void *gemm_event_begin, *gemm_event_end;
  /* fp8 = 1: x and W are OCP e4m3 bytes (spb_quantize_e4m3) with per-tensor
   * scales, multiplied on v_mfma_scale_f32_32x32x64_f8f6f4, acc scaled by
   * scale_x * scale_w before the epilogue; k % 128 == 0.  0: bf16 operands. */
  int32_t fp8;
  float scale_x, scale_w;
} spb_linear_args;
spb_status spb_linear(const spb_linear_args *args, void *stream);

/* dst[i] = e4m3(src[i] / scale) for i < n: the nearest OCP e4m3fn value (ties
 * to the even significand), saturated to +-448 -- the per-tensor static
 * quantization of the pages' fp8s checkpoints [man page "spinf-serve",
 * DESCRIPTION].  src: f32 or bf16 (src_dtype SPB_F32 / SPB_BF16), dst: bytes;
 * device memory, 16-byte aligned (src) and 8-byte aligned (dst). */
typedef struct {
  const void *src;
  int32_t src_dtype;
  void *dst;
  int64_t n;
  float scale;
} spb_quantize_args;
spb_status spb_quantize_e4m3(const spb_quantize_args *args, void *stream);

/* --------------------------------------------------------- extraction slots
 * A slot ({*} text, {n} a number, {$} an amount) is decoded from the same
 * read, with its answers' probabilities [PyPI "spinf-serve 0.1.1", "What it
 * does": Extraction and generation]; the slots of many inputs are decoded
 * together [PyPI "Speed and scale"].  The search is a beam search of width B:
 * step 0 takes the k best allowed tokens after the slot question's template
 * (its scored last row), every later step feeds each live beam's last token
 * through the decoder stack (spb_gather_rows, the layer calls with
 * spb_decode_attention in place of branch attention, the lm head as
 * spb_linear SPB_LINEAR_F32) and spb_topk_lse, and spb_beam_step keeps the B
 * best candidates: score (sum of the tokens' vocab-wide log-probabilities)
 * descending, then the earlier beam, then the smaller token id; finished
 * beams (the stop token chosen) stay candidates with their scores.  A step's
 * rows are slot-major: row r = slot * B + beam; the decode K/V cache of a
 * layer holds the rows of depth j (1-based) at rows (j - 1) * R + r. */

/* The slot question's template row and its prefix in the pass: the key rows
 * that row attends to (itself included), as runs (first pass row, count) in
 * attention order.  logical_branch: as in spb_plan_branches. */
enum { SPB_MAX_SLOT_RANGES = 16, SPB_MAX_TOPK = 16, SPB_MAX_BEAMS = 16 };
typedef struct {
  int32_t pass;
  int32_t row;
  int32_t position;
  int32_t n_ranges;
  int32_t ranges[SPB_MAX_SLOT_RANGES][2];
} spb_slot_info;
spb_status spb_plan_slot(const spb_plan *plan, int32_t logical_branch, spb_slot_info *out);

/* dst[r] = src[idx[r]] for r < rows (bf16 rows of dim; dst as f32 or bf16,
 * exactly one non-NULL), idx clamped into [0, n_src); with pos non-NULL also
 * pos[r] = pos_base[r / per] + pos_add (the positions of a decode step's rows). */
typedef struct {
  const void *src;
  int32_t n_src;
  const int32_t *idx;
  int64_t rows;
  int32_t dim;
  float *dst_f32;
  void *dst_bf16;
  int32_t *pos;
  const int32_t *pos_base;
  int32_t per, pos_add;
} spb_gather_args;
spb_status spb_gather_rows(const spb_gather_args *args, void *stream);

/* Per row of f32 logits [rows][vocab]: lse = log sum exp over the whole
 * vocabulary (a fixed-order reduction), and the k (<= 16) best tokens the
 * row's mask allows (the row's stop token always allowed) in the order
 * logit descending, then smaller id, as ids [rows][k] and lp = logit - lse;
 * -1 / -inf when fewer are allowed.  masks: [n_masks][ceil(vocab / 32)]
 * bit sets, mask_of_row[r] in [-1, n_masks) (-1: every token); both may be
 * NULL (every token); stop_of_row may be NULL. */
typedef struct {
  const float *logits;
  int64_t rows;
  int32_t vocab, k;
  const uint32_t *masks;
  int32_t n_masks;
  const int32_t *mask_of_row;
  const int32_t *stop_of_row;
  int32_t *ids;
  float *lp;
  float *lse;
  void *workspace; /* device, spb_topk_workspace_bytes, 16-byte aligned */
  size_t workspace_bytes;
} spb_topk_args;
spb_status spb_topk_workspace_bytes(int64_t rows, int32_t vocab, size_t *out);
spb_status spb_topk_lse(const spb_topk_args *args, void *stream);

/* Attention of a decode step's rows (q [rows][hq][d], after RoPE): row r of
 * slot s = r / beams attends to its slot's prefix ranges (spb_plan_slot) in
 * the pass's K/V of this layer (k_pass, v_pass [n_pass_rows][hkv][d]), then
 * to its n_path ancestors path[r][0 .. n_path) in the decode cache (k_dec,
 * v_dec [t_cap * rows][hkv][d]), then to itself at decode row
 * n_path * rows + r.  o [rows][hq][d] bf16.  Scores, softmax and P.V in f32.
 * ranges [n_slots][16][2] and n_ranges [n_slots] are device copies of
 * spb_plan_slot's; row indices are clamped into the caches. */
typedef struct {
  const void *q;
  const void *k_pass, *v_pass;
  int32_t n_pass_rows;
  const void *k_dec, *v_dec;
  void *o;
  int32_t rows, beams, hq, hkv, head_dim;
  const int32_t *ranges, *n_ranges;
  const int32_t *path;
  int32_t t_cap, n_path;
  float softmax_scale;
} spb_decode_attn_args;
spb_status spb_decode_attention(const spb_decode_attn_args *args, void *stream);

/* One beam-search step for n_slots slots of `beams` beams (<= 16).  step 0:
 * ids / lp [n_slots][k] are the candidates after each slot's template row;
 * step >= 1: [n_slots * beams][k] after each beam's fed row.  State, device
 * arrays per beam (slot-major): tok [t_cap] (decoded tokens, -1 past len),
 * len, fin (1: finished), score (sum of lp), path [t_cap] (decode-cache rows
 * of the fed tokens), and per slot nb (live beam count); *_in is read (not at
 * step 0), *_out written.  feed[r]: the token row r feeds at the next step
 * (the stop token for a finished beam). */
typedef struct {
  int32_t n_slots, beams, k, t_cap, step;
  const int32_t *stop;
  const int32_t *ids;
  const float *lp;
  const int32_t *tok_in, *len_in, *fin_in, *path_in, *nb_in;
  const float *score_in;
  int32_t *tok_out, *len_out, *fin_out, *path_out, *nb_out;
  float *score_out;
  int32_t *feed;
} spb_beam_args;
spb_status spb_beam_step(const spb_beam_args *args, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* SPB_H */
