/*
 * sks.h -- C ABI of libsks, sparse-sketch long-context decode attention for
 * AMD Instinct MI355X (gfx950).
 *
 * One decode-attention step over one layer, as described on the page
 * "8 agents x 250K context, concurrently, on two 3090s" (claims list: every
 * decode step each attention layer reads ~1% of the tokens, picked with a tiny
 * rank-64 key sketch; "What it took": build the sketch, score every token,
 * pick the top ~2K and pack them for attention, CUDA-graph safe) and on the
 * "Agens SGLang" README ("What it adds": a 4,096-token sliding window plus a
 * 4:1 mean-pooled far field merged under one softmax; "Quick start": the
 * speculative-decoding verify step served as a chain).
 *
 * A step is:  sks_sketch_build (append the current tokens' key sketches)
 *             -> sks_sketch_build_query -> sks_sketch_score -> sks_topk_select
 *             -> sks_sparse_decode_attn (gathers the picked rows itself);
 *             sks_gather_pack materialises the same rows as a packed copy.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every tensor argument is a DEVICE pointer to caller-owned, contiguous,
 *   row-major memory; 16-byte alignment is required for K, V, S, Kp, Vp,
 *   K_out, V_out, out, scores and the workspace, 4-byte for the rest.
 * - The library allocates nothing, frees nothing and never synchronises: a
 *   call validates its host-visible arguments, enqueues kernels on `stream`
 *   (NULL = the null stream of the current device) and returns.  All calls
 *   can therefore be captured into a HIP graph.  Lengths are read on the
 *   device (`seq_len`), so one captured step serves every decode position.
 * - Errors: a call whose arguments are invalid returns SKS_ERR_ARG (or
 *   SKS_ERR_UNSUPPORTED / SKS_ERR_WORKSPACE) BEFORE launching anything, and
 *   sks_last_error() describes it.  SKS_ERR_HIP reports a failed launch; the
 *   outputs may then be partly written.
 * - Device lengths are clamped to [0, T_max - rows + 1] inside the kernels,
 *   so a bad length gives unspecified but memory-safe results.
 * - Results are bit-deterministic for identical inputs, whatever the batch
 *   composition and the number of verify rows: no floating-point atomics,
 *   attention split counts fixed by the per-row parameters (window, topk,
 *   pool, KV storage), fixed merge order.  A verify row gives the bits of a
 *   one-row step at its length.
 *
 * Geometry of query row i (0 <= i < rows) of sequence b, with r = pool:
 *   L_i   = seq_len[b] + i        tokens visible to the row (its own included;
 *                                  row i sits at position seq_len[b]-1+i)
 *   n_far = L_i > window ? (L_i - window) / r : 0       far tokens / r-blocks
 *   ws    = n_far * r              first token of the exact window
 *   k_eff = min(topk, n_far)
 *   The row attends to its k_eff selected far entries (pooled rows when r > 1)
 *   and to every token in [ws, L_i), under one softmax.  Query head h uses KV
 *   head h / (Hq / Hkv); the selection is per (sequence, row, KV head).
 */
#ifndef SKS_H
#define SKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *sks_stream_t; /* a hipStream_t */

enum sks_status {
  SKS_OK = 0,
  SKS_ERR_ARG = 1,          /* invalid argument; nothing was launched          */
  SKS_ERR_UNSUPPORTED = 2,  /* valid but not implemented (e.g. int8/int4 + pooling) */
  SKS_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required       */
  SKS_ERR_HIP = 4           /* a HIP launch failed                              */
};

enum sks_kv_dtype {
  SKS_KV_BF16 = 0,          /* K, V hold bfloat16                               */
  SKS_KV_I8 = 1,            /* K, V hold int8 codes; x = code * fp16 row scale  */
  SKS_KV_I4 = 2             /* K, V hold int4 codes, 64 bytes per row: byte j
                               has dim 2j in its low and dim 2j+1 in its high
                               nibble, two's complement in [-8, 7];
                               x = code * fp16 row scale (the int4 KV of the
                               claims list of "8 agents x 250K context ...")  */
};

#define SKS_HEAD_DIM 128
#define SKS_RANK 64
#define SKS_MAX_ROWS 8
#define SKS_MAX_POOL 64
#define SKS_APPEND (-1)     /* t_begin value: sketch the current rows' tokens  */
#define SKS_MAX_EXTENT (1 << 24) /* upper bound of window and topk               */

/* One layer's KV cache. */
typedef struct sks_kv {
  int32_t B;                /* sequences                                        */
  int32_t Hkv;              /* KV heads                                         */
  int32_t D;                /* head dim, must be 128                            */
  int32_t T_max;            /* cache capacity in tokens                         */
  int32_t dtype;            /* enum sks_kv_dtype                                */
  const void *K;            /* [B][Hkv][T_max][D] bf16 or int8, [..][D/2] int4   */
  const void *V;            /* [B][Hkv][T_max][D]                               */
  const uint16_t *K_scale;  /* [B][Hkv][T_max] fp16 bits, int8/int4, else NULL  */
  const uint16_t *V_scale;  /* [B][Hkv][T_max] fp16 bits, int8/int4, else NULL  */
  const int32_t *seq_len;   /* [B] device: L of query row 0 (own token included) */
  /* Hot tier (optional, all NULL / 0 without one).  "8 agents x 250K
   * context ...", claims list: the full KV cache lives in host RAM, the GPU
   * keeps the sketch and a small hot set, and only the picked tokens cross
   * PCIe.  With a hot tier, K, V (and their scales) may be pinned host memory
   * mapped into the device's address space (pass the device address, e.g.
   * from hipHostGetDevicePointer); they are then read only for the selected
   * far rows, for host-range key sketch builds and, in a dense step, for the
   * window positions older than the ring.  The exact window and the rows' own
   * tokens (APPEND) are read from the ring below, in which position p sits
   * in slot p % W_hot.  The caller keeps the ring current:
   * it must hold every position in [L_0 + rows - 1 - W_hot, L_0 + rows - 1).
   * Needs pool == 1 (SKS_ERR_UNSUPPORTED otherwise). */
  const void *K_hot;        /* [B][Hkv][W_hot][row] same format as K, or NULL   */
  const void *V_hot;        /* [B][Hkv][W_hot][row]                             */
  const uint16_t *K_hot_scale; /* [B][Hkv][W_hot] fp16 bits, int8/int4, else NULL */
  const uint16_t *V_hot_scale; /* [B][Hkv][W_hot]                               */
  int32_t W_hot;            /* ring slots, window + rows <= W_hot <= T_max      */
} sks_kv;

/* Selection parameters of the step. */
typedef struct sks_params {
  int32_t window;           /* exact sliding window, 0 <= W <= SKS_MAX_EXTENT   */
  int32_t topk;             /* far entries per (sequence, row, KV head),
                               1 <= k <= SKS_MAX_EXTENT (k >= n_far: all)      */
  int32_t pool;             /* far-field pooling ratio r, 1 <= r <= 64          */
  int32_t rank;             /* sketch rank, must be 64                          */
  int32_t rows;             /* query rows per sequence R, 1 <= R <= 8           */
} sks_params;

/* Number of sketch rows (tokens, or r-blocks) per (sequence, KV head):
 * NB = T_max / pool.  S, Kp, Vp and each scores row have NB entries. */

/* Text of the last error returned on this thread ("" if none). */
const char *sks_last_error(void);

/* HIP runtime version seen by the library (hipRuntimeGetVersion). */
int32_t sks_runtime_version(void);

/* Workspace bytes that sks_sketch_score, sks_topk_select and
 * sks_sparse_decode_attn need for this shape; one buffer serves the whole
 * step.  Returns 0 on invalid arguments.
 * The workspace starts with a region that must be ZERO AT REST (per-segment
 * selection histograms): sks_sketch_score (with a workspace) and the
 * selection add into it, and sks_topk_select returns it to zero.  Zero a new
 * workspace once with sks_workspace_init.  A workspace that is not zero at
 * rest costs time (the selection then falls back to a full pass over the
 * scores), never correctness.  The rest is scratch, clobbered by each call.
 * Calls that share one workspace must be ordered (same stream). */
size_t sks_workspace_bytes(const sks_kv *kv, const sks_params *p, int32_t Hq);

/* Zero-fill ws_bytes of a workspace on `stream` (a fill kernel, no memset
 * node, so it may be captured in a graph). */
int sks_workspace_init(void *ws, size_t ws_bytes, sks_stream_t stream);

/* Key sketch build.  "What it took" (build the sketch) and the claims list
 * (rank-64 key sketch) of "8 agents x 250K context ...", plus the frozen
 * sketch basis of the same list; pooling from "What it adds" of
 * "Agens SGLang".
 *
 * For every sequence b, KV head h and sketch row j:
 *   pool == 1: rows are tokens t in the position range;
 *              S[b][h][t][c] = clamp(rne((P_h . x_t)_c / key_scale[h]), +-127)
 *              with x_t the (dequantised) key; Kp, Vp must be NULL.
 *   pool  > 1: rows are blocks j whose LAST token r*j + r - 1 lies in the
 *              position range; Kp/Vp[b][h][j] = bf16(rne(mean of the block's
 *              r keys / values)) and S[b][h][j] is the sketch of Kp[b][h][j].
 *              bf16 caches only (SKS_ERR_UNSUPPORTED otherwise).
 * basis: [1][64][128] (basis_per_head == 0) or [Hkv][64][128] fp32, row c of
 *        P_h being the c-th basis vector.  key_scale: [Hkv] fp32, > 0.
 * Position range: [t_begin, t_end) clamped to [0, T_max) for every sequence,
 *   or, with t_begin == SKS_APPEND, the current rows' own tokens
 *   [seq_len[b] - 1, seq_len[b] - 1 + rows) read on the device (t_end ignored).
 * S: [B][Hkv][NB][64] int8.  Kp, Vp: [B][Hkv][NB][128] bf16 (pool > 1). */
int sks_sketch_build(const sks_kv *kv, const sks_params *p, const float *basis,
                     int32_t basis_per_head, const float *key_scale, int32_t t_begin,
                     int32_t t_end, int8_t *S, uint16_t *Kp, uint16_t *Vp,
                     sks_stream_t stream);

/* Query sketch.  Same passages as the key sketch; under grouped-query
 * attention the query side of KV head h is the mean qbar of its g = Hq/Hkv
 * query vectors:  y = P_h qbar,  qscale = max|y| / 127,
 *   qsk = clamp(rne(y / qscale), +-127)   (all zero and qscale 0 if y == 0).
 * q: [B][R][Hq][128] bf16.  qsk: [B][R][Hkv][64] int8.  qscale: [B][R][Hkv]
 * fp32 (may be NULL). */
int sks_sketch_build_query(const uint16_t *q, int32_t B, int32_t R, int32_t Hq, int32_t Hkv,
                           const float *basis, int32_t basis_per_head, int8_t *qsk,
                           float *qscale, sks_stream_t stream);

/* Score every far token ("What it took": score every token):
 *   scores[b][i][h][t] = sum_c qsk[b][i][h][c] * S[b][h][t][c]   (exact int32)
 * for t < n_far of the row with the most far entries; one pass over S serves
 * all rows.  Entries past that are not written.
 * scores: [B][R][Hkv][NB] int32.
 * ws (optional, may be NULL): a step workspace; when given, the call also
 * accumulates the selection's level-1 histogram into it, and the following
 * sks_topk_select on these scores is called with SKS_TOPK_HIST_READY. */
int sks_sketch_score(const int8_t *qsk, const int8_t *S, const sks_kv *kv,
                     const sks_params *p, int32_t *scores, void *ws, size_t ws_bytes,
                     sks_stream_t stream);

/* Top-k selection ("What it took": pick the top ~2K).  For every (b, i, h):
 * the k_eff far entries with the largest scores[b][i][h][0 .. n_far), the
 * lower index first among equal scores, written in ascending order to
 * idx[b][i][h][0 .. k_eff) and padded with -1 up to topk.
 * n_sel: [B][R][Hkv] int32 receives k_eff (may be NULL).
 * Caches of up to 8,388,608 sketch rows (T_max / pool): above that the call
 * returns SKS_ERR_UNSUPPORTED (so does sks_decode_step).
 * flags: 0, or SKS_TOPK_HIST_READY when sks_sketch_score produced these
 *        scores with this workspace (its histogram is then reused).
 * ws: at least sks_workspace_bytes(); its zero-at-rest region is returned to
 *     zero. */
#define SKS_TOPK_HIST_READY 1
int sks_topk_select(const int32_t *scores, const sks_kv *kv, const sks_params *p,
                    int32_t flags, int32_t *idx, int32_t *n_sel, void *ws, size_t ws_bytes,
                    sks_stream_t stream);

/* Candidate mode of the score pass and the selection: the same selection as
 * sks_sketch_score(ws) + sks_topk_select(SKS_TOPK_HIST_READY), bit for bit,
 * without storing the scores, so that the score pass streams only the
 * sketches.  sks_score_candidates
 *   1. (without SKS_CAND_KEEP_ESTIMATE) scores every 64th far entry of each
 *      (b, i, h) into a sample histogram in ws;
 *   2. derives from that histogram an estimate E of each (b, i, h)'s k-th
 *      largest biased score (score + 2^20), set low enough that with high
 *      probability at least k entries reach it (where a (b, i, h) has at most
 *      1,024 sampled entries, step 1 derives E at once and keeps E in ws
 *      instead of the histogram); scores every far token as sks_sketch_score
 *      does and keeps in ws, instead of the scores, every far entry whose
 *      biased score is at least E (index and biased score, ascending).
 * sks_topk_select_candidates then selects as sks_topk_select, from those
 * entries.  Where fewer than k entries reached E, it recomputes that
 * segment's scores from qsk and S into `scores` ([B][R][Hkv][NB] int32,
 * scratch: its contents afterwards are unspecified) and selects from them.
 * E only decides the time taken, never the result.
 * Flags of sks_score_candidates:
 *   SKS_CAND_KEEP_ESTIMATE  reuse the sample histograms (or estimates)
 *                           already in ws (step 2 only;
 *                           sks_topk_select_candidates returns histograms
 *                           to zero, after which E is 0);
 *   SKS_CAND_TEST_HIGH      (tests) E above every score: every segment with
 *                           k_eff < n_far takes the recomputing path;
 *   SKS_CAND_TEST_ZERO      (tests) E = 0: every far entry is kept.
 * ws: at least sks_workspace_bytes(); the two calls use the same ws, in this
 * order, with no other selection call on it in between. */
#define SKS_CAND_KEEP_ESTIMATE 1
#define SKS_CAND_TEST_HIGH 2
#define SKS_CAND_TEST_ZERO 4
int sks_score_candidates(const int8_t *qsk, const int8_t *S, const sks_kv *kv,
                         const sks_params *p, int32_t flags, void *ws, size_t ws_bytes,
                         sks_stream_t stream);
int sks_topk_select_candidates(const int8_t *qsk, const int8_t *S, const sks_kv *kv,
                               const sks_params *p, int32_t *scores, int32_t *idx,
                               int32_t *n_sel, void *ws, size_t ws_bytes,
                               sks_stream_t stream);

/* Gather/pack ("What it took": pack the picked tokens for the attention
 * kernel).  For every (b, i, h) writes the row's attention set, selected far
 * entries first (ascending, rows of Kp/Vp when pool > 1, else of K/V), then
 * the window tokens [ws, L_i) ascending, into
 *   K_out, V_out: [B][R][Hkv][C][row] with C = topk + window + pool - 1,
 * rows in the cache's own format (int8 and int4 caches also write the fp16
 * row scales to Ks_out, Vs_out [B][R][Hkv][C]; NULL for bf16), and the entry
 * count to
 * n_out [B][R][Hkv].  Slots past n_out are not written. */
int sks_gather_pack(const sks_kv *kv, const sks_params *p, const int32_t *idx,
                    const uint16_t *Kp, const uint16_t *Vp, void *K_out, void *V_out,
                    uint16_t *Ks_out, uint16_t *Vs_out, int32_t *n_out,
                    sks_stream_t stream);

/* Sparse decode attention, one merged softmax over the selected far entries
 * and the exact window ("What it adds" of "Agens SGLang"; "int8 attention"
 * of "What it took" for int8 and int4 caches, dequantised in registers).  For query
 * head hq of row i of sequence b, with U its row's attention set:
 *   z_j = sm_scale * (q . K_j),  out = sum_j softmax(z)_j V_j,
 *   lse = log sum_j exp(z_j)     (U empty: out = 0, lse = -inf).
 * The rows are gathered from K/V (and Kp/Vp for selected blocks when
 * pool > 1) by idx [B][R][Hkv][topk] as written by sks_topk_select.
 * q: [B][R][Hq][128] bf16.  out: [B][R][Hq][128] fp32.  lse: [B][R][Hq] fp32
 * (may be NULL).  ws: at least sks_workspace_bytes(). */
int sks_sparse_decode_attn(const uint16_t *q, int32_t Hq, const sks_kv *kv,
                           const sks_params *p, const int32_t *idx, const uint16_t *Kp,
                           const uint16_t *Vp, float sm_scale, float *out, float *lse,
                           void *ws, size_t ws_bytes, sks_stream_t stream);

/* One whole decode step of one layer in a single call: the work of
 *   sks_sketch_build(APPEND)      (with SKS_STEP_APPEND)
 *   sks_sketch_build_query
 *   sks_sketch_score(ws)
 *   sks_topk_select(SKS_TOPK_HIST_READY)
 *   sks_sparse_decode_attn
 * in that order, with the same results bit for bit (the pages' statement of
 * the work in "What it took": build the sketch, score every token, pick the
 * top ~2K, attend, all graph-safe).  Grouping the calls lets launches share
 * work that the order allows: the query sketch and the append run in one
 * launch.
 * With SKS_STEP_DENSE the step skips scoring and selection (the dense half of
 * the per-step dense/sparse switch of "What it took", so that short chats
 * stay at full speed): every row attends, under one softmax, to its last
 * window + topk tokens -- all of [0, L_i) when L_i <= window + topk, which is
 * exactly the set the sparse step attends for such rows when pool == 1.  The
 * attention entries are then in position order, so out and lse equal the
 * sparse step's up to rounding, not bit for bit.  scores, idx and n_sel are
 * left as they are (idx must still point at a buffer of its size); the
 * APPEND sketch rows are written as usual, so that later sparse steps find
 * the sketch current.  Which mode a step takes is the caller's choice (it
 * knows its lengths); the workspace of the sparse step serves both.
 * With SKS_STEP_NO_SCORES the caller does not read `scores` after the step:
 * where it pays (rows of more than 8,192 far entries, and either at most
 * 65,536 far entries per row, or one row per sequence and at least 2^20 far
 * entries over all (b, h)), the step scores and selects in candidate
 * mode (sks_score_candidates + sks_topk_select_candidates), which stores no
 * scores; idx, n_sel, out and lse are the same bit for bit, and `scores` is
 * then scratch with unspecified contents.
 * Every buffer is caller-owned and keeps the layout of the individual call
 * that writes or reads it; NULL is allowed where the individual call allows
 * it (qscale, n_sel, lse; Kp/Vp when pool == 1).  The same validation as the
 * individual calls happens before any launch. */
typedef struct sks_step {
  const uint16_t *q;        /* [B][R][Hq][128] bf16 queries of the rows         */
  int32_t Hq;               /* query heads: a multiple of Hkv, Hq / Hkv <= 8    */
  const float *basis;       /* [1 or Hkv][64][128] fp32 sketch basis            */
  int32_t basis_per_head;   /* 0: one basis for all KV heads, 1: one per head   */
  const float *key_scale;   /* [Hkv] frozen key-sketch scales                   */
  int8_t *S;                /* [B][Hkv][NB][64] key sketch (APPEND rows written) */
  uint16_t *Kp, *Vp;        /* [B][Hkv][NB][128] bf16 pooled rows (pool > 1)    */
  float sm_scale;           /* logit scale, > 0 (1/sqrt(128) for the pages)     */
  int8_t *qsk;              /* out: [B][R][Hkv][64] query sketch codes          */
  float *qscale;            /* out: [B][R][Hkv] query sketch scales, or NULL    */
  int32_t *scores;          /* out: [B][R][Hkv][NB] scores                      */
  int32_t *idx;             /* out: [B][R][Hkv][topk] selected entries          */
  int32_t *n_sel;           /* out: [B][R][Hkv] k_eff, or NULL                  */
  float *out;               /* out: [B][R][Hq][128] fp32 attention output       */
  float *lse;               /* out: [B][R][Hq] fp32 log-sum-exp, or NULL        */
} sks_step;
#define SKS_STEP_APPEND 1   /* sketch the rows' own tokens first */
#define SKS_STEP_DENSE 2    /* no selection: attend the last window + topk tokens */
#define SKS_STEP_NO_SCORES 4  /* scores are scratch: candidate mode where it pays */
int sks_decode_step(const sks_kv *kv, const sks_params *p, const sks_step *step, int32_t flags,
                    void *ws, size_t ws_bytes, sks_stream_t stream);

/* sks_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a static array of
 * SKS_STATIC_WORKSPACE_BYTES that the library holds on every GPU it runs on
 * until the process ends; the call itself allocates and frees nothing.
 * Same arguments, flags, validation and results (bit for bit) as
 * sks_decode_step; the caller still provides every input and output.
 * - A shape whose workspace (sks_workspace_bytes) exceeds the static array
 *   returns SKS_ERR_WORKSPACE before any launch (every workload shape of this
 *   library fits: 8 x 250,000 tokens with 24/4 heads needs about 67 MB).
 * - The array of a GPU is shared by every call on that GPU (the GPU of
 *   `stream`; the current device for the null stream) and keeps the last
 *   call's contents.  Calls that may overlap on one GPU -- on streams not
 *   ordered with each other, or from several host threads -- race on it and
 *   must not be issued.
 * - The first call on a GPU looks up that GPU's copy of the array
 *   (hipGetSymbolAddress; issue it once outside a graph capture if the
 *   capture must contain only the step).  The first call and every call whose
 *   shape differs from the previous call's on that GPU also clear the
 *   selection histograms with a fill kernel (a dirty region would cost time,
 *   never correctness). */
#define SKS_STATIC_WORKSPACE_BYTES (96u << 20)
int sks_decode_step_static(const sks_kv *kv, const sks_params *p, const sks_step *step,
                           int32_t flags, sks_stream_t stream);

/* ---------------------------------------------------------------- basis refit
 * "What it took" of "8 agents x 250K context ...": a frozen sketch basis in
 * one file plus the script that refits it.  A refit reads the captured keys
 * of every sequence b and KV head h at positions [t_begin, min(t_end,
 * seq_len[b])) of a bf16 cache (int8/int4 caches: SKS_ERR_UNSUPPORTED) and
 * computes, in three calls on one stream:
 *   G = sum of x x^T over the keys (fp64 [128][128], per KV head or over all),
 *   basis = the 64 eigenvectors of G with the largest eigenvalues, as rows in
 *           descending eigenvalue order, each signed so that its
 *           largest-magnitude component (the first one on ties) is positive,
 *   key_scale[h] = max over the keys of (b, h) of max_c |(P x)_c| / 127, so
 *           that no captured key's code clips (1 if every projection is 0).
 * The outputs can be handed to every other call as basis / key_scale.  Same
 * conventions as above: device pointers, nothing allocated, errors before any
 * launch.  The Gram matrix accumulates exact bf16 products in fp32 per
 * 8,192-key chunk and the chunks in fp64; the eigen-decomposition is cyclic
 * Jacobi in fp64.  Equal eigenvalues leave the order among them, and hence
 * the basis, to the solver. */

/* Workspace bytes for sks_refit_gram and sks_refit_key_scale on this key
 * range; it also covers sks_refit_basis for up to Hkv matrices.  0 on
 * invalid arguments. */
size_t sks_refit_workspace_bytes(const sks_kv *kv, int32_t t_begin, int32_t t_end);

/* gram: [per_head ? Hkv : 1][128][128] fp64, symmetric, 8-byte aligned. */
int sks_refit_gram(const sks_kv *kv, int32_t t_begin, int32_t t_end, int32_t per_head,
                   double *gram, void *ws, size_t ws_bytes, sks_stream_t stream);

/* From n Gram matrices [n][128][128] fp64: basis [n][64][128] fp32 and, if
 * eigval is not NULL, all eigenvalues [n][128] fp64 in descending order.
 * ws: at least n * 128 * 128 * 8 bytes (scratch). */
int sks_refit_basis(const double *gram, int32_t n, float *basis, double *eigval, void *ws,
                    size_t ws_bytes, sks_stream_t stream);

/* key_scale: [Hkv] fp32, from basis [1 or Hkv][64][128] (basis_per_head). */
int sks_refit_key_scale(const sks_kv *kv, int32_t t_begin, int32_t t_end, const float *basis,
                        int32_t basis_per_head, float *key_scale, void *ws, size_t ws_bytes,
                        sks_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SKS_H */
