/*
 * kvfix.h — C ABI of the cross-context KV-cache correction library for
 * AMD Instinct MI355X (gfx950).
 *
 * The library corrects a reused KV cache of a shared segment so that it can
 * stand in for a fresh prefill under a new prefix.  Its calls are the steps of
 * that correction and of the block-sparse storage of sibling caches:
 *
 *   kvfix_rope_shift   rotary re-alignment of cached keys to new positions
 *   kvfix_score        fresh-vs-reused L2 divergence per token at a check layer
 *   kvfix_score_draft  attention mass that draft query rows pay each token
 *   kvfix_select_topb  exactly b tokens with the largest score (probe set)
 *   kvfix_chunk_budget / kvfix_chunk_means / kvfix_expand_chunks
 *                      probe sets of whole fixed-size chunks (BCR-chunk, coin)
 *   kvfix_select_grow  probe sets of spans grown around the best rows (BCR-grow)
 *   kvfix_fit_mean     per-layer mean residual over the probe set (+ fresh scatter)
 *   kvfix_apply        fused re-align + weighted mean + rank-r correction
 *   kvfix_*_ex         the same with per-head probe sets and a covered prefix
 *   kvfix_diff_encode  block-sparse diff of N sibling caches against a master
 *   kvfix_diff_decode  fused restore: master + diff blocks + rotation, per sibling
 *   kvfix_select_master  the group's master: lowest total deviation
 *   kvfix_anchor_match / kvfix_anchor_apply
 *                      anchor-pool token weights, reliability gate, and the
 *                      blended low-rank correction
 *
 * Sources (page titles; sections named, not quoted):
 *   [KVCMAS] "KVCMAS: Efficient KV cache Correction for Shared Context in
 *            Multi-Agent Systems" (arXiv 2609.34060)
 *   [AKS]    "AgentKVShift: Correcting Reused KV" (review page)
 *   [TD]     "TokenDance: Scaling Multi-Agent LLM Serving via Collective KV
 *            Cache Sharing" (summary page)
 *   [BCR]    "Budgeted Cache Repair for Cross-Context KV-Cache Reuse"
 *            (arXiv 2610.02233)
 *
 * Conventions shared by every call
 *   - Every tensor pointer is a CALLER-OWNED DEVICE pointer (memory from
 *     hipMalloc or a framework allocator on the current device).  The library
 *     never allocates device memory; temporary space comes from a caller
 *     workspace whose size a *_workspace_size() call returns.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  No call synchronises.  Host-side argument checks run before
 *     any launch; on failure nothing is launched and a status is returned.
 *   - Results are bitwise identical from run to run (no floating-point
 *     atomics; every reduction has a fixed order).
 *   - Layout: a plane is one K or V cache, [layer][segment][kv_head][token]
 *     [head_dim] with free element strides (head_dim contiguous), or a paged
 *     pool [layer][page][page_size][kv_head][head_dim] addressed through a
 *     per-segment page table.
 *   - Alignment: data pointers and every row must be 16-byte aligned (the
 *     kernels move 128-bit vectors); otherwise KVFIX_ERR_ALIGN.
 *   - Arithmetic: fp32 storage is computed in fp64.  For bf16 storage:
 *     kvfix_apply, kvfix_diff_decode and the anchor calls compute in fp32;
 *     kvfix_rope_shift, kvfix_score, kvfix_fit_mean and kvfix_diff_encode's
 *     compare compute in fp64.  Each output element is rounded once (round
 *     to nearest even).
 */
#ifndef KVFIX_H
#define KVFIX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVFIX_OK = 0,
  KVFIX_ERR_ARG = 1,          /* null pointer, size or index out of range, shape mismatch */
  KVFIX_ERR_ALIGN = 2,        /* pointer or row stride not 16-byte aligned */
  KVFIX_ERR_CAPACITY = 3,     /* diff encode listed more blocks than the diff can hold, or a
                                 call needs more than a fixed library buffer holds */
  KVFIX_ERR_HIP = 4,          /* a HIP runtime or launch error */
  KVFIX_ERR_UNSUPPORTED = 5   /* dtype / head_dim / rank outside the compiled set */
} kvfix_status;

typedef enum { KVFIX_F32 = 0, KVFIX_BF16 = 1 } kvfix_dtype;

/* Rotary pairing.  HALF pairs dims (i, i + hd/2) (Llama / Qwen checkpoints);
 * INTERLEAVED pairs (2i, 2i + 1).  Pair i has frequency theta^(-2i/hd). */
typedef enum { KVFIX_ROPE_HALF = 0, KVFIX_ROPE_INTERLEAVED = 1 } kvfix_rope_style;

/* One K or V plane.
 *   contiguous (page_table == NULL):
 *     row (l, s, h, j) starts at  data + l*s_layer + s*s_seg + h*s_head + j*s_token
 *   paged (page_table != NULL):
 *     row (l, s, h, j) starts at  data + l*s_layer + page*s_page + (j % page_size)*s_token
 *                                      + h*s_head,  page = page_table[s*pages_per_seg + j/page_size]
 *   Strides count elements of `dtype`.  A row holds head_dim contiguous elements.
 *   Rows whose page id is outside [0, n_pool_pages) are skipped (neither read
 *   nor written): a bad id cannot make a kernel touch memory outside the pool.
 *   s_seg may be 0 (every segment reads the same data: a broadcast source). */
typedef struct {
  void*          data;
  int32_t        dtype;          /* kvfix_dtype */
  int32_t        n_layers;
  int32_t        n_segs;
  int32_t        n_heads;        /* KV heads */
  int32_t        n_tokens;       /* tokens per segment */
  int32_t        head_dim;       /* 64, 128 or 256 */
  int64_t        s_layer, s_seg, s_head, s_token;
  const int32_t* page_table;     /* device int32 [n_segs][pages_per_seg], or NULL */
  int32_t        page_size;
  int32_t        pages_per_seg;
  int64_t        s_page;
  int64_t        n_pool_pages;
} kvfix_plane;

/* Rotary shift: segment s is rotated forward by delta[s] positions, i.e. pair
 * i turns by delta[s] * theta^(-2i/hd) radians.  Angles are formed in fp64
 * and their sine/cosine taken by the library's own routines (within about one
 * unit of 2^-53 of the exact values; the fp32 tables of bf16 applies within
 * about one unit of 2^-24).  Limit: |delta[s]| < 2^23 positions, below which
 * the reduction of the angle by pi/2 is exact; larger shifts are not
 * detected (delta is device data) and lose accuracy.  [KVCMAS §2.2, App. A.3
 * "Correction Weighting and Positional Alignment"; TD Algorithm 1, RoPERecover] */
typedef struct {
  double         theta;
  int32_t        style;          /* kvfix_rope_style */
  const int64_t* delta;          /* device int64 [n_segs] */
} kvfix_rope;

/* Rank-r residual state Z = A B per (layer, segment, head).  [KVCMAS eq. 7-8]
 *   A: fp32, element (l, s, h, j, k) at  A + l*sA_layer + s*sA_seg + h*sA_head + j*rank + k
 *   B: fp32, element (l, s, h, k, d) at  B + l*sB_layer + s*sB_seg + h*sB_head + k*head_dim + d
 *   j is the token index within the segment; sA_head (or any A stride) may be
 *   0 to share A.  rank 0 means no state. */
typedef struct {
  const float* A;
  const float* B;
  int32_t      rank;             /* 0..8 */
  int64_t      sA_layer, sA_seg, sA_head;
  int64_t      sB_layer, sB_seg, sB_head;
} kvfix_lowrank;

/* ---------------------------------------------------------------------------
 * a1. Rotary re-alignment.  dst(l, s, h, j) = R(delta[s]) src(l, s, h, j).
 * [KVCMAS §2.2: every method re-aligns cached keys to their target positions
 * before reuse; TD §4.2: one batched rotary call for the whole group]
 * src and dst have the same shape and dtype; dst may alias src exactly
 * (in place).  Only keys are rotated; values need no call.
 * Arithmetic: fp64, one rounding per element.
 * ------------------------------------------------------------------------- */
kvfix_status kvfix_rope_shift(const kvfix_plane* src, const kvfix_plane* dst,
                              const kvfix_rope* rope, void* stream);

/* ---------------------------------------------------------------------------
 * a2. L2 divergence score at a check layer.
 *   scores[s][j] = || fresh(fresh_layer, s, :, j, :) - align(reuse(reuse_layer, s, :, j, :)) ||_2
 * taken over all heads and dims of token j.  rope == NULL scores a value plane
 * (no rotation).  [AKS "Core idea and method", step 1 and the equation for d;
 * TD §4.2, one batched difference pass at the check layer]
 * fresh and reuse must agree in n_segs, n_heads, n_tokens, head_dim and dtype.
 * scores: device fp32 [n_segs][n_tokens], written in full.
 * Arithmetic: fp64 accumulation, rounded once to fp32.
 * ------------------------------------------------------------------------- */
kvfix_status kvfix_score(const kvfix_plane* fresh, int32_t fresh_layer,
                         const kvfix_plane* reuse, int32_t reuse_layer,
                         const kvfix_rope* rope, float* scores, void* stream);

/* ---------------------------------------------------------------------------
 * a3. Draft attention-mass score.
 *   scores[s][j] = sum_{l >= first_layer} sum_t sum_h softmax_j( q'(s,l,h,t) . k(l,s,g(h),j) )
 *   q' = R(-delta[s]) q / sqrt(head_dim),   g(h) = h / (n_q_heads / n_heads)
 * i.e. the attention the draft query rows pay each re-aligned key
 * (q . R(delta) k = R(-delta) q . k, so keys are scored without rotating them).
 * [BCR §3 "The repair" (the score a_j), App. B Algorithm 2 and "The policy",
 * step 2 (grouped-query keys expanded to the query heads)]
 * q: device bf16 [n_segs][n_layers][n_q_heads][n_draft][head_dim], contiguous.
 * k: bf16 plane; n_q_heads must be a multiple of k->n_heads; n_q_heads/n_heads
 *    * n_draft <= 16.  head_dim 128 only.
 * scores: device fp32 [n_segs][n_tokens].
 * ws: device workspace of kvfix_score_draft_workspace(...) bytes, 256-byte aligned.
 * Arithmetic: bf16 MFMA on a 3-term bf16 split of q' (fp32-accurate logits),
 * fp32 exp, fp64 mass accumulation, rounded once to fp32.
 * ------------------------------------------------------------------------- */
size_t kvfix_score_draft_workspace(int32_t n_segs, int32_t n_layers, int32_t first_layer,
                                   int32_t n_q_heads, int32_t n_draft, int32_t n_tokens);
kvfix_status kvfix_score_draft(const void* q, int32_t n_q_heads, int32_t n_draft,
                               const kvfix_plane* k, int32_t first_layer, const kvfix_rope* rope,
                               float* scores, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * a4. Top-b selection.  For each of n_rows rows of n scores, exactly b indices
 * with the largest score; equal scores go to the lower index; -0 equals +0;
 * NaN ranks below every number.  [AKS step 2, b = ceil(r n); BCR-single]
 * scores: device fp32 [n_rows][n].  idx: device int32 [n_rows][b], ascending.
 * mask: device uint32 [n_rows][ceil(n/32)], bit j%32 of word j/32 set iff j
 * is selected (all words written).  0 <= b <= n.
 * ------------------------------------------------------------------------- */
kvfix_status kvfix_select_topb(const float* scores, int32_t n_rows, int32_t n, int32_t b,
                               int32_t* idx, uint32_t* mask, void* stream);

/* ---------------------------------------------------------------------------
 * BCR layouts of the probe budget.  [BCR §3 "The layouts" and "The repair";
 * §4.3; App. A.2 "The policy", "The random control" and Table 8; App. B
 * Algorithm 1]
 *
 * Whole chunks (BCR-chunk): chunk i of a row of n scores holds tokens
 * [i*chunk, min((i+1)*chunk, n)) and scores the mean of its tokens' scores.
 * The layout is: kvfix_chunk_means, then kvfix_select_topb over the means with
 * c = kvfix_chunk_budget(...) chunks, then kvfix_expand_chunks to token
 * indices and the token mask, which kvfix_fit_mean and kvfix_apply take.  The
 * coin control draws the chunks at random at the same budget: the same chain
 * with kvfix_select_topb run over caller-drawn uniform random keys, one per
 * chunk, instead of the means.
 * ------------------------------------------------------------------------- */
typedef enum {
  KVFIX_BUDGET_SKIP = 0,          /* 0 when M < 2 chunk or rho M < chunk, else round(rho M / chunk) */
  KVFIX_BUDGET_AT_LEAST_ONE = 1   /* max(1, round(rho * ceil(M / chunk))) */
} kvfix_budget_rule;

/* Number of chunks to repair among M = n_tokens cached tokens at budget
 * rho = rho_num / rho_den (exact; a half rounds up), never more than
 * ceil(M / chunk).  KVFIX_BUDGET_SKIP is BCR's Algorithm 1 (serve unrepaired
 * when the segment is shorter than two chunks or the budget is less than one
 * chunk); KVFIX_BUDGET_AT_LEAST_ONE is BCR's Table 8 rule.  Host-only (no
 * device work).  Returns -1 for chunk < 1, n_tokens outside [0, 2^31],
 * rho_den outside [1, 2^30], rho_num outside [0, rho_den] or another rule. */
int64_t kvfix_chunk_budget(int64_t n_tokens, int32_t chunk, int64_t rho_num, int64_t rho_den,
                           int32_t rule);

/* means[r][i] = mean of scores[r][j] over the tokens j of chunk i, summed in
 * fp64 in token order, divided by the chunk's own length (the last chunk may
 * be short) and rounded once to fp32.
 * scores: device fp32 [n_rows][n].  means: device fp32 [n_rows][ceil(n/chunk)]. */
kvfix_status kvfix_chunk_means(const float* scores, int32_t n_rows, int32_t n, int32_t chunk,
                               float* means, void* stream);

/* The tokens of c listed chunks per row.  chunk_idx: device int32 [n_rows][c]
 * (kvfix_select_topb's output: ascending); an id outside [0, ceil(n/chunk))
 * lists no tokens.  idx: device int32 [n_rows][c*chunk]: the listed chunks'
 * tokens in list order (ascending for an ascending list), then -1 padding
 * for the tokens a short last chunk does not have (kvfix_fit_mean reads -1
 * as padding).  counts: device int32 [n_rows], the tokens listed.  mask:
 * device uint32 [n_rows][ceil(n/32)], all words written.  c * chunk < 2^31. */
kvfix_status kvfix_expand_chunks(const int32_t* chunk_idx, int32_t n_rows, int32_t c, int32_t n,
                                 int32_t chunk, int32_t* idx, int32_t* counts, uint32_t* mask,
                                 void* stream);

/* Grown spans (BCR-grow): exactly b tokens per row.  While fewer than b are
 * chosen, the seed is the best-scoring token not yet chosen (equal scores:
 * the lower index; -0 equals +0; NaN ranks lowest); it is chosen, and its
 * span widens one token at a time to the higher-scoring of the two tokens
 * just outside it (the left one on a tie), while that token is not chosen
 * yet, scores at least tau times the seed (compared in fp64) and the budget
 * lasts.  tau > 1 with positive scores gives kvfix_select_topb's set.
 * scores: device fp32 [n_rows][n].  idx: device int32 [n_rows][b],
 * ascending.  mask: as kvfix_select_topb.  0 <= b <= n; tau not NaN.
 * KVFIX_ERR_UNSUPPORTED when the seed sort (8 bytes per seed, b rounded up
 * to a power of two), the seeds (4 bytes each) and the chosen-token bitmap
 * (n/8 bytes) exceed one block's LDS (with 160 KiB: b <= 8192 for n up to
 * about 500 000).  The scores are staged in LDS as well when they fit. */
kvfix_status kvfix_select_grow(const float* scores, int32_t n_rows, int32_t n, int32_t b,
                               double tau, int32_t* idx, uint32_t* mask, void* stream);

/* ---------------------------------------------------------------------------
 * a5. Probe mean residual, re-estimated per layer, and fresh scatter.
 *   mu[l][s][h][:] = (1/m) sum_{k : j in [0, n)} ( fresh_k - align(reuse_j) - A_j B ),
 *   j = idx[s][k],  m = the number of k < b with j in [0, n_tokens)
 * An index outside [0, n_tokens) is padding, not a probe: a layout whose
 * row count depends on the data (whole chunks, the last one short) pads its
 * fixed-width list with -1.  m == 0 (b == 0, or padding only) gives mu = 0.
 * fresh_k is fresh row j (fresh_by_slot == 0) or fresh row k (fresh_by_slot
 * == 1: fresh holds the probe rows by slot, in idx order).  If out != NULL
 * the fresh rows are also copied into out at the probe positions (exact
 * copy).  [AKS step 3 and the equation for mu-hat (the mean over the probe
 * set); KVCMAS eq. 7]
 * mu: device fp32 [n_layers][n_segs][n_heads][head_dim], contiguous.
 * idx: device int32 [n_segs][b]; b >= 0 is the list width and may exceed
 * n_tokens (device data is not checked on the host).
 * out may alias reuse (in-place correction).  When it does, the members of
 * each list must be distinct (a repeated index could read the fresh row
 * that an earlier member already scattered over the reused one, which
 * changes mu); kvfix_select_topb and kvfix_select_grow lists are distinct,
 * and so is a kvfix_expand_chunks list whose chunk ids are.  Out of place,
 * a repeated index is a repeated member and counts once per occurrence
 * (with fresh_by_slot, which occurrence's fresh row lands in out is
 * unspecified).
 * ws: device workspace of kvfix_fit_mean_workspace(...) bytes, 16-byte
 * aligned (fp64 partial sums of 256-probe slices); KVFIX_ERR_ARG when it is
 * missing, short or misaligned.
 * Arithmetic: fp64 residuals and sums in a fixed order, rounded once to fp32.
 * ------------------------------------------------------------------------- */
size_t kvfix_fit_mean_workspace(int32_t n_layers, int32_t n_segs, int32_t n_heads,
                                int32_t head_dim, int32_t b);
kvfix_status kvfix_fit_mean(const kvfix_plane* fresh, int32_t fresh_by_slot,
                            const kvfix_plane* reuse, const kvfix_plane* out,
                            const int32_t* idx, int32_t b, const kvfix_rope* rope,
                            const kvfix_lowrank* lowrank, float* mu, void* ws, size_t ws_bytes,
                            void* stream);

/* kvfix_fit_mean without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The slice partials live in a fixed
 * library array of KVFIX_NOALLOC_SCRATCH_BYTES per device, held by every GPU
 * the library runs on until the process ends; the call allocates nothing
 * (no hipMalloc / hipFree).  Same arguments, results and checks as
 * kvfix_fit_mean; KVFIX_ERR_CAPACITY when kvfix_fit_mean_workspace(...)
 * exceeds the array (64 MiB: at head_dim 128, b <= 512 for 80 layers x 32
 * segments x 8 heads, b <= 61 184 for 32 layers x 8 heads).  Calls
 * share their device's array: two calls that overlap on one device (other
 * streams, other threads) race and give undefined means.  The array's
 * address is looked up on a device's first call (KVFIX_ERR_HIP if that
 * fails). */
#define KVFIX_NOALLOC_SCRATCH_BYTES (64u << 20)
kvfix_status kvfix_fit_mean_noalloc(const kvfix_plane* fresh, int32_t fresh_by_slot,
                                    const kvfix_plane* reuse, const kvfix_plane* out,
                                    const int32_t* idx, int32_t b, const kvfix_rope* rope,
                                    const kvfix_lowrank* lowrank, float* mu, void* stream);

/* ---------------------------------------------------------------------------
 * a6. Fused apply.  For every token j whose mask bit is clear:
 *   out_j = round( align(reuse_j) + w_j mu + A_j B ),   w_j = clamp(scores[s][j], w_lo, w_hi)
 * (w = 1 when scores == NULL).  Rows whose mask bit is set are not touched.
 * [AKS equation for the corrected key: probes keep their fresh rows, others
 * get reuse + w mu-hat; KVCMAS eq. 3 (selective recompute) and eq. 4 / eq. 8
 * (add the estimated deviation to the aligned source cache)]
 * mask: device uint32 [n_segs][ceil(n_tokens/32)] or NULL (no probes).
 * mu: device fp32 [n_layers][n_segs][n_heads][head_dim], contiguous, 16-byte
 * aligned (KVFIX_ERR_ALIGN otherwise).
 * lowrank: A rows may use any 4-byte-aligned strides (16-byte-aligned rows
 * of rank 4 or 8 are read as vectors); rank <= 8.
 * out may alias reuse exactly (in place; each row is read and written by the
 * same lanes).  rope == NULL for value planes.
 * Arithmetic: fp32 for bf16 planes, fp64 for fp32 planes; one rounding.
 * ------------------------------------------------------------------------- */
kvfix_status kvfix_apply(const kvfix_plane* reuse, const kvfix_plane* out,
                         const uint32_t* mask, const float* scores, float w_lo, float w_hi,
                         const float* mu, const kvfix_lowrank* lowrank,
                         const kvfix_rope* rope, void* stream);

/* ---------------------------------------------------------------------------
 * Master selection.  [TD §4.2 "reuse plan output": the reuse path accumulates
 * a deviation score per request, and the master of a group is the request
 * closest to the group's shared structure, usually the one with the lowest
 * total deviation from the shared blocks]
 * totals[a] = sum over j of scores[a][j] in fp64, added in a fixed order:
 * each 64-token block in token order, then the block sums in block order
 * (deterministic; within (63 + ceil(n/64)) 2^-53 sum_j |scores[a][j]| of the
 * exact sum); *master = the a with the lowest total, ties to the lower index
 * (a NaN total ranks last).  The scores are per-token deviation scores, e.g.
 * kvfix_score of each request's cache against the shared blocks at the
 * check layer.  scores: device fp32 [n_agents][n]; totals: device fp64
 * [n_agents]; master: device int32 [1].  n_agents >= 1.
 * ------------------------------------------------------------------------- */
kvfix_status kvfix_select_master(const float* scores, int32_t n_agents, int32_t n,
                                 double* totals, int32_t* master, void* stream);

/* ---------------------------------------------------------------------------
 * Probe granularity and covered prefix.  [AKS "Core idea and method": the
 * construction is for one layer and one attention head; KVCMAS App. A.3
 * "Variable Segment Lengths": when the correction state covers only a prefix
 * of a segment, that prefix is corrected and the rest keeps the re-aligned
 * source cache]
 *
 * The _ex calls take these options; the calls above are the _ex calls with
 * opt == NULL (one probe set per segment, every row covered).
 * ------------------------------------------------------------------------- */
typedef struct {
  /* 0: one score row, probe list and mask per segment, shared by its heads
   *    (scores [n_segs][n], idx [n_segs][b], mask [n_segs][ceil(n/32)]);
   * 1: one per (segment, head): scores [n_segs][n_heads][n], idx
   *    [n_segs][n_heads][b], mask [n_segs][n_heads][ceil(n/32)], and the
   *    score of a token is taken over its head's head_dim elements only. */
  int32_t per_head;
  /* NULL, or device int32 [n_segs]: segment s is covered by the correction
   * state for tokens j < cover[s] only.  kvfix_apply_ex writes
   * round(align(reuse_j)) for non-probe tokens j >= cover[s] (no weighted
   * mean, no rank term); kvfix_fit_mean_ex takes A_j = 0 for probes
   * j >= cover[s].  Values outside [0, n_tokens] act as the nearest end. */
  const int32_t* cover;
} kvfix_granularity;

kvfix_status kvfix_score_ex(const kvfix_plane* fresh, int32_t fresh_layer,
                            const kvfix_plane* reuse, int32_t reuse_layer,
                            const kvfix_rope* rope, const kvfix_granularity* opt, float* scores,
                            void* stream);
kvfix_status kvfix_fit_mean_ex(const kvfix_plane* fresh, int32_t fresh_by_slot,
                               const kvfix_plane* reuse, const kvfix_plane* out,
                               const int32_t* idx, int32_t b, const kvfix_rope* rope,
                               const kvfix_lowrank* lowrank, const kvfix_granularity* opt,
                               float* mu, void* ws, size_t ws_bytes, void* stream);
kvfix_status kvfix_apply_ex(const kvfix_plane* reuse, const kvfix_plane* out,
                            const uint32_t* mask, const float* scores, float w_lo, float w_hi,
                            const float* mu, const kvfix_lowrank* lowrank,
                            const kvfix_rope* rope, const kvfix_granularity* opt, void* stream);

/* ---------------------------------------------------------------------------
 * a8 / a9. Master-mirror block-sparse diff.  [TD §4.3 master-mirror layout and
 * block-sparse diff representation; §5, one index list shared by K and V;
 * §4.4 and Algorithm 1, fused diff restore]
 *
 * A block is (agent a, layer l, token block beta) = tokens
 * [beta*block_tokens, min(n, (beta+1)*block_tokens)) of every head.
 *   mask      device uint32 [n_agents][n_layers][ceil(n_blocks/32)]
 *   offsets   device int64  [n_agents*n_layers + 1]: exclusive prefix count of
 *             listed blocks in (agent, layer) order; offsets[last] = total
 *   block_idx device int32  [capacity_blocks]: beta of each packed slot
 *   vals_k/v  device, plane dtype, [capacity_blocks][n_heads][block_tokens][head_dim]
 *             (rows past a ragged last block are left unwritten)
 * Packed slots are in (agent, layer, beta)-ascending order.
 * ------------------------------------------------------------------------- */
typedef struct {
  uint32_t* mask;
  int64_t*  offsets;
  int32_t*  block_idx;
  void*     vals_k;
  void*     vals_v;
  int64_t   capacity_blocks;
  int32_t   block_tokens;        /* 1..64 */
} kvfix_diff;

/* Encode: sibling a's keys are re-aligned into the master frame by
 * to_master->delta[a] positions (fp64); a block is listed when any element of
 * K or V differs from the master by more than eps (|x - m| > eps).  The listed
 * blocks' re-aligned K (rounded once) and raw V are packed.
 * master_k/v: planes with n_segs == 1; sib_k/v: planes with n_segs = n_agents.
 * dev_status: device int32, set to KVFIX_OK or KVFIX_ERR_CAPACITY (more listed
 * blocks than capacity_blocks: no slot past the capacity is written; the
 * packed values are then incomplete, mask and offsets are still exact).
 * ws: device workspace of kvfix_diff_encode_workspace(...) bytes. */
size_t kvfix_diff_encode_workspace(int32_t n_agents, int32_t n_layers, int32_t n_tokens,
                                   int32_t block_tokens);
kvfix_status kvfix_diff_encode(const kvfix_plane* master_k, const kvfix_plane* master_v,
                               const kvfix_plane* sib_k, const kvfix_plane* sib_v,
                               const kvfix_rope* to_master, float eps, const kvfix_diff* out,
                               int32_t* dev_status, void* ws, size_t ws_bytes, void* stream);

/* Decode: for every agent a, out(l, a) = master(l) with the listed blocks of
 * (a, l) overwritten by their packed values, keys then rotated forward by
 * from_master->delta[a] positions (fp32 for bf16 planes, fp64 for fp32
 * planes; sine and cosine from fp64; one rounding); values copied.  No
 * dense mirror is materialised: each master block is read from HBM once per
 * group of 16 agents and written to each of them.  out_k/out_v: planes with
 * n_segs = n_agents.
 * A listed block whose slot lies at or past capacity_blocks (an encode that
 * reported KVFIX_ERR_CAPACITY) is restored from the master instead.
 * ws: device workspace of kvfix_diff_decode_workspace(...) bytes (the
 * per-agent rotary table), 256-byte aligned. */
size_t kvfix_diff_decode_workspace(int32_t n_agents, int32_t head_dim);
kvfix_status kvfix_diff_decode(const kvfix_plane* master_k, const kvfix_plane* master_v,
                               const kvfix_diff* diff, const kvfix_rope* from_master,
                               const kvfix_plane* out_k, const kvfix_plane* out_v,
                               void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Anchor-blended low-rank correction and the reliability gate.
 * [KVCMAS eq. 7: an anchor stores rank-r factors A B (A: rows x r, B: r x D)
 *  of its base cache and of its delta correction; eq. 8: the correction is
 *  the weighted sum of the anchors' deltas; App. A.3 "Reliability Gate"
 *  eq. 9-11, "Correction Weighting and Positional Alignment", "Variable
 *  Segment Lengths"; eq. 4 / 6 / 12: the correction is added to the aligned
 *  source cache.]
 *
 * A pool holds the factors of V <= KVFIX_ANCHOR_MAX anchors of one shared
 * segment slot, in canonical (segment-relative) positions, rank
 * KVFIX_ANCHOR_RANK (a lower rank is passed zero-padded, which is exact):
 *   a   device bf16 [V][n_layers][2][n_max][r]   (plane 0 = K, 1 = V)
 *   bt  device bf16 [V][n_layers][2][n_heads*128][r]   B transposed: row
 *       h*128 + d holds column (h, d) of B
 *   lengths  HOST int32 [V]: tokens stored by each anchor, 0..n_max
 * The base factors (the anchors' source caches) feed kvfix_anchor_match,
 * the delta factors of the consuming agent feed kvfix_anchor_apply, with the
 * same lengths.  Both pointers 16-byte aligned (KVFIX_ERR_ALIGN otherwise).
 *
 * Eligible anchors E: those storing the whole n-token segment; if none does,
 * those storing the longest prefix, and the covered prefix is then that
 * length (else n).  The source segment is segment `seg` of bf16 planes with
 * head_dim 128 (KVFIX_ERR_UNSUPPORTED otherwise); its keys are cached at
 * positions src_off + j.  Offsets (and their differences) up to 2^23.
 * ------------------------------------------------------------------------- */
#define KVFIX_ANCHOR_MAX 16
#define KVFIX_ANCHOR_RANK 32

typedef struct {
  int32_t        n_anchors;      /* V, 0..KVFIX_ANCHOR_MAX */
  int32_t        rank;           /* must be KVFIX_ANCHOR_RANK */
  int64_t        n_max;
  const int32_t* lengths;        /* host */
  const void*    a;
  const void*    bt;
} kvfix_anchor_pool;

/* Match: token weights and the gate.
 * weights: device fp32 [n_layers][2][V][n].  For covered rows j and plane p,
 *   w[l][p][v][j] = softmax over v in E of -dist_v (T = 1), dist_v = the mean
 *   over all heads and dims of |source row - A_v[j] B_v| (keys first rotated
 *   by -src_off to canonical positions); 0 for v outside E and for rows past
 *   the covered prefix.
 * gate: device fp64 [V + 1].  The comparison prefix is the first k_gate
 *   tokens (clamped to [0, n]); A_k = anchors storing at least that many.
 *   gate[v] = d_v = sqrt(sum over layers, prefix rows, heads, dims of
 *   (value - A_v B_v)^2) for v in A_k, NaN otherwise; gate[V] = the
 *   normalized entropy of softmax(-d) over A_k, clamped to [0, 1] (NaN with
 *   fewer than two compared anchors).
 * accept: device int32, 1 iff |A_k| >= 2 and gate[V] <= tau (else dense
 *   prefill is due).
 * ws: device workspace of kvfix_anchor_match_workspace(...) bytes, 256-byte
 *   aligned: distance sums of both planes per group of heads (fp32
 *   [L][2][V][G][n], G = n_heads / 2 for an even head count, else n_heads)
 *   and the gate's fp64 partial sums (per layer, 128-token block, head group
 *   and anchor, then per layer, 256-token block and anchor).
 * Arithmetic: bf16 MFMA products; fp32 distance sums (per head; a group's
 * heads added in order, then the groups in order); gate squares summed in fp32 per head over 32-token
 * groups, those groups and all further totals in fp64. */
size_t kvfix_anchor_match_workspace(int32_t n_layers, int32_t n_heads, int32_t n_tokens,
                                    int32_t n_anchors);
kvfix_status kvfix_anchor_match(const kvfix_plane* src_k, const kvfix_plane* src_v, int32_t seg,
                                const kvfix_anchor_pool* base, int64_t src_off, double theta,
                                int32_t rope_style, int64_t k_gate, double tau, float* weights,
                                double* gate, int32_t* accept, void* ws, size_t ws_bytes,
                                void* stream);

/* Apply: the corrected target segment.  For covered rows j:
 *   delta_j = sum over v in E of weights[l][p][v][j] A_v[j] B_v (canonical),
 *   keys    out = R(tgt_off - src_off) x + R(tgt_off) delta_j
 *   values  out = x + delta_j
 * and past the covered prefix out = R(tgt_off - src_off) x (keys), x (values).
 * out_k/out_v: bf16 planes of the same shape (dense or paged), written at
 * segment `seg`; they may alias src_k/src_v exactly (in place: each row is
 * read and written by the same lanes).  weights: as produced by
 * kvfix_anchor_match (may be NULL when E is empty).
 * Arithmetic: bf16 MFMA products, fp32 blend and rotation, one rounding. */
kvfix_status kvfix_anchor_apply(const kvfix_plane* src_k, const kvfix_plane* src_v, int32_t seg,
                                const kvfix_anchor_pool* delta, const float* weights,
                                int64_t src_off, int64_t tgt_off, double theta, int32_t rope_style,
                                const kvfix_plane* out_k, const kvfix_plane* out_v, void* stream);

/* Human-readable name of a status code (static storage). */
const char* kvfix_status_string(kvfix_status status);

/* Library version, major*10000 + minor*100 + patch. */
int32_t kvfix_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVFIX_H */
