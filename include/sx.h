/*
 * sx.h -- C ABI of libsx, the MI355X (gfx950) SparseX prefill-layer path.
 *
 * One SparseX prefill layer over a prompt assembled from reused KV segments
 * ("SparseX: Efficient Segment-Level KV Cache Sharing for Interleaved LLM
 * Serving", arXiv 2606.01751):
 *   1. RoPE re-alignment of each reused segment's cached keys     (§3.1)
 *   2. Sparse-Q attention-mass scoring and per-request top-k      (§3.2, §3.3)
 *   3. Sparse-KV recomputation: gather, QKV GEMM, RoPE, scatter    (§3.4)
 *   4. causal GQA attention of the active rows over the mixed
 *      paged cache; full causal prefill before the threshold      (§3.4, §4.5)
 * and around it the segment lookup that finds the reused blocks (§4.1-§4.5)
 * and decode attention over the mixed cache afterwards (§4.5).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers unless the parameter name ends in `_h`
 *   (host memory).  The caller owns every buffer; the library allocates and
 *   frees nothing and keeps no state between calls -- except the segment
 *   index (sx_index_*), a host object the caller creates and destroys, and
 *   the static scratch array of sx_decode_attn_noalloc.
 * - Every compute call enqueues its kernels on `stream` (a hipStream_t; NULL
 *   is the null stream) and returns without synchronising.  Results are
 *   valid in stream order.
 * - Scalars and host arrays are validated before anything is launched; on
 *   a bad argument the call returns a negative sx_status, launches nothing
 *   and sx_last_error() describes the problem.  Device-resident index data
 *   (request offsets, block tables, row lists, realign jobs) is not
 *   inspected on the host.  The kernels bound-check every index they
 *   dereference, so bad index data never makes them touch memory outside
 *   the buffers the call was given; instead: a page id outside [0, n_pages)
 *   reads page 0 and its writes are skipped; a realign job whose pages,
 *   slots, count or |delta| (>= rope_len) are out of range is skipped, its
 *   destination slots keeping their old contents; a RoPE position outside
 *   the table is clamped into it; a row that is not a token of the batch
 *   reads row 0 of x and writes nothing; a row outside its request or out
 *   of order is clamped to the request's keys.  The outputs that depend on
 *   a bad index are then unspecified.
 * - Debug mode: with the environment variable SX_DEBUG set (to anything but
 *   "0") every device entry point except sx_topk first runs device-side
 *   checks of the index data it will read -- request offsets (ascending,
 *   from 0 to n_tok), the block-table page ids of every request's tokens
 *   (in [0, n_pages), within max_pages columns), RoPE positions
 *   (sx_recompute_kv: in [0, rope_len)), row lists (tokens of the batch;
 *   where rows are grouped by request: ascending inside their request) and
 *   realign jobs (pages, slots, counts, |delta| < rope_len).  If any check
 *   fails the call returns SX_EDEVICE, sx_last_error() names what failed,
 *   and none of its compute kernels is launched.  Debug mode waits for the
 *   stream inside the call (it cannot be captured into a graph).
 * - Storage type: all of x, weights, Q, K/V pages and outputs of one call
 *   share `dims->dtype` (bf16 or fp32).  Accumulation is fp32.  Results
 *   are bitwise reproducible: reductions run in a fixed order, with no
 *   floating-point atomics.
 * - Packed token ids: the tokens of all requests of a batch are numbered
 *   0..n_tok-1, request r owning [seq_start[r], seq_start[r+1]).  Token t of
 *   request r has index i = t - seq_start[r] inside the request; its RoPE
 *   position is i + pos_offset[r] (pos_offset NULL means 0).
 * - Paged KV cache of one layer (the paper's PagedAttention blocks, §4.1):
 *     K pool: [n_pages][n_kv_heads][page_size][head_dim]
 *     V pool: [n_pages][n_kv_heads][head_dim][page_size]   (V transposed
 *             inside a page so attention reads 16 keys per head dimension
 *             contiguously)
 *   Token index i of request r lives in page block_table[r][i / page_size],
 *   slot i % page_size.  page_size is 16.
 * - RoPE (the rotation R_m of §3.1): rotate-half pairs (e, e + d/2) with
 *   omega_e = theta^(-2e/d).  `rope_tab` holds cos and sin of m*omega_e for
 *   m = 0..rope_len-1, built in double precision by sx_rope_table().
 */
#ifndef SX_H
#define SX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SX_OK = 0,
  SX_EINVAL = -1,        /* bad pointer, size or inconsistent argument      */
  SX_EUNSUPPORTED = -2,  /* valid but not implemented (e.g. head_dim 96)    */
  SX_EWORKSPACE = -3,    /* workspace missing or smaller than required      */
  SX_EDEVICE = -4,       /* a HIP call or kernel launch failed              */
  SX_ENOMEM = -5         /* the block pool cannot supply the blocks asked for */
} sx_status;

typedef enum { SX_F32 = 0, SX_BF16 = 1 } sx_dtype;

/* Model shape of one layer.  head_dim is 64 or 128 (fp32) or 128 (bf16);
 * n_q_heads is a multiple of n_kv_heads with n_q_heads / n_kv_heads <= 8;
 * page_size must be 16. */
typedef struct {
  int32_t hidden;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t dtype;         /* sx_dtype */
} sx_dims;

/* One layer's paged K and V pools (layouts above). */
typedef struct {
  void *k;
  void *v;
  int32_t n_pages;
} sx_pages;

/* Request layout of a batch: the paper's scheduler output (§4.5: request
 * layout, block table, slot mapping).  n_tok, n_req, max_pages and rope_len
 * are host values; the arrays are device arrays. */
typedef struct {
  int32_t n_req;
  int32_t n_tok;                 /* == seq_start[n_req]                    */
  int32_t max_pages;             /* columns of block_table                 */
  int32_t rope_len;              /* rows of rope_tab                       */
  const int32_t *seq_start;      /* [n_req + 1]                            */
  const int32_t *block_table;    /* [n_req][max_pages] physical page ids   */
  const int32_t *pos_offset;     /* [n_req] or NULL                        */
  const float *rope_tab;         /* [rope_len][head_dim / 2][2] cos, sin   */
} sx_layout;

/* One block-granular copy of the fused copy-Delta-RoPE step (§4.4, §4.5):
 * n_tok consecutive tokens from src page slots [src_slot, src_slot+n_tok)
 * to dst page slots [dst_slot, dst_slot+n_tok); keys rotated by R_delta,
 * values copied. */
typedef struct {
  int32_t src_page;
  int32_t dst_page;
  int32_t src_slot;
  int32_t dst_slot;
  int32_t n_tok;
  int32_t delta;
} sx_realign_job;

/* A reused run of a request, as the host scheduler knows it (§4.5). */
typedef struct {
  int32_t req;            /* destination request                              */
  int32_t dst_start;      /* token index of the run's first token in req      */
  int32_t len;            /* tokens                                           */
  int32_t p_src;          /* RoPE position the cached keys of token 0 carry   */
  int32_t src_slot0;      /* slot of token 0 in its first source page         */
  int32_t src_pages_off;  /* index of that page in the source page-id array   */
} sx_segment;

/* ----------------------------------------------------------------------- */
/* Host-side planning (pure host code, no GPU needed).                     */
/* ----------------------------------------------------------------------- */

/* RoPE table (§3.1, the rotation R_m): tab_h[m][e][0] = cos(m*omega_e),
 * tab_h[m][e][1] = sin(m*omega_e), omega_e = theta^(-2e/head_dim), formed in
 * double precision and rounded to float.  tab_h holds n_pos*head_dim
 * floats.  Returns SX_EINVAL for theta <= 0, odd or non-positive head_dim,
 * n_pos <= 0 or a NULL pointer. */
sx_status sx_rope_table(double theta, int32_t head_dim, int32_t n_pos, float *tab_h);

/* Token classes and selection budgets of a batch (§3.2: the index sets
 * I_reuse and I_nr, and the tail fallback; §3.3: overflow).
 *   Request r consists of pieces piece_start_h[r] .. piece_start_h[r+1]-1;
 *   piece p is piece_len_h[p] tokens, reused if piece_reuse_h[p] != 0.
 *   Empty pieces are ignored.  If a request's last token is reused, the last
 *   min(fallback_tokens, L) tokens of its final reused piece join I_nr.
 *   Overflow (off when overflow_tokens is 0; one block = 16 tokens in the
 *   paper's setting): for every run of new pieces, the last
 *   min(overflow_tokens, L) tokens of the reused piece right before it and
 *   the first min(overflow_tokens, L) tokens of the reused piece right after
 *   it join I_nr too (the Sparse-Q interval widened by one block per side).
 * Outputs (host, caller-allocated):
 *   seq_start_h [n_req+1]        packed token offsets
 *   tok_class_h [n_tok_cap]      0 = selection candidate (reused, not in
 *                                I_nr), 1 = Sparse-Q row (in I_nr)
 *   sq_rows_h   [n_tok_cap]      packed ids of I_nr, ascending
 *   sq_start_h  [n_req+1]        request r's I_nr rows are
 *                                sq_rows_h[sq_start_h[r] .. sq_start_h[r+1])
 *   n_cand_h    [n_req]          number of candidates R_r
 *   k_h         [n_req]          floor(ratio_num_h[r] * R_r / ratio_den_h[r])
 * The ratio is a fraction of the candidates in [0, 1].  Returns SX_EINVAL
 * for negative lengths, a ratio outside [0,1], a zero denominator, a
 * negative fallback_tokens or overflow_tokens, or a batch longer than
 * n_tok_cap tokens. */
sx_status sx_plan_layout(int32_t n_req, const int32_t *piece_start_h, const int32_t *piece_reuse_h,
                         const int32_t *piece_len_h, const int32_t *ratio_num_h,
                         const int32_t *ratio_den_h, int32_t fallback_tokens,
                         int32_t overflow_tokens, int32_t n_tok_cap, int32_t *seq_start_h,
                         uint8_t *tok_class_h, int32_t *sq_rows_h, int32_t *sq_start_h,
                         int32_t *n_cand_h, int32_t *k_h);

/* Split reused runs into page-granular realign jobs (§4.5: allocate fresh
 * blocks for hits, then copy-Delta-RoPE them).  Token j of run s comes from
 * source page src_page_ids_h[s.src_pages_off + (s.src_slot0 + j) / ps], slot
 * (s.src_slot0 + j) % ps, and goes to request s.req at token index
 * s.dst_start + j; delta = s.dst_start + pos_offset_h[s.req] - s.p_src
 * (pos_offset_h may be NULL).  A job never crosses a page boundary on
 * either side.  Writes at most max_jobs jobs to jobs_h and their count to
 * *n_jobs_h; SX_EINVAL if a run leaves its page arrays or max_jobs is too
 * small (sx_realign_jobs_bound() is always enough). */
sx_status sx_plan_realign(const sx_segment *segs_h, int32_t n_segs, const int32_t *src_page_ids_h,
                          int32_t n_src_ids, const int32_t *block_table_h, int32_t n_req,
                          int32_t max_pages, int32_t page_size, const int32_t *pos_offset_h,
                          sx_realign_job *jobs_h, int32_t max_jobs, int32_t *n_jobs_h);

/* Upper bound on the job count sx_plan_realign() produces. */
int32_t sx_realign_jobs_bound(const sx_segment *segs_h, int32_t n_segs, int32_t page_size);

/* ----------------------------------------------------------------------- */
/* Segment lookup (host; §4.1-§4.5).  Turns a reused segment's token ids    */
/* and extra key into cached blocks and realign descriptors.                */
/* ----------------------------------------------------------------------- */

/* h_virt = H(B, e) of §4.3 for the n_tok token ids of a block and an extra
 * key e: SHA-256 (FIPS 180-4) over e as 8 little-endian bytes followed by
 * each token id as 4 little-endian bytes; *hash_h = the first 8 digest bytes
 * as a little-endian integer.  Position- and prefix-independent (§4.4): no
 * parent hash is chained in. */
sx_status sx_virtual_hash(const int32_t *tokens_h, int32_t n_tok, uint64_t extra_key,
                          uint64_t *hash_h);

/* The block pool and its virtual-block index (§4.1 frozen blocks, §4.2 the
 * frozen-block pool, §4.4 virtual blocks).  One pool of n_blocks physical
 * KV blocks (the page ids of sx_pages) of block_size tokens.  Per block:
 * in use or free, a reference count, a frozen flag and a hit count.  A
 * virtual entry {h_virt, block, position of its first token in the cached
 * copy, its token ids, extra key} owns no KV memory.  Frozen blocks stay in
 * use at reference count 0; when more than evict_num/evict_den of the pool
 * is in use after an allocation (§4.1: 90% -> 9/10), frozen blocks nobody
 * holds are evicted, fewest hits first, then the earliest frozen, then the
 * lowest id.  Not thread-safe: calls on one index must not overlap.  Calls
 * that take a list of ids check the whole list first; a failed call leaves
 * the index unchanged.  *index_h is NULL on failure. */
typedef struct sx_index sx_index;
sx_status sx_index_create(int32_t n_blocks, int32_t block_size, int32_t evict_num,
                          int32_t evict_den, sx_index **index_h);
void sx_index_destroy(sx_index *index);

/* Allocate n blocks (the lowest free ids, ascending, reference count 1) into
 * ids_h [n]: a request's carrier blocks (§4.5) or a segment being cached.
 * Evicts unheld frozen blocks when fewer than n are free; SX_ENOMEM if even
 * that cannot supply n.  Then evicts while the pool is above the threshold. */
sx_status sx_index_alloc(sx_index *index, int32_t n, int32_t *ids_h);

/* Drop one reference per listed id (an id may repeat).  A block that reaches
 * 0 and is not frozen is freed with its virtual entries.  SX_EINVAL if a
 * block is free or would drop below 0. */
sx_status sx_index_release(sx_index *index, const int32_t *ids_h, int32_t n);

/* Register a cached segment (§4.2 insert API; §4.4): its n_tok token ids
 * tokens_h, extra key, the ceil(n_tok / block_size) blocks ids_h holding it
 * (all in use) and p_src, the RoPE position of its first token in that
 * copy.  Every full block j gets a virtual entry at position
 * p_src + j*block_size; the partial last block gets none.  frozen != 0 also
 * freezes the full blocks. */
sx_status sx_index_insert(sx_index *index, const int32_t *tokens_h, int32_t n_tok,
                          uint64_t extra_key, const int32_t *ids_h, int32_t p_src, int32_t frozen);

/* Look up the n_tok / block_size full blocks of a reused segment (§4.3,
 * §4.5): block j hits a live entry whose hash, extra key and token ids all
 * equal its own (the most recently inserted of several).  Writes block_h[j]
 * (the physical block) and pos_h[j] (its cached position), or -1 / -1 on a
 * miss.  Each hit takes a reference on its block, to be released once the
 * realign copy out of it is done, and counts one hit. */
sx_status sx_index_lookup(sx_index *index, const int32_t *tokens_h, int32_t n_tok,
                          uint64_t extra_key, int32_t *block_h, int32_t *pos_h);

/* Delete blocks from the index (§4.2 delete API): their virtual entries go,
 * they are unfrozen, and those nobody holds are freed. */
sx_status sx_index_remove(sx_index *index, const int32_t *ids_h, int32_t n);

/* stats_h[4] = {blocks in use, free blocks, frozen blocks, live entries}. */
sx_status sx_index_stats(const sx_index *index, int32_t *stats_h);

/* Realign descriptors of one reused piece from its lookup (§4.5).  The piece
 * is n_tok tokens at token index dst_start of request req; block_h/pos_h
 * hold the lookup of its n_tok / block_size full blocks.  Each run of hits
 * whose cached positions continue block after block becomes one sx_segment
 * (src_slot0 0, src_pages_off = ids_off + its first id's index in src_ids_h);
 * src_ids_h receives the hit blocks in order.  piece_reuse_h/piece_len_h
 * receive the piece's split into reused (1) and to-prefill (0) runs -- misses
 * and the partial last block -- in sx_plan_layout's piece format.  Each
 * output array needs n_tok / block_size + 1 entries; counts go to
 * *n_segs_h, *n_ids_h and *n_pieces_h. */
sx_status sx_plan_segments(int32_t req, int32_t dst_start, const int32_t *block_h,
                           const int32_t *pos_h, int32_t n_tok, int32_t block_size,
                           int32_t ids_off, sx_segment *segs_h, int32_t *n_segs_h,
                           int32_t *src_ids_h, int32_t *n_ids_h, int32_t *piece_reuse_h,
                           int32_t *piece_len_h, int32_t *n_pieces_h);

/* ----------------------------------------------------------------------- */
/* Device entry points.                                                     */
/* ----------------------------------------------------------------------- */

/* Operation ids for sx_workspace_bytes(). */
enum { SX_OP_REALIGN = 0, SX_OP_RECOMPUTE = 1, SX_OP_SELECT = 2, SX_OP_TOPK = 3,
       SX_OP_SPARSE_ATTN = 4, SX_OP_FULL_ATTN = 5, SX_OP_DECODE = 6 };

/* Bytes of device workspace `op` needs (0 if none).  n_tok: tokens of the
 * batch; n_rows: rows of the call (Sparse-Q rows for SX_OP_SELECT, active
 * rows for SX_OP_SPARSE_ATTN); n_req: requests. */
size_t sx_workspace_bytes(int32_t op, const sx_dims *dims, int32_t n_tok, int32_t n_rows,
                          int32_t n_req);

/* Step 1 -- RoPE re-alignment (§3.1 delta equation; §4.4 copy semantics;
 * §4.5 fused copy-Delta-RoPE kernel).  For every job and every kv head:
 *   K_dst[dst_page][h][dst_slot+j] = R_delta K_src[src_page][h][src_slot+j]
 *   V_dst[dst_page][h][:][dst_slot+j] = V_src[src_page][h][:][src_slot+j]
 * for j < n_tok.  R_delta uses rope_tab row |delta| (sin negated when
 * delta < 0), so rope_len must exceed every |delta|.  Source pools are only
 * read (virtual blocks share them, §4.4); src and dst may be the same pool
 * if the pages are disjoint.  jobs: device array of n_jobs jobs. */
sx_status sx_rope_realign(const sx_dims *dims, const sx_layout *lay, const sx_pages *src,
                          const sx_pages *dst, const sx_realign_job *jobs, int32_t n_jobs,
                          void *stream);

/* Step 3 -- Sparse-KV recomputation (§3.4; §4.5 "normal attention
 * computation" for recomputed tokens).  For each of the n_rows packed token
 * ids rows[m]:  [q | k | v] = x[rows[m]] . w_qkv^T  (fp32 accumulation),
 * q and k rotated by R_pos at the token's position, then
 *   k, v scattered into the pages of the token's request (overwriting any
 *   realigned copy), q written to q_out[m] ([n_rows][n_q_heads][head_dim]).
 * x: [n_tok][hidden]; w_qkv: [(Hq + 2 Hkv) * head_dim][hidden], rows of W_q
 * then W_k then W_v.  q_out may be NULL (K/V only, e.g. to build a cache).
 * rows need not be sorted; a token listed twice is written twice with the
 * same values.  rope_len must exceed every position. */
sx_status sx_recompute_kv(const sx_dims *dims, const sx_layout *lay, const void *x,
                          const int32_t *rows, int32_t n_rows, const void *w_qkv,
                          const sx_pages *kv, void *q_out, void *stream);

/* Steps 3 and 1 of two consecutive sparse layers in one call:
 * sx_recompute_kv(dims, lay, x, rows, n_rows, w_qkv, kv, q_out) for layer l
 * and sx_rope_realign(dims, lay, rsrc, rdst, jobs, n_jobs) for layer l+1's
 * cache (§3.4 recomputation; §3.1 delta equation and §4.4 copy semantics),
 * with the same results as the two calls in either order.  Layer l+1's
 * realign only has to finish before its own recomputation, so when the
 * projection's tiles leave compute units free (bf16, more than 64 rows) the
 * realign jobs run on those units inside the same launch; otherwise the two
 * are launched one after the other.  rdst must not share pages with kv (a
 * different pool; the call rejects rdst == kv with SX_EINVAL, and partial
 * overlaps are undefined).  Errors: those of the two calls. */
sx_status sx_recompute_kv_realign(const sx_dims *dims, const sx_layout *lay, const void *x,
                                  const int32_t *rows, int32_t n_rows, const void *w_qkv,
                                  const sx_pages *kv, void *q_out, const sx_pages *rsrc,
                                  const sx_pages *rdst, const sx_realign_job *jobs, int32_t n_jobs,
                                  void *stream);

/* Step 2 -- Sparse-Q scoring and top-k (§3.2 probe cost equation and the
 * paragraph after it: one score per token aggregated across heads; §3.3
 * first sentence: top-k per request).  For every token j of request r:
 *   scores[j] = sum_h sum_{i in I_nr(r), i >= j} exp(q_i^h . k_j / sqrt(d)
 *               - lse_i^h)
 * (the causal attention probability Sparse-Q row i, head h puts on key j).
 *   q: query rows; Sparse-Q row i (0..n_sq-1) is q[q_index[i]] (q_index NULL
 *      means q[i]); layout [*][n_q_heads][head_dim].
 *   sq_rows: packed token ids of I_nr, ascending within each request and
 *      grouped by request as given by sq_start [n_req+1].
 *   lse: natural-log softmax normaliser of each Sparse-Q row and head, same
 *      row indexing as q ([*][n_q_heads]); NULL: computed here over the
 *      cache (keys 0..i of the row's request).
 *   tok_class: [n_tok], 0 marks the selection candidates.
 *   k_sel: [n_req] budgets (clamped to [0, #candidates]).
 * Outputs: sel_rows -- for request r, the k_sel[r] candidates with the
 *   largest score (ties: lower token id first), ascending, stored at offset
 *   sum_{r'<r} k_sel[r'].  act_rows (may be NULL) -- the active set
 *   I_nr(r) U S(r) ascending, at offset sq_start[r] + sum_{r'<r} k_sel[r'].
 *   scores (may be NULL) -- [n_tok] fp32.
 * ws: sx_workspace_bytes(SX_OP_SELECT, dims, n_tok, n_sq, n_req) bytes. */
sx_status sx_select_topk(const sx_dims *dims, const sx_layout *lay, const void *q,
                         const int32_t *q_index, const int32_t *sq_rows, const int32_t *sq_start,
                         int32_t n_sq, const float *lse, const sx_pages *kv,
                         const uint8_t *tok_class, const int32_t *k_sel, int32_t *sel_rows,
                         int32_t *act_rows, float *scores, void *ws, size_t ws_bytes,
                         void *stream);

/* The selection half of sx_select_topk on given scores (§3.3 first
 * sentence): per request r (tokens seq_start[r]..seq_start[r+1]-1), the
 * k_sel[r] tokens with tok_class 0 and the largest scores[j] (-0.0 equals
 * +0.0; ties: lower id first), ascending, at offset sum_{r'<r} k_sel[r'].
 * NaN scores give an unspecified (but in-bounds) selection.
 * ws: sx_workspace_bytes(SX_OP_TOPK, dims, n_tok, 0, n_req) bytes (per-request
 * digit histograms and per-chunk counts of the multi-workgroup radix select);
 * a smaller or NULL ws returns SX_EWORKSPACE. */
sx_status sx_topk(const float *scores, const uint8_t *tok_class, const int32_t *seq_start,
                  int32_t n_req, int32_t n_tok, const int32_t *k_sel, int32_t *sel_rows,
                  void *ws, size_t ws_bytes, void *stream);

/* Step 4 -- attention of the active rows (§3.2: Sparse-Q rows interact with
 * all available keys at their true positions; §4.5 last paragraph).  For
 * each active row m (packed token id rows[m], index i in its request) and
 * query head h with kv head g = h / (Hq/Hkv):
 *   o[m][h*d:(h+1)*d] = sum_{j<=i} softmax_j(q[m][h] . k_j^g / sqrt(d)) v_j^g
 * over the request's paged cache.  q: [n_rows][Hq][d]; o: [n_rows][Hq*d];
 * lse (may be NULL): [n_rows][Hq] natural-log normalisers.  rows are
 * grouped by request per row_start [n_req+1] and ascending within a
 * request.  ws: sx_workspace_bytes(SX_OP_SPARSE_ATTN, ...) bytes. */
sx_status sx_sparse_attn(const sx_dims *dims, const sx_layout *lay, const void *q,
                         const int32_t *rows, const int32_t *row_start, int32_t n_rows,
                         const sx_pages *kv, void *o, float *lse, void *ws, size_t ws_bytes,
                         void *stream);

/* sx_sparse_attn in two calls, for callers that attend over the same active
 * rows in many layers (after the boundary selection of §3.4 the set
 * A = I_nr U S is fixed for every later layer).
 * sx_sparse_attn_plan: the work list of the attention over rows / row_start
 *   (as for sx_sparse_attn), written into ws; only ws is written.
 * sx_sparse_attn_run: sx_sparse_attn over the work list already in ws.
 *   dims, lay, rows, row_start's content and n_rows must be those the plan
 *   was built for, and ws must not have been written in between (by this
 *   library or the caller); any number of runs may follow one plan, with any
 *   q, kv, o and lse.  Violations give unspecified outputs (in-bounds
 *   accesses only).  sx_sparse_attn(...) equals the plan followed by a run
 *   and gives the same bits.
 * ws: sx_workspace_bytes(SX_OP_SPARSE_ATTN, ...) bytes for both.  Errors as
 * for sx_sparse_attn. */
sx_status sx_sparse_attn_plan(const sx_dims *dims, const sx_layout *lay, const int32_t *rows,
                              const int32_t *row_start, int32_t n_rows, void *ws, size_t ws_bytes,
                              void *stream);
sx_status sx_sparse_attn_run(const sx_dims *dims, const sx_layout *lay, const void *q,
                             const int32_t *rows, int32_t n_rows, const sx_pages *kv, void *o,
                             float *lse, void *ws, size_t ws_bytes, void *stream);

/* Full causal prefill attention of every token (the layers before the
 * threshold, §3.4): sx_sparse_attn with rows = 0..n_tok-1.  q: [n_tok][Hq][d],
 * o: [n_tok][Hq*d], lse: [n_tok][Hq] or NULL. */
sx_status sx_full_attn(const sx_dims *dims, const sx_layout *lay, const void *q,
                       const sx_pages *kv, void *o, float *lse, void *ws, size_t ws_bytes,
                       void *stream);

/* Decode attention over the mixed paged cache (§4.5 last paragraph: after
 * the first prefill pass, decode reads the realigned and recomputed blocks
 * through the block table).  One query row per request, at its last token:
 * request r holds T_r = seq_start[r+1] - seq_start[r] tokens in its pages,
 * the new token's k/v already written (sx_recompute_kv of that row), and
 *   o[r][h*d:(h+1)*d] = sum_{j<T_r} softmax_j(q[r][h] . k_j^g / sqrt(d)) v_j^g
 * with g = h / (Hq/Hkv).  q: [n_req][Hq][d]; o: [n_req][Hq*d]; lse (may be
 * NULL): [n_req][Hq] natural-log normalisers.  A request with no tokens
 * gets o = 0 and lse = -inf.  bf16 only (SX_EUNSUPPORTED for fp32).
 * ws: sx_workspace_bytes(SX_OP_DECODE, dims, n_tok, 0, n_req) bytes. */
sx_status sx_decode_attn(const sx_dims *dims, const sx_layout *lay, const void *q,
                         const sx_pages *kv, void *o, float *lse, void *ws, size_t ws_bytes,
                         void *stream);

/* sx_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory around the call: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The partial results
 * go to a static scratch array of SX_DECODE_NOALLOC_SCRATCH_BYTES (4 MiB)
 * inside the library; each GPU holds its own copy until the process ends.
 * The first call on a device looks up that device's copy (the stream must
 * belong to the current device).  Calls whose workspace need
 * (sx_workspace_bytes(SX_OP_DECODE, ...)) exceeds the scratch return
 * SX_EWORKSPACE and launch nothing; with Llama-3-8B shapes that is above
 * about 250 requests per call.  Every call on one GPU shares its scratch, so
 * calls that overlap on one GPU (different streams without ordering, or
 * different host threads) race and give wrong results.  The call allocates
 * and frees nothing.  Arguments, outputs and other errors as for
 * sx_decode_attn; the results are bitwise those of sx_decode_attn. */
#define SX_DECODE_NOALLOC_SCRATCH_BYTES (4u << 20)
sx_status sx_decode_attn_noalloc(const sx_dims *dims, const sx_layout *lay, const void *q,
                                 const sx_pages *kv, void *o, float *lse, void *stream);

/* Measurement utility, not a step of the method: a throughput probe of the
 * MFMA units, the measured counterpart of the data-sheet bf16 peak that the
 * attention utilisation is also quoted against.  Launches n_workgroups
 * workgroups of 8 waves (two per SIMD when one workgroup runs per compute
 * unit); every wave issues iters x 16 back-to-back v_mfma_f32_32x32x16_bf16
 * (32768 flop each), eight in a row on each of two accumulators, so the
 * launch performs n_workgroups * 8 * iters * 16 * 32768 flop.  Operands are
 * small constants (random_operands == 0) or random bf16 values in [-2, 2)
 * from eight register sets in turn (random_operands != 0): the chip draws
 * more power and holds a lower clock on random data, so the two rates
 * bracket what an MFMA-bound kernel can reach.  Time it with events on
 * `stream`.  out: device, n_workgroups * 8 floats (one reduced value per
 * wave, written so the work is not optimised away; the values carry no
 * meaning).  Errors: SX_EINVAL for n_workgroups or iters outside [1, 2^20]
 * or a NULL out; SX_EDEVICE if the launch fails. */
sx_status sx_mfma_peak_probe(int32_t n_workgroups, int32_t iters, int32_t random_operands, float *out,
                             void *stream);

/* Text of the last non-OK status returned on the calling thread. */
const char *sx_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SX_H */
