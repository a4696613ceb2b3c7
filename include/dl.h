/*
 * dl.h — C ABI of the sparse-attention MoE decode layer step for AMD MI355X (gfx950).
 *
 * One decode step of a long-context sparse-attention mixture-of-experts layer:
 *   S1  an int8 indexer scores every cached position of each sequence,
 *   S2  the best `top_k` positions are kept,
 *   S3-S5 attention runs over only those FP8 latent entries, then W_UV, W_O and the residual,
 *   S6  a router picks each token's experts,
 *   S7-S9 the chosen FP8 SwiGLU experts (plus shared experts) stream through the FFN.
 * Sources (the pages this follows):
 *   "RunanywhereAI/trnrt" summary, "The interesting bit": sparse attention over the top 2,048
 *     positions; decode layers as fused kernels.
 *   "Introducing Kiln: LLM Inference on AWS Trainium":
 *     "How was Kiln measured against vLLM on H200?" — sparse attention over a compressed latent
 *       cache that is not split across heads; routed experts (8 per token) and a shared expert;
 *       FP8 weights with 128 x 128 block scales;
 *     "What moved the number from 19.4 to 122.9 tokens a second?" — separate scoring and top-k
 *       kernels over a separate pool-key cache; MoE tile skip;
 *     "A collective costs per graph, so the graphs got big" — each expert applied once to all of
 *       its tokens;
 *     "The decode kernels, and why they are opt-in" — gather the selected entries, do not mask;
 *     "What could only a device show?" — padded rows must not write what others read; a host copy
 *       is not ordered behind work already queued.
 *
 * Conventions for every entry point
 *   Memory      Every tensor pointer is a DEVICE pointer owned by the caller, 16-byte aligned,
 *               row-major and densely packed in the stated shape.  The library never allocates,
 *               frees or keeps device memory; scratch comes from the caller's workspace `ws` of
 *               `ws_bytes` bytes (query the size first; 256-byte alignment).  A workspace also carries
 *               a scheduling hint from one call to the next (the expert kernels' per-XCD shares of
 *               their work, from the rates measured in the last call); it never changes a result, so
 *               any workspace of the right size works, and reusing one per stream is fastest.  Inputs are never
 *               modified; outputs are overwritten completely (including -1 padding).  Descriptor structs (dl_pages,
 *               dl_mat, dl_layer_desc, dl_layer_io) live in HOST memory and are read during the
 *               call only.
 *   Streams     Work is only enqueued on `stream` (a hipStream_t passed as void*).  NULL is HIP's null
 *               stream, which is torch's default stream: work goes there only when the caller passes
 *               it, exactly as on any other stream.  The library never synchronises a stream or the
 *               device; the caller orders its own writes of the inputs on that stream.  Concurrent
 *               calls need distinct workspaces.
 *   Errors      Arguments are checked on the host before anything is enqueued.  On error the call
 *               returns a negative dl_status, enqueues nothing and sets dl_last_error().  A request
 *               the kernels do not support is rejected (DL_ERR_UNSUPPORTED), never degraded.  A
 *               failed launch returns DL_ERR_HIP.
 *   Padding     seq_lens[b] == 0 marks a padding row: its sel is all -1, its attention output is 0
 *               (so its hidden state is the residual), and it writes only its own output rows.
 *   Determinism Identical inputs give bitwise identical outputs (no floating-point atomics).
 */
#ifndef DL_H
#define DL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DL_ABI_VERSION 3

typedef enum {
    DL_OK = 0,
    DL_ERR_NULL = -1,        /* a required pointer is NULL */
    DL_ERR_SHAPE = -2,       /* sizes inconsistent or out of range */
    DL_ERR_DTYPE = -3,       /* unsupported dtype or dtype combination */
    DL_ERR_UNSUPPORTED = -4, /* valid request the kernels do not implement */
    DL_ERR_WORKSPACE = -5,   /* workspace NULL, misaligned or too small */
    DL_ERR_HIP = -6          /* a HIP launch failed */
} dl_status;

typedef enum { DL_F32 = 0, DL_BF16 = 1, DL_FP8_E4M3 = 2, DL_I8 = 3, DL_I32 = 4 } dl_dtype;

/* Paged cache geometry of a batch.  Position p of row b lives in page
 * page_table[b * max_pages_per_seq + p / page_size], slot p % page_size.
 * page_size is a power of two; entries past ceil(seq_lens[b] / page_size) are never read.
 * key_layout is the layout of the int8 index-key cache (k_pool, or the pool-key cache) that the calls taking
 * these pages read or write; every other cache is row-major:
 *   DL_LAYOUT_ROWS  (0): [n_pages, items per page, dim], item-major.
 *   DL_LAYOUT_TILES (1): the same bytes regrouped per 16 consecutive items of a page (item index i of the
 *     whole array, group i / 16): inside a group's 16 * dim bytes, byte kc*1024 + g*256 + (i % 16)*16 + j holds
 *     key byte kc*64 + g*16 + j of item i (kc < dim / 64, g < 4, j < 16).  These are the operand bytes of the
 *     scoring kernel's int8 matrix instructions, so each of its loads reads 1 KB contiguous instead of sixteen
 *     64-byte pieces of different lines.  Needs dim % 64 == 0 and items per page a multiple of 16;
 *     dl_tile_index_keys converts a row-major cache. */
typedef struct {
    int32_t batch;             /* B >= 1 */
    int32_t page_size;         /* tokens per page, power of two, 1..1024 */
    int32_t max_pages_per_seq; /* columns of page_table; max seq_len <= this * page_size */
    const int32_t *seq_lens;   /* device int32 [B], 0 <= seq_lens[b] <= max_pages_per_seq * page_size */
    const int32_t *page_table; /* device int32 [B, max_pages_per_seq], page ids of the pools */
    int32_t key_layout;        /* DL_LAYOUT_ROWS or DL_LAYOUT_TILES (index-key cache only) */
} dl_pages;

/* A stack of weight matrices [count][rows = out][cols = in].
 * DL_FP8_E4M3: w holds OCP e4m3fn codes and scale holds one fp32 per 128 x 128 block,
 * [count][ceil(rows/128)][ceil(cols/128)]; the weight is code * scale ("FP8 weights with
 * 128 x 128 block scales", Kiln, "How was Kiln measured against vLLM on H200?").
 * DL_F32: w holds fp32 values, scale is NULL.
 * layout DL_LAYOUT_ROWS: row-major.  DL_LAYOUT_TILES (FP8 only): the loader's re-tiling done by
 * dl_pack_weights — every 16-row x 128-column tile is 2,048 contiguous bytes, tiles ordered by
 * (matrix, 16-row tile, 128-column block), and inside a tile byte h*1024 + l*16 + i holds
 * row l % 16, column h*64 + (l / 16)*16 + i (h < 2, l < 64, i < 16): the operand of one matrix-core
 * instruction, so every weight load is a contiguous 1 KB. */
#define DL_LAYOUT_ROWS 0
#define DL_LAYOUT_TILES 1
typedef struct {
    const void *w;
    const float *scale;
    int32_t dtype;
    int32_t count, rows, cols;
    int32_t layout;
} dl_mat;

int dl_abi_version(void);
/* HIP_VERSION the library was compiled against (major * 10^7 + minor * 10^5 + patch).  A loader refuses a
 * library whose HIP major version differs from the runtime it will share the process with (the library runs on
 * whatever libamdhip64 the process loaded first, e.g. the one bundled with torch). */
int dl_hip_version(void);

/* Re-tile a row-major FP8 weight stack (src->layout == DL_LAYOUT_ROWS, rows % 16 == 0,
 * cols % 128 == 0) into DL_LAYOUT_TILES at dst (device, count*rows*cols bytes, not overlapping src).
 * Scales are unchanged.  Done once when weights are loaded, the way Kiln's loader fits each
 * 128 x 128 block to a kernel tile ("Expert parallelism without an all-to-all"). */
int dl_pack_weights(const dl_mat *src, void *dst, void *stream);
/* Regroup a row-major int8 index-key cache (n_items = n_pages * items per page rows of dim bytes) into
 * DL_LAYOUT_TILES at dst (device, n_items * dim bytes, not overlapping src).  n_items % 16 == 0,
 * dim % 64 == 0, 64 <= dim <= 256.  Done once when a cache is loaded; dl_kv_append keeps it tiled. */
int dl_tile_index_keys(const int8_t *src, int8_t *dst, int64_t n_items, int32_t dim, void *stream);
/* Message of the last failed call on this host thread (library-owned, valid until the next call). */
const char *dl_last_error(void);

/* ---------------------------------------------------------------- current-token append
 * The step before S1: write each row's new token into its cache slot, in the layout S1 and S3 read
 * (Kiln, "How was Kiln measured ...": a compressed latent cache in FP8; "What moved the number ...":
 * a separate key cache for the scoring kernel).  The pages do not print the quantiser; this is the
 * plainest one that fits the stored layout.  The new token is position p = seq_lens[b] - 1 (the
 * lengths already count it), page page_table[b, p / page_size], slot p % page_size:
 *   kv_scale[page, slot, j] = s_j = amax_j / 448 in fp32, amax_j = max |latent[b, d]| over the
 *                             128-feature block j (s_j = 0 for an all-zero block);
 *   kv_pool[page, slot, d]  = e4m3fn code of latent[b, d] / s_j (fp32 quotient, nearest, ties to even,
 *                             saturating at 448; 0 when s_j == 0);
 *   k_pool[page, slot, i]   = round-half-even(key[b, i] / key_scale) clamped to [-127, 127], one
 *                             key_scale for every position so that the integer scores stay comparable.
 * Padding rows (seq_lens[b] == 0) write nothing ("What could only a device show?": padded rows that
 * wrote one shared slot raced).  When several rows address the same physical slot, only the lowest
 * row writes it, so the result never depends on the order the rows run in.
 *   latent   [B, d_c] in lat_dt (DL_F32 or DL_BF16)
 *   key      [B, idx_dim] in key_dt (DL_F32 or DL_BF16); unused (may be NULL) when idx_dim == 0
 *   kv_pool  FP8 codes [n_pages, page_size, d_c], kv_scale fp32 [n_pages, page_size, ceil(d_c/128)],
 *   k_pool   int8 [n_pages, page_size, idx_dim] in pages->key_layout: in/out — only the addressed slots are written, every
 *            other byte of the pools is left unchanged (the exception to "outputs are overwritten").
 * page_table entries of the written pages must be valid page ids of the pools (not checked).
 * Limits: 1 <= d_c <= 1024; 0 <= idx_dim <= 1024; key_scale finite and > 0 when idx_dim > 0.
 * No workspace. */
int dl_kv_append(const dl_pages *pages, const void *latent, int32_t lat_dt, int32_t d_c, const void *key,
                 int32_t key_dt, int32_t idx_dim, float key_scale, uint8_t *kv_pool, float *kv_scale, int8_t *k_pool,
                 void *stream);

/* ---------------------------------------------------------------- S1 + S2
 * Indexer scoring and exact top-k selection (Kiln, "What moved the number ...": a scoring kernel
 * and a top-k kernel over a separate key cache; trnrt summary: the top 2,048 positions are kept).
 * For every row b and position p < seq_lens[b]:
 *   score[p] = sum_{h < n_heads} max(0, sum_{d < dim} q_idx[b,h,d] * k_pool[page, slot, d])
 * accumulated exactly in int32.  The kept set is the first min(top_k, seq_lens[b]) positions under
 * the order (score descending, position ascending) — ties go to the lower position.
 *   q_idx   int8 [B, n_heads, dim]
 *   k_pool  int8 [n_pages, page_size, dim] in pages->key_layout
 *   sel     int32 [B, top_k]  out: kept positions in ascending order, then -1
 *   sel_score int32 [B, top_k] out, nullable: score of each kept position (0 for padding)
 * Limits: 1 <= n_heads <= 64, dim % 16 == 0, dim <= 256, n_heads * dim <= 131071 (int32 bound),
 * 1 <= top_k <= 65536.  Workspace: dl_indexer_topk_workspace(pages). */
size_t dl_indexer_topk_workspace(const dl_pages *pages);
int dl_indexer_topk(const dl_pages *pages, const int8_t *q_idx, const int8_t *k_pool, int32_t n_heads,
                    int32_t dim, int32_t top_k, int32_t *sel, int32_t *sel_score, void *ws, size_t ws_bytes,
                    void *stream);

/* Pool-granular selection (Kiln, "What moved the number ...": a separate pool-key cache scored by its own
 * kernel; "The decode kernels, and why they are opt-in": decode attention gathers the 512 selected pools).
 * The pages do not say how a pool's key is formed, so the pool-key cache is an input: one int8 key per pool
 * of `pool` consecutive positions (pool p = positions [p pool, (p + 1) pool)), paged like the position keys
 * with page_size / pool pools per page: pool_keys int8 [n_pages, page_size / pool, dim] in pages->key_layout
 * (tiles need 16 | page_size / pool), pool p of row b at
 * page page_table[b, p / (page_size / pool)], entry p % (page_size / pool).  Every pool holding a cached
 * position (ceil(seq_lens[b] / pool) of them) is scored exactly as in dl_indexer_topk; the kept pools are
 * the first min(top_pools, pool count) under (score descending, pool ascending), in ascending order, and
 * each is written as its `pool` positions:
 *   sel        int32 [B, top_pools * pool]  out: positions ascending; positions >= seq_lens[b] and unused
 *              slots are -1 (all -1 entries come after the valid ones)
 *   pool_score int32 [B, top_pools]         out, nullable: scores of the kept pools, then 0
 * pool = 1 is dl_indexer_topk on pool_keys.  Limits: pool a power of two <= page_size; top_pools * pool
 * <= 65536; otherwise as dl_indexer_topk.  Workspace: dl_indexer_topk_pooled_workspace(pages, pool). */
size_t dl_indexer_topk_pooled_workspace(const dl_pages *pages, int32_t pool);
int dl_indexer_topk_pooled(const dl_pages *pages, int32_t pool, const int8_t *q_idx, const int8_t *pool_keys,
                           int32_t n_heads, int32_t dim, int32_t top_pools, int32_t *sel, int32_t *pool_score,
                           void *ws, size_t ws_bytes, void *stream);

/* Multi-row decode (multi-token-prediction verification: TileRT, "Running the Generation Example with
 * Multi-Token Prediction (MTP)", depth 1 or 3; Kiln, "What did we measure that did not pay?": MTP
 * drafts verified in one step).  Each sequence b carries R = rows_per_seq query rows, the last R tokens
 * of the sequence (seq_lens already counts them): row r (0-based) is the token at position
 * seq_lens[b] - R + r and scores only the positions p <= its own, i.e. its visible length is
 * seq_lens[b] - (R - 1 - r) (causal among the R rows; a row with no visible position is padding).
 * The key pages of a sequence are read once for all of its rows.  Rows are numbered i = b * R + r:
 *   q_idx int8 [B * R, n_heads, dim]; sel [B * R, top_k], sel_score [B * R, top_k] as in dl_indexer_topk.
 * R = 1 is dl_indexer_topk.  Limits: 1 <= R <= 4, B * R <= 4096, as dl_indexer_topk otherwise.
 * Workspace: dl_indexer_topk_rows_workspace(pages, rows_per_seq). */
size_t dl_indexer_topk_rows_workspace(const dl_pages *pages, int32_t rows_per_seq);
int dl_indexer_topk_rows(const dl_pages *pages, int32_t rows_per_seq, const int8_t *q_idx, const int8_t *k_pool,
                         int32_t n_heads, int32_t dim, int32_t top_k, int32_t *sel, int32_t *sel_score, void *ws,
                         size_t ws_bytes, void *stream);

/* Multi-row decode with pool-granular selection: R = rows_per_seq rows per sequence as in
 * dl_indexer_topk_rows, each selecting whole pools as in dl_indexer_topk_pooled over its own visible
 * length (row r of sequence b sees the ceil((seq_lens[b] - (R - 1 - r)) / pool) pools holding its visible
 * positions, and writes the positions of its kept pools below that length, -1 after):
 *   q_idx int8 [B * R, n_heads, dim]; sel int32 [B * R, top_pools * pool]; pool_score int32 [B * R,
 *   top_pools] (nullable).
 * R = 1 is dl_indexer_topk_pooled; pool = 1 is dl_indexer_topk_rows.  Limits as those two.
 * Workspace: dl_indexer_topk_rows_pooled_workspace(pages, rows_per_seq, pool); 0 for unsupported values. */
size_t dl_indexer_topk_rows_pooled_workspace(const dl_pages *pages, int32_t rows_per_seq, int32_t pool);
int dl_indexer_topk_rows_pooled(const dl_pages *pages, int32_t rows_per_seq, int32_t pool, const int8_t *q_idx,
                                const int8_t *pool_keys, int32_t n_heads, int32_t dim, int32_t top_pools,
                                int32_t *sel, int32_t *pool_score, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------- S3 - S5
 * Sparse MLA decode attention over the kept positions only (Kiln, "The decode kernels ...":
 * gather the selected entries instead of masking all keys), every head reading the same latent
 * vector (Kiln, "How was Kiln measured ...": compressed latent cache not split across heads):
 *   c_j     = latent of position sel[b,j] (FP8 code * scale of its 128-feature block, or fp32)
 *   logit   = sm_scale * q[b,h,:] . c_j          (all d_c features act as the key)
 *   p       = softmax over the kept j            (fp32, max subtracted)
 *   o[b,h]  = sum_j p_j * c_j[:d_v]              (the first d_v features act as the value)
 * then, when w_o is given:  out[b] = residual[b] + W_O concat_h(W_UV[h] o[b,h])  (W_UV optional),
 * else out = o.
 *   q        bf16 or fp32 [B, n_heads, d_c]
 *   kv_pool  FP8 codes [n_pages, page_size, d_c] with kv_scale fp32 [n_pages, page_size, ceil(d_c/128)],
 *            or fp32 [n_pages, page_size, d_c] with kv_scale NULL
 *   sel      int32 [B, top_k] as written by dl_indexer_topk (-1 entries skipped)
 *   w_uv     nullable; count = n_heads, cols = d_v, rows = head_dim
 *   w_o      nullable; rows = D, cols = n_heads * (w_uv ? head_dim : d_v)
 *   residual bf16 or fp32 [B, D] (required with w_o)
 *   out      fp32 [B, n_heads, d_v] (no w_o) or fp32 [B, D]
 * Limits: d_v <= d_c <= 1024; FP8 weights need rows % 32 == 0 and cols % 128 == 0; W_O cols <= 262144.
 * Workspace: dl_sparse_attn_workspace(...). */
size_t dl_sparse_attn_workspace(int32_t batch, int32_t n_heads, int32_t d_v, int32_t top_k, const dl_mat *w_uv,
                                const dl_mat *w_o);
int dl_sparse_attn_decode(const dl_pages *pages, const void *q, int32_t q_dt, const void *kv_pool,
                          const float *kv_scale, int32_t kv_dt, int32_t n_heads, int32_t d_c, int32_t d_v,
                          float sm_scale, const int32_t *sel, int32_t top_k, const dl_mat *w_uv, const dl_mat *w_o,
                          const void *residual, int32_t res_dt, float *out, void *ws, size_t ws_bytes,
                          void *stream);

/* ---------------------------------------------------------------- S6
 * Router (Kiln, "How was Kiln measured ...": routed experts, 8 per token):
 *   logits[b,e] = W_r[e] . h[b] + bias[e]     (fp64 accumulation of fp32 products)
 *   experts[b]  = the top_k experts by (logit descending, expert id ascending), in that order
 *   gates[b]    = softmax over those top_k logits
 *   h fp32 [B, D]; w_r fp32 [n_experts, D]; bias fp32 [n_experts] nullable;
 *   experts int32 [B, top_k]; gates fp32 [B, top_k]; logits fp32 [B, n_experts] nullable.
 * Limits: 1 <= top_k <= 32, top_k <= n_experts <= 1024, D % 4 == 0, D <= 16384.
 * Workspace: dl_moe_route_workspace(B, D, n_experts). */
size_t dl_moe_route_workspace(int32_t B, int32_t D, int32_t n_experts);
int dl_moe_route(const float *h, int32_t B, int32_t D, const float *w_r, const float *bias, int32_t n_experts,
                 int32_t top_k, int32_t *experts, float *gates, float *logits, void *ws, size_t ws_bytes, void *stream);

/* dl_moe_route for callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same computation and results as dl_moe_route, with no workspace
 * argument.  Its scratch (the router's fp64 chunk partials) is a file-scope device array of
 * DL_MOE_ROUTE_NOALLOC_MAX_SCRATCH bytes inside the library, one per GPU the library runs on, held until the
 * process ends; the call allocates nothing.  Calls that overlap on one GPU share that array and race: order them
 * (one stream, or events).  Nothing in the array needs clearing: every call writes what it reads.
 * Limits: as dl_moe_route, and ceil(D / 1024) * B * n_experts * 8 <= DL_MOE_ROUTE_NOALLOC_MAX_SCRATCH
 * (DL_ERR_SHAPE otherwise; e.g. B <= 128 at D = 6144 with 256 experts). */
#define DL_MOE_ROUTE_NOALLOC_MAX_SCRATCH (2u << 20)
int dl_moe_route_noalloc(const float *h, int32_t B, int32_t D, const float *w_r, const float *bias, int32_t n_experts,
                         int32_t top_k, int32_t *experts, float *gates, float *logits, void *stream);

/* ---------------------------------------------------------------- S7 - S9
 * Expert FFN (Kiln, "A collective costs per graph ...": each expert applied once to all of its
 * tokens; "What moved the number ...": experts with no token are skipped):
 *   f_e(h) = W_down[e] (silu(W_gate[e] h) * (W_up[e] h)),  silu(g) = g / (1 + e^-g)
 *   out[b] = residual[b] + sum_{j<top_k} gates[b,j] f_{experts[b,j]}(h[b]) + sum_s f_{n_routed+s}(h[b])
 * summed in that order (residual NULL: 0).
 *   h fp32 [B, D]; experts int32 [B, top_k] (each < n_routed, larger ids are clamped to n_routed - 1;
 *   a negative id marks a slot whose expert is not applied here, e.g. one another GPU holds in an
 *   expert-parallel layout: the slot adds nothing, as if its gate were 0); gates fp32 [B, top_k];
 *   w_gate, w_up: count = n_routed + n_shared, rows = inter, cols = D;
 *   w_down: count = n_routed + n_shared, rows = D, cols = inter;
 *   residual fp32 [B, D] nullable; out [B, D] in out_dt (DL_F32 or DL_BF16, rounded once, RNE).
 * Limits: D % 4 == 0; D <= 65536; inter <= 16384; B * (top_k + n_shared) <= 16384;
 * top_k + n_shared <= 40; n_routed <= 1024; n_routed + n_shared <= 4096.  With FP8 weights the
 * activations enter the matrix cores as two FP8 parts (value and remainder) with per-128-block
 * scales.  Workspace: dl_moe_ffn_workspace(...). */
size_t dl_moe_ffn_workspace(int32_t B, int32_t D, int32_t inter, int32_t top_k, int32_t n_routed, int32_t n_shared);
int dl_moe_ffn(const float *h, int32_t B, int32_t D, int32_t inter, const int32_t *experts, const float *gates,
               int32_t top_k, const dl_mat *w_gate, const dl_mat *w_up, const dl_mat *w_down, int32_t n_routed,
               int32_t n_shared, const float *residual, void *out, int32_t out_dt, void *ws, size_t ws_bytes,
               void *stream);

/* One GPU's expert-parallel share of the expert FFN (the layout Kiln weighs against tensor-parallel experts in
 * "Expert parallelism without an all-to-all"): the weight stacks hold the routed experts
 * [expert_lo, expert_lo + n_local) followed by n_shared shared experts (count = n_local + n_shared).  experts
 * holds the router's global ids; a pick inside the range is applied with its local index, any other pick is
 * skipped (another GPU applies it), so summing the shares of all GPUs, with the shared experts and the residual
 * counted on one of them, gives dl_moe_ffn of the whole layer.  Otherwise as dl_moe_ffn, except that top_k may
 * exceed n_local.  expert_lo >= 0 (else DL_ERR_SHAPE).  Workspace: dl_moe_ffn_workspace(B, D, inter, top_k,
 * n_local, n_shared). */
int dl_moe_ffn_ep(const float *h, int32_t B, int32_t D, int32_t inter, const int32_t *experts, const float *gates,
                  int32_t top_k, int32_t expert_lo, const dl_mat *w_gate, const dl_mat *w_up, const dl_mat *w_down,
                  int32_t n_local, int32_t n_shared, const float *residual, void *out, int32_t out_dt, void *ws,
                  size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------- the whole step
 * dl_layer_step == dl_indexer_topk -> dl_sparse_attn_decode(w_uv, w_o, residual = x) -> dl_moe_route
 * -> dl_moe_ffn(residual = h), with every intermediate kept in the workspace. */
typedef struct dl_layer_desc {
    int32_t D;           /* hidden size */
    int32_t n_heads;     /* query heads */
    int32_t d_c, d_v;    /* latent (key) width and value width */
    int32_t idx_heads;   /* indexer heads */
    int32_t idx_dim;     /* indexer dim */
    int32_t top_k;       /* positions kept */
    int32_t n_routed, n_shared, expert_top_k, inter;
    float sm_scale;
    int32_t q_dt;        /* DL_BF16 | DL_F32 (q and x) */
    int32_t kv_dt;       /* DL_FP8_E4M3 | DL_F32 */
    int32_t out_dt;      /* DL_BF16 | DL_F32 */
    dl_mat w_uv;         /* w == NULL: no W_UV */
    dl_mat w_o;
    const float *w_r;    /* fp32 [n_routed, D] */
    const float *r_bias; /* fp32 [n_routed], nullable */
    dl_mat w_gate, w_up, w_down;
} dl_layer_desc;

typedef struct dl_layer_io {
    dl_pages pages;
    const void *x;        /* [B, D] q_dt */
    const void *q;        /* [B, n_heads, d_c] q_dt */
    const int8_t *q_idx;  /* [B, idx_heads, idx_dim] */
    const void *kv_pool;  /* [n_pages, page_size, d_c] kv_dt */
    const float *kv_scale;/* [n_pages, page_size, ceil(d_c/128)] or NULL */
    const int8_t *k_pool; /* [n_pages, page_size, idx_dim] in pages.key_layout */
    void *y;              /* out [B, D] out_dt */
    /* optional debug outputs (nullable), for stage-wise checks of the fused step */
    int32_t *sel;         /* [B, top_k] */
    float *h;             /* [B, D] fp32 hidden state after attention + residual */
    int32_t *experts;     /* [B, expert_top_k] */
    float *gates;         /* [B, expert_top_k] */
    float *o;             /* [B, n_heads, d_v] attention output before projection */
    float *y32;           /* [B, D] the output in fp32 before its one rounding */
    float *logits;        /* [B, n_routed] router logits W_r h + bias (fp64 sums rounded to fp32) */
} dl_layer_io;

size_t dl_layer_workspace(const dl_layer_desc *desc, const dl_pages *pages);
int dl_layer_step(const dl_layer_desc *desc, const dl_layer_io *io, void *ws, size_t ws_bytes, void *stream);
/* The step over R = rows_per_seq query rows per sequence (multi-row decode, as dl_indexer_topk_rows):
 * io->pages describes the B sequences; x, q, q_idx, y and the debug outputs hold B * R rows (row
 * i = b * R + r).  Row r selects among the positions up to its own, and every later stage treats each row
 * as one token (B * R tokens into the router and the FFN).  R = 1 is dl_layer_step.
 * Limits: 1 <= R <= 4, B * R <= 4096.  Workspace: dl_layer_workspace_rows(desc, pages, rows_per_seq). */
size_t dl_layer_workspace_rows(const dl_layer_desc *desc, const dl_pages *pages, int32_t rows_per_seq);
int dl_layer_step_rows(const dl_layer_desc *desc, const dl_layer_io *io, int32_t rows_per_seq, void *ws,
                       size_t ws_bytes, void *stream);
/* The step with pool-granular selection (as dl_indexer_topk_pooled): io->k_pool is the pool-key cache
 * [n_pages, page_size / pool, idx_dim]; desc->top_k counts positions and must be a multiple of pool; the
 * top_k / pool best pools are kept and expanded to their positions, which attention then reads.  pool = 1
 * is dl_layer_step.  Limits: pool a power of two <= page_size; as dl_layer_step otherwise (one row per
 * sequence).  Workspace: dl_layer_workspace_pooled(desc, pages, pool); 0 for an unsupported pool. */
size_t dl_layer_workspace_pooled(const dl_layer_desc *desc, const dl_pages *pages, int32_t pool);
int dl_layer_step_pooled(const dl_layer_desc *desc, const dl_layer_io *io, int32_t pool, void *ws, size_t ws_bytes,
                         void *stream);

/* The step over R = rows_per_seq rows per sequence with pool-granular selection: the multi-token-prediction
 * verification step of dl_layer_step_rows reading the pool-key cache like dl_layer_step_pooled (each row
 * selects top_k / pool pools over its own visible length, dl_indexer_topk_rows_pooled).  R = 1 is
 * dl_layer_step_pooled, pool = 1 is dl_layer_step_rows; limits as those two.
 * Workspace: dl_layer_workspace_rows_pooled(desc, pages, rows_per_seq, pool); 0 for unsupported values. */
size_t dl_layer_workspace_rows_pooled(const dl_layer_desc *desc, const dl_pages *pages, int32_t rows_per_seq,
                                      int32_t pool);
int dl_layer_step_rows_pooled(const dl_layer_desc *desc, const dl_layer_io *io, int32_t rows_per_seq, int32_t pool,
                              void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* DL_H */
