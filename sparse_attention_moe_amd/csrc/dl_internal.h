// Host-side internals shared by the launch code of the decode layer step.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/dl.h"

namespace dl {

// Sets the thread's last-error message and returns `st`.
int fail(int st, const char *fmt, ...);
int hip_check(const char *what);  // DL_OK or DL_ERR_HIP after a launch
// Workgroups of `threads` threads of `kernel` resident on the current device at once (cached).
int resident_blocks(const void *kernel, int threads);

// Carves 256-byte-aligned regions out of a workspace.  With base == nullptr it only measures.
struct Ws {
    char *base;
    size_t off = 0;
    explicit Ws(void *b) : base((char *)b) {}
    template <class T>
    T *take(size_t n)
    {
        off = (off + 255) & ~(size_t)255;
        T *p = base ? (T *)(base + off) : nullptr;
        off += n * sizeof(T);
        return p;
    }
    size_t used() const { return (off + 255) & ~(size_t)255; }
};

// ------------------------------------------------------------- indexer + top-k
struct Thr {           // the selection threshold of a row: items scoring above hi are kept,
    int lo, hi, need;  // need of the items inside [lo, hi]
};
struct TopkWs {
    int32_t *scores;   // [B, Lmax] scores of the row's items
    unsigned *hist1;   // [B, NB1] log-linear histogram of the scores
    unsigned long long *hflag;  // [sequences] epoch of the launch that last cleared the sequence's histograms
    unsigned *bits;    // [B, nchunk * 128] kept items, one bit each (whole 4,096-item chunks)
    int2 *cand;        // [B, nchunk * 4,096] (item, score) inside the threshold bin, per chunk
    int32_t *ccnt;     // [B, nchunk] how many per chunk
    int32_t *acnt;     // [B, nchunk] items marked (above the bin) per chunk
    Thr *thr;          // [B]
};
void topk_ws_layout(Ws &w, const dl_pages &pg, TopkWs &t, int R = 1, int pool = 1);
int launch_probe_read(const void *buf, size_t bytes, size_t *bytes_read, hipStream_t s);
int launch_probe_null(int n_kernels, int blocks, hipStream_t s);
int launch_kv_append(const dl_pages &pg, const void *latent, int lat_dt, int Dc, const void *key, int key_dt, int DI,
                     float key_scale, uint8_t *kv, float *kv_scale, int8_t *kp, hipStream_t s);
// R query rows per sequence (multi-row decode): q_idx [B*R, HI, DI], sel [B*R, top_k]; row i is the token at
// position seq_lens[i / R] - R + i % R and sees the positions up to its own.
static constexpr int DL_MAX_ROWS_PER_SEQ = 4;
int launch_indexer_topk(const dl_pages &pg, const int8_t *q_idx, const int8_t *k_pool, int HI, int DI, int top_k,
                        int32_t *sel, int32_t *sel_score, const TopkWs &t, hipStream_t s, int R = 1, int pool = 1);

// ------------------------------------------------------------- GEMV engine
enum { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2 };

struct GemvArgs {
    // weights: FP8 codes + block scales, or fp32 (wf)
    const uint8_t *w;  const float *wsc;  const float *wf;
    const uint8_t *w2; const float *wsc2; const float *wf2;   // second matrix of SwiGLU (up)
    long mat_elems;
    int rows, cols, nrb, nkb;
    int tiled;               // FP8 weights in DL_LAYOUT_TILES
    // which matrices and which tokens
    const int *active;       // matrix id of active slot u (nullptr: u itself)
    const int *n_active_dev; // device count of active slots (nullptr: n_active_host)
    int n_active_host;
    const int *tok_off, *tok_cnt;  // plan mode: pairs of slot u are [tok_off[u], +tok_cnt[u])
    int ntok_host;                 // uniform mode: tokens 0..ntok-1 for every matrix
    int max_groups;                // fp32 path: upper bound of ceil(tokens per matrix / 16)
    const int *grp_off;            // plan mode: prefix over active slots of their token groups (16 / NS tokens)
    const int *pair_act;           // plan mode: activation row of global pair p
    int a_ts, a_ms;                // uniform mode: activation row = t*a_ts + m*a_ms
    long o_ts, o_ms;               // output offset = t*o_ts + m*o_ms (uniform) or p*o_ts (plan)
    // activations: NS FP8 parts [part][row][cols] + scales [part][row][nkb], or fp32 [row][cols]
    const uint8_t *aq; const float *asc;
    long aq_part, asc_part;
    const float *af;
    // output
    float *out;
    const void *resid; int resid_dt; long r_ts;    // EPI_RESID: resid[t*r_ts + row]
    // split of K into ksplit chunks of kchunk blocks: raw partial sums go to part[chunk][out offset]
    // (and part2 for the second SwiGLU matrix), then a reduction applies the epilogue
    int ksplit, kchunk;
    int flat;          // balanced step ranges; a chunk may be split in two partial slots (see k_gemv.hip)
    int oneshot;       // one-shot projection kernel: partial slot per group of 8 K-blocks
    float *part, *part2;
    long n_out;        // elements of the output array (partial buffer stride)
    int *queue;        // work queue mode (plan mode only): piece counter, zero on entry; npc pieces per unit
    int npc;
    bool reduce_in_consumer;  // the next kernel sums the partials itself (no reduction launch)
};
// Partial slots the GEMV writes: 2 per K chunk in flat mode, else 1 per chunk (0 without a split).
__host__ __device__ inline int gemv_slots(const GemvArgs &a) { return a.queue ? a.npc : a.flat ? 2 * a.ksplit : a.ksplit; }
static constexpr int MAX_KSPLIT = 16;
static constexpr int GEMV_MAXCHUNK = 128;  // most 128-wide K-blocks in one chunk of the FP8 GEMV
static constexpr int GEMV_MAXMAT = 4096;  // active matrices of one FP8 GEMV (plan mode)
// Work-queue state of one FP8 GEMV: GEMV_QPOOLS pools, one line of GEMV_QSTRIDE ints (256 B) each: [0] the
// pool's piece counter, [1] its finished waves, [2..3] and [4..5] the start and end time of its last launch
// (s_memrealtime ticks).  Ints [GEMV_QTAB, GEMV_QTAB + GEMV_QPOOLS) of pool 0's line hold the pools' shares of a
// round of GEMV_QROUND pieces (written by the plan from the pools' measured rates).
static constexpr int GEMV_QPOOLS = 8, GEMV_QSTRIDE = 64, GEMV_QINTS = GEMV_QPOOLS * GEMV_QSTRIDE;
static constexpr int GEMV_QROUND = 512, GEMV_QTAB = 16;

// The pools' shares m[0..7] of a round from the stored raw[0..7]: at least 1 each and GEMV_QROUND in all, else
// (never written) equal ones.
__device__ inline void gemv_shares_valid(const int raw[GEMV_QPOOLS], int m[GEMV_QPOOLS])
{
    int tot = 0;
    bool ok = true;
#pragma unroll
    for (int p = 0; p < GEMV_QPOOLS; p++) {
        m[p] = raw[p];
        ok = ok && m[p] >= 1 && m[p] <= GEMV_QROUND;
        tot += ok ? m[p] : 0;
    }
    if (!ok || tot != GEMV_QROUND)
#pragma unroll
        for (int p = 0; p < GEMV_QPOOLS; p++) m[p] = GEMV_QROUND / GEMV_QPOOLS;
}
__device__ inline void gemv_shares_read(const int *q, int m[GEMV_QPOOLS])
{
    int raw[GEMV_QPOOLS];
#pragma unroll
    for (int p = 0; p < GEMV_QPOOLS; p++) raw[p] = q[GEMV_QTAB + p];
    gemv_shares_valid(raw, m);
}

// Position in its round of pool p's k-th slot (k < m[p]).  The slots of all pools are ordered by (k + 1/2) / m_p,
// ties to the lower pool, so each pool's slots are spread evenly over the round and the pools advance through the
// pieces side by side; equal shares give the plain interleave p, p + 8, ....  The positions of all (p, k) are a
// permutation of the round: the position is the number of slots ordered before (p, k).
__device__ inline int gemv_slot_pos(const int m[GEMV_QPOOLS], int p, int k)
{
    const int B = m[p], B2 = 2 * m[p];
    int pos = k;
#pragma unroll
    for (int q = 0; q < GEMV_QPOOLS; q++) {
        if (q == p) continue;
        const int A = (2 * k + 1) * m[q];  // slot k' of pool q comes first iff (2k' + 1) m_p < A (<= A for q < p)
        pos += min(m[q], (A + B - (q < p ? 0 : 1)) / B2);
    }
    return pos;
}
int launch_gemv(const GemvArgs &a, int ns, int epi, bool fp8, hipStream_t s);
// Gate/up, SwiGLU + FP8 split and down of the expert FFN in one launch (k_ffn_fp8): g the gate/up GEMV (queue and
// plan mode, tiled, partial slots in part / part2), d the down GEMV (plan mode, tiled, npc <= 2 K pieces into as
// many slots of part, activations aq / asc = the FP8 parts of Z).  sync: [gmax][I / 128] finished gate/up pieces per (token group,
// 128-row block of Z), then [gmax] finished blocks per token group; zero on entry (the plan clears them).
struct FfnFused {
    GemvArgs g, d;
    int *sync;
    int gmax;
};
int launch_ffn_fused(const FfnFused &f, hipStream_t s);
// Flat mode for an FP8 GEMV of about `units_est` units: the K split (<= max_ksplit chunks) with chunks no
// longer than a wave's share of steps.
void gemv_flat(GemvArgs &a, int ns, int epi, long units_est, int max_ksplit);
// One-shot mode for a single FP8 matrix in uniform mode (rows % 128 == 0, K % 1024 == 0); false if
// the shape does not fit (then nothing is changed).
bool gemv_oneshot(GemvArgs &a, bool fp8);
int launch_pack(const uint8_t *src, uint8_t *dst, long count, int rows, int cols, hipStream_t s);
// Row-major int8 index keys [n_items][DI] -> the tiled key layout (n_items % 16 == 0, DI % 64 == 0).
int launch_tile_keys(const int8_t *src, int8_t *dst, long n_items, int DI, hipStream_t s);

// SwiGLU of summed gate/up partial slots, split into NS FP8 parts (rows may come from the device).
int launch_swiglu_quant(const float *pg, const float *pu, int nslot, long stride, long rows_host,
                        const int *rows_dev, int cols, uint8_t *q, float *sc, long q_part, long sc_part, int ns,
                        hipStream_t s);
// x fp32 rows -> NS FP8 parts with one dynamic scale per (part, row, 128 block).
int launch_quant(const float *x, long rows_host, const int *rows_dev, int cols, uint8_t *q, float *sc,
                 long q_part, long sc_part, int ns, hipStream_t s);

// ------------------------------------------------------------- attention
// opart [B, splits, H, Dv] and ml [B, splits, H, 2] are scratch for the matrix-core path.
bool attention_mfma_ok(int H, int Dc, int Dv, int q_dt, int kv_dt);
int attention_splits(int top_k, int B, int H);
// With the matrix-core path and o == nullptr only the split partials are written (the caller merges).
int launch_attention(const dl_pages &pg, const void *q, int q_dt, const void *kv, const float *kv_scale, int kv_dt,
                     int H, int Dc, int Dv, float sm_scale, const int32_t *sel, int top_k, float *o, float *opart,
                     float *ml, hipStream_t s, int R = 1);
bool attention_merge_uv_ok(int Dv, int hd);
// Merge of the split partials + W_UV (fp32, exact decode) + 4-part FP8 split of u for W_O.
int launch_attn_merge_uv(int B, int H, int Dv, int top_k, const float *opart, const float *ml, float *o,
                         const uint8_t *wuv, const float *wsc, int hd, int tiled, uint8_t *uq, float *uqs,
                         long uq_part, long uqs_part, hipStream_t s);
// h = resid + sum of W_O's K-chunk partials; with hq != nullptr also h split into 2 FP8 parts.
int launch_resid_reduce_split(const GemvArgs &a, float *h, uint8_t *hq, float *hqs, long hq_part, long hqs_part,
                              hipStream_t s);

// ------------------------------------------------------------- MoE
static constexpr int PLAN_TPG = 8;  // tokens per group of the expert GEMV (16 MFMA columns / 2 FP8 parts)
struct MoePlan {
    int *n_active;   // [1]
    int *n_pairs;    // [1]
    int *grp_off;    // [NE + 1] prefix over active slots of ceil(tokens / PLAN_TPG)
    int *active;     // [NE]
    int *tok_off;    // [NE]
    int *tok_cnt;    // [NE]
    int *pair_tok;   // [B*(ke+S)]
    int *pair_idx;   // [B, ke+S]
    int *queue;      // [2 GEMV_QINTS] work-queue counters of the expert GEMVs, cleared with the plan (nullptr: none)
    int *ffn_sync;   // hand-off counters of the fused FFN (FfnFused::sync), cleared with the plan (nullptr: none)
    int ffn_gmax, ffn_nrb;
};
int route_chunks(int D);  // hidden-size chunks of the router's partial dot products
// part [route_chunks(D), B, E] is scratch (fp64).
int launch_route(const float *h, int B, int D, const float *w_r, const float *bias, int E, int ke, int32_t *experts,
                 float *gates, float *logits, double *part, hipStream_t s);
// lo < 0: picks are stack indices (negative: computed elsewhere); lo >= 0: the stack holds experts [lo, lo + E)
int launch_plan(const int32_t *experts, int B, int ke, int E, int S, const MoePlan &p, hipStream_t s, int lo = -1);
// Router top-k (from launch_route_partial's chunk partials), with p != nullptr fused with the dispatch plan.
bool route_plan_ok(int E, int ke, int B);
int launch_route_partial(const float *h, int B, int D, const float *w_r, int E, double *part, hipStream_t s);
int launch_route_plan(const double *part, int B, int D, const float *bias, int E, int ke, int S, int32_t *experts,
                      float *gates, float *logits, const MoePlan *p, hipStream_t s);
// F: nslot partial slots of the expert outputs, fstride floats apart, summed in slot order.
int launch_combine(const float *F, int nslot, long fstride, const MoePlan &p, const float *gates, int B, int D, int ke,
                   int S,
                   const void *resid, int resid_dt, void *out, int out_dt, float *out32, hipStream_t s);

}  // namespace dl
