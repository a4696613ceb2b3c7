// Host side of the C ABI: argument checks, workspace layout and the launch sequence of each entry
// point.  Nothing here computes; every step of the path runs in the gfx950 kernels.
#include <stdarg.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include "dl_common.h"
#include "dl_internal.h"
#include "../../include/dl_measure.h"

#include <hip/hip_version.h>

#include <algorithm>
#include <mutex>

namespace dl {

static thread_local char g_err[512] = "";

int fail(int st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

int hip_check(const char *what)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(DL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return DL_OK;
}

int resident_blocks(const void *kernel, int threads)
{
    // per device and kernel; the few kernels of the library make a tiny linear cache enough
    struct Entry { int dev; const void *k; int blocks; };
    static thread_local Entry cache[64];
    static thread_local int n = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    for (int i = 0; i < n; i++)
        if (cache[i].dev == dev && cache[i].k == kernel) return cache[i].blocks;
    int per_cu = 1, cus = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu < 1) per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 1;
    const int blocks = per_cu * cus;
    if (n < 64) cache[n++] = Entry{dev, kernel, blocks};
    return blocks;
}

#define DL_TRY(x)              \
    do {                       \
        int _r = (x);          \
        if (_r != DL_OK) return _r; \
    } while (0)

static bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

// ------------------------------------------------------------------ phase events (measurement only)
struct StepMarks {
    hipEvent_t ev[DL_N_PHASES + 1];
};
static bool g_prof = false;
static int g_ffn_fused = -1;  // the last expert FFN ran fused (1), as three kernels (0), none yet (-1)
static StepMarks *g_pend = nullptr;  // recorded, not yet read
static int g_npend = 0, g_cap = 0;
static StepMarks *g_free = nullptr;
static int g_nfree = 0, g_fcap = 0;

struct Marks {
    StepMarks *m = nullptr;
    hipStream_t s = nullptr;
    void at(int i) const
    {
        // a record that fails leaves its event unrecorded, which dl_profile_read reports (elapsed time fails)
        if (m) (void)hipEventRecord(m->ev[i], s);
    }
};

static int marks_begin(Marks &mk, hipStream_t s)
{
    mk.s = s;
    mk.m = nullptr;
    if (!g_prof) return DL_OK;
    if (g_npend == g_cap) {
        g_cap = g_cap ? 2 * g_cap : 64;
        g_pend = (StepMarks *)realloc(g_pend, sizeof(StepMarks) * g_cap);
        if (!g_pend) return fail(DL_ERR_HIP, "profile: out of host memory");
    }
    StepMarks sm;
    if (g_nfree) {
        sm = g_free[--g_nfree];
    } else {
        for (int i = 0; i <= DL_N_PHASES; i++)
            if (hipEventCreate(&sm.ev[i]) != hipSuccess) return fail(DL_ERR_HIP, "profile: hipEventCreate");
    }
    g_pend[g_npend] = sm;
    mk.m = &g_pend[g_npend++];
    return DL_OK;
}

static int check_pages(const dl_pages *pg)
{
    if (!pg) return fail(DL_ERR_NULL, "pages is NULL");
    if (!pg->seq_lens || !pg->page_table) return fail(DL_ERR_NULL, "seq_lens/page_table NULL");
    if (pg->batch < 1 || pg->batch > 4096) return fail(DL_ERR_SHAPE, "batch %d", pg->batch);
    if (!pow2(pg->page_size) || pg->page_size > 1024) return fail(DL_ERR_SHAPE, "page_size %d", pg->page_size);
    if (pg->max_pages_per_seq < 1) return fail(DL_ERR_SHAPE, "max_pages_per_seq %d", pg->max_pages_per_seq);
    if ((long)pg->max_pages_per_seq * pg->page_size > (1L << 30)) return fail(DL_ERR_SHAPE, "context too long");
    if (pg->key_layout != DL_LAYOUT_ROWS && pg->key_layout != DL_LAYOUT_TILES)
        return fail(DL_ERR_SHAPE, "key_layout %d", pg->key_layout);
    return DL_OK;
}

// Tiled index keys need whole 64-byte chunks and whole 16-item groups in every page.
static int check_key_tiles(const dl_pages *pg, int dim, int pool)
{
    if (pg->key_layout == DL_LAYOUT_TILES && (dim % 64 || (pg->page_size / pool) % 16))
        return fail(DL_ERR_UNSUPPORTED, "tiled index keys need dim %% 64 == 0 (%d) and 16 | items per page (%d)", dim,
                    pg->page_size / pool);
    return DL_OK;
}

// FP8 weights need 16-row tiles and 128-column blocks; fp32 weights any shape.
static int check_mat(const dl_mat *m, const char *name, int count, int rows, int cols)
{
    if (!m || !m->w) return fail(DL_ERR_NULL, "%s: weights NULL", name);
    if (m->count != count || m->rows != rows || m->cols != cols)
        return fail(DL_ERR_SHAPE, "%s: [%d,%d,%d] expected [%d,%d,%d]", name, m->count, m->rows, m->cols, count, rows,
                    cols);
    if (m->layout != DL_LAYOUT_ROWS && m->layout != DL_LAYOUT_TILES) return fail(DL_ERR_SHAPE, "%s: layout %d", name, m->layout);
    if (m->layout == DL_LAYOUT_TILES && m->dtype != DL_FP8_E4M3) return fail(DL_ERR_DTYPE, "%s: tiles need FP8", name);
    if (m->dtype == DL_FP8_E4M3) {
        if (!m->scale) return fail(DL_ERR_NULL, "%s: FP8 needs block scales", name);
        if (rows % 32 || cols % 128) return fail(DL_ERR_UNSUPPORTED, "%s: FP8 needs rows%%32==0, cols%%128==0", name);
    } else if (m->dtype == DL_F32) {
        if (m->scale) return fail(DL_ERR_DTYPE, "%s: fp32 weights take no scale", name);
    } else {
        return fail(DL_ERR_DTYPE, "%s: dtype %d", name, m->dtype);
    }
    return DL_OK;
}

static int check_ws(void *ws, size_t have, size_t need)
{
    if (need == 0) return DL_OK;
    if (!ws) return fail(DL_ERR_WORKSPACE, "workspace NULL (%zu bytes needed)", need);
    if (((uintptr_t)ws) & 255) return fail(DL_ERR_WORKSPACE, "workspace not 256-byte aligned");
    if (have < need) return fail(DL_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", have, need);
    return DL_OK;
}

static int check_indexer(int HI, int DI, int top_k)
{
    if (HI < 1 || HI > 64) return fail(DL_ERR_UNSUPPORTED, "indexer heads %d (1..64)", HI);
    if (DI < 16 || DI > 256 || DI % 16) return fail(DL_ERR_UNSUPPORTED, "indexer dim %d (16..256, %%16)", DI);
    if ((long)HI * DI > 131071) return fail(DL_ERR_SHAPE, "indexer heads*dim may overflow int32");
    if (top_k < 1 || top_k > 65536) return fail(DL_ERR_SHAPE, "top_k %d", top_k);
    return DL_OK;
}

// ------------------------------------------------------------------ attention + projection

struct AttnWs {
    float *opart, *ml;         // split partials of the matrix-core attention
    float *kpart;              // [2 MAX_KSPLIT, B, D] partial slots of W_O
    float *o;                  // [B, H, Dv] (when the caller's out is not o)
    uint8_t *oq; float *oqs;   // 4 parts of o for W_UV
    float *u;                  // [B, H*hd]
    uint8_t *uq; float *uqs;   // 4 parts of u for W_O
};
static constexpr int PROJ_PARTS = 4;  // projections ahead of the router keep ~16 significant bits
static constexpr int FFN_PARTS = 2;

static void attn_split_ws(Ws &w, int B, int H, int Dv, int top_k, AttnWs &a)
{
    const long ns = attention_splits(top_k, B, H);
    a.opart = w.take<float>((long)B * ns * H * Dv);
    a.ml = w.take<float>((long)B * ns * H * 2);
}

static void attn_ws_layout(Ws &w, int B, int H, int Dv, int top_k, const dl_mat *w_uv, const dl_mat *w_o, AttnWs &a)
{
    a = AttnWs{};
    attn_split_ws(w, B, H, Dv, top_k, a);
    if (!w_o) return;
    const long BH = (long)B * H;
    a.o = w.take<float>(BH * Dv);
    const int hd = w_uv ? w_uv->rows : Dv;
    if (w_uv) {
        if (w_uv->dtype == DL_FP8_E4M3) {
            a.oq = w.take<uint8_t>(PROJ_PARTS * BH * Dv);
            a.oqs = w.take<float>(PROJ_PARTS * BH * (Dv / 128));
        }
        a.u = w.take<float>(BH * hd);
    }
    if (w_o->dtype == DL_FP8_E4M3) {
        a.uq = w.take<uint8_t>(PROJ_PARTS * BH * hd);
        a.uqs = w.take<float>(PROJ_PARTS * BH * (hd / 128));
        a.kpart = w.take<float>(2L * MAX_KSPLIT * B * w_o->rows);
    }
}

static GemvArgs mat_args(const dl_mat *m)
{
    GemvArgs g;
    memset(&g, 0, sizeof g);
    if (m->dtype == DL_FP8_E4M3) {
        g.w = (const uint8_t *)m->w;
        g.wsc = m->scale;
        g.tiled = m->layout == DL_LAYOUT_TILES;
    } else {
        g.wf = (const float *)m->w;
    }
    g.ksplit = 1;
    g.kchunk = (m->cols + 127) / 128;
    g.mat_elems = (long)m->rows * m->cols;
    g.rows = m->rows;
    g.cols = m->cols;
    g.nrb = (m->rows + 127) / 128;
    g.nkb = (m->cols + 127) / 128;
    return g;
}

// out = residual + W_O concat_h(W_UV[h] o[b,h]), o fp32 [B, H, Dv].
static int run_projection(int B, int H, int Dv, const float *o, const dl_mat *w_uv, const dl_mat *w_o,
                          const void *resid, int resid_dt, float *out, const AttnWs &a, hipStream_t s)
{

    const long BH = (long)B * H;
    const float *act = o;
    int K = Dv;
    if (w_uv) {
        const int hd = w_uv->rows;
        GemvArgs g = mat_args(w_uv);
        g.n_active_host = H;
        g.ntok_host = B;
        g.max_groups = (B + 15) / 16;
        g.a_ts = H;
        g.a_ms = 1;
        g.o_ts = (long)H * hd;
        g.o_ms = hd;
        g.out = a.u;
        const bool f8 = w_uv->dtype == DL_FP8_E4M3;
        if (f8) {
            DL_TRY(launch_quant(o, BH, nullptr, Dv, a.oq, a.oqs, BH * Dv, BH * (Dv / 128), PROJ_PARTS, s));
            g.aq = a.oq; g.asc = a.oqs; g.aq_part = BH * Dv; g.asc_part = BH * (Dv / 128);
        } else {
            g.af = o;
        }
        DL_TRY(launch_gemv(g, PROJ_PARTS, EPI_STORE, f8, s));
        act = a.u;
        K = H * hd;
    } else {
        K = H * Dv;
    }
    GemvArgs g = mat_args(w_o);
    g.n_active_host = 1;
    g.ntok_host = B;
    g.max_groups = (B + 15) / 16;
    g.a_ts = 1;
    g.a_ms = 0;
    g.o_ts = w_o->rows;
    g.o_ms = 0;
    g.out = out;
    g.resid = resid;
    g.resid_dt = resid_dt;
    g.r_ts = w_o->rows;
    const bool f8 = w_o->dtype == DL_FP8_E4M3;
    if (f8) {
        DL_TRY(launch_quant(act, B, nullptr, K, a.uq, a.uqs, (long)B * K, (long)B * (K / 128), PROJ_PARTS, s));
        g.aq = a.uq; g.asc = a.uqs; g.aq_part = (long)B * K; g.asc_part = (long)B * (K / 128);
        if (!gemv_oneshot(g, true))
            gemv_flat(g, PROJ_PARTS, resid ? EPI_RESID : EPI_STORE, (long)(w_o->rows / 32) * g.max_groups, MAX_KSPLIT);
        g.part = a.kpart;
        g.n_out = (long)B * w_o->rows;
    } else {
        g.af = act;
    }
    return launch_gemv(g, PROJ_PARTS, resid ? EPI_RESID : EPI_STORE, f8, s);
}

// Attention over the kept positions, then (with w_o) out = residual + W_O concat_h(W_UV[h] o[h]).
// With the matrix-core attention, FP8 W_UV/W_O and hd = 128 or 256, the split merge, W_UV and the split
// of u run as one kernel, and W_O's K-chunk reduction adds the residual (and, with hq, splits h for the
// FFN).  Both entry points use this routine, so the fused step and the separate calls agree bit for bit.
static int run_attn_proj(const dl_pages &pg, const void *q, int q_dt, const void *kv, const float *kv_scale,
                         int kv_dt, int H, int Dc, int Dv, float sm_scale, const int32_t *sel, int top_k,
                         const dl_mat *w_uv, const dl_mat *w_o, const void *resid, int resid_dt, float *o,
                         float *out, const AttnWs &a, uint8_t *hq, float *hqs, bool *h_split, hipStream_t s,
                         const Marks &mk, int R = 1, bool o_wanted = true)
{
    const int B = pg.batch * R;  // rows
    if (h_split) *h_split = false;
    const int hd = w_uv ? w_uv->rows : Dv;
    const bool fuse = w_o && w_uv && attention_mfma_ok(H, Dc, Dv, q_dt, kv_dt) && w_uv->dtype == DL_FP8_E4M3 &&
                      w_o->dtype == DL_FP8_E4M3 && attention_merge_uv_ok(Dv, hd);
    if (!fuse) {
        DL_TRY(launch_attention(pg, q, q_dt, kv, kv_scale, kv_dt, H, Dc, Dv, sm_scale, sel, top_k, o, a.opart, a.ml, s,
                                R));
        mk.at(2);
        if (!w_o) return DL_OK;
        return run_projection(B, H, Dv, o, w_uv, w_o, resid, resid_dt, out, a, s);
    }
    DL_TRY(launch_attention(pg, q, q_dt, kv, kv_scale, kv_dt, H, Dc, Dv, sm_scale, sel, top_k, nullptr, a.opart, a.ml,
                            s, R));
    mk.at(2);
    const long K = (long)H * hd;
    // with W_UV fused into the merge, o is only an output when the caller asks for it
    DL_TRY(launch_attn_merge_uv(B, H, Dv, top_k, a.opart, a.ml, o_wanted ? o : nullptr, (const uint8_t *)w_uv->w,
                                w_uv->scale, hd,
                                w_uv->layout == DL_LAYOUT_TILES, a.uq, a.uqs, (long)B * K, (long)B * (K / 128), s));
    GemvArgs g = mat_args(w_o);
    g.n_active_host = 1;
    g.ntok_host = B;
    g.max_groups = (B + 15) / 16;
    g.a_ts = 1;
    g.o_ts = w_o->rows;
    g.out = out;
    g.resid = resid;
    g.resid_dt = resid_dt;
    g.r_ts = w_o->rows;
    g.aq = a.uq; g.asc = a.uqs; g.aq_part = (long)B * K; g.asc_part = (long)B * (K / 128);
    if (!gemv_oneshot(g, true)) gemv_flat(g, PROJ_PARTS, EPI_RESID, (long)(w_o->rows / 32) * g.max_groups, MAX_KSPLIT);
    g.part = a.kpart;
    g.n_out = (long)B * w_o->rows;
    g.reduce_in_consumer = true;
    DL_TRY(launch_gemv(g, PROJ_PARTS, EPI_RESID, true, s));
    DL_TRY(launch_resid_reduce_split(g, out, hq, hqs, (long)B * w_o->rows, (long)B * (w_o->rows / 128), s));
    if (h_split) *h_split = hq != nullptr;
    return DL_OK;
}

// ------------------------------------------------------------------ FFN
static constexpr int GU_MAXK = 4;  // most K chunks of the FP8 gate/up pass (partial slots: twice that)
// Work-queue pieces per unit of the FP8 expert GEMVs (partial slots): gate/up and down.
static constexpr int GU_NPC = 2, DN_NPC = 1;
static constexpr int FUSED_DN_NPC = 2;  // K pieces (output slots) of the down pieces in the fused FFN
// at most the bit length of nkb, so no piece is empty
static int fused_dn_npc(int nkb)
{
    int maxp = 0;
    while ((nkb >> maxp) > 0) maxp++;
    return std::min(FUSED_DN_NPC, maxp);
}
static_assert(GU_NPC <= 2 * GU_MAXK, "gate/up pieces exceed the partial slots");

// Queue mode for a plan-mode FP8 GEMV of `pairs` (token, expert) pairs: npc pieces per unit (at most the bit
// length of nkb, so none is empty).  False (the caller keeps a static split) when the pieces could not be
// numbered in 31 bits or a piece would exceed the scale registers' 128 K-blocks.
static bool gemv_queue(GemvArgs &a, int *counter, int npc, long pairs)
{
    int maxp = 0;
    while ((a.nkb >> maxp) > 0) maxp++;
    if (a.nkb > GEMV_MAXCHUNK || !a.grp_off) return false;
    // units <= row tiles x token groups, and the groups of all slots are at most the pairs plus one per slot
    if ((long)(a.rows / 32) * (a.n_active_host + pairs) * std::min(npc, maxp) >= (1L << 31)) return false;
    a.queue = counter;
    a.npc = std::min(npc, maxp);
    a.flat = 0;
    a.ksplit = 1;
    a.kchunk = a.nkb;
    return true;
}

struct FfnWs {
    MoePlan plan;
    uint8_t *hq; float *hqs;   // 2 parts of h  [2][B][D]
    float *gpart, *upart;      // [2 GU_MAXK, P, I] gate/up partial slots (FP8 path)
    float *Z;                  // [P, I]
    uint8_t *zq; float *zqs;   // 2 parts of Z
    float *F;                  // [max(DN_NPC, FUSED_DN_NPC), P, D] expert outputs (partial slots in the FP8 path)
    int *queue;                // [2 GEMV_QINTS] work-queue counters (gate/up, down)
    int *sync;                 // hand-off counters of the fused FFN (FfnFused::sync; FP8 path)
};

// Gate/up, SwiGLU and down as one launch where the weights allow it (k_ffn_fp8); 0 keeps three launches.
#ifndef DL_FFN_FUSE
#define DL_FFN_FUSE 1
#endif

static void ffn_ws_layout(Ws &w, int B, int D, int I, int ke, int E, int S, bool fp8, FfnWs &f)
{
    const int NE = E + S;
    const long P = (long)B * (ke + S);
    f.plan.n_active = w.take<int>(1);
    f.plan.n_pairs = w.take<int>(1);
    f.plan.grp_off = w.take<int>(NE + 1);
    f.plan.active = w.take<int>(NE);
    f.plan.tok_off = w.take<int>(NE);
    f.plan.tok_cnt = w.take<int>(NE);
    f.plan.pair_tok = w.take<int>(P);
    f.plan.pair_idx = w.take<int>(P);
    f.queue = w.take<int>(2 * GEMV_QINTS);
    f.plan.queue = fp8 ? f.queue : nullptr;
    f.hq = nullptr; f.hqs = nullptr; f.zq = nullptr; f.zqs = nullptr;
    if (fp8) {
        f.hq = w.take<uint8_t>((long)FFN_PARTS * B * D);
        f.hqs = w.take<float>((long)FFN_PARTS * B * (D / 128));
    }
    f.Z = w.take<float>(P * I);
    f.gpart = f.upart = nullptr;
    if (fp8) {
        f.gpart = w.take<float>(2L * GU_MAXK * P * I);
        f.upart = w.take<float>(2L * GU_MAXK * P * I);
        f.zq = w.take<uint8_t>((long)FFN_PARTS * P * I);
        f.zqs = w.take<float>((long)FFN_PARTS * P * (I / 128));
    }
    f.F = w.take<float>((fp8 ? std::max(DN_NPC, FUSED_DN_NPC) : 1) * P * D);
    // token groups: at most one per active slot plus one per pair
    f.plan.ffn_gmax = (int)(NE + P);
    f.plan.ffn_nrb = I / 128;
    f.sync = fp8 ? w.take<int>((long)f.plan.ffn_gmax * (I / 128 + 1)) : nullptr;
    f.plan.ffn_sync = f.sync;
}

static int run_ffn(const float *h, int B, int D, int I, const int32_t *experts, const float *gates, int ke,
                   const dl_mat *wg, const dl_mat *wu, const dl_mat *wd, int E, int S, const void *resid,
                   int resid_dt, void *out, int out_dt, const FfnWs &f, hipStream_t s, const Marks &mk = Marks(),
                   float *out32 = nullptr, bool plan_ready = false, bool h_split_ready = false, int expert_lo = -1)
{
    const bool f8 = wg->dtype == DL_FP8_E4M3;
    const int NE = E + S;
    const long P = (long)B * (ke + S);
    if (!plan_ready) DL_TRY(launch_plan(experts, B, ke, E, S, f.plan, s, expert_lo));
    // gate/up + SwiGLU -> Z
    GemvArgs g = mat_args(wg);
    g.w2 = (const uint8_t *)(f8 ? wu->w : nullptr);
    g.wsc2 = f8 ? wu->scale : nullptr;
    g.wf2 = f8 ? nullptr : (const float *)wu->w;
    // active experts: at most every routed pick plus the shared experts
    const int na_est = (int)std::min<long>(NE, (long)B * ke + S);
    g.active = f.plan.active;
    g.n_active_dev = f.plan.n_active;
    g.n_active_host = na_est;
    g.tok_off = f.plan.tok_off;
    g.tok_cnt = f.plan.tok_cnt;
    g.max_groups = (B + 15) / 16;
    g.grp_off = f8 ? f.plan.grp_off : nullptr;
    g.pair_act = f.plan.pair_tok;
    g.o_ts = I;
    g.out = f.Z;
    if (f8) {
        if (!h_split_ready)
            DL_TRY(launch_quant(h, B, nullptr, D, f.hq, f.hqs, (long)B * D, (long)B * (D / 128), FFN_PARTS, s));
        g.aq = f.hq; g.asc = f.hqs; g.aq_part = (long)B * D; g.asc_part = (long)B * (D / 128);
        if (!gemv_queue(g, f.queue, GU_NPC, P))
            gemv_flat(g, FFN_PARTS, EPI_SWIGLU, (long)na_est * (I / 32) * g.max_groups, GU_MAXK);
        g.part = f.gpart;
        g.part2 = f.upart;
        g.n_out = P * I;
        g.reduce_in_consumer = true;
    } else {
        g.af = h;
    }
    // down -> F (set up before the gate/up launch: the fused form takes both)
    GemvArgs d = mat_args(wd);
    d.active = f.plan.active;
    d.n_active_dev = f.plan.n_active;
    d.n_active_host = na_est;
    d.tok_off = f.plan.tok_off;
    d.tok_cnt = f.plan.tok_cnt;
    d.max_groups = (B + 15) / 16;
    d.grp_off = f8 ? f.plan.grp_off : nullptr;
    d.pair_act = nullptr;  // Z rows are per pair
    d.o_ts = D;
    d.out = f.F;
    bool fused = false;
    if (f8) {
        d.aq = f.zq; d.asc = f.zqs; d.aq_part = P * I; d.asc_part = P * (I / 128);
        if (gemv_queue(d, f.queue + GEMV_QINTS, DN_NPC, P)) {
            d.part = f.F;
            d.n_out = P * D;
            d.reduce_in_consumer = true;
        }
        fused = DL_FFN_FUSE && f.sync && g.queue && d.queue && g.tiled && d.tiled && g.npc <= 2 && d.npc == 1 &&
                I % 128 == 0 && D % 64 == 0;
    } else {
        d.af = f.Z;
    }
    g_ffn_fused = fused;
    mk.at(5);
    if (fused) {
        FfnFused ff;
        ff.g = g;
        ff.d = d;
        ff.sync = f.sync;
        ff.gmax = f.plan.ffn_gmax;
        ff.d.npc = fused_dn_npc(d.nkb);
        DL_TRY(launch_ffn_fused(ff, s));
        mk.at(6);
        mk.at(7);
    } else {
        DL_TRY(launch_gemv(g, FFN_PARTS, EPI_SWIGLU, f8, s));
        mk.at(6);
        if (f8)
            DL_TRY(launch_swiglu_quant(f.gpart, f.upart, gemv_slots(g), P * I, P, f.plan.n_pairs, I, f.zq, f.zqs,
                                       P * I, P * (I / 128), FFN_PARTS, s));
        mk.at(7);
        DL_TRY(launch_gemv(d, FFN_PARTS, EPI_STORE, f8, s));
    }
    mk.at(8);
    DL_TRY(launch_combine(f.F, fused ? fused_dn_npc(d.nkb) : d.queue ? d.npc : 1, P * D, f.plan, gates, B, D, ke, S, resid, resid_dt, out, out_dt,
                          out32, s));
    mk.at(9);
    return DL_OK;
}

struct LayerWs {
    TopkWs topk;
    int32_t *sel;
    AttnWs attn;
    float *o, *h;
    double *rpart;
    int32_t *experts;
    float *gates;
    FfnWs ffn;
};

static void layer_ws_layout(Ws &w, const dl_layer_desc *d, const dl_pages *pg, const dl_layer_io *io, LayerWs &L,
                            int R = 1, int pool = 1)
{
    const int B = pg->batch * R;  // rows
    topk_ws_layout(w, *pg, L.topk, R, pool);
    L.sel = (io && io->sel) ? io->sel : w.take<int32_t>((long)B * d->top_k);
    L.o = (io && io->o) ? io->o : w.take<float>((long)B * d->n_heads * d->d_v);
    attn_ws_layout(w, B, d->n_heads, d->d_v, d->top_k, d->w_uv.w ? &d->w_uv : nullptr, nullptr, L.attn);
    const int hd = d->w_uv.w ? d->w_uv.rows : d->d_v;
    const long BH = (long)B * d->n_heads;
    L.attn.o = L.o;
    if (d->w_uv.w) {
        if (d->w_uv.dtype == DL_FP8_E4M3) {
            L.attn.oq = w.take<uint8_t>(PROJ_PARTS * BH * d->d_v);
            L.attn.oqs = w.take<float>(PROJ_PARTS * BH * (d->d_v / 128));
        }
        L.attn.u = w.take<float>(BH * hd);
    }
    if (d->w_o.dtype == DL_FP8_E4M3) {
        L.attn.uq = w.take<uint8_t>(PROJ_PARTS * BH * hd);
        L.attn.uqs = w.take<float>(PROJ_PARTS * BH * (hd / 128));
        L.attn.kpart = w.take<float>(2L * MAX_KSPLIT * B * d->w_o.rows);
    }
    L.h = (io && io->h) ? io->h : w.take<float>((long)B * d->D);
    L.rpart = w.take<double>((long)route_chunks(d->D) * B * d->n_routed);
    L.experts = (io && io->experts) ? io->experts : w.take<int32_t>((long)B * d->expert_top_k);
    L.gates = (io && io->gates) ? io->gates : w.take<float>((long)B * d->expert_top_k);
    ffn_ws_layout(w, B, d->D, d->inter, d->expert_top_k, d->n_routed, d->n_shared, d->w_gate.dtype == DL_FP8_E4M3,
                  L.ffn);
}

// local: the stack holds one GPU's share of the routed experts, so a token may pick more experts than it holds
static int check_ffn_shapes(int B, int D, int I, int ke, int E, int S, const dl_mat *wg, const dl_mat *wu,
                            const dl_mat *wd, bool local = false)
{
    if (B < 1 || D < 1 || I < 1) return fail(DL_ERR_SHAPE, "ffn B=%d D=%d I=%d", B, D, I);
    if (D % 4) return fail(DL_ERR_UNSUPPORTED, "ffn hidden size %d (multiple of 4)", D);
    if (D > 65536 || I > 16384) return fail(DL_ERR_UNSUPPORTED, "ffn D=%d (<= 65536) I=%d (<= 16384)", D, I);
    if (E < 1) return fail(DL_ERR_SHAPE, "routed experts %d", E);
    if (ke < 1 || ke > 32 || (!local && ke > E)) return fail(DL_ERR_SHAPE, "expert top_k %d of %d", ke, E);
    if (ke + S > 40) return fail(DL_ERR_UNSUPPORTED, "top_k + shared experts %d (<= 40)", ke + S);
    if (S < 0 || E > 1024 || E + S > 4096) return fail(DL_ERR_SHAPE, "experts %d + %d", E, S);
    if ((long)B * (ke + S) > 16384) return fail(DL_ERR_SHAPE, "B*(top_k+shared) > 16384");
    if ((long)B * ke > 16384) return fail(DL_ERR_SHAPE, "B*top_k > 16384");
    DL_TRY(check_mat(wg, "w_gate", E + S, I, D));
    DL_TRY(check_mat(wu, "w_up", E + S, I, D));
    DL_TRY(check_mat(wd, "w_down", E + S, D, I));
    if (wg->dtype != wu->dtype || wg->dtype != wd->dtype) return fail(DL_ERR_DTYPE, "expert weights mix dtypes");
    if (wg->layout != wu->layout) return fail(DL_ERR_SHAPE, "gate and up weights need the same layout");
    return DL_OK;
}

static int check_attn_shapes(int B, int H, int Dc, int Dv, int top_k, int q_dt, int kv_dt, const float *kv_scale,
                             bool check_scale = true)
{
    if (H < 1 || Dc < 4 || Dv < 4 || Dv > Dc || Dc > 1024) return fail(DL_ERR_SHAPE, "H=%d d_c=%d d_v=%d", H, Dc, Dv);
    if (top_k < 1 || top_k > 4096) return fail(DL_ERR_UNSUPPORTED, "attention top_k %d (1..4096)", top_k);
    if (q_dt != DL_BF16 && q_dt != DL_F32) return fail(DL_ERR_DTYPE, "q dtype %d", q_dt);
    if (kv_dt == DL_FP8_E4M3) {
        if (check_scale && !kv_scale) return fail(DL_ERR_NULL, "FP8 KV needs scales");
    } else if (kv_dt == DL_F32) {
        if (check_scale && kv_scale) return fail(DL_ERR_DTYPE, "fp32 KV takes no scales");
    } else {
        return fail(DL_ERR_DTYPE, "kv dtype %d", kv_dt);
    }
    (void)B;
    return DL_OK;
}

static int check_proj(int H, int Dv, const dl_mat *w_uv, const dl_mat *w_o, int *D_out)
{
    int hd = Dv;
    if (w_uv) {
        if (!w_uv->w) return fail(DL_ERR_NULL, "w_uv");
        DL_TRY(check_mat(w_uv, "w_uv", H, w_uv->rows, Dv));
        hd = w_uv->rows;
    }
    if (!w_o || !w_o->w) return fail(DL_ERR_NULL, "w_o");
    DL_TRY(check_mat(w_o, "w_o", 1, w_o->rows, H * hd));
    if ((long)H * hd > (long)MAX_KSPLIT * GEMV_MAXCHUNK * 128)
        return fail(DL_ERR_UNSUPPORTED, "W_O input width %ld (<= %d)", (long)H * hd, MAX_KSPLIT * GEMV_MAXCHUNK * 128);
    *D_out = w_o->rows;
    return DL_OK;
}

// ------------------------------------------------------------------ the router without a workspace
// Scratch of dl_moe_route_noalloc: the router's fp64 chunk partials live in this file-scope device array (each
// device that runs the library holds its own copy until the process ends).  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in); it takes the device address from hipGetSymbolAddress,
// once per device, and passes that.
static constexpr size_t DL_ROUTE_SCRATCH_BYTES = (size_t)DL_MOE_ROUTE_NOALLOC_MAX_SCRATCH;
static __device__ __align__(256) double scratch[DL_ROUTE_SCRATCH_BYTES / sizeof(double)];

static constexpr int DL_MAX_DEVICES = 64;
static double *g_scratch_ptr[DL_MAX_DEVICES];
static bool g_scratch_init[DL_MAX_DEVICES];
static std::mutex g_scratch_mu;

// The scratch array's device address on the current device (looked up once per device).
static int route_scratch(double **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(DL_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= DL_MAX_DEVICES) return fail(DL_ERR_UNSUPPORTED, "device %d (< %d)", dev, DL_MAX_DEVICES);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_init[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(DL_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = (double *)ptr;
        g_scratch_init[dev] = true;
    }
    *out = g_scratch_ptr[dev];
    return DL_OK;
}

}  // namespace dl

using namespace dl;

extern "C" {

int dl_abi_version(void) { return DL_ABI_VERSION; }
int dl_hip_version(void) { return HIP_VERSION; }

int dl_pack_weights(const dl_mat *src, void *dst, void *stream)
{
    g_err[0] = 0;
    if (!src || !src->w || !dst) return fail(DL_ERR_NULL, "src/dst NULL");
    if (src->dtype != DL_FP8_E4M3) return fail(DL_ERR_DTYPE, "only FP8 weights are tiled");
    if (src->layout != DL_LAYOUT_ROWS) return fail(DL_ERR_SHAPE, "source must be row-major");
    if (src->count < 1 || src->rows < 16 || src->rows % 16 || src->cols < 128 || src->cols % 128)
        return fail(DL_ERR_SHAPE, "pack needs rows %% 16 == 0 and cols %% 128 == 0");
    const long bytes = (long)src->count * src->rows * src->cols;
    const char *a = (const char *)src->w, *b = (const char *)dst;
    if (a < b + bytes && b < a + bytes) return fail(DL_ERR_SHAPE, "src and dst overlap");
    (void)hipGetLastError();
    return launch_pack((const uint8_t *)src->w, (uint8_t *)dst, src->count, src->rows, src->cols, (hipStream_t)stream);
}
int dl_tile_index_keys(const int8_t *src, int8_t *dst, int64_t n_items, int32_t dim, void *stream)
{
    g_err[0] = 0;
    if (!src || !dst) return fail(DL_ERR_NULL, "src/dst NULL");
    if (n_items < 16 || n_items % 16 || dim < 64 || dim > 256 || dim % 64)
        return fail(DL_ERR_SHAPE, "tile keys: n_items %lld (multiple of 16), dim %d (64, 128, 192 or 256)",
                    (long long)n_items, dim);
    const long bytes = (long)n_items * dim;
    const char *a = (const char *)src, *b = (const char *)dst;
    if (a < b + bytes && b < a + bytes) return fail(DL_ERR_SHAPE, "src and dst overlap");
    (void)hipGetLastError();
    return launch_tile_keys(src, dst, n_items, dim, (hipStream_t)stream);
}
const char *dl_last_error(void) { return g_err; }

size_t dl_indexer_topk_rows_workspace(const dl_pages *pages, int32_t rows_per_seq)
{
    if (!pages || rows_per_seq < 1 || rows_per_seq > DL_MAX_ROWS_PER_SEQ) return 0;
    Ws w(nullptr);
    TopkWs t;
    topk_ws_layout(w, *pages, t, rows_per_seq);
    return w.used();
}

size_t dl_indexer_topk_workspace(const dl_pages *pages) { return dl_indexer_topk_rows_workspace(pages, 1); }

size_t dl_indexer_topk_pooled_workspace(const dl_pages *pages, int32_t pool)
{
    if (!pages || pool < 1 || pool > pages->page_size || (pool & (pool - 1))) return 0;
    Ws w(nullptr);
    TopkWs t;
    topk_ws_layout(w, *pages, t, 1, pool);
    return w.used();
}

int dl_indexer_topk_pooled(const dl_pages *pages, int32_t pool, const int8_t *q_idx, const int8_t *pool_keys,
                           int32_t n_heads, int32_t dim, int32_t top_pools, int32_t *sel, int32_t *pool_score,
                           void *ws, size_t ws_bytes, void *stream)
{
    g_err[0] = 0;
    DL_TRY(check_pages(pages));
    if (pool < 1 || pool > pages->page_size || (pool & (pool - 1)))
        return fail(DL_ERR_UNSUPPORTED, "pool %d (power of two, <= page size %d)", pool, pages->page_size);
    if (!q_idx || !pool_keys || !sel) return fail(DL_ERR_NULL, "q_idx/pool_keys/sel NULL");
    DL_TRY(check_indexer(n_heads, dim, top_pools));
    DL_TRY(check_key_tiles(pages, dim, pool));
    if ((long)top_pools * pool > 65536) return fail(DL_ERR_SHAPE, "top_pools * pool %ld (<= 65536)", (long)top_pools * pool);
    DL_TRY(check_ws(ws, ws_bytes, dl_indexer_topk_pooled_workspace(pages, pool)));
    (void)hipGetLastError();
    Ws w(ws);
    TopkWs t;
    topk_ws_layout(w, *pages, t, 1, pool);
    return launch_indexer_topk(*pages, q_idx, pool_keys, n_heads, dim, top_pools, sel, pool_score, t,
                               (hipStream_t)stream, 1, pool);
}

size_t dl_indexer_topk_rows_pooled_workspace(const dl_pages *pages, int32_t rows_per_seq, int32_t pool)
{
    if (!pages || rows_per_seq < 1 || rows_per_seq > DL_MAX_ROWS_PER_SEQ) return 0;
    if (pool < 1 || pool > pages->page_size || (pool & (pool - 1))) return 0;
    Ws w(nullptr);
    TopkWs t;
    topk_ws_layout(w, *pages, t, rows_per_seq, pool);
    return w.used();
}

int dl_indexer_topk_rows_pooled(const dl_pages *pages, int32_t rows_per_seq, int32_t pool, const int8_t *q_idx,
                                const int8_t *pool_keys, int32_t n_heads, int32_t dim, int32_t top_pools,
                                int32_t *sel, int32_t *pool_score, void *ws, size_t ws_bytes, void *stream)
{
    g_err[0] = 0;
    DL_TRY(check_pages(pages));
    const int R = rows_per_seq;
    if (R < 1 || R > DL_MAX_ROWS_PER_SEQ) return fail(DL_ERR_UNSUPPORTED, "rows per sequence %d (1..%d)", R, DL_MAX_ROWS_PER_SEQ);
    if ((long)pages->batch * R > 4096) return fail(DL_ERR_SHAPE, "rows %ld (<= 4096)", (long)pages->batch * R);
    if (pool < 1 || pool > pages->page_size || (pool & (pool - 1)))
        return fail(DL_ERR_UNSUPPORTED, "pool %d (power of two, <= page size %d)", pool, pages->page_size);
    if (!q_idx || !pool_keys || !sel) return fail(DL_ERR_NULL, "q_idx/pool_keys/sel NULL");
    DL_TRY(check_indexer(n_heads, dim, top_pools));
    DL_TRY(check_key_tiles(pages, dim, pool));
    if ((long)top_pools * pool > 65536) return fail(DL_ERR_SHAPE, "top_pools * pool %ld (<= 65536)", (long)top_pools * pool);
    DL_TRY(check_ws(ws, ws_bytes, dl_indexer_topk_rows_pooled_workspace(pages, R, pool)));
    (void)hipGetLastError();
    Ws w(ws);
    TopkWs t;
    topk_ws_layout(w, *pages, t, R, pool);
    return launch_indexer_topk(*pages, q_idx, pool_keys, n_heads, dim, top_pools, sel, pool_score, t,
                               (hipStream_t)stream, R, pool);
}

int dl_kv_append(const dl_pages *pages, const void *latent, int32_t lat_dt, int32_t d_c, const void *key,
                 int32_t key_dt, int32_t idx_dim, float key_scale, uint8_t *kv_pool, float *kv_scale, int8_t *k_pool,
                 void *stream)
{
    g_err[0] = 0;
    DL_TRY(check_pages(pages));
    if (!latent || !kv_pool || !kv_scale) return fail(DL_ERR_NULL, "latent/kv_pool/kv_scale NULL");
    if (idx_dim > 0 && (!key || !k_pool)) return fail(DL_ERR_NULL, "key/k_pool NULL");
    if (d_c < 1 || d_c > 1024 || idx_dim < 0 || idx_dim > 1024)
        return fail(DL_ERR_SHAPE, "append d_c=%d idx_dim=%d", d_c, idx_dim);
    if (lat_dt != DL_F32 && lat_dt != DL_BF16) return fail(DL_ERR_DTYPE, "latent dtype %d", lat_dt);
    if (idx_dim > 0 && key_dt != DL_F32 && key_dt != DL_BF16) return fail(DL_ERR_DTYPE, "key dtype %d", key_dt);
    if (idx_dim > 0 && !(key_scale > 0.f && key_scale <= 3.4028235e38f))
        return fail(DL_ERR_SHAPE, "key_scale %g (finite, > 0)", (double)key_scale);
    if (idx_dim > 0) DL_TRY(check_key_tiles(pages, idx_dim, 1));
    (void)hipGetLastError();
    return launch_kv_append(*pages, latent, lat_dt, d_c, key, key_dt, idx_dim, key_scale, kv_pool, kv_scale, k_pool,
                            (hipStream_t)stream);
}

int dl_indexer_topk_rows(const dl_pages *pages, int32_t rows_per_seq, const int8_t *q_idx, const int8_t *k_pool,
                         int32_t n_heads, int32_t dim, int32_t top_k, int32_t *sel, int32_t *sel_score, void *ws,
                         size_t ws_bytes, void *stream)
{
    g_err[0] = 0;
    DL_TRY(check_pages(pages));
    const int R = rows_per_seq;
    if (R < 1 || R > DL_MAX_ROWS_PER_SEQ) return fail(DL_ERR_UNSUPPORTED, "rows per sequence %d (1..%d)", R, DL_MAX_ROWS_PER_SEQ);
    if ((long)pages->batch * R > 4096) return fail(DL_ERR_SHAPE, "rows %ld (<= 4096)", (long)pages->batch * R);
    if (!q_idx || !k_pool || !sel) return fail(DL_ERR_NULL, "q_idx/k_pool/sel NULL");
    DL_TRY(check_indexer(n_heads, dim, top_k));
    DL_TRY(check_key_tiles(pages, dim, 1));
    DL_TRY(check_ws(ws, ws_bytes, dl_indexer_topk_rows_workspace(pages, R)));
    (void)hipGetLastError();
    Ws w(ws);
    TopkWs t;
    topk_ws_layout(w, *pages, t, R);
    return launch_indexer_topk(*pages, q_idx, k_pool, n_heads, dim, top_k, sel, sel_score, t, (hipStream_t)stream, R);
}

int dl_indexer_topk(const dl_pages *pages, const int8_t *q_idx, const int8_t *k_pool, int32_t n_heads, int32_t dim,
                    int32_t top_k, int32_t *sel, int32_t *sel_score, void *ws, size_t ws_bytes, void *stream)
{
    return dl_indexer_topk_rows(pages, 1, q_idx, k_pool, n_heads, dim, top_k, sel, sel_score, ws, ws_bytes, stream);
}

size_t dl_sparse_attn_workspace(int32_t batch, int32_t n_heads, int32_t d_v, int32_t top_k, const dl_mat *w_uv,
                                const dl_mat *w_o)
{
    Ws w(nullptr);
    AttnWs a;
    attn_ws_layout(w, batch, n_heads, d_v, top_k, w_uv, w_o, a);
    return w.used();
}

int dl_sparse_attn_decode(const dl_pages *pages, const void *q, int32_t q_dt, const void *kv_pool,
                          const float *kv_scale, int32_t kv_dt, int32_t n_heads, int32_t d_c, int32_t d_v,
                          float sm_scale, const int32_t *sel, int32_t top_k, const dl_mat *w_uv, const dl_mat *w_o,
                          const void *residual, int32_t res_dt, float *out, void *ws, size_t ws_bytes, void *stream)
{
    g_err[0] = 0;
    DL_TRY(check_pages(pages));
    if (!q || !kv_pool || !sel || !out) return fail(DL_ERR_NULL, "q/kv_pool/sel/out NULL");
    DL_TRY(check_attn_shapes(pages->batch, n_heads, d_c, d_v, top_k, q_dt, kv_dt, kv_scale));
    if (w_uv && !w_o) return fail(DL_ERR_SHAPE, "w_uv given without w_o");
    int D = 0;
    if (w_o) {
        DL_TRY(check_proj(n_heads, d_v, w_uv, w_o, &D));
        if (!residual) return fail(DL_ERR_NULL, "residual required with w_o");
        if (res_dt != DL_BF16 && res_dt != DL_F32) return fail(DL_ERR_DTYPE, "residual dtype %d", res_dt);
    }
    DL_TRY(check_ws(ws, ws_bytes, dl_sparse_attn_workspace(pages->batch, n_heads, d_v, top_k, w_uv, w_o)));
    (void)hipGetLastError();
    hipStream_t s = (hipStream_t)stream;
    Ws w(ws);
    AttnWs a;
    attn_ws_layout(w, pages->batch, n_heads, d_v, top_k, w_uv, w_o, a);
    float *o = w_o ? a.o : out;
    return run_attn_proj(*pages, q, q_dt, kv_pool, kv_scale, kv_dt, n_heads, d_c, d_v, sm_scale, sel, top_k, w_uv, w_o,
                         residual, res_dt, o, out, a, nullptr, nullptr, nullptr, s, Marks(), 1, !w_o);
}

size_t dl_moe_route_workspace(int32_t B, int32_t D, int32_t n_experts)
{
    Ws w(nullptr);
    w.take<double>((long)route_chunks(D) * B * n_experts);
    return w.used();
}

int dl_moe_route(const float *h, int32_t B, int32_t D, const float *w_r, const float *bias, int32_t n_experts,
                 int32_t top_k, int32_t *experts, float *gates, float *logits, void *ws, size_t ws_bytes, void *stream)
{
    g_err[0] = 0;
    if (!h || !w_r || !experts || !gates) return fail(DL_ERR_NULL, "h/w_r/experts/gates NULL");
    if (B < 1 || B > 65536 || D < 1) return fail(DL_ERR_SHAPE, "B=%d D=%d", B, D);
    if (top_k < 1 || top_k > 32 || n_experts < top_k || n_experts > 1024)
        return fail(DL_ERR_SHAPE, "top_k %d of %d experts", top_k, n_experts);
    if (D % 4 || D > 16384) return fail(DL_ERR_UNSUPPORTED, "router hidden size %d (multiple of 4, <= 16384)", D);
    DL_TRY(check_ws(ws, ws_bytes, dl_moe_route_workspace(B, D, n_experts)));
    (void)hipGetLastError();
    Ws w(ws);
    double *part = w.take<double>((long)route_chunks(D) * B * n_experts);
    return launch_route(h, B, D, w_r, bias, n_experts, top_k, experts, gates, logits, part, (hipStream_t)stream);
}


int dl_moe_route_noalloc(const float *h, int32_t B, int32_t D, const float *w_r, const float *bias, int32_t n_experts,
                         int32_t top_k, int32_t *experts, float *gates, float *logits, void *stream)
{
    g_err[0] = 0;
    if (!h || !w_r || !experts || !gates) return fail(DL_ERR_NULL, "h/w_r/experts/gates NULL");
    if (B < 1 || B > 65536 || D < 1) return fail(DL_ERR_SHAPE, "B=%d D=%d", B, D);
    if (top_k < 1 || top_k > 32 || n_experts < top_k || n_experts > 1024)
        return fail(DL_ERR_SHAPE, "top_k %d of %d experts", top_k, n_experts);
    if (D % 4 || D > 16384) return fail(DL_ERR_UNSUPPORTED, "router hidden size %d (multiple of 4, <= 16384)", D);
    const size_t need = (size_t)route_chunks(D) * B * n_experts * sizeof(double);
    if (need > DL_ROUTE_SCRATCH_BYTES)
        return fail(DL_ERR_SHAPE, "router scratch %zu bytes > %zu (chunks of 1,024 features x B x experts x 8 B)",
                    need, DL_ROUTE_SCRATCH_BYTES);
    double *part = nullptr;
    DL_TRY(route_scratch(&part));
    (void)hipGetLastError();
    return launch_route(h, B, D, w_r, bias, n_experts, top_k, experts, gates, logits, part, (hipStream_t)stream);
}

size_t dl_moe_ffn_workspace(int32_t B, int32_t D, int32_t inter, int32_t top_k, int32_t n_routed, int32_t n_shared)
{
    Ws w(nullptr);
    FfnWs f;
    ffn_ws_layout(w, B, D, inter, top_k, n_routed, n_shared, true, f);
    return w.used();
}

int dl_moe_ffn(const float *h, int32_t B, int32_t D, int32_t inter, const int32_t *experts, const float *gates,
               int32_t top_k, const dl_mat *w_gate, const dl_mat *w_up, const dl_mat *w_down, int32_t n_routed,
               int32_t n_shared, const float *residual, void *out, int32_t out_dt, void *ws, size_t ws_bytes,
               void *stream)
{
    g_err[0] = 0;
    if (!h || !experts || !gates || !out) return fail(DL_ERR_NULL, "h/experts/gates/out NULL");
    DL_TRY(check_ffn_shapes(B, D, inter, top_k, n_routed, n_shared, w_gate, w_up, w_down));
    if (out_dt != DL_F32 && out_dt != DL_BF16) return fail(DL_ERR_DTYPE, "out dtype %d", out_dt);
    DL_TRY(check_ws(ws, ws_bytes, dl_moe_ffn_workspace(B, D, inter, top_k, n_routed, n_shared)));
    (void)hipGetLastError();
    Ws w(ws);
    FfnWs f;
    ffn_ws_layout(w, B, D, inter, top_k, n_routed, n_shared, w_gate->dtype == DL_FP8_E4M3, f);
    return run_ffn(h, B, D, inter, experts, gates, top_k, w_gate, w_up, w_down, n_routed, n_shared, residual, DL_F32,
                   out, out_dt, f, (hipStream_t)stream);
}

int dl_moe_ffn_ep(const float *h, int32_t B, int32_t D, int32_t inter, const int32_t *experts, const float *gates,
                  int32_t top_k, int32_t expert_lo, const dl_mat *w_gate, const dl_mat *w_up, const dl_mat *w_down,
                  int32_t n_local, int32_t n_shared, const float *residual, void *out, int32_t out_dt, void *ws,
                  size_t ws_bytes, void *stream)
{
    g_err[0] = 0;
    if (!h || !experts || !gates || !out) return fail(DL_ERR_NULL, "h/experts/gates/out NULL");
    if (expert_lo < 0) return fail(DL_ERR_SHAPE, "expert_lo %d", expert_lo);
    DL_TRY(check_ffn_shapes(B, D, inter, top_k, n_local, n_shared, w_gate, w_up, w_down, true));
    if (out_dt != DL_F32 && out_dt != DL_BF16) return fail(DL_ERR_DTYPE, "out dtype %d", out_dt);
    DL_TRY(check_ws(ws, ws_bytes, dl_moe_ffn_workspace(B, D, inter, top_k, n_local, n_shared)));
    (void)hipGetLastError();
    Ws w(ws);
    FfnWs f;
    ffn_ws_layout(w, B, D, inter, top_k, n_local, n_shared, w_gate->dtype == DL_FP8_E4M3, f);
    return run_ffn(h, B, D, inter, experts, gates, top_k, w_gate, w_up, w_down, n_local, n_shared, residual, DL_F32,
                   out, out_dt, f, (hipStream_t)stream, Marks(), nullptr, false, false, expert_lo);
}

static int check_layer(const dl_layer_desc *d, const dl_pages *pg, int R = 1)
{
    if (!d) return fail(DL_ERR_NULL, "desc NULL");
    DL_TRY(check_pages(pg));
    if ((long)pg->batch * R > 4096) return fail(DL_ERR_SHAPE, "rows %ld (<= 4096)", (long)pg->batch * R);
    DL_TRY(check_indexer(d->idx_heads, d->idx_dim, d->top_k));
    DL_TRY(check_attn_shapes(pg->batch * R, d->n_heads, d->d_c, d->d_v, d->top_k, d->q_dt, d->kv_dt, nullptr, false));
    int D = 0;
    DL_TRY(check_proj(d->n_heads, d->d_v, d->w_uv.w ? &d->w_uv : nullptr, &d->w_o, &D));
    if (D != d->D) return fail(DL_ERR_SHAPE, "w_o rows %d != D %d", D, d->D);
    if (!d->w_r) return fail(DL_ERR_NULL, "w_r");
    DL_TRY(check_ffn_shapes(pg->batch * R, d->D, d->inter, d->expert_top_k, d->n_routed, d->n_shared, &d->w_gate,
                            &d->w_up, &d->w_down));
    if (d->out_dt != DL_F32 && d->out_dt != DL_BF16) return fail(DL_ERR_DTYPE, "out dtype %d", d->out_dt);
    if (d->D % 4 || d->D > 16384) return fail(DL_ERR_UNSUPPORTED, "hidden size %d (multiple of 4, <= 16384)", d->D);
    return DL_OK;
}

static bool pool_ok(const dl_pages *pg, int pool)
{
    return pool >= 1 && pool <= pg->page_size && !(pool & (pool - 1));
}

// Workspace of the step with R rows per sequence and selection by pools of `pool` positions.
static size_t layer_workspace(const dl_layer_desc *desc, const dl_pages *pages, int R, int pool)
{
    if (!desc || !pages || R < 1 || R > DL_MAX_ROWS_PER_SEQ || !pool_ok(pages, pool)) return 0;
    Ws w(nullptr);
    LayerWs L;
    layer_ws_layout(w, desc, pages, nullptr, L, R, pool);
    return w.used();
}

size_t dl_layer_workspace_rows(const dl_layer_desc *desc, const dl_pages *pages, int32_t rows_per_seq)
{
    return layer_workspace(desc, pages, rows_per_seq, 1);
}

size_t dl_layer_workspace(const dl_layer_desc *desc, const dl_pages *pages)
{
    return layer_workspace(desc, pages, 1, 1);
}

size_t dl_layer_workspace_pooled(const dl_layer_desc *desc, const dl_pages *pages, int32_t pool)
{
    return layer_workspace(desc, pages, 1, pool);
}

static int layer_step(const dl_layer_desc *d, const dl_layer_io *io, int R, int pool, void *ws, size_t ws_bytes,
                      void *stream)
{
    g_err[0] = 0;
    if (!io) return fail(DL_ERR_NULL, "io NULL");
    if (R < 1 || R > DL_MAX_ROWS_PER_SEQ) return fail(DL_ERR_UNSUPPORTED, "rows per sequence %d (1..%d)", R, DL_MAX_ROWS_PER_SEQ);
    DL_TRY(check_layer(d, &io->pages, R));
    if (!pool_ok(&io->pages, pool))
        return fail(DL_ERR_UNSUPPORTED, "pool %d (power of two, <= page size %d)", pool, io->pages.page_size);
    if (d->top_k % pool) return fail(DL_ERR_SHAPE, "top_k %d is not a multiple of pool %d", d->top_k, pool);
    DL_TRY(check_key_tiles(&io->pages, d->idx_dim, pool));
    if (d->kv_dt == DL_FP8_E4M3 && !io->kv_scale) return fail(DL_ERR_NULL, "FP8 KV needs kv_scale");
    if (d->kv_dt == DL_F32 && io->kv_scale) return fail(DL_ERR_DTYPE, "fp32 KV takes no kv_scale");
    if (!io->x || !io->q || !io->q_idx || !io->kv_pool || !io->k_pool || !io->y) return fail(DL_ERR_NULL, "io tensor NULL");
    DL_TRY(check_ws(ws, ws_bytes, layer_workspace(d, &io->pages, R, pool)));
    (void)hipGetLastError();
    hipStream_t s = (hipStream_t)stream;
    const dl_pages &pg = io->pages;
    const int B = pg.batch * R;  // rows: every row is a token of the step from here on
    Ws w(ws);
    LayerWs L;
    layer_ws_layout(w, d, &pg, io, L, R, pool);
    Marks mk;
    DL_TRY(marks_begin(mk, s));
    const dl_mat *wuv = d->w_uv.w ? &d->w_uv : nullptr;
    const bool f8_ffn = d->w_gate.dtype == DL_FP8_E4M3;
    const bool fuse_route = route_plan_ok(d->n_routed, d->expert_top_k, B);
    mk.at(0);
    DL_TRY(launch_indexer_topk(pg, io->q_idx, io->k_pool, d->idx_heads, d->idx_dim, d->top_k / pool, L.sel, nullptr,
                               L.topk, s, R, pool));
    mk.at(1);
    bool h_split = false;
    DL_TRY(run_attn_proj(pg, io->q, d->q_dt, io->kv_pool, io->kv_scale, d->kv_dt, d->n_heads, d->d_c, d->d_v,
                         d->sm_scale, L.sel, d->top_k, wuv, &d->w_o, io->x, d->q_dt, L.o, L.h, L.attn,
                         f8_ffn ? L.ffn.hq : nullptr, L.ffn.hqs, &h_split, s, mk, R, io->o != nullptr));
    mk.at(3);
    if (fuse_route) {
        DL_TRY(launch_route_partial(L.h, B, d->D, d->w_r, d->n_routed, L.rpart, s));
        DL_TRY(launch_route_plan(L.rpart, B, d->D, d->r_bias, d->n_routed, d->expert_top_k, d->n_shared, L.experts,
                                 L.gates, io->logits, &L.ffn.plan, s));
    } else {
        DL_TRY(launch_route(L.h, B, d->D, d->w_r, d->r_bias, d->n_routed, d->expert_top_k, L.experts, L.gates,
                            io->logits, L.rpart, s));
    }
    mk.at(4);
    return run_ffn(L.h, B, d->D, d->inter, L.experts, L.gates, d->expert_top_k, &d->w_gate, &d->w_up, &d->w_down,
                   d->n_routed, d->n_shared, L.h, DL_F32, io->y, d->out_dt, L.ffn, s, mk, io->y32, fuse_route, h_split);
}

int dl_layer_step_rows(const dl_layer_desc *d, const dl_layer_io *io, int32_t rows_per_seq, void *ws, size_t ws_bytes,
                       void *stream)
{
    return layer_step(d, io, rows_per_seq, 1, ws, ws_bytes, stream);
}

int dl_layer_step_pooled(const dl_layer_desc *d, const dl_layer_io *io, int32_t pool, void *ws, size_t ws_bytes,
                         void *stream)
{
    return layer_step(d, io, 1, pool, ws, ws_bytes, stream);
}

size_t dl_layer_workspace_rows_pooled(const dl_layer_desc *desc, const dl_pages *pages, int32_t rows_per_seq,
                                      int32_t pool)
{
    return layer_workspace(desc, pages, rows_per_seq, pool);
}

int dl_layer_step_rows_pooled(const dl_layer_desc *d, const dl_layer_io *io, int32_t rows_per_seq, int32_t pool,
                              void *ws, size_t ws_bytes, void *stream)
{
    return layer_step(d, io, rows_per_seq, pool, ws, ws_bytes, stream);
}

int dl_layer_step(const dl_layer_desc *d, const dl_layer_io *io, void *ws, size_t ws_bytes, void *stream)
{
    return layer_step(d, io, 1, 1, ws, ws_bytes, stream);
}

int dl_probe_read(const void *buf, size_t bytes, size_t *bytes_read, void *stream)
{
    g_err[0] = 0;
    if (!buf) return fail(DL_ERR_NULL, "probe_read: buffer NULL");
    (void)hipGetLastError();
    return launch_probe_read(buf, bytes, bytes_read, (hipStream_t)stream);
}

int dl_probe_null(int32_t n_kernels, int32_t blocks, void *stream)
{
    g_err[0] = 0;
    if (n_kernels < 1 || n_kernels > 1024 || blocks < 1 || blocks > 65536)
        return fail(DL_ERR_SHAPE, "probe_null: %d kernels of %d workgroups (1..1024, 1..65536)", n_kernels, blocks);
    (void)hipGetLastError();
    return launch_probe_null(n_kernels, blocks, (hipStream_t)stream);
}

int dl_profile_enable(int on)
{
    g_err[0] = 0;
    g_prof = on != 0;
    if (!g_prof) {
        for (int i = 0; i < g_npend; i++)
            for (int j = 0; j <= DL_N_PHASES; j++) (void)hipEventDestroy(g_pend[i].ev[j]);
        for (int i = 0; i < g_nfree; i++)
            for (int j = 0; j <= DL_N_PHASES; j++) (void)hipEventDestroy(g_free[i].ev[j]);
        g_npend = g_nfree = 0;
    }
    return DL_OK;
}

int dl_profile_ffn_fused(void) { return g_ffn_fused; }

int dl_profile_read(double *ms_sum, int64_t *steps)
{
    g_err[0] = 0;
    if (!ms_sum || !steps) return fail(DL_ERR_NULL, "ms_sum/steps NULL");
    for (int j = 0; j < DL_N_PHASES; j++) ms_sum[j] = 0.0;
    *steps = g_npend;
    for (int i = 0; i < g_npend; i++) {
        StepMarks &m = g_pend[i];
        if (hipEventSynchronize(m.ev[DL_N_PHASES]) != hipSuccess) return fail(DL_ERR_HIP, "profile: sync");
        for (int j = 0; j < DL_N_PHASES; j++) {
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, m.ev[j], m.ev[j + 1]) != hipSuccess) return fail(DL_ERR_HIP, "profile: elapsed");
            ms_sum[j] += ms;
        }
        if (g_nfree == g_fcap) {
            g_fcap = g_fcap ? 2 * g_fcap : 64;
            g_free = (StepMarks *)realloc(g_free, sizeof(StepMarks) * g_fcap);
            if (!g_free) return fail(DL_ERR_HIP, "profile: out of host memory");
        }
        g_free[g_nfree++] = m;
    }
    g_npend = 0;
    return DL_OK;
}

}  // extern "C"
