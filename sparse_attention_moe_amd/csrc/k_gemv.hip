// Weight-streaming GEMV engine for FP8 block-scaled weights (W_UV, W_O, expert gate/up/down).
//
// The weights are OCP e4m3fn codes with one fp32 scale per 128 x 128 block ("FP8 weights with
// 128 x 128 block scales", Introducing Kiln, "How was Kiln measured against vLLM on H200?").  Kiln
// aligned each block with a kernel tile so one scale serves the tile ("Expert parallelism without an
// all-to-all", per-tile dequantisation).  Here a wave owns 16 weight rows and walks K in 128-wide
// blocks: each block is exactly one v_mfma_f32_16x16x128_f8f6f4 on the raw codes, and the block's
// partial sums are scaled once — the codes are never decoded on the vector units.
//
// The activations enter as NS FP8 parts: part 0 is the value rounded to e4m3 with a per-(row, 128-block)
// scale, part s the remainder of parts < s with its own scale.  Two parts carry about 10 significant bits,
// four about 16, so the projections ahead of the router keep near-fp32 accuracy while the expert FFN uses
// two.  The parts share the 16 columns (the N side) of one instruction: a token group is 16 / NS tokens x NS
// parts, each lane scales its column by its own part's scale, and the parts of a token are added once at
// the end of an item (DPP within the 16-lane row).  An expert with one or two tokens thus costs one
// instruction, one activation load and one scale load per weight tile and K block.
//
// Work items are (active matrix, 16-row tile, token group); matrices and token groups come from a
// device-side plan in the MoE (experts with no token are simply absent: the MoE tile skip of Kiln's
// "What moved the number ..." section).  Every weight byte is read once with 16-byte loads.
#include "dl_common.h"
#include "dl_internal.h"

namespace dl {

__device__ __forceinline__ v8i ld32(const uint8_t *p)
{
    v4i a = *(const v4i *)p, b = *(const v4i *)(p + 16);
    return v8i{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ v4f mfma_fp8(v8i a, v8i b)
{
    v4f z = {0.f, 0.f, 0.f, 0.f};
    // cbsz = blgp = 0: both operands e4m3; no MX scaling.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// A ticket from a queue counter into tk (lane 0; the other lanes keep theirs): the counter's old value, waited for
// only where it is read.  The address passes through a register the compiler cannot see into: with a uniform address
// it rewrites the atomic into a wave-wide form and waits for its result at once, and that wait (in issue order)
// also drains the weight loads issued just before it.
__device__ __forceinline__ void q_take(int *qc, int lane, int &tk)
{
    __attribute__((address_space(1))) int *p = (__attribute__((address_space(1))) int *)qc;
    asm volatile("" : "+v"(p));
    if (lane == 0) tk = __hip_atomic_fetch_add(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The NS FP8 parts of a wave's 128 values (two per lane, at element e of the row): part 0 is the value rounded to
// e4m3 with an amax / 448 scale over the 128, part s the remainder of parts < s with its own scale.  Codes go to
// q + s * q_part + e, scales to sc + s * sc_part + si; DEV: device-scope stores.
template <int NS, bool DEV>
__device__ __forceinline__ void split_store(float r0, float r1, uint8_t *q, float *sc, long q_part, long sc_part, long e,
                                            long si, int lane)
{
#pragma unroll
    for (int s = 0; s < NS; s++) {
        const float amax = wave_max(fmaxf(fabsf(r0), fabsf(r1)));
        const float scale = amax > 0.f ? amax * (1.0f / 448.0f) : 1.0f;
        const float inv = 1.0f / scale;
        const float c0 = fminf(fmaxf(r0 * inv, -448.f), 448.f);
        const float c1 = fminf(fmaxf(r1 * inv, -448.f), 448.f);
        const uint32_t code = f32x2_to_fp8(c0, c1);
        uint16_t *qp = (uint16_t *)(q + s * q_part + e);
        if (DEV) st_dev(qp, (uint16_t)code);
        else *qp = (uint16_t)code;
        if (lane == 0) {
            if (DEV) st_dev(sc + s * sc_part + si, scale);
            else sc[s * sc_part + si] = scale;
        }
        const v2f d = fp8x2_lo(code);
        r0 -= d.x * scale;
        r1 -= d.y * scale;
    }
}

// Work: units (active matrix u, RT*16-row tile, group of 16 tokens), numbered with the token group fastest,
// then the tile, then u; a unit's K range is nkb steps of one 128-wide block, cut into chunks of kchunk
// blocks.  The steps of all units form one sequence.  Without `flat` each wave owns a contiguous share of whole
// (unit, chunk) items; with `flat` each wave owns an equal share of steps (at least kchunk), so a chunk may be
// split between two neighbouring waves: the first writes partial slot 2 kc, the second 2 kc + 1, and a chunk
// done by one wave zero-fills 2 kc + 1.  Either way consecutive segments of a wave mostly share the matrix
// and token group (no new metadata) and the load pipeline runs on across segment boundaries.
//
// With a work queue the waves take pieces instead of fixed shares.  Every unit's K range is cut at the same
// npc - 1 points (halving: the first piece is half the range, the next a quarter, ..., the last two equal; one
// piece is the whole range), and piece j of every unit writes partial slot j, so the sums do not depend on which
// wave ran a piece.  Pieces are numbered piece-major (all units' first pieces, then all units' second ones, ...),
// so the long pieces go first and the short ones last.  The pieces are dealt into GEMV_QPOOLS pools in rounds of
// GEMV_QROUND: pool p takes m_p slots of every round, spread evenly over it (equal shares give piece i to pool
// i % GEMV_QPOOLS), so each pool keeps the long-first order and the pools advance through the weights side by
// side; the shares come from the pools' measured rates in the previous launch (set by the plan).  Workgroup b
// draws from pool b % GEMV_QPOOLS, which with the round-robin dispatch over the eight XCDs is its XCD's own.  Each wave's first piece of its pool is fixed by its index, each further one comes from the
// pool's device counter, drawn right after the current piece's first loads so that the atomic's round trip stays
// off the wait for any load issued before it.  A counter serves one atomic at a
// time: a single one for the whole device made the waves queue for their tickets (and a wave's loads complete
// in order behind its atomic).  Balance between the pools comes from their shares: moving drained pools' waves
// on to the others evened the XCDs out but piled them onto the remaining counters, and both passes got slower.
template <bool SW, int RT>
struct Stage {
    v8i A[RT], A2[RT];
    v8i Bv;
    float as;
};

// Weight scales of the segment's K range (at most 128 blocks): lane j holds the scale of K-block kb0 + j in wsv
// and of kb0 + 64 + j in wsvB; the compute loop reads them with readlane, so no scale is loaded per K-block.
struct Ctx {
    int u, m, cnt, off, t0, r0, kc, kb0, kb1, piece, whole;
    bool valid, tv;
    int tt;
    const uint8_t *wp, *wp2, *ap;
    const float *wsp, *wsp2, *asp;
    float wsv, wsv2, wsvB, wsvB2;
};

// Two 16-byte halves of an operand: at p and p + gap.
__device__ __forceinline__ v8i ld16x2(const uint8_t *p, int gap)
{
    v4i a = *(const v4i *)p, b = *(const v4i *)(p + gap);
    return v8i{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// Weight bytes are read once per step: streaming (non-temporal) loads keep them from displacing the
// step's small intermediates in the caches.
__device__ __forceinline__ v8i ldw16x2(const uint8_t *p, int gap)
{
    v4i a = __builtin_nontemporal_load((const v4i *)p), b = __builtin_nontemporal_load((const v4i *)(p + gap));
    return v8i{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Operand bytes of lane l = (ln, lg): row ln of the tile, K bytes {lg*16 .. +16} and {64 + lg*16 .. +16}
// of the 128-wide block.  Row-major weights: two loads 64 B apart in the row; tiled weights: 16 B at
// l*16 and 1024 + l*16 of the tile's 2 KB.  The activations use the same K assignment.
template <bool SW, int RT, bool TL, bool COH = false>
__device__ __forceinline__ void load_stage(Stage<SW, RT> &st, const Ctx &c, long cols, int kb)
{
#pragma unroll
    for (int r = 0; r < RT; r++) {
        if (TL) {
            // consecutive 16-row tiles are cols/128 blocks of 2 KB apart
            const uint8_t *t = c.wp + (long)r * (cols / 128) * 2048 + (long)kb * 2048;
            st.A[r] = ldw16x2(t, 1024);
            if (SW) st.A2[r] = ldw16x2(c.wp2 + (long)r * (cols / 128) * 2048 + (long)kb * 2048, 1024);
        } else {
            st.A[r] = ldw16x2(c.wp + r * 16 * cols + kb * 128, 64);
            if (SW) st.A2[r] = ldw16x2(c.wp2 + r * 16 * cols + kb * 128, 64);
        }
    }
    // lanes of empty token slots read a valid row of the group (their column is scaled by 0); every lane
    // loads, so each step issues the same loads
    st.Bv = ld16x2(c.ap + kb * 128, 64);
    st.as = COH ? ld_dev(c.asp + kb) : c.asp[kb];
}

// Segment (steps [s, e) of one unit's chunk) -> context.  Units are (u, tile, g) with g fastest; in plan mode
// matrix slot u has goff[u+1] - goff[u] token groups (goff in LDS), else every matrix has `groups`.  Reuses
// `prev` (same matrix and token group) when possible: then no memory is read.
template <int NS, int RT, bool SW, bool TL>
__device__ __forceinline__ void make_ctx(const GemvArgs &a, long s, long e, int groups, int tiles, int n_act,
                                         const int *goff, const Ctx *prev, Ctx &c)
{
    constexpr int TPG = 16 / NS;
    const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
    const int unit = (int)(s / a.nkb);
    const int kb = (int)(s - (long)unit * a.nkb);
    const int kc = kb / a.kchunk;
    int u, tile, g;
    if (goff) {
        int lo = 0, hi = n_act - 1;  // last slot with tiles * goff[slot] <= unit
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tiles * goff[mid] <= unit) lo = mid; else hi = mid - 1;
        }
        u = lo;
        const int gc = goff[u + 1] - goff[u], r = unit - tiles * goff[u];
        tile = r / gc;
        g = r - tile * gc;
    } else {
        g = unit % groups;
        tile = (unit / groups) % tiles;
        u = unit / groups / tiles;
    }
    if (prev && prev->u == u && prev->t0 == g * TPG) {
        c = *prev;
    } else {
        c.u = u;
        c.m = __builtin_amdgcn_readfirstlane(a.active ? a.active[u] : u);
        c.cnt = a.tok_cnt ? a.tok_cnt[u] : a.ntok_host;
        c.off = a.tok_cnt ? a.tok_off[u] : 0;
        c.t0 = g * TPG;
        c.valid = c.t0 < c.cnt;
        // column ln = token t0 + ln % TPG, part ln / TPG
        c.tt = c.t0 + ln % TPG;
        c.tv = c.tt < c.cnt;
        const int ts = c.tv ? c.tt : c.t0;
        const long arow = !c.valid ? 0
                          : a.pair_act ? a.pair_act[c.off + ts]
                          : a.tok_cnt  ? (long)(c.off + ts)
                                       : (long)ts * a.a_ts + (long)c.m * a.a_ms;
        const int sp = ln / TPG;
        c.ap = a.aq + sp * a.aq_part + arow * a.cols + lg * 16;
        c.asp = a.asc + sp * a.asc_part + arow * a.nkb;
    }
    const int kb_end = min(a.nkb, (kc + 1) * a.kchunk);
    c.kc = kc;
    c.kb0 = kb;
    c.kb1 = kb + (int)(e - s);
    c.piece = kb != kc * a.kchunk;
    c.whole = !c.piece && c.kb1 == kb_end;
    c.r0 = tile * 16 * RT;
    const long wrow = TL ? (long)c.m * a.mat_elems + (long)(c.r0 / 16) * a.nkb * 2048 + lane * 16
                         : (long)c.m * a.mat_elems + (long)(c.r0 + ln) * a.cols + lg * 16;
    c.wp = a.w + wrow;
    c.wp2 = SW ? a.w2 + wrow : nullptr;
    const long sbase = ((long)c.m * a.nrb + (c.r0 >> 7)) * a.nkb;
    c.wsp = a.wsc + sbase;
    c.wsp2 = SW ? a.wsc2 + sbase : nullptr;
    // every lane loads (indices clamped to the segment), so no load here depends on the lane
    const int last = c.kb1 - c.kb0 - 1;
    const int i0 = c.kb0 + min(lane, last), i1 = c.kb0 + min(lane + 64, last);
    c.wsv = c.wsp[i0];
    c.wsvB = c.wsp[i1];
    c.wsv2 = SW ? c.wsp2[i0] : 0.f;
    c.wsvB2 = SW ? c.wsp2[i1] : 0.f;
}

__device__ __forceinline__ float lane_f(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }

// Sum over the NS part columns of a token (lanes ln, ln + 16/NS, ... of the 16-lane row), on the DPP network.
__device__ __forceinline__ float row_ror(float v, int n8)
{
    return n8 ? __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false))
              : __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false));
}
template <int NS>
__device__ __forceinline__ v4f sum_parts(v4f v)
{
#pragma unroll
    for (int i = 0; i < 4; i++) {
        if (NS == 4) v[i] += row_ror(v[i], 0);
        if (NS >= 2) v[i] += row_ror(v[i], 1);
    }
    return v;
}

template <int NS, int EPI, int RT, bool TL>
__global__ __launch_bounds__(256, (EPI == EPI_SWIGLU || NS == 4) ? 2 : 3) void k_gemv_fp8(GemvArgs a)
{
    constexpr bool SW = EPI == EPI_SWIGLU;
    constexpr int TPG = 16 / NS;  // tokens per group (the parts share the 16 columns)
    __shared__ int s_goff[GEMV_MAXMAT + 1];
    const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nwaves = gridDim.x * 4;
    const int n_act = a.n_active_dev ? *a.n_active_dev : a.n_active_host;
    const int groups = (a.ntok_host + TPG - 1) / TPG;  // uniform mode
    const int tiles = a.rows / (16 * RT);
    // queue: pieces, pool, tickets handed out by index, the pool's counter, the next ticket (lane 0), this slot,
    // the pools' shares of a round
    int qtot = 0, npool = 1, pool = 0, qbase = 0, qtk = 0, qslot = 0;
    int qm[GEMV_QPOOLS];
    int *qc = nullptr;
    if (a.queue) {
        npool = min((int)gridDim.x, GEMV_QPOOLS);
        pool = blockIdx.x % npool;
        qc = a.queue + pool * GEMV_QSTRIDE;
        qbase = 4 * (((int)gridDim.x - pool + npool - 1) / npool);  // the pool's waves
        gemv_shares_read(a.queue, qm);
        if (blockIdx.x < npool && threadIdx.x == 0)
            *(unsigned long long *)(qc + 2) = __builtin_amdgcn_s_memrealtime();
    }
    // a wave of the pool is done: the last one records the time
    auto q_done = [&]() {
        if (a.queue && lane == 0 && atomicAdd(qc + 1, 1) == qbase - 1)
            *(unsigned long long *)(qc + 4) = __builtin_amdgcn_s_memrealtime();
    };
    long units;
    if (a.grp_off) {
        for (int i = threadIdx.x; i <= n_act; i += 256) s_goff[i] = a.grp_off[i];
        __syncthreads();
        units = (long)tiles * s_goff[n_act];
    } else {
        units = (long)n_act * tiles * groups;
    }
    const int *goff = a.grp_off ? s_goff : nullptr;
    const long S = units * a.nkb;  // steps of all units
    long s0, s1;
    // ticket t of the wave's pool -> piece: its (t mod m_pool)-th slot of round t / m_pool
    auto qindex = [&](int t) {
        if (npool < GEMV_QPOOLS) return (long)t * npool + pool;
        const int n = qm[pool];
        return (long)(t / n) * GEMV_QROUND + gemv_slot_pos(qm, pool, t % n);
    };
    // piece t -> steps [s0, s1) of unit t % units, K-blocks [nkb - nkb >> j, nkb - nkb >> (j + 1)) with j = t / units
    auto qpiece = [&](int t, long &ps, long &pe, int &slot) {
        const int j = (int)(t / units);
        const long u0 = (t - (long)j * units) * a.nkb;
        ps = u0 + a.nkb - (a.nkb >> j);
        pe = u0 + (j + 1 >= a.npc ? a.nkb : a.nkb - (a.nkb >> (j + 1)));
        slot = j;
    };
    if (a.queue) {
        qtot = (int)(units * a.npc);
        const int t0 = (blockIdx.x / npool) * 4 + (threadIdx.x >> 6);
        if (qindex(t0) >= qtot) {
            q_done();
            return;
        }
        qpiece((int)qindex(t0), s0, s1, qslot);
    } else if (a.flat) {
        // at least kchunk steps per wave, so a chunk is split at most once
        long W = nwaves;
        if (S / a.kchunk < W) W = S / a.kchunk > 0 ? S / a.kchunk : 1;
        if (wave >= W) return;
        s0 = wave * S / W;
        s1 = (wave + 1) * S / W;
    } else {
        // whole (unit, chunk) items
        const long items = units * a.ksplit;
        const long i0 = wave * items / nwaves, i1 = (wave + 1) * items / nwaves;
        s0 = (i0 / a.ksplit) * a.nkb + min((long)a.nkb, (i0 % a.ksplit) * a.kchunk);
        s1 = (i1 / a.ksplit) * a.nkb + min((long)a.nkb, (i1 % a.ksplit) * a.kchunk);
    }
    if (s0 >= s1) {
        q_done();
        return;
    }
    // end of the segment starting at step x: the end of its chunk, or s1
    auto seg_end = [&](long x) {
        const long unit = x / a.nkb;
        const int kb = (int)(x - unit * a.nkb);
        const long ce = unit * a.nkb + min(a.nkb, (kb / a.kchunk + 1) * a.kchunk);
        return ce < s1 ? ce : s1;
    };
    // the segment after the one ending at e: the rest of the wave's share, or the next piece from the queue
    auto next_seg = [&](long e_cur, long &ns, long &ne, int &nslot) -> bool {
        if (a.queue) {
            const long t = qindex(qbase + __builtin_amdgcn_readlane(qtk, 0));
            if (t >= qtot) return false;
            qpiece((int)t, ns, ne, nslot);
            return true;
        }
        if (e_cur >= s1) return false;
        ns = e_cur;
        ne = seg_end(e_cur);
        return true;
    };
    const bool parts = a.flat || a.ksplit > 1 || a.queue;
    Ctx c, n;
    long e = a.queue ? s1 : seg_end(s0), ns = 0, ne = 0;
    int slot = qslot, nslot = 0;
    bool more = false;
    make_ctx<NS, RT, SW, TL>(a, s0, e, groups, tiles, n_act, goff, nullptr, c);
    if (!a.queue) slot = a.flat ? 2 * c.kc + c.piece : c.kc;
    v4f tot[RT], tot2[RT];
#pragma unroll
    for (int r = 0; r < RT; r++) tot[r] = tot2[r] = v4f{0.f, 0.f, 0.f, 0.f};
    Stage<SW, RT> X, Y;
    int kb = c.kb0;  // K-block of step s, in segment c
    long s = s0;
    load_stage<SW, RT, TL>(X, c, a.cols, kb);
    if (a.queue) q_take(qc, lane, qtk);
    // Step s: first the loads of step s + 1 into the other stage (from the next segment's context when s + 1
    // starts one; the last step re-reads its own tile, so every step issues the same loads), then the
    // arithmetic of step s, which waits only for the older stage.  The stages alternate by unrolling two
    // steps, never by copying registers that loads are still filling.
    auto step = [&](Stage<SW, RT> &P, Stage<SW, RT> &Q) __attribute__((always_inline)) -> bool {
        if (s + 1 == e) {
            more = next_seg(e, ns, ne, nslot);
            if (more) {
                make_ctx<NS, RT, SW, TL>(a, ns, ne, groups, tiles, n_act, goff, &c, n);
                if (!a.queue) nslot = a.flat ? 2 * n.kc + n.piece : n.kc;
                load_stage<SW, RT, TL>(Q, n, a.cols, n.kb0);
                if (a.queue) q_take(qc, lane, qtk);
            } else {
                load_stage<SW, RT, TL>(Q, c, a.cols, kb);
            }
        } else {
            load_stage<SW, RT, TL>(Q, c, a.cols, kb + 1);
        }
        const int kr = kb - c.kb0;
        const float tmask = c.tv ? 1.f : 0.f;
        const float ws = lane_f(kr < 64 ? c.wsv : c.wsvB, kr & 63) * tmask;
        const float ws2 = SW ? lane_f(kr < 64 ? c.wsv2 : c.wsvB2, kr & 63) * tmask : 0.f;
        const float f = ws * P.as, f2 = ws2 * P.as;
#pragma unroll
        for (int r = 0; r < RT; r++) {
            tot[r] += mfma_fp8(P.A[r], P.Bv) * f;
            if (SW) tot2[r] += mfma_fp8(P.A2[r], P.Bv) * f2;
        }
        if (s + 1 == e) {
            // end of the segment: add the parts of each token (columns ln, ln + TPG, ...), then store
#pragma unroll
            for (int r = 0; r < RT; r++) {
                tot[r] = sum_parts<NS>(tot[r]);
                if (SW) tot2[r] = sum_parts<NS>(tot2[r]);
            }
            if (c.tv && ln < TPG) {
                const long ooff = a.tok_cnt ? (long)(c.off + c.tt) * a.o_ts : (long)c.tt * a.o_ts + (long)c.m * a.o_ms;
#pragma unroll
                for (int r = 0; r < RT; r++) {
                    const int rr = c.r0 + r * 16 + 4 * lg;
                    if (parts) {
                        *(v4f *)(a.part + slot * a.n_out + ooff + rr) = tot[r];
                        if (SW) *(v4f *)(a.part2 + slot * a.n_out + ooff + rr) = tot2[r];
                        if (a.flat && c.whole) {
                            const v4f z = {0.f, 0.f, 0.f, 0.f};
                            *(v4f *)(a.part + (slot + 1) * a.n_out + ooff + rr) = z;
                            if (SW) *(v4f *)(a.part2 + (slot + 1) * a.n_out + ooff + rr) = z;
                        }
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            float v = tot[r][i];
                            if (EPI == EPI_RESID) v += act_load(a.resid, a.resid_dt, (long)c.tt * a.r_ts + rr + i);
                            if (SW) v = silu(v) * tot2[r][i];
                            a.out[ooff + rr + i] = v;
                        }
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < RT; r++) tot[r] = tot2[r] = v4f{0.f, 0.f, 0.f, 0.f};
            if (!more) return false;
            c = n;
            s = ns;
            e = ne;
            slot = nslot;
            kb = c.kb0;
            return true;
        }
        kb++;
        ++s;
        return true;
    };
    while (step(X, Y) && step(Y, X)) {
    }
    q_done();
}

// ------------------------------------------------------------------ fused expert FFN
// Gate/up, the SwiGLU with its FP8 split, and down in one launch over one work queue per XCD pool, so the waves that
// run out of gate/up pieces go on to down pieces instead of idling until the slowest one ends.  Pieces are
// numbered gate/up first (units (slot, 32-row tile, token group), npc K pieces each, unit-major), then down
// (units (slot, 64-row tile, token group), d.npc K pieces each into as many output slots, unit-major: the shorter
// pieces shorten the launch's tail, where the last waves finish their last pieces); each pool's
// tickets follow that order, so a pool hands out down pieces only after all of its gate/up pieces.  The hand-offs
// between phases go through device-scope stores and counters instead of a kernel boundary:
// - a gate/up piece stores its partial sums device-scope and then counts itself in done[group][block] (group: token
//   group of a slot, block: 128 rows of the intermediate).  The count is taken one step into the wave's next piece,
//   right after that step's loads are issued: the wait for all but those loads, which the step's arithmetic needs
//   anyway, has then covered the stores, so the weight stream does not drain for it;
// - the piece that completes a block forms Z = silu(G) * U for the group's tokens over those 128 rows, split into
//   FP8 parts as k_swiglu_quant does (same sums in slot order, same rounding), stores it device-scope and counts
//   the block in ready[group];
// - a down piece begins once ready[group] holds every block of its group.  Its count is read in the first step of
//   the wave's previous piece, so only the hand-over from gate/up to down ever spins.
// A wave waits only for pieces that running waves have taken: a taken gate/up piece runs to its end without
// waiting, every gate/up ticket of a pool precedes its down tickets, and the grid is what the device holds at
// once.  A wait that still passes its bound (about a third of a second) stops and fills the piece's outputs with
// NaN, so the launch always ends and such a failure cannot go unnoticed.
static constexpr int FFN_SPIN = 1 << 18;

template <bool TL>
__global__ __launch_bounds__(256, 2) void k_ffn_fp8(FfnFused f)
{
    constexpr int NS = 2, RT = 2, TPG = 16 / NS;
    constexpr int NLD = 4 * RT + 2 + 1;  // vector memory instructions of one load_stage<true, RT>
    __shared__ int s_goff[GEMV_MAXMAT + 1];
    const GemvArgs &g = f.g, &d = f.d;
    const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
    const int n_act = *g.n_active_dev;
    for (int i = threadIdx.x; i <= n_act; i += 256) s_goff[i] = g.grp_off[i];
    __syncthreads();
    const int ngrp = s_goff[n_act];
    const int tiles_g = g.rows / (16 * RT), tiles_d = d.rows / (32 * RT);
    const long units_g = (long)tiles_g * ngrp, units_d = (long)tiles_d * ngrp;
    const long qgu = units_g * g.npc, qtot = qgu + units_d * d.npc;
    const int nrb = g.rows / 128, ppb = 128 / (16 * RT) * g.npc;  // blocks of Z per group; gate/up pieces per block
    int *const done = f.sync, *const ready = f.sync + (long)f.gmax * nrb;
    // the queue, as in k_gemv_fp8
    const int npool = min((int)gridDim.x, GEMV_QPOOLS);
    const int pool = blockIdx.x % npool;
    int *qc = g.queue + pool * GEMV_QSTRIDE;
    const int qbase = 4 * (((int)gridDim.x - pool + npool - 1) / npool);
    int qm[GEMV_QPOOLS];
    gemv_shares_read(g.queue, qm);
    if (blockIdx.x < npool && threadIdx.x == 0)
        *(unsigned long long *)(qc + 2) = __builtin_amdgcn_s_memrealtime();
    // a wave is done: the pool's last one records the time (the pools' shares follow their rates over the launch)
    auto q_done = [&]() {
        if (lane == 0 && atomicAdd(qc + 1, 1) == qbase - 1)
            *(unsigned long long *)(qc + 4) = __builtin_amdgcn_s_memrealtime();
    };
    auto qindex = [&](int t) -> long {
        if (npool < GEMV_QPOOLS) return (long)t * npool + pool;
        const int n = qm[pool];
        return (long)(t / n) * GEMV_QROUND + gemv_slot_pos(qm, pool, t % n);
    };
    // slot of token group G: the last slot u with goff[u] <= G
    auto group_slot = [&](int G) {
        int lo = 0, hi = n_act - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_goff[mid] <= G) lo = mid; else hi = mid - 1;
        }
        return lo;
    };
    // token group of down unit x (units numbered group fastest, then tile, then slot)
    auto dn_group = [&](long x) {
        int lo = 0, hi = n_act - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if ((long)tiles_d * s_goff[mid] <= x) lo = mid; else hi = mid - 1;
        }
        const int gc = s_goff[lo + 1] - s_goff[lo];
        return s_goff[lo] + (int)((x - (long)tiles_d * s_goff[lo]) % gc);
    };
    // gate/up piece t -> steps [ps, pe) and partial slot: the K pieces of k_gemv_fp8, numbered unit-major here
    // (a unit's pieces side by side), so the slots' blocks complete in slot order from early on and the down
    // pieces, which follow the same slot order, find them ready
    auto gu_piece = [&](long t, long &ps, long &pe, int &sl) {
        const long unit = t / g.npc;
        const int j = (int)(t - unit * g.npc);
        const long u0 = unit * g.nkb;
        ps = u0 + g.nkb - (g.nkb >> j);
        pe = u0 + (j + 1 >= g.npc ? g.nkb : g.nkb - (g.nkb >> (j + 1)));
        sl = j;
    };
    // down piece x (after the gate/up ones) -> steps [ps, pe) and output slot: K pieces as for gate/up, unit-major
    auto dn_piece = [&](long x, long &ps, long &pe, int &sl) {
        const long unit = x / d.npc;
        const int j = (int)(x - unit * d.npc);
        const long u0 = unit * d.nkb;
        ps = u0 + d.nkb - (d.nkb >> j);
        pe = u0 + (j + 1 >= d.npc ? d.nkb : d.nkb - (d.nkb >> (j + 1)));
        sl = j;
    };
    // a down context covers 64 rows: tiles 0-1 in A, 2-3 in A2 (same 128-row scale block)
    auto fix_dn = [&](Ctx &x) {
        x.wp2 = x.wp + (TL ? 2L * d.nkb * 2048 : 32L * d.cols);
        x.wsp2 = x.wsp;
        x.wsv2 = x.wsv;
        x.wsvB2 = x.wsvB;
    };
    // block idx = G * nrb + rb of Z: SwiGLU of the group's tokens over rows [128 rb, +128), split into FP8 parts
    auto swiglu_block = [&](int idx) {
        const int G = idx / nrb, rb = idx - G * nrb;
        const int u = group_slot(G);
        const int t0 = (G - s_goff[u]) * TPG, off = g.tok_off[u] + t0;
        const int nt = min(TPG, g.tok_cnt[u] - t0), nsl = g.npc;
        const long base = (long)rb * 128 + lane * 2;
        // TB tokens at a time: all their loads in flight together, within the registers the piece loop leaves
        constexpr int TB = 2;
#pragma unroll 1
        for (int t0b = 0; t0b < nt; t0b += TB) {
            v2f gc[TB][2], uc[TB][2];
#pragma unroll
            for (int t = 0; t < TB; t++)
#pragma unroll
                for (int c = 0; c < 2; c++) {
                    const long o = (long)min(c, nsl - 1) * g.n_out + (long)(off + min(t0b + t, nt - 1)) * g.o_ts + base;
                    gc[t][c] = v2f{ld_dev(g.part + o), ld_dev(g.part + o + 1)};
                    uc[t][c] = v2f{ld_dev(g.part2 + o), ld_dev(g.part2 + o + 1)};
                }
#pragma unroll
            for (int t = 0; t < TB; t++) {
                if (t0b + t >= nt) break;
                v2f gs = {0.f, 0.f}, us = {0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 2; c++)
                    if (c < nsl) { gs += gc[t][c]; us += uc[t][c]; }
                const long row = off + t0b + t;
                split_store<NS, true>(silu(gs.x) * us.x, silu(gs.y) * us.y, const_cast<uint8_t *>(d.aq),
                                      const_cast<float *>(d.asc), d.aq_part, d.asc_part, row * g.rows + base,
                                      row * nrb + rb, lane);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the parts are stored before the block is counted
        if (lane == 0) atomicAdd(ready + G, 1);
    };
    bool poison = false;
    // until ready[G] holds every block (v: its value as last read)
    auto wait_ready = [&](int G, int v) {
        for (int it = 0; v < nrb && it < FFN_SPIN; it++) {
            __builtin_amdgcn_s_sleep(8);
            v = __builtin_amdgcn_readfirstlane(ld_dev(ready + G));
        }
        if (v < nrb) poison = true;
    };

    // the wave's first piece, fixed by its index: dealt wave-major over the pool's workgroups (wave 0 of every
    // workgroup, then wave 1, ...), so that when the pieces are fewer than the waves the busy waves spread over
    // the compute units instead of filling the first workgroups' units (a unit streams at a bounded rate, and a
    // unit holding twice the busy waves finishes its pieces twice as late)
    long t = qindex((threadIdx.x >> 6) * (qbase / 4) + (int)(blockIdx.x / npool));
    if (t >= qtot) {
        q_done();
        return;
    }
    Ctx c, n;
    Stage<true, RT> X, Y;
    v4f tot[RT], tot2[RT];
#pragma unroll
    for (int r = 0; r < RT; r++) tot[r] = tot2[r] = v4f{0.f, 0.f, 0.f, 0.f};
    long s = 0, e = 0, ns = 0, ne = 0;
    int kb = 0, slot = 0, nslot = 0, qtk = 0;
    int gn = -1, rdy = 0;  // down: group of the wave's next piece and its ready count (read early; lane values)
    bool more = false;

    // ---- gate/up pieces
    if (t < qgu) {
        int pend = -1;              // block of the last piece, stored but not yet counted
        int cnt_idx = -1, cnt_old = 0;  // block counted one piece ago, and the count it found (lane 0)
        auto count_back = [&]() {  // the count taken one piece ago: did that piece complete its block?
            if (cnt_idx >= 0 && __builtin_amdgcn_readlane(cnt_old, 0) == ppb - 1) swiglu_block(cnt_idx);
            cnt_idx = -1;
        };
        gu_piece(t, s, e, slot);
        make_ctx<NS, RT, true, TL>(g, s, e, 0, tiles_g, n_act, s_goff, nullptr, c);
        kb = c.kb0;
        load_stage<true, RT, TL>(X, c, g.cols, kb);
        q_take(qc, lane, qtk);
        auto step = [&](Stage<true, RT> &P, Stage<true, RT> &Q) __attribute__((always_inline)) -> bool {
            if (s + 1 == e) {
                // first (before the next piece's loads hold registers) a count not yet read (a short piece)
                count_back();
                t = qindex(qbase + __builtin_amdgcn_readlane(qtk, 0));
                more = t < qgu;
                if (more) {
                    gu_piece(t, ns, ne, nslot);
                    make_ctx<NS, RT, true, TL>(g, ns, ne, 0, tiles_g, n_act, s_goff, &c, n);
                    load_stage<true, RT, TL>(Q, n, g.cols, n.kb0);
                    q_take(qc, lane, qtk);
                } else {
                    load_stage<true, RT, TL>(Q, c, g.cols, kb);
                }
            } else {
                load_stage<true, RT, TL>(Q, c, g.cols, kb + 1);
            }
            if (pend >= 0) {
                // only this step's loads may still be outstanding: the previous piece's stores are complete
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NLD) : "memory");
                if (lane == 0) cnt_old = atomicAdd(done + pend, 1);
                cnt_idx = pend;
                pend = -1;
            }
            const int kr = kb - c.kb0;
            const float tmask = c.tv ? 1.f : 0.f;
            const float ws = lane_f(kr < 64 ? c.wsv : c.wsvB, kr & 63) * tmask;
            const float ws2 = lane_f(kr < 64 ? c.wsv2 : c.wsvB2, kr & 63) * tmask;
            const float f1 = ws * P.as, f2 = ws2 * P.as;
#pragma unroll
            for (int r = 0; r < RT; r++) {
                tot[r] += mfma_fp8(P.A[r], P.Bv) * f1;
                tot2[r] += mfma_fp8(P.A2[r], P.Bv) * f2;
            }
            if (s + 1 != e && kb == c.kb0 + 2) count_back();  // the count has returned by now
            if (s + 1 == e) {
#pragma unroll
                for (int r = 0; r < RT; r++) {
                    tot[r] = sum_parts<NS>(tot[r]);
                    tot2[r] = sum_parts<NS>(tot2[r]);
                }
                if (c.tv && ln < TPG) {
                    const long ooff = (long)(c.off + c.tt) * g.o_ts + (long)slot * g.n_out;
#pragma unroll
                    for (int r = 0; r < RT; r++) {
                        const long o = ooff + c.r0 + r * 16 + 4 * lg;
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            st_dev(g.part + o + i, tot[r][i]);
                            st_dev(g.part2 + o + i, tot2[r][i]);
                        }
                    }
                }
                pend = (s_goff[c.u] + c.t0 / TPG) * nrb + c.r0 / 128;
#pragma unroll
                for (int r = 0; r < RT; r++) tot[r] = tot2[r] = v4f{0.f, 0.f, 0.f, 0.f};
                if (!more) return false;
                c = n;
                s = ns;
                e = ne;
                slot = nslot;
                kb = c.kb0;
                return true;
            }
            kb++;
            ++s;
            return true;
        };
        while (step(X, Y) && step(Y, X)) {
        }
        // the wave's last gate/up piece: counted once its stores are complete (after any count still unread)
        count_back();
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (lane == 0) cnt_old = atomicAdd(done + pend, 1);
        cnt_idx = pend;
        count_back();
    }

    // ---- down pieces
    if (t >= qgu && t < qtot) {
        {
            const int G = dn_group((t - qgu) / d.npc);
            wait_ready(G, __builtin_amdgcn_readfirstlane(ld_dev(ready + G)));
        }
        dn_piece(t - qgu, s, e, slot);
        make_ctx<NS, 2 * RT, false, TL>(d, s, e, 0, tiles_d, n_act, s_goff, nullptr, c);
        fix_dn(c);
        kb = c.kb0;
        load_stage<true, RT, TL, true>(X, c, d.cols, kb);
        q_take(qc, lane, qtk);
        auto step = [&](Stage<true, RT> &P, Stage<true, RT> &Q) __attribute__((always_inline)) -> bool {
            if (s + 1 == e) {
                const long tn = qindex(qbase + __builtin_amdgcn_readlane(qtk, 0));
                more = tn < qtot;
                if (more) {
                    if (c.kb1 - c.kb0 < 2) {  // a one-step piece: no step read the count early
                        gn = dn_group((tn - qgu) / d.npc);
                        rdy = ld_dev(ready + gn);
                    }
                    wait_ready(gn, __builtin_amdgcn_readfirstlane(rdy));
                    dn_piece(tn - qgu, ns, ne, nslot);
                    make_ctx<NS, 2 * RT, false, TL>(d, ns, ne, 0, tiles_d, n_act, s_goff, &c, n);
                    fix_dn(n);
                    load_stage<true, RT, TL, true>(Q, n, d.cols, n.kb0);
                    q_take(qc, lane, qtk);
                } else {
                    load_stage<true, RT, TL, true>(Q, c, d.cols, kb);
                }
            } else {
                load_stage<true, RT, TL, true>(Q, c, d.cols, kb + 1);
                if (kb == c.kb0) {
                    // the next ticket has returned by now: read its group's count, used at the piece's end
                    const long tn = qindex(qbase + __builtin_amdgcn_readlane(qtk, 0));
                    gn = dn_group((min(tn, qtot - 1) - qgu) / d.npc);
                    rdy = ld_dev(ready + gn);
                }
            }
            const int kr = kb - c.kb0;
            const float tmask = c.tv ? 1.f : 0.f;
            const float ws = lane_f(kr < 64 ? c.wsv : c.wsvB, kr & 63) * tmask;
            const float ws2 = lane_f(kr < 64 ? c.wsv2 : c.wsvB2, kr & 63) * tmask;
            const float f1 = ws * P.as, f2 = ws2 * P.as;
#pragma unroll
            for (int r = 0; r < RT; r++) {
                tot[r] += mfma_fp8(P.A[r], P.Bv) * f1;
                tot2[r] += mfma_fp8(P.A2[r], P.Bv) * f2;
            }
            if (s + 1 == e) {
#pragma unroll
                for (int r = 0; r < RT; r++) {
                    tot[r] = sum_parts<NS>(tot[r]);
                    tot2[r] = sum_parts<NS>(tot2[r]);
                }
                if (c.tv && ln < TPG) {
                    const float bad = poison ? __builtin_nanf("") : 0.f;
                    const long ooff = (long)(c.off + c.tt) * d.o_ts + (long)slot * d.n_out;
#pragma unroll
                    for (int r = 0; r < RT; r++) {
                        const long o = ooff + c.r0 + r * 16 + 4 * lg;
                        *(v4f *)(d.part + o) = tot[r] + bad;
                        *(v4f *)(d.part + o + 32) = tot2[r] + bad;
                    }
                }
#pragma unroll
                for (int r = 0; r < RT; r++) tot[r] = tot2[r] = v4f{0.f, 0.f, 0.f, 0.f};
                if (!more) return false;
                c = n;
                s = ns;
                e = ne;
                slot = nslot;
                kb = c.kb0;
                return true;
            }
            kb++;
            ++s;
            return true;
        };
        while (step(X, Y) && step(Y, X)) {
        }
    }
    q_done();
}

int launch_ffn_fused(const FfnFused &f, hipStream_t s)
{
    const GemvArgs &g = f.g, &d = f.d;
    if (!g.queue || !g.grp_off || !g.n_active_dev || !d.grp_off || !g.tiled || !d.tiled || g.npc < 1 || g.npc > 2 ||
        d.npc < 1 || d.npc > 2 || (d.nkb >> (d.npc - 1)) < 1 || g.rows % 128 || d.rows % 64 || g.cols != d.rows || d.cols != g.rows || !g.part || !g.part2 ||
        !d.part || !f.sync || f.gmax < 1)
        return fail(DL_ERR_UNSUPPORTED, "fused FFN: unsupported arguments");
    const void *k = (const void *)k_ffn_fp8<true>;
    FfnFused arg = f;
    void *args[] = {(void *)&arg};
    if (hipLaunchKernel(k, dim3(resident_blocks(k, 256)), dim3(256), args, 0, s) != hipSuccess)
        return hip_check("ffn_fp8");
    return hip_check("ffn_fp8");
}

// One-shot projection GEMV (one FP8 matrix, either layout, tokens 0..ntok-1): a workgroup owns PROJ_RT * 16
// rows (PROJ_RT tiles) and a group of 8 K-blocks, wave w the blocks 2w and 2w + 1 of it.  Every wave issues all
// of its weight loads (PROJ_RT * 4 KB) before any arithmetic, so the whole matrix is in flight at once instead of
// a few blocks per wave, then adds its token groups' activations; the four waves' sums go through LDS and are
// added in wave order into partial slot (K group) of [slot][token][row].  Four tiles per workgroup give W_O
// (6,144 rows x 64 K-blocks) 768 workgroups, three per compute unit; eight gave 384, so half the units held two
// and half one, and the kernel lasted as long as the units reading twice the bytes.  The token groups run one
// after another (16 of them at 64 tokens), each loading the next group's activations before its own products.
static constexpr int PROJ_RT = 4;
template <int NS, bool TL>
__global__ __launch_bounds__(256) void k_proj_shot(GemvArgs a)
{
    constexpr int RT = PROJ_RT, KB = 2;
    __shared__ v4f s_acc[2][4][RT][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, ln = lane & 15, lg = lane >> 4;
    const int rb = blockIdx.x, kq = blockIdx.y;
    const int kb0 = kq * 8 + w * KB;
    if (a.ntok_host <= 0) return;
    v8i A[KB][RT];
#pragma unroll
    for (int k = 0; k < KB; k++)
#pragma unroll
        for (int r = 0; r < RT; r++)
            A[k][r] = TL ? ldw16x2(a.w + ((long)(rb * RT + r) * a.nkb + kb0 + k) * 2048 + lane * 16, 1024)
                         : ldw16x2(a.w + (long)((rb * RT + r) * 16 + ln) * a.cols + (kb0 + k) * 128 + lg * 16, 64);
    float ws[KB];
#pragma unroll
    for (int k = 0; k < KB; k++) ws[k] = a.wsc[(long)(rb * RT / 8) * a.nkb + kb0 + k];  // 128-row scale blocks
    constexpr int TPG = 16 / NS;  // tokens per group: the NS parts share the 16 columns
    const int ntok = a.ntok_host, tl = ln % TPG, sp = ln / TPG;
    const int tlast = (ntok - 1) / TPG * TPG;  // the last group's first token
    // a token group's activation codes and scales; the token clamped into range (every load unconditional, so
    // they are in flight together; a lane past the last token repeats it and its scale is zeroed below)
    auto load_b = [&](int t0, v8i (&Bv)[KB], float (&as)[KB]) {
        const int t = min(t0 + tl, ntok - 1);
#pragma unroll
        for (int k = 0; k < KB; k++) {
            Bv[k] = ld16x2(a.aq + sp * a.aq_part + (long)t * a.cols + (kb0 + k) * 128 + lg * 16, 64);
            as[k] = a.asc[sp * a.asc_part + (long)t * a.nkb + kb0 + k];
        }
    };
    // one token group: the next group's operands are loaded before this one's products, so their latency
    // overlaps the arithmetic and the sums; the four waves' sums go through LDS buffer buf (two buffers
    // alternate, so one barrier per group suffices: a buffer is written again only after the barrier of the
    // group in between, which every wave passes after reading it)
    auto group = [&](int t0, int buf, v8i (&Bc)[KB], float (&sc)[KB], v8i (&Bn)[KB], float (&sn)[KB]) {
        load_b(min(t0 + TPG, tlast), Bn, sn);
        const int t = t0 + tl;
        const bool tv = t < ntok;
        v4f tot[RT];
#pragma unroll
        for (int r = 0; r < RT; r++) tot[r] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KB; k++) {
            const float f = tv ? ws[k] * sc[k] : 0.f;
#pragma unroll
            for (int r = 0; r < RT; r++) tot[r] += mfma_fp8(A[k][r], Bc[k]) * f;
        }
#pragma unroll
        for (int r = 0; r < RT; r++) s_acc[buf][w][r][lane] = sum_parts<NS>(tot[r]);
        __syncthreads();
        // wave w adds the four waves' sums of its RT / 4 tiles
        if (tv && sp == 0) {
#pragma unroll
            for (int q = 0; q < RT / 4; q++) {
                const int r = (RT / 4) * w + q;
                const v4f v = ((s_acc[buf][0][r][lane] + s_acc[buf][1][r][lane]) + s_acc[buf][2][r][lane]) +
                              s_acc[buf][3][r][lane];
                *(v4f *)(a.part + (long)kq * a.n_out + (long)t * a.o_ts + (rb * RT + r) * 16 + 4 * lg) = v;
            }
        }
    };
    v8i B0[KB], B1[KB];
    float s0[KB], s1[KB];
    load_b(0, B0, s0);
    for (int t0 = 0; t0 < ntok; t0 += 2 * TPG) {
        group(t0, 0, B0, s0, B1, s1);
        if (t0 + TPG < ntok) group(t0 + TPG, 1, B1, s1, B0, s0);
    }
}

bool gemv_oneshot(GemvArgs &a, bool fp8)
{
    if (!fp8 || a.n_active_host != 1 || a.tok_cnt || a.a_ts != 1 || a.rows % 128 || a.nkb % 8 ||
        a.nkb / 8 > MAX_KSPLIT)
        return false;
    a.oneshot = 1;
    a.flat = 0;
    a.ksplit = a.nkb / 8;
    a.kchunk = 8;
    return true;
}

// Sum of the K-chunk partials in chunk order, then the epilogue.  EPI_RESID here needs the residual laid
// out like the output (r_ts == o_ts, uniform mode with one matrix).
template <int EPI>
__global__ __launch_bounds__(256) void k_gemv_reduce(GemvArgs a)
{
    constexpr bool SW = EPI == EPI_SWIGLU;
    const long e = (long)blockIdx.x * 256 + threadIdx.x;
    if (e >= a.n_out) return;
    const int nslot = gemv_slots(a);
    float v = 0.f, v2 = 0.f;
    for (int k = 0; k < nslot; k++) {
        v += a.part[(long)k * a.n_out + e];
        if (SW) v2 += a.part2[(long)k * a.n_out + e];
    }
    if (EPI == EPI_RESID) v += act_load(a.resid, a.resid_dt, e);
    if (SW) v = silu(v) * v2;
    a.out[e] = v;
}

// fp32 weights: one wave per (matrix, row, token group); lanes split the columns.
template <int EPI>
__global__ __launch_bounds__(256) void k_gemv_f32(GemvArgs a)
{
    constexpr bool SW = EPI == EPI_SWIGLU;
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nwaves = gridDim.x * 4;
    const int n_act = a.n_active_dev ? *a.n_active_dev : a.n_active_host;
    const long total = (long)n_act * a.rows * a.max_groups;
    for (long item = wave; item < total; item += nwaves) {
        const int g = (int)(item % a.max_groups);
        const long t2 = item / a.max_groups;
        const int row = (int)(t2 % a.rows);
        const int u = (int)(t2 / a.rows);
        const int m = a.active ? a.active[u] : u;
        const int cnt = a.tok_cnt ? a.tok_cnt[u] : a.ntok_host;
        const int off = a.tok_cnt ? a.tok_off[u] : 0;
        const int t0 = g * 16;
        if (t0 >= cnt) continue;
        const int nt = min(16, cnt - t0);
        const float *w = a.wf + (long)m * a.mat_elems + (long)row * a.cols;
        const float *w2 = SW ? a.wf2 + (long)m * a.mat_elems + (long)row * a.cols : nullptr;
        float acc[16], acc2[16];
        long arow[16];
#pragma unroll
        for (int t = 0; t < 16; t++) {
            acc[t] = acc2[t] = 0.f;
            const int tt = t0 + t;
            arow[t] = t < nt ? (a.pair_act ? a.pair_act[off + tt] : a.tok_cnt ? (long)(off + tt) : (long)tt * a.a_ts + (long)m * a.a_ms) : 0;
        }
        for (int c = lane; c < a.cols; c += 64) {
            const float wv = w[c];
            const float wv2 = SW ? w2[c] : 0.f;
#pragma unroll
            for (int t = 0; t < 16; t++)
                if (t < nt) {
                    const float x = a.af[arow[t] * a.cols + c];
                    acc[t] = fmaf(wv, x, acc[t]);
                    if (SW) acc2[t] = fmaf(wv2, x, acc2[t]);
                }
        }
#pragma unroll
        for (int t = 0; t < 16; t++) {
            if (t >= nt) continue;  // (uniform over the wave)
            float v = wave_sum(acc[t]);
            const float v2 = SW ? wave_sum(acc2[t]) : 0.f;
            if (lane == 0) {
                const int tt = t0 + t;
                const long ooff = a.tok_cnt ? (long)(off + tt) * a.o_ts : (long)tt * a.o_ts + (long)m * a.o_ms;
                if (EPI == EPI_RESID) v += act_load(a.resid, a.resid_dt, (long)tt * a.r_ts + row);
                if (SW) v = silu(v) * v2;
                a.out[ooff + row] = v;
            }
        }
    }
}

// One wave per (row, 128-block): NS parts, each rounded to e4m3 with its own amax/448 scale.
template <int NS>
__global__ __launch_bounds__(256) void k_quant(const float *__restrict__ x, long rows_host, const int *rows_dev,
                                               int cols, uint8_t *__restrict__ q, float *__restrict__ sc, long q_part,
                                               long sc_part)
{
    const int lane = threadIdx.x & 63;
    const long wave = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const long nwaves = (long)gridDim.x * 4;
    const long rows = rows_dev ? *rows_dev : rows_host;
    const int nkb = cols >> 7;
    for (long it = wave; it < rows * nkb; it += nwaves) {
        const long row = it / nkb;
        const int kb = (int)(it % nkb);
        const long e = row * cols + kb * 128 + lane * 2;
        const v2f v = *(const v2f *)(x + e);
        split_store<NS, false>(v.x, v.y, q, sc, q_part, sc_part, e, row * nkb + kb, lane);
    }
}

// Z = silu(sum_c G_c) * (sum_c U_c) from the nslot (<= 8) partial slots of the gate/up pass, summed in slot
// order, split into NS FP8 parts like k_quant.  rows come from the device (pairs of the plan).
template <int NS>
__global__ __launch_bounds__(256) void k_swiglu_quant(const float *__restrict__ pg, const float *__restrict__ pu,
                                                      int nslot, long stride, long rows_host, const int *rows_dev,
                                                      int cols, uint8_t *__restrict__ q, float *__restrict__ sc,
                                                      long q_part, long sc_part)
{
    const int lane = threadIdx.x & 63;
    const long wave = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const long nwaves = (long)gridDim.x * 4;
    const long rows = rows_dev ? *rows_dev : rows_host;
    const int nkb = cols >> 7;
    for (long it = wave; it < rows * nkb; it += nwaves) {
        const long row = it / nkb;
        const int kb = (int)(it % nkb);
        const long e = row * cols + kb * 128 + lane * 2;
        v2f gc[8], uc[8];
#pragma unroll
        for (int c = 0; c < 8; c++) {
            gc[c] = c < nslot ? *(const v2f *)(pg + c * stride + e) : v2f{0.f, 0.f};
            uc[c] = c < nslot ? *(const v2f *)(pu + c * stride + e) : v2f{0.f, 0.f};
        }
        v2f g = {0.f, 0.f}, u = {0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 8; c++)
            if (c < nslot) { g += gc[c]; u += uc[c]; }
        split_store<NS, false>(silu(g.x) * u.x, silu(g.y) * u.y, q, sc, q_part, sc_part, e, row * nkb + kb, lane);
    }
}

static int grid_for(long items, int per_block_waves = 4, int max_blocks = 8192)
{
    long b = (items + per_block_waves - 1) / per_block_waves;
    if (b < 1) b = 1;
    if (b > max_blocks) b = max_blocks;
    return (int)b;
}

static const void *gemv_kernel(int ns, int epi, bool tiled)
{
#define DL_K(NS_, E_, TL_) \
    if (ns == NS_ && epi == E_ && tiled == TL_) return (const void *)k_gemv_fp8<NS_, E_, 2, TL_>;
    DL_K(2, EPI_STORE, false) DL_K(2, EPI_RESID, false) DL_K(2, EPI_SWIGLU, false)
    DL_K(4, EPI_STORE, false) DL_K(4, EPI_RESID, false) DL_K(4, EPI_SWIGLU, false)
    DL_K(2, EPI_STORE, true) DL_K(2, EPI_RESID, true) DL_K(2, EPI_SWIGLU, true)
    DL_K(4, EPI_STORE, true) DL_K(4, EPI_RESID, true) DL_K(4, EPI_SWIGLU, true)
#undef DL_K
    return nullptr;
}

void gemv_flat(GemvArgs &a, int ns, int epi, long units_est, int max_ksplit)
{
    const void *k = gemv_kernel(ns, epi, a.tiled != 0);
    const long waves = k ? 4L * resident_blocks(k, 256) : 1024;
    const long spw = units_est * a.nkb / waves;  // steps per wave
    // fewest chunks that fit a wave's share, preferring equal chunks; never more than GEMV_MAXCHUNK blocks each
    int ks = 1;
    while (ks < max_ksplit && !(a.nkb % ks == 0 && a.nkb / ks <= spw)) ks++;
    while (ks > 1 && a.nkb % ks) ks--;
    while (ks < max_ksplit && (a.nkb + ks - 1) / ks > GEMV_MAXCHUNK) ks++;
    a.flat = 1;
    a.kchunk = (a.nkb + ks - 1) / ks;
    a.ksplit = (a.nkb + a.kchunk - 1) / a.kchunk;
}

int launch_gemv(const GemvArgs &a, int ns, int epi, bool fp8, hipStream_t s)
{
    // upper bound of the item count (device-side counts can only be smaller)
    const long n_act = a.n_active_host;
    if (fp8) {
        // persistent grid: exactly the workgroups that fit on the device at once, so every wave's equal
        // share of the items runs concurrently
        if (a.oneshot) {
            if (ns != 4 || !a.part) return fail(DL_ERR_UNSUPPORTED, "one-shot gemv parts=%d", ns);
            const dim3 g(a.rows / (PROJ_RT * 16), a.nkb / 8);
            if (a.tiled) hipLaunchKernelGGL((k_proj_shot<4, true>), g, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((k_proj_shot<4, false>), g, dim3(256), 0, s, a);
            if (!a.reduce_in_consumer) {
                const dim3 gr((unsigned)((a.n_out + 255) / 256));
                if (epi == EPI_RESID) hipLaunchKernelGGL((k_gemv_reduce<EPI_RESID>), gr, dim3(256), 0, s, a);
                else hipLaunchKernelGGL((k_gemv_reduce<EPI_STORE>), gr, dim3(256), 0, s, a);
            }
            return hip_check("proj_shot");
        }
        const void *k = gemv_kernel(ns, epi, a.tiled != 0);
        if (!k) return fail(DL_ERR_UNSUPPORTED, "gemv parts=%d", ns);
        if ((a.flat || a.ksplit > 1 || a.queue) && !a.part) return fail(DL_ERR_UNSUPPORTED, "gemv split without partials");
        if (a.queue && (!a.grp_off || a.npc < 1 || (a.nkb >> (a.npc - 1)) < 1))
            return fail(DL_ERR_UNSUPPORTED, "gemv queue of %d pieces over %d K-blocks", a.npc, a.nkb);
        if (a.kchunk > GEMV_MAXCHUNK)
            return fail(DL_ERR_UNSUPPORTED, "gemv K chunk of %d blocks (<= %d)", a.kchunk, GEMV_MAXCHUNK);
        GemvArgs arg = a;
        void *args[] = {(void *)&arg};
        if (hipLaunchKernel(k, dim3(resident_blocks(k, 256)), dim3(256), args, 0, s) != hipSuccess)
            return hip_check("gemv_fp8");
        if ((a.ksplit > 1 || a.flat || a.queue) && !a.reduce_in_consumer) {
            const dim3 gr((unsigned)((a.n_out + 255) / 256));
            if (epi == EPI_STORE) hipLaunchKernelGGL((k_gemv_reduce<EPI_STORE>), gr, dim3(256), 0, s, a);
            else if (epi == EPI_RESID) hipLaunchKernelGGL((k_gemv_reduce<EPI_RESID>), gr, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((k_gemv_reduce<EPI_SWIGLU>), gr, dim3(256), 0, s, a);
        }
        return hip_check("gemv_fp8");
    }
    const long items = n_act * a.rows * a.max_groups;
    const dim3 g(grid_for(items, 4, 4096));
    if (epi == EPI_STORE) hipLaunchKernelGGL((k_gemv_f32<EPI_STORE>), g, dim3(256), 0, s, a);
    else if (epi == EPI_RESID) hipLaunchKernelGGL((k_gemv_f32<EPI_RESID>), g, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_gemv_f32<EPI_SWIGLU>), g, dim3(256), 0, s, a);
    return hip_check("gemv_f32");
}

// Row-major FP8 [count][rows][cols] -> tiles (see dl.h): one thread per 16-byte output chunk.
__global__ __launch_bounds__(256) void k_pack(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, long count,
                                              int rows, int cols)
{
    const long nkb = cols / 128, tiles = rows / 16;
    const long n16 = count * tiles * nkb * 128;  // 16-byte chunks
    for (long o = (long)blockIdx.x * 256 + threadIdx.x; o < n16; o += (long)gridDim.x * 256) {
        const int l = (int)(o % 64);
        const int h = (int)((o / 64) % 2);
        long t = o / 128;  // (matrix, tile, block)
        const long kb = t % nkb;
        t /= nkb;
        const long tile = t % tiles;
        const long m = t / tiles;
        const long row = tile * 16 + (l % 16);
        const long col = kb * 128 + h * 64 + (l / 16) * 16;
        *(v4i *)(dst + o * 16) = *(const v4i *)(src + (m * rows + row) * cols + col);
    }
}

int launch_pack(const uint8_t *src, uint8_t *dst, long count, int rows, int cols, hipStream_t s)
{
    const long n16 = count * (long)rows * cols / 16;
    long blocks = (n16 + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_pack, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, count, rows, cols);
    return hip_check("pack");
}

// h = resid + sum_c part[c]: one wave per (row, 128-block); optionally h split into 2 FP8 parts.
__global__ __launch_bounds__(256) void k_resid_reduce_split(GemvArgs a, float *__restrict__ h, uint8_t *__restrict__ hq,
                                                            float *__restrict__ hqs, long hq_part, long hqs_part)
{
    const int lane = threadIdx.x & 63;
    const long wave = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int D = a.rows, nkb = D / 128;
    const long rows = a.n_out / D;
    if (wave >= rows * nkb) return;
    const long row = wave / nkb;
    const int kb = (int)(wave % nkb);
    const long e = row * D + kb * 128 + lane * 2;
    const int nslot = gemv_slots(a);
    // eight slots' loads at a time, unconditional (the slot index clamped; unused values dropped), issued before
    // the residual's (whose type decides its load), so that they are in flight together: a load under a
    // condition is waited for on its own
    v2f v = {0.f, 0.f};
    float x0 = 0.f, x1 = 0.f;
    for (int c0 = 0; c0 < nslot; c0 += 8) {
        v2f pc[8];
#pragma unroll
        for (int c = 0; c < 8; c++) pc[c] = *(const v2f *)(a.part + (long)min(c0 + c, nslot - 1) * a.n_out + e);
        if (c0 == 0) {
            x0 = act_load(a.resid, a.resid_dt, e);
            x1 = act_load(a.resid, a.resid_dt, e + 1);
        }
#pragma unroll
        for (int c = 0; c < 8; c++)
            if (c0 + c < nslot) v += pc[c];
    }
    float r0 = v.x + x0, r1 = v.y + x1;
    *(v2f *)(h + e) = v2f{r0, r1};
    if (!hq) return;
#pragma unroll
    for (int s = 0; s < 2; s++) {
        const float amax = wave_max(fmaxf(fabsf(r0), fabsf(r1)));
        const float scale = amax > 0.f ? amax * (1.0f / 448.0f) : 1.0f;
        const float inv = 1.0f / scale;
        const uint32_t code = f32x2_to_fp8(fminf(fmaxf(r0 * inv, -448.f), 448.f), fminf(fmaxf(r1 * inv, -448.f), 448.f));
        *(uint16_t *)(hq + s * hq_part + e) = (uint16_t)code;
        if (lane == 0) hqs[s * hqs_part + row * nkb + kb] = scale;
        const v2f d = fp8x2_lo(code);
        r0 -= d.x * scale;
        r1 -= d.y * scale;
    }
}

int launch_resid_reduce_split(const GemvArgs &a, float *h, uint8_t *hq, float *hqs, long hq_part, long hqs_part,
                              hipStream_t s)
{
    const long waves = a.n_out / 128;
    hipLaunchKernelGGL(k_resid_reduce_split, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a, h, hq, hqs, hq_part,
                       hqs_part);
    return hip_check("resid_reduce_split");
}

int launch_swiglu_quant(const float *pg, const float *pu, int nslot, long stride, long rows_host,
                        const int *rows_dev, int cols, uint8_t *q, float *sc, long q_part, long sc_part, int ns,
                        hipStream_t s)
{
    const long items = rows_host * (cols / 128);
    const dim3 g(grid_for(items, 4, 4096));
    if (ns == 2)
        hipLaunchKernelGGL((k_swiglu_quant<2>), g, dim3(256), 0, s, pg, pu, nslot, stride, rows_host, rows_dev, cols, q,
                           sc, q_part, sc_part);
    else return fail(DL_ERR_UNSUPPORTED, "swiglu quant parts=%d", ns);
    return hip_check("swiglu_quant");
}

int launch_quant(const float *x, long rows_host, const int *rows_dev, int cols, uint8_t *q, float *sc, long q_part,
                 long sc_part, int ns, hipStream_t s)
{
    const long items = rows_host * (cols / 128);
    const dim3 g(grid_for(items, 4, 4096));
    if (ns == 2) hipLaunchKernelGGL((k_quant<2>), g, dim3(256), 0, s, x, rows_host, rows_dev, cols, q, sc, q_part, sc_part);
    else if (ns == 4) hipLaunchKernelGGL((k_quant<4>), g, dim3(256), 0, s, x, rows_host, rows_dev, cols, q, sc, q_part, sc_part);
    else return fail(DL_ERR_UNSUPPORTED, "quant parts=%d", ns);
    return hip_check("quant");
}

}  // namespace dl
