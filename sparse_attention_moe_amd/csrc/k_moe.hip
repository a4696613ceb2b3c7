// S6 + S7 + combine: router, dispatch plan and the fixed-order sum of expert outputs.
//
// The model routes every token to 8 experts plus a shared one (Introducing Kiln, "How was Kiln
// measured against vLLM on H200?"); its expert kernel applies each expert once to all of its tokens
// ("A collective costs per graph, so the graphs got big") from a routing plan, and experts without
// tokens are skipped ("What moved the number ...").  Router logits accumulate fp32 products in fp64
// so the expert choice matches an exact evaluation except for genuinely near-equal logits.
#include "dl_common.h"
#include "dl_internal.h"

#include <string.h>

namespace dl {

static constexpr int ROUTE_KW = 256;  // hidden features per wave
static constexpr int ROUTE_KC = 4 * ROUTE_KW;  // hidden features per workgroup
static constexpr int ROUTE_MAXC = 16; // chunks: hidden size <= 16,384
static constexpr int RP_MAXE = 1024;  // experts the router + plan kernel handles
static constexpr int RP_LCAP = 8192;  // logits held in LDS at once (tokens per block = RP_LCAP / E)

typedef double v4d __attribute__((ext_vector_type(4)));

// Partial router logits on the fp64 matrix cores: part[c, b, e] = sum over hidden chunk c of w_r[e, d] * h[b, d].
// A workgroup owns 16 experts (the M side of v_mfma_f64_16x16x4f64) and a chunk of ROUTE_KC features,
// ROUTE_KW per wave; 16 tokens form the N side.  Every fp32 product is exact in fp64 and the sums are fp64.
// Lane (r, g) = (lane % 16, lane / 16) holds expert r's and token r's features 16 j + 4 g .. + 4 of the wave's
// range; instruction i of a group takes the i-th of those four, so A and B agree on the K index.  The four
// waves' sums are added in order through LDS.  The grid's third axis strides over the 16-token tiles, so a large
// batch spreads over more workgroups instead of lengthening each one's serial loop.
__global__ __launch_bounds__(256) void k_route_partial(const float *__restrict__ h, int B, int D,
                                                       const float *__restrict__ wr, int E, double *__restrict__ part)
{
    constexpr int NJ = ROUTE_KW / 16;
    __shared__ double s_d[4][16][17];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int e0 = blockIdx.x * 16, c = blockIdx.y;
    const int kq = c * ROUTE_KC + w * ROUTE_KW + 4 * g;
    const int e = e0 + r;
    // every load unconditional (expert, token and feature clamped into range, the values masked to zero after),
    // and the first token tile's activations issued with the weights, so both are in flight together (the grid
    // covers up to 1,024 tokens with one tile per workgroup; beyond that a workgroup loads its later tiles in turn)
    const bool ev = e < E;
    v4f wv[NJ];
#pragma unroll
    for (int j = 0; j < NJ; j++) wv[j] = *(const v4f *)(wr + (long)min(e, E - 1) * D + min(kq + 16 * j, D - 4));
    auto load_h = [&](int t0, v4f (&hv)[NJ]) {
        const int t = min(t0 + r, B - 1);
#pragma unroll
        for (int j = 0; j < NJ; j++) hv[j] = *(const v4f *)(h + (long)t * D + min(kq + 16 * j, D - 4));
    };
    v4f hn[NJ];
    load_h(blockIdx.z * 16, hn);
#pragma unroll
    for (int j = 0; j < NJ; j++)
        if (!(ev && kq + 16 * j < D)) wv[j] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int t0 = blockIdx.z * 16; t0 < B; t0 += gridDim.z * 16) {
        const int t = t0 + r;
        if (t0 != (int)blockIdx.z * 16) load_h(t0, hn);
        v4f hv[NJ];
#pragma unroll
        for (int j = 0; j < NJ; j++) hv[j] = (t < B && kq + 16 * j < D) ? hn[j] : v4f{0.f, 0.f, 0.f, 0.f};
        v4d acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int j = 0; j < NJ; j++)
#pragma unroll
            for (int i = 0; i < 4; i++)
                acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)wv[j][i], (double)hv[j][i], acc, 0, 0, 0);
        // the fp64 instruction's result layout: acc[i] of lane (r, g) = row 4 i + g (expert), column r (token)
#pragma unroll
        for (int i = 0; i < 4; i++) s_d[w][4 * i + g][r] = acc[i];
        __syncthreads();
        {
            const int ee = threadIdx.x >> 4, tt = threadIdx.x & 15;
            if (e0 + ee < E && t0 + tt < B)
                part[((long)c * B + t0 + tt) * E + e0 + ee] =
                    ((s_d[0][ee][tt] + s_d[1][ee][tt]) + s_d[2][ee][tt]) + s_d[3][ee][tt];
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ wave reductions on the DPP network
// Maximum of an unsigned over the wave, broadcast.  Row prefix maxima (shifts 1, 2, 4, 8), then rows are
// combined with the row-broadcast forms; lane 63 ends up with the maximum.  Zero is the identity.
__device__ __forceinline__ unsigned wave_max_u32(unsigned v)
{
    v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));  // row_shr:1
    v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));  // row_shr:2
    v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));  // row_shr:4
    v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));  // row_shr:8
    v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
    v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
    return (unsigned)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ unsigned wave_min_u32(unsigned v) { return ~wave_max_u32(~v); }

// Order-preserving map of a float to an unsigned (x < y  =>  key(x) < key(y)); every finite value and the
// infinities map above 0.
__device__ __forceinline__ unsigned ordered_key(float f)
{
    const unsigned u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exact top-k of one token's fp64 logits by (logit desc, id asc) in one wave: each lane owns experts
// lane + 64 i; ke rounds of a wave argmax, the owner retiring its pick.  Lane j < ke returns pick j.
template <int NSLOT>
__device__ __forceinline__ int token_topk_exact(const double *lrow, int E, int ke)
{
    const int lane = threadIdx.x & 63;
    double l[NSLOT];
#pragma unroll
    for (int i = 0; i < NSLOT; i++) {
        const int e = lane + 64 * i;
        l[i] = e < E ? lrow[e] : -INFINITY;
    }
    int my_e = 0;
    for (int j = 0; j < ke; j++) {
        double best = -INFINITY;
        int bi = 0, be = 0x7FFFFFFF;
#pragma unroll
        for (int i = 0; i < NSLOT; i++) {
            const int e = lane + 64 * i;
            if (e < E && (l[i] > best || (l[i] == best && e < be))) { best = l[i]; be = e; bi = i; }
        }
        const int me = be;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const double ov = __shfl_xor(best, o, 64);
            const int oe = __shfl_xor(be, o, 64);
            if (ov > best || (ov == best && oe < be)) { best = ov; be = oe; }
        }
        if (me == be) {
#pragma unroll
            for (int i = 0; i < NSLOT; i++)
                if (i == bi) l[i] = -INFINITY;
        }
        if (lane == j) my_e = be;
    }
    return my_e;
}

// Top-k of one token in one wave.  Selection runs on fp32 keys of the fp64 logits (an order-preserving
// map: a strictly larger key means a strictly larger logit) with two DPP reductions per round: the
// largest key, then the lowest expert id holding it.  ke + 1 rounds are taken; when no two of those
// ke + 1 keys are equal, the keys order the picks and the boundary exactly as the fp64 logits do.
// Otherwise (a rounding tie) the exact fp64 selection decides.  Lane j < ke returns pick j.
template <int NSLOT>
__device__ __forceinline__ int token_topk(const double *lrow, int E, int ke)
{
    const int lane = threadIdx.x & 63;
    unsigned key[NSLOT];
#pragma unroll
    for (int i = 0; i < NSLOT; i++) {
        const int e = lane + 64 * i;
        key[i] = e < E ? ordered_key((float)lrow[e]) : 0u;
    }
    int my_e = 0;
    unsigned prev = 0;
    bool tie = false;
    const int rounds = ke < E ? ke + 1 : ke;
    for (int j = 0; j < rounds; j++) {
        unsigned bk = 0;
        int bi = 0;
#pragma unroll
        for (int i = 0; i < NSLOT; i++)
            if (key[i] > bk) { bk = key[i]; bi = i; }
        const unsigned K = wave_max_u32(bk);
        const unsigned id = wave_min_u32(bk == K ? (unsigned)(lane + 64 * bi) : 0xFFFFFFFFu);
        if (j > 0 && K == prev) tie = true;
        prev = K;
        if (j < ke) {
            if (lane == (int)(id & 63)) {
#pragma unroll
                for (int i = 0; i < NSLOT; i++)
                    if (i == (int)(id >> 6)) key[i] = 0u;
            }
            if (lane == j) my_e = (int)id;
        }
    }
    if (tie) my_e = token_topk_exact<NSLOT>(lrow, E, ke);
    return my_e;
}

// ------------------------------------------------------------------ dispatch plan
// From the picks s_exp[b * ke + j] (in LDS) of a whole workgroup of 1024 threads: active experts, the shared
// ones first, then the routed ones in ascending id, each expert's pairs in (token, slot) order, the pair index of every
// (token, slot), and the prefix over active experts of their token groups of PLAN_TPG (grp_off, n_active + 1
// entries) that the expert GEMV enumerates its work by.  `distinct`: no token picks an expert twice (router
// output), so an expert's pair rank is the number of earlier tokens in its token mask (B <= 64); otherwise the
// earlier picks are counted.  A negative pick is skipped: its pair index is -1 and the pairs computed here stay
// contiguous (shared experts' pairs right after the routed ones).  s_cnt holds E + 1 entries.
// The pools' shares of the next launch of one expert GEMV (q: its GEMV_QINTS block), from the last launch's
// measured times: pool p ran m_p of every GEMV_QROUND pieces and took T_p, so its rate is m_p / T_p; the new
// shares move three quarters of the way to the rates' proportions, within half and one and a half times an equal
// share.  (The pools are the XCDs: the dispatch deals workgroups round-robin over them, and their read rates
// differ by up to about 15% on one device, the slow ones the same from launch to launch.)  Which
// pool runs a piece never changes a result (piece j of a unit always writes partial slot j).  Shares or times
// that were never written give equal shares.  Lanes 0..7 of one wave.
// The inputs of the shares, split from the arithmetic below so that a caller can issue these loads early and
// use them later: the current shares and lane l's pool's start and end times (lanes 8..63 read pool 7's, unused).
struct PoolIn {
    int m[GEMV_QPOOLS];
    unsigned long long t0, t1;
};
__device__ __forceinline__ void gemv_pool_load(const int *q, int lane, PoolIn &in)
{
#pragma unroll
    for (int p = 0; p < GEMV_QPOOLS; p++) in.m[p] = q[GEMV_QTAB + p];
    const int l = min(lane, GEMV_QPOOLS - 1);
    in.t0 = *(const unsigned long long *)(q + l * GEMV_QSTRIDE + 2);
    in.t1 = *(const unsigned long long *)(q + l * GEMV_QSTRIDE + 4);
}
__device__ void gemv_pool_shares(int *q, int lane, const PoolIn &in)
{
    int m[GEMV_QPOOLS];
    gemv_shares_valid(in.m, m);
    float rl = 0.f;
    bool okl = true;
    if (lane < GEMV_QPOOLS) {
        const unsigned long long t0 = in.t0, t1 = in.t1;
        int ml = 0;
#pragma unroll
        for (int p = 0; p < GEMV_QPOOLS; p++) ml = lane == p ? m[p] : ml;
        okl = t1 > t0 && t1 - t0 < 100000000ull;  // under a second of 100 MHz ticks
        rl = okl ? ml / (float)(t1 - t0) : 0.f;
    }
    const bool ok = __builtin_amdgcn_ballot_w64(!okl) == 0;
    float r[GEMV_QPOOLS], rs = 0.f;
#pragma unroll
    for (int p = 0; p < GEMV_QPOOLS; p++) {
        r[p] = __shfl(rl, p, 64);
        rs += r[p];
    }
    constexpr int EQ = GEMV_QROUND / GEMV_QPOOLS, LO = EQ / 2, HI = EQ + EQ / 2;
    int n[GEMV_QPOOLS];
    if (!ok || !(rs > 0.f)) {
#pragma unroll
        for (int p = 0; p < GEMV_QPOOLS; p++) n[p] = EQ;
    } else {
        float x[GEMV_QPOOLS];
        int tot = 0;
#pragma unroll
        for (int p = 0; p < GEMV_QPOOLS; p++) {
            x[p] = fminf(fmaxf(0.25f * m[p] + 0.75f * GEMV_QROUND * r[p] / rs, (float)LO), (float)HI);
            n[p] = (int)x[p];
            tot += n[p];
        }
        // the remaining slots to the largest remainders (at most HI each)
        for (; tot < GEMV_QROUND; tot++) {
            int b = 0;
            float bf = -1.f;
#pragma unroll
            for (int p = 0; p < GEMV_QPOOLS; p++)
                if (n[p] < HI && x[p] - n[p] > bf) { b = p; bf = x[p] - n[p]; }
#pragma unroll
            for (int p = 0; p < GEMV_QPOOLS; p++) n[p] += p == b;
        }
    }
    if (lane < GEMV_QPOOLS) {
        int nl = 0;
#pragma unroll
        for (int p = 0; p < GEMV_QPOOLS; p++) nl = lane == p ? n[p] : nl;
        q[GEMV_QTAB + lane] = nl;
    }
}

__device__ void build_plan(const int *s_exp, int B, int ke, int E, int S, bool distinct, int *s_cnt, int *s_off,
                           unsigned long long *s_mask, const MoePlan &p, bool shares)
{
    const int tid = threadIdx.x, lane = tid & 63;
    const int nT = blockDim.x;
    const int kk = ke + S;
    const int np = B * ke;
    const bool use_mask = distinct && B <= 64;
    __shared__ int s_ngrp;  // token groups of the plan
    for (int e = tid; e < E; e += nT) { s_cnt[e] = 0; s_mask[e] = 0ull; }
    __syncthreads();
    for (int i = tid; i < np; i += nT) {
        const int e = s_exp[i];
        if (e < 0) continue;  // a pair computed elsewhere
        atomicAdd(&s_cnt[e], 1);
        if (use_mask) atomicOr(&s_mask[e], 1ull << (i / ke));
    }
    __syncthreads();
    // the expert GEMVs' work queues: the pools' shares from their last launch, cleared counters
    if (shares && p.queue && nT >= 256 && (tid >> 6) >= 2 && (tid >> 6) < 4) {
        PoolIn in;
        gemv_pool_load(p.queue + ((tid >> 6) - 2) * GEMV_QINTS, lane, in);
        gemv_pool_shares(p.queue + ((tid >> 6) - 2) * GEMV_QINTS, lane, in);
    }
    if (p.queue && tid < 2 * GEMV_QPOOLS) {
        p.queue[tid * GEMV_QSTRIDE] = 0;
        p.queue[tid * GEMV_QSTRIDE + 1] = 0;
    }
    if (tid < 64) {
        // lane owns experts [lane * per, (lane + 1) * per)
        const int per = (E + 63) / 64;
        int na = 0, npl = 0, ng = 0;
        for (int i = 0; i < per; i++) {
            const int e = lane * per + i;
            if (e < E) {
                const int c = s_cnt[e];
                na += c > 0;
                npl += c;
                ng += (c + PLAN_TPG - 1) / PLAN_TPG;
            }
        }
        int ia = na, ip = npl, ig = ng;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int ta = __shfl_up(ia, o, 64), tp = __shfl_up(ip, o, 64), tg = __shfl_up(ig, o, 64);
            if (lane >= o) { ia += ta; ip += tp; ig += tg; }
        }
        const int na_tot = __shfl(ia, 63, 64), ng_tot = __shfl(ig, 63, 64);
        const int npr = __shfl(ip, 63, 64);  // routed pairs computed here (skipped ones excluded)
        // slots: the shared experts first (the most tokens: the fused FFN finishes their gate/up, and so can start
        // their down pieces, earliest), then the routed ones in expert order; pairs: routed, then shared
        const int gs = (B + PLAN_TPG - 1) / PLAN_TPG;  // token groups of a shared expert
        int a = S + ia - na, q = ip - npl, gq = S * gs + ig - ng;
        for (int i = 0; i < per; i++) {
            const int e = lane * per + i;
            if (e < E && s_cnt[e] > 0) {
                p.active[a] = e;
                p.tok_off[a] = q;
                p.tok_cnt[a] = s_cnt[e];
                p.grp_off[a] = gq;
                s_off[e] = q;
                a++;
                q += s_cnt[e];
                gq += (s_cnt[e] + PLAN_TPG - 1) / PLAN_TPG;
            }
        }
        for (int sx = lane; sx < S; sx += 64) {
            p.active[sx] = E + sx;
            p.tok_off[sx] = npr + sx * B;
            p.tok_cnt[sx] = B;
            p.grp_off[sx] = sx * gs;
        }
        if (lane == 0) {
            p.grp_off[na_tot + S] = ng_tot + S * gs;
            *p.n_active = na_tot + S;
            *p.n_pairs = npr + S * B;
            s_cnt[E] = npr;  // for the shared pairs below (s_cnt holds E + 1 entries)
            s_ngrp = ng_tot + S * gs;
        }
    }
    __syncthreads();
    const int npr = s_cnt[E];
    if (p.ffn_sync) {
        // the fused FFN's counters of the plan's token groups
        const int ng = min(s_ngrp, p.ffn_gmax);
        int *ready = p.ffn_sync + (long)p.ffn_gmax * p.ffn_nrb;
        for (int i = tid; i < ng * p.ffn_nrb; i += nT) p.ffn_sync[i] = 0;
        for (int i = tid; i < ng; i += nT) ready[i] = 0;
    }
    for (int i = tid; i < np; i += nT) {
        const int b = i / ke, j = i - b * ke, e = s_exp[i];
        if (e < 0) {
            p.pair_idx[(long)b * kk + j] = -1;
            continue;
        }
        int rank = 0;
        if (use_mask) rank = __popcll(s_mask[e] & ((1ull << b) - 1ull));
        else
            for (int i2 = 0; i2 < i; i2++) rank += s_exp[i2] == e;
        const int q = s_off[e] + rank;
        p.pair_tok[q] = b;
        p.pair_idx[(long)b * kk + j] = q;
    }
    for (int i = tid; i < S * B; i += nT) {
        const int sx = i / B, b = i - sx * B;
        const int q = npr + sx * B + b;
        p.pair_tok[q] = b;
        p.pair_idx[(long)b * kk + ke + sx] = q;
    }
}

// Dispatch plan of caller-given picks (experts [B, ke]).  A negative id marks a pair computed elsewhere (an
// expert another GPU holds): it gets no row and adds nothing.  lo < 0: ids of E or more are clamped to E - 1 so
// that no access leaves the arrays.  lo >= 0 (one GPU's expert-parallel share): the stack holds experts
// [lo, lo + E); a pick in that range becomes its local index, any other pick is computed elsewhere.  Picks with
// no expert twice in a token (the router's) take the token-mask ranks; each pick looks back over its own token.
__global__ __launch_bounds__(1024) void k_plan(const int32_t *__restrict__ experts, int B, int ke, int E, int S,
                                               int lo, MoePlan p)
{
    __shared__ int s_exp[16384];
    __shared__ int s_cnt[RP_MAXE + 1], s_off[RP_MAXE];  // s_cnt[E]: routed pairs computed
    __shared__ unsigned long long s_mask[RP_MAXE];
    for (int i = threadIdx.x; i < B * ke; i += blockDim.x) {
        const int e = experts[i];
        s_exp[i] = lo < 0 ? (e < 0 ? -1 : min(e, E - 1)) : (e >= lo && e - lo < E ? e - lo : -1);
    }
    __syncthreads();
    int dup = 0;
    for (int i = threadIdx.x; i < B * ke; i += blockDim.x) {
        const int e = s_exp[i];
        if (e >= 0)
            for (int i2 = i - i % ke; i2 < i; i2++) dup |= s_exp[i2] == e;
    }
    const bool distinct = !__syncthreads_or(dup);
    build_plan(s_exp, B, ke, E, S, distinct, s_cnt, s_off, s_mask, p, true);
}

// Router top-k, fused with the dispatch plan when one workgroup of 1024 threads routes every token.  A workgroup
// routes tokens [blockIdx.x * tpb, + tpb), in blocks of RP_LCAP / E: the block's logits (chunk partials summed in
// chunk order, plus the bias) go to LDS, then wave w picks the experts of tokens w, w + 16, ... and their gates
// (softmax over the picked logits, summed in pick order).  With p.active != nullptr (a single workgroup) the plan
// follows (B * ke <= 16384).
template <int NSLOT>  // experts per lane: E <= 64 * NSLOT
__global__ __launch_bounds__(1024) void k_route_plan(const double *__restrict__ part, int nchunk, int B, int E, int ke,
                                                     int S, const float *__restrict__ bias,
                                                     int32_t *__restrict__ experts, float *__restrict__ gates,
                                                     float *__restrict__ logits, MoePlan p, int tpb)
{
    __shared__ double s_l[RP_LCAP];
    __shared__ int s_exp[16384];
    __shared__ int s_cnt[RP_MAXE + 1], s_off[RP_MAXE];  // s_cnt[E]: routed pairs computed
    __shared__ unsigned long long s_mask[RP_MAXE];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nT = 1024;
    const bool plan = p.active != nullptr;
    // the expert GEMVs' pool shares for this step, by the last two waves: their inputs loaded now, the arithmetic
    // while waves 0..nb-1 pick the experts of the first block's tokens
    const bool shares = plan && p.queue && wv >= 14;
    PoolIn pin;
    if (shares) gemv_pool_load(p.queue + (wv - 14) * GEMV_QINTS, lane, pin);
    const int tb = RP_LCAP / E;
    const int t0 = blockIdx.x * tpb, t1 = min(B, t0 + tpb);  // this workgroup's tokens
    for (int b0 = t0; b0 < t1; b0 += tb) {
        const int nb = min(tb, t1 - b0);
        // two logits per thread per pass, summed in chunk order; eight chunks' partials of both are loaded at
        // once, unconditionally (indices clamped into the arrays), so that the loads are in flight together: a
        // load under a condition is waited for on its own
        for (int i0 = tid; i0 < nb * E; i0 += 2 * nT) {
            double v2[2] = {0.0, 0.0};
            float bv[2];  // the biases, loaded with the partials (without a bias: any readable word, unused)
#pragma unroll
            for (int k = 0; k < 2; k++) {
                const int i = min(i0 + k * nT, nb * E - 1);
                bv[k] = *(bias ? bias + i % E : (const float *)part);
            }
            for (int c0 = 0; c0 < nchunk; c0 += 8) {
                double pc[2][8];
#pragma unroll
                for (int k = 0; k < 2; k++) {
                    const int i = min(i0 + k * nT, nb * E - 1);
                    const int b = b0 + i / E, e = i % E;
#pragma unroll
                    for (int c = 0; c < 8; c++) pc[k][c] = part[((long)min(c0 + c, nchunk - 1) * B + b) * E + e];
                }
#pragma unroll
                for (int k = 0; k < 2; k++)
#pragma unroll
                    for (int c = 0; c < 8; c++)
                        if (c0 + c < nchunk) v2[k] += pc[k][c];
            }
#pragma unroll
            for (int k = 0; k < 2; k++) {
                const int i = i0 + k * nT;
                if (i >= nb * E) break;
                const int b = b0 + i / E, e = i % E;
                double v = v2[k];
                if (bias) v += (double)bv[k];
                s_l[i] = v;
                if (logits) logits[(long)b * E + e] = (float)v;
            }
        }
        __syncthreads();
        for (int bl = wv; bl < nb; bl += 16) {
            const double *lrow = s_l + (long)bl * E;
            const int me = token_topk<NSLOT>(lrow, E, ke);
            const double lm = lane < ke ? lrow[me] : 0.0;
            const double l0 = __shfl(lm, 0, 64);
            const double gx = exp(lm - l0);
            double z = 0.0;
            for (int j = 0; j < ke; j++) z += __shfl(gx, j, 64);
            if (lane < ke) {
                const int b = b0 + bl;
                experts[(long)b * ke + lane] = me;
                gates[(long)b * ke + lane] = (float)(gx / z);
                if (plan) s_exp[b * ke + lane] = me;
            }
        }
        if (shares && b0 == t0) gemv_pool_shares(p.queue + (wv - 14) * GEMV_QINTS, lane, pin);
        __syncthreads();
    }
    if (plan) build_plan(s_exp, B, ke, E, S, true, s_cnt, s_off, s_mask, p, false);
}

int route_chunks(int D) { return (D + ROUTE_KC - 1) / ROUTE_KC; }

bool route_plan_ok(int E, int ke, int B) { return E <= RP_MAXE && ke <= 32 && (long)B * ke <= 16384; }

int launch_route_partial(const float *h, int B, int D, const float *w_r, int E, double *part, hipStream_t s)
{
    dim3 g((E + 15) / 16, route_chunks(D), max(1, min((B + 15) / 16, 64)));
    hipLaunchKernelGGL(k_route_partial, g, dim3(256), 0, s, h, B, D, w_r, E, part);
    return hip_check("route_partial");
}

int launch_route_plan(const double *part, int B, int D, const float *bias, int E, int ke, int S, int32_t *experts,
                      float *gates, float *logits, const MoePlan *p, hipStream_t s)
{
    MoePlan none;
    memset(&none, 0, sizeof none);
    // up to 16 tokens one workgroup routes them all and builds the plan; more are routed 16 per workgroup (one
    // token per wave), and the plan kernel follows: the single workgroup's token loop was the cost at batch 64
    const bool one = B <= 16;
    const MoePlan &pp = p && one ? *p : none;
    const dim3 g(one ? 1 : (B + 15) / 16);
    const int tpb = one ? B : 16;
#define DL_RP(NS_)                                                                                                  \
    hipLaunchKernelGGL((k_route_plan<NS_>), g, dim3(1024), 0, s, part, route_chunks(D), B, E, ke, S, bias, experts, \
                       gates, logits, pp, tpb)
    if (E <= 256) DL_RP(4); else DL_RP(16);
#undef DL_RP
    if (p && !one) return launch_plan(experts, B, ke, E, S, *p, s);
    return hip_check("route_plan");
}

int launch_route(const float *h, int B, int D, const float *w_r, const float *bias, int E, int ke, int32_t *experts,
                 float *gates, float *logits, double *part, hipStream_t s)
{
    int st = launch_route_partial(h, B, D, w_r, E, part, s);
    if (st != DL_OK) return st;
    return launch_route_plan(part, B, D, bias, E, ke, 0, experts, gates, logits, nullptr, s);
}

int launch_plan(const int32_t *experts, int B, int ke, int E, int S, const MoePlan &p, hipStream_t s, int lo)
{
    hipLaunchKernelGGL(k_plan, dim3(1), dim3(1024), 0, s, experts, B, ke, E, S, lo, p);
    return hip_check("plan");
}

// out[b, d] = resid[b, d] + sum_j gate[b, j] f_j[d] + sum_s f_s[d], in that order, where f is the sum of the
// expert output's nslot partial slots (in slot order).  A thread owns 4 consecutive features of one token (a
// workgroup's threads all hold the same token).  Lane j of a wave loads the token's pair index j and gate j, and
// the wave reads them back with readlane, so those loads are one round trip (scalar loads of the same words were
// each waited for before the next); the residual is loaded in both layouts at once (the one not used reads another
// array in bounds), and the expert outputs 16 pairs at a time, so all of a thread's loads are in flight together.
__global__ __launch_bounds__(256) void k_combine(const float *__restrict__ F, int nslot, long fstride,
                                                 const int *__restrict__ pair_idx,
                                                 const float *__restrict__ gates, int B, int D, int ke, int S,
                                                 const void *__restrict__ resid, int resid_dt, void *__restrict__ out,
                                                 int out_dt, float *__restrict__ out32)
{
    constexpr int PU = 16;  // pairs per round
    const int b = blockIdx.y, lane = threadIdx.x & 63;
    const int d0 = (blockIdx.x * 256 + threadIdx.x) * 4;
    const bool dv = d0 < D;
    const int d = min(d0, D - 4);  // lanes past the row compute on its last features and store nothing
    const int kk = ke + S;
    const long row = (long)b * D + d;
    const int *pi = pair_idx + (long)b * kk;
    const float *gt = gates + (long)b * ke;
    const bool rbf = resid && resid_dt == DL_BF16, rf32 = resid && resid_dt != DL_BF16;
    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
    bool first = true;
    for (int j0 = 0; j0 < max(kk, 1); j0 += 64) {
        // pair indices and gates j0 .. j0 + 63, one per lane (with no pairs at all: any readable words, unused)
        const int qv = kk > 0 ? pi[min(j0 + lane, kk - 1)] : 0;
        const float gv = ke > 0 ? gt[min(j0 + lane, ke - 1)] : 0.f;
        if (first) {
            // the residual, loaded after the indices so that one wait covers both, and taken into the sum first
            const uint2 r16 = *(const uint2 *)((rbf ? (const uint16_t *)resid : (const uint16_t *)F) + row);
            const v4f r32 = *(const v4f *)((rf32 ? (const float *)resid : F) + row);
            const v4f a16 = v4f{__uint_as_float(r16.x << 16), __uint_as_float(r16.x & 0xFFFF0000u),
                                __uint_as_float(r16.y << 16), __uint_as_float(r16.y & 0xFFFF0000u)};
            acc = rbf ? a16 : rf32 ? r32 : acc;
            first = false;
        }
        for (int j1 = j0; j1 < min(kk, j0 + 64); j1 += PU) {
            v4f f[PU], f2[PU];
            int q[PU];
            // the indices read back from their lanes (all shuffles first, then one wait), then every load
            // unconditional (a missing pair reads pair 0's row and is dropped below)
#pragma unroll
            for (int u = 0; u < PU; u++) q[u] = __shfl(qv, min(j1 + u - j0, 63), 64);
#pragma unroll
            for (int u = 0; u < PU; u++) q[u] = j1 + u < kk ? q[u] : -1;  // -1: past the slots, or elsewhere
#pragma unroll
            for (int u = 0; u < PU; u++) {
                f[u] = *(const v4f *)(F + (long)max(q[u], 0) * D + d);
                f2[u] = *(const v4f *)(F + (nslot > 1 ? fstride : 0) + (long)max(q[u], 0) * D + d);
            }
            if (nslot > 1)
#pragma unroll
                for (int u = 0; u < PU; u++) f[u] += f2[u];
            for (int k = 2; k < nslot; k++) {
                v4f f3[PU];
#pragma unroll
                for (int u = 0; u < PU; u++) f3[u] = *(const v4f *)(F + k * fstride + (long)max(q[u], 0) * D + d);
#pragma unroll
                for (int u = 0; u < PU; u++) f[u] += f3[u];
            }
#pragma unroll
            for (int u = 0; u < PU; u++) {
                const int j = j1 + u;
                const float g = __shfl(gv, min(j - j0, 63), 64);
                if (q[u] >= 0) {
                    if (j < ke) {
                        acc.x = fmaf(g, f[u].x, acc.x); acc.y = fmaf(g, f[u].y, acc.y);
                        acc.z = fmaf(g, f[u].z, acc.z); acc.w = fmaf(g, f[u].w, acc.w);
                    } else acc += f[u];
                }
            }
        }
    }
    if (!dv) return;
    if (out32) *(v4f *)(out32 + row) = acc;
    if (out_dt == DL_BF16) {
        uint2 o;
        o.x = (uint32_t)f32_to_bf16(acc.x) | ((uint32_t)f32_to_bf16(acc.y) << 16);
        o.y = (uint32_t)f32_to_bf16(acc.z) | ((uint32_t)f32_to_bf16(acc.w) << 16);
        *(uint2 *)((uint16_t *)out + row) = o;
    } else *(v4f *)((float *)out + row) = acc;
}

int launch_combine(const float *F, int nslot, long fstride, const MoePlan &p, const float *gates, int B, int D, int ke,
                   int S,
                   const void *resid, int resid_dt, void *out, int out_dt, float *out32, hipStream_t s)
{
    dim3 g((D / 4 + 255) / 256, B);
    hipLaunchKernelGGL(k_combine, g, dim3(256), 0, s, F, nslot, fstride, p.pair_idx, gates, B, D, ke, S, resid, resid_dt, out, out_dt,
                       out32);
    return hip_check("combine");
}

}  // namespace dl
