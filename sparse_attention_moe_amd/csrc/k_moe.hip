// S6 + S7 + combine: router, dispatch plan and the fixed-order sum of expert outputs.
//
// The model routes every token to 8 experts plus a shared one (Introducing Kiln, "How was Kiln
// measured against vLLM on H200?"); its expert kernel applies each expert once to all of its tokens
// ("A collective costs per graph, so the graphs got big") from a routing plan, and experts without
// tokens are skipped ("What moved the number ...").  Router logits accumulate fp32 products in fp64
// so the expert choice matches an exact evaluation except for genuinely near-equal logits.
#include "dl_common.h"
#include "dl_internal.h"

namespace dl {

static constexpr int ROUTE_EXP = 4;   // experts per wave
static constexpr int ROUTE_TB = 4;    // tokens per pass of a wave
static constexpr int ROUTE_KC = 512;  // hidden features per wave (8 per lane)
static constexpr int ROUTE_MAXC = 32; // chunks: hidden size <= 16,384

// Partial router logits: part[c, b, e] = sum over hidden chunk c of w_r[e, d] * h[b, d], with the fp32
// products formed exactly in fp64 and summed in fp64.  One wave per (4 experts, chunk); each lane owns 8
// consecutive features, holds the 4 experts' weights in fp32 and walks the tokens 4 at a time.
__global__ __launch_bounds__(64) void k_route_partial(const float *__restrict__ h, int B, int D,
                                                      const float *__restrict__ wr, int E,
                                                      double *__restrict__ part)
{
    const int lane = threadIdx.x;
    const int e0 = blockIdx.x * ROUTE_EXP;
    const int c = blockIdx.y;
    const int d0 = c * ROUTE_KC + lane * 8;
    v4f w[ROUTE_EXP][2];
#pragma unroll
    for (int x = 0; x < ROUTE_EXP; x++)
#pragma unroll
        for (int q = 0; q < 2; q++) {
            const int e = e0 + x, d = d0 + q * 4;
            w[x][q] = (e < E && d < D) ? *(const v4f *)(wr + (long)e * D + d) : v4f{0.f, 0.f, 0.f, 0.f};
        }
    for (int b0 = 0; b0 < B; b0 += ROUTE_TB) {
        v4f hv[ROUTE_TB][2];
#pragma unroll
        for (int t = 0; t < ROUTE_TB; t++)
#pragma unroll
            for (int q = 0; q < 2; q++) {
                const int d = d0 + q * 4;
                hv[t][q] = (b0 + t < B && d < D) ? *(const v4f *)(h + (long)(b0 + t) * D + d) : v4f{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
        for (int x = 0; x < ROUTE_EXP; x++)
#pragma unroll
            for (int t = 0; t < ROUTE_TB; t++) {
                double acc = 0.0;
#pragma unroll
                for (int q = 0; q < 2; q++)
#pragma unroll
                    for (int i = 0; i < 4; i++) acc = fma((double)w[x][q][i], (double)hv[t][q][i], acc);
                acc = wave_sum_d(acc);
                if (lane == 0 && e0 + x < E && b0 + t < B) part[((long)c * B + b0 + t) * E + e0 + x] = acc;
            }
    }
}

// Top-k of one token's logits by (logit desc, id asc) in one wave: each lane owns experts lane + 64 i;
// ke rounds of a wave argmax, the owner retiring its pick.  Lane j < ke returns pick j and its softmax
// gate over the picked logits.  (Shared by the routing entry point and the fused router + plan kernel.)
template <int NSLOT>
__device__ __forceinline__ void token_topk(const double *__restrict__ lrow, int E, int ke, int &my_e, float &my_gate)
{
    const int lane = threadIdx.x & 63;
    double l[NSLOT];
#pragma unroll
    for (int i = 0; i < NSLOT; i++) {
        const int e = lane + 64 * i;
        l[i] = e < E ? lrow[e] : -INFINITY;
    }
    double top0 = 0.0, z = 0.0, my_g = 0.0;
    my_e = 0;
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
        if (j == 0) top0 = best;
        const double g = exp(best - top0);
        z += g;
        if (lane == j) { my_g = g; my_e = be; }
    }
    my_gate = (float)(my_g / z);
}

// logits64[b, e] = chunk partials summed in chunk order + bias (all threads), then one wave per token.
template <int NSLOT>
__global__ __launch_bounds__(256) void k_route_topk(const double *__restrict__ part, int nchunk, int B, int E, int ke,
                                                    const float *__restrict__ bias, int32_t *__restrict__ experts,
                                                    float *__restrict__ gates, float *__restrict__ logits,
                                                    double *__restrict__ logits64)
{
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (b >= B) return;
    double *l = logits64 + (long)b * E;
    for (int e = lane; e < E; e += 64) {
        double pc[ROUTE_MAXC];
#pragma unroll
        for (int c = 0; c < ROUTE_MAXC; c++) pc[c] = c < nchunk ? part[((long)c * B + b) * E + e] : 0.0;
        double v = 0.0;
#pragma unroll
        for (int c = 0; c < ROUTE_MAXC; c++)
            if (c < nchunk) v += pc[c];
        if (bias) v += (double)bias[e];
        l[e] = v;
        if (logits) logits[(long)b * E + e] = (float)v;
    }
    // each lane reads back only the logits it wrote itself (same thread, same addresses)
    int me;
    float mg;
    token_topk<NSLOT>(l, E, ke, me, mg);
    if (lane < ke) {
        experts[(long)b * ke + lane] = me;
        gates[(long)b * ke + lane] = mg;
    }
}

// Dispatch plan in one workgroup: active experts in ascending id (shared experts last), each
// expert's tokens in ascending order, and the pair index of every (token, slot).
__global__ __launch_bounds__(1024) void k_plan(const int32_t *__restrict__ experts, int B, int ke, int E, int S,
                                               int *__restrict__ n_active, int *__restrict__ n_pairs,
                                               int *__restrict__ n_groups,
                                               int *__restrict__ active, int *__restrict__ tok_off,
                                               int *__restrict__ tok_cnt, int *__restrict__ pair_tok,
                                               int *__restrict__ pair_idx)
{
    __shared__ int s_cnt[4096];
    __shared__ int s_scan[1024];
    __shared__ int s_exp[16384];
    const int tid = threadIdx.x;
    const int nT = 1024;
    const int per = (E + nT - 1) / nT;
    const int kk = ke + S;
    // tokens per routed expert
    for (int e = tid; e < E; e += nT) s_cnt[e] = 0;
    __syncthreads();
    for (int i = tid; i < B * ke; i += nT) {
        const int e = experts[i];
        s_exp[i] = e;
        atomicAdd(&s_cnt[e], 1);
    }
    __syncthreads();
    // thread t owns experts [t*per, (t+1)*per): count its active experts and pairs
    int na = 0, np = 0;
    for (int i = 0; i < per; i++) {
        const int e = tid * per + i;
        if (e < E && s_cnt[e] > 0) { na++; np += s_cnt[e]; }
    }
    // exclusive scans of the active-expert and pair counts
    s_scan[tid] = na;
    __syncthreads();
    for (int o = 1; o < nT; o <<= 1) {
        const int v = tid >= o ? s_scan[tid - o] : 0;
        __syncthreads();
        s_scan[tid] += v;
        __syncthreads();
    }
    const int a0 = s_scan[tid] - na;
    const int na_tot = s_scan[nT - 1];
    __syncthreads();
    s_scan[tid] = np;
    __syncthreads();
    for (int o = 1; o < nT; o <<= 1) {
        const int v = tid >= o ? s_scan[tid - o] : 0;
        __syncthreads();
        s_scan[tid] += v;
        __syncthreads();
    }
    int p0 = s_scan[tid] - np;
    int a = a0;
    for (int i = 0; i < per; i++) {
        const int e = tid * per + i;
        if (e >= E || s_cnt[e] == 0) continue;
        active[a] = e;
        tok_off[a] = p0;
        tok_cnt[a] = s_cnt[e];
        int p = p0;
        for (int b = 0; b < B; b++)
            for (int j = 0; j < ke; j++)
                if (s_exp[b * ke + j] == e) {
                    pair_tok[p] = b;
                    pair_idx[(long)b * kk + j] = p;
                    p++;
                }
        p0 = p;
        a++;
    }
    // shared experts: every token, after all routed pairs
    const int routed_pairs = B * ke;
    for (int i = tid; i < S * B; i += nT) {
        const int s = i / B, b = i % B;
        const int p = routed_pairs + s * B + b;
        pair_tok[p] = b;
        pair_idx[(long)b * kk + ke + s] = p;
    }
    if (tid < S) {
        active[na_tot + tid] = E + tid;
        tok_off[na_tot + tid] = routed_pairs + tid * B;
        tok_cnt[na_tot + tid] = B;
    }
    // largest token group count over the active experts (shared experts have B tokens)
    int mx = S > 0 ? B : 0;
    for (int e = tid; e < E; e += nT) mx = max(mx, s_cnt[e]);
    mx = wave_max_i(mx);
    __syncthreads();
    if ((tid & 63) == 0) s_scan[tid >> 6] = mx;
    __syncthreads();
    if (tid == 0) {
        int m2 = 0;
        for (int w = 0; w < nT / 64; w++) m2 = max(m2, s_scan[w]);
        *n_active = na_tot + S;
        *n_pairs = routed_pairs + S * B;
        *n_groups = (m2 + 15) / 16;
    }
}

// Router top-k fused with the dispatch plan, one workgroup of 1024 threads:
//   1. wave w takes tokens b = w, w + 16, ...: each lane owns experts e = lane + 64 i (i < 16), whose logit is
//      the sum of the chunk partials (in chunk order) plus the bias; ke rounds of a wave argmax by
//      (logit desc, id asc) pick the experts; gates are the softmax over the picked logits.
//   2. the plan, exactly as k_plan, from the picked experts kept in LDS.
static constexpr int RP_MAXE = 1024;

// Exclusive scan of one int over the 1024 threads (16 waves); also returns the total.
__device__ __forceinline__ int block_excl_scan_1024(int v, int *s_w, int &total)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(inc, o, 64);
        if (lane >= o) inc += t;
    }
    __syncthreads();
    if (lane == 63) s_w[wv] = inc;
    __syncthreads();
    int before = 0;
    total = 0;
    for (int w = 0; w < 16; w++) {
        const int x = s_w[w];
        if (w < wv) before += x;
        total += x;
    }
    return before + inc - v;
}

template <int NSLOT>  // experts per lane: E <= 64 * NSLOT
__global__ __launch_bounds__(1024) void k_route_plan(const double *__restrict__ part, int nchunk, int B, int E, int ke,
                                                     int S, const float *__restrict__ bias,
                                                     double *__restrict__ logits64, int32_t *__restrict__ experts,
                                                     float *__restrict__ gates, float *__restrict__ logits,
                                                     int *__restrict__ n_active, int *__restrict__ n_pairs,
                                                     int *__restrict__ n_groups, int *__restrict__ active,
                                                     int *__restrict__ tok_off, int *__restrict__ tok_cnt,
                                                     int *__restrict__ pair_tok, int *__restrict__ pair_idx)
{
    __shared__ int s_cnt[RP_MAXE];
    __shared__ int s_w[16];
    __shared__ int s_exp[16384];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nT = 1024;
    const int kk = ke + S;
    for (int e = tid; e < E; e += nT) s_cnt[e] = 0;
    // 1. logits = chunk partials summed in chunk order, plus the bias
    for (int i = tid; i < B * E; i += nT) {
        const int b = i / E, e = i % E;
        double pc[ROUTE_MAXC];  // every chunk's partial in flight at once, then summed in chunk order
#pragma unroll
        for (int c = 0; c < ROUTE_MAXC; c++) pc[c] = c < nchunk ? part[((long)c * B + b) * E + e] : 0.0;
        double v = 0.0;
#pragma unroll
        for (int c = 0; c < ROUTE_MAXC; c++)
            if (c < nchunk) v += pc[c];
        if (bias) v += (double)bias[e];
        logits64[i] = v;
        if (logits) logits[i] = (float)v;
    }
    __syncthreads();
    // 2. per token: the picked experts and gates
    for (int b = wv; b < B; b += 16) {
        int me;
        float mg;
        token_topk<NSLOT>(logits64 + (long)b * E, E, ke, me, mg);
        if (lane < ke) {
            experts[(long)b * ke + lane] = me;
            gates[(long)b * ke + lane] = mg;
            s_exp[b * ke + lane] = me;
        }
    }
    __syncthreads();
    // 3. dispatch plan (same rules as k_plan)
    for (int i = tid; i < B * ke; i += nT) atomicAdd(&s_cnt[s_exp[i]], 1);
    __syncthreads();
    const int per = (E + nT - 1) / nT;
    int na = 0, np = 0;
    for (int i = 0; i < per; i++) {
        const int e = tid * per + i;
        if (e < E && s_cnt[e] > 0) { na++; np += s_cnt[e]; }
    }
    int na_tot, np_tot;
    const int a0 = block_excl_scan_1024(na, s_w, na_tot);
    int p0 = block_excl_scan_1024(np, s_w, np_tot);
    int a = a0;
    for (int i = 0; i < per; i++) {
        const int e = tid * per + i;
        if (e >= E || s_cnt[e] == 0) continue;
        active[a] = e;
        tok_off[a] = p0;
        tok_cnt[a] = s_cnt[e];
        int p = p0;
        for (int b = 0; b < B; b++)
            for (int j = 0; j < ke; j++)
                if (s_exp[b * ke + j] == e) {
                    pair_tok[p] = b;
                    pair_idx[(long)b * kk + j] = p;
                    p++;
                }
        p0 = p;
        a++;
    }
    const int routed_pairs = B * ke;
    for (int i = tid; i < S * B; i += nT) {
        const int s2 = i / B, b = i % B;
        const int p = routed_pairs + s2 * B + b;
        pair_tok[p] = b;
        pair_idx[(long)b * kk + ke + s2] = p;
    }
    if (tid < S) {
        active[na_tot + tid] = E + tid;
        tok_off[na_tot + tid] = routed_pairs + tid * B;
        tok_cnt[na_tot + tid] = B;
    }
    int mx = S > 0 ? B : 0;
    for (int e = tid; e < E; e += nT) mx = max(mx, s_cnt[e]);
    mx = wave_max_i(mx);
    __syncthreads();
    if (lane == 0) s_w[wv] = mx;
    __syncthreads();
    if (tid == 0) {
        int m2 = 0;
        for (int w = 0; w < 16; w++) m2 = max(m2, s_w[w]);
        *n_active = na_tot + S;
        *n_pairs = routed_pairs + S * B;
        *n_groups = (m2 + 15) / 16;
    }
}

// out[b, d] = resid[b, d] + sum_j gate[b, j] f_j[d] + sum_s f_s[d], in that order.  A thread owns 4
// consecutive features of one token; the token's pair indices and gates are wave-uniform (scalar loads), and
// the expert outputs are fetched 8 slots at a time so their loads are in flight together.
__global__ __launch_bounds__(256) void k_combine(const float *__restrict__ F, const int *__restrict__ pair_idx,
                                                 const float *__restrict__ gates, int B, int D, int ke, int S,
                                                 const void *__restrict__ resid, int resid_dt, void *__restrict__ out,
                                                 int out_dt, float *__restrict__ out32)
{
    const int b = blockIdx.y;
    const int d = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (d >= D) return;
    const int kk = ke + S;
    const long row = (long)b * D + d;
    v4f acc;
    if (!resid) acc = v4f{0.f, 0.f, 0.f, 0.f};
    else if (resid_dt == DL_BF16) {
        const uint2 r = *(const uint2 *)((const uint16_t *)resid + row);
        acc = v4f{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xFFFF0000u), __uint_as_float(r.y << 16),
                  __uint_as_float(r.y & 0xFFFF0000u)};
    } else acc = *(const v4f *)((const float *)resid + row);
    const int *pi = pair_idx + (long)b * kk;
    const float *gt = gates + (long)b * ke;
    for (int j0 = 0; j0 < kk; j0 += 8) {
        v4f f[8];
#pragma unroll
        for (int u = 0; u < 8; u++)
            if (j0 + u < kk) f[u] = *(const v4f *)(F + (long)pi[j0 + u] * D + d);
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const int j = j0 + u;
            if (j < kk) {
                if (j < ke) {
                    const float g = gt[j];
                    acc.x = fmaf(g, f[u].x, acc.x); acc.y = fmaf(g, f[u].y, acc.y);
                    acc.z = fmaf(g, f[u].z, acc.z); acc.w = fmaf(g, f[u].w, acc.w);
                } else acc += f[u];
            }
        }
    }
    if (out32) *(v4f *)(out32 + row) = acc;
    if (out_dt == DL_BF16) {
        uint2 o;
        o.x = (uint32_t)f32_to_bf16(acc.x) | ((uint32_t)f32_to_bf16(acc.y) << 16);
        o.y = (uint32_t)f32_to_bf16(acc.z) | ((uint32_t)f32_to_bf16(acc.w) << 16);
        *(uint2 *)((uint16_t *)out + row) = o;
    } else *(v4f *)((float *)out + row) = acc;
}

int route_chunks(int D) { return (D + ROUTE_KC - 1) / ROUTE_KC; }

int launch_route(const float *h, int B, int D, const float *w_r, const float *bias, int E, int ke, int32_t *experts,
                 float *gates, float *logits, double *logits64, double *part, hipStream_t s)
{
    const int nc = route_chunks(D);
    dim3 g((E + ROUTE_EXP - 1) / ROUTE_EXP, nc);
    hipLaunchKernelGGL(k_route_partial, g, dim3(64), 0, s, h, B, D, w_r, E, part);
    if (E <= 256)
        hipLaunchKernelGGL((k_route_topk<4>), dim3((B + 3) / 4), dim3(256), 0, s, part, nc, B, E, ke, bias, experts,
                           gates, logits, logits64);
    else
        hipLaunchKernelGGL((k_route_topk<16>), dim3((B + 3) / 4), dim3(256), 0, s, part, nc, B, E, ke, bias, experts,
                           gates, logits, logits64);
    return hip_check("route");
}

bool route_plan_ok(int E, int ke, int B) { return E <= RP_MAXE && ke <= 32 && (long)B * ke <= 16384; }

int launch_route_partial(const float *h, int B, int D, const float *w_r, int E, double *part, hipStream_t s)
{
    dim3 g((E + ROUTE_EXP - 1) / ROUTE_EXP, route_chunks(D));
    hipLaunchKernelGGL(k_route_partial, g, dim3(64), 0, s, h, B, D, w_r, E, part);
    return hip_check("route_partial");
}

int launch_route_plan(const double *part, int B, int D, const float *bias, int E, int ke, int S, int32_t *experts,
                      float *gates, float *logits, double *logits64, const MoePlan &p, hipStream_t s)
{
#define DL_RP(NS_)                                                                                                  \
    hipLaunchKernelGGL((k_route_plan<NS_>), dim3(1), dim3(1024), 0, s, part, route_chunks(D), B, E, ke, S, bias,     \
                       logits64, experts, gates, logits, p.n_active, p.n_pairs, p.n_groups, p.active, p.tok_off,     \
                       p.tok_cnt, p.pair_tok, p.pair_idx)
    if (E <= 256) DL_RP(4); else DL_RP(16);
#undef DL_RP
    return hip_check("route_plan");
}

int launch_plan(const int32_t *experts, int B, int ke, int E, int S, const MoePlan &p, hipStream_t s)
{
    hipLaunchKernelGGL(k_plan, dim3(1), dim3(1024), 0, s, experts, B, ke, E, S, p.n_active, p.n_pairs, p.n_groups,
                       p.active,
                       p.tok_off, p.tok_cnt, p.pair_tok, p.pair_idx);
    return hip_check("plan");
}

int launch_combine(const float *F, const MoePlan &p, const float *gates, int B, int D, int ke, int S,
                   const void *resid, int resid_dt, void *out, int out_dt, float *out32, hipStream_t s)
{
    dim3 g((D / 4 + 255) / 256, B);
    hipLaunchKernelGGL(k_combine, g, dim3(256), 0, s, F, p.pair_idx, gates, B, D, ke, S, resid, resid_dt, out, out_dt,
                       out32);
    return hip_check("combine");
}

}  // namespace dl
