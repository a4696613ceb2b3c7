// Weight-streaming GEMV engine for FP8 block-scaled weights (W_UV, W_O, expert gate/up/down).
//
// The weights are OCP e4m3fn codes with one fp32 scale per 128 x 128 block ("FP8 weights with
// 128 x 128 block scales", Introducing Kiln, "How was Kiln measured against vLLM on H200?").  Kiln
// aligned each block with a kernel tile so one scale serves the tile ("Expert parallelism without an
// all-to-all", per-tile dequantisation).  Here a wave owns 16 weight rows and walks K in 128-wide
// blocks: each block is exactly one v_mfma_f32_16x16x128_f8f6f4 on the raw codes, and the block's
// partial sums are scaled once — the codes are never decoded on the vector units.
//
// The activations (up to 16 tokens per pass, the N side of the instruction) enter as NS FP8 parts:
// part 0 is the value rounded to e4m3 with a per-(row, 128-block) scale, part s the remainder of
// parts < s with its own scale.  Two parts carry about 10 significant bits, four about 16, so the
// projections ahead of the router keep near-fp32 accuracy while the expert FFN uses two.
//
// Work items are (active matrix, 16-row tile, group of 16 tokens); matrices and tokens can come
// from a device-side plan (experts with no token are simply absent: the MoE tile skip of Kiln's
// "What moved the number ..." section).  Waves take items round-robin; every weight byte is read
// once with 16-byte loads.
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

struct ItemInfo {
    int m, off, cnt, t0, r0;
};

__device__ __forceinline__ bool decode_item(const GemvArgs &a, long item, int tiles, ItemInfo &it)
{
    const int g = (int)(item % a.max_groups);
    const long t2 = item / a.max_groups;
    const int tile = (int)(t2 % tiles);
    const int u = (int)(t2 / tiles);
    it.m = a.active ? a.active[u] : u;
    if (a.tok_cnt) {
        it.cnt = a.tok_cnt[u];
        it.off = a.tok_off[u];
    } else {
        it.cnt = a.ntok_host;
        it.off = 0;
    }
    it.t0 = g * 16;
    it.r0 = tile * 16;
    return it.t0 < it.cnt;
}

template <int NS, int EPI>
__global__ __launch_bounds__(256) void k_gemv_fp8(GemvArgs a)
{
    constexpr bool SW = EPI == EPI_SWIGLU;
    const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nwaves = gridDim.x * 4;
    const int n_act = a.n_active_dev ? *a.n_active_dev : a.n_active_host;
    const int tiles = a.rows >> 4;
    const long total = (long)n_act * tiles * a.max_groups * a.ksplit;
    for (long item0 = wave; item0 < total; item0 += nwaves) {
        const int kc = (int)(item0 % a.ksplit);
        const long item = item0 / a.ksplit;
        ItemInfo it;
        if (!decode_item(a, item, tiles, it)) continue;
        const int kb0 = kc * a.kchunk, kb1 = min(a.nkb, kb0 + a.kchunk);
        const int tt = it.t0 + ln;
        const bool tv = tt < it.cnt;
        long arow = 0;
        if (tv) arow = a.pair_act ? a.pair_act[it.off + tt] : a.tok_cnt ? (long)(it.off + tt) : (long)tt * a.a_ts + (long)it.m * a.a_ms;
        const long wrow = (long)it.m * a.mat_elems + (long)(it.r0 + ln) * a.cols + lg * 32;
        const uint8_t *wp = a.w + wrow;
        const uint8_t *wp2 = SW ? a.w2 + wrow : nullptr;
        const long sbase = ((long)it.m * a.nrb + (it.r0 >> 7)) * a.nkb;
        const float *wsp = a.wsc + sbase;
        const float *wsp2 = SW ? a.wsc2 + sbase : nullptr;
        const uint8_t *ap = a.aq + arow * a.cols + lg * 32;
        const float *asp = a.asc + arow * a.nkb;
        v4f tot = {0.f, 0.f, 0.f, 0.f}, tot2 = {0.f, 0.f, 0.f, 0.f};
        for (int kb = kb0; kb < kb1; kb++) {
            const v8i A = ld32(wp + kb * 128);
            v8i A2;
            if (SW) A2 = ld32(wp2 + kb * 128);
            v8i Bv[NS];
            float as[NS];
#pragma unroll
            for (int s = 0; s < NS; s++) {
                Bv[s] = tv ? ld32(ap + s * a.aq_part + kb * 128) : v8i{0, 0, 0, 0, 0, 0, 0, 0};
                as[s] = tv ? asp[s * a.asc_part + kb] : 0.f;
            }
            const float ws = wsp[kb];
            const float ws2 = SW ? wsp2[kb] : 0.f;
#pragma unroll
            for (int s = 0; s < NS; s++) {
                const v4f acc = mfma_fp8(A, Bv[s]);
                const float f = ws * as[s];
                tot += acc * f;
                if (SW) {
                    const v4f acc2 = mfma_fp8(A2, Bv[s]);
                    tot2 += acc2 * (ws2 * as[s]);
                }
            }
        }
        if (!tv) continue;
        const long ooff = a.tok_cnt ? (long)(it.off + tt) * a.o_ts : (long)tt * a.o_ts + (long)it.m * a.o_ms;
        if (a.ksplit > 1) {
            float *p = a.part + (long)kc * a.n_out + ooff + it.r0 + 4 * lg;
            *(v4f *)p = tot;
            if (SW) *(v4f *)(a.part2 + (long)kc * a.n_out + ooff + it.r0 + 4 * lg) = tot2;
            continue;
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int r = it.r0 + 4 * lg + i;
            float v = tot[i];
            if (EPI == EPI_RESID) v += act_load(a.resid, a.resid_dt, (long)tt * a.r_ts + r);
            if (SW) v = silu(v) * tot2[i];
            a.out[ooff + r] = v;
        }
    }
}

// Sum of the K-chunk partials in chunk order, then the epilogue.  EPI_RESID here needs the residual laid
// out like the output (r_ts == o_ts, uniform mode with one matrix).
template <int EPI>
__global__ __launch_bounds__(256) void k_gemv_reduce(GemvArgs a)
{
    constexpr bool SW = EPI == EPI_SWIGLU;
    const long e = (long)blockIdx.x * 256 + threadIdx.x;
    if (e >= a.n_out) return;
    float v = 0.f, v2 = 0.f;
    for (int kc = 0; kc < a.ksplit; kc++) {
        v += a.part[(long)kc * a.n_out + e];
        if (SW) v2 += a.part2[(long)kc * a.n_out + e];
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
            if (t >= nt) break;
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
        float r0 = v.x, r1 = v.y;
#pragma unroll
        for (int s = 0; s < NS; s++) {
            const float amax = wave_max(fmaxf(fabsf(r0), fabsf(r1)));
            const float scale = amax > 0.f ? amax * (1.0f / 448.0f) : 1.0f;
            const float inv = 1.0f / scale;
            const float c0 = fminf(fmaxf(r0 * inv, -448.f), 448.f);
            const float c1 = fminf(fmaxf(r1 * inv, -448.f), 448.f);
            const uint32_t code = f32x2_to_fp8(c0, c1);
            *(uint16_t *)(q + s * q_part + e) = (uint16_t)code;
            if (lane == 0) sc[s * sc_part + row * nkb + kb] = scale;
            const v2f d = fp8x2_lo(code);
            r0 -= d.x * scale;
            r1 -= d.y * scale;
        }
    }
}

static int grid_for(long items, int per_block_waves = 4, int max_blocks = 8192)
{
    long b = (items + per_block_waves - 1) / per_block_waves;
    if (b < 1) b = 1;
    if (b > max_blocks) b = max_blocks;
    return (int)b;
}

int launch_gemv(const GemvArgs &a, int ns, int epi, bool fp8, hipStream_t s)
{
    // upper bound of the item count (device-side counts can only be smaller)
    const long n_act = a.n_active_host;
    if (fp8) {
        const long items = n_act * (a.rows / 16) * a.max_groups * a.ksplit;
        const dim3 g(grid_for(items, 4, 2048));
        bool done = false;
#define DL_G(NS_, E_) \
    if (!done && ns == NS_ && epi == E_) { hipLaunchKernelGGL((k_gemv_fp8<NS_, E_>), g, dim3(256), 0, s, a); done = true; }
        DL_G(2, EPI_STORE) DL_G(2, EPI_RESID) DL_G(2, EPI_SWIGLU)
        DL_G(4, EPI_STORE) DL_G(4, EPI_RESID) DL_G(4, EPI_SWIGLU)
#undef DL_G
        if (!done) return fail(DL_ERR_UNSUPPORTED, "gemv parts=%d", ns);
        if (a.ksplit > 1) {
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
