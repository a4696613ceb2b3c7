// S3 + S4: sparse MLA decode attention over the kept positions only.
//
// Kiln's decode kernel gathers the selected entries instead of masking every key ("The decode
// kernels, and why they are opt-in", Introducing Kiln); the cache is one compressed latent per
// position shared by all heads ("How was Kiln measured against vLLM on H200?").  The key is the
// whole latent (d_c features), the value its first d_v features.
//
// A workgroup owns HG heads of one row: it resolves the page of every kept position once, scores
// all of them for its heads (each latent row is decoded once for HG heads), takes an exact fp32
// softmax, and accumulates the values with 4 consecutive features per thread.
#include "dl_common.h"
#include "dl_internal.h"

namespace dl {

static constexpr int ATT_HG = 4;
static constexpr int ATT_MAX_K = 4096;
static constexpr int ATT_MAX_DC = 1024;

// Decoded latent feature d of cache row `row` (FP8 code * block scale, or fp32).
__device__ __forceinline__ float lat(const void *kv, const float *ks, int fp8, long row, int Dc, int nb, int d)
{
    if (fp8) {
        const uint32_t c = ((const uint8_t *)kv)[row * Dc + d];
        return fp8x2_lo(c).x * ks[row * nb + (d >> 7)];
    }
    return ((const float *)kv)[row * Dc + d];
}

__global__ __launch_bounds__(256) void k_attn(const void *__restrict__ q, int q_dt, const void *__restrict__ kv,
                                              const float *__restrict__ ks, int fp8, const int32_t *__restrict__ pt,
                                              int max_pages, int ps_shift, const int32_t *__restrict__ sel, int top_k,
                                              int H, int Dc, int Dv, float sm_scale, float *__restrict__ o)
{
    __shared__ float s_q[ATT_HG][ATT_MAX_DC];
    __shared__ float s_p[ATT_HG][ATT_MAX_K];
    __shared__ long s_row[ATT_MAX_K];
    __shared__ float s_red[ATT_HG][8];
    const int b = blockIdx.y, h0 = blockIdx.x * ATT_HG;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nb = (Dc + 127) >> 7;
    const int ps_mask = (1 << ps_shift) - 1;
    const int hn = min(ATT_HG, H - h0);
    for (int i = tid; i < ATT_HG * Dc; i += 256) {
        const int hh = i / Dc, d = i % Dc;
        s_q[hh][d] = hh < hn ? act_load(q, q_dt, ((long)b * H + h0 + hh) * Dc + d) : 0.f;
    }
    for (int j = tid; j < top_k; j += 256) {
        const int p = sel[(long)b * top_k + j];
        s_row[j] = p < 0 ? -1 : ((long)pt[(long)b * max_pages + (p >> ps_shift)] << ps_shift) + (p & ps_mask);
    }
    __syncthreads();
    // logits
    float mx[ATT_HG];
#pragma unroll
    for (int hh = 0; hh < ATT_HG; hh++) mx[hh] = -INFINITY;
    for (int j = tid; j < top_k; j += 256) {
        const long row = s_row[j];
        float lgt[ATT_HG];
        if (row < 0) {
#pragma unroll
            for (int hh = 0; hh < ATT_HG; hh++) lgt[hh] = -INFINITY;
        } else {
            float acc[ATT_HG] = {};
            for (int blk = 0; blk < nb; blk++) {
                float part[ATT_HG] = {};
                const int dend = min(Dc, blk * 128 + 128);
                if (fp8) {
                    const uint8_t *cp = (const uint8_t *)kv + row * Dc;
                    for (int d = blk * 128; d < dend; d += 4) {
                        const uint32_t w = *(const uint32_t *)(cp + d);
                        const v2f lo = fp8x2_lo(w), hi = fp8x2_hi(w);
#pragma unroll
                        for (int hh = 0; hh < ATT_HG; hh++)
                            part[hh] += s_q[hh][d] * lo.x + s_q[hh][d + 1] * lo.y + s_q[hh][d + 2] * hi.x +
                                        s_q[hh][d + 3] * hi.y;
                    }
                    const float scl = ks[row * nb + blk];
#pragma unroll
                    for (int hh = 0; hh < ATT_HG; hh++) acc[hh] += part[hh] * scl;
                } else {
                    const float *cp = (const float *)kv + row * Dc;
                    for (int d = blk * 128; d < dend; d++) {
                        const float c = cp[d];
#pragma unroll
                        for (int hh = 0; hh < ATT_HG; hh++) acc[hh] += s_q[hh][d] * c;
                    }
                }
            }
#pragma unroll
            for (int hh = 0; hh < ATT_HG; hh++) lgt[hh] = acc[hh] * sm_scale;
        }
#pragma unroll
        for (int hh = 0; hh < ATT_HG; hh++) {
            s_p[hh][j] = lgt[hh];
            mx[hh] = fmaxf(mx[hh], lgt[hh]);
        }
    }
#pragma unroll
    for (int hh = 0; hh < ATT_HG; hh++) {
        float m = wave_max(mx[hh]);
        if (lane == 0) s_red[hh][wave] = m;
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < ATT_HG; hh++)
        mx[hh] = fmaxf(fmaxf(s_red[hh][0], s_red[hh][1]), fmaxf(s_red[hh][2], s_red[hh][3]));
    __syncthreads();
    float sm[ATT_HG] = {};
    for (int j = tid; j < top_k; j += 256) {
#pragma unroll
        for (int hh = 0; hh < ATT_HG; hh++) {
            const float lv = s_p[hh][j];
            const float e = (lv == -INFINITY) ? 0.f : expf(lv - mx[hh]);
            s_p[hh][j] = e;
            sm[hh] += e;
        }
    }
#pragma unroll
    for (int hh = 0; hh < ATT_HG; hh++) {
        float v = wave_sum(sm[hh]);
        if (lane == 0) s_red[hh][4 + wave] = v;
    }
    __syncthreads();
    float inv[ATT_HG];
#pragma unroll
    for (int hh = 0; hh < ATT_HG; hh++) {
        const float z = s_red[hh][4] + s_red[hh][5] + s_red[hh][6] + s_red[hh][7];
        inv[hh] = z > 0.f ? 1.0f / z : 0.f;
    }
    // values: thread -> 4 consecutive features, NSTR independent j streams
    const int nv4 = Dv >> 2;             // threads per stream
    const int nstr = 256 / nv4;          // streams
    const int v0 = (tid % nv4) * 4, str = tid / nv4;
    float acc[ATT_HG][4] = {};
    for (int j = str; j < top_k; j += nstr) {
        const long row = s_row[j];
        if (row < 0) continue;
        float c[4];
        if (fp8) {
            const uint32_t w = *(const uint32_t *)((const uint8_t *)kv + row * Dc + v0);
            const float scl = ks[row * nb + (v0 >> 7)];
            const v2f lo = fp8x2_lo(w), hi = fp8x2_hi(w);
            c[0] = lo.x * scl; c[1] = lo.y * scl; c[2] = hi.x * scl; c[3] = hi.y * scl;
        } else {
            const v4f w = *(const v4f *)((const float *)kv + row * Dc + v0);
            c[0] = w[0]; c[1] = w[1]; c[2] = w[2]; c[3] = w[3];
        }
#pragma unroll
        for (int hh = 0; hh < ATT_HG; hh++) {
            const float p = s_p[hh][j];
#pragma unroll
            for (int i = 0; i < 4; i++) acc[hh][i] = fmaf(p, c[i], acc[hh][i]);
        }
    }
    __syncthreads();
    // reduce the streams through LDS (reuse s_p)
    float *red = &s_p[0][0];  // [nstr][ATT_HG][Dv] <= 256*4*4 floats
#pragma unroll
    for (int hh = 0; hh < ATT_HG; hh++)
#pragma unroll
        for (int i = 0; i < 4; i++) red[((long)str * ATT_HG + hh) * Dv + v0 + i] = acc[hh][i];
    __syncthreads();
    for (int i = tid; i < hn * Dv; i += 256) {
        const int hh = i / Dv, v = i % Dv;
        float s = 0.f;
        for (int t = 0; t < nstr; t++) s += red[((long)t * ATT_HG + hh) * Dv + v];
        o[((long)b * H + h0 + hh) * Dv + v] = s * inv[hh];
    }
}

int launch_attention(const dl_pages &pg, const void *q, int q_dt, const void *kv, const float *kv_scale, int kv_dt,
                     int H, int Dc, int Dv, float sm_scale, const int32_t *sel, int top_k, float *o, hipStream_t s)
{
    if (top_k > ATT_MAX_K || Dc > ATT_MAX_DC) return fail(DL_ERR_UNSUPPORTED, "attention top_k %d / d_c %d", top_k, Dc);
    if (Dv % 4 || (256 % (Dv / 4))) return fail(DL_ERR_UNSUPPORTED, "attention d_v %d (power of two 4..1024)", Dv);
    if (Dc % 4) return fail(DL_ERR_UNSUPPORTED, "attention d_c %d", Dc);
    const int ps_shift = __builtin_ctz((unsigned)pg.page_size);
    dim3 g((H + ATT_HG - 1) / ATT_HG, pg.batch);
    hipLaunchKernelGGL(k_attn, g, dim3(256), 0, s, q, q_dt, kv, kv_scale, kv_dt == DL_FP8_E4M3 ? 1 : 0, pg.page_table,
                       pg.max_pages_per_seq, ps_shift, sel, top_k, H, Dc, Dv, sm_scale, o);
    return hip_check("attention");
}

}  // namespace dl
