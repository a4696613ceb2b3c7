// S3 + S4: sparse MLA decode attention over the kept positions only.
//
// Kiln's decode kernel gathers the selected entries instead of masking every key ("The decode
// kernels, and why they are opt-in", Introducing Kiln); the cache is one compressed latent per
// position shared by all heads ("How was Kiln measured against vLLM on H200?").  The key is the
// whole latent (d_c features), the value its first d_v features.
//
// Two kernels:
//  * k_attn_mla (FP8 latents, bf16 queries, 16 | heads): split over the kept positions like flash
//    decoding.  A workgroup owns one row, a run of kept positions and up to 64 heads (16 per wave), so
//    every kept latent is gathered once for all heads; positions are staged 64 at a time into LDS through
//    the page table.  Scores are [16 heads x 64] x [64 x d_c] products on the matrix cores
//    (v_mfma_f32_16x16x32_bf16): the queries are bf16 already and every e4m3 code is exactly a bf16, so the
//    products are exact and each 128-feature block's sum takes its scale once.  The softmax runs online in
//    fp32 inside each wave.  The values are transposed once per chunk into bf16 [feature][position] rows in
//    LDS, and O += P' C with P' = p * (block scale) split into bf16 high and low halves (about 16
//    significant bits), so the output keeps fp32-level accuracy.  The splits are merged afterwards
//    (max-rescaled sums).
//  * k_attn (any shape, fp32 or FP8 latents): a workgroup owns 4 heads of one row and scores every
//    kept position on the vector units in fp32.
#include "dl_common.h"
#include "dl_internal.h"

#include <algorithm>

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
                                              int max_pages, int R, int ps_shift, const int32_t *__restrict__ sel, int top_k,
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
        s_row[j] = p < 0 ? -1 : ((long)pt[(long)(b / R) * max_pages + (p >> ps_shift)] << ps_shift) + (p & ps_mask);
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


// ----------------------------------------------------------------------------- matrix-core path
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

static constexpr int AM_NJ = 64;        // kept positions per chunk
static constexpr int AM_MAXSPLIT = 32;  // splits of the kept positions
static constexpr int AM_MAXPPS = 512;   // kept positions per split (8 chunks)

// 8 e4m3 codes (two dwords) -> 8 bf16, exactly.
__device__ __forceinline__ v8bf fp8x8_to_bf16(uint32_t w0, uint32_t w1)
{
    const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
    const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
    const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
    const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
    return v8bf{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

__device__ __forceinline__ v4f mfma_bf16(v8bf a, v8bf b, v4f c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float max16(float v)
{
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float sum16(float v)
{
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Row-wide (16-lane) reductions on the DPP network: butterflies within quads, then rotations of the row;
// every lane of the row ends with the result.
__device__ __forceinline__ float dpp_f(float v, int ctrl_sel)
{
    switch (ctrl_sel) {
    case 0: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false));
    case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, false));
    case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false));
    default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));
    }
}
__device__ __forceinline__ float row_max16(float v)
{
#pragma unroll
    for (int c = 0; c < 4; c++) v = fmaxf(v, dpp_f(v, c));
    return v;
}
__device__ __forceinline__ float row_sum16(float v)
{
#pragma unroll
    for (int c = 0; c < 4; c++) v += dpp_f(v, c);
    return v;
}

// Byte transpose of four dwords: out[k] = (a.k, b.k, c.k, d.k).
__device__ __forceinline__ void tr4x4(uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t out[4])
{
    const uint32_t t0 = __builtin_amdgcn_perm(b, a, 0x05010400u), t1 = __builtin_amdgcn_perm(b, a, 0x07030602u);
    const uint32_t t2 = __builtin_amdgcn_perm(d, c, 0x05010400u), t3 = __builtin_amdgcn_perm(d, c, 0x07030602u);
    out[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
    out[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
    out[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
    out[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// grid (nsplit, ceil(H/64), B), 256 threads.  A workgroup owns one row, one run of kept positions (the split)
// and up to 64 heads: wave w takes heads 16 (4 blockIdx.y + w) .. +16, so each kept latent is gathered once
// for all heads.  Per chunk of 64 positions:
//   gather   the latent codes (through the page table), converted exactly to bf16 once, as [position][feature]
//            rows in LDS;
//   values   the first Dv features transposed once into [feature][position] rows (position groups XOR-swizzled
//            by the feature's 16-group);
//   scores   S = Q C^T on v_mfma_f32_16x16x32_bf16 (queries in registers), each 128-feature block's sum taking
//            its scale once;
//   softmax  online per head in fp32, entirely inside the wave (DPP row reductions);
//   output   O += P' C with P' = p * (block scale) in bf16 high and low halves (about 16 significant bits).
// P of each wave reuses the LDS of the bf16 latents once every wave's scores are done.
// opart [B, nsplit, H, Dv] holds the unnormalised sums, ml [B, nsplit, H, 2] the running (max, sum).
template <int KQ, int NVB, bool MULTI>  // MULTI: more than one chunk of 64 positions per split
__global__ __launch_bounds__(256, 1) void k_attn_mla(const uint16_t *__restrict__ q, const uint8_t *__restrict__ kv,
                                                     const float *__restrict__ ks, const int32_t *__restrict__ pt,
                                                     int max_pages, int R, int ps_shift, const int32_t *__restrict__ sel,
                                                     int top_k, int H, int pps, float sm_scale,
                                                     float *__restrict__ opart, float *__restrict__ ml)
{
    constexpr int Dc = KQ * 32, NB = (Dc + 127) / 128, Dv = NVB * 128;
    constexpr int CBP = Dc + 8;                         // bf16 latent row pitch
    constexpr int PP = AM_NJ + 8;                       // value row pitch (bf16)
    constexpr int NLD = (AM_NJ * (Dc / 16) + 255) / 256;  // 16-byte code loads per thread per chunk
    constexpr int CB_BYTES = AM_NJ * CBP * 2;
    constexpr int P_BYTES = 4 * 16 * (AM_NJ + 4) * 4;
    __shared__ __attribute__((aligned(16))) uint8_t s_cbuf[CB_BYTES > P_BYTES ? CB_BYTES : P_BYTES];
    __shared__ __attribute__((aligned(16))) __bf16 s_v[Dv * PP];
    __shared__ __attribute__((aligned(16))) float s_sc[NB][AM_NJ];
    __shared__ long s_row[AM_MAXPPS];
    __bf16 *s_cb = (__bf16 *)s_cbuf;                       // [position][CBP] bf16 latents
    float(*s_p)[16][AM_NJ + 4] = (float(*)[16][AM_NJ + 4])s_cbuf;  // [wave][head][position] after the scores
    const int split = blockIdx.x, b = blockIdx.z;
    const int nsplit = gridDim.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, ln = lane & 15, lg = lane >> 4;
    const int h0 = (blockIdx.y * 4 + w) * 16;
    const bool active = h0 < H;
    const int ps_mask = (1 << ps_shift) - 1;
    const int jbase = split * pps;
    // queries of this wave's 16 heads, as the A operand of every K step: head ln, features 32 kk + 8 lg .. + 8
    v8bf Aq[KQ];
#pragma unroll
    for (int kk = 0; kk < KQ; kk++)
        Aq[kk] = active ? *(const v8bf *)(q + ((long)b * H + h0 + ln) * Dc + kk * 32 + lg * 8) : v8bf{};
    for (int i = tid; i < pps; i += 256) {
        const int j = jbase + i;
        const int p = j < top_k ? sel[(long)b * top_k + j] : -1;
        s_row[i] = p < 0 ? -1 : ((long)pt[(long)(b / R) * max_pages + (p >> ps_shift)] << ps_shift) + (p & ps_mask);
    }
    const int nch = MULTI ? max(0, min(pps, top_k - jbase) + AM_NJ - 1) / AM_NJ : (jbase < top_k ? 1 : 0);
    // scores in log2 units: p = 2^(S - m) with S = sm_scale * log2(e) * q.c, so the exponentials are exp2
    const float sl2 = sm_scale * 1.4426950408889634f;
    float m[4], l[4];
    v4f acc[NVB][8];
#pragma unroll
    for (int i = 0; i < 4; i++) { m[i] = -INFINITY; l[i] = 0.f; }
#pragma unroll
    for (int vb = 0; vb < NVB; vb++)
#pragma unroll
        for (int t = 0; t < 8; t++) acc[vb][t] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int ch = 0; ch < nch; ch++) {
        const int cb = ch * AM_NJ;  // chunk base within the split
        __syncthreads();            // s_row is complete; the previous chunk's LDS reads are done
        // gather: 16 codes per load, converted to bf16 in registers, two 16-byte LDS writes
        {
            v4i R[NLD];
#pragma unroll
            for (int k = 0; k < NLD; k++) {
                const int id = k * 256 + tid;
                R[k] = v4i{0, 0, 0, 0};
                if (id < AM_NJ * (Dc / 16)) {
                    const long row = s_row[cb + id / (Dc / 16)];
                    if (row >= 0) R[k] = *(const v4i *)(kv + row * Dc + (id % (Dc / 16)) * 16);
                }
            }
            for (int i = tid; i < AM_NJ * NB; i += 256) {
                const int pos = i / NB, blk = i % NB;
                const long row = s_row[cb + pos];
                s_sc[blk][pos] = row < 0 ? 0.f : ks[row * NB + blk];
            }
#pragma unroll
            for (int k = 0; k < NLD; k++) {
                const int id = k * 256 + tid;
                if (id < AM_NJ * (Dc / 16)) {
                    __bf16 *dst = s_cb + (id / (Dc / 16)) * CBP + (id % (Dc / 16)) * 16;
                    *(v8bf *)dst = fp8x8_to_bf16((uint32_t)R[k][0], (uint32_t)R[k][1]);
                    *(v8bf *)(dst + 8) = fp8x8_to_bf16((uint32_t)R[k][2], (uint32_t)R[k][3]);
                }
            }
        }
        __syncthreads();
        // values: thread -> 8 features x 8 positions, transposed to [feature][position]
        for (int u = tid; u < (Dv / 8) * (AM_NJ / 8); u += 256) {
            const int fq = u % (Dv / 8), pg = u / (Dv / 8);
            v4i r[8];
#pragma unroll
            for (int e = 0; e < 8; e++) r[e] = *(const v4i *)(s_cb + (pg * 8 + e) * CBP + fq * 8);
#pragma unroll
            for (int k = 0; k < 8; k++) {
                const uint32_t sl = (k & 1) ? 0x07060302u : 0x05040100u;
                v4i o;
#pragma unroll
                for (int mm = 0; mm < 4; mm++)
                    o[mm] = (int)__builtin_amdgcn_perm((uint32_t)r[2 * mm + 1][k >> 1], (uint32_t)r[2 * mm][k >> 1], sl);
                const int f = fq * 8 + k;
                *(v4i *)(s_v + f * PP + ((pg ^ ((f >> 4) & 7)) << 3)) = o;
            }
        }
        // scores: S[j] = 16 heads x positions j*16 .. +16; lane holds heads 4 lg + i of position cb + j*16 + ln
        v4f S[4];
        if (active) {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const __bf16 *cr = s_cb + (j * 16 + ln) * CBP + lg * 8;
                v4f sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int blk = 0; blk < NB; blk++) {
                    v4f a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = blk * 4; kk < (blk * 4 + 4 < KQ ? blk * 4 + 4 : KQ); kk++)
                        a = mfma_bf16(Aq[kk], *(const v8bf *)(cr + kk * 32), a);
                    sacc += a * s_sc[blk][j * 16 + ln];
                }
                const bool valid = s_row[cb + j * 16 + ln] >= 0;
#pragma unroll
                for (int i = 0; i < 4; i++) S[j][i] = valid ? sacc[i] * sl2 : -INFINITY;
            }
        }
        __syncthreads();  // every wave's scores are done: the latent rows become P; the values are complete
        if (!active) continue;
        // online softmax per head (row 4 lg + i), within the wave
        float alpha[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float mc = row_max16(fmaxf(fmaxf(S[0][i], S[1][i]), fmaxf(S[2][i], S[3][i])));
            const float mn = fmaxf(m[i], mc);
            alpha[i] = mn == -INFINITY ? 1.f : exp2f(m[i] - mn);
            m[i] = mn;
            float ps = 0.f;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float pv = S[j][i] == -INFINITY ? 0.f : exp2f(S[j][i] - mn);
                s_p[w][4 * lg + i][j * 16 + ln] = pv;
                ps += pv;
            }
            l[i] = l[i] * alpha[i] + row_sum16(ps);
        }
        if (MULTI && ch > 0) {  // rescale the running sums (still zero in the first chunk)
#pragma unroll
            for (int vb = 0; vb < NVB; vb++)
#pragma unroll
                for (int t = 0; t < 8; t++)
#pragma unroll
                    for (int i = 0; i < 4; i++) acc[vb][t][i] *= alpha[i];
        }
        // O += P' C over two K steps of 32 positions: A = P' (head ln, positions 8 lg .. + 8), B = values
        // (feature 16 t + ln of block vb, the same positions)
#pragma unroll
        for (int kstep = 0; kstep < 2; kstep++) {
            const int pl = kstep * 32 + lg * 8;  // first position of this lane's K group (within the chunk)
            const v4f p0 = *(const v4f *)&s_p[w][ln][pl], p1 = *(const v4f *)&s_p[w][ln][pl + 4];
            const float pr[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
#pragma unroll
            for (int vb = 0; vb < NVB; vb++) {
                const v4f c0 = *(const v4f *)&s_sc[vb][pl], c1 = *(const v4f *)&s_sc[vb][pl + 4];
                const float sc[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
                v8bf Ah, Al;
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const float x = pr[e] * sc[e];
                    const __bf16 hb = (__bf16)x;
                    Ah[e] = hb;
                    Al[e] = (__bf16)(x - (float)hb);
                }
#pragma unroll
                for (int t = 0; t < 8; t++) {
                    const int f = vb * 128 + t * 16 + ln;
                    const v8bf Bv = *(const v8bf *)(s_v + f * PP + (((kstep * 4 + lg) ^ ((vb * 8 + t) & 7)) << 3));
                    acc[vb][t] = mfma_bf16(Ah, Bv, acc[vb][t]);
                    acc[vb][t] = mfma_bf16(Al, Bv, acc[vb][t]);
                }
            }
        }
    }
    if (!active) return;
    // lane holds O[head h0 + 4 lg + i][feature vb*128 + 16 t + ln]; each 128-feature block goes through this
    // wave's P rows in LDS (free now) and out as 16-byte stores
    float *op = opart + (((long)b * nsplit + split) * H + h0) * Dv;
    float(*st)[AM_NJ + 4] = s_p[w];
#pragma unroll
    for (int vb = 0; vb < NVB; vb++) {
        // two halves of 64 features per pass (the rows hold 64 + 4 floats)
#pragma unroll
        for (int half = 0; half < 2; half++) {
#pragma unroll
            for (int t = 0; t < 4; t++)
#pragma unroll
                for (int i = 0; i < 4; i++) st[4 * lg + i][t * 16 + ln] = acc[vb][half * 4 + t][i];
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int head = r * 4 + lg, col = ln * 4;
                // streaming store: read once by the merge, so it should not sit dirty in the last-level
                // cache until the expert weight stream evicts it (its write-back would then compete with
                // that stream for HBM)
                __builtin_nontemporal_store(*(const v4f *)&st[head][col],
                                            (v4f *)(op + (long)head * Dv + vb * 128 + half * 64 + col));
            }
        }
    }
    if (ln == 0) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            float *m2 = ml + (((long)b * nsplit + split) * H + h0 + 4 * lg + i) * 2;
            m2[0] = m[i] * 0.6931471805599453f;  // natural-log units for the merge
            m2[1] = l[i];
        }
    }
}

// o[b, h, v] = sum_s e^(m_s - M) O_s[v] / sum_s e^(m_s - M) l_s, splits merged in order.
__global__ __launch_bounds__(256) void k_attn_merge(const float *__restrict__ opart, const float *__restrict__ ml,
                                                    int nsplit, int H, int Dv, float *__restrict__ o)
{
    const int bh = blockIdx.x;  // b*H + h
    const int b = bh / H, h = bh % H;
    // every split's (m, l) in flight at once; weights w_s = e^(m_s - M)
    float sm[AM_MAXSPLIT], sl[AM_MAXSPLIT];
#pragma unroll
    for (int s2 = 0; s2 < AM_MAXSPLIT; s2++) {
        const bool ok = s2 < nsplit;
        sm[s2] = ok ? ml[(((long)b * nsplit + s2) * H + h) * 2] : -INFINITY;
        sl[s2] = ok ? ml[(((long)b * nsplit + s2) * H + h) * 2 + 1] : 0.f;
    }
    float M = -INFINITY;
#pragma unroll
    for (int s2 = 0; s2 < AM_MAXSPLIT; s2++) M = fmaxf(M, sm[s2]);
    float den = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < AM_MAXSPLIT; s2++) {
        sm[s2] = sm[s2] == -INFINITY ? 0.f : expf(sm[s2] - M);  // weight of split s2 (0 if empty)
        den += sm[s2] * sl[s2];
    }
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    for (int v = threadIdx.x; v < Dv; v += 256) {
        float op[AM_MAXSPLIT];
#pragma unroll
        for (int s2 = 0; s2 < AM_MAXSPLIT; s2++)
            op[s2] = s2 < nsplit ? opart[(((long)b * nsplit + s2) * H + h) * Dv + v] : 0.f;
        float num = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < AM_MAXSPLIT; s2++)
            if (s2 < nsplit && sm[s2] != 0.f) num += sm[s2] * op[s2];
        o[(long)bh * Dv + v] = num * inv;
    }
}

// Split merge fused with the per-head value up-projection and its FP8 split: one workgroup per (row, head).
//   o      = merged attention output (also stored: [B, H, Dv])
//   u[r]   = sum_v W_UV[h][r][v] o[v]   on the vector units in fp32 (each code decoded exactly, one scale
//            per 128-column block), hd = 128 or 256 rows
//   uq, uqs: u split into NSU FP8 parts with one scale per (part, row b, 128-block) — the activation layout
//            the W_O pass reads ([part][B][H*hd] and [part][B][H*hd/128]).
// Every global load (split maxima and sums, the partial sums, the W_UV codes) is issued up front.  Threads
// take 4 features of one half of the splits; the halves meet in LDS.
template <int NSU>
__global__ __launch_bounds__(256) void k_attn_merge_uv(const float *__restrict__ opart, const float *__restrict__ ml,
                                                       int nsplit, int H, int Dv, float *__restrict__ o,
                                                       const uint8_t *__restrict__ wuv, const float *__restrict__ wsc,
                                                       int hd, int tiled, uint8_t *__restrict__ uq,
                                                       float *__restrict__ uqs, long uq_part, long uqs_part)
{
    constexpr int HS = AM_MAXSPLIT / 2;  // splits per half
    __shared__ __attribute__((aligned(16))) float s_half[2][1024];
    __shared__ float s_o[1024];
    __shared__ float s_u[256][2];
    __shared__ float s_wt[AM_MAXSPLIT];
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    // W_UV codes of this thread: row r, columns [c_lo, c_hi) (16 codes per load)
    const int nkb = Dv / 128, nrb = (hd + 127) / 128;
    const int per_row = 256 / hd;  // 2 (hd = 128) or 1 (hd = 256)
    const int r = tid / per_row, part = tid % per_row;
    // ncol <= 256 for every shape attention_merge_uv_ok admits (Dv <= 512 with two threads a row, Dv <= 256 with
    // one), so 16 code vectors a thread: 64 registers fewer than room for 512 columns, three workgroups a unit
    const int c_lo = part * (Dv / per_row), ncol = Dv / per_row;
    const uint8_t *wm = wuv + (long)h * hd * Dv;
    v4i wcode[16];
#pragma unroll
    for (int q = 0; q < 16; q++) {
        wcode[q] = v4i{0, 0, 0, 0};
        const int c = c_lo + q * 16;
        if (q * 16 < ncol) {
            const int kb = c / 128;
            long off;
            if (tiled) {
                const int hh = (c % 128) / 64, lgq = (c % 64) / 16, l = lgq * 16 + r % 16;
                off = ((long)(r / 16) * nkb + kb) * 2048 + hh * 1024 + l * 16;
            } else {
                off = (long)r * Dv + c;
            }
            wcode[q] = *(const v4i *)(wm + off);
        }
    }
    // partial sums: thread -> features 4 fq .. + 4 of splits [HS sh, HS sh + HS)
    const int fq = tid & 127, sh = tid >> 7;
    v4f pv[HS];
#pragma unroll
    for (int k = 0; k < HS; k++) {
        const int s2 = sh * HS + k;
        pv[k] = (s2 < nsplit && fq * 4 < Dv) ? *(const v4f *)(opart + (((long)b * nsplit + s2) * H + h) * Dv + fq * 4)
                                            : v4f{0.f, 0.f, 0.f, 0.f};
    }
    // split weights w_s = e^(m_s - M) / sum_s e^(m_s - M) l_s (0 for an empty split), by wave 0
    if (wv == 0) {
        const bool ok = lane < nsplit;
        const float m = ok ? ml[(((long)b * nsplit + lane) * H + h) * 2] : -INFINITY;
        const float l = ok ? ml[(((long)b * nsplit + lane) * H + h) * 2 + 1] : 0.f;
        const float M = wave_max(m);
        const float e = m == -INFINITY ? 0.f : expf(m - M);
        const float den = wave_sum(e * l);
        if (lane < AM_MAXSPLIT) s_wt[lane] = den > 0.f ? e / den : 0.f;
    }
    __syncthreads();
    // 1. merge: each half in split order, then half 0 + half 1
    {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < HS; k++) {
            const float wk = s_wt[sh * HS + k];
            if (wk != 0.f) acc += pv[k] * wk;
        }
        if (fq * 4 < Dv) *(v4f *)&s_half[sh][fq * 4] = acc;
    }
    __syncthreads();
    for (int v = tid; v < Dv; v += 256) {
        const float ov = s_half[0][v] + s_half[1][v];
        s_o[v] = ov;
        o[(long)bh * Dv + v] = ov;
    }
    __syncthreads();
    // 2. u = W_UV[h] o: thread -> (row r, its columns)
    float acc = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
        if (kb * 128 >= ncol) break;
        float blk = 0.f;
#pragma unroll
        for (int qq = 0; qq < 8; qq++) {
            const int q = kb * 8 + qq, c = c_lo + q * 16;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const v2f lo = fp8x2_lo((uint32_t)wcode[q][i]), hi = fp8x2_hi((uint32_t)wcode[q][i]);
                blk = fmaf(lo.x, s_o[c + 4 * i], blk);
                blk = fmaf(lo.y, s_o[c + 4 * i + 1], blk);
                blk = fmaf(hi.x, s_o[c + 4 * i + 2], blk);
                blk = fmaf(hi.y, s_o[c + 4 * i + 3], blk);
            }
        }
        acc = fmaf(blk, wsc[((long)h * nrb + r / 128) * nkb + (c_lo / 128 + kb)], acc);
    }
    s_u[r][part] = acc;
    __syncthreads();
    // 3. split u into NSU parts, one wave per 128-row block of u
    const int nub = hd / 128;
    const long K = (long)H * hd;
    if (wv < nub) {
        const int r0 = wv * 128 + lane * 2;
        float x0 = s_u[r0][0] + (per_row > 1 ? s_u[r0][1] : 0.f);
        float x1 = s_u[r0 + 1][0] + (per_row > 1 ? s_u[r0 + 1][1] : 0.f);
        const long e = (long)b * K + (long)h * hd + r0;
        const long sc_i = (long)b * (K / 128) + (long)h * nub + wv;
#pragma unroll
        for (int s = 0; s < NSU; s++) {
            const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
            const float scale = amax > 0.f ? amax * (1.0f / 448.0f) : 1.0f;
            const float iv = 1.0f / scale;
            const uint32_t code = f32x2_to_fp8(fminf(fmaxf(x0 * iv, -448.f), 448.f), fminf(fmaxf(x1 * iv, -448.f), 448.f));
            *(uint16_t *)(uq + s * uq_part + e) = (uint16_t)code;
            if (lane == 0) uqs[s * uqs_part + sc_i] = scale;
            const v2f d = fp8x2_lo(code);
            x0 -= d.x * scale;
            x1 -= d.y * scale;
        }
    }
}

bool attention_merge_uv_ok(int Dv, int hd)
{
    return Dv % 128 == 0 && Dv <= 512 && (hd == 128 || (hd == 256 && Dv <= 256));
}

int launch_attn_merge_uv(int B, int H, int Dv, int top_k, const float *opart, const float *ml, float *o,
                         const uint8_t *wuv, const float *wsc, int hd, int tiled, uint8_t *uq, float *uqs,
                         long uq_part, long uqs_part, hipStream_t s)
{
    hipLaunchKernelGGL((k_attn_merge_uv<4>), dim3(B * H), dim3(256), 0, s, opart, ml, attention_splits(top_k, B, H), H, Dv,
                       o, wuv, wsc, hd, tiled, uq, uqs, uq_part, uqs_part);
    return hip_check("attn_merge_uv");
}

bool attention_mfma_ok(int H, int Dc, int Dv, int q_dt, int kv_dt)
{
    return kv_dt == DL_FP8_E4M3 && q_dt == DL_BF16 && H % 16 == 0 &&
           (Dc == 576 || Dc == 512 || Dc == 256 || Dc == 128) && (Dv == 128 || Dv == 256 || Dv == 512) && Dv <= Dc;
}

// Kept positions per split: about 256 workgroups over the batch, whole chunks of 64, at most 512; the number
// of splits follows (at most 32).
static int attention_pps(int top_k, int B, int H)
{
    const int hs = (H + 63) / 64;
    const long want = std::max(1L, 256L / ((long)B * hs));
    int ch = (int)((top_k + AM_NJ * want - 1) / (AM_NJ * want));
    ch = std::max(ch, (top_k + AM_NJ * AM_MAXSPLIT - 1) / (AM_NJ * AM_MAXSPLIT));
    ch = std::min(std::max(ch, 1), AM_MAXPPS / AM_NJ);
    return ch * AM_NJ;
}

int attention_splits(int top_k, int B, int H)
{
    const int pps = attention_pps(top_k, B, H);
    return (top_k + pps - 1) / pps;
}

int launch_attention(const dl_pages &pg, const void *q, int q_dt, const void *kv, const float *kv_scale, int kv_dt,
                     int H, int Dc, int Dv, float sm_scale, const int32_t *sel, int top_k, float *o, float *opart,
                     float *ml, hipStream_t s, int R)
{
    const int rows = pg.batch * R;  // row i reads the cache of sequence i / R
    if (attention_mfma_ok(H, Dc, Dv, q_dt, kv_dt) && opart && ml) {
        if (top_k > AM_MAXPPS * AM_MAXSPLIT) return fail(DL_ERR_UNSUPPORTED, "attention top_k %d", top_k);
        const int ps_shift = __builtin_ctz((unsigned)pg.page_size);
        const int pps = attention_pps(top_k, rows, H);
        const int nsplit = (top_k + pps - 1) / pps;
        dim3 g(nsplit, (H + 63) / 64, rows);
#define DL_AM(KQ_, NVB_)                                                                                            \
    if (Dc == KQ_ * 32 && Dv == NVB_ * 128) {                                                                       \
        if (pps > AM_NJ)                                                                                            \
            hipLaunchKernelGGL((k_attn_mla<KQ_, NVB_, true>), g, dim3(256), 0, s, (const uint16_t *)q,              \
                               (const uint8_t *)kv, kv_scale, pg.page_table, pg.max_pages_per_seq, R, ps_shift, sel,    \
                               top_k, H, pps, sm_scale, opart, ml);                                                 \
        else                                                                                                        \
            hipLaunchKernelGGL((k_attn_mla<KQ_, NVB_, false>), g, dim3(256), 0, s, (const uint16_t *)q,             \
                               (const uint8_t *)kv, kv_scale, pg.page_table, pg.max_pages_per_seq, R, ps_shift, sel,    \
                               top_k, H, pps, sm_scale, opart, ml);                                                 \
    }
        DL_AM(18, 4) DL_AM(18, 2) DL_AM(18, 1) DL_AM(16, 4) DL_AM(16, 2) DL_AM(16, 1) DL_AM(8, 2) DL_AM(8, 1)
        DL_AM(4, 1)
#undef DL_AM
        if (o) hipLaunchKernelGGL(k_attn_merge, dim3(rows * H), dim3(256), 0, s, opart, ml, nsplit, H, Dv, o);
        return hip_check("attention_mfma");
    }
    if (top_k > ATT_MAX_K || Dc > ATT_MAX_DC) return fail(DL_ERR_UNSUPPORTED, "attention top_k %d / d_c %d", top_k, Dc);
    if (Dv % 4 || (256 % (Dv / 4))) return fail(DL_ERR_UNSUPPORTED, "attention d_v %d (power of two 4..1024)", Dv);
    if (Dc % 4) return fail(DL_ERR_UNSUPPORTED, "attention d_c %d", Dc);
    const int ps_shift = __builtin_ctz((unsigned)pg.page_size);
    dim3 g((H + ATT_HG - 1) / ATT_HG, rows);
    hipLaunchKernelGGL(k_attn, g, dim3(256), 0, s, q, q_dt, kv, kv_scale, kv_dt == DL_FP8_E4M3 ? 1 : 0, pg.page_table,
                       pg.max_pages_per_seq, R, ps_shift, sel, top_k, H, Dc, Dv, sm_scale, o);
    return hip_check("attention");
}

}  // namespace dl
