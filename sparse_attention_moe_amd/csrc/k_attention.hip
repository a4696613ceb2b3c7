// S3 + S4: sparse MLA decode attention over the kept positions only.
//
// Kiln's decode kernel gathers the selected entries instead of masking every key ("The decode
// kernels, and why they are opt-in", Introducing Kiln); the cache is one compressed latent per
// position shared by all heads ("How was Kiln measured against vLLM on H200?").  The key is the
// whole latent (d_c features), the value its first d_v features.
//
// Two kernels:
//  * k_attn_mla, k_attn_mla1 (FP8 latents, bf16 queries, 16 | heads): split over the kept positions like
//    flash decoding.  A workgroup owns one row, a run of kept positions (the split) and up to 64 heads, so
//    every kept latent is gathered once for all heads; positions are staged 64 at a time (a chunk) in LDS.
//    k_attn_mla (splits of several chunks, 512 threads, two waves per 16 heads): the chunk's raw e4m3 bytes
//    arrive by the direct global-to-LDS loads, the next chunk landing while the current one is computed;
//    scores on the FP8 matrix cores (v_mfma_f32_16x16x128_f8f6f4) with each query, scaled by a power of two,
//    split into two e4m3 parts whose sum is the bf16 query exactly.  k_attn_mla1 (one chunk, 256 threads):
//    the codes are converted once to bf16 in LDS and scored on v_mfma_f32_16x16x32_bf16 (every e4m3 code is
//    exactly a bf16).  Either way the products are exact and each 128-feature block's sum takes its scale
//    once; the softmax runs online in fp32; the values are transposed once per chunk into [feature][position]
//    rows, and O += P' C with P' = p * (block scale) split into bf16 high and low halves (about 16
//    significant bits), so the output keeps fp32-level accuracy.  The splits are merged afterwards
//    (max-rescaled sums), with W_UV applied in the merge.
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

#ifndef DL_ATT_NT_STORE
#define DL_ATT_NT_STORE 1
#endif
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

// A workgroup barrier over LDS alone: this wave's LDS writes complete, then every wave meets.  Unlike
// __syncthreads it leaves the wave's global loads in flight (the direct-to-LDS ones included).
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt left at their maxima
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// O += A B on v_mfma_f32_16x16x128_f8f6f4, both operands e4m3 without block scales.  Lane (l % 16, l / 16)
// holds 32 K bytes of row l % 16 of A and of column l % 16 of B; any K order works if A and B share it.
__device__ __forceinline__ v4f mfma_fp8_acc(v8i a, v8i b, v4f c)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
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

// Splits of one chunk (64 kept positions): grid (nsplit, ceil(H/64), B), 256 threads.  A workgroup owns one row,
// its split and up to 64 heads: wave w takes heads 16 (4 blockIdx.y + w) .. +16, so each kept latent is gathered
// once for all heads.  With nothing to prefetch, the fewer fixed steps of this form beat the chunked kernel below
// (batch 8 / 128K: 18.6 against 21.9 us; batch 1 / 1M: 13.6 against 16.3 us).  For its chunk:
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
template <int KQ, int NVB>
__global__ __launch_bounds__(256, 1) void k_attn_mla1(const uint16_t *__restrict__ q, const uint8_t *__restrict__ kv,
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
    // (loads unconditional, with clamped indices: a load under a condition is waited for on its own; a wave past
    // the heads reads the last head's row and computes nothing with it)
    v8bf Aq[KQ];
    const int hq = min(h0 + ln, H - 1);
#pragma unroll
    for (int kk = 0; kk < KQ; kk++) Aq[kk] = *(const v8bf *)(q + ((long)b * H + hq) * Dc + kk * 32 + lg * 8);
    for (int i = tid; i < pps; i += 256) {
        const int j = jbase + i;
        const int ps = sel[(long)b * top_k + min(j, top_k - 1)];
        const int p = j < top_k ? ps : -1;
        const int pg = pt[(long)(b / R) * max_pages + (max(p, 0) >> ps_shift)];
        s_row[i] = p < 0 ? -1 : ((long)pg << ps_shift) + (p & ps_mask);
    }
    const int nch = jbase < top_k ? 1 : 0;
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
    // gather of chunk c into registers: 16 codes per load, and the chunk's block scales (a position past the
    // kept ones reads code 0 and scale 0)
    constexpr int NSC = (AM_NJ * NB + 255) / 256;  // scales per thread
    v4i GR[NLD];
    float GS[NSC];
    auto gather = [&](int c) __attribute__((always_inline)) {
        const int cbase = c * AM_NJ;
#pragma unroll
        for (int k = 0; k < NLD; k++) {
            const int id = k * 256 + tid;
            GR[k] = v4i{0, 0, 0, 0};
            if (id < AM_NJ * (Dc / 16)) {
                const long row = s_row[cbase + id / (Dc / 16)];
                if (row >= 0) GR[k] = *(const v4i *)(kv + row * Dc + (id % (Dc / 16)) * 16);
            }
        }
#pragma unroll
        for (int k = 0; k < NSC; k++) {
            const int i = k * 256 + tid;
            GS[k] = 0.f;
            if (i < AM_NJ * NB) {
                const long row = s_row[cbase + i / NB];
                if (row >= 0) GS[k] = ks[row * NB + i % NB];
            }
        }
    };
    for (int ch = 0; ch < nch; ch++) {
        const int cb = ch * AM_NJ;  // chunk base within the split
        __syncthreads();            // s_row is complete; the previous chunk's LDS reads are done
        gather(ch);
        // chunk ch's codes converted to bf16 (two 16-byte LDS writes per load) and its scales into LDS
#pragma unroll
        for (int k = 0; k < NLD; k++) {
            const int id = k * 256 + tid;
            if (id < AM_NJ * (Dc / 16)) {
                __bf16 *dst = s_cb + (id / (Dc / 16)) * CBP + (id % (Dc / 16)) * 16;
                *(v8bf *)dst = fp8x8_to_bf16((uint32_t)GR[k][0], (uint32_t)GR[k][1]);
                *(v8bf *)(dst + 8) = fp8x8_to_bf16((uint32_t)GR[k][2], (uint32_t)GR[k][3]);
            }
        }
#pragma unroll
        for (int k = 0; k < NSC; k++) {
            const int i = k * 256 + tid;
            if (i < AM_NJ * NB) s_sc[i % NB][i / NB] = GS[k];
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
            // the four position tiles are four independent accumulator chains, interleaved so that consecutive
            // instructions do not wait on each other; each 128-feature block's operands are read before its
            // instructions (one wave per SIMD: nothing else would hide the LDS latency)
            v4f sacc[4];
#pragma unroll
            for (int j = 0; j < 4; j++) sacc[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int blk = 0; blk < NB; blk++) {
                v4f a[4];
#pragma unroll
                for (int j = 0; j < 4; j++) a[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int q2 = 0; q2 < 4; q2 += 2) {
                    v8bf Bt[2][4];
#pragma unroll
                    for (int q = 0; q < 2; q++)
#pragma unroll
                        for (int j = 0; j < 4; j++)
                            if (blk * 4 + q2 + q < KQ)
                                Bt[q][j] = *(const v8bf *)(s_cb + (j * 16 + ln) * CBP + lg * 8 + (blk * 4 + q2 + q) * 32);
#pragma unroll
                    for (int q = 0; q < 2; q++)
#pragma unroll
                        for (int j = 0; j < 4; j++)
                            if (blk * 4 + q2 + q < KQ) a[j] = mfma_bf16(Aq[blk * 4 + q2 + q], Bt[q][j], a[j]);
                }
#pragma unroll
                for (int j = 0; j < 4; j++) sacc[j] += a[j] * s_sc[blk][j * 16 + ln];
            }
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const bool valid = s_row[cb + j * 16 + ln] >= 0;
#pragma unroll
                for (int i = 0; i < 4; i++) S[j][i] = valid ? sacc[j][i] * sl2 : -INFINITY;
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
                v8bf Bv[8];
#pragma unroll
                for (int t = 0; t < 8; t++) {
                    const int f = vb * 128 + t * 16 + ln;
                    Bv[t] = *(const v8bf *)(s_v + f * PP + (((kstep * 4 + lg) ^ ((vb * 8 + t) & 7)) << 3));
                }
#pragma unroll
                for (int t = 0; t < 8; t++) {
                    acc[vb][t] = mfma_bf16(Ah, Bv[t], acc[vb][t]);
                    acc[vb][t] = mfma_bf16(Al, Bv[t], acc[vb][t]);
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
#if DL_ATT_NT_STORE
                __builtin_nontemporal_store(*(const v4f *)&st[head][col],
                                            (v4f *)(op + (long)head * Dv + vb * 128 + half * 64 + col));
#else
                *(v4f *)(op + (long)head * Dv + vb * 128 + half * 64 + col) = *(const v4f *)&st[head][col];
#endif
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

// Sixteen zero bytes: the source of every direct-to-LDS load that has nothing to load.
static __device__ __attribute__((aligned(16))) uint32_t g_zero16[4] = {0u, 0u, 0u, 0u};  // never written
// Running maxima move only when a chunk's maximum exceeds them by more than this (log2 units), so p <= 2^8 and the
// sums are rescaled rarely.
static constexpr float AM_TAU = 8.f;

// Splits of several chunks: grid (nsplit, ceil(H/64), B), 512 threads.  A workgroup owns one row, one run of kept
// positions (the split)
// and up to 64 heads, so each kept latent is gathered once for all of them.  Waves w and w + 4 share the 16
// heads 16 (4 blockIdx.y + w % 4) .. +16, so two waves share each SIMD and hide each other's latencies: wave w
// holds the query's first NBA = (NB + 1) / 2 128-feature blocks, owns positions 0..31 of every chunk of 64 and
// accumulates value features 0..d_v/2; wave w + 4 the other blocks, positions 32..63 and features d_v/2..d_v.
// Per chunk:
//   gather   the latent codes and block scales of the chunk's positions (through the page table) straight into
//            LDS as raw e4m3 bytes with the direct global-to-LDS loads, one chunk ahead: chunk c + 1 lands in
//            the other of two buffers while chunk c is computed, and no register holds it meanwhile;
//   values   the first Dv features transposed once into [feature][position] byte rows;
//   scores   S = Q C^T on v_mfma_f32_16x16x128_f8f6f4 straight from the e4m3 codes: each wave's part of a
//            head's query is scaled by a power of two and split into two e4m3 parts whose sum is the scaled
//            bf16 query exactly (bar elements 2^9 below that part's largest), so the products and sums are those
//            of the bf16 query; each 128-feature block's sum takes its scale once.  Each wave scores all 64
//            positions over its blocks and hands its partner the partial sums of the partner's positions;
//   softmax  online per head in fp32, each wave over its own positions with its own running reference (raised
//            only when a chunk exceeds it by more than AM_TAU, so the rescaling of the sums is rare); both waves'
//            p and references go to LDS, and p is rescaled to the larger of the two as it is read;
//   output   O += P' C with P' = p * (block scale) in bf16 high and low halves (about 16 significant bits) on
//            v_mfma_f32_16x16x32_bf16, the e4m3 values converted to bf16 (exactly) as they are read.
// opart [B, nsplit, H, Dv] holds the unnormalised sums, ml [B, nsplit, H, 2] the (max, sum) they refer to.
template <int KQ, int NVB>
__global__ __launch_bounds__(512, 1) void k_attn_mla(const uint16_t *__restrict__ q, const uint8_t *__restrict__ kv,
                                                     const float *__restrict__ ks, const int32_t *__restrict__ pt,
                                                     int max_pages, int R, int ps_shift, const int32_t *__restrict__ sel,
                                                     int top_k, int H, int pps, float sm_scale,
                                                     float *__restrict__ opart, float *__restrict__ ml)
{
    constexpr int Dc = KQ * 32, NB = (Dc + 127) / 128, Dv = NVB * 128;
    constexpr int NBA = (NB + 1) / 2;        // query blocks of the first wave of a pair (the second: NB - NBA)
    constexpr int NG = Dc / 16 + 1;          // 16-byte granules per position row in LDS (one unused, so that
    constexpr int RP = NG * 16;              // consecutive rows start in different banks); row pitch
    constexpr int NIW = (NG + 7) / 8;        // 64-lane code loads per wave and chunk (NG in all)
    constexpr int NSW = (NB + 7) / 8;        // 64-lane scale loads per wave and chunk (NB in all)
    constexpr int VP = AM_NJ + 8;            // value row pitch (bytes)
    constexpr int FV = Dv / 2;               // value features per wave
    constexpr int NT = FV / 16;              // 16-feature tiles per wave
    constexpr int NVW = (FV + 127) / 128;    // 128-feature scale blocks per wave
    constexpr int TPB = NT / NVW;            // tiles per scale block
    constexpr int SPP = 76;                  // s_p row pitch (floats)
    static_assert(AM_NJ == 64 && Dv <= 512 && Dv <= Dc, "one position per lane in a scale load; a value per thread");
    // [position][RP] codes and [block][position] scales, each followed by the padding the last loads fill
    __shared__ __attribute__((aligned(16))) uint8_t s_c0[NIW * 8 * 1024], s_c1[NIW * 8 * 1024];
    __shared__ __attribute__((aligned(16))) float s_s0[NSW * 8 * 64], s_s1[NSW * 8 * 64];
    __shared__ __attribute__((aligned(16))) uint8_t s_vt[Dv * VP];     // [feature][position] values
    // (flat arrays indexed by one integer: the compiler can then tell every access apart from the direct loads'
    // targets; through a deep chain of address steps it cannot, and waits for those loads first)
    __shared__ __attribute__((aligned(16))) float s_p[4 * 16 * SPP];  // [head group][head][position]
    __shared__ float s_mx[2 * 64];                                      // running maxima [half][group, head]
    __shared__ float s_l[64];
    __shared__ long s_row[AM_MAXPPS];
    const int split = blockIdx.x, b = blockIdx.z;
    const int nsplit = gridDim.x;
    const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
    const int hg = w & 3, half = w >> 2;
    const int h0 = (blockIdx.y * 4 + hg) * 16;
    const bool active = h0 < H;
    const int kb0 = half ? NBA : 0, nkb = half ? NB - NBA : NBA;
    const int ps_mask = (1 << ps_shift) - 1;
    const int jbase = split * pps;
    // the split's kept positions -> cache rows (first: their two dependent loads overlap the query's)
    for (int i = tid; i < pps; i += 512) {
        const int j = jbase + i;
        const int p = j < top_k ? sel[(long)b * top_k + j] : -1;
        s_row[i] = p < 0 ? -1 : ((long)pt[(long)(b / R) * max_pages + (p >> ps_shift)] << ps_shift) + (p & ps_mask);
    }
    // this wave's query blocks as FP8 A operands: head ln, features 128 kb + 32 lg .. + 32 (zero past d_c),
    // times 2^e with e chosen per head so that the largest |q| of these blocks lies in [128, 256), as e4m3 high
    // and low parts; qi[i] = 2^-e of head 4 lg + i
    v8i Qh[NBA], Ql[NBA];
    float qi[4];
    {
        uint4 qv[NBA][4];
        float mx = 0.f;
#pragma unroll
        for (int kk = 0; kk < NBA; kk++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int f = (kb0 + kk) * 128 + lg * 32 + e * 8;
                qv[kk][e] = active && kk < nkb && f < Dc ? *(const uint4 *)(q + ((long)b * H + h0 + ln) * Dc + f)
                                                         : uint4{0, 0, 0, 0};
                const uint32_t x[4] = {qv[kk][e].x, qv[kk][e].y, qv[kk][e].z, qv[kk][e].w};
#pragma unroll
                for (int k = 0; k < 4; k++)
                    mx = fmaxf(mx, fmaxf(fabsf(__uint_as_float(x[k] << 16)), fabsf(__uint_as_float(x[k] & 0xFFFF0000u))));
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // mx in [2^ex, 2^(ex+1)); scale 2^se, se = 7 - ex (kept where both 2^se and 2^-se are normal floats)
        const int ex = mx > 0.f ? (int)((__float_as_uint(mx) >> 23) & 255u) - 127 : 7;
        const int se = min(max(7 - ex, -126), 126);
        const float sc = __uint_as_float((uint32_t)(se + 127) << 23);
        const float inv = __uint_as_float((uint32_t)(127 - se) << 23);
#pragma unroll
        for (int kk = 0; kk < NBA; kk++) {
            uint32_t hw[8], lw[8];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const uint32_t x[4] = {qv[kk][e].x, qv[kk][e].y, qv[kk][e].z, qv[kk][e].w};
#pragma unroll
                for (int k = 0; k < 4; k += 2) {
                    // 4 consecutive elements (two dwords of bf16 pairs) -> one dword of codes per part
                    const float v0 = __uint_as_float(x[k] << 16) * sc, v1 = __uint_as_float(x[k] & 0xFFFF0000u) * sc;
                    const float v2 = __uint_as_float(x[k + 1] << 16) * sc;
                    const float v3 = __uint_as_float(x[k + 1] & 0xFFFF0000u) * sc;
                    const uint32_t h01 = f32x2_to_fp8(v0, v1), h23 = f32x2_to_fp8(v2, v3);
                    const v2f b01 = fp8x2_lo(h01), b23 = fp8x2_lo(h23);
                    const uint32_t l01 = f32x2_to_fp8(v0 - b01.x, v1 - b01.y), l23 = f32x2_to_fp8(v2 - b23.x, v3 - b23.y);
                    hw[e * 2 + k / 2] = h01 | h23 << 16;
                    lw[e * 2 + k / 2] = l01 | l23 << 16;
                }
            }
            Qh[kk] = v8i{(int)hw[0], (int)hw[1], (int)hw[2], (int)hw[3], (int)hw[4], (int)hw[5], (int)hw[6], (int)hw[7]};
            Ql[kk] = v8i{(int)lw[0], (int)lw[1], (int)lw[2], (int)lw[3], (int)lw[4], (int)lw[5], (int)lw[6], (int)lw[7]};
        }
#pragma unroll
        for (int i = 0; i < 4; i++) qi[i] = __shfl(inv, 4 * lg + i, 64);
    }
    // scores in log2 units: p = 2^(S - m) with S = sm_scale * log2(e) * q.c, so the exponentials are exp2
    const float sl2 = sm_scale * 1.4426950408889634f;
    const int nch = max(0, min(pps, top_k - jbase) + AM_NJ - 1) / AM_NJ;
    // chunk c's codes and scales into LDS.  Code load i (of a wave: i = w, w + 8, ...) fills 64 consecutive 16-byte
    // slots; slot s is granule s % NG of position s / NG (granule NG - 1 is padding).  Scale load i fills 64 floats:
    // block i of the chunk's positions.  Every wave issues the same number of loads, all of them unconditionally:
    // a slot with nothing to load (padding, a position past the kept ones, no next chunk) reads zeros, so such a
    // position has value 0 and scale 0.  (A direct-to-LDS load on a conditional path makes the compiler wait for
    // it before later LDS accesses, which would undo the overlap.)
    const uint8_t *const dummy = (const uint8_t *)g_zero16;
    auto gather = [&](int c, bool more, uint8_t *dc, float *dsc) __attribute__((always_inline)) {
        const int cbase = c * AM_NJ;
        // the lane's slot arithmetic is redone per chunk: hoisted out of the chunk loop its results would stay
        // live across the chunk's arithmetic and spill
        int ln64 = lane;
        asm volatile("" : "+v"(ln64));
        long rows[NIW], srows[NSW];
#pragma unroll
        for (int k = 0; k < NIW; k++) rows[k] = s_row[min(cbase + ((k * 8 + w) * 64 + ln64) / NG, AM_MAXPPS - 1)];
#pragma unroll
        for (int k = 0; k < NSW; k++) srows[k] = s_row[min(cbase + ln64, AM_MAXPPS - 1)];
#pragma unroll
        for (int k = 0; k < NIW; k++) {
            const int i = k * 8 + w, sl = i * 64 + ln64, p = sl / NG, g = sl - p * NG;
            const bool ok = more && p < AM_NJ && g < Dc / 16 && rows[k] >= 0;
            const uint8_t *src = ok ? kv + rows[k] * Dc + g * 16 : dummy;
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                             (__attribute__((address_space(3))) void *)(dc + i * 1024), 16, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < NSW; k++) {
            const int blk = k * 8 + w;
            const bool ok = more && blk < NB && srows[k] >= 0;
            const void *src = ok ? (const void *)(ks + srows[k] * NB + blk) : (const void *)dummy;
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                             (__attribute__((address_space(3))) void *)(dsc + blk * 64), 4, 0, 0);
        }
    };
    // mh, lh: this wave's running max and sum over its own positions, heads 4 lg + i; ma: the max acc refers to
    float mh[4], lh[4], ma[4];
    v4f acc[NT];
#pragma unroll
    for (int i = 0; i < 4; i++) { mh[i] = -INFINITY; lh[i] = 0.f; ma[i] = -INFINITY; }
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
    // chunk c from buffers (cc, cs), prefetching chunk c + 1 into (nc, ns)
    auto chunk = [&](int c, const uint8_t *cc, const float *cs, uint8_t *nc, float *ns) __attribute__((always_inline)) {
        const int cb = c * AM_NJ;
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of chunk c have landed
        __syncthreads();                // everyone's have; every wave is done with chunk c - 1
        gather(c + 1, c + 1 < nch, nc, ns);
        // per-lane offsets are recomputed per chunk (a few VALU operations) rather than held in registers
        // across it: the lane id passes through an opaque copy
        int lnc = lane;
        asm volatile("" : "+v"(lnc));
        const int ln = lnc & 15, lg = lnc >> 4, tid = w * 64 + lnc;
        // values: thread u -> 8 features x 8 positions, a byte transpose to [feature][position].  Lane l of a wave
        // takes position group l % 8 and feature group l / 8; it reads its 8 rows starting at row (l % 8) of
        // the group, so the 64 lanes' reads and writes each spread over all banks, and rotates each feature's
        // 8 bytes back into position order.  (Positions past the kept ones were loaded as zeros.)
        if (tid < Dv) {
            const int pg = tid & 7, fq = tid >> 3;
            uint32_t r0[8], r1[8];
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const uint2 v = *(const uint2 *)(cc + (pg * 8 + ((e + pg) & 7)) * RP + fq * 8);
                r0[e] = v.x;
                r1[e] = v.y;
            }
            uint32_t lo0[4], lo1[4], hi0[4], hi1[4];
            tr4x4(r0[0], r0[1], r0[2], r0[3], lo0);
            tr4x4(r0[4], r0[5], r0[6], r0[7], lo1);
            tr4x4(r1[0], r1[1], r1[2], r1[3], hi0);
            tr4x4(r1[4], r1[5], r1[6], r1[7], hi1);
            const int sh = pg * 8;
#pragma unroll
            for (int k = 0; k < 8; k++) {
                const uint64_t x = k < 4 ? ((uint64_t)lo1[k] << 32 | lo0[k]) : ((uint64_t)hi1[k - 4] << 32 | hi0[k - 4]);
                *(uint64_t *)(s_vt + (fq * 8 + k) * VP + pg * 8) = x << sh | x >> ((64 - sh) & 63);
            }
        }
        // partial scores over this wave's blocks, all four position tiles: tile j covers positions
        // 16 ((j + 2 half) % 4) + ln, so tiles 0, 1 are this wave's own positions and 2, 3 its partner's; lane
        // holds heads 4 lg + i, in true units (times 2^-e)
        v4f sp[4];
#pragma unroll
        for (int j = 0; j < 4; j++) sp[j] = v4f{0.f, 0.f, 0.f, 0.f};
        if (active) {
#pragma unroll
            for (int kk = 0; kk < NBA; kk++) {
                if (kk >= nkb) break;
                const int kb = kb0 + kk;
                // B: 32 code bytes of the position, the lane's K range of block kb (re-read within d_c where the
                // block is half past it: the query's part there is zero)
                const int f = kb * 128 + lg * 32 < Dc ? kb * 128 + lg * 32 : kb * 128 + (lg & 1) * 32;
#pragma unroll
                for (int jp = 0; jp < 4; jp += 2) {
                    v8i Bc[2];
#pragma unroll
                    for (int jj = 0; jj < 2; jj++) {
                        const uint8_t *src = cc + (((jp + jj + 2 * half) & 3) * 16 + ln) * RP + f;
                        const v4i x0 = *(const v4i *)src, x1 = *(const v4i *)(src + 16);
                        Bc[jj] = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
                    }
#pragma unroll
                    for (int jj = 0; jj < 2; jj++) {
                        v4f a = mfma_fp8_acc(Qh[kk], Bc[jj], v4f{0.f, 0.f, 0.f, 0.f});
                        a = mfma_fp8_acc(Ql[kk], Bc[jj], a);
                        sp[jp + jj] += a * cs[kb * AM_NJ + ((jp + jj + 2 * half) & 3) * 16 + ln];
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int i = 0; i < 4; i++) sp[j][i] *= qi[i];
            // the partner's positions (tiles 2, 3) into its P rows
#pragma unroll
            for (int jj = 0; jj < 2; jj++)
#pragma unroll
                for (int i = 0; i < 4; i++)
                    s_p[(hg * 16 + 4 * lg + i) * SPP + (2 * (1 - half) + jj) * 16 + ln] = sp[2 + jj][i];
        }
        lds_barrier();  // the values and the partial scores are complete (the next chunk's loads stay in flight)
        if (active) {
            // own positions (tiles 0, 1: positions 32 half + 16 jj + ln); whole scores, then the online softmax
            v4f S[2];
#pragma unroll
            for (int jj = 0; jj < 2; jj++) {
                const int j = half * 2 + jj;
                const bool valid = s_row[cb + j * 16 + ln] >= 0;
#pragma unroll
                for (int i = 0; i < 4; i++)
                    S[jj][i] = valid ? (sp[jj][i] + s_p[(hg * 16 + 4 * lg + i) * SPP + j * 16 + ln]) * sl2 : -INFINITY;
            }
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float mc = row_max16(fmaxf(S[0][i], S[1][i]));
                const float mn = mc > mh[i] + AM_TAU || mh[i] == -INFINITY ? mc : mh[i];
                const float al = mn == mh[i] ? 1.f : __builtin_amdgcn_exp2f(mh[i] - mn);
                mh[i] = mn;
                float ps = 0.f;
#pragma unroll
                for (int jj = 0; jj < 2; jj++) {
                    const float pv = S[jj][i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(S[jj][i] - mn);
                    s_p[(hg * 16 + 4 * lg + i) * SPP + (half * 2 + jj) * 16 + ln] = pv;
                    ps += pv;
                }
                lh[i] = lh[i] * al + row_sum16(ps);
                if (ln == 0) s_mx[half * 64 + hg * 16 + 4 * lg + i] = mn;
            }
        }
        lds_barrier();  // p of all 64 positions and both halves' maxima are in LDS
        if (!active) return;
        // acc refers to the larger of the two references from now on (a rare change: AM_TAU)
        {
            float al[4];
            bool moved = false;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float mn = fmaxf(s_mx[hg * 16 + 4 * lg + i], s_mx[64 + hg * 16 + 4 * lg + i]);
                al[i] = mn == ma[i] ? 1.f : __builtin_amdgcn_exp2f(ma[i] - mn);
                moved |= mn != ma[i];
                ma[i] = mn;
            }
            if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
                for (int t = 0; t < NT; t++)
#pragma unroll
                    for (int i = 0; i < 4; i++) acc[t][i] *= al[i];
            }
        }
        // p of half h (positions 32 h ..) is relative to that half's max: factor 2^(m_h - max) for head ln
        float corr[2];
        {
            const float m0 = s_mx[hg * 16 + ln], m1 = s_mx[64 + hg * 16 + ln], mn = fmaxf(m0, m1);
            corr[0] = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m0 - mn);
            corr[1] = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mn);
        }
        // O += P' C over two K steps of 32 positions (the two halves): A = P' (head ln, positions 8 lg .. + 8),
        // B = values (feature half FV + 16 t + ln, the same positions)
#pragma unroll
        for (int kstep = 0; kstep < 2; kstep++) {
            const int pl = kstep * 32 + lg * 8;  // first position of this lane's K group (within the chunk)
            const v4f p0 = *(const v4f *)&s_p[(hg * 16 + ln) * SPP + pl], p1 = *(const v4f *)&s_p[(hg * 16 + ln) * SPP + pl + 4];
            const float pr[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
#pragma unroll
            for (int vw = 0; vw < NVW; vw++) {
                const int vb = half * FV / 128 + vw;  // scale block of these features
                const v4f c0 = *(const v4f *)&cs[vb * AM_NJ + pl], c1 = *(const v4f *)&cs[vb * AM_NJ + pl + 4];
                const float sc[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
                v8bf Ah, Al;
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    // (a position past the kept ones has p = 0 and scale 0)
                    const float x = pr[e] * corr[kstep] * sc[e];
                    const __bf16 hb = (__bf16)x;
                    Ah[e] = hb;
                    Al[e] = (__bf16)(x - (float)hb);
                }
#pragma unroll
                for (int t0 = 0; t0 < TPB; t0 += 4) {
                    uint2 Bv[4];
#pragma unroll
                    for (int t = 0; t < 4; t++)
                        if (t0 + t < TPB) Bv[t] = *(const uint2 *)(s_vt + (half * FV + vw * 128 + (t0 + t) * 16 + ln) * VP + pl);
#pragma unroll
                    for (int t = 0; t < 4; t++) {
                        if (t0 + t >= TPB) break;
                        const v8bf Bb = fp8x8_to_bf16(Bv[t].x, Bv[t].y);
                        acc[vw * TPB + t0 + t] = mfma_bf16(Ah, Bb, acc[vw * TPB + t0 + t]);
                        acc[vw * TPB + t0 + t] = mfma_bf16(Al, Bb, acc[vw * TPB + t0 + t]);
                    }
                }
            }
        }
    };
    __syncthreads();  // s_row is complete
    if (nch > 0) gather(0, true, s_c0, s_s0);
    for (int ch = 0; ch < nch; ch += 2) {
        chunk(ch, s_c0, s_s0, s_c1, s_s1);
        if (ch + 1 >= nch) break;
        chunk(ch + 1, s_c1, s_s1, s_c0, s_s0);
    }
    __syncthreads();  // every wave is done with s_p
    // lane holds O[head h0 + 4 lg + i][feature half FV + 16 t + ln]; 32 features at a time go through this
    // wave's half of its group's P rows in LDS ([16][36] floats) and out as 16-byte stores
    if (active) {
        float *op = opart + (((long)b * nsplit + split) * H + h0) * Dv + half * FV;
        float *st = s_p + hg * 16 * SPP + half * 16 * 36;
#pragma unroll
        for (int pass = 0; pass < NT / 2; pass++) {
#pragma unroll
            for (int tt = 0; tt < 2; tt++)
#pragma unroll
                for (int i = 0; i < 4; i++) st[(4 * lg + i) * 36 + tt * 16 + ln] = acc[pass * 2 + tt][i];
#pragma unroll
            for (int r = 0; r < 2; r++) {
                const int head = r * 8 + (lane >> 3), col = (lane & 7) * 4;
                // streaming store: read once by the merge, so it should not sit dirty in the last-level
                // cache until the expert weight stream evicts it (its write-back would then compete with
                // that stream for HBM)
#if DL_ATT_NT_STORE
                __builtin_nontemporal_store(*(const v4f *)&st[head * 36 + col],
                                            (v4f *)(op + (long)head * Dv + pass * 32 + col));
#else
                *(v4f *)(op + (long)head * Dv + pass * 32 + col) = *(const v4f *)&st[head * 36 + col];
#endif
            }
        }
        // the sum over all 64 positions of every chunk, relative to ma: each half's sum rescaled from its max
        if (half == 1 && ln == 0)
#pragma unroll
            for (int i = 0; i < 4; i++) s_l[hg * 16 + 4 * lg + i] = mh[i] == -INFINITY ? 0.f : lh[i] * __builtin_amdgcn_exp2f(mh[i] - ma[i]);
    }
    __syncthreads();  // the second halves' sums are in LDS
    if (active && half == 0 && ln == 0) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            float *m2 = ml + (((long)b * nsplit + split) * H + h0 + 4 * lg + i) * 2;
            m2[0] = ma[i] * 0.6931471805599453f;  // natural-log units for the merge
            m2[1] = (mh[i] == -INFINITY ? 0.f : lh[i] * __builtin_amdgcn_exp2f(mh[i] - ma[i])) + s_l[hg * 16 + 4 * lg + i];
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

// Split merge fused with the per-head value up-projection and its FP8 split, one workgroup per (row, head): the
// form for a few rows with many splits each (at batch 8, 32 splits a row it is ~3 µs faster than the per-head
// form below, which wins once several rows share a head's W_UV).
//   o      = merged attention output (also stored: [B, H, Dv])
//   u[r]   = sum_v W_UV[h][r][v] o[v]   on the vector units in fp32 (each code decoded exactly, one scale
//            per 128-column block), hd = 128 or 256 rows
//   uq, uqs: u split into NSU FP8 parts with one scale per (part, row b, 128-block) — the activation layout
//            the W_O pass reads ([part][B][H*hd] and [part][B][H*hd/128]).
// Every global load (split maxima and sums, the partial sums, the W_UV codes) is issued up front.  Threads
// take 4 features of one half of the splits; the halves meet in LDS.
template <int NSU>
__global__ __launch_bounds__(256) void k_attn_merge_uv_row(const float *__restrict__ opart, const float *__restrict__ ml,
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
    // this thread's two W_UV block scales, loaded now rather than where they are used
    float wsv[2];
#pragma unroll
    for (int kb = 0; kb < 2; kb++) wsv[kb] = wsc[((long)h * nrb + r / 128) * nkb + min(c_lo / 128 + kb, nkb - 1)];
    // (every load unconditional, with clamped indices, and masked after: a load under a condition is waited for
    // on its own)
    v4f pv[HS];
    const int fqc = min(fq, Dv / 4 - 1);
#pragma unroll
    for (int k = 0; k < HS; k++) {
        const int s2 = min(sh * HS + k, nsplit - 1);
        pv[k] = *(const v4f *)(opart + (((long)b * nsplit + s2) * H + h) * Dv + fqc * 4);
    }
#pragma unroll
    for (int k = 0; k < HS; k++)
        if (!(sh * HS + k < nsplit && fq * 4 < Dv)) pv[k] = v4f{0.f, 0.f, 0.f, 0.f};
    // split weights w_s = e^(m_s - M) / sum_s e^(m_s - M) l_s (0 for an empty split), by wave 0
    if (wv == 0) {
        const bool ok = lane < nsplit;
        const int lc = min(lane, nsplit - 1);
        const float m0 = ml[(((long)b * nsplit + lc) * H + h) * 2], l0 = ml[(((long)b * nsplit + lc) * H + h) * 2 + 1];
        const float m = ok ? m0 : -INFINITY;
        const float l = ok ? l0 : 0.f;
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
        if (o) o[(long)bh * Dv + v] = ov;
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
            if (q * 16 >= ncol) break;  // Dv = 128 with two threads a row: 64 columns, s_o holds only Dv values
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const v2f lo = fp8x2_lo((uint32_t)wcode[q][i]), hi = fp8x2_hi((uint32_t)wcode[q][i]);
                blk = fmaf(lo.x, s_o[c + 4 * i], blk);
                blk = fmaf(lo.y, s_o[c + 4 * i + 1], blk);
                blk = fmaf(hi.x, s_o[c + 4 * i + 2], blk);
                blk = fmaf(hi.y, s_o[c + 4 * i + 3], blk);
            }
        }
        acc = fmaf(blk, wsv[kb], acc);
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

// Split merge fused with the per-head value up-projection and its FP8 split: one workgroup per (head h, block of at
// most MW_RB rows), so W_UV[h] is read once per block of rows instead of once per row, and applied on the matrix
// cores.  Blocks of one head are MW_HEADS workgroups apart in the grid, so they share an XCD and its L2.
//   o      = merged attention output, o[b] = sum_s w_s O_s[b] with w_s = e^(m_s - M) / sum_s e^(m_s - M) l_s
//            summed in split order (also stored when o != nullptr: [rows, H, Dv]);
//   u[b]   = W_UV[h] o[b]: the FP8 codes of W_UV are exact bf16 values, and o enters as bf16 high and low halves
//            (o * block scale, about 16 significant bits), so v_mfma_f32_16x16x32_bf16 forms every product
//            exactly and sums in fp32: [16 W_UV rows] x [32 features] x [16 rows of the block] per instruction;
//   uq, uqs: u split into NSU FP8 parts with one scale per (part, row b, 128-block) — the activation layout the
//            W_O pass reads ([part][rows][H*hd] and [part][rows][H*hd/128]).
// Every partial of the block (at most 128 KB: rb * nsplit * Dv <= 32,768 floats) is loaded up front, 32 16-byte
// loads a thread, together with this wave's W_UV codes.
static constexpr int MW_RB = 16;      // rows per workgroup at most (the N side of one instruction)
static constexpr int MW_ROW_FORM_MAX_ROWS = 8;  // up to this many rows, one workgroup per (row, head)
static constexpr int MW_LOADS = 32;   // 16-byte partial loads per thread

// Row tiles of W_UV[h] per wave (hd / 64) and K-blocks (Dv / 128).
template <int TPW, int NKB, int NSU, bool TL>
__global__ __launch_bounds__(256, 2) void k_merge_wuv(const float *__restrict__ opart, const float *__restrict__ ml,
                                                      int nsplit, int rows, int H, int rb, float *__restrict__ o,
                                                      const uint8_t *__restrict__ wuv, const float *__restrict__ wsc,
                                                      uint8_t *__restrict__ uq, float *__restrict__ uqs, long uq_part,
                                                      long uqs_part)
{
    constexpr int Dv = NKB * 128, hd = TPW * 64, NRB = hd / 128;
    constexpr int FQ = Dv / 4;  // feature quads of a row
    __shared__ float s_wt[MW_RB][AM_MAXSPLIT];
    __shared__ __attribute__((aligned(16))) float s_o[MW_RB][Dv + 4];  // padded: the operand reads take 16 rows
    __shared__ float s_u[MW_RB][hd + 1];
    const int h = blockIdx.x, b0 = blockIdx.y * rb;
    const int nb = min(rb, rows - b0);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, ln = lane & 15, lg = lane >> 4;
    // 1. the split maxima and sums of this wave's rows (w, w + 4, ...), first, so that the weights below wait
    //    only for them
    float mv[MW_RB / 4], lv[MW_RB / 4];
#pragma unroll
    for (int q = 0; q < MW_RB / 4; q++) {
        const int b = min(w + 4 * q, nb - 1);
        const int sp = min(lane, nsplit - 1);
        const long mi = (((long)(b0 + b) * nsplit + sp) * H + h) * 2;
        mv[q] = ml[mi];
        lv[q] = ml[mi + 1];
    }
    // 2. this wave's W_UV[h] operands: row tiles w * TPW .. + TPW (16 rows each), every 128-column block; lane
    //    (ln, lg) holds row ln's columns lg*16 .. +16 and 64 + lg*16 .. +16 of the block (32 codes)
    v4i A[TPW][NKB][2];
#pragma unroll
    for (int t = 0; t < TPW; t++)
#pragma unroll
        for (int kb = 0; kb < NKB; kb++) {
            const int tile = w * TPW + t;
            const uint8_t *p = TL ? wuv + (((long)h * (hd / 16) + tile) * NKB + kb) * 2048 + lane * 16
                                  : wuv + ((long)h * hd + tile * 16 + ln) * Dv + kb * 128 + lg * 16;
            A[t][kb][0] = __builtin_nontemporal_load((const v4i *)p);
            A[t][kb][1] = __builtin_nontemporal_load((const v4i *)(p + (TL ? 1024 : 64)));
        }
    // 3. every partial of the block: load k of a thread is split k % nsplit of its pair k / nsplit, where pair j of
    //    thread tid is (row, feature quad) number tid + 256 j; so a pair's splits are summed in one thread, in order.
    //    Every load is issued (loads past the thread's pairs re-read a valid one and are not used).
    const int npair = MW_LOADS / nsplit;
    const long sstride = (long)H * Dv;
    auto pair_ptr = [&](int j) {
        const int pi = tid + 256 * min(j, npair - 1);
        const int b = min(pi / FQ, nb - 1), fq = pi % FQ;
        return opart + ((long)(b0 + b) * nsplit * H + h) * Dv + fq * 4;
    };
    v4f pv[MW_LOADS];
    {
        const float *ptr = pair_ptr(0);
        int sp = 0, j = 0;
#pragma unroll
        for (int k = 0; k < MW_LOADS; k++) {
            pv[k] = *(const v4f *)ptr;
            ptr += sstride;
            if (++sp == nsplit) {
                sp = 0;
                ptr = pair_ptr(++j);
            }
        }
    }
    // split weights w_s = e^(m_s - M) / sum_s e^(m_s - M) l_s (0 for an empty split)
#pragma unroll
    for (int q = 0; q < MW_RB / 4; q++) {
        const int b = w + 4 * q;
        if (b < nb) {
            const bool ok = lane < nsplit;
            const float m = ok ? mv[q] : -INFINITY;
            const float l = ok ? lv[q] : 0.f;
            const float M = wave_max(m);
            const float e = m == -INFINITY ? 0.f : expf(m - M);
            const float den = wave_sum(e * l);
            if (lane < AM_MAXSPLIT) s_wt[b][lane] = den > 0.f ? e / den : 0.f;
        }
    }
    __syncthreads();
    // 3. merge: o[b] = sum over the splits in order of w_s O_s[b]
    {
        int sp = 0, j = 0;
        v4f cur = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < MW_LOADS; k++) {
            const int pi = tid + 256 * j, b = pi / FQ, fq = pi % FQ;
            if (j < npair && b < nb) {
                const float wt = s_wt[b][sp];
                if (wt != 0.f) cur += pv[k] * wt;
                if (sp == nsplit - 1) {
                    *(v4f *)&s_o[b][fq * 4] = cur;
                    cur = v4f{0.f, 0.f, 0.f, 0.f};
                }
            }
            if (++sp == nsplit) { sp = 0; j++; }
        }
    }
    __syncthreads();
    if (o)
        for (int i = tid; i < nb * FQ; i += 256) {
            const int b = i / FQ, fq = i % FQ;
            *(v4f *)(o + ((long)(b0 + b) * H + h) * Dv + fq * 4) = *(const v4f *)&s_o[b][fq * 4];
        }
    // 4. u = W_UV[h] o on the matrix cores.  K order inside a 128-column block: step ks takes lane byte range
    //    [8 ks, 8 ks + 8) of its 32 codes, i.e. columns (ks < 2 ? 0 : 64) + lg*16 + (ks & 1) * 8 .. + 8; the o side
    //    reads the same columns.
    {
        v4f acc[TPW];
#pragma unroll
        for (int t = 0; t < TPW; t++) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
        const int rblk = (w * TPW * 16) / 128;  // this wave's tiles lie in one 128-row scale block
        const bool bv = ln < nb;
#pragma unroll
        for (int kb = 0; kb < NKB; kb++) {
            const float sc = wsc[((long)h * NRB + rblk) * NKB + kb];
#pragma unroll
            for (int ks = 0; ks < 4; ks++) {
                const int c = kb * 128 + (ks < 2 ? 0 : 64) + lg * 16 + (ks & 1) * 8;
                v4f x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
                if (bv) {
                    x0 = *(const v4f *)&s_o[ln][c] * sc;
                    x1 = *(const v4f *)&s_o[ln][c + 4] * sc;
                }
                const float xs[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
                v8bf Bh, Bl;
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const __bf16 hb = (__bf16)xs[e];
                    Bh[e] = hb;
                    Bl[e] = (__bf16)(xs[e] - (float)hb);
                }
#pragma unroll
                for (int t = 0; t < TPW; t++) {
                    const uint32_t w0 = (uint32_t)A[t][kb][ks >> 1][(ks & 1) * 2];
                    const uint32_t w1 = (uint32_t)A[t][kb][ks >> 1][(ks & 1) * 2 + 1];
                    const v8bf Aw = fp8x8_to_bf16(w0, w1);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Aw, Bh, acc[t], 0, 0, 0);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Aw, Bl, acc[t], 0, 0, 0);
                }
            }
        }
        // lane (ln, lg) holds u[row ln][W_UV rows tile*16 + 4 lg .. + 4]
        if (bv) {
#pragma unroll
            for (int t = 0; t < TPW; t++)
#pragma unroll
                for (int i = 0; i < 4; i++) s_u[ln][(w * TPW + t) * 16 + 4 * lg + i] = acc[t][i];
        }
    }
    __syncthreads();
    // 5. split u into NSU parts, one wave per (row, 128-row block of u)
    const long K = (long)H * hd;
    for (int it = w; it < nb * NRB; it += 4) {
        const int b = it / NRB, j = it % NRB;
        const int r0 = j * 128 + lane * 2;
        float x0 = s_u[b][r0], x1 = s_u[b][r0 + 1];
        const long e = (long)(b0 + b) * K + (long)h * hd + r0;
        const long sc_i = (long)(b0 + b) * (K / 128) + (long)h * NRB + j;
#pragma unroll
        for (int sp = 0; sp < NSU; sp++) {
            const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
            const float scale = amax > 0.f ? amax * (1.0f / 448.0f) : 1.0f;
            const float iv = 1.0f / scale;
            const uint32_t code = f32x2_to_fp8(fminf(fmaxf(x0 * iv, -448.f), 448.f), fminf(fmaxf(x1 * iv, -448.f), 448.f));
            *(uint16_t *)(uq + sp * uq_part + e) = (uint16_t)code;
            if (lane == 0) uqs[sp * uqs_part + sc_i] = scale;
            const v2f d = fp8x2_lo(code);
            x0 -= d.x * scale;
            x1 -= d.y * scale;
        }
    }
}

// Value widths 128, 256 or 512 with hd = 128, and 128 or 256 with hd = 256 (the kernel's register budget).
bool attention_merge_uv_ok(int Dv, int hd)
{
    return (Dv == 128 || Dv == 256 || Dv == 512) && (hd == 128 || (hd == 256 && Dv <= 256));
}

// Rows per merge workgroup: every partial of the block fits the threads' loads, and about 256 workgroups.
static int merge_rows(int rows, int H, int nsplit, int Dv)
{
    // pairs (row, feature quad) per thread: MW_LOADS / nsplit, so rb * Dv / 4 <= 256 * (MW_LOADS / nsplit)
    int rb = std::max(1, std::min(MW_RB, (256 * (MW_LOADS / nsplit)) / (Dv / 4)));
    const int want = std::max(1, (rows * H + 255) / 256);
    return std::min(rb, std::max(1, std::min(want, rows)));
}

int launch_attn_merge_uv(int B, int H, int Dv, int top_k, const float *opart, const float *ml, float *o,
                         const uint8_t *wuv, const float *wsc, int hd, int tiled, uint8_t *uq, float *uqs,
                         long uq_part, long uqs_part, hipStream_t s)
{
    const int nsplit = attention_splits(top_k, B, H);
    if (B <= MW_ROW_FORM_MAX_ROWS) {
        hipLaunchKernelGGL((k_attn_merge_uv_row<4>), dim3(B * H), dim3(256), 0, s, opart, ml, nsplit, H, Dv, o, wuv, wsc, hd,
                           tiled, uq, uqs, uq_part, uqs_part);
        return hip_check("attn_merge_uv_row");
    }
    const int rb = merge_rows(B, H, nsplit, Dv);
    const dim3 g(H, (B + rb - 1) / rb);
#define DL_MW(TPW_, NKB_)                                                                                           \
    if (hd == TPW_ * 64 && Dv == NKB_ * 128) {                                                                     \
        if (tiled)                                                                                                 \
            hipLaunchKernelGGL((k_merge_wuv<TPW_, NKB_, 4, true>), g, dim3(256), 0, s, opart, ml, nsplit, B, H, rb, o, \
                               wuv, wsc, uq, uqs, uq_part, uqs_part);                                               \
        else                                                                                                       \
            hipLaunchKernelGGL((k_merge_wuv<TPW_, NKB_, 4, false>), g, dim3(256), 0, s, opart, ml, nsplit, B, H, rb,  \
                               o, wuv, wsc, uq, uqs, uq_part, uqs_part);                                            \
        return hip_check("attn_merge_uv");                                                                          \
    }
    DL_MW(2, 1) DL_MW(2, 2) DL_MW(2, 4) DL_MW(4, 1) DL_MW(4, 2)
#undef DL_MW
    return fail(DL_ERR_UNSUPPORTED, "attention merge: d_v %d with head_dim %d", Dv, hd);
}

bool attention_mfma_ok(int H, int Dc, int Dv, int q_dt, int kv_dt)
{
    return kv_dt == DL_FP8_E4M3 && q_dt == DL_BF16 && H % 16 == 0 &&
           (Dc == 576 || Dc == 512 || Dc == 256 || Dc == 128) && (Dv == 128 || Dv == 256 || Dv == 512) && Dv <= Dc;
}

// Kept positions per split: about 256 workgroups over the batch, whole chunks of 64, at most 512; the number
// of splits follows (at most 32).
#ifndef DL_ATT_WGS
#define DL_ATT_WGS 256
#endif
static int attention_pps(int top_k, int B, int H)
{
    const int hs = (H + 63) / 64;
    const long want = std::max(1L, (long)DL_ATT_WGS / ((long)B * hs));
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
            hipLaunchKernelGGL((k_attn_mla<KQ_, NVB_>), g, dim3(512), 0, s, (const uint16_t *)q,                    \
                               (const uint8_t *)kv, kv_scale, pg.page_table, pg.max_pages_per_seq, R, ps_shift, sel,    \
                               top_k, H, pps, sm_scale, opart, ml);                                                 \
        else                                                                                                        \
            hipLaunchKernelGGL((k_attn_mla1<KQ_, NVB_>), g, dim3(256), 0, s, (const uint16_t *)q,                   \
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
