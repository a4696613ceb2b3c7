// S3 + S4: sparse MLA decode attention over the kept positions only.
//
// Kiln's decode kernel gathers the selected entries instead of masking every key ("The decode
// kernels, and why they are opt-in", Introducing Kiln); the cache is one compressed latent per
// position shared by all heads ("How was Kiln measured against vLLM on H200?").  The key is the
// whole latent (d_c features), the value its first d_v features.
//
// Two kernels:
//  * k_attn_mfma (FP8 latents, bf16 queries, 16 | heads): split over the kept positions like flash
//    decoding.  A workgroup owns 16 heads of one row and a run of kept positions, staged 64 at a time
//    into LDS through the page table.  Scores are a [16 heads x 64] x [64 x d_c] product on the matrix
//    cores (v_mfma_f32_16x16x32_bf16): the queries are bf16 already and every e4m3 code is exactly a
//    bf16, so the products are exact and each 128-feature block's sum takes its scale once.  The
//    softmax runs online across chunks in fp32.  For the values, wave w owns a quarter of the d_v
//    features and computes O^T = C^T P' with P' = p * (block scale) split into bf16 high and low
//    halves (about 16 significant bits), so the output keeps fp32-level accuracy.  A small kernel
//    merges the splits (max-rescaled sums).
//  * k_attn (any shape, fp32 or FP8 latents): a workgroup owns 4 heads of one row and scores every
//    kept position on the vector units in fp32.
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


// ----------------------------------------------------------------------------- matrix-core path
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

static constexpr int AM_NJ = 64;     // kept positions per chunk (one 16-position tile per wave)
static constexpr int AM_MAXDC = 1024;
static constexpr int AM_MAXNB = 8;   // 128-feature blocks of the latent
static constexpr int AM_MAXSPLIT = 32;  // splits of the kept positions (top_k <= 4,096)
static constexpr int AM_CHUNKS = 2;     // chunks per split: 128 kept positions per workgroup

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

// grid (nsplit, H/16, B), 256 threads.  opart [B, nsplit, H, Dv] unnormalised sums, ml [B, nsplit, H, 2].
// The split's page-table lookups happen once up front; chunk c+1's latent codes are loaded into registers
// while chunk c is computed (double buffering through LDS); the queries sit in LDS.
template <int KQ, int CH>  // d_c / 32, chunks of 64 positions per split
__global__ __launch_bounds__(256) void k_attn_mfma(const uint16_t *__restrict__ q, const uint8_t *__restrict__ kv,
                                                   const float *__restrict__ ks, const int32_t *__restrict__ pt,
                                                   int max_pages, int ps_shift, const int32_t *__restrict__ sel,
                                                   int top_k, int H, int Dv, float sm_scale,
                                                   float *__restrict__ opart, float *__restrict__ ml)
{
    constexpr int Dc = KQ * 32;
    constexpr int DCP = Dc + 16;  // padded LDS row: conflict-free 8-byte reads across 16 positions
    constexpr int NB = (Dc + 127) / 128;
    constexpr int NP = CH * AM_NJ;                       // positions of the split
    constexpr int NLD = (AM_NJ * (Dc / 16) + 255) / 256;  // 16-byte code loads per thread per chunk
    __shared__ __attribute__((aligned(16))) uint8_t s_c[AM_NJ * DCP];
    __shared__ __attribute__((aligned(16))) uint16_t s_q[16 * Dc];
    __shared__ float s_sc[NP][NB];
    __shared__ float s_p[16][AM_NJ + 4];
    __shared__ long s_row[NP];
    __shared__ float s_red[4][16];
    __shared__ float s_m[16], s_l[16], s_alpha[16];
    const int split = blockIdx.x, h0 = blockIdx.y * 16, b = blockIdx.z;
    const int nsplit = gridDim.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, ln = lane & 15, lg = lane >> 4;
    const int ps_mask = (1 << ps_shift) - 1;
    const int jbase = split * NP;
    // queries of the 16 heads -> LDS; rows and scales of every position of the split
    for (int i = tid; i < 16 * Dc / 8; i += 256)
        *(v4i *)(s_q + i * 8) = *(const v4i *)(q + ((long)b * H + h0) * Dc + i * 8);
    for (int i = tid; i < NP; i += 256) {
        const int j = jbase + i;
        const int p = j < top_k ? sel[(long)b * top_k + j] : -1;
        s_row[i] = p < 0 ? -1 : ((long)pt[(long)b * max_pages + (p >> ps_shift)] << ps_shift) + (p & ps_mask);
    }
    if (tid < 16) { s_m[tid] = -INFINITY; s_l[tid] = 0.f; }
    __syncthreads();
    for (int i = tid; i < NP * NB; i += 256) {
        const long row = s_row[i / NB];
        s_sc[i / NB][i % NB] = row < 0 ? 0.f : ks[row * NB + i % NB];
    }
    const int nch = min(CH, (top_k - jbase + AM_NJ - 1) / AM_NJ);
    // chunk 0's codes into registers
    v4i R[NLD];
    auto load_chunk = [&](int ch) {
#pragma unroll
        for (int k = 0; k < NLD; k++) {
            const int id = k * 256 + tid;
            R[k] = v4i{0, 0, 0, 0};
            if (id < AM_NJ * (Dc / 16)) {
                const int pos = id / (Dc / 16), c16 = id % (Dc / 16);
                const long row = s_row[ch * AM_NJ + pos];
                if (row >= 0) R[k] = *(const v4i *)(kv + row * Dc + c16 * 16);
            }
        }
    };
    if (nch > 0) load_chunk(0);
    const int vw = Dv >> 2, vt0 = w * (vw >> 4), nvt = vw >> 4;
    v4f acc[8];
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int ch = 0; ch < nch; ch++) {
        __syncthreads();  // the previous chunk's LDS reads are done
#pragma unroll
        for (int k = 0; k < NLD; k++) {
            const int id = k * 256 + tid;
            if (id < AM_NJ * (Dc / 16)) *(v4i *)(s_c + (id / (Dc / 16)) * DCP + (id % (Dc / 16)) * 16) = R[k];
        }
        __syncthreads();
        if (ch + 1 < nch) load_chunk(ch + 1);  // in flight while this chunk is computed
        const int jl = w * 16 + ln;             // this lane's position within the chunk
        const int jp = ch * AM_NJ + jl;         // ... within the split
        v4f S = {0.f, 0.f, 0.f, 0.f};
        const uint8_t *cr = s_c + jl * DCP + lg * 8;
        const uint16_t *qr = s_q + ln * Dc + lg * 8;
#pragma unroll
        for (int blk = 0; blk < NB; blk++) {
            v4f a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = blk * 4; kk < (blk * 4 + 4 < KQ ? blk * 4 + 4 : KQ); kk++) {
                const uint2 cw = *(const uint2 *)(cr + kk * 32);
                const v8bf Aq = *(const v8bf *)(qr + kk * 32);
                a = mfma_bf16(Aq, fp8x8_to_bf16(cw.x, cw.y), a);
            }
            S += a * s_sc[jp][blk];
        }
        const bool valid = s_row[jp] >= 0;
        float sv[4];
#pragma unroll
        for (int i = 0; i < 4; i++) sv[i] = valid ? S[i] * sm_scale : -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float m = max16(sv[i]);
            if (ln == 0) s_red[w][4 * lg + i] = m;
        }
        __syncthreads();
        if (tid < 16) {
            const float mc = fmaxf(fmaxf(s_red[0][tid], s_red[1][tid]), fmaxf(s_red[2][tid], s_red[3][tid]));
            const float mo = s_m[tid], mn = fmaxf(mo, mc);
            s_alpha[tid] = (mn == -INFINITY) ? 1.f : expf(mo - mn);
            s_m[tid] = mn;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int hh = 4 * lg + i;
            const float mn = s_m[hh];
            const float pv = (sv[i] == -INFINITY) ? 0.f : expf(sv[i] - mn);
            s_p[hh][jl] = pv;
            const float ssum = sum16(pv);
            if (ln == 0) s_red[w][hh] = ssum;
        }
        __syncthreads();
        if (tid < 16) s_l[tid] = s_l[tid] * s_alpha[tid] + (s_red[0][tid] + s_red[1][tid] + s_red[2][tid] + s_red[3][tid]);
        const float al = s_alpha[ln];
#pragma unroll
        for (int i = 0; i < 8; i++) acc[i] *= al;
#pragma unroll
        for (int kk = 0; kk < AM_NJ / 32; kk++) {
            const int jj = kk * 32 + lg * 8;
            float pr[8];
#pragma unroll
            for (int e = 0; e < 8; e++) pr[e] = s_p[ln][jj + e];
            int cur_blk = -1;
            v8bf Bh, Bl;
#pragma unroll
            for (int t = 0; t < 8; t++) {
                if (t >= nvt) break;
                const int v0 = (vt0 + t) * 16;
                const int blk = v0 >> 7;
                if (blk != cur_blk) {
                    cur_blk = blk;
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        const float x = pr[e] * s_sc[ch * AM_NJ + jj + e][blk];
                        const __bf16 hi = (__bf16)x;
                        Bh[e] = hi;
                        Bl[e] = (__bf16)(x - (float)hi);
                    }
                }
                const uint8_t *cc = s_c + jj * DCP + v0 + ln;
                uint32_t w0 = 0, w1 = 0;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    w0 |= (uint32_t)cc[e * DCP] << (8 * e);
                    w1 |= (uint32_t)cc[(e + 4) * DCP] << (8 * e);
                }
                const v8bf Av = fp8x8_to_bf16(w0, w1);
                acc[t] = mfma_bf16(Av, Bh, acc[t]);
                acc[t] = mfma_bf16(Av, Bl, acc[t]);
            }
        }
    }
    __syncthreads();
    float *op = opart + (((long)b * nsplit + split) * H + h0 + ln) * Dv;
#pragma unroll
    for (int t = 0; t < 8; t++) {
        if (t >= nvt) break;
        *(v4f *)(op + (vt0 + t) * 16 + 4 * lg) = acc[t];
    }
    if (tid < 16) {
        float *m2 = ml + (((long)b * nsplit + split) * H + h0 + tid) * 2;
        m2[0] = s_m[tid];
        m2[1] = s_l[tid];
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
template <int NSU>
__global__ __launch_bounds__(256) void k_attn_merge_uv(const float *__restrict__ opart, const float *__restrict__ ml,
                                                       int nsplit, int H, int Dv, float *__restrict__ o,
                                                       const uint8_t *__restrict__ wuv, const float *__restrict__ wsc,
                                                       int hd, int tiled, uint8_t *__restrict__ uq,
                                                       float *__restrict__ uqs, long uq_part, long uqs_part)
{
    __shared__ float s_o[1024];
    __shared__ float s_u[256][2];
    __shared__ float s_w[4];
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    // 1. merge the splits
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
    for (int v = tid; v < Dv; v += 256) {
        float op[AM_MAXSPLIT];
#pragma unroll
        for (int s2 = 0; s2 < AM_MAXSPLIT; s2++)
            op[s2] = s2 < nsplit ? opart[(((long)b * nsplit + s2) * H + h) * Dv + v] : 0.f;
        float num = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < AM_MAXSPLIT; s2++)
            if (s2 < nsplit && sm[s2] != 0.f) num += sm[s2] * op[s2];
        const float ov = num * inv;
        s_o[v] = ov;
        o[(long)bh * Dv + v] = ov;
    }
    __syncthreads();
    // 2. u = W_UV[h] o: thread -> (row r, half of the columns); 16 codes per load
    const int nkb = Dv / 128, nrb = (hd + 127) / 128;
    const int per_row = 256 / hd;  // 2 (hd = 128) or 1 (hd = 256)
    const int r = tid / per_row, part = tid % per_row;
    const int c_lo = part * (Dv / per_row), c_hi = c_lo + Dv / per_row;
    const uint8_t *wm = wuv + (long)h * hd * Dv;
    float acc = 0.f;
    for (int c0 = c_lo; c0 < c_hi; c0 += 128) {
        const int kb = c0 / 128;
        float blk = 0.f;
#pragma unroll
        for (int q = 0; q < 8; q++) {
            const int c = c0 + q * 16;
            long off;
            if (tiled) {
                const int hh = (c % 128) / 64, lg = (c % 64) / 16, l = lg * 16 + r % 16;
                off = ((long)(r / 16) * nkb + kb) * 2048 + hh * 1024 + l * 16;
            } else {
                off = (long)r * Dv + c;
            }
            const v4i w = *(const v4i *)(wm + off);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const v2f lo = fp8x2_lo((uint32_t)w[i]), hi = fp8x2_hi((uint32_t)w[i]);
                blk = fmaf(lo.x, s_o[c + 4 * i], blk);
                blk = fmaf(lo.y, s_o[c + 4 * i + 1], blk);
                blk = fmaf(hi.x, s_o[c + 4 * i + 2], blk);
                blk = fmaf(hi.y, s_o[c + 4 * i + 3], blk);
            }
        }
        acc = fmaf(blk, wsc[((long)h * nrb + r / 128) * nkb + kb], acc);
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
    (void)s_w;
}

bool attention_merge_uv_ok(int Dv, int hd) { return Dv % 128 == 0 && Dv <= 1024 && (hd == 128 || hd == 256); }

int launch_attn_merge_uv(int B, int H, int Dv, int top_k, const float *opart, const float *ml, float *o,
                         const uint8_t *wuv, const float *wsc, int hd, int tiled, uint8_t *uq, float *uqs,
                         long uq_part, long uqs_part, hipStream_t s)
{
    hipLaunchKernelGGL((k_attn_merge_uv<4>), dim3(B * H), dim3(256), 0, s, opart, ml, attention_splits(top_k), H, Dv,
                       o, wuv, wsc, hd, tiled, uq, uqs, uq_part, uqs_part);
    return hip_check("attn_merge_uv");
}

bool attention_mfma_ok(int H, int Dc, int Dv, int q_dt, int kv_dt)
{
    return kv_dt == DL_FP8_E4M3 && q_dt == DL_BF16 && H % 16 == 0 && (Dc == 576 || Dc == 512 || Dc == 256 ||
           Dc == 128) && Dv % 64 == 0 && Dv / 4 <= 128 && Dv <= Dc;
}

int attention_splits(int top_k) { return (top_k + AM_NJ * AM_CHUNKS - 1) / (AM_NJ * AM_CHUNKS); }

int launch_attention(const dl_pages &pg, const void *q, int q_dt, const void *kv, const float *kv_scale, int kv_dt,
                     int H, int Dc, int Dv, float sm_scale, const int32_t *sel, int top_k, float *o, float *opart,
                     float *ml, hipStream_t s)
{
    if (attention_mfma_ok(H, Dc, Dv, q_dt, kv_dt) && opart && ml) {
        const int ps_shift = __builtin_ctz((unsigned)pg.page_size);
        const int nsplit = attention_splits(top_k);
        dim3 g(nsplit, H / 16, pg.batch);
#define DL_AM(KQ_)                                                                                                  \
    if (Dc == KQ_ * 32)                                                                                             \
        hipLaunchKernelGGL((k_attn_mfma<KQ_, AM_CHUNKS>), g, dim3(256), 0, s, (const uint16_t *)q, (const uint8_t *)kv, \
                           kv_scale, pg.page_table, pg.max_pages_per_seq, ps_shift, sel, top_k, H, Dv, sm_scale,     \
                           opart, ml);
        DL_AM(18) DL_AM(16) DL_AM(8) DL_AM(4)
#undef DL_AM
        if (o) hipLaunchKernelGGL(k_attn_merge, dim3(pg.batch * H), dim3(256), 0, s, opart, ml, nsplit, H, Dv, o);
        return hip_check("attention_mfma");
    }
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
