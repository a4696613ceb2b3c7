// Current-token append: the new token's latent and indexer key are quantised and written into the
// token's cache slot, in the layout the indexer (S1) and the attention gather (S3) read.
//
// The latent cache holds OCP e4m3fn codes with one fp32 scale per (token, 128-feature block) and the key
// cache holds int8 keys (Introducing Kiln, "How was Kiln measured against vLLM on H200?": an FP8 latent
// cache; "What moved the number ...": a separate key cache scored by its own kernel).  Per block the scale
// is amax / 448 and the codes are the fp32 quotients rounded to e4m3 (nearest, ties to even, clamped to
// +-448 first, so nothing overflows); the key is key / key_scale rounded half to even and clamped to
// +-127.  Padding rows write nothing, and of several rows that address one physical slot only the lowest
// writes it ("What could only a device show?": padded rows that raced for one slot changed real outputs).
#include "dl_common.h"
#include "dl_internal.h"

namespace dl {

__device__ __forceinline__ float wave_max_f(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// One workgroup (256 threads) per row.  Wave w quantises latent blocks w, w + 4, ...; lane l holds features
// 128 j + l and 128 j + 64 + l of block j.
__global__ __launch_bounds__(256) void k_kv_append(const int *__restrict__ seq_lens, const int *__restrict__ pt,
                                                    int max_pages, int ps_shift, const void *latent, int lat_dt, int Dc,
                                                    const void *key, int key_dt, int DI, float key_scale,
                                                    uint8_t *kv, float *kv_scale, int8_t *kp, int key_tiles)
{
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int ps_mask = (1 << ps_shift) - 1;
    const int L = seq_lens[b];
    if (L <= 0) return;  // padding row
    const int p = L - 1;
    const long slot = ((long)pt[(long)b * max_pages + (p >> ps_shift)] << ps_shift) + (p & ps_mask);
    // the lowest row addressing this slot writes it; every other one stops here
    int clash = 0;
    for (int j = tid; j < b; j += 256) {
        const int Lj = seq_lens[j];
        if (Lj > 0) {
            const int pj = Lj - 1;
            const long sj = ((long)pt[(long)j * max_pages + (pj >> ps_shift)] << ps_shift) + (pj & ps_mask);
            clash |= sj == slot;
        }
    }
    if (__syncthreads_or(clash)) return;

    const int nb = (Dc + 127) / 128;
    for (int j = w; j < nb; j += 4) {
        const int d0 = j * 128 + lane, d1 = d0 + 64, end = min(Dc, j * 128 + 128);
        const float v0 = d0 < end ? act_load(latent, lat_dt, (long)b * Dc + d0) : 0.f;
        const float v1 = d1 < end ? act_load(latent, lat_dt, (long)b * Dc + d1) : 0.f;
        const float amax = wave_max_f(fmaxf(fabsf(v0), fabsf(v1)));
        const float s = __fdiv_rn(amax, 448.f);
        uint32_t c0 = 0, c1 = 0;
        if (s != 0.f) {
            const float q0 = fminf(fmaxf(__fdiv_rn(v0, s), -448.f), 448.f);
            const float q1 = fminf(fmaxf(__fdiv_rn(v1, s), -448.f), 448.f);
            const uint32_t c = f32x2_to_fp8(q0, q1);
            c0 = c & 0xFFu;
            c1 = (c >> 8) & 0xFFu;
        }
        if (d0 < end) kv[slot * Dc + d0] = (uint8_t)c0;
        if (d1 < end) kv[slot * Dc + d1] = (uint8_t)c1;
        if (lane == 0) kv_scale[slot * nb + j] = s;
    }
    for (int i = tid; i < DI; i += 256) {
        const float t = __builtin_rintf(__fdiv_rn(act_load(key, key_dt, (long)b * DI + i), key_scale));
        kp[key_offset(slot, i, DI, key_tiles)] = (int8_t)fminf(fmaxf(t, -127.f), 127.f);
    }
}

// Row-major key cache -> tiles: thread o writes the 16 bytes at tiled offset 16 o, read from their item's row.
__global__ __launch_bounds__(256) void k_tile_keys(const int8_t *__restrict__ src, int8_t *__restrict__ dst, long n16,
                                                   int DI)
{
    for (long o = (long)blockIdx.x * 256 + threadIdx.x; o < n16; o += (long)gridDim.x * 256) {
        const long byte = o * 16, gsz = 16L * DI, grp = byte / gsz;
        const int in = (int)(byte - grp * gsz);  // kc * 1024 + g * 256 + p * 16
        const int kc = in >> 10, g = (in >> 8) & 3, p = (in >> 4) & 15;
        *(v4i *)(dst + byte) = *(const v4i *)(src + (grp * 16 + p) * DI + kc * 64 + g * 16);
    }
}

int launch_tile_keys(const int8_t *src, int8_t *dst, long n_items, int DI, hipStream_t s)
{
    const long n16 = n_items * DI / 16;
    const long blocks = std::min<long>((n16 + 255) / 256, 65536);
    hipLaunchKernelGGL(k_tile_keys, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, n16, DI);
    return hip_check("tile_keys");
}

int launch_kv_append(const dl_pages &pg, const void *latent, int lat_dt, int Dc, const void *key, int key_dt, int DI,
                     float key_scale, uint8_t *kv, float *kv_scale, int8_t *kp, hipStream_t s)
{
    int shift = 0;
    while ((1 << shift) < pg.page_size) shift++;
    hipLaunchKernelGGL(k_kv_append, dim3(pg.batch), dim3(256), 0, s, pg.seq_lens, pg.page_table, pg.max_pages_per_seq,
                       shift, latent, lat_dt, Dc, key, key_dt, DI, key_scale, kv, kv_scale, kp,
                       pg.key_layout == DL_LAYOUT_TILES);
    return hip_check("kv_append");
}

}  // namespace dl
