// Measurement aids, not part of the decode step.
// - A plain streaming read of a device buffer, to measure the HBM read rate the weight streams can reach for a
//   given content (the rate depends on the bytes read).  Every wave reads its own contiguous range with 16-byte
//   non-temporal loads, 16 in flight per lane, the way the expert GEMV streams weights.
// - A chain of kernels that do no work (Kiln's "null" kernel, used there to expose fixed costs, "What moved the
//   number from 19.4 to 122.9 tokens a second?"): the time of one dependent launch with nothing in it.
#include "dl_common.h"
#include "dl_internal.h"

namespace dl {

__device__ int g_probe_sink;  // externally visible, so the store (and the loads behind it) stay

constexpr int PROBE_U = 16;

__global__ __launch_bounds__(256) void k_probe_read(const v4i *__restrict__ p, long per_wave)
{
    const int lane = threadIdx.x & 63;
    const long w = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const v4i *q = p + w * per_wave;
    v4i acc = {0, 0, 0, 0};
    for (long i = 0; i < per_wave; i += PROBE_U * 64) {
        v4i a[PROBE_U];
#pragma unroll
        for (int u = 0; u < PROBE_U; u++) a[u] = __builtin_nontemporal_load(q + i + u * 64 + lane);
#pragma unroll
        for (int u = 0; u < PROBE_U; u++) acc ^= a[u];
    }
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x5EED5EED) g_probe_sink = 1;  // keeps the loads live
}

int launch_probe_read(const void *buf, size_t bytes, size_t *bytes_read, hipStream_t s)
{
    int dev = 0, cus = 1;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return hip_check("probe_read: device query");
    const long blocks = 4L * cus, waves = 4 * blocks;
    const long step = (long)PROBE_U * 64;  // 16-byte vectors per wave iteration
    const long per_wave = (long)(bytes / 16) / waves / step * step;
    if (per_wave <= 0) return fail(DL_ERR_SHAPE, "probe_read: %zu bytes is too small", bytes);
    hipLaunchKernelGGL(k_probe_read, dim3((unsigned)blocks), dim3(256), 0, s, (const v4i *)buf, per_wave);
    if (bytes_read) *bytes_read = (size_t)(per_wave * waves * 16);
    return hip_check("probe_read");
}

__global__ __launch_bounds__(256) void k_probe_null() {}

int launch_probe_null(int n_kernels, int blocks, hipStream_t s)
{
    for (int i = 0; i < n_kernels; i++) hipLaunchKernelGGL(k_probe_null, dim3(blocks), dim3(256), 0, s);
    return hip_check("probe_null");
}

}  // namespace dl
