// Practical-ceiling probes of the device, for the measurements that report
// each kernel against its roofline: a streaming copy (the HBM rate a plain
// read + write stream reaches) and an int8 MFMA loop (the matrix-core rate
// with no memory traffic).  Not part of the convolution path.
#include "ifx_probe.h"

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "ifx_internal.h"

namespace ifx {
namespace {

// Grid-stride copy of 16-byte chunks, non-temporal loads and stores (data moved once).
__global__ __launch_bounds__(256) void probe_copy_kernel(const v4i *src, v4i *dst, long long chunks)
{
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < chunks; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// A 4 x 4 tile of independent accumulator chains of v_mfma_i32_16x16x64_i8 per wave (the shape of
// the convolution kernels' main loop) on register operands: the loop issues matrix instructions
// only.  Each wave writes one sum so nothing is dropped.
__global__ __launch_bounds__(256) void probe_mfma_kernel(int *out, int iters, int seed)
{
    const int lane = threadIdx.x & 63;
    v4i af[4], bf[4], acc[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        af[t] = (v4i){seed + lane + t, seed ^ lane, lane * 3 + t, seed - lane};
        bf[t] = (v4i){lane ^ t, seed + t, lane ^ 5, seed + 1 - t};
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
#pragma unroll
            for (int tn = 0; tn < 4; ++tn)
                acc[tm][tn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[tm], bf[tn], it == 0 ? (v4i){0, 0, 0, 0}
                                                                                            : acc[tm][tn], 0, 0, 0);
    }
    v4i s = {0, 0, 0, 0};
#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) s += acc[tm][tn];
    if (lane == 0) out[blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = s.x + s.y + s.z + s.w;
}

}  // namespace
}  // namespace ifx

extern "C" {

int32_t ifx_probe_copy(const void *src, void *dst, size_t bytes, void *stream)
{
    if (!src || !dst) return 1;
    if ((bytes & 15u) || ((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u)) return 4;
    const long long chunks = (long long)(bytes / 16);
    if (chunks == 0) return 0;
    int cus = 0;
    if (ifx::current_cus(&cus) != hipSuccess) return 6;
    long long grid = (chunks + 255) / 256;
    if (grid > 64LL * cus) grid = 64LL * cus;
    hipLaunchKernelGGL(ifx::probe_copy_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                       (const ifx::v4i *)src, (ifx::v4i *)dst, chunks);
    return hipGetLastError() == hipSuccess ? 0 : 6;
}

int32_t ifx_probe_mfma_i8(int32_t *out, int32_t blocks, int32_t iters, void *stream)
{
    if (!out) return 1;
    if (blocks <= 0 || iters <= 0) return 2;
    hipLaunchKernelGGL(ifx::probe_mfma_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, out,
                       iters, 7);
    return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // extern "C"
