// Quantisation of the input image and dequantisation of the logits on the device.
//
// The Alibaba inference article (Hanguang 800 section) runs the engine on
// integer data and moves the quantisation before it and the dequantisation
// after it, which had run on the host and taken most of the latency, into the
// accelerated pre- and post-processing.  With the path's symmetric int8 codes
// (real = s_x * code), per element of an NHWC tensor (channel = index mod c):
//   fp32 image:  code = sat8(round_half_away(x * mult[ch]))
//   uint8 image: code = sat8(round_half_away(((float)u - mean[ch]) * mult[ch]))
//   logits:      y = (float)q * scale
// Every step is one IEEE single-precision operation (round to nearest even;
// contraction is off in this file), so the codes are reproducible bit for bit.
//
// The kernels are streaming and HBM-bound (5 bytes per image element, 8 per
// logit): each thread converts four consecutive elements per step, one 16- or
// 4-byte load and one 4- or 16-byte store, in a grid-stride loop.
#include "device_common.h"
#include "ifx_internal.h"

#pragma clang fp contract(off)

namespace ifx {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

// round half away from zero (roundf), saturated; NaN -> 0.  Clamping first keeps the conversion
// to int in range for any finite or infinite value.
__device__ __forceinline__ int code_of(float t)
{
    if (t != t) return 0;
    t = fminf(fmaxf(t, -1024.0f), 1024.0f);
    return min(max((int)roundf(t), -128), 127);
}

template <bool U8>
__device__ __forceinline__ float pre(const void *x, int i, const float *mean, int ch)
{
    if (U8) return (float)((const uint8_t *)x)[i] - mean[ch];
    return ((const float *)x)[i];
}

// Four elements i0 .. i0+3 per step; ch advances with the element and wraps at c.
template <bool U8>
__global__ __launch_bounds__(256) void quantize_kernel(const void *x, int8_t *q, int count, int c, unsigned cmul,
                                                       int cshr, const float *mean, const float *mult)
{
    const int nv = count >> 2;
    const int stride = (int)gridDim.x * 256;
    for (int v = (int)blockIdx.x * 256 + (int)threadIdx.x; v < nv; v += stride) {
        const int i0 = 4 * v;
        int ch = i0 - fdiv(i0, cmul, cshr) * c;
        float f[4];
        if (U8) {
            const unsigned w = ((const unsigned *)x)[v];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[e] = (float)((w >> (8 * e)) & 255u) - mean[ch];
                f[e] = f[e] * mult[ch];
                ch = ch + 1 == c ? 0 : ch + 1;
            }
        } else {
            const v4f w = ((const v4f *)x)[v];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[e] = w[e] * mult[ch];
                ch = ch + 1 == c ? 0 : ch + 1;
            }
        }
        ((unsigned *)q)[v] = pack4(code_of(f[0]), code_of(f[1]), code_of(f[2]), code_of(f[3]));
    }
    // the last count % 4 elements
    const int i = (nv << 2) + (int)threadIdx.x;
    if (blockIdx.x == 0 && i < count) {
        const int ch = i - fdiv(i, cmul, cshr) * c;
        q[i] = (int8_t)code_of(pre<U8>(x, i, mean, ch) * mult[ch]);
    }
}

__global__ __launch_bounds__(256) void dequantize_kernel(const int32_t *q, float *y, int count, float scale)
{
    const int nv = count >> 2;
    const int stride = (int)gridDim.x * 256;
    for (int v = (int)blockIdx.x * 256 + (int)threadIdx.x; v < nv; v += stride) {
        const v4i w = ((const v4i *)q)[v];
        v4f o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (float)w[e] * scale;
        ((v4f *)y)[v] = o;
    }
    const int i = (nv << 2) + (int)threadIdx.x;
    if (blockIdx.x == 0 && i < count) y[i] = (float)q[i] * scale;
}

int grid_for(int count)
{
    int cus = 0;
    if (current_cus(&cus) != hipSuccess || cus <= 0) cus = 256;
    const long long want = ((long long)(count >> 2) + 255) / 256;
    const long long cap = 8LL * cus;
    return (int)(want < 1 ? 1 : (want > cap ? cap : want));
}

}  // namespace

hipError_t launch_quantize(const void *x, bool u8, int8_t *q, int count, int c, const float *mean, const float *mult,
                           hipStream_t s)
{
    unsigned cmul = 0;
    int cshr = 0;
    fastdiv_magic((unsigned)c, &cmul, &cshr);
    const int g = grid_for(count);
    if (u8)
        hipLaunchKernelGGL(quantize_kernel<true>, dim3((unsigned)g), dim3(256), 0, s, x, q, count, c, cmul, cshr, mean,
                           mult);
    else
        hipLaunchKernelGGL(quantize_kernel<false>, dim3((unsigned)g), dim3(256), 0, s, x, q, count, c, cmul, cshr,
                           mean, mult);
    return hipGetLastError();
}

hipError_t launch_dequantize(const int32_t *q, float *y, int count, float scale, hipStream_t s)
{
    hipLaunchKernelGGL(dequantize_kernel, dim3((unsigned)grid_for(count)), dim3(256), 0, s, q, y, count, scale);
    return hipGetLastError();
}

}  // namespace ifx
