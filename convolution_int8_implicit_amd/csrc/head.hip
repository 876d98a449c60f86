// Global average pool of a packed int8 tensor to int8 (the head in front of
// the FC layer).  The pages' only head is the float AdaptiveAvgPool + Linear
// of the quantisation example in the "Benchmark Device to SOTA Device" page;
// the integer reading used here is out[b,c] = round_half_away(sum_hw x / HW),
// saturated to int8, in the packed layout [n, c1, 1, 1, 32].
//
// HBM-bound.  Two mappings of lanes to pixels and channels:
//   * few planes (small batches): one wave owns one (image, channel block) plane; lane l reads
//     word l % 8 (4 channels) of pixels l / 8, l / 8 + 8, ..., so each load instruction covers
//     256 contiguous bytes, and the 8 partial sums of a word are combined across the wave;
//   * many planes: one wave owns eight consecutive planes, lane l summing word l % 8 of plane
//     l / 8 over all of the plane's pixels.  No lanes need combining and each lane keeps many
//     independent loads in flight; the four loads that read one 128-byte line come from
//     consecutive instructions of the same wave (cached loads, so the line is fetched once).
#include "ifx_internal.h"

namespace ifx {
namespace {

constexpr int kPoolPlanesPerWave = 8;  // the many-plane mapping
constexpr long long kPoolManyPlanes = 4096;

// int8 average of a 4-channel word sum over hw pixels, rounded half away from zero, saturated
__device__ __forceinline__ unsigned pool_word(const int (&s)[4], int hw)
{
    unsigned out = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int mag = s[e] < 0 ? -s[e] : s[e];
        int q = (2 * mag + hw) / (2 * hw);  // floor(|s|/hw + 1/2)
        q = s[e] < 0 ? -q : q;
        q = min(max(q, -128), 127);
        out |= (unsigned)(q & 0xff) << (8 * e);
    }
    return out;
}

__global__ __launch_bounds__(256) void avgpool_kernel(const int8_t *__restrict__ x, int8_t *__restrict__ y,
                                                      long long planes, int hw)
{
    const long long plane = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, word = lane & 7;
    if (plane >= planes) return;  // the whole wave leaves together
    const unsigned *src = (const unsigned *)(x + plane * hw * 32) + word;
    int s[4] = {0, 0, 0, 0};
#pragma unroll 4
    for (int p = lane >> 3; p < hw; p += 8) {
        const unsigned v = __builtin_nontemporal_load(src + p * 8);  // read once
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] += (int)(signed char)(v >> (8 * e));
    }
#pragma unroll
    for (int o = 8; o < 64; o <<= 1)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] += __shfl_xor(s[e], o);
    if (lane >= 8) return;
    ((unsigned *)(y + plane * 32))[word] = pool_word(s, hw);
}

__global__ __launch_bounds__(256) void avgpool_lanes_kernel(const int8_t *__restrict__ x, int8_t *__restrict__ y,
                                                            long long planes, int hw)
{
    const int lane = threadIdx.x & 63, word = lane & 7;
    const long long plane = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * kPoolPlanesPerWave + (lane >> 3);
    if (plane >= planes) return;  // no cross-lane work follows
    const unsigned *src = (const unsigned *)(x + plane * hw * 32) + word;
    int s[4] = {0, 0, 0, 0};
#pragma unroll 8
    for (int p = 0; p < hw; ++p) {
        const unsigned v = src[p * 8];
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] += (int)(signed char)(v >> (8 * e));
    }
    ((unsigned *)(y + plane * 32))[word] = pool_word(s, hw);
}

}  // namespace

hipError_t launch_avgpool(const int8_t *x, int8_t *y, int n, int c1, int hw, hipStream_t s)
{
    const long long planes = (long long)n * c1;
    if (planes <= 0) return hipSuccess;
    if (planes < kPoolManyPlanes) {  // one wave per plane, four per workgroup
        hipLaunchKernelGGL(avgpool_kernel, dim3((unsigned)((planes + 3) / 4)), dim3(256), 0, s, x, y, planes, hw);
    } else {  // eight planes per wave
        const long long waves = (planes + kPoolPlanesPerWave - 1) / kPoolPlanesPerWave;
        hipLaunchKernelGGL(avgpool_lanes_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, x, y, planes,
                           hw);
    }
    return hipGetLastError();
}

}  // namespace ifx
