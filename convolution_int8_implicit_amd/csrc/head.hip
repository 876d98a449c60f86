// Global average pool of a packed int8 tensor to int8 (the head in front of
// the FC layer).  The pages' only head is the float AdaptiveAvgPool + Linear
// of the quantisation example in the "Benchmark Device to SOTA Device" page;
// the integer reading used here is out[b,c] = round_half_away(sum_hw x / HW),
// saturated to int8, in the packed layout [n, c1, 1, 1, 32].
//
// HBM-bound: one wave owns one (image, channel block) plane.  Lane l reads
// word l % 8 (4 channels) of pixels l / 8, l / 8 + 8, ..., so each load
// instruction covers 8 consecutive 32-byte pixel vectors (256 contiguous
// bytes); the 8 pixel-group sums are then combined across the wave.
#include "ifx_internal.h"

namespace ifx {
namespace {

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
    unsigned out = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int mag = s[e] < 0 ? -s[e] : s[e];
        int q = (2 * mag + hw) / (2 * hw);  // floor(|s|/hw + 1/2)
        q = s[e] < 0 ? -q : q;
        q = min(max(q, -128), 127);
        out |= (unsigned)(q & 0xff) << (8 * e);
    }
    ((unsigned *)(y + plane * 32))[word] = out;
}

}  // namespace

hipError_t launch_avgpool(const int8_t *x, int8_t *y, int n, int c1, int hw, hipStream_t s)
{
    long long planes = (long long)n * c1;
    long long blocks = (planes + 3) / 4;  // one wave per plane, four per workgroup
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(avgpool_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, y, planes, hw);
    return hipGetLastError();
}

}  // namespace ifx
