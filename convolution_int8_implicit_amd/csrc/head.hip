// Global average pool of a packed int8 tensor to int8 (the head in front of
// the FC layer).  The pages' only head is the float AdaptiveAvgPool + Linear
// of the quantisation example in the "Benchmark Device to SOTA Device" page;
// the integer reading used here is out[b,c] = round_half_away(sum_hw x / HW),
// saturated to int8, in the packed layout [n, c1, 1, 1, 32].
//
// HBM-bound: one thread owns 4 channels (one 32-bit word) of one
// (image, channel block) plane and streams its HW words; 8 consecutive
// threads cover a plane's 32-byte pixel vectors.
#include "ifx_internal.h"

namespace ifx {
namespace {

__global__ __launch_bounds__(256) void avgpool_kernel(const int8_t *__restrict__ x, int8_t *__restrict__ y,
                                                      long long planes, int hw)
{
    long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    long long plane = t >> 3;
    int word = (int)(t & 7);
    if (plane >= planes) return;
    const unsigned *src = (const unsigned *)(x + plane * hw * 32) + word;
    int s0 = 0, s1 = 0, s2 = 0, s3 = 0;
    for (int p = 0; p < hw; ++p) {
        unsigned v = __builtin_nontemporal_load(src + p * 8);  // read once
        s0 += (int)(signed char)(v);
        s1 += (int)(signed char)(v >> 8);
        s2 += (int)(signed char)(v >> 16);
        s3 += (int)(signed char)(v >> 24);
    }
    int s[4] = {s0, s1, s2, s3};
    unsigned out = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        int mag = s[e] < 0 ? -s[e] : s[e];
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
    long long threads = planes * 8;
    long long blocks = (threads + 255) / 256;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(avgpool_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, y, planes, hw);
    return hipGetLastError();
}

}  // namespace ifx
