// Layout transforms (Inspur conv-merge article, section 3.1): activations
// NHWC <-> NC/32HW32 and weights OHWI -> [O1, KH, KW, I1, O2, 32] (plus the
// compact 7x7 stem layout [Oc, 8, 8, 4]).  All are HBM-bound copies: each
// thread produces one 16-byte chunk of the destination with a single 16-byte
// store; sources are read with 16-byte loads when the channel count allows
// it, byte loads otherwise.
#include "ifx_internal.h"

namespace ifx {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

// One 16-byte chunk of a packed activation: (pixel, channel block, half).
__global__ __launch_bounds__(256) void pack_act_kernel(const int8_t *__restrict__ x, int8_t *__restrict__ blk,
                                                       long long chunks, int hw, int c, int c1n, int vec)
{
    long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= chunks) return;
    // destination order: [b][c1][pix][half]
    int half = (int)(t & 1);
    long long u = t >> 1;
    long long pix = u % hw;
    long long v = u / hw;
    int c1 = (int)(v % c1n);
    long long b = v / c1n;
    int ch0 = c1 * 32 + half * 16;
    const int8_t *src = x + (b * hw + pix) * c + ch0;
    v4i out;
    if (vec && ch0 + 16 <= c) {
        out = *(const v4i *)src;
    } else {
        union { v4i v; int8_t b[16]; } tmp;
#pragma unroll
        for (int j = 0; j < 16; ++j) tmp.b[j] = (ch0 + j < c) ? src[j] : (int8_t)0;
        out = tmp.v;
    }
    *(v4i *)(blk + t * 16) = out;
}

// One 16-channel chunk of an NHWC pixel from a packed activation.
__global__ __launch_bounds__(256) void unpack_act_kernel(const int8_t *__restrict__ blk, int8_t *__restrict__ x,
                                                         long long items, int hw, int c, int c1n, int cchunks,
                                                         int vec)
{
    long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= items) return;
    int k = (int)(t % cchunks);
    long long u = t / cchunks;  // b * hw + pix
    long long pix = u % hw;
    long long b = u / hw;
    int ch0 = k * 16;
    const int8_t *src = blk + ((b * c1n + (ch0 >> 5)) * hw + pix) * 32 + (ch0 & 31);
    int8_t *dst = x + u * c + ch0;
    if (vec && ch0 + 16 <= c) {
        *(v4i *)dst = *(const v4i *)src;
    } else {
        for (int j = 0; j < 16 && ch0 + j < c; ++j) dst[j] = src[j];
    }
}

// One 16-byte chunk of the blocked weights [o1][ky][kx][i1][o2][half].
__global__ __launch_bounds__(256) void pack_weights_kernel(const int8_t *__restrict__ w, int8_t *__restrict__ blk,
                                                           long long chunks, int oc, int kh, int kw, int ic,
                                                           int o2n, int i1n)
{
    long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= chunks) return;
    int half = (int)(t & 1);
    long long u = t >> 1;
    int o2 = (int)(u % o2n);
    u /= o2n;
    int i1 = (int)(u % i1n);
    u /= i1n;
    int x = (int)(u % kw);
    u /= kw;
    int y = (int)(u % kh);
    int o1 = (int)(u / kh);
    int o = o1 * o2n + o2;
    int i0 = i1 * 32 + half * 16;
    union { v4i v; int8_t b[16]; } tmp;
    const int8_t *src = w + (((long long)o * kh + y) * kw + x) * ic + i0;
#pragma unroll
    for (int j = 0; j < 16; ++j) tmp.b[j] = (o < oc && i0 + j < ic) ? src[j] : (int8_t)0;
    *(v4i *)(blk + t * 16) = tmp.v;
}

// Stem weights [oc][8][8][4]: one thread per byte (16 KB in total).
__global__ __launch_bounds__(256) void pack_weights_stem_kernel(const int8_t *__restrict__ w,
                                                                int8_t *__restrict__ blk, int oc, int ic)
{
    int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= oc * 256) return;
    int ch = t & 3, x = (t >> 2) & 7, y = (t >> 5) & 7, o = t >> 8;
    blk[t] = (y < 7 && x < 7 && ch < ic) ? w[((o * 7 + y) * 7 + x) * ic + ch] : (int8_t)0;
}

inline unsigned grid_for(long long n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t launch_pack_act(const int8_t *x, int8_t *blk, int n, int h, int w, int c, hipStream_t s)
{
    int c1n = (c + 31) / 32;
    long long chunks = (long long)n * c1n * h * w * 2;
    if (chunks == 0) return hipSuccess;
    int vec = (c % 16 == 0) && (((uintptr_t)x & 15) == 0);
    hipLaunchKernelGGL(pack_act_kernel, dim3(grid_for(chunks)), dim3(256), 0, s, x, blk, chunks, h * w, c, c1n,
                       vec);
    return hipGetLastError();
}

hipError_t launch_unpack_act(const int8_t *blk, int8_t *x, int n, int h, int w, int c, hipStream_t s)
{
    int c1n = (c + 31) / 32;
    int cchunks = (c + 15) / 16;
    long long items = (long long)n * h * w * cchunks;
    if (items == 0) return hipSuccess;
    int vec = (c % 16 == 0) && (((uintptr_t)x & 15) == 0);
    hipLaunchKernelGGL(unpack_act_kernel, dim3(grid_for(items)), dim3(256), 0, s, blk, x, items, h * w, c, c1n,
                       cchunks, vec);
    return hipGetLastError();
}

hipError_t launch_pack_weights(const int8_t *w, int8_t *blk, int oc, int kh, int kw, int ic, int o2,
                               hipStream_t s)
{
    int o1n = (oc + o2 - 1) / o2, i1n = (ic + 31) / 32;
    long long chunks = (long long)o1n * kh * kw * i1n * o2 * 2;
    hipLaunchKernelGGL(pack_weights_kernel, dim3(grid_for(chunks)), dim3(256), 0, s, w, blk, chunks, oc, kh, kw,
                       ic, o2, i1n);
    return hipGetLastError();
}

hipError_t launch_pack_weights_stem(const int8_t *w, int8_t *blk, int oc, int ic, hipStream_t s)
{
    hipLaunchKernelGGL(pack_weights_stem_kernel, dim3(grid_for((long long)oc * 256)), dim3(256), 0, s, w, blk,
                       oc, ic);
    return hipGetLastError();
}

}  // namespace ifx
