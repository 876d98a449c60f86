// Internal interface between the C ABI (api.cpp) and the gfx950 kernels.
// Everything here is launched on the caller's stream; nothing synchronises.
#pragma once

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

namespace ifx {

// Arguments of one implicit-GEMM convolution launch.
struct ConvArgs {
    const int8_t *x;       // packed input  [n, i1, h, w, 32]
    const int8_t *wt;      // packed weights [o1, kh, kw, i1, o2, 32]
    const int32_t *bias;   // [oc]
    const int32_t *mult;   // [oc]
    const int32_t *shift;  // [oc]
    const int8_t *res;     // packed shortcut [n, oc1, ho, wo, 32] or null
    void *y;               // packed int8 output, or int32 NHWC when out_i32
    int n, h, w, i1;       // input batch, size, channel blocks
    int ho, wo, oc, oc1;   // output size, channels, channel blocks
    int o2;                // output-channel group of the weight layout
    int stride, pad;
    int m;                 // n * ho * wo (GEMM rows)
    int nkb;               // kh * kw * i1 (32-wide reduction blocks)
    int relu, residual, out_i32;
    int out_even;          // store only the even rows and columns of the output (chained conv3)
    // or null: also store the even rows and columns of the output, densely, here
    // ([n, oc1, ceil(ho / 2), ceil(wo / 2), 32]): the input of a following stride-2 projection
    int8_t *y_even;
    // phase-split layout [n][c1][2][2][h/2][w/2][32] (even sizes): plane (y % 2, x % 2) holds the
    // pixels of that row and column parity, so a stride-2 3x3 reads contiguous runs for every tap
    int in_ps, out_ps;
    // split-K (partial launches only): workgroup row blockIdx.y covers 32-channel blocks
    // [blockIdx.y * kb_per, +kb_per) of the reduction and writes its int32 sums, without the
    // bias, to slice blockIdx.y of y ([ksplit][m][oc]); ksplit = 1 is the whole reduction
    int ksplit, kb_per;
    // magic numbers for exact unsigned division of n < 2^31 by ho*wo, wo, o2
    // (q = n when d == 1, else umulhi(n, mul) >> shr); see fastdiv_magic()
    unsigned howo_mul, wo_mul, o2_mul;
    int howo_shr, wo_shr, o2_shr;
};

// Host-side kernel-name query.  While a thread has a query armed, the launchers it reaches
// launch nothing: the first one writes the name of the kernel instance it would launch, as
// profilers print it (e.g. "igemm_kernel<3, 3, 128, 128, 2, false, true, false>"), and returns
// hipSuccess.  The query therefore runs exactly the dispatch code of the launch it describes.
struct KernelQuery {
    char name[160];
    bool answered;
    bool even_copy;  // the answering launcher writes ConvArgs::y_even
};
KernelQuery *&armed_query();  // this thread's armed query, or null

// Called first by every leaf launcher: true when a query took the call (nothing to launch).
// even_copy: the launcher writes ConvArgs::y_even.
inline bool answer_query_e(bool even_copy, const char *fmt, va_list ap)
{
    KernelQuery *q = armed_query();
    if (!q) return false;
    if (!q->answered) {
        vsnprintf(q->name, sizeof(q->name), fmt, ap);
        q->answered = true;
        q->even_copy = even_copy;
    }
    return true;
}
inline bool answer_query_even(bool even_copy, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    const bool r = answer_query_e(even_copy, fmt, ap);
    va_end(ap);
    return r;
}
inline bool answer_query(const char *fmt, ...)
{
    KernelQuery *q = armed_query();
    if (!q) return false;
    if (!q->answered) {
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(q->name, sizeof(q->name), fmt, ap);
        va_end(ap);
        q->answered = true;
        q->even_copy = false;
    }
    return true;
}

inline const char *tf(bool b) { return b ? "true" : "false"; }

// Compute units of the current device: a device property the runtime keeps on the host, so
// reading it launches nothing and is safe while a stream is being captured.  The persistent
// kernels size their grids from it and from their compile-time residency per CU.
inline hipError_t current_cus(int *cus)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess && *cus < 1) *cus = 1;
    return e;
}

// Magic multiplier and shift for q = floor(n / d), 0 <= n < 2^31, d >= 1:
// with p = 31 + ceil(log2 d) and m = ceil(2^p / d), floor(n * m / 2^p) = floor(n / d)
// (the classic round-up method for dividing by an invariant integer; m < 2^32).
inline void fastdiv_magic(unsigned d, unsigned *mul, int *shr)
{
    if (d <= 1) {
        *mul = 0;
        *shr = 0;
        return;
    }
    int l = 0;
    while ((1ull << l) < d) ++l;
    const int p = 31 + l;
    *mul = (unsigned)(((1ull << p) + d - 1) / d);
    *shr = p - 32;
}

// Arguments of the fused stem (7x7/s2/p3 conv + ReLU + 3x3/s2/p1 max-pool).
struct StemArgs {
    const int8_t *x;       // packed input [n, 1, h, w, 32], or compact NHWC [n, h, w, c] when nhwc
    const int8_t *wt;      // stem weights [oc=64, 8, 8, 4]
    const int32_t *bias, *mult, *shift;
    int8_t *y;             // packed pooled output [n, 2, ph, pw, 32]
    int n, h, w, c;        // input (c <= 4)
    int nhwc;              // input layout: 0 packed, 1 compact NHWC
    int ho, wo;            // conv output
    int ph, pw;            // pooled output
    int relu;
};

// Inputs of the BN folding kernel (device pointers; see ifx_fold_bn).
struct FoldArgs {
    int c_out;
    float x_scale, y_scale, eps;
    int w_per_channel;
    const float *w_scale, *conv_bias, *gamma, *beta, *mean, *var;
};

hipError_t launch_conv(const ConvArgs &a, int kh, int kw, hipStream_t s);
// Whether the kernel launch_conv_split picks for `a` honours a.in_ps / a.out_ps (the general
// kernel does; a launch it would split over K is not given a phase-split output).
bool conv_phase_supported(const ConvArgs &a, int kh, int kw);
// Bytes of int32 partial sums launch_conv_split would use for `a` (0: it would not split).  A
// convolution on few output tiles with a long reduction is split over workgroups along K.
size_t splitk_bytes(const ConvArgs &a, int kh, int kw);
// launch_conv, split along K when that pays and `part` (part_bytes of device memory) holds the
// partial sums; a second kernel then sums them and applies the epilogue.  Results are identical.
hipError_t launch_conv_split(const ConvArgs &a, int kh, int kw, int32_t *part, size_t part_bytes, hipStream_t s);
// The 1x1 shortcut conv `a` (RESIDUAL) of a bottleneck fused with its 1x1 projection shortcut
// `pj` (same output pixels and channels, no ReLU): the projection's requantised output is the
// shortcut and never reaches HBM; a.res is not read.
hipError_t launch_conv_proj(const ConvArgs &a, const ConvArgs &pj, hipStream_t s);
// input quantisation (fp32 or uint8 NHWC image -> int8 codes) and logits dequantisation, quant.hip
hipError_t launch_quantize(const void *x, bool u8, int8_t *q, int count, int c, const float *mean, const float *mult,
                           hipStream_t s);
hipError_t launch_dequantize(const int32_t *q, float *y, int count, float scale, hipStream_t s);
hipError_t launch_fold_bn(const FoldArgs &f, int32_t *bias, int32_t *mult, int32_t *shift, int32_t *status,
                          hipStream_t s);
// 1x1 convolutions with at most 128 input channels (conv1x1.hip)
bool conv1x1_small_k_supported(const ConvArgs &a, int kh, int kw);
bool conv1x1_proj_supported(const ConvArgs &a, const ConvArgs &pj);
bool conv1x1_ring_proj_supported(const ConvArgs &a, const ConvArgs &pj);
bool conv1x1_ring_wide_supported(const ConvArgs &a);
hipError_t launch_conv1x1_ring_wide(const ConvArgs &a, hipStream_t s);
hipError_t launch_conv1x1_ring_proj(const ConvArgs &a, const ConvArgs &pj, hipStream_t s);
hipError_t launch_conv1x1_proj(const ConvArgs &a, const ConvArgs &pj, hipStream_t s);
hipError_t launch_conv1x1_small_k(const ConvArgs &a, hipStream_t s);
// conv3 of one bottleneck (a, with its shortcut) chained with conv1 of the next (b): the block
// output a.y is stored and conv1 reads it from LDS (conv1x1.hip)
bool conv1x1_chain_supported(const ConvArgs &a, const ConvArgs &b);
hipError_t launch_conv1x1_chain(const ConvArgs &a, const ConvArgs &b, hipStream_t s);
bool conv1x1_proj_chain_supported(const ConvArgs &a, const ConvArgs &pj, const ConvArgs &b);
hipError_t launch_conv1x1_proj_chain(const ConvArgs &a, const ConvArgs &pj, const ConvArgs &b, hipStream_t s);
hipError_t launch_stem(const StemArgs &a, hipStream_t s);
hipError_t launch_avgpool(const int8_t *x, int8_t *y, int n, int c1, int hw, hipStream_t s);
hipError_t launch_pack_act(const int8_t *x, int8_t *blk, int n, int h, int w, int c, hipStream_t s);
hipError_t launch_unpack_act(const int8_t *blk, int8_t *x, int n, int h, int w, int c, hipStream_t s);
hipError_t launch_pack_weights(const int8_t *w, int8_t *blk, int oc, int kh, int kw, int ic, int o2,
                               hipStream_t s);
hipError_t launch_pack_weights_stem(const int8_t *w, int8_t *blk, int oc, int ic, hipStream_t s);

}  // namespace ifx
