// Float -> fixed-point epilogue parameters of a conv + BN layer (BN folding).
//
// The pages fuse BN into the convolution (DiDi IFX DAWNBench blog, inference
// section: CONV+BN+RELU as one function; Inspur conv-merge article, section
// 3.4: BN applied to the accumulators; the optimisation guide's Conv+BN fusion
// pattern) and quantise with per-layer scales after calibration (DiDi blog,
// quantisation section), but print no formula.  With symmetric int8
// quantisation (real = scale * code, zero point 0), one output channel o:
//   conv real  = s_x * s_w[o] * acc + b_conv[o]
//   BN         = gamma (conv - mean) / sqrt(var + eps) + beta
//   code       = BN / s_y
//              = M[o] * (acc + B[o])
//   M[o] = gamma s_x s_w / (s_y sqrt(var + eps))
//   B[o] = (b_conv - mean) / (s_x s_w) + beta sqrt(var + eps) / (gamma s_x s_w)
// and the library's epilogue takes bias = round_half_away(B) and
// M ~= mult * 2^-(31 + shift) with mult in [2^30, 2^31).
//
// Every value is computed in IEEE double with one rounding per operation in
// the order written above (no fused multiply-add), so the integers that come
// out are reproducible bit for bit.
#include "ifx_internal.h"

namespace ifx {
namespace {

// round half away from zero, exact for every finite double (no x + 0.5 rounding)
__device__ double round_away(double x)
{
    const double a = fabs(x);
    const double r = floor(a);
    const double q = (a - r >= 0.5) ? r + 1.0 : r;
    return x < 0 ? -q : q;
}

__global__ __launch_bounds__(256) void fold_bn_kernel(FoldArgs f, int32_t *bias, int32_t *mult, int32_t *shift,
                                                      int32_t *status)
{
    const int o = blockIdx.x * blockDim.x + threadIdx.x;
    if (o >= f.c_out) return;
    const double sx = f.x_scale, sy = f.y_scale, eps = f.eps;
    const double sw = f.w_scale[f.w_per_channel ? o : 0];
    const double cb = f.conv_bias ? (double)f.conv_bias[o] : 0.0;
    const double g = f.gamma[o], be = f.beta[o], mu = f.mean[o], var = f.var[o];

    const double sd = __dsqrt_rn(__dadd_rn(var, eps));
    const double sxw = __dmul_rn(sx, sw);
    const double M = __ddiv_rn(__dmul_rn(g, sxw), __dmul_rn(sy, sd));
    const double B = __dadd_rn(__ddiv_rn(__dsub_rn(cb, mu), sxw), __ddiv_rn(__dmul_rn(be, sd), __dmul_rn(g, sxw)));

    int st = 0;
    int32_t m = 0, s = 0, b = 0;
    if (!(M > 0.0) || !isfinite(M) || !isfinite(B)) {
        st = 2;  // not representable: non-positive or non-finite scale
    } else {
        int e = 0;
        const double fr = frexp(M, &e);      // M = fr * 2^e, fr in [0.5, 1)
        long long sh = -(long long)e;
        double t = ldexp(fr, 31);            // exact, in [2^30, 2^31)
        if (sh > 31) {                       // tiny scale: shift 31, mult below 2^30
            t = ldexp(fr, 31 - (int)(sh - 31));
            sh = 31;
        }
        double mr = round_away(t);
        if (mr >= 2147483648.0) {            // rounded up to 2^31
            mr = 1073741824.0;
            --sh;
        }
        if (sh < 0) {                        // scale >= 1: not representable
            st = 1;
            m = 2147483647;
            s = 0;
        } else {
            m = (int32_t)mr;
            s = (int32_t)sh;
        }
        const double br = round_away(B);
        if (br > 2147483647.0 || br < -2147483648.0) {
            st = st ? st : 3;                // bias outside int32: clamped
            b = br > 0 ? 2147483647 : (int32_t)-2147483647 - 1;
        } else {
            b = (int32_t)br;
        }
    }
    bias[o] = b;
    mult[o] = m;
    shift[o] = s;
    status[o] = st;
}

}  // namespace

hipError_t launch_fold_bn(const FoldArgs &f, int32_t *bias, int32_t *mult, int32_t *shift, int32_t *status,
                          hipStream_t s)
{
    const int blocks = (f.c_out + 255) / 256;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(fold_bn_kernel, dim3(blocks), dim3(256), 0, s, f, bias, mult, shift, status);
    return hipGetLastError();
}

}  // namespace ifx
