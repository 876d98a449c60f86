/*
 * oracle.c -- plain CPU definition of the fused int8 ResNet convolution path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle: the slow, obviously
 * correct statement of what the GPU library must compute.  Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or helper with the GPU library, and the
 * library never calls it.
 *
 * Sources (the pages are cited by title and section):
 *  - Inspur, MLPerf v2.0 ResNet50 convolution-merge article ("Inspur
 *    conv-merge article"): section 2.2 gives the res3.x bottleneck
 *    (Conv1+BN+ReLU, Conv2+BN+ReLU, Conv3+BN, Sum with the block input,
 *    ReLU); section 3 the Conv3 shapes; section 3.1 the NC/32HW32 data and
 *    [O1,I1,O2,I2] weight layouts; section 3.3 the GEMM view
 *    data[M,K] . weight[N,K]^T = out[M,N]; section 3.4 the fused
 *    BN+Sum+ReLU epilogue.
 *  - DiDi Cloud IFX DAWNBench blog, section "inference optimisation"
 *    (极致推理优化): CONV+BN+RELU and CONV+BN+RELU+MAXPOOL as single
 *    fused functions.
 *
 * Readings where the pages are silent:
 *  - BN is folded into an int32 bias plus a per-output-channel fixed-point
 *    scale mult * 2^-(31+shift), mult in [0, 2^31), shift in [0, 31].
 *  - One rounding, half away from zero, of (acc + bias) * mult / 2^(31+shift).
 *  - The shortcut is added in the output's quantised domain, before ReLU and
 *    before the single saturation to int8.
 *  - Zero point 0 everywhere; convolution padding contributes 0; max-pool
 *    ignores out-of-range taps.
 *
 * All arithmetic is integer.  Accumulation runs in int64 and any value that
 * leaves the int32 range is reported (ORC_E_OVERFLOW) instead of wrapping.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_E_OVERFLOW 1
#define ORC_E_ARG 2
#define ORC_E_NOMEM 3

#define ORC_RELU 1
#define ORC_RESIDUAL 2
#define ORC_MAXPOOL 4

/* Output size of a convolution or pooling window: floor((in + 2p - k)/s) + 1. */
int orc_out_dim(int in, int k, int s, int p)
{
    int span = in + 2 * p - k;
    if (span < 0 || s <= 0) return 0;
    return span / s + 1;
}

/*
 * Convolution accumulation (Inspur conv-merge article, section 3.3: the
 * convolution as data[M,K] . weight[N,K]^T, here written out directly over
 * the kernel window).
 *   acc[b,oy,ox,o] = sum_{ky,kx,i} x[b, oy*s-p+ky, ox*s-p+kx, i] * w[o,ky,kx,i]
 * x is NHWC int8, w is OHWI int8, acc is NHWC int32.  Taps outside the
 * image contribute 0.  Returns ORC_E_OVERFLOW if any sum leaves int32.
 */
int orc_conv_acc(const int8_t *x, int n, int h, int w, int c,
                 const int8_t *wt, int oc, int kh, int kw, int stride, int pad,
                 int32_t *acc)
{
    int ho = orc_out_dim(h, kh, stride, pad);
    int wo = orc_out_dim(w, kw, stride, pad);
    if (n < 0 || h <= 0 || w <= 0 || c <= 0 || oc <= 0 || kh <= 0 || kw <= 0 ||
        stride <= 0 || pad < 0 || ho <= 0 || wo <= 0)
        return ORC_E_ARG;
    int overflow = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(| : overflow)
    for (int b = 0; b < n; b++) {
        for (int oy = 0; oy < ho; oy++) {
            for (int ox = 0; ox < wo; ox++) {
                for (int o = 0; o < oc; o++) {
                    int64_t sum = 0;
                    for (int ky = 0; ky < kh; ky++) {
                        int iy = oy * stride - pad + ky;
                        if (iy < 0 || iy >= h) continue;
                        for (int kx = 0; kx < kw; kx++) {
                            int ix = ox * stride - pad + kx;
                            if (ix < 0 || ix >= w) continue;
                            const int8_t *xp = x + (((int64_t)b * h + iy) * w + ix) * c;
                            const int8_t *wp = wt + (((int64_t)o * kh + ky) * kw + kx) * c;
                            for (int i = 0; i < c; i++)
                                sum += (int64_t)xp[i] * (int64_t)wp[i];
                        }
                    }
                    if (sum < INT32_MIN || sum > INT32_MAX) overflow = 1;
                    acc[(((int64_t)b * ho + oy) * wo + ox) * oc + o] = (int32_t)sum;
                }
            }
        }
    }
    return overflow ? ORC_E_OVERFLOW : ORC_OK;
}

/*
 * Round-half-away-from-zero division by a power of two:
 *   sign(p) * floor((|p| + 2^(s-1)) / 2^s),  1 <= s <= 62.
 */
int64_t orc_round_shift(int64_t p, int s)
{
    uint64_t mag = p < 0 ? (uint64_t)0 - (uint64_t)p : (uint64_t)p;
    uint64_t half = (uint64_t)1 << (s - 1);
    uint64_t q = (mag + half) >> s;
    return p < 0 ? -(int64_t)q : (int64_t)q;
}

/*
 * Folded BN plus requantisation of one accumulator (the "BN" of the Inspur
 * conv-merge article, sections 2.2 and 3.4, with the fixed-point reading):
 *   y = acc + bias                  (must stay in int32)
 *   q = round_half_away(y * mult / 2^(31 + shift))
 * The product is exact in int64 because |y| <= 2^31 and mult < 2^31.
 */
int orc_requant(int32_t acc, int32_t bias, int32_t mult, int32_t shift, int64_t *q)
{
    if (mult < 0 || shift < 0 || shift > 31) return ORC_E_ARG;
    int64_t y = (int64_t)acc + (int64_t)bias;
    if (y < INT32_MIN || y > INT32_MAX) return ORC_E_OVERFLOW;
    int64_t p = y * (int64_t)mult;
    *q = orc_round_shift(p, 31 + shift);
    return ORC_OK;
}

/*
 * Fused epilogue on accumulators (Inspur conv-merge article, section 3.4:
 * BN, then Sum with the shortcut, then ReLU; DiDi IFX blog: CONV+BN+RELU):
 *   q = requant(acc + bias); if RESIDUAL q += r; if RELU q = max(q, 0);
 *   out = saturate_int8(q)
 * acc, residual and out are NHWC with `oc` channels and `npix` pixels.
 */
int orc_epilogue(const int32_t *acc, int64_t npix, int oc,
                 const int32_t *bias, const int32_t *mult, const int32_t *shift,
                 const int8_t *residual, int flags, int8_t *out)
{
    for (int o = 0; o < oc; o++)
        if (mult[o] < 0 || shift[o] < 0 || shift[o] > 31) return ORC_E_ARG;
    if ((flags & ORC_RESIDUAL) && !residual) return ORC_E_ARG;
    int err = 0;
#pragma omp parallel for schedule(static) reduction(| : err)
    for (int64_t p = 0; p < npix; p++) {
        for (int o = 0; o < oc; o++) {
            int64_t idx = p * oc + o;
            int64_t q;
            if (orc_requant(acc[idx], bias[o], mult[o], shift[o], &q) != ORC_OK) {
                err = 1;
                continue;
            }
            if (flags & ORC_RESIDUAL) q += residual[idx];
            if ((flags & ORC_RELU) && q < 0) q = 0;
            if (q > 127) q = 127;
            if (q < -128) q = -128;
            out[idx] = (int8_t)q;
        }
    }
    return err ? ORC_E_OVERFLOW : ORC_OK;
}

/*
 * 3x3 stride-2 pad-1 max-pool (the MAXPOOL of the DiDi IFX blog's fused
 * CONV+BN+RELU+MAXPOOL).  Out-of-range taps are ignored.
 */
int orc_maxpool3s2p1(const int8_t *in, int n, int h, int w, int c, int8_t *out)
{
    int ph = orc_out_dim(h, 3, 2, 1), pw = orc_out_dim(w, 3, 2, 1);
    if (ph <= 0 || pw <= 0) return ORC_E_ARG;
    for (int b = 0; b < n; b++)
        for (int py = 0; py < ph; py++)
            for (int px = 0; px < pw; px++)
                for (int ch = 0; ch < c; ch++) {
                    int best = -129;
                    for (int dy = 0; dy < 3; dy++) {
                        int y = 2 * py - 1 + dy;
                        if (y < 0 || y >= h) continue;
                        for (int dx = 0; dx < 3; dx++) {
                            int xx = 2 * px - 1 + dx;
                            if (xx < 0 || xx >= w) continue;
                            int v = in[(((int64_t)b * h + y) * w + xx) * c + ch];
                            if (v > best) best = v;
                        }
                    }
                    out[(((int64_t)b * ph + py) * pw + px) * c + ch] = (int8_t)best;
                }
    return ORC_OK;
}

/*
 * One fused convolution: conv -> folded BN + requant -> [shortcut sum] ->
 * [ReLU] -> saturate -> [3x3/s2 max-pool].  out has the pooled shape when
 * MAXPOOL is set.
 */
int orc_conv_fused(const int8_t *x, int n, int h, int w, int c,
                   const int8_t *wt, int oc, int kh, int kw, int stride, int pad,
                   const int32_t *bias, const int32_t *mult, const int32_t *shift,
                   const int8_t *residual, int flags, int8_t *out)
{
    int ho = orc_out_dim(h, kh, stride, pad);
    int wo = orc_out_dim(w, kw, stride, pad);
    if (ho <= 0 || wo <= 0) return ORC_E_ARG;
    if ((flags & ORC_MAXPOOL) && (flags & ORC_RESIDUAL)) return ORC_E_ARG;
    int64_t npix = (int64_t)n * ho * wo;
    int32_t *acc = (int32_t *)malloc((size_t)(npix * oc) * sizeof(int32_t));
    if (!acc) return ORC_E_NOMEM;
    int rc = orc_conv_acc(x, n, h, w, c, wt, oc, kh, kw, stride, pad, acc);
    if (rc == ORC_OK) {
        if (flags & ORC_MAXPOOL) {
            int8_t *pre = (int8_t *)malloc((size_t)(npix * oc));
            if (!pre) {
                free(acc);
                return ORC_E_NOMEM;
            }
            rc = orc_epilogue(acc, npix, oc, bias, mult, shift, NULL, flags & ORC_RELU, pre);
            if (rc == ORC_OK) rc = orc_maxpool3s2p1(pre, n, ho, wo, oc, out);
            free(pre);
        } else {
            rc = orc_epilogue(acc, npix, oc, bias, mult, shift, residual, flags, out);
        }
    }
    free(acc);
    return rc;
}

/*
 * Global average pool to int8: a[b,c] = round_half_away(sum_{y,x} t[b,y,x,c] / (h*w)).
 * Not on the pages (their float example ends in an average pool and a
 * linear layer); this integer form is the reading used for the head.
 */
int orc_avgpool(const int8_t *in, int n, int h, int w, int c, int8_t *out)
{
    int64_t cnt = (int64_t)h * w;
    if (cnt <= 0) return ORC_E_ARG;
    for (int b = 0; b < n; b++)
        for (int ch = 0; ch < c; ch++) {
            int64_t s = 0;
            for (int64_t p = 0; p < cnt; p++) s += in[((int64_t)b * cnt + p) * c + ch];
            int64_t mag = s < 0 ? -s : s;
            int64_t q = (2 * mag + cnt) / (2 * cnt); /* floor(|s|/cnt + 1/2) */
            q = s < 0 ? -q : q;
            if (q > 127) q = 127;
            if (q < -128) q = -128;
            out[(int64_t)b * c + ch] = (int8_t)q;
        }
    return ORC_OK;
}

/*
 * Fully connected layer with int32 logits: logits[b,o] = sum_c a[b,c]*w[o,c] + bias[o].
 */
int orc_fc(const int8_t *a, int n, int k, const int8_t *wt, int o_n,
           const int32_t *bias, int32_t *logits)
{
    int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
    for (int b = 0; b < n; b++)
        for (int o = 0; o < o_n; o++) {
            int64_t s = bias[o];
            for (int i = 0; i < k; i++) s += (int64_t)a[(int64_t)b * k + i] * wt[(int64_t)o * k + i];
            if (s < INT32_MIN || s > INT32_MAX) overflow = 1;
            logits[(int64_t)b * o_n + o] = (int32_t)s;
        }
    return overflow ? ORC_E_OVERFLOW : ORC_OK;
}

/* ------------------------------------------------------------------------
 * Layout maps (Inspur conv-merge article, section 3.1).  These define the
 * packed byte layouts the GPU packers must produce; tests compare the GPU
 * packers with these byte for byte.
 * ------------------------------------------------------------------------ */

/* Activations: NHWC -> [N, ceil(C/32), H, W, 32], channels >= C zero-filled. */
int orc_pack_act(const int8_t *x, int n, int h, int w, int c, int8_t *blk)
{
    int c1n = (c + 31) / 32;
    for (int b = 0; b < n; b++)
        for (int c1 = 0; c1 < c1n; c1++)
            for (int y = 0; y < h; y++)
                for (int xx = 0; xx < w; xx++)
                    for (int c2 = 0; c2 < 32; c2++) {
                        int ch = c1 * 32 + c2;
                        int64_t dst = ((((int64_t)b * c1n + c1) * h + y) * w + xx) * 32 + c2;
                        blk[dst] = ch < c ? x[(((int64_t)b * h + y) * w + xx) * c + ch] : 0;
                    }
    return ORC_OK;
}

/* Inverse of orc_pack_act (padding channels are dropped). */
int orc_unpack_act(const int8_t *blk, int n, int h, int w, int c, int8_t *x)
{
    int c1n = (c + 31) / 32;
    for (int b = 0; b < n; b++)
        for (int y = 0; y < h; y++)
            for (int xx = 0; xx < w; xx++)
                for (int ch = 0; ch < c; ch++)
                    x[(((int64_t)b * h + y) * w + xx) * c + ch] =
                        blk[((((int64_t)b * c1n + ch / 32) * h + y) * w + xx) * 32 + ch % 32];
    return ORC_OK;
}

/* Output-channel group width of the blocked weight layout: min(128, Oc rounded up to 32). */
int orc_wgroup(int oc)
{
    int r = (oc + 31) / 32 * 32;
    return r < 128 ? r : 128;
}

/*
 * Weights: OHWI [Oc,KH,KW,Ic] -> [O1, KH, KW, I1, O2, I2=32] with
 * O2 = orc_wgroup(Oc), O1 = ceil(Oc/O2), I1 = ceil(Ic/32); out-of-range
 * positions are zero.  For KH = KW = 1 this is the article's [O1,I1,O2,I2].
 */
int orc_pack_weights(const int8_t *wt, int oc, int kh, int kw, int ic, int8_t *blk)
{
    int o2n = orc_wgroup(oc), o1n = (oc + o2n - 1) / o2n, i1n = (ic + 31) / 32;
    for (int o1 = 0; o1 < o1n; o1++)
        for (int y = 0; y < kh; y++)
            for (int xx = 0; xx < kw; xx++)
                for (int i1 = 0; i1 < i1n; i1++)
                    for (int o2 = 0; o2 < o2n; o2++)
                        for (int i2 = 0; i2 < 32; i2++) {
                            int o = o1 * o2n + o2, i = i1 * 32 + i2;
                            int64_t dst =
                                (((((int64_t)o1 * kh + y) * kw + xx) * i1n + i1) * o2n + o2) * 32 + i2;
                            blk[dst] = (o < oc && i < ic)
                                           ? wt[(((int64_t)o * kh + y) * kw + xx) * ic + i]
                                           : 0;
                        }
    return ORC_OK;
}

/*
 * Stem weights (7x7 kernel over at most 4 input channels): OHWI ->
 * [Oc, 8, 8, 4]; row 7, column 7 and channels >= Ic are zero.  The reduction
 * index of one output channel is (ky, kx, c) with 32 bytes per kernel row.
 */
int orc_pack_weights_stem(const int8_t *wt, int oc, int ic, int8_t *blk)
{
    if (ic > 4) return ORC_E_ARG;
    for (int o = 0; o < oc; o++)
        for (int y = 0; y < 8; y++)
            for (int xx = 0; xx < 8; xx++)
                for (int ch = 0; ch < 4; ch++) {
                    int64_t dst = (((int64_t)o * 8 + y) * 8 + xx) * 4 + ch;
                    blk[dst] = (y < 7 && xx < 7 && ch < ic)
                                   ? wt[(((int64_t)o * 7 + y) * 7 + xx) * ic + ch]
                                   : 0;
                }
    return ORC_OK;
}

/*
 * BN folding into the integer epilogue (DiDi IFX DAWNBench blog: CONV+BN+RELU
 * as one function after post-training quantisation; Inspur conv-merge
 * article section 3.4: BN applied to the accumulators).  The pages print no
 * formula; the reading: symmetric int8 quantisation (real = scale * code), so
 * for output channel o the output code is M * (acc + B) with
 *   M = gamma * s_x * s_w / (s_y * sqrt(var + eps))
 *   B = (b_conv - mean) / (s_x * s_w) + beta * sqrt(var + eps) / (gamma * s_x * s_w)
 * Each value is one IEEE double operation after another, in this order, so a
 * decision taken on them (a rounding to an integer) is reproducible:
 *   sd = sqrt(var + eps); sxw = s_x * s_w; M = (gamma * sxw) / (s_y * sd);
 *   B = (b_conv - mean) / sxw + (beta * sd) / (gamma * sxw).
 * Then bias = round_half_away(B) and M = f * 2^e (f in [0.5, 1)) gives
 * shift = -e and mult = round_half_away(f * 2^31), renormalised when that
 * reaches 2^31; a shift beyond 31 keeps 31 with mult = round(f * 2^(62 + e)).
 * status: 0 ok; 1 M >= 1 (mult = 2^31 - 1, shift 0); 2 M <= 0 or not finite
 * (all zero); 3 bias outside int32 (clamped).
 */
static double orc_round_half_away(double x)
{
    double a = fabs(x);
    double r = floor(a);
    double q = (a - r >= 0.5) ? r + 1.0 : r;
    return x < 0 ? -q : q;
}

int orc_fold_bn(int c_out, double x_scale, double y_scale, double eps, int w_per_channel, const float *w_scale,
                const float *conv_bias, const float *gamma, const float *beta, const float *mean, const float *var,
                int32_t *bias, int32_t *mult, int32_t *shift, int32_t *status)
{
    for (int o = 0; o < c_out; o++) {
        double sw = w_scale[w_per_channel ? o : 0];
        double cb = conv_bias ? conv_bias[o] : 0.0;
        double g = gamma[o];
        double sd = sqrt((double)var[o] + eps);
        double sxw = x_scale * sw;
        double num = g * sxw;
        double den = y_scale * sd;
        double M = num / den;
        double t1 = (cb - (double)mean[o]) / sxw;
        double t2 = ((double)beta[o] * sd) / (g * sxw);
        double B = t1 + t2;
        int st = 0;
        int32_t m = 0, s = 0, b = 0;
        if (!(M > 0.0) || !isfinite(M) || !isfinite(B)) {
            st = 2;
        } else {
            int e = 0;
            double f = frexp(M, &e);
            long sh = -(long)e;
            double tm;
            if (sh > 31) {
                tm = ldexp(f, 62 + e);
                sh = 31;
            } else {
                tm = ldexp(f, 31);
            }
            double mr = orc_round_half_away(tm);
            if (mr >= 2147483648.0) {
                mr = 1073741824.0;
                sh -= 1;
            }
            if (sh < 0) {
                st = 1;
                m = 2147483647;
                s = 0;
            } else {
                m = (int32_t)mr;
                s = (int32_t)sh;
            }
            double br = orc_round_half_away(B);
            if (br > 2147483647.0 || br < -2147483648.0) {
                if (!st) st = 3;
                b = br > 0 ? 2147483647 : INT32_MIN;
            } else {
                b = (int32_t)br;
            }
        }
        bias[o] = b;
        mult[o] = m;
        shift[o] = s;
        status[o] = st;
    }
    return ORC_OK;
}

/*
 * Quantisation of the input image and dequantisation of the logits (Alibaba
 * inference article, Hanguang 800 section: the accelerator takes integer
 * data, and the quantisation before the engine and the dequantisation after
 * it, which had run on the host and taken most of the latency, belong with
 * the accelerated pre- and post-processing).  The page prints no formula.
 * The reading, with the path's symmetric int8 codes (real = s_x * code, zero
 * point 0), one IEEE single-precision operation at a time (round to nearest
 * even, no fused multiply-add):
 *   fp32 image:  t = x * mult[ch]
 *   uint8 image: t = ((float)u - mean[ch]) * mult[ch]
 *                (the per-channel mean subtraction and 1 / (std * s_x)
 *                scaling of an ImageNet-style pre-processing, fused into the
 *                quantisation)
 *   code = saturate_int8(round_half_away(t)); a NaN t gives code 0
 * where ch = element index mod c (NHWC: channels innermost), and
 *   logits:      y = (float)q * scale.
 */
static int8_t orc_code_of(float t)
{
    if (t != t) return 0;
    double r = orc_round_half_away((double)t);
    if (r > 127.0) r = 127.0;
    if (r < -128.0) r = -128.0;
    return (int8_t)r;
}

int orc_quantize_f32(const float *x, int64_t count, int c, const float *mult, int8_t *q)
{
    if (c <= 0 || count < 0 || count % c) return ORC_E_ARG;
    for (int64_t i = 0; i < count; i++) {
        float t = x[i] * mult[i % c];
        q[i] = orc_code_of(t);
    }
    return ORC_OK;
}

int orc_quantize_u8(const uint8_t *x, int64_t count, int c, const float *mean, const float *mult, int8_t *q)
{
    if (c <= 0 || count < 0 || count % c) return ORC_E_ARG;
    for (int64_t i = 0; i < count; i++) {
        int ch = (int)(i % c);
        float d = (float)x[i] - mean[ch];
        float t = d * mult[ch];
        q[i] = orc_code_of(t);
    }
    return ORC_OK;
}

int orc_dequantize_i32(const int32_t *q, int64_t count, float scale, float *y)
{
    if (count < 0) return ORC_E_ARG;
    for (int64_t i = 0; i < count; i++) {
        float v = (float)q[i];
        y[i] = v * scale;
    }
    return ORC_OK;
}
