// Fused stem: 7x7 stride-2 pad-3 convolution over <= 4 input channels, folded
// BN, ReLU and a 3x3 stride-2 pad-1 max-pool, in one kernel (the
// CONV+BN+RELU+MAXPOOL single function of the DiDi IFX DAWNBench blog,
// inference-optimisation section).  The pre-pool tensor is never written.
//
// gfx950 design:
//   * one 256-thread workgroup produces an 8x8 tile of pooled pixels x 64
//     channels; it needs the 17x17 convolution pixels under those windows
//     (the one-row/column halo shared with neighbouring tiles is recomputed);
//   * the input window (40x40 pixels) is staged in LDS with only the four
//     channel bytes the stem uses, so one 16-byte MFMA operand is four
//     consecutive kernel columns x four channels;
//   * reduction order per output channel: (ky, kx, c) with 32 bytes per
//     kernel row (column 7 and channel 3 are zero weights) and the 8th row a
//     zero row: K = 256 = four v_mfma_i32_16x16x64_i8 steps instead of the
//     49 x 32 = 1568 of the channel-padded layout;
//   * int32 accumulators go to LDS and the max-pool runs on them: with
//     mult >= 0 the epilogue (bias, requant, ReLU, saturate) is monotone
//     non-decreasing per channel, so pooling before the epilogue gives the
//     same bytes as pooling after it, with a quarter of the requant work.
#include "ifx_internal.h"

namespace ifx {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kPT = 8;               // pooled tile edge
constexpr int kCT = 2 * kPT + 1;     // convolution tile edge (17)
constexpr int kCPix = kCT * kCT;     // 289 convolution pixels
constexpr int kMT = (kCPix + 15) / 16;  // 19 MFMA row tiles
constexpr int kIT = 2 * kCT + 6;     // 40 input rows/cols staged
constexpr int kOC = 64;

__device__ __forceinline__ int requant_any(int y, int m, int sh)
{
    long long p = (long long)y * (long long)m + (1ll << (30 + sh)) - (y < 0 ? 1 : 0);
    return (int)(p >> (31 + sh));
}

__global__ __launch_bounds__(kThreads) void stem_kernel(StemArgs a)
{
    __shared__ __attribute__((aligned(16))) int32_t sIn[kIT * kIT];      // 4 channel bytes per pixel
    __shared__ __attribute__((aligned(16))) int32_t sAcc[kCPix * kOC];  // conv accumulators

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    const int tiles_x = (a.pw + kPT - 1) / kPT;
    const int tiles_y = (a.ph + kPT - 1) / kPT;
    int t = blockIdx.x;
    const int tx = t % tiles_x;
    t /= tiles_x;
    const int ty = t % tiles_y;
    const int b = t / tiles_y;
    const int py0 = ty * kPT, px0 = tx * kPT;
    const int cy0 = 2 * py0 - 1, cx0 = 2 * px0 - 1;  // first conv pixel of the tile
    const int iy0 = 2 * cy0 - 3, ix0 = 2 * cx0 - 3;  // first input pixel staged

    // ---- stage the input window: 4 channel bytes of each pixel ----
    const int8_t *img = a.x + (long long)b * a.h * a.w * 32;
    for (int i = tid; i < kIT * kIT; i += kThreads) {
        int ry = i / kIT, rx = i - ry * kIT;
        int iy = iy0 + ry, ix = ix0 + rx;
        int v = 0;
        if ((unsigned)iy < (unsigned)a.h && (unsigned)ix < (unsigned)a.w)
            v = *(const int32_t *)(img + ((long long)iy * a.w + ix) * 32);
        sIn[i] = v;
    }

    // ---- weights for this lane: 4 column tiles x 4 K steps of 16 bytes ----
    const int c = lane & 15, g = lane >> 4;
    v4i wf[4][4];
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
        const int8_t *wp = a.wt + (4 * c + tn) * 256 + g * 16;  // MFMA column c of tile tn = channel 4c+tn
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) wf[tn][ks] = *(const v4i *)(wp + ks * 64);
    }
    __syncthreads();

    // ---- convolution: MFMA rows = conv pixels, columns = channels ----
    const int kh_off = g >> 1;       // kernel row within a K step (two rows per step)
    const int kw0 = 4 * (g & 1);     // first kernel column of this lane's chunk
    for (int tm = wave; tm < kMT; tm += 4) {
        int q = 16 * tm + (lane & 15);
        if (q >= kCPix) q = kCPix - 1;  // padding rows: any valid address, results dropped
        const int ly = q / kCT, lx = q - (q / kCT) * kCT;
        v4i acc[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int ry = 2 * ly + 2 * ks + kh_off;
            const int rx = 2 * lx + kw0;
            const v2i *src = (const v2i *)&sIn[ry * kIT + rx];
            v2i lo = src[0], hi = src[1];
            v4i af = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
            for (int tn = 0; tn < 4; ++tn)
                acc[tn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, wf[tn][ks], acc[tn], 0, 0, 0);
        }
        // lane (g, c) holds conv pixels 16tm + 4g + i, channels 4c + tn
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int qq = 16 * tm + 4 * g + i;
            if (qq >= kCPix) continue;
            const int qy = qq / kCT, qx = qq - (qq / kCT) * kCT;
            const bool inside = (unsigned)(cy0 + qy) < (unsigned)a.ho && (unsigned)(cx0 + qx) < (unsigned)a.wo;
            v4i v = inside ? (v4i){acc[0][i], acc[1][i], acc[2][i], acc[3][i]}
                           : (v4i){INT32_MIN, INT32_MIN, INT32_MIN, INT32_MIN};
            *(v4i *)&sAcc[qq * kOC + 4 * c] = v;
        }
    }
    __syncthreads();

    // ---- max-pool on accumulators, then the epilogue on 16 channels ----
    const int pp = tid >> 2;            // pooled pixel of the 8x8 tile
    const int cg = (tid & 3) * 16;      // 16-channel group
    const int ply = pp / kPT, plx = pp - (pp / kPT) * kPT;
    const int py = py0 + ply, px = px0 + plx;
    if (py >= a.ph || px >= a.pw) return;
    v4i mx[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) mx[k] = (v4i){INT32_MIN, INT32_MIN, INT32_MIN, INT32_MIN};
#pragma unroll
    for (int dy = 0; dy < 3; ++dy)
#pragma unroll
        for (int dx = 0; dx < 3; ++dx) {
            const int qq = (2 * ply + dy) * kCT + 2 * plx + dx;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v4i v = *(const v4i *)&sAcc[qq * kOC + cg + 4 * k];
                mx[k].x = max(mx[k].x, v.x);
                mx[k].y = max(mx[k].y, v.y);
                mx[k].z = max(mx[k].z, v.z);
                mx[k].w = max(mx[k].w, v.w);
            }
        }
    unsigned words[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        unsigned wv = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int o = cg + 4 * k + e;
            int yv = mx[k][e] + a.bias[o];
            int q = requant_any(yv, a.mult[o], a.shift[o]);
            if (a.relu) q = max(q, 0);
            q = min(max(q, -128), 127);
            wv |= (unsigned)(q & 0xff) << (8 * e);
        }
        words[k] = wv;
    }
    int8_t *dst = a.y + ((((long long)b * 2 + (cg >> 5)) * a.ph + py) * a.pw + px) * 32 + (cg & 31);
    *(v4i *)dst = (v4i){(int)words[0], (int)words[1], (int)words[2], (int)words[3]};
}

}  // namespace

hipError_t launch_stem(const StemArgs &a, hipStream_t s)
{
    long long tiles = (long long)a.n * ((a.ph + kPT - 1) / kPT) * ((a.pw + kPT - 1) / kPT);
    if (tiles <= 0) return hipSuccess;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(stem_kernel, dim3((unsigned)tiles), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace ifx
