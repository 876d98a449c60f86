// Implicit-GEMM int8 convolution with the fused requant / shortcut / ReLU
// epilogue, for gfx950 (CDNA4) int8 MFMA.
//
// What is computed (Inspur conv-merge article, section 3.3): the convolution
// is the matrix product data[M,K] . weight[N,K]^T with M = batch*Ho*Wo output
// pixels, N = output channels and K = KH*KW*Ic, both operands K-contiguous
// thanks to the NC/32HW32 activation and [O1,KH,KW,I1,O2,32] weight layouts
// (section 3.1).  The epilogue (section 3.4: BN, Sum with the shortcut, ReLU)
// runs on the int32 accumulators before anything is written.
//
// How (the gfx950 design, not the article's A100 tiling):
//   * one 256-thread workgroup (4 wave64s) owns a BM x BN output tile; each
//     wave owns a 64x64 sub-tile = 4x4 tiles of v_mfma_i32_16x16x64_i8;
//   * the K loop steps 64 bytes (two 32-channel blocks of one or two kernel
//     taps) at a time through a double-buffered LDS stage: 16-byte global
//     loads for step k+1 are in flight while the MFMAs consume step k;
//   * implicit GEMM: row m of the activation operand at tap (ky,kx) is the
//     32-byte channel vector of input pixel (oy*s-p+ky, ox*s-p+kx), or zero
//     outside the image; nothing is materialised (no im2col);
//   * MFMA rows/columns are permuted so that each lane ends up holding four
//     consecutive output channels of one pixel: the epilogue reads the
//     shortcut and writes the output as whole 32-bit words that a wave
//     assembles into 128-byte runs of the NC/32HW32 output;
//   * the bias is folded into the accumulator initial value;
//   * workgroups are renumbered so that the tiles sharing an activation tile
//     run on the same XCD (own L2) back to back.
#include "ifx_internal.h"

namespace ifx {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaveM = 64;
constexpr int kWaveN = 64;

// 16-byte-chunk XOR swizzle of a 64-byte LDS row: keeps the ds_write_b128 of
// the loaders and the ds_read_b128 of the MFMA operand fetch conflict-free.
__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

// Requantisation, exact for every |y| < 2^31, 0 <= m < 2^31, 0 <= sh <= 31:
//   q = sign(y) * floor((|y|*m + 2^(30+sh)) / 2^(31+sh))
// which is round-half-away-from-zero of y*m/2^(31+sh).  Using arithmetic
// shifts (floor): q = floor((y*m + 2^(30+sh) - [y<0]) / 2^(31+sh)).
// General form: one 64-bit product and one 64-bit shift.
__device__ __forceinline__ int requant_any(int y, int m, int sh)
{
    long long p = (long long)y * (long long)m + (1ll << (30 + sh)) - (y < 0 ? 1 : 0);
    return (int)(p >> (31 + sh));
}

// Fast form for sh >= 2: the rounding term 2^(30+sh) - [y<0] has high word
// 2^(sh-2) + sgn and low word sgn (sgn = y >> 31), so the whole sum is one
// v_mad_i64_i32, and floor(p / 2^(31+sh)) = (high word of p) >> (sh - 1).
__device__ __forceinline__ int requant_fast(int y, int m, int rnd_hi, int sh_m1)
{
    int sgn = y >> 31;
    long long add = (long long)(((unsigned long long)(unsigned)(rnd_hi + sgn) << 32) | (unsigned)sgn);
    long long p = (long long)y * (long long)m + add;
    return ((int)(p >> 32)) >> sh_m1;
}

template <int KH, int KW, int BM, int BN>
__global__ __launch_bounds__(kThreads) void conv_kernel(ConvArgs a)
{
    constexpr int WAVES_M = BM / kWaveM;
    constexpr int WAVES_N = BN / kWaveN;
    static_assert(WAVES_M * WAVES_N == kThreads / 64, "4 waves per workgroup");
    constexpr int MT = kWaveM / 16;  // MFMA tiles along M per wave
    constexpr int NT = kWaveN / 16;  // MFMA tiles along N per wave
    constexpr int AR = BM / 64;      // activation rows loaded per thread per step
    constexpr int BR = BN / 64;      // weight rows loaded per thread per step

    __shared__ __attribute__((aligned(16))) int8_t smem[2 * (BM + BN) * 64];
    int8_t *sA = smem;               // [2][BM][64]
    int8_t *sB = smem + 2 * BM * 64; // [2][BN][64]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm0 = (wave % WAVES_M) * kWaveM;
    const int wn0 = (wave / WAVES_M) * kWaveN;

    // ---- tile of this workgroup (XCD-aware renumbering) ----
    const int tiles_n = (a.oc1 * 32 + BN - 1) / BN;
    const int G = gridDim.x;
    const int bid = blockIdx.x;
    const int per_xcd = G >> 3;
    const int lin = bid < (per_xcd << 3) ? (bid & 7) * per_xcd + (bid >> 3) : bid;
    const int tile_n = lin % tiles_n;
    const int tile_m = lin / tiles_n;
    const int m0 = tile_m * BM;
    const int n0 = tile_n * BN;

    const int HoWo = a.ho * a.wo;
    const int HW = a.h * a.w;

    // ---- per-thread load assignment: row r0 + 64j, 16-byte chunk cq ----
    const int cq = tid & 3;
    const int r0 = tid >> 2;
    const int half = cq & 1;
    const int bpar = cq >> 1;  // which of the two 32-channel blocks of a step

    const int8_t *img[AR];
    int iy0[AR], ix0[AR];
    bool mval[AR];
#pragma unroll
    for (int j = 0; j < AR; ++j) {
        int p = m0 + r0 + 64 * j;
        mval[j] = p < a.m;
        int pp = mval[j] ? p : 0;
        int b = pp / HoWo;
        int rem = pp - b * HoWo;
        int oy = rem / a.wo;
        int ox = rem - oy * a.wo;
        iy0[j] = oy * a.stride - a.pad;
        ix0[j] = ox * a.stride - a.pad;
        img[j] = a.x + (long long)b * a.i1 * HW * 32 + half * 16;
    }
    const int wrows = ((a.oc + a.o2 - 1) / a.o2) * a.o2;
    const int8_t *wrow[BR];
    bool nval[BR];
#pragma unroll
    for (int j = 0; j < BR; ++j) {
        int R = n0 + r0 + 64 * j;
        nval[j] = R < wrows;
        int RR = nval[j] ? R : 0;
        int o1 = RR / a.o2;
        int o2i = RR - o1 * a.o2;
        wrow[j] = a.wt + ((long long)o1 * KH * KW * a.i1 * a.o2 + o2i) * 32 + half * 16;
    }

    // reduction-block counters for block kb = 2*step + bpar: (ky, kx, c1)
    int kb = bpar;
    int c1 = kb % a.i1;
    int tap = kb / a.i1;
    int kx = tap % KW;
    int ky = tap / KW;

    const int nsteps = (a.nkb + 1) >> 1;
    const long long wstride_c1 = (long long)a.o2 * 32;

    v4i pa[AR], pb[BR];
    auto load_step = [&]() {
        const bool kval = kb < a.nkb;
#pragma unroll
        for (int j = 0; j < AR; ++j) {
            v4i v = {0, 0, 0, 0};
            int iy = iy0[j] + ky;
            int ix = ix0[j] + kx;
            bool ok = kval && mval[j];
            if (KH > 1) ok = ok && (unsigned)iy < (unsigned)a.h;
            if (KW > 1) ok = ok && (unsigned)ix < (unsigned)a.w;
            if (ok) v = *(const v4i *)(img[j] + ((long long)c1 * HW + (long long)iy * a.w + ix) * 32);
            pa[j] = v;
        }
#pragma unroll
        for (int j = 0; j < BR; ++j) {
            v4i v = {0, 0, 0, 0};
            if (kval && nval[j])
                v = *(const v4i *)(wrow[j] + ((long long)(ky * KW + kx) * a.i1 + c1) * wstride_c1);
            pb[j] = v;
        }
        // advance two reduction blocks
        kb += 2;
        c1 += 2;
        while (c1 >= a.i1) {
            c1 -= a.i1;
            if (++kx == KW) {
                kx = 0;
                ++ky;
            }
        }
    };
    auto store_step = [&](int buf) {
#pragma unroll
        for (int j = 0; j < AR; ++j) {
            int row = r0 + 64 * j;
            *(v4i *)(sA + (buf * BM + row) * 64 + ((cq ^ swz(row)) << 4)) = pa[j];
        }
#pragma unroll
        for (int j = 0; j < BR; ++j) {
            // within each 64-channel group, channel o goes to row (o%4)*16 + o/4
            int row = 64 * j + (r0 & 3) * 16 + (r0 >> 2);
            *(v4i *)(sB + (buf * BN + row) * 64 + ((cq ^ swz(row)) << 4)) = pb[j];
        }
    };

    // ---- accumulators, initialised with the folded BN bias ----
    const int c = lane & 15;
    const int g = lane >> 4;
    const int ocl = n0 + wn0 + 4 * c;  // first of this lane's four output channels
    v4i acc[MT][NT];
#pragma unroll
    for (int tn = 0; tn < NT; ++tn) {
        int o = ocl + tn;
        int bv = o < a.oc ? a.bias[o] : 0;
#pragma unroll
        for (int tm = 0; tm < MT; ++tm) acc[tm][tn] = (v4i){bv, bv, bv, bv};
    }

    // ---- K loop: double-buffered LDS ----
    load_step();
    store_step(0);
    __syncthreads();
    for (int step = 0; step < nsteps; ++step) {
        const int buf = step & 1;
        const bool more = step + 1 < nsteps;
        if (more) load_step();
        v4i af[MT], bf[NT];
#pragma unroll
        for (int tm = 0; tm < MT; ++tm) {
            int r = lane & 15;
            int row = wm0 + 16 * tm + 4 * (r & 3) + (r >> 2);
            af[tm] = *(const v4i *)(sA + (buf * BM + row) * 64 + ((g ^ swz(row)) << 4));
        }
#pragma unroll
        for (int tn = 0; tn < NT; ++tn) {
            int row = wn0 + 16 * tn + c;
            bf[tn] = *(const v4i *)(sB + (buf * BN + row) * 64 + ((g ^ swz(row)) << 4));
        }
#pragma unroll
        for (int tm = 0; tm < MT; ++tm)
#pragma unroll
            for (int tn = 0; tn < NT; ++tn)
                acc[tm][tn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[tm], bf[tn], acc[tm][tn], 0, 0, 0);
        if (more) store_step(buf ^ 1);
        __syncthreads();
    }

    // ---- fused epilogue ----
    // lane (g, c) of MFMA tile (tm, tn) holds pixel wm0 + 16tm + 4i + g and
    // output channel ocl + tn, for i = 0..3.
    const int pbase = m0 + wm0;
    const int b0 = pbase / HoWo;
    const int hw0 = pbase - b0 * HoWo;

    if (a.out_i32) {
        int32_t *y = (int32_t *)a.y;
        const bool vec = (a.oc & 3) == 0 && ocl + 3 < a.oc;
#pragma unroll
        for (int tm = 0; tm < MT; ++tm)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int p = pbase + 16 * tm + 4 * i + g;
                if (p >= a.m) continue;
                long long off = (long long)p * a.oc + ocl;
                if (vec) {
                    *(v4i *)(y + off) = (v4i){acc[tm][0][i], acc[tm][1][i], acc[tm][2][i], acc[tm][3][i]};
                } else {
#pragma unroll
                    for (int tn = 0; tn < NT; ++tn)
                        if (ocl + tn < a.oc) y[off + tn] = acc[tm][tn][i];
                }
            }
        return;
    }

    if (ocl >= a.oc1 * 32) return;  // this lane's channels are past the last output block

    int mul[NT], rnd[NT], shm[NT], shf[NT];
    bool fast_lane = true;
#pragma unroll
    for (int tn = 0; tn < NT; ++tn) {
        int o = ocl + tn;
        bool v = o < a.oc;
        mul[tn] = v ? a.mult[o] : 0;
        shf[tn] = v ? a.shift[o] : 2;
        fast_lane = fast_lane && shf[tn] >= 2;
        rnd[tn] = 1 << ((shf[tn] - 2) & 31);
        shm[tn] = shf[tn] - 1;
    }
    const bool fast = __all(fast_lane);
    int keep[NT];
#pragma unroll
    for (int tn = 0; tn < NT; ++tn) keep[tn] = ocl + tn < a.oc ? 0xff : 0;

    int8_t *y = (int8_t *)a.y;
    const long long cblk = ocl >> 5;
    const int cbyte = ocl & 31;
#pragma unroll
    for (int tm = 0; tm < MT; ++tm)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int off = 16 * tm + 4 * i + g;
            if (pbase + off >= a.m) continue;
            int b = b0;
            int hw = hw0 + off;
            while (hw >= HoWo) {
                hw -= HoWo;
                ++b;
            }
            const long long addr = (((long long)b * a.oc1 + cblk) * HoWo + hw) * 32 + cbyte;
            unsigned rr = 0;
            if (a.residual) rr = *(const unsigned *)(a.res + addr);
            unsigned packed = 0;
#pragma unroll
            for (int tn = 0; tn < NT; ++tn) {
                int yv = acc[tm][tn][i];
                int q = fast ? requant_fast(yv, mul[tn], rnd[tn], shm[tn]) : requant_any(yv, mul[tn], shf[tn]);
                if (a.residual) q += (int)(signed char)(rr >> (8 * tn));
                if (a.relu) q = max(q, 0);
                q = min(max(q, -128), 127);
                packed |= (unsigned)(q & keep[tn]) << (8 * tn);
            }
            *(unsigned *)(y + addr) = packed;
        }
}

template <int KH, int KW, int BM, int BN>
hipError_t launch_tiles(const ConvArgs &a, hipStream_t s)
{
    long long tiles_m = (a.m + BM - 1) / BM;
    long long tiles_n = (a.oc1 * 32 + BN - 1) / BN;
    long long blocks = tiles_m * tiles_n;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((conv_kernel<KH, KW, BM, BN>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int KH, int KW>
hipError_t launch_k(const ConvArgs &a, hipStream_t s)
{
    if (a.oc1 * 32 > 64) return launch_tiles<KH, KW, 128, 128>(a, s);
    return launch_tiles<KH, KW, 256, 64>(a, s);
}

}  // namespace

hipError_t launch_conv(const ConvArgs &a, int kh, int kw, hipStream_t s)
{
    if (kh == 1 && kw == 1) return launch_k<1, 1>(a, s);
    if (kh == 3 && kw == 3) return launch_k<3, 3>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace ifx
