// Fused stem: 7x7 stride-2 pad-3 convolution over <= 4 input channels, folded
// BN, ReLU and a 3x3 stride-2 pad-1 max-pool, in one kernel (the
// CONV+BN+RELU+MAXPOOL single function of the DiDi IFX DAWNBench blog,
// inference-optimisation section).  The pre-pool tensor never leaves LDS.
//
// gfx950 design:
//   * persistent 256-thread workgroups, each walking a list of 8x8 tiles of
//     pooled pixels x 64 channels; the 64 filters stay in registers for the
//     whole launch, and the next tile's input window is loaded into
//     registers while the current tile computes;
//   * per tile, the 17x17 convolution pixels under the pooling windows are
//     computed (the one-pixel halo shared with neighbouring tiles is
//     recomputed) from a 40x40-pixel input window staged in LDS as 4 bytes
//     per pixel (the <= 4 channels, zero-filled), so one 16-byte MFMA operand
//     is four consecutive kernel columns x four channels;
//   * the window is read either from the packed NC/32HW32 tensor (first word
//     of each 32-byte pixel vector) or straight from the compact NHWC image
//     (aligned dword loads of three-byte pixels, unpacked with v_perm), which
//     folds the input pack into the stem;
//   * reduction order per output channel: (ky, kx, c) with 32 bytes per
//     kernel row (column 7 and channel 3 are zero weights, row 7 a zero row):
//     K = 256 = four v_mfma_i32_16x16x64_i8 steps;
//   * each convolution pixel is requantised (bias, fixed-point scale, ReLU,
//     saturation) as soon as its MFMAs finish and kept as a biased byte in
//     LDS; the 3x3 max-pool runs on those bytes, exactly as the layer is
//     defined, and writes whole 16-byte chunks of the packed output;
//   * tiles are dealt out in contiguous runs per XCD, so the input rows two
//     neighbouring tiles share are read through the same L2.
#include "device_common.h"
#include "ifx_internal.h"

namespace ifx {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kPT = 8;                  // pooled tile edge
constexpr int kCT = 2 * kPT + 1;        // convolution tile edge (17)
constexpr int kCPix = kCT * kCT;        // 289 convolution pixels
constexpr int kMT = (kCPix + 15) / 16;  // 19 MFMA row tiles
constexpr int kIT = 2 * kCT + 6;        // 40 input rows/cols staged
constexpr int kOC = 64;

// input paths
constexpr int kPacked = 0;   // packed [n, 1, h, w, 32]
constexpr int kNhwc3 = 1;    // compact NHWC, c == 3, w % 4 == 0: 12-byte groups of 4 pixels
constexpr int kNhwcAny = 2;  // compact NHWC, any c <= 4 and w: byte loads

constexpr int kPkSlots = (kIT * kIT + kThreads - 1) / kThreads;      // 7 pixels per thread
constexpr int kGroups = kIT / 4 + 1;                                // 11 groups cover a window row
constexpr int kG3Slots = (kIT * kGroups + kThreads - 1) / kThreads;  // 2 groups per thread
constexpr int kPre = 8;                                             // prefetch registers
static_assert(kPkSlots <= kPre && 3 * kG3Slots <= kPre, "prefetch registers");

struct Tile {
    int b, py0, px0, cy0, cx0, iy0, ix0;
};

__device__ __forceinline__ Tile tile_geo(int t, int tiles_x, int tiles_y)
{
    Tile g;
    const int tx = t % tiles_x;
    t /= tiles_x;
    const int ty = t % tiles_y;
    g.b = t / tiles_y;
    g.py0 = ty * kPT;
    g.px0 = tx * kPT;
    g.cy0 = 2 * g.py0 - 1;  // first convolution pixel of the tile
    g.cx0 = 2 * g.px0 - 1;
    g.iy0 = 2 * g.cy0 - 3;  // first input pixel of the window
    g.ix0 = 2 * g.cx0 - 3;
    return g;
}

// Issue the loads of a tile's input window into registers.
template <int PATH>
__device__ __forceinline__ void fetch(const StemArgs &a, const Tile &g, unsigned (&pre)[kPre])
{
    const int tid = threadIdx.x;
    if (PATH == kPacked) {
        const int8_t *img = a.x + (long long)g.b * a.h * a.w * 32;
#pragma unroll
        for (int s = 0; s < kPkSlots; ++s) {
            const int i = tid + s * kThreads;
            const int ry = i / kIT, rx = i - (i / kIT) * kIT;
            const int iy = g.iy0 + ry, ix = g.ix0 + rx;
            unsigned v = 0;
            if (i < kIT * kIT && (unsigned)iy < (unsigned)a.h && (unsigned)ix < (unsigned)a.w)
                v = *(const unsigned *)(img + ((long long)iy * a.w + ix) * 32);
            pre[s] = v;
        }
    } else if (PATH == kNhwc3) {
        // ix0 = 4 px0 - 5 = 3 (mod 4): the groups of 4 pixels start at ix0 - 3
        const int8_t *img = a.x + (long long)g.b * a.h * a.w * 3;
#pragma unroll
        for (int s = 0; s < kG3Slots; ++s) {
            const int i = tid + s * kThreads;
            const int ry = i / kGroups, gi = i - (i / kGroups) * kGroups;
            const int iy = g.iy0 + ry, gx = g.ix0 - 3 + 4 * gi;
            unsigned d0 = 0, d1 = 0, d2 = 0;
            // w % 4 == 0 and gx % 4 == 0: a group lies wholly inside or outside the row
            if (i < kIT * kGroups && (unsigned)iy < (unsigned)a.h && (unsigned)gx < (unsigned)a.w) {
                const unsigned *src = (const unsigned *)(img + ((long long)iy * a.w + gx) * 3);
                d0 = __builtin_nontemporal_load(src);
                d1 = __builtin_nontemporal_load(src + 1);
                d2 = __builtin_nontemporal_load(src + 2);
            }
            pre[3 * s] = d0;
            pre[3 * s + 1] = d1;
            pre[3 * s + 2] = d2;
        }
    }
}

// Write a tile's input window into LDS: sIn[ry][rx] = the channel bytes of
// input pixel (iy0 + ry, ix0 + rx), zero outside the image.
template <int PATH>
__device__ __forceinline__ void put(const StemArgs &a, const Tile &g, const unsigned (&pre)[kPre], int32_t *sIn)
{
    const int tid = threadIdx.x;
    if (PATH == kPacked) {
#pragma unroll
        for (int s = 0; s < kPkSlots; ++s) {
            const int i = tid + s * kThreads;
            if (i < kIT * kIT) sIn[i] = (int)pre[s];
        }
    } else if (PATH == kNhwc3) {
#pragma unroll
        for (int s = 0; s < kG3Slots; ++s) {
            const int i = tid + s * kThreads;
            if (i >= kIT * kGroups) continue;
            const int ry = i / kGroups, gi = i - (i / kGroups) * kGroups;
            const unsigned d0 = pre[3 * s], d1 = pre[3 * s + 1], d2 = pre[3 * s + 2];
            unsigned p[4];
            p[0] = __builtin_amdgcn_perm(d1, d0, 0x0c020100u);  // bytes 0..2
            p[1] = __builtin_amdgcn_perm(d1, d0, 0x0c050403u);  // bytes 3..5
            p[2] = __builtin_amdgcn_perm(d2, d1, 0x0c040302u);  // bytes 6..8
            p[3] = __builtin_amdgcn_perm(d2, d2, 0x0c030201u);  // bytes 9..11
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rx = 4 * gi + e - 3;  // window column of pixel e of the group
                if ((unsigned)rx < (unsigned)kIT) sIn[ry * kIT + rx] = (int)p[e];
            }
        }
    } else {
        const int8_t *img = a.x + (long long)g.b * a.h * a.w * a.c;
        for (int i = tid; i < kIT * kIT; i += kThreads) {
            const int ry = i / kIT, rx = i - (i / kIT) * kIT;
            const int iy = g.iy0 + ry, ix = g.ix0 + rx;
            unsigned v = 0;
            if ((unsigned)iy < (unsigned)a.h && (unsigned)ix < (unsigned)a.w) {
                const unsigned char *src = (const unsigned char *)(img + ((long long)iy * a.w + ix) * a.c);
                for (int ch = 0; ch < a.c; ++ch) v |= (unsigned)src[ch] << (8 * ch);
            }
            sIn[i] = (int)v;
        }
    }
}

// Packed 16-bit maxima: the pooled tile keeps int8 values biased to unsigned
// (q + 128), so the 3x3 maximum runs on the even and odd bytes separately.
__device__ __forceinline__ unsigned pkmax(unsigned x, unsigned y)
{
    const u16x2 r = __builtin_elementwise_max(__builtin_bit_cast(u16x2, x), __builtin_bit_cast(u16x2, y));
    return __builtin_bit_cast(unsigned, r);
}

// Per-channel parameters in LDS, one int32 per channel each: bias, multiplier,
// shift, and for shift >= 2 the rounding high word 2^(shift-2) and shift - 1.
struct ChanParams {
    int bias[kOC], mul[kOC], shf[kOC], rnd[kOC], shm[kOC];
    int add_lo[kOC], add_hi[kOC];  // bias * mult + (rnd << 32): the bias folded into mode 1's constant
};

// Convolution of one tile into sConv (biased int8 [pixel][channel]).
// MODE 0: general requant, ReLU if a.relu; 1: shift >= 2 with ReLU; 2: shift >= 2, no ReLU.
template <int MODE>
__device__ __forceinline__ void conv_tile(const StemArgs &a, const Tile &g, const int32_t *sIn, int8_t *sConv,
                                          const v4i (&wf)[4][4], const ChanParams &P)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane & 15, grp = lane >> 4;
    const int kh_off = grp >> 1;    // kernel row within a K step (two rows per step)
    const bool interior = g.cy0 >= 0 && g.cx0 >= 0 && g.cy0 + kCT <= a.ho && g.cx0 + kCT <= a.wo;
    const int kw0 = 4 * (grp & 1);  // first kernel column of this lane's 16 bytes
    for (int tm = wave; tm < kMT; tm += 4) {
        int q = 16 * tm + (lane & 15);
        if (q >= kCPix) q = kCPix - 1;  // padding rows: any valid address, results dropped
        const int ly = q / kCT, lx = q - (q / kCT) * kCT;
        v4i acc[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const v2i *src = (const v2i *)&sIn[(2 * ly + 2 * ks + kh_off) * kIT + 2 * lx + kw0];
            const v2i lo = src[0], hi = src[1];
            const v4i af = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
            for (int tn = 0; tn < 4; ++tn)
                acc[tn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, wf[tn][ks], acc[tn], 0, 0, 0);
        }
        const v4i bias = *(const v4i *)&P.bias[4 * c];
        const v4i mul = *(const v4i *)&P.mul[4 * c];
        const v4i shf = *(const v4i *)&P.shf[4 * c];
        const v4i rnd = *(const v4i *)&P.rnd[4 * c];
        const v4i shm = *(const v4i *)&P.shm[4 * c];
        const v4i alo = *(const v4i *)&P.add_lo[4 * c];
        const v4i ahi = *(const v4i *)&P.add_hi[4 * c];
        // only tiles at the image border (or the last, partial row tile) need per-pixel checks
        const bool edge = !interior || tm == kMT - 1;
        // lane (grp, c) holds conv pixels 16tm + 4grp + i, channels 4c + tn; pixels outside
        // the convolution output are stored as 0 (= -128) so the max ignores them (every
        // pooling window holds its centre pixel, which is inside)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int qq = 16 * tm + 4 * grp + i;
            bool inside = true;
            if (edge) {
                const int qy = qq / kCT, qx = qq - (qq / kCT) * kCT;
                inside = qq < kCPix && (unsigned)(g.cy0 + qy) < (unsigned)a.ho && (unsigned)(g.cx0 + qx) < (unsigned)a.wo;
            }
            int r[4];
#pragma unroll
            for (int tn = 0; tn < 4; ++tn) {
                int v;
                if (MODE == 0) {
                    v = requant_any(acc[tn][i] + bias[tn], mul[tn], shf[tn]);
                    if (a.relu) v = max(v, 0);
                } else if (MODE == 1) {
                    const long long add = (long long)(((unsigned long long)(unsigned)ahi[tn] << 32) | (unsigned)alo[tn]);
                    v = max(((int)(((long long)acc[tn][i] * (long long)mul[tn] + add) >> 32)) >> shm[tn], 0);
                } else {
                    v = requant_fast(acc[tn][i] + bias[tn], mul[tn], rnd[tn], shm[tn]);
                }
                r[tn] = min(max(v, -128), 127);
            }
            const unsigned word = inside ? (pack4(r[0], r[1], r[2], r[3]) ^ 0x80808080u) : 0u;
            if (!edge || qq < kCPix) *(unsigned *)&sConv[qq * kOC + 4 * c] = word;
        }
    }
}

// Workgroups resident per CU: the register budget (at most 168 VGPRs, three waves per SIMD)
// sets it; the launch bounds hold the compiler to it and the persistent grid is sized by it.
constexpr int kStemPerCu = 3;

template <int PATH>
__global__ __launch_bounds__(kThreads, kStemPerCu) void stem_kernel(StemArgs a, int tiles, int per_xcd)
{
    __shared__ __attribute__((aligned(16))) int32_t sIn[kIT * kIT];      // 4 channel bytes per pixel
    __shared__ __attribute__((aligned(16))) int8_t sConv[kCPix * kOC];  // biased int8 conv outputs [px][ch]
    __shared__ __attribute__((aligned(16))) ChanParams sP;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int tiles_x = (a.pw + kPT - 1) / kPT;
    const int tiles_y = (a.ph + kPT - 1) / kPT;

    // tile list: XCD x = blockIdx % 8 owns tiles [x * per_xcd, (x + 1) * per_xcd); its
    // workgroups take them round robin
    const int xcd = blockIdx.x & 7;
    const int stride = gridDim.x >> 3;
    const int t_end = min(tiles, (xcd + 1) * per_xcd);
    int t = xcd * per_xcd + (int)(blockIdx.x >> 3);
    if (t >= t_end) return;

    // filters and per-channel parameters of this lane: MFMA column c of tile tn = channel 4c + tn
    const int c = lane & 15, grp = lane >> 4;
    v4i wf[4][4];
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
        const int8_t *wp = a.wt + (4 * c + tn) * 256 + grp * 16;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) wf[tn][ks] = *(const v4i *)(wp + ks * 64);
    }
    if (tid < kOC) {
        const int sh = a.shift[tid];
        sP.bias[tid] = a.bias[tid];
        sP.mul[tid] = a.mult[tid];
        sP.shf[tid] = sh;
        sP.rnd[tid] = 1 << ((sh - 2) & 31);
        sP.shm[tid] = sh - 1;
        const long long add = (long long)a.bias[tid] * a.mult[tid] + ((long long)(1 << ((sh - 2) & 31)) << 32);
        sP.add_lo[tid] = (int)(unsigned)(add & 0xffffffffLL);
        sP.add_hi[tid] = (int)(add >> 32);
    }
    // one wave reads all 64 shifts, and every wave takes the same decision
    const bool fast = __all(a.shift[lane] >= 2);
    const int mode = !fast ? 0 : (a.relu ? 1 : 2);

    unsigned pre[kPre];
    Tile g = tile_geo(t, tiles_x, tiles_y);
    fetch<PATH>(a, g, pre);
    for (;;) {
        // sIn is free: every wave's MFMA reads of the previous tile are behind the
        // barrier before its pool; sConv is free once every wave passes this barrier,
        // since each wave's pool reads come before it
        put<PATH>(a, g, pre, sIn);
        lds_barrier();
        const int t_next = t + stride;
        if (t_next < t_end) fetch<PATH>(a, tile_geo(t_next, tiles_x, tiles_y), pre);  // in flight during this tile
        if (mode == 0)
            conv_tile<0>(a, g, sIn, sConv, wf, sP);
        else if (mode == 1)
            conv_tile<1>(a, g, sIn, sConv, wf, sP);
        else
            conv_tile<2>(a, g, sIn, sConv, wf, sP);
        lds_barrier();

        // 3x3/s2 max-pool of the biased bytes: thread = pooled pixel x 16 channels
        const int pp = tid >> 2;
        const int cg = (tid & 3) * 16;
        const int ply = pp / kPT, plx = pp - (pp / kPT) * kPT;
        const int py = g.py0 + ply, px = g.px0 + plx;
        if (py < a.ph && px < a.pw) {
            unsigned ev[4] = {0u, 0u, 0u, 0u}, od[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int dy = 0; dy < 3; ++dy)
#pragma unroll
                for (int dx = 0; dx < 3; ++dx) {
                    const v4i v = *(const v4i *)&sConv[((2 * ply + dy) * kCT + 2 * plx + dx) * kOC + cg];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        ev[j] = pkmax(ev[j], (unsigned)v[j] & 0x00ff00ffu);
                        od[j] = pkmax(od[j], ((unsigned)v[j] >> 8) & 0x00ff00ffu);
                    }
                }
            v4i mx;
#pragma unroll
            for (int j = 0; j < 4; ++j) mx[j] = (int)((ev[j] | (od[j] << 8)) ^ 0x80808080u);
            int8_t *dst = a.y + ((((long long)g.b * 2 + (cg >> 5)) * a.ph + py) * a.pw + px) * 32 + (cg & 31);
            store16_stream(dst, mx);
        }
        if (t_next >= t_end) break;
        t = t_next;
        g = tile_geo(t, tiles_x, tiles_y);
    }
}

template <int PATH>
hipError_t launch_path(const StemArgs &a, int tiles, hipStream_t s)
{
    // as many workgroups as the chip holds at once (never more, so none waits for another)
    int cus = 0;
    hipError_t e = current_cus(&cus);
    if (e != hipSuccess) return e;
    long long g = (long long)kStemPerCu * cus;
    g = g / 8 * 8;  // a multiple of 8 so every XCD gets the same number
    if (g < 8) g = 8;
    const long long need = (tiles + 7LL) / 8 * 8;
    if (g > need) g = need;
    const int per_xcd = (int)((tiles + 7LL) / 8);
    hipLaunchKernelGGL(stem_kernel<PATH>, dim3((unsigned)g), dim3(kThreads), 0, s, a, tiles, per_xcd);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_stem(const StemArgs &a, hipStream_t s)
{
    const long long tiles = (long long)a.n * ((a.ph + kPT - 1) / kPT) * ((a.pw + kPT - 1) / kPT);
    if (tiles <= 0) return hipSuccess;
    if (tiles > 0x7ffffff0LL) return hipErrorInvalidConfiguration;
    if (!a.nhwc) return launch_path<kPacked>(a, (int)tiles, s);
    if (a.c == 3 && (a.w & 3) == 0) return launch_path<kNhwc3>(a, (int)tiles, s);
    return launch_path<kNhwcAny>(a, (int)tiles, s);
}

}  // namespace ifx
