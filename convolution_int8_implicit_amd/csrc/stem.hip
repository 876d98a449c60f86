// Fused stem: 7x7 stride-2 pad-3 convolution over <= 4 input channels, folded
// BN, ReLU and a 3x3 stride-2 pad-1 max-pool, in one kernel (the
// CONV+BN+RELU+MAXPOOL single function of the DiDi IFX DAWNBench blog,
// inference-optimisation section).  The pre-pool tensor never leaves the
// registers.
//
// gfx950 design:
//   * persistent 256-thread workgroups walk units of 8 pooled rows x 28
//     pooled columns x 64 channels; the 64 filters stay in registers for the
//     whole launch;
//   * the v_mfma_i32_16x16x64_i8 operands are oriented so that a lane's
//     results are 16 consecutive output channels of ONE convolution pixel:
//     the filters are the A operand (rows = channels), the input patches the
//     B operand (columns = 16 consecutive convolution columns of one row, a
//     "strip"); each wave owns a strip and walks down the 17 convolution
//     rows of the unit;
//   * the max-pool runs on the int32 accumulators, before requantisation:
//     the epilogue (bias, fixed-point scale with a non-negative multiplier,
//     ReLU, saturation) is non-decreasing, so the maximum of the epilogues is
//     the epilogue of the maximum.  Rows pool in registers (each odd
//     convolution row serves two pooled rows), columns across neighbouring
//     lanes of a 16-lane DPP row; only the pooled outputs are requantised,
//     two pooled rows packed into one register set;
//   * reduction order per output channel: (ky, kx, c) with 32 bytes per
//     kernel row (column 7 and channel 3 are zero weights, row 7 a zero row):
//     K = 256 = four K-steps; the input window sits in LDS at 4 bytes per
//     pixel, so a lane's 16 K-bytes are 4 consecutive pixels of one row;
//   * the window of the next unit is fetched while the current one computes:
//     the compact NHWC image (3 bytes per pixel) goes by buffer->LDS DMA into
//     a staging area as whole row segments, and one pass spreads it to 4
//     bytes per pixel with zeros outside the image (the input pack folded
//     into the stem).  A packed NC/32HW32 input (first word of each pixel) or
//     an NHWC image of other channel counts is gathered into the window at
//     the start of its unit;
//   * units are dealt out in contiguous runs per XCD, so the input rows two
//     neighbouring units share are read through the same L2.
#include "device_common.h"
#include "ifx_internal.h"

namespace ifx {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;               // four waves, one strip each
constexpr int kOC = 64;
constexpr int kPR = 8;                      // pooled rows per unit
constexpr int kSP = 7;                      // pooled columns per strip (centres at odd lanes 1..13)
constexpr int kStrips = 4;                  // strips per unit
constexpr int kUnitPW = kStrips * kSP;      // 28 pooled columns per unit
static_assert(kPR % 2 == 0, "pooled rows are requantised in pairs");
constexpr int kCR = 2 * kPR + 1;            // convolution rows per unit (17)
constexpr int kWR = 2 * (kCR - 1) + 8;      // window rows (40)
constexpr int kWC = 128;                    // window columns, 4 bytes per pixel
constexpr int kWPitch = kWC * 4;            // 512 bytes
constexpr int kWinBytes = kWR * kWPitch;    // 20 KB
// A staged raw row starts 16 pixels (48 bytes, three whole DMA chunks) before input column
// 4 px0, so at the image's first row and column the chunks fall either wholly before the image
// (read as zeros) or wholly inside it.  Window column wc is raw pixel wc + 9, i.e. raw byte
// 3 wc + 27: the four window columns 4j .. 4j + 3 (one aligned 16-byte LDS word) come from raw
// bytes 12j + 27 .. 12j + 38, inside the four dwords at 12j + 24.
constexpr int kRawLead = 16;                // raw pixels before input column 4 px0
constexpr int kRawChunks = 27;              // 16-byte DMA chunks per raw row (432 >= 12 * 31 + 40 bytes)
constexpr int kRawPitch = 16 * kRawChunks;  // 432 bytes per raw row in the staging area
constexpr int kRawDma = 5;                  // DMA instructions per wave per unit (4 waves x 5 x 64 >= 40 x 27)
constexpr int kStageBytes = kRawDma * 4 * 1024;  // 20 KB: every lane of those instructions lands inside
static_assert(kRawDma * 4 * 64 >= kWR * kRawChunks, "one DMA lane per raw chunk");
static_assert(12 * (kWC / 4 - 1) + 40 <= kRawPitch, "the last window word's raw bytes fit the pitch");
static_assert(3 * (kRawLead - 7) == 27, "window column wc is raw byte 3 wc + 27");

// input paths
constexpr int kPacked = 0;   // packed [n, 1, h, w, 32]: the first word of each pixel
constexpr int kNhwc3 = 1;    // compact NHWC, c == 3, w % 4 == 0: raw row segments by DMA
constexpr int kNhwcAny = 2;  // compact NHWC, any c <= 4 and w: byte loads

// Unit geometry: pooled rows [py0, py0 + 8), pooled columns [px0, px0 + 28) of image b.
// Convolution row r of the unit is y = 2 py0 - 1 + r; window row wr holds input row
// 4 py0 - 5 + wr and window column wc input column 4 px0 - 7 + wc (odd, so every B fragment
// starts on an 8-byte boundary); raw pixel p of a staging row is input column 4 px0 - 16 + p.
struct Unit {
    int b, py0, px0;
};

__device__ __forceinline__ Unit unit_geo(int u, int bands, int halves)
{
    Unit g;
    const int half = u % halves;
    u /= halves;
    g.px0 = half * kUnitPW;
    g.py0 = (u % bands) * kPR;
    g.b = u / bands;
    return g;
}

// Per-channel parameters in LDS.
struct ChanParams {
    int bias[kOC], mul[kOC], shf[kOC], rnd[kOC], shm[kOC];
    int add_lo[kOC], add_hi[kOC];  // bias * mult + (rnd << 32): the bias folded into mode 1's constant
};

// DMA the raw NHWC (3-byte) row segments of unit g into the staging area: chunk k (16 bytes)
// of window row wr is lane idx = 27 wr + k of this workgroup's 20 instructions, which lands at
// staging byte 16 idx = 432 wr + 16 k.
__device__ __forceinline__ void issue_raw(const StemArgs &a, const Unit &g, int8_t *stage, int wave, int lane)
{
    const long long img = (long long)a.h * a.w * 3;
    const v4i rs = make_rsrc(a.x + (long long)g.b * img, img);
    const int iy0 = 4 * g.py0 - 5, rx0 = 4 * g.px0 - kRawLead;
#pragma unroll
    for (int q = 0; q < kRawDma; ++q) {
        const int inst = q * 4 + wave;
        const int idx = inst * 64 + lane;
        const int wr = idx / kRawChunks, k = idx - wr * kRawChunks;
        const int iy = iy0 + wr;
        const long long off = ((long long)iy * a.w + rx0) * 3 + 16 * k;
        const bool ok = wr < kWR && (unsigned)iy < (unsigned)a.h && off >= 0;
        load16_lds_stream(rs, stage + inst * 1024, ok ? (unsigned)off : kOOB);
    }
}

// Spread the staged raw rows into the window: 4 bytes per pixel (channel 3 = 0), zero outside
// the image.  Thread item (wr, j) writes window columns 4j .. 4j + 3 as one 16-byte word.
__device__ __forceinline__ void unpack_raw(const StemArgs &a, const Unit &g, const int8_t *stage, int8_t *win,
                                           int tid)
{
    const int iy0 = 4 * g.py0 - 5, wx0 = 4 * g.px0 - 7;
    for (int it = tid; it < kWR * (kWC / 4); it += kThreads) {
        const int wr = it / (kWC / 4), j = it - wr * (kWC / 4);
        const unsigned *src = (const unsigned *)(stage + wr * kRawPitch + 12 * j + 24);
        const unsigned d0 = src[0], d1 = src[1], d2 = src[2], d3 = src[3];
        // pixel k of the word starts at byte 3 + 3k of d0..d3
        unsigned p[4];
        p[0] = __builtin_amdgcn_perm(d1, d0, 0x0c050403u);  // d0[3], d1[0], d1[1]
        p[1] = __builtin_amdgcn_perm(d2, d1, 0x0c040302u);  // d1[2], d1[3], d2[0]
        p[2] = __builtin_amdgcn_perm(d2, d2, 0x0c030201u);  // d2[1], d2[2], d2[3]
        p[3] = __builtin_amdgcn_perm(d3, d3, 0x0c020100u);  // d3[0], d3[1], d3[2]
        const bool row_ok = (unsigned)(iy0 + wr) < (unsigned)a.h;
        v4i w;
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = (row_ok && (unsigned)(wx0 + 4 * j + k) < (unsigned)a.w) ? (int)p[k] : 0;
        *(v4i *)(win + wr * kWPitch + 16 * j) = w;
    }
}

// Fill the window of unit g directly (paths without a staging area); the caller waits.
template <int PATH>
__device__ __forceinline__ void gather_window(const StemArgs &a, const Unit &g, int8_t *win, int wave, int lane,
                                              int tid)
{
    const int iy0 = 4 * g.py0 - 5, wx0 = 4 * g.px0 - 7;
    if (PATH == kPacked) {
        // one word per lane: window row wr, half hh covers columns [64 hh, 64 hh + 64)
        const long long img = (long long)a.h * a.w * 32;
        const v4i rs = make_rsrc(a.x + (long long)g.b * img, img);
        for (int q = wave; q < 2 * kWR; q += 4) {
            const int wr = q >> 1, wc = (q & 1) * 64 + lane;
            const int iy = iy0 + wr, ix = wx0 + wc;
            const bool ok = (unsigned)iy < (unsigned)a.h && (unsigned)ix < (unsigned)a.w;
            ifx_raw_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)(win + q * 256), 4,
                                    ok ? (unsigned)((iy * a.w + ix) * 32) : kOOB, 0, 0, 0);
        }
    } else {
        const int8_t *img = a.x + (long long)g.b * a.h * a.w * a.c;
        for (int i = tid; i < kWR * kWC; i += kThreads) {
            const int wr = i / kWC, wc = i - wr * kWC;
            const int iy = iy0 + wr, ix = wx0 + wc;
            unsigned v = 0;
            if ((unsigned)iy < (unsigned)a.h && (unsigned)ix < (unsigned)a.w) {
                const unsigned char *src = (const unsigned char *)(img + ((long long)iy * a.w + ix) * a.c);
                for (int ch = 0; ch < a.c; ++ch) v |= (unsigned)src[ch] << (8 * ch);
            }
            ((unsigned *)win)[i] = v;
        }
    }
}

constexpr int kIMin = (int)0x80000000;

// Lane c of a 16-lane DPP row gets lane c - 1's value / lane c + 1's / lane c + 2's; a lane
// without a source in its row gets 0 (lanes 0, 14 and 15, whose results are never stored).
__device__ __forceinline__ int from_left(int v) { return __builtin_amdgcn_mov_dpp(v, 0x111, 0xf, 0xf, true); }
__device__ __forceinline__ int from_right(int v) { return __builtin_amdgcn_mov_dpp(v, 0x101, 0xf, 0xf, true); }
__device__ __forceinline__ int from_right2(int v) { return __builtin_amdgcn_mov_dpp(v, 0x102, 0xf, 0xf, true); }
__device__ __forceinline__ int max3(int a, int b, int c) { return max(max(a, b), c); }
// max(a, dpp(b)) then max(., dpp(b)) as two-operand maxima: the empty barrier keeps the compiler
// from merging them into one three-input max, so each DPP move folds into its max (v_max_i32
// with a DPP operand) instead of costing an instruction of its own
__device__ __forceinline__ int max_lr(int v, int l, int r)
{
    int t = max(v, l);
    asm volatile("" : "+v"(t));
    return max(t, r);
}

// One convolution row of the wave's strip: acc[tn][i] = channel 16 (lane / 16) + 4 tn + i of
// convolution column c = lane % 16.  wrow: the window bytes of the row's first K-step at this
// lane's fragment offset.
__device__ __forceinline__ void conv_row(const int8_t *wrow, const v4i (&wf)[4][4], v4i (&acc)[4])
{
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const v2i lo = *(const v2i *)(wrow + ks * 2 * kWPitch);
        const v2i hi = *(const v2i *)(wrow + ks * 2 * kWPitch + 8);
        const v4i bfrag = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
            acc[tn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[tn][ks], bfrag, ks == 0 ? (v4i){0, 0, 0, 0} : acc[tn], 0,
                                                            0, 0);
    }
}

// Requantise channel groups K0 and K0 + 1 of a lane's 16 pooled accumulators (channels
// ch0 + 4 k + i, held at m[k][i]) and pack them into words 0 and 1 of the result: half of the
// lane's 16 output bytes.  MODE 0: general form (ReLU if relu); 1: shift >= 2 with ReLU;
// 2: shift >= 2, no ReLU.
template <int MODE, int K0>
__device__ __forceinline__ v2i requant8(const v4i (&m)[4], const ChanParams &P, int ch0, bool relu)
{
    v2i out;
#pragma unroll
    for (int k = K0; k < K0 + 2; ++k) {
        // one channel group's parameters in flight at a time (register pressure)
        if (k > K0) asm volatile("" ::: "memory");
        const int ch = ch0 + 4 * k;
        int r[4];
        if (MODE == 1) {
            const v4i mul = *(const v4i *)&P.mul[ch], shm = *(const v4i *)&P.shm[ch];
            const v4i alo = *(const v4i *)&P.add_lo[ch], ahi = *(const v4i *)&P.add_hi[ch];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const long long add = (long long)(((unsigned long long)(unsigned)ahi[i] << 32) | (unsigned)alo[i]);
                const int v = ((int)(((long long)m[k][i] * (long long)mul[i] + add) >> 32)) >> shm[i];
                r[i] = min(max(v, 0), 127);
            }
        } else if (MODE == 2) {
            const v4i bias = *(const v4i *)&P.bias[ch], mul = *(const v4i *)&P.mul[ch];
            const v4i rnd = *(const v4i *)&P.rnd[ch], shm = *(const v4i *)&P.shm[ch];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                r[i] = min(max(requant_fast(m[k][i] + bias[i], mul[i], rnd[i], shm[i]), -128), 127);
        } else {
            const v4i bias = *(const v4i *)&P.bias[ch], mul = *(const v4i *)&P.mul[ch];
            const v4i shf = *(const v4i *)&P.shf[ch];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int v = requant_any(m[k][i] + bias[i], mul[i], shf[i]);
                if (relu) v = max(v, 0);
                r[i] = min(max(v, -128), 127);
            }
        }
        out[k - K0] = (int)pack4(r[0], r[1], r[2], r[3]);
    }
    return out;
}

// The wave's strip of unit g: 17 convolution rows, pooled rows in pairs.  Pooled row p is the
// maximum over convolution rows 2p, 2p + 1, 2p + 2 and, per centre column, over its neighbours.
// Rows and columns outside the convolution output are replaced by the nearest row or column
// inside it, which belongs to the same pooling window, so the maximum is unchanged and no
// masking is needed (a strip or row past the output reads in-window data that is never stored).
//
// Software pipeline: once the vertical maximum of pooled row p is taken, rows 2p and 2p + 1
// are dead, and the matrix pipe computes convolution rows 2p + 3 and 2p + 4 into their
// registers while the VALU finishes row p (the horizontal maximum, and half of a pair's
// requantisation, see requant_lo / requant_store).  Rows
// live in three rotating register sets (row r in set r % 3); the band is unrolled so every set
// index is a constant.
template <int MODE>
__device__ __forceinline__ void compute_unit(const StemArgs &a, const Unit &g, const int8_t *win,
                                             const v4i (&wf)[4][4], const ChanParams &P, int wave, int lane)
{
    const int c = lane & 15, grp = lane >> 4;
    const int xs = 2 * g.px0 - 1 + 14 * wave;  // convolution column of lane c = 0
    const int x = max(min(max(xs + c, 0), a.wo - 1), xs);
    // window bytes of this lane's B fragment for convolution row 0, K-step 0: window column
    // 2 x - 3 + 4 (grp & 1) - (4 px0 - 7)
    const int8_t *wl = win + (grp >> 1) * kWPitch + (2 * (x - xs) + 28 * wave + 4 * (grp & 1) + 2) * 4;
    const int y0 = 2 * g.py0 - 1;
    const int ymax = max(a.ho - 1, y0);
    v4i R[3][4], vm[4];
    auto row = [&](int r) __attribute__((always_inline)) {
        const int re = min(max(y0 + r, 0), ymax) - y0;  // nearest row inside the output
        conv_row(wl + re * 2 * kWPitch, wf, R[r % 3]);
    };
    auto vertical = [&](int p) __attribute__((always_inline)) {
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                vm[tn][i] = max3(R[(2 * p) % 3][tn][i], R[(2 * p + 1) % 3][tn][i], R[(2 * p + 2) % 3][tn][i]);
    };
    v4i pm[4];
    // pooled row p into pm: odd (centre) lanes of a first row of a pair keep their own 3-max;
    // even lanes of a second row take the 3-max of the lane to their right (a centre column,
    // moved one lane left)
    auto pool = [&](int p) __attribute__((always_inline)) {
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int v = vm[tn][i];
                if ((p & 1) == 0) {
                    pm[tn][i] = max_lr(v, from_left(v), from_right(v));
                } else {
                    // computed in every lane: a DPP read of a lane that the exec mask has switched
                    // off returns the old value, and the compiler would otherwise compute it only
                    // in the even lanes that use it (the volatile barrier keeps it out of any branch)
                    int t = max_lr(v, from_right(v), from_right2(v));
                    asm volatile("" : "+v"(t));
                    pm[tn][i] = (c & 1) ? pm[tn][i] : t;
                }
            }
    };
    // A pair of pooled rows is requantised in two halves, each in a scheduling region that also
    // issues 32 MFMAs of later convolution rows: channel groups 0-1 right after the pair's second
    // row is pooled, groups 2-3 in the next pooled row's region, before its pooling overwrites
    // pm.  Both halves are computed in every lane, outside the store's branch (the empty register
    // barriers), so the compiler can interleave them with the matrix instructions instead of
    // running them on their own after the branch.  The parameters are re-read from LDS each time
    // (a fence keeps the compiler from hoisting all 64 of a lane's words out of the band).
    const long long out_img = 2LL * a.ph * a.pw * 32;  // the image's two 32-channel blocks
    const v4i ys = make_rsrc(a.y + (long long)g.b * out_img, out_img);
    v2i q01;
    auto requant_lo = [&]() __attribute__((always_inline)) {
        asm volatile("" ::: "memory");
        q01 = requant8<MODE, 0>(pm, P, 16 * grp, a.relu != 0);
        asm volatile("" : "+v"(q01));
    };
    auto requant_store = [&](int pp) __attribute__((always_inline)) {
        asm volatile("" ::: "memory");
        v2i q23 = requant8<MODE, 2>(pm, P, 16 * grp, a.relu != 0);
        asm volatile("" : "+v"(q23));
        const v4i q = {q01.x, q01.y, q23.x, q23.y};
        // before the unit's last store, this wave's memory operations are waited for: the next
        // unit's raw rows (requested a whole unit of work ago) and the earlier stores.  Loads and
        // stores share one counter whose order is not guaranteed between them, so this is a
        // wait for zero; at the top of the next unit no store is left to wait for but this one.
        if (pp == kPR / 2 - 1) wait_vmcnt<0>();
        // odd lanes: pooled row 2pp, column (c - 1) / 2 of the strip; even lanes: row 2pp + 1,
        // column c / 2.  A buffer store with no branch (a branch would end the scheduling region
        // and leave the next pooling without matrix work to overlap): lanes without an output
        // (c >= 14, or a row or column past the image) take an offset past the range.
        const int py = g.py0 + 2 * pp + ((c & 1) ? 0 : 1);
        const int px = g.px0 + kSP * wave + (c >> 1);
        const bool ok = c < 14 && py < a.ph && px < a.pw;
        const unsigned off = ok ? (unsigned)((((grp >> 1) * a.ph + py) * a.pw + px) * 32 + 16 * (grp & 1)) : kOOB;
        ifx_raw_buffer_store_v4i32(q, ys, off, 0, kCachePolicyNT);
    };

    row(0);
    row(1);
    row(2);
#pragma unroll
    for (int p = 0; p < kPR; ++p) {
        // one scheduling region per pooled row: nothing is hoisted into the previous one, which
        // would only cost registers
        __builtin_amdgcn_sched_barrier(0);
        vertical(p);
        if (p + 1 < kPR) {
            row(2 * p + 3);
            row(2 * p + 4);
        }
        if (p & 1) {
            pool(p);
            requant_lo();
        } else {
            if (p > 0) requant_store((p >> 1) - 1);
            pool(p);
        }
    }
    requant_store(kPR / 2 - 1);
}

// Workgroups resident per CU: the register budget (at most 256 VGPRs, two waves per SIMD)
// sets it; the launch bounds hold the compiler to it and the persistent grid is sized by it.
constexpr int kStemPerCu = 2;

template <int PATH>
__global__ __launch_bounds__(kThreads, waves_per_simd(kThreads, kStemPerCu)) void stem_kernel(StemArgs a, int units, int per_xcd)
{
    __shared__ __attribute__((aligned(1024))) int8_t sWin[kWinBytes];
    __shared__ __attribute__((aligned(1024))) int8_t sStage[PATH == kNhwc3 ? kStageBytes : 16];
    __shared__ __attribute__((aligned(16))) ChanParams sP;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bands = (a.ph + kPR - 1) / kPR;
    const int halves = (a.pw + kUnitPW - 1) / kUnitPW;

    // unit list: XCD x = blockIdx % 8 owns units [x * per_xcd, (x + 1) * per_xcd); its
    // workgroups take them round robin
    const int xcd = blockIdx.x & 7;
    const int stride = gridDim.x >> 3;
    const int u_end = min(units, (xcd + 1) * per_xcd);
    int u = xcd * per_xcd + (int)(blockIdx.x >> 3);
    if (u >= u_end) return;

    // filters: A operand of tile tn, K-step ks; MFMA row m = lane % 16 is output channel
    // 16 (m / 4) + 4 tn + m % 4, so a lane's results are 16 consecutive channels
    const int c = lane & 15, grp = lane >> 4;
    v4i wf[4][4];
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
        const int8_t *wp = a.wt + (16 * (c >> 2) + 4 * tn + (c & 3)) * 256 + grp * 16;
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

    Unit g = unit_geo(u, bands, halves);
    if (PATH == kNhwc3) {
        issue_raw(a, g, sStage, wave, lane);
        wait_vmcnt<0>();
    }
    for (;;) {
        // the previous unit's reads of the window are behind this barrier
        if (PATH == kNhwc3) {
            lds_barrier();  // every wave's raw DMAs have landed (each waited before its last store)
            unpack_raw(a, g, sStage, sWin, tid);
            lds_barrier();  // the window is complete and the staging area free
        } else {
            lds_barrier();
            gather_window<PATH>(a, g, sWin, wave, lane, tid);
            wait_vmcnt<0>();
            lds_barrier();
        }
        const int u_next = u + stride;
        const Unit gn = unit_geo(u_next < u_end ? u_next : u, bands, halves);
        if (PATH == kNhwc3 && u_next < u_end) issue_raw(a, gn, sStage, wave, lane);  // lands during this unit
        if (mode == 0)
            compute_unit<0>(a, g, sWin, wf, sP, wave, lane);
        else if (mode == 1)
            compute_unit<1>(a, g, sWin, wf, sP, wave, lane);
        else
            compute_unit<2>(a, g, sWin, wf, sP, wave, lane);
        if (u_next >= u_end) break;
        u = u_next;
        g = gn;
    }
}

template <int PATH>
hipError_t launch_path(const StemArgs &a, int units, hipStream_t s)
{
    if (answer_query("stem_kernel<%d>", PATH)) return hipSuccess;
    // as many workgroups as the chip holds at once (never more, so none waits for another)
    int cus = 0;
    hipError_t e = current_cus(&cus);
    if (e != hipSuccess) return e;
    long long g = (long long)kStemPerCu * cus;
    g = g / 8 * 8;  // a multiple of 8 so every XCD gets the same number
    if (g < 8) g = 8;
    const long long need = (units + 7LL) / 8 * 8;
    if (g > need) g = need;
    const int per_xcd = (int)((units + 7LL) / 8);
    hipLaunchKernelGGL(stem_kernel<PATH>, dim3((unsigned)g), dim3(kThreads), 0, s, a, units, per_xcd);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_stem(const StemArgs &a, hipStream_t s)
{
    const long long units = (long long)a.n * ((a.ph + kPR - 1) / kPR) * ((a.pw + kUnitPW - 1) / kUnitPW);
    if (units <= 0) return hipSuccess;
    if (units > 0x7ffffff0LL) return hipErrorInvalidConfiguration;
    if ((long long)a.h * a.w * 32 >= 0x7fffffffLL) return hipErrorInvalidValue;  // per-image offsets
    if (!a.nhwc) return launch_path<kPacked>(a, (int)units, s);
    if (a.c == 3 && (a.w & 3) == 0) return launch_path<kNhwc3>(a, (int)units, s);
    return launch_path<kNhwcAny>(a, (int)units, s);
}

}  // namespace ifx
