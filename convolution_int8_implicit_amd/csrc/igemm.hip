// General implicit-GEMM convolution (any kernel size, stride, padding and
// channel count): one BM x BN output tile per workgroup.
//
// Computation: Inspur conv-merge article, section 3.3 (data[M,K] .
// weight[N,K]^T over NC/32HW32 activations and [O1,KH,KW,I1,O2,32] weights)
// and section 3.4 (BN + Sum + ReLU applied to the accumulators before the
// store).  The design is the gfx950 one:
//   * K advances 64 bytes per step: two 32-channel blocks, taken in the flat
//     (tap, channel-block) order of the weight layout, so any channel count
//     and any kernel size share one loop;
//   * each step's operands reach LDS by buffer->LDS DMA in 1 KB
//     instructions, and every instruction reads ONE contiguous 1 KB piece of
//     HBM: 32 pixels x 32 channels of one block of the activation (a run of
//     consecutive pixels, shifted by the tap), or 32 output channels x 32
//     input channels of one weight block.  Gathering several segments per
//     instruction (as a row-per-pixel layout would) costs more than half of
//     the DMA rate on this chip;
//   * out-of-image taps, rows past the end and blocks past K read through
//     the buffer range check as zeros (no im2col, no branches);
//   * two LDS stages (double buffer, one barrier per step) and small LDS
//     (33-50 KB), so 3-4 workgroups share a CU and hide each other's
//     latency, prologue and epilogue;
//   * within a stage an operand block is [rows][32 B] with a 16-byte-slot
//     swizzle per 128-byte line, so the DMA writes whole lines and the
//     ds_read_b128 fragment reads of v_mfma_i32_16x16x64_i8 are free of bank
//     conflicts;
//   * the epilogue (per-channel bias, fixed-point requant, shortcut add,
//     ReLU, saturate) runs on the accumulators and writes whole 16-byte
//     chunks of the NC/32HW32 output.
#include "device_common.h"
#include "ifx_internal.h"

namespace ifx {
namespace {

// BM x BN tiles, a ring of ST stages; each wave owns a 64 x WN sub-tile (WN = 64 or 128: a wider
// sub-tile reuses each activation fragment for twice the MACs, halving the LDS reads per MAC)
template <int BM, int BN, int ST, int WN = 64>
struct IgCfg {
    static constexpr int WAVES_M = BM / 64;
    static constexpr int WNH = WN / 64;  // 64-channel halves of a wave's sub-tile
    static constexpr int WAVES = WAVES_M * (BN / WN);
    static_assert(WN == 64 || WN == 128, "64- or 128-channel wave sub-tiles");
    static_assert(WAVES == 4 || WAVES == 8 || WAVES == 16, "four, eight or sixteen waves");
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int A_CH = BM / 32;  // 32-row chunks of a tile's pixels
    static constexpr int B_CH = BN / 32;  // 32-row chunks of a tile's output channels
    static constexpr int AI = 2 * A_CH / WAVES;  // activation DMAs per wave per K-step
    static constexpr int BI = 2 * B_CH / WAVES;  // weight DMAs per wave per K-step
    static_assert(AI * WAVES == 2 * A_CH && BI * WAVES == 2 * B_CH, "whole DMAs");
    static constexpr int STAGE = (BM + BN) * 64;  // A: [2][BM][32 B], then B: [2][BN][32 B]
    static constexpr int PARAM = WAVES * WNH * 768;  // per wave and half: bias, mult, shift of 64 channels
    static constexpr int LPS = AI + BI;          // DMAs per wave per stage
    // a fused projection with 64x128 wave sub-tiles keeps its requantised output (the shortcut) in
    // registers, 32 per lane, and its parameters in a second parameter region
    static constexpr bool sc_regs(bool proj) { return proj && WNH == 2; }
    // ring | parameters | shortcut tile (RES), or the projection's parameters (register shortcut)
    static constexpr int lds(bool res, bool proj = false)
    {
        return ST * STAGE + PARAM + (sc_regs(proj) ? PARAM : (res ? BM * BN : 0));
    }
    // at most four waves per SIMD (so up to 128 VGPRs each; two, with up to 256, for the wide
    // sub-tile's accumulators), as LDS allows
    static constexpr int MAXW = WN == 64 ? 16 : 8;
    static constexpr int wg_per_cu(bool res, bool proj = false)
    {
        return kLdsBytes / lds(res, proj) > MAXW / WAVES ? MAXW / WAVES : kLdsBytes / lds(res, proj);
    }
    // the epilogue stages each wave's 64x64 output in the ring slot no wave reads any more, or,
    // when the waves' 4 KB parts do not fit one slot, across the ring after a workgroup barrier
    static constexpr bool STAGE_IN_SLOT = WAVES * WNH * 4096 <= STAGE;
    static_assert(WAVES * WNH * 4096 <= ST * STAGE, "the output staging fits the ring");
};

// LDS layouts of one operand block of a stage (32 K-bytes per row, two 16-byte halves h).
// Rows go four to a 128-byte line, so each 8-lane group of a DMA fetches one whole
// 128-byte line of consecutive pixels or weight rows; the slot of (row, h) inside its
// line is XOR-swizzled against the ds_read_b128 fragment reads.  Such a read serves
// its 64 lanes in four passes of 16 lanes, {0-7, 24-31}, {8-15, 16-23}, {32-39, 56-63}
// and {40-47, 48-55}; a pass takes one cycle when its lanes hit 16 different 16-byte
// bank slots (16 per 256 bytes).  Fragment lane (c = l % 16, g = l / 16) reads half
// g % 2 of pixel row 4(c%4) + c/4 of a 16-row group, or of weight row 4c + tn, so each
// pass reads half 0 of eight rows and half 1 of eight others; both swizzles give every
// pass 16 distinct slots.
__device__ __forceinline__ int a_swz(int row, int h)
{
    return ((row >> 2) << 7) | (((((row & 3) ^ ((row >> 2) & 3)) << 1) | (h ^ (row & 1))) << 4);
}
__device__ __forceinline__ int b_swz(int row, int h)
{
    return ((row >> 2) << 7) | ((((row & 3) << 1 | h) ^ ((row >> 2) & 6)) << 4);
}
// Inverses for the DMA: lane l of an instruction that fills rows [32 c, 32 c + 32) lands at
// byte 16 l of that 1 KB and must fetch half dma_*_h(l) of row 32 c + dma_*_row(l); lanes
// 8k..8k+7 fetch rows 4k..4k+3.
__device__ __forceinline__ int dma_a_row(int lane) { return 4 * (lane >> 3) + (((lane & 7) >> 1) ^ ((lane >> 3) & 3)); }
__device__ __forceinline__ int dma_a_h(int lane) { return (lane & 1) ^ (dma_a_row(lane) & 1); }
__device__ __forceinline__ int dma_b_row(int lane) { return 4 * (lane >> 3) + (((lane & 7) ^ ((lane >> 3) & 6)) >> 1); }
__device__ __forceinline__ int dma_b_h(int lane) { return lane & 1; }

template <int V>
struct Slot {
    static constexpr int value = V;
};

// f(Slot<I>()), ..., f(Slot<N - 1>()), unrolled at compile time
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(Slot<I>());
        static_for<I + 1, N>(f);
    }
}

// Requantise the wave's accumulators (MODE picked by a wave vote on the shifts) into the LDS tile
// at rbase (row stride 64 B), adding the shortcut bytes already there when RES.  ADD_BIAS: the
// accumulators do not hold the bias yet.
template <bool RES, bool RELU, bool ADD_BIAS>
__device__ __forceinline__ void requant_to_lds(const v4i (&acc)[4][4], int8_t *rbase, const int8_t *Pw, int c,
                                               int ocl, int oc)
{
    RqLane r;
    const int mode = rq_setup<RES, RELU>(r, *(const v4i *)(Pw + c * 16), *(const v4i *)(Pw + 256 + c * 16),
                                         *(const v4i *)(Pw + 512 + c * 16), !ADD_BIAS, ocl, oc);
    requant_tile_any<RES, RELU, 64>(mode, acc, rbase, r);
}

// One convolution `a` (with its epilogue), or, when PROJ, the last 1x1 convolution `a` of a
// bottleneck whose shortcut is the 1x1 projection `pj` of the block input: the tile's
// projection is computed first and requantised (no ReLU) into the LDS that otherwise receives
// a shortcut tile, so the shortcut never goes through HBM.
template <int KH, int KW, int BM, int BN, int ST, int WN, bool RES, bool RELU, bool PROJ>
__global__ __launch_bounds__((IgCfg<BM, BN, ST, WN>::THREADS),
                              (waves_per_simd(IgCfg<BM, BN, ST, WN>::THREADS, IgCfg<BM, BN, ST, WN>::wg_per_cu(RES, PROJ))))
void igemm_kernel(ConvArgs a, ConvArgs pj, int tiles_n, int per_xcd)
{
    using C = IgCfg<BM, BN, ST, WN>;
    constexpr int WNH = C::WNH;
    constexpr int NWV = C::WAVES;
    static_assert(!PROJ || (RES && KH == 1 && KW == 1), "a projection shortcut feeds a 1x1 shortcut conv");
    static_assert(!PROJ || ST == 2, "the stream switches convolutions one stage ahead");
    constexpr bool SCR = C::sc_regs(PROJ);  // the shortcut stays in registers
    __shared__ __attribute__((aligned(1024))) int8_t smem[C::lds(RES, PROJ)];
    int8_t *const Pm = smem + ST * C::STAGE;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm0 = (wave % C::WAVES_M) * 64;
    const int wn0 = (wave / C::WAVES_M) * WN;
    // half hh of the wave's channels (64 each): parameters at Pw + 768 hh (bias, mult, shift), the
    // RES shortcut / output staging [64 pixels][64 B] at Rres + 4096 hh
    int8_t *const Pw = Pm + wave * WNH * 768;
    int8_t *const Rres = Pm + C::PARAM + wave * WNH * 4096;
    int8_t *const Ppj = Pm + C::PARAM + wave * WNH * 768;  // the projection's parameters (SCR)

    // tile: XCD x (blockIdx & 7) owns M-tiles [x * per_xcd, (x + 1) * per_xcd), so neighbouring
    // pixel tiles (which share 3x3 halo rows) and the N-tiles of one pixel tile share an L2
    const int xcd = blockIdx.x & 7;
    const int kk = blockIdx.x >> 3;
    const int mq = kk / tiles_n;
    const int m0 = (xcd * per_xcd + mq) * BM;
    if (m0 >= a.m) return;
    const int n0 = (kk - mq * tiles_n) * BN;
    const int ch0 = n0 + wn0;

    const int HoWo = a.ho * a.wo;
    const long long out_img = (long long)a.oc1 * HoWo * 32;
    const int img0 = fdiv(m0, a.howo_mul, a.howo_shr);

    // ---- fragment addresses (stage-relative): lane (r = lane % 16, g = lane / 16) reads
    //      pixel row 4(r%4) + r/4 of each 16-row group and weight row 4r + tn, K bytes [16g, 16g+16)
    const int c = lane & 15;
    const int g = lane >> 4;
    // rows 16 apart sit 4 lines (512 B) apart with the same slot; weight row 4c + tn sits at
    // the slot of row 4c XOR 32 tn
    const int a_frag = (g >> 1) * (BM * 32) + a_swz(wm0 + 4 * (c & 3) + (c >> 2), g & 1);
    int b_frag[WNH][4];
#pragma unroll
    for (int hh = 0; hh < WNH; ++hh)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
            b_frag[hh][tn] = (BM * 64 + (g >> 1) * (BN * 32) + b_swz(wn0 + 64 * hh + 4 * c, g & 1)) ^ (tn << 5);

    v4i acc[WNH][4][4];
    unsigned sc[SCR ? WNH : 1][4][4];  // the requantised projection (SCR): rows 16tm + 4i + g, channels 4c..4c+3

    // ---- per-lane DMA plans of convolution q.  Activation DMA j of wave w fills chunk
    //      (4j + w) % A_CH of block (4j + w) / A_CH: the lane's pixel, its tap-validity mask and
    //      base offset.  Weight DMA j likewise for B_CH.
    // geometry of the convolution whose K-steps are being issued
    int HW = 0, wblk = 0, qi1 = 0, qnkb = 0, qw = 0, qkb0 = 0;
    bool in_ps = false;
    v4i rsA, rsB;
    int a_base[C::AI], b_base[C::BI];
    unsigned a_nmask[C::AI];  // complement of the lane's tap-validity mask (bit 31 always set)
    unsigned b_bad[C::BI];    // 1 << 31 for a weight row past the buffer, else 0
    auto plan = [&](const ConvArgs &q) __attribute__((always_inline)) {
        HW = q.h * q.w;
        qi1 = q.i1;
        in_ps = q.in_ps != 0;
        // this workgroup's part of the reduction: blocks [qkb0, qnkb)
        qkb0 = (PROJ || q.ksplit <= 1) ? 0 : (int)blockIdx.y * q.kb_per;
        qnkb = (PROJ || q.ksplit <= 1) ? q.nkb : min(q.nkb, qkb0 + q.kb_per);
        qw = q.w;
        const long long in_img = (long long)q.i1 * HW * 32;
        rsA = make_rsrc(q.x + (long long)img0 * in_img, (long long)(q.n - img0) * in_img);
        const int wrows = ((q.oc + q.o2 - 1) / q.o2) * q.o2;
        rsB = make_rsrc(q.wt, (long long)wrows * KH * KW * q.i1 * 32);
        wblk = q.o2 * 32;  // bytes of one (tap, channel-block) slice of an O1 group
#pragma unroll
        for (int j = 0; j < C::AI; ++j) {
            const int chunk = (j * NWV + wave) % C::A_CH;
            const int row = chunk * 32 + dma_a_row(lane);
            const int h = dma_a_h(lane);
            const int p = m0 + row;
            const bool ok = p < q.m;
            const int pp = ok ? p : m0;
            const int b = fdiv(pp, q.howo_mul, q.howo_shr);
            const int rem = pp - b * HoWo;
            const int oy = fdiv(rem, q.wo_mul, q.wo_shr);
            const int ox = rem - oy * q.wo;
            const int iy0 = oy * q.stride - q.pad;
            const int ix0 = ox * q.stride - q.pad;
            // phase-split input (stride 2, pad 1): every tap of pixel (oy, ox) reads position
            // (oy, ox) of a parity plane, shifted by at most one row and column (step offsets)
            const int pix = q.in_ps ? oy * (q.w >> 1) + ox : iy0 * q.w + ix0;
            a_base[j] = (int)((long long)(b - img0) * in_img) + pix * 32 + h * 16;
            unsigned mask = 0;
#pragma unroll
            for (int ky = 0; ky < KH; ++ky)
#pragma unroll
                for (int kx = 0; kx < KW; ++kx)
                    if ((unsigned)(iy0 + ky) < (unsigned)q.h && (unsigned)(ix0 + kx) < (unsigned)q.w)
                        mask |= 1u << (ky * KW + kx);
            a_nmask[j] = ok ? ~mask : ~0u;
        }
#pragma unroll
        for (int j = 0; j < C::BI; ++j) {
            const int chunk = (j * NWV + wave) % C::B_CH;
            const int row = chunk * 32 + dma_b_row(lane);
            const int h = dma_b_h(lane);
            const int R = n0 + row;
            const bool rok = R < wrows;
            b_bad[j] = rok ? 0u : 0x80000000u;
            const int RR = rok ? R : 0;
            const int o1 = fdiv(RR, q.o2_mul, q.o2_shr);
            b_base[j] = o1 * (KH * KW * q.i1 * wblk) + (RR - o1 * q.o2) * 32 + h * 16;
        }
    };

    // ---- the K-step stream: the steps of pj (PROJ only), then those of a.  Step s covers
    //      the flat 32-channel blocks kb = 2s, 2s+1 of its convolution, kb -> (tap, channel block).
    const int n1 = PROJ ? (pj.nkb + 1) >> 1 : 0;
    int iss = 0;                  // next step to issue
    int cur_c1 = 0, cur_tap = 0;  // block 2s of that step, within its convolution
    if (PROJ)
        plan(pj);
    else
        plan(a);
    if (!PROJ && qkb0 > 0) {  // a split-K part starts inside the reduction
        cur_tap = qkb0 / qi1;
        cur_c1 = qkb0 - cur_tap * qi1;
    }
    const int nsteps = n1 + (PROJ ? (a.nkb + 1) >> 1 : (qnkb - qkb0 + 1) >> 1);
    auto issue = [&](int slot) __attribute__((always_inline)) {
        const int s = iss - (iss >= n1 ? n1 : 0);
        ++iss;
        int8_t *st = smem + slot * C::STAGE;
        int c1b = cur_c1 + 1, tapb = cur_tap;  // block 2s + 1
        if (c1b == qi1) {
            c1b = 0;
            ++tapb;
        }
        const int kb0 = qkb0 + 2 * s;
        const bool v0 = kb0 < qnkb, v1 = kb0 + 1 < qnkb;
        const int ky0 = cur_tap / KW, kx0 = cur_tap - ky0 * KW;
        const int ky1 = tapb / KW, kx1 = tapb - ky1 * KW;
        // tap (ky, kx) of a stride-2 pad-1 3x3 on a phase-split input: parity plane
        // ((ky + 1) % 2, (kx + 1) % 2), shifted one row / column back for ky = 0 / kx = 0
        auto tap_off = [&](int ky, int kx) __attribute__((always_inline)) {
            if (!in_ps) return (ky * qw + kx) * 32;
            const int py = (ky + 1) & 1, px = (kx + 1) & 1;
            return ((py * 2 + px) * (HW >> 2) + ((ky - 1 - py) >> 1) * (qw >> 1) + ((kx - 1 - px) >> 1)) * 32;
        };
        const int dA0 = cur_c1 * HW * 32 + tap_off(ky0, kx0);
        const int dA1 = c1b * HW * 32 + tap_off(ky1, kx1);
        const int dB0 = kb0 * wblk, dB1 = dB0 + wblk;
        // a block past the convolution's K reads tap 31 of the complemented masks (always invalid)
        // and ORs bit 31 into the weight offsets: either way its lanes fall outside every buffer
        const int tap0 = v0 ? cur_tap : 31, tap1 = v1 ? tapb : 31;
        const unsigned nv0 = v0 ? 0u : 0x80000000u, nv1 = v1 ? 0u : 0x80000000u;
#pragma unroll
        for (int j = 0; j < C::AI; ++j) {
            const int blk = (j * NWV + wave) / C::A_CH;
            const int chunk = (j * NWV + wave) % C::A_CH;
            // an invalid lane gets bit 31 set: past every buffer range, so its DMA writes zeros
            const unsigned bad = (a_nmask[j] >> (blk ? tap1 : tap0)) & 1u;
            const unsigned off = (unsigned)(a_base[j] + (blk ? dA1 : dA0)) | (bad << 31);
            load16_lds(rsA, st + blk * (BM * 32) + chunk * 1024, off);
        }
#pragma unroll
        for (int j = 0; j < C::BI; ++j) {
            const int qq = j * NWV + wave;
            const int blk = qq / C::B_CH;
            const int chunk = qq % C::B_CH;
            const unsigned off = (unsigned)(b_base[j] + (blk ? dB1 : dB0)) | b_bad[j] | (blk ? nv1 : nv0);
            load16_lds(rsB, st + BM * 64 + blk * (BN * 32) + chunk * 1024, off);
        }
        cur_c1 += 2;
        while (cur_c1 >= qi1) {
            cur_c1 -= qi1;
            ++cur_tap;
        }
    };

    issue(0);
    // per-channel parameters and the shortcut part of this wave
    auto issue_params = [&](const ConvArgs &q, int8_t *dst, int chh) __attribute__((always_inline)) {
        if (lane < 16) {
            const bool v = chh + 4 * lane < q.oc;
            const unsigned off = v ? (unsigned)(chh + 4 * lane) * 4 : kOOB;
            load16_lds(make_rsrc(q.bias, (long long)q.oc * 4), dst, off);
            if (!q.out_i32) {
                load16_lds(make_rsrc(q.mult, (long long)q.oc * 4), dst + 256, off);
                load16_lds(make_rsrc(q.shift, (long long)q.oc * 4), dst + 512, off);
            }
        }
    };
#pragma unroll
    for (int hh = 0; hh < WNH; ++hh) issue_params(a, Pw + 768 * hh, ch0 + 64 * hh);
    // PROJ: the projection's parameters wait in the wave's shortcut region, which the
    // projection's requantisation overwrites only after reading them
    if (PROJ)
#pragma unroll
        for (int hh = 0; hh < WNH; ++hh) issue_params(pj, (SCR ? Ppj + 768 * hh : Rres + 4096 * hh), ch0 + 64 * hh);
    if (RES && !PROJ) {
        const v4i rsR = make_rsrc(a.res + (long long)img0 * out_img, (long long)(a.n - img0) * out_img);
#pragma unroll
        for (int hh = 0; hh < WNH; ++hh)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int p = m0 + wm0 + 16 * j + (lane >> 2);
                const int oc = ch0 + 64 * hh + (lane & 3) * 16;
                unsigned off = kOOB;
                if (p < a.m && oc < a.oc1 * 32) {
                    const int b = fdiv(p, a.howo_mul, a.howo_shr), hw = p - b * HoWo;
                    off = (unsigned)((((long long)(b - img0) * a.oc1 + (oc >> 5)) * HoWo + hw) * 32 + (oc & 31));
                }
                load16_lds_stream(rsR, Rres + 4096 * hh + j * 1024, off);
            }
    }
    // Stages after the tile inputs, so the first wait needs no count of them.  A stream that fits
    // the ring (nsteps <= ST, the short 1x1 convolutions) is requested whole, up front; a longer
    // one keeps ST-1 stages in flight and requests stage s+ST-1 at step s.
    const bool upfront = nsteps <= ST;
    if (upfront) {
        for (int s = 1; s < nsteps; ++s) {
            if (PROJ && s == n1) {  // the stream moves on to a's first step
                plan(a);
                cur_c1 = 0;
                cur_tap = 0;
            }
            issue(s);
        }
    } else {
#pragma unroll
        for (int s = 1; s < ST - 1; ++s)
            if (s < nsteps) issue(s);
    }

    // ---- epilogue geometry: lane (g, c) holds pixel rows 16tm + 4i + g and channels 4c .. 4c+3
    const int ocl = ch0 + 4 * c;
    const int pbase = m0 + wm0;

    // The first K-step of a contraction takes 0 as the MFMA's C operand, so no accumulator is
    // ever cleared; the per-channel bias enters in the requantisation (folded into its added
    // constant, free in the common mode).

    static_assert(ST >= 2 && ST <= 4, "a ring of two to four stages");
    // step s reads ring slot SL = s % ST, a compile-time constant so the fragment addresses
    // need no per-step arithmetic
    auto step = [&](auto slot, auto first, int s) __attribute__((always_inline)) {
        constexpr int SL = decltype(slot)::value;
        constexpr bool FIRST = decltype(first)::value != 0;
        // this wave's DMAs of stage s (and, at s = 0, the tile inputs): later stages requested
        // before them may stay in flight (one when up front, ST-2 in the ring)
        if (upfront ? s + 1 < nsteps : (ST > 2 && s + ST - 2 < nsteps))
            wait_vmcnt<(ST > 2 ? ST - 2 : 1) * C::LPS>();
        else if (!upfront && ST > 3 && s + 1 < nsteps)
            wait_vmcnt<C::LPS>();  // the ring's tail: one later stage in flight
        else
            wait_vmcnt<0>();
        ring_barrier();  // ... and every other wave's; stage s-1's slot is free again
        if (!upfront && s + ST - 1 < nsteps) issue((SL + ST - 1) % ST);
        const int8_t *st = smem + SL * C::STAGE;
        v4i af[4], bf[WNH][4];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) af[tm] = *(const v4i *)(st + a_frag + 512 * tm);
#pragma unroll
        for (int hh = 0; hh < WNH; ++hh)
#pragma unroll
            for (int tn = 0; tn < 4; ++tn) bf[hh][tn] = *(const v4i *)(st + b_frag[hh][tn]);
#pragma unroll
        for (int hh = 0; hh < WNH; ++hh)
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int tn = 0; tn < 4; ++tn)
                    if constexpr (FIRST)
                        acc[hh][tm][tn] =
                            __builtin_amdgcn_mfma_i32_16x16x64_i8(af[tm], bf[hh][tn], (v4i){0, 0, 0, 0}, 0, 0, 0);
                    else
                        acc[hh][tm][tn] =
                            __builtin_amdgcn_mfma_i32_16x16x64_i8(af[tm], bf[hh][tn], acc[hh][tm][tn], 0, 0, 0);
    };
    // fused form (ST == 2): steps s0 <= s < s1 of one contraction, none its first, slots alternating
    // inside the loop (a run-time slot choice per step would merge two register allocations of the
    // accumulators every iteration)
    auto run_range = [&](int s0, int s1) __attribute__((always_inline)) {
        int s = s0;
        if (s < s1 && (s & 1)) step(Slot<1>(), Slot<0>(), s++);
        for (; s + 1 < s1; s += 2) {
            step(Slot<0>(), Slot<0>(), s);
            step(Slot<1>(), Slot<0>(), s + 1);
        }
        if (s < s1) step(Slot<0>(), Slot<0>(), s);
    };
    if (PROJ) {
        // the projection's steps 0 .. n1-1; its last one requests a's first stage
        auto switch_to_a = [&]() __attribute__((always_inline)) {
            if (!upfront) {
                plan(a);
                cur_c1 = 0;
                cur_tap = 0;
            }
        };
        if (n1 == 1) {
            switch_to_a();
            step(Slot<0>(), Slot<1>(), 0);
        } else {
            step(Slot<0>(), Slot<1>(), 0);
            run_range(1, n1 - 1);
            switch_to_a();
            run_range(n1 - 1, n1);
        }
        // the projection is complete: its requantised output (no ReLU) is the shortcut, in registers
        // (SCR) or in the shortcut tile
        if constexpr (SCR) {
#pragma unroll
            for (int hh = 0; hh < WNH; ++hh) {
                const int8_t *const pp = Ppj + 768 * hh + c * 16;
                RqLane rp;
                const int mp = rq_setup<false, false>(rp, *(const v4i *)pp, *(const v4i *)(pp + 256),
                                                      *(const v4i *)(pp + 512), false, ocl + 64 * hh, pj.oc);
                requant_regs_any(mp, acc[hh], rp, sc[hh]);
            }
        } else {
#pragma unroll
            for (int hh = 0; hh < WNH; ++hh)
                requant_to_lds<false, false, true>(acc[hh], Rres + 4096 * hh + g * 64 + 4 * c, Rres + 4096 * hh, c,
                                                   ocl + 64 * hh, pj.oc);
        }
        if (n1 & 1)
            step(Slot<1>(), Slot<1>(), n1);
        else
            step(Slot<0>(), Slot<1>(), n1);
        run_range(n1 + 1, nsteps);
    } else {
        step(Slot<0>(), Slot<1>(), 0);
        static_for<1, ST>([&](auto sl) __attribute__((always_inline)) {
            if (decltype(sl)::value < nsteps) step(sl, Slot<0>(), decltype(sl)::value);
        });
        for (int s = ST; s < nsteps; s += ST)
            static_for<0, ST>([&](auto sl) __attribute__((always_inline)) {
                if (s + decltype(sl)::value < nsteps) step(sl, Slot<0>(), s + decltype(sl)::value);
            });
    }
    if (a.out_i32) {
        // a split-K part writes its own slice of partial sums; the bias is added once, after the sum
        int32_t *y = (int32_t *)a.y + (a.ksplit > 1 ? (long long)blockIdx.y * a.m * a.oc : 0LL);
#pragma unroll
        for (int hh = 0; hh < WNH; ++hh) {
            const int oh = ocl + 64 * hh;
            const bool vec = (a.oc & 3) == 0 && oh + 3 < a.oc;
            const v4i bias4 = a.ksplit > 1 ? (v4i){0, 0, 0, 0}
                                           : *(const v4i *)(Pw + 768 * hh + c * 16);  // zero past Oc
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int p = pbase + 16 * tm + 4 * i + g;
                    if (p >= a.m) continue;
                    const long long off = (long long)p * a.oc + oh;
                    const v4i v =
                        (v4i){acc[hh][tm][0][i], acc[hh][tm][1][i], acc[hh][tm][2][i], acc[hh][tm][3][i]} + bias4;
                    if (vec) {
                        *(v4i *)(y + off) = v;
                    } else {
#pragma unroll
                        for (int tn = 0; tn < 4; ++tn)
                            if (oh + tn < a.oc) y[off + tn] = v[tn];
                    }
                }
        }
        return;
    }
    // staging: the shortcut tile itself (requantised in place), else free ring memory
    constexpr bool IN_RING = !RES || SCR;
    if (IN_RING && !C::STAGE_IN_SLOT) lds_barrier();
    int8_t *const Rw =
        !IN_RING ? Rres : smem + (C::STAGE_IN_SLOT ? (nsteps % ST) * C::STAGE : 0) + wave * WNH * 4096;
    if constexpr (SCR) {
#pragma unroll
        for (int hh = 0; hh < WNH; ++hh) {
            const int8_t *const pa = Pw + 768 * hh + c * 16;
            RqLane r;
            const int mode = rq_setup<true, RELU>(r, *(const v4i *)pa, *(const v4i *)(pa + 256), *(const v4i *)(pa + 512),
                                                  false, ocl + 64 * hh, a.oc);
            requant_tile_sc_any<RELU, 64>(mode, acc[hh], Rw + 4096 * hh + g * 64 + 4 * c, r, sc[hh]);
        }
    } else {
#pragma unroll
        for (int hh = 0; hh < WNH; ++hh)
            requant_to_lds<RES, RELU, true>(acc[hh], Rw + 4096 * hh + g * 64 + 4 * c, Pw + 768 * hh, c,
                                            ocl + 64 * hh, a.oc);
    }
    wave_lds_sync();

    // 16-byte stores of the wave's 64 pixels x 64 (or 128) channels
    if (pbase >= a.m) return;
    int8_t *y = (int8_t *)a.y;
    const int k = lane & 3;
    const int b0 = fdiv(pbase, a.howo_mul, a.howo_shr);
    const int hw0 = pbase - b0 * HoWo;
    const int we = (a.wo + 1) >> 1;  // the even-pixel copy (y_even): ceil(ho / 2) x ceil(wo / 2) planes
    const long long plane_e = (long long)((a.ho + 1) >> 1) * we;
#pragma unroll
    for (int hh = 0; hh < WNH; ++hh) {
        const int och = ch0 + 64 * hh + 16 * k;  // first channel of this lane's chunk
        if (och >= a.oc1 * 32) break;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int prow = 16 * j + (lane >> 2);
            if (pbase + prow >= a.m) break;
            int b = b0, hw = hw0 + prow;
            while (hw >= HoWo) {
                hw -= HoWo;
                ++b;
            }
            const v4i v = *(const v4i *)(Rw + 4096 * hh + prow * 64 + 16 * k);
            long long pix = hw;
            if (a.out_ps) {  // phase-split output: the pixel's parity plane, then its place in it
                const int oy = fdiv(hw, a.wo_mul, a.wo_shr), ox = hw - oy * a.wo;
                pix = (long long)((oy & 1) * 2 + (ox & 1)) * (HoWo >> 2) + (oy >> 1) * (a.wo >> 1) + (ox >> 1);
            }
            int8_t *dst = y + (((long long)b * a.oc1 + (och >> 5)) * HoWo + pix) * 32 + (och & 31);
            if (RES)
                store16_stream(dst, v);
            else
                *(v4i *)dst = v;
            if (a.y_even) {
                const int oy = fdiv(hw, a.wo_mul, a.wo_shr), ox = hw - oy * a.wo;
                if (!((oy | ox) & 1))
                    store16_stream(a.y_even + (((long long)b * a.oc1 + (och >> 5)) * plane_e + (oy >> 1) * we +
                                               (ox >> 1)) * 32 + (och & 31),
                                   v);
            }
        }
    }
}

template <int KH, int KW, int BM, int BN, int ST, bool RES, bool PROJ, int WN = 64>
hipError_t launch_ig(const ConvArgs &a, const ConvArgs &pj, hipStream_t s)
{
    if (answer_query_even(!a.out_i32, "igemm_kernel<%d, %d, %d, %d, %d, %d, %s, %s, %s>", KH, KW, BM, BN, ST, WN,
                          tf(RES), tf(a.relu != 0), tf(PROJ)))
        return hipSuccess;
    const int tiles_n = (a.oc1 * 32 + BN - 1) / BN;
    const long long tiles_m = (a.m + BM - 1) / BM;
    const long long per = (tiles_m + 7) / 8;
    const long long grid = 8 * per * tiles_n;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    // activation offsets are taken relative to a tile's first image and must fit 31 bits
    const long long imgs = BM / ((long long)a.ho * a.wo) + 2;
    if (imgs * (long long)a.i1 * a.h * a.w * 32 >= 0x7fffffffLL) return hipErrorInvalidValue;
    if (PROJ && imgs * (long long)pj.i1 * pj.h * pj.w * 32 >= 0x7fffffffLL) return hipErrorInvalidValue;
    if (a.relu)
        hipLaunchKernelGGL((igemm_kernel<KH, KW, BM, BN, ST, WN, RES, true, PROJ>),
                           dim3((unsigned)grid, (unsigned)(a.ksplit > 1 ? a.ksplit : 1)),
                           dim3(IgCfg<BM, BN, ST, WN>::THREADS), 0, s, a, pj, tiles_n, (int)per);
    else
        hipLaunchKernelGGL((igemm_kernel<KH, KW, BM, BN, ST, WN, RES, false, PROJ>),
                           dim3((unsigned)grid, (unsigned)(a.ksplit > 1 ? a.ksplit : 1)),
                           dim3(IgCfg<BM, BN, ST, WN>::THREADS), 0, s, a, pj, tiles_n, (int)per);
    return hipGetLastError();
}

// ---- stride-1 3x3 over 128 or more input channels: haloed windows per 64-channel chunk ------
//
// The general kernel fetches each activation row again for every tap: nine 64-byte K-steps per
// pixel and 64 input channels.  Here a workgroup's tile is 224 output pixels of whole rows (8 rows
// of a 28-wide image, 16 of a 14-wide one) by 128 output channels, and the reduction runs over
// 64-channel chunks and, inside a chunk, over the nine taps.  A chunk's input window is fetched
// once, into one of two buffers, while the previous chunk computes; each tap's weights stream
// through a ring of three 8 KB stages.  Per K-step the activation DMA falls from 64 bytes per
// output pixel to about 7, and each weight byte serves 224 pixels instead of 128.
//
// Window rows: for a tile whose first output row is row y0 of image i0, output pixel (image i,
// row y, column x) reads, at tap (ky, kx), window row (i - i0)(H + 2) + (y - y0) + ky and window
// column x + kx.  Every image the tile touches thus contributes the rows it needs plus one halo
// row above and one below (zero outside the image).  The window pitch P (16 or 32 pixels, at
// least W + 2) is a multiple of 16, so a row shifted by ky keeps its slot swizzle and each lane
// needs base addresses only for the three column shifts.  The order of the reduction differs
// from the weight layout's, which integer sums do not see.

constexpr int kWinTile = 224;                  // output pixels per tile (14 groups of 16)
constexpr int kWinPx = 384;                    // window pixels per 32-channel block (rows x P)
constexpr int kWinBuf = 2 * kWinPx * 32;       // one chunk's window, two blocks: 24 KB
constexpr int kWinStage = 128 * 64;            // one K-step of 128 channels' weights: 8 KB
constexpr int kWinRows = kWinTile / 2;         // output pixels per wave (two waves along M)
constexpr int kWinLds = 2 * kWinBuf + 3 * kWinStage + 4 * 768;
constexpr int kWinDma = 2 * kWinPx / 32 / 4;   // window DMAs per wave per chunk (6)
static_assert(4 * kWinRows * 64 <= 2 * kWinBuf, "the output tile is staged over the windows");
static_assert(2 * kWinLds <= kLdsBytes, "two workgroups per CU");

template <int P, bool RELU>
__global__ __launch_bounds__(256, waves_per_simd(256, 2)) void conv3x3_win_kernel(ConvArgs a, int tiles_n, int per_xcd,
                                                                                  int tr)
{
    constexpr int TM = kWinRows / 16;  // 16-row groups per wave (7)
    __shared__ __attribute__((aligned(1024))) int8_t smem[kWinLds];
    int8_t *const Bs = smem + 2 * kWinBuf;  // weight ring [slot][block][128 rows][32 B], slots as b_swz
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int8_t *const Pw = Bs + 3 * kWinStage + wave * 768;
    const int mw = wave & 1, nw = wave >> 1;  // the wave's 112 pixels and 64 channels

    // tile: XCD x (blockIdx & 7) owns pixel tiles [x * per_xcd, (x + 1) * per_xcd), so tiles that
    // share halo rows, and the channel tiles of one pixel tile, share an L2
    const int xcd = blockIdx.x & 7;
    const int kk = blockIdx.x >> 3;
    const int mq = kk / tiles_n;
    const int m0 = (xcd * per_xcd + mq) * kWinTile;
    if (m0 >= a.m) return;
    const int n0 = (kk - mq * tiles_n) * 128;
    const int ch0 = n0 + 64 * nw;

    const int H = a.h, W = a.w, HW = H * W, H2 = H + 2;
    const int img0 = fdiv(m0, a.howo_mul, a.howo_shr);
    const int y0 = fdiv(m0 - img0 * HW, a.wo_mul, a.wo_shr);
    const int segs = fdiv(m0 + kWinTile - 1, a.howo_mul, a.howo_shr) - img0 + 1;  // images touched
    const int rows = tr + 2 * segs;                                                // window rows read
    const long long in_img = (long long)a.i1 * HW * 32;
    const v4i rsA = make_rsrc(a.x + (long long)img0 * in_img, (long long)(a.n - img0) * in_img);

    // window DMA q = 4j + wave fills 32 window pixels (1 KB) of block q / 12: with P = 32 one
    // window row, with P = 16 two (lanes 32-63 take the second).  A lane's column is the same in
    // every DMA; a row's source (image, input row), or its absence (halo rows outside the image,
    // rows the tile does not read), is wave-uniform.
    const int dr = dma_a_row(lane);
    const int lx = (dr & (P - 1)) - 1;
    const bool lsecond = P == 16 && dr >= 16;
    const unsigned lane_off = (unsigned)(lx * 32 + dma_a_h(lane) * 16);
    const bool col_ok = (unsigned)lx < (unsigned)W;
    auto row_src = [&](int wr) __attribute__((always_inline)) {  // chunk-0 offset of window row wr, or -1
        int u = wr + y0, sg = 0;
        while (u >= H2) {
            u -= H2;
            ++sg;
        }
        const int r_in = u - 1;
        const bool ok = wr < rows && (unsigned)r_in < (unsigned)H && img0 + sg < a.n;
        return ok ? (sg * a.i1 * HW + r_in * W) * 32 : -1;
    };
    auto issue_window = [&](int chunk, int buf) __attribute__((always_inline)) {
        int8_t *const dst = smem + buf * kWinBuf;
#pragma unroll
        for (int j = 0; j < kWinDma; ++j) {
            const int q = 4 * j + wave;
            const int blk = q >= 12 ? 1 : 0;
            const int cq = q - 12 * blk;
            const int src = P == 32 ? row_src(cq) : (lsecond ? row_src(2 * cq + 1) : row_src(2 * cq));
            const unsigned off =
                src >= 0 && col_ok ? (unsigned)(src + (2 * chunk + blk) * HW * 32) + lane_off : kOOB;
            load16_lds(rsA, dst + blk * (kWinPx * 32) + cq * 1024, off);
        }
    };

    // weight DMA q = 4j + wave fills 32 rows of block q / 4 of a stage
    const int wblk = a.o2 * 32;
    const int wrows = ((a.oc + a.o2 - 1) / a.o2) * a.o2;
    const v4i rsB = make_rsrc(a.wt, (long long)wrows * 9 * a.i1 * 32);
    int b_off[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int q = 4 * j + wave;
        const int R = n0 + 32 * (q & 3) + dma_b_row(lane);
        const int o1 = fdiv(R, a.o2_mul, a.o2_shr);
        b_off[j] = o1 * (9 * a.i1 * wblk) + (q >> 2) * wblk + (R - o1 * a.o2) * 32 + dma_b_h(lane) * 16;
    }
    auto issue_b = [&](int tap, int chunk, int slot) __attribute__((always_inline)) {
        // opaque per step: otherwise each tap's offset is hoisted out of the loop into a register
        int add = (tap * a.i1 + 2 * chunk) * wblk;
        asm volatile("" : "+s"(add));
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int q = 4 * j + wave;
            load16_lds(rsB, Bs + slot * kWinStage + (q >> 2) * 4096 + (q & 3) * 1024, (unsigned)(b_off[j] + add));
        }
    };

    // per-channel parameters of the wave's 64 channels, then chunk 0's window and two weight stages
    if (lane < 16) {
        const unsigned off = (unsigned)(ch0 + 4 * lane) * 4;
        load16_lds(make_rsrc(a.bias, (long long)a.oc * 4), Pw, off);
        load16_lds(make_rsrc(a.mult, (long long)a.oc * 4), Pw + 256, off);
        load16_lds(make_rsrc(a.shift, (long long)a.oc * 4), Pw + 512, off);
    }
    issue_window(0, 0);
    issue_b(0, 0, 0);
    issue_b(1, 0, 1);

    // fragment addresses: lane (c, g) reads half g % 2 of block g / 2 of output pixel
    // 16 tm + 4 (c % 4) + c / 4 of the wave's rows (window-relative, per column shift), and
    // weight row 4c + tn of the wave's channels
    const int c = lane & 15;
    const int g = lane >> 4;
    int abase[TM][3];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int p = m0 + kWinRows * mw + 16 * tm + 4 * (c & 3) + (c >> 2);
        const int i = fdiv(p, a.howo_mul, a.howo_shr);
        const int rem = p - i * HW;
        const int y = fdiv(rem, a.wo_mul, a.wo_shr);
        const int R0 = ((i - img0) * H2 + y - y0) * P + (rem - y * W);
#pragma unroll
        for (int kx = 0; kx < 3; ++kx) abase[tm][kx] = (g >> 1) * (kWinPx * 32) + a_swz(R0 + kx, g & 1);
    }
    int b_frag[4];
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) b_frag[tn] = ((g >> 1) * 4096 + b_swz(64 * nw + 4 * c, g & 1)) ^ (tn << 5);

    v4i acc[TM][4];

    // K-step (chunk, tap T) reads window buffer chunk % 2 and weight slot T % 3 (nine taps per
    // chunk keep the slot a compile-time constant).  Its weights were requested two steps before;
    // the next chunk's window is requested at tap 0, after that step's barrier has freed the
    // buffer.  Loads complete in order, so each wait counts what this wave requested later: the
    // next step's weights (2), and at taps 1 and 2 also the next window (kWinDma).
    // (the first step takes 0 as the MFMAs' C operand, so no accumulator is ever cleared)
    auto step = [&](auto tap, auto buf, auto first, int chunk, bool last) __attribute__((always_inline)) {
        constexpr int T = decltype(tap)::value, BUF = decltype(buf)::value;
        constexpr bool FIRST = decltype(first)::value != 0;
        if constexpr (T == 1 || T == 2) {
            if (last)
                wait_vmcnt<2>();
            else
                wait_vmcnt<2 + kWinDma>();
        } else if constexpr (T == 8) {
            if (last)
                wait_vmcnt<0>();
            else
                wait_vmcnt<2>();
        } else {
            wait_vmcnt<2>();
        }
        // every wave's part of this step has landed, and every wave's reads of step - 1 are done
        // (the compiler may sink a step's last fragment reads past the next barrier; the slot and
        // window this step refills must not be overwritten under them)
        lds_barrier();
        if constexpr (T <= 6)
            issue_b(T + 2, chunk, (T + 2) % 3);
        else if (!last)
            issue_b(T - 7, chunk + 1, (T + 2) % 3);
        if constexpr (T == 0)
            if (!last) issue_window(chunk + 1, BUF ^ 1);
        const int8_t *const win = smem + BUF * kWinBuf + (T / 3) * P * 32;  // offsets in the instructions
        const int8_t *const bst = Bs + (T % 3) * kWinStage;
        v4i bf[4], af[TM];
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) bf[tn] = *(const v4i *)(bst + b_frag[tn]);
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) af[tm] = *(const v4i *)(win + abase[tm][T % 3]);
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < 4; ++tn)
                acc[tm][tn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[tm], bf[tn],
                                                                    FIRST ? (v4i){0, 0, 0, 0} : acc[tm][tn], 0, 0, 0);
    };
    // chunks ck (window buffer 0) and ck + 1 (buffer 1)
    auto pair = [&](auto first, int ck, bool last) __attribute__((always_inline)) {
        // opaque per pair of chunks: otherwise every (buffer, tap, row group) address is hoisted out
        // of the loop into a register of its own
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
            for (int kx = 0; kx < 3; ++kx) asm volatile("" : "+v"(abase[tm][kx]));
        static_for<0, 9>([&](auto t) __attribute__((always_inline)) {
            step(t, Slot<0>(), Slot<(decltype(first)::value && decltype(t)::value == 0) ? 1 : 0>(), ck, false);
        });
        static_for<0, 9>([&](auto t) __attribute__((always_inline)) { step(t, Slot<1>(), Slot<0>(), ck + 1, last); });
    };
    const int nc = a.i1 >> 1;  // 64-channel chunks (an even number)
    pair(Slot<1>(), 0, nc <= 2);
    for (int ck = 2; ck < nc; ck += 2) pair(Slot<0>(), ck, ck + 2 >= nc);

    // every wave's fragment reads are done: the windows take the staged output tile
    lds_barrier();
    int8_t *const Rw = smem + wave * (kWinRows * 64);
    RqLane r;
    const int mode = rq_setup<false, RELU>(r, *(const v4i *)(Pw + c * 16), *(const v4i *)(Pw + 256 + c * 16),
                                           *(const v4i *)(Pw + 512 + c * 16), false, ch0 + 4 * c, a.oc);
    requant_tile_any<false, RELU, 64>(mode, acc, Rw + g * 64 + 4 * c, r);
    wave_lds_sync();

    // 16-byte stores: lane -> row 16 j + lane / 4 of the wave's pixels, channels och .. och + 15
    const int k = lane & 3;
    const int och = ch0 + 16 * k;
    const int we = (a.wo + 1) >> 1;  // the even-pixel copy: ceil(ho / 2) x ceil(wo / 2) planes
    const long long plane_e = (long long)((a.ho + 1) >> 1) * we;
    int p = m0 + kWinRows * mw + (lane >> 2);
    int b = fdiv(p, a.howo_mul, a.howo_shr), hw = p - b * HW;  // rows 16 apart: at most one image apart
#pragma unroll
    for (int j = 0; j < TM; ++j, p += 16, hw += 16) {
        if (hw >= HW) {
            hw -= HW;
            ++b;
        }
        if (p >= a.m) break;
        const v4i v = *(const v4i *)(Rw + (16 * j + (lane >> 2)) * 64 + 16 * k);
        *(v4i *)((int8_t *)a.y + (((long long)b * a.oc1 + (och >> 5)) * HW + hw) * 32 + (och & 31)) = v;
        if (a.y_even) {
            const int oy = fdiv(hw, a.wo_mul, a.wo_shr), ox = hw - oy * W;
            if (!((oy | ox) & 1))
                store16_stream(a.y_even + (((long long)b * a.oc1 + (och >> 5)) * plane_e + (oy >> 1) * we + (ox >> 1)) *
                                              32 + (och & 31),
                               v);
        }
    }
}

bool conv3x3_win_supported(const ConvArgs &a, int kh, int kw)
{
    if (kh != 3 || kw != 3 || a.stride != 1 || a.pad != 1 || a.ho != a.h || a.wo != a.w) return false;
    if (a.residual || a.out_i32 || a.in_ps || a.out_ps || a.out_even || a.ksplit > 1) return false;
    if (a.i1 % 4 != 0 || a.oc % 128 != 0 || a.oc1 * 32 != a.oc || a.o2 % 32 != 0) return false;
    if (a.w < 1 || kWinTile % a.w != 0 || a.w + 2 > 32 || a.h * a.w < 16) return false;
    const int pitch = a.w + 2 <= 16 ? 16 : 32;
    const int tr = kWinTile / a.w;
    const int segs = (tr - 1 + a.h - 1) / a.h + 1;  // most images a run of tr rows touches
    if ((tr + 2 * segs) * pitch > kWinPx) return false;
    if ((long long)segs * a.i1 * a.h * a.w * 32 >= 0x7fffffffLL) return false;
    // enough tiles for one per CU
    return (long long)(a.m + kWinTile - 1) / kWinTile * (a.oc / 128) >= 256;
}

hipError_t launch_conv3x3_win(const ConvArgs &a, hipStream_t s)
{
    const int pitch = a.w + 2 <= 16 ? 16 : 32;
    if (answer_query_even(true, "conv3x3_win_kernel<%d, %s>", pitch, tf(a.relu != 0))) return hipSuccess;
    const int tiles_n = a.oc / 128;
    const long long tiles_m = (a.m + kWinTile - 1) / kWinTile;
    const long long per = (tiles_m + 7) / 8;
    const long long grid = 8 * per * tiles_n;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const int tr = kWinTile / a.w;
    if (pitch == 16) {
        if (a.relu)
            hipLaunchKernelGGL((conv3x3_win_kernel<16, true>), dim3((unsigned)grid), dim3(256), 0, s, a, tiles_n, (int)per, tr);
        else
            hipLaunchKernelGGL((conv3x3_win_kernel<16, false>), dim3((unsigned)grid), dim3(256), 0, s, a, tiles_n, (int)per, tr);
    } else {
        if (a.relu)
            hipLaunchKernelGGL((conv3x3_win_kernel<32, true>), dim3((unsigned)grid), dim3(256), 0, s, a, tiles_n, (int)per, tr);
        else
            hipLaunchKernelGGL((conv3x3_win_kernel<32, false>), dim3((unsigned)grid), dim3(256), 0, s, a, tiles_n, (int)per, tr);
    }
    return hipGetLastError();
}

template <int KH, int KW>
hipError_t launch_ig_k(const ConvArgs &a, hipStream_t s)
{
    constexpr int ST = 2;
    const bool wide = a.oc1 * 32 > 64;
    if (KH == 3 && KW == 3 && conv3x3_win_supported(a, KH, KW)) return launch_conv3x3_win(a, s);
    if (KH == 1 && KW == 1 && conv1x1_ring_wide_supported(a)) return launch_conv1x1_ring_wide(a, s);
    if (a.residual)
        return wide ? launch_ig<KH, KW, 128, 128, ST, true, false>(a, a, s)
                    : launch_ig<KH, KW, 256, 64, ST, true, false>(a, a, s);
    // the wide 1x1 convolutions without a shortcut (K of 256..2048, few pixels per tile column)
    // run eight-wave 256x128 tiles on a three-stage ring: twice the MACs per operand byte
    if (KH == 1 && KW == 1 && wide) return launch_ig<1, 1, 256, 128, 3, false, false>(a, a, s);
    // strided 3x3 with >= 256 output channels on the plain layout: each activation DMA gathers
    // 32-byte pieces, so 128x256 tiles (eight waves) that read each activation tile once for 256
    // channels win; on the phase-split layout the runs are contiguous and 128x128 tiles are
    // faster (28x28x256: 147 -> 131 us per 1024 images)
    if (KH == 3 && a.stride == 2 && a.oc1 * 32 >= 256 && !a.in_ps)
        return launch_ig<3, 3, 128, 256, ST, false, false>(a, a, s);
    // 3x3 layers with 512 output channels, and the phase-split strided ones with 256 or more: four
    // waves of 64x128 sub-tiles on a three-stage ring (two workgroups per CU) read each activation
    // fragment for twice the MACs; 5-12 % faster there (7x7x512: 112 -> 106 us, strided 14x14x512:
    // 129 -> 113 us per 1024 images), slower for 256 channels at unit stride and for 128
    if (KH == 3 && !a.out_i32 && (a.oc1 * 32 >= 512 || (a.in_ps && a.oc1 * 32 >= 256)))
        return launch_ig<3, 3, 128, 256, 3, false, false, 128>(a, a, s);
    return wide ? launch_ig<KH, KW, 128, 128, ST, false, false>(a, a, s)
                : launch_ig<KH, KW, 256, 64, ST, false, false>(a, a, s);
}

}  // namespace

hipError_t launch_conv_proj(const ConvArgs &a, const ConvArgs &pj, hipStream_t s)
{
    if (conv1x1_proj_supported(a, pj)) return launch_conv1x1_proj(a, pj, s);
    if (conv1x1_ring_proj_supported(a, pj)) return launch_conv1x1_ring_proj(a, pj, s);
    constexpr int ST = 2;
    // 256 or more output channels and at least 2048 such tiles: 128x256 tiles of 64x128 sub-tiles
    // read each activation tile once for twice the channels, the shortcut held in registers (two
    // workgroups per CU); fewer, larger tiles lose at small batches (res5.1 at 1024 images:
    // 200 -> 182 us; at 5 images: 18 -> 24 us)
    if (a.oc1 * 32 >= 256 && (long long)((a.m + 127) / 128) * ((a.oc1 * 32 + 255) / 256) >= 2048)
        return launch_ig<1, 1, 128, 256, ST, true, true, 128>(a, pj, s);
    if (a.oc1 * 32 > 64) return launch_ig<1, 1, 128, 128, ST, true, true>(a, pj, s);
    return launch_ig<1, 1, 256, 64, ST, true, true>(a, pj, s);
}

namespace {

// ---- stride-1 3x3 over at most 64 input channels: haloed input windows ------------------------
//
// The general kernel fetches each tap's activation rows again (nine 64-byte K-steps per pixel
// for 64 input channels), so for the res2-shaped 3x3 (56x56, 64 -> 64) the activation DMA is its
// largest cost.  Here a persistent workgroup of eight waves owns one 64-channel output tile: it
// stages all nine taps of those weights (and their parameters) in LDS once, then walks a
// contiguous run of 8-row bands of whole image rows.  Each band's input window (10 rows at a
// pitch of 64 pixels, both 32-channel blocks, zero outside the image) is fetched once, into one
// of two buffers, while the previous band computes; the nine K-steps read shifted window rows.
// The window keeps the general kernel's row swizzle; with a pitch that is a multiple of 16 rows
// the kernel-row offset is a constant (2048 bytes per row), so only the three column offsets
// need swizzled base addresses, and those do not depend on the band.

constexpr int kHaloPitch = 64;                          // window row pitch (pixels), >= W + 2
constexpr int kHaloTR = 8;                              // output rows per band
constexpr int kHaloRows = (kHaloTR + 2) * kHaloPitch;  // 640 window pixels per 32-channel block
constexpr int kHaloWin = 2 * kHaloRows * 32;            // one window: 40 KB
constexpr int kHaloB = 9 * 2 * 64 * 32;                 // weights: 9 taps x 2 blocks x 64 rows, 36 KB
constexpr int kHaloLds = kHaloB + 2 * kHaloWin + 8 * 768;
constexpr int kHaloWinDma = kHaloWin / 1024 / 8;        // window DMAs per wave (5)
static_assert(kHaloWinDma * 8 * 1024 == kHaloWin, "whole window DMAs per wave");

template <bool RELU>
__global__ __launch_bounds__(512, waves_per_simd(512, 1)) void conv3x3_halo_kernel(ConvArgs a, int bands, int tiles_n, int per_wg)
{
    __shared__ __attribute__((aligned(1024))) int8_t smem[kHaloLds];
    int8_t *const WB = smem;                      // [tap][block][64 rows][32 B], slots as b_swz
    int8_t *const Win = smem + kHaloB;            // two windows [block][640 rows][32 B], slots as a_swz
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int8_t *const Pw = smem + kHaloB + 2 * kHaloWin + wave * 768;

    const int n0 = (int)(blockIdx.x % (unsigned)tiles_n) * 64;
    const int first = (int)(blockIdx.x / (unsigned)tiles_n) * per_wg;  // this workgroup's bands
    const int nbands = min(per_wg, a.n * bands - first);
    if (nbands <= 0) return;
    const int W = a.w, H = a.h, HW = H * W;
    const long long in_img = (long long)a.i1 * HW * 32;
    const long long out_img = (long long)a.oc1 * HW * 32;

    // weights and parameters of channels n0 .. n0+63, once: 36 DMAs over the eight waves
    const int wrows = ((a.oc + a.o2 - 1) / a.o2) * a.o2;
    const v4i rsB = make_rsrc(a.wt, (long long)wrows * 9 * a.i1 * 32);
    const int wblk = a.o2 * 32;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
        const int q = j * 8 + wave;
        if (q >= 36) break;
        const int tb = q >> 1, chunk = q & 1;  // (tap, block) slice and its 32-row half
        const int tap = tb >> 1, blk = tb & 1;
        const int R = n0 + chunk * 32 + dma_b_row(lane);
        const int h = dma_b_h(lane);
        const bool rok = R < wrows;
        const int RR = rok ? R : 0;
        const int o1 = fdiv(RR, a.o2_mul, a.o2_shr);
        const bool ok = rok && blk < a.i1;
        const unsigned off =
            ok ? (unsigned)(o1 * (9 * a.i1 * wblk) + (tap * a.i1 + blk) * wblk + (RR - o1 * a.o2) * 32 + h * 16) : kOOB;
        load16_lds(rsB, WB + tb * 2048 + chunk * 1024, off);
    }
    if (lane < 16) {
        const bool v = n0 + 4 * lane < a.oc;
        const unsigned off = v ? (unsigned)(n0 + 4 * lane) * 4 : kOOB;
        load16_lds(make_rsrc(a.bias, (long long)a.oc * 4), Pw, off);
        load16_lds(make_rsrc(a.mult, (long long)a.oc * 4), Pw + 256, off);
        load16_lds(make_rsrc(a.shift, (long long)a.oc * 4), Pw + 512, off);
    }

    // a band's window into buffer buf: 2 blocks x 20 DMAs of 32 rows, 5 per wave; row R is window
    // pixel (R / 64, R % 64), image pixel (y0 - 1 + R / 64, R % 64 - 1)
    auto issue_window = [&](int band_id, int buf) __attribute__((always_inline)) {
        const int b = band_id / bands;
        const int y0 = (band_id - b * bands) * kHaloTR;
        const v4i rsA = make_rsrc(a.x + (long long)b * in_img, in_img);
        int8_t *const dst = Win + buf * kHaloWin;
#pragma unroll
        for (int j = 0; j < kHaloWinDma; ++j) {
            const int q = j * 8 + wave;
            const int blk = q / 20, chunk = q - blk * 20;
            const int R = chunk * 32 + dma_a_row(lane);
            const int h = dma_a_h(lane);
            const int y = y0 - 1 + (R >> 6), x = (R & 63) - 1;
            const bool ok = blk < a.i1 && (unsigned)y < (unsigned)H && (unsigned)x < (unsigned)W;
            const unsigned off = ok ? (unsigned)((blk * HW + y * W + x) * 32 + h * 16) : kOOB;
            load16_lds(rsA, dst + blk * (kHaloRows * 32) + chunk * 1024, off);
        }
    };

    // fragment addresses (band-independent): lane (c, g) reads half g % 2 of block g / 2 at
    // window pixel R0 + 64 ky + kx of its output pixel m = 64 wave + 16 tm + 4 (c % 4) + c / 4
    // of the band (rows past the band repeat its last row; they are never stored)
    const int c = lane & 15;
    const int g = lane >> 4;
    const int wm0 = wave * 64;
    const int m_band = kHaloTR * W;  // <= 496
    int abase[4][3];
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
        const int m = min(wm0 + 16 * tm + 4 * (c & 3) + (c >> 2), m_band - 1);
        const int oy = fdiv(m, a.wo_mul, a.wo_shr);
        const int R0 = oy * kHaloPitch + (m - oy * W);
#pragma unroll
        for (int kx = 0; kx < 3; ++kx) abase[tm][kx] = (g >> 1) * (kHaloRows * 32) + a_swz(R0 + kx, g & 1);
    }
    int bfr[4];
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) bfr[tn] = ((g >> 1) * 2048 + b_swz(4 * c, g & 1)) ^ (tn << 5);
    const int k = lane & 3;
    const int och = n0 + 16 * k;  // first channel of this lane's 16-byte output chunk

    issue_window(first, 0);
    for (int i = 0; i < nbands; ++i) {
        const int buf = i & 1;
        // the other buffer's last readers (band i-1's staging) are behind this barrier
        if (i > 0) ring_barrier();
        if (i + 1 < nbands) {
            issue_window(first + i + 1, buf ^ 1);
            wait_vmcnt<kHaloWinDma>();  // all but the next window's DMAs have landed
        } else {
            wait_vmcnt<0>();
        }
        ring_barrier();  // ... for every wave: band i's window (and the weights) are visible
        const int8_t *const win = Win + buf * kHaloWin;
        v4i acc[4][4];
#pragma unroll
        for (int ky = 0; ky < 3; ++ky)
#pragma unroll
            for (int kx = 0; kx < 3; ++kx) {
                const int8_t *wb = WB + (ky * 3 + kx) * 4096;
                v4i bf[4];
#pragma unroll
                for (int tn = 0; tn < 4; ++tn) bf[tn] = *(const v4i *)(wb + bfr[tn]);
#pragma unroll
                for (int tm = 0; tm < 4; ++tm) {
                    const v4i af = *(const v4i *)(win + abase[tm][kx] + 2048 * ky);
#pragma unroll
                    for (int tn = 0; tn < 4; ++tn)
                        acc[tm][tn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                            af, bf[tn], (ky == 0 && kx == 0) ? (v4i){0, 0, 0, 0} : acc[tm][tn], 0, 0, 0);
                }
            }
        // every wave's fragment reads of this window are done (waited for: the compiler may leave
        // the last ones in flight here): it takes the 4 KB staging tiles
        lds_barrier();
        int8_t *const Rw = (int8_t *)win + wave * 4096;
        requant_to_lds<false, RELU, true>(acc, Rw + g * 64 + 4 * c, Pw, c, n0 + 4 * c, a.oc);
        wave_lds_sync();
        // 16-byte stores: lane -> band row 16 j + lane / 4, channels och .. och + 15
        const int band_id = first + i;
        const int b = band_id / bands;
        const int y0 = (band_id - b * bands) * kHaloTR;
        const int m_valid = min(kHaloTR, H - y0) * W;
        if (och < a.oc1 * 32) {
            int8_t *const yb = (int8_t *)a.y + (long long)b * out_img + ((long long)(och >> 5) * HW + y0 * W) * 32 +
                               (och & 31);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * j + (lane >> 2);
                if (wm0 + r < m_valid) *(v4i *)(yb + (long long)(wm0 + r) * 32) = *(const v4i *)(Rw + r * 64 + 16 * k);
            }
        }
    }
}

bool conv3x3_halo_supported(const ConvArgs &a, int kh, int kw)
{
    return kh == 3 && kw == 3 && a.stride == 1 && a.pad == 1 && a.i1 <= 2 && a.w >= 48 && a.w + 2 <= kHaloPitch &&
           !a.residual && !a.out_i32 && a.ksplit <= 1 && a.ho == a.h && a.wo == a.w;
}

// Persistent grid: one eight-wave workgroup per CU (its LDS leaves room for no second one), in
// groups of tiles_n (one per 64-channel output tile), each group taking an equal contiguous run
// of bands.
static_assert(2 * kHaloLds > kLdsBytes, "one haloed-window workgroup per CU");

hipError_t launch_conv3x3_halo(const ConvArgs &a, hipStream_t s)
{
    if (answer_query("conv3x3_halo_kernel<%s>", tf(a.relu != 0))) return hipSuccess;
    int slots = 0;
    hipError_t e = current_cus(&slots);
    if (e != hipSuccess) return e;
    const int bands = (a.h + kHaloTR - 1) / kHaloTR;
    const int tiles_n = (a.oc1 * 32 + 63) / 64;
    const long long total = (long long)a.n * bands;  // bands of the whole batch
    if (total <= 0) return hipSuccess;
    if (total > 0x7ffffff0LL) return hipErrorInvalidConfiguration;
    if ((long long)a.i1 * a.h * a.w * 32 >= 0x7fffffffLL) return hipErrorInvalidValue;
    long long groups = slots / tiles_n;
    if (groups < 1) groups = 1;
    if (groups > total) groups = total;
    const int per_wg = (int)((total + groups - 1) / groups);
    groups = (total + per_wg - 1) / per_wg;
    const dim3 grid((unsigned)(groups * tiles_n));
    if (a.relu)
        hipLaunchKernelGGL(conv3x3_halo_kernel<true>, grid, dim3(512), 0, s, a, bands, tiles_n, per_wg);
    else
        hipLaunchKernelGGL(conv3x3_halo_kernel<false>, grid, dim3(512), 0, s, a, bands, tiles_n, per_wg);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv(const ConvArgs &a, int kh, int kw, hipStream_t s)
{
    if (conv3x3_halo_supported(a, kh, kw)) return launch_conv3x3_halo(a, s);
    if (conv1x1_small_k_supported(a, kh, kw)) return launch_conv1x1_small_k(a, s);
    if (kh == 1 && kw == 1) return launch_ig_k<1, 1>(a, s);
    if (kh == 3 && kw == 3) return launch_ig_k<3, 3>(a, s);
    return hipErrorInvalidValue;
}

// ---- split-K: few output tiles, long reduction (the batch-1 layers) ----------------------------

namespace {

// Output tile of the general kernel for `a` without a shortcut (the partial launch drops it).
void partial_tile(const ConvArgs &a, int kh, int kw, int *bm, int *bn)
{
    const bool wide = a.oc1 * 32 > 64;
    *bm = wide ? 128 : 256;
    *bn = wide ? 128 : 64;
    if (kh == 1 && kw == 1 && wide) {
        *bm = 256;
        *bn = 128;
    } else if (kh == 3 && a.stride == 2 && a.oc1 * 32 >= 256) {
        *bm = 128;
        *bn = 256;
    }
}

// Number of K parts for `a` (1: no split) and the 32-channel blocks per part (even).  A launch
// with fewer than 64 output tiles and at least 16 K-steps is split into at most 16 parts of at
// least two K-steps, aiming at 256 workgroups, while the int32 partial sums fit in 8 MB.
int split_count(const ConvArgs &a, int kh, int kw, int *kb_per)
{
    // the reduction kernel writes the plain layout
    if (a.out_ps || conv1x1_small_k_supported(a, kh, kw) || (a.oc & 3) != 0) return 1;
    if (!((kh == 1 && kw == 1) || (kh == 3 && kw == 3))) return 1;
    int bm, bn;
    partial_tile(a, kh, kw, &bm, &bn);
    const long long tiles = (long long)((a.m + bm - 1) / bm) * ((a.oc1 * 32 + bn - 1) / bn);
    const int nsteps = (a.nkb + 1) / 2;
    if (tiles >= 64 || nsteps < 16) return 1;
    long long parts = (256 + tiles - 1) / tiles;
    if (parts > nsteps / 2) parts = nsteps / 2;
    if (parts > 16) parts = 16;
    const int per = 2 * (int)((nsteps + parts - 1) / parts);
    const int n = (a.nkb + per - 1) / per;
    if (n < 2 || (long long)n * a.m * a.oc * 4 > (8LL << 20)) return 1;
    *kb_per = per;
    return n;
}

// Sum of the K parts, bias, then the epilogue of `a`: fixed-point requantisation, shortcut, ReLU
// and saturation into the NC/32HW32 output (padding channels of a 32-channel block written as
// 0), or the int32 sums for an int32 output.  An item is one pixel and 4 channels; a workgroup
// takes 64 items, its four waves summing every fourth part with 16-byte loads, wave 0 adding
// the three other waves' sums from LDS.  Requires Oc % 4 == 0 (16-byte aligned part rows).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(ConvArgs a, const int32_t *part, int parts)
{
    __shared__ v4i red[3][64];
    const int groups = a.out_i32 ? a.oc >> 2 : a.oc1 * 8;
    const int t = threadIdx.x & 63, pl = threadIdx.x >> 6;
    const int idx = blockIdx.x * 64 + t;
    const bool live = idx < a.m * groups;
    const int p = live ? idx / groups : 0;
    const int ch = (idx - p * groups) * 4;
    const bool real = live && ch < a.oc;
    v4i acc = {0, 0, 0, 0};
    if (real) {
        const long long slice = (long long)a.m * a.oc;
        const int32_t *src = part + (long long)p * a.oc + ch;
#pragma unroll 4
        for (int q = pl; q < parts; q += 4) acc += *(const v4i *)(src + q * slice);
    }
    if (pl) red[pl - 1][t] = acc;
    __syncthreads();
    if (pl || !live) return;
    acc += red[0][t] + red[1][t] + red[2][t];
    if (a.out_i32) {
        const v4i b = {a.bias[ch], a.bias[ch + 1], a.bias[ch + 2], a.bias[ch + 3]};
        *(v4i *)((int32_t *)a.y + (long long)p * a.oc + ch) = acc + b;
        return;
    }
    const int HoWo = a.ho * a.wo;
    const int b = p / HoWo, hw = p - b * HoWo;
    const long long off = (((long long)b * a.oc1 + (ch >> 5)) * HoWo + hw) * 32 + (ch & 31);
    int v[4] = {0, 0, 0, 0};
    if (real) {
        const unsigned rr = a.residual ? *(const unsigned *)(a.res + off) : 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int r = requant_any(acc[j] + a.bias[ch + j], a.mult[ch + j], a.shift[ch + j]);
            if (a.residual) r += (int)(signed char)(rr >> (8 * j));
            if (a.relu) r = max(r, 0);
            v[j] = min(max(r, -128), 127);
        }
    }
    *(unsigned *)((int8_t *)a.y + off) = pack4(v[0], v[1], v[2], v[3]);
}

}  // namespace

bool conv_phase_supported(const ConvArgs &a, int kh, int kw)
{
    if (a.in_ps && !(kh == 3 && kw == 3 && a.stride == 2 && a.pad == 1 && !(a.h & 1) && !(a.w & 1))) return false;
    if (a.out_ps && (((a.ho | a.wo) & 1) || a.out_i32)) return false;
    // only the general kernel reads and writes the phase-split layout
    if (conv3x3_halo_supported(a, kh, kw) || conv1x1_small_k_supported(a, kh, kw)) return false;
    if (a.out_ps) {  // and a launch that would be split over K keeps its split (batch-1 latency)
        ConvArgs q = a;
        q.out_ps = 0;
        int per = 0;
        if (split_count(q, kh, kw, &per) > 1) return false;
    }
    return true;
}

size_t splitk_bytes(const ConvArgs &a, int kh, int kw)
{
    int per = 0;
    const int n = split_count(a, kh, kw, &per);
    return n > 1 ? (((size_t)n * a.m * a.oc * 4 + 255) & ~(size_t)255) : 0;
}

hipError_t launch_conv_split(const ConvArgs &a, int kh, int kw, int32_t *part, size_t part_bytes, hipStream_t s)
{
    int per = 0;
    const int n = part ? split_count(a, kh, kw, &per) : 1;
    if (n <= 1 || (size_t)n * a.m * a.oc * 4 > part_bytes) return launch_conv(a, kh, kw, s);
    ConvArgs q = a;  // the partial launch: int32 sums of each K part, no shortcut, no bias
    q.out_i32 = 1;
    q.residual = 0;
    q.res = nullptr;
    q.relu = 0;
    q.y = part;
    q.ksplit = n;
    q.kb_per = per;
    hipError_t e = kh == 1 ? launch_ig_k<1, 1>(q, s) : launch_ig_k<3, 3>(q, s);
    if (e != hipSuccess) return e;
    if (armed_query()) return hipSuccess;  // the partial launch named the kernel
    const long long items = (long long)a.m * (a.out_i32 ? a.oc / 4 : a.oc1 * 8);
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((items + 63) / 64)), dim3(256), 0, s, a, part, n);
    return hipGetLastError();
}

}  // namespace ifx
