// 1x1 convolutions with at most 128 input channels: one output tile per
// workgroup, every operand of the tile requested at once.
//
// Same computation as the implicit-GEMM core (Inspur conv-merge article,
// sections 3.3-3.4: data[M,K] . weight[N,K]^T, then BN + Sum + ReLU on the
// accumulators), for the layers where K = Ic <= 128 is only one or two
// 64-byte K-steps.  Those layers are HBM-bound (res2 conv3 and projection,
// res3 conv3 of ResNet-50: ~100 ops per byte) and their tiles are short, so a
// persistent pipeline spends most of each tile waiting for the shortcut it
// needs a step later.  Here instead:
//   * a workgroup owns one BM x BN output tile and issues, at its start, the
//     DMA of all its activation and weight K-steps into LDS, then the
//     shortcut and per-channel parameters of each wave's 64x64 part;
//   * LDS use is small (35-52 KB), so 3-4 workgroups share a CU and one
//     workgroup's epilogue overlaps the others' loads;
//   * tiles are numbered so that the N-tiles of one activation tile run back
//     to back on one XCD, reading the activation tile from HBM once;
//   * operand layout, MFMA tiling and epilogue are those of the general
//     kernel (64-byte XOR-swizzled LDS rows, v_mfma_i32_16x16x64_i8, 4
//     consecutive output channels per lane, exact fixed-point requant,
//     16-byte stores of whole NC/32HW32 chunks).
#include "device_common.h"
#include "ifx_internal.h"

namespace ifx {
namespace {

template <int BM, int BN, int NST>
struct C1Cfg {
    static constexpr int WAVES_M = BM / 64;
    static constexpr int WAVES = WAVES_M * (BN / 64);
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int AI = BM * 64 / 16 / THREADS;  // activation loads per thread per K-step
    static constexpr int BI = BN * 64 / 16 / THREADS;  // weight loads per thread per K-step
    static_assert(AI * THREADS * 16 == BM * 64 && BI * THREADS * 16 == BN * 64, "whole 16-byte loads");
    static constexpr int STAGE = (BM + BN) * 64;
    static constexpr int LDS = NST * STAGE + BM * BN + WAVES * 768;  // stages | staging | params
    static constexpr int WG_PER_CU = kLdsBytes / LDS > 4 ? 4 : kLdsBytes / LDS;
    static constexpr int TILE_IN = 4 + 3;  // per-wave shortcut and parameter DMAs (with a shortcut)
};

// Issue the DMAs of all NST K-steps of `q`'s operands for output tile (m0, n0) into `stages`
// (NST stages of (BM + BN) x 64 bytes, activations then weights).
template <int BM, int BN, int NST>
__device__ __forceinline__ void issue_operands(const ConvArgs &q, int8_t *stages, int m0, int n0, int wave, int lane)
{
    using C = C1Cfg<BM, BN, NST>;
    constexpr int NWV = C::WAVES;
    const int HoWo = q.ho * q.wo;
    const int HW = q.h * q.w;
    const long long in_img = (long long)q.i1 * HW * 32;
    const int img0 = fdiv(m0, q.howo_mul, q.howo_shr);
    // activations: instruction j of wave w fills rows [(j*NWV + w)*16, +16) of a stage; lane l ->
    // row (j*NWV + w)*16 + l/4, physical chunk l%4 holding logical chunk (l%4)^swz(row)
    const v4i rsA = make_rsrc(q.x + (long long)img0 * in_img, (long long)(q.n - img0) * in_img);
#pragma unroll
    for (int j = 0; j < C::AI; ++j) {
        const int row = (j * NWV + wave) * 16 + (lane >> 2);
        const int lch = (lane & 3) ^ swz(row);
        const int sel = lch >> 1;  // which 32-channel block of the step
        const int p = m0 + row;
        const bool ok = p < q.m;
        const int pp = ok ? p : m0;
        const int b = fdiv(pp, q.howo_mul, q.howo_shr);
        const int rem = pp - b * HoWo;
        const int oy = fdiv(rem, q.wo_mul, q.wo_shr);
        const int ox = rem - oy * q.wo;
        const unsigned base = (unsigned)((long long)(b - img0) * in_img) + (unsigned)(sel * HW * 32) +
                              (unsigned)((oy * q.stride * q.w + ox * q.stride) * 32) + (lch & 1) * 16;
#pragma unroll
        for (int s = 0; s < NST; ++s) {
            const bool v = ok && 2 * s + sel < q.i1;
            load16_lds(rsA, stages + s * C::STAGE + (j * NWV + wave) * 1024,
                       v ? base + (unsigned)(2 * s * HW * 32) : kOOB);
        }
    }
    // weights: physical row r of a 64-row group holds output channel (r%16)*4 + r/16
    const int wrows = ((q.oc + q.o2 - 1) / q.o2) * q.o2;
    const v4i rsB = make_rsrc(q.wt, (long long)wrows * q.i1 * 32);
#pragma unroll
    for (int j = 0; j < C::BI; ++j) {
        const int prow = (j * NWV + wave) * 16 + (lane >> 2);
        const int lch = (lane & 3) ^ swz(prow);
        const int sel = lch >> 1;
        const int o = (prow & ~63) + (prow & 15) * 4 + ((prow & 63) >> 4);
        const int rw = n0 + o;
        const bool ok = rw < wrows;
        const int o1 = fdiv(ok ? rw : 0, q.o2_mul, q.o2_shr);
        const int o2i = (ok ? rw : 0) - o1 * q.o2;
        const unsigned base = (unsigned)(((o1 * q.i1 + sel) * q.o2 + o2i) * 32) + (lch & 1) * 16;
#pragma unroll
        for (int s = 0; s < NST; ++s) {
            const bool v = ok && 2 * s + sel < q.i1;
            load16_lds(rsB, stages + s * C::STAGE + BM * 64 + (j * NWV + wave) * 1024,
                       v ? base + (unsigned)(2 * s * q.o2 * 32) : kOOB);
        }
    }
}

// Bias, multipliers and shifts of channels ch0 .. ch0+63 into a wave's 768-byte region: 3 DMAs.
__device__ __forceinline__ void issue_params(const ConvArgs &q, int8_t *Pw, int ch0, int lane)
{
    if (lane < 16) {
        const bool v = ch0 + 4 * lane < q.oc;
        const unsigned off = v ? (unsigned)(ch0 + 4 * lane) * 4 : kOOB;
        load16_lds(make_rsrc(q.bias, (long long)q.oc * 4), Pw, off);
        load16_lds(make_rsrc(q.mult, (long long)q.oc * 4), Pw + 256, off);
        load16_lds(make_rsrc(q.shift, (long long)q.oc * 4), Pw + 512, off);
    }
}

// The wave's 64x64 part of the contraction over NST landed stages (zero C on the first step).
template <int BM, int BN, int NST>
__device__ __forceinline__ void contract(const int8_t *stages, v4i (&acc)[4][4], int wm0, int wn0, int lane)
{
    using C = C1Cfg<BM, BN, NST>;
    const int c = lane & 15;
    const int g = lane >> 4;
#pragma unroll
    for (int s = 0; s < NST; ++s) {
        const int8_t *st = stages + s * C::STAGE;
        v4i af[4], bf[4];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
            const int r = lane & 15;
            const int row = wm0 + 16 * tm + 4 * (r & 3) + (r >> 2);
            af[tm] = *(const v4i *)(st + row * 64 + ((g ^ swz(row)) << 4));
        }
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) {
            const int row = wn0 + 16 * tn + c;
            bf[tn] = *(const v4i *)(st + BM * 64 + row * 64 + ((g ^ swz(row)) << 4));
        }
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
#pragma unroll
            for (int tn = 0; tn < 4; ++tn)
                acc[tm][tn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[tm], bf[tn],
                                                                    s == 0 ? (v4i){0, 0, 0, 0} : acc[tm][tn], 0, 0, 0);
    }
}

// 16-byte stores of a wave's staged 64 pixels x 64 channels (Rw: [64 rows][64 B]) into the
// NC/32HW32 output, non-temporal when NT.
template <bool NT>
__device__ __forceinline__ void store_wave_tile(const ConvArgs &a, const int8_t *Rw, int m0, int wm0, int ch0,
                                                int lane)
{
    int8_t *y = (int8_t *)a.y;
    const int HoWo = a.ho * a.wo;
    const int k = lane & 3;
    const int och = ch0 + 16 * k;  // first channel of this lane's chunk
    if (och >= a.oc1 * 32) return;
    const int pbase = m0 + wm0;
    if (pbase >= a.m) return;
    const int b0 = fdiv(pbase, a.howo_mul, a.howo_shr);
    const int hw0 = pbase - b0 * HoWo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int prow = 16 * j + (lane >> 2);
        if (pbase + prow >= a.m) break;
        int b = b0, hw = hw0 + prow;
        while (hw >= HoWo) {
            hw -= HoWo;
            ++b;
        }
        const v4i v = *(const v4i *)(Rw + prow * 64 + 16 * k);
        int8_t *dst = y + (((long long)b * a.oc1 + (och >> 5)) * HoWo + hw) * 32 + (och & 31);
        if (NT)
            store16_stream(dst, v);
        else
            *(v4i *)dst = v;
    }
}

template <int BM, int BN, int NST, bool RES, bool RELU>
__global__ __launch_bounds__((C1Cfg<BM, BN, NST>::THREADS), (waves_per_simd(C1Cfg<BM, BN, NST>::THREADS, C1Cfg<BM, BN, NST>::WG_PER_CU)))
void conv1x1_kernel(ConvArgs a, int tiles_n)
{
    using C = C1Cfg<BM, BN, NST>;
    __shared__ __attribute__((aligned(1024))) int8_t smem[C::LDS];
    int8_t *const R = smem + NST * C::STAGE;  // per wave: [64 rows][64 B] shortcut in, output out
    int8_t *const Pm = R + BM * BN;           // per wave: bias, mult, shift of its 64 channels

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave % C::WAVES_M) * 64;
    const int wn0 = (wave / C::WAVES_M) * 64;
    int8_t *const Rw = R + wave * 4096;
    int8_t *const Pw = Pm + wave * 768;

    // tile: workgroup k of XCD x (blockIdx = 8k + x) takes M-tile 8 (k / tiles_n) + x, N-tile k % tiles_n
    const int xcd = blockIdx.x & 7;
    const int kk = blockIdx.x >> 3;
    const int mt = (kk / tiles_n) * 8 + xcd;
    const int m0 = mt * BM;
    if (m0 >= a.m) return;
    const int n0 = (kk - (kk / tiles_n) * tiles_n) * BN;

    const int HoWo = a.ho * a.wo;
    const long long out_img = (long long)a.oc1 * HoWo * 32;
    const int img0 = fdiv(m0, a.howo_mul, a.howo_shr);
    issue_operands<BM, BN, NST>(a, smem, m0, n0, wave, lane);
    // ---- this wave's shortcut tile and parameters (always 7 DMAs with a shortcut, 3 without)
    const int ch0 = n0 + wn0;
    issue_params(a, Pw, ch0, lane);
    if (RES) {
        const v4i rsR = make_rsrc(a.res + (long long)img0 * out_img, (long long)(a.n - img0) * out_img);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int p = m0 + wm0 + 16 * j + (lane >> 2);
            const int oc = ch0 + (lane & 3) * 16;
            unsigned off = kOOB;
            if (p < a.m && oc < a.oc1 * 32) {
                const int b = fdiv(p, a.howo_mul, a.howo_shr), hw = p - b * HoWo;
                off = (unsigned)((((long long)(b - img0) * a.oc1 + (oc >> 5)) * HoWo + hw) * 32 + (oc & 31));
            }
            load16_lds_stream(rsR, Rw + j * 1024, off);
        }
    }

    // ---- contraction: operands landed once only the shortcut/parameter DMAs remain
    if (RES)
        wait_vmcnt<C::TILE_IN>();
    else
        wait_vmcnt<3>();
    ring_barrier();
    const int c = lane & 15;
    const int g = lane >> 4;
    // the first K-step's MFMAs take 0 as their C operand: no accumulator is cleared
    v4i acc[4][4];
    contract<BM, BN, NST>(smem, acc, wm0, wn0, lane);

    // ---- epilogue: this wave's own shortcut and parameters (no other wave's data)
    wait_vmcnt<0>();
    const int ocl = ch0 + 4 * c;  // first of this lane's four output channels
    RqLane r;
    const int mode = rq_setup<RES, RELU>(r, *(const v4i *)(Pw + c * 16), *(const v4i *)(Pw + 256 + c * 16),
                                         *(const v4i *)(Pw + 512 + c * 16), false, ocl, a.oc);
    requant_tile_any<RES, RELU, 64>(mode, acc, Rw + g * 64 + 4 * c, r);
    wave_lds_sync();

    // 16-byte stores of the wave's 64 pixels x 64 channels; with a shortcut stream, both streams
    // go non-temporal (measured faster); without, plain stores
    store_wave_tile<RES>(a, Rw, m0, wm0, ch0, lane);
}

// ---- conv3 of a bottleneck fused with its 1x1 projection shortcut, both with K <= 128 ----
//
// y = ReLU(requant(conv3(t)) + requant(proj(x))) for one output tile per workgroup: the
// operands of both convolutions (every K-step) and both parameter sets are requested at tile
// start; the projection's accumulators are requantised (no ReLU) into 16 registers per lane,
// which then take conv3's contraction, and the final epilogue adds the shortcut bytes from
// those registers: the MFMA layout gives the lane that produced a shortcut value the same pixel
// and channels in conv3's tile.  The shortcut never reaches LDS or HBM.
template <int BM, int BN, int NSP, int NSA>
struct C1PCfg {
    using C = C1Cfg<BM, BN, 1>;
    static constexpr int WAVES = C::WAVES;
    static constexpr int THREADS = C::THREADS;
    static constexpr int STAGE = C::STAGE;
    static constexpr int LDS = (NSP + NSA) * STAGE + WAVES * 1536;  // stages | params (conv3, projection)
    static constexpr int WG_PER_CU = kLdsBytes / LDS > 4 ? 4 : kLdsBytes / LDS;
    // each wave stages its 64x64 output over the projection's stages, which no wave reads
    // once every wave has passed the barrier in front of conv3's contraction
    static_assert(WAVES * 4096 <= NSP * STAGE, "staging fits the projection stages");
};

template <int BM, int BN, int NSP, int NSA, bool RELU>
__global__ __launch_bounds__((C1PCfg<BM, BN, NSP, NSA>::THREADS),
                              (waves_per_simd(C1PCfg<BM, BN, NSP, NSA>::THREADS, C1PCfg<BM, BN, NSP, NSA>::WG_PER_CU)))
void conv1x1_proj_kernel(ConvArgs a, ConvArgs pj, int tiles_n)
{
    using P = C1PCfg<BM, BN, NSP, NSA>;
    using C = C1Cfg<BM, BN, 1>;
    __shared__ __attribute__((aligned(1024))) int8_t smem[P::LDS];
    int8_t *const SP = smem;                               // projection stages, later the output staging
    int8_t *const SA = smem + NSP * P::STAGE;              // conv3 stages
    int8_t *const Pm = smem + (NSP + NSA) * P::STAGE;      // per wave: conv3 parameters, projection's

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave % C::WAVES_M) * 64;
    const int wn0 = (wave / C::WAVES_M) * 64;
    int8_t *const Pw = Pm + wave * 1536;
    int8_t *const Pp = Pw + 768;

    // tile: workgroup k of XCD x (blockIdx = 8k + x) takes M-tile 8 (k / tiles_n) + x, N-tile k % tiles_n
    const int xcd = blockIdx.x & 7;
    const int kk = blockIdx.x >> 3;
    const int mt = (kk / tiles_n) * 8 + xcd;
    const int m0 = mt * BM;
    if (m0 >= a.m) return;
    const int n0 = (kk - (kk / tiles_n) * tiles_n) * BN;
    const int ch0 = n0 + wn0;

    // projection first (it is consumed first), then conv3: (AI + BI) x NSA + 3 DMAs after the
    // projection's operands and parameters
    issue_operands<BM, BN, NSP>(pj, SP, m0, n0, wave, lane);
    issue_params(pj, Pp, ch0, lane);
    issue_operands<BM, BN, NSA>(a, SA, m0, n0, wave, lane);
    issue_params(a, Pw, ch0, lane);

    const int c = lane & 15;
    const int g = lane >> 4;
    const int ocl = ch0 + 4 * c;  // first of this lane's four output channels
    v4i acc[4][4];
    unsigned sc[4][4];
    wait_vmcnt<(C::AI + C::BI) * NSA + 3>();
    ring_barrier();
    contract<BM, BN, NSP>(SP, acc, wm0, wn0, lane);
    {
        RqLane r;
        const int mode = rq_setup<false, false>(r, *(const v4i *)(Pp + c * 16), *(const v4i *)(Pp + 256 + c * 16),
                                                *(const v4i *)(Pp + 512 + c * 16), false, ocl, pj.oc);
        requant_regs_any(mode, acc, r, sc);
    }
    wait_vmcnt<0>();
    ring_barrier();
    contract<BM, BN, NSA>(SA, acc, wm0, wn0, lane);
    RqLane r;
    const int mode = rq_setup<true, RELU>(r, *(const v4i *)(Pw + c * 16), *(const v4i *)(Pw + 256 + c * 16),
                                          *(const v4i *)(Pw + 512 + c * 16), false, ocl, a.oc);
    int8_t *const Rw = SP + wave * 4096;
    requant_tile_sc_any<RELU, 64>(mode, acc, Rw + g * 64 + 4 * c, r, sc);
    wave_lds_sync();
    store_wave_tile<false>(a, Rw, m0, wm0, ch0, lane);
}

template <int BM, int BN, int NSP, int NSA>
hipError_t launch_1x1_proj(const ConvArgs &a, const ConvArgs &pj, hipStream_t s)
{
    if (answer_query("conv1x1_proj_kernel<%d, %d, %d, %d, %s>", BM, BN, NSP, NSA, tf(a.relu != 0))) return hipSuccess;
    using P = C1PCfg<BM, BN, NSP, NSA>;
    const int tiles_n = (a.oc1 * 32 + BN - 1) / BN;
    const long long tiles_m = (a.m + BM - 1) / BM;
    const long long grid = (tiles_m + 7) / 8 * 8 * tiles_n;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (a.relu)
        hipLaunchKernelGGL((conv1x1_proj_kernel<BM, BN, NSP, NSA, true>), dim3((unsigned)grid), dim3(P::THREADS), 0, s,
                           a, pj, tiles_n);
    else
        hipLaunchKernelGGL((conv1x1_proj_kernel<BM, BN, NSP, NSA, false>), dim3((unsigned)grid), dim3(P::THREADS), 0,
                           s, a, pj, tiles_n);
    return hipGetLastError();
}

template <int BM, int BN>
hipError_t launch_1x1_proj_k(const ConvArgs &a, const ConvArgs &pj, hipStream_t s)
{
    if (pj.i1 <= 2)
        return a.i1 <= 2 ? launch_1x1_proj<BM, BN, 1, 1>(a, pj, s) : launch_1x1_proj<BM, BN, 1, 2>(a, pj, s);
    return a.i1 <= 2 ? launch_1x1_proj<BM, BN, 2, 1>(a, pj, s) : launch_1x1_proj<BM, BN, 2, 2>(a, pj, s);
}

template <int BM, int BN, int NST, bool RES>
hipError_t launch_1x1(const ConvArgs &a, hipStream_t s)
{
    if (answer_query("conv1x1_kernel<%d, %d, %d, %s, %s>", BM, BN, NST, tf(RES), tf(a.relu != 0))) return hipSuccess;
    using C = C1Cfg<BM, BN, NST>;
    const int tiles_n = (a.oc1 * 32 + BN - 1) / BN;
    const long long tiles_m = (a.m + BM - 1) / BM;
    const long long grid = (tiles_m + 7) / 8 * 8 * tiles_n;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (a.relu)
        hipLaunchKernelGGL((conv1x1_kernel<BM, BN, NST, RES, true>), dim3((unsigned)grid), dim3(C::THREADS), 0, s, a,
                           tiles_n);
    else
        hipLaunchKernelGGL((conv1x1_kernel<BM, BN, NST, RES, false>), dim3((unsigned)grid), dim3(C::THREADS), 0, s,
                           a, tiles_n);
    return hipGetLastError();
}

template <int BM, int BN, int NST>
hipError_t launch_1x1_res(const ConvArgs &a, hipStream_t s)
{
    return a.residual ? launch_1x1<BM, BN, NST, true>(a, s) : launch_1x1<BM, BN, NST, false>(a, s);
}


// ---- conv3 of one bottleneck chained with conv1 of the next (256-channel block output) ----
//
// y  = ReLU(requant(conv3(t2)) + shortcut)          the block output, stored (the next block's
//                                                    shortcut) and kept in LDS
// t1 = [ReLU](requant(conv1'(y)))                   the next block's first convolution
// The Inspur conv-merge article (section 2.1) merges consecutive operators so that the tensor
// passed between them is neither written by one nor read back by the other; here y is still
// written (the next block adds it as its shortcut) but conv1' reads it from LDS, saving one full
// read of the block output.  Persistent workgroups of four waves walk 64-pixel tiles:
//   * both convolutions' weights live in registers for the whole launch (conv3: 16 bytes x 4 per
//     lane, conv1': 16 bytes x 4 K-steps per 16 output channels), as do their parameters;
//   * a ring of kChainNB LDS buffers holds each tile's activations (64 x 64 bytes) and shortcut
//     (four 64 x 64 byte regions, one per wave's 64 channels, in the XOR-swizzled row layout of
//     an MFMA operand); the DMAs of the tiles kChainNB - 2 ahead stay in flight while a tile is
//     computed, which is what keeps HBM busy: a tile carries ~40 KB of traffic and ~2 us of work;
//   * phase 1 (each wave 64 pixels x 64 channels, K <= 64) requantises in place, turning its
//     shortcut region into y; those four regions are exactly conv1''s four 64-byte K-steps;
//   * phase 2 multiplies with the weights as the row operand (each wave N1/4 channels x 64
//     pixels), so a lane ends with 4 (N1 = 64) or 8 (N1 = 128) consecutive channels of one pixel
//     and stores them straight from registers.
// With PROJ the block's shortcut is its 1x1 projection (the first block of a stage, Inspur article
// section 2.2): a slot holds the projection's input tile (64 pixels x K <= 64) instead of the
// shortcut, each wave computes the projection of its 64 channels, requantises it (no ReLU) into
// registers and adds it in conv3's epilogue, as the fused projection kernel does; y is staged in
// one region after the ring (conv1' with 64 output channels only: the projection's weights and
// parameters take the registers that 128 would need).
// The block output has 64 NW channels (NW waves: 256 at res2, 512 at res3); conv3 has KS 64-byte
// K-steps (K <= 64 NW / 4 ... 128).
constexpr int kChainA = 4096;  // one K-step of a tile's conv3 input (or projection input): [64 rows][64 B]

template <int NW, int KS, bool PROJ>
struct ChainLay {
    // slot: KS K-steps of conv3 activations + the NW shortcut / y regions; y is computed in place
    static constexpr int SLOT = KS * kChainA + NW * 4096;
    static constexpr int NB = 4;                     // ring depth (tiles resident in LDS)
    static constexpr int PER_CU = NW == 4 ? 2 : 1;   // resident workgroups per CU
    static constexpr int ADMA = KS * 4 / NW;         // activation DMAs per wave per tile
    static constexpr int DMA = ADMA + 4;             // + 4 shortcut DMAs
    static constexpr int LDS = NB * SLOT;
    static_assert(ADMA >= 1 && ADMA * NW == KS * 4, "every wave issues the same DMAs");
};
template <>
struct ChainLay<4, 1, true> {
    // slot: conv3 activations + projection input; y in one region after the ring
    static constexpr int SLOT = 2 * kChainA;
    static constexpr int NB = 6;
    static constexpr int PER_CU = 2;
    static constexpr int ADMA = 1;
    static constexpr int DMA = 2;  // 1 activation, 1 projection input
    static constexpr int LDS = NB * SLOT + 4 * 4096;
};
static_assert(2 * ChainLay<4, 1, false>::LDS <= kLdsBytes && 2 * ChainLay<4, 1, true>::LDS <= kLdsBytes &&
                  ChainLay<8, 2, false>::LDS <= kLdsBytes,
              "ring fits the LDS");

// Physical LDS byte of logical 16-byte chunk k of row r in a [rows][64 B] swizzled region.
__device__ __forceinline__ int swz_at(int r, int k) { return r * 64 + ((k ^ swz(r)) << 4); }

// Where a 64-pixel tile starts (unit stride, so input and output pixels coincide): first pixel
// m0, its image img0 and position hw0 in that image, the image size and the per-image byte
// counts of a packed tensor with c1 channel blocks (c1 * HoWo * 32).  All wave-uniform.
struct TileOrg {
    int m0, img0, hw0, HoWo;
};

__device__ __forceinline__ TileOrg tile_org(const ConvArgs &a, int m0)
{
    TileOrg t;
    t.m0 = m0;
    t.HoWo = a.ho * a.wo;
    t.img0 = fdiv(m0, a.howo_mul, a.howo_shr);
    t.hw0 = m0 - t.img0 * t.HoWo;
    return t;
}

// Pixel m0 + r (0 <= r < 64) of the tile: image img0 + d, position hw.  Images of at least 64
// pixels take one conditional subtraction; smaller ones a short loop.
__device__ __forceinline__ void split_px(const TileOrg &t, int r, int &d, int &hw)
{
    hw = t.hw0 + r;
    d = 0;
    if (t.HoWo >= 64) {
        if (hw >= t.HoWo) {
            hw -= t.HoWo;
            d = 1;
        }
    } else {
        while (hw >= t.HoWo) {
            hw -= t.HoWo;
            ++d;
        }
    }
}

// Rows 16 grp .. +15 of K-step ks (32-channel blocks 2 ks, 2 ks + 1, zero past q.i1) of a 64-pixel
// tile of q's input into a [64 rows][64 B] swizzled region: one DMA.
__device__ __forceinline__ void tile_rows_issue(const ConvArgs &q, const TileOrg &t, int8_t *dst, int grp, int ks,
                                                int lane)
{
    const unsigned plane = (unsigned)t.HoWo * 32;  // bytes of one 32-channel block of an image
    const unsigned in_img = (unsigned)q.i1 * plane;
    const v4i rs = make_rsrc(q.x + (long long)t.img0 * in_img, (long long)(q.n - t.img0) * in_img);
    const int row = 16 * grp + (lane >> 2);
    const int lch = (lane & 3) ^ swz(row);  // logical chunk: input channels 64 ks + 16 lch .. +15
    const int blk = 2 * ks + (lch >> 1);
    int d, hw;
    split_px(t, row, d, hw);
    const bool ok = t.m0 + row < q.m && blk < q.i1;
    const unsigned off = (unsigned)d * in_img + (unsigned)blk * plane + (unsigned)hw * 32 + (lch & 1) * 16;
    load16_lds_stream(rs, dst + grp * 1024, ok ? off : kOOB);
}

// This wave's DMAs of the tile at pixel m0 (m0 >= a.m: every load is out of range, so the
// slot fills with zeros and the count of DMAs stays the same): conv3 activation rows 16 wave ..
// +15 into the slot's first 4 KB, then the shortcut bytes of channels 64 wave .. +63 into the
// wave's region or, with PROJ, the projection input's rows into the second 4 KB.
template <int NW, int KS, bool PROJ>
__device__ __forceinline__ void chain_issue(const ConvArgs &a, const ConvArgs &pj, int8_t *buf, int m0, int wave,
                                            int lane)
{
    using L = ChainLay<NW, KS, PROJ>;
    const TileOrg t = tile_org(a, m0);
    const unsigned plane = (unsigned)t.HoWo * 32;
#pragma unroll
    for (int j = 0; j < L::ADMA; ++j) {  // 16-row group q % 4 of K-step q / 4
        const int q = j * NW + wave;
        tile_rows_issue(a, t, buf + (q >> 2) * kChainA, q & 3, q >> 2, lane);
    }
    if (PROJ) {
        tile_rows_issue(pj, t, buf + kChainA, wave, 0, lane);
        return;
    }
    {
        const unsigned out_img = (unsigned)a.oc1 * plane;
        const v4i rsR = make_rsrc(a.res + (long long)t.img0 * out_img, (long long)(a.n - t.img0) * out_img);
        int8_t *const Rw = buf + KS * kChainA + wave * 4096;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 16 * j + (lane >> 2);
            const int k = (lane & 3) ^ swz(row);  // logical chunk: channels 64 wave + 16k .. +15
            const int oc = 64 * wave + 16 * k;
            int d, hw;
            split_px(t, row, d, hw);
            const unsigned off = (unsigned)d * out_img + (unsigned)(oc >> 5) * plane + (unsigned)hw * 32 + (oc & 31);
            load16_lds_stream(rsR, Rw + j * 1024, m0 + row < a.m ? off : kOOB);
        }
    }
}

// 16 weight bytes of output channel o, reduction bytes 16 kc .. +15 (zero past the input
// channels), from the [o1][i1][o2][32] layout of a 1x1 convolution.
__device__ __forceinline__ v4i chain_weights(const ConvArgs &q, int o, int kc)
{
    const int kb = kc >> 1;
    if (kb >= q.i1) return (v4i){0, 0, 0, 0};
    const int o1 = fdiv(o, q.o2_mul, q.o2_shr), o2i = o - o1 * q.o2;
    return *(const v4i *)(q.wt + ((long long)(o1 * q.i1 + kb) * q.o2 + o2i) * 32 + (kc & 1) * 16);
}

// Phase 2's output channel for row r (0..15) of channel tile mt of a wave that owns CPW conv1'
// channels: CPW = 16 gives it 16 consecutive channels; CPW = 32 gives it 32 (one 32-channel block)
// with rows ordered so that accumulator row 4g + i of tiles 0 and 1 are channels 8g + i and
// 8g + 4 + i.
template <int CPW>
__device__ __forceinline__ int chain_ch2(int wave, int mt, int r)
{
    static_assert(CPW == 16 || CPW == 32, "16 or 32 conv1' channels per wave");
    return CPW == 16 ? 16 * wave + r : 32 * wave + 8 * (r >> 2) + 4 * mt + (r & 3);
}

template <int NW, int KS, int N1, bool RELU1, bool EVEN, bool PROJ>
__global__ __launch_bounds__(64 * NW, (waves_per_simd(64 * NW, ChainLay<NW, KS, PROJ>::PER_CU))) void conv1x1_chain_kernel(ConvArgs a,
                                                                                                   ConvArgs b,
                                                                                                   ConvArgs pj,
                                                                                                   int tiles)
{
    using L = ChainLay<NW, KS, PROJ>;
    constexpr int CPW = N1 / NW;   // conv1' channels per wave
    constexpr int MT2 = CPW / 16;  // phase-2 channel tiles per wave
    __shared__ __attribute__((aligned(1024))) int8_t smem[L::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, g = lane >> 4;
    const int ch0 = 64 * wave;  // this wave's phase-1 channels
    const int HoWo = a.ho * a.wo;
    const int first = blockIdx.x;
    if (first >= tiles) return;
    const int ntile = (tiles - 1 - first) / (int)gridDim.x + 1;

    // ---- weights and parameters into registers (before any DMA, so their waits are short)
    v4i w3[KS][4];  // phase-1 column operand: lane (c, g), tile tn -> channel ch0 + 4c + tn, bytes 64s + 16g ..
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) w3[s][tn] = chain_weights(a, ch0 + 4 * c + tn, 4 * s + g);
    v4i w1[MT2][NW];  // phase-2 row operand: lane (c, g), K-step s -> channel chain_ch2(c), bytes 64s + 16g ..
#pragma unroll
    for (int mt = 0; mt < MT2; ++mt)
#pragma unroll
        for (int s = 0; s < NW; ++s) w1[mt][s] = chain_weights(b, chain_ch2<CPW>(wave, mt, c), 4 * s + g);
    RqPacked r1;
    int mode1;
    {
        RqLane r;
        mode1 = rq_setup<true, true>(r, *(const v4i *)(a.bias + ch0 + 4 * c), *(const v4i *)(a.mult + ch0 + 4 * c),
                                     *(const v4i *)(a.shift + ch0 + 4 * c), false, ch0 + 4 * c, a.oc);
        r1 = rq_pack(r, mode1);
    }
    v4i wp[4];  // the projection's weights, as w3 (PROJ only)
    RqPacked rpj;
    int modep = 0;
    if (PROJ) {
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) wp[tn] = chain_weights(pj, ch0 + 4 * c + tn, g);
        RqLane r;
        modep = rq_setup<false, false>(r, *(const v4i *)(pj.bias + ch0 + 4 * c), *(const v4i *)(pj.mult + ch0 + 4 * c),
                                       *(const v4i *)(pj.shift + ch0 + 4 * c), false, ch0 + 4 * c, pj.oc);
        rpj = rq_pack(r, modep);
    }
    RqPacked r2[MT2];
    int mode2 = 1;
    {
        RqLane r[MT2];
#pragma unroll
        for (int mt = 0; mt < MT2; ++mt) {
            const int cb = chain_ch2<CPW>(wave, mt, 4 * g);  // the lane's 4 consecutive channels
            const int md = rq_setup<false, RELU1>(r[mt], *(const v4i *)(b.bias + cb), *(const v4i *)(b.mult + cb),
                                                  *(const v4i *)(b.shift + cb), false, cb, b.oc);
            mode2 = (md == 0 || mode2 == 0) ? 0 : (md == 1 && mode2 == 1 ? 1 : 2);  // valid for both sets
        }
#pragma unroll
        for (int mt = 0; mt < MT2; ++mt) r2[mt] = rq_pack(r[mt], mode2);
    }

    // ---- ring prologue: tiles 0 .. NB-2 (tiles past the end load zeros)
    auto tile_m0 = [&](int j) { const int t = first + j * (int)gridDim.x; return t < tiles ? t * 64 : a.m; };
#pragma unroll
    for (int j = 0; j < L::NB - 1; ++j) chain_issue<NW, KS, PROJ>(a, pj, smem + j * L::SLOT, tile_m0(j), wave, lane);

    for (int j = 0; j < ntile; ++j) {
        int8_t *const buf = smem + (j % L::NB) * L::SLOT;
        const int m0 = tile_m0(j);
        // exactly NB - 2 tiles were issued after this one; loads land in issue order, so this
        // leaves only theirs in flight (pending stores only make the wait longer)
        wait_vmcnt<(L::NB - 2) * L::DMA>();
        ring_barrier();  // tile j visible to every wave; every wave is done with tile j - 1
        chain_issue<NW, KS, PROJ>(a, pj, smem + ((j + L::NB - 1) % L::NB) * L::SLOT, tile_m0(j + L::NB - 1), wave,
                                  lane);

        // ---- phase 1: conv3, 64 pixels x this wave's 64 channels, one K-step, in two halves of
        //      32 pixels (half the accumulators live at a time)
        int8_t *const Rb = PROJ ? smem + L::NB * L::SLOT : buf + KS * kChainA;  // the NW y regions
        int8_t *const Rw = Rb + wave * 4096;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            v4i acc[4][4];  // rows 2h, 2h+1 of the 16-row tiles used
            // lane (g, c) holds rows 16 tm + 4 i + g, channels 4c .. 4c+3 (logical chunk c / 4 of
            // the row); the shortcut words of those rows: the projection's, requantised into
            // registers, or the DMA'd shortcut bytes, which y then overwrites in place
            unsigned rr[2][4];
            if (PROJ) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int tm = 2 * h + t;
                    const v4i af = *(const v4i *)(buf + kChainA + swz_at(16 * tm + 4 * (c & 3) + (c >> 2), g));
#pragma unroll
                    for (int tn = 0; tn < 4; ++tn)
                        acc[t][tn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, wp[tn], (v4i){0, 0, 0, 0}, 0, 0, 0);
                }
                auto rqp = [&](auto md) __attribute__((always_inline)) {
                    constexpr int MD = decltype(md)::value;
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int i = 0; i < 4; ++i) rr[t][i] = requant_row_p<MD, false, false>(acc, t, i, rpj, 0u);
                };
                if (modep == 0)
                    rqp(Slot0());
                else if (modep == 1)
                    rqp(Slot1());
                else
                    rqp(Slot2());
            } else {
                // every shortcut word first: the reads overlap, not read-wait-write
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        rr[t][i] = *(const unsigned *)(Rw + swz_at(16 * (2 * h + t) + 4 * i + g, c >> 2) + 4 * (c & 3));
            }
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int tm = 2 * h + t;
                    const v4i af = *(const v4i *)(buf + s * kChainA + swz_at(16 * tm + 4 * (c & 3) + (c >> 2), g));
#pragma unroll
                    for (int tn = 0; tn < 4; ++tn)
                        acc[t][tn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, w3[s][tn],
                                                                           s == 0 ? (v4i){0, 0, 0, 0} : acc[t][tn],
                                                                           0, 0, 0);
                }
            auto rq = [&](auto md) __attribute__((always_inline)) {
                constexpr int MD = decltype(md)::value;
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        *(unsigned *)(Rw + swz_at(16 * (2 * h + t) + 4 * i + g, c >> 2) + 4 * (c & 3)) =
                            requant_row_p<MD, true, true>(acc, t, i, r1, rr[t][i]);
            };
            if (mode1 == 0)
                rq(Slot0());
            else if (mode1 == 1)
                rq(Slot1());
            else
                rq(Slot2());
        }
        lds_barrier();  // y complete in all four regions

        // y (the block output) to HBM: the wave's region, 16-byte chunks; with EVEN only the
        // pixels at even rows and columns, into a tensor of half the height and width (rounded up)
        const TileOrg to = tile_org(a, m0);
        {
            const int k = lane & 3;
            const int och = ch0 + 16 * k;
            const int ho2 = (a.ho + 1) >> 1, wo2 = (a.wo + 1) >> 1;
            const unsigned plane = (unsigned)(EVEN ? ho2 * wo2 : to.HoWo) * 32;
            const unsigned out_img = (unsigned)a.oc1 * plane;
            int8_t *const ybase = (int8_t *)a.y + (long long)to.img0 * out_img;
            v4i v[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) v[jj] = *(const v4i *)(Rw + swz_at(16 * jj + (lane >> 2), k));
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int row = 16 * jj + (lane >> 2);
                int d, hw;
                split_px(to, row, d, hw);
                bool ok = m0 + row < a.m;
                unsigned pix = (unsigned)hw;
                if (EVEN) {
                    const int oy = fdiv(hw, a.wo_mul, a.wo_shr), ox = hw - oy * a.wo;
                    ok = ok && ((oy | ox) & 1) == 0;
                    pix = (unsigned)((oy >> 1) * wo2 + (ox >> 1));
                }
                if (ok)
                    store16_stream(ybase + ((unsigned)d * out_img + (unsigned)(och >> 5) * plane + pix * 32 + (och & 31)),
                                   v[jj]);
            }
        }

        // ---- phase 2: conv1' = W1 . y^T, this wave's CPW channels x 64 pixels, K = 64 NW (the
        //      NW regions); lane (c, g) gets channels chain_ch2(4g .. 4g+3) of pixel 16 pg + c
        v4i acc2[4][MT2];
#pragma unroll
        for (int s = 0; s < NW; ++s) {
            const int8_t *const Rs = Rb + s * 4096;
#pragma unroll
            for (int pg = 0; pg < 4; ++pg) {
                const v4i bf = *(const v4i *)(Rs + swz_at(16 * pg + c, g));
#pragma unroll
                for (int mt = 0; mt < MT2; ++mt)
                    acc2[pg][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w1[mt][s], bf,
                                                                         s == 0 ? (v4i){0, 0, 0, 0} : acc2[pg][mt], 0, 0, 0);
            }
        }
        {
            const int cb = chain_ch2<CPW>(wave, 0, 4 * g);
            const unsigned plane = (unsigned)to.HoWo * 32;
            const unsigned t1_img = (unsigned)b.oc1 * plane;
            int8_t *const t1 = (int8_t *)b.y + (long long)to.img0 * t1_img + (unsigned)(cb >> 5) * plane + (cb & 31);
            auto rq2 = [&](auto md) __attribute__((always_inline)) {
                constexpr int MD = decltype(md)::value;
#pragma unroll
                for (int pg = 0; pg < 4; ++pg) {
                    const int row = 16 * pg + c;
                    if (m0 + row < b.m) {
                        int d, hw;
                        split_px(to, row, d, hw);
                        unsigned pix = (unsigned)hw;
                        if (b.out_ps) {  // phase-split t1: the pixel's parity plane, then its place
                            const int oy = fdiv(hw, a.wo_mul, a.wo_shr), ox = hw - oy * a.wo;
                            pix = (unsigned)(((oy & 1) * 2 + (ox & 1)) * (to.HoWo >> 2) + (oy >> 1) * (a.wo >> 1) +
                                             (ox >> 1));
                        }
                        int8_t *dst = t1 + ((unsigned)d * t1_img + pix * 32);
                        if (MT2 == 1) {
                            *(unsigned *)dst = requant_quad_p<MD, RELU1>(acc2[pg][0], r2[0]);
                        } else {
                            const unsigned lo = requant_quad_p<MD, RELU1>(acc2[pg][0], r2[0]);
                            const unsigned hi = requant_quad_p<MD, RELU1>(acc2[pg][MT2 - 1], r2[MT2 - 1]);
                            *(uint2 *)dst = make_uint2(lo, hi);
                        }
                    }
                }
            };
            if (mode2 == 0)
                rq2(Slot0());
            else if (mode2 == 1)
                rq2(Slot1());
            else
                rq2(Slot2());
        }
    }
    wait_vmcnt<0>();  // the ring's last (zero-fill) DMAs land before the workgroup's LDS is released
}

template <int NW, int KS, int N1, bool RELU1, bool EVEN, bool PROJ>
hipError_t launch_chain_k(const ConvArgs &a, const ConvArgs &b, const ConvArgs &pj, long long tiles, hipStream_t s)
{
    using L = ChainLay<NW, KS, PROJ>;
    int cus = 0;
    const hipError_t e = current_cus(&cus);
    if (e != hipSuccess) return e;
    const long long slots = (long long)L::PER_CU * cus;
    const long long grid = tiles < slots ? tiles : slots;
    hipLaunchKernelGGL((conv1x1_chain_kernel<NW, KS, N1, RELU1, EVEN, PROJ>), dim3((unsigned)grid), dim3(64 * NW), 0,
                       s, a, b, pj, (int)tiles);
    return hipGetLastError();
}

template <int NW, int KS, int N1, bool PROJ>
hipError_t launch_chain_flags(const ConvArgs &a, const ConvArgs &b, const ConvArgs &pj, long long tiles,
                              hipStream_t s)
{
    const bool relu = b.relu != 0, even = a.out_even != 0;
    if constexpr (PROJ) {  // the projection's block output is read whole by the next block
        if (even) return hipErrorInvalidValue;
    } else {
        if (even)
            return relu ? launch_chain_k<NW, KS, N1, true, true, PROJ>(a, b, pj, tiles, s)
                        : launch_chain_k<NW, KS, N1, false, true, PROJ>(a, b, pj, tiles, s);
    }
    return relu ? launch_chain_k<NW, KS, N1, true, false, PROJ>(a, b, pj, tiles, s)
                : launch_chain_k<NW, KS, N1, false, false, PROJ>(a, b, pj, tiles, s);
}

// The instances: 256-channel block outputs (four waves, conv3 K <= 64) chained with a conv1 to 64
// or 128 channels, with the projection (conv1 to 64) or without; 512-channel block outputs (eight
// waves, conv3 K <= 128) chained with a conv1 to 128 channels.  pj: the block's projection (conv3's
// shortcut computed in the kernel) or null (DMA'd shortcut).
hipError_t launch_chain(const ConvArgs &a, const ConvArgs &b, const ConvArgs *pj, hipStream_t s)
{
    const int nw = a.oc / 64, ks = a.i1 <= 2 && nw == 4 ? 1 : 2;
    const bool relu = b.relu != 0, even = a.out_even != 0, proj = pj != nullptr;
    if (answer_query("conv1x1_chain_kernel<%d, %d, %d, %s, %s, %s>", nw, ks, b.oc, tf(relu), tf(even), tf(proj)))
        return hipSuccess;
    const long long tiles = (a.m + 63) / 64;
    if (tiles <= 0) return hipSuccess;
    if (tiles > 0x7fffffffLL / 64) return hipErrorInvalidConfiguration;
    if (nw == 4 && ks == 1) {
        if (proj) return b.oc == 64 ? launch_chain_flags<4, 1, 64, true>(a, b, *pj, tiles, s) : hipErrorInvalidValue;
        if (b.oc == 64) return launch_chain_flags<4, 1, 64, false>(a, b, a, tiles, s);
        if (b.oc == 128) return launch_chain_flags<4, 1, 128, false>(a, b, a, tiles, s);
    }
    if (nw == 8 && ks == 2 && !proj && b.oc == 128) return launch_chain_flags<8, 2, 128, false>(a, b, a, tiles, s);
    return hipErrorInvalidValue;
}


// ---- 1x1 with a shortcut, K <= 128, 256 or 512 output channels: persistent, ring-buffered ----
//
// The same layers as conv1x1_kernel (res3 conv3, the 28x28x128 -> 512 fused layer, unchained res2
// conv3), walked by persistent workgroups the way the chained kernel walks its tiles: one wave per
// 64 output channels holds its weights (KS x 4 x 16 bytes per lane) and parameters in registers
// for the whole launch, and a ring of NB LDS buffers, each a 64-pixel tile's activations (KS
// 64-byte K-steps) and shortcut (one 64 x 64-byte region per wave), keeps NB - 2 tiles of DMA in
// flight while one is computed.  The shortcut region is requantised in place and stored from
// there by its own wave, so a tile needs one barrier.  These layers read and write ~60 KB of HBM
// per 64-pixel tile for ~1.5 MOP of MFMA work: the bytes in flight, not the arithmetic, set the
// rate.
// KP > 0: the layer's shortcut is its 1x1 projection (stride 1, KP K-steps; the first block of a
// stage, whose stride-2 input the previous block stored subsampled): a slot holds the projection's
// input tile instead of the shortcut, each wave requantises the projection of its 64 channels (no
// ReLU) into registers and adds it in the epilogue, and y is staged in one region per wave after
// the ring.
template <int NW, int KS, int KP = 0, int TR = 64>
struct RingCfg {
    static constexpr int KB = TR * 64;                   // one K-step of a tile: [TR rows][64 B]
    static constexpr int A = KS * KB;                    // activations
    static constexpr int X = KP * KB;                    // projection input
    static constexpr int BUF = A + (KP ? X : NW * KB);   // + shortcut / output, one region per wave
    static constexpr int YST = KP ? NW * KB : 0;         // output staging after the ring (projection)
    static constexpr int PER_CU = NW == 4 ? 2 : 1;
    static constexpr int AVAIL = kLdsBytes / PER_CU - YST;
    static constexpr int NBMAX = (KP || TR == 32) ? 6 : 4;
    static constexpr int NB = AVAIL / BUF > NBMAX ? NBMAX : AVAIL / BUF;
    static constexpr int GRPS = TR / 16;                 // 16-row groups of a tile (1 KB DMAs per K-step)
    static constexpr int ADMA = KS * GRPS / NW;          // activation DMAs per wave per tile
    static constexpr int XDMA = KP * GRPS / NW;          // projection-input DMAs per wave per tile
    static constexpr int DMA = ADMA + (KP ? XDMA : GRPS);  // (+ the shortcut DMAs without a projection)
    static constexpr int LDS = NB * BUF + YST;
    static_assert(TR == 64 || (TR == 32 && KP == 0), "32-pixel tiles without a projection only");
    static_assert(ADMA >= 1 && ADMA * NW == KS * GRPS, "every wave issues the same DMAs");
    static_assert(XDMA * NW == KP * GRPS, "every wave issues the same DMAs");
    static_assert(NB >= 3, "a ring of at least three tiles");
};

// soc: the first output channel of the workgroup's slice
template <int NW, int KS, int KP, int TR>
__device__ __forceinline__ void ring_issue(const ConvArgs &a, const ConvArgs &pj, int8_t *buf, int m0, int wave,
                                           int lane, int soc)
{
    using C = RingCfg<NW, KS, KP, TR>;
    const TileOrg t = tile_org(a, m0);
    const unsigned plane = (unsigned)t.HoWo * 32;
#pragma unroll
    for (int j = 0; j < C::ADMA; ++j) {  // 16-row group q % GRPS of K-step q / GRPS
        const int q = j * NW + wave;
        tile_rows_issue(a, t, buf + (q / C::GRPS) * C::KB, q % C::GRPS, q / C::GRPS, lane);
    }
    if (KP) {
#pragma unroll
        for (int j = 0; j < C::XDMA; ++j) {
            const int q = j * NW + wave;
            tile_rows_issue(pj, t, buf + C::A + (q / C::GRPS) * C::KB, q % C::GRPS, q / C::GRPS, lane);
        }
        return;
    }
    {
        const unsigned out_img = (unsigned)a.oc1 * plane;
        const v4i rsR = make_rsrc(a.res + (long long)t.img0 * out_img, (long long)(a.n - t.img0) * out_img);
        int8_t *const Rw = buf + C::A + wave * C::KB;
#pragma unroll
        for (int j = 0; j < C::GRPS; ++j) {
            const int row = 16 * j + (lane >> 2);
            const int k = (lane & 3) ^ swz(row);
            const int oc = soc + 64 * wave + 16 * k;
            int d, hw;
            split_px(t, row, d, hw);
            const unsigned off = (unsigned)d * out_img + (unsigned)(oc >> 5) * plane + (unsigned)hw * 32 + (oc & 31);
            load16_lds_stream(rsR, Rw + j * 1024, m0 + row < a.m ? off : kOOB);
        }
    }
}

template <int NW, int KS, int KP, int TR, bool RELU>
__global__ __launch_bounds__(64 * NW, (waves_per_simd(64 * NW, RingCfg<NW, KS, KP, TR>::PER_CU))) void conv1x1_ring_kernel(ConvArgs a,
                                                                                               ConvArgs pj,
                                                                                               int tiles, int slices)
{
    using C = RingCfg<NW, KS, KP, TR>;
    __shared__ __attribute__((aligned(1024))) int8_t smem[C::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, g = lane >> 4;
    // slices > 1 (no projection): workgroup b owns output channels [64 NW (b % slices), +64 NW)
    // and walks tiles b / slices, + gridDim.x / slices, ...
    const int slice = (int)(blockIdx.x % (unsigned)slices);
    const int soc = slice * 64 * NW;
    const int ch0 = soc + 64 * wave;
    const int first = (int)(blockIdx.x / (unsigned)slices);
    const int gstride = (int)(gridDim.x / (unsigned)slices);
    if (first >= tiles) return;
    const int ntile = (tiles - 1 - first) / gstride + 1;

    // weights (column operand: lane (c, g), tile tn -> channel ch0 + 4c + tn, K-step s bytes
    // 64s + 16g ..) and parameters into registers, before any DMA
    v4i w[KS][4];
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) w[s][tn] = chain_weights(a, ch0 + 4 * c + tn, 4 * s + g);
    RqPacked rp;
    int mode;
    {
        RqLane r;
        mode = rq_setup<true, RELU>(r, *(const v4i *)(a.bias + ch0 + 4 * c), *(const v4i *)(a.mult + ch0 + 4 * c),
                                    *(const v4i *)(a.shift + ch0 + 4 * c), false, ch0 + 4 * c, a.oc);
        rp = rq_pack(r, mode);
    }
    v4i wp[KP ? KP : 1][4];  // the projection's weights (KP > 0)
    RqPacked rpj;
    int modep = 0;
    if (KP) {
#pragma unroll
        for (int s = 0; s < KP; ++s)
#pragma unroll
            for (int tn = 0; tn < 4; ++tn) wp[s][tn] = chain_weights(pj, ch0 + 4 * c + tn, 4 * s + g);
        RqLane r;
        modep = rq_setup<false, false>(r, *(const v4i *)(pj.bias + ch0 + 4 * c), *(const v4i *)(pj.mult + ch0 + 4 * c),
                                       *(const v4i *)(pj.shift + ch0 + 4 * c), false, ch0 + 4 * c, pj.oc);
        rpj = rq_pack(r, modep);
    }

    auto tile_m0 = [&](int j) { const int t = first + j * gstride; return t < tiles ? t * TR : a.m; };
#pragma unroll
    for (int j = 0; j < C::NB - 1; ++j)
        ring_issue<NW, KS, KP, TR>(a, pj, smem + j * C::BUF, tile_m0(j), wave, lane, soc);

    int8_t *y = (int8_t *)a.y;
    const int k4 = lane & 3;
    const int och = ch0 + 16 * k4;  // this lane's 16-byte output chunk
    for (int j = 0; j < ntile; ++j) {
        int8_t *const buf = smem + (j % C::NB) * C::BUF;
        const int m0 = tile_m0(j);
        wait_vmcnt<(C::NB - 2) * C::DMA>();  // tile j landed (loads complete in issue order)
        ring_barrier();                        // ... for every wave; every wave is done with tile j - 1
        ring_issue<NW, KS, KP, TR>(a, pj, smem + ((j + C::NB - 1) % C::NB) * C::BUF, tile_m0(j + C::NB - 1),
                                   wave, lane, soc);

        // the wave's output region: its shortcut bytes in the slot (requantised in place), or its
        // own staging region after the ring
        int8_t *const Rw = KP ? smem + C::NB * C::BUF + wave * C::KB : buf + C::A + wave * C::KB;
        auto contract = [&](v4i (&acc)[4][4], const int8_t *src, const v4i (*wt)[4], int steps, int tm)
            __attribute__((always_inline)) {
#pragma unroll
            for (int s = 0; s < steps; ++s) {
                const v4i af = *(const v4i *)(src + s * C::KB + swz_at(16 * tm + 4 * (c & 3) + (c >> 2), g));
#pragma unroll
                for (int tn = 0; tn < 4; ++tn)
                    acc[tm & 1][tn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, wt[s][tn], s == 0 ? (v4i){0, 0, 0, 0}
                                                                                                   : acc[tm & 1][tn],
                                                                            0, 0, 0);
            }
        };
        auto store_rows = [&](auto md, const v4i (&acc)[4][4], int tm, const unsigned *rr)
            __attribute__((always_inline)) {
            constexpr int MD = decltype(md)::value;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *(unsigned *)(Rw + swz_at(16 * tm + 4 * i + g, c >> 2) + 4 * (c & 3)) =
                    requant_row_p<MD, true, RELU>(acc, tm & 1, i, rp, rr[i]);
        };
        if constexpr (KP > 0) {
            // one 16-pixel row block at a time: the projection, requantised into shortcut words, then
            // conv3 (keeps the live accumulators to one block)
#pragma unroll
            for (int tm = 0; tm < 4; ++tm) {
                v4i acc[4][4];
                unsigned rr[4];
                contract(acc, buf + C::A, wp, KP, tm);
                auto rqp = [&](auto md) __attribute__((always_inline)) {
                    constexpr int MD = decltype(md)::value;
#pragma unroll
                    for (int i = 0; i < 4; ++i) rr[i] = requant_row_p<MD, false, false>(acc, tm & 1, i, rpj, 0u);
                };
                if (modep == 0)
                    rqp(Slot0());
                else if (modep == 1)
                    rqp(Slot1());
                else
                    rqp(Slot2());
                contract(acc, buf, w, KS, tm);
                if (mode == 0)
                    store_rows(Slot0(), acc, tm, rr);
                else if (mode == 1)
                    store_rows(Slot1(), acc, tm, rr);
                else
                    store_rows(Slot2(), acc, tm, rr);
            }
        } else {
#pragma unroll
            for (int h = 0; h < TR / 32; ++h) {  // halves of 32 pixels
                v4i acc[4][4];
                unsigned rr[2][4];  // the shortcut words of rows 16 (2h + t) + 4i + g, channels 4c ..
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        rr[t][i] = *(const unsigned *)(Rw + swz_at(16 * (2 * h + t) + 4 * i + g, c >> 2) + 4 * (c & 3));
#pragma unroll
                for (int s = 0; s < KS; ++s)
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const int tm = 2 * h + t;
                        const v4i af = *(const v4i *)(buf + s * C::KB + swz_at(16 * tm + 4 * (c & 3) + (c >> 2), g));
#pragma unroll
                        for (int tn = 0; tn < 4; ++tn)
                            acc[t][tn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, w[s][tn], s == 0 ? (v4i){0, 0, 0, 0}
                                                                                                     : acc[t][tn], 0, 0, 0);
                    }
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    if (mode == 0)
                        store_rows(Slot0(), acc, 2 * h + t, rr[t]);
                    else if (mode == 1)
                        store_rows(Slot1(), acc, 2 * h + t, rr[t]);
                    else
                        store_rows(Slot2(), acc, 2 * h + t, rr[t]);
                }
            }
        }
        wave_lds_sync();  // the wave's own region: no other wave reads it
        v4i v[C::GRPS];
#pragma unroll
        for (int jj = 0; jj < C::GRPS; ++jj) v[jj] = *(const v4i *)(Rw + swz_at(16 * jj + (lane >> 2), k4));
        const TileOrg to = tile_org(a, m0);
        const unsigned plane = (unsigned)to.HoWo * 32;
        const unsigned out_img = (unsigned)a.oc1 * plane;
        int8_t *const ybase = y + (long long)to.img0 * out_img + (unsigned)(och >> 5) * plane + (och & 31);
        // the even-pixel copy (y_even): its plane is ceil(ho / 2) x ceil(wo / 2)
        const int we = (a.wo + 1) >> 1;
        const unsigned plane_e = (unsigned)(((a.ho + 1) >> 1) * we) * 32;
        const unsigned img_e = (unsigned)a.oc1 * plane_e;
        int8_t *const ebase =
            a.y_even ? a.y_even + (long long)to.img0 * img_e + (unsigned)(och >> 5) * plane_e + (och & 31) : nullptr;
#pragma unroll
        for (int jj = 0; jj < C::GRPS; ++jj) {
            const int row = 16 * jj + (lane >> 2);
            if (m0 + row < a.m) {
                int d, hw;
                split_px(to, row, d, hw);
                store16_stream(ybase + ((unsigned)d * out_img + (unsigned)hw * 32), v[jj]);
                if (ebase) {
                    const int oy = fdiv(hw, a.wo_mul, a.wo_shr), ox = hw - oy * a.wo;
                    if (!((oy | ox) & 1))
                        store16_stream(ebase + ((unsigned)d * img_e + (unsigned)((oy >> 1) * we + (ox >> 1)) * 32),
                                       v[jj]);
                }
            }
        }
    }
    wait_vmcnt<0>();  // the ring's last (zero-fill) DMAs land before the workgroup's LDS is released
}

// pj: the projection (KP > 0) or `a` itself (unused); TR: pixels per tile (64, or 32 for a
// deeper ring)
template <int NW, int KS, int KP, int TR = 64>
hipError_t launch_ring(const ConvArgs &a, const ConvArgs &pj, hipStream_t s)
{
    using C = RingCfg<NW, KS, KP, TR>;
    if (answer_query_even(KP == 0, "conv1x1_ring_kernel<%d, %d, %d, %d, %s>", NW, KS, KP, TR, tf(a.relu != 0)))
        return hipSuccess;
    const long long tiles = (a.m + TR - 1) / TR;
    if (tiles <= 0) return hipSuccess;
    if (tiles > 0x7fffffffLL / TR) return hipErrorInvalidConfiguration;
    int cus = 0;
    const hipError_t e = current_cus(&cus);
    if (e != hipSuccess) return e;
    // output-channel slices of 64 NW channels (one without a projection's fixed pairing)
    const int slices = KP ? 1 : a.oc / (64 * NW);
    if (!KP && (slices < 1 || slices * 64 * NW != a.oc)) return hipErrorInvalidValue;
    const long long slots = (long long)C::PER_CU * cus / slices * slices;
    const long long want = tiles * slices;
    long long grid = want < slots ? want : slots;
    if (grid < slices) grid = slices;
    if (a.relu)
        hipLaunchKernelGGL((conv1x1_ring_kernel<NW, KS, KP, TR, true>), dim3((unsigned)grid), dim3(64 * NW), 0, s,
                           a, pj, (int)tiles, slices);
    else
        hipLaunchKernelGGL((conv1x1_ring_kernel<NW, KS, KP, TR, false>), dim3((unsigned)grid), dim3(64 * NW), 0, s,
                           a, pj, (int)tiles, slices);
    return hipGetLastError();
}

}  // namespace

bool conv1x1_small_k_supported(const ConvArgs &a, int kh, int kw)
{
    return kh == 1 && kw == 1 && a.pad == 0 && !a.out_i32 && a.i1 <= 4;
}

// conv3 + projection in one small-K launch: both 1x1 with K <= 128, conv3 unit stride (the
// projection's stride is free), the same output pixels and channels.
bool conv1x1_proj_supported(const ConvArgs &a, const ConvArgs &pj)
{
    return a.i1 <= 4 && pj.i1 <= 4 && a.stride == 1 && a.pad == 0 && pj.pad == 0 && !a.out_i32 && !pj.out_i32 &&
           a.m == pj.m && a.oc == pj.oc && a.ho == pj.ho && a.wo == pj.wo && a.n == pj.n;
}

hipError_t launch_conv1x1_proj(const ConvArgs &a, const ConvArgs &pj, hipStream_t s)
{
    return a.oc1 * 32 > 64 ? launch_1x1_proj_k<128, 128>(a, pj, s) : launch_1x1_proj_k<256, 64>(a, pj, s);
}

// conv3 (a: 1x1, unit stride, shortcut and ReLU) chained with the next block's conv1 (b: 1x1, unit
// stride, the same pixels): a 256-channel block output with conv3 K <= 64 and conv1 to 64 or 128
// channels, or a 512-channel one with conv3 K <= 128 and conv1 to 128.
bool conv1x1_chain_supported(const ConvArgs &a, const ConvArgs &b)
{
    if (a.in_ps || a.out_ps || b.in_ps || (b.out_ps && ((b.ho | b.wo) & 1))) return false;
    const bool shape = (a.oc == 256 && a.i1 <= 2 && (b.oc == 64 || b.oc == 128)) ||
                       (a.oc == 512 && a.i1 <= 4 && b.oc == 128);
    return shape && a.stride == 1 && a.pad == 0 && a.residual && a.relu && !a.out_i32 && b.i1 * 32 == a.oc &&
           b.stride == 1 && b.pad == 0 && !b.residual && !b.out_i32 && a.m == b.m && a.ho == b.h && a.wo == b.w &&
           a.n == b.n && b.ho == b.h && b.wo == b.w;
}

hipError_t launch_conv1x1_chain(const ConvArgs &a, const ConvArgs &b, hipStream_t s)
{
    return launch_chain(a, b, nullptr, s);
}

// The same with conv3's shortcut its 1x1 projection pj (unit stride, K <= 64, conv3's pixels and
// channels, no ReLU), computed in the kernel.
bool conv1x1_proj_chain_supported(const ConvArgs &a, const ConvArgs &pj, const ConvArgs &b)
{
    return conv1x1_chain_supported(a, b) && a.oc == 256 && b.oc == 64 && !a.out_even && !pj.in_ps && !pj.out_ps &&
           pj.i1 <= 2 &&
           pj.oc == a.oc &&
           pj.stride == 1 && pj.pad == 0 && !pj.relu && !pj.residual && !pj.out_i32 && pj.m == a.m &&
           pj.ho == a.ho && pj.wo == a.wo && pj.h == a.h && pj.w == a.w && pj.n == a.n;
}

hipError_t launch_conv1x1_proj_chain(const ConvArgs &a, const ConvArgs &pj, const ConvArgs &b, hipStream_t s)
{
    return launch_chain(a, b, &pj, s);
}

// conv3 (a: 1x1, unit stride, 64 < K <= 128, 512 output channels, its shortcut the projection)
// with its 1x1 projection pj (unit stride, 128 < K <= 256: the first block of res3, whose stride-2
// input arrives subsampled) in the persistent ring kernel.
bool conv1x1_ring_proj_supported(const ConvArgs &a, const ConvArgs &pj)
{
    return a.oc == 512 && a.i1 > 2 && a.i1 <= 4 && a.stride == 1 && a.pad == 0 && !a.out_i32 && !a.in_ps &&
           !a.out_ps && pj.oc == a.oc && pj.i1 > 4 && pj.i1 <= 8 && pj.stride == 1 && pj.pad == 0 && !pj.relu &&
           !pj.residual && !pj.out_i32 && !pj.in_ps && !pj.out_ps && pj.n == a.n && pj.h == a.ho && pj.w == a.wo &&
           a.h == a.ho && a.w == a.wo && pj.m == a.m;
}

hipError_t launch_conv1x1_ring_proj(const ConvArgs &a, const ConvArgs &pj, hipStream_t s)
{
    return launch_ring<8, 2, 4>(a, pj, s);
}

// The 1x1 conv3 with shortcut of res4 (K = 256, 1024 output channels): the ring kernel with all
// four K-steps of weights in registers, in slices of 512 output channels, on 32-pixel tiles (a
// 64-pixel slot, 48 KB, would leave a ring of three), for batches that give every CU's workgroup
// a run of tiles (at least 1024 tiles of 32 pixels).
bool conv1x1_ring_wide_supported(const ConvArgs &a)
{
    return a.residual && a.stride == 1 && a.pad == 0 && a.ho == a.h && a.wo == a.w && a.i1 > 4 && a.i1 <= 8 &&
           a.oc >= 512 && a.oc % 512 == 0 && a.m >= 64 * 512 && !a.out_i32 && !a.in_ps && !a.out_ps &&
           !a.out_even && a.ksplit <= 1;
}

hipError_t launch_conv1x1_ring_wide(const ConvArgs &a, hipStream_t s) { return launch_ring<8, 4, 0, 32>(a, a, s); }

hipError_t launch_conv1x1_small_k(const ConvArgs &a, hipStream_t s)
{
    // unit-stride layers with a shortcut and 256 or 512 output channels: the persistent ring kernel
    if (a.residual && a.stride == 1 && a.pad == 0 && a.ho == a.h && a.wo == a.w) {
        if (a.oc == 256) return a.i1 <= 2 ? launch_ring<4, 1, 0>(a, a, s) : launch_ring<4, 2, 0>(a, a, s);
        if (a.oc == 512 && a.i1 > 2) return launch_ring<8, 2, 0>(a, a, s);
    }
    const bool wide = a.oc1 * 32 > 64;
    if (a.i1 <= 2) return wide ? launch_1x1_res<128, 128, 1>(a, s) : launch_1x1_res<256, 64, 1>(a, s);
    return wide ? launch_1x1_res<128, 128, 2>(a, s) : launch_1x1_res<256, 64, 2>(a, s);
}

}  // namespace ifx
