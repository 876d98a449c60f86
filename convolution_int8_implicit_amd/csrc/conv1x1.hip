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
__global__ __launch_bounds__((C1Cfg<BM, BN, NST>::THREADS), (C1Cfg<BM, BN, NST>::WG_PER_CU))
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
__global__ __launch_bounds__((C1PCfg<BM, BN, NSP, NSA>::THREADS), (C1PCfg<BM, BN, NSP, NSA>::WG_PER_CU))
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

hipError_t launch_conv1x1_small_k(const ConvArgs &a, hipStream_t s)
{
    const bool wide = a.oc1 * 32 > 64;
    if (a.i1 <= 2) return wide ? launch_1x1_res<128, 128, 1>(a, s) : launch_1x1_res<256, 64, 1>(a, s);
    return wide ? launch_1x1_res<128, 128, 2>(a, s) : launch_1x1_res<256, 64, 2>(a, s);
}

}  // namespace ifx
