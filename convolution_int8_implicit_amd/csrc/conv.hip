// Implicit-GEMM int8 convolution with the fused requant / shortcut / ReLU
// epilogue, for gfx950 (CDNA4) int8 MFMA.
//
// What is computed (Inspur conv-merge article, section 3.3): the convolution
// is the matrix product data[M,K] . weight[N,K]^T with M = batch*Ho*Wo output
// pixels, N = output channels and K = KH*KW*Ic, both operands K-contiguous
// thanks to the NC/32HW32 activation and [O1,KH,KW,I1,O2,32] weight layouts
// (section 3.1).  The epilogue (section 3.4: BN, Sum with the shortcut, ReLU)
// runs on the int32 accumulators before anything is written, and the
// shortcut tile is fetched while the contraction runs (the article's early
// asynchronous shortcut copy).
//
// gfx950 design (not the article's A100 tiling):
//   * persistent workgroups of one wave64 per 64x64 sub-tile, as many per CU
//     as LDS allows; each owns a list of BM x BN output tiles and streams the
//     flattened sequence of
//     (tile, K-step) stages through an ST-deep LDS ring, so the loads of
//     the next tile are in flight while the current tile's epilogue runs;
//   * ring stages are filled by direct buffer->LDS 16-byte loads
//     (buffer_load_dwordx4 ... lds), no register staging; the buffer range
//     check turns every out-of-image tap, ragged row or padded channel into
//     zeros, so the implicit GEMM needs neither im2col nor branches;
//   * each wave owns 64x64 outputs = 4x4 v_mfma_i32_16x16x64_i8 tiles; one
//     K-step is 64 bytes = two 32-channel blocks;
//   * LDS rows are 64 bytes with an XOR swizzle of their four 16-byte
//     chunks, realised by choosing which global chunk each lane fetches;
//   * MFMA columns are permuted so that each lane holds four consecutive
//     output channels of a pixel; the epilogue requantises in registers,
//     stages bytes through LDS and writes whole 16-byte chunks of the
//     NC/32HW32 output (the shortcut and the per-channel parameters arrive
//     in LDS by DMA as well);
//   * tiles are dealt out XCD by XCD so the tiles sharing an activation tile
//     run together on one XCD (own L2).
#include "ifx_internal.h"
#include "device_common.h"

namespace ifx {
namespace {

// Tile geometry: a BM x BN workgroup tile, one wave per 64x64 sub-tile, and
// an ST-stage LDS ring.
template <int BM, int BN, int ST>
struct ConvCfg {
    static constexpr int WAVES_M = BM / 64;
    static constexpr int WAVES_N = BN / 64;
    static constexpr int WAVES = WAVES_M * WAVES_N;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int AI = BM * 64 / 16 / THREADS;  // A-tile loads per thread per stage
    static constexpr int BI = BN * 64 / 16 / THREADS;  // B-tile loads per thread per stage
    static_assert(AI * THREADS * 16 == BM * 64 && BI * THREADS * 16 == BN * 64, "whole 16-byte loads");
    static constexpr int LPS = AI + BI;                 // loads per thread per stage
    static constexpr int STAGE = (BM + BN) * 64;        // bytes per ring stage
    static constexpr int RI = BM * BN / 16 / THREADS;   // shortcut loads per thread
    static constexpr int RING = ST * STAGE;
    static constexpr int LDS = RING + BM * BN + 3 * 1024;  // ring | staging tile | bias,mult,shift
    static constexpr int WG_PER_CU = kLdsBytes / LDS > 2 ? 2 : kLdsBytes / LDS;
    static_assert(WG_PER_CU >= 1, "LDS budget");
    static_assert(ST >= 2 && (ST - 1) * LPS < 64, "ring depth");
};

template <int KH, int KW, int BM, int BN, int ST, bool RES, bool RELU>
__global__ __launch_bounds__((ConvCfg<BM, BN, ST>::THREADS), (ConvCfg<BM, BN, ST>::WG_PER_CU * ConvCfg<BM, BN, ST>::WAVES / 4))
void conv_kernel(ConvArgs a)
{
    using C = ConvCfg<BM, BN, ST>;
    constexpr int NWV = C::WAVES;
    constexpr int kStages = ST;
    constexpr int AI = C::AI, BI = C::BI, LPS = C::LPS, STAGE = C::STAGE;
    __shared__ __attribute__((aligned(1024))) int8_t smem[C::LDS];
    int8_t *const R = smem + C::RING;      // [BM][BN] shortcut in, packed output out
    int8_t *const Pm = R + BM * BN;        // [3][1024 B]: bias, mult, shift of the tile's channels

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS bases stay scalar
    const int wm0 = (wave % C::WAVES_M) * 64;
    const int wn0 = (wave / C::WAVES_M) * 64;

    // ---- this workgroup's tiles: XCD x takes the x-th eighth of the tile
    //      list (row-major over (m, n)); its workgroups deal it round robin ----
    const int tiles_n = (a.oc1 * 32 + BN - 1) / BN;
    const int tiles_m = (a.m + BM - 1) / BM;
    const long long T = (long long)tiles_m * tiles_n;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per = gridDim.x >> 3;
    const long long xb = T * xcd / 8;
    const long long span = T * (xcd + 1) / 8 - xb;
    if (span <= slot) return;
    const int n_items = (int)((span - slot + per - 1) / per);
    const int nsteps = (a.nkb + 1) >> 1;

    const int HoWo = a.ho * a.wo;
    const int HW = a.h * a.w;
    const long long in_img = (long long)a.i1 * HW * 32;
    const long long in_total = (long long)a.n * in_img;
    const long long out_img = (long long)a.oc1 * HoWo * 32;
    const int wrows = ((a.oc + a.o2 - 1) / a.o2) * a.o2;
    const v4i rsB = make_rsrc(a.wt, (long long)wrows * KH * KW * a.i1 * 32);
    const unsigned wstride_c1 = (unsigned)a.o2 * 32;

    auto item_tile = [&](int it, int &m0, int &n0) {
        const long long lin = xb + slot + (long long)it * per;
        const int li = (int)lin;
        const int tm_ = li / tiles_n;
        m0 = tm_ * BM;
        n0 = (li - tm_ * tiles_n) * BN;
    };

    // ---------------- issue cursor: next (tile, K-step) stage to load ----------------
    int is_it = 0, is_ks = 0;
    int s_c1 = 0, s_kx = 0, s_ky = 0, s_kb = 0;  // first block of the step: (ky, kx, c1), flat index
    v4i rsA;
    // general path (any channel-block count): pieces recombined every step
    unsigned a_img[AI];
    int a_iy[AI], a_ix[AI], a_sel[AI];
    bool a_ok[AI];
    unsigned b_off[BI];
    int b_sel[BI];
    bool b_ok[BI];
    // even channel-block count: both blocks of a step share the kernel tap, so a
    // lane's offset is its base plus a uniform per-step delta, and 3x3 padding
    // is a per-lane mask of valid taps
    const bool even_i1 = (a.i1 & 1) == 0;
    unsigned a_base[AI], b_base[BI];
    unsigned a_mask[AI];

    auto plan = [&]() {  // per-lane load plans of tile is_it
        int m0, n0;
        item_tile(is_it, m0, n0);
        const int img0 = fdiv(m0, a.howo_mul, a.howo_shr);
        rsA = make_rsrc(a.x + (long long)img0 * in_img, in_total - (long long)img0 * in_img);
        // A: instruction j of wave w fills stage rows [(4j+w)*16, +16); lane l -> row (4j+w)*16 + l/4,
        //    physical chunk l%4, which holds logical chunk (l%4) ^ swz(row).
#pragma unroll
        for (int j = 0; j < AI; ++j) {
            const int row = (j * NWV + wave) * 16 + (lane >> 2);
            const int lch = (lane & 3) ^ swz(row);
            const int p = m0 + row;
            a_ok[j] = p < a.m;
            const int pp = a_ok[j] ? p : m0;  // rows past the end load pixel m0 (result discarded)
            const int b = fdiv(pp, a.howo_mul, a.howo_shr);
            const int rem = pp - b * HoWo;
            const int oy = fdiv(rem, a.wo_mul, a.wo_shr);
            const int ox = rem - oy * a.wo;
            a_iy[j] = oy * a.stride - a.pad;
            a_ix[j] = ox * a.stride - a.pad;
            a_img[j] = (unsigned)((long long)(b - img0) * in_img) + (lch & 1) * 16;
            a_sel[j] = lch >> 1;  // which of the step's two 32-channel blocks
            a_base[j] = a_img[j] + (unsigned)(a_sel[j] * HW * 32) + (unsigned)((a_iy[j] * a.w + a_ix[j]) * 32);
            unsigned mask = 0;
#pragma unroll
            for (int ky = 0; ky < KH; ++ky)
#pragma unroll
                for (int kx = 0; kx < KW; ++kx)
                    if ((unsigned)(a_iy[j] + ky) < (unsigned)a.h && (unsigned)(a_ix[j] + kx) < (unsigned)a.w)
                        mask |= 1u << (ky * KW + kx);
            a_mask[j] = mask;
        }
        // B: instruction j of wave w fills physical rows [(4j+w)*16, +16); within each
        //    64-row group physical row r holds output channel (r%16)*4 + r/16.
#pragma unroll
        for (int j = 0; j < BI; ++j) {
            const int prow = (j * NWV + wave) * 16 + (lane >> 2);
            const int lch = (lane & 3) ^ swz(prow);
            const int o = (prow & ~63) + (prow & 15) * 4 + ((prow & 63) >> 4);
            const int Rw = n0 + o;
            b_ok[j] = Rw < wrows;
            const int RR = b_ok[j] ? Rw : 0;
            const int o1 = fdiv(RR, a.o2_mul, a.o2_shr), o2i = RR - o1 * a.o2;
            b_off[j] = (unsigned)(((long long)o1 * KH * KW * a.i1 * a.o2 + o2i) * 32) + (lch & 1) * 16;
            b_sel[j] = lch >> 1;
            b_base[j] = b_off[j] + (unsigned)b_sel[j] * wstride_c1;
        }
        s_c1 = s_kx = s_ky = s_kb = 0;
    };

    auto issue = [&](int ring_slot) {
        int8_t *st = smem + ring_slot * STAGE;
        if (is_it < n_items && even_i1) {
            const int tap = s_ky * KW + s_kx;
            const unsigned ua = (unsigned)((s_ky * a.w + s_kx) * 32 + s_c1 * HW * 32);
#pragma unroll
            for (int j = 0; j < AI; ++j) {
                unsigned off = a_base[j] + ua;
                if (KH > 1 || KW > 1) off = ((a_mask[j] >> tap) & 1u) ? off : kOOB;
                load16_lds(rsA, st + (j * NWV + wave) * 1024, off);
            }
            const unsigned ub = (unsigned)(tap * a.i1 + s_c1) * wstride_c1;
#pragma unroll
            for (int j = 0; j < BI; ++j) load16_lds(rsB, st + BM * 64 + (j * NWV + wave) * 1024, b_base[j] + ub);
            s_kb += 2;
            s_c1 += 2;
            if (s_c1 >= a.i1) {
                s_c1 = 0;
                if (++s_kx == KW) {
                    s_kx = 0;
                    ++s_ky;
                }
            }
            if (++is_ks == nsteps) {
                is_ks = 0;
                if (++is_it < n_items) plan();
            }
        } else if (is_it < n_items) {
            int c1b = s_c1 + 1, kxb = s_kx, kyb = s_ky;  // the step's second block
            if (c1b == a.i1) {
                c1b = 0;
                if (++kxb == KW) {
                    kxb = 0;
                    ++kyb;
                }
            }
#pragma unroll
            for (int j = 0; j < AI; ++j) {
                const int sel = a_sel[j];
                const int c1 = sel ? c1b : s_c1;
                const int kx = sel ? kxb : s_kx;
                const int ky = sel ? kyb : s_ky;
                const int iy = a_iy[j] + ky, ix = a_ix[j] + kx;
                bool ok = a_ok[j] && (s_kb + sel) < a.nkb;
                if (KH > 1) ok = ok && (unsigned)iy < (unsigned)a.h;
                if (KW > 1) ok = ok && (unsigned)ix < (unsigned)a.w;
                const unsigned off = ok ? a_img[j] + (unsigned)(((c1 * a.h + iy) * a.w + ix) * 32) : kOOB;
                load16_lds(rsA, st + (j * NWV + wave) * 1024, off);
            }
#pragma unroll
            for (int j = 0; j < BI; ++j) {
                const int sel = b_sel[j];
                const int c1 = sel ? c1b : s_c1;
                const int kx = sel ? kxb : s_kx;
                const int ky = sel ? kyb : s_ky;
                const bool ok = b_ok[j] && (s_kb + sel) < a.nkb;
                const unsigned off = ok ? b_off[j] + (unsigned)((ky * KW + kx) * a.i1 + c1) * wstride_c1 : kOOB;
                load16_lds(rsB, st + BM * 64 + (j * NWV + wave) * 1024, off);
            }
            s_kb += 2;
            s_c1 += 2;
            while (s_c1 >= a.i1) {
                s_c1 -= a.i1;
                if (++s_kx == KW) {
                    s_kx = 0;
                    ++s_ky;
                }
            }
            if (++is_ks == nsteps) {
                is_ks = 0;
                if (++is_it < n_items) plan();
            }
        } else {
            // past the last tile: same number of loads, all out of range (they write zeros)
#pragma unroll
            for (int j = 0; j < AI; ++j) load16_lds(rsB, st + (j * NWV + wave) * 1024, kOOB);
#pragma unroll
            for (int j = 0; j < BI; ++j) load16_lds(rsB, st + BM * 64 + (j * NWV + wave) * 1024, kOOB);
        }
    };

    // per-channel parameters and shortcut of the tile being computed -> LDS
    auto issue_tile_inputs = [&](int m0, int n0) {
        if (wave == 0) {
            const bool v = 4 * lane < BN && n0 + 4 * lane < a.oc;
            const unsigned off = v ? (unsigned)(n0 + 4 * lane) * 4 : kOOB;
            load16_lds(make_rsrc(a.bias, (long long)a.oc * 4), Pm, off);
            if (!a.out_i32) {
                load16_lds(make_rsrc(a.mult, (long long)a.oc * 4), Pm + 1024, off);
                load16_lds(make_rsrc(a.shift, (long long)a.oc * 4), Pm + 2048, off);
            }
        }
        if (RES) {
            const int img0 = fdiv(m0, a.howo_mul, a.howo_shr);
            const v4i rsR = make_rsrc(a.res + (long long)img0 * out_img, (long long)(a.n - img0) * out_img);
            constexpr int CPR = BN / 16;  // 16-byte chunks per staged row
#pragma unroll
            for (int j = 0; j < C::RI; ++j) {
                const int q = (j * NWV + wave) * 64 + lane;  // 16-byte slot of R
                const int row = q / CPR, ch = q % CPR;
                const int p = m0 + row;
                const int oc = n0 + ch * 16;
                unsigned off = kOOB;
                if (p < a.m && oc < a.oc1 * 32) {
                    const int b = fdiv(p, a.howo_mul, a.howo_shr), hw = p - b * HoWo;
                    off = (unsigned)((((long long)(b - img0) * a.oc1 + (oc >> 5)) * HoWo + hw) * 32 + (oc & 31));
                }
                load16_lds_stream(rsR, R + (j * NWV + wave) * 1024, off);
            }
        }
    };

    const int c = lane & 15;
    const int g = lane >> 4;
    v4i acc[4][4];

    auto epilogue = [&](int m0, int n0) {
        // the tile's parameters and shortcut were issued at its first K-step;
        // at most min(nsteps-1, ST-1) stages of later loads may stay in flight
        const int later = min(nsteps - 1, kStages - 1);
        if (later <= 0)
            wait_vmcnt<0>();
        else if (later == 1)
            wait_vmcnt<LPS>();
        else if (later == 2 || ST <= 3)
            wait_vmcnt<2 * LPS>();
        else if (later == 3 || ST <= 4)
            wait_vmcnt<(ST > 3 ? 3 : 2) * LPS>();
        else if (later == 4 || ST <= 5)
            wait_vmcnt<(ST > 4 ? 4 : 2) * LPS>();
        else
            wait_vmcnt<(ST > 5 ? 5 : 2) * LPS>();
        ring_barrier();

        const int ocl = n0 + wn0 + 4 * c;  // first of this lane's four output channels
        const v4i bias4 = *(const v4i *)(Pm + (wn0 + 4 * c) * 4);
        const int pbase = m0 + wm0;
        if (a.out_i32) {
            int32_t *y = (int32_t *)a.y;
            const bool vec = (a.oc & 3) == 0 && ocl + 3 < a.oc;
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int p = pbase + 16 * tm + 4 * i + g;
                    if (p >= a.m) continue;
                    const long long off = (long long)p * a.oc + ocl;
                    const v4i v = {acc[tm][0][i] + bias4.x, acc[tm][1][i] + bias4.y, acc[tm][2][i] + bias4.z,
                                   acc[tm][3][i] + bias4.w};
                    if (vec) {
                        *(v4i *)(y + off) = v;
                    } else {
#pragma unroll
                        for (int tn = 0; tn < 4; ++tn)
                            if (ocl + tn < a.oc) y[off + tn] = v[tn];
                    }
                }
            return;
        }
        const v4i mult4 = *(const v4i *)(Pm + 1024 + (wn0 + 4 * c) * 4);
        const v4i shift4 = *(const v4i *)(Pm + 2048 + (wn0 + 4 * c) * 4);
        int bias[4], mul[4], rnd[4], shm[4], shf[4];
        bool fast_lane = true;
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) {
            const bool v = ocl + tn < a.oc;  // padded channels: bias = mult = 0 gives 0
            bias[tn] = v ? bias4[tn] : 0;
            mul[tn] = v ? mult4[tn] : 0;
            shf[tn] = v ? shift4[tn] : 2;
            fast_lane = fast_lane && shf[tn] >= 2;
            rnd[tn] = 1 << ((shf[tn] - 2) & 31);
            shm[tn] = shf[tn] - 1;
        }
        int8_t *rbase = R + (wm0 + g) * BN + wn0 + 4 * c;
        if (!__all(fast_lane))
            requant_tile<0, RES, RELU, BN>(acc, rbase, bias, mul, rnd, shm, shf);
        else if (!RES && RELU)
            requant_tile<1, RES, RELU, BN>(acc, rbase, bias, mul, rnd, shm, shf);
        else
            requant_tile<2, RES, RELU, BN>(acc, rbase, bias, mul, rnd, shm, shf);
        wave_lds_sync();

        // 16-byte stores of the wave's 64 pixels x 64 channels
        int8_t *y = (int8_t *)a.y;
        const int k = lane & 3;
        const int och = n0 + wn0 + 16 * k;  // first channel of this lane's chunk
        if (och >= a.oc1 * 32) return;
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
            const v4i v = *(const v4i *)(R + (wm0 + prow) * BN + wn0 + 16 * k);
            int8_t *dst = y + (((long long)b * a.oc1 + (och >> 5)) * HoWo + hw) * 32 + (och & 31);
            // with a shortcut stream, both streams go non-temporal (measured faster); without, plain stores
            if (RES)
                store16_stream(dst, v);
            else
                *(v4i *)dst = v;
        }
    };

    // ---------------- main stream ----------------
    plan();
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) issue(s);

    int c_it = 0, c_ks = 0, c_m0, c_n0;
    item_tile(0, c_m0, c_n0);
    const int S = n_items * nsteps;
    for (int s = 0; s < S; ++s) {
        wait_vmcnt<(kStages - 2) * LPS>();
        ring_barrier();
        issue((s + kStages - 1) % kStages);
        if (c_ks == 0) {
            issue_tile_inputs(c_m0, c_n0);
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int tn = 0; tn < 4; ++tn) acc[tm][tn] = (v4i){0, 0, 0, 0};
        }
        const int8_t *st = smem + (s % kStages) * STAGE;
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
                acc[tm][tn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[tm], bf[tn], acc[tm][tn], 0, 0, 0);
        if (++c_ks == nsteps) {
            epilogue(c_m0, c_n0);
            c_ks = 0;
            if (++c_it < n_items) item_tile(c_it, c_m0, c_n0);
        }
    }
    wait_vmcnt<0>();  // trailing out-of-range ring loads
}

int g_cus = 0;

int device_cus()
{
    if (g_cus <= 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            g_cus = n;
        else
            g_cus = 256;
    }
    return g_cus;
}

template <int KH, int KW, int BM, int BN, int ST, bool RES>
hipError_t launch_tiles(const ConvArgs &a, hipStream_t s)
{
    using C = ConvCfg<BM, BN, ST>;
    const long long tiles = (long long)((a.m + BM - 1) / BM) * ((a.oc1 * 32 + BN - 1) / BN);
    if (tiles <= 0) return hipSuccess;
    // as many persistent workgroups as fit on the chip, a multiple of 8 (one share per XCD)
    long long g = (long long)C::WG_PER_CU * device_cus();
    if (g > tiles) g = (tiles + 7) / 8 * 8;
    g = g / 8 * 8;
    if (g < 8) g = 8;
    if (a.relu)
        hipLaunchKernelGGL((conv_kernel<KH, KW, BM, BN, ST, RES, true>), dim3((unsigned)g), dim3(C::THREADS), 0, s, a);
    else
        hipLaunchKernelGGL((conv_kernel<KH, KW, BM, BN, ST, RES, false>), dim3((unsigned)g), dim3(C::THREADS), 0, s,
                           a);
    return hipGetLastError();
}

template <int KH, int KW, int BM, int BN, int ST>
hipError_t launch_res(const ConvArgs &a, hipStream_t s)
{
    if (a.residual) return launch_tiles<KH, KW, BM, BN, ST, true>(a, s);
    return launch_tiles<KH, KW, BM, BN, ST, false>(a, s);
}

template <int KH, int KW>
hipError_t launch_k(const ConvArgs &a, hipStream_t s)
{
    if (a.oc1 * 32 > 64) return launch_res<KH, KW, 128, 128, 3>(a, s);
    return launch_res<KH, KW, 256, 64, 3>(a, s);
}

}  // namespace

void warm_conv_queries() { (void)device_cus(); }

hipError_t launch_conv(const ConvArgs &a, int kh, int kw, hipStream_t s)
{
    if (conv1x1_small_k_supported(a, kh, kw)) return launch_conv1x1_small_k(a, s);
    return launch_igemm(a, kh, kw, s);
}

}  // namespace ifx
