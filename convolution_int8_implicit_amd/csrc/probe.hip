// Practical-ceiling probes of the device, for the measurements that report
// each kernel against its roofline: a streaming copy (the HBM rate a plain
// read + write stream reaches), an int8 MFMA loop (the matrix-core rate with
// no memory traffic), the buffer->LDS DMA rate of contiguous 1 KB runs from an
// L2-resident buffer (how the convolution kernels stage their operands), and
// the ds_read_b128 rate of a given lane pattern (LDS bank conflicts).  Not
// part of the convolution path.
#include "ifx_probe.h"

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "ifx_internal.h"

namespace ifx {
namespace {

// Grid-stride copy of 16-byte chunks, non-temporal loads and stores (data moved once).
__global__ __launch_bounds__(256) void probe_copy_kernel(const v4i *src, v4i *dst, long long chunks)
{
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < chunks; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// A 4 x 4 tile of independent accumulator chains of v_mfma_i32_16x16x64_i8 per wave (the shape of
// the convolution kernels' main loop) on register operands: the loop issues matrix instructions
// only.  Each wave writes one sum so nothing is dropped.
__global__ __launch_bounds__(256) void probe_mfma_kernel(int *out, int iters, int seed)
{
    const int lane = threadIdx.x & 63;
    v4i af[4], bf[4], acc[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        af[t] = (v4i){seed + lane + t, seed ^ lane, lane * 3 + t, seed - lane};
        bf[t] = (v4i){lane ^ t, seed + t, lane ^ 5, seed + 1 - t};
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
#pragma unroll
            for (int tn = 0; tn < 4; ++tn)
                acc[tm][tn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[tm], bf[tn], it == 0 ? (v4i){0, 0, 0, 0}
                                                                                            : acc[tm][tn], 0, 0, 0);
    }
    v4i s = {0, 0, 0, 0};
#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) s += acc[tm][tn];
    if (lane == 0) out[blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = s.x + s.y + s.z + s.w;
}

// The same tile shape with operands that change from one MFMA to the next, as a contraction's do:
// four sets of random operand bits (a 32-bit integer hash of the lane and a counter) cycled
// through, so every instruction multiplies fresh bytes.  The matrix pipe's rate with toggling
// inputs, against the constant operands above.
__device__ __forceinline__ unsigned probe_hash(unsigned x)
{
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

__global__ __launch_bounds__(256) void probe_mfma_data_kernel(int *out, int iters, unsigned seed)
{
    const int lane = threadIdx.x & 63;
    v4i af[4][4], bf[4][4], acc[4][4];
    unsigned h = seed ^ ((blockIdx.x * 256u + threadIdx.x) * 0x9e3779b9u);
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                h = probe_hash(h + 1u);
                af[st][t][e] = (int)h;
                h = probe_hash(h + 1u);
                bf[st][t][e] = (int)h;
            }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int tn = 0; tn < 4; ++tn)
                    acc[tm][tn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                        af[st][tm], bf[st][tn], (it == 0 && st == 0) ? (v4i){0, 0, 0, 0} : acc[tm][tn], 0, 0, 0);
    }
    v4i sum = {0, 0, 0, 0};
#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) sum += acc[tm][tn];
    if (lane == 0) out[blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = sum.x + sum.y + sum.z + sum.w;
}

// Each wave moves 8 contiguous 1 KB runs per round from src into its own 8 KB of LDS by
// buffer->LDS DMA, then waits for them: run j of round i of wave w is 1 KB piece
// (8 (w iters + i) + j) mod pieces of src, so a src that fits L2 is read from L2.
constexpr int kProbeDmaLds = 4 * 8192;
__global__ __launch_bounds__(256) void probe_dma_lds_kernel(const int8_t *src, unsigned pieces, int iters, int *out)
{
    __shared__ __attribute__((aligned(1024))) int8_t lds[kProbeDmaLds];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const v4i rs = make_rsrc(src, (long long)pieces * 1024);
    const unsigned w = blockIdx.x * 4u + (unsigned)wave;
    int8_t *const mine = lds + wave * 8192;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const unsigned piece = (8u * (w * (unsigned)iters + (unsigned)i) + (unsigned)j) % pieces;
            load16_lds(rs, mine + j * 1024, piece * 1024u + (unsigned)lane * 16u);
        }
        wait_vmcnt<0>();
    }
    wave_lds_sync();
    const v4i v = *(const v4i *)(mine + lane * 16);
    if (lane == 0) out[w] = v.x ^ v.y ^ v.z ^ v.w;
}

// Each wave issues 8 independent ds_read_b128 per round, lane l at byte offsets[l] (masked into a
// 16 KB buffer, 16-byte aligned) plus 1 KB j (the same banks), and keeps the data live with an
// empty asm statement, so no other instruction competes with the reads.
constexpr int kProbeLds = 16384;
__global__ __launch_bounds__(256) void probe_lds_read_kernel(const int *offsets, int iters, int *out)
{
    __shared__ __attribute__((aligned(1024))) int8_t lds[kProbeLds + 8 * 1024];
    const int lane = threadIdx.x & 63;
    for (int i = threadIdx.x; i < (kProbeLds + 8 * 1024) / 16; i += blockDim.x)
        *(v4i *)(lds + 16 * i) = (v4i){i, i ^ 5, i + 7, (int)blockIdx.x};
    __syncthreads();
    const int off = offsets[lane] & (kProbeLds - 16);
    v4i keep = {0, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
        v4i v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = *(const v4i *)(lds + off + j * 1024);
#pragma unroll
        for (int j = 0; j < 8; ++j) asm volatile("" : : "v"(v[j]));
        keep = v[it & 7];
    }
    if (keep.x == 0x7fffffff) out[blockIdx.x] = keep.y;
}

// VALU issue rate of the fixed-point requantisation core against plain integer work: each lane
// runs `iters` rounds of 8 independent chains of one operation pair (kind 0: v_mad_i64_i32 then
// an arithmetic shift of the high word, the mode-1 requantisation; 1: an integer add then an
// xor; 2: int32 -> f64, an f64 fused multiply-add, f64 -> int32, the exact double-precision
// alternative).  The operands are launch arguments, so nothing folds at compile time; each
// lane's result is kept live by a store that happens only for an impossible value.
template <int KIND>
__global__ __launch_bounds__(256) void probe_valu_kernel(int *out, int iters, int m, long long add, int sh, double dm,
                                                         double dc)
{
    int v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (int)threadIdx.x * 7 + j;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (KIND == 0)
                v[j] = ((int)(((long long)v[j] * m + add) >> 32)) >> sh;
            else if (KIND == 1)
                v[j] = (v[j] + m) ^ sh;
            else
                v[j] = (int)__builtin_fma((double)v[j], dm, dc);
        }
    }
    int s = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += v[j];
    if (s == 0x12345678) out[blockIdx.x] = s;
}

}  // namespace
}  // namespace ifx

extern "C" {

int32_t ifx_probe_copy(const void *src, void *dst, size_t bytes, void *stream)
{
    if (!src || !dst) return 1;
    if ((bytes & 15u) || ((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u)) return 4;
    const long long chunks = (long long)(bytes / 16);
    if (chunks == 0) return 0;
    int cus = 0;
    if (ifx::current_cus(&cus) != hipSuccess) return 6;
    long long grid = (chunks + 255) / 256;
    if (grid > 64LL * cus) grid = 64LL * cus;
    hipLaunchKernelGGL(ifx::probe_copy_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                       (const ifx::v4i *)src, (ifx::v4i *)dst, chunks);
    return hipGetLastError() == hipSuccess ? 0 : 6;
}

int32_t ifx_probe_mfma_i8(int32_t *out, int32_t blocks, int32_t iters, void *stream)
{
    if (!out) return 1;
    if (blocks <= 0 || iters <= 0) return 2;
    hipLaunchKernelGGL(ifx::probe_mfma_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, out,
                       iters, 7);
    return hipGetLastError() == hipSuccess ? 0 : 6;
}

int32_t ifx_probe_mfma_i8_data(int32_t *out, int32_t blocks, int32_t iters, void *stream)
{
    if (!out) return 1;
    if (blocks <= 0 || iters <= 0) return 2;
    hipLaunchKernelGGL(ifx::probe_mfma_data_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, out,
                       iters, 0x5eedu);
    return hipGetLastError() == hipSuccess ? 0 : 6;
}

int32_t ifx_probe_dma_lds(const void *src, size_t bytes, int32_t blocks, int32_t iters, int32_t *out,
                          void *stream)
{
    if (!src || !out) return 1;
    if (blocks <= 0 || iters <= 0 || bytes < 1024 || (bytes & 1023u) || bytes > 0x7fffffffu) return 2;
    if ((uintptr_t)src & 15u) return 4;
    hipLaunchKernelGGL(ifx::probe_dma_lds_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       (const int8_t *)src, (unsigned)(bytes / 1024), iters, out);
    return hipGetLastError() == hipSuccess ? 0 : 6;
}

int32_t ifx_probe_lds_read(const int32_t *offsets, int32_t blocks, int32_t iters, int32_t *out, void *stream)
{
    if (!offsets || !out) return 1;
    if (blocks <= 0 || iters <= 0) return 2;
    hipLaunchKernelGGL(ifx::probe_lds_read_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       offsets, iters, out);
    return hipGetLastError() == hipSuccess ? 0 : 6;
}

int32_t ifx_probe_valu(int32_t kind, int32_t *out, int32_t blocks, int32_t iters, void *stream)
{
    if (!out) return 1;
    if (blocks <= 0 || iters <= 0 || kind < 0 || kind > 2) return 2;
    const dim3 g((unsigned)blocks), b(256);
    const hipStream_t st = (hipStream_t)stream;
    if (kind == 0)
        hipLaunchKernelGGL(ifx::probe_valu_kernel<0>, g, b, 0, st, out, iters, 1234567, (1LL << 40) + 5, 9, 1e-5, 0.5);
    else if (kind == 1)
        hipLaunchKernelGGL(ifx::probe_valu_kernel<1>, g, b, 0, st, out, iters, 1234567, (1LL << 40) + 5, 9, 1e-5, 0.5);
    else
        hipLaunchKernelGGL(ifx::probe_valu_kernel<2>, g, b, 0, st, out, iters, 1234567, (1LL << 40) + 5, 9, 1e-5, 0.5);
    return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // extern "C"
