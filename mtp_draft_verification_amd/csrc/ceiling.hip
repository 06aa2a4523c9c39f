// Achievable-rate probes for the roofline report: what a plain kernel reaches on
// this part for the two resources the verify path is bound by, measured on the same
// box and in the same process as the verify calls.
//
//  * read_kernel: one sweep of a buffer with 16-byte non-temporal loads, eight in
//    flight per thread, each workgroup reading 8 KB blocks spaced by the grid (of the
//    sweep layouts tried here the one that streams HBM best: ~7.0 TB/s against
//    ~6.8 TB/s with one contiguous range per workgroup and ~5.6 TB/s with a plain
//    per-load grid stride, 1.2-1.9 GB buffers); the words are folded into a
//    register that is written out only when a kernel argument the host always
//    passes as 0 is set, so the loads are kept and nothing is written.
//  * mfma_kernel: back-to-back v_mfma_f32_16x16x32_bf16 on 16 independent
//    accumulators per wave, 4 waves per compute unit (one per SIMD), on operands
//    with varied bit patterns (bf16 values of magnitude about 1 with random signs and
//    mantissas: constant operands draw less power and let the clock run higher than
//    the head product's data does).
#include "mtpv_internal.h"

#include <algorithm>

namespace mtpv {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(kReadThreads) void read_kernel(const u32x4_t* __restrict__ src, size_t n,
                                                            unsigned int* sink, int keep) {
    // workgroup w reads blocks w, w + grid, w + 2 grid, ... of kReadUnroll * 256
    // consecutive 16-byte words (8 KB), one word per thread per load
    const size_t blk = (size_t)kReadUnroll * kReadThreads;
    const size_t step = blk * gridDim.x;
    unsigned int acc = 0;
    size_t i = (size_t)blockIdx.x * blk + threadIdx.x;
    for (; i + (size_t)(kReadUnroll - 1) * kReadThreads < n; i += step) {
        u32x4_t v[kReadUnroll];
#pragma unroll
        for (int j = 0; j < kReadUnroll; ++j) v[j] = __builtin_nontemporal_load(src + i + (size_t)j * kReadThreads);
#pragma unroll
        for (int j = 0; j < kReadUnroll; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
    }
    for (; i < n; i += kReadThreads) {  // the last, partial block
        const u32x4_t v = __builtin_nontemporal_load(src + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (keep != 0) *sink = acc;
}

constexpr int kMfmaAcc = 16;

__device__ __forceinline__ unsigned int mix32(unsigned int x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

// bf16 pair with random signs and mantissas and exponents 126..127 (|v| in [0.5, 2))
__device__ __forceinline__ unsigned int bf16_pair(unsigned int r) {
    const unsigned int lo = (r & 0x807fu) | ((0x7eu + ((r >> 7) & 1u)) << 7);
    const unsigned int h = r >> 16;
    const unsigned int hi = (h & 0x807fu) | ((0x7eu + ((h >> 7) & 1u)) << 7);
    return lo | (hi << 16);
}

__global__ __launch_bounds__(256) void mfma_kernel(int iters, float* sink, int keep) {
    const unsigned int seed = blockIdx.x * 256u + threadIdx.x;
    u32x4_t a, b;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        a[j] = bf16_pair(mix32(seed * 8u + j));
        b[j] = bf16_pair(mix32(seed * 8u + 4u + j));
    }
    f32x4_t acc[kMfmaAcc];
#pragma unroll
    for (int j = 0; j < kMfmaAcc; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kMfmaAcc; ++j)
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc[j]) : "v"(a), "v"(b));
    }
    // the accumulators are read next: wait out the last MFMAs (the compiler does not
    // see inside the asm); the asm statements after it take every accumulator as an
    // operand, so no read of one can be placed before the wait
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int j = 0; j < kMfmaAcc; ++j) asm volatile("" : "+v"(acc[j]));
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kMfmaAcc; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    if (keep != 0) *sink = s;
}

}  // namespace

hipError_t launch_read(const void* src, size_t bytes, void* sink, hipStream_t stream) {
    const size_t n = bytes / 16;
    // 16 workgroups per compute unit, fewer when the buffer has fewer 8 KB blocks
    const size_t blocks = (n + (size_t)kReadUnroll * kReadThreads - 1) / ((size_t)kReadUnroll * kReadThreads);
    const int grid = (int)std::min<size_t>(4096, std::max<size_t>(1, blocks));
    hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(kReadThreads), 0, stream, static_cast<const u32x4_t*>(src), n,
                       static_cast<unsigned int*>(sink), 0);
    return hipGetLastError();
}

int64_t launch_mfma_rate(int iters, void* sink, hipStream_t stream) {
    constexpr int grid = 256;  // one workgroup of 4 waves per compute unit
    hipLaunchKernelGGL(mfma_kernel, dim3(grid), dim3(256), 0, stream, iters, static_cast<float*>(sink), 0);
    if (hipGetLastError() != hipSuccess) return -1;
    return (int64_t)grid * 4 * iters * kMfmaAcc * 16 * 16 * 32 * 2;
}

}  // namespace mtpv
