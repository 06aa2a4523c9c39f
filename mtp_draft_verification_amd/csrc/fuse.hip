// Input fusion of the MTP module in front of the drafter: per request, the RMS-
// normalized embedding of the chosen token and the RMS-normalized hidden state,
// concatenated into the 2H-wide input of the module's fc projection ("The Tiny Draft
// Model Hidden Inside Qwen", section "One step deeper than the main model": the
// module normalizes the hidden state and the new token's embedding, concatenates
// them and projects back to the hidden width; the embedding table is the main
// model's). The projection itself runs on the LM-head kernels (W_fc [H, 2H] in the
// place of the head, the fused rows in the place of the hidden states).
//
// One workgroup per request row: 16-byte loads of both rows, fp32 sums of squares
// (per-thread partials, then a fixed-order wave and workgroup reduction), then the
// scaled values n(v) = v / sqrt(mean(v^2) + eps) * g in fp32. The projection's
// operands are bf16, so each fp32 value x is carried as two bf16 numbers: hi =
// bf16(x) (round to nearest even) and lo = bf16(x - hi) (x - hi is exact in fp32);
// hi + lo is x to 2^-17 relative. The fused input is written as 2B rows,
//   row b     = hi parts of [n_e(E[tok]) | n_h(h)],
//   row B + b = lo parts,
// and the fc sums the two rows' products (bf16 x bf16 products are exact in fp32).
// A token outside [0, V) contributes a zero row; workgroup 0 sets the call's device
// error word from all tokens (one writer, so it also clears stale bits).
#include "mtpv.h"
#include "mtpv_internal.h"

namespace mtpv {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(unsigned int w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned int w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ unsigned int to_bf16(float f) {
    const unsigned int u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float sq8(u32x4_t v) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = bf16_lo(v[i]), b = bf16_hi(v[i]);
        s = fmaf(a, a, s);
        s = fmaf(b, b, s);
    }
    return s;
}

// 8 values of v scaled by r and the matching 8 weights of g, as bf16 hi and lo parts
__device__ __forceinline__ void scale8(u32x4_t v, u32x4_t g, float r, u32x4_t& hi, u32x4_t& lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = bf16_lo(v[i]) * r * bf16_lo(g[i]);
        const float b = bf16_hi(v[i]) * r * bf16_hi(g[i]);
        const unsigned int ah = to_bf16(a), bh = to_bf16(b);
        const unsigned int al = to_bf16(a - __uint_as_float(ah << 16));
        const unsigned int bl = to_bf16(b - __uint_as_float(bh << 16));
        hi[i] = ah | (bh << 16);
        lo[i] = al | (bl << 16);
    }
}

__device__ __forceinline__ float block_sum(float v, float* sh) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh[wave] = v;
    __syncthreads();
    const float t = ((sh[0] + sh[1]) + sh[2]) + sh[3];
    __syncthreads();
    return t;
}

__global__ __launch_bounds__(256) void fuse_kernel(FuseArgs p) {
    __shared__ float sh[4];
    __shared__ int sh_err;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int nv = p.H / 8;  // 16-byte vectors per row
    const int tok = p.tokens[b];
    const bool ok = tok >= 0 && tok < p.V;
    const u32x4_t* e = reinterpret_cast<const u32x4_t*>(p.embed + (size_t)(ok ? tok : 0) * p.H * 2);
    const u32x4_t* h = reinterpret_cast<const u32x4_t*>(p.hidden + (size_t)b * p.H * 2);
    const u32x4_t zero = u32x4_t{0u, 0u, 0u, 0u};

    if (b == 0) {  // device error word: any token out of range
        if (tid == 0) sh_err = 0;
        __syncthreads();
        int bad = 0;
        for (int i = tid; i < p.B; i += 256) {
            const int t = p.tokens[i];
            bad |= (t < 0 || t >= p.V) ? 1 : 0;
        }
        if (bad) atomicOr(&sh_err, 1);
        __syncthreads();
        if (tid == 0) *p.err = sh_err ? MTPV_DEVERR_TOKEN_RANGE : 0;
    }

    float se = 0.f, shh = 0.f;
    for (int i = tid; i < nv; i += 256) {
        const u32x4_t ev = ok ? e[i] : zero;
        se += sq8(ev);
        shh += sq8(h[i]);
    }
    se = block_sum(se, sh);
    shh = block_sum(shh, sh);
    const float re = 1.0f / sqrtf(se / (float)p.H + p.eps);
    const float rh = 1.0f / sqrtf(shh / (float)p.H + p.eps);

    const u32x4_t* ge = reinterpret_cast<const u32x4_t*>(p.g_e);
    const u32x4_t* gh = reinterpret_cast<const u32x4_t*>(p.g_h);
    u32x4_t* xh = reinterpret_cast<u32x4_t*>(p.x + (size_t)b * p.H * 4);
    u32x4_t* xl = reinterpret_cast<u32x4_t*>(p.x + (size_t)(p.B + b) * p.H * 4);
    for (int i = tid; i < nv; i += 256) {
        const u32x4_t ev = ok ? e[i] : zero;
        u32x4_t hi, lo;
        scale8(ev, ge[i], re, hi, lo);
        xh[i] = hi;
        xl[i] = lo;
        scale8(h[i], gh[i], rh, hi, lo);
        xh[nv + i] = hi;
        xl[nv + i] = lo;
    }
}

}  // namespace

hipError_t launch_fuse(const FuseArgs& args, hipStream_t stream) {
    hipLaunchKernelGGL(fuse_kernel, dim3(args.B), dim3(256), 0, stream, args);
    return hipGetLastError();
}

}  // namespace mtpv
