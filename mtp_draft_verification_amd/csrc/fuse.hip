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
// scaled values rounded to bf16 (round to nearest even), written as
// x[b] = [n_e(E[tok]) | n_h(h)], n(v) = v / sqrt(mean(v^2) + eps) * g.
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

// 8 values of v scaled by r and the matching 8 weights of g, packed back to bf16
__device__ __forceinline__ u32x4_t scale8(u32x4_t v, u32x4_t g, float r) {
    u32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const unsigned int lo = to_bf16(bf16_lo(v[i]) * r * bf16_lo(g[i]));
        const unsigned int hi = to_bf16(bf16_hi(v[i]) * r * bf16_hi(g[i]));
        o[i] = lo | (hi << 16);
    }
    return o;
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
    u32x4_t* x = reinterpret_cast<u32x4_t*>(p.x + (size_t)b * p.H * 4);
    for (int i = tid; i < nv; i += 256) {
        const u32x4_t ev = ok ? e[i] : zero;
        x[i] = scale8(ev, ge[i], re);
        x[nv + i] = scale8(h[i], gh[i], rh);
    }
}

}  // namespace

hipError_t launch_fuse(const FuseArgs& args, hipStream_t stream) {
    hipLaunchKernelGGL(fuse_kernel, dim3(args.B), dim3(256), 0, stream, args);
    return hipGetLastError();
}

}  // namespace mtpv
