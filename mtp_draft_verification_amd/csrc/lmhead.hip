// LM-head tile kernel for an fp32 head with more than 16 positions (the tiny
// fp32-head workload), with the fused vocab-split softmax / argmax epilogue. bf16
// heads take the streaming kernel (skinny.hip) or the LDS-tiled kernel (wide.hip).
//
// The verify step pushes every target verify position and every drafter
// position through the one shared vocabulary head ("The Tiny Draft Model Hidden
// Inside Qwen", sections "One step deeper than the main model" and "How the
// draft becomes real output"); one read of the weights serves all positions of
// the pass ("Speculative Decoding and MTP: Why Guessing Is Free", section "The
// part that got me"):
//
//  * a workgroup owns 64 consecutive vocabulary rows and one chunk of up to
//    16*NT rows (positions); each of its 4 waves owns 16 vocabulary rows;
//  * the positions' hidden states are staged in LDS (all of H at once when they
//    fit, else in K chunks), W goes from HBM straight into MFMA A-operand
//    registers with 16-byte loads, PF steps ahead of its use;
//  * four v_mfma_f32_16x16x4_f32 per 16-byte fragment pair. Accumulation is fp32
//    over the whole of H (no split-K), in a fixed order;
//  * the epilogue reduces each position over the workgroup's vocabulary rows
//    to {max of l/T (log2 units), sum of exp, argmax (lowest id on ties)},
//    gathers the logit of the position's draft token, and optionally writes the
//    fp32 logits out for the sampling pass.
//
// MFMA 16x16 layouts used (wave64): A fragment lane l holds row l%16 and 16
// bytes of K (lane group l/16 selects which 16 bytes); B fragment lane l holds
// column l%16 with the same K slice; accumulator lane l holds column l%16,
// rows 4*(l/16) .. 4*(l/16)+3. Any assignment of K to lane groups works as long
// as A and B use the same one.
#include "mtpv_internal.h"

#include <climits>

namespace mtpv {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <int ES>
struct Mma;

template <>
struct Mma<4> {  // fp32 storage: 4 elements per fragment, K = 16 per step
    __device__ __forceinline__ static f32x4_t run(u32x4_t a, u32x4_t b, f32x4_t c) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[0]), __uint_as_float(b[0]), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[1]), __uint_as_float(b[1]), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[2]), __uint_as_float(b[2]), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[3]), __uint_as_float(b[3]), c, 0, 0, 0);
        return c;
    }
};

__device__ __forceinline__ Partial merge_partial(Partial a, Partial b) {
    const float ninf = -__builtin_inff();
    Partial o;
    o.x = fmaxf(a.x, b.x);
    const float sa = (a.x == ninf) ? 0.f : a.s * exp2f(a.x - o.x);
    const float sb = (b.x == ninf) ? 0.f : b.s * exp2f(b.x - o.x);
    o.s = sa + sb;
    const bool take_b = (b.bv > a.bv) || (b.bv == a.bv && b.bi < a.bi);
    o.bv = take_b ? b.bv : a.bv;
    o.bi = take_b ? b.bi : a.bi;
    return o;
}

// W is read exactly once per call: non-temporal loads keep it from displacing
// the staged positions and partials in the caches.
__device__ __forceinline__ u32x4_t load_w(const uint8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

template <int ES, int VA, int NT, int PF>
__global__ __launch_bounds__(256) void lmhead_kernel(LmHeadArgs p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int EPV = 16 / ES;   // elements per 16-byte fragment
    constexpr int KSTEP = 4 * EPV; // hidden elements consumed per fragment step
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lrow = lane & 15;
    const int lgrp = lane >> 4;

    // Workgroup -> (vocab block, M chunk). With several M chunks, the chunks of one
    // vocab block go to the same XCD (workgroups are dealt to XCDs round-robin)
    // one after another, so the block's W tile is reused from that XCD's L2.
    int vb, mc;
    if (p.MC == 1) {
        vb = blockIdx.x;
        mc = 0;
    } else {
        const int L = blockIdx.x;
        const int slot = L >> 3;
        mc = slot % p.MC;
        vb = (slot / p.MC) * 8 + (L & 7);
        if (vb >= p.S) return;  // uniform over the workgroup
    }
    if (vb == 0 && mc == 0 && tid == 0 && p.err != nullptr) *p.err = 0;

    const int m0 = mc * 16 * NT;
    const int mrows = min(16 * NT, p.Meff - m0);
    const int vw0 = vb * 64 * VA + wave * 16 * VA;
    const int H = p.H;
    const int V = p.V;
    const size_t rowbytes = (size_t)H * ES;

    const uint8_t* wp[VA];
#pragma unroll
    for (int va = 0; va < VA; ++va) {
        const int v = min(vw0 + va * 16 + lrow, V - 1);
        wp[va] = p.w + (size_t)v * rowbytes + lgrp * 16;
    }

    f32x4_t acc[VA][NT];
#pragma unroll
    for (int va = 0; va < VA; ++va)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[va][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nsteps = (H + KSTEP - 1) / KSTEP;
    const int steps_per_chunk = p.kc / KSTEP;
    const int ldsstride = p.kc * ES + 16;
    const u32x4_t zero4 = u32x4_t{0u, 0u, 0u, 0u};
    // Byte offset of this lane's 16 bytes of W at step g. Past H the address is
    // clamped into the row: those products meet zero-filled hidden states.
    const int hmax = H - EPV;
    auto w_off = [&](int g) -> size_t {
        const int k = min(g * KSTEP + lgrp * EPV, hmax);
        return (size_t)(k - lgrp * EPV) * ES;
    };

    // Stage hidden elements [g0*KSTEP, g1*KSTEP) of this chunk's positions into
    // LDS, zero-filled past H.
    auto stage = [&](int g0, int g1) {
        const int kbase = g0 * KSTEP;
        const int vpr = (g1 - g0) * KSTEP / EPV;  // 16-byte vectors per row
        for (int e = tid; e < mrows * vpr; e += 256) {
            const int r = e / vpr;
            const int c = e - r * vpr;
            const int kk = kbase + c * EPV;
            u32x4_t val = zero4;
            if (kk < H) {
                const int gr = m0 + r;
                const uint8_t* src = gr < p.Mt ? p.xt + (size_t)gr * rowbytes : p.xd + (size_t)(gr - p.Mt) * rowbytes;
                val = *(const u32x4_t*)(src + (size_t)kk * ES);
            }
            *(u32x4_t*)(smem + r * ldsstride + c * 16) = val;
        }
    };

    // W ring: wb[i] holds the fragments of the step currently PF - i steps ahead.
    // The loads are unconditional (clamped addresses) so the compiler can keep
    // PF steps of loads in flight and wait for exactly the one it needs.
    u32x4_t wb[PF][VA];
    auto prologue = [&](int g0, int g1) {
#pragma unroll
        for (int i = 0; i < PF; ++i)
#pragma unroll
            for (int va = 0; va < VA; ++va) wb[i][va] = load_w(wp[va] + w_off(min(g0 + i, g1 - 1)));
    };
    auto consume = [&](int i, int sl) {
        u32x4_t xb[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int r = nt * 16 + lrow;
            xb[nt] = (r < mrows) ? *(const u32x4_t*)(smem + r * ldsstride + (sl * KSTEP + lgrp * EPV) * ES) : zero4;
        }
#pragma unroll
        for (int va = 0; va < VA; ++va)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[va][nt] = Mma<ES>::run(wb[i][va], xb[nt], acc[va][nt]);
    };
    // Stream W over steps [g0, g1) against the staged chunk that starts at g0;
    // the ring must already hold steps g0 .. g0 + PF - 1.
    auto body = [&](int g0, int g1) {
        int g = g0;
        for (; g + PF <= g1; g += PF) {
#pragma unroll
            for (int i = 0; i < PF; ++i) {
                consume(i, g + i - g0);
                const int gn = min(g + i + PF, g1 - 1);
#pragma unroll
                for (int va = 0; va < VA; ++va) wb[i][va] = load_w(wp[va] + w_off(gn));
            }
        }
        // tail: fewer than PF steps left, their W already in registers
#pragma unroll
        for (int i = 0; i < PF; ++i)
            if (g + i < g1) consume(i, g + i - g0);
    };

    if (nsteps <= steps_per_chunk) {
        // All of H fits: start the W stream, stage the positions once, then one
        // uninterrupted stream over W.
        prologue(0, nsteps);
        stage(0, nsteps);
        __syncthreads();
        body(0, nsteps);
    } else {
        for (int g0 = 0; g0 < nsteps; g0 += steps_per_chunk) {
            const int g1 = min(nsteps, g0 + steps_per_chunk);
            __syncthreads();
            prologue(g0, g1);
            stage(g0, g1);
            __syncthreads();
            body(g0, g1);
        }
    }

    // ------------------------------------------------------------------ epilogue
    __syncthreads();  // every wave is done reading the staged hidden states
    Partial* red = reinterpret_cast<Partial*>(smem);  // [4][16*NT]
    const float ninf = -__builtin_inff();
    const float c2 = p.c2;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int rl = nt * 16 + lrow;
        const int r = m0 + rl;
        const bool rv = rl < mrows;
        int d = -1;
        if (rv && p.drafts != nullptr) {
            if (r < p.Mt) {
                const int b = r / (p.k + 1);
                const int j = r - b * (p.k + 1);
                d = (j < p.k) ? p.drafts[b * p.k + j] : -1;
            } else {
                d = p.drafts[r - p.Mt];
            }
        }
        float mx = ninf, bv = ninf;
        int bi = INT_MAX;
#pragma unroll
        for (int va = 0; va < VA; ++va)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int v = vw0 + va * 16 + lgrp * 4 + t;
                const float l = acc[va][nt][t];
                if (v < V) {
                    mx = fmaxf(mx, l * c2);
                    if (l > bv) {
                        bv = l;
                        bi = v;
                    }
                    if (v == d) p.dlogit[r] = l;
                }
            }
        if (p.spill != nullptr && rv) {
#pragma unroll
            for (int va = 0; va < VA; ++va) {
                const int v0 = vw0 + va * 16 + lgrp * 4;
                float* dst = p.spill + (size_t)r * V + v0;
                if ((V & 3) == 0 && v0 + 3 < V) {
                    *(f32x4_t*)dst = acc[va][nt];
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (v0 + t < V) dst[t] = acc[va][nt][t];
                }
            }
        }
        // reduce over the four lane groups that share this position
#pragma unroll
        for (int off = 16; off <= 32; off <<= 1) {
            mx = fmaxf(mx, __shfl_xor(mx, off));
            const float obv = __shfl_xor(bv, off);
            const int obi = __shfl_xor(bi, off);
            if (obv > bv || (obv == bv && obi < bi)) {
                bv = obv;
                bi = obi;
            }
        }
        float s = 0.f;
        if (mx != ninf) {
#pragma unroll
            for (int va = 0; va < VA; ++va)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int v = vw0 + va * 16 + lgrp * 4 + t;
                    if (v < V) s += exp2f(acc[va][nt][t] * c2 - mx);
                }
        }
        s += __shfl_xor(s, 16);
        s += __shfl_xor(s, 32);
        if (lgrp == 0) red[wave * 16 * NT + rl] = Partial{mx, s, bv, bi};
    }
    __syncthreads();
    if (tid < mrows) {
        Partial o = red[tid];
#pragma unroll
        for (int w = 1; w < 4; ++w) o = merge_partial(o, red[w * 16 * NT + tid]);
        p.partials[(size_t)(m0 + tid) * p.S + vb] = o;
    }
}

template <int ES, int VA, int NT>
hipError_t launch_one(const Plan& plan, const LmHeadArgs& args, hipStream_t stream) {
    constexpr int PF = (VA * NT <= 1) ? 8 : (VA * NT <= 4) ? 4 : 2;
    hipLaunchKernelGGL((lmhead_kernel<ES, VA, NT, PF>), dim3(plan.grid), dim3(256), plan.lds, stream, args);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lmhead(const Plan& plan, const LmHeadArgs& args, hipStream_t stream) {
    if (plan.es == 4 && plan.va == 1) {
        switch (plan.nt) {
            case 1: return launch_one<4, 1, 1>(plan, args, stream);
            case 2: return launch_one<4, 1, 2>(plan, args, stream);
            default: break;
        }
    }
    return hipErrorInvalidConfiguration;
}

}  // namespace mtpv
