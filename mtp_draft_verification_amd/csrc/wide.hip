// LM-head kernel for many positions (more than 16): batched verification and the
// large-batch rollout shape.
//
// The verify pass is a contraction l[m, v] = sum_h x[m, h] W[v, h] over every
// target and drafter position m of the batch, with W read from HBM once ("One step
// deeper than the main model" / "How the draft becomes real output", "The Tiny
// Draft Model Hidden Inside Qwen": one shared head for target and drafter rows).
// With hundreds of positions it approaches and then crosses the point where the
// MFMA units, not HBM, set the pace ("Larger batches can also push the target model
// from memory-bound toward compute-bound", same page).
//
// Layout of the work:
//  * one 8-wave workgroup per compute unit (two waves per SIMD), persistent over
//    1/256 of the vocabulary (rows split evenly) and one chunk of at most 32*FM <=
//    128 positions; with several position chunks, the chunks of one vocabulary
//    range go to the same XCD side by side so that range's W is served from that
//    XCD's L2 after the first read;
//  * wave w owns column w % 4 of the range's rows and half w / 4 of the positions;
//    the column is processed 64 rows (4 MFMA row fragments) at a time against the
//    wave's 16*FM positions: 4*FM independent 16x16x32 bf16 MFMA accumulators;
//  * W fragments go from HBM straight into registers with 16-byte loads, one K-chunk (4 steps of 32 hidden elements) ahead, the prefetch running
//    on across chunk boundaries; the two waves of a column load the same W (the
//    second from L2), every W byte comes from HBM once;
//  * the positions' hidden states are staged through LDS in K-chunks of 128
//    elements, double buffered (one barrier per K-chunk); B fragments are read with
//    ds_read_b128: one 1 KB fragment feeds 4 MFMAs;
//  * after each 64-row column chunk the wave folds its logits into running per-
//    position statistics kept in LDS (max of l*c2, sum of exp2, argmax), gathers the
//    draft logits and writes the fp32 logits out when asked; at the end the four
//    columns are merged into one partial per (position, workgroup).
// Accumulation is fp32 over all of H in a fixed order; no split-K, no atomics.
#include "mtpv_internal.h"

#include <climits>

namespace mtpv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int KC = 128;                // hidden elements per staged K-chunk
constexpr int KSTEP = 32;              // hidden elements per MFMA step
constexpr int SPC = KC / KSTEP;        // MFMA steps per K-chunk
constexpr int PITCH = KC * 2 + 16;     // LDS bytes per staged position row

struct WStat {
    float x, s, bv;
    int bi;
};

__device__ __forceinline__ WStat merge_wstat(WStat a, WStat b) {
    const float ninf = -__builtin_inff();
    WStat o;
    o.x = fmaxf(a.x, b.x);
    const float sa = (a.x == ninf) ? 0.f : a.s * exp2f(a.x - o.x);
    const float sb = (b.x == ninf) ? 0.f : b.s * exp2f(b.x - o.x);
    o.s = sa + sb;
    const bool take_b = (b.bv > a.bv) || (b.bv == a.bv && b.bi < a.bi);
    o.bv = take_b ? b.bv : a.bv;
    o.bi = take_b ? b.bi : a.bi;
    return o;
}

// W bytes are reused from L2: by the second wave of a column and by the other
// position chunks of the range. Plain (temporal) loads, so the first read
// allocates in L2.
__device__ __forceinline__ u32x4_t load_w(const uint8_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// Position of the next W step to load: column chunk, K-chunk index (before
// rotation), step within the K-chunk. A value type, advanced by a pure function,
// so it stays in registers.
struct WCursor {
    int c, ki, s;
};

__device__ __forceinline__ WCursor advance(WCursor u, int nkc, int nch) {
    // past the last step the cursor stays there (a re-read, no new traffic)
    if (u.s + 1 < SPC) return WCursor{u.c, u.ki, u.s + 1};
    if (u.ki + 1 < nkc) return WCursor{u.c, u.ki + 1, 0};
    if (u.c + 1 < nch) return WCursor{u.c + 1, 0, 0};
    return u;
}

struct WFrags {
    u32x4_t f[4];
};

template <int FM>
__global__ __launch_bounds__(512, 1) void wide_kernel(LmHeadArgs p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int NT = 512;        // threads per workgroup
    constexpr int PF = SPC;        // W ring depth: one K-chunk, so a step's slot is its index
    constexpr int ROWS = 32 * FM;  // position rows per chunk (two halves of 16 * FM)
    uint8_t* xbuf0 = smem;
    uint8_t* xbuf1 = smem + ROWS * PITCH;
    WStat* stats = reinterpret_cast<WStat*>(smem + 2 * ROWS * PITCH);  // [4][ROWS]
    int* dtok = reinterpret_cast<int*>(stats + 4 * ROWS);              // [ROWS] draft id per position

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = (tid >> 6) & 3;  // vocabulary column
    const int half = tid >> 8;        // half of the positions
    const int lrow = lane & 15;
    const int lgrp = lane >> 4;
    const int H = p.H;
    const int V = p.V;
    const int R = p.S;  // vocabulary ranges (= partials per position)

    // workgroup -> (range, position chunk); chunks of one range share an XCD
    int rg, mc;
    if (p.MC == 1) {
        rg = blockIdx.x;
        mc = 0;
    } else {
        const int L = blockIdx.x;
        const int slot = L >> 3;
        mc = slot % p.MC;
        rg = (slot / p.MC) * 8 + (L & 7);
        if (rg >= R) return;  // uniform over the workgroup
    }
    if (rg == 0 && mc == 0 && tid == 0) *p.err = 0;

    const int m0 = mc * ROWS;
    const int mrows = min(ROWS, p.Meff - m0);
    // this range's rows, and this wave's column of them
    const int r0 = (int)((long long)rg * V / R);
    const int r1 = (int)((long long)(rg + 1) * V / R);
    const int n = r1 - r0;
    const int cs = r0 + (int)((long long)wave * n / 4);
    const int ce = r0 + (int)((long long)(wave + 1) * n / 4);
    const int colmax = (n + 3) / 4;
    const int nch = max(1, (colmax + 63) / 64);  // 64-row chunks, same count for all waves
    const int nkc = (H + KC - 1) / KC;
    const int total_it = nch * nkc;
    const size_t rowbytes = (size_t)H * 2;
    const int kc0 = p.rotate ? (int)(((unsigned)rg * 7u) % (unsigned)nkc) : 0;

    // ---------------------------------------------------------------- staging
    const u32x4_t zero4 = u32x4_t{0u, 0u, 0u, 0u};
    constexpr int VPR = KC * 2 / 16;               // 16-byte vectors per staged row
    constexpr int NXV = (ROWS * VPR + NT - 1) / NT;  // vectors per thread
    // Loads are unconditional (clamped addresses) so the compiler can count them
    // exactly; rows past the chunk and elements past H are zeroed at store time.
    u32x4_t xr[NXV];
    int xk = 0;  // K-chunk of the values in xr
    auto x_load = [&](int kc) {
        xk = kc;
#pragma unroll
        for (int i = 0; i < NXV; ++i) {
            const int e = tid + i * NT;
            const int r = min(e / VPR, mrows - 1);
            const int c = e % VPR;
            const int kk = min(kc * KC + c * 8, H - 8);
            const int gr = m0 + r;
            const uint8_t* src = gr < p.Mt ? p.xt + (size_t)gr * rowbytes : p.xd + (size_t)(gr - p.Mt) * rowbytes;
            xr[i] = *(const u32x4_t*)(src + (size_t)kk * 2);
        }
    };
    auto x_store = [&](uint8_t* buf) {
#pragma unroll
        for (int i = 0; i < NXV; ++i) {
            const int e = tid + i * NT;
            const int r = e / VPR;
            const int c = e - r * VPR;
            const bool live = r < mrows && xk * KC + c * 8 < H;
            if (r < ROWS) *(u32x4_t*)(buf + r * PITCH + c * 16) = live ? xr[i] : zero4;
        }
    };

    // ------------------------------------------------------ W stream (registers)
    const int vhi = max(min(ce, V) - 1, 0);
    auto w_load = [&](WCursor u) -> WFrags {
        int kc = kc0 + u.ki;
        if (kc >= nkc) kc -= nkc;
        const int k = min(kc * KC + u.s * KSTEP + lgrp * 8, H - 8);
        const int base = cs + 64 * u.c;
        WFrags r;
#pragma unroll
        for (int fv = 0; fv < 4; ++fv) {
            const int v = max(min(base + 16 * fv + lrow, vhi), 0);
            r.f[fv] = load_w(p.w + (size_t)v * rowbytes + (size_t)k * 2);
        }
        return r;
    };

    f32x4_t acc[4][FM];
#pragma unroll
    for (int fv = 0; fv < 4; ++fv)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) acc[fv][fm] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // running statistics of this wave's positions, draft id of each position
    const float ninf = -__builtin_inff();
    for (int i = tid; i < 4 * ROWS; i += NT) stats[i] = WStat{ninf, 0.f, ninf, INT_MAX};
    for (int i = tid; i < ROWS; i += NT) {
        int d = -1;
        const int pos = m0 + i;
        if (i < mrows && p.drafts != nullptr) {
            if (pos < p.Mt) {
                const int b = pos / (p.k + 1);
                const int j = pos - b * (p.k + 1);
                d = (j < p.k) ? p.drafts[b * p.k + j] : -1;
            } else {
                d = p.drafts[pos - p.Mt];
            }
        }
        dtok[i] = d;
    }

    WFrags wb[PF];
    WCursor cur{0, 0, 0};
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        wb[i] = w_load(cur);
        cur = advance(cur, nkc, nch);
    }
    x_load(kc0);
    x_store(xbuf0);
    __syncthreads();

    const float c2 = p.c2;
    const bool vec_spill = (V & 3) == 0;

    // Fold this wave's logits of column chunk c into the running statistics.
    auto epilogue = [&](int c) {
        const int vbase = cs + 64 * c;
        const int vr = min(64, ce - vbase);  // valid rows of this chunk (may be <= 0)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int pl = half * 16 * FM + 16 * fm + lrow;  // position within the chunk
            const bool pv = pl < mrows;
            const int pos = m0 + pl;
            float mx = ninf, bv = ninf;
            int bi = INT_MAX;
#pragma unroll
            for (int fv = 0; fv < 4; ++fv)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int vo = 16 * fv + 4 * lgrp + t;
                    const float l = acc[fv][fm][t];
                    if (vo < vr) {
                        mx = fmaxf(mx, l * c2);
                        if (l > bv) {
                            bv = l;
                            bi = vbase + vo;
                        }
                    }
                }
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
                for (int fv = 0; fv < 4; ++fv)
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (16 * fv + 4 * lgrp + t < vr) s += exp2f(acc[fv][fm][t] * c2 - mx);
            }
            s += __shfl_xor(s, 16);
            s += __shfl_xor(s, 32);
            if (pv) {
                // draft logit and fp32 logits of this chunk
                const int dd = dtok[pl] - vbase;
                if (dd >= 0 && dd < vr && ((dd >> 2) & 3) == lgrp) {
                    // select the element without a runtime index into the accumulators
                    const int fv = dd >> 4, t = dd & 3;
                    float l = 0.f;
#pragma unroll
                    for (int f = 0; f < 4; ++f) {
                        const f32x4_t a = acc[f][fm];
                        const float e = t == 0 ? a[0] : t == 1 ? a[1] : t == 2 ? a[2] : a[3];
                        l = (f == fv) ? e : l;
                    }
                    p.dlogit[pos] = l;
                }
                if (p.spill != nullptr) {
#pragma unroll
                    for (int fv = 0; fv < 4; ++fv) {
                        const int vo = 16 * fv + 4 * lgrp;
                        if (vo < vr) {
                            float* dst = p.spill + (size_t)pos * V + vbase + vo;
                            if (vec_spill && vo + 3 < vr) {
                                *(f32x4_t*)dst = acc[fv][fm];
                            } else {
#pragma unroll
                                for (int t = 0; t < 4; ++t)
                                    if (vo + t < vr) dst[t] = acc[fv][fm][t];
                            }
                        }
                    }
                }
                if (lgrp == 0 && mx != ninf) {
                    WStat& st = stats[wave * ROWS + pl];
                    st = merge_wstat(st, WStat{mx, s, bv, bi});
                }
            }
#pragma unroll
            for (int fv = 0; fv < 4; ++fv) acc[fv][fm] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            __builtin_amdgcn_sched_barrier(0);  // one fragment's temporaries at a time
        }
    };

    for (int it = 0; it < total_it; ++it) {
        const int c = it / nkc;
        const int kci = it - c * nkc;
        {
            // next K-chunk's hidden states (the last iteration re-stages a valid
            // chunk nobody reads: no branch around the loads keeps the wait counts exact)
            int kn = kc0 + (kci + 1 == nkc ? 0 : kci + 1);
            if (kn >= nkc) kn -= nkc;
            x_load(kn);
        }
        const uint8_t* xb = (it & 1) ? xbuf1 : xbuf0;
        const int nfv = min(4, max(0, (min(64, ce - (cs + 64 * c)) + 15) / 16));
#pragma unroll
        for (int s = 0; s < SPC; ++s) {  // ring slot s holds this step (PF == SPC)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const u32x4_t bx =
                    *(const u32x4_t*)(xb + (half * 16 * FM + 16 * fm + lrow) * PITCH + (s * KSTEP + lgrp * 8) * 2);
#pragma unroll
                for (int fv = 0; fv < 4; ++fv)
                    if (fv < nfv)
                        acc[fv][fm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, wb[s].f[fv]), __builtin_bit_cast(bf16x8_t, bx), acc[fv][fm], 0,
                            0, 0);
            }
            wb[s] = w_load(cur);
            cur = advance(cur, nkc, nch);
        }
        x_store((it & 1) ? xbuf0 : xbuf1);
        if (kci == nkc - 1) epilogue(c);
        __syncthreads();
    }

    // merge the four columns' statistics per position
    if (tid < mrows) {
        WStat o = stats[tid];
#pragma unroll
        for (int w = 1; w < 4; ++w) o = merge_wstat(o, stats[w * ROWS + tid]);
        p.partials[(size_t)(m0 + tid) * R + rg] = Partial{o.x, o.s, o.bv, o.bi};
    }
}

template <int FM>
hipError_t launch_fm(const Plan& plan, const LmHeadArgs& args, hipStream_t stream) {
    auto kern = wide_kernel<FM>;
    const size_t lds = plan.lds;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(plan.grid), dim3(512), lds, stream, args);
    return hipGetLastError();
}

}  // namespace

size_t wide_lds_bytes(int fm) {
    const size_t rows = (size_t)32 * fm;
    return 2 * rows * PITCH + 4 * rows * sizeof(WStat) + rows * sizeof(int);
}

hipError_t launch_wide(const Plan& plan, const LmHeadArgs& args, hipStream_t stream) {
    switch (plan.nt) {
        case 1: return launch_fm<1>(plan, args, stream);
        case 2: return launch_fm<2>(plan, args, stream);
        case 3: return launch_fm<3>(plan, args, stream);
        case 4: return launch_fm<4>(plan, args, stream);
        default: return hipErrorInvalidConfiguration;
    }
}

}  // namespace mtpv
