// LM-head kernel for many positions (more than 16, bf16): batched verification
// and the large-batch rollout shape.
//
// The verify pass is a contraction l[m, v] = sum_h x[m, h] W[v, h] over every
// target and drafter position m of the batch, with one head W for both ("The Tiny
// Draft Model Hidden Inside Qwen", sections "One step deeper than the main model"
// and "How the draft becomes real output"). With hundreds of positions it
// approaches and then crosses the point where the MFMA units, not HBM, set the
// pace (same page: larger batches push the target from memory-bound toward
// compute-bound), so it is written as an LDS-tiled matrix product:
//
//  * one workgroup (8 waves) per tile of BV = 256 vocabulary rows by BM positions
//    (BM = 64, 128 or 256); the tiles of one vocabulary block go to the same XCD side
//    by side, so after the first one its W comes from that XCD's L2;
//  * both operands are staged in LDS in K-stages of 64 hidden elements (128 bytes
//    per row) with 16-byte direct-to-LDS loads: one load instruction fills 1 KB,
//    eight whole 128-byte rows, so every cache line fetched is used in full and no
//    register holds staged data; NS stages rotate (the loads of stage kb + NS - 1
//    are issued while stage kb is multiplied);
//  * within a staged row the eight 16-byte chunks are XOR-swizzled by row, which
//    makes the MFMA fragment reads (ds_read_b128, 16 rows per 16 lanes) free of bank
//    conflicts;
//  * wave w owns vocabulary rows 64 (w % 4) .. + 63 and positions (w / 4) BM / 2 ..
//    + BM / 2 - 1 of the tile: 4 x BM / 32 accumulators of 16x16x32 bf16 MFMAs (a
//    wave whose positions end inside its half skips the padded fragments);
//  * after the last stage each wave folds its logits into per-position statistics
//    (max of l * c2, sum of exp2, argmax), gathers the draft logits and writes the
//    fp32 logits out when asked; the four vocabulary waves are merged into one
//    partial per (position, vocabulary block).
// Accumulation is fp32 over all of H in a fixed order, no atomics; the K-split launch
// of the input fusion writes each slice's raw products, which ksum_kernel adds in
// slice order.
#include "mtpv_internal.h"

#include <algorithm>
#include <atomic>
#include <type_traits>

#include <climits>

namespace mtpv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BV = 256;        // vocabulary rows per tile
constexpr int NT = 512;        // threads per workgroup
constexpr int LDS_MAX = 160 * 1024;

// Sixteen zero bytes: the source of the hidden-state chunks past H in the last
// stage when H is not a multiple of 64 (a direct-to-LDS load cannot zero-fill).
__device__ __attribute__((aligned(16))) const unsigned int kZero16[4] = {0u, 0u, 0u, 0u};

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

// s_waitcnt with only the vector-memory count set (expcnt and lgkmcnt at their
// maxima): gfx9 encoding, vmcnt split over bits 3:0 and 15:14.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Tile of at most BV vocabulary rows by BM positions, K-stages of BK = 64 hidden
// elements. W and the positions have rings of their own in LDS: NSW stages of W (the
// operand that streams from HBM, so it runs one stage further ahead) and NSX of X.
template <int BM>
struct WideCfg {
    static constexpr int BK = 64;
    static constexpr int ROWB = BK * 2;                      // LDS bytes per staged row
    static constexpr int CPR = BK / 8;                       // 16-byte chunks per staged row
    static constexpr int RPI = 64 / CPR;                     // rows filled by one load instruction
    static constexpr int WSTAGE = BV * ROWB;                 // bytes of one W stage
    static constexpr int XSTAGE = BM * ROWB;                 // bytes of one X stage
    static constexpr int NSX = BM == 256 ? 2 : 3;            // X stages
    static constexpr int NSW = (LDS_MAX - NSX * XSTAGE) / WSTAGE;  // W stages
    static constexpr int LPW_W = BV / RPI / (NT / 64);       // W load instructions per wave per stage
    static constexpr int LPW_X = BM / RPI / (NT / 64);       // X load instructions per wave per stage
    static constexpr int FM = BM / 32;                       // position fragments per wave
    static constexpr int KS = BK / 32;                       // MFMA K-steps per stage
    static constexpr int LDS = NSW * WSTAGE + NSX * XSTAGE;
    static_assert(NSW >= NSX && NSX >= 2 && LDS <= LDS_MAX, "rings");
    static_assert(LPW_W * RPI * (NT / 64) == BV && LPW_X * RPI * (NT / 64) == BM, "whole instructions");
    // The loop issues, in the middle of iteration i, X(i + NSX) then W(i + NSW)
    // (the prologue does so for i = -NSW .. -1). WAIT: loads issued after the later
    // of X(kb + 1) and W(kb + 1) when iteration kb waits for stage kb + 1; PRO_WAIT:
    // loads issued after the later of X(0) and W(0) at the end of the prologue.
    static constexpr int WAIT = NSW > NSX ? LPW_W + (NSX - 2) * (LPW_W + LPW_X) : (NSX - 2) * (LPW_W + LPW_X);
    static constexpr int PRO_WAIT = NSW > NSX ? LPW_W + (NSX - 1) * (LPW_W + LPW_X) : (NSX - 1) * (LPW_W + LPW_X);
    static_assert(NSW - NSX <= 1 && PRO_WAIT < 64, "wait counts");
};

// Calls f(std::integral_constant<int, n>) for the run-time n in [0, N]: one
// instantiation of f per count.
template <int N, typename F>
__device__ __forceinline__ void with_live(int n, F&& f) {
    if constexpr (N == 0) {
        f(std::integral_constant<int, 0>{});
    } else {
        if (n == N)
            f(std::integral_constant<int, N>{});
        else
            with_live<N - 1>(n, f);
    }
}

// Workgroup barrier for the stage ring. __syncthreads() would also make every wave
// wait for all of its direct-to-LDS loads (vmcnt(0): its release fence covers them),
// which drains the ring at every stage; the ring's own vmcnt wait already covers
// the stage about to be read, so only the barrier itself is needed. The empty asm
// statements keep the compiler from moving LDS accesses across it.
// It also waits for this wave's LDS reads (lgkmcnt(0)), so that once every wave is
// past it the buffers they read may be refilled.
__device__ __forceinline__ void stage_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maxima
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Chunk swizzle of staged row r: any 16 consecutive rows read at one chunk index
// land on 16 distinct 16-byte bank groups (of a 256-byte bank row).
template <int CPR>
__device__ __forceinline__ int chunk_swz(int r) { return (r / (16 / CPR)) % CPR; }

// NTW: W is read by one workgroup only (one position chunk per vocabulary tile, K
// not split), so its loads carry the non-temporal hint; with several chunks per tile
// they share W through L2 and load it normally (a K-split launch measured slower
// with the hint).
template <int BM, bool NTW>
__global__ __launch_bounds__(512, 1) void wide_kernel(LmHeadArgs p) {
    using Cfg = WideCfg<BM>;
    constexpr int NSW = Cfg::NSW;
    constexpr int NSX = Cfg::NSX;
    constexpr int LPW_W = Cfg::LPW_W;
    constexpr int LPW_X = Cfg::LPW_X;
    constexpr int FM = Cfg::FM;
    constexpr int BK = Cfg::BK;
    constexpr int ROWB = Cfg::ROWB;
    constexpr int CPR = Cfg::CPR;
    constexpr int RPI = Cfg::RPI;
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    uint8_t* wring = smem;                            // NSW stages of BV rows
    uint8_t* xring = smem + NSW * Cfg::WSTAGE;        // NSX stages of BM rows

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int vw = wave & 3;   // vocabulary quarter of the tile
    const int mw = wave >> 2;  // position half of the tile
    const int H = p.H;
    const int V = p.V;
    const int S = p.S;  // vocabulary tiles (= partials per position)

    // workgroup -> (vocabulary tile, position chunk); the chunks of one tile share an XCD.
    // With K split in ks slices, workgroup g takes slice g % ks of position chunk
    // (g / ks) % MC of tile g / (ks MC): with ks = 8 each XCD works on one slice of K.
    int vt, mt, ksl = 0;
    if (p.ks > 1) {
        const int rest = blockIdx.x / p.ks;
        ksl = blockIdx.x - rest * p.ks;
        mt = rest % p.MC;
        vt = rest / p.MC;
    } else if (p.MC == 1) {
        vt = blockIdx.x;
        mt = 0;
    } else {
        const int g = blockIdx.x;
        const int idx = g >> 3;
        mt = idx % p.MC;
        vt = (idx / p.MC) * 8 + (g & 7);
        if (vt >= S) return;  // uniform over the workgroup
    }
    if (vt == 0 && mt == 0 && tid == 0 && p.err != nullptr) *p.err = 0;

    // vocabulary rows [v0, v1) of this tile: the 16-row groups of V split evenly over
    // the S tiles (edges on 16-row boundaries keep the fp32 spill's vector stores
    // aligned; at most 16 groups per tile since S >= V / 256)
    const int G = (V + 15) / 16;
    const int v0 = min(V, 16 * (int)((long long)vt * G / S));
    const int v1 = min(V, 16 * (int)((long long)(vt + 1) * G / S));
    const int m0 = mt * BM;
    // K stages [kbeg, kbeg + nk) of the nk_all in H (all of them unless K is split)
    const int nk_all = (H + BK - 1) / BK;
    const int nk_per = (nk_all + p.ks - 1) / p.ks;
    const int kbeg = min(nk_all, ksl * nk_per);
    const int nk = min(nk_all, kbeg + nk_per) - kbeg;
    const size_t rowbytes = (size_t)H * 2;
    // optional rotation of the K order per vocabulary tile (the position chunks of
    // one tile share it, and so their W in L2)
    const int kb0 = p.ks > 1 ? kbeg : p.rotate ? (int)(((unsigned)vt * 7u) % (unsigned)nk) : 0;

    // ------------------------------------------------------------ stage loads
    // W instruction j (j = wave * LPW_W + i) fills staged W rows RPI j .. RPI j + RPI - 1,
    // X instruction j likewise for positions. Lane l writes LDS slot l % CPR of row
    // RPI j + l / CPR and fetches chunk (l % CPR) ^ swz(row). Rows past the tile and
    // positions past Meff re-read the last valid row (results ignored).
    const uint8_t* w_row[LPW_W];
    int w_chunk[LPW_W];
    const uint8_t* x_row[LPW_X];
    int x_chunk[LPW_X];
#pragma unroll
    for (int i = 0; i < LPW_W; ++i) {
        const int r = RPI * (wave * LPW_W + i) + lane / CPR;
        w_chunk[i] = (lane % CPR) ^ chunk_swz<CPR>(r);
        w_row[i] = p.w + (size_t)min(v0 + r, v1 - 1) * rowbytes;
    }
#pragma unroll
    for (int i = 0; i < LPW_X; ++i) {
        const int r = RPI * (wave * LPW_X + i) + lane / CPR;
        x_chunk[i] = (lane % CPR) ^ chunk_swz<CPR>(r);
        const int m = min(m0 + r, p.Meff - 1);
        x_row[i] = m < p.Mt ? p.xt + (size_t)m * rowbytes : p.xd + (size_t)(m - p.Mt) * rowbytes;
    }
    auto stage_k = [&](int kb) {
        const int kk = kb + kb0;
        return kk >= nk_all ? kk - nk_all : kk;
    };
    // chunks past H: W re-reads the row start, X reads sixteen zero bytes
    auto issue_w = [&](int kb) {
        const int kk = stage_k(kb);
        uint8_t* dst = wring + (kb % NSW) * Cfg::WSTAGE + wave * LPW_W * 1024;
#pragma unroll
        for (int i = 0; i < LPW_W; ++i) {
            const int k = kk * BK + 8 * w_chunk[i];
            const uint8_t* src = k < H ? w_row[i] + (size_t)k * 2 : w_row[i];
            __builtin_amdgcn_global_load_lds(src, (lds_void*)(dst + i * 1024), 16, 0, NTW ? 2 : 0);  // 2: nt
        }
    };
    auto issue_x = [&](int kb) {
        const int kk = stage_k(kb);
        uint8_t* dst = xring + (kb % NSX) * Cfg::XSTAGE + wave * LPW_X * 1024;
#pragma unroll
        for (int i = 0; i < LPW_X; ++i) {
            const int k = kk * BK + 8 * x_chunk[i];
            const uint8_t* src = k < H ? x_row[i] + (size_t)k * 2 : reinterpret_cast<const uint8_t*>(kZero16);
            __builtin_amdgcn_global_load_lds(src, (lds_void*)(dst + i * 1024), 16, 0, 0);
        }
    };
    // the middle of iteration i issues X(i + NSX), then W(i + NSW), each if it exists,
    // into the buffers of stage i (read to registers by then)
    auto issue_mid = [&](int i) {
        if (i + NSX >= 0 && i + NSX < nk) issue_x(i + NSX);
        if (i + NSW >= 0 && i + NSW < nk) issue_w(i + NSW);
    };

    // fragment read offsets: row (l & 15) of a 16-row block, chunk 4 s + l / 16 for
    // K-step s of the stage (the swizzle of row 16 q + lrow is that of lrow)
    const int lrow = lane & 15;
    const int lgrp = lane >> 4;
    const int lswz = chunk_swz<CPR>(lrow);
    const int frag_off0 = lrow * ROWB + ((lgrp ^ lswz) << 4);
    const int frag_off1 = lrow * ROWB + ((((4 + lgrp) % CPR) ^ lswz) << 4);

    f32x4_t acc[4][FM];
#pragma unroll
    for (int fv = 0; fv < 4; ++fv)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) acc[fv][fm] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // The K-steps of stage kb: fragments of K-step 0 were read before the stage
    // began, those of K-step 1 are read before K-step 0's MFMAs. In the middle of the
    // stage every wave holds all of stage kb in registers, so after the barrier its
    // buffers take the loads of later stages, and K-step 0 of stage kb + 1 is read
    // before K-step 1's MFMAs: the MFMAs already issued cover the barrier, the load
    // issue and the LDS latency.
    // The stage loop for NL live position fragments of this wave: the fragments past
    // the last position hold padding whose products would be discarded, so their X
    // fragments are not read and their MFMAs not issued (the accumulators stay 0).
    auto stage_loop = [&](auto nl_tag) {
        constexpr int NL = decltype(nl_tag)::value;
        auto read_frags = [&](int kb, int s, u32x4_t (&a)[4], u32x4_t (&b)[NL > 0 ? NL : 1]) {
            const uint8_t* wbase = wring + (kb % NSW) * Cfg::WSTAGE + (vw * 64) * ROWB;
            const uint8_t* xbase = xring + (kb % NSX) * Cfg::XSTAGE + (mw * (BM / 2)) * ROWB;
            const int fo = s == 0 ? frag_off0 : frag_off1;
#pragma unroll
            for (int fv = 0; fv < 4; ++fv) a[fv] = *(const u32x4_t*)(wbase + fv * 16 * ROWB + fo);
#pragma unroll
            for (int fm = 0; fm < NL; ++fm) b[fm] = *(const u32x4_t*)(xbase + fm * 16 * ROWB + fo);
        };
        auto mma = [&](const u32x4_t (&a)[4], const u32x4_t (&b)[NL > 0 ? NL : 1]) {
#pragma unroll
            for (int fm = 0; fm < NL; ++fm)
#pragma unroll
                for (int fv = 0; fv < 4; ++fv)
                    acc[fv][fm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[fv]),
                                                                          __builtin_bit_cast(bf16x8_t, b[fm]),
                                                                          acc[fv][fm], 0, 0, 0);
        };
        static_assert(Cfg::KS == 2, "two K-steps per stage");

#pragma unroll
        for (int i = -NSW; i < 0; ++i) issue_mid(i);
        if (nk >= NSW) wait_vm<Cfg::PRO_WAIT>();
        else wait_vm<0>();
        stage_barrier();  // stage 0 landed in every wave
        u32x4_t a0[4], b0[NL > 0 ? NL : 1], a1[4], b1[NL > 0 ? NL : 1];
        read_frags(0, 0, a0, b0);

        for (int kb = 0; kb < nk; ++kb) {
            read_frags(kb, 1, a1, b1);
            mma(a0, b0);
            if (kb + 1 < nk) {
                // this wave's loads of stage kb + 1 are done when only later ones remain;
                // the last of those counted, W(kb + NSW - 1), exists iff kb + NSW - 1 < nk
                if (kb + NSW - 1 < nk) wait_vm<Cfg::WAIT>();
                else wait_vm<0>();
                stage_barrier();  // stage kb + 1 landed everywhere; stage kb is in registers
                issue_mid(kb);
                read_frags(kb + 1, 0, a0, b0);
            }
            mma(a1, b1);
        }
    };
    // live fragments of this wave (uniform over the wave): all of them unless the
    // tile's last positions are padding; a wave with none still issues its share of
    // the stage loads and meets every barrier
    const int nlive = min(FM, max(0, (p.Meff - m0 - mw * (BM / 2) + 15) / 16));
    with_live<FM>(nlive, stage_loop);
    __syncthreads();  // all stages read: the LDS is reused for the statistics

    // ------------------------------------------------------------- epilogue
    WStat* stats = reinterpret_cast<WStat*>(smem);  // [4][BM]
    const float ninf = -__builtin_inff();
    const float c2 = p.c2;
    const bool vec_spill = (V & 3) == 0;
    const int vbase = v0 + vw * 64;
    const int vr = min(64, v1 - vbase);  // valid rows of this wave (may be <= 0)
    const int mrows = min(BM, p.Meff - m0);
    if (p.ks > 1) {
        // K split: this slice's raw products into slice ksl of [ks, Meff, V]
        float* part = p.spill + (size_t)ksl * p.Meff * V;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int pl = mw * (BM / 2) + 16 * fm + lrow;
            if (pl < mrows) {
#pragma unroll
                for (int fv = 0; fv < 4; ++fv) {
                    const int vo = 16 * fv + 4 * lgrp;
                    if (vo < vr) {
                        float* dst = part + (size_t)(m0 + pl) * V + vbase + vo;
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
        }
        return;
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int pl = mw * (BM / 2) + 16 * fm + lrow;  // position within the tile
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
            // draft id of this position: slot j < k of a target row, or a drafter row
            int d = -1;
            if (p.drafts != nullptr) {
                if (pos < p.Mt) {
                    const int b = pos / (p.k + 1);
                    const int j = pos - b * (p.k + 1);
                    if (j < p.k) d = p.drafts[b * p.k + j];
                } else {
                    d = p.drafts[pos - p.Mt];
                }
            }
            const int dd = d - vbase;
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
        }
        if (lgrp == 0) stats[vw * BM + pl] = WStat{mx, s, bv, bi};
        __builtin_amdgcn_sched_barrier(0);  // one fragment's temporaries at a time
    }
    __syncthreads();
    if (tid < mrows) {
        WStat o = stats[tid];
#pragma unroll
        for (int w = 1; w < 4; ++w) o = merge_wstat(o, stats[w * BM + tid]);
        p.partials[(size_t)(m0 + tid) * S + vt] = Partial{o.x, o.s, o.bv, o.bi};
    }
}

// Raises the kernel's dynamic-LDS limit to its ring size, once per device: the call
// costs host time on every launch otherwise (and the limit never changes).
template <int BM, bool NTW>
hipError_t allow_lds() {
    static std::atomic<uint64_t> done{0};  // bit d: done on device d (devices past 63: every call)
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? (1ull << dev) : 0ull;
    if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
    e = hipFuncSetAttribute((const void*)wide_kernel<BM, NTW>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)WideCfg<BM>::LDS);
    if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_release);
    return e;
}

template <int BM, bool NTW>
hipError_t launch_bm_nt(const Plan& plan, const LmHeadArgs& args, hipStream_t stream) {
    const hipError_t e = allow_lds<BM, NTW>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((wide_kernel<BM, NTW>), dim3(plan.grid), dim3(NT), plan.lds, stream, args);
    return hipGetLastError();
}

template <int BM>
hipError_t launch_bm(const Plan& plan, const LmHeadArgs& args, hipStream_t stream) {
    if (plan.lds > (size_t)WideCfg<BM>::LDS) return hipErrorInvalidConfiguration;
    return (plan.MC == 1 && plan.ks == 1) ? launch_bm_nt<BM, true>(plan, args, stream)
                                          : launch_bm_nt<BM, false>(plan, args, stream);
}

}  // namespace

int wide_rows() { return BV; }

size_t wide_lds_bytes(int bm) {
    return bm == 256 ? WideCfg<256>::LDS : bm == 128 ? WideCfg<128>::LDS : WideCfg<64>::LDS;
}

namespace {

__global__ __launch_bounds__(256) void ksum_kernel(const float4* __restrict__ part, float4* __restrict__ out, int ks,
                                                   int halves, size_t n4) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
        float4 o;
        for (int h = 0; h < halves; ++h) {
            float4 a = part[(size_t)h * n4 + i];
            for (int s = 1; s < ks; ++s) {
                const float4 b = part[((size_t)s * halves + h) * n4 + i];
                a.x += b.x;
                a.y += b.y;
                a.z += b.z;
                a.w += b.w;
            }
            if (h == 0) {
                o = a;
            } else {
                o.x += a.x;
                o.y += a.y;
                o.z += a.z;
                o.w += a.w;
            }
        }
        out[i] = o;
    }
}

}  // namespace

hipError_t launch_ksum(const float* part, float* out, int ks, int halves, size_t n, hipStream_t stream) {
    const size_t n4 = n / 4;
    const unsigned int blocks = (unsigned int)std::min<size_t>((n4 + 255) / 256, 2048);
    if (blocks == 0 || ks < 1 || halves < 1) return hipSuccess;
    hipLaunchKernelGGL(ksum_kernel, dim3(blocks), dim3(256), 0, stream, reinterpret_cast<const float4*>(part),
                       reinterpret_cast<float4*>(out), ks, halves, n4);
    return hipGetLastError();
}

hipError_t launch_wide(const Plan& plan, const LmHeadArgs& args, hipStream_t stream) {
    switch (plan.nt) {
        case 64: return launch_bm<64>(plan, args, stream);
        case 128: return launch_bm<128>(plan, args, stream);
        case 256: return launch_bm<256>(plan, args, stream);
        default: return hipErrorInvalidConfiguration;
    }
}

}  // namespace mtpv
