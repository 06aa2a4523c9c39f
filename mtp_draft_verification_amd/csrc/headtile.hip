// LM-head kernel for many positions (more than 96, bf16): batched verification,
// the depth-5 chain and the large-batch rollout shape.
//
// The verify pass is a contraction l[m, v] = sum_h x[m, h] W[v, h] over every target
// and drafter position m of the batch with the one head W ("The Tiny Draft Model
// Hidden Inside Qwen", sections "One step deeper than the main model" and "How the
// draft becomes real output"). With hundreds of positions the MFMA units, not HBM,
// set the pace (same page: larger batches push the target from memory-bound toward
// compute-bound), so it is an LDS-tiled matrix product laid out for gfx950:
//
//  * persistent: one workgroup of 4 waves per compute unit walks a list of items
//    (vocabulary tile, position chunk). Workgroup w runs on XCD w % 8 and takes the
//    items of the vocabulary tiles t = w % 8 (mod 8) in order, the position chunks of
//    a tile next to each other: the workgroups of one XCD work on the chunks of the
//    same tiles at the same time, so each W tile comes from HBM once and from that
//    XCD's L2 for the other chunks;
//  * a tile is at most 2 FV x 16 vocabulary rows by 2 FM x 16 positions, each split
//    in two halves: wave w owns vocabulary half w % 2 and position half w / 2, FV x FM
//    accumulators of 16x16x32 bf16 MFMAs in AGPRs, one wave per SIMD. Two geometries:
//    FV x FM = 8 x 7 (256 x 224 tiles; per K-step a wave reads 15 fragments from LDS
//    for 56 MFMAs) and, for at most 128 positions, 6 x 4 (192 x 128) with a deeper W
//    ring;
//  * both operands are staged in LDS in K-stages of 64 hidden elements (128 bytes per
//    row) with 16-byte direct-to-LDS loads (one instruction = 8 whole 128-byte rows),
//    3 (or 5) stages of W and 2 of positions; 16-byte chunks XOR-swizzled by row so
//    the fragment reads have no bank conflicts;
//  * a wave whose position half ends early skips the padded fragments' reads and
//    MFMAs (one instance of the stage loop per live-fragment count);
//  * after the last stage each wave folds its logits into per-position statistics
//    (max of l * c2, sum of exp2, argmax), gathers the draft logits and writes the fp32
//    logits out when asked; the two vocabulary halves are merged in LDS into one
//    partial per (position, vocabulary tile);
//  * with one position chunk, the vocabulary tiles left over after whole rounds are
//    cut along K into pieces run by otherwise idle workgroups; head_tile_tail_kernel
//    adds the pieces' raw accumulators and runs the same epilogue.
// Accumulation is fp32 over all of H in a fixed order (split tiles: the pieces in
// order), no atomics.
#include "mtpv_internal.h"

#include <algorithm>
#include <atomic>
#include <climits>
#include <type_traits>

namespace mtpv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int NT = 256;         // threads per workgroup (4 waves)
constexpr int BK = 64;          // hidden elements per stage
constexpr int ROWB = BK * 2;    // LDS bytes per staged row
constexpr int CPR = BK / 8;     // 16-byte chunks per staged row
constexpr int RPI = 64 / CPR;   // rows filled by one load instruction
constexpr int PF_DIST = 5;     // L2 prefetch distance, in stages

// Tile geometry: a wave holds FV x FM accumulator fragments (vocabulary x positions),
// the workgroup's tile is 2 FV x 2 FM fragments, and the W ring has NSW stages (the
// position ring 2). The prologue issues W(0) .. W(NSW - NSX - 1), then X(0), W(NSW -
// NSX), X(1), W(NSW - 1); phase 2 of iteration i issues X(i + NSX) then W(i + NSW) (and,
// with prefetching, one prefetch after them). WAIT: loads issued after X(kb + 1) when
// iteration kb waits for stage kb + 1 (W(kb + NSW - 1), plus the prefetch issued with
// it from iteration 1 on; W(kb + 1) came before X(kb + 1)); PRO_WAIT: loads issued
// after X(0).
template <int FV_, int FM_, int NSW_>
struct Geo {
    static constexpr int FV = FV_;           // vocabulary fragments per wave
    static constexpr int FM = FM_;           // position fragments per wave
    static constexpr int VH = 16 * FV;       // vocabulary rows per half tile
    static constexpr int BV = 2 * VH;        // vocabulary rows per tile
    static constexpr int MH = 16 * FM;       // positions per half chunk
    static constexpr int BM = 2 * MH;        // positions per chunk
    static constexpr int WSTAGE = BV * ROWB;
    static constexpr int XSTAGE = BM * ROWB;
    static constexpr int NSW = NSW_;         // W stages
    static constexpr int NSX = 2;            // position stages
    static constexpr int LPW_W = BV / RPI / (NT / 64);  // W load instructions per wave per stage
    static constexpr int LPW_X = BM / RPI / (NT / 64);  // position load instructions per wave per stage
    static constexpr int STATS = 2 * BM * 16;           // per-half statistics of a chunk
    static constexpr int PF_OFF = NSW * WSTAGE + NSX * XSTAGE + STATS;  // landing zone of the L2 prefetches
    static constexpr int LDS = PF_OFF + 1024;
    static constexpr int WAIT = LPW_W;
    static constexpr int PRO_WAIT = LPW_W + (NSX - 1) * (LPW_W + LPW_X);
    static_assert(LDS <= 160 * 1024, "LDS");
    static_assert(LPW_W * RPI * (NT / 64) == BV && LPW_X * RPI * (NT / 64) == BM, "whole instructions");
    static_assert(NSW > NSX && PRO_WAIT < 64, "wait counts");
};
// 256 vocabulary rows x 224 positions, 3 W stages (152 KB); 192 x 128 with 5 W stages
// (4 in flight, 152 KB) for at most 128 positions, where the W stream sets the pace
using GeoL = Geo<8, 7, 3>;
using GeoS = Geo<6, 4, 5>;

// Sixteen zero bytes: the source of the hidden-state chunks past H in the last stage
// when H is not a multiple of 64 (a direct-to-LDS load cannot zero-fill).
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

// Workgroup barrier for the stage ring: waits for this wave's LDS reads (lgkmcnt(0))
// and meets the other waves, but not for outstanding direct-to-LDS loads
// (__syncthreads() would wait for all of them, draining the ring); the ring's own
// vmcnt wait covers the stage about to be read. The empty asm statements keep the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maxima
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Chunk swizzle of staged row r: any 16 consecutive rows read at one chunk index land
// on 16 distinct 16-byte bank groups (of a 256-byte bank row).
__device__ __forceinline__ int chunk_swz(int r) { return (r / (16 / CPR)) % CPR; }

// Calls f(std::integral_constant<int, n>) for the run-time n in [0, N].
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

// One K-step of a wave: acc[fv][fm] += A fragment fv x B fragment fm for the NL live
// position fragments, with N other instructions (LDS fragment reads, direct-to-LDS
// loads) spread evenly between the MFMAs: item i goes after MFMA (i + 1) 8 NL / (N + 1)
// - 1, so the wave issues them while the matrix pipe works. The accumulators live in
// AGPRs ("+a"): with 224 of them the compiler's own allocation moved them between
// registers around every MFMA. The MFMAs are volatile asm, which keeps their order
// against the memory instructions around them.
template <int I, int END, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < END) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, END>(f);
    }
}

template <class G, int NL, int N, typename F>
__device__ __forceinline__ void mma_step(f32x4_t (&acc)[G::FV][G::FM], const u32x4_t (&a)[G::FV],
                                         const u32x4_t (&b)[NL > 0 ? NL : 1], F&& item) {
    constexpr int FV = G::FV;
    constexpr int T = FV * NL;  // MFMAs
    if constexpr (T == 0) {
        static_for<0, N>(item);
    } else {
        static_for<0, T>([&](auto t_tag) __attribute__((always_inline)) {
            constexpr int t = decltype(t_tag)::value;
            constexpr int fm = t / FV, fv = t % FV;
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[fv][fm]) : "v"(a[fv]), "v"(b[fm]));
            static_for<0, N>([&](auto i_tag) __attribute__((always_inline)) {
                constexpr int i = decltype(i_tag)::value;
                if constexpr ((i + 1) * T / (N + 1) == t) item(i_tag);
            });
        });
    }
}

__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Where an item's rows are: vocabulary fragments [vf0, vf1) of tile vt (halves of g0
// and vf1 - vf0 - g0 fragments), position fragments [pf0, pf1) of chunk mc (halves of
// h0 and pf1 - pf0 - h0), and this wave's share (vocabulary half vh, position half mh).
struct Item {
    int vt, vf0, vf1, g0, vlast, vbase_h, vr;
    int pf0, pf1, h0, plast, pbase_h, nlive;
};

__device__ __forceinline__ Item item_at(const LmHeadArgs& p, int vt, int mc, int vh, int mh) {
    const int G = (p.V + 15) / 16;
    const int Mf = (p.Meff + 15) / 16;
    Item t;
    t.vt = vt;
    t.vf0 = (int)((long long)vt * G / p.S);
    t.vf1 = (int)((long long)(vt + 1) * G / p.S);
    t.g0 = (t.vf1 - t.vf0 + 1) / 2;
    t.vlast = min(p.V, 16 * t.vf1) - 1;
    t.vbase_h = 16 * t.vf0 + (vh ? 16 * t.g0 : 0);                               // this wave's first row
    t.vr = min(16 * (vh ? (t.vf1 - t.vf0) / 2 : t.g0), p.V - t.vbase_h);  // its valid rows (may be <= 0)
    t.pf0 = (int)((long long)mc * Mf / p.MC);
    t.pf1 = (int)((long long)(mc + 1) * Mf / p.MC);
    t.h0 = (t.pf1 - t.pf0 + 1) / 2;
    t.plast = min(p.Meff, 16 * t.pf1) - 1;
    t.pbase_h = 16 * t.pf0 + (mh ? 16 * t.h0 : 0);
    t.nlive = mh ? (t.pf1 - t.pf0) / 2 : t.h0;  // live position fragments of this wave
    return t;
}

// One position fragment fm of a wave's share of an item (accumulators a[fv] = rows
// 16 fv + 4 (lane / 16) .. + 3 of the wave's vocabulary half, positions 16 fm + lane % 16
// of its position half): the statistics of each position over those rows (max of
// l * c2, sum of exp2, argmax, combined across the four lane groups), the draft logits
// gathered and the fp32 logits written out when asked. Returns the statistics (valid in
// every lane; the caller keeps those of lane group 0).
template <class G>
__device__ __forceinline__ WStat frag_stats(const LmHeadArgs& p, const Item& t, const f32x4_t (&a)[G::FV], int fm,
                                            int lrow, int lgrp) {
    constexpr int FV = G::FV;
    const float ninf = -__builtin_inff();
    const float c2 = p.c2;
    const int V = p.V;
    const bool vec_spill = (V & 3) == 0;
    const int pos = t.pbase_h + 16 * fm + lrow;
    const bool pv = fm < t.nlive && pos <= t.plast;
    float mx = ninf, bv = ninf;
    int bi = INT_MAX;
#pragma unroll
    for (int fv = 0; fv < FV; ++fv)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int vo = 16 * fv + 4 * lgrp + q;
            const float l = a[fv][q];
            if (vo < t.vr) {
                mx = fmaxf(mx, l * c2);
                if (l > bv) {
                    bv = l;
                    bi = t.vbase_h + vo;
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
    // every argument is at most 0: the hardware exp2 (which flushes results below
    // 2^-126, far below what a sum of at least 1 can hold) gives what the library exp2
    // would, without its denormal-range guard
    float s = 0.f;
    if (mx != ninf) {
#pragma unroll
        for (int fv = 0; fv < FV; ++fv)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (16 * fv + 4 * lgrp + q < t.vr) s += __builtin_amdgcn_exp2f(a[fv][q] * c2 - mx);
    }
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    if (pv) {
        // draft id of this position: slot j < k of a target row, or a drafter row
        int d = -1;
        if (p.drafts != nullptr) {
            if (pos < p.Mt) {
                const int b = pos / (p.k + 1);
                const int jj = pos - b * (p.k + 1);
                if (jj < p.k) d = p.drafts[b * p.k + jj];
            } else {
                d = p.drafts[pos - p.Mt];
            }
        }
        const int dd = d - t.vbase_h;
        if (dd >= 0 && dd < t.vr && ((dd >> 2) & 3) == lgrp) {
            // the element without a run-time index into the accumulators
            const int fsel = dd >> 4, q = dd & 3;
            float l = 0.f;
#pragma unroll
            for (int f = 0; f < FV; ++f) {
                const f32x4_t v = a[f];
                const float e = q == 0 ? v[0] : q == 1 ? v[1] : q == 2 ? v[2] : v[3];
                l = (f == fsel) ? e : l;
            }
            p.dlogit[pos] = l;
        }
        if (p.spill != nullptr) {
#pragma unroll
            for (int fv = 0; fv < FV; ++fv) {
                const int vo = 16 * fv + 4 * lgrp;
                if (vo < t.vr) {
                    float* dst = p.spill + (size_t)pos * V + t.vbase_h + vo;
                    if (vec_spill && vo + 3 < t.vr) {
                        *(f32x4_t*)dst = a[fv];
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            if (vo + q < t.vr) dst[q] = a[fv][q];
                    }
                }
            }
        }
    }
    return WStat{mx, s, bv, bi};
}

// After the last stage of an item: every position fragment of each wave through
// frag_stats, then the two vocabulary halves merged in LDS into one partial per
// (position, vocabulary tile). Ends with the workgroup's LDS barrier.
template <class G>
__device__ __forceinline__ void epilogue(const LmHeadArgs& p, const Item& t, f32x4_t (&acc)[G::FV][G::FM],
                                         WStat* stats, int tid, int vh, int mh) {
    constexpr int FV = G::FV, FM = G::FM, MH = G::MH, BM = G::BM;
    const int lane = tid & 63;
    const int lrow = lane & 15;
    const int lgrp = lane >> 4;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        f32x4_t a[FV];
#pragma unroll
        for (int fv = 0; fv < FV; ++fv) a[fv] = acc[fv][fm];
        const WStat w = frag_stats<G>(p, t, a, fm, lrow, lgrp);
        if (lgrp == 0) stats[vh * BM + mh * MH + 16 * fm + lrow] = w;
        __builtin_amdgcn_sched_barrier(0);  // one fragment's temporaries at a time
    }
    // the statistics are in LDS: a barrier on LDS only, so the spill stores keep
    // draining while the workgroup goes on (__syncthreads() would wait for them)
    stage_barrier();
    // merge the two vocabulary halves: one partial per (position, tile)
    if (tid < BM) {
        const int hm = tid < MH ? 0 : 1;
        const int r = tid - hm * MH;
        const int pos = 16 * t.pf0 + (hm ? 16 * t.h0 : 0) + r;
        const int live = hm ? (t.pf1 - t.pf0) / 2 : t.h0;
        if (r < 16 * live && pos <= t.plast) {
            const WStat o = merge_wstat(stats[tid], stats[BM + tid]);
            p.partials[(size_t)pos * p.S + t.vt] = Partial{o.x, o.s, o.bv, o.bi};
        }
    }
    stage_barrier();  // statistics read: the next item may write them
}

// Raw accumulators of one K piece of a split tile with fl live position fragments per
// wave: register (fv, fm < fl) of thread tid at float4 (fv * fl + fm) * NT + tid of the
// piece (each store instruction writes 4 KB in a row).
template <class G>
__device__ __forceinline__ size_t piece_float4(int fl) { return (size_t)G::FV * fl * NT; }

// NTW: each W tile is read by one workgroup only (one position chunk), so its loads
// carry the non-temporal hint. PF: several chunks share each W tile and each chunk is
// shared by several tiles of a round, so every workgroup brings its share of both into
// L2 PF_DIST stages ahead (one 4-byte load per 128-byte line; the loads of the sharers
// then hit L2 instead of all waiting on the same misses). HFULL: H % 64 == 0, no
// stage reads past the end of a row.
//
// Items: the whole-K items of tiles [0, S') (S' = tail_f when tiles are split, else
// S), then, when tiles are split, workgroup q < tail_r * tail_ks takes K piece q /
// tail_r of tile tail_f + q % tail_r: the stages [piece * nk / ks, (piece + 1) * nk /
// ks), whose raw accumulators go to p.tail for head_tile_tail_kernel.
template <class G, bool NTW, bool PF, bool HFULL>
__global__ __launch_bounds__(NT, 1) void head_tile_kernel(LmHeadArgs p) {
    constexpr int FV = G::FV, FM = G::FM, VH = G::VH, MH = G::MH;
    constexpr int WSTAGE = G::WSTAGE, XSTAGE = G::XSTAGE, NSW = G::NSW, NSX = G::NSX;
    constexpr int LPW_W = G::LPW_W, LPW_X = G::LPW_X, PF_OFF = G::PF_OFF, WAIT = G::WAIT, PRO_WAIT = G::PRO_WAIT;
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    uint8_t* wring = smem;                                     // NSW stages of BV rows
    uint8_t* xring = smem + NSW * WSTAGE;                      // NSX stages of BM rows
    WStat* stats = reinterpret_cast<WStat*>(smem + NSW * WSTAGE + NSX * XSTAGE);  // [2][BM]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS addresses in SGPRs
    const int vh = wave & 1;   // vocabulary half of the tile
    const int mh = wave >> 1;  // position half of the chunk
    const int H = p.H, MC = p.MC;
    const int nk = (H + BK - 1) / BK;
    const size_t rowbytes = (size_t)H * 2;
    if (blockIdx.x == 0 && tid == 0 && p.err != nullptr) *p.err = 0;

    // this workgroup's whole-K items: XCD x = blockIdx.x % 8 owns tiles x, x + 8, ...;
    // item j of the XCD is (tile x + 8 (j / MC), chunk j % MC); the XCD's workgroups
    // take j = c, c + per_xcd, ...
    const int x = blockIdx.x & 7;
    const int c = blockIdx.x >> 3;
    const int per_xcd = gridDim.x >> 3;
    const int S_whole = p.tail_r > 0 ? p.tail_f : p.S;
    const int nvt_x = S_whole > x ? (S_whole - x + 7) / 8 : 0;
    const int nx = nvt_x * MC;

    const int lrow = lane & 15;
    const int lgrp = lane >> 4;
    const int lswz = chunk_swz(lrow);
    const int frag_off0 = lrow * ROWB + ((lgrp ^ lswz) << 4);
    const int frag_off1 = lrow * ROWB + ((((4 + lgrp) % CPR) ^ lswz) << 4);

    // one item: stages [k0, k0 + nki) of (tile vt, chunk mc); piece >= 0: a K piece of a
    // split tile (raw accumulators out, no epilogue)
    auto run_item = [&](int vt, int mc, int k0, int nki, int piece) __attribute__((always_inline)) {
        const Item t = item_at(p, vt, mc, vh, mh);
        const int vf0 = t.vf0, g0 = t.g0, vlast = t.vlast;
        const int pf0 = t.pf0, h0 = t.h0, plast = t.plast;

        // stage loads: W instruction i of this wave fills staged rows 8 LPW_W wave + 8 i
        // .. + 7 (one vocabulary half per pair of waves), position instruction i fills
        // rows 8 LPW_X wave + 8 i .. + 7 (waves 0, 1: first half, 2, 3: second half). Lane
        // l writes slot l % CPR of row 8 i + l / CPR of its block and fetches chunk
        // (l % CPR) ^ swz(row); swz(row) = (4 LPW wave + 4 i + l / 16) % 8.
        // Rows past the valid ones re-read the last valid row (results ignored).
        const int lr = lane / CPR, lc = lane % CPR;
        const int w_v0 = 16 * vf0 + (wave >= 2 ? 16 * g0 : 0) + 8 * LPW_W * (wave & 1) + lr;  // row of instruction 0
        const int x_m0 = 16 * pf0 + (wave >= 2 ? 16 * h0 : 0) + 8 * LPW_X * (wave & 1) + lr;
        // load instruction i of the W (position) ring: the data of stage k0 + kd into the
        // buffer of stage ks (they differ only past the last stage, where a free buffer
        // takes a repeat of the last stage so that every phase issues the same loads)
        auto load_w = [&](int kd, int ks, int i) __attribute__((always_inline)) {
            uint8_t* dst = wring + (ks % NSW) * WSTAGE + wave * LPW_W * 1024;
            const int chunk = lc ^ ((4 * LPW_W * wave + 4 * i + (lane >> 4)) & 7);
            const int k = (k0 + kd) * BK + 8 * chunk;
            const uint8_t* row = p.w + (size_t)min(w_v0 + 8 * i, vlast) * rowbytes;
            const uint8_t* src = (HFULL || k < H) ? row + (size_t)k * 2 : row;
            __builtin_amdgcn_global_load_lds(src, (lds_void*)(dst + i * 1024), 16, 0, NTW ? 2 : 0);
        };
        auto load_x = [&](int kd, int ks, int i) __attribute__((always_inline)) {
            uint8_t* dst = xring + (ks % NSX) * XSTAGE + wave * LPW_X * 1024;
            const int chunk = lc ^ ((4 * LPW_X * wave + 4 * i + (lane >> 4)) & 7);
            const int k = (k0 + kd) * BK + 8 * chunk;
            const int m = min(x_m0 + 8 * i, plast);
            const uint8_t* row = m < p.Mt ? p.xt + (size_t)m * rowbytes : p.xd + (size_t)(m - p.Mt) * rowbytes;
            const uint8_t* src = (HFULL || k < H) ? row + (size_t)k * 2 : reinterpret_cast<const uint8_t*>(kZero16);
            __builtin_amdgcn_global_load_lds(src, (lds_void*)(dst + i * 1024), 16, 0, 0);
        };
        // prefetch shares: rows [wlo, whi) of the W tile (1 / MC of them, by chunk) and
        // rows [xlo, xhi) of the position chunk (1 / nsh of them, nsh = items of a round
        // with this chunk, by the tile's place in the round); one 128-byte line of each
        // row per stage, spread over the lanes of the four waves
        const int nrows_t = min(p.V, 16 * t.vf1) - 16 * vf0;
        const int wlo = nrows_t * mc / MC, whi = nrows_t * (mc + 1) / MC;
        const int nsh = max(1, per_xcd / MC);
        const int tr = (vt / 8) % nsh;
        const int nrows_c = plast + 1 - 16 * pf0;
        const int xlo = nrows_c * tr / nsh, xhi = nrows_c * (tr + 1) / nsh;
        auto prefetch = [&](int kd) __attribute__((always_inline)) {
            const int q = wave * 64 + lane;
            const int nw = whi - wlo;
            const uint8_t* src;
            if (q < nw) {
                src = p.w + (size_t)(16 * vf0 + wlo + q) * rowbytes;
            } else if (q < nw + (xhi - xlo)) {
                const int m = 16 * pf0 + xlo + (q - nw);
                src = m < p.Mt ? p.xt + (size_t)m * rowbytes : p.xd + (size_t)(m - p.Mt) * rowbytes;
            } else {
                src = p.w + (size_t)(16 * vf0) * rowbytes;
            }
            src += (size_t)(k0 + kd) * BK * 2;
            __builtin_amdgcn_global_load_lds(src, (lds_void*)(smem + PF_OFF + wave * 256), 4, 0, 0);
        };
        auto issue_w = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < LPW_W; ++i) load_w(kb, kb, i);
        };
        auto issue_x = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < LPW_X; ++i) load_x(kb, kb, i);
        };
        auto issue_mid = [&](int i) __attribute__((always_inline)) {
            if (i + NSX >= 0 && i + NSX < nki) issue_x(i + NSX);
            if (i + NSW >= 0 && i + NSW < nki) issue_w(i + NSW);
        };

        f32x4_t acc[FV][FM];
#pragma unroll
        for (int fv = 0; fv < FV; ++fv)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) acc[fv][fm] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        // Stage loop for NL live position fragments. Registers X hold the fragments of
        // K-step 0 of stage kb, Y those of K-step 1. Phase 1: the MFMAs on X, with the
        // reads of Y between them. Then this wave's loads of stage kb + 1 are waited for
        // and the workgroup meets (every wave has read stage kb and holds it in
        // registers). Phase 2: the MFMAs on Y, with the loads of later stages into
        // stage kb's buffers and the reads of X for stage kb + 1 between them. Each
        // phase ends with lgkmcnt(0), so the next phase's operands are complete.
        auto stage_loop = [&](auto nl_tag) __attribute__((always_inline)) {
            constexpr int NL = decltype(nl_tag)::value;
            constexpr int NB = NL > 0 ? NL : 1;
            constexpr int NR = FV + NL;  // fragment reads of one K-step
            auto rd = [&](int kb, int s, u32x4_t (&a)[FV], u32x4_t (&b)[NB], auto i_tag) {
                constexpr int i = decltype(i_tag)::value;
                const int fo = s == 0 ? frag_off0 : frag_off1;
                if constexpr (i < FV) {
                    a[i] = *(const u32x4_t*)(wring + (kb % NSW) * WSTAGE + (vh * VH + i * 16) * ROWB + fo);
                } else if constexpr (i - FV < NL) {
                    b[i - FV] = *(const u32x4_t*)(xring + (kb % NSX) * XSTAGE + (mh * MH + (i - FV) * 16) * ROWB + fo);
                }
            };
#pragma unroll
            for (int i = -NSW; i < 0; ++i) issue_mid(i);
            if (nki >= NSW) wait_vm<PRO_WAIT>();
            else wait_vm<0>();
            stage_barrier();  // stage 0 landed in every wave
            u32x4_t a0[FV], b0[NB], a1[FV], b1[NB];
            static_for<0, NR>([&](auto i) __attribute__((always_inline)) { rd(0, 0, a0, b0, i); });
            wait_lgkm0();
            for (int kb = 0; kb < nki; ++kb) {
                mma_step<G, NL, NR>(acc, a0, b0, [&](auto i) __attribute__((always_inline)) { rd(kb, 1, a1, b1, i); });
                wait_lgkm0();
                if (kb + 1 < nki) {
                    // this wave's loads of stage kb + 1 are done when only later ones remain:
                    // after X(kb + 1) come W(kb + 2) (issued by the prologue or by phase 2 of
                    // iteration kb - 1, always) and, from iteration 1 on, that phase's prefetch
                    if (kb == 0 && NSW - 1 >= nki) wait_vm<0>();
                    else if (PF && kb >= 1) wait_vm<WAIT + 1>();
                    else wait_vm<WAIT>();
                }
                // stage kb + 1 landed everywhere, and every wave holds stage kb in registers,
                // so its buffers may be refilled (also after the last stage: the repeat loads
                // below must not land while another wave still reads them)
                stage_barrier();
                // Every phase 2 issues the same loads (past the last stage, repeats of the last
                // stage into buffers no longer read), so the wait counts above hold; after the
                // last stage the reads below fetch stale LDS, never used.
                const int kx = min(kb + NSX, nki - 1), kw = min(kb + NSW, nki - 1);
                mma_step<G, NL, LPW_X + LPW_W + NR>(acc, a1, b1, [&](auto i_tag) __attribute__((always_inline)) {
                    constexpr int i = decltype(i_tag)::value;
                    if constexpr (i < LPW_X) {
                        load_x(kx, kb + NSX, i);
                    } else if constexpr (i < LPW_X + LPW_W) {
                        load_w(kw, kb + NSW, i - LPW_X);
                        if constexpr (PF && i == LPW_X + LPW_W - 1) prefetch(min(kb + PF_DIST, nki - 1));
                    } else {
                        rd(kb + 1, 0, a0, b0, std::integral_constant<int, i - LPW_X - LPW_W>{});
                    }
                });
                wait_lgkm0();
            }
            // the accumulators are read by VALU instructions next: wait out the last
            // MFMAs (the compiler does not see inside the asm)
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
            if (piece >= 0) {
                // a K piece: this wave's live accumulators out
                f32x4_t* dst = reinterpret_cast<f32x4_t*>(p.tail) + (size_t)piece * piece_float4<G>(p.tail_fm) + tid;
                const int fl = p.tail_fm;
#pragma unroll
                for (int fv = 0; fv < FV; ++fv)
#pragma unroll
                    for (int fm = 0; fm < NL; ++fm) dst[(fv * fl + fm) * NT] = acc[fv][fm];
            }
        };
        with_live<FM>(t.nlive, stage_loop);

        if (piece < 0) epilogue<G>(p, t, acc, stats, tid, vh, mh);
        else stage_barrier();  // every wave is past its stage loop
    };

    for (int j = c; j < nx; j += per_xcd) run_item(x + 8 * (j / MC), j - (j / MC) * MC, 0, nk, -1);
    if (p.tail_r > 0 && (int)blockIdx.x < p.tail_r * p.tail_ks) {
        const int q = blockIdx.x;
        const int kp = q / p.tail_r;
        const int kbeg = (int)((long long)kp * nk / p.tail_ks), kend = (int)((long long)(kp + 1) * nk / p.tail_ks);
        run_item(p.tail_f + q % p.tail_r, 0, kbeg, kend - kbeg, q);
    }
    // no direct-to-LDS load may still be landing when the workgroup's LDS is released
    wait_vm<0>();
}

// Finishes the split tiles, one position fragment of one position half of a tile per
// workgroup of two waves (the two vocabulary halves): workgroup ((u * 2 + mh) * FM + fm)
// takes tile tail_f + u. Each thread adds, in piece order, the raw accumulators that the
// head kernel's thread (vh + 2 mh) * 64 + lane held for that fragment, runs frag_stats on
// the sums and the halves are merged as in the head kernel's epilogue.
template <class G>
__global__ __launch_bounds__(128) void head_tile_tail_kernel(LmHeadArgs p) {
    constexpr int FV = G::FV, FM = G::FM;
    __shared__ WStat stats[2][16];
    const int u = blockIdx.x / (2 * FM);
    const int mh = (blockIdx.x / FM) % 2;
    const int fm = blockIdx.x % FM;
    const int vh = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const Item t = item_at(p, p.tail_f + u, 0, vh, mh);
    if (fm >= t.nlive) return;  // the same for both waves of the workgroup
    const int tid = (vh + 2 * mh) * 64 + lane;
    const int fl = p.tail_fm;
    f32x4_t v[4][FV];
    f32x4_t a[FV];
#pragma unroll
    for (int fv = 0; fv < FV; ++fv) a[fv] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < p.tail_ks; k0 += 4) {
        // up to 4 pieces' loads in flight, then their sums in piece order
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
            if (k0 + kq < p.tail_ks) {
                const f32x4_t* src = reinterpret_cast<const f32x4_t*>(p.tail) +
                                     (size_t)(u + (k0 + kq) * p.tail_r) * piece_float4<G>(fl) + fm * NT + tid;
#pragma unroll
                for (int fv = 0; fv < FV; ++fv) v[kq][fv] = src[(size_t)fv * fl * NT];
            }
        }
#pragma unroll
        for (int kq = 0; kq < 4; ++kq)
            if (k0 + kq < p.tail_ks) {
#pragma unroll
                for (int fv = 0; fv < FV; ++fv) a[fv] += v[kq][fv];
            }
    }
    const WStat w = frag_stats<G>(p, t, a, fm, lane & 15, lane >> 4);
    if ((lane >> 4) == 0) stats[vh][lane & 15] = w;
    __syncthreads();
    if (threadIdx.x < 16) {
        const int r = threadIdx.x;
        const int pos = t.pbase_h + 16 * fm + r;
        if (pos <= t.plast) {
            const WStat o = merge_wstat(stats[0][r], stats[1][r]);
            p.partials[(size_t)pos * p.S + t.vt] = Partial{o.x, o.s, o.bv, o.bi};
        }
    }
}

// Raises the kernel's dynamic-LDS limit, once per device.
template <class G, bool NTW, bool PF, bool HFULL>
hipError_t allow_lds() {
    static std::atomic<uint64_t> done{0};  // bit d: done on device d (devices past 63: every call)
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? (1ull << dev) : 0ull;
    if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
    e = hipFuncSetAttribute((const void*)head_tile_kernel<G, NTW, PF, HFULL>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            G::LDS);
    if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_release);
    return e;
}

template <class G, bool NTW, bool PF, bool HFULL>
hipError_t launch_t(const Plan& plan, const LmHeadArgs& args, hipStream_t stream) {
    const hipError_t e = allow_lds<G, NTW, PF, HFULL>();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((head_tile_kernel<G, NTW, PF, HFULL>), dim3(plan.grid), dim3(NT), G::LDS, stream, args);
    if (args.tail_r > 0) {
        const hipError_t le = hipGetLastError();
        if (le != hipSuccess) return le;
        hipLaunchKernelGGL(head_tile_tail_kernel<G>, dim3(args.tail_r * 2 * G::FM), dim3(128), 0, stream, args);
    }
    return hipGetLastError();
}

template <bool HFULL>
hipError_t launch_h(const Plan& plan, const LmHeadArgs& args, hipStream_t stream) {
    // one chunk per tile: W streams once (non-temporal); several: shared, prefetched.
    // The small geometry serves one chunk only.
    if (plan.geo == 1) return launch_t<GeoS, true, false, HFULL>(plan, args, stream);
    return plan.MC == 1 ? launch_t<GeoL, true, false, HFULL>(plan, args, stream)
                        : launch_t<GeoL, false, true, HFULL>(plan, args, stream);
}

template <class G>
bool geometry_fits(const Plan& plan, const LmHeadArgs& args) {
    const int G16 = (plan.V + 15) / 16, Mf = (plan.Meff + 15) / 16;
    // every tile at most 2 FV fragments, every chunk at most 2 FM
    return (long long)plan.S * 2 * G::FV >= G16 && (long long)plan.MC * 2 * G::FM >= Mf &&
           (args.tail_r == 0 || (args.tail_fm >= 1 && args.tail_fm <= G::FM));
}

}  // namespace

int head_tile_max_positions(int geo) { return geo == 1 ? GeoS::BM : GeoL::BM; }

int head_tile_rows(int geo) { return geo == 1 ? GeoS::BV : GeoL::BV; }

size_t head_tile_piece_bytes(int fm, int geo) { return (size_t)(geo == 1 ? GeoS::FV : GeoL::FV) * fm * NT * 16; }

hipError_t launch_head_tile(const Plan& plan, const LmHeadArgs& args, hipStream_t stream) {
    if (plan.grid % 8 != 0 || plan.grid < 8) return hipErrorInvalidConfiguration;
    // split tiles: one chunk, every piece a workgroup of the grid, a non-empty K range each
    if (args.tail_r > 0 && (plan.MC != 1 || args.tail == nullptr || args.tail_ks < 2 ||
                            args.tail_r * args.tail_ks > plan.grid || args.tail_f + args.tail_r != plan.S ||
                            args.tail_ks > (plan.H + BK - 1) / BK))
        return hipErrorInvalidConfiguration;
    if (plan.geo == 1 ? (plan.MC != 1 || !geometry_fits<GeoS>(plan, args)) : !geometry_fits<GeoL>(plan, args))
        return hipErrorInvalidConfiguration;
    return plan.H % BK == 0 ? launch_h<true>(plan, args, stream) : launch_h<false>(plan, args, stream);
}

}  // namespace mtpv
