// LM-head streaming kernel for few positions (at most 16 rows): the decode regime.
//
// With a handful of positions the step is pure weight streaming: every byte of
// W_lm [V, H] is read once and feeds only 2*M flops ("Speculative Decoding and
// MTP: Why Guessing Is Free", section "The part that got me": one read of the
// weights serves every position of the pass). What decides the speed is how the
// loads meet HBM: a load instruction that touches many rows with short runs each
// leaves DRAM pages half used. Here each wave streams 4 vocabulary rows at a time,
// 256 contiguous bytes of each row per 16-byte load instruction, 16 instructions
// in flight (4 KB of each row outstanding), with non-temporal loads.
//
// The contraction runs on the 16-block MFMA v_mfma_f32_4x4x4_16b_bf16 (fp32
// heads: v_mfma_f32_4x4x1_16b_f32). Block b of lane (i + 4b) carries row i's
// elements [16 b, 16 b + 16) bytes of the current 256-byte step; the matching B
// lane (j + 4b) carries position j's same elements; block b accumulates the
// partial dot products over its residue class of K, and a sum over the 16 blocks at
// the end of each 4-row tile (DPP row rotations, then permlane swaps) gives the full
// logits. Accumulation is fp32 over all of H, fixed order.
//
// The epilogue runs once per 4-row tile, in the middle of the stream (the next
// tile's loads are already in flight): running max of l*c2 (log2 units), sum of
// exp2, argmax (lowest id on ties), the draft token's logit, and optionally the
// fp32 logits for the sampling pass. At the end the four waves' statistics are
// merged in LDS into one partial per (position, workgroup).
#include "mtpv_internal.h"

#include <climits>

namespace mtpv {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

template <int ES>
struct Mma4;

template <>
struct Mma4<2> {  // bf16: 8 elements per 16 bytes = two 4x4x4 blocks-of-K steps
    static constexpr int EPV = 8;
    __device__ __forceinline__ static f32x4_t run(u32x4_t a, u32x4_t b, f32x4_t c) {
        typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t a0{a[0], a[1]}, a1{a[2], a[3]}, b0{b[0], b[1]}, b1{b[2], b[3]};
        c = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4_t, a0), __builtin_bit_cast(s16x4_t, b0),
                                                   c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4_t, a1), __builtin_bit_cast(s16x4_t, b1),
                                                   c, 0, 0, 0);
        return c;
    }
};

template <>
struct Mma4<4> {  // fp32: 4 elements per 16 bytes = four 4x4x1 steps
    static constexpr int EPV = 4;
    __device__ __forceinline__ static f32x4_t run(u32x4_t a, u32x4_t b, f32x4_t c) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            c = __builtin_amdgcn_mfma_f32_4x4x1f32(__uint_as_float(a[e]), __uint_as_float(b[e]), c, 0, 0, 0);
        return c;
    }
};

__device__ __forceinline__ u32x4_t load_w(const uint8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

struct Stat {
    float x, s, bv;
    int bi;
};

__device__ __forceinline__ Stat merge_stat(Stat a, Stat b) {
    const float ninf = -__builtin_inff();
    Stat o;
    o.x = fmaxf(a.x, b.x);
    const float sa = (a.x == ninf) ? 0.f : a.s * exp2f(a.x - o.x);
    const float sb = (b.x == ninf) ? 0.f : b.s * exp2f(b.x - o.x);
    o.s = sa + sb;
    const bool take_b = (b.bv > a.bv) || (b.bv == a.bv && b.bi < a.bi);
    o.bv = take_b ? b.bv : a.bv;
    o.bi = take_b ? b.bi : a.bi;
    return o;
}

// Sum over the 16 K-blocks of the 16-block 4x4x4 layout (lane = i + 4 b): rotating
// by 4 and by 8 lanes inside each 16-lane row adds the row's four blocks and keeps
// i = lane % 4; then row pairs and wave halves are swapped in and added. Every
// lane ends with the same total for its i, added in the same order.
__device__ __forceinline__ float block_sum16(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));  // row_ror:4
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror:8
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// NG groups of 4 positions, PF steps of W in flight per wave. The grid is sized
// to what the GPU holds at once (every workgroup resident, no second round). The
// ceil(V / 4) row tiles are dealt to the waves round by round: in round r wave w
// takes tile r * n + w (n waves in the grid), so at any moment all waves stream
// from one window of consecutive tiles; the tiles of the last, partial round are
// spread evenly over the waves. Each workgroup writes one partial per position.
//
// A step's load address is a wave-uniform base (the tile's first row and the K
// step, in scalar registers) plus a per-lane offset that changes only between
// tiles, so the step loop spends no vector instructions on W addresses.
template <int ES, int NG, int PF>
__global__ __launch_bounds__(256) void skinny_kernel(LmHeadArgs p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int EPV = Mma4<ES>::EPV;
    constexpr int KS = 16 * EPV;  // hidden elements per step
    constexpr int SB = KS * ES;   // bytes of a row per step (256)
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 3;   // A: row within the tile; B / D: position within the group
    const int lb = lane >> 2;  // block: 16-byte segment of the step
    const int H = p.H;
    const int V = p.V;
    const int vb = blockIdx.x;
    const int ntile = (V + 3) / 4;
    const int nw = 4 * gridDim.x;
    const int gw = vb * 4 + wave;
    const int full = ntile / nw;          // rounds in which every wave takes a tile
    const int rem = ntile - full * nw;    // tiles of the last, partial round
    const int last_tile = full * nw + (int)((long long)gw * rem / nw);
    const bool has_last = (int)((long long)(gw + 1) * rem / nw) > (int)((long long)gw * rem / nw);
    const int T = full + (has_last ? 1 : 0);  // tiles of this wave (may be 0)
    auto tile_row = [&](int t) { return 4 * (t < full ? t * nw + gw : last_tile); };
    const int rowbytes = H * ES;  // < 64 KB: the staged rows fit the LDS budget
    const int nsteps = (H + KS - 1) / KS;
    const int total = max(T, 1) * nsteps;  // a wave without tiles streams nothing new
    const int mrows = p.Meff;  // all positions fit one workgroup here
    const int pitch = nsteps * SB + 64;

    if (vb == 0 && tid == 0 && p.err != nullptr) *p.err = 0;

    // Steps advance through K of the current tile, then on to the next tile; past
    // the last step the address stays on the last step (a re-read, no new HBM
    // traffic). Each wave walks K starting at its own rotation `rot` (any order of K
    // gives the same dot products): waves whose rows sit at power-of-two strides
    // would otherwise hit the same HBM channels at the same moment. Rows past V
    // re-read row V - 1; in the last step of a row that is not a whole number of
    // steps long, segments past H re-read the row's last 16 bytes.
    const int rot = p.rotate ? (int)(((unsigned)gw * 5u) % (unsigned)nsteps) : 0;
    const bool ragged = nsteps * KS != H;
    const unsigned seg = (unsigned)(lb * 16);
    const unsigned seg_last = (unsigned)min(lb * 16, rowbytes - 16 - (nsteps - 1) * SB);
    auto row_off = [&](int row0) { return (unsigned)(min(row0 + li, V - 1) - row0) * (unsigned)rowbytes; };
    int lt = 0, lks = 0;
    int lrow0 = tile_row(0);
    unsigned loff = row_off(lrow0);
    auto next_w = [&]() -> u32x4_t {
        int kstep = lks + rot;
        if (kstep >= nsteps) kstep -= nsteps;
        const uint8_t* base = p.w + (size_t)lrow0 * rowbytes + (size_t)kstep * SB;  // wave-uniform
        const unsigned off = loff + ((ragged && kstep == nsteps - 1) ? seg_last : seg);
        const u32x4_t r = load_w(base + off);
        if (lks + 1 < nsteps) {
            ++lks;
        } else if (lt + 1 < T) {
            lks = 0;
            ++lt;
            lrow0 = tile_row(lt);
            loff = row_off(lrow0);
        }
        return r;
    };

    // The ring is filled unconditionally: a wave without tiles (T = 0) re-reads its
    // would-be first tile, which lies inside W (tile_row(0) < 4 * ntile).
    u32x4_t wb[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) wb[i] = next_w();

    // per-lane position bookkeeping: position m = 4g + li (read before the staging
    // below, whose wait covers these loads too)
    int dtok[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const int m = 4 * g + li;
        int d = -1;
        if (m < mrows && p.drafts != nullptr) {
            if (m < p.Mt) {
                const int b = m / (p.k + 1);
                const int j = m - b * (p.k + 1);
                d = (j < p.k) ? p.drafts[b * p.k + j] : -1;
            } else {
                d = p.drafts[m - p.Mt];
            }
        }
        dtok[g] = d;
    }

    // Stage all positions' hidden states, zero-filled to nsteps * KS elements.
    {
        const int vpr = nsteps * KS / EPV;
        for (int e = tid; e < mrows * vpr; e += 256) {
            const int r = e / vpr;
            const int c = e - r * vpr;
            const int kk = c * EPV;
            u32x4_t val = u32x4_t{0u, 0u, 0u, 0u};
            if (kk < H) {
                const uint8_t* src = r < p.Mt ? p.xt + (size_t)r * rowbytes : p.xd + (size_t)(r - p.Mt) * rowbytes;
                val = *(const u32x4_t*)(src + (size_t)kk * ES);
            }
            *(u32x4_t*)(smem + r * pitch + c * 16) = val;
        }
    }
    // Every load issued so far (the ring, the draft ids, the staging) is complete
    // here in practice: the staging waits for its own loads, which were issued last.
    // Saying so explicitly keeps the compiler from waiting for the draft ids inside
    // the step loop, where that wait would drain the ring.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt at their maxima

    const float ninf = -__builtin_inff();
    Stat st[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) st[g] = Stat{ninf, 0.f, ninf, INT_MAX};
    f32x4_t acc[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) acc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    __syncthreads();

    const float c2 = p.c2;
    const bool vec_spill = (V & 3) == 0;
    // This lane's B fragment at K step 0, per group. A lane of a missing position
    // (past the last one in a partial group of 4) reads the last position's row: the
    // MFMA keeps B's columns apart, so that column's logits are computed and ignored.
    unsigned xoff[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) xoff[g] = (unsigned)(min(4 * g + li, mrows - 1) * pitch) + seg;

    auto consume = [&](const u32x4_t& w, int ks) {
        const uint8_t* xs = smem + ks * SB;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const u32x4_t x = *(const u32x4_t*)(xs + xoff[g]);
            acc[g] = Mma4<ES>::run(w, x, acc[g]);
        }
    };

    // End of a 4-row tile: sum the 16 K-blocks, update the running statistics.
    auto finish_tile = [&](int t) {
        const int v0 = tile_row(t);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            f32x4_t a;
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] = block_sum16(acc[g][e]);
            acc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            const int m = 4 * g + li;
            float tx = ninf;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (v0 + e < V) tx = fmaxf(tx, a[e] * c2);
            if (m < mrows && tx != ninf) {  // else: no position here, or tile past V
                Stat s = st[g];
                const float nx = fmaxf(s.x, tx);
                float sum = (s.x == ninf) ? 0.f : s.s * exp2f(s.x - nx);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int v = v0 + e;
                    if (v < V) {
                        sum += exp2f(a[e] * c2 - nx);
                        if (a[e] > s.bv) {
                            s.bv = a[e];
                            s.bi = v;
                        }
                    }
                }
                s.x = nx;
                s.s = sum;
                st[g] = s;
                if (lb == 0) {
                    const int d = dtok[g];
                    if (d >= v0 && d < v0 + 4) {
                        const int t = d - v0;
                        p.dlogit[m] = t == 0 ? a[0] : t == 1 ? a[1] : t == 2 ? a[2] : a[3];
                    }
                    if (p.spill != nullptr) {
                        float* dst = p.spill + (size_t)m * V + v0;
                        if (vec_spill && v0 + 3 < V) {
                            *(f32x4_t*)dst = a;
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (v0 + e < V) dst[e] = a[e];
                        }
                    }
                }
            }
        }
    };

    // ks counts steps within the tile; kr is the K step they map to after rotation.
    // One loop covers every step: the steps of the last batch past `work` consume
    // nothing, and their loads (re-reads of the last step) are never waited for.
    int ks = 0, kr = rot, t = 0;
    const int work = T > 0 ? total : 0;
    for (int s = 0; s < work; s += PF) {
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            const bool live = s + i < work;  // wave-uniform
            if (live) consume(wb[i], kr);
            wb[i] = next_w();
            if (live) {
                if (++kr == nsteps) kr = 0;
                if (++ks == nsteps) {
                    finish_tile(t);
                    ks = 0;
                    ++t;
                }
            }
        }
    }

    // merge the four waves' statistics per position (positions < 4 * NG <= 16)
    __syncthreads();
    Stat* red = reinterpret_cast<Stat*>(smem);  // [4][16]
    if (lb == 0) {
#pragma unroll
        for (int g = 0; g < NG; ++g) red[wave * 16 + 4 * g + li] = st[g];
    }
    __syncthreads();
    if (tid < mrows) {
        Stat o = red[tid];
#pragma unroll
        for (int w = 1; w < 4; ++w) o = merge_stat(o, red[w * 16 + tid]);
        p.partials[(size_t)tid * p.S + vb] = Partial{o.x, o.s, o.bv, o.bi};
    }
}

template <int ES, int NG>
hipError_t launch_ng(const Plan& plan, const LmHeadArgs& args, hipStream_t stream) {
    hipLaunchKernelGGL((skinny_kernel<ES, NG, 16>), dim3(plan.grid), dim3(256), plan.lds, stream, args);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_skinny(const Plan& plan, const LmHeadArgs& args, hipStream_t stream) {
    const int ng = (plan.Meff + 3) / 4;
    if (plan.es == 2) {
        switch (ng) {
            case 1: return launch_ng<2, 1>(plan, args, stream);
            case 2: return launch_ng<2, 2>(plan, args, stream);
            case 3: return launch_ng<2, 3>(plan, args, stream);
            case 4: return launch_ng<2, 4>(plan, args, stream);
            default: break;
        }
    } else {
        switch (ng) {
            case 1: return launch_ng<4, 1>(plan, args, stream);
            case 2: return launch_ng<4, 2>(plan, args, stream);
            case 3: return launch_ng<4, 3>(plan, args, stream);
            case 4: return launch_ng<4, 4>(plan, args, stream);
            default: break;
        }
    }
    return hipErrorInvalidConfiguration;
}

}  // namespace mtpv
