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
// partial dot products over its residue class of K, and a lane butterfly over the
// 16 blocks at the end of each 4-row tile gives the full logits. Accumulation is
// fp32 over all of H, fixed order.
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

// NG groups of 4 positions, PF steps of W in flight per wave. The grid is sized
// to what the GPU holds at once (every workgroup resident, no second round) and
// the ceil(V / 4) row tiles are split as evenly as possible over all its waves:
// wave w owns tiles [w * nt / nw, (w + 1) * nt / nw). A workgroup's rows are
// contiguous and it writes one partial per position.
template <int ES, int NG, int PF>
__global__ __launch_bounds__(256) void skinny_kernel(LmHeadArgs p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int EPV = Mma4<ES>::EPV;
    constexpr int KS = 16 * EPV;  // hidden elements per step (256 bytes of a row)
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
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
    const size_t rowbytes = (size_t)H * ES;
    const int nsteps = (H + KS - 1) / KS;
    const int total = max(T, 1) * nsteps;  // a wave without tiles streams nothing new
    const int mrows = p.Meff;  // all positions fit one workgroup here
    const int pitch = nsteps * KS * ES + 64;

    if (vb == 0 && tid == 0 && p.err != nullptr) *p.err = 0;

    // Address of this lane's 16 bytes for the next step to load; steps advance
    // through K of the current tile, then on to the next tile. Past the last step
    // the address stays on the last step (a re-read, no new HBM traffic).
    // Each wave walks K starting at its own rotation `rot` (any order of K gives
    // the same dot products): waves whose rows sit at power-of-two strides would
    // otherwise hit the same HBM channels at the same moment.
    const int kmax = H - EPV;
    const int rot = p.rotate ? (int)(((unsigned)(vb * 4 + wave) * 5u) % (unsigned)nsteps) : 0;
    int lt = 0, lks = 0;
    auto next_w = [&]() -> u32x4_t {
        const int v = min(tile_row(lt) + li, V - 1);
        int kstep = lks + rot;
        if (kstep >= nsteps) kstep -= nsteps;
        const int k = min(kstep * KS + lb * EPV, kmax);
        const u32x4_t r = load_w(p.w + (size_t)v * rowbytes + (size_t)k * ES);
        if (lks + 1 < nsteps) {
            ++lks;
        } else if (lt + 1 < T) {
            lks = 0;
            ++lt;
        }
        return r;
    };

    u32x4_t wb[PF];
    if (T > 0) {
#pragma unroll
        for (int i = 0; i < PF; ++i) wb[i] = next_w();
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

    // per-lane position bookkeeping: position m = 4g + li
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

    auto consume = [&](const u32x4_t& w, int ks) {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int m = 4 * g + li;
            const u32x4_t x = (m < mrows) ? *(const u32x4_t*)(smem + m * pitch + (ks * KS + lb * EPV) * ES)
                                          : u32x4_t{0u, 0u, 0u, 0u};
            acc[g] = Mma4<ES>::run(w, x, acc[g]);
        }
    };

    // End of a 4-row tile: sum the 16 K-blocks, update the running statistics.
    auto finish_tile = [&](int t) {
        const int v0 = tile_row(t);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            f32x4_t a = acc[g];
#pragma unroll
            for (int off = 4; off < 64; off <<= 1) {
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e] += __shfl_xor(a[e], off);
            }
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
    int ks = 0, kr = rot, t = 0;
    int s = 0;
    const int work = T > 0 ? total : 0;
    for (; s + PF <= work; s += PF) {
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            consume(wb[i], kr);
            wb[i] = next_w();
            if (++kr == nsteps) kr = 0;
            if (++ks == nsteps) {
                finish_tile(t);
                ks = 0;
                ++t;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        if (s + i < work) {
            consume(wb[i], kr);
            if (++kr == nsteps) kr = 0;
            if (++ks == nsteps) {
                finish_tile(t);
                ks = 0;
                ++t;
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
