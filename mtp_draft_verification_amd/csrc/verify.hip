// Cross-block combine, acceptance decisions, longest-prefix scan and the fp64
// inverse-CDF sampler of the verify step.
//
// decide_kernel (one workgroup per request) merges the LM-head kernel's
// per-(row, vocab block) partials in a fixed order into per-row {max, sum of
// exp, argmax}, takes the acceptance decisions slot by slot and scans for the
// first rejection (the correct prefix is kept: "Speculative Decoding
// and MTP: Why Guessing Is Free", section "Speculative decoding: draft, then
// verify"; "The Tiny Draft Model Hidden Inside Qwen", section "How the draft
// becomes real output"), writes accepted_len / out_tokens and, when a token
// must be drawn, one sampling job.
//
// The draw itself (correction from normalize(max(0, p - q)) at the first
// rejection, bonus from p_k after k acceptances, or a drafter draw from q)
// runs over the spilled fp32 logits in three passes over the one or two rows a
// job needs, with fp64 sums: per-chunk sums of exp(l/T - ref) (the normaliser,
// recomputed here with the exact 1/T from the same per-element values the weights
// use), per-64-token tile sums of the weights, and a search over those sums in a
// fixed order followed by a scan inside the chosen tile in the same order as its
// tile sum. Every comparison uses sums built in one fixed order, so the search is
// consistent and bit-reproducible.
#include "mtpv_internal.h"

#include <algorithm>
#include <climits>

namespace mtpv {
namespace {

constexpr double kLn2 = 0.693147180559945309417232121458176568;

// ---------------------------------------------------------------- Philox4x32-10
// Salmon, Moraes, Dror & Shaw, SC'11: ten rounds over a 4-word counter with a
// 2-word key bumped by two Weyl constants between rounds.
__device__ __forceinline__ void philox_block(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                             uint32_t k0, uint32_t k1, uint32_t out[4]) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint32_t hi0 = __umulhi(0xD2511F53u, c0);
        const uint32_t lo0 = 0xD2511F53u * c0;
        const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2);
        const uint32_t lo1 = 0xCD9E8D57u * c2;
        const uint32_t n0 = hi1 ^ c1 ^ k0;
        const uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

// Uniform on the 24-bit grid: (x >> 8) * 2^-24, exact in fp64.
__device__ __forceinline__ double uniform24(uint32_t x) { return (double)(x >> 8) * 0x1p-24; }

// Word `word` of Philox(key = seed; counter = (slot, request, offset lo, offset hi)).
__device__ __forceinline__ double slot_uniform(uint64_t seed, uint64_t offset, int slot, int req, int word) {
    uint32_t o[4];
    philox_block((uint32_t)slot, (uint32_t)req, (uint32_t)offset, (uint32_t)(offset >> 32), (uint32_t)seed,
                 (uint32_t)(seed >> 32), o);
    return uniform24(o[word]);
}

// ------------------------------------------------------------ row combination
struct Acc {
    double x;   // running max (log2 units)
    double z;   // sum of exp2(. - x)
    float bv;
    int bi;
};

__device__ __forceinline__ int request_row(const DecideArgs& p, int b, int i) {
    if (p.mode == 2) return b * p.k + i;
    if (i <= p.k) return b * (p.k + 1) + i;
    return p.Mt + b * p.k + (i - p.k - 1);
}

// One workgroup per request, one wave per row up to 8 waves. Wave w of nw merges
// rows w, w + nw, ... of the request:
// each lane loads its share of the row's S partials (all loads of a batch issued
// before any use), reduces them (max first, then one exp2 per partial, no serial
// exp chain), and a wave butterfly finishes the row; all in a fixed order. While
// the waves reduce, the decision inputs (draft ids, draft logits, Philox uniforms)
// are fetched by other lanes. Then one slot per thread is decided and thread 0
// scans for the first rejection. Draft mode only writes one sampling job per row.
constexpr int kDecideWaves = 8;

__global__ __launch_bounds__(64 * kDecideWaves) void decide_kernel(DecideArgs p) {
    constexpr int U = 16;
    __shared__ RowStat rows[129];
    __shared__ int s_draft[64];
    __shared__ float s_lt[64], s_ld[64];
    __shared__ double s_u[64];
    __shared__ int keep[64];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int nw = blockDim.x >> 6;
    const int k = p.k;
    const int nrows = p.mode == 0 ? k + 1 : p.mode == 1 ? 2 * k + 1 : k;
    // drafts judged for this request (k_b <= k; the rest of its rows are unused)
    int kb = k;
    if (p.mode != 2 && p.draft_len != nullptr) {
        const int v = p.draft_len[b];
        kb = min(max(v, 0), k);
        if (v != kb && tid == 0) atomicOr(p.err, 2);
    }
    const float ninf = -__builtin_inff();

    // Decision inputs, independent of the row statistics. They are fetched by the
    // wave of the last row (after its row's loads are issued) so no wave's partial
    // loads wait behind them; the draft-logit loads do not depend on the draft ids (a
    // logit slot of an out-of-range draft is never written and never used).
    const int fetch_wave = max(0, nrows - 1) % nw;
    auto fetch_inputs = [&]() {
        if (p.mode != 2 && wave == fetch_wave && lane < k) {
            const int j = lane;
            const int d = p.drafts[b * k + j];
            const float lt = p.dlogit[b * (k + 1) + j];
            const float ld = p.mode == 1 ? p.dlogit[p.Mt + b * k + j] : 0.f;
            s_draft[j] = d;
            s_lt[j] = lt;
            s_ld[j] = ld;
            s_u[j] = p.mode == 1 ? slot_uniform(p.seed, p.offset, j, b, 0) : 0.0;
        }
    };
    if (wave >= nrows) fetch_inputs();

    for (int i = wave; i < nrows; i += nw) {
        const int r = request_row(p, b, i);
        const Partial* row = p.partials + (size_t)r * p.S;
        // Pass 1 over the row (usually one batch held in registers): the row max.
        // Pass 2: every lane rescales its partial sums to that max with one exp2
        // each; then plain fp64 sums. No exp2 inside the cross-lane reduction.
        float m = ninf;
        double z = 0.0;
        float bv = ninf;
        int bi = INT_MAX;
        const bool one_batch = p.S <= 64 * U;
        Partial q[U];
        for (int base = 0; base < p.S; base += 64 * U) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int s = base + u * 64 + lane;
                q[u] = s < p.S ? row[s] : Partial{ninf, 0.f, ninf, INT_MAX};
            }
            if (base == 0 && i + nw >= nrows) fetch_inputs();  // overlap with this wave's loads
#pragma unroll
            for (int u = 0; u < U; ++u) {
                m = fmaxf(m, q[u].x);
                if (q[u].bv > bv || (q[u].bv == bv && q[u].bi < bi)) {
                    bv = q[u].bv;
                    bi = q[u].bi;
                }
            }
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            m = fmaxf(m, __shfl_xor(m, off));
            const float obv = __shfl_xor(bv, off);
            const int obi = __shfl_xor(bi, off);
            if (obv > bv || (obv == bv && obi < bi)) {
                bv = obv;
                bi = obi;
            }
        }
        if (m != ninf) {
            for (int base = 0; base < p.S; base += 64 * U) {
                if (!one_batch) {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int s = base + u * 64 + lane;
                        q[u] = s < p.S ? row[s] : Partial{ninf, 0.f, ninf, INT_MAX};
                    }
                }
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (q[u].x != ninf) z += (double)q[u].s * (double)exp2f(q[u].x - m);
            }
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) z += __shfl_xor(z, off);
        const Acc a{(double)m, z, bv, bi};
        if (lane == 0) {
            RowStat rs;
            rs.x = a.x;
            rs.z = a.z;
            rs.bv = a.bv;
            rs.bi = a.bi;
            rs.pad[0] = rs.pad[1] = 0;
            rows[i] = rs;
            p.rowstat[r] = rs;
            if (p.dbg_argmax) p.dbg_argmax[r] = a.bi;
            if (p.dbg_rowstats) {
                p.dbg_rowstats[2 * r] = a.x * kLn2;
                p.dbg_rowstats[2 * r + 1] = a.z;
            }
            if (p.mode == 2) {  // drafter draw: one job per row, no decision
                Job job;
                job.row_p = r;
                job.row_q = -1;
                job.out_index = r;
                job.pad = 0;
                job.u = slot_uniform(p.seed, p.offset, p.depth0 + i, b, 2);
                job.ref_p = a.x;
                job.ref_q = 0.0;
                p.jobs[r] = job;
            }
        }
    }
    if (p.mode == 2) return;
    __syncthreads();

    if (tid < kb) {
        const int j = tid;
        const int d = s_draft[j];
        const bool in_range = d >= 0 && d < p.V;
        if (!in_range) atomicOr(p.err, 1);
        double pj = -1.0, qj = -1.0;
        bool kp = false;
        if (in_range) {
            const RowStat& st = rows[j];
            pj = exp2((double)(s_lt[j] * p.c2f) - st.x) / st.z;
            if (p.mode == 0) {
                qj = 0.0;
                kp = (d == st.bi);
            } else {
                const RowStat& sd = rows[k + 1 + j];
                qj = exp2((double)(s_ld[j] * p.c2f) - sd.x) / sd.z;
                kp = s_u[j] * qj < pj;
            }
        }
        if (p.dbg_pdqd) {
            p.dbg_pdqd[2 * (b * k + j)] = pj;
            p.dbg_pdqd[2 * (b * k + j) + 1] = qj;
        }
        keep[j] = kp ? 1 : 0;
    }
    __syncthreads();
    if (tid != 0) return;
    int al = kb;
    for (int j = 0; j < kb; ++j)
        if (!keep[j]) {
            al = j;
            break;
        }
    p.accepted_len[b] = al;
    int32_t* out = p.out_tokens + (size_t)b * (k + 1);
    for (int j = 0; j <= k; ++j) {
        int t = -1;
        if (j < al) t = s_draft[j];
        else if (j == al && p.mode == 0) t = rows[al].bi;
        out[j] = t;
    }
    if (p.mode == 1) {
        Job job;
        job.row_p = b * (k + 1) + al;
        job.row_q = (al < kb) ? p.Mt + b * k + al : -1;
        job.out_index = b * (k + 1) + al;
        job.pad = 0;
        job.u = slot_uniform(p.seed, p.offset, al, b, 1);
        job.ref_p = rows[al].x;
        job.ref_q = (al < kb) ? rows[k + 1 + al].x : 0.0;
        p.jobs[b] = job;
    }
}

// ------------------------------------------------------------ sampling passes
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off);
    return v;
}

// Four consecutive logits of `row` from token v (v % 4 == 0): one 16-byte load when
// rows are 16-byte aligned (V % 4 == 0), else four loads. Addresses are clamped into
// the row, so tokens at or past V (and rows < 0) read some logit of the row; callers
// give those tokens weight 0.
struct F4 {
    float a[4];
};

// VEC (V % 4 == 0, so every row starts 16-byte aligned): one 16-byte load; else four
// 4-byte loads. A template parameter, not a run-time test: with both paths in one
// function the compiler merged them into 4-byte loads.
template <bool VEC>
__device__ __forceinline__ F4 row_logit4(const float* logits, int row, int V, int v) {
    const float* base = logits + (size_t)max(row, 0) * V;
    F4 r;
    if (VEC) {
        typedef float f32x4_t __attribute__((ext_vector_type(4)));
        const f32x4_t x = *reinterpret_cast<const f32x4_t*>(base + min(v, V - 4));
        r.a[0] = x[0];
        r.a[1] = x[1];
        r.a[2] = x[2];
        r.a[3] = x[3];
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) r.a[e] = base[min(v + e, V - 1)];
    }
    return r;
}

// exp(l / T) up to the job's common factor, as 2^n * 2^f: t = l log2(e) / T - ref in
// fp64 (ref: the row max in log2 units), n = round(t), f = t - n in [-1/2, 1/2], 2^f
// from the hardware exp2 (f exact to 2^-25, no range reduction needed in that
// interval, the result to about 1e-7 relative), scaled by 2^n exactly. The error is a
// small random relative factor per element: the job's normaliser sums these same
// values, so a common scale cancels, and the cumulative sums stay in fp64.
__device__ __forceinline__ double row_exp_of(float l, bool live, double c2d, double ref) {
    if (!live) return 0.0;
    const double t = fma((double)l, c2d, -ref);
    const double n = rint(t);
    return ldexp((double)__builtin_amdgcn_exp2f((float)(t - n)), (int)n);
}

// Holds a wave-uniform job constant in a vector register once, so the fma above (which
// may read only one scalar operand on this chip) does not copy it in per element.
__device__ __forceinline__ void in_vgpr(double& x) { asm volatile("" : "+v"(x)); }

// Weight of one element for a job from its two logits: max(0, p - q) with a drafter
// row, else p; rp and rq are the reciprocals of the rows' normalisers.
__device__ __forceinline__ double weight_of(float lp, float lq, bool live, bool use_q, double c2d, const Job& job,
                                            double rp, double rq) {
    const double pv = row_exp_of(lp, live, c2d, job.ref_p) * rp;
    if (!use_q) return pv;
    const double qv = row_exp_of(lq, live, c2d, job.ref_q) * rq;
    const double d = pv - qv;
    return d > 0.0 ? d : 0.0;
}

// The fixed order of a 64-token tile, shared by the tile-sum pass and the search:
// lane q of a 16-lane group holds tokens 4q .. 4q + 3 of the tile, sums them in token
// order (w0 + w1) + w2 + w3, and the group takes the inclusive scan of those lane
// sums (Hillis-Steele, 16 lanes). The tile total is lane 15's scan value.
struct Lane4 {
    double w[4];
    double s;  // ((w0 + w1) + w2) + w3
};

__device__ __forceinline__ Lane4 lane_weights(const F4& lp, const F4& lq, int v, int vend, bool use_q, double c2d,
                                              const Job& job, double rp, double rq) {
    Lane4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r.w[e] = weight_of(lp.a[e], lq.a[e], v + e < vend, use_q, c2d, job, rp, rq);
    r.s = ((r.w[0] + r.w[1]) + r.w[2]) + r.w[3];
    return r;
}

__device__ __forceinline__ double scan16(double x, int q) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
        const double y = __shfl_up(x, off, 16);
        if (q >= off) x += y;
    }
    return x;
}

__device__ __forceinline__ double wave_scan(double x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}

// Reciprocals of the job's normalisers: lane c of each wave loads chunk c's partials
// (C <= 64) and a butterfly adds them; every lane ends with the same sums, in the
// same order wherever this is called.
__device__ __forceinline__ void normalisers(const ResidualArgs& p, int j, double* rp, double* rq) {
    const int lane = threadIdx.x & 63;
    const double* zpart = p.zpart + (size_t)j * p.C * 2;
    double a = 0.0, b = 0.0;
    if (lane < p.C) {
        a = zpart[2 * lane];
        b = zpart[2 * lane + 1];
    }
    a = wave_sum(a);
    b = wave_sum(b);
    *rp = 1.0 / a;
    *rq = 1.0 / b;
}

// 16-byte loads per lane and row per loop trip in the sampling passes. The loads of
// the next trip are issued before the fp64 arithmetic of the current one (past the
// chunk's end they re-read clamped addresses and are not used).
constexpr int UR = 4;

// Pass 1: per-chunk sums of exp(l/T - ref) for the job's p row and q row.
template <bool VEC>
__global__ __launch_bounds__(256) void zsum_kernel(ResidualArgs p) {
    __shared__ double sh[2][4];
    const int j = blockIdx.y, c = blockIdx.x;
    Job job = p.jobs[j];
    in_vgpr(job.ref_p);
    in_vgpr(job.ref_q);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int t0 = c * p.tpc, t1 = min(p.ntiles, t0 + p.tpc);
    const int e1 = min(p.V, t1 * 64);
    const bool has_q = job.row_q >= 0;
    double sp = 0.0, sq = 0.0;
    F4 np[UR], nq[UR];
    auto fetch = [&](int base) {
#pragma unroll
        for (int i = 0; i < UR; ++i) {
            const int v = base + 1024 * i + 4 * tid;
            np[i] = row_logit4<VEC>(p.logits, job.row_p, p.V, v);
            nq[i] = row_logit4<VEC>(p.logits, has_q ? job.row_q : job.row_p, p.V, v);
        }
    };
    fetch(t0 * 64);
    for (int base = t0 * 64; base < e1; base += 1024 * UR) {
        F4 lp[UR], lq[UR];
#pragma unroll
        for (int i = 0; i < UR; ++i) {
            lp[i] = np[i];
            lq[i] = nq[i];
        }
        if (base + 1024 * UR < e1) fetch(base + 1024 * UR);
#pragma unroll
        for (int i = 0; i < UR; ++i) {
            const int v = base + 1024 * i + 4 * tid;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool live = v + e < e1;
                sp += row_exp_of(lp[i].a[e], live, p.c2d, job.ref_p);
                sq += row_exp_of(lq[i].a[e], live && has_q, p.c2d, job.ref_q);
            }
        }
    }
    sp = wave_sum(sp);
    sq = wave_sum(sq);
    if (lane == 0) {
        sh[0][wave] = sp;
        sh[1][wave] = sq;
    }
    __syncthreads();
    if (tid == 0) {
        double* out = p.zpart + ((size_t)j * p.C + c) * 2;
        out[0] = ((sh[0][0] + sh[0][1]) + sh[0][2]) + sh[0][3];
        out[1] = ((sh[1][0] + sh[1][1]) + sh[1][2]) + sh[1][3];
    }
}

// Pass 2: per-tile sums of the job's weights in the tile's fixed order. Each wave
// load covers four consecutive tiles (1 KB of each row); wave w of the workgroup takes
// tiles 4 w .. 4 w + 3 of every 16.
template <bool VEC>
__global__ __launch_bounds__(256) void tsum_kernel(ResidualArgs p) {
    const int j = blockIdx.y, c = blockIdx.x;
    Job job = p.jobs[j];
    in_vgpr(job.ref_p);
    in_vgpr(job.ref_q);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, q = lane & 15;
    const bool use_q = job.row_q >= 0;
    const int t0 = c * p.tpc, t1 = min(p.ntiles, t0 + p.tpc);
    F4 np[UR], nq[UR];
    auto fetch = [&](int tb) {
#pragma unroll
        for (int i = 0; i < UR; ++i) {
            const int v = (tb + 16 * i) * 64 + 4 * q;
            np[i] = row_logit4<VEC>(p.logits, job.row_p, p.V, v);
            nq[i] = row_logit4<VEC>(p.logits, use_q ? job.row_q : job.row_p, p.V, v);
        }
    };
    fetch(t0 + 4 * wave + g);
    double rp, rq;  // (their loads wait behind the first logits)
    normalisers(p, j, &rp, &rq);
    for (int tb = t0 + 4 * wave + g; tb < t1; tb += 16 * UR) {  // uniform within each 16-lane group
        F4 lp[UR], lq[UR];
#pragma unroll
        for (int i = 0; i < UR; ++i) {
            lp[i] = np[i];
            lq[i] = nq[i];
        }
        if (tb + 16 * UR < t1) fetch(tb + 16 * UR);
#pragma unroll
        for (int i = 0; i < UR; ++i) {
            const int t = tb + 16 * i;
            const Lane4 w = lane_weights(lp[i], lq[i], t * 64 + 4 * q, p.V, use_q, p.c2d, job, rp, rq);
            const double incl = scan16(w.s, q);
            if (q == 15 && t < t1) p.tsum[(size_t)j * p.ntiles + t] = incl;
        }
    }
}

// Tile sums [i, i + SB) of a thread's run (0.0 past its end i1), all loads issued
// before any is used.
constexpr int SB = 16;
__device__ __forceinline__ void load_sums(const double* ts, int i, int i1, double (&tb)[SB]) {
#pragma unroll
    for (int u = 0; u < SB; ++u) tb[u] = i + u < i1 ? ts[i + u] : 0.0;
}

// Pass 3: locate u * (total weight) in the fixed-order sums and emit the token.
template <bool VEC>
__global__ __launch_bounds__(256) void search_kernel(ResidualArgs p) {
    __shared__ double wave_tot[4];
    __shared__ int sh_tile, sh_last, sh_pick;
    __shared__ double sh_base;
    __shared__ double sh_target;
    const int j = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    Job job = p.jobs[j];
    in_vgpr(job.ref_p);
    in_vgpr(job.ref_q);
    double rp, rq;
    normalisers(p, j, &rp, &rq);
    bool use_q = job.row_q >= 0;
    double* ts = p.tsum + (size_t)j * p.ntiles;
    const int per = (p.ntiles + 255) / 256;

    for (int pass = 0; pass < 2; ++pass) {
        if (pass == 1) {
            // Residual mass was zero: draw from p instead (tile sums rebuilt for p,
            // in the tile order of the tile-sum pass).
            const int g = lane >> 4, q = lane & 15;
            for (int tb = 4 * wave + g; tb < p.ntiles; tb += 16) {  // uniform within each 16-lane group
                const int v = tb * 64 + 4 * q;
                const F4 lp = row_logit4<VEC>(p.logits, job.row_p, p.V, v);
                const Lane4 w = lane_weights(lp, lp, v, p.V, false, p.c2d, job, rp, rq);
                const double incl = scan16(w.s, q);
                if (q == 15 && tb < p.ntiles) ts[tb] = incl;
            }
            __syncthreads();
        }
        // Each thread owns a run of consecutive tiles and sums it in tile order; a block
        // scan of the run totals gives every run its starting point, so each thread can
        // walk its own tiles from there. The first tile (over all threads) whose running
        // sum passes the target is the draw's tile; its base is the running sum before it.
        const int i0 = min(p.ntiles, tid * per), i1 = min(p.ntiles, i0 + per);
        double tot = 0.0;  // (adding the 0.0 of a padded slot leaves the sum as it is)
        int lastpos_tile = -1;
        for (int i = i0; i < i1; i += SB) {
            double tb[SB];
            load_sums(ts, i, i1, tb);
#pragma unroll
            for (int u = 0; u < SB; ++u) {
                tot += tb[u];
                if (tb[u] > 0.0) lastpos_tile = i + u;
            }
        }
        const double incl = wave_scan(tot, lane);
        double excl = __shfl_up(incl, 1);
        if (lane == 0) excl = 0.0;
        if (lane == 63) wave_tot[wave] = incl;
        if (tid == 0) {
            sh_tile = INT_MAX;
            sh_last = -1;
        }
        __syncthreads();
        double R = 0.0, wbase = 0.0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            if (w == wave) wbase = R;
            R += wave_tot[w];
        }
        if (!(R > 0.0)) {
            if (pass == 0 && use_q) {  // residual mass is zero: draw from p (uniform over the block)
                use_q = false;
                __syncthreads();
                continue;
            }
            // degenerate: every weight is zero; take token 0
            if (tid == 0) {
                sh_pick = 0;
                sh_base = 0.0;
                sh_target = -1.0;
            }
        } else {
            const double target = job.u * R;
            double run = wbase + excl;
            int cand = -1;
            for (int i = i0; i < i1 && cand < 0; i += SB) {
                double tb[SB];
                load_sums(ts, i, i1, tb);
#pragma unroll
                for (int u = 0; u < SB; ++u) {
                    if (cand < 0 && i + u < i1) {
                        if (run + tb[u] > target) cand = i + u;
                        else run += tb[u];
                    }
                }
            }
            if (cand >= 0) atomicMin(&sh_tile, cand);
            if (lastpos_tile >= 0) atomicMax(&sh_last, lastpos_tile);
            __syncthreads();
            const int tile = sh_tile;
            if (tile == INT_MAX) {
                // rounding put the target past the end: the last tile with mass, searched
                // with a target no prefix reaches, which selects its last positive token
                if (tid == 0) {
                    sh_pick = sh_last;
                    sh_base = 0.0;
                    sh_target = __builtin_huge_val();
                }
            } else if (cand == tile) {  // the one thread whose walk stopped there
                sh_pick = tile;
                sh_base = run;
                sh_target = target;
            }
        }
        __syncthreads();
        if (wave == 0) {
            // the chosen tile in the tile-sum pass's order: lanes 0..15 hold 4 tokens each
            // (lanes 16..63 repeat the computation and are left out of the ballots)
            const int q = lane & 15;
            const int v = sh_pick * 64 + 4 * q;
            const F4 lp = row_logit4<VEC>(p.logits, job.row_p, p.V, v);
            const F4 lq = row_logit4<VEC>(p.logits, use_q ? job.row_q : job.row_p, p.V, v);
            const Lane4 w = lane_weights(lp, lq, v, p.V, use_q, p.c2d, job, rp, rq);
            const double incl = scan16(w.s, q);
            double excl = __shfl_up(incl, 1, 16);
            if (q == 0) excl = 0.0;
            // cumulative weight through each token of the lane: the scan value of the
            // lane before, plus the lane's partial sums in token order; the lane's last
            // token takes its own scan value, so the tile's last token carries exactly
            // the tile total the walk compared
            const double b = sh_base, tg = sh_target;
            const double c0 = excl + w.w[0];
            const double c1 = excl + (w.w[0] + w.w[1]);
            const double c2 = excl + ((w.w[0] + w.w[1]) + w.w[2]);
            const int first = (b + c0 > tg) ? 0 : (b + c1 > tg) ? 1 : (b + c2 > tg) ? 2 : (b + incl > tg) ? 3 : 4;
            const int lastpos = w.w[3] > 0.0 ? 3 : w.w[2] > 0.0 ? 2 : w.w[1] > 0.0 ? 1 : w.w[0] > 0.0 ? 0 : -1;
            const unsigned long long group = 0xFFFFull;
            const unsigned long long hit = __ballot(first < 4) & group;
            const unsigned long long pos = __ballot(lastpos >= 0) & group;
            int ln = 0, e = 0;
            if (hit) {
                ln = __ffsll(hit) - 1;
                e = __shfl(first, ln);
            } else if (pos) {  // rounding left the target past the tile: its last positive token
                ln = 63 - __clzll(pos);
                e = __shfl(lastpos, ln);
            }
            if (lane == 0) p.out[job.out_index] = min(sh_pick * 64 + 4 * ln + e, p.V - 1);
        }
        break;
    }
}

// Debug export: probs[r][v] = exp2(l * c2 - x_r) / z_r with the kernels' own row statistics.
__global__ __launch_bounds__(256) void probs_kernel(ProbsArgs p) {
    const int r = blockIdx.y;
    const int v = blockIdx.x * 256 + threadIdx.x;
    if (v >= p.V) return;
    const RowStat st = p.rowstat[r];
    const float l = p.logits[(size_t)r * p.V + v];
    p.probs[(size_t)r * p.V + v] = (float)(exp2((double)(l * p.c2f) - st.x) / st.z);
}

__global__ __launch_bounds__(256) void copy_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src, size_t n) {
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

hipError_t launch_decide(const Plan& plan, const DecideArgs& args, hipStream_t stream) {
    const int nrows = args.mode == 0 ? args.k + 1 : args.mode == 1 ? 2 * args.k + 1 : args.k;
    // one wave per row, up to 8 (the first wave alone covers the k <= 64 decision slots)
    const int nw = std::max(1, std::min(kDecideWaves, nrows));
    hipLaunchKernelGGL(decide_kernel, dim3(plan.B), dim3(64 * nw), 0, stream, args);
    return hipGetLastError();
}

template <bool VEC>
hipError_t launch_residual_vec(const ResidualArgs& args, hipStream_t stream) {
    hipLaunchKernelGGL(zsum_kernel<VEC>, dim3(args.C, args.NJ), dim3(256), 0, stream, args);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(tsum_kernel<VEC>, dim3(args.C, args.NJ), dim3(256), 0, stream, args);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(search_kernel<VEC>, dim3(args.NJ), dim3(256), 0, stream, args);
    return hipGetLastError();
}

hipError_t launch_residual(const Plan& plan, const ResidualArgs& args, hipStream_t stream) {
    // the logit rows start 16-byte aligned when V % 4 == 0 (the buffer itself is)
    const bool vec = (args.V & 3) == 0 && ((uintptr_t)args.logits & 15) == 0;
    return vec ? launch_residual_vec<true>(args, stream) : launch_residual_vec<false>(args, stream);
}

hipError_t launch_probs(const ProbsArgs& args, hipStream_t stream) {
    hipLaunchKernelGGL(probs_kernel, dim3((args.V + 255) / 256, args.Meff), dim3(256), 0, stream, args);
    return hipGetLastError();
}

hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
    const size_t n = bytes / 16;
    const unsigned grid = (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, stream, (uint4*)dst, (const uint4*)src, n);
    return hipGetLastError();
}

}  // namespace mtpv
