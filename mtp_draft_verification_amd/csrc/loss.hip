// Top-k soft cross-entropy draft loss ("Faster Rollouts with MTP Speculative
// Decoding", SkyRL docs, sections "Overview" and "How does it work?": the MTP head is
// distilled toward the detached policy's next-token distribution with a soft
// cross-entropy over the policy's top-k tokens, k = 256 in the section "Example").
// Per row n of teacher logits t and student logits s over the vocabulary:
//   K      = the k largest t (equal logits: lower index first; -0.0 equals +0.0)
//   pt_j   = exp(t_j) / sum_{i in K} exp(t_i)           (j in K)
//   loss_n = logsumexp_v(s) - sum_{j in K} pt_j s_j      (= - sum pt_j log q_j)
//   grad   = scale * (softmax(s) - pt scattered on K)   (the teacher gets none)
//
// Selection kernel: one workgroup (4 waves) per row streams the teacher row and the
// student row once with non-temporal 16-byte loads. Each wave keeps, in LDS, the entries of its
// share that beat a running threshold; when its buffer nears full it cuts it to about
// its k best (a radix search for the k-th key, stopped early once the cut is within
// a few entries of k) and raises the threshold, and publishes a bound under which
// fewer than k / 4 of its entries lie, so that the four waves together screen with
// about the k-th best of all their tokens; a plain float compare against the
// threshold's value screens each token first. The student side keeps a per-lane
// running maximum and an fp64 sum of exp(s - max) (hardware exp2 of the scaled
// difference, summed in fp32 per 4 tokens). At the end the four
// waves' lists are merged and cut to k, ranked, and the soft targets, the gathered
// student logits and the loss are reduced in fp64 in a fixed order.
//
// Gradient (optional): a second streaming pass over the student rows writes
// scale * (exp(s - lse) - pt) for every token (pt = 0 off the kept list), each chunk
// of a row first marking its kept tokens in LDS.
#include "mtpv.h"
#include "mtpv_internal.h"

#include <climits>
#include <cmath>

namespace mtpv {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kCap = 1120;                 // entries per wave buffer
constexpr int kRoom = 256;                 // most entries one pass can add (64 lanes x 4)
constexpr int kDepth = 4;                  // passes of loads in flight per wave
constexpr int kPerWave = (kCap + 63) / 64; // buffer entries per lane when a wave compacts
constexpr int kSlack = 64;                 // a cut may keep this many entries beyond k
constexpr int kPerKept = (MTPV_LOSS_MAX_TOPK + kSlack + 63) / 64;  // entries per lane after a cut
static_assert(kCap - kRoom >= MTPV_LOSS_MAX_TOPK + kSlack + 256, "room between compactions");
static_assert(kCap % 4 == 0 && kCap >= 2 * MTPV_LOSS_MAX_TOPK, "16-byte rank reads; rank area after the kept entries");

// Monotone map of an fp32 value to an unsigned key (larger value, larger key);
// -0.0 maps to the key of +0.0.
__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t b = __float_as_uint(x);
    if (b == 0x80000000u) b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// (key, index) ordering: larger key first, then lower index
__device__ __forceinline__ bool beats(uint32_t k, int i, uint32_t tk, int ti) {
    return k > tk || (k == tk && i < ti);
}

__device__ __forceinline__ int lanes_below(unsigned long long m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Wave-wide inclusive prefix sum and maximum over the lanes in ascending order, with
// DPP row shifts and row broadcasts (register-to-register, no LDS round trip).
__device__ __forceinline__ int wave_prefix_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
    return x;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

__device__ __forceinline__ int wave_max_int(int x) {
    x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x111, 0xF, 0xF, false));
    x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x112, 0xF, 0xF, false));
    x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x114, 0xF, 0xF, false));
    x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x118, 0xF, 0xF, false));
    x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x142, 0xA, 0xF, false));
    x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x143, 0xC, 0xF, false));
    return __builtin_amdgcn_readlane(x, 63);
}

// Radix search over the first n keys of bk for a bound T with at least `want` keys
// >= T (1 <= want <= n), one byte at a time from the top: count the keys that share
// the bits fixed so far by their next 8 bits, then take the digit where the count
// from the top reaches the number still needed. The bits common to all keys are
// fixed first (they would put every key in one bin). The search stops when every
// bit is fixed (exact = true: T is the want-th largest key and `need` keys equal to
// T are still needed) or when the chosen bin holds at most `slack` keys more than
// are still needed (exact = false: T is the bin's lowest key, bits below zero, and
// at most want + slack keys are >= T). Runs on one whole wave with its own 256-bin
// LDS histogram; n <= 64 * PER.
template <int PER>
__device__ uint32_t radix_bound(const uint32_t* bk, int n, int want, int slack, int lane, uint32_t* hist, int& need,
                                bool& exact) {
    // Loops stay rolled and read the buffer from LDS each time: this runs rarely,
    // inside the streaming loop, and kept small it leaves that loop's code compact.
    uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
#pragma nounroll
    for (int e = 0; e < PER; ++e) {
        const int pos = e * 64 + lane;
        if (pos < n) {
            const uint32_t key = bk[pos];
            kmax = max(kmax, key);
            kmin = min(kmin, key);
        }
    }
    kmax = wave_max_u32(kmax);
    kmin = ~wave_max_u32(~kmin);
    const uint32_t diff = kmax ^ kmin;
    const int top = diff ? 31 - __clz(diff) : -1;  // highest differing bit (-1: all equal)
    uint32_t pmask = top < 0 ? 0xFFFFFFFFu : top == 31 ? 0u : ~((2u << top) - 1u);  // bits fixed so far
    uint32_t prefix = kmax & pmask;
    need = want;
    exact = true;
#pragma nounroll
    for (int hi = top; hi >= 0; hi -= 8) {
        const int lo = max(hi - 7, 0);
        const uint32_t dmask = (2u << (hi - lo)) - 1u;
        *reinterpret_cast<uint4*>(hist + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
#pragma nounroll
        for (int e = 0; e < PER; ++e) {
            const int pos = e * 64 + lane;
            if (pos < n) {
                const uint32_t key = bk[pos];
                if ((key & pmask) == prefix) atomicAdd(&hist[255u - ((key >> lo) & dmask)], 1u);
            }
        }
        // lane l holds bins 255-4l .. 252-4l (high digits on low lanes), so a prefix
        // sum over the lanes counts the entries at or above each lane's lowest digit
        const uint4 h = *reinterpret_cast<const uint4*>(hist + 4 * lane);
        const int c = (int)(h.x + h.y + h.z + h.w);
        const int S = wave_prefix_sum(c);
        const unsigned long long reach = __ballot(S >= need);  // lanes L..63 (S grows with the lane)
        const int L = __ffsll((long long)reach) - 1;
        int above = S - c;  // entries in higher bins than this lane's four
        int digit, inbin;
        if (above + (int)h.x >= need) {
            digit = 255 - 4 * lane;
            inbin = (int)h.x;
        } else if (above + (int)(h.x + h.y) >= need) {
            digit = 254 - 4 * lane;
            above += (int)h.x;
            inbin = (int)h.y;
        } else if (above + (int)(h.x + h.y + h.z) >= need) {
            digit = 253 - 4 * lane;
            above += (int)(h.x + h.y);
            inbin = (int)h.z;
        } else {
            digit = 252 - 4 * lane;
            above += (int)(h.x + h.y + h.z);
            inbin = (int)h.w;
        }
        digit = __builtin_amdgcn_readlane(digit, L);
        above = __builtin_amdgcn_readlane(above, L);
        inbin = __builtin_amdgcn_readlane(inbin, L);
        need -= above;
        prefix |= (uint32_t)digit << lo;
        pmask |= dmask << lo;
        if (lo > 0 && inbin - need <= slack) {
            exact = false;
            break;
        }
    }
    return prefix;
}

// Keeps at least the `want` best entries (larger key, then lower index) among the
// first n of (bk, bi), moved to the front in no particular order, and returns how
// many were kept. The bound found by radix_bound decides: exact, the want best are
// kept and (tk, ti) is the worst of them; otherwise every entry of key >= T is kept
// (at most want + slack) and (tk, ti) = (T, INT_MAX), which every key >= T beats.
// Either way at least `want` kept entries beat or equal (tk, ti), so no entry below
// it can be among the row's k best.
template <int PER>
__device__ int wave_keep(uint32_t* bk, int32_t* bi, int n, int want, int slack, int lane, uint32_t* hist,
                         uint32_t& tk, int& ti) {
    int need;
    bool exact;
    const uint32_t T = radix_bound<PER>(bk, n, want, slack, lane, hist, need, exact);
    int I = INT_MAX;
    if (exact) {  // need = entries of key T to keep, the lowest indices first
        int ties = 0, tie_max = -1;
#pragma nounroll
        for (int e = 0; e < PER; ++e) {
            const int pos = e * 64 + lane;
            const bool t = pos < n && bk[pos] == T;
            ties += __popcll(__ballot(t));
            if (t) tie_max = max(tie_max, bi[pos]);
        }
        tie_max = wave_max_int(tie_max);
        I = tie_max;
        if (need < ties) {
            int lo = 0, hi = tie_max;
            while (lo < hi) {
                const int mid = lo + ((hi - lo) >> 1);
                int c = 0;
#pragma nounroll
                for (int e = 0; e < PER; ++e) {
                    const int pos = e * 64 + lane;
                    c += __popcll(__ballot(pos < n && bk[pos] == T && bi[pos] <= mid));
                }
                if (c >= need)
                    hi = mid;
                else
                    lo = mid + 1;
            }
            I = lo;
        }
    }
    // compact in place: an entry's new slot is never above its old one, and each
    // group of 64 is read before any of it is overwritten
    int base = 0;
#pragma nounroll
    for (int e = 0; e < PER; ++e) {
        const int pos = e * 64 + lane;
        uint32_t key = 0u;
        int idx = INT_MAX;
        if (pos < n) {
            key = bk[pos];
            idx = bi[pos];
        }
        const bool s = pos < n && (key > T || (key == T && idx <= I));
        const unsigned long long m = __ballot(s);
        if (s) {
            const int to = base + lanes_below(m);
            bk[to] = key;
            bi[to] = idx;
        }
        base += __popcll(m);
    }
    tk = T;
    ti = I;
    return base;
}

__device__ __forceinline__ double block_sum(double v, double* sh) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[wave] = v;
    __syncthreads();
    return ((sh[0] + sh[1]) + sh[2]) + sh[3];
}

__device__ __forceinline__ float block_max(float v, float* sh) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[wave] = v;
    __syncthreads();
    return fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
}

struct F4 {
    float x[4];
};

// Four consecutive values of a row from token v; past the row's end the address is
// clamped to its last values (callers mask tokens >= V), so the load is never
// predicated and the loads of a ring stay in flight together.
template <bool VEC>
__device__ __forceinline__ F4 load4(const float* row, int v, int V) {
    F4 r;
    // non-temporal: each row is streamed once here (the gradient pass, if any, comes
    // long after the row has left the caches)
    if (VEC) {
        const f32x4_t q = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(row + min(v, V - 4)));
        r.x[0] = q[0];
        r.x[1] = q[1];
        r.x[2] = q[2];
        r.x[3] = q[3];
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) r.x[j] = __builtin_nontemporal_load(row + min(v + j, V - 1));
    }
    return r;
}

// Per-wave state of the stream: the kept-entry count and the worst kept entry
// (key tk, index ti; thr = its value, a cheap first test), and the lane's running
// student maximum m with sum of exp(s - m).
struct StreamState {
    int cnt = 0;
    uint32_t tk = 0u;
    int ti = INT_MAX;
    float thr = -INFINITY;
    float m = -INFINITY;
    double sum = 0.0;
};

constexpr float kLog2eF = 1.44269504088896340736f;

// One pass of a wave: 4 teacher and 4 student values per lane from token v. CHECK:
// the pass reaches past the row's end (tokens >= V are masked).
//
// The threshold (tk, ti) a token must beat is the stronger of this wave's own (the
// worst entry its last cut kept) and a bound shared by the four waves: after each
// cut a wave publishes a key q_w below which fewer than ceil(k / 4) of its kept
// entries lie, so the four lists hold at least k entries of key >= min_w q_w and no
// token below that minimum can be among the row's k best. It rises as soon as every
// wave has cut once, to about the k-th best of all four waves' tokens so far, where
// a wave's own threshold only reflects its quarter of them.
template <bool CHECK>
__device__ __forceinline__ void consume(const F4& t4, const F4& s4, int v, int V, int lane, uint32_t* bk,
                                        int32_t* bi, uint32_t* hist, uint32_t* sq, int wave, int K,
                                        StreamState& st) {
    {
        // relaxed workgroup-scope loads: fresh each pass, with no wait on the ring
        uint32_t q[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) q[w] = __hip_atomic_load(sq + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const uint32_t qmin = min(min(q[0], q[1]), min(q[2], q[3]));
        if (qmin > st.tk) {
            st.tk = qmin;
            st.ti = INT_MAX;
            st.thr = key_value(qmin);
        }
    }
    // teacher: with thr the value of the threshold key tk, a token beats (tk, ti)
    // exactly when t > thr, or t == thr and its index is lower (equal floats have
    // equal keys, -0.0 included); before the first cut thr = -inf and ti = INT_MAX
    // admit every token
    bool sel[4];
    int nsel = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        sel[j] = (!CHECK || v + j < V) && (t4.x[j] > st.thr || (t4.x[j] == st.thr && v + j < st.ti));
        nsel += sel[j] ? 1 : 0;
    }
    if (__ballot(nsel != 0)) {
        // slots for the lane's picks: an exclusive prefix sum over the lanes
        const int incl = wave_prefix_sum(nsel);
        int pos = st.cnt + incl - nsel;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (sel[j]) {
                bk[pos] = order_key(t4.x[j]);
                bi[pos] = v + j;
                ++pos;
            }
        }
        st.cnt += __builtin_amdgcn_readlane(incl, 63);
        if (st.cnt > kCap - kRoom) {
            st.cnt = wave_keep<kPerWave>(bk, bi, st.cnt, K, kSlack, lane, hist, st.tk, st.ti);
            st.thr = key_value(st.tk);
            int need;
            bool exact;
            const uint32_t q = radix_bound<kPerKept>(bk, st.cnt, (K + 3) / 4, kSlack, lane, hist, need, exact);
            if (lane == 0)
                __hip_atomic_store(sq + wave, max(sq[wave], q), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    }
    // student: running maximum, then exp2 of the scaled differences (<= 0)
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (!CHECK || v + j < V) mx = fmaxf(mx, s4.x[j]);
    if (mx > st.m) {
        if (st.m != -INFINITY) st.sum *= exp((double)st.m - (double)mx);
        st.m = mx;
    }
    if (st.m != -INFINITY) {
        float part = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (!CHECK || v + j < V) part += __builtin_amdgcn_exp2f((s4.x[j] - st.m) * kLog2eF);
        st.sum += (double)part;
    }
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void loss_select_kernel(LossArgs p) {
    __shared__ __attribute__((aligned(16))) uint32_t s_key[kWaves * kCap];
    __shared__ __attribute__((aligned(16))) int32_t s_id[kWaves * kCap];
    __shared__ uint32_t s_u[8];
    __shared__ int s_i[8];
    __shared__ uint4 s_hist[kWaves][64];  // a 256-bin histogram per wave
    __shared__ int s_cnt[kWaves];
    __shared__ double s_red[kWaves];
    __shared__ float s_redf[kWaves];
    __shared__ uint32_t s_q[kWaves];  // the waves' shared bounds (0: none yet)
    const int row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int V = p.V, K = p.k;
    const float* trow = p.teacher + (size_t)row * V;
    const float* srow = p.student + (size_t)row * V;
    uint32_t* bk = s_key + wave * kCap;
    int32_t* bi = s_id + wave * kCap;
    uint32_t* hist = reinterpret_cast<uint32_t*>(s_hist[wave]);

    StreamState st;
    if (tid < kWaves) s_q[tid] = 0u;
    __syncthreads();  // before any load is in flight (a barrier would wait for them)
    // Each pass of the workgroup covers 4 * kThreads consecutive tokens (a wave 256,
    // a lane 4); kDepth - 1 passes of loads stay in flight while one is consumed.
    constexpr int kStep = 4 * kThreads;
    const int nit = (V + kStep - 1) / kStep;
    const int v0 = wave * 256 + lane * 4;
    F4 tr[kDepth], sr[kDepth];
    // issued in slot order (the order the loop refills them), so the wait before each
    // slot's first use counts the same on the first trip as on every later one
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
        tr[d] = load4<VEC>(trow, v0 + d * kStep, V);
        sr[d] = load4<VEC>(srow, v0 + d * kStep, V);
        asm volatile("" ::: "memory");
    }
    for (int it = 0; it < nit; it += kDepth) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            const int v = v0 + (it + d) * kStep;
            if ((it + d + 1) * kStep <= V)
                consume<false>(tr[d], sr[d], v, V, lane, bk, bi, hist, s_q, wave, K, st);
            else
                consume<true>(tr[d], sr[d], v, V, lane, bk, bi, hist, s_q, wave, K, st);
            // refill the slot only once its values are consumed (the same registers)
            tr[d] = load4<VEC>(trow, v + kDepth * kStep, V);
            sr[d] = load4<VEC>(srow, v + kDepth * kStep, V);
        }
    }
    // student: logsumexp from the lanes' (max, sum) pairs (the barriers in the block
    // reductions also publish every wave's list length)
    if (lane == 0) s_cnt[wave] = st.cnt;
    const float m = st.m;
    const float M = block_max(m, s_redf);
    const double lane_part = (m == -INFINITY) ? 0.0 : st.sum * exp((double)m - (double)M);
    const double Z = block_sum(lane_part, s_red);
    const double lse = (double)M + log(Z);

    // The row's k best over the four lists (waves keep theirs where they are): a radix
    // select by all waves over one shared histogram, then each wave cuts its own list
    // in place. Uniform over the workgroup (every thread sees the same counts).
    const int own = st.cnt;
    const int n_all = s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
    int kept = own;
    if (n_all > K) {
        uint32_t* hist0 = reinterpret_cast<uint32_t*>(s_hist);  // 256 bins
        uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
        for (int e = 0; e < kPerWave; ++e) {
            const int pos = e * 64 + lane;
            if (pos < own) {
                const uint32_t key = bk[pos];
                kmax = max(kmax, key);
                kmin = min(kmin, key);
            }
        }
        kmax = wave_max_u32(kmax);
        const uint32_t nkmin = wave_max_u32(~kmin);
        if (lane == 0) {
            s_u[wave] = kmax;
            s_u[4 + wave] = nkmin;
        }
        __syncthreads();
        kmax = max(max(s_u[0], s_u[1]), max(s_u[2], s_u[3]));
        kmin = ~max(max(s_u[4], s_u[5]), max(s_u[6], s_u[7]));
        const uint32_t diff = kmax ^ kmin;
        const int top = diff ? 31 - __clz(diff) : -1;
        uint32_t pmask = top < 0 ? 0xFFFFFFFFu : top == 31 ? 0u : ~((2u << top) - 1u);
        uint32_t prefix = kmax & pmask;
        int need = K;
        for (int hi = top; hi >= 0; hi -= 8) {
            const int lo = max(hi - 7, 0);
            const uint32_t dmask = (2u << (hi - lo)) - 1u;
            hist0[tid] = 0u;
            __syncthreads();
            for (int e = 0; e < kPerWave; ++e) {
                const int pos = e * 64 + lane;
                if (pos < own) {
                    const uint32_t key = bk[pos];
                    if ((key & pmask) == prefix) atomicAdd(&hist0[255u - ((key >> lo) & dmask)], 1u);
                }
            }
            __syncthreads();
            if (wave == 0) {
                // lane l holds bins 255-4l .. 252-4l; a prefix sum over the lanes counts
                // the entries at or above each lane's lowest digit
                const uint4 h = reinterpret_cast<const uint4*>(hist0)[lane];
                const int c = (int)(h.x + h.y + h.z + h.w);
                const int S = wave_prefix_sum(c);
                const int L = __ffsll((long long)__ballot(S >= need)) - 1;
                int above = S - c;
                int digit;
                if (above + (int)h.x >= need) {
                    digit = 255 - 4 * lane;
                } else if (above + (int)(h.x + h.y) >= need) {
                    digit = 254 - 4 * lane;
                    above += (int)h.x;
                } else if (above + (int)(h.x + h.y + h.z) >= need) {
                    digit = 253 - 4 * lane;
                    above += (int)(h.x + h.y);
                } else {
                    digit = 252 - 4 * lane;
                    above += (int)(h.x + h.y + h.z);
                }
                if (lane == L) {
                    s_i[0] = digit;
                    s_i[1] = above;
                }
            }
            __syncthreads();
            need -= s_i[1];
            prefix |= (uint32_t)s_i[0] << lo;
            pmask |= dmask << lo;
            __syncthreads();  // s_i is read by all before it is written again
        }
        const uint32_t T = prefix;  // need = entries of key T to keep, the lowest indices first
        int ties = 0, tmax = -1;
        for (int e = 0; e < kPerWave; ++e) {
            const int pos = e * 64 + lane;
            const bool t = pos < own && bk[pos] == T;
            ties += __popcll(__ballot(t));
            if (t) tmax = max(tmax, bi[pos]);
        }
        tmax = wave_max_int(tmax);
        if (lane == 0) {
            s_i[wave] = ties;
            s_i[4 + wave] = tmax;
        }
        __syncthreads();
        const int ties_all = s_i[0] + s_i[1] + s_i[2] + s_i[3];
        int I = max(max(s_i[4], s_i[5]), max(s_i[6], s_i[7]));
        __syncthreads();
        if (need < ties_all) {
            int lo = 0, hi = I;
            while (lo < hi) {
                const int mid = lo + ((hi - lo) >> 1);
                int c = 0;
                for (int e = 0; e < kPerWave; ++e) {
                    const int pos = e * 64 + lane;
                    c += __popcll(__ballot(pos < own && bk[pos] == T && bi[pos] <= mid));
                }
                if (lane == 0) s_i[wave] = c;
                __syncthreads();
                const int call = s_i[0] + s_i[1] + s_i[2] + s_i[3];
                __syncthreads();
                if (call >= need)
                    hi = mid;
                else
                    lo = mid + 1;
            }
            I = lo;
        }
        // cut this wave's list in place: an entry's new slot is never above its old one
        int base = 0;
        for (int e = 0; e < kPerWave; ++e) {
            const int pos = e * 64 + lane;
            uint32_t key = 0u;
            int idx = INT_MAX;
            if (pos < own) {
                key = bk[pos];
                idx = bi[pos];
            }
            const bool keep = pos < own && (key > T || (key == T && idx <= I));
            const unsigned long long mk = __ballot(keep);
            if (keep) {
                const int to = base + lanes_below(mk);
                bk[to] = key;
                bi[to] = idx;
            }
            base += __popcll(mk);
        }
        kept = base;
    }
    __syncthreads();
    if (lane == 0) s_cnt[wave] = kept;
    __syncthreads();

    // rank the k kept entries (distinct under the ordering) into the tail of the last
    // wave's buffer (its kept entries end before k <= 512 < kCap - 512). Each entry is
    // first packed as key * 2^32 + (2^32 - 1 - index) into the free histogram area
    // (512 slots; the slots up to a multiple of 4 past k hold 0, which beats nothing):
    // one 64-bit compare then orders two entries, larger key first, lower index first.
    uint32_t* rk = s_key + kWaves * kCap - MTPV_LOSS_MAX_TOPK;
    int32_t* ri = s_id + kWaves * kCap - MTPV_LOSS_MAX_TOPK;
    uint64_t* comp = reinterpret_cast<uint64_t*>(s_hist);
    static_assert(sizeof(s_hist) >= MTPV_LOSS_MAX_TOPK * sizeof(uint64_t), "packed entries fit the histograms");
    const int k4 = (K + 3) & ~3;
    for (int a = tid; a < k4; a += kThreads) {
        uint64_t c = 0u;
        if (a < K) {
            int w = 0, j = a;
            while (j >= s_cnt[w]) {
                j -= s_cnt[w];
                ++w;
            }
            c = ((uint64_t)s_key[w * kCap + j] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)s_id[w * kCap + j]);
        }
        comp[a] = c;
    }
    __syncthreads();
    for (int a = tid; a < K; a += kThreads) {
        const uint64_t ca = comp[a];
        int rank = 0;
        const ulonglong2* cq = reinterpret_cast<const ulonglong2*>(comp);
        for (int q = 0; q < k4 / 2; ++q) {
            const ulonglong2 cc = cq[q];
            rank += (cc.x > ca) ? 1 : 0;
            rank += (cc.y > ca) ? 1 : 0;
        }
        rk[rank] = (uint32_t)(ca >> 32);
        ri[rank] = (int32_t)(0xFFFFFFFFu - (uint32_t)ca);
    }
    __syncthreads();

    // soft targets over the kept teacher logits, the student logits at them, the loss
    const double t0 = (double)key_value(rk[0]);
    double e_own[2] = {0.0, 0.0};
    double z_part = 0.0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int a = tid + h * kThreads;
        if (a < K) {
            e_own[h] = exp((double)key_value(rk[a]) - t0);
            z_part += e_own[h];
        }
    }
    const double Zt = block_sum(z_part, s_red);
    double dot_part = 0.0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int a = tid + h * kThreads;
        if (a < K) {
            const int id = ri[a];
            const double pt = e_own[h] / Zt;
            dot_part += pt * (double)srow[id];
            p.index[(size_t)row * K + a] = id;
            p.pt[(size_t)row * K + a] = pt;
        }
    }
    const double dot = block_sum(dot_part, s_red);
    if (tid == 0) {
        p.loss[row] = (float)(lse - dot);
        p.lse[row] = lse;
    }
}

// grad[n, v] = scale * (q_v - pt_v), q_v = exp(s[n, v] - lse[n]), over one chunk of a
// row; the chunk's kept tokens are first marked in LDS (their place in the kept
// list, plus one) so every token is written once.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void loss_grad_kernel(LossArgs p) {
    __shared__ uint64_t slot4[kLossChunk / 4];      // 16-bit slot per token
    __shared__ double pt[MTPV_LOSS_MAX_TOPK + 1];   // soft target per slot (slot 0: none)
    const int row = blockIdx.x / p.chunks;
    const int c = blockIdx.x - row * p.chunks;
    const int v0 = c * kLossChunk;
    for (int i = threadIdx.x; i < kLossChunk / 4; i += kThreads) slot4[i] = 0ull;
    if (threadIdx.x == 0) pt[0] = 0.0;
    __syncthreads();
    uint16_t* slot = reinterpret_cast<uint16_t*>(slot4);
    const int32_t* kept = p.index + (size_t)row * p.k;
    const double* kept_pt = p.pt + (size_t)row * p.k;
    for (int r = threadIdx.x; r < p.k; r += kThreads) {
        const int id = kept[r];
        if (id >= v0 && id < v0 + kLossChunk) {
            slot[id - v0] = (uint16_t)(r + 1);
            pt[r + 1] = kept_pt[r];
        }
    }
    __syncthreads();
    const double lse = p.lse[row];
    const float* srow = p.student + (size_t)row * p.V;
    float* grow = p.grad + (size_t)row * p.V;
    constexpr int kU = kLossChunk / (4 * kThreads);
    F4 sv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) sv[u] = load4<VEC>(srow, v0 + u * 4 * kThreads + 4 * threadIdx.x, p.V);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int off = u * 4 * kThreads + 4 * threadIdx.x;
        const int v = v0 + off;
        const uint64_t sl = slot4[off >> 2];
        float g[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float q = expf((float)((double)sv[u].x[j] - lse));
            const int r = (int)((sl >> (16 * j)) & 0xFFFFu);
            g[j] = r ? (float)((double)p.scale * ((double)q - pt[r])) : p.scale * q;
        }
        // non-temporal stores: the gradient is written once and not read here again
        if (VEC) {
            if (v < p.V)
                __builtin_nontemporal_store(f32x4_t{g[0], g[1], g[2], g[3]}, reinterpret_cast<f32x4_t*>(grow + v));
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (v + j < p.V) __builtin_nontemporal_store(g[j], grow + v + j);
        }
    }
}

}  // namespace

hipError_t launch_loss(const LossArgs& a, bool vec, hipStream_t stream) {
    if (a.N == 0) return hipSuccess;
    hipEvent_t t0, t1;  // the selection kernel is the timed one
    const bool timed = timed_launch_events(&t0, &t1);
    if (timed) {
        const hipError_t re = hipEventRecord(t0, stream);
        if (re != hipSuccess) return re;
    }
    if (vec)
        hipLaunchKernelGGL(loss_select_kernel<true>, dim3(a.N), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(loss_select_kernel<false>, dim3(a.N), dim3(kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && timed) e = hipEventRecord(t1, stream);
    if (e != hipSuccess || a.grad == nullptr) return e;
    const unsigned int blocks = (unsigned int)((size_t)a.N * a.chunks);
    if (vec)
        hipLaunchKernelGGL(loss_grad_kernel<true>, dim3(blocks), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(loss_grad_kernel<false>, dim3(blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mtpv

using namespace mtpv;

namespace {

bool loss_aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t loss_ws_layout(int N, int k, size_t* off_pt, size_t* off_index) {
    const size_t lse = ((size_t)N * sizeof(double) + 255) / 256 * 256;
    const size_t pt = ((size_t)N * k * sizeof(double) + 255) / 256 * 256;
    const size_t idx = ((size_t)N * k * sizeof(int32_t) + 255) / 256 * 256;
    *off_pt = lse;
    *off_index = lse + pt;
    return lse + pt + idx;
}

}  // namespace

extern "C" {

size_t mtpv_loss_workspace_bytes(int N, int topk) {
    if (N < 0 || topk < 1 || topk > MTPV_LOSS_MAX_TOPK) return 0;
    size_t a, b;
    return loss_ws_layout(N, topk, &a, &b);
}

int mtp_draft_loss_topk(const float* teacher, const float* student, int N, int V, int topk, float grad_scale,
                        float* loss, int32_t* topk_index, float* grad, void* workspace, size_t workspace_bytes,
                        void* stream) {
    if (N < 0 || V < 1 || V > (1 << 30) || topk < 1 || topk > MTPV_LOSS_MAX_TOPK || topk > V ||
        !std::isfinite(grad_scale))
        return MTPV_EINVAL;
    const size_t chunks = ((size_t)V + kLossChunk - 1) / kLossChunk;
    if (grad != nullptr && (size_t)N * chunks > (size_t)INT_MAX) return MTPV_EINVAL;
    if (N == 0) return MTPV_OK;
    if (!teacher || !student || !loss) return MTPV_ENULL;
    if (!loss_aligned(teacher, 4) || !loss_aligned(student, 4) || !loss_aligned(loss, 4) ||
        !loss_aligned(topk_index, 4) || !loss_aligned(grad, 4))
        return MTPV_EALIGN;
    size_t off_pt, off_index;
    const size_t need = loss_ws_layout(N, topk, &off_pt, &off_index);
    if (workspace == nullptr || !loss_aligned(workspace, 256) || workspace_bytes < need) return MTPV_EWORKSPACE;
    uint8_t* base = static_cast<uint8_t*>(workspace);
    LossArgs a;
    a.teacher = teacher;
    a.student = student;
    a.loss = loss;
    a.index = topk_index ? topk_index : reinterpret_cast<int32_t*>(base + off_index);
    a.pt = reinterpret_cast<double*>(base + off_pt);
    a.lse = reinterpret_cast<double*>(base);
    a.grad = grad;
    a.scale = grad_scale;
    a.N = N;
    a.V = V;
    a.k = topk;
    a.chunks = (int)chunks;
    // 16-byte loads when every row starts on a 16-byte boundary
    const bool vec = V % 4 == 0 && loss_aligned(teacher, 16) && loss_aligned(student, 16) &&
                     (grad == nullptr || loss_aligned(grad, 16));
    return launch_loss(a, vec, static_cast<hipStream_t>(stream)) == hipSuccess ? MTPV_OK : MTPV_ELAUNCH;
}

}  // extern "C"
