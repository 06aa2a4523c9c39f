// Host side of the C ABI declared in include/mtpv.h: argument checks, the
// stream-ordered launch sequence and the measurement hooks (the launch plan and
// workspace layout are in plan.hip).
#include "mtpv.h"
#include "mtpv_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <utility>
#include <vector>

namespace mtpv {

namespace {

constexpr double kLog2e = 1.442695040888963407359924681001892137;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Rotation of the K order per wave in the streaming kernel (MTPV_K_ROTATE=0 turns
// it off, for measurements).
int k_rotate() {
    static const int r = [] {
        const char* e = std::getenv("MTPV_K_ROTATE");
        return (e && std::atoi(e) == 0) ? 0 : 1;
    }();
    return r;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// ------------------------------------------------------------- timing hooks
struct Timing {
    std::mutex mu;
    bool on = false;
    int every = 1;    // time one launch in `every`
    size_t seen = 0;  // launches offered since enabling or the last reset
    std::vector<std::pair<hipEvent_t, hipEvent_t>> events;
    size_t used = 0;
};

Timing& timing() {
    static Timing t;
    return t;
}

constexpr size_t kMaxTimed = 65536;

// Returns the event pair to record around this launch, or nullptr.
std::pair<hipEvent_t, hipEvent_t>* timing_slot() {
    Timing& t = timing();
    std::lock_guard<std::mutex> lk(t.mu);
    if (!t.on) return nullptr;
    if (t.seen++ % (size_t)t.every != 0 || t.used >= kMaxTimed) return nullptr;
    if (t.used == t.events.size()) {
        hipEvent_t a, b;
        if (hipEventCreate(&a) != hipSuccess) return nullptr;
        if (hipEventCreate(&b) != hipSuccess) {
            (void)hipEventDestroy(a);
            return nullptr;
        }
        t.events.emplace_back(a, b);
    }
    return &t.events[t.used++];
}

int common_check(int mode, int B, int k, int H, int V, int dtype, double temperature, const void* xt,
                 const void* xd, const void* w, const int32_t* drafts, const int32_t* alen,
                 const int32_t* out, const void* ws, size_t ws_bytes, Plan* plan) {
    const int st = make_plan(mode, B, k, H, V, dtype, plan);
    if (st != MTPV_OK) return st;
    if (mode != MTPV_MODE_GREEDY && !(std::isfinite(temperature) && temperature > 0.0)) return MTPV_EINVAL;
    if (w == nullptr) return MTPV_ENULL;
    if (mode == MTPV_MODE_DRAFT) {
        if (xd == nullptr || drafts == nullptr) return MTPV_ENULL;
    } else {
        if (xt == nullptr || alen == nullptr || out == nullptr) return MTPV_ENULL;
        if (k > 0 && drafts == nullptr) return MTPV_ENULL;
        if (mode == MTPV_MODE_SAMPLE && k > 0 && xd == nullptr) return MTPV_ENULL;
    }
    if (!aligned(w, 16) || (xt && !aligned(xt, 16)) || (xd && !aligned(xd, 16))) return MTPV_EALIGN;
    if ((drafts && !aligned(drafts, 4)) || (alen && !aligned(alen, 4)) || (out && !aligned(out, 4)))
        return MTPV_EALIGN;
    if (ws == nullptr || !aligned(ws, 256) || ws_bytes < plan->total) return MTPV_EWORKSPACE;
    return MTPV_OK;
}

int check_debug(const Plan& plan, const mtpv_debug* dbg) {
    if (dbg == nullptr) return MTPV_OK;
    if (dbg->logits && !aligned(dbg->logits, 16)) return MTPV_EALIGN;
    if (dbg->probs && !dbg->logits && plan.mode == MTPV_MODE_GREEDY) return MTPV_EINVAL;
    return MTPV_OK;
}

// The LM-head kernel of `plan` on rows xt (then xd) against w, with the timing
// events around it when enabled.
int launch_head(const Plan& plan, const void* xt, const void* xd, const void* w, const int32_t* drafts, float c2f,
                Partial* partials, float* dlogit, float* spill, int32_t* err, float* tail, hipStream_t stream,
                bool timed = true) {
    LmHeadArgs la;
    la.xt = static_cast<const uint8_t*>(xt);
    la.xd = static_cast<const uint8_t*>(xd);
    la.w = static_cast<const uint8_t*>(w);
    la.drafts = drafts;
    la.Mt = plan.Mt;
    la.Meff = plan.Meff;
    la.H = plan.H;
    la.V = plan.V;
    la.k = plan.k;
    la.S = plan.S;
    la.MC = plan.MC;
    la.kc = plan.kc;
    la.c2 = c2f;
    la.partials = partials;
    la.dlogit = dlogit;
    la.spill = spill;
    la.err = err;
    la.tiles = plan.tiles;
    // The streaming kernels spread their waves over the K order; the wide kernel keeps
    // every tile at the same K offset so that the tiles running together on an XCD
    // share their hidden-state and W chunks in L2.
    la.rotate = plan.kind == KIND_WIDE ? 0 : k_rotate();
    la.ks = plan.kind == KIND_WIDE ? plan.ks : 1;
    la.tail = tail;
    la.tail_f = plan.tail_f;
    la.tail_r = plan.tail_r;
    la.tail_ks = plan.tail_ks;
    la.tail_fm = plan.tail_fm;

    std::pair<hipEvent_t, hipEvent_t>* ev = timed ? timing_slot() : nullptr;
    if (ev && hipEventRecord(ev->first, stream) != hipSuccess) return MTPV_EDEVICE;
    const hipError_t le = plan.kind == KIND_SKINNY  ? launch_skinny(plan, la, stream)
                          : plan.kind == KIND_HTILE ? launch_head_tile(plan, la, stream)
                          : plan.kind == KIND_WIDE  ? launch_wide(plan, la, stream)
                                                    : launch_lmhead(plan, la, stream);
    if (le != hipSuccess) return MTPV_ELAUNCH;
    if (ev && hipEventRecord(ev->second, stream) != hipSuccess) return MTPV_EDEVICE;
    return MTPV_OK;
}

// One call: the LM-head launch, the decision pass (two passes for the dual call,
// greedy first, into alen_g / out_g), and the sampling passes. err_word: where the
// call's device error word goes (NULL: the workspace's own); timed: whether the
// measurement hooks may record events around the LM-head launch.
int run(const Plan& plan, const void* xt, const void* xd, const void* w, const int32_t* drafts,
        const int32_t* draft_len, double temperature, uint64_t seed, uint64_t offset, int depth0,
        int32_t* alen, int32_t* out, void* ws, const mtpv_debug* dbg, hipStream_t stream,
        int32_t* alen_g = nullptr, int32_t* out_g = nullptr, int32_t* err_word = nullptr, bool timed = true) {
    uint8_t* base = static_cast<uint8_t*>(ws);
    int32_t* err = err_word != nullptr ? err_word : reinterpret_cast<int32_t*>(base + plan.off_err);
    Partial* partials = reinterpret_cast<Partial*>(base + plan.off_partials);
    float* dlogit = reinterpret_cast<float*>(base + plan.off_dlogit);
    RowStat* rowstat = reinterpret_cast<RowStat*>(base + plan.off_rowstat);
    Job* jobs = reinterpret_cast<Job*>(base + plan.off_jobs);
    double* zpart = reinterpret_cast<double*>(base + plan.off_zpart);
    double* tsum = reinterpret_cast<double*>(base + plan.off_tsum);
    float* spill = nullptr;
    if (plan.mode != MTPV_MODE_GREEDY) spill = reinterpret_cast<float*>(base + plan.off_spill);
    if (dbg && dbg->logits) spill = dbg->logits;

    const double T = plan.mode == MTPV_MODE_GREEDY ? 1.0 : temperature;
    const float c2f = (float)(kLog2e / T);

    float* tail = reinterpret_cast<float*>(base + plan.off_tail);
    const int hs = launch_head(plan, xt, xd, w, plan.mode == MTPV_MODE_DRAFT ? nullptr : drafts, c2f, partials,
                               dlogit, spill, err, tail, stream, timed);
    if (hs != MTPV_OK) return hs;

    DecideArgs da;
    da.partials = partials;
    da.dlogit = dlogit;
    da.drafts = plan.mode == MTPV_MODE_DRAFT ? nullptr : drafts;
    da.draft_len = plan.mode == MTPV_MODE_DRAFT ? nullptr : draft_len;
    da.mode = plan.mode;
    da.B = plan.B;
    da.k = plan.k;
    da.V = plan.V;
    da.Mt = plan.Mt;
    da.Meff = plan.Meff;
    da.S = plan.S;
    da.depth0 = depth0;
    da.c2f = c2f;
    da.inv_t = 1.0 / T;
    da.seed = seed;
    da.offset = offset;
    da.rowstat = rowstat;
    da.accepted_len = alen;
    da.out_tokens = out;
    da.jobs = jobs;
    da.err = err;
    da.dbg_pdqd = (dbg && plan.mode != MTPV_MODE_DRAFT) ? dbg->pd_qd : nullptr;
    da.dbg_argmax = dbg ? dbg->argmax : nullptr;
    da.dbg_rowstats = dbg ? dbg->row_stats : nullptr;
    if (alen_g != nullptr) {
        // the greedy outcome of the same pass: decisions on the target rows only
        DecideArgs dg = da;
        dg.mode = MTPV_MODE_GREEDY;
        dg.accepted_len = alen_g;
        dg.out_tokens = out_g;
        dg.dbg_pdqd = nullptr;
        dg.dbg_argmax = nullptr;
        dg.dbg_rowstats = nullptr;
        if (launch_decide(plan, dg, stream) != hipSuccess) return MTPV_ELAUNCH;
    }
    if (launch_decide(plan, da, stream) != hipSuccess) return MTPV_ELAUNCH;

    if (plan.NJ > 0) {
        ResidualArgs ra;
        ra.logits = spill;
        ra.jobs = jobs;
        ra.NJ = plan.NJ;
        ra.V = plan.V;
        ra.C = plan.C;
        ra.tpc = plan.tpc;
        ra.ntiles = plan.ntiles;
        ra.c2d = 1.442695040888963407359924681001892137 / T;
        ra.zpart = zpart;
        ra.tsum = tsum;
        ra.out = plan.mode == MTPV_MODE_DRAFT ? const_cast<int32_t*>(drafts) : out;
        if (launch_residual(plan, ra, stream) != hipSuccess) return MTPV_ELAUNCH;
    }
    if (dbg && dbg->probs) {
        ProbsArgs pa;
        pa.logits = spill;
        pa.rowstat = rowstat;
        pa.c2f = c2f;
        pa.Meff = plan.Meff;
        pa.V = plan.V;
        pa.probs = dbg->probs;
        if (launch_probs(pa, stream) != hipSuccess) return MTPV_ELAUNCH;
    }
    return MTPV_OK;
}

// ------------------------------------------------ allocation-free entry point
// spec_verify_greedy_noalloc keeps its workspace in this file-scope device array: one
// copy per GPU, allocated with the code object and held until the process ends.
// In host code the array's name is only a stand-in; the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and only that
// address is ever handed to kernels.
constexpr size_t kScratchBytes = MTPV_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of the scratch array, or nullptr (HIP error).
void* scratch_address() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (dev < kMaxDevices && g_scratch_ptr[dev] != nullptr) return g_scratch_ptr[dev];
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    if (dev < kMaxDevices) g_scratch_ptr[dev] = p;
    return p;
}

}  // namespace

bool timed_launch_events(hipEvent_t* start, hipEvent_t* stop) {
    std::pair<hipEvent_t, hipEvent_t>* ev = timing_slot();
    if (ev == nullptr) return false;
    *start = ev->first;
    *stop = ev->second;
    return true;
}

}  // namespace mtpv

using namespace mtpv;

extern "C" {

int mtpv_version(void) { return 100; }

const char* mtpv_status_string(int status) {
    switch (status) {
        case MTPV_OK: return "ok";
        case MTPV_EINVAL: return "invalid size or scalar argument";
        case MTPV_EALIGN: return "H not a multiple of 8 or pointer not 16-byte aligned";
        case MTPV_EWORKSPACE: return "workspace missing, misaligned or too small";
        case MTPV_EDTYPE: return "unknown dtype";
        case MTPV_ENULL: return "required pointer is NULL";
        case MTPV_ELAUNCH: return "kernel launch failed";
        case MTPV_EDEVICE: return "HIP runtime error";
        case MTPV_ESCRATCH: return "shape needs more workspace than the allocation-free call's scratch holds";
        default: return "unknown status";
    }
}

size_t mtpv_workspace_bytes(int B, int k, int H, int V, int dtype, int mode) {
    Plan p;
    if (make_plan(mode, B, k, H, V, dtype, &p) != MTPV_OK) return 0;
    return p.total;
}

int mtpv_check_args(int mode, int B, int k, int H, int V, int dtype, double temperature,
                    const void* target_hidden, const void* draft_hidden, const void* W_lm,
                    const int32_t* draft_tokens, const int32_t* accepted_len, const int32_t* out_tokens,
                    const void* workspace, size_t workspace_bytes) {
    Plan p;
    return common_check(mode, B, k, H, V, dtype, temperature, target_hidden, draft_hidden, W_lm, draft_tokens,
                        accepted_len, out_tokens, workspace, workspace_bytes, &p);
}

int spec_verify_greedy(const void* hidden, const void* W_lm, const int32_t* draft_tokens, int B, int k, int H,
                       int V, int dtype, int32_t* accepted_len, int32_t* out_tokens, void* workspace,
                       size_t workspace_bytes, const mtpv_debug* debug, void* stream) {
    Plan p;
    int st = common_check(MTPV_MODE_GREEDY, B, k, H, V, dtype, 1.0, hidden, nullptr, W_lm, draft_tokens,
                          accepted_len, out_tokens, workspace, workspace_bytes, &p);
    if (st == MTPV_OK) st = check_debug(p, debug);
    if (st != MTPV_OK) return st;
    return run(p, hidden, nullptr, W_lm, draft_tokens, nullptr, 1.0, 0, 0, 0, accepted_len, out_tokens, workspace,
               debug, static_cast<hipStream_t>(stream));
}

int spec_verify_greedy_ragged(const void* hidden, const void* W_lm, const int32_t* draft_tokens,
                              const int32_t* draft_len, int B, int k, int H, int V, int dtype,
                              int32_t* accepted_len, int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                              const mtpv_debug* debug, void* stream) {
    Plan p;
    int st = common_check(MTPV_MODE_GREEDY, B, k, H, V, dtype, 1.0, hidden, nullptr, W_lm, draft_tokens,
                          accepted_len, out_tokens, workspace, workspace_bytes, &p);
    if (st == MTPV_OK && draft_len && !aligned(draft_len, 4)) st = MTPV_EALIGN;
    if (st == MTPV_OK) st = check_debug(p, debug);
    if (st != MTPV_OK) return st;
    return run(p, hidden, nullptr, W_lm, draft_tokens, draft_len, 1.0, 0, 0, 0, accepted_len, out_tokens,
               workspace, debug, static_cast<hipStream_t>(stream));
}

int spec_verify_sample(const void* target_hidden, const void* draft_hidden, const void* W_lm,
                       const int32_t* draft_tokens, int B, int k, int H, int V, int dtype, double temperature,
                       uint64_t seed, uint64_t offset, int32_t* accepted_len, int32_t* out_tokens,
                       void* workspace, size_t workspace_bytes, const mtpv_debug* debug, void* stream) {
    Plan p;
    int st = common_check(MTPV_MODE_SAMPLE, B, k, H, V, dtype, temperature, target_hidden, draft_hidden, W_lm,
                          draft_tokens, accepted_len, out_tokens, workspace, workspace_bytes, &p);
    if (st == MTPV_OK) st = check_debug(p, debug);
    if (st != MTPV_OK) return st;
    return run(p, target_hidden, draft_hidden, W_lm, draft_tokens, nullptr, temperature, seed, offset, 0,
               accepted_len, out_tokens, workspace, debug, static_cast<hipStream_t>(stream));
}

int spec_verify_sample_ragged(const void* target_hidden, const void* draft_hidden, const void* W_lm,
                              const int32_t* draft_tokens, const int32_t* draft_len, int B, int k, int H, int V,
                              int dtype, double temperature, uint64_t seed, uint64_t offset,
                              int32_t* accepted_len, int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                              const mtpv_debug* debug, void* stream) {
    Plan p;
    int st = common_check(MTPV_MODE_SAMPLE, B, k, H, V, dtype, temperature, target_hidden, draft_hidden, W_lm,
                          draft_tokens, accepted_len, out_tokens, workspace, workspace_bytes, &p);
    if (st == MTPV_OK && draft_len && !aligned(draft_len, 4)) st = MTPV_EALIGN;
    if (st == MTPV_OK) st = check_debug(p, debug);
    if (st != MTPV_OK) return st;
    return run(p, target_hidden, draft_hidden, W_lm, draft_tokens, draft_len, temperature, seed, offset, 0,
               accepted_len, out_tokens, workspace, debug, static_cast<hipStream_t>(stream));
}

int spec_verify_dual(const void* target_hidden, const void* draft_hidden, const void* W_lm,
                     const int32_t* draft_tokens, const int32_t* draft_len, int B, int k, int H, int V, int dtype,
                     double temperature, uint64_t seed, uint64_t offset, int32_t* accepted_len_greedy,
                     int32_t* out_tokens_greedy, int32_t* accepted_len_sample, int32_t* out_tokens_sample,
                     void* workspace, size_t workspace_bytes, const mtpv_debug* debug, void* stream) {
    Plan p;
    int st = common_check(MTPV_MODE_SAMPLE, B, k, H, V, dtype, temperature, target_hidden, draft_hidden, W_lm,
                          draft_tokens, accepted_len_sample, out_tokens_sample, workspace, workspace_bytes, &p);
    if (st == MTPV_OK && (accepted_len_greedy == nullptr || out_tokens_greedy == nullptr)) st = MTPV_ENULL;
    if (st == MTPV_OK && (!aligned(accepted_len_greedy, 4) || !aligned(out_tokens_greedy, 4))) st = MTPV_EALIGN;
    if (st == MTPV_OK && draft_len && !aligned(draft_len, 4)) st = MTPV_EALIGN;
    if (st == MTPV_OK) st = check_debug(p, debug);
    if (st != MTPV_OK) return st;
    return run(p, target_hidden, draft_hidden, W_lm, draft_tokens, draft_len, temperature, seed, offset, 0,
               accepted_len_sample, out_tokens_sample, workspace, debug, static_cast<hipStream_t>(stream),
               accepted_len_greedy, out_tokens_greedy);
}

// Workspace of mtp_input_fuse: the projection's LM-head workspace (its error word
// first), then the fused rows [2B, 2H] bf16 (hi parts, then lo parts), then the
// projection's raw products [ks, 2B, H] fp32.
// The fc projection [2H -> H] runs on the LM-head kernels with W_fc as the head over
// the 2B fused rows; a fixed-order sum adds each request's hi and lo rows (and the K
// slices). On the tiled kernel, which these shapes take beyond a few rows, there are
// only H output rows, so K is split in 8 slices, one per XCD (the slice of the fused
// rows is shared in that XCD's L2, every W_fc byte is read once), with the H rows in
// tiles so that slices x position chunks x tiles fill whole rounds of the compute
// units.
static int fuse_plan(int B, int H, Plan* p, size_t* x_off, size_t* part_off, size_t* total) {
    if (H < 8 || H > (1 << 19) || B < 1 || B > (1 << 19)) return MTPV_EINVAL;
    const int st = make_plan(MTPV_MODE_GREEDY, 2 * B, 0, 2 * H, H, MTPV_BF16, p, KIND_WIDE);
    if (st != MTPV_OK) return st;
    if (p->kind == KIND_WIDE) {
        constexpr int kCUs = 256;
        // K slices: 8 fill the compute units for few rows; with more than 256 rows (two
        // position chunks) 4 do, and the slices' raw products in the workspace (written
        // and read back once each) are half as many bytes
        p->ks = 2 * B > 256 ? 4 : 8;
        const long long per_tile = (long long)p->ks * p->MC;  // workgroups per row tile
        const long long s_min = (H + wide_rows() - 1) / wide_rows();
        const long long s_max = std::max(s_min, (long long)(H + 15) / 16);
        long long S = std::max(s_min, (kCUs + per_tile - 1) / per_tile);
        const long long rounds = (S * per_tile + kCUs - 1) / kCUs;
        S = std::min(s_max, std::max(S, rounds * kCUs / per_tile));
        p->S = (int)S;
        p->grid = (int)(S * per_tile);
    }
    *x_off = align_up(p->total, 256);
    *part_off = align_up(*x_off + (size_t)2 * B * 2 * H * 2, 256);
    *total = *part_off + align_up((size_t)p->ks * 2 * B * H * sizeof(float), 256);
    return MTPV_OK;
}

size_t mtpv_fuse_workspace_bytes(int B, int H) {
    Plan p;
    size_t x_off, part_off, total;
    return fuse_plan(B, H, &p, &x_off, &part_off, &total) == MTPV_OK ? total : 0;
}

int mtp_input_fuse(const int32_t* tokens, const void* embed, const void* hidden, const void* norm_emb,
                   const void* norm_hidden, const void* W_fc, int B, int H, int V, double eps, float* out,
                   void* workspace, size_t workspace_bytes, void* stream) {
    Plan p;
    size_t x_off, part_off, total;
    if (B < 1 || V < 1 || V > (1 << 26) || !(std::isfinite(eps) && eps >= 0.0)) return MTPV_EINVAL;
    int st = fuse_plan(B, H, &p, &x_off, &part_off, &total);
    if (st != MTPV_OK) return st;
    if (H % 8 != 0) return MTPV_EALIGN;
    if (!tokens || !embed || !hidden || !norm_emb || !norm_hidden || !W_fc || !out) return MTPV_ENULL;
    if (!aligned(tokens, 4) || !aligned(embed, 16) || !aligned(hidden, 16) || !aligned(norm_emb, 16) ||
        !aligned(norm_hidden, 16) || !aligned(W_fc, 16) || !aligned(out, 16))
        return MTPV_EALIGN;
    if (workspace == nullptr || !aligned(workspace, 256) || workspace_bytes < total) return MTPV_EWORKSPACE;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* base = static_cast<uint8_t*>(workspace);
    FuseArgs fa;
    fa.tokens = tokens;
    fa.embed = static_cast<const uint8_t*>(embed);
    fa.hidden = static_cast<const uint8_t*>(hidden);
    fa.g_e = static_cast<const uint8_t*>(norm_emb);
    fa.g_h = static_cast<const uint8_t*>(norm_hidden);
    fa.x = base + x_off;
    fa.err = reinterpret_cast<int32_t*>(base + p.off_err);
    fa.B = B;
    fa.H = H;
    fa.V = V;
    fa.eps = (float)eps;
    if (launch_fuse(fa, s) != hipSuccess) return MTPV_ELAUNCH;
    // the projection: fused rows in the place of hidden states, W_fc in the place of
    // the head, the raw fp32 products of every row (and K slice) through the logit
    // output, then their fixed-order sum; the error word is the fusion kernel's
    float* part = reinterpret_cast<float*>(base + part_off);
    st = launch_head(p, base + x_off, nullptr, W_fc, nullptr, (float)kLog2e,
                     reinterpret_cast<Partial*>(base + p.off_partials), reinterpret_cast<float*>(base + p.off_dlogit),
                     part, nullptr, nullptr, s);
    if (st != MTPV_OK) return st;
    return launch_ksum(part, out, p.ks, 2, (size_t)B * H, s) == hipSuccess ? MTPV_OK : MTPV_ELAUNCH;
}

int spec_draft_sample(const void* draft_hidden, const void* W_lm, int B, int kd, int depth0, int H, int V,
                      int dtype, double temperature, uint64_t seed, uint64_t offset, int32_t* draft_tokens,
                      void* workspace, size_t workspace_bytes, const mtpv_debug* debug, void* stream) {
    Plan p;
    if (depth0 < 0) return MTPV_EINVAL;
    int st = common_check(MTPV_MODE_DRAFT, B, kd, H, V, dtype, temperature, nullptr, draft_hidden, W_lm,
                          draft_tokens, nullptr, nullptr, workspace, workspace_bytes, &p);
    if (st == MTPV_OK) st = check_debug(p, debug);
    if (st != MTPV_OK) return st;
    return run(p, nullptr, draft_hidden, W_lm, draft_tokens, nullptr, temperature, seed, offset, depth0, nullptr,
               nullptr, workspace, debug, static_cast<hipStream_t>(stream));
}

int spec_verify_greedy_noalloc(const void* hidden, const void* W_lm, const int32_t* draft_tokens, int B, int k,
                               int H, int V, int dtype, int32_t* accepted_len, int32_t* out_tokens,
                               int32_t* device_error, void* stream) {
    Plan p;
    // the argument check of spec_verify_greedy, with a stand-in workspace of the
    // scratch array's size (checked for size only, never used)
    int st = common_check(MTPV_MODE_GREEDY, B, k, H, V, dtype, 1.0, hidden, nullptr, W_lm, draft_tokens,
                          accepted_len, out_tokens, reinterpret_cast<const void*>((uintptr_t)256), kScratchBytes,
                          &p);
    if (st == MTPV_EWORKSPACE) return MTPV_ESCRATCH;  // the shape needs more than the scratch array
    if (st != MTPV_OK) return st;
    if (device_error != nullptr && !aligned(device_error, 4)) return MTPV_EALIGN;
    void* ws = scratch_address();
    if (ws == nullptr) return MTPV_EDEVICE;
    return run(p, hidden, nullptr, W_lm, draft_tokens, nullptr, 1.0, 0, 0, 0, accepted_len, out_tokens, ws, nullptr,
               static_cast<hipStream_t>(stream), nullptr, nullptr, device_error, false);
}

int mtpv_get_device_error(const void* workspace, int32_t* err, void* stream) {
    if (workspace == nullptr || err == nullptr) return MTPV_ENULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipStreamSynchronize(s) != hipSuccess) return MTPV_EDEVICE;
    if (hipMemcpy(err, workspace, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess) return MTPV_EDEVICE;
    return MTPV_OK;
}

int mtpv_timing_enable(int every) {
    if (every < 0) return MTPV_EINVAL;
    Timing& t = timing();
    std::lock_guard<std::mutex> lk(t.mu);
    t.on = every != 0;
    t.every = every > 0 ? every : 1;
    t.seen = 0;
    return MTPV_OK;
}

int mtpv_timing_read(double* ms_total, int64_t* launches, int reset) {
    if (ms_total == nullptr || launches == nullptr) return MTPV_ENULL;
    Timing& t = timing();
    std::lock_guard<std::mutex> lk(t.mu);
    double total = 0.0;
    for (size_t i = 0; i < t.used; ++i) {
        if (hipEventSynchronize(t.events[i].second) != hipSuccess) return MTPV_EDEVICE;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, t.events[i].first, t.events[i].second) != hipSuccess) return MTPV_EDEVICE;
        total += ms;
    }
    *ms_total = total;
    *launches = (int64_t)t.used;
    if (reset) {
        t.used = 0;
        t.seen = 0;
    }
    return MTPV_OK;
}

int mtpv_copy_bytes(void* dst, const void* src, size_t bytes, void* stream) {
    if (dst == nullptr || src == nullptr) return MTPV_ENULL;
    if (!aligned(dst, 16) || !aligned(src, 16) || bytes % 16 != 0) return MTPV_EALIGN;
    if (launch_copy(dst, src, bytes, static_cast<hipStream_t>(stream)) != hipSuccess) return MTPV_ELAUNCH;
    return MTPV_OK;
}

int mtpv_read_bytes(const void* src, size_t bytes, void* sink, void* stream) {
    if (src == nullptr || sink == nullptr) return MTPV_ENULL;
    if (!aligned(src, 16) || !aligned(sink, 4) || bytes % 16 != 0) return MTPV_EALIGN;
    if (bytes == 0) return MTPV_OK;
    if (launch_read(src, bytes, sink, static_cast<hipStream_t>(stream)) != hipSuccess) return MTPV_ELAUNCH;
    return MTPV_OK;
}

int mtpv_mfma_rate(int iters, void* sink, int64_t* flops, void* stream) {
    if (sink == nullptr || flops == nullptr) return MTPV_ENULL;
    if (!aligned(sink, 4)) return MTPV_EALIGN;
    if (iters < 1 || iters > (1 << 24)) return MTPV_EINVAL;
    const int64_t f = launch_mfma_rate(iters, sink, static_cast<hipStream_t>(stream));
    if (f < 0) return MTPV_ELAUNCH;
    *flops = f;
    return MTPV_OK;
}

}  // extern "C"
