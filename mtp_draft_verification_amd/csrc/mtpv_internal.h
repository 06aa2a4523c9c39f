// Internal declarations shared by the host API (api.hip) and the kernel files.
// Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mtpv {

// Per-(row, vocab block) statistics written by the LM-head kernel's epilogue.
//   x  = max over the block of l * c2 (c2 = log2(e) / T, fp32), i.e. log2 units
//   s  = sum over the block of exp2(l * c2 - x)
//   bv = largest raw logit in the block, bi = its lowest vocabulary id
struct Partial {
    float x;
    float s;
    float bv;
    int bi;
};

// Per-row statistics after combining every vocab block (fixed order).
struct RowStat {
    double x;   // max of l * c2 (log2 units)
    double z;   // sum of exp2(l * c2 - x)
    float bv;   // max raw logit
    int bi;     // its lowest id
    int pad[2];
};

// One inverse-CDF draw: from normalize(max(0, p - q)) when row_q >= 0, else from p.
struct Job {
    int row_p;      // row of the spilled logits giving p
    int row_q;      // row giving q, or -1
    int out_index;  // element of the output token array to write
    int pad;
    double u;       // uniform in [0, 1)
    double ref_p;   // reference: the row max of l log2(e) / T (log2 units) for the exponentials
    double ref_q;
};

enum { KIND_TILE = 0, KIND_SKINNY = 1, KIND_WIDE = 2, KIND_HTILE = 3 };

struct Plan {
    int mode, B, k, H, V, dtype;
    int es;          // element size (2 for bf16, 4 for fp32)
    int Mt, Meff;    // target rows, all rows the head sees
    int va, nt;      // tile kernel: 16*va vocab rows per wave, 16*nt positions per chunk;
                     // wide kernel: nt = positions per tile (64, 128 or 256)
    int vblock;      // vocab rows per workgroup (64 * va)
    int S;           // vocab blocks (wide kernel: tiles, V split evenly, at most 256 rows each)
    int MC;          // M chunks
    int kc;          // hidden elements staged per LDS pass
    int kind;        // LM-head kernel: KIND_SKINNY, KIND_HTILE, KIND_WIDE or KIND_TILE
    int tiles;       // skinny kernel: 4-row tiles per wave
    size_t lds;      // dynamic LDS bytes of the LM-head kernel
    int grid;        // LM-head workgroups (1-D, XCD-aware ordering when MC > 1)
    int ks;          // wide kernel: K slices (1: whole K per tile; > 1: raw partial
                     // products per slice into the spill, summed by launch_ksum; grid
                     // = S * MC * ks, slice fastest)
    int tail_f, tail_r, tail_ks;  // tiled kernel, one position chunk: tiles [tail_f, tail_f + tail_r) are
                                  // split along K in tail_ks pieces (0 tail tiles: none split)
    int tail_fm;                  // live position fragments per wave of those tiles
    int geo;                      // tiled kernel: 0 = 256-row x 224-position tiles, 1 = 192 x 128
    int NJ;          // inverse-CDF jobs (0 in greedy mode)
    int C;           // chunks per job in the residual passes
    int tpc;         // tiles per chunk (a multiple of the passes' 64-tile trip)
    int ntiles;      // 64-element tiles per vocabulary row
    // workspace layout (byte offsets)
    size_t off_err, off_partials, off_dlogit, off_rowstat, off_jobs, off_zpart, off_tsum, off_spill, off_tail;
    size_t total;
};

// Returns 0 and fills *plan, or a negative status for an invalid shape. many_kind: the
// kernel for more positions than the streaming kernel holds, bf16 (KIND_HTILE; the
// MTP input fusion's K-split projection asks for KIND_WIDE).
int make_plan(int mode, int B, int k, int H, int V, int dtype, Plan* plan, int many_kind = KIND_HTILE);

struct LmHeadArgs {
    const uint8_t* xt;      // target rows [Mt, H]
    const uint8_t* xd;      // drafter rows [Meff - Mt, H]
    const uint8_t* w;       // head [V, H]
    const int32_t* drafts;  // [B, k] or NULL (draft mode)
    int Mt, Meff, H, V, k;
    int S, MC, kc;
    float c2;               // log2(e) / T
    Partial* partials;      // [Meff, S]
    float* dlogit;          // [Meff]
    float* spill;           // [Meff, V] or NULL
    int32_t* err;           // cleared by the first workgroup (NULL: left alone)
    int tiles;              // skinny kernel: 4-row tiles per wave
    int rotate;             // skinny / wide kernels: rotation of the K order per wave / workgroup
    int ks;                 // wide kernel: K slices (> 1: raw products per slice, spill = [ks, Meff, V])
    float* tail;            // tiled kernel: raw accumulators of the K pieces of the split tiles
    int tail_f, tail_r, tail_ks, tail_fm;
};

// out[i] = sum over h < halves of (sum over s < ks of part[(s * halves + h) * n + i]),
// each sum in order (n % 4 == 0, 16-byte aligned): the K slices of a split wide-kernel
// launch, and the hi and lo rows of the fused MTP input.
hipError_t launch_ksum(const float* part, float* out, int ks, int halves, size_t n, hipStream_t stream);

hipError_t launch_lmhead(const Plan& plan, const LmHeadArgs& args, hipStream_t stream);
hipError_t launch_skinny(const Plan& plan, const LmHeadArgs& args, hipStream_t stream);
hipError_t launch_wide(const Plan& plan, const LmHeadArgs& args, hipStream_t stream);
hipError_t launch_head_tile(const Plan& plan, const LmHeadArgs& args, hipStream_t stream);
int head_tile_max_positions(int geo);  // positions per chunk of the persistent tiled kernel's geometry
int head_tile_rows(int geo);           // vocabulary rows per tile of that geometry
size_t head_tile_piece_bytes(int fm, int geo);  // raw accumulators of one K piece of a split tile (fm live fragments)
size_t wide_lds_bytes(int bm);  // dynamic LDS of the wide kernel for bm (64, 128 or 256) positions per tile
int wide_rows();                // most vocabulary rows per wide-kernel tile

struct DecideArgs {
    const Partial* partials;
    const float* dlogit;
    const int32_t* drafts;  // [B, k] (greedy, sample)
    const int32_t* draft_len;  // [B] drafts judged per request, or NULL (all k)
    int mode, B, k, V, Mt, Meff, S, depth0;
    float c2f;              // the fp32 constant the epilogue used
    double inv_t;           // 1 / T in fp64
    uint64_t seed, offset;
    RowStat* rowstat;       // [Meff]
    int32_t* accepted_len;  // [B]
    int32_t* out_tokens;    // [B, k+1] (greedy, sample) or [B, k] (draft)
    Job* jobs;              // [NJ]
    int32_t* err;
    double* dbg_pdqd;       // [B, k, 2] or NULL
    int32_t* dbg_argmax;    // [Meff] or NULL
    double* dbg_rowstats;   // [Meff, 2] or NULL
};

hipError_t launch_decide(const Plan& plan, const DecideArgs& args, hipStream_t stream);

struct ResidualArgs {
    const float* logits;    // spilled logits [Meff, V]
    const Job* jobs;
    int NJ, V, C, tpc, ntiles;
    double c2d;             // log2(e) / T in fp64
    double* zpart;          // [NJ, C, 2]
    double* tsum;           // [NJ, ntiles]
    int32_t* out;           // token output array (indexed by Job::out_index)
};

hipError_t launch_residual(const Plan& plan, const ResidualArgs& args, hipStream_t stream);

struct ProbsArgs {
    const float* logits;
    const RowStat* rowstat;
    float c2f;
    int Meff, V;
    float* probs;
};

hipError_t launch_probs(const ProbsArgs& args, hipStream_t stream);

hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

// Achievable-rate probes (ceiling.hip): one non-temporal read sweep of `bytes`; and
// back-to-back bf16 MFMAs, returning the flops of the launch (-1 on a launch error).
hipError_t launch_read(const void* src, size_t bytes, void* sink, hipStream_t stream);
int64_t launch_mfma_rate(int iters, void* sink, hipStream_t stream);

struct FuseArgs {
    const int32_t* tokens;  // [B]
    const uint8_t* embed;   // [V, H] bf16
    const uint8_t* hidden;  // [B, H] bf16
    const uint8_t* g_e;     // [H] bf16
    const uint8_t* g_h;     // [H] bf16
    uint8_t* x;             // [2B, 2H] bf16 (output): hi parts in rows 0..B-1, lo parts in B..2B-1
    int32_t* err;           // device error word (written by workgroup 0)
    int B, H, V;
    float eps;
};

hipError_t launch_fuse(const FuseArgs& args, hipStream_t stream);

// While measurement is on (mtpv_timing_enable), hands out the start/stop event pair
// to record around one launch of a call's dominant kernel and returns true.
bool timed_launch_events(hipEvent_t* start, hipEvent_t* stop);

// Top-k soft cross-entropy draft loss.
constexpr int kLossChunk = 8192;  // tokens per workgroup of the gradient pass

struct LossArgs {
    const float* teacher;  // [N, V]
    const float* student;  // [N, V]
    float* loss;           // [N]
    int32_t* index;        // [N, k]: kept tokens, best first
    double* pt;            // [N, k]: soft targets in the same order
    double* lse;           // [N]: logsumexp of each student row
    float* grad;           // [N, V] or NULL
    float scale;
    int N, V, k;
    int chunks;            // gradient workgroups per row
};

hipError_t launch_loss(const LossArgs& args, bool vec, hipStream_t stream);

}  // namespace mtpv
