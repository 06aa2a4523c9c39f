// Launch plan of a verify call: which LM-head kernel, its tiling and grid, the
// sampling-pass chunking, and the workspace layout. Host code only; everything that
// decides how the LM-head kernels are launched lives here.
#include "mtpv.h"
#include "mtpv_internal.h"

#include <algorithm>
#include <cstdlib>
#include <cstring>

namespace mtpv {

namespace {

constexpr int kMaxK = 64;
constexpr int kLdsBudget = 64 * 1024;   // staging budget per workgroup (two workgroups fit per CU)
constexpr size_t kLdsPerCU = 160 * 1024; // LDS of one gfx950 compute unit
constexpr int kCUs = 256;                // compute units of one MI355X
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// MTPV_WIDE_KERNEL=old selects the earlier tiled kernel for many positions (A/B
// measurements only).
bool wide_forced() {
    static const bool f = [] {
        const char* e = std::getenv("MTPV_WIDE_KERNEL");
        return e != nullptr && std::strcmp(e, "old") == 0;
    }();
    return f;
}

int shape_status(int mode, int B, int k, int H, int V, int dtype) {
    if (dtype != MTPV_BF16 && dtype != MTPV_F32) return MTPV_EDTYPE;
    if (mode < MTPV_MODE_GREEDY || mode > MTPV_MODE_DRAFT) return MTPV_EINVAL;
    if (B < 1 || B > (1 << 20) || k < 0 || k > kMaxK || H < 8 || H > (1 << 20) || V < 1 || V > (1 << 26))
        return MTPV_EINVAL;
    if (mode == MTPV_MODE_DRAFT && k < 1) return MTPV_EINVAL;
    if (H % 8 != 0) return MTPV_EALIGN;
    const long long meff = (long long)B * (k + 1) + (mode == MTPV_MODE_SAMPLE ? (long long)B * k : 0);
    if (meff > (1 << 22)) return MTPV_EINVAL;
    // sampling jobs and debug rows index the second grid dimension (at most 65535)
    if (mode == MTPV_MODE_DRAFT && (long long)B * k > 65535) return MTPV_EINVAL;
    if (meff > 65535) return MTPV_EINVAL;
    return MTPV_OK;
}

}  // namespace

int make_plan(int mode, int B, int k, int H, int V, int dtype, Plan* pl, int many_kind) {
    const int st = shape_status(mode, B, k, H, V, dtype);
    if (st != MTPV_OK) return st;
    Plan p;
    std::memset(&p, 0, sizeof(p));
    p.mode = mode;
    p.B = B;
    p.k = k;
    p.H = H;
    p.V = V;
    p.dtype = dtype;
    p.es = dtype == MTPV_BF16 ? 2 : 4;
    p.ks = 1;
    p.tail_ks = 1;
    if (mode == MTPV_MODE_DRAFT) {
        p.Mt = 0;
        p.Meff = B * k;
    } else {
        p.Mt = B * (k + 1);
        p.Meff = p.Mt + (mode == MTPV_MODE_SAMPLE ? B * k : 0);
    }
    const int epv = 16 / p.es;
    // Few positions (<= 16) whose hidden states fit in LDS: the streaming kernel
    // with 4-row tiles (p.tiles tiles per wave, 16 * tiles rows per workgroup).
    {
        const int ks = 16 * epv;
        const int nsteps = (H + ks - 1) / ks;
        const size_t pitch = (size_t)nsteps * ks * p.es + 64;
        const size_t x_lds = (size_t)p.Meff * pitch;
        if (p.Meff <= 16 && x_lds <= (size_t)kLdsBudget) {
            // One resident round: kCUs compute units times the workgroups they hold
            // at once (by LDS, and by registers: 4 waves per SIMD up to 8 positions,
            // 3 beyond), but no more workgroups than one tile per wave. With at most 4
            // positions, 2 workgroups per unit stream as fast as 4 and leave half as
            // many partials to merge (decode step 0.1894 -> 0.1891 ms).
            p.kind = KIND_SKINNY;
            const int by_regs = p.Meff <= 4 ? 2 : p.Meff <= 8 ? 4 : 3;
            const int per_cu = (int)std::min<size_t>(by_regs, kLdsPerCU / std::max<size_t>(x_lds, 1024));
            const int tiles = (V + 3) / 4;
            p.grid = std::max(1, std::min(kCUs * std::max(per_cu, 1), (tiles + 3) / 4));
            p.tiles = (tiles + 4 * p.grid - 1) / (4 * p.grid);
            p.vblock = 0;
            p.S = p.grid;
            p.MC = 1;
            p.lds = std::max(x_lds, (size_t)4 * 16 * 16);
            p.va = p.nt = 0;
            p.kc = H;
        }
    }
    // Up to 96 head rows the W stream sets the time and the wide kernel's one-tile
    // workgroups keep more of it in flight (H = 5120, V = 151936 greedy: 242 against
    // 277 us at 20 rows, 300 against 310 us at 96); from 112 rows on the tiled kernel
    // is as fast or faster (326 against 342 us at 128, 350 against 404 us at 160).
    constexpr int kWideMaxRows = 96;
    if (many_kind == KIND_HTILE && !wide_forced() && p.kind != KIND_SKINNY && p.es == 2 &&
        p.Meff > kWideMaxRows) {
        // Many positions, bf16: the persistent tiled kernel. Position chunks of at most
        // the geometry's positions, split evenly; vocabulary tiles of at most its rows, as
        // many as make whole rounds of items over the compute units (tile edges on 16-row
        // boundaries, every tile at least one fragment).
        p.kind = KIND_HTILE;
        // At most 128 head rows (one chunk of the small geometry): 192-row tiles with five
        // W stages, four of them in flight, since there the W stream sets the pace; more
        // rows: 256-row x 224-position tiles with three W stages.
        const long long Mf = (p.Meff + 15) / 16;
        p.geo = Mf <= head_tile_max_positions(1) / 16 ? 1 : 0;
        const int cap = head_tile_max_positions(p.geo) / 16;
        const int tfr = head_tile_rows(p.geo) / 16;  // fragments per whole tile
        p.MC = (int)((Mf + cap - 1) / cap);
        const long long G = (V + 15) / 16;
        const long long nvt_min = (G + tfr - 1) / tfr;
        const long long rounds = (nvt_min * p.MC + kCUs - 1) / kCUs;
        long long S = std::max(nvt_min, rounds * kCUs / p.MC);
        S = std::min(S, G);
        // One position chunk and whole tiles that leave the last round part full: the
        // whole rounds as they are, the tiles left over cut along K into
        // pieces that fill the compute units instead (raw accumulators to the
        // workspace, added in piece order by a second kernel that finishes those
        // tiles). Padding the rounds with smaller tiles instead keeps the MFMA work of
        // 256-row tiles for fewer live rows.
        const long long full = nvt_min / kCUs * kCUs, left = nvt_min - full;
        if (p.MC == 1 && full > 0 && left > 0 && kCUs / left >= 2) {
            S = nvt_min;
            p.tail_f = (int)full;
            p.tail_r = (int)left;
            p.tail_ks = (int)std::min<long long>(std::min<long long>(8, kCUs / left), (H + 63) / 64);
            p.tail_fm = (int)((Mf + 1) / 2);
            if (p.tail_ks < 2) p.tail_f = p.tail_r = p.tail_fm = 0, p.tail_ks = 1;
        }
        p.S = (int)S;
        const long long items = S * p.MC;
        p.grid = (int)std::min<long long>(kCUs, (items + 7) / 8 * 8);
        p.nt = head_tile_max_positions(p.geo);
        p.kc = 64;
        p.lds = 0;
        p.vblock = 0;
        p.va = 0;
    }
    if (p.kind != KIND_SKINNY && p.kind != KIND_HTILE && p.es == 2) {
        // Many positions, bf16: LDS-tiled matrix product, one workgroup per tile of at
        // most 256 vocabulary rows by 64, 128 or 256 positions (whichever pads fewer
        // rows; 256 on a tie, so W is re-read from L2 fewer times), the position
        // chunks of one vocabulary tile on one XCD. With few tiles the vocabulary is
        // cut into more, smaller tiles so that every compute unit gets the same
        // number (at least 16 rows per tile).
        p.kind = KIND_WIDE;
        const int pad64 = (p.Meff + 63) / 64 * 64;
        const int pad128 = (p.Meff + 127) / 128 * 128;
        const int pad256 = (p.Meff + 255) / 256 * 256;
        const int bm = pad256 <= pad128 ? 256 : pad128 <= pad64 ? 128 : 64;
        p.nt = bm;
        p.MC = (p.Meff + bm - 1) / bm;
        p.va = 0;
        const long long s0 = (V + wide_rows() - 1) / wide_rows();
        long long S = s0;
        if (s0 * p.MC < 4LL * kCUs) {
            const long long rounds = (s0 * p.MC + kCUs - 1) / kCUs;
            S = std::max(s0, (rounds * kCUs + p.MC - 1) / p.MC);
            S = std::min(S, std::max(s0, (long long)(V + 15) / 16));
        }
        p.S = (int)S;
        p.grid = p.MC == 1 ? p.S : ((p.S + 7) / 8) * 8 * p.MC;
        p.kc = 64;
        p.lds = wide_lds_bytes(bm);
        p.vblock = 0;
    }
    if (p.kind == KIND_TILE) {
        // LM-head tile (fp32 heads only; every bf16 shape took one of the kernels
        // above): positions in chunks of 16*nt, 16 vocab rows per wave.
        const int need = (p.Meff + 15) / 16;
        p.va = 1;
        p.nt = need <= 1 ? 1 : 2;
        p.vblock = 64 * p.va;
        p.S = (V + p.vblock - 1) / p.vblock;
        p.MC = (p.Meff + 16 * p.nt - 1) / (16 * p.nt);
        const int kstep = 4 * epv;
        const int rows = std::min(16 * p.nt, p.Meff);
        const int h_pad = (H + kstep - 1) / kstep * kstep;
        int kc = ((kLdsBudget / rows - 16) / p.es) / kstep * kstep;
        if (kc < kstep) kc = kstep;
        p.kc = std::min(kc, h_pad);
        const size_t stage = (size_t)rows * (p.kc * p.es + 16);
        const size_t red = (size_t)4 * 16 * p.nt * sizeof(Partial);
        p.lds = std::max(stage, red);
        p.grid = p.MC == 1 ? p.S : ((p.S + 7) / 8) * 8 * p.MC;
    }
    // sampling jobs
    p.ntiles = (V + 63) / 64;
    p.NJ = mode == MTPV_MODE_GREEDY ? 0 : mode == MTPV_MODE_SAMPLE ? B : B * k;
    if (p.NJ > 0) {
        // About 1024 workgroups over all jobs where V allows, each chunk a whole number
        // of the passes' 64-tile trips (no half-empty trips), at most 64 chunks per job.
        // Short chunks are rounded down (more workgroups hide more latency); long ones
        // are rounded up when rounding down would pass the 1024 workgroups resident at
        // once (4 per compute unit), which would leave a second round of long chunks.
        int c = (1024 + p.NJ - 1) / p.NJ;
        c = std::max(1, std::min(c, 64));
        const int trip = 64;
        p.tpc = std::max(trip, p.ntiles / c / trip * trip);
        const long long wgs = (long long)p.NJ * ((p.ntiles + p.tpc - 1) / p.tpc);
        if ((p.ntiles + p.tpc - 1) / p.tpc > 64 || (wgs > 1024 && p.tpc >= 4 * trip))
            p.tpc = ((p.ntiles + c - 1) / c + trip - 1) / trip * trip;
        p.C = (p.ntiles + p.tpc - 1) / p.tpc;
    }
    // workspace layout
    size_t off = 0;
    p.off_err = off;
    off = align_up(off + 4, 256);
    p.off_partials = off;
    off = align_up(off + (size_t)p.Meff * p.S * sizeof(Partial), 256);
    p.off_dlogit = off;
    off = align_up(off + (size_t)p.Meff * sizeof(float), 256);
    p.off_rowstat = off;
    off = align_up(off + (size_t)p.Meff * sizeof(RowStat), 256);
    p.off_jobs = off;
    off = align_up(off + (size_t)p.NJ * sizeof(Job), 256);
    p.off_zpart = off;
    off = align_up(off + (size_t)p.NJ * p.C * 2 * sizeof(double), 256);
    p.off_tsum = off;
    off = align_up(off + (size_t)p.NJ * p.ntiles * sizeof(double), 256);
    p.off_spill = off;
    if (mode != MTPV_MODE_GREEDY) off = align_up(off + (size_t)p.Meff * V * sizeof(float), 256);
    p.off_tail = off;
    off = align_up(off + (size_t)p.tail_r * p.tail_ks * head_tile_piece_bytes(p.tail_fm, p.geo), 256);
    p.total = off;
    *pl = p;
    return MTPV_OK;
}

}  // namespace mtpv
