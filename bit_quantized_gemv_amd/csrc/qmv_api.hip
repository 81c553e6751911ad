// qmv_api.hip -- the C ABI of include/qmv.h: argument validation, launch
// planning and dispatch to the gfx950 kernel instances.
//
// Validation is plain host code and runs before any HIP call, so every error
// path is reachable (and tested) on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <mutex>

#include "qmv.h"
#include "qmv_dispatch.hpp"

namespace {

using qmv::KernelFn;
using qmv::Params;


int dtype_bytes(int dt) { return dt == QMV_DT_F32 ? 4 : 2; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

int r_index(int R) { return R - 1; }   // R in 1..4

static_assert(qmv::kStamps == QMV_STAMPS, "per-wavefront stamp record size");

// Pure argument check (no HIP calls).
int check_args(const uint32_t* w, const void* s, const void* b, const void* x, void* y, int M,
               int N, int K, int bits, int gs, int x_dt, int sb_dt, int y_dt, int R)
{
    if (!w || !s || !b || !x || !y) return QMV_E_NULL;
    if (bits != 2 && bits != 4) return QMV_E_BITS;
    if (gs != 64 && gs != 128) return QMV_E_GROUP;
    if (M < 1 || M > QMV_MAX_M) return QMV_E_M_RANGE;
    if (N < 1 || N > QMV_MAX_N || K < gs || K > QMV_MAX_K || K % gs != 0) return QMV_E_SHAPE;
    if (x_dt != QMV_DT_F32 && x_dt != QMV_DT_BF16) return QMV_E_DTYPE;
    if (sb_dt != QMV_DT_F16 && sb_dt != QMV_DT_BF16) return QMV_E_DTYPE;
    if (y_dt != QMV_DT_F32 && y_dt != QMV_DT_BF16) return QMV_E_DTYPE;
    if (R < 0 || R > 4) return QMV_E_ROWS;
    const long long G = K / gs;
    if (!aligned(w, 16) || !aligned(s, 16) || !aligned(b, 16) || !aligned(x, 16)) return QMV_E_ALIGN;
    if (!aligned(y, (size_t)dtype_bytes(y_dt))) return QMV_E_ALIGN;
    const size_t nw = (size_t)N * (size_t)K * bits / 8;
    const size_t nsb = (size_t)N * (size_t)G * 2;
    const size_t nx = (size_t)M * (size_t)K * dtype_bytes(x_dt);
    const size_t ny = (size_t)M * (size_t)N * dtype_bytes(y_dt);
    if (overlap(y, ny, w, nw) || overlap(y, ny, s, nsb) || overlap(y, ny, b, nsb) ||
        overlap(y, ny, x, nx))
        return QMV_E_ALIAS;
    return QMV_OK;
}

// Kernel instance for (bits, group size, activation and scale/bias dtypes,
// rows per wavefront, vectors, K windows); every instance keeps one unit in
// flight per wavefront.
KernelFn pick_kernel(int bits, int gs, bool xf32, bool sbf, int R, int PF, int M, bool win)
{
    if (PF != 1) return nullptr;
    const int ri = r_index(R);
    const int mi = M - 1;
    const int si = sbf ? 1 : 0;
    if (win) {
        if (bits == 4 && gs == 64) return xf32 ? qmv::qmv_wtable_b4_g64_f32[ri][mi][si] : qmv::qmv_wtable_b4_g64_bf16[ri][mi][si];
        if (bits == 4 && gs == 128) return xf32 ? qmv::qmv_wtable_b4_g128_f32[ri][mi][si] : qmv::qmv_wtable_b4_g128_bf16[ri][mi][si];
        if (bits == 2 && gs == 64) return xf32 ? qmv::qmv_wtable_b2_g64_f32[ri][mi][si] : qmv::qmv_wtable_b2_g64_bf16[ri][mi][si];
        return xf32 ? qmv::qmv_wtable_b2_g128_f32[ri][mi][si] : qmv::qmv_wtable_b2_g128_bf16[ri][mi][si];
    }
    if (bits == 4 && gs == 64) return xf32 ? qmv::qmv_table_b4_g64_f32[ri][mi][si] : qmv::qmv_table_b4_g64_bf16[ri][mi][si];
    if (bits == 4 && gs == 128) return xf32 ? qmv::qmv_table_b4_g128_f32[ri][mi][si] : qmv::qmv_table_b4_g128_bf16[ri][mi][si];
    if (bits == 2 && gs == 64) return xf32 ? qmv::qmv_table_b2_g64_f32[ri][mi][si] : qmv::qmv_table_b2_g64_bf16[ri][mi][si];
    return xf32 ? qmv::qmv_table_b2_g128_f32[ri][mi][si] : qmv::qmv_table_b2_g128_bf16[ri][mi][si];
}

struct Plan {
    Params p;
    KernelFn fn;
    bool win;   // fn is a K-windowed instance
    int R, W, PF, lds, grid, blocks_per_cu;
};

// LDS layout and K windows for workgroups of W wavefronts that walk up to
// `per` row blocks each.  Returns QMV_E_SHAPE if one wave step of activations
// for all M vectors does not fit in LDS.
int make_plan(int M, int N, int K, int bits, int gs, bool xf32, bool sbf, int R, int W, int PF, int per,
              Plan& pl)
{
    const int G = K / gs;
    const int chunks = K * bits / 128;
    const int nsteps = (chunks + qmv::kWave - 1) / qmv::kWave;
    const int xcb = (128 / bits) * (xf32 ? 4 : 2);
    // Whole K, scale/bias copies in LDS (the instances without K windows):
    // each of a wavefront's `per` row blocks takes a slot of whole 16-byte
    // pieces from the piece that holds its rows' first byte, and the slots
    // of all of them must fit one wave-wide load (kMetaBytes); the copies sit
    // in a static array of kMaxWaves * 2 * kMetaBytes bytes, and the lane
    // offsets of the loads are 32-bit.
    const long long m_slot = 16 * ((14 + 2LL * R * G + 15) / 16);
    const long long sb_bytes = (long long)N * G * 2;
    const int lpg = gs * bits / 128;
    const bool own_rows = (lpg == 2 || lpg == 4) && R % lpg == 0;   // instances that hold copies
    const bool copies_fit = per * m_slot <= qmv::kMetaBytes && sb_bytes <= (1LL << 31) - 16;
    const long long static_lds = (long long)qmv::kMaxWaves * 2 * qmv::kMetaBytes;
    // per vector and window: padded activations and a float2 per chunk
    // (dot-chain start, group sum).  Padding: 16 bytes after every 256.  With
    // one window a vector's slot holds the row's chunks and one zero chunk
    // after them (which the lanes past the row's end read), not the whole last
    // wave step; with more, every window's chunks (the last window's zero
    // chunk lies inside its slot).
    auto phys = [](long long o) { return o + ((o >> 8) << 4); };
    auto slot_bytes = [&](int w) -> int {
        if (w < nsteps) return (int)phys((long long)w * qmv::kWave * xcb);
        return (int)phys((long long)chunks * xcb) + (chunks < w * qmv::kWave ? xcb : 0);
    };
    int ws = nsteps, x_m = 0, sc_bytes = 0;
    long long total = 0;
    for (;;) {
        x_m = slot_bytes(ws);
        sc_bytes = M * ws * qmv::kWave * 8;
        total = (long long)M * x_m + sc_bytes;
        if (total <= qmv::kLdsBytes || ws == 1) break;
        --ws;
    }
    if (total > qmv::kLdsBytes) return QMV_E_SHAPE;
    const int nwin = (nsteps + ws - 1) / ws;
    ws = (nsteps + nwin - 1) / nwin;  // even windows
    x_m = nwin == 1 ? slot_bytes(ws) : (int)phys((long long)ws * qmv::kWave * xcb);
    sc_bytes = M * ws * qmv::kWave * 8;
    Params& p = pl.p;
    p.N = N;
    p.K = K;
    p.G = G;
    p.chunks = chunks;
    p.nsteps = nsteps;
    p.row_bytes = chunks * 16;
    p.win_steps = ws;
    p.nwin = nwin;
    p.n_rb = (N + W * R - 1) / (W * R);
    p.x_m_bytes = x_m;
    p.s_off = M * x_m;
    pl.lds = p.s_off + sc_bytes;
    // Whole K: instances whose lanes fold their own rows hold the copies when
    // they fit (beside the static array); where they do not, the K-windowed
    // instance, which loads the scales and biases per unit, serves one window.
    const bool mlds = nwin == 1 && own_rows && copies_fit && pl.lds + static_lds <= qmv::kLdsBytes;
    p.m_slot = mlds ? (int)m_slot : 0;
    p.sb_last = mlds ? (int)((sb_bytes - 1) & ~15LL) : 0;
    p.m_div = mlds ? (8192 + (int)(m_slot / 16) - 1) / (int)(m_slot / 16) : 0;
    // staging rounds per vector: 16-byte units (8 values; 16 for bf16
    // activations with 2-bit codes) of a window over the workgroup's threads
    {
        const int uv = (!xf32 && bits == 2) ? 16 : 8;
        const int vpc = 128 / bits;
        const int nthr = W * qmv::kWave;
        auto rounds_of = [&](int c_n) { return (c_n * vpc / uv + nthr - 1) / nthr; };
        p.rpm_full = rounds_of(std::min(chunks, ws * qmv::kWave));
        p.rpm_last = rounds_of(chunks - (nwin - 1) * ws * qmv::kWave);
    }
    p.rb_per = 0;    // set with the grid
    p.rb_full = 0;
    pl.R = R;
    pl.W = W;
    pl.PF = PF;
    pl.win = nwin > 1 || (own_rows && !mlds);
    pl.fn = pick_kernel(bits, gs, xf32, sbf, R, PF, M, pl.win);
    return QMV_OK;
}

// Per-device launch-shape cache: compute-unit count, and for each kernel
// instance, workgroup size and LDS size the resident workgroups per CU (after
// raising the instance's dynamic-LDS limit) and the instance's private
// (spill) bytes per lane.  Filled on first use; never invalidated.
struct OccEntry {
    const void* fn;
    int dev;
    int lds;
    int w;
    int blocks;
    int scratch;
};

std::mutex g_mu;
int g_cus[64] = {0};
OccEntry g_occ[1024];
int g_nocc = 0;

int cu_count_locked(int dev)
{
    if (dev < 0 || dev >= 64) return 256;
    if (g_cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        g_cus[dev] = n;
    }
    return g_cus[dev];
}

int cu_count(int dev)
{
    std::lock_guard<std::mutex> lk(g_mu);
    return cu_count_locked(dev);
}

// Resident workgroups per CU of an instance at a workgroup size and LDS size,
// and its private bytes per lane.  False on a HIP error.
bool occupancy(const void* fn, int W, int lds, int dev, int& blocks, int& scratch)
{
    std::lock_guard<std::mutex> lk(g_mu);
    for (int i = 0; i < g_nocc; ++i)
        if (g_occ[i].fn == fn && g_occ[i].dev == dev && g_occ[i].lds == lds && g_occ[i].w == W) {
            blocks = g_occ[i].blocks;
            scratch = g_occ[i].scratch;
            return true;
        }
    if (lds > 65536 && hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
        return false;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, W * qmv::kWave, lds) != hipSuccess) return false;
    hipFuncAttributes attr;
    if (hipFuncGetAttributes(&attr, fn) != hipSuccess) return false;
    blocks = nb < 0 ? 0 : nb;
    scratch = (int)attr.localSizeBytes;
    if (g_nocc < 1024) g_occ[g_nocc++] = OccEntry{fn, dev, lds, W, blocks, scratch};
    return true;
}

// A candidate launch: the plan for (R, W, PF) with its grid, or false when
// the shape has no instance or no resident workgroup.  Returns -1 on a HIP
// error.
int try_plan(int M, int N, int K, int bits, int gs, bool xf32, bool sbf, int R, int W, int PF,
             int dev, int cus, Plan& pl, bool& shape_ok)
{
    // Whether a whole-K plan holds the scale/bias copies of its row blocks
    // depends on the row blocks per workgroup, which follow from the resident
    // workgroups, which the instance and its LDS decide: start from one block
    // and plan again until the plan holds every block its workgroups walk.
    int reserve = 1;
    for (int iter = 0; iter < 16; ++iter) {
        if (make_plan(M, N, K, bits, gs, xf32, sbf, R, W, PF, reserve, pl) != QMV_OK) return 0;
        shape_ok = true;
        if (pl.fn == nullptr) return 0;
        int nb = 0, scratch = 0;
        if (!occupancy(reinterpret_cast<const void*>(pl.fn), W, pl.lds, dev, nb, scratch)) return -1;
        if (nb == 0) return 0;
        const int n_rb = pl.p.n_rb;
        const int cap = nb * cus;
        int per = (n_rb + cap - 1) / cap;         // row blocks per workgroup
        // Memory-bound calls: at least two row blocks per workgroup while that
        // still leaves a workgroup for every compute unit -- the activations
        // are staged once for both and the second block's loads overlap the
        // first's compute (measured: 1% on 15360 x 3840 at 4 bits, and the
        // choice the occupancy already makes at 2 bits, where a row is one
        // wave step).
        if (M <= 2 && per == 1 && n_rb >= 2 * cus) per = 2;
        if (pl.p.m_slot > 0 && per > reserve) {
            reserve = per;
            continue;
        }
        pl.grid = (n_rb + per - 1) / per;
        pl.blocks_per_cu = nb;
        pl.p.rb_per = (n_rb + pl.grid - 1) / pl.grid;
        pl.p.rb_full = n_rb - (pl.p.rb_per - 1) * pl.grid;
        return 1;
    }
    return 0;
}

// Rows the busiest compute unit processes: workgroups are dealt out whole, so
// a compute unit holds up to ceil(grid / CUs) of them, each covering `per` row
// blocks of W*R rows.
int busiest_cu_rows(const Plan& pl, int cus)
{
    const int per = (pl.p.n_rb + pl.grid - 1) / pl.grid;
    return ((pl.grid + cus - 1) / cus) * per * pl.W * pl.R;
}

// Launch shape (measured on MI355X over the 12B- and 27B-class projection
// shapes; an explicit rows-per-wavefront request is honoured in both cases):
//   * M <= 2, bound by memory: 8 wavefronts, one unit in flight, and the rows
//     per wavefront that put the fewest rows on the busiest compute unit
//     (ties: 2, 3, 1, 4 rows; one row's many small workgroups measure slower
//     than three rows at equal rows per CU; fewer wavefronts when 8 do not
//     fit) -- then, for 4-bit codes, one workgroup per compute unit at four or
//     three rows where that keeps the busiest unit's rows (below).  Four rows
//     on 15360 rows (240 workgroups of two 32-row blocks, 64 rows per CU, as
//     two-row workgroups have); two on 3840 (240 workgroups of 16 rows); three
//     on 5120 (214 workgroups of 24 rows instead of 320 of 16, 16% faster) and
//     on 17408 (242 workgroups of three 24-row blocks, 72 rows per CU; by row
//     count alone one row per wavefront in 726 workgroups, which beat 363
//     workgroups of two 24-row blocks by 14%); two on the 2-bit shapes.
//   * M >= 3, bound by the vector ALUs: 8 wavefronts, one unit in flight, and
//     the R that minimises the rows the busiest compute unit processes,
//     weighted by the per-row cost of fewer rows per wavefront (the
//     activations read from LDS and the decode are shared by fewer rows): 1.2x
//     for three rows (ungrouped folds), 1.1x for two and 2.5x for one,
//     relative to four (one row per wavefront reads the activations from LDS
//     once per row, which makes it LDS-bound where the vector ALUs are busy).
//   * 2-bit codes have no four-row instances; K-windowed calls have one unit
//     in flight.
int choose_plan(int M, int N, int K, int bits, int gs, bool xf32, bool sbf, int R_req, Plan& best)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QMV_E_LAUNCH;
    const int cus = cu_count(dev);
    if (bits == 2 && R_req >= 3) R_req = 2;      // no three- or four-row 2-bit instances
    bool shape_ok = false;
    if (M <= 2) {
        // bound by memory: rows are equally cheap at any R, so the R that puts
        // the fewest rows on the busiest compute unit, ties in this order
        const int Rs[4] = {2, 3, 1, 4};
        int best_rows = 0;
        bool found = false;
        for (int R : Rs) {
            if ((R_req != 0 && R != R_req) || (bits == 2 && R >= 3)) continue;
            for (int W = qmv::kMaxWaves; W >= 1; --W) {
                Plan pl;
                const int st = try_plan(M, N, K, bits, gs, xf32, sbf, R, W, 1, dev, cus, pl, shape_ok);
                if (st < 0) return QMV_E_LAUNCH;
                if (st == 0) continue;
                const int rows_cu = busiest_cu_rows(pl, cus);
                if (!found || rows_cu < best_rows) {
                    found = true;
                    best_rows = rows_cu;
                    best = pl;
                }
                break;
            }
        }
        // One workgroup of eight wavefronts per compute unit, with four (else
        // three) rows per wavefront, where that puts no more rows on the
        // busiest compute unit: no second workgroup stages its activations
        // behind the first one's weight requests, and 8 x R KiB of weights
        // stay in flight per compute unit, 24-32 KiB at R = 3-4.  Measured
        // (bench.py --sweep-launch, two boxes): 15360 x 3840, R = 4, 240
        // workgroups of two row blocks: 3-4% faster at M = 1 and 5.5% at M = 2
        // than 480 two-row workgroups; 17408 x 5120, R = 3, 242 workgroups of
        // three blocks: 2-3% and 5.5-8.6% faster than 726 one-row workgroups.
        // (At two rows, 16 KiB in flight, one workgroup per compute unit is
        // slower: 2-bit 15360 x 3840, 5-7%.)
        if (found && bits == 4) {
            for (int R : {4, 3}) {
                if (R_req != 0 && R != R_req) continue;
                constexpr int W = qmv::kMaxWaves;
                const int n_rb = (N + W * R - 1) / (W * R);
                const int per = (n_rb + cus - 1) / cus;
                Plan pl;
                if (make_plan(M, N, K, bits, gs, xf32, sbf, R, W, 1, per, pl) != QMV_OK || pl.fn == nullptr)
                    continue;
                int nb = 0, scratch = 0;
                if (!occupancy(reinterpret_cast<const void*>(pl.fn), W, pl.lds, dev, nb, scratch)) return QMV_E_LAUNCH;
                if (nb == 0) continue;
                pl.grid = (n_rb + per - 1) / per;
                pl.blocks_per_cu = nb;
                pl.p.rb_per = (n_rb + pl.grid - 1) / pl.grid;
                pl.p.rb_full = n_rb - (pl.p.rb_per - 1) * pl.grid;
                if (busiest_cu_rows(pl, cus) <= best_rows) {
                    best = pl;
                    break;
                }
            }
        }
        if (found) return QMV_OK;
    } else {
        const int Rs[4] = {4, 3, 2, 1};
        const double cost[4] = {1.0, 1.2, 1.1, 2.5};
        double best_score = 0.0;
        bool found = false;
        for (int i = 0; i < 4; ++i) {
            const int R = Rs[i];
            if ((R_req != 0 && R != R_req) || (bits == 2 && R >= 3)) continue;
            for (int W = qmv::kMaxWaves; W >= 1; --W) {
                Plan pl;
                const int st = try_plan(M, N, K, bits, gs, xf32, sbf, R, W, 1, dev, cus, pl, shape_ok);
                if (st < 0) return QMV_E_LAUNCH;
                if (st == 0) continue;
                const double score = busiest_cu_rows(pl, cus) * cost[i];
                if (!found || score < best_score - 1e-9) {
                    found = true;
                    best_score = score;
                    best = pl;
                }
                break;
            }
        }
        if (found) return QMV_OK;
    }
    return shape_ok ? QMV_E_LAUNCH : QMV_E_SHAPE;
}

// Vectors per launch: at most QMV_TILE_M, and at most as many as one wave
// step of activations of fits in LDS (fewer only for fp32 activations with
// 2-bit codes); the M vectors are then cut into equal tiles of at most that
// many.  Vectors are independent, so tiling M changes no result bit.
int vectors_per_launch(int M, int N, int K, int bits, int gs, bool xf32)
{
    int cap = 0;
    for (int mc = std::min(M, QMV_TILE_M); mc >= 1; --mc) {
        Plan pl;
        if (make_plan(mc, N, K, bits, gs, xf32, true, 1, 1, 1, 1, pl) == QMV_OK) {
            cap = mc;
            break;
        }
    }
    if (cap == 0) return 0;
    const int tiles = (M + cap - 1) / cap;
    return (M + tiles - 1) / tiles;
}

// Vectors per launch, final: when a launch of vectors_per_launch() vectors
// would window K (its activations do not fit in LDS whole) and its workgroups
// walk more than one row block each, every block restages every window.  If
// tiles of at least half as many vectors fit whole K, the vectors are cut
// into those instead (measured on the 17408 x 5120 projection at M = 13:
// two whole-K launches take ~20% less time than one windowed launch).
int tile_vectors(int M, int N, int K, int bits, int gs, bool xf32, bool sbf, int R_req)
{
    const int mc = vectors_per_launch(M, N, K, bits, gs, xf32);
    if (mc < 2) return mc;
    Plan pl;
    if (choose_plan(mc, N, K, bits, gs, xf32, sbf, R_req, pl) != QMV_OK) return mc;
    if (pl.p.nwin == 1 || pl.p.n_rb <= pl.grid) return mc;
    for (int mk = mc - 1; mk >= (mc + 1) / 2; --mk) {
        Plan q;
        if (make_plan(mk, N, K, bits, gs, xf32, sbf, 1, 1, 1, 1, q) == QMV_OK && q.p.nwin == 1) {
            const int tiles = (M + mk - 1) / mk;
            return (M + tiles - 1) / tiles;
        }
    }
    return mc;
}

}  // namespace

extern "C" {

int qmv_affine_ex(const uint32_t* w_packed, const void* scales, const void* biases,
                  const void* x, void* y, int M, int N, int K, int bits, int group_size,
                  qmv_dtype x_dt, qmv_dtype sb_dt, qmv_dtype y_dt, int rows_per_wave,
                  void* stream)
{
    int st = check_args(w_packed, scales, biases, x, y, M, N, K, bits, group_size, x_dt, sb_dt,
                        y_dt, rows_per_wave);
    if (st != QMV_OK) return st;
    const bool xf32 = (x_dt == QMV_DT_F32);
    const bool sbf = (sb_dt == QMV_DT_BF16);
    const int mc = tile_vectors(M, N, K, bits, group_size, xf32, sbf, rows_per_wave);
    if (mc < 1) return QMV_E_SHAPE;
    // Tiles of mc vectors and, when M is not a multiple of mc, one last tile
    // of M % mc: both plans are made before the first launch is enqueued, so a
    // plan that fails leaves y untouched.
    const int last = M % mc;
    Plan plans[2];
    st = choose_plan(mc, N, K, bits, group_size, xf32, sbf, rows_per_wave, plans[0]);
    if (st != QMV_OK) return st;
    if (last != 0) {
        st = choose_plan(last, N, K, bits, group_size, xf32, sbf, rows_per_wave, plans[1]);
        if (st != QMV_OK) return st;
    }
    for (int m0 = 0; m0 < M; m0 += mc) {
        Plan& pl = plans[(M - m0 < mc) ? 1 : 0];
        Params& p = pl.p;
        p.w = w_packed;
        p.s = static_cast<const uint16_t*>(scales);
        p.b = static_cast<const uint16_t*>(biases);
        p.x = static_cast<const uint8_t*>(x) + (size_t)m0 * K * dtype_bytes(x_dt);
        p.y = static_cast<uint8_t*>(y) + (size_t)m0 * N * dtype_bytes(y_dt);
        p.y_bf16 = (y_dt == QMV_DT_BF16);
        void* args[] = {&p};
        const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(pl.fn), dim3(pl.grid),
                                             dim3(pl.W * qmv::kWave), args, (size_t)pl.lds,
                                             static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return QMV_E_LAUNCH;
    }
    return QMV_OK;
}

int qmv_affine(const uint32_t* w_packed, const void* scales, const void* biases, const void* x,
               void* y, int M, int N, int K, int bits, int group_size, void* stream)
{
    return qmv_affine_ex(w_packed, scales, biases, x, y, M, N, K, bits, group_size, QMV_DT_BF16,
                         QMV_DT_BF16, QMV_DT_BF16, 0, stream);
}

int qmv_kernel_info(int M, int N, int K, int bits, int group_size, qmv_dtype x_dt,
                    qmv_dtype sb_dt, qmv_dtype y_dt, int rows_per_wave, qmv_kernel_info_t* out)
{
    if (!out) return QMV_E_NULL;
    // validate the shape with stand-in aligned, non-overlapping pointers
    const uintptr_t base = 1u << 20;
    const uintptr_t stride = (uintptr_t)1 << 40;
    int st = check_args(reinterpret_cast<const uint32_t*>(base), reinterpret_cast<const void*>(base + stride),
                        reinterpret_cast<const void*>(base + 2 * stride), reinterpret_cast<const void*>(base + 3 * stride),
                        reinterpret_cast<void*>(base + 4 * stride), M, N, K, bits, group_size, x_dt,
                        sb_dt, y_dt, rows_per_wave);
    if (st != QMV_OK) return st;
    const bool xf32 = (x_dt == QMV_DT_F32);
    const bool sbf = (sb_dt == QMV_DT_BF16);
    const int mc = tile_vectors(M, N, K, bits, group_size, xf32, sbf, rows_per_wave);
    if (mc < 1) return QMV_E_SHAPE;
    Plan pl;
    st = choose_plan(mc, N, K, bits, group_size, xf32, sbf, rows_per_wave, pl);
    if (st != QMV_OK) return st;
    hipFuncAttributes attr;
    if (hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(pl.fn)) != hipSuccess) return QMV_E_LAUNCH;
    out->vgprs = attr.numRegs;
    out->scratch_bytes = (int)attr.localSizeBytes;
    out->lds_bytes = pl.lds + (int)attr.sharedSizeBytes;
    out->wg_size = pl.W * qmv::kWave;
    out->grid = pl.grid;
    // workgroups on the busiest compute unit (at most the resident count),
    // times their wavefronts, over the four SIMDs of a compute unit
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QMV_E_LAUNCH;
    const int cus = cu_count(dev);
    out->waves_per_simd = (std::min(pl.blocks_per_cu, (pl.grid + cus - 1) / cus) * pl.W + 3) / 4;
    out->rows_per_wave = pl.R;
    out->k_windows = pl.p.nwin;
    out->prefetch_units = pl.PF;
    out->meta_lds = pl.p.m_slot > 0 ? 1 : 0;
    return QMV_OK;
}

int qmv_affine_shape(const uint32_t* w_packed, const void* scales, const void* biases,
                     const void* x, void* y, int M, int N, int K, int bits, int group_size,
                     qmv_dtype x_dt, qmv_dtype sb_dt, qmv_dtype y_dt, int rows_per_wave,
                     int waves_per_wg, int row_blocks_per_wg, qmv_kernel_info_t* info, void* stream)
{
    if (rows_per_wave < 1) return QMV_E_ROWS;
    int st = check_args(w_packed, scales, biases, x, y, M, N, K, bits, group_size, x_dt, sb_dt,
                        y_dt, rows_per_wave);
    if (st != QMV_OK) return st;
    if (bits == 2 && rows_per_wave >= 3) return QMV_E_ROWS;    // no three- or four-row 2-bit instances
    if (waves_per_wg < 1 || waves_per_wg > qmv::kMaxWaves || row_blocks_per_wg < 1) return QMV_E_SHAPE;
    const bool xf32 = (x_dt == QMV_DT_F32);
    const bool sbf = (sb_dt == QMV_DT_BF16);
    // one launch: at most the vectors qmv_affine_ex launches together
    const int mc = tile_vectors(M, N, K, bits, group_size, xf32, sbf, rows_per_wave);
    if (mc < 1) return QMV_E_SHAPE;
    if (mc < M) return QMV_E_M_RANGE;
    Plan pl;
    st = make_plan(M, N, K, bits, group_size, xf32, sbf, rows_per_wave, waves_per_wg, 1, row_blocks_per_wg, pl);
    if (st != QMV_OK) return st;
    if (pl.fn == nullptr) return QMV_E_ROWS;
    int dev = 0, nb = 0, scratch = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QMV_E_LAUNCH;
    if (!occupancy(reinterpret_cast<const void*>(pl.fn), waves_per_wg, pl.lds, dev, nb, scratch)) return QMV_E_LAUNCH;
    if (nb == 0) return QMV_E_LAUNCH;
    // workgroups of row_blocks_per_wg row blocks each (the last ones one fewer
    // where the count does not divide)
    const int n_rb = pl.p.n_rb;
    pl.grid = (n_rb + row_blocks_per_wg - 1) / row_blocks_per_wg;
    pl.blocks_per_cu = nb;
    pl.p.rb_per = (n_rb + pl.grid - 1) / pl.grid;
    pl.p.rb_full = n_rb - (pl.p.rb_per - 1) * pl.grid;
    if (info) {
        hipFuncAttributes attr;
        if (hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(pl.fn)) != hipSuccess) return QMV_E_LAUNCH;
        const int cus = cu_count(dev);
        info->vgprs = attr.numRegs;
        info->scratch_bytes = (int)attr.localSizeBytes;
        info->lds_bytes = pl.lds + (int)attr.sharedSizeBytes;
        info->wg_size = waves_per_wg * qmv::kWave;
        info->grid = pl.grid;
        info->waves_per_simd = (std::min(nb, (pl.grid + cus - 1) / cus) * waves_per_wg + 3) / 4;
        info->rows_per_wave = rows_per_wave;
        info->k_windows = pl.p.nwin;
        info->prefetch_units = pl.PF;
        info->meta_lds = pl.p.m_slot > 0 ? 1 : 0;
    }
    Params& p = pl.p;
    p.w = w_packed;
    p.s = static_cast<const uint16_t*>(scales);
    p.b = static_cast<const uint16_t*>(biases);
    p.x = x;
    p.y = y;
    p.y_bf16 = (y_dt == QMV_DT_BF16);
    void* args[] = {&p};
    if (hipLaunchKernel(reinterpret_cast<const void*>(pl.fn), dim3(pl.grid), dim3(waves_per_wg * qmv::kWave), args,
                        (size_t)pl.lds, static_cast<hipStream_t>(stream)) != hipSuccess)
        return QMV_E_LAUNCH;
    return QMV_OK;
}

int qmv_affine_timeline(const uint32_t* w_packed, const void* scales, const void* biases,
                        const void* x, void* y, int M, int N, int K, int bits, int group_size,
                        qmv_dtype y_dt, int rows_per_wave, uint64_t* stamps, long long stamps_len,
                        qmv_timeline_info_t* info, void* stream)
{
    if (!info) return QMV_E_NULL;
    int st = check_args(w_packed, scales, biases, x, y, M, N, K, bits, group_size, QMV_DT_BF16,
                        QMV_DT_BF16, y_dt, rows_per_wave);
    if (st != QMV_OK) return st;
    // the stamped sets: 4-bit codes in groups of 64, 2-bit codes in groups of 128
    if ((bits == 4) != (group_size == 64)) return QMV_E_GROUP;
    if (M > QMV_TILE_M) return QMV_E_M_RANGE;
    if (stamps && !aligned(stamps, 8)) return QMV_E_ALIGN;
    if (stamps && stamps_len < 1) return QMV_E_SHAPE;
    if (stamps) {
        const size_t nst = (size_t)stamps_len * 8;
        const size_t nw = (size_t)N * (size_t)K * bits / 8, nsb = (size_t)N * (size_t)(K / group_size) * 2;
        const size_t nx = (size_t)M * (size_t)K * 2, ny = (size_t)M * (size_t)N * dtype_bytes(y_dt);
        if (overlap(stamps, nst, w_packed, nw) || overlap(stamps, nst, scales, nsb) ||
            overlap(stamps, nst, biases, nsb) || overlap(stamps, nst, x, nx) || overlap(stamps, nst, y, ny))
            return QMV_E_ALIAS;
    }
    // the call must be the one launch qmv_affine_ex would make
    const int mc = tile_vectors(M, N, K, bits, group_size, false, true, rows_per_wave);
    if (mc < 1) return QMV_E_SHAPE;
    if (mc < M) return QMV_E_M_RANGE;
    Plan pl;
    st = choose_plan(M, N, K, bits, group_size, false, true, rows_per_wave, pl);
    if (st != QMV_OK) return st;
    const qmv::TimelineFn tfn = (bits == 4 ? qmv::qmv_timeline_b4_g64_bf16
                                           : qmv::qmv_timeline_b2_g128_bf16)[pl.win ? 1 : 0][pl.R - 1][M - 1];
    if (tfn == nullptr) return QMV_E_LAUNCH;
    int dev = 0, khz = 0, nb = 0, scratch = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QMV_E_LAUNCH;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return QMV_E_LAUNCH;
    if (!occupancy(reinterpret_cast<const void*>(tfn), pl.W, pl.lds, dev, nb, scratch)) return QMV_E_LAUNCH;
    hipFuncAttributes ta, pa;
    if (hipFuncGetAttributes(&ta, reinterpret_cast<const void*>(tfn)) != hipSuccess ||
        hipFuncGetAttributes(&pa, reinterpret_cast<const void*>(pl.fn)) != hipSuccess)
        return QMV_E_LAUNCH;
    info->waves = pl.grid * pl.W;
    info->wg_size = pl.W * qmv::kWave;
    info->grid = pl.grid;
    info->clock_khz = khz;
    info->blocks_per_cu = nb;
    info->product_blocks_per_cu = pl.blocks_per_cu;
    info->vgprs = ta.numRegs;
    info->product_vgprs = pa.numRegs;
    if (!stamps) return QMV_OK;
    if (stamps_len < (long long)info->waves * QMV_STAMPS) return QMV_E_SHAPE;
    Params& p = pl.p;
    p.w = w_packed;
    p.s = static_cast<const uint16_t*>(scales);
    p.b = static_cast<const uint16_t*>(biases);
    p.x = static_cast<const uint8_t*>(x);
    p.y = y;
    p.y_bf16 = (y_dt == QMV_DT_BF16);
    void* args[] = {&p, &stamps};
    if (hipLaunchKernel(reinterpret_cast<const void*>(tfn), dim3(pl.grid), dim3(pl.W * qmv::kWave), args,
                        (size_t)pl.lds, static_cast<hipStream_t>(stream)) != hipSuccess)
        return QMV_E_LAUNCH;
    return QMV_OK;
}

const char* qmv_status_string(int status)
{
    switch (status) {
    case QMV_OK: return "QMV_OK";
    case QMV_E_NULL: return "QMV_E_NULL";
    case QMV_E_BITS: return "QMV_E_BITS";
    case QMV_E_GROUP: return "QMV_E_GROUP";
    case QMV_E_SHAPE: return "QMV_E_SHAPE";
    case QMV_E_M_RANGE: return "QMV_E_M_RANGE";
    case QMV_E_ALIGN: return "QMV_E_ALIGN";
    case QMV_E_DTYPE: return "QMV_E_DTYPE";
    case QMV_E_ROWS: return "QMV_E_ROWS";
    case QMV_E_ALIAS: return "QMV_E_ALIAS";
    case QMV_E_LAUNCH: return "QMV_E_LAUNCH";
    default: return "QMV_E_UNKNOWN";
    }
}

}  // extern "C"
