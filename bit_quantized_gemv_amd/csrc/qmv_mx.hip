// qmv_mx.hip -- gfx950 kernel and C ABI of the mxfp4 mode of the streamed qmv:
//
//   y[m][n] = sum_b X[n][b] * sum_{k in b} e2m1(q[n][k]) * x[m][k]
//
// with FP4 E2M1 codes q packed 8 per uint32 (field 0 in the low bits), one
// E8M0 scale X = 2^(E - 127) per block of 32 values along K, and bf16 or
// fp32 activations.  The MLX pages list this quantization mode beside the affine
// one (mlxcel issue "an order-preserving streamed qmv would give MTP the fast
// kernel and byte-identity together", section "Scope limits") without
// defining the format; the element and scale formats are those of the OCP
// Microscaling Formats (MX) specification v1.0.
//
// Work decomposition and order (the affine kernel's, without bias and with
// one block per lane):
//   * Chunk c (16 bytes = 32 codes = one block) of a row is read by lane c % 64
//     in wave step c / 64; a wavefront owns R consecutive rows; a workgroup of
//     W wavefronts stages x[0..M)[0..K) in LDS (its own dtype, natural order,
//     one zero chunk past the row's last, which the lanes past the row's end
//     read) and walks row blocks of W*R rows.
//   * Per row, chunk and vector: the codes of each byte become an exact bf16
//     pair (v_cvt_scalef32_pk_bf16_fp4 with scale 1: low nibble first); D is
//     the v_dot2_f32_bf16 chain over the chunk's 16 pairs, in byte order,
//     from 0; the lane folds acc = fma(X, D, acc) over its chunks in
//     ascending step.  A lane owns its chunk's block, so no lanes combine.
//   * Row total: lanes l and l ^ d combined for d = 32, 16, 8, 4, 2, 1, then
//     round-to-nearest-even to y's dtype.
//   None of this depends on M, R, W or the grid, so every output vector equals
//   the one-vector call on that vector bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <utility>

#include "qmv.h"
#include "qmv_kernel.hpp"

namespace qmv {

struct MxParams {
    const uint32_t* w;
    const uint8_t* s;
    const void* x;
    void* y;
    int N;
    int K;
    int chunks;      // K / 32
    int nsteps;      // ceil(chunks / 64)
    int row_bytes;   // K / 2
    int n_rb;        // row blocks of W*R rows
    int y_bf16;
    int win_steps;   // wave steps per K window (even unless one window covers K)
    int nwin;        // K windows
    int xm_bytes;    // LDS bytes of one vector's slot, padded: a window's chunks (win_steps*64),
                     // or with the whole K the row's chunks and one zero chunk (at most nsteps*64)
    uint32_t ipm_magic;  // i / (16-byte pieces per vector slot) is
    int ipm_shift;       // umulhi(i, ipm_magic) >> ipm_shift for every staging index i
};

// 2^(E - 127) as fp32 from an E8M0 byte: E = 0 is the subnormal 2^-127 and
// E = 255 is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e)
{
    const uint32_t bits = (e == 0u) ? 0x00400000u : ((e == 255u) ? 0x7fc00000u : (e << 23));
    return __uint_as_float(bits);
}

// The four bytes of a word of E2M1 codes as exact bf16 pairs, byte j ->
// (code 2j, code 2j+1) with the low nibble in the low half (the byte select of
// the conversion must be a constant).
__device__ __forceinline__ uint4 fp4_word_to_bf16_pairs(uint32_t w)
{
    return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3)));
}

// The eight codes of a word as exact fp32 values, code 0 (low nibble of byte 0)
// first.
__device__ __forceinline__ void fp4_word_to_f32(uint32_t w, float (&out)[8])
{
    const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    out[0] = p0[0]; out[1] = p0[1]; out[2] = p1[0]; out[3] = p1[1];
    out[4] = p2[0]; out[5] = p2[1]; out[6] = p3[0]; out[7] = p3[1];
}

// WIN: the activations do not fit in LDS whole for this launch; they are
// staged window by window (win_steps wave steps at a time) for every row block,
// with the accumulators kept in registers across windows, which gives the
// same bits as staging them whole.
// XF32: fp32 activations -- each code becomes an exact fp32
// (v_cvt_scalef32_pk_f32_fp4, scale 1) and the chunk's dot is the fma chain
// over its 32 values in ascending k, from 0.
template <int R, int M, bool WIN, bool XF32>
__global__ __launch_bounds__(kMaxWaves * kWave) void qmv_mx_kernel(MxParams p)
{
    constexpr int V = R * M;
    constexpr int P = pow2_at_least(V);
    static_assert(P <= kWave, "too many row totals per lane");
    extern __shared__ __align__(16) uint8_t lds[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int W = blockDim.x / kWave;
    const int grid = gridDim.x;
    // (the grid never exceeds the row blocks, so every workgroup has one; a
    // test of that here would hold back the other argument loads)

    const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w, -1);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.s, -1);
    uint4 wb[2][R];
    uint32_t eb[2][R];
    // loads of step t of row block rb (rows past N read row N-1, chunks past
    // the row's end its last chunk)
    auto issue = [&](int slot, int rb, int t) {
        const int n0 = (rb * W + wave) * R;
        const int c = min(t * kWave + lane, p.chunks - 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int n = min(n0 + r, p.N - 1);
            wb[slot][r] = buf_load_nt(wr, n * p.row_bytes + c * 16, 0);
            eb[slot][r] = __builtin_amdgcn_raw_buffer_load_b8(sr, n * p.chunks + c, 0, 0);
        }
    };

    // ---- stage x[0..M)[window]: 16-byte pieces, four per chunk; pieces of
    // chunks past the row's end are zero.  All of a thread's loads of a batch
    // are issued before any store; the first batch of the first window carries
    // the first weight step behind it.
    const int cwin = p.win_steps * kWave;                 // chunks per window
    // Chunks in a vector's LDS slot: a window's, or with the whole K the row's
    // and one zero chunk after them (which the lanes past the row's end read)
    const int cslot = WIN ? cwin : min(p.chunks + 1, cwin);
    constexpr int XB = XF32 ? 4 : 2;                      // activation bytes
    constexpr int PSH = XF32 ? 3 : 2;                     // log2 of 16-byte pieces per chunk
    constexpr int PPC = 1 << PSH;
    constexpr int CB = 32 * XB;                           // LDS bytes per chunk
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.x, M * p.K * XB);
    // 16-byte pieces per thread and batch: a window of one or two vectors has
    // few per thread, and the clamped re-reads that fill a larger batch cost
    // more than the second batch a long window then needs
    constexpr int SB = (M == 1) ? 2 : (M == 2 ? 4 : 8);
    auto stage = [&](int win, auto first_tag) {
        const int items = M * cslot * PPC;
        const int c0 = win * cwin;
        auto batch = [&](int i0, auto with_issue) {
            uint4 v[SB];
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                const int i = min(i0 + j * (int)blockDim.x + (int)threadIdx.x, items - 1);
                const int m = (int)(__umulhi((uint32_t)i, p.ipm_magic) >> p.ipm_shift), rem = i - m * (cslot * PPC);
                const int c = min(c0 + (rem >> PSH), p.chunks - 1), piece = rem & (PPC - 1);
                v[j] = buf_load(xr, (m * p.K + c * 32) * XB + piece * 16);
            }
            if constexpr (decltype(with_issue)::value) issue(0, blockIdx.x, 0);
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                const int i = i0 + j * (int)blockDim.x + (int)threadIdx.x;
                if (i < items) {
                    const int m = (int)(__umulhi((uint32_t)i, p.ipm_magic) >> p.ipm_shift), rem = i - m * (cslot * PPC);
                    const int cl = rem >> PSH, piece = rem & (PPC - 1);
                    const uint4 d = (c0 + cl < p.chunks) ? v[j] : make_uint4(0, 0, 0, 0);
                    *reinterpret_cast<uint4*>(lds + m * p.xm_bytes + lds_phys(cl * CB + piece * 16)) = d;
                }
            }
        };
        batch(0, first_tag);
        for (int i0 = SB * (int)blockDim.x; i0 < items; i0 += SB * (int)blockDim.x) batch(i0, std::false_type{});
    };
    if constexpr (!WIN) {
        stage(0, std::true_type{});
        __syncthreads();
    }

    for (int rb = blockIdx.x; rb < p.n_rb; rb += grid) {
        const int n0 = (rb * W + wave) * R;
        float acc[R][M];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

        // one step: the next step's loads go out, then this step's chunk is
        // decoded and every vector's chain and fold run (the slot is a
        // compile-time constant, so the ring stays in registers)
        auto step = [&](auto slot_tag, int t) {
            constexpr int slot = decltype(slot_tag)::value;
            // next loads: this row block's next step; after its last step, the
            // next row block's first step when that lands in slot 0 (an even
            // step count), else a harmless reload of this step
            const bool last = t + 1 == p.nsteps;
            const bool cross = last && rb + grid < p.n_rb && (p.nsteps & 1) == 0;
            issue(slot ^ 1, cross ? rb + grid : rb, cross ? 0 : min(t + 1, p.nsteps - 1));
            __builtin_amdgcn_sched_barrier(0);
            const int cl = (t - (t / p.win_steps) * p.win_steps) * kWave + lane;   // chunk in its window
            float sc[R];
#pragma unroll
            for (int r = 0; r < R; ++r) sc[r] = e8m0_to_f32(eb[slot][r] & 0xffu);
            // (whole K: lanes past the row's end read the zero chunk)
            const uint8_t* xs = lds + lds_phys((WIN ? cl : min(cl, p.chunks)) * CB);
            if constexpr (!XF32) {
                uint32_t pr[R][16];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t wd[4] = {wb[slot][r].x, wb[slot][r].y, wb[slot][r].z, wb[slot][r].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint4 q4 = fp4_word_to_bf16_pairs(wd[i]);
                        pr[r][4 * i] = q4.x;
                        pr[r][4 * i + 1] = q4.y;
                        pr[r][4 * i + 2] = q4.z;
                        pr[r][4 * i + 3] = q4.w;
                    }
                }
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    uint32_t xp[16];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint4 q = *reinterpret_cast<const uint4*>(xs + m * p.xm_bytes + 16 * i);
                        xp[4 * i] = q.x;
                        xp[4 * i + 1] = q.y;
                        xp[4 * i + 2] = q.z;
                        xp[4 * i + 3] = q.w;
                    }
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        float d = 0.0f;
#pragma unroll
                        for (int i = 0; i < 16; ++i) d = dot2(pr[r][i], xp[i], d);
                        acc[r][m] = pinned(__builtin_fmaf(sc[r], d, acc[r][m]));
                    }
                }
            } else {
                // one word (8 values) of every row at a time; each (row, vector)
                // chain runs through the words in order
                float d[R][M];
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int m = 0; m < M; ++m) d[r][m] = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float cv[R][8];
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const uint32_t w = (i == 0) ? wb[slot][r].x : (i == 1) ? wb[slot][r].y
                                         : (i == 2) ? wb[slot][r].z : wb[slot][r].w;
                        fp4_word_to_f32(w, cv[r]);
                    }
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        const float4 xa = *reinterpret_cast<const float4*>(xs + m * p.xm_bytes + 32 * i);
                        const float4 xb = *reinterpret_cast<const float4*>(xs + m * p.xm_bytes + 32 * i + 16);
                        const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
                        for (int r = 0; r < R; ++r)
#pragma unroll
                            for (int k = 0; k < 8; ++k) d[r][m] = __builtin_fmaf(cv[r][k], xv[k], d[r][m]);
                    }
                }
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int m = 0; m < M; ++m) acc[r][m] = pinned(__builtin_fmaf(sc[r], d[r][m], acc[r][m]));
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        // the first row block's first step went out with the activation loads,
        // a later one's with the previous row block's last step (even step
        // counts)
        if (rb != (int)blockIdx.x && (p.nsteps & 1) != 0) issue(0, rb, 0);
        for (int win = 0; win < p.nwin; ++win) {
            if constexpr (WIN) {
                // every wavefront is past the previous window's reads
                if (win > 0 || rb != (int)blockIdx.x) __syncthreads();
                if (win == 0 && rb == (int)blockIdx.x)
                    stage(win, std::true_type{});
                else
                    stage(win, std::false_type{});
                __syncthreads();
            }
            // windows hold an even number of steps (all but the last), so every
            // window starts on slot 0
            const int t1 = min(p.nsteps, (win + 1) * p.win_steps);
            for (int t = win * p.win_steps; t < t1; t += 2) {
                step(std::integral_constant<int, 0>{}, t);
                if (t + 1 < t1) step(std::integral_constant<int, 1>{}, t + 1);
            }
        }

        // row totals: lane l ends with value reduce_index<P>(l)
        float v[P];
#pragma unroll
        for (int i = 0; i < P; ++i) v[i] = (i < V) ? acc[i / M][i % M] : 0.0f;
        lane_reduce<P>(v, lane);
        const int idx = reduce_index<P>(lane);
        const bool holder = (lane % (kWave / P)) == 0;
        if (holder && idx < V) {
            const int r = idx / M, m = idx - (idx / M) * M;
            if (n0 + r < p.N) {
                const size_t o = (size_t)m * p.N + n0 + r;
                if (p.y_bf16)
                    static_cast<uint16_t*>(p.y)[o] = (uint16_t)f32_to_bf16_rne(v[0]);
                else
                    static_cast<float*>(p.y)[o] = v[0];
            }
        }
    }
}

}  // namespace qmv

namespace {

using MxKernelFn = void (*)(qmv::MxParams);

template <int R, bool WIN, bool XF32, int... Ms>
constexpr MxKernelFn mx_pick(int M, std::integer_sequence<int, Ms...>)
{
    MxKernelFn f = nullptr;
    ((f = (M == Ms + 1) ? &qmv::qmv_mx_kernel<R, Ms + 1, WIN, XF32> : f), ...);
    return f;
}

// fp32 activations: two rows per wavefront and at most kMxF32Tile vectors per
// launch (their chains and accumulators stay in registers).
constexpr int kMxF32Tile = 4;

MxKernelFn mx_kernel(int R, int M, bool win, bool xf32)
{
    if (xf32) {
        const auto seq = std::make_integer_sequence<int, kMxF32Tile>{};
        if (R != 2 || M > kMxF32Tile) return nullptr;
        return win ? mx_pick<2, true, true>(M, seq) : mx_pick<2, false, true>(M, seq);
    }
    const auto seq = std::make_integer_sequence<int, QMV_TILE_M>{};
    if (win) return R == 2 ? mx_pick<2, true, false>(M, seq) : mx_pick<4, true, false>(M, seq);
    return R == 2 ? mx_pick<2, false, false>(M, seq) : mx_pick<4, false, false>(M, seq);
}

constexpr int kMxW = 8;                      // wavefronts per workgroup
constexpr int kMxLds = 160 * 1024;

bool overlap_mx(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + nb && pb < pa + na;
}

// one vector's wave step in LDS (padded): 64 chunks of 32 activations
int mx_step_bytes(bool xf32) { return qmv::kWave * 32 * (xf32 ? 4 : 2) * 17 / 16; }

int mx_steps(int K) { return (K / 32 + qmv::kWave - 1) / qmv::kWave; }

// LDS bytes of one vector's activations with the whole K: the row's chunks and
// one zero chunk after them (16 bytes of padding after every 256), at most the
// whole wave steps
int mx_whole_bytes(int K, bool xf32)
{
    const long long cb = 32LL * (xf32 ? 4 : 2);
    const long long cs = std::min<long long>(K / 32 + 1, (long long)mx_steps(K) * qmv::kWave);
    const long long o = cs * cb;
    return (int)(o + ((o >> 8) << 4));
}

// Rows per wavefront: four (activations read once per four rows) when M >= 3
// and the row blocks still cover every compute unit, else two.  A K-windowed
// launch also takes four when two would give workgroups more than one row
// block (each would restage every window per row block).
int mx_rows(int Mt, int N, int cus, bool win)
{
    const int n_rb4 = (N + kMxW * 4 - 1) / (kMxW * 4);
    const int n_rb2 = (N + kMxW * 2 - 1) / (kMxW * 2);
    return (Mt >= 3 && (n_rb4 >= cus || (win && n_rb2 > cus))) ? 4 : 2;
}

// Vectors per launch and K windows.  Activations that fit in LDS whole for
// all of a launch's vectors are staged once.  Otherwise the launch keeps up to
// QMV_TILE_M vectors and stages K in windows of an even number of wave steps
// (one pass over the weights), unless four-row blocks would still outnumber
// the compute units -- each workgroup would then restage every window for
// each of its row blocks -- and two tiles that fit whole suffice (two passes
// over the weights, no restaging).
struct MxShape {
    int per_launch;   // vectors per launch (before balancing)
    int win_steps;    // 0 = whole K
};

MxShape mx_shape(int M, int N, int K, int cus, bool xf32)
{
    const int tile = xf32 ? kMxF32Tile : QMV_TILE_M;
    const int whole = kMxLds / mx_whole_bytes(K, xf32);
    const int Mt = std::min(M, tile);
    if (whole >= Mt) return {tile, 0};
    const int n_rb4 = (N + kMxW * 4 - 1) / (kMxW * 4);
    if (whole >= 1 && n_rb4 > cus && (Mt + whole - 1) / whole <= 2) return {whole, 0};
    int ws = kMxLds / (Mt * mx_step_bytes(xf32));
    ws -= ws & 1;
    return {tile, std::max(2, ws)};
}

std::mutex g_mx_mu;
struct MxOcc {
    MxKernelFn fn;
    int dev, lds, blocks;
};
MxOcc g_mx_occ[256];
int g_mx_nocc = 0;

int mx_resident(MxKernelFn fn, int dev, int lds)
{
    std::lock_guard<std::mutex> lk(g_mx_mu);
    for (int i = 0; i < g_mx_nocc; ++i)
        if (g_mx_occ[i].fn == fn && g_mx_occ[i].dev == dev && g_mx_occ[i].lds == lds) return g_mx_occ[i].blocks;
    const void* f = reinterpret_cast<const void*>(fn);
    if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kMxLds) != hipSuccess) return -1;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, f, kMxW * qmv::kWave, lds) != hipSuccess) return -1;
    if (g_mx_nocc < 256) g_mx_occ[g_mx_nocc++] = MxOcc{fn, dev, lds, nb};
    return nb;
}

int mx_check(const uint32_t* w, const uint8_t* s, const void* x, void* y, int M, int N, int K,
             int x_dt, int y_dt)
{
    if (!w || !s || !x || !y) return QMV_E_NULL;
    if (M < 1 || M > QMV_MAX_M) return QMV_E_M_RANGE;
    if (N < 1 || N > QMV_MAX_N || K < 32 || K % 32 != 0 || K > QMV_MX_MAX_K) return QMV_E_SHAPE;
    if ((x_dt != QMV_DT_F32 && x_dt != QMV_DT_BF16) || (y_dt != QMV_DT_F32 && y_dt != QMV_DT_BF16))
        return QMV_E_DTYPE;
    const size_t yb = (y_dt == QMV_DT_F32) ? 4 : 2;
    if ((reinterpret_cast<uintptr_t>(w) % 16) || (reinterpret_cast<uintptr_t>(x) % 16) ||
        (reinterpret_cast<uintptr_t>(y) % yb))
        return QMV_E_ALIGN;
    const size_t nw = (size_t)N * (size_t)K / 2, ns = (size_t)N * (size_t)(K / 32);
    const size_t nx = (size_t)M * (size_t)K * (x_dt == QMV_DT_F32 ? 4 : 2), ny = (size_t)M * (size_t)N * yb;
    if (overlap_mx(y, ny, w, nw) || overlap_mx(y, ny, s, ns) || overlap_mx(y, ny, x, nx))
        return QMV_E_ALIAS;
    // the kernel's row offsets are 32-bit
    if (nw >= (size_t)1 << 31) return QMV_E_SHAPE;
    return QMV_OK;
}

}  // namespace

extern "C" int qmv_mxfp4(const uint32_t* w_packed, const uint8_t* scales, const void* x, void* y,
                         int M, int N, int K, qmv_dtype x_dt, qmv_dtype y_dt, void* stream)
{
    const int st = mx_check(w_packed, scales, x, y, M, N, K, (int)x_dt, (int)y_dt);
    if (st != QMV_OK) return st;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QMV_E_LAUNCH;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return QMV_E_LAUNCH;
    const size_t yb = (y_dt == QMV_DT_F32) ? 4 : 2;
    const bool xf32 = x_dt == QMV_DT_F32;
    const size_t xb = xf32 ? 4 : 2;
    const int step_bytes = mx_step_bytes(xf32);
    const MxShape shape = mx_shape(M, N, K, cus, xf32);
    const int tiles = (M + shape.per_launch - 1) / shape.per_launch;
    // Balanced tiles: the first M % tiles get one more vector, so there are at
    // most two tile sizes.  Both launches are planned (instance, LDS,
    // residency) before the first one is enqueued, so a refused plan leaves y
    // untouched.
    struct MxLaunch {
        qmv::MxParams p;
        MxKernelFn fn;
        int lds, grid;
    };
    MxLaunch plans[2];
    const int sizes[2] = {M / tiles + (M % tiles ? 1 : 0), M / tiles};
    for (int i = 0; i < 2; ++i) {
        const int Mt = sizes[i];
        if (Mt < 1) continue;
        const bool win = shape.win_steps > 0 && Mt * mx_whole_bytes(K, xf32) > kMxLds;
        const int R = xf32 ? 2 : mx_rows(Mt, N, cus, win);
        qmv::MxParams& p = plans[i].p;
        p.w = w_packed;
        p.s = scales;
        p.N = N;
        p.K = K;
        p.chunks = K / 32;
        p.nsteps = mx_steps(K);
        p.row_bytes = K / 2;
        p.n_rb = (N + kMxW * R - 1) / (kMxW * R);
        p.y_bf16 = (y_dt == QMV_DT_BF16) ? 1 : 0;
        p.win_steps = win ? shape.win_steps : p.nsteps;
        p.nwin = (p.nsteps + p.win_steps - 1) / p.win_steps;
        p.xm_bytes = win ? p.win_steps * step_bytes : mx_whole_bytes(K, xf32);
        {
            // exact division by d = pieces per vector and window for every
            // index below 2^21 (at most 13 * 2^14 here): with k >= 21 +
            // ceil(log2 d) and magic = ceil(2^k / d), i * d < 2^k makes
            // floor(i * magic / 2^k) = floor(i / d); k >= 32 keeps it one
            // high-half multiply, and magic < 2^32
            const uint32_t cslot = win ? (uint32_t)p.win_steps * qmv::kWave
                                       : (uint32_t)std::min(p.chunks + 1, p.nsteps * qmv::kWave);
            const uint32_t d = cslot * (xf32 ? 8u : 4u);
            int lg = 0;
            while ((1u << lg) < d) ++lg;
            const int k = std::max(32, 21 + lg);
            p.ipm_shift = k - 32;
            p.ipm_magic = (uint32_t)(((1ULL << k) + d - 1) / d);
        }
        const int lds = Mt * p.xm_bytes;
        if (lds > kMxLds) return QMV_E_SHAPE;
        const MxKernelFn fn = mx_kernel(R, Mt, win, xf32);
        if (!fn) return QMV_E_LAUNCH;
        const int nb = mx_resident(fn, dev, lds);
        if (nb <= 0) return QMV_E_LAUNCH;
        // row blocks per workgroup: as the affine launch -- every workgroup the
        // same count, and two for memory-bound calls while that still leaves a
        // workgroup for every compute unit
        int per = (p.n_rb + nb * cus - 1) / (nb * cus);
        if (Mt <= 2 && per == 1 && p.n_rb >= 2 * cus) per = 2;
        plans[i].fn = fn;
        plans[i].lds = lds;
        plans[i].grid = (p.n_rb + per - 1) / per;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    int m0 = 0;
    for (int t = 0; t < tiles; ++t) {
        const int i = (t < M % tiles || M % tiles == 0) ? 0 : 1;
        const int Mt = sizes[i];
        MxLaunch& L = plans[i];
        L.p.x = static_cast<const uint8_t*>(x) + (size_t)m0 * K * xb;
        L.p.y = static_cast<uint8_t*>(y) + (size_t)m0 * N * yb;
        void* args[] = {&L.p};
        if (hipLaunchKernel(reinterpret_cast<const void*>(L.fn), dim3(L.grid), dim3(kMxW * qmv::kWave), args,
                            (size_t)L.lds, s) != hipSuccess)
            return QMV_E_LAUNCH;
        m0 += Mt;
    }
    return QMV_OK;
}
