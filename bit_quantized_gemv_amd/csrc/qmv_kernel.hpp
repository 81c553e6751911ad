// qmv_kernel.hpp -- gfx950 kernels of the affine group-quantized
// matrix-vector product streamed over M <= 13 activation vectors.
//
//   y[m][n] = sum_g ( scale[n][g] * sum_{k in g} q[n][k] x[m][k]
//                   + bias[n][g]  * sum_{k in g} x[m][k] )
//
// (mlxcel issue "an order-preserving streamed qmv would give MTP the fast
// kernel and byte-identity together", sections "Correction to the obvious
// sketch" and "Step 2"; mlxcel PR "block output rows per warp in qmv below
// Ampere", sections "What lands" and "Not covered").
//
// Work decomposition
//   * A row of packed weights is a sequence of 16-byte chunks.  Chunk c is read
//     by lane c % 64 in wave step c / 64, so one wave-wide 128-bit load covers
//     1 KiB of a row contiguously.
//   * A wavefront owns R consecutive rows (row blocking): in a step it loads the
//     chunk of each of its rows and reads the activations of that chunk from
//     LDS once for all R rows.  A (row block, step) pair is a unit.  Each
//     wavefront keeps the weights (and, where loaded per unit, the scales and
//     biases) of the next PF units in flight in a register ring; the loads of a unit are issued before the
//     compute of the unit PF places earlier, and a scheduling barrier keeps
//     the compiler from sinking them below it.
//   * A workgroup of W wavefronts stages the activations x[0..M)[K-window] in
//     LDS, together with each chunk's dot-chain start and group sum, and walks
//     row blocks of W*R rows (one per workgroup when the grid fits on the chip
//     in one round).
//     All activation loads are issued before the first weight load, and the
//     weight prologue is in flight while the activations are converted.
//   * Each lane uses the scale and bias of its own group, of the rows whose
//     group it owns (step 4 below) when the rows per wavefront are a multiple
//     of lpg, else of every row (zeroing them in registers where it does not
//     own the group).  Whole-K instances with a multiple of lpg rows per
//     wavefront fetch the scale and bias rows of all the wavefront's row
//     blocks once (two wave-wide 128-bit loads) into LDS and read them there;
//     the others load each unit's values with its weights.  Rows past N and
//     chunks past a row's end read clamped, in-bounds addresses; the
//     activations, chain starts and group sums of chunks past the row's end
//     are zero in LDS, so those lanes add nothing.
//   * Activation staging issues the loads of a batch of rounds together; long
//     windows and many vectors take several batches.
//   * The weight decode of a chunk happens once per step, outside the loop over
//     the M vectors; every vector then reuses the decoded registers.
//   * A measurement instance of the same kernel (one more argument) records,
//     per wavefront, the real-time counter at its start, after staging and at
//     its end, and where it ran; the product instances compile to the same
//     code as without it.
//
// Per-row arithmetic (fixed by K, bits, group size and activation dtype; it
// never depends on M, R, W, PF, the grid or the K-window size):
//   1. bf16 activations: the chunk's codes become exact bf16 pairs
//      (2^bits + q_a, 2^bits + q_b) -- the code sits in the top mantissa bits
//      of a number in [2^bits, 2^(bits+1)) -- and D_c is the chain of
//      v_dot2_f32_bf16 over the chunk's pairs in word order then pair order,
//      starting from -2^bits * S_c (S_c: the chunk's activation sum), so it
//      ends at the chunk's raw integer dot sum_k q_k x_k.  Pair j of a word
//      holds fields (j, j + 32/(2 bits)); the matching activation pairs are
//      laid out that way in LDS.
//      fp32 activations: D_c is the fma chain over the chunk's values in
//      ascending k, from 0, with exact fp32 codes.
//   2. The lpg = gs*bits/128 chunks of a group sit in adjacent lanes; their
//      partials are combined by a DPP butterfly (xor 1, then xor 2).
//   3. S[m][g] is the fp32 sum of the group's activations.  bf16 activations:
//      each 8-value block (16 at 2 bits) is a v_dot2_f32_bf16 chain of its
//      natural pairs (x_2i, x_2i+1) against (1, 1) from 0 (at 2 bits two
//      8-value chains, then added); fp32 activations: 8-value blocks summed
//      left to right.  Blocks are combined pairwise (xor-1, xor-2, ... tree);
//      the level that completes a chunk gives S_c of step 1.
//   4. Each group is folded once, by its owner lane -- for row n, the lane l
//      of the group with l % lpg == n % lpg -- as
//      acc = fma(scale, D, fma(bias, S, acc)), over its groups in ascending
//      step: the scale multiplies the group's raw integer dot D, the bias its
//      activation sum S.  With lpg = 2 or 4, a multiple of lpg rows per
//      wavefront and more than one vector, the lpg lanes of a group run the
//      chains of all rows of a row group, in an order rotated by the lane's
//      place in the group, so the DPP adds of step 2 (same addends, same
//      grouping) leave each lane the group dot of its own row and each lane
//      folds only its own rows.  Otherwise
//      every lane executes the fold of every row, with scale and bias zeroed
//      on lanes that do not own the group, which leaves their accumulators at
//      +0.
//   5. Row total: lanes l and l ^ d combined for d = 32, 16, 8, 4, 2, 1 in that
//      order (lanes that own none of the row's groups contribute +0); then
//      round-to-nearest-even to y's dtype.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include <type_traits>

namespace qmv {

constexpr int kWave = 64;
constexpr int kLdsBytes = 163840;

struct Params {
    const uint32_t* w;
    const uint16_t* s;
    const uint16_t* b;
    const void* x;
    void* y;
    int N;
    int K;
    int G;               // groups per row
    int chunks;          // 16-byte weight chunks per row
    int nsteps;          // wave steps per row, ceil(chunks / 64)
    int row_bytes;       // chunks * 16
    int win_steps;       // wave steps per K window
    int nwin;            // K windows
    int n_rb;            // row blocks of W*R rows
    int y_bf16;          // y: 1 = bf16, 0 = fp32
    int x_m_bytes;       // LDS bytes of one vector's activation window (padded); with one
                         // window, only the row's chunks and one zero chunk after them
    int s_off;           // LDS offset of SC[M][win_steps * 64]: per chunk a float2 (dot-chain
                         // start -2^bits * chunk sum for bf16 activations, 0 for fp32;
                         // sum of the chunk's group)
    int m_slot;          // whole-K instances: bytes of a row block's scale (bias) copy,
                         // 16 * ceil((14 + 2 * R * G) / 16); at most kMetaBytes per wavefront
                         // for all its row blocks
    int sb_last;         // offset of the last 16-byte piece of the scale (bias) tensor
    int m_div;           // ceil(8192 / (m_slot / 16)): lane / (m_slot / 16) is (lane * m_div) >> 13
    int rpm_full;        // staging rounds per vector of a full K window (of the whole K if one)
    int rpm_last;        // ... of the last K window
    int rb_per;          // row blocks of the workgroups that walk the most: ceil(n_rb / grid)
    int rb_full;         // workgroups below this index walk rb_per blocks, the others rb_per - 1
};

// Whole-K instances: LDS bytes per wavefront for its copy of the scales (and
// as many for the biases) of all its row blocks -- one 16-byte piece per lane
// of one wave-wide load.
constexpr int kMetaBytes = 1024;

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h)
{
    return __half2float(__ushort_as_half(static_cast<unsigned short>(h)));
}

// IEEE round-to-nearest-even binary32 -> bfloat16 (NaN stays quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// LDS activation layout: 16 bytes of padding after every 256 bytes, so that
// 16 lanes reading 16-byte pieces at a 64/128/256-byte lane stride hit 64
// distinct banks.
__device__ __forceinline__ int lds_phys(int o) { return o + ((o >> 8) << 4); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Sum over the lanes of a group of n (1, 2, 4, 8 or 16) adjacent lanes; every
// lane of the group ends with the same bits (each step adds two values that
// the partner lane adds in the other order).
template <int NL>
__device__ __forceinline__ float lane_group_sum(float v)
{
    if constexpr (NL >= 2) v = v + dpp<kQuadXor1>(v);
    if constexpr (NL >= 4) v = v + dpp<kQuadXor2>(v);
    if constexpr (NL >= 8) v = v + dpp<kRowHalfMirror>(v);
    if constexpr (NL >= 16) v = v + dpp<kRowMirror>(v);
    return v;
}

// The levels of lane_group_sum<TO> past those of lane_group_sum<FROM>: applied to
// lane_group_sum<FROM>(v) it gives lane_group_sum<TO>(v) bit for bit.
template <int FROM, int TO>
__device__ __forceinline__ float lane_group_sum_from(float v)
{
    if constexpr (TO >= 2 && FROM < 2) v = v + dpp<kQuadXor1>(v);
    if constexpr (TO >= 4 && FROM < 4) v = v + dpp<kQuadXor2>(v);
    if constexpr (TO >= 8 && FROM < 8) v = v + dpp<kRowHalfMirror>(v);
    if constexpr (TO >= 16 && FROM < 16) v = v + dpp<kRowMirror>(v);
    return v;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

// (a & mask) | magic.  gfx9 VOP3 instructions take no literal constants and
// read at most one scalar operand; with the magic held in a VGPR (see
// opaque_u32) and the mask in an SGPR this is one v_and_or_b32.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t magic)
{
    return (a & mask) | magic;
}

// v unchanged, as a value the compiler cannot fold into a constant (so a
// constant used by a VOP3 instruction stays in a register).
__device__ __forceinline__ uint32_t opaque_u32(uint32_t v)
{
    asm volatile("" : "+v"(v));
    return v;
}

template <int BITS>
constexpr uint32_t code_magic() { return BITS == 4 ? 0x41804180u : 0x40804080u; }

// Exact bf16 pair (2^BITS + field j, 2^BITS + field j + 32/(2 BITS)) of a word.
// 4-bit: 16 + q = 0x4180 | q << 3 (code in mantissa bits 3..6).
// 2-bit:  4 + q = 0x4080 | q << 5 (code in mantissa bits 5..6).
// `magic` is code_magic<BITS>() held in a VGPR.
template <int BITS>
__device__ __forceinline__ uint32_t code_pair(uint32_t w, int j, uint32_t magic)
{
    if constexpr (BITS == 4) {
        const uint32_t t = (j == 0) ? (w << 3) : (w >> (4 * j - 3));
        return and_or(t, 0x00780078u, magic);
    } else {
        const int sh = 5 - 2 * j;
        const uint32_t t = (sh >= 0) ? (w << sh) : (w >> (-sh));
        return and_or(t, 0x00600060u, magic);
    }
}

// Buffer resources and loads.  Every lane of every load the kernels issue
// addresses memory inside its tensor (rows past N, lanes past a row's last
// chunk and groups past a row's last group are clamped to the last valid
// one), so a resource either spans all of memory (record count 0xffffffff) or
// nothing (record count 0: a prefetch slot past the last unit, which reads
// zero without touching memory).  Loads whose lanes fall outside the record
// count are avoided elsewhere: on gfx950 they are not free.
constexpr int kRsrcWord3 = 0x00020000;   // gfx9-family raw buffer

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int records)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, records, kRsrcWord3);
}

// 128-bit load with the non-temporal hint (weights are streamed once).
// `soff` rides in an SGPR and is added after the lane offset.
__device__ __forceinline__ uint4 buf_load_nt(__amdgpu_buffer_rsrc_t r, int off, int soff)
{
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 2);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint4 buf_load(__amdgpu_buffer_rsrc_t r, int off)
{
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ unsigned short buf_load_u16(__amdgpu_buffer_rsrc_t r, int off, int soff)
{
    return (unsigned short)__builtin_amdgcn_raw_buffer_load_b16(r, off, soff, 0);
}

// fp32 value of a bf16 / fp16 held in the low half of a register.  Written as
// volatile asm so the conversion stays where the value is consumed: left to
// the compiler it is scheduled right after the loop's previous step, which
// makes the wavefront wait there for every load still in flight.
__device__ __forceinline__ float bf16_to_f32_here(unsigned short h)
{
    float f;
    asm volatile("v_lshlrev_b32 %0, 16, %1" : "=v"(f) : "v"(h));
    return f;
}
__device__ __forceinline__ float f16_to_f32_here(unsigned short h)
{
    float f;
    asm volatile("v_cvt_f32_f16 %0, %1" : "=v"(f) : "v"(h));
    return f;
}

// v as a scalar register.  A value derived from scalars only is uniform, but
// after divergent control flow the compiler may keep it in a vector register
// (dropping a readfirstlane as redundant), and a buffer resource built from a
// vector register costs a waterfall loop around every load that uses it.  The
// "s" constraints make it materialize the value in an SGPR.
__device__ __forceinline__ int in_sgpr(int v)
{
    int r;
    asm("s_mov_b32 %0, %1" : "=s"(r) : "s"(v));
    return r;
}

// Hides how an offset was computed, so the compiler keeps one unconditional
// load instead of re-splitting a masked offset into guarded branches.
__device__ __forceinline__ int opaque(int v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// Returns v unchanged from an empty volatile asm: the computation of v stays
// where it is written (it cannot be sunk into later blocks, which would keep
// its inputs live).
__device__ __forceinline__ float pinned(float v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// Returns v unchanged, as a value that exists only once `dep` has been
// computed: a memory access addressed by it cannot be moved (by IR passes or
// the scheduler) above the computation of `dep`.
__device__ __forceinline__ int after(int v, float dep)
{
    asm volatile("" : "+v"(v) : "v"(dep));
    return v;
}

// ------------------------------------------------------ activation staging
// Stages x[0..M)[window] into LDS (bf16 pairs in code-pair order, or fp32 in
// natural order), writes each chunk's (dot-chain start, group sum) pair, and
// zeroes the activations and pairs of the window's chunks past the row's end.
// Work is cut into units of UV consecutive values of one vector; a round is
// one unit per thread of one vector's window.  The loads of up to XB rounds
// are issued together before any of them is consumed.
constexpr uint32_t kOnePair = 0x3f803f80u;   // bf16 pair (1.0, 1.0)

template <int BITS, int GS, int M, bool XF32>
struct Stager {
    static constexpr int VPC = 128 / BITS;                    // values per weight chunk
    static constexpr int LPG = GS * BITS / 128;               // chunks per group
    static constexpr int XCB = VPC * (XF32 ? 4 : 2);          // LDS bytes per chunk
    static constexpr int UV = (!XF32 && BITS == 2) ? 16 : 8;  // values per unit
    static constexpr int UPG = GS / UV;                       // units per group
    static constexpr int UPC = VPC / UV;                      // units per chunk
    static constexpr int NLD = (XF32 || BITS == 2) ? 2 : 1;   // 16-byte loads per unit
    // Rounds in flight per batch: 4 at one or two vectors, 8 to six, 16 beyond
    // (halved where a unit is two loads); from nine vectors with bf16
    // activations exactly M, so a window whose vectors take one round each is
    // one batch with no clamped re-reads, and one whose vectors take two is two
    // equal batches (measured 0.3-7% faster at M = 9-13 on the four 4-bit
    // projection shapes and 2-4% on the 2-bit one; at M = 7 and 8 mixed, -2%
    // to +2%, and at M = 3 slower).
    static constexpr int XB = (M >= 9 && (NLD == 1 || (!XF32 && BITS == 2))) ? M : ((M <= 2) ? 4 : (M <= 6 ? 8 : 16)) / NLD;

    int nthr;     // threads in the workgroup
    int upm;      // units per vector in this window
    int rpm;      // rounds per vector
    int rounds;   // M * rpm
    int k_lo;     // first value of the window
    int c_n;      // chunks in this window

    __device__ void begin(const Params& p, int win)
    {
        const int c_lo = win * p.win_steps * kWave;
        c_n = min(p.chunks - c_lo, p.win_steps * kWave);
        upm = c_n * VPC / UV;
        rpm = (win == p.nwin - 1) ? p.rpm_last : p.rpm_full;   // ceil(upm / threads)
        rounds = M * rpm;
        k_lo = c_lo * VPC;
    }

    // Loads of the round (vector m, j-th round of that vector).  Threads past
    // the window, and rounds past the last (m >= M), re-read an in-bounds
    // unit; their data is not stored.
    __device__ void load(const Params& p, __amdgpu_buffer_rsrc_t xr, int m, int j, uint4 (&d)[NLD]) const
    {
        const int l = j * nthr + (int)threadIdx.x;
        const int lc = min(l, upm - 1);
        const int mc = min(m, M - 1);
        const int off = (mc * p.K + k_lo + lc * UV) * (XF32 ? 4 : 2);
#pragma unroll
        for (int k = 0; k < NLD; ++k) d[k] = buf_load(xr, off + 16 * k);
    }

    __device__ void store(const Params& p, uint8_t* lds, int m, int j, const uint4 (&d)[NLD]) const
    {
        const int l = j * nthr + (int)threadIdx.x;
        const bool valid = l < upm;
        float2* SC = reinterpret_cast<float2*>(lds + p.s_off);
        uint8_t* dst = lds + m * p.x_m_bytes;
        float part;
        if constexpr (XF32) {
            const float v[8] = {__uint_as_float(d[0].x), __uint_as_float(d[0].y),
                                __uint_as_float(d[0].z), __uint_as_float(d[0].w),
                                __uint_as_float(d[1].x), __uint_as_float(d[1].y),
                                __uint_as_float(d[1].z), __uint_as_float(d[1].w)};
            part = v[0];
#pragma unroll
            for (int k = 1; k < 8; ++k) part = part + v[k];
            if (valid) {
                *reinterpret_cast<uint4*>(dst + lds_phys(l * 32)) = d[0];
                *reinterpret_cast<uint4*>(dst + lds_phys(l * 32 + 16)) = d[1];
            }
        } else if constexpr (BITS == 4) {
            // sum: a v_dot2_f32_bf16 chain of the unit's four natural pairs
            // (x_2i, x_2i+1) against (1, 1), from 0
            const uint4 q0 = d[0];
            part = dot2(q0.x, kOnePair, 0.0f);
            part = dot2(q0.y, kOnePair, part);
            part = dot2(q0.z, kOnePair, part);
            part = dot2(q0.w, kOnePair, part);
            if (valid) {
                // pairs (x_j, x_{j+4}), j = 0..3
                uint4 q;
                q.x = __builtin_amdgcn_perm(q0.z, q0.x, 0x05040100u);
                q.y = __builtin_amdgcn_perm(q0.z, q0.x, 0x07060302u);
                q.z = __builtin_amdgcn_perm(q0.w, q0.y, 0x05040100u);
                q.w = __builtin_amdgcn_perm(q0.w, q0.y, 0x07060302u);
                *reinterpret_cast<uint4*>(dst + lds_phys(l * 16)) = q;
            }
        } else {
            // sum: v_dot2_f32_bf16 chains of each half's four natural pairs against
            // (1, 1), from 0; then the two halves added
            const uint32_t dw[8] = {d[0].x, d[0].y, d[0].z, d[0].w, d[1].x, d[1].y, d[1].z, d[1].w};
            float pa = dot2(dw[0], kOnePair, 0.0f);
            float pb = dot2(dw[4], kOnePair, 0.0f);
#pragma unroll
            for (int k = 1; k < 4; ++k) {
                pa = dot2(dw[k], kOnePair, pa);
                pb = dot2(dw[4 + k], kOnePair, pb);
            }
            part = pa + pb;
            if (valid) {
                // pairs (x_j, x_{j+8}), j = 0..7
                uint32_t pr[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    pr[j] = __builtin_amdgcn_perm(dw[4 + (j >> 1)], dw[j >> 1], (j & 1) ? 0x07060302u : 0x05040100u);
                *reinterpret_cast<uint4*>(dst + lds_phys(l * 32)) = make_uint4(pr[0], pr[1], pr[2], pr[3]);
                *reinterpret_cast<uint4*>(dst + lds_phys(l * 32 + 16)) = make_uint4(pr[4], pr[5], pr[6], pr[7]);
            }
        }
        // group sum: the UPG units of a group sit in UPG adjacent lanes (a
        // round starts at a multiple of the wavefront size and a window holds
        // whole groups, so the lanes past the window form whole groups too)
        // chunk sums (the UPC units of a chunk sit in adjacent lanes), then group
        // sums (the LPG chunks of a group sit in adjacent lanes, and a window
        // holds whole groups); each chunk's lane pair stores (start, group sum)
        float c0 = 0.0f;
        part = lane_group_sum<UPC>(part);
        if constexpr (!XF32) c0 = -(float)(1 << BITS) * part;
        part = lane_group_sum_from<UPC, UPG>(part);
        if (valid && (l % UPC) == 0) SC[m * p.win_steps * kWave + l / UPC] = make_float2(c0, part);
    }

    // zero the activations past the window's chunks -- with one window only the
    // chunk after them, which the lanes past the row's end read; with several,
    // the rest of the last window's slot -- and the chain starts and group
    // sums of the window's chunks past the row's end (only the last window of
    // a row has them)
    __device__ void zero_tail(const Params& p, uint8_t* lds) const
    {
        const int cw = p.win_steps * kWave;
        const int pieces = (p.nwin > 1) ? (cw - c_n) * XCB / 16 : (c_n < cw) ? XCB / 16 : 0;
        float2* SC = reinterpret_cast<float2*>(lds + p.s_off);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            for (int j = (int)threadIdx.x; j < pieces; j += nthr)
                *reinterpret_cast<uint4*>(lds + m * p.x_m_bytes + lds_phys(c_n * XCB + 16 * j)) =
                    make_uint4(0, 0, 0, 0);
            for (int j = (int)threadIdx.x; j < cw - c_n; j += nthr)
                SC[m * cw + c_n + j] = make_float2(0.0f, 0.0f);
        }
    }

    // Stage a window.  The loads of the first XB rounds are issued together,
    // unconditionally (so the compiler counts the loads in flight exactly);
    // `between` runs next (the caller issues its weight prologue there, so the
    // activation requests are ahead of the weight stream); then those rounds
    // are converted and stored.  Rounds past XB (long windows, many vectors)
    // follow in batches of XB, each batch's loads issued together.
    template <class F>
    __device__ void stage(const Params& p, __amdgpu_buffer_rsrc_t xr, uint8_t* lds, int win, F&& between)
    {
        begin(p, win);
        {
            uint4 d[XB][NLD];
            int m = 0, j = 0;
#pragma unroll
            for (int i = 0; i < XB; ++i) {
                load(p, xr, m, j, d[i]);
                if (++j == rpm) {
                    j = 0;
                    ++m;
                }
            }
            // (more vectors: nothing of `between` moves above the loads)
            if constexpr (M != 1) __builtin_amdgcn_sched_barrier(0);
            between();
            m = 0;
            j = 0;
#pragma unroll
            for (int i = 0; i < XB; ++i) {
                if (i < rounds) store(p, lds, m, j, d[i]);
                if (++j == rpm) {
                    j = 0;
                    ++m;
                }
            }
        }
        for (int base = XB; base < rounds; base += XB) {
            uint4 d[XB][NLD];
            int m = base / rpm, j = base - (base / rpm) * rpm;
#pragma unroll
            for (int i = 0; i < XB; ++i) {
                load(p, xr, m, j, d[i]);
                if (++j == rpm) {
                    j = 0;
                    ++m;
                }
            }
            m = base / rpm;
            j = base - (base / rpm) * rpm;
#pragma unroll
            for (int i = 0; i < XB; ++i) {
                if (base + i < rounds) store(p, lds, m, j, d[i]);
                if (++j == rpm) {
                    j = 0;
                    ++m;
                }
            }
        }
        zero_tail(p, lds);
    }
};

// --------------------------------------------------------- row reductions
// Cross-lane exchange partner l ^ D for D in {1, 2, 4, 8}, within 16-lane rows.
template <int D>
__device__ __forceinline__ float xor_lanes(float v)
{
    const int i = __float_as_int(v);
    if constexpr (D == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, i, kQuadXor1, 0xF, 0xF, false));
    if constexpr (D == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, i, kQuadXor2, 0xF, 0xF, false));
    // banks are the 4-lane quarters of a row; row_shl:n reads lane l + n, row_shr:n lane l - n
    if constexpr (D == 4) {
        int t = __builtin_amdgcn_update_dpp(0, i, 0x104, 0xF, 0x5, false);
        return __int_as_float(__builtin_amdgcn_update_dpp(t, i, 0x114, 0xF, 0xA, false));
    }
    int t = __builtin_amdgcn_update_dpp(0, i, 0x108, 0xF, 0x3, false);
    return __int_as_float(__builtin_amdgcn_update_dpp(t, i, 0x118, 0xF, 0xC, false));
}

constexpr int pow2_at_least(int v) { return v <= 1 ? 1 : 2 * pow2_at_least((v + 1) / 2); }

// Row totals of V per-lane partials (rows x vectors), all at once.  Every value is summed
// over the 64 lanes by the same tree -- pairs of lanes l, l ^ d combined for
// d = 32, 16, 8, 4, 2, 1 in that order -- so a value's bits do not depend on
// how many other values share the reduction.  While several values remain per
// lane, each level exchanges halves (permlane32/16 swaps, then DPP) so lane l
// keeps a different value than lane l ^ d; once one value remains, the level
// is a butterfly.  On return, v[0] of lane l holds the total of value
// reduce_index<P>(l); lanes l with l % (64/P) == 0 hold distinct values.
// SKIP > 0 (row-grouped folds): the lanes of each aligned group of 2^SKIP
// lanes hold partials of different rows; the levels d = 32 .. 2^SKIP run as
// above, and the levels below are the adds of the +0 that lanes owning none
// of a row's groups contribute to it (one add of +0 gives the same bits).
template <int P, int SKIP = 0>
__device__ __forceinline__ void lane_reduce(float (&v)[P], int lane)
{
    static_assert(P >= 1 && P <= 64 && (P & (P - 1)) == 0, "P must be a power of two <= 64");
    static_assert(P <= (64 >> SKIP), "too many values for the lanes left");
    // d = 32
    if constexpr (P >= 2) {
#pragma unroll
        for (int i = 0; i < P / 2; ++i) {
            auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i + P / 2]), false, false);
            v[i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        }
    } else {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0]), __float_as_uint(v[0]), false, false);
        v[0] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    // d = 16
    if constexpr (P >= 4) {
#pragma unroll
        for (int i = 0; i < P / 4; ++i) {
            auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + P / 4]), false, false);
            v[i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        }
    } else {
        auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[0]), __float_as_uint(v[0]), false, false);
        v[0] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    // d = 8, 4, 2, 1
    auto level = [&](auto dtag, auto ntag) {
        constexpr int D = decltype(dtag)::value;
        constexpr int NV = decltype(ntag)::value;   // values per lane before this level
        if constexpr (NV >= 2) {
            const bool hi = (lane & D) != 0;
#pragma unroll
            for (int i = 0; i < NV / 2; ++i) {
                const float send = hi ? v[i] : v[i + NV / 2];
                const float keep = hi ? v[i + NV / 2] : v[i];
                v[i] = keep + xor_lanes<D>(send);
            }
        } else {
            v[0] = v[0] + xor_lanes<D>(v[0]);
        }
    };
    level(std::integral_constant<int, 8>{}, std::integral_constant<int, (P >= 8 ? P / 4 : 1)>{});
    level(std::integral_constant<int, 4>{}, std::integral_constant<int, (P >= 16 ? P / 8 : 1)>{});
    if constexpr (SKIP < 2)
        level(std::integral_constant<int, 2>{}, std::integral_constant<int, (P >= 32 ? P / 16 : 1)>{});
    if constexpr (SKIP < 1)
        level(std::integral_constant<int, 1>{}, std::integral_constant<int, (P >= 64 ? P / 32 : 1)>{});
    // skipped levels: the value plus +0, i.e. unchanged except that -0 becomes +0
    if constexpr (SKIP > 0) v[0] = v[0] + 0.0f;
}

// Which value lane l holds after lane_reduce<P, SKIP>.
template <int P, int SKIP = 0>
__device__ __forceinline__ int reduce_index(int lane)
{
    int idx = 0, n = P;
#pragma unroll
    for (int d = 32; d >= (1 << SKIP); d >>= 1) {
        if (n >= 2) {
            if (lane & d) idx += n / 2;
            n /= 2;
        }
    }
    return idx;
}

// ------------------------------------------------------------------- kernel
// Largest workgroup (in wavefronts) an instance is compiled for.
constexpr int kMaxWaves = 8;

// Resident wavefronts per SIMD an instance asks the register allocator for:
// eight (at most 64 VGPRs) for the memory-bound 4-bit, bf16-activation,
// one-vector instances with at most two rows, one unit in flight and no K
// windows, so a grid of one workgroup per row block is resident in one round;
// else no constraint.
constexpr int waves_hint(int BITS, bool XF32, int R, int M, int PF, bool WIN)
{
    return (BITS == 4 && !XF32 && M == 1 && R <= 2 && PF == 1 && !WIN) ? 8 : 1;
}

// Per-wavefront record of the stamped (measurement) instances: the constant-
// rate counter at the wavefront's start, once the activations are staged
// (after the workgroup barrier) and at its end, and the hardware ids of where
// it ran (XCC id in the high word, HW_ID in the low word).  Nothing is stamped
// inside the unit loop: a stamp there changes the loop's code and register
// use.
constexpr int kStamps = 4;

// Reads the constant-rate real-time counter and waits for it in the same asm
// block, so no later wait on LDS reads waits on it.
__device__ __forceinline__ uint64_t stamp_now()
{
    uint64_t t;
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t));
    __builtin_amdgcn_sched_barrier(0);
    return t;
}

// WIN: the instance restages the activations per K window (when x[0..M)[0..K)
// does not fit in LDS) and loads each unit's scales and biases with its
// weights; it also serves one window where the scale/bias copies of the
// instances without it do not fit.  Instances without it require p.nwin == 1
// and p.m_slot > 0.
// Stamps: the product instances take no further argument (Stamps empty).  The
// measurement instance takes one, a uint64_t* to which lane 0 of each
// wavefront writes its kStamps values at stamps[(workgroup * W + wave) *
// kStamps ...] after its last unit; its code is the product's with three
// counter reads, two hardware-register reads and that store added (the
// scheduling barriers around the counter reads keep some of the product's
// setup instructions on their side).  The stamps stay inside this one
// definition: a kernel body moved into a device function compiles to
// different code.
template <int BITS, int GS, int R, int M, int PF, bool XF32, bool SBF, bool WIN, class... Stamps>
__global__ __launch_bounds__(kMaxWaves * kWave) __attribute__((amdgpu_waves_per_eu(waves_hint(BITS, XF32, R, M, PF, WIN))))
void qmv_affine_kernel(const Params p, Stamps... stamp_ptr)
{
    constexpr bool STAMP = sizeof...(Stamps) > 0;
    static_assert(sizeof...(Stamps) == 0 || (sizeof...(Stamps) == 1 && (std::is_same_v<Stamps, uint64_t*> && ...)),
                  "the only extra argument is the stamps pointer");
    uint64_t ts_start = 0, ts_staged = 0;
    if constexpr (STAMP) ts_start = stamp_now();
    constexpr int LPG = GS * BITS / 128;          // lanes (chunks) per group
    constexpr int VPC = 128 / BITS;               // values per chunk
    constexpr int XCB = VPC * (XF32 ? 4 : 2);     // activation bytes per chunk in LDS
    constexpr int XSTEP = kWave * XCB + kWave * XCB / 16;  // padded LDS bytes per wave step
    constexpr int NS = PF + 1;                    // ring slots
    // Grouped folds: with lpg = 2 or 4 lanes per group and a
    // multiple of lpg rows per wavefront, lane l of a group folds the rows
    // lpg*k + l % lpg -- so each lane loads the metadata of R/lpg rows, and
    // one combine and one fold serve lpg rows.  (Every instance uses this
    // ownership; other instances zero the scale and bias of the rows a lane
    // does not own, which gives the same bits.  One vector keeps that form:
    // its short compute after the last load is latency-bound, and grouping
    // adds the per-word lane selects to it.)
    constexpr bool GROUPED = !XF32 && (R % LPG == 0) && ((LPG == 2 && M >= 2) || (LPG == 4 && M >= 9));
    constexpr int RS = GROUPED ? R / LPG : R;      // rows each lane folds (accumulator sets)
    // Rows whose scale and bias a lane loads: with a multiple of lpg rows per
    // wavefront a lane owns the groups of one row in lpg, in either form, so
    // it loads only those rows' values (the rows lpg*k + l % lpg).
    constexpr bool OWNLOAD = (LPG == 2 || LPG == 4) && (R % LPG == 0);
    constexpr int RL = OWNLOAD ? R / LPG : R;
    // Whole-K instances whose lanes each fold their own rows (OWNLOAD) read
    // each group's scale and bias from LDS: with the weight prologue every
    // wavefront loads the scale and bias rows of all its row blocks (two
    // wave-wide loads), and its first unit stores them in a static LDS array,
    // so the unit loop issues weight loads only.  The other instances --
    // and the K-windowed one, also used for whole K where the copies would
    // not fit -- load the values of each unit with its weights.
    constexpr bool MLDS = !WIN && OWNLOAD;
    constexpr int SKIP = GROUPED ? (LPG == 4 ? 2 : 1) : 0;   // reduction levels inside a group
    constexpr int V = RS * M;
    constexpr int P = pow2_at_least(V);
    static_assert(P <= (64 >> SKIP), "too many row totals per lane");

    extern __shared__ __align__(16) uint8_t lds[];
    const int lane = threadIdx.x & (kWave - 1);
    // wave-uniform by construction; readfirstlane lets the compiler keep it
    // (and everything derived from it) in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int W = blockDim.x / kWave;
    const int grid = gridDim.x;
    const float2* SClds = reinterpret_cast<const float2*>(lds + p.s_off);
    const int cwin = p.win_steps * kWave;                  // chunks per window

    // (The grid never exceeds the row blocks, so every workgroup has one; a
    // test of that here would cost a round trip to the kernel arguments
    // before the others are requested.)
    const int n_my = p.rb_per - ((int)blockIdx.x >= p.rb_full ? 1 : 0);   // row blocks of this workgroup
    const int n_units = n_my * p.nsteps;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.x, M * p.K * (XF32 ? 4 : 2));

    // Units are issued in order: unit (irb, it) is row block
    // blockIdx.x + irb * gridDim.x, wave step it.  Rows past N read row N-1;
    // a lane past the row's last chunk (group) reads the last chunk (group).
    // Slots past the last unit get an empty resource and read nothing.  The
    // resources and row offsets of the row block being issued live in scalar
    // registers and are rebuilt only when the issue moves to the next block;
    // the lane offsets advance by one step per issue.
    int is_t = 0, is_rb = 0;
    int i_row0 = ((int)blockIdx.x * W + wave) * R;   // first row of the block being issued
    const int row_step = grid * W * R;
    __amdgpu_buffer_rsrc_t i_wr, i_sr, i_br;
    int i_sw[R], i_ss[R];                            // per-row scalar offsets (weights, scales/biases)
    int i_ps[RL];                                    // offset of the lane's own row of each row group
    auto set_block = [&]() {
        // every input of the resources is wave-uniform; readfirstlane makes that
        // explicit (a resource the compiler cannot prove uniform costs a
        // waterfall loop around every load)
        const int rbase = in_sgpr(__builtin_amdgcn_readfirstlane(min(i_row0, p.N - 1)));
        const int records = in_sgpr(__builtin_amdgcn_readfirstlane((is_rb < n_my) ? -1 : 0));
        i_wr = make_rsrc(reinterpret_cast<const uint8_t*>(p.w) + (size_t)rbase * p.row_bytes, records);
        i_sr = make_rsrc(p.s + (size_t)rbase * p.G, records);
        i_br = make_rsrc(p.b + (size_t)rbase * p.G, records);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int rr = min(r, p.N - 1 - rbase);
            i_sw[r] = rr * p.row_bytes;
            i_ss[r] = rr * p.G * 2;
        }
        if constexpr (OWNLOAD) {
#pragma unroll
            for (int k = 0; k < RL; ++k) i_ps[k] = min(k * LPG + lane % LPG, p.N - 1 - rbase) * p.G * 2;
        }
    };
    // One vector: the row block's resources first, so that the first weight
    // requests follow the activation loads at once.  More vectors: the
    // activation loads first (their staging is the longer wait), the
    // resources while they are in flight.
    if constexpr (M == 1) set_block();
    const int wo0 = lane * 16;                       // lane's chunk offset in a row's first step
    const int mo0 = (lane / LPG) * 2;                // lane's group offset in a row's first step
    int i_wo = wo0, i_mo = mo0;
    const int wo_max = p.row_bytes - 16, mo_max = p.G * 2 - 2;
    auto issue = [&](uint4 (&wv)[R], unsigned short (&sv)[RL], unsigned short (&bv)[RL]) {
        const int wo = min(i_wo, wo_max);
        const int mo = min(i_mo, mo_max);
#pragma unroll
        for (int r = 0; r < R; ++r) wv[r] = buf_load_nt(i_wr, wo, i_sw[r]);
#pragma unroll
        for (int k = 0; k < (MLDS ? 0 : RL); ++k) {
            if constexpr (OWNLOAD) {
                sv[k] = buf_load_u16(i_sr, mo + i_ps[k], 0);
                bv[k] = buf_load_u16(i_br, mo + i_ps[k], 0);
            } else {
                sv[k] = buf_load_u16(i_sr, mo, i_ss[k]);
                bv[k] = buf_load_u16(i_br, mo, i_ss[k]);
            }
        }
        if (++is_t == p.nsteps) {
            is_t = 0;
            ++is_rb;
            i_row0 += row_step;
            set_block();
            i_wo = wo0;
            i_mo = mo0;
        } else {
            i_wo += kWave * 16;
            i_mo += (kWave / LPG) * 2;
        }
    };

    // Whole K: one wave-wide 128-bit load fetches the scales of all row
    // blocks of this wavefront (another the biases), issued with the weight
    // prologue; the first unit, which waits for the prologue's weights anyway,
    // stores them in this wavefront's part of a static LDS array, where every
    // unit reads them.  Lane l takes piece l % SP of block l / SP, SP =
    // m_slot / 16 pieces per block: block b's rows [r0, r0 + nr) (a block past
    // N reads row N-1) are the bytes from r0*G*2, taken from the 16-byte piece
    // that holds their first byte, so they start (r0*G*2) % 16 bytes into the
    // block's slot.  Lanes past the last block, and pieces past the tensor's
    // last piece, read that last piece again.  The tensors start 16-byte
    // aligned, so every piece holds tensor bytes and lies in their page.
    uint8_t* mcopy = nullptr;
    uint4 mpiece_s = make_uint4(0, 0, 0, 0), mpiece_b = make_uint4(0, 0, 0, 0);
    if constexpr (MLDS) {
        __shared__ __align__(16) uint8_t meta_lds[kMaxWaves][2][kMetaBytes];
        mcopy = &meta_lds[wave][0][0];
    }
    auto load_meta = [&]() {
        const int sp = p.m_slot >> 4;
        const int b = (lane * p.m_div) >> 13;   // lane / sp (exact for lane < 64, sp <= 64)
        const int pc = lane - b * sp;
        const int bb = min(b, n_my - 1);
        const int r0 = min((((int)blockIdx.x + bb * grid) * W + wave) * R, p.N - 1);
        const int start = (int)(((uint32_t)r0 * (uint32_t)(p.G * 2)) & ~15u);
        const int off = min(start + pc * 16, p.sb_last);
        mpiece_s = buf_load(make_rsrc(p.s, -1), off);
        mpiece_b = buf_load(make_rsrc(p.b, -1), off);
    };

    const uint32_t magic = opaque_u32(code_magic<BITS>());
    Stager<BITS, GS, M, XF32> stg;
    stg.nthr = W * kWave;
    uint4 wb[NS][R];
    unsigned short sb[NS][RL], bb[NS][RL];  // scale and bias bits (of the lane's own rows with OWNLOAD)
    auto prologue = [&]() {
#pragma unroll
        for (int s = 0; s < PF; ++s) issue(wb[s], sb[s], bb[s]);
    };
    // activation loads first, then (whole K) the scale/bias pieces, then the
    // weight prologue, then the conversion
    stg.stage(p, xr, lds, 0, [&]() {
        if constexpr (M != 1) set_block();
        if constexpr (MLDS) load_meta();
        prologue();
    });
    __syncthreads();
    if constexpr (STAMP) ts_staged = stamp_now();

    float acc[RS][M];
#pragma unroll
    for (int r = 0; r < RS; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
    int c_rb = 0, c_t = 0, c_tw = 0, c_win = 0;   // unit consumed next; its step within the window
    // Whole K: byte offsets of the lane's scale in the LDS copies.  Per row
    // block: the block's slot, the rows' start in it, and row k of the lane
    // (rows past N read row N-1); per unit the lane's group, clamped to the
    // row's last group.
    int m_roff[RL];
    const int m_goff = (lane / LPG) * 2, m_gmax = (p.G - 1) * 2;
    auto meta_block = [&](int rb) {
        if constexpr (MLDS) {
            const int r0 = min((((int)blockIdx.x + rb * grid) * W + wave) * R, p.N - 1);
            const int nr1 = min(R, p.N - r0) - 1;
            const int base = rb * p.m_slot + (int)(((uint32_t)r0 * (uint32_t)(p.G * 2)) & 15u);
#pragma unroll
            for (int k = 0; k < RL; ++k) m_roff[k] = base + min(k * LPG + lane % LPG, nr1) * p.G * 2;
        }
    };
    meta_block(0);
    const int xl = lds_phys(lane * XCB);          // LDS offset of the lane's chunk in a window's first step
    // Lanes past the row's end (the last step of the last window) read the zero
    // chunk that follows that window's chunks: every valid chunk's offset is
    // below it, so one minimum does the clamp.  (Computed here from loaded
    // arguments: a further kernel argument regrouped the argument loads into a
    // serial pair, +2.5% at one vector.)
    const int xz = lds_phys((p.chunks - (p.nwin - 1) * cwin) * XCB);
    // (K-windowed layouts keep every window's slot whole, with its tail zeroed,
    // so only a one-window layout clamps.)  Held per lane, as the room between
    // the lane's first-step offset and the limit: a scalar kept across the
    // unit loop costs the windowed instances two more scalar-register reloads
    // per unit.
    const int xroom = ((WIN && p.nwin > 1) ? 0x3fffffff : xz) - xl;
    for (int ub = 0; ub < n_units; ub += NS) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            // the slot consumed one unit ago takes the unit PF ahead
            issue(wb[(s + PF) % NS], sb[(s + PF) % NS], bb[(s + PF) % NS]);
            __builtin_amdgcn_sched_barrier(0);
            if (ub + s < n_units) {
                const int t = c_t;
                if constexpr (WIN) {
                    if (c_tw == p.win_steps) {
                        c_tw = 0;
                        ++c_win;
                    }
                    if (p.nwin > 1 && c_tw == 0 && (c_rb > 0 || t > 0)) {
                        // K windows: restage this window (the first one was staged
                        // above; with one window, used for whole K where the
                        // scale/bias copies do not fit, it stays)
                        __syncthreads();
                        stg.stage(p, xr, lds, c_win, [] {});
                        __syncthreads();
                    }
                }
                const uint4 (&wcur)[R] = wb[s];
                // Scale and bias of each row's group.  The group's owner is the lane
                // l with l % lpg == n % lpg for row n.  Ungrouped, every lane folds
                // every row with the scale and bias zeroed on all lanes but the
                // owner, so the fold acc = s*D + (b*S + acc) leaves a non-owner's
                // accumulator unchanged without a branch; grouped, each lane folds
                // only its own rows.  With a multiple of lpg rows per wavefront the
                // block's first row is a multiple of lpg, so row r's owner is the
                // lane with l % lpg == r % lpg, and a lane loaded only the values of
                // the rows it owns.
                const int rb0 = (((int)blockIdx.x + c_rb * grid) * W + wave) * R;   // block's first row
                float sv[RS], bv[RS];
                float fs[RL], fb[RL];
                auto own_select = [&]() {
#pragma unroll
                    for (int k = 0; k < RS; ++k) {
                        if constexpr (GROUPED) {
                            sv[k] = fs[k];
                            bv[k] = fb[k];
                        } else if constexpr (OWNLOAD) {
                            const bool own = (lane % LPG) == (k % LPG);
                            sv[k] = own ? fs[k / LPG] : 0.0f;
                            bv[k] = own ? fb[k / LPG] : 0.0f;
                        } else {
                            const bool own = (lane % LPG) == ((rb0 + k) % LPG);
                            sv[k] = own ? fs[k] : 0.0f;
                            bv[k] = own ? fb[k] : 0.0f;
                        }
                    }
                };
                if constexpr (!MLDS) {
#pragma unroll
                    for (int k = 0; k < RL; ++k) {
                        fs[k] = SBF ? bf16_to_f32_here(sb[s][k]) : f16_to_f32_here(sb[s][k]);
                        fb[k] = SBF ? bf16_to_f32_here(bb[s][k]) : f16_to_f32_here(bb[s][k]);
                    }
                    own_select();
                }
                // Whole K: the scale and bias of this unit come from the LDS
                // copies, read ahead of the activations.  The first unit stores
                // the copies after its activation reads (the store waits for the
                // pieces) and reads them again there.  Each path calls
                // finish_meta() once its activation reads are issued; the
                // conversion there waits for the copies' reads only.
                uint32_t hs[RL], hb[RL];
                const bool first_unit = (ub == 0 && s == 0);
                auto meta_read = [&]() {
                    const int gofs = min(t * (kWave / LPG) * 2 + m_goff, m_gmax);
#pragma unroll
                    for (int k = 0; k < RL; ++k) {
                        const uint8_t* e = mcopy + m_roff[k] + gofs;
                        hs[k] = *reinterpret_cast<const unsigned short*>(e);
                        hb[k] = *reinterpret_cast<const unsigned short*>(e + kMetaBytes);
                    }
                };
                if constexpr (MLDS) meta_read();   // (first unit: read again after its store)
                auto finish_meta = [&]() {
                    if constexpr (MLDS) {
                        if (first_unit) {
                            __builtin_amdgcn_sched_barrier(0);
                            *reinterpret_cast<uint4*>(mcopy + lane * 16) = mpiece_s;
                            *reinterpret_cast<uint4*>(mcopy + kMetaBytes + lane * 16) = mpiece_b;
                            meta_read();
                        }
#pragma unroll
                        for (int k = 0; k < RL; ++k) {
                            // (volatile: the conversion stays here, after the
                            // activation reads, instead of next to the reads)
                            const unsigned short s16 = (unsigned short)hs[k], b16 = (unsigned short)hb[k];
                            fs[k] = SBF ? bf16_to_f32_here(s16) : f16_to_f32_here(s16);
                            fb[k] = SBF ? bf16_to_f32_here(b16) : f16_to_f32_here(b16);
                        }
                        own_select();
                    }
                };
                // chunk's LDS offset (never straddles padding); past the row's end the zero chunk
                const int xo0 = xl + min(c_tw * XSTEP, xroom);
                const int cl = c_tw * kWave + lane;           // chunk within the window

                if constexpr (!XF32) {
                    // ---- bf16 activations: exact code pairs and v_dot2_f32_bf16
                    constexpr int NP = 64 / BITS;              // code pairs per chunk
                    constexpr int PPW = 16 / BITS;             // pairs per word
                    // activation pairs of vector m for this lane's chunk, the chunk's
                    // chain start and the group's sum
                    auto read_x = [&](int m, int xo, uint32_t (&xp)[NP], float& S, float& c0) {
                        const uint8_t* xs = lds + m * p.x_m_bytes + xo;
                        const float2 sc = SClds[m * cwin + cl];
                        c0 = sc.x;
                        S = sc.y;
                        // the chain start is needed first: keep its read ahead of the
                        // activation reads, so the chain can begin as they arrive
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int v = 0; v < NP / 4; ++v) {
                            const uint4 t4 = *reinterpret_cast<const uint4*>(xs + v * 16);
                            xp[4 * v + 0] = t4.x; xp[4 * v + 1] = t4.y;
                            xp[4 * v + 2] = t4.z; xp[4 * v + 3] = t4.w;
                        }
                    };
                    auto decode = [&](const uint4& w4, uint32_t (&qp)[NP]) {
                        const uint32_t wd[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int j = 0; j < PPW; ++j) qp[i * PPW + j] = code_pair<BITS>(wd[i], j, magic);
                    };
                    // one vector's chain over a row's pairs from the chunk's start
                    // -2^bits*S_chunk (so it ends at the raw integer dot), the group's
                    // combine, and the fold (a no-op on all lanes but the owner)
                    auto chain_fold = [&](const uint32_t (&qp)[NP], const uint32_t (&xp)[NP], float S,
                                          float c0, int r, float& a) {
                        float d = c0;
#pragma unroll
                        for (int i = 0; i < NP; ++i) d = dot2(qp[i], xp[i], d);
                        d = lane_group_sum<LPG>(d);
                        a = pinned(__builtin_fmaf(sv[r], d, __builtin_fmaf(bv[r], S, a)));
                    };
                    // Row groups (grouped folds): register j of group k holds row
                    // LPG*k + (j ^ lane % LPG), so the lanes of a weight group run the
                    // group's rows in rotated order.  `combine` adds, for the lane's own
                    // row, its chain and its partners' -- xor 1 first, then xor 2 --
                    // which are the addends and grouping of the plain butterfly.
                    auto swap_words = [&](int k, int i, uint32_t (&out)[LPG]) {
                        uint32_t w[LPG];
#pragma unroll
                        for (int t = 0; t < LPG; ++t) {
                            const uint4& wr = wcur[GROUPED ? LPG * k + t : 0];
                            w[t] = (i == 0) ? wr.x : (i == 1) ? wr.y : (i == 2) ? wr.z : wr.w;
                        }
                        const bool b0 = (lane & 1) != 0;
#pragma unroll
                        for (int t = 0; t < LPG; ++t) out[t] = b0 ? w[(t ^ 1) % LPG] : w[t];
                        if constexpr (LPG == 4) {
                            const bool b1 = (lane & 2) != 0;
                            uint32_t a[LPG];
#pragma unroll
                            for (int t = 0; t < LPG; ++t) a[t] = out[t];
#pragma unroll
                            for (int t = 0; t < LPG; ++t) out[t] = b1 ? a[t ^ 2] : a[t];
                        }
                    };
                    auto combine = [&](const float (&d)[LPG]) -> float {
                        if constexpr (LPG <= 2) {
                            return d[0] + dpp<kQuadXor1>(d[1 % LPG]);
                        } else {
                            const float w0 = d[0] + dpp<kQuadXor1>(d[1]);
                            const float w1 = d[2 % LPG] + dpp<kQuadXor1>(d[3 % LPG]);
                            return w0 + dpp<kQuadXor2>(w1);
                        }
                    };
                    if constexpr (M <= R) {
                        // few vectors: activation pairs of all M vectors first, then one
                        // row at a time, one weight word at a time: decode the word's
                        // pairs and extend every vector's chain with them (the same chain
                        // order as decoding the whole chunk first; only the pairs of one
                        // word are live at once)
                        uint32_t xp[M][NP];
                        float S[M], c0[M];
#pragma unroll
                        for (int m = 0; m < M; ++m) read_x(m, xo0, xp[m], S[m], c0[m]);
                        finish_meta();
                        if constexpr (GROUPED) {
#pragma unroll
                            for (int k = 0; k < RS; ++k) {
                                float d[LPG][M];
#pragma unroll
                                for (int j = 0; j < LPG; ++j)
#pragma unroll
                                    for (int m = 0; m < M; ++m) d[j][m] = c0[m];
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    uint32_t ws[LPG];
                                    swap_words(k, i, ws);
                                    uint32_t q[LPG][PPW];
#pragma unroll
                                    for (int j = 0; j < LPG; ++j)
#pragma unroll
                                        for (int jj = 0; jj < PPW; ++jj) q[j][jj] = code_pair<BITS>(ws[j], jj, magic);
#pragma unroll
                                    for (int m = 0; m < M; ++m)
#pragma unroll
                                        for (int jj = 0; jj < PPW; ++jj)
#pragma unroll
                                            for (int j = 0; j < LPG; ++j)
                                                d[j][m] = dot2(q[j][jj], xp[m][i * PPW + jj], d[j][m]);
                                    __builtin_amdgcn_sched_barrier(0);
                                }
#pragma unroll
                                for (int m = 0; m < M; ++m) {
                                    float dv[LPG];
#pragma unroll
                                    for (int j = 0; j < LPG; ++j) dv[j] = d[j][m];
                                    const float dd = combine(dv);
                                    acc[k][m] = pinned(__builtin_fmaf(sv[k], dd, __builtin_fmaf(bv[k], S[m], acc[k][m])));
                                }
                            }
                        } else {
#pragma unroll
                            for (int r = 0; r < R; ++r) {
                                const uint32_t wd[4] = {wcur[r].x, wcur[r].y, wcur[r].z, wcur[r].w};
                                float d[M];
#pragma unroll
                                for (int m = 0; m < M; ++m) d[m] = c0[m];
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    uint32_t qw[PPW];
#pragma unroll
                                    for (int j = 0; j < PPW; ++j) qw[j] = code_pair<BITS>(wd[i], j, magic);
#pragma unroll
                                    for (int m = 0; m < M; ++m)
#pragma unroll
                                        for (int j = 0; j < PPW; ++j) d[m] = dot2(qw[j], xp[m][i * PPW + j], d[m]);
                                    __builtin_amdgcn_sched_barrier(0);
                                }
#pragma unroll
                                for (int m = 0; m < M; ++m) {
                                    const float dd = lane_group_sum<LPG>(d[m]);
                                    acc[r][m] = pinned(__builtin_fmaf(sv[r], dd, __builtin_fmaf(bv[r], S[m], acc[r][m])));
                                }
                            }
                        }
                    } else {
                        // many vectors: decode every row once, then one vector at a time.
                        // Vector m+1's pairs are read while vector m's chains run; the
                        // read is tied to vector m-1's last result, so the compiler
                        // cannot hoist every vector's reads (and registers) up front.
                        uint32_t xq[2][NP];
                        float Sq[2], cq[2][R];
                        // Every row's chain needs the start in a register of its own (the
                        // dot2 accumulates in place); reading it once per row from LDS
                        // (volatile, so the reads are not merged) spares a vector-ALU
                        // copy per row and vector.
                        auto read_xr = [&](int m, int xo, uint32_t (&xp)[NP], float& S, float (&c0)[R]) {
                            read_x(m, xo, xp, S, c0[0]);
                            typedef __attribute__((address_space(3))) const volatile float lds_f32;
                            lds_f32* cs = (lds_f32*)(&SClds[m * cwin + cl].x);
#pragma unroll
                            for (int r = 1; r < R; ++r) c0[r] = *cs;
                        };
                        read_xr(0, xo0, xq[0], Sq[0], cq[0]);
                        finish_meta();
                        uint32_t qp[R][NP];
                        if constexpr (GROUPED) {
#pragma unroll
                            for (int k = 0; k < RS; ++k) {
                                uint32_t ws[4][LPG];
#pragma unroll
                                for (int i = 0; i < 4; ++i) swap_words(k, i, ws[i]);
#pragma unroll
                                for (int j = 0; j < LPG; ++j)
                                    decode(make_uint4(ws[0][j], ws[1][j], ws[2][j], ws[3][j]), qp[LPG * k + j]);
                            }
                        } else {
#pragma unroll
                            for (int r = 0; r < R; ++r) decode(wcur[r], qp[r]);
                        }
#pragma unroll
                        for (int m = 0; m < M; ++m) {
                            if (m + 1 < M) {
                                const int xo = (m == 0) ? xo0 : after(xo0, acc[RS - 1][m - 1]);
                                read_xr(m + 1, xo, xq[(m + 1) & 1], Sq[(m + 1) & 1], cq[(m + 1) & 1]);
                            }
                            if constexpr (GROUPED) {
                                float d[R];
#pragma unroll
                                for (int r = 0; r < R; ++r) {
                                    d[r] = cq[m & 1][r];
#pragma unroll
                                    for (int i = 0; i < NP; ++i) d[r] = dot2(qp[r][i], xq[m & 1][i], d[r]);
                                }
#pragma unroll
                                for (int k = 0; k < RS; ++k) {
                                    float dv[LPG];
#pragma unroll
                                    for (int j = 0; j < LPG; ++j) dv[j] = d[GROUPED ? LPG * k + j : 0];
                                    const float dd = combine(dv);
                                    acc[k][m] = pinned(__builtin_fmaf(sv[k], dd, __builtin_fmaf(bv[k], Sq[m & 1], acc[k][m])));
                                }
                            } else {
#pragma unroll
                                for (int r = 0; r < R; ++r) chain_fold(qp[r], xq[m & 1], Sq[m & 1], cq[m & 1][r], r, acc[r][m]);
                            }
                            // keep each vector's folds next to its chains (left free, the
                            // scheduler sinks them and holds every chain result live)
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                } else {
                    // ---- fp32 activations: exact fp32 codes and an fma chain, one
                    // weight word at a time; the activations of step k+1 (word, vector)
                    // are read while step k's chains run
                    constexpr int VPW = 32 / BITS;             // values per word
                    float dsum[R][M];
                    float xq[2][VPW];
                    auto read_x = [&](int k, int xo, float (&xv)[VPW]) {
                        const int i = k / M, m = k % M;
                        const uint8_t* xs = lds + m * p.x_m_bytes + xo + i * VPW * 4;
#pragma unroll
                        for (int v = 0; v < VPW / 4; ++v) {
                            const float4 t4 = *reinterpret_cast<const float4*>(xs + v * 16);
                            xv[4 * v + 0] = t4.x; xv[4 * v + 1] = t4.y;
                            xv[4 * v + 2] = t4.z; xv[4 * v + 3] = t4.w;
                        }
                    };
                    read_x(0, xo0, xq[0]);
                    finish_meta();
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float qv[R][VPW];
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            const uint32_t wd = (i == 0) ? wcur[r].x : (i == 1) ? wcur[r].y
                                              : (i == 2) ? wcur[r].z : wcur[r].w;
#pragma unroll
                            for (int j = 0; j < VPW; ++j)
                                qv[r][j] = (float)((wd >> (BITS * j)) & ((1u << BITS) - 1u));
                        }
#pragma unroll
                        for (int m = 0; m < M; ++m) {
                            // step k+1's read is tied to step k-1's last chain result
                            const int k = i * M + m;
                            if (k + 1 < 4 * M) {
                                const int xo = (k == 0) ? xo0 : after(xo0, dsum[R - 1][(k - 1) % M]);
                                read_x(k + 1, xo, xq[(k + 1) & 1]);
                            }
                            const float (&xv)[VPW] = xq[k & 1];
#pragma unroll
                            for (int r = 0; r < R; ++r) {
                                float d = (i == 0) ? 0.0f : dsum[r][m];
#pragma unroll
                                for (int j = 0; j < VPW; ++j) d = __builtin_fmaf(qv[r][j], xv[j], d);
                                dsum[r][m] = d;
                            }
                        }
                    }
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        const float S = SClds[m * cwin + cl].y;
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            const float d = lane_group_sum<LPG>(dsum[r][m]);
                            acc[r][m] = pinned(__builtin_fmaf(sv[r], d, __builtin_fmaf(bv[r], S, acc[r][m])));
                        }
                    }
                }

                if (t == p.nsteps - 1) {
                    // row totals and output: lane l stores value reduce_index(l)
                    float v[P];
#pragma unroll
                    for (int i = 0; i < P; ++i) v[i] = (i < V) ? acc[i / M][i % M] : 0.0f;
                    lane_reduce<P, SKIP>(v, lane);
                    const int idx = reduce_index<P, SKIP>(lane);
                    const int k = idx / M, m = idx - (idx / M) * M;
                    const int r = GROUPED ? LPG * k + lane % LPG : k;
                    const bool holder = ((lane >> SKIP) % ((64 >> SKIP) / P)) == 0;
                    if (holder && idx < V && rb0 + r < p.N) {
                        const size_t o = (size_t)m * p.N + rb0 + r;
                        if (p.y_bf16)
                            static_cast<uint16_t*>(p.y)[o] = (uint16_t)f32_to_bf16_rne(v[0]);
                        else
                            static_cast<float*>(p.y)[o] = v[0];
                    }
#pragma unroll
                    for (int rr = 0; rr < RS; ++rr)
#pragma unroll
                        for (int mm = 0; mm < M; ++mm) acc[rr][mm] = 0.0f;
                    c_t = 0;
                    c_tw = 0;
                    c_win = 0;
                    ++c_rb;
                    meta_block(c_rb);
                } else {
                    ++c_t;
                    ++c_tw;
                }
            }
        }
    }
    if constexpr (STAMP) {
        const uint64_t ts_end = stamp_now();
        const uint32_t xcc = __builtin_amdgcn_s_getreg(0xf814);   // hwreg(HW_REG_XCC_ID)
        const uint32_t hwid = __builtin_amdgcn_s_getreg(0xf804);  // hwreg(HW_REG_HW_ID)
        // lane 0, from the lane count (the lane id in a register of its own
        // would stay live through the unit loop)
        if (__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) == 0) {
            uint64_t* const stamps[] = {stamp_ptr...};
            uint64_t* o = stamps[0] + ((size_t)blockIdx.x * W + wave) * kStamps;
            o[0] = ts_start;
            o[1] = ts_staged;
            o[2] = ts_end;
            o[3] = ((uint64_t)xcc << 32) | hwid;
        }
    }
}

}  // namespace qmv
