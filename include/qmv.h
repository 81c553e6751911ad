/*
 * qmv.h -- C ABI of the MI355X (gfx950) affine group-quantized
 * matrix-vector product, streamed over up to 13 activation vectors.
 *
 * The operation.  For m < M and n < N,
 *
 *   y[m][n] = sum_{g < K/gs} ( scale[n][g] * sum_{k in g} q[n][k] * x[m][k]
 *                            + bias[n][g]  * sum_{k in g} x[m][k] )
 *
 * i.e. the product of x with the affine-dequantized weights
 * W[n][k] = scale[n][g(k)] * q[n][k] + bias[n][g(k)], with the group
 * parameters applied once per group, to the raw integer dot and to sum(x).
 * Defined in mlxcel issue "an order-preserving streamed qmv would give MTP the
 * fast kernel and byte-identity together" (section "Correction to the obvious
 * sketch: qdot does not dequantize": the qdot fold scale*accum + sum*bias) and
 * mlxcel PR "block output rows per warp in qmv below Ampere" (section "Not
 * covered": the per-group form).  The M vectors are those of a speculative /
 * MTP verify block (same issue, sections "Problem" and "Scope limits").
 *
 * Layouts (all row-major, dense, no padding):
 *   w_packed  uint32 [N][K*bits/32]; field j of a word (j < 32/bits) occupies
 *             bits [bits*j, bits*(j+1)) -- field 0 in the low bits -- and
 *             holds q[n][k] for k = word*(32/bits) + j.
 *   scales, biases  [N][K/gs] of the parameter dtype (fp16 or bf16).
 *   x         [M][K] of the activation dtype (fp32 or bf16).
 *   y         [M][N] of the output dtype (fp32 or bf16), written with
 *             round-to-nearest-even from the fp32 accumulator.
 *
 * Numerics.  Accumulation is fp32 in one fixed per-row order that depends on
 * (K, bits, group_size, activation dtype) only: never on M, rows_per_wave, the
 * launch shape or the stream.  Output vector m of an M-vector call is
 * therefore bit-identical to a 1-vector call on x[m], and repeated calls are
 * bit-identical.
 *
 * Ownership and concurrency.  Every pointer is device memory owned by the
 * caller; the library never allocates, frees, or keeps a pointer past the
 * call, and uses no workspace.  Inputs are read only; y must not overlap any
 * input.  Calls are asynchronous on `stream` (a hipStream_t, NULL = the
 * default stream): they return after the launch is enqueued and y is valid
 * once the stream has been synchronized.  The only state the library keeps
 * is a per-device cache of launch-shape queries (compute-unit count and
 * occupancy per kernel instance), filled on first use under a lock;
 * concurrent calls from several host threads are safe.  When one wave step
 * of activations for all M vectors does not fit in LDS (fp32 activations with
 * 2-bit codes and large M), a call is issued as several launches on the same
 * stream, each over a subset of the vectors; the results do not change.
 *
 * Errors.  Arguments are validated, and every launch of the call (one per
 * tile of vectors, below) is planned, on the host before anything is
 * enqueued; a status other than QMV_OK from validation or planning means that
 * nothing was launched and y is untouched.  QMV_E_LAUNCH from the HIP runtime
 * refusing a launch is the one exception: in a call cut into several tiles,
 * the tiles enqueued before the refused one may already have written their
 * part of y.  Faults inside a kernel surface, as with any HIP kernel, at the
 * caller's next synchronization.  The C ABI sees pointers, not buffer
 * lengths: the caller guarantees that each buffer holds the shape given by
 * (M, N, K, bits, group_size) and its dtype (the Python binding checks the
 * tensor shapes before calling).
 */
#ifndef QMV_H
#define QMV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { QMV_DT_F32 = 0, QMV_DT_F16 = 1, QMV_DT_BF16 = 2 } qmv_dtype;

enum {
    QMV_OK = 0,
    QMV_E_NULL = 1,     /* a required pointer is NULL */
    QMV_E_BITS = 2,     /* bits is not 2 or 4 */
    QMV_E_GROUP = 3,    /* group_size is not 64 or 128 */
    QMV_E_SHAPE = 4,    /* N < 1, K < 1, K % group_size != 0, or the shape exceeds
                           the limits below */
    QMV_E_M_RANGE = 5,  /* M is not in [1, QMV_MAX_M] */
    QMV_E_ALIGN = 6,    /* w_packed, scales, biases or x is not 16-byte aligned, or y
                           is not aligned to its element size */
    QMV_E_DTYPE = 7,    /* unsupported dtype (x: f32/bf16; scales and biases:
                           f16/bf16; y: f32/bf16) */
    QMV_E_ROWS = 8,     /* rows_per_wave is not 0, 1, 2, 3 or 4 */
    QMV_E_ALIAS = 9,    /* y overlaps an input buffer */
    QMV_E_LAUNCH = 10   /* the HIP runtime refused the launch (e.g. no gfx950 device) */
};

/* Vectors per call.  One kernel launch serves at most QMV_TILE_M vectors (the
 * served range of the streamed qmv: mlxcel issue "an order-preserving streamed
 * qmv would give MTP the fast kernel and byte-identity together", section
 * "Scope limits"); a call with more runs them as balanced tiles of at most
 * QMV_TILE_M vectors, launched in order on the stream.  Fewer vectors per tile
 * are used where the activations of QMV_TILE_M vectors do not fit in LDS whole
 * (long K).  Each vector's arithmetic is the same in every tile, so every output
 * vector is bit-identical to the one-vector call on that vector for any M. */
#define QMV_MAX_M 65536
#define QMV_TILE_M 13
/* Largest K (keeps every LDS and row offset inside 32-bit arithmetic). */
#define QMV_MAX_K (1 << 20)
#define QMV_MAX_N (1 << 28)

/*
 * y = qmv(x) with the common dtypes: x bf16, scales and biases bf16, y bf16.
 *   w_packed, scales, biases, x, y: device pointers as laid out above.
 *   M in [1, QMV_MAX_M]; N >= 1; K >= group_size, K % group_size == 0;
 *   bits in {2, 4}; group_size in {64, 128}; stream: hipStream_t or NULL.
 * Returns QMV_OK or a QMV_E_* status.
 */
int qmv_affine(const uint32_t* w_packed, const void* scales, const void* biases,
               const void* x, void* y, int M, int N, int K, int bits, int group_size,
               void* stream);

/*
 * Same operation and kernel family with explicit dtypes and row blocking.
 *   x_dt: QMV_DT_F32 or QMV_DT_BF16; sb_dt (scales and biases): QMV_DT_F16 or
 *   QMV_DT_BF16; y_dt: QMV_DT_F32 or QMV_DT_BF16.
 *   rows_per_wave: output rows owned by one wavefront (1, 2, 3 or 4; 2-bit codes
 *   use at most 2), or 0 for the library's choice.  It changes the launch shape only, never the result
 *   (mlxcel PR "block output rows per warp in qmv below Ampere", section "What
 *   lands": row blocking leaves the per-row arithmetic untouched).
 */
int qmv_affine_ex(const uint32_t* w_packed, const void* scales, const void* biases,
                  const void* x, void* y, int M, int N, int K, int bits, int group_size,
                  qmv_dtype x_dt, qmv_dtype sb_dt, qmv_dtype y_dt, int rows_per_wave,
                  void* stream);

/* Resources and launch shape of the kernel the library would use for a call
 * with these arguments (its first launch, when the call is cut into several
 * tiles of vectors; no launch is made; needs a gfx950 device for the
 * occupancy query).  The arguments are those of qmv_affine_ex without the
 * pointers and the stream, validated the same way; y_dt selects no instance
 * (the output dtype is a run-time flag of every kernel) and is validated
 * only.  Fields: vgprs (architected VGPRs per lane as compiled),
 * scratch_bytes (private memory per lane; 0 = no register spills), lds_bytes
 * per workgroup (dynamic plus static), wg_size (threads), grid (workgroups),
 * waves_per_simd (wavefronts per SIMD on the busiest compute unit: its
 * resident workgroups times their wavefronts over its four SIMDs),
 * rows_per_wave, k_windows (K windows the activation tile is staged in;
 * 1 = whole K), prefetch_units (units of R rows x one 64-lane step whose
 * loads each wavefront keeps in flight), meta_lds (1: each wavefront loads
 * the scales and biases of all its rows once and reads them from LDS; 0: it
 * loads each unit's with the unit's weights).  The HIP runtime's function
 * attributes report no scalar register count, so there is no sgprs field. */
typedef struct {
    int vgprs;
    int scratch_bytes;
    int lds_bytes;
    int wg_size;
    int grid;
    int waves_per_simd;
    int rows_per_wave;
    int k_windows;
    int prefetch_units;
    int meta_lds;
} qmv_kernel_info_t;

int qmv_kernel_info(int M, int N, int K, int bits, int group_size, qmv_dtype x_dt,
                    qmv_dtype sb_dt, qmv_dtype y_dt, int rows_per_wave,
                    qmv_kernel_info_t* out);

/* Measurement aid, not part of the product: reads `bytes` bytes at `buf` (device
 * memory, 16-byte aligned, bytes a positive multiple of 16) with four
 * 8-wavefront workgroups per compute unit and 128-bit non-temporal loads.  Its time is the
 * streaming-read ceiling a one-launch kernel of that shape reaches on that many
 * bytes, against which the qmv's fraction of the HBM peak is read.  With
 * `checksum` nonzero it also XORs the XOR of all 32-bit words of the buffer into
 * *out (device memory, 4-byte aligned; clear it first), one atomic per
 * wavefront on that one address -- slow, for checking; with `checksum` zero it
 * only reads (it may store to *out).  Asynchronous on `stream`; one kernel
 * launch, no other work.  Returns QMV_E_NULL, QMV_E_SHAPE, QMV_E_ALIGN or
 * QMV_E_LAUNCH on bad arguments or a refused launch. */
int qmv_stream_read(const void* buf, long long bytes, uint32_t* out, int checksum, void* stream);

/* The same measurement aid with its launch shape as arguments, for sweeping
 * the ceiling: wg_per_cu workgroups per compute unit (1..32), waves_per_wg
 * wavefronts per workgroup (1..16), batch loads in flight per lane (1, 2, 4,
 * 8 or 16), and interleave = 0 (each wavefront reads its own contiguous span
 * of 1 KiB runs) or 1 (instruction j of wavefront w reads run j*TW + w, TW the
 * wavefronts in the grid).  qmv_stream_read is (4, 8, 4, 0).  Other values
 * return QMV_E_SHAPE. */
int qmv_stream_read_ex(const void* buf, long long bytes, uint32_t* out, int checksum,
                       int wg_per_cu, int waves_per_wg, int batch, int interleave, void* stream);

/* Measurement aid, not part of the product: the one launch qmv_affine_ex
 * makes for these arguments with bf16 activations and bf16 scales and
 * biases, and 4-bit codes in groups of 64 or 2-bit codes in groups of 128
 * (the library's choice of launch, or rows_per_wave as there), run by the
 * same kernel with per-wavefront stamps added.  y is written exactly as qmv_affine_ex writes it.  For wavefront
 * w = workgroup * (wg_size / 64) + wavefront-in-workgroup, lane 0 writes
 * QMV_STAMPS values to stamps[w * QMV_STAMPS ...]: the device's constant-rate
 * counter (s_memrealtime, clock_khz ticks per millisecond) at the wavefront's
 * start, once its activations are staged (after the workgroup barrier), and
 * at its end; then (XCC id << 32) | HW_ID, the hardware register that names
 * the wavefront's compute unit (bits 8..11), shader array (bit 12), shader
 * engine (bits 13..15) and SIMD (bits 4..5).  Nothing is stamped inside the
 * unit loop, whose code stays the product's; each counter read waits for its
 * own result (and any LDS or scalar load still in flight), so the stamped
 * kernel runs as the product one does, give or take three such reads and one
 * 32-byte store per wavefront.
 *   stamps: device memory, 8-byte aligned, stamps_len >= waves * QMV_STAMPS
 *   entries, not overlapping any other buffer; NULL only fills *info (no
 *   launch).  info (host memory, required): waves and grid of the launch,
 *   wg_size (threads), clock_khz, and resident workgroups per compute unit and
 *   VGPRs of the stamped instance beside those of the product instance (equal
 *   when the stamps change nothing of the launch's residency).
 * M must be in [1, QMV_TILE_M] and the call one launch (else QMV_E_M_RANGE);
 * QMV_E_GROUP for another pairing of bits and group size; other errors as for
 * qmv_affine_ex, plus QMV_E_SHAPE for too few stamps,
 * QMV_E_ALIGN and QMV_E_ALIAS for the stamps buffer.  Asynchronous on
 * `stream`; the stamps are valid once it has been synchronized. */
#define QMV_STAMPS 4
typedef struct {
    int waves;
    int wg_size;
    int grid;
    int clock_khz;
    int blocks_per_cu;
    int product_blocks_per_cu;
    int vgprs;
    int product_vgprs;
} qmv_timeline_info_t;

int qmv_affine_timeline(const uint32_t* w_packed, const void* scales, const void* biases,
                        const void* x, void* y, int M, int N, int K, int bits, int group_size,
                        qmv_dtype y_dt, int rows_per_wave, uint64_t* stamps, long long stamps_len,
                        qmv_timeline_info_t* info, void* stream);

/* Measurement aid, not part of the product: one launch of the qmv_affine_ex
 * kernels with its launch shape given instead of chosen -- rows_per_wave R in
 * 1..4 (1..2 for 2-bit codes), waves_per_wg W in 1..8 wavefronts per
 * workgroup, and row_blocks_per_wg: each workgroup walks that many row blocks
 * of W*R rows (the last workgroups one fewer where it does not divide), so the
 * grid is ceil(ceil(N / (W*R)) / row_blocks_per_wg) workgroups.  For sweeping
 * the launch shape; the per-row arithmetic does not depend on R, W or the
 * grid, so y is bit-identical to qmv_affine_ex's.  Arguments, ownership and
 * numerics as for qmv_affine_ex; M must fit one launch (else QMV_E_M_RANGE);
 * QMV_E_ROWS for an R with no instance, QMV_E_SHAPE for W or row_blocks_per_wg
 * out of range or activations that do not fit LDS, QMV_E_LAUNCH if no
 * workgroup of that shape is resident.  info (host memory, optional) receives
 * the launch as qmv_kernel_info describes one.  Asynchronous on `stream`. */
int qmv_affine_shape(const uint32_t* w_packed, const void* scales, const void* biases,
                     const void* x, void* y, int M, int N, int K, int bits, int group_size,
                     qmv_dtype x_dt, qmv_dtype sb_dt, qmv_dtype y_dt, int rows_per_wave,
                     int waves_per_wg, int row_blocks_per_wg, qmv_kernel_info_t* info, void* stream);

/*
 * mxfp4 mode: y = qmv(x) with FP4 (E2M1) codes and one E8M0 scale per block of
 * 32 values along K, no bias:
 *
 *   y[m][n] = sum_b 2^(E[n][b] - 127) * sum_{k in b} e2m1(q[n][k]) * x[m][k]
 *
 * The MLX pages list this quantization mode beside the affine one (mlxcel
 * issue "an order-preserving streamed qmv would give MTP the fast kernel and
 * byte-identity together", section "Scope limits") without defining it; the
 * element and scale formats are those of the OCP Microscaling Formats (MX)
 * specification v1.0: E2M1 is sign bit 3, exponent bits 2..1 (bias 1),
 * mantissa bit 0, exponent 0 subnormal (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and
 * their negatives); E8M0 is 2^(E - 127), E = 255 NaN.
 *   w_packed  uint32 [N][K/8], code k of a row in field k % 8 (bits
 *             [4*(k%8), 4*(k%8)+4)) of word k / 8 -- field 0 in the low bits.
 *   scales    uint8 [N][K/32] (E8M0), no alignment requirement.
 *   x         [M][K] of x_dt (QMV_DT_BF16 or QMV_DT_F32); y [M][N] of y_dt
 *             (QMV_DT_F32 or QMV_DT_BF16, RNE).
 *   M in [1, QMV_MAX_M]; N in [1, QMV_MAX_N]; K a multiple of 32 in
 *   [32, QMV_MX_MAX_K] with N*K/2 < 2^31; w_packed and x 16-byte aligned, y
 *   aligned to its element size; y must not overlap an input.
 * Numerics: each block's dot is an fp32 v_dot2 chain over its exact bf16 code
 * pairs in K order (fp32 x: an fma chain over its exact fp32 codes in K order),
 * from 0, folded once as acc = fma(2^(E-127), D, acc) in ascending block order
 * per lane, then a fixed 64-lane butterfly; every output vector
 * equals the one-vector call on that vector bit for bit.  Ownership, streams
 * and errors as for qmv_affine.  At most QMV_TILE_M vectors per launch (fp32 x:
 * four; more run as balanced tiles); x is staged in LDS whole or, when it does not fit,
 * in K windows (or, for many rows, as two tiles of vectors that fit whole) --
 * none of which changes a result bit.
 */
#define QMV_MX_MAX_K 65536
int qmv_mxfp4(const uint32_t* w_packed, const uint8_t* scales, const void* x, void* y,
              int M, int N, int K, qmv_dtype x_dt, qmv_dtype y_dt, void* stream);

/* Static string naming a status code ("QMV_OK", "QMV_E_BITS", ...). */
const char* qmv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* QMV_H */
