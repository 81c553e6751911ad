/*
 * qmv_oracle.c -- plain CPU oracle for the affine group-quantized
 * matrix-vector product (qmv).
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this file's library.  The GPU
 * library never includes, links or calls it, and it shares no code, header,
 * table or helper with the GPU path.
 *
 * What it computes (fp64 accumulation, no blocking, no reordering beyond the
 * grouped definition itself; the mxfp4 mode further below):
 *
 *   y[m][n] = sum_g ( scale[n][g] * sum_{k in g} q[n][k] * x[m][k]
 *                   + bias[n][g]  * sum_{k in g} x[m][k] )
 *
 * Sources (cited by page title and section):
 *  - mlxcel issue "an order-preserving streamed qmv would give MTP the fast
 *    kernel and byte-identity together", section "Correction to the obvious
 *    sketch: qdot does not dequantize": the weight of element i is
 *    scale*q_i + bias; the group parameters are applied once, to the raw
 *    integer dot and to sum(x) (the `scale * accum + sum * bias` fold).
 *  - mlxcel PR "block output rows per warp in qmv below Ampere", section
 *    "Not covered": the per-group form sum_g [scale*sum(x*w_int) + bias*sum(x)].
 *  - same issue, section "Step 2": row-major packed rows (row n starts at
 *    ws + n*in_vec_size_w) and per-group scales/biases rows
 *    (scales + n*in_vec_size_g); section "The observation this rests on":
 *    vector m of the block starts at x + m*in_vec_size, its output at
 *    y + m*out_vec_size.
 *  - field order "field 0 in the low bits": the 4-bit masks 0x000f, 0x00f0,
 *    0x0f00, 0xf000 in the "Correction" section (fields 0..3 of a 16-bit
 *    half, lowest first) and llama.cpp PR "PQ2_0 and Q2_0 mat-vec dot in
 *    exact float", section "How" (plain bit packing keeps field 0 in the low
 *    bits).
 *
 * Every input value (bf16, fp16, fp32 activations and parameters, and the
 * integers q) converts to double exactly; each product q*x, scale*D and
 * bias*S of bf16/fp16 operands is exact in double, so the only rounding is
 * that of the fp64 sums.
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* dtype codes of the oracle's own interface (same numbering as the library's
 * public header by convention only; nothing is shared) */
enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

/* IEEE 754 binary16 -> double, from the format's definition:
 * sign 1 bit, exponent 5 bits (bias 15), fraction 10 bits; exponent 0 holds
 * zero and subnormals (fraction * 2^-24), exponent 31 holds inf/NaN. */
double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f | 0x400), e - 25);
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double orc_bf16_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double elem(const void* p, size_t i, int dt)
{
    if (dt == ORC_F32) return (double)((const float*)p)[i];
    if (dt == ORC_F16) return orc_f16_to_f64(((const uint16_t*)p)[i]);
    return orc_bf16_to_f64(((const uint16_t*)p)[i]);
}

/* field k of a packed row: word k / (32/bits), field j = k mod (32/bits)
 * occupying bits [bits*j, bits*(j+1)) of that word (field 0 lowest). */
unsigned orc_field(const uint32_t* row, int k, int bits)
{
    int pf = 32 / bits;
    uint32_t w = row[k / pf];
    int j = k % pf;
    return (w >> (bits * j)) & ((1u << bits) - 1u);
}

/* unpack one packed row of K fields into q[0..K) */
void orc_unpack_row(const uint32_t* row, int K, int bits, uint8_t* q)
{
    for (int k = 0; k < K; ++k) q[k] = (uint8_t)orc_field(row, k, bits);
}

static int check(int M, int N, int K, int bits, int gs)
{
    if (bits != 2 && bits != 4) return -1;
    if (gs != 64 && gs != 128) return -2;
    if (M < 0 || N < 0 || K < 0) return -3;
    if (K % gs) return -4;
    return 0;
}

/* y_ref for one output row n and one vector m, in the grouped form. */
static double one(const uint32_t* w, const void* scales, const void* biases, int sb_dt,
                  const void* x, int x_dt, int m, int n, int K, int bits, int gs)
{
    const int G = K / gs;
    const uint32_t* row = w + (size_t)n * (size_t)(K * bits / 32);
    double acc = 0.0;
    for (int g = 0; g < G; ++g) {
        double D = 0.0, S = 0.0;
        for (int k = g * gs; k < (g + 1) * gs; ++k) {
            double q = (double)orc_field(row, k, bits);
            double xv = elem(x, (size_t)m * (size_t)K + (size_t)k, x_dt);
            D += q * xv;
            S += xv;
        }
        double s = elem(scales, (size_t)n * G + g, sb_dt);
        double b = elem(biases, (size_t)n * G + g, sb_dt);
        acc += s * D + b * S;
    }
    return acc;
}

/*
 * Full oracle: y[m*N + n] (double) for all m < M, n < N.
 * w: [N][K*bits/32] uint32; scales, biases: [N][K/gs] (sb_dt); x: [M][K] (x_dt).
 * nthreads <= 0 uses the OpenMP default.  Returns 0, or a negative code for a
 * shape the definition does not cover.
 */
int orc_qmv_affine(const uint32_t* w, const void* scales, const void* biases, int sb_dt,
                   const void* x, int x_dt, double* y, int M, int N, int K, int bits, int gs,
                   int nthreads)
{
    int rc = check(M, N, K, bits, gs);
    if (rc) return rc;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    #pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n)
        for (int m = 0; m < M; ++m)
            y[(size_t)m * N + n] = one(w, scales, biases, sb_dt, x, x_dt, m, n, K, bits, gs);
    return 0;
}

/*
 * Sampled oracle: the same value for a list of (m, n) pairs, for checks of
 * full-size launches element by element.  out[i] = y_ref[ms[i]][ns[i]].
 */
int orc_qmv_affine_at(const uint32_t* w, const void* scales, const void* biases, int sb_dt,
                      const void* x, int x_dt, const int* ms, const int* ns, int count,
                      double* out, int N, int K, int bits, int gs, int nthreads)
{
    int rc = check(1, N, K, bits, gs);
    if (rc) return rc;
    for (int i = 0; i < count; ++i)
        if (ns[i] < 0 || ns[i] >= N || ms[i] < 0) return -5;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    #pragma omp parallel for schedule(static)
    for (int i = 0; i < count; ++i)
        out[i] = one(w, scales, biases, sb_dt, x, x_dt, ms[i], ns[i], K, bits, gs);
    return 0;
}

/*
 * Term magnitude of each output, for an a-priori bound on the rounding error
 * of any fp32 evaluation of the grouped form:
 *
 *   mag[m][n] = sum_g ( 2^(bits+2) |scale[n][g]| + |bias[n][g]| ) * sum_{k in g} |x[m][k]|
 *
 * Every code satisfies 0 <= q < 2^bits.  An evaluation may add an offset
 * 0 <= c <= 2^bits to every code and remove it again as -c*scale*sum(x) (equal
 * in real arithmetic, as the grouped and dequantized forms are: mlxcel issue
 * "an order-preserving streamed qmv would give MTP the fast kernel and
 * byte-identity together", section "Correction to the obvious sketch"); its
 * terms scale*(q + c)*x, -c*scale*x and bias*x then have magnitudes summing to
 * at most (3*2^bits |scale| + |bias|)|x| < (2^(bits+2) |scale| + |bias|)|x|.
 * A sum evaluated in fp32 through at most d roundings per
 * term differs from the exact sum by at most gamma_d = d*u/(1 - d*u) (u = 2^-24)
 * times the sum of the magnitudes of its terms (the standard bound for
 * floating-point summation), so |y - y_ref| <= gamma_d * mag.  The bound holds
 * whatever the value of y, including outputs that cancel far below their
 * terms.  The codes do not enter it, so w is not an argument.
 */
int orc_qmv_affine_mag(const void* scales, const void* biases, int sb_dt, const void* x,
                       int x_dt, double* mag, int M, int N, int K, int bits, int gs,
                       int nthreads)
{
    int rc = check(M, N, K, bits, gs);
    if (rc) return rc;
    const int G = K / gs;
    const double span = ldexp(1.0, bits + 2);
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    #pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n)
        for (int m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int g = 0; g < G; ++g) {
                double A = 0.0;
                for (int k = g * gs; k < (g + 1) * gs; ++k)
                    A += fabs(elem(x, (size_t)m * (size_t)K + (size_t)k, x_dt));
                double s = fabs(elem(scales, (size_t)n * G + g, sb_dt));
                double b = fabs(elem(biases, (size_t)n * G + g, sb_dt));
                acc += (span * s + b) * A;
            }
            mag[(size_t)m * N + n] = acc;
        }
    return 0;
}

/* ------------------------------------------------------------------ mxfp4
 * Microscaling FP4 (the "mxfp4" quantization mode the MLX pages list beside
 * the affine one; the pages do not define it, so the definition is the OCP
 * Microscaling Formats (MX) specification v1.0): blocks of 32 elements share
 * one E8M0 scale X = 2^(E - 127) (E = 255 encodes NaN); each element is FP4
 * E2M1 -- sign bit 3, exponent bits 2..1 with bias 1, mantissa bit 0;
 * exponent 0 is the subnormal range, 2^(1-1) * (m / 2); no inf or NaN.
 * Elements are packed 8 per uint32 with field 0 in the low bits (the affine
 * 4-bit packing), scales are uint8 [N][K/32]:
 *
 *   y[m][n] = sum_b X[n][b] * sum_{k in b} e2m1(q[n][k]) * x[m][k]
 *
 * Every element, scale and activation converts to double exactly, and each
 * product is exact in double.
 */
double orc_e2m1_to_f64(unsigned c)
{
    int sign = (c >> 3) & 1;
    int e = (c >> 1) & 3;
    int m = c & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -v : v;
}

double orc_e8m0_to_f64(unsigned E)
{
    return (E & 0xffu) == 0xffu ? NAN : ldexp(1.0, (int)(E & 0xffu) - 127);
}

static double one_mx(const uint32_t* w, const uint8_t* scales, const void* x, int x_dt,
                     int m, int n, int K)
{
    const int B = K / 32;
    const uint32_t* row = w + (size_t)n * (size_t)(K / 8);
    double acc = 0.0;
    for (int b = 0; b < B; ++b) {
        double D = 0.0;
        for (int k = b * 32; k < (b + 1) * 32; ++k)
            D += orc_e2m1_to_f64(orc_field(row, k, 4)) *
                 elem(x, (size_t)m * (size_t)K + (size_t)k, x_dt);
        acc += orc_e8m0_to_f64(scales[(size_t)n * B + b]) * D;
    }
    return acc;
}

/* y[m*N + n] (double) for all m < M, n < N; K a multiple of 32. */
int orc_qmv_mxfp4(const uint32_t* w, const uint8_t* scales, const void* x, int x_dt,
                  double* y, int M, int N, int K, int nthreads)
{
    if (M < 0 || N < 0 || K < 0) return -3;
    if (K % 32) return -4;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    #pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n)
        for (int m = 0; m < M; ++m)
            y[(size_t)m * N + n] = one_mx(w, scales, x, x_dt, m, n, K);
    return 0;
}

/*
 * Term magnitude of each mxfp4 output, for the same kind of a-priori bound:
 *   mag[m][n] = sum_b X[n][b] * 6 * sum_{k in b} |x[m][k]|
 * (6 is the largest E2M1 magnitude, so X*6 bounds |X * e2m1(q)|).  A block
 * scale of NaN (E = 255) gives NaN.
 */
int orc_qmv_mxfp4_mag(const uint8_t* scales, const void* x, int x_dt, double* mag,
                      int M, int N, int K, int nthreads)
{
    if (M < 0 || N < 0 || K < 0) return -3;
    if (K % 32) return -4;
    const int B = K / 32;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    #pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n)
        for (int m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int b = 0; b < B; ++b) {
                double A = 0.0;
                for (int k = b * 32; k < (b + 1) * 32; ++k)
                    A += fabs(elem(x, (size_t)m * (size_t)K + (size_t)k, x_dt));
                acc += orc_e8m0_to_f64(scales[(size_t)n * B + b]) * 6.0 * A;
            }
            mag[(size_t)m * N + n] = acc;
        }
    return 0;
}

/* IEEE round-to-nearest-even of a binary32 to bfloat16, from the definition:
 * keep the upper 16 bits, rounding on the discarded lower 16 (ties to the
 * even upper half); NaN stays a quiet NaN. */
uint16_t orc_f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t upper = u >> 16;
    uint32_t lower = u & 0xffffu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
    return (uint16_t)upper;
}

/* double -> binary32 with the default (round-to-nearest-even) mode, then -> bf16 */
void orc_round_outputs(const double* y, size_t count, float* y32, uint16_t* y16)
{
    for (size_t i = 0; i < count; ++i) {
        float f = (float)y[i];
        if (y32) y32[i] = f;
        if (y16) y16[i] = orc_f32_to_bf16_rne(f);
    }
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
