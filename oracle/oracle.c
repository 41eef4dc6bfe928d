/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the matrix-core
 * GEMM library.  TEST INFRASTRUCTURE ONLY: nothing in the product path may
 * include, link, load or call this file.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg use it.  It shares no code, header,
 * table or constant with the GPU library; its dtype and layout codes are its
 * own (the Python wrapper maps names to them).
 *
 * What it computes (sources are the three pages this project is built from):
 *
 *  - The matrix fused multiply-add D = A*B + C, element by element,
 *        d_ij = sum_{l=1..k} a_il * b_lj + c_ij
 *    ("Accurate Models of AMD Matrix Cores", Section 2, Notations and
 *    Definitions, the definition of MFMA and Eq. (1)), generalised to
 *    D = alpha*sA*sB*(A*B) + beta*C (alpha/beta as in BLAS; sA/sB are the
 *    per-tensor dequantisation scales of fp8 operands).  beta == 0 means C is
 *    never read.
 *  - Input formats are decoded exactly from their bits, with the format
 *    parameters of Table 1 of the same paper (precision, smallest normal,
 *    largest finite): bfloat16, binary16, fp8 E4M3 and fp8 E5M2 in their OCP
 *    encodings, and signed 8-bit integers ("CDNA3 dense MFMA builtins",
 *    INT32-accumulate builtins: the i8 inputs are signed).
 *  - Float paths: every product a*b of two decoded inputs is exact in binary64
 *    (at most 11+11 significant bits), the k sum runs in ascending k order in
 *    binary64, and the result is rounded ONCE to binary32 (round to nearest
 *    even, the C cast).  The same loop returns S = sum_k |a_ik*b_kj| for the
 *    error bound.
 *  - Float paths may also deliver D (and read C) in bfloat16 or binary16: the
 *    exact binary64 value t is then rounded ONCE, directly to that format
 *    (round to nearest, ties to even; gradual underflow; magnitudes beyond the
 *    largest finite value become infinities), with the format parameters of
 *    Table 1 (precision 8 / 11, smallest normal 2^-126 / 2^-14, largest
 *    finite (2 - 2^-7) 2^127 / 65504).
 *  - int8 path: exact int64 accumulation, t = alpha*acc + beta*c, wrapped to
 *    int32 (mod 2^32).
 *  - binary64 path (the FP64-accumulate matrix instructions of "CDNA3 dense
 *    MFMA builtins", FP64-accumulate builtins: binary64 inputs and outputs):
 *    every product of two binary64 inputs is exact in binary128 (at most
 *    106 significant bits of its 113, and the exponent range cannot be
 *    left), the k sum runs in ascending k order in binary128, alpha*acc +
 *    beta*c is formed in binary128, and the result is rounded ONCE to
 *    binary64 (nearest even).  The binary128 sum's own error is at most
 *    (K+2) 2^-113 (|alpha| S + |beta c|), far below the binary64 bound.
 *  - 2:4 structured sparsity ("RDNA4 sparse WMMA builtins", Structured
 *    sparsity (2:4 pattern) and Common parameters, the index operand): in each
 *    contiguous group of four along K at most two values are non-zero; the
 *    compressed form keeps two values per group, in ascending position order,
 *    and a 4-bit code per group made of two 2-bit positions (p0 | p1 << 2,
 *    p0 < p1).  Codes of consecutive groups are packed LSB first, eight per
 *    32-bit word.  Groups with fewer than two non-zeros are padded with the
 *    lowest unused positions.  The sparse GEMM is "decompress, then the dense
 *    float GEMM" and is composed in the Python wrapper.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -shared -fPIC.
 * OpenMP parallelises over independent output elements only; each element's
 * sum is computed by one thread in ascending k order.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

enum { ORC_BF16 = 0, ORC_F16 = 1, ORC_I8 = 2, ORC_E4M3 = 3, ORC_E5M2 = 4 };
enum { ORC_K_CONTIG = 0, ORC_MN_CONTIG = 1 };
enum { ORC_OK = 0, ORC_BAD_ARG = -1, ORC_BAD_INDEX = -2 };
/* output (and C) formats of the float GEMM */
enum { ORC_OUT_F32 = 0, ORC_OUT_BF16 = 1, ORC_OUT_F16 = 2 };

/* ---------------------------------------------------------------- decoders */

/* bfloat16: the upper 16 bits of a binary32 (Table 1: precision 8). */
static double dec_bf16(uint16_t h) {
    uint32_t w = (uint32_t)h << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits (Table 1:
 * precision 11, smallest normal 2^-14, largest 65504). */
static double dec_f16(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                    /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);        /* (1 + m/2^10) * 2^(e-15) */
    return s ? -v : v;
}

/* fp8 E4M3, OCP encoding: 1 sign, 4 exponent (bias 7), 3 fraction bits; no
 * infinities; S.1111.111 is NaN (Table 1: precision 4, smallest normal 2^-6,
 * largest 448). */
static double dec_e4m3(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 0xf, m = c & 7;
    double v;
    if (e == 0)
        v = ldexp((double)m, -9);                     /* m/8 * 2^-6 */
    else if (e == 15 && m == 7)
        v = NAN;
    else
        v = ldexp((double)(8 + m), e - 10);           /* (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

/* fp8 E5M2, OCP encoding: 1 sign, 5 exponent (bias 15), 2 fraction bits;
 * exponent 31 holds Inf/NaN (Table 1: precision 3, smallest normal 2^-14,
 * largest 57344). */
static double dec_e5m2(uint8_t c) {
    int s = c >> 7, e = (c >> 2) & 0x1f, m = c & 3;
    double v;
    if (e == 0)
        v = ldexp((double)m, -16);                    /* m/4 * 2^-14 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(4 + m), e - 17);           /* (1 + m/4) * 2^(e-15) */
    return s ? -v : v;
}

static double dec(int dtype, const void* base, int64_t idx) {
    switch (dtype) {
    case ORC_BF16: return dec_bf16(((const uint16_t*)base)[idx]);
    case ORC_F16:  return dec_f16(((const uint16_t*)base)[idx]);
    case ORC_I8:   return (double)((const int8_t*)base)[idx];
    case ORC_E4M3: return dec_e4m3(((const uint8_t*)base)[idx]);
    case ORC_E5M2: return dec_e5m2(((const uint8_t*)base)[idx]);
    default:       return NAN;
    }
}

static int elem_bytes(int dtype) {
    return (dtype == ORC_BF16 || dtype == ORC_F16) ? 2 : 1;
}

static int valid_dtype(int d) { return d >= ORC_BF16 && d <= ORC_E5M2; }

/* ------------------------------------------------------------- rounding */

/* Round t to the binary format with p significant bits, smallest normal
 * exponent emin and largest exponent emax: the representable numbers near t
 * are the integer multiples of the quantum 2^(max(E, emin) - p + 1), where E
 * is the exponent of t's leading bit; the nearest multiple is taken, a tie
 * going to the even multiple (rint in the default rounding mode); results
 * beyond the largest finite value (2 - 2^(1-p)) 2^emax become infinities.
 * Scaling by powers of two is exact in binary64 for every t used here. */
static double round_to_format(double t, int p, int emin, int emax) {
    if (t == 0.0 || !isfinite(t)) return t;
    int ex;
    frexp(t, &ex);                       /* |t| = m 2^ex, 0.5 <= m < 1 */
    const int E = ex - 1;                /* exponent of the leading bit */
    const int q = (E > emin ? E : emin) - p + 1;
    const double r = ldexp(rint(ldexp(t, -q)), q);
    const double maxf = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
    if (fabs(r) > maxf) return r > 0 ? INFINITY : -INFINITY;
    return r;
}

static double round_out(int outfmt, double t) {
    switch (outfmt) {
    case ORC_OUT_BF16: return round_to_format(t, 8, -126, 127);
    case ORC_OUT_F16:  return round_to_format(t, 11, -14, 15);
    default:           return (double)(float)t;  /* binary32: the C cast rounds to nearest even */
    }
}

static double dec_out(int outfmt, const void* base, int64_t idx) {
    switch (outfmt) {
    case ORC_OUT_BF16: return dec_bf16(((const uint16_t*)base)[idx]);
    case ORC_OUT_F16:  return dec_f16(((const uint16_t*)base)[idx]);
    default:           return (double)((const float*)base)[idx];
    }
}

/* Element-wise rounding (exposed so that the rounding itself can be tested). */
int orc_round(int outfmt, int64_t n, const double* src, double* dst) {
    if (outfmt < ORC_OUT_F32 || outfmt > ORC_OUT_F16 || n < 0 || (n > 0 && (!src || !dst))) return ORC_BAD_ARG;
    for (int64_t i = 0; i < n; ++i) dst[i] = round_out(outfmt, src[i]);
    return ORC_OK;
}

int orc_decode(int dtype, int64_t n, const void* src, double* dst) {
    if (!valid_dtype(dtype) || n < 0 || (n > 0 && (!src || !dst))) return ORC_BAD_ARG;
    for (int64_t t = 0; t < n; ++t) dst[t] = dec(dtype, src, t);
    return ORC_OK;
}

/* ---------------------------------------------------------------- addressing
 * A is logically M x K, B is logically K x N.
 *   K-contiguous A: a(i,k) = A[i*lda + k]   (row-major A)
 *   MN-contiguous A: a(i,k) = A[k*lda + i]  (column-major A)
 *   K-contiguous B: b(k,j) = B[j*ldb + k]   (column-major B)
 *   MN-contiguous B: b(k,j) = B[k*ldb + j]  (row-major B)
 * C and D are row-major M x N with leading dimension ldc. */
static int64_t a_off(int lay, int64_t i, int64_t k, int64_t lda) {
    return lay == ORC_K_CONTIG ? i * lda + k : k * lda + i;
}
static int64_t b_off(int lay, int64_t k, int64_t j, int64_t ldb) {
    return lay == ORC_K_CONTIG ? j * ldb + k : k * ldb + j;
}

typedef struct {
    int dtA, dtB, layA, layB;
    int64_t M, N, K;
    const void* A; int64_t lda;
    const void* B; int64_t ldb;
    const void* C; int64_t ldc;
    int outfmt;
} Gemm;

static int check_gemm(const Gemm* g, int need_c) {
    if (!valid_dtype(g->dtA) || !valid_dtype(g->dtB)) return ORC_BAD_ARG;
    if ((g->layA != ORC_K_CONTIG && g->layA != ORC_MN_CONTIG) ||
        (g->layB != ORC_K_CONTIG && g->layB != ORC_MN_CONTIG)) return ORC_BAD_ARG;
    if (g->M < 0 || g->N < 0 || g->K < 0) return ORC_BAD_ARG;
    if (g->K > 0 && g->M > 0 && !g->A) return ORC_BAD_ARG;
    if (g->K > 0 && g->N > 0 && !g->B) return ORC_BAD_ARG;
    if (need_c && !g->C) return ORC_BAD_ARG;
    return ORC_OK;
}

/* One output element of the float GEMM: ascending-k binary64 sum of exact
 * products, then the alpha/beta combination, then one rounding to the output
 * format (the rounded value is exact in binary32, which carries it back). */
static void float_elem(const Gemm* g, double alpha, double beta, double sA, double sB,
                       int64_t i, int64_t j, float* d, double* s) {
    double acc = 0.0, sabs = 0.0;
    for (int64_t k = 0; k < g->K; ++k) {
        double p = dec(g->dtA, g->A, a_off(g->layA, i, k, g->lda)) *
                   dec(g->dtB, g->B, b_off(g->layB, k, j, g->ldb));
        acc += p;
        sabs += fabs(p);
    }
    double t = (alpha * sA * sB) * acc;
    if (beta != 0.0) t += beta * dec_out(g->outfmt, g->C, i * g->ldc + j);
    *d = (float)round_out(g->outfmt, t);
    *s = sabs;
}

/* One output element of the int8 GEMM: exact sum, then wrap to int32. */
static int32_t i8_elem(const Gemm* g, int64_t alpha, int64_t beta, int64_t i, int64_t j) {
    int64_t acc = 0;
    for (int64_t k = 0; k < g->K; ++k)
        acc += (int64_t)((const int8_t*)g->A)[a_off(g->layA, i, k, g->lda)] *
               (int64_t)((const int8_t*)g->B)[b_off(g->layB, k, j, g->ldb)];
    uint64_t t = (uint64_t)alpha * (uint64_t)acc;
    if (beta != 0) t += (uint64_t)beta * (uint64_t)(int64_t)((const int32_t*)g->C)[i * g->ldc + j];
    return (int32_t)(uint32_t)t;
}

/* Float GEMM over a list of output coordinates (rows[t], cols[t]).
 * d_ref[t] is the binary32 reference, abs_sum[t] = sum_k |a_ik b_kj| (of the
 * decoded codes, scales not applied). */
int orc_gemm_float_elems(int dtA, int dtB, int layA, int layB,
                         int64_t M, int64_t N, int64_t K,
                         const void* A, int64_t lda, const void* B, int64_t ldb,
                         const void* C, int64_t ldc, int outfmt,
                         double alpha, double beta, double sA, double sB,
                         int64_t n, const int64_t* rows, const int64_t* cols,
                         float* d_ref, double* abs_sum) {
    Gemm g = {dtA, dtB, layA, layB, M, N, K, A, lda, B, ldb, C, ldc, outfmt};
    if (dtA == ORC_I8 || dtB == ORC_I8) return ORC_BAD_ARG;
    if (outfmt < ORC_OUT_F32 || outfmt > ORC_OUT_F16) return ORC_BAD_ARG;
    if (check_gemm(&g, beta != 0.0) != ORC_OK || n < 0) return ORC_BAD_ARG;
    for (int64_t t = 0; t < n; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return ORC_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t t = 0; t < n; ++t)
        float_elem(&g, alpha, beta, sA, sB, rows[t], cols[t], &d_ref[t], &abs_sum[t]);
    return ORC_OK;
}

/* Float GEMM over the whole M x N output (row-major, leading dimension N). */
int orc_gemm_float_full(int dtA, int dtB, int layA, int layB,
                        int64_t M, int64_t N, int64_t K,
                        const void* A, int64_t lda, const void* B, int64_t ldb,
                        const void* C, int64_t ldc, int outfmt,
                        double alpha, double beta, double sA, double sB,
                        float* d_ref, double* abs_sum) {
    Gemm g = {dtA, dtB, layA, layB, M, N, K, A, lda, B, ldb, C, ldc, outfmt};
    if (dtA == ORC_I8 || dtB == ORC_I8) return ORC_BAD_ARG;
    if (outfmt < ORC_OUT_F32 || outfmt > ORC_OUT_F16) return ORC_BAD_ARG;
    if (check_gemm(&g, beta != 0.0) != ORC_OK) return ORC_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            float_elem(&g, alpha, beta, sA, sB, i, j, &d_ref[i * N + j], &abs_sum[i * N + j]);
    return ORC_OK;
}

/* int8 x int8 -> int32 GEMM over a list of output coordinates. */
int orc_gemm_i8_elems(int layA, int layB, int64_t M, int64_t N, int64_t K,
                      const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb,
                      const int32_t* C, int64_t ldc, int64_t alpha, int64_t beta,
                      int64_t n, const int64_t* rows, const int64_t* cols, int32_t* d_ref) {
    Gemm g = {ORC_I8, ORC_I8, layA, layB, M, N, K, A, lda, B, ldb, C, ldc, ORC_OUT_F32};
    if (check_gemm(&g, beta != 0) != ORC_OK || n < 0) return ORC_BAD_ARG;
    for (int64_t t = 0; t < n; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return ORC_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t t = 0; t < n; ++t) d_ref[t] = i8_elem(&g, alpha, beta, rows[t], cols[t]);
    return ORC_OK;
}

/* int8 x int8 -> int32 GEMM over the whole output (row-major, ld N). */
int orc_gemm_i8_full(int layA, int layB, int64_t M, int64_t N, int64_t K,
                     const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb,
                     const int32_t* C, int64_t ldc, int64_t alpha, int64_t beta, int32_t* d_ref) {
    Gemm g = {ORC_I8, ORC_I8, layA, layB, M, N, K, A, lda, B, ldb, C, ldc, ORC_OUT_F32};
    if (check_gemm(&g, beta != 0) != ORC_OK) return ORC_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) d_ref[i * N + j] = i8_elem(&g, alpha, beta, i, j);
    return ORC_OK;
}

/* ------------------------------------------------------------ binary64 GEMM */

typedef __float128 quad;

/* One output element of the binary64 GEMM: ascending-k binary128 sum of the
 * exact products, then alpha*acc + beta*c in binary128, rounded once to
 * binary64.  *s receives S = sum_k |a_ik b_kj| (rounded to binary64). */
static void f64_elem(int layA, int layB, const double* A, int64_t lda, const double* B, int64_t ldb,
                     const double* C, int64_t ldc, int64_t K, double alpha, double beta,
                     int64_t i, int64_t j, double* d, double* s) {
    quad acc = 0, sabs = 0;
    for (int64_t k = 0; k < K; ++k) {
        const double a = A[a_off(layA, i, k, lda)], b = B[b_off(layB, k, j, ldb)];
        const quad p = (quad)a * (quad)b;
        acc += p;
        sabs += (quad)fabs(a) * (quad)fabs(b);
    }
    quad t = (quad)alpha * acc;
    if (beta != 0.0) t += (quad)beta * (quad)C[i * ldc + j];
    *d = (double)t;
    *s = (double)sabs;
}

static int check_f64(int layA, int layB, int64_t M, int64_t N, int64_t K, const double* A,
                     const double* B, const double* C, double beta) {
    if ((layA != ORC_K_CONTIG && layA != ORC_MN_CONTIG) || (layB != ORC_K_CONTIG && layB != ORC_MN_CONTIG))
        return ORC_BAD_ARG;
    if (M < 0 || N < 0 || K < 0) return ORC_BAD_ARG;
    if (K > 0 && M > 0 && !A) return ORC_BAD_ARG;
    if (K > 0 && N > 0 && !B) return ORC_BAD_ARG;
    if (beta != 0.0 && !C) return ORC_BAD_ARG;
    return ORC_OK;
}

/* binary64 GEMM over a list of output coordinates (rows[t], cols[t]). */
int orc_gemm_f64_elems(int layA, int layB, int64_t M, int64_t N, int64_t K,
                       const double* A, int64_t lda, const double* B, int64_t ldb,
                       const double* C, int64_t ldc, double alpha, double beta,
                       int64_t n, const int64_t* rows, const int64_t* cols,
                       double* d_ref, double* abs_sum) {
    if (check_f64(layA, layB, M, N, K, A, B, C, beta) != ORC_OK || n < 0) return ORC_BAD_ARG;
    for (int64_t t = 0; t < n; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return ORC_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t t = 0; t < n; ++t)
        f64_elem(layA, layB, A, lda, B, ldb, C, ldc, K, alpha, beta, rows[t], cols[t], &d_ref[t], &abs_sum[t]);
    return ORC_OK;
}

/* binary64 GEMM over the whole M x N output (row-major, leading dimension N). */
int orc_gemm_f64_full(int layA, int layB, int64_t M, int64_t N, int64_t K,
                      const double* A, int64_t lda, const double* B, int64_t ldb,
                      const double* C, int64_t ldc, double alpha, double beta,
                      double* d_ref, double* abs_sum) {
    if (check_f64(layA, layB, M, N, K, A, B, C, beta) != ORC_OK) return ORC_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            f64_elem(layA, layB, A, lda, B, ldb, C, ldc, K, alpha, beta, i, j, &d_ref[i * N + j], &abs_sum[i * N + j]);
    return ORC_OK;
}

/* ------------------------------------------------------------ 2:4 sparsity */

/* Is element (row-major, element index idx) a non-zero for sparsity purposes?
 * Both signed zeros count as zero; a NaN counts as non-zero. */
static int is_nonzero(int dtype, const void* base, int64_t idx) {
    switch (dtype) {
    case ORC_BF16:
    case ORC_F16:  return (((const uint16_t*)base)[idx] & 0x7fff) != 0;
    case ORC_I8:   return ((const int8_t*)base)[idx] != 0;
    case ORC_E4M3:
    case ORC_E5M2: return (((const uint8_t*)base)[idx] & 0x7f) != 0;
    default:       return 0;
    }
}

static void copy_elem(int eb, void* dst, int64_t di, const void* src, int64_t si) {
    memcpy((char*)dst + di * eb, (const char*)src + si * eb, (size_t)eb);
}

/* Compress a row-major M x K matrix (leading dimension lda) that obeys 2:4
 * sparsity along K.  Outputs: vals, M x K/2 (leading dimension ldv), and idx,
 * M x ceil(K/32) uint32 words (leading dimension ldi).  Returns the number of
 * groups that held more than two non-zeros (those groups are written as two
 * zero values with code 0b0100, i.e. positions 0 and 1), or a negative code
 * on bad arguments. */
int64_t orc_compress24(int dtype, int64_t M, int64_t K, const void* A, int64_t lda,
                       void* vals, int64_t ldv, uint32_t* idx, int64_t ldi) {
    if (!valid_dtype(dtype) || M < 0 || K < 0 || K % 4 != 0) return ORC_BAD_ARG;
    if (lda < K || ldv < K / 2 || ldi < (K + 31) / 32) return ORC_BAD_ARG;
    if (M > 0 && K > 0 && (!A || !vals || !idx)) return ORC_BAD_ARG;
    const int eb = elem_bytes(dtype);
    const int64_t words = (K + 31) / 32;
    int64_t violations = 0;
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t w = 0; w < words; ++w) idx[i * ldi + w] = 0;
        for (int64_t g = 0; g < K / 4; ++g) {
            int pos[4], nz = 0;
            for (int p = 0; p < 4; ++p)
                if (is_nonzero(dtype, A, i * lda + 4 * g + p)) pos[nz++] = p;
            int p0, p1;
            if (nz > 2) {
                ++violations;
                memset((char*)vals + (i * ldv + 2 * g) * eb, 0, (size_t)(2 * eb));
                idx[i * ldi + g / 8] |= (uint32_t)(0 | (1 << 2)) << (4 * (g % 8));
                continue;
            }
            /* pad with the lowest positions not already selected */
            for (int p = 0; nz < 2 && p < 4; ++p) {
                int used = 0;
                for (int q = 0; q < nz; ++q) used |= (pos[q] == p);
                if (!used) pos[nz++] = p;
            }
            p0 = pos[0] < pos[1] ? pos[0] : pos[1];
            p1 = pos[0] < pos[1] ? pos[1] : pos[0];
            copy_elem(eb, vals, i * ldv + 2 * g, A, i * lda + 4 * g + p0);
            copy_elem(eb, vals, i * ldv + 2 * g + 1, A, i * lda + 4 * g + p1);
            idx[i * ldi + g / 8] |= (uint32_t)(p0 | (p1 << 2)) << (4 * (g % 8));
        }
    }
    return violations;
}

/* Expand the compressed form back to a dense row-major M x K matrix
 * (leading dimension lda): each group's two values go to positions p0 and p1
 * of its code, the other two positions become zero.  Returns ORC_BAD_INDEX if
 * a code does not name two distinct positions in ascending order. */
int orc_decompress24(int dtype, int64_t M, int64_t K, const void* vals, int64_t ldv,
                     const uint32_t* idx, int64_t ldi, void* A, int64_t lda) {
    if (!valid_dtype(dtype) || M < 0 || K < 0 || K % 4 != 0) return ORC_BAD_ARG;
    if (lda < K || ldv < K / 2 || ldi < (K + 31) / 32) return ORC_BAD_ARG;
    if (M > 0 && K > 0 && (!A || !vals || !idx)) return ORC_BAD_ARG;
    const int eb = elem_bytes(dtype);
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t g = 0; g < K / 4; ++g) {
            uint32_t code = (idx[i * ldi + g / 8] >> (4 * (g % 8))) & 0xf;
            int p0 = code & 3, p1 = code >> 2;
            if (p0 >= p1) return ORC_BAD_INDEX;
            memset((char*)A + (i * lda + 4 * g) * eb, 0, (size_t)(4 * eb));
            copy_elem(eb, A, i * lda + 4 * g + p0, vals, i * ldv + 2 * g);
            copy_elem(eb, A, i * lda + 4 * g + p1, vals, i * ldv + 2 * g + 1);
        }
    }
    return ORC_OK;
}

/* Number of OpenMP threads a parallel region of this library uses. */
int orc_max_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the number of OpenMP threads later parallel regions use (n >= 1); the
   CPU baseline times the oracle single-threaded with it.  No arithmetic. */
void orc_set_threads(int n) {
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
