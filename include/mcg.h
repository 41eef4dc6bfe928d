/*
 * mcg.h -- C ABI of the MI355X (gfx950, CDNA4) matrix-core GEMM library.
 *
 * The library multiplies matrices with the wavefront-level matrix fused
 * multiply-add instructions (MFMA, and the 2:4-sparse SMFMAC) of gfx950:
 *
 *     D = alpha * scaleA * scaleB * (A . B) + beta * C
 *
 * The operation is the matrix fused multiply-add D = A B + C of "Accurate
 * Models of AMD Matrix Cores" (Section 2, Notations and Definitions, Eq. (1)),
 * with BLAS-style alpha/beta and per-tensor fp8 dequantisation scales.  One
 * MFMA instruction computes one K-step of a small tile; the library tiles and
 * loops over K ("CDNA3 dense MFMA builtins", Naming convention; Using MFMA
 * builtins as a compute policy).  The sparse variant takes A in the 2:4
 * compressed form of "RDNA4 sparse WMMA builtins" (Structured sparsity (2:4
 * pattern); Common parameters, index), with the compressed values and the
 * index stored separately (Using sparse WMMA builtins as a compute policy).
 *
 * Conventions common to every entry point
 *  - Pointers named A, B, C, D, A_compressed, A_index, d_violations are
 *    DEVICE pointers (gfx950 global memory) owned by the caller.  The library
 *    keeps no state, allocates no device memory and never frees caller memory.
 *  - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL is
 *    the null stream) and return as soon as the work is enqueued.
 *  - Leading dimensions are in ELEMENTS.  Sizes are int64.
 *  - Return value: 0 (MCG_SUCCESS) or a positive mcg_status.  Argument errors
 *    are found on the host before anything is launched; then nothing is read
 *    or written.  The library never aborts and never throws.
 *  - Only gfx950 devices are supported (MCG_ERR_UNSUPPORTED_ARCH otherwise).
 *  - Thread-safe: no global mutable state beyond a per-device arch check.
 */
#ifndef MCG_H
#define MCG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  Float formats are decoded as in "Accurate Models of AMD
 * Matrix Cores", Table 1: bfloat16, binary16, fp8 E4M3 and fp8 E5M2 in their
 * OCP encodings (E4M3: bias 7, no infinities, largest 448; E5M2: bias 15,
 * largest 57344).  MCG_I8 is signed ("CDNA3 dense MFMA builtins",
 * INT32-accumulate builtins).  MCG_F64 is IEEE binary64, the operand and
 * accumulator format of the FP64-accumulate builtins of the same page. */
typedef enum {
    MCG_BF16 = 0,
    MCG_F16 = 1,
    MCG_I8 = 2,
    MCG_FP8_E4M3 = 3,
    MCG_FP8_E5M2 = 4,
    MCG_F32 = 5,
    MCG_I32 = 6,
    MCG_F64 = 7
} mcg_dtype;

/* Storage order of the operands.  A is logically M x K, B is K x N.
 *   MCG_K_CONTIG : A row-major    (A[i*lda + k], lda >= K)
 *                  B column-major (B[j*ldb + k], ldb >= K)
 *   MCG_MN_CONTIG: A column-major (A[k*lda + i], lda >= M)
 *                  B row-major    (B[k*ldb + j], ldb >= N)
 * C and D are always row-major M x N (C[i*ldc + j], ldc >= N). */
typedef enum {
    MCG_K_CONTIG = 0,
    MCG_MN_CONTIG = 1
} mcg_layout;

typedef enum {
    MCG_SUCCESS = 0,
    MCG_ERR_NULL_POINTER = 1,      /* a required pointer is NULL                     */
    MCG_ERR_INVALID_SIZE = 2,      /* negative size, or K % 4 != 0 for 2:4           */
    MCG_ERR_INVALID_LD = 3,        /* a leading dimension below its minimum          */
    MCG_ERR_UNSUPPORTED_DTYPE = 4, /* dtype/layout combination not provided          */
    MCG_ERR_MISALIGNED = 5,        /* pointer/ld alignment the entry point requires  */
    MCG_ERR_NOT_2_4_SPARSE = 6,    /* a group of four holds more than two non-zeros  */
    MCG_ERR_INVALID_INDEX = 7,     /* a 2:4 index code with p0 >= p1 (decompress24_host) */
    MCG_ERR_UNSUPPORTED_ARCH = 8,  /* current device is not gfx950                   */
    MCG_ERR_HIP = 9,               /* a HIP runtime call failed                      */
    MCG_ERR_INVALID_VALUE = 10,    /* alpha/beta/scale not usable for this dtype     */
    MCG_ERR_SCRATCH_LIMIT = 11     /* gemm_dense_noalloc: plan needs more scratch    */
} mcg_status;

/*
 * gemm_dense -- D = alpha*scaleA*scaleB*(A.B) + beta*C on MFMA.
 *
 * dtypeA/dtypeB : supported pairs are BF16xBF16, F16xF16, I8xI8, F64xF64 and
 *                 any pair of FP8_E4M3/FP8_E5M2.
 * layoutA/B     : mcg_layout (all four combinations for every pair).
 * M, N, K       : any sizes >= 0.  M == 0 or N == 0 is a no-op.  K == 0 gives
 *                 D = beta*C.  Ragged edges are handled inside the kernels.
 * A, lda        : logical M x K in layoutA; lda >= K (K_CONTIG) or >= M.
 * B, ldb        : logical K x N in layoutB; ldb >= K (K_CONTIG) or >= N.
 * C             : row-major M x N of dtypeD, read only when beta != 0 (may be
 *                 NULL then).  D: row-major M x N of dtypeD; D may alias C
 *                 exactly (same pointer); other overlaps are undefined.
 * ldc           : leading dimension of both C and D, ldc >= N.
 * dtypeD        : format of C and D.  Float inputs: MCG_F32, MCG_BF16 or
 *                 MCG_F16 (fp32 accumulation; a bfloat16/binary16 D is the
 *                 fp32 result rounded once to nearest-even, C is read in the
 *                 same format).  int8: MCG_I32 (exact int32 accumulation,
 *                 wrapping mod 2^32).  F64: MCG_F64 (binary64 accumulation on
 *                 the FP64 matrix instructions, alpha and beta used as
 *                 binary64).
 * alpha, beta   : float paths use them as fp32: MCG_ERR_INVALID_VALUE when
 *                 alpha*scaleA*scaleB or beta is not finite once rounded to
 *                 fp32 (e.g. 1e39).  The int8 path requires
 *                 integral values in int32 range and computes
 *                 alpha*acc + beta*C in wrapping int32 arithmetic.
 * scaleA/scaleB : per-tensor dequantisation scales of fp8 operands (real
 *                 value = scale * decoded code), folded into the epilogue as
 *                 fp32 alpha*scaleA*scaleB.  Must be 1.0f for non-fp8 inputs.
 * stream        : hipStream_t or NULL.
 * Accuracy      : float results are the fp32 result of a non-IEEE matrix-core
 *                 accumulation, not bit-reproducible across architectures
 *                 ("Accurate Models of AMD Matrix Cores", Abstract); int8
 *                 results are exact.  Every float result stays within
 *                 4*2^-24*(K+2)*|alpha*scaleA*scaleB|*sum|a*b| + 2^-24*|D| of
 *                 the exact value (plus the output rounding for 16-bit D).
 *                 The native fp8 instructions keep only about 13 bits below
 *                 the largest product of each group they sum (measured), which
 *                 fits that bound from K = 6144 on; below it fp8 operands are
 *                 widened exactly to bfloat16 and multiplied on the bfloat16
 *                 instructions.  Binary64 results stay within
 *                 4*2^-53*(K+2)*|alpha|*sum|a*b| + 2^-53*|D| of the exact value
 *                 (plus 2^-53*|beta*c| when beta is not 0 or +-1); unless K is
 *                 split they are deterministic: the FP64 instructions are
 *                 chains of correctly rounded binary64 fused multiply-adds
 *                 (measured), applied in a fixed K order.
 * Alignment     : none beyond the element size (binary64 operands take the
 *                 same path at any leading dimension); 16-byte aligned
 *                 pointers and leading
 *                 dimensions whose byte size is a multiple of 16 take the
 *                 vector-load path, anything else a slower element path.
 * Split K       : problems with too few output tiles to fill the device
 *                 (e.g. N <= 32, M <= 32, or a long K over a small D) may cut
 *                 K into ranges run by separate workgroups when D is MCG_F32,
 *                 MCG_I32 or MCG_F64 and is not C with beta != 0.  D is then zeroed,
 *                 receives the partial sums through device-scope atomic adds
 *                 and is finally set to alpha*D + beta*C, so D must be
 *                 ordinary device memory.  Float results of a split problem
 *                 may differ in the last bits between runs (the order of the
 *                 additions is not fixed); int32 results are exact.
 *                 mcg_dense_splits reports the split a call would use.
 */
int gemm_dense(int dtypeA, int dtypeB, int layoutA, int layoutB,
               int64_t M, int64_t N, int64_t K,
               const void* A, int64_t lda, const void* B, int64_t ldb,
               const void* C, void* D, int64_t ldc, int dtypeD,
               double alpha, double beta, float scaleA, float scaleB, void* stream);

/*
 * gemm_dense_ws -- gemm_dense with a caller-provided device workspace.
 *
 * Computes exactly what gemm_dense computes (the matrix fused multiply-add of
 * "Accurate Models of AMD Matrix Cores", Section 2, Eq. (1)), with the same
 * arguments, validation, accuracy bound and errors.  The workspace lets problems
 * on the pipelined kernel (256 x 256 tiles, or its 128 x 128 form for mid-size
 * problems) whose tile count leaves the device's last round of tiles partly
 * idle run in stream-K form: the whole rounds as usual, and the K
 * iterations of the remaining tiles spread evenly over all compute units, each
 * piece of a tile leaving its partial sums in the workspace, from which a
 * second kernel adds them in a fixed order (K ascending) and applies the
 * epilogue.  Results stay deterministic.  A problem on the 128 x 128 form
 * whose tiles cannot be cut that way although its last round leaves compute
 * units idle takes the 256 x 256 split instead when K is long (at least 256 K
 * tiles of 128 bytes: 16384 16-bit or 32768 8-bit values), and an aligned
 * problem of at least 128 x 128 with so few tiles and so long a K that
 * gemm_dense runs it on the general kernel takes the 128 x 128 form's split
 * when it has one.  This decomposition is not from the pages; it is a
 * scheduling choice of this library.
 *
 * workspace       : device memory owned by the caller, 16-byte aligned, or
 *                   NULL.  The call may use its first
 *                   mcg_dense_workspace_bytes(...) bytes as scratch; their
 *                   contents on entry do not matter and are unspecified after
 *                   the call.  Calls that share a workspace must not overlap
 *                   (same stream, or synchronised).
 * workspace_bytes : its size.  When the workspace is NULL or smaller than the
 *                   plan needs, the call runs exactly as gemm_dense.
 * Errors          : those of gemm_dense; MCG_ERR_MISALIGNED for a workspace
 *                   that is not 16-byte aligned, MCG_ERR_INVALID_SIZE for a
 *                   negative workspace_bytes.
 */
int gemm_dense_ws(int dtypeA, int dtypeB, int layoutA, int layoutB,
                  int64_t M, int64_t N, int64_t K,
                  const void* A, int64_t lda, const void* B, int64_t ldb,
                  const void* C, void* D, int64_t ldc, int dtypeD,
                  double alpha, double beta, float scaleA, float scaleB,
                  void* workspace, int64_t workspace_bytes, void* stream);

/*
 * gemm_dense_noalloc -- gemm_dense_ws for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the stream-K slots come from a static device array inside
 * the library, mcg_dense_noalloc_scratch_bytes() (32 MiB) per GPU, held until
 * the process ends.  The call allocates nothing and frees nothing.
 *
 * Arguments, results and errors are those of gemm_dense_ws with a workspace
 * of that size, except that a problem whose stream-K plan needs more than the
 * static array (mcg_dense_workspace_bytes > mcg_dense_noalloc_scratch_bytes)
 * returns MCG_ERR_SCRATCH_LIMIT before anything is launched or written;
 * problems without a stream-K plan run as gemm_dense.  The long-K 256 x 256
 * split of a 128 x 128 problem and the 128 x 128 split of a general-kernel
 * problem (see gemm_dense_ws) are optional: each is taken only when it fits
 * the array, and otherwise the problem runs as gemm_dense.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams, other
 * host threads) race and must be ordered by the caller.
 */
int gemm_dense_noalloc(int dtypeA, int dtypeB, int layoutA, int layoutB,
                       int64_t M, int64_t N, int64_t K,
                       const void* A, int64_t lda, const void* B, int64_t ldb,
                       const void* C, void* D, int64_t ldc, int dtypeD,
                       double alpha, double beta, float scaleA, float scaleB, void* stream);
int64_t mcg_dense_noalloc_scratch_bytes(void);

/* mcg_dense_workspace_bytes -- bytes of workspace gemm_dense_ws uses for these
 * operands (host-only, no device work): one binary32 tile per piece of a
 * remainder tile (256 KiB with 256 x 256 tiles, 64 KiB with 128 x 128 ones),
 * or 0 when the problem does not take the stream-K form (another kernel, a
 * tile count that fills the device's rounds, or too little to gain).  Reads the
 * current device's compute-unit count (256 when there is no device). */
int64_t mcg_dense_workspace_bytes(int dtypeA, int layoutA, int layoutB, int64_t M, int64_t N, int64_t K,
                                  const void* A, int64_t lda, const void* B, int64_t ldb);

/*
 * gemm_sparse24 -- D = alpha*(A.B) + beta*C with A given in 2:4 compressed
 * form and multiplied on the sparse matrix cores (SMFMAC).
 *
 * dtypeA/dtypeB : MCG_BF16 x MCG_BF16, MCG_F16 x MCG_F16 (dtypeD MCG_F32,
 *                 MCG_BF16 or MCG_F16), any pair of MCG_FP8_E4M3 / MCG_FP8_E5M2
 *                 (same outputs; per-tensor dequantisation scales are folded
 *                 into alpha by the caller), or MCG_I8 x MCG_I8 (dtypeD
 *                 MCG_I32, integral alpha/beta, exact wrapping int32 as for
 *                 gemm_dense).  fp8 with K below 6144 is widened exactly to
 *                 bfloat16 and multiplied on the bfloat16 sparse instruction
 *                 (see Accuracy at gemm_dense).
 * layoutB       : mcg_layout of B (A is always the compressed row-major form).
 * K             : the DENSE K; K % 4 == 0.
 * A_compressed  : M x K/2 values, row-major, lda_c >= K/2.  Row i holds, for
 *                 each group g of four along K, the two kept values of that
 *                 group in ascending position order.
 * A_index       : M x ceil(K/32) uint32 words, row-major, ld_idx >=
 *                 ceil(K/32).  Group g of row i has the 4-bit code
 *                 p0 | (p1 << 2) (positions 0..3 of its two kept values,
 *                 p0 < p1) at bits 4*(g % 8) of word g/8; unused trailing
 *                 codes are zero.  This is the canonical layout produced by
 *                 compress24 / compress24_host; kernels re-pack it per lane.
 *                 The codes are not checked here (checking them would cost a
 *                 pass over the index on every call): a code with p0 >= p1
 *                 gives unspecified values in the outputs of its rows, but
 *                 every memory access stays inside the arguments' extents.
 *                 decompress24_host checks every code.
 * B, ldb, C, D, ldc, alpha, beta, stream: as for gemm_dense.
 */
int gemm_sparse24(int dtypeA, int dtypeB, int layoutB, int64_t M, int64_t N, int64_t K,
                  const void* A_compressed, int64_t lda_c,
                  const uint32_t* A_index, int64_t ld_idx,
                  const void* B, int64_t ldb, const void* C, void* D, int64_t ldc,
                  int dtypeD, double alpha, double beta, void* stream);

/*
 * gemm_sparse24_ws -- gemm_sparse24 with a caller-provided device workspace.
 *
 * Computes exactly what gemm_sparse24 computes (the 2:4 compressed form of
 * "RDNA4 sparse WMMA builtins", Structured sparsity (2:4 pattern), multiplied as
 * in "Accurate Models of AMD Matrix Cores", Section 2, Eq. (1)), with the same
 * arguments, validation, accuracy bound and errors.  Problems on the 256 x 256
 * sparse kernel whose tile count leaves the device's last round of tiles partly
 * idle run in stream-K form, as gemm_dense_ws does: the remainder tiles' K range
 * is cut into equal pieces over all compute units, each piece leaves its partial
 * sums in the workspace, and a second kernel adds them in K order and applies
 * the epilogue (deterministic).  A scheduling choice of this library, not of the
 * pages.
 * workspace, workspace_bytes : as for gemm_dense_ws (16-byte aligned device
 *                 memory, contents irrelevant on entry and unspecified after;
 *                 NULL or too small: the call runs as gemm_sparse24).
 *                 mcg_sparse24_workspace_bytes reports the plan's size: 256 KiB
 *                 per piece, 0 without a stream-K plan.
 */
int gemm_sparse24_ws(int dtypeA, int dtypeB, int layoutB, int64_t M, int64_t N, int64_t K,
                     const void* A_compressed, int64_t lda_c, const uint32_t* A_index, int64_t ld_idx,
                     const void* B, int64_t ldb, const void* C, void* D, int64_t ldc, int dtypeD,
                     double alpha, double beta, void* workspace, int64_t workspace_bytes, void* stream);
int64_t mcg_sparse24_workspace_bytes(int dtypeA, int layoutB, int64_t M, int64_t N, int64_t K,
                                     const void* A_compressed, int64_t lda_c, const uint32_t* A_index,
                                     int64_t ld_idx, const void* B, int64_t ldb);

/*
 * compress24 -- 2:4 compressor on the device ("RDNA4 sparse WMMA builtins",
 * Structured sparsity (2:4 pattern): walk K in groups of four and keep the
 * two non-zero positions).
 *
 * dtype         : MCG_BF16, MCG_F16, MCG_I8, MCG_FP8_E4M3 or MCG_FP8_E5M2.
 * A, lda        : dense row-major M x K, lda >= K, K % 4 == 0.
 * A_compressed, lda_c, A_index, ld_idx: outputs in the layout described at
 *                 gemm_sparse24.  A group with fewer than two non-zeros keeps
 *                 the lowest unused positions; +0 and -0 count as zero and NaN
 *                 as non-zero.  A group with more than two non-zeros is
 *                 written as two zeros with code p0=0, p1=1.
 * d_violations  : optional device int32; if not NULL it is set to the number
 *                 of groups with more than two non-zeros (the library zeroes
 *                 it first, in stream order).
 */
int compress24(int dtype, int64_t M, int64_t K, const void* A, int64_t lda,
               void* A_compressed, int64_t lda_c, uint32_t* A_index, int64_t ld_idx,
               int32_t* d_violations, void* stream);

/*
 * compress24_host -- the same compressor for HOST pointers, synchronous, for
 * preparing weights offline.  Returns MCG_ERR_NOT_2_4_SPARSE if any group
 * held more than two non-zeros (outputs are still fully written).
 */
int compress24_host(int dtype, int64_t M, int64_t K, const void* A, int64_t lda,
                    void* A_compressed, int64_t lda_c, uint32_t* A_index, int64_t ld_idx);

/*
 * decompress24_host -- the inverse of compress24_host ("RDNA4 sparse WMMA
 * builtins", Structured sparsity (2:4 pattern): each group of four along K
 * holds its two kept values at the two positions its index bits name, and
 * zeros elsewhere; Common parameters, index: two bits per kept value).
 *
 * Pointers are HOST pointers; the call is synchronous and touches no device.
 * dtype         : MCG_BF16, MCG_F16, MCG_I8, MCG_FP8_E4M3 or MCG_FP8_E5M2.
 * A_compressed, lda_c, A_index, ld_idx: the compressed form described at
 *                 gemm_sparse24 (M x K/2 values, M x ceil(K/32) index words).
 * A, lda        : output, dense row-major M x K, lda >= K; for every group
 *                 the four elements are written (the kept values at p0 and
 *                 p1, zero bits at the other two positions).
 * Errors        : MCG_ERR_INVALID_INDEX if any used group's code has
 *                 p0 >= p1 (codes of groups past K/4 in a row's last word are
 *                 ignored); all codes are checked first, so on this error
 *                 nothing is written.  Argument errors as for compress24_host.
 */
int decompress24_host(int dtype, int64_t M, int64_t K, const void* A_compressed, int64_t lda_c,
                      const uint32_t* A_index, int64_t ld_idx, void* A, int64_t lda);

/* Host-only argument checks: the exact validation the entry points above run
 * before touching the device (same arguments, minus outputs' contents and the
 * stream).  They never call HIP and return an mcg_status. */
int mcg_validate_dense(int dtypeA, int dtypeB, int layoutA, int layoutB, int64_t M, int64_t N,
                       int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                       const void* C, const void* D, int64_t ldc, int dtypeD, double alpha,
                       double beta, float scaleA, float scaleB);
int mcg_validate_sparse24(int dtypeA, int dtypeB, int layoutB, int64_t M, int64_t N, int64_t K,
                          const void* A_compressed, int64_t lda_c, const uint32_t* A_index,
                          int64_t ld_idx, const void* B, int64_t ldb, const void* C, const void* D,
                          int64_t ldc, int dtypeD, double alpha, double beta);
int mcg_validate_compress24(int dtype, int64_t M, int64_t K, const void* A, int64_t lda,
                            const void* A_compressed, int64_t lda_c, const uint32_t* A_index,
                            int64_t ld_idx);

/* Kernel selection, for callers that tune shapes and for tests.  Host-only,
   no validation, no device memory access; the cost model uses the current
   device's compute-unit count (256, an MI355X's, when no device is visible).
   mcg_dense_path: the kernel gemm_dense runs for these operands with a
     binary32/int32 D that is not C: 0 general kernel, 128 x 128 tiles (any
     shape, alignment or leading dimension); 1 the 256 x 256 pipelined kernel;
     2 general kernel with 128 x 32 tiles (N <= 32, aligned operands, the
     M x K operand MN-contiguous with M < 2048, or operand windows of 2 GiB);
     3 general kernel with 32 x 128 tiles (M <= 32, likewise for B and N);
     4 the streaming kernel (N <= 32 or M <= 32, aligned operands in any
     storage order, otherwise); 5 the binary64 kernel (dtypeA MCG_F64, any shape); 6 the
     pipelined kernel with 128 x 128 tiles (aligned operands, M and N >= 128,
     too few 256 x 256 tiles to fill the chip, faster than kernel 0 by the
     planner's cost model).
   mcg_dense_splits: the number of K ranges (1 = no split) gemm_dense uses
     with exactly these arguments.
   mcg_sparse24_path: 1 if gemm_sparse24 runs the 256 x 256 pipelined kernel,
     0 for the general one. */
int mcg_dense_path(int dtypeA, int layoutA, int layoutB, int64_t M, int64_t N, int64_t K, const void* A,
                   int64_t lda, const void* B, int64_t ldb);
int mcg_dense_splits(int dtypeA, int layoutA, int layoutB, int64_t M, int64_t N, int64_t K, const void* A,
                     int64_t lda, const void* B, int64_t ldb, const void* C, const void* D, int dtypeD,
                     double beta);
int mcg_sparse24_path(int dtypeA, int layoutB, int64_t M, int64_t N, int64_t K, const void* A_compressed,
                      int64_t lda_c, const uint32_t* A_index, int64_t ld_idx, const void* B, int64_t ldb);

/*
 * mcg_mfma_eval -- one gfx950 matrix-core instruction per test vector, for
 * numerical characterisation ("Accurate Models of AMD Matrix Cores", Section 2,
 * Eq. (1): d = sum_l a_l b_l + c for one output element; Section 3: targeted
 * and randomised test vectors).
 *
 * dtype  : MCG_BF16, MCG_F16, MCG_FP8_E4M3 or MCG_FP8_E5M2 (a and b alike),
 *          or MCG_F64 (the FP64-accumulate builtins of "CDNA3 dense MFMA
 *          builtins").
 * shape  : 16 (mfma_f32_16x16x32_{bf16,f16}, mfma_scale_f32_16x16x128_f8f6f4,
 *          mfma_f64_16x16x4f64) or 32 (mfma_f32_32x32x16_{bf16,f16},
 *          mfma_scale_f32_32x32x64_f8f6f4); for MCG_F64 also 4 (block 0 of
 *          mfma_f64_4x4x4f64).
 * a, b   : DEVICE arrays of n * k element codes, k = mcg_mfma_eval_k(dtype,
 *          shape); test vector t is a[t*k .. t*k + k) and b[t*k .. t*k + k).
 *          Element l goes to operand slot l: lane group g holds slots
 *          [g*E, (g+1)*E) in register order (E = 8 for 16-bit, 32 for fp8
 *          elements per lane; for MCG_F64 slot l is the K index l, k = 4).
 * c, d   : DEVICE arrays of n accumulator elements (float; double for
 *          MCG_F64): c[t] is accumulator element (0, 0) of test t, d[t]
 *          receives result element (0, 0).  All other operand elements are
 *          zero.
 * Returns an mcg_status; asynchronous on stream.
 */
int mcg_mfma_eval(int dtype, int shape, int64_t n, const void* a, const void* b, const void* c, void* d,
                  void* stream);
/* Elements per test vector for mcg_mfma_eval (0 if unsupported). */
int mcg_mfma_eval_k(int dtype, int shape);

/*
 * mcg_mfma_probe -- sustained matrix-core rate on given operand bits (a
 * measurement aid for the GEMM roofline; computes no GEMM).
 *
 * The published peak of an instruction ("CDNA3 dense MFMA builtins",
 * Instruction throughput: operations per instruction x instructions per cycle
 * x CUs x clock) assumes the peak clock; under full matrix-core load the
 * gfx950 clock depends on the operand bits.  The probe runs the instructions
 * of the GEMM kernels (mfma 32x32x16 bf16/f16, 32x32x32 i8, 32x32x64 fp8; for
 * 2:4 the smfmac of "RDNA4 sparse WMMA builtins", Structured sparsity) in their
 * arrangement -- num_wg workgroups of 8 wavefronts, one per CU, two wavefronts
 * per SIMD alternating between workgroup barriers, 16 instructions per
 * wavefront and phase on a 4 x 2 grid of 32 x 32 accumulators -- on fragments
 * loaded once, with no other memory traffic.  Its rate bounds what any data
 * movement schedule can reach with those operand bits.
 *
 * dtypeA/B        : as for gemm_dense (sparse == 0: BF16xBF16, F16xF16,
 *                   I8xI8, any FP8 pair) or gemm_sparse24 (sparse == 1).
 * a, b            : DEVICE operand bytes (for 2:4: kept values and dense B),
 *                   16-byte aligned, at least 65536 readable bytes each; lane
 *                   l of wavefront w of workgroup g takes its fragments from
 *                   the 128 bytes at ((4096 g) mod 32768) + 64 (64 w + l).
 * idx             : DEVICE 2:4 index words (sparse == 1 only; 16-byte
 *                   aligned, 65536 readable bytes), else ignored.
 * instr_per_wave  : matrix instructions per wavefront, a positive multiple of
 *                   16, at most 2^24.
 * num_wg          : workgroups (the CU count fills the chip once), 1..65536.
 * sink            : DEVICE float[num_wg * 512], receives each thread's sum of
 *                   its accumulators (keeps the work live; with every operand
 *                   byte of the 16-bit kinds equal to bf16/f16 1.0 it is
 *                   256 * instr_per_wave exactly).
 * clocks          : DEVICE int64[2 * num_wg]: per workgroup, shader-clock
 *                   cycles and 100 MHz reference ticks between its first and
 *                   last matrix phase (s_memtime, s_memrealtime).
 * Errors: MCG_ERR_UNSUPPORTED_DTYPE, MCG_ERR_INVALID_SIZE, MCG_ERR_NULL_POINTER,
 * MCG_ERR_MISALIGNED, MCG_ERR_UNSUPPORTED_ARCH, MCG_ERR_HIP.  Asynchronous on
 * stream; the caller times it (one launch).
 */
int mcg_mfma_probe(int dtypeA, int dtypeB, int sparse, const void* a, const void* b, const void* idx,
                   int64_t instr_per_wave, int num_wg, float* sink, int64_t* clocks, void* stream);

/* Human-readable name of an mcg_status value (static storage). */
const char* mcg_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int mcg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MCG_H */
