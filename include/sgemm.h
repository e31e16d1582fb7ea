/*
 * sgemm.h -- C ABI of the MI355X (gfx950) FP32 matrix multiply.
 *
 * Operation ("Shared Memory Tiling for Matrix Multiplication", opening
 * definition; "Matrix Multiplication -- Naive to Tiled", section 02):
 *
 *     C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j],   0 <= i < M, 0 <= j < N
 *
 * A is M x K, B is K x N, C is M x N, all float32 and row-major: element
 * (r, c) of a matrix with leading dimension ld lives at ptr[r * ld + c]
 * ("Matrix Multiplication -- Naive to Tiled", section 02 indexes A[row*K+i],
 * B[i*N+col], C[row*N+col]; leading dimensions generalise the row length as
 * the BLAS call of section 07 does). C is overwritten: its old contents are
 * never read (section 07's vendor call with alpha = 1, beta = 0; every kernel
 * on the pages stores with '='). Elements of C's rows beyond column N-1 (the
 * padding up to ldc) are never touched.
 *
 * Products are formed and summed in float32 (fused multiply-add, round to
 * nearest even). The summation order is the kernel's own; the result is within
 * 1e-5 * sum_k |A[i][k]| * |B[k][j]| + 1e-6 of the exact sum, and exact when
 * every partial sum is an integer below 2^24 (small-integer inputs).
 *
 * All matrix pointers are DEVICE pointers on the calling thread's current HIP
 * device. The caller owns every buffer; the library allocates nothing per
 * call (sgemm_ex_ws works in scratch memory the caller passes), keeps no
 * pointer after returning and has no mutable global state besides a
 * per-device cache of the device's architecture, so calls from several host
 * threads are safe. The one exception is sgemm_ex_noalloc, which works in a
 * static device buffer of the library's own (see there).
 */
#ifndef SGEMM_H
#define SGEMM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. Every entry point returns one; none ever exits the process
 * (unlike the pages' error macro, which prints and calls exit()). */
typedef enum sgemm_status {
    SGEMM_OK = 0,
    SGEMM_ERR_DIM = -1,      /* M, N or K negative                              */
    SGEMM_ERR_LD = -2,       /* lda < max(1,K), ldb < max(1,N) or ldc < max(1,N) */
    SGEMM_ERR_NULL = -3,     /* NULL matrix pointer with a non-empty extent      */
    SGEMM_ERR_VARIANT = -4,  /* unknown variant code                             */
    SGEMM_ERR_LAUNCH = -5,   /* the HIP launch itself failed (hipGetLastError)   */
    SGEMM_ERR_DEVICE = -6,   /* no usable HIP device, or it is not gfx950        */
    SGEMM_ERR_ALIAS = -7,    /* C's extent overlaps A's or B's                   */
    SGEMM_ERR_OP = -8,       /* transpose flag not SGEMM_OP_N or SGEMM_OP_T      */
    SGEMM_ERR_DTYPE = -9,    /* 16-bit type not SGEMM_LP_BF16 or SGEMM_LP_F16    */
    SGEMM_ERR_SCRATCH = -10  /* sgemm_ex_noalloc: the product needs more scratch
                                than the library's static buffer holds          */
} sgemm_status;

/* 16-bit operand types of sgemm_lp. */
typedef enum sgemm_lp_type {
    SGEMM_LP_BF16 = 1,  /* bfloat16: the upper 16 bits of an IEEE binary32     */
    SGEMM_LP_F16 = 2    /* IEEE 754 binary16                                   */
} sgemm_lp_type;

/* Transpose flags of sgemm_ex: how an operand is stored. */
typedef enum sgemm_op {
    SGEMM_OP_N = 0,  /* as is: op(X) = X                   */
    SGEMM_OP_T = 1   /* transposed: op(X) = X^T            */
} sgemm_op;

/* Kernel variants: the ladder from the pages' naive kernel to matrix cores.
 *  NAIVE    one work-item per element of C, operands straight from global
 *           memory ("Matrix Multiplication -- Naive to Tiled", section 02).
 *  TILED    T x T tiles of A and B staged in LDS, zero-filled at the edges,
 *           two barriers per K step (same page, sections 04-05), with the
 *           tile size T chosen per shape from 8, 16 and 32 (same page,
 *           exercise 2; "Naive GEMM vs Tiled GEMM", the kernel with 32 x 32
 *           tiles). TILED_T8, TILED_T16 and TILED_T32 fix T.
 *  REGBLOCK 128 x 128 LDS tiles, an 8 x 8 block of C per work-item in
 *           registers, 128-bit global loads, double-buffered LDS (same page,
 *           section 07; "From 306 ms to 86 ms", "Register blocking"); 64 x 64
 *           (4 x 4), 32 x 32 (2 x 2) or 16 x 16 (1 x 1) tiles for products
 *           with too few 128 x 128 tiles to occupy the device
 *           (sgemm_regblock_tile).
 *  MFMA     the same tiling fed to the CDNA matrix cores with
 *           v_mfma_f32_32x32x2_f32 (FP32 in, FP32 accumulate), with the tile
 *           shape chosen per product (sgemm_mfma_tile, sgemm_mfma_shape).
 *  BEST     whichever variant is fastest for the shape (currently MFMA). */
typedef enum sgemm_variant {
    SGEMM_BEST = -1,
    SGEMM_NAIVE = 0,
    SGEMM_TILED = 1,
    SGEMM_REGBLOCK = 2,
    SGEMM_MFMA = 3,
    SGEMM_TILED_T8 = 4,
    SGEMM_TILED_T16 = 5,
    SGEMM_TILED_T32 = 6
} sgemm_variant;

/*
 * C = A * B on `stream` (a hipStream_t of the current device; NULL means the
 * null stream).
 *
 * Arguments
 *   M, N, K        sizes; each >= 0.
 *   A, lda         M x K operand, lda >= max(1, K).
 *   B, ldb         K x N operand, ldb >= max(1, N).
 *   C, ldc         M x N result, ldc >= max(1, N); overwritten.
 *   stream         queue to launch on; the call returns without waiting.
 *   variant        an sgemm_variant code.
 *
 * Behaviour
 *   - Arguments are checked on the host, in this order, before any HIP call:
 *     sizes, leading dimensions, variant, then (only if M > 0 and N > 0)
 *     NULL pointers and overlap of C with A or B.
 *   - M == 0 or N == 0: nothing to do; returns SGEMM_OK without touching the
 *     GPU (pointers may then be NULL).
 *   - K == 0: the sum is empty, so the M x N window of C is set to 0
 *     (A and B are not read and may be NULL).
 *   - Otherwise one kernel is enqueued. Errors a kernel meets while running
 *     (a fault from a bad pointer, say) are not seen here; they surface at the
 *     caller's next synchronisation, as for any asynchronous HIP launch.
 *   - C must not overlap A or B (checked: SGEMM_ERR_ALIAS).
 *
 * Returns SGEMM_OK or a negative sgemm_status.
 */
int sgemm(int M, int N, int K,
          const float *A, int lda,
          const float *B, int ldb,
          float *C, int ldc,
          void *stream, int variant);

/*
 * The general form of the vendor call on "Matrix Multiplication -- Naive to
 * Tiled", section 07 (which uses alpha = 1, beta = 0 and no transposes):
 *
 *     C = alpha * op(A) * op(B) + beta * C
 *
 * with op(A) of M x K, op(B) of K x N and C of M x N, all row-major float32
 * on `stream` (as for sgemm).
 *
 * Arguments
 *   transA         SGEMM_OP_N: A is stored M x K, lda >= max(1, K);
 *                  SGEMM_OP_T: A is stored K x M (op(A) = A^T), lda >= max(1, M).
 *   transB         SGEMM_OP_N: B is stored K x N, ldb >= max(1, N);
 *                  SGEMM_OP_T: B is stored N x K (op(B) = B^T), ldb >= max(1, K).
 *   M, N, K        sizes of the product; each >= 0.
 *   alpha, beta    scalars.
 *   C, ldc         M x N, ldc >= max(1, N); read (when beta != 0) and written.
 *   stream, variant  as for sgemm; every variant takes every transpose pair.
 *
 * Behaviour (the BLAS conventions)
 *   - Checks, in this order, before any HIP call: transpose flags, sizes,
 *     leading dimensions, variant, then (only if M > 0 and N > 0) C == NULL,
 *     and, when A and B are read, NULL A or B and overlap of C with them.
 *   - M == 0 or N == 0: returns SGEMM_OK without touching the GPU.
 *   - beta == 0: C is not read (NaN or Inf in C does not propagate).
 *   - K == 0 or alpha == 0: A and B are not read (and may be NULL, or overlap
 *     C); C becomes beta * C, and with beta == 1 the call returns SGEMM_OK
 *     without touching the GPU.
 *   - Otherwise each element is alpha * s + beta * c (one fused multiply-add
 *     of alpha and s onto the rounded beta * c; alpha * s alone when beta ==
 *     0), s being the float32 sum of section 02 formed as for sgemm; the
 *     result is within 1e-5 * (|alpha| sum_k |op(A)[i][k]| |op(B)[k][j]| +
 *     |beta c|) + 1e-6 of the exact value.
 *   - sgemm(M, N, K, A, lda, B, ldb, C, ldc, stream, v) is exactly
 *     sgemm_ex(SGEMM_OP_N, SGEMM_OP_N, M, N, K, 1, A, lda, B, ldb, 0, C, ldc,
 *     stream, v).
 *
 * Returns SGEMM_OK or a negative sgemm_status.
 */
int sgemm_ex(int transA, int transB, int M, int N, int K,
             float alpha,
             const float *A, int lda,
             const float *B, int ldb,
             float beta,
             float *C, int ldc,
             void *stream, int variant);

/*
 * The host-side argument checks of sgemm() alone, with the same codes and in
 * the same order; makes no HIP call and touches no memory. Returns SGEMM_OK
 * when sgemm() would go on to launch (or return early for an empty C).
 */
int sgemm_check_args(int M, int N, int K,
                     const float *A, int lda,
                     const float *B, int ldb,
                     const float *C, int ldc,
                     int variant);

/* The host-side argument checks of sgemm_ex() alone (same codes, same
 * order); makes no HIP call and touches no memory. */
int sgemm_ex_check_args(int transA, int transB, int M, int N, int K,
                        float alpha,
                        const float *A, int lda,
                        const float *B, int ldb,
                        float beta,
                        const float *C, int ldc,
                        int variant);

/*
 * sgemm_ex with a device workspace, so that the matrix-core variant can run
 * products whose tiles would load the compute units unevenly on a split
 * schedule. Tiles are tuned per problem as section 07 and exercise 2 of
 * "Matrix Multiplication -- Naive to Tiled" describe; splitting a tile's K
 * range over several work-groups is this library's addition to that.
 *
 * Split schedule: the product's (tile, K slab) iterations, tile after tile,
 * are dealt out in equal runs to one work-group per compute unit (two with
 * 128 x 128 tiles). A tile whose slabs all fall to one work-group is
 * computed and stored as in sgemm_ex; a tile shared by several is computed
 * in pieces whose unscaled sums go to the workspace, and a second kernel adds
 * each shared tile's pieces in K order and applies alpha and beta. The result
 * is therefore the same on every run, and within the bound sgemm_ex states
 * (its last bits may differ from sgemm_ex's, whose sums are not split).
 *
 * Arguments: those of sgemm_ex, plus
 *   workspace        16-byte aligned device memory the call may use
 *                    (contents undefined afterwards; the caller owns it);
 *                    NULL, an address that is not 16-byte aligned, or
 *   workspace_bytes  smaller than sgemm_ex_workspace_size() for this product,
 *                    makes the call exactly sgemm_ex.
 * The library decides per product whether the split schedule is faster; only
 * the matrix-core variant (and SGEMM_BEST) uses it. Calls that share a
 * workspace must be ordered on one stream: concurrent calls race on it.
 *
 * Behaviour: as sgemm_ex, with one more check after sgemm_ex's: a non-empty
 * workspace that overlaps C, or A or B when they are read, is SGEMM_ERR_ALIAS.
 * Returns SGEMM_OK or a negative sgemm_status.
 */
int sgemm_ex_ws(int transA, int transB, int M, int N, int K,
                float alpha,
                const float *A, int lda,
                const float *B, int ldb,
                float beta,
                float *C, int ldc,
                void *workspace, size_t workspace_bytes,
                void *stream, int variant);

/* The host-side argument checks of sgemm_ex_ws() alone (same codes, same
 * order); makes no HIP call and touches no memory. */
int sgemm_ex_ws_check_args(int transA, int transB, int M, int N, int K,
                           float alpha,
                           const float *A, int lda,
                           const float *B, int ldb,
                           float beta,
                           const float *C, int ldc,
                           const void *workspace, size_t workspace_bytes,
                           int variant);

/*
 * Workspace bytes sgemm_ex_ws needs to run this product on the split
 * schedule on a device with `cus` compute units (cus <= 0: 256, an MI355X),
 * or 0 when it would not split it (the whole-tile schedule is estimated to
 * be as fast, or the arguments are invalid). Pure host logic: no HIP call.
 */
size_t sgemm_ex_workspace_size(int transA, int transB, int M, int N, int K, int cus);

/*
 * sgemm_ex_ws without a workspace argument, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses
 * that forbid hipMalloc): the split schedule's partial tiles go to a static
 * device buffer the library holds, sgemm_ex_noalloc_scratch_bytes() bytes
 * (128 MiB: the largest workspace the split schedule asks for on a 256-CU
 * MI355X) on each GPU the library runs on, from when the library's code is
 * loaded on that GPU until the process ends. The call itself allocates
 * nothing and calls no allocating routine.
 *
 * Arguments and behaviour: those of sgemm_ex (same checks, same order), and
 * the same product as sgemm_ex_ws given a large enough workspace: the same
 * plan, kernels and bits. After the checks, a product that the matrix-core
 * variant (or SGEMM_BEST) would put on the split schedule with more scratch
 * than the buffer holds returns SGEMM_ERR_SCRATCH without launching anything
 * (not on a 256-CU MI355X, where every plan fits). The first call on a device
 * looks up that device's address of the buffer (SGEMM_ERR_DEVICE if that
 * fails).
 *
 * Every call on one GPU shares that GPU's buffer, and what a call leaves in
 * it is never read by the next (each partial tile is written before it is
 * read). Calls whose kernels may run at the same time on one GPU (different
 * streams with no ordering between them) race on the buffer: order them on
 * one stream, or use sgemm_ex_ws with a workspace per stream.
 */
int sgemm_ex_noalloc(int transA, int transB, int M, int N, int K,
                     float alpha,
                     const float *A, int lda,
                     const float *B, int ldb,
                     float beta,
                     float *C, int ldc,
                     void *stream, int variant);

/* The host-side checks of sgemm_ex_noalloc() alone, for a device with `cus`
 * compute units (cus <= 0: 256): sgemm_ex's checks, then SGEMM_ERR_SCRATCH
 * where the product would need more than the static buffer. Makes no HIP
 * call and touches no memory. */
int sgemm_ex_noalloc_check_args(int transA, int transB, int M, int N, int K,
                                float alpha,
                                const float *A, int lda,
                                const float *B, int ldb,
                                float beta,
                                const float *C, int ldc,
                                int variant, int cus);

/* Bytes of the static scratch buffer sgemm_ex_noalloc works in. */
size_t sgemm_ex_noalloc_scratch_bytes(void);

/*
 * The reduced-precision workload: the tensor-core variant "Matrix
 * Multiplication -- Naive to Tiled", section 07 names (16-bit inputs, FP32
 * accumulation), in the general form of sgemm_ex:
 *
 *     C = alpha * op(A) * op(B) + beta * C
 *
 * with A and B holding 16-bit encodings of type `dtype` (SGEMM_LP_BF16 or
 * SGEMM_LP_F16) and C float32. Every product of two 16-bit values is exact in
 * float32, and the products are summed in float32 on the matrix cores
 * (v_mfma_f32_32x32x16_bf16 / _f16), in an order of the kernel's own.
 *
 * Arguments are those of sgemm_ex with A and B typed `const void *` (16-bit
 * elements; leading dimensions in elements; any 2-byte alignment), and no
 * variant: the matrix-core kernel always runs (a one-work-item-per-element
 * kernel takes products whose row-contiguous operand is under 8 wide).
 *
 * Behaviour: as sgemm_ex (the same checks in the same order, with the type
 * first: SGEMM_ERR_DTYPE; the same BLAS read rules; C must not overlap A or B
 * when they are read). Returns SGEMM_OK or a negative sgemm_status.
 */
int sgemm_lp(int dtype, int transA, int transB, int M, int N, int K,
             float alpha,
             const void *A, int lda,
             const void *B, int ldb,
             float beta,
             float *C, int ldc,
             void *stream);

/* The host-side argument checks of sgemm_lp() alone (same codes, same
 * order); makes no HIP call and touches no memory. */
int sgemm_lp_check_args(int dtype, int transA, int transB, int M, int N, int K,
                        float alpha,
                        const void *A, int lda,
                        const void *B, int ldb,
                        float beta,
                        const float *C, int ldc);

/* Static English text for a status code ("unknown status" otherwise). */
const char *sgemm_status_string(int status);

/* Static name of a variant code ("naive", "tiled", "regblock", "mfma",
 * "best"), or NULL for an unknown code. */
const char *sgemm_variant_name(int variant);

/* The concrete variant SGEMM_BEST resolves to for an M x N x K product. */
int sgemm_best_variant(int M, int N, int K);

/*
 * Edge of the square tile (128, 64, 32 or 16) the REGBLOCK variant uses for an
 * M x N product on a device with `cus` compute units (cus <= 0: 256, an
 * MI355X): the pages' 128 x 128 tile ("From 306 ms to 86 ms", "Register
 * blocking") where C holds enough of them to occupy the compute units, else
 * a smaller one, tuned per problem as section 07 of "Matrix Multiplication --
 * Naive to Tiled" describes. Pure host logic: no HIP call. Returns the edge,
 * or SGEMM_ERR_DIM when M or N is negative.
 */
int sgemm_regblock_tile(int M, int N, int cus);

/*
 * The interior tile (BM x BN) the MFMA variant uses for an M x N x K product
 * on a device with `cus` compute units (cus <= 0: 256, an MI355X); tiles are
 * tuned per problem as section 07 and exercise 2 of "Matrix Multiplication --
 * Naive to Tiled" describe. The choice estimates each shape's launch time
 * from how its work-groups fall into rounds over the compute units and the
 * throughput measured for that shape, and takes the fastest; K counts only
 * for the 64 x 64 tile whose K range is split over its waves (taken for a K
 * that is not a multiple of 32 only with one tile per compute unit). Pure
 * host logic: no HIP call. Returns SGEMM_OK, SGEMM_ERR_DIM (M, N or K
 * negative) or SGEMM_ERR_NULL (BM or BN NULL).
 */
int sgemm_mfma_tile(int M, int N, int K, int cus, int *BM, int *BN);

/*
 * The whole kernel shape behind sgemm_mfma_tile's choice, in shape[0..5]:
 * BM, BN, BK (slab depth; for the split tile below, the k per chunk), the
 * waves per work-group along M and N, and the number of wave sets that
 * split the K range between them: 1; 2 for the 64 x 64 and 32 x 32 tiles
 * whose two sets share each slab, which put two waves on each SIMD where one
 * tile per compute unit would leave one; 4 for the 64 x 64 tile whose four
 * waves each hold the whole tile over a quarter of K's chunks (1 x 1 waves
 * per set). Pure host logic. Returns SGEMM_OK, SGEMM_ERR_DIM or
 * SGEMM_ERR_NULL (shape NULL).
 */
int sgemm_mfma_shape(int M, int N, int K, int cus, int *shape);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_H */
