// Host-side argument checks, status strings and variant names of the C ABI.
//
// Pure C++: no HIP header and no device call, so these entry points work
// (and are tested, also under the host sanitizers) on a machine without a GPU.
#include <cstddef>
#include <cstdint>

#include "select.hpp"
#include "sgemm.h"

namespace {

// Byte range [lo, hi) spanned by a rows x cols row-major matrix with leading
// dimension ld (elements); empty when rows or cols is 0.
struct Span {
    std::uintptr_t lo, hi;
};

Span span_of(const void *p, int rows, int cols, int ld, std::size_t elem = sizeof(float))
{
    const std::uintptr_t base = reinterpret_cast<std::uintptr_t>(p);
    if (rows <= 0 || cols <= 0) return {base, base};
    const std::uint64_t last = static_cast<std::uint64_t>(rows - 1) * static_cast<std::uint64_t>(ld) +
                               static_cast<std::uint64_t>(cols);
    return {base, base + last * elem};
}

bool overlap(Span a, Span b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

bool known_variant(int v) { return v >= SGEMM_BEST && v <= SGEMM_TILED_T32; }

bool known_op(int op) { return op == SGEMM_OP_N || op == SGEMM_OP_T; }

int at_least_1(int x) { return x > 1 ? x : 1; }

}  // namespace

extern "C" int sgemm_ex_check_args(int transA, int transB, int M, int N, int K, float alpha, const float *A,
                                   int lda, const float *B, int ldb, float beta, const float *C, int ldc,
                                   int variant)
{
    (void)beta;
    if (!known_op(transA) || !known_op(transB)) return SGEMM_ERR_OP;
    if (M < 0 || N < 0 || K < 0) return SGEMM_ERR_DIM;
    // Stored shapes: A is M x K (K x M when transposed), B is K x N (N x K).
    const bool ta = transA == SGEMM_OP_T, tb = transB == SGEMM_OP_T;
    const int a_rows = ta ? K : M, a_cols = ta ? M : K;
    const int b_rows = tb ? N : K, b_cols = tb ? K : N;
    if (lda < at_least_1(a_cols) || ldb < at_least_1(b_cols) || ldc < at_least_1(N)) return SGEMM_ERR_LD;
    if (!known_variant(variant)) return SGEMM_ERR_VARIANT;
    if (M == 0 || N == 0) return SGEMM_OK;
    if (C == nullptr) return SGEMM_ERR_NULL;
    const bool reads_ab = K > 0 && alpha != 0.0f;
    if (reads_ab) {
        if (A == nullptr || B == nullptr) return SGEMM_ERR_NULL;
        const Span c = span_of(C, M, N, ldc);
        if (overlap(c, span_of(A, a_rows, a_cols, lda)) || overlap(c, span_of(B, b_rows, b_cols, ldb)))
            return SGEMM_ERR_ALIAS;
    }
    return SGEMM_OK;
}

extern "C" int sgemm_ex_ws_check_args(int transA, int transB, int M, int N, int K, float alpha, const float *A,
                                      int lda, const float *B, int ldb, float beta, const float *C, int ldc,
                                      const void *workspace, std::size_t workspace_bytes, int variant)
{
    const int rc = sgemm_ex_check_args(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, variant);
    if (rc != SGEMM_OK || M == 0 || N == 0) return rc;
    if (workspace == nullptr || workspace_bytes == 0) return SGEMM_OK;
    const std::uintptr_t base = reinterpret_cast<std::uintptr_t>(workspace);
    const Span ws{base, base + workspace_bytes};
    if (overlap(ws, span_of(C, M, N, ldc))) return SGEMM_ERR_ALIAS;
    if (K > 0 && alpha != 0.0f) {
        const bool ta = transA == SGEMM_OP_T, tb = transB == SGEMM_OP_T;
        if (overlap(ws, span_of(A, ta ? K : M, ta ? M : K, lda)) || overlap(ws, span_of(B, tb ? N : K, tb ? K : N, ldb)))
            return SGEMM_ERR_ALIAS;
    }
    return SGEMM_OK;
}

extern "C" int sgemm_lp_check_args(int dtype, int transA, int transB, int M, int N, int K, float alpha,
                                   const void *A, int lda, const void *B, int ldb, float beta, const float *C,
                                   int ldc)
{
    (void)beta;
    if (dtype != SGEMM_LP_BF16 && dtype != SGEMM_LP_F16) return SGEMM_ERR_DTYPE;
    if (!known_op(transA) || !known_op(transB)) return SGEMM_ERR_OP;
    if (M < 0 || N < 0 || K < 0) return SGEMM_ERR_DIM;
    const bool ta = transA == SGEMM_OP_T, tb = transB == SGEMM_OP_T;
    const int a_rows = ta ? K : M, a_cols = ta ? M : K;
    const int b_rows = tb ? N : K, b_cols = tb ? K : N;
    if (lda < at_least_1(a_cols) || ldb < at_least_1(b_cols) || ldc < at_least_1(N)) return SGEMM_ERR_LD;
    if (M == 0 || N == 0) return SGEMM_OK;
    if (C == nullptr) return SGEMM_ERR_NULL;
    if (K > 0 && alpha != 0.0f) {
        if (A == nullptr || B == nullptr) return SGEMM_ERR_NULL;
        const Span c = span_of(C, M, N, ldc);
        if (overlap(c, span_of(A, a_rows, a_cols, lda, 2)) || overlap(c, span_of(B, b_rows, b_cols, ldb, 2)))
            return SGEMM_ERR_ALIAS;
    }
    return SGEMM_OK;
}

extern "C" int sgemm_check_args(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
                                const float *C, int ldc, int variant)
{
    return sgemm_ex_check_args(SGEMM_OP_N, SGEMM_OP_N, M, N, K, 1.0f, A, lda, B, ldb, 0.0f, C, ldc, variant);
}

extern "C" const char *sgemm_status_string(int status)
{
    switch (status) {
    case SGEMM_OK: return "success";
    case SGEMM_ERR_DIM: return "negative matrix dimension";
    case SGEMM_ERR_LD: return "leading dimension smaller than the row length";
    case SGEMM_ERR_NULL: return "NULL matrix pointer with a non-empty extent";
    case SGEMM_ERR_VARIANT: return "unknown kernel variant";
    case SGEMM_ERR_LAUNCH: return "kernel launch failed";
    case SGEMM_ERR_DEVICE: return "no usable gfx950 HIP device";
    case SGEMM_ERR_ALIAS: return "C overlaps A or B";
    case SGEMM_ERR_OP: return "transpose flag is neither SGEMM_OP_N nor SGEMM_OP_T";
    case SGEMM_ERR_DTYPE: return "16-bit operand type is neither SGEMM_LP_BF16 nor SGEMM_LP_F16";
    case SGEMM_ERR_SCRATCH: return "the product needs more scratch than the library's static buffer holds";
    default: return "unknown status";
    }
}

extern "C" const char *sgemm_variant_name(int variant)
{
    switch (variant) {
    case SGEMM_BEST: return "best";
    case SGEMM_NAIVE: return "naive";
    case SGEMM_TILED: return "tiled";
    case SGEMM_REGBLOCK: return "regblock";
    case SGEMM_MFMA: return "mfma";
    case SGEMM_TILED_T8: return "tiled8";
    case SGEMM_TILED_T16: return "tiled16";
    case SGEMM_TILED_T32: return "tiled32";
    default: return nullptr;
    }
}

extern "C" int sgemm_best_variant(int M, int N, int K)
{
    (void)M;
    (void)N;
    (void)K;
    return SGEMM_MFMA;
}

extern "C" int sgemm_ex_noalloc_check_args(int transA, int transB, int M, int N, int K, float alpha,
                                           const float *A, int lda, const float *B, int ldb, float beta,
                                           const float *C, int ldc, int variant, int cus)
{
    const int rc = sgemm_ex_check_args(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, variant);
    if (rc != SGEMM_OK || M == 0 || N == 0 || K == 0 || alpha == 0.0f) return rc;
    const int v = variant == SGEMM_BEST ? sgemm_best_variant(M, N, K) : variant;
    if (v != SGEMM_MFMA) return SGEMM_OK;  // only the split schedule uses scratch
    if (sgemm_ex_workspace_size(transA, transB, M, N, K, cus) > sgemm_impl::kNoallocScratchBytes)
        return SGEMM_ERR_SCRATCH;
    return SGEMM_OK;
}

extern "C" size_t sgemm_ex_noalloc_scratch_bytes(void) { return sgemm_impl::kNoallocScratchBytes; }
