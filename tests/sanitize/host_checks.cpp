// Host-only entry points of the C ABI (argument checks, status strings,
// variant names, the tile and split-schedule choices) driven over edge-case
// arguments, for a build under AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_sanitizers.py). No pointer passed here is ever dereferenced by
// these functions: they compare addresses only. Exits non-zero on a failed
// expectation; the sanitizers abort on any undefined behaviour or bad access.
#include <climits>
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "sgemm.h"

namespace {

int failures = 0;

void expect(bool ok, const char *what, long long a = 0, long long b = 0, long long c = 0)
{
    if (!ok) {
        std::fprintf(stderr, "FAILED: %s (%lld, %lld, %lld)\n", what, a, b, c);
        ++failures;
    }
}

bool is_status(int s) { return s <= 0 && s >= SGEMM_ERR_DTYPE; }

const float *fake(std::uintptr_t addr) { return reinterpret_cast<const float *>(addr); }

}  // namespace

int main()
{
    const int sizes[] = {INT_MIN, -7, -1, 0, 1, 3, 4, 7, 8, 31, 64, 255, 256, 4093, 4096, 46400, 65600, 1 << 30,
                         INT_MAX};
    const int lds[] = {INT_MIN, -1, 0, 1, 4, 8, 4096, 4100, INT_MAX};
    const int variants[] = {-2, SGEMM_BEST, SGEMM_NAIVE, SGEMM_TILED, SGEMM_REGBLOCK, SGEMM_MFMA, SGEMM_TILED_T8,
                            SGEMM_TILED_T16, SGEMM_TILED_T32, 7, INT_MAX};

    // Plain and general argument checks: every combination returns a status,
    // and the status string exists.
    const std::uintptr_t a = 0x100000, b = 0x40000000000, c = 0x80000000000;
    for (int M : sizes)
        for (int N : sizes)
            for (int K : sizes)
                for (int ld : lds) {
                    const int s = sgemm_check_args(M, N, K, fake(a), ld, fake(b), ld, fake(c), ld, SGEMM_MFMA);
                    expect(is_status(s), "sgemm_check_args status", M, N, K);
                    expect(sgemm_status_string(s) != nullptr, "status string");
                    if (M < 0 || N < 0 || K < 0) expect(s == SGEMM_ERR_DIM, "negative size -> ERR_DIM", M, N, K);
                    for (int ta = -1; ta <= 2; ++ta) {
                        const int se = sgemm_ex_check_args(ta, 1 - ta, M, N, K, 0.5f, fake(a), ld, fake(b), ld, 1.0f,
                                                           fake(c), ld, SGEMM_BEST);
                        expect(is_status(se), "sgemm_ex_check_args status", M, N, K);
                        const int sw = sgemm_ex_ws_check_args(ta, 0, M, N, K, 1.0f, fake(a), ld, fake(b), ld, 0.0f,
                                                              fake(c), ld, reinterpret_cast<void *>(c), 1u << 20,
                                                              SGEMM_MFMA);
                        expect(is_status(sw), "sgemm_ex_ws_check_args status", M, N, K);
                        const int sl = sgemm_lp_check_args(1 + (ta & 1), ta, 0, M, N, K, 1.0f, fake(a), ld, fake(b),
                                                           ld, 0.0f, fake(c), ld);
                        expect(is_status(sl), "sgemm_lp_check_args status", M, N, K);
                    }
                }
    for (int v : variants) {
        const int s = sgemm_check_args(8, 8, 8, fake(a), 8, fake(b), 8, fake(c), 8, v);
        expect(is_status(s), "variant status", v);
        expect((v >= SGEMM_BEST && v <= SGEMM_TILED_T32) == (s == SGEMM_OK), "variant validity", v, s);
        const char *name = sgemm_variant_name(v);
        expect((name != nullptr) == (v >= SGEMM_BEST && v <= SGEMM_TILED_T32), "variant name", v);
    }
    for (int s = -20; s <= 5; ++s) expect(sgemm_status_string(s) != nullptr, "status string of any code", s);

    // Overlap checks at the top of the address space and at huge extents:
    // the span arithmetic must not overflow.
    const std::uintptr_t top = UINTPTR_MAX - (std::uintptr_t(1) << 20);
    expect(is_status(sgemm_check_args(INT_MAX, INT_MAX, INT_MAX, fake(top), INT_MAX, fake(top), INT_MAX, fake(top),
                                      INT_MAX, SGEMM_MFMA)),
           "huge extents");
    expect(sgemm_check_args(64, 64, 64, fake(a), 64, fake(b), 64, fake(a + 64 * 63 * 4), 64, SGEMM_MFMA) ==
               SGEMM_ERR_ALIAS,
           "C inside A is an alias");
    expect(sgemm_check_args(64, 64, 64, fake(a), 64, fake(b), 64, fake(a + 64 * 64 * 4), 64, SGEMM_MFMA) == SGEMM_OK,
           "C just past A is not");

    // Tile and split-schedule choice over sizes and compute-unit counts.
    const int cus_list[] = {INT_MIN, -1, 0, 1, 80, 256, 304, 1024, INT_MAX};
    for (int M : sizes)
        for (int N : sizes)
            for (int cus : cus_list) {
                for (int K : sizes) {
                    int bm = -1, bn = -1;
                    const int rt = sgemm_mfma_tile(M, N, K, cus, &bm, &bn);
                    expect(is_status(rt), "sgemm_mfma_tile status", M, N, cus);
                    if (rt == SGEMM_OK)
                        expect(((bm == 32 || bm == 64 || bm == 96 || bm == 128 || bm == 256) && bn == bm) ||
                                   (bm == 192 && bn == 128) || (bm == 128 && bn == 192),
                               "tile", M, N, bm);
                    int shape[6] = {-1, -1, -1, -1, -1, -1};
                    const int rs = sgemm_mfma_shape(M, N, K, cus, shape);
                    expect(is_status(rs), "sgemm_mfma_shape status", M, N, cus);
                    if (rs == SGEMM_OK)
                        expect(shape[0] > 0 && shape[1] > 0 && shape[2] > 0 && shape[3] > 0 && shape[4] > 0 &&
                                   (shape[5] == 1 || shape[5] == 2 || shape[5] == 4),
                               "shape", M, N, cus);
                }
                for (int K : sizes) {
                    const std::size_t w = sgemm_ex_workspace_size(0, 1, M, N, K, cus);
                    if (M <= 0 || N <= 0 || K <= 0) expect(w == 0, "no workspace for an empty product", M, N, K);
                    expect(w <= (std::size_t(1) << 40), "workspace size bounded", M, N, K);
                }
            }
    expect(sgemm_best_variant(4096, 4096, 4096) == SGEMM_MFMA, "best variant");

    if (failures) {
        std::fprintf(stderr, "%d failed expectations\n", failures);
        return 1;
    }
    std::printf("host checks ok\n");
    return 0;
}
