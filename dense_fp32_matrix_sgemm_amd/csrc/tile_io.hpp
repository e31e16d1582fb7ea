// Device helpers shared by the LDS-staged kernels: guarded 4-wide loads and
// stores, and the mapping from work-group number to output tile.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace sgemm_impl {

// Four consecutive elements (row, c .. c+3) of a row-major rows x cols matrix
// with leading dimension ld; elements outside the matrix read as 0 (the
// zero-padding that makes ragged tiles correct: "Matrix Multiplication --
// Naive to Tiled", section 05; "Shared Memory Tiling for Matrix
// Multiplication", traps). `inside` is the caller's promise that the whole
// chunk lies in the matrix. With VEC the chunk is then read with one 16-byte
// load; the caller guarantees 16-byte alignment (base aligned, ld and c
// multiples of 4).
template <bool VEC>
__device__ __forceinline__ float4 load4(const float *base, std::int64_t ld, std::int64_t row, int c,
                                        std::int64_t rows, int cols, bool inside)
{
    const float *p = base + row * ld + c;
    if (inside) {
        if constexpr (VEC) {
            return *reinterpret_cast<const float4 *>(p);
        } else {
            return make_float4(p[0], p[1], p[2], p[3]);
        }
    }
    const bool r = row < rows;
    float4 v;
    v.x = (r && c + 0 < cols) ? p[0] : 0.0f;
    v.y = (r && c + 1 < cols) ? p[1] : 0.0f;
    v.z = (r && c + 2 < cols) ? p[2] : 0.0f;
    v.w = (r && c + 3 < cols) ? p[3] : 0.0f;
    return v;
}

// 16 bytes at a float address that need only be 4-byte aligned. gfx950 has
// unaligned global access, so this is still a single 128-bit load or store.
typedef float f32x4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4u load16u(const float *p)
{
    f32x4u v;
    __builtin_memcpy(&v, p, sizeof(v));
    return v;
}
__device__ __forceinline__ void store16u(float *p, f32x4u v) { __builtin_memcpy(p, &v, sizeof(v)); }
__device__ __forceinline__ void store8u(float *p, float a, float b)
{
    const float v[2] = {a, b};
    __builtin_memcpy(p, v, sizeof(v));
}

// Four consecutive elements known to lie inside the matrix (no guard).
template <bool VEC>
__device__ __forceinline__ float4 load4_inside(const float *base, std::int64_t ld, std::int64_t row, int c)
{
    const float *p = base + row * ld + c;
    if constexpr (VEC) {
        return *reinterpret_cast<const float4 *>(p);
    } else {
        return make_float4(p[0], p[1], p[2], p[3]);
    }
}

// Four consecutive elements (row, c .. c+3) of which some may lie outside the
// matrix: every address is clamped into it (rows, cols >= 1), so all four
// loads are in bounds and unconditional. The values read for outside
// elements are junk until zero_outside() replaces them; keeping that select
// away from the loads stops the compiler from turning each load into a
// branch that waits for its own result.
__device__ __forceinline__ float4 load4_clamped(const float *base, std::int64_t ld, std::int64_t row, int c,
                                                std::int64_t rows, int cols)
{
    const float *p = base + (row < rows ? row : rows - 1) * ld;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = p[c + e < cols ? c + e : cols - 1];
    return make_float4(v[0], v[1], v[2], v[3]);
}

// Zero the elements of a chunk loaded by load4_clamped that lie outside the
// rows x cols matrix (the zero padding of ragged tiles).
__device__ __forceinline__ void zero_outside(float4 &v, std::int64_t row, int c, std::int64_t rows, int cols)
{
    const bool r = row < rows;
    v.x = (r && c + 0 < cols) ? v.x : 0.0f;
    v.y = (r && c + 1 < cols) ? v.y : 0.0f;
    v.z = (r && c + 2 < cols) ? v.z : 0.0f;
    v.w = (r && c + 3 < cols) ? v.w : 0.0f;
}

// The epilogue's update of one element: alpha * acc, plus beta * old when
// beta != 0 (old, C's value before the call, is read only then).
__device__ __forceinline__ float axpby(float alpha, float acc, float beta, float old)
{
    return __builtin_fmaf(alpha, acc, beta * old);
}

// C <- alpha * v + beta * C for N (1, 2 or 4) consecutive elements (row, c ..)
// of C, reading C only when beta != 0. `inside` promises the whole run lies in
// C; it then moves as one access (any 4-byte aligned address: gfx950 performs
// unaligned global accesses). Otherwise elements outside rows x cols are
// skipped.
template <int N>
__device__ __forceinline__ void update_n(float *base, std::int64_t ld, std::int64_t row, int c, std::int64_t rows,
                                         int cols, const float (&v)[N], bool inside, float alpha, float beta)
{
    float *p = base + row * ld + c;
    if (inside) {
        if constexpr (N == 4) {
            f32x4u o = {alpha * v[0], alpha * v[1], alpha * v[2], alpha * v[3]};
            if (beta != 0.0f) {
                const f32x4u old = load16u(p);
                o = f32x4u{axpby(alpha, v[0], beta, old[0]), axpby(alpha, v[1], beta, old[1]),
                           axpby(alpha, v[2], beta, old[2]), axpby(alpha, v[3], beta, old[3])};
            }
            store16u(p, o);
        } else if constexpr (N == 2) {
            float o[2] = {alpha * v[0], alpha * v[1]};
            if (beta != 0.0f) {
                float old[2];
                __builtin_memcpy(old, p, sizeof(old));
                o[0] = axpby(alpha, v[0], beta, old[0]);
                o[1] = axpby(alpha, v[1], beta, old[1]);
            }
            store8u(p, o[0], o[1]);
        } else {
            p[0] = beta != 0.0f ? axpby(alpha, v[0], beta, p[0]) : alpha * v[0];
        }
        return;
    }
    if (row >= rows) return;
#pragma unroll
    for (int e = 0; e < N; ++e)
        if (c + e < cols) p[e] = beta != 0.0f ? axpby(alpha, v[e], beta, p[e]) : alpha * v[e];
}

// The two halves of update_n for callers that update many runs of C with
// beta != 0: read_c reads the N elements of a run (0 where a run at the edge
// has none), write_c writes alpha * v + beta * old over them. Reading every
// run of a batch before writing any keeps the reads in flight together;
// update_n, run by run, waits for each read before the next.
template <int N>
__device__ __forceinline__ void read_c(const float *base, std::int64_t ld, std::int64_t row, int c, std::int64_t rows,
                                       int cols, bool inside, float (&old)[N])
{
    const float *p = base + row * ld + c;
    if (inside) {
        if constexpr (N == 4) {
            const f32x4u x = load16u(p);
            old[0] = x[0];
            old[1] = x[1];
            old[2] = x[2];
            old[3] = x[3];
        } else {
            __builtin_memcpy(old, p, sizeof(old));
        }
        return;
    }
#pragma unroll
    for (int e = 0; e < N; ++e) old[e] = row < rows && c + e < cols ? p[e] : 0.0f;
}

template <int N>
__device__ __forceinline__ void write_c(float *base, std::int64_t ld, std::int64_t row, int c, std::int64_t rows,
                                        int cols, const float (&v)[N], const float (&old)[N], bool inside, float alpha,
                                        float beta)
{
    float o[N];
#pragma unroll
    for (int e = 0; e < N; ++e) o[e] = axpby(alpha, v[e], beta, old[e]);
    float *p = base + row * ld + c;
    if (inside) {
        if constexpr (N == 4)
            store16u(p, f32x4u{o[0], o[1], o[2], o[3]});
        else if constexpr (N == 2)
            store8u(p, o[0], o[1]);
        else
            p[0] = o[0];
        return;
    }
    if (row >= rows) return;
#pragma unroll
    for (int e = 0; e < N; ++e)
        if (c + e < cols) p[e] = o[e];
}

// Work-group number -> output tile (tm, tn).
//
// The dispatcher hands consecutive work-group numbers to the eight XCDs in
// turn (number w runs on XCD w % 8), and each XCD has its own L2. The first
// step renumbers so that each XCD receives one contiguous run of logical
// tiles; the second walks the logical tiles in bands of `group_m` tile rows,
// column by column inside a band, so that the tiles resident on one XCD at a
// time share a few row panels of A and column panels of B in its L2.
// Both steps are bijections on [0, tiles_m * tiles_n).
__device__ __forceinline__ unsigned logical_workgroup(unsigned w, unsigned n_wg)
{
    constexpr unsigned kXcds = 8;
    const unsigned q = n_wg / kXcds, r = n_wg % kXcds;
    const unsigned xcd = w % kXcds, idx = w / kXcds;
    return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

// Logical tile number -> (tm, tn), in bands of group_m tile rows walked
// column by column (the second step above).
__device__ __forceinline__ void tile_of_index(unsigned logical, int tiles_m, unsigned tiles_n, int group_m, int &tm,
                                              int &tn)
{
    const unsigned band = unsigned(group_m) * tiles_n;
    const unsigned first_m = (logical / band) * unsigned(group_m);
    const unsigned rows_in_band = min(unsigned(tiles_m) - first_m, unsigned(group_m));
    const unsigned in_band = logical % band;
    tm = int(first_m + in_band % rows_in_band);
    tn = int(in_band / rows_in_band);
}

__device__ __forceinline__ void tile_of_workgroup(unsigned w, unsigned n_wg, int tiles_m, int group_m, int &tm,
                                                  int &tn)
{
    tile_of_index(logical_workgroup(w, n_wg), tiles_m, n_wg / unsigned(tiles_m), group_m, tm, tn);
}

}  // namespace sgemm_impl
