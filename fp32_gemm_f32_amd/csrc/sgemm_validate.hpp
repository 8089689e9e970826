// sgemm_validate.hpp -- argument validation for the C ABI (pure host code, no HIP calls).
//
// Everything here runs before the library touches the HIP runtime, so a host without a
// GPU can exercise every error path. The rules are the ones stated in sgemm_f32.h.
#pragma once

#include <cstdint>

#include "sgemm_f32.h"

namespace sgemm {

// Element span of a row-major rows x cols matrix with leading dimension ld (0 if empty).
inline int64_t span_elems(int64_t rows, int64_t cols, int64_t ld)
{
    if (rows <= 0 || cols <= 0) return 0;
    return (rows - 1) * ld + cols;
}

inline bool bad_ptr(const void *p, int64_t elems)
{
    if (elems == 0) return false;
    return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 3u) != 0;
}

inline bool overlap(const void *a, int64_t a_elems, const void *b, int64_t b_elems)
{
    if (a_elems == 0 || b_elems == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), a1 = a0 + uintptr_t(a_elems) * 4u;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(b), b1 = b0 + uintptr_t(b_elems) * 4u;
    return a0 < b1 && b0 < a1;
}

// The shape rules alone (dimensions, then leading dimensions), for the entry points that
// plan without operands.
inline int validate_shape(int M, int N, int K, int lda, int ldb, int ldc)
{
    if (M < 0 || N < 0 || K < 0) return SGEMM_EINVAL_DIM;
    if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1))
        return SGEMM_EINVAL_LD;
    return SGEMM_OK;
}

inline int validate(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
                    const float *C, int ldc)
{
    const int st = validate_shape(M, N, K, lda, ldb, ldc);
    if (st != SGEMM_OK) return st;
    const int64_t sa = span_elems(M, K, lda);
    const int64_t sb = span_elems(K, N, ldb);
    const int64_t sc = span_elems(M, N, ldc);
    if (bad_ptr(A, sa) || bad_ptr(B, sb) || bad_ptr(C, sc)) return SGEMM_EINVAL_PTR;
    if (overlap(C, sc, A, sa) || overlap(C, sc, B, sb)) return SGEMM_EALIAS;
    return SGEMM_OK;
}

}  // namespace sgemm
