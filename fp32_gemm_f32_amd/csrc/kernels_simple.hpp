// kernels_simple.hpp -- the two rungs below the hot kernel, plus the K == 0 fill.
//
//  * k_sgemm_naive: one work-item per element of C, a dot product of length K read
//    straight from global memory ("Shared Memory Tiling", "The naive kernel"), generalised
//    to M x N x K, leading dimensions and bounds checks.
//  * k_sgemm_lds_tiled<TILE, PAD>: the cooperative shared-memory tiled kernel ("SGEMM:
//    Shared Memory Tiling Visualizer", code panel; "Shared Memory Tiling", "The tiled
//    kernel"): TILE x TILE work-items per block, each tile of A and B loaded once into LDS
//    with out-of-range elements set to zero, ceil(K/TILE) tile steps (the ceiling keeps
//    the last partial tile that a plain integer division would drop), two barriers per
//    step, and a store guarded for ragged M and N.
//    On gfx950 a wavefront is 64 work-items: with TILE = 16 one wave spans four rows of
//    the block, with TILE = 32 two rows. At a fixed k the wave reads one A word per row
//    (a broadcast within each row) and TILE consecutive B words (distinct banks), so the
//    unpadded layout has no bank conflicts; PAD = 1 gives the padded rows of "Shared
//    Memory Tiling", "Conflict-free layout", so the two can be measured side by side.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace sgemm {

__global__ void k_sgemm_naive(int M, int N, int K, const float *__restrict__ A, int lda,
                              const float *__restrict__ B, int ldb, float *__restrict__ C,
                              int ldc)
{
    const int col = blockIdx.x * blockDim.x + threadIdx.x;
    if (col >= N) return;
    // rows are strided over the grid's y extent, which the launcher caps
    for (int64_t row = int64_t(blockIdx.y) * blockDim.y + threadIdx.y; row < M;
         row += int64_t(gridDim.y) * blockDim.y) {
        const float *a = A + row * lda;
        const float *b = B + col;
        float acc = 0.0f;
        for (int k = 0; k < K; ++k) acc = __builtin_fmaf(a[k], b[int64_t(k) * ldb], acc);
        C[row * ldc + col] = acc;
    }
}

template <int TILE, int PAD>
__global__ __launch_bounds__(TILE *TILE) void k_sgemm_lds_tiled(
    int M, int N, int K, const float *__restrict__ A, int lda, const float *__restrict__ B,
    int ldb, float *__restrict__ C, int ldc)
{
    __shared__ float tileA[TILE][TILE + PAD];
    __shared__ float tileB[TILE][TILE + PAD];
    const int tx = threadIdx.x, ty = threadIdx.y;
    const int col = blockIdx.x * TILE + tx;
    const int steps = (K + TILE - 1) / TILE;
    // block rows are strided over the grid's y extent (uniform per block, so the
    // barriers inside stay convergent)
    for (int64_t row0 = int64_t(blockIdx.y) * TILE; row0 < M;
         row0 += int64_t(gridDim.y) * TILE) {
        const int64_t row = row0 + ty;
        float acc = 0.0f;
        for (int t = 0; t < steps; ++t) {
            const int ka = t * TILE + tx;  // column of A this work-item loads
            const int kb = t * TILE + ty;  // row of B this work-item loads
            tileA[ty][tx] = (row < M && ka < K) ? A[row * lda + ka] : 0.0f;
            tileB[ty][tx] = (kb < K && col < N) ? B[int64_t(kb) * ldb + col] : 0.0f;
            __syncthreads();
#pragma unroll
            for (int k = 0; k < TILE; ++k)
                acc = __builtin_fmaf(tileA[ty][k], tileB[k][tx], acc);
            __syncthreads();
        }
        if (row < M && col < N) C[row * ldc + col] = acc;
    }
}

// C[i][j] = 0 for i < M, j < N: the empty sum when K == 0 (grid-stride over elements).
__global__ void k_fill_zero(int M, int N, float *__restrict__ C, int ldc)
{
    const int64_t total = int64_t(M) * N;
    for (int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
         e += int64_t(gridDim.x) * blockDim.x)
        C[(e / N) * ldc + e % N] = 0.0f;
}

}  // namespace sgemm
