// kernels_ladder.hpp -- the measurable rungs between the shared-memory tiled kernel and the
// matrix-core kernel, and the bank-geometry microbenchmark.
//
//  * k_sgemm_regtile<BM, BN, BK, TM, TN>: scalar register tiling ("SGEMM: 2D Register
//    Tiling Visualizer", code panel and "Why 2D Register Tiling Dominates"). A block of
//    (BM/TM) x (BN/TN) threads owns a BM x BN tile of C; per K step of BK it stages a
//    BM x BK tile of A and a BK x BN tile of B in LDS (zero past the edges), and per inner
//    step each thread loads TM values of A into regM and TN values of B into regN and does
//    TM*TN FMAs into its TM x TN results. TM = 4, TN = 1 is the 1-D strip of that page
//    (5 shared reads per 4 FMAs); 4 x 4 and 8 x 8 are its 2-D tiles (8 per 16, 16 per 64).
//    The LDS layout is the page's: As[row][k], Bs[k][col].
//  * k_lds_transpose<T, PAD>: out = in^T through a T x (T + PAD) LDS tile, written by rows
//    and read by columns ("Visual walkthrough - Memory hierarchy", Step 6; "Shared Memory
//    Tiling", "Conflict-free layout"). With PAD = 0 every lane of a column read hits the
//    same bank; with PAD = 1 consecutive rows shift by one bank. It exists to measure the
//    LDS bank geometry of gfx950 with SQ_LDS_BANK_CONFLICT.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace sgemm {

template <int BM, int BN, int BK, int TM, int TN>
__global__ __launch_bounds__((BM / TM) * (BN / TN)) void k_sgemm_regtile(
    int M, int N, int K, const float *__restrict__ A, int lda, const float *__restrict__ B,
    int ldb, float *__restrict__ C, int ldc)
{
    constexpr int TX = BN / TN, TY = BM / TM, NT = TX * TY;
    static_assert(BM % TM == 0 && BN % TN == 0, "register tile divides the block tile");
    __shared__ float As[BM][BK];
    __shared__ float Bs[BK][BN];
    const int tid = threadIdx.x;
    const int tx = tid % TX, ty = tid / TX;
    const int64_t m0 = int64_t(blockIdx.y) * BM, n0 = int64_t(blockIdx.x) * BN;
    float res[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) res[i][j] = 0.0f;
    float regM[TM], regN[TN];
    for (int k0 = 0; k0 < K; k0 += BK) {
        // cooperative, masked loads of both tiles
        for (int e = tid; e < BM * BK; e += NT) {
            const int r = e / BK, k = e % BK;
            As[r][k] = (m0 + r < M && k0 + k < K) ? A[(m0 + r) * lda + k0 + k] : 0.0f;
        }
        for (int e = tid; e < BK * BN; e += NT) {
            const int k = e / BN, c = e % BN;
            Bs[k][c] = (k0 + k < K && n0 + c < N) ? B[int64_t(k0 + k) * ldb + n0 + c] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int d = 0; d < BK; ++d) {
#pragma unroll
            for (int i = 0; i < TM; ++i) regM[i] = As[ty * TM + i][d];
#pragma unroll
            for (int j = 0; j < TN; ++j) regN[j] = Bs[d][tx * TN + j];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) res[i][j] = __builtin_fmaf(regM[i], regN[j], res[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t row = m0 + ty * TM + i;
        if (row >= M) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t col = n0 + tx * TN + j;
            if (col < N) C[row * ldc + col] = res[i][j];
        }
    }
}

// out[j][i] = in[i][j] for i < rows, j < cols. Block: T x (T / 4) threads; each moves a
// T x T tile, four rows per thread.
template <int T, int PAD>
__global__ __launch_bounds__(T *(T / 4)) void k_lds_transpose(int rows, int cols,
                                                             const float *__restrict__ in,
                                                             int ldi, float *__restrict__ out,
                                                             int ldo)
{
    __shared__ float tile[T][T + PAD];
    const int tx = threadIdx.x % T, ty = threadIdx.x / T;
    const int64_t r0 = int64_t(blockIdx.y) * T, c0 = int64_t(blockIdx.x) * T;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int r = ty + k * (T / 4);
        tile[r][tx] = (r0 + r < rows && c0 + tx < cols) ? in[(r0 + r) * ldi + c0 + tx] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int c = ty + k * (T / 4);   // output row = input column c0 + c
        if (c0 + c < cols && r0 + tx < rows) out[(c0 + c) * ldo + r0 + tx] = tile[tx][c];
    }
}

}  // namespace sgemm
