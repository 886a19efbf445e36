// Host-side interface of the dense Wt GEMM (bf16, 256 x 128 x 64 tiles).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace poetx {

bool dense_gemm_supported(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb);
// C[M][N] = A[M][K] . B^T (b_nn = false, B is [N][K]) or A . B (b_nn = true, B is [K][N]).
hipError_t dense_gemm_bf16(bool b_nn, const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                           int M, int N, int K, hipStream_t stream);

}  // namespace poetx
