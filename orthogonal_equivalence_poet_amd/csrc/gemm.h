// Host-side interface of the MFMA GEMM used by every product in libpoetx.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace poetx {

// (A layout, B layout): NT = A[M][K] . B[N][K]^T, NN = A[M][K] . B[K][N],
// TN = A[K][M]^T . B[K][N].
enum class GemmLayout { NT, NN, TN };
// Workgroup tile: Large 256x128 (bf16 only), Medium 128x128, Small 64x64.
enum class GemmTile { Large, Medium, Small };

struct GemmArgs {
    const void* A = nullptr;
    int64_t lda = 0, strideA = 0;
    const void* B = nullptr;
    int64_t ldb = 0, strideB = 0;
    void* C = nullptr;            // output in the output dtype (may be null)
    int64_t ldc = 0, strideC = 0;
    int64_t strideSplit = 0;      // offset between split-K partial outputs
    void* C2 = nullptr;           // optional second output in the compute dtype
    int64_t ldc2 = 0, strideC2 = 0;
    const float* Cin1 = nullptr;  // optional float32 addends
    int64_t ldcin1 = 0, strideCin1 = 0;
    const float* Cin2 = nullptr;
    int64_t ldcin2 = 0, strideCin2 = 0;
    float alpha = 1.f, beta1 = 0.f, beta2 = 0.f, gamma = 0.f;
    // Epilogue mode 1 (Cayley-Neumann square): with v = alpha * acc and
    // Q = Cin1, writes C = 2Q + 2v (float32), C2 = v and C3 = 2Q + v (compute dtype).
    int mode = 0;
    void* C3 = nullptr;
    int M = 0, N = 0, K = 0;
    int batch = 1;
    int splits = 1;
    int k_per_split = 0;          // multiple of the tile's k extent
};

hipError_t gemm_launch(const GemmArgs& p, GemmLayout layout, GemmTile tile, bool compute_bf16,
                       bool out_bf16, hipStream_t stream);
int gemm_tile_rows(GemmTile tile, bool bf16);
int gemm_tile_cols(GemmTile tile, bool bf16);
int gemm_tile_k(bool bf16);

}  // namespace poetx
