// Host-side interface of the memory-bound libpoetx kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace poetx {

// Q = unpack(q) in float32 or bf16; with Q2_bf16 set, a bf16 copy is written too.
hipError_t skew_unpack(const float* q, void* Q, bool bf16, int64_t nblk, int b, hipStream_t s,
                       void* Q2_bf16 = nullptr);
hipError_t skew_pack(const float* dQ, float* dq, int64_t nblk, int b, hipStream_t s);
hipError_t permute_2d(const void* src, void* dst, bool bf16, int64_t rows, int64_t cols, const int* row_idx,
                      const int* col_idx, bool scatter, hipStream_t s);
hipError_t splitk_reduce(const float* part, float* out, int64_t count, int splits, hipStream_t s);
hipError_t combine(int64_t nblk, int b, const float* in0, float c0, const float* in1, float c1, const float* in2,
                   float c2, float gamma, float* out32, void* outc, bool outc_bf16, hipStream_t s);
hipError_t fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t compose_perm(const int* pi_old, const int* pi_new, int* inv_tmp, int* sigma, int64_t len,
                        hipStream_t s);
hipError_t check_perm(const int* pi, int64_t len, int* ok, int* counts, int* bad, hipStream_t s);

}  // namespace poetx
