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
// dst[r][c] = sum_{g < nsum} src[r][idx[g dst_cols + c]] (float32 sum, one rounding);
// src [rows, src_cols], dst [rows, dst_cols], both 16-byte rows.
hipError_t gather_sum(const void* src, void* dst, bool bf16, int64_t rows, int64_t src_cols, int64_t dst_cols,
                      const int* idx, int nsum, hipStream_t s);
// The index tables of a group of `count` linears sharing an input of width n,
// the linear g owning output rows [off[g], off[g + 1]):
// out_R[i] = pi_R[i] + off[g] (its R permutation in the concatenated outputs) and
// inv_P[g n + pi_P[g n + j]] = g n + j (its P permutation inverted, offset by g n).
struct PermSegments {
    int count = 0;
    int64_t n = 0;
    int64_t off[9] = {};
};
hipError_t group_perms(const int* pi_R, const int* pi_P, int* out_R, int* inv_P, const PermSegments& seg,
                       hipStream_t s);
// Symmetric int8 storage per row: scale[i] = max_j |W[i][j]| / 127, q[i][j] = nearest
// integer to W[i][j] / scale[i] (ties to even) in [-127, 127]; zero rows: scale 0, codes 0.
hipError_t quantize_rows(const void* W, bool bf16, int64_t m, int64_t n, int8_t* q, float* scale, hipStream_t s);
// out (bf16 [m, n], 16-byte aligned, n % 16 == 0) = q[i][j] * scale[i].
hipError_t dequantize_rows(const int8_t* q, const float* scale, void* out, int64_t m, int64_t n, hipStream_t s);
// inv[pi[i]] = i.
hipError_t invert_perm(const int* pi, int* inv, int64_t len, hipStream_t s);
// out (d x d, 16-byte aligned, d % b == 0) = Pi^T diag(G) Pi as a dense matrix, given
// inv = pi^-1 and the blocks G [d / b, b, b] in the same dtype.
hipError_t blockdiag_dense(const void* G, const int* inv, void* out, bool bf16, int64_t d, int b, hipStream_t s);
// dG [d / b, b, b] = the diagonal blocks of Pi D Pi^T, D dense float32 d x d.
hipError_t blockdiag_gather(const float* D, const int* pi, float* dG, int64_t d, int b, hipStream_t s);

// AdamW coefficients for one step, worked out on the host in double:
// decay = 1 - eta wd, step = eta / (1 - beta1^t), inv_sqrt_bc2 = 1 / sqrt(1 - beta2^t)
// with eta = lr * gamma.  Per element:  m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
// q = decay q - step m / (sqrt(v) inv_sqrt_bc2 + eps).
struct AdamwCoef {
    float beta1, one_minus_beta1, beta2, one_minus_beta2, eps, decay, step, inv_sqrt_bc2;
};
hipError_t adamw_step(float* q, const float* g, float* m, float* v, int64_t count, const AdamwCoef& c,
                      hipStream_t s);
// a[i] = b[i] = 0 for i < count (a fill kernel, so a captured graph replays it).
hipError_t zero_pair(float* a, float* b, int64_t count, hipStream_t s);

}  // namespace poetx
