// Host-side interface of the pipelined bf16 MFMA GEMM (256 x 128 x 64 tiles,
// direct-to-LDS loads) that runs the dense Wt products, the batched block
// products and the block gradients of the layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace poetx {

// One product of a grouped launch (pipe_gemm with ngroups > 0): output columns
// [n_begin, next n_begin) use A + a_off and B + b_off (element offsets) and run
// k over [0, k).
struct PipeGroup {
    int n_begin = 0;
    int k = 0;
    int64_t a_off = 0;
    int64_t b_off = 0;
};
constexpr int kMaxPipeGroups = 8;

struct PipeArgs {
    const void* A = nullptr;   // bf16
    int64_t lda = 0, strideA = 0;
    const void* B = nullptr;   // bf16
    int64_t ldb = 0, strideB = 0;
    void* C = nullptr;         // bf16 or float32
    int64_t ldc = 0, strideC = 0, strideSplit = 0;
    int M = 0, N = 0, K = 0;
    int batch = 1;
    int splits = 1;
    int k_per_split = 0;       // multiple of 64
    // General epilogue (pipe_gemm_general only).  With v = alpha * acc:
    //   mode 0: o = v + beta1 Cin1 + beta2 Cin2 + gamma [row == col];
    //           C = o (output dtype, if C), C2 = o (bf16, if C2);
    //   mode 1 (Cayley-Neumann square, k = 3): C = 2 Cin1 + 2 v, C2 = v, C3 = 2 Cin1 + v;
    //   mode 3 (Cayley-Neumann square, k = 4): C = v, C2 = v, C3 = Cin1 + v
    //           (pipe_gemm_general only).
    void* C2 = nullptr;        // bf16
    void* C3 = nullptr;        // bf16, same layout as C2
    int64_t ldc2 = 0, strideC2 = 0;
    const float* Cin1 = nullptr;
    int64_t ldcin1 = 0, strideCin1 = 0;
    const float* Cin2 = nullptr;
    int64_t ldcin2 = 0, strideCin2 = 0;
    float alpha = 1.f, beta1 = 0.f, beta2 = 0.f, gamma = 0.f;
    int mode = 0;
    int epi_vec = 0;           // set by pipe_gemm_general: epilogue may use vector accesses
    // Second product of pipe_gemm_dual: A2^T B2 with A2 [K][M] and B2 [K][N] (m/n-major).
    const void* A2 = nullptr;
    int64_t lda2 = 0, strideA2 = 0;
    const void* B2 = nullptr;
    int64_t ldb2 = 0, strideB2 = 0;
    // Grouped product (pipe_gemm with k-major A, bf16 output, tile Tall, Square
    // or Slim; batch 1, no split): ngroups entries with ascending n_begin,
    // grp[0].n_begin == 0, each a multiple of 128; K must be the largest group k.
    int ngroups = 0;
    PipeGroup grp[kMaxPipeGroups];
    // Column scale of the plain epilogue (int8 dense forward, scaled block
    // product): C[r][c] = acc * colscale[c] (batch entry z: colscale + z strideScale).
    const float* colscale = nullptr;
    int64_t strideScale = 0;
    // The R blocks of the folded forward (dense_fold_r): b x b bf16 blocks, block
    // j for output columns [256 j, 256 j + 256).
    const void* Gfold = nullptr;
};

// a_mn: A is [K][M] (m contiguous) instead of [M][K]; b_mn: B is [K][N] instead
// of [N][K].  C[z] (M x N) = op(A[z]) op(B[z]) over the k range of each split;
// with splits > 1 split s writes its partial sum at C + s * strideSplit.
// Requirements (pipe_gemm_supported): K-contiguous operands need K % 64 == 0;
// every leading dimension, stride and contiguous extent a multiple of 8.
// Workgroup tiles, k-major A with bf16 output (dense and block products): Big
// 256 x 256, Tall 256 x 128, Wide 128 x 256 (a block product's workgroup spans
// a whole block of 256 outputs), Square 128 x 128 and Slim 64 x 128; callers
// take the largest whose grid still gives every CU a workgroup.  m/n-major A
// and B with float32 output (block gradients): Square 128 x 128 and Small
// 64 x 64 (enough tiles to fill the chip without splitting the token axis).
// Dense products of the weight-centric variant: k-major A with float32 output
// and m/n-major A and B with bf16 output, each in Tall and Square.
enum class PipeTile { Tall, Wide, Square, Small, Big, Slim };
bool pipe_gemm_supported(bool a_mn, bool b_mn, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                         int64_t strideA, int64_t strideB);
hipError_t pipe_gemm(bool a_mn, bool b_mn, bool out_f32, const PipeArgs& p, hipStream_t stream, PipeTile tile);
int pipe_tile_rows(PipeTile t);
// Batched products of small matrices (the Cayley-Neumann b x b products) with the
// general epilogue above: 64 x 64 workgroup tiles, or 128 x 128 when the batch is
// large enough to fill the chip with them.  Operand layouts as in pipe_gemm
// ((a_mn, b_mn) = (0, 0), (0, 1) or (1, 1)); no split-K.
hipError_t pipe_gemm_general(bool a_mn, bool b_mn, bool out_f32, const PipeArgs& p, hipStream_t stream);
// Two products of the same b x b shape in one launch (64 x 64 tiles, general
// epilogue): A B^T (k-major A and B) and A2^T B2 (m/n-major A2 and B2).
// separate = false: the general epilogue sees their sum (modes 0 and 1);
// separate = true:  mode 2, C = alpha P1 + beta1 Cin1 and C2 (bf16) = alpha (P1 + P2) + beta2 Cin1.
hipError_t pipe_gemm_dual(bool separate, bool out_f32, const PipeArgs& p, hipStream_t stream);
int pipe_tile_cols(PipeTile t);

// The last product pair of the Cayley-Neumann backward with the skew pack
// folded in, for b x b blocks with b % 64 == 0 (M = N = K = b, A and B k-major,
// A2 and B2 m/n-major, no C outputs): with dQ = alpha (A B^T + A2^T B2) +
// beta1 Cin1 + beta2 Cin2, writes dq [batch, b(b-1)/2] with
// dq[idx(r, c)] = dQ[r][c] - dQ[c][r] for r < c (row-major upper triangle).
hipError_t cnp_pack_pair(const PipeArgs& p, float* dq, int b, hipStream_t stream);

// The k = 3 Cayley-Neumann backward in two passes over units of two tiles (bf16
// operands, b % 64 == 0, all [nblk, b, b] row-major): with X1 = dG S,
// X2 = T^T dG, dS = 2 dG + X1 + X2, Sigma = dS + dS^T,
//   cnp_bwd_sym:  sigma = Sigma (bf16), dq = 2 (dA - dA^T) packed (dA = dG + X1);
//   cnp_bwd_sigq: dq += pack(-(P - P^T)), P = Sigma Q.
// dG is float32 (16-byte aligned): the products take it rounded to bf16 on chip,
// the leading terms exactly.
hipError_t cnp_bwd_sym(const float* dG, const void* S, const void* T, void* sigma, float* dq, int64_t nblk, int b,
                       hipStream_t stream);
hipError_t cnp_bwd_sigq(const void* sigma, const void* Q, float* dq, int64_t nblk, int b, hipStream_t stream);
// The same k = 3 backward with one b = 256 block per workgroup (every
// intermediate on chip, no Sigma or partial dq in memory): dq [nblk, b(b-1)/2]
// from dG float32 and the bf16 S, T, Q of each block.  dGh [nblk, b, b] bf16 is
// scratch (the kernel writes dG / 2 there once and reads it back).
hipError_t cnp_bwd_block(const float* dG, const void* S, const void* T, const void* Q, void* dGh, float* dq,
                         int64_t nblk, int b, hipStream_t stream);

// The k = 3 Cayley-Neumann forward with one b = 256 block per workgroup, from
// the packed parameters q [nblk, b(b-1)/2] to G [nblk, b, b] bf16, with S and T
// (required) and Q (optional) kept in bf16 as the saving forward keeps them.
hipError_t cnp_fwd_block(const float* q, void* G, void* Qc, void* S, void* T, int64_t nblk, int b,
                         hipStream_t stream);

// Fused Cayley-Neumann forward for bf16 blocks of b = 128 or 256 (see the
// kernel): packed float32 parameters q [nblk, b(b-1)/2] -> G bf16 [nblk, b, b];
// with Qc given also Q in bf16, with S and T given (k >= 2) also S = Q Q and
// T = 2Q + S in bf16.  One workgroup per 64-row (few blocks: 32-row) panel.
bool cnp_fused_supported(int64_t b, int k);
hipError_t cnp_fused_fwd(const float* q, void* G, void* Qc, void* S, void* T, int64_t nblk, int64_t b, int k,
                         hipStream_t stream);

// Dense products with an int8 B operand (the quantized weight: codes [N][K]
// k-major for b_nn = false, [K][N] n-major for b_nn = true; int8, ld in
// elements): the codes travel global -> LDS as bytes and are widened to bf16 in
// LDS (exact: |code| <= 127), a tile ahead of their use.  b_nn = false scales
// output column c by colscale[c]; b_nn = true applies no scale (the caller folds
// the row scales of the weight into A's columns).  Needs K % 64 == 0 for
// b_nn = false, N % 16 == 0, lda % 8 == 0, ldb % 16 == 0, 16-byte aligned operands.
bool dense_gemm_q8_supported(bool b_nn, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb);
hipError_t dense_gemm_q8(bool b_nn, const void* A, int64_t lda, const int8_t* B, int64_t ldb, const float* colscale,
                         void* C, int64_t ldc, int M, int N, int K, hipStream_t stream);
// The block product of pipe_gemm (k-major A, bf16 out, n-major B: out = in . G)
// with its output columns scaled: out[:, c] *= colscale[c] over the whole
// [T, d] activation (tiles as block_apply picks them).
hipError_t pipe_gemm_colscale(const PipeArgs& p, hipStream_t stream, PipeTile tile);

// The layer forward's dense product with its R-side block product folded in
// (b = 256): z = (A B^T) blockdiag(G)^T for A = h1 [M][K], B = Wt [N][K] (bf16,
// or int8 codes with q8 and output column c of A B^T scaled by colscale[c]
// first), G [N / 256][256][256] bf16; h2 = A B^T (bf16) is also written when h2
// is given.  z equals the dense product, bf16 rounding of h2 and block product
// run one after another, bit for bit.  N % 256 == 0, K % 64 == 0.
bool dense_fold_r_supported(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int64_t ldc2,
                            int b);
hipError_t dense_fold_r(bool q8, const void* A, int64_t lda, const void* B, int64_t ldb, const float* colscale,
                        const void* G, void* h2, int64_t ldh2, void* z, int64_t ldz, int M, int N, int K, int b,
                        hipStream_t stream);

// Dense convenience wrappers (batch 1, no split).
bool dense_gemm_supported(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb);
// C[M][N] = A[M][K] . B^T (b_nn = false, B is [N][K]) or A . B (b_nn = true, B is [K][N]).
hipError_t dense_gemm_bf16(bool b_nn, const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                           int M, int N, int K, hipStream_t stream);

}  // namespace poetx
