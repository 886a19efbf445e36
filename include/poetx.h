/*
 * libpoetx: the POET-X linear layer on AMD Instinct MI355X (gfx950).
 *
 * The layer trains a frozen weight W0 (m x n, d_out x d_in) through an
 * orthogonal equivalence  W_RP = R W0 P  ("POET-X: Memory-efficient LLM
 * Training by Scaling Orthogonal Transformation", SAI replication review,
 * Summary; agidaily.cc article, formula W_RP = R . W0 . P).  R (m x m) and
 * P (n x n) are block-diagonal orthogonal matrices in a random permuted basis;
 * every b x b block G is the Cayley map of a skew-symmetric Q truncated after
 * the k-th Neumann term, and Q is stored as its b(b-1)/2 upper-triangle values
 * (review Summary; Reproducibility, "Partial coverage ...").
 *
 * Conventions fixed by this library (readings of points the pages leave open):
 *   - compact layout: q[idx(r,c)] = Q[r,c] for r < c with
 *     idx(r,c) = r*b - r*(r+1)/2 + (c - r - 1)  (row-major strict upper
 *     triangle), Q[c,r] = -Q[r,c], Q[r,r] = 0;
 *   - G = (I + Q) * sum_{i=0..k} Q^i  (first-order term I + 2Q, as the
 *     review's "Cayley approximation" weakness states);
 *   - a permutation pi (int32, length d) gathers: (Pi v)[i] = v[pi[i]];
 *     R = Pi_R^T diag(G_R,0, G_R,1, ...) Pi_R, P likewise; block j covers the
 *     permuted indices [j*b, (j+1)*b);
 *   - the two permutations next to W0 are absorbed into the stored weight
 *     Wt = Pi_R W0 Pi_P^T, Wt[i][j] = W0[pi_R[i]][pi_P[j]] (review Summary,
 *     "permutation reduction");
 *   - activations are row-major [T, features] (one token per row); the layer
 *     computes y_t = R W0 P x_t for every row.
 *
 * Memory and execution model (all entry points):
 *   - every tensor pointer is a caller-owned DEVICE pointer, contiguous
 *     row-major, 16-byte aligned; the library never allocates or frees device
 *     memory and keeps no pointer after the call returns.  The layer and group
 *     calls (poetx_linear_*, poetx_group_*) check the alignment of every
 *     pointer they take and return POETX_ERR_INVALID_ARG for one that is not
 *     16-byte aligned (a contiguous view at an odd element offset, say);
 *   - work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*, NULL = the null stream); results are ready when the stream is;
 *   - scratch memory comes from the caller's workspace `ws` of `ws_bytes`
 *     bytes (256-byte aligned); the matching *_workspace_bytes() query returns
 *     the size needed (0 means ws may be NULL);
 *   - all arguments are validated on the host BEFORE any HIP call: a bad
 *     argument returns an error code and enqueues nothing;
 *   - nothing aborts and no C++ exception crosses this interface.
 *   - calls on different streams that share output or workspace memory race.
 *
 * Data types: POETX_F32 or POETX_BF16 for activations, Wt and G blocks (bf16
 * is stored as the upper 16 bits of an IEEE float, round-to-nearest-even on
 * every conversion); the compact parameters q, dq and the block gradients dG
 * are always float32.  Every product accumulates in float32 (MFMA).
 *
 * Supported sizes: 16 <= b <= 1024 with b % 16 == 0, b | m, b | n,
 * 1 <= k <= 8, T >= 0 (T == 0 is an empty batch), every extent below 2^31.
 */
#ifndef POETX_H
#define POETX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
enum {
    POETX_OK = 0,
    POETX_ERR_INVALID_ARG = 1, /* null pointer, unknown enum value */
    POETX_ERR_SHAPE = 2,       /* b does not divide m/n, T < 0, b % 16 != 0, ... */
    POETX_ERR_UNSUPPORTED = 3, /* b or k outside the supported range */
    POETX_ERR_WORKSPACE = 4,   /* ws_bytes below the *_workspace_bytes() value */
    POETX_ERR_HIP = 5          /* a HIP call failed; see poetx_last_hip_error() */
};

enum { POETX_F32 = 0, POETX_BF16 = 1 };

/* fast saves h2 (the dense product's output) and a (x gathered by pi_P) for
 * the backward; mem keeps only x and recomputes both (review Summary:
 * POET-X_fast / checkpointed POET-X_mem).
 *
 * Two comparison variants compute the same y, dx, dG_R and dG_P (to rounding)
 * without one of the reformulations, for measuring what that reformulation
 * buys (review Summary, "permutation reduction" and the original weight-centric
 * POET; Reproducibility & code, the original-POET single-layer timing and the
 * 4-permute against 2-permute comparison):
 *   four_perm:       the fast chain over W0 itself, applying all four
 *                    permutations to the activations (two gathers and two
 *                    scatters each way) instead of absorbing two into Wt;
 *   weight_centric:  the original POET: R and P are built as dense m x m and
 *                    n x n matrices, W_RP = R (W0 P) is formed and y = x W_RP^T;
 *                    the backward forms dW_RP = dy^T x and takes
 *                    dR = dW_RP (W0 P)^T and dP = W0^T (R^T dW_RP) from it.
 * With either of them the weight argument of poetx_linear_fwd / _bwd is W0
 * [m, n] itself, not the pre-permuted Wt, and poetx_merge does not apply
 * (POETX_ERR_UNSUPPORTED). */
enum { POETX_FAST = 0, POETX_MEM = 1, POETX_FOUR_PERM = 2, POETX_WEIGHT_CENTRIC = 3, POETX_MEM_Q8 = 4 };

/* mem_q8 (the review's POET-XQ, Summary and Strengths: quantized training
 * through the checkpointed variant, which never keeps a dequantized weight):
 * the stored weight is the quantized buffer of poetx_quantize_weight (int8 per
 * output row, see below) and poetx_linear_fwd / _bwd run the mem chain with the
 * int8 codes read straight into the dense products: the codes are widened to
 * bf16 inside the product (exact), the row scales are applied in float32 (to
 * the output columns of h2 in the forward, to the columns of dh2 in the
 * backward), so the weight the chain computes with is code * scale and no
 * dequantized copy of it is made; bf16 only, b % 64 == 0 (POETX_ERR_SHAPE
 * otherwise).  The pages give no format: symmetric int8 with one float32 scale
 * per row of Wt is this library's reading of their 8-bit setting.  poetx_merge
 * on a mem_q8 descriptor expands the weight into its workspace, merges in bf16
 * and stores the result quantized again. */

typedef struct poetx_linear_desc {
    int64_t T;       /* tokens (rows of x and y), >= 0 */
    int64_t m;       /* d_out: rows of W0, size of R */
    int64_t n;       /* d_in: columns of W0, size of P */
    int64_t b;       /* block size of R and P */
    int32_t k;       /* Neumann order (highest power of Q kept) */
    int32_t dtype;   /* POETX_F32 or POETX_BF16 */
    int32_t variant; /* POETX_FAST, POETX_MEM, POETX_FOUR_PERM, POETX_WEIGHT_CENTRIC or POETX_MEM_Q8 */
    int32_t reserved;/* must be 0 */
} poetx_linear_desc;

/* Library version string, e.g. "libpoetx 0.1.0 gfx950". */
const char* poetx_version(void);
/* Static text for a status code. */
const char* poetx_status_string(int status);
/* Text of the last HIP failure seen by the calling thread ("" if none). */
const char* poetx_last_hip_error(void);

/* ------------------------------------------------ compact skew parameters */
/* Q[j] = unpack(q[j]) for nblk blocks (compact skew storage, review Summary).
 * q: float32 [nblk, b(b-1)/2]; Q: dtype [nblk, b, b].  Bit-exact. */
int poetx_skew_unpack(const float* q, void* Q, int dtype, int64_t nblk, int64_t b,
                      void* stream);

/* Adjoint of unpack: dq[j][idx(r,c)] = dQ[j][r][c] - dQ[j][c][r].
 * dQ: float32 [nblk, b, b]; dq: float32 [nblk, b(b-1)/2]. */
int poetx_skew_pack(const float* dQ, float* dq, int64_t nblk, int64_t b, void* stream);

/* ----------------------------------------------- Cayley-Neumann transform */
/* G[j] = (I + Q_j) sum_{i<=k} Q_j^i for a flat batch of nblk blocks (the
 * review's fused Cayley-Neumann kernel, Summary and Reproducibility).
 * q: float32 [nblk, b(b-1)/2]; G: G_dtype [nblk, b, b].  With G_dtype
 * POETX_BF16 the powers of Q are multiplied in bf16 with float32
 * accumulation and the terms I + 2Q are added in float32; POETX_F32 keeps
 * every operand in float32.  One call may cover the blocks of many layers. */
size_t poetx_cnp_fwd_workspace_bytes(int64_t nblk, int64_t b, int k, int G_dtype);
int poetx_cnp_fwd(const float* q, int64_t nblk, int64_t b, int k, void* G, int G_dtype,
                  void* ws, size_t ws_bytes, void* stream);

/* Adjoint of poetx_cnp_fwd followed by the skew pack:
 * dq = pack(L_f(Q^T)[dG]).  dG: float32 [nblk, b, b]; dq: float32
 * [nblk, b(b-1)/2].  `dtype` selects the operand precision of the products
 * as for poetx_cnp_fwd. */
size_t poetx_cnp_bwd_workspace_bytes(int64_t nblk, int64_t b, int k, int dtype);
int poetx_cnp_bwd(const float* q, const float* dG, int64_t nblk, int64_t b, int k,
                  float* dq, int dtype, void* ws, size_t ws_bytes, void* stream);

/* Save / reuse variant of the pair above (the fast-versus-memory trade of the
 * review's POET-X_fast / POET-X_mem, applied to the transform): the forward
 * keeps Q and the square of Q with its companion terms in the caller's
 * `saved` buffer (device memory of at least poetx_cnp_saved_bytes bytes,
 * 256-byte aligned), and the backward reads them instead of recomputing.
 * The backward's `saved` must hold what poetx_cnp_fwd_save wrote for the same
 * q, nblk, b, k and dtype, unchanged since; results are bit-identical to
 * poetx_cnp_fwd / poetx_cnp_bwd.  `ws` as for the plain calls (their
 * *_workspace_bytes suffice).  Errors: a null `saved` is POETX_ERR_INVALID_ARG,
 * saved_bytes too small is POETX_ERR_WORKSPACE. */
size_t poetx_cnp_saved_bytes(int64_t nblk, int64_t b, int k, int dtype);
int poetx_cnp_fwd_save(const float* q, int64_t nblk, int64_t b, int k, void* G, int G_dtype,
                       void* saved, size_t saved_bytes, void* ws, size_t ws_bytes, void* stream);
int poetx_cnp_bwd_saved(const float* q, const float* dG, int64_t nblk, int64_t b, int k,
                        float* dq, int dtype, const void* saved, size_t saved_bytes,
                        void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------ permutations */
/* dst[i][j] = src[row_idx[i]][col_idx[j]] (row_idx / col_idx may be NULL for
 * the identity).  src, dst: dtype [rows, cols] with leading dimension cols.
 * With scatter_cols != 0 the columns are scattered instead:
 * dst[i][col_idx[j]] = src[row_idx[i]][j].  Bit-exact.  The index arrays
 * must be permutations (see poetx_check_perm); src and dst must not overlap. */
int poetx_permute(const void* src, void* dst, int dtype, int64_t rows, int64_t cols,
                  const int32_t* row_idx, const int32_t* col_idx, int scatter_cols,
                  void* stream);

/* Wt = Pi_R W0 Pi_P^T, i.e. Wt[i][j] = W0[pi_R[i]][pi_P[j]] (the review's
 * permutation reduction).  W0, Wt: dtype [m, n].  Bit-exact. */
int poetx_prepermute(const void* W0, void* Wt, int dtype, int64_t m, int64_t n,
                     const int32_t* pi_R, const int32_t* pi_P, void* stream);

/* Debug check that pi is a bijection of [0, len): writes 1 (yes) or 0 to the
 * device int32 *ok.  Needs poetx_check_perm_workspace_bytes(len) of ws. */
size_t poetx_check_perm_workspace_bytes(int64_t len);
int poetx_check_perm(const int32_t* pi, int64_t len, int32_t* ok, void* ws, size_t ws_bytes,
                     void* stream);

/* ------------------------------------------------------------- the layer */
/* Forward of the input-centric chain (review Summary):
 *   a  = x gathered by pi_P          [T, n]
 *   h1 = a . blockdiag(G_P)^T        [T, n]
 *   h2 = h1 . Wt^T                   [T, m]
 *   z  = h2 . blockdiag(G_R)^T       [T, m]
 *   y  = z scattered by pi_R         [T, m]   (y = x P^T W0^T R^T)
 * x: dtype [T, n]; Wt: dtype [m, n]; G_R: dtype [m/b, b, b]; G_P: dtype
 * [n/b, b, b]; y: dtype [T, m].  FAST writes h2 (dtype [T, m]) and a (dtype
 * [T, n], at the next 256-byte boundary after h2) to `saved`, which must hold
 * poetx_linear_saved_bytes(d) bytes; MEM writes nothing there (saved may be
 * NULL).  FOUR_PERM saves the same two tensors (h2 here is the dense product's
 * output gathered by pi_R).  WEIGHT_CENTRIC saves the dense R (dtype [m, m]),
 * W0 P and W_RP (dtype [m, n] each), each at a 256-byte boundary. */
size_t poetx_linear_saved_bytes(const poetx_linear_desc* d);
size_t poetx_linear_fwd_workspace_bytes(const poetx_linear_desc* d);
int poetx_linear_fwd(const poetx_linear_desc* d, const void* x, const void* Wt,
                     const void* G_R, const void* G_P, const int32_t* pi_R,
                     const int32_t* pi_P, void* y, void* saved, void* ws, size_t ws_bytes,
                     void* stream);

/* poetx_linear_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same forward, same arguments and results, bit for bit, but without a
 * workspace argument.  Its scratch is a device array of the library's own,
 * POETX_NOALLOC_SCRATCH_BYTES bytes, one copy on each GPU the library runs on,
 * held from the first call on that GPU until the process ends.  The caller
 * still passes x, y, saved and the weights.
 *   - a descriptor whose poetx_linear_fwd_workspace_bytes exceeds
 *     POETX_NOALLOC_SCRATCH_BYTES returns POETX_ERR_WORKSPACE before any HIP
 *     call (at bf16 that admits, e.g., the fast forward at T * max(m, n) up to
 *     16 Mi elements: 2048 tokens of a 4096-wide layer);
 *   - the call allocates and frees nothing (no hipMalloc, hipFree or
 *     allocating library routine); on a device's first call it looks up the
 *     array's address once (hipGetSymbolAddress);
 *   - every call on one GPU shares that GPU's array: calls that overlap on one
 *     GPU (different streams or threads without ordering) race; calls ordered
 *     on one stream do not.  Nothing in the array needs to start at zero.
 * Other errors as for poetx_linear_fwd. */
#define POETX_NOALLOC_SCRATCH_BYTES (64u << 20)
int poetx_linear_fwd_noalloc(const poetx_linear_desc* d, const void* x, const void* Wt,
                             const void* G_R, const void* G_P, const int32_t* pi_R,
                             const int32_t* pi_P, void* y, void* saved, void* stream);

/* Backward of the chain for L = <dy, y>; W0 is frozen, so there is no dW0.
 *   dx  = dy R W0 P                              dtype [T, n]
 *   dG_R[j] = (Pi_R dR Pi_R^T) block j, dR = dy^T x P^T W0^T     float32 [m/b, b, b]
 *   dG_P[j] = (Pi_P dP Pi_P^T) block j, dP = W0^T R^T dy^T x     float32 [n/b, b, b]
 * FAST, FOUR_PERM and WEIGHT_CENTRIC read what poetx_linear_fwd saved for the
 * same inputs; MEM recomputes h2 and a from x.  Feed dG_R / dG_P to poetx_cnp_bwd
 * to obtain dq_R / dq_P.  T == 0 writes zero block gradients. */
size_t poetx_linear_bwd_workspace_bytes(const poetx_linear_desc* d);
int poetx_linear_bwd(const poetx_linear_desc* d, const void* dy, const void* x,
                     const void* Wt, const void* G_R, const void* G_P, const int32_t* pi_R,
                     const int32_t* pi_P, const void* saved, void* dx, float* dG_R,
                     float* dG_P, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------- groups of linears */
/* Linears that read the same input (a decoder layer's q, k and v projections,
 * or its gate and up projections) as one chain, so that each stage is one
 * launch over the whole group instead of one per linear.  This extends the
 * review's batch-parallel block products (Summary: all blocks of a transform
 * in one batched product) across the linears of a group; the pages do not
 * describe it.  Every linear keeps its own W0, R, P and permutations: linear g
 * computes y_g = R_g W0_g P_g x exactly as poetx_linear_fwd does, and the group
 * computes all of them from one read of x.
 *
 * With off_g = m_0 + ... + m_{g-1} and M = off_count:
 *   Wt   dtype [M, n]           the pre-permuted weights stacked by rows (linear g
 *                               in rows [off_g, off_g + m_g));
 *   G_R  dtype [M/b, b, b]      linear g's R blocks from block off_g / b;
 *   G_P  dtype [count n/b, b, b] linear g's P blocks from block g n / b;
 *   pi_R int32 [M]              linear g's own permutation of [0, m_g) at off_g;
 *   pi_P int32 [count n]        linear g's own permutation of [0, n) at g n;
 *   y, dy dtype [T, M]          linear g's output in columns [off_g, off_g + m_g);
 *   dx   dtype [T, n]           sum over the group of the input gradients
 *                               (float32 sum, one rounding);
 *   dG_R float32 [M/b, b, b], dG_P float32 [count n/b, b, b], in the G layout.
 * FAST saves the dense products' outputs [T, M] and the gathered inputs [T, count n]
 * (at the next 256-byte boundary); MEM saves nothing.  The dense products of
 * a bf16 group whose m_g and n are multiples of 128 run as one launch. */
#define POETX_MAX_GROUP 8
typedef struct poetx_group_desc {
    int64_t T;        /* tokens, >= 0 */
    int64_t n;        /* width of the shared input (d_in of every linear) */
    int64_t b;        /* block size of every R and P */
    int32_t k;        /* Neumann order */
    int32_t dtype;    /* POETX_F32 or POETX_BF16 */
    int32_t variant;  /* POETX_FAST or POETX_MEM */
    int32_t count;    /* linears in the group, 1 .. POETX_MAX_GROUP */
    int32_t reserved; /* must be 0 */
    int32_t pad;      /* ignored */
    int64_t m[POETX_MAX_GROUP]; /* d_out of each linear (the first `count`); b | m_g */
} poetx_group_desc;
size_t poetx_group_saved_bytes(const poetx_group_desc* g);
size_t poetx_group_fwd_workspace_bytes(const poetx_group_desc* g);
int poetx_group_fwd(const poetx_group_desc* g, const void* x, const void* Wt, const void* G_R,
                    const void* G_P, const int32_t* pi_R, const int32_t* pi_P, void* y, void* saved,
                    void* ws, size_t ws_bytes, void* stream);
size_t poetx_group_bwd_workspace_bytes(const poetx_group_desc* g);
int poetx_group_bwd(const poetx_group_desc* g, const void* dy, const void* x, const void* Wt,
                    const void* G_R, const void* G_P, const int32_t* pi_R, const int32_t* pi_P,
                    const void* saved, void* dx, float* dG_R, float* dG_P, void* ws, size_t ws_bytes,
                    void* stream);

/* ------------------------------------------------------------------ merge */
/* Merge-then-reinitialize (agidaily.cc article; review "merge_then_reinitialize"):
 * with G from q_R / q_P (k = d->k, products in d->dtype),
 *   M   = diag(G_R) . Wt . diag(G_P)      (Wt in the old permuted bases)
 *   Wt' [i][j] = M[s_R[i]][s_P[j]],  s = pi_old^-1 o pi_new
 * so that Wt' = Pi_R' (R W0 P) Pi_P'^T; then q_R and q_P are set to zero.
 * Wt is updated in place (dtype [m, n]); the caller draws pi_new (no RNG in
 * the library) and uses it from then on.  Passing pi_new == pi_old gives a
 * pure fold; with q == 0 as well the call leaves Wt bit-identical.
 * d->T is ignored.  With POETX_MEM_Q8, Wt is the quantized buffer: the merge
 * runs on its bf16 expansion and writes the merged weight back quantized.
 * POETX_FOUR_PERM and POETX_WEIGHT_CENTRIC keep W0 itself, not Wt:
 * POETX_ERR_UNSUPPORTED. */
size_t poetx_merge_workspace_bytes(const poetx_linear_desc* d);
int poetx_merge(const poetx_linear_desc* d, void* Wt, float* q_R, float* q_P,
                const int32_t* pi_R_old, const int32_t* pi_P_old, const int32_t* pi_R_new,
                const int32_t* pi_P_new, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------- quantized weight (mem_q8) */
/* Wq layout: int8 codes [m, n] row-major, then float32 scales [m] at the next
 * 256-byte boundary; poetx_qweight_bytes gives the size (0 for bad sizes).
 * Quantize (W float32 or bf16 [m, n], n % 16 == 0, Wq 16-byte aligned):
 *   scale_i = max_j |W_ij| / 127,  q_ij = nearest integer to W_ij / scale_i (ties
 *   to even) in [-127, 127], computed in float32; a zero row gets scale 0.
 * Dequantize: W (bf16 [m, n]) = bf16(q_ij * scale_i). */
size_t poetx_qweight_bytes(int64_t m, int64_t n);
int poetx_quantize_weight(const void* W, int dtype, int64_t m, int64_t n, void* Wq, void* stream);
int poetx_dequantize_weight(const void* Wq, int64_t m, int64_t n, void* W, void* stream);

/* ------------------------------------------------- building blocks (stages) */
/* The MFMA GEMM every stage of the layer runs on, exposed for composition and
 * per-stage measurement.  C[z] = op(A[z]) op(B[z]) for z < batch, with
 *   POETX_GEMM_NT:  A [M][K] (lda), B [N][K] (ldb)      C = A B^T
 *   POETX_GEMM_NN:  A [M][K] (lda), B [K][N] (ldb)      C = A B
 *   POETX_GEMM_TN:  A [K][M] (lda), B [K][N] (ldb)      C = A^T B
 * C [M][N] (ldc), all of `dtype`, float32 accumulation; strides are the
 * element offsets between batch entries.  The contiguous extent of every
 * operand, every leading dimension and every stride must be a multiple of
 * 16 bytes.  With dense != 0 the call uses the tile schedule of the layer's
 * dense Wt products (batch must be 1), otherwise that of the block products. */
enum { POETX_GEMM_NT = 0, POETX_GEMM_NN = 1, POETX_GEMM_TN = 2 };
int poetx_gemm(int layout, int dtype, int dense, int64_t M, int64_t N, int64_t K, int64_t batch,
               const void* A, int64_t lda, int64_t strideA, const void* B, int64_t ldb, int64_t strideB,
               void* C, int64_t ldc, int64_t strideC, void* stream);

/* Batch-wise block-diagonal product (review Summary: the block-diagonal matmul
 * done per block, never building the sparse matrix): for j < d/b
 *   transpose_G == 1:  out[:, jb:(j+1)b] = in[:, jb:(j+1)b] . G[j]^T
 *   transpose_G == 0:  out[:, jb:(j+1)b] = in[:, jb:(j+1)b] . G[j]
 * in, out: dtype [T, d]; G: dtype [d/b, b, b].  out must not overlap in. */
int poetx_block_apply(int dtype, int transpose_G, int64_t T, int64_t d, int64_t b, const void* in, const void* G,
                      void* out, void* stream);

/* The layer forward's dense product with its R-side block product folded
 * into the same launch (review Summary: the input-centric chain as a few
 * fused products; agidaily article, the operator fusion of the W_RP section):
 *   h2 = h1 . Wt^T,   z[:, jb:(j+1)b] = h2[:, jb:(j+1)b] . G_R[j]^T
 * h1: bf16 [T, n]; Wt: bf16 [m, n]; G_R: bf16 [m/b, b, b]; z: bf16 [T, m];
 * h2: bf16 [T, m], written when not NULL.  b must be 256 and n a multiple of
 * 64 (else POETX_ERR_UNSUPPORTED); dtype must be POETX_BF16.  h2 is rounded to
 * bf16 before the block product, so z equals poetx_gemm (dense NT) followed by
 * poetx_block_apply bit for bit.  z and h2 must not overlap h1 or Wt.
 * poetx_linear_fwd takes this path for bf16 chains with b = 256 whose grid of
 * ceil(T / 128) * m / 256 tiles is a multiple of 256 or at least 1024. */
int poetx_dense_fold_r(int dtype, int64_t T, int64_t m, int64_t n, int64_t b, const void* h1, const void* Wt,
                       const void* G_R, void* h2, void* z, void* stream);

/* Block gradients of the batch-wise block products (the backward of the
 * review's "batch-wise block-diagonal matmul"): for j < d/b
 *   dG[j] = A[:, jb:(j+1)b]^T B[:, jb:(j+1)b]      (sum over the T rows)
 * A, B: dtype [T, d]; dG: float32 [d/b, b, b].  The token axis is split over
 * workgroups and the partial sums are added in a fixed order (deterministic).
 * T == 0 writes zeros. */
size_t poetx_block_grad_workspace_bytes(int64_t T, int64_t d, int64_t b, int dtype);
int poetx_block_grad(int dtype, int64_t T, int64_t d, int64_t b, const void* A, const void* B, float* dG,
                     void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------ training step */
/* The optimizer on the compact parameters (the review's Summary: optimizer
 * state lives on the b(b-1)/2 values per block only; Weaknesses, single-run
 * 8B/13B remark: the POET learning-rate scaling gamma = 0.5 and a reset gap of
 * 400 steps).  The update is decoupled-decay AdamW with bias-corrected moments at
 * the rate eta = lr * gamma (gamma = 0.5 on the pages: R - I is about 2Q, the
 * review's "Cayley approximation" weakness, so q takes half the step):
 *   m = beta1 m + (1 - beta1) dq
 *   v = beta2 v + (1 - beta2) dq^2
 *   q = q - eta ( m / (1 - beta1^step) / (sqrt(v / (1 - beta2^step)) + eps)
 *                 + weight_decay q )
 * The schedule is the caller's: every reset gap updates it calls poetx_merge
 * (which zeroes q) and poetx_adamw_reset on the same parameters, and counts
 * `step` from 1 again. */
typedef struct poetx_adamw_params {
    double lr;           /* base learning rate (finite) */
    double gamma;        /* POET learning-rate scaling (finite; 0.5 on the pages) */
    double beta1, beta2; /* moment decay rates, in [0, 1) */
    double eps;          /* added to the root of the second moment, >= 0 */
    double weight_decay; /* decoupled decay on q, >= 0 (0 keeps q's origin, R = I) */
} poetx_adamw_params;

/* One update of count float32 parameters in place.  q, m, v: float32 [count]
 * (updated); dq: float32 [count] (read).  step >= 1 counts the updates since
 * the last reset.  The four arrays must not overlap (16-byte aligned arrays
 * take the vector path, others a scalar one with identical results).  The
 * arithmetic is float32 with IEEE sqrt and division; the coefficients
 * (1 - beta, the bias corrections, eta) are formed on the host in double from
 * the double parameters and then rounded once, so 1 - beta2 keeps its digits.
 * Non-finite gradients propagate.
 * Errors: p NULL, step < 1, a rate outside its range -> INVALID_ARG;
 * count < 0 or >= 2^31 -> SHAPE; count == 0 does nothing. */
int poetx_adamw_step(float* q, const float* dq, float* m, float* v, int64_t count, int64_t step,
                     const poetx_adamw_params* p, void* stream);

/* m[i] = v[i] = 0 for i < count: the optimizer reset that follows a merge.
 * A fill kernel (no memset node), so a captured graph replays it. */
int poetx_adamw_reset(float* m, float* v, int64_t count, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* POETX_H */
