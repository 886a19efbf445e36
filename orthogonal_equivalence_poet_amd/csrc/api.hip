// libpoetx C ABI: argument validation, workspace planning and the stream-ordered
// kernel sequences of the POET-X layer.  No device memory is allocated here:
// every scratch buffer is carved from the caller's workspace.
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>

#include "dense_gemm.h"
#include "elementwise.h"
#include "gemm.h"
#include "poetx.h"

using namespace poetx;

namespace {

thread_local std::string g_last_hip_error;

int hip_fail(hipError_t e) {
    g_last_hip_error = hipGetErrorString(e);
    return POETX_ERR_HIP;
}

#define HIP_TRY(expr)                                   \
    do {                                                \
        const hipError_t e_ = (expr);                   \
        if (e_ != hipSuccess) return hip_fail(e_);      \
    } while (0)

#define POETX_TRY(expr)                                 \
    do {                                                \
        const int s_ = (expr);                          \
        if (s_ != POETX_OK) return s_;                  \
    } while (0)

constexpr int64_t kMaxExtent = (int64_t(1) << 31) - 1;

// Bump allocator over the caller's workspace; with a null base it only measures.
struct Carver {
    char* base;
    size_t off = 0;
    explicit Carver(void* b) : base(static_cast<char*>(b)) {}
    void* take(size_t bytes) {
        off = (off + 255) & ~size_t(255);
        void* p = base ? base + off : nullptr;
        off += bytes;
        return p;
    }
    template <typename T> T* take_n(int64_t n) { return static_cast<T*>(take(sizeof(T) * (size_t)std::max<int64_t>(n, 0))); }
};

inline bool dtype_ok(int d) { return d == POETX_F32 || d == POETX_BF16; }

// Every tensor the layer entry points take is read or written with 16-byte
// vector accesses (and the direct-to-LDS operand loads): a pointer off that
// alignment is an argument error, not a misaligned access.
inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
template <typename... P>
inline bool all_al16(const P*... p) { return (al16(p) && ...); }
inline size_t esize(int d) { return d == POETX_BF16 ? 2 : 4; }
inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

int check_block(int64_t b) {
    if (b <= 0) return POETX_ERR_SHAPE;
    if (b < 16 || b > 1024 || b % 16 != 0) return POETX_ERR_UNSUPPORTED;
    return POETX_OK;
}

int check_k(int k) { return (k >= 1 && k <= 8) ? POETX_OK : POETX_ERR_UNSUPPORTED; }

int check_nblk(int64_t nblk, int64_t b) {
    if (nblk < 0) return POETX_ERR_SHAPE;
    if (nblk > 0 && nblk > kMaxExtent / (b * b)) return POETX_ERR_SHAPE;
    return POETX_OK;
}

int check_desc(const poetx_linear_desc* d) {
    if (!d) return POETX_ERR_INVALID_ARG;
    if (!dtype_ok(d->dtype) || d->variant < POETX_FAST || d->variant > POETX_MEM_Q8 || d->reserved != 0)
        return POETX_ERR_INVALID_ARG;
    if (d->variant == POETX_MEM_Q8 && d->dtype != POETX_BF16) return POETX_ERR_UNSUPPORTED;
    POETX_TRY(check_block(d->b));
    // the int8 weight feeds products tiled in 64-k steps over both m and n
    if (d->variant == POETX_MEM_Q8 && d->b % 64 != 0) return POETX_ERR_SHAPE;
    POETX_TRY(check_k(d->k));
    if (d->T < 0 || d->m <= 0 || d->n <= 0) return POETX_ERR_SHAPE;
    if (d->m % d->b != 0 || d->n % d->b != 0) return POETX_ERR_SHAPE;
    if (d->T > kMaxExtent || d->m > kMaxExtent || d->n > kMaxExtent) return POETX_ERR_SHAPE;
    return POETX_OK;
}

// ------------------------------------------------------------- GEMM helpers
// Largest workgroup tile that still gives about one workgroup per CU (256 CUs);
// small problems fall through to the 64 x 64 tile.
GemmTile pick_tile(bool bf16, int64_t M, int64_t N, int64_t batch) {
    auto wgs = [&](int64_t tm, int64_t tn) { return ((M + tm - 1) / tm) * ((N + tn - 1) / tn) * std::max<int64_t>(batch, 1); };
    if (bf16) {
        if (M >= 256 && N >= 128 && wgs(256, 128) >= 240) return GemmTile::Large;
        if (M >= 128 && N >= 128 && wgs(128, 128) >= 240) return GemmTile::Medium;
        return GemmTile::Small;
    }
    if (M >= 128 && N >= 128 && wgs(128, 128) >= 240) return GemmTile::Medium;
    return GemmTile::Small;
}

struct Mat {
    const void* p;
    int64_t ld;
    int64_t stride;
};

// Products of small matrices (the Cayley-Neumann b x b products): bf16 operands
// that meet the direct-to-LDS load rules go to the pipelined kernel with the
// general epilogue, everything else to the register-staged kernel.
hipError_t small_gemm(const GemmArgs& g, GemmLayout layout, bool cbf16, bool obf16, hipStream_t s) {
    const bool a_mn = layout == GemmLayout::TN;
    const bool b_mn = layout != GemmLayout::NT;
    const bool aligned = ((uintptr_t)g.A | (uintptr_t)g.B) % 16 == 0;
    if (cbf16 && aligned && g.M <= 1024 && g.N <= 1024 && g.splits == 1 &&
        pipe_gemm_supported(a_mn, b_mn, g.M, g.N, g.K, g.lda, g.ldb, g.strideA, g.strideB)) {
        PipeArgs p;
        p.A = g.A; p.lda = g.lda; p.strideA = g.strideA;
        p.B = g.B; p.ldb = g.ldb; p.strideB = g.strideB;
        p.C = g.C; p.ldc = g.ldc; p.strideC = g.strideC;
        p.C2 = g.C2; p.C3 = g.C3; p.ldc2 = g.ldc2; p.strideC2 = g.strideC2;
        p.Cin1 = g.Cin1; p.ldcin1 = g.ldcin1; p.strideCin1 = g.strideCin1;
        p.Cin2 = g.Cin2; p.ldcin2 = g.ldcin2; p.strideCin2 = g.strideCin2;
        p.alpha = g.alpha; p.beta1 = g.beta1; p.beta2 = g.beta2; p.gamma = g.gamma; p.mode = g.mode;
        p.M = g.M; p.N = g.N; p.K = g.K;
        p.batch = g.batch;
        p.k_per_split = g.K;
        return pipe_gemm_general(a_mn, b_mn, !obf16, p, s);
    }
    return gemm_launch(g, layout, pick_tile(cbf16, g.M, g.N, g.batch), cbf16, obf16, s);
}

hipError_t gemm(GemmLayout layout, bool cbf16, bool obf16, int64_t M, int64_t N, int64_t K, int64_t batch, Mat A,
                Mat B, void* C, int64_t ldc, int64_t sC, hipStream_t s, float alpha = 1.f,
                const float* cin1 = nullptr, float beta1 = 0.f, const float* cin2 = nullptr, float beta2 = 0.f,
                float gamma = 0.f, void* C2 = nullptr, bool dense = false) {
    GemmArgs g;
    g.A = A.p; g.lda = A.ld; g.strideA = A.stride;
    g.B = B.p; g.ldb = B.ld; g.strideB = B.stride;
    g.C = C; g.ldc = ldc; g.strideC = sC;
    g.C2 = C2; g.ldc2 = ldc; g.strideC2 = sC;
    g.Cin1 = cin1; g.ldcin1 = ldc; g.strideCin1 = sC; g.beta1 = beta1;
    g.Cin2 = cin2; g.ldcin2 = ldc; g.strideCin2 = sC; g.beta2 = beta2;
    g.alpha = alpha; g.gamma = gamma;
    g.M = (int)M; g.N = (int)N; g.K = (int)K;
    g.batch = (int)batch;
    g.splits = 1;
    g.k_per_split = (int)std::max<int64_t>(K, 1);
    if (!dense) return small_gemm(g, layout, cbf16, obf16, s);
    return gemm_launch(g, layout, pick_tile(cbf16, M, N, batch), cbf16, obf16, s);
}

// The dense Wt products of the chain: [T, K] x Wt (NT forward, NN backward).
hipError_t dense_gemm(GemmLayout layout, bool bf, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                      const void* B, int64_t ldb, void* C, int64_t ldc, hipStream_t s) {
    if (bf && layout != GemmLayout::TN && dense_gemm_supported(M, N, K, lda, ldb) && ldc % 8 == 0)
        return dense_gemm_bf16(layout == GemmLayout::NN, A, lda, B, ldb, C, ldc, (int)M, (int)N, (int)K, s);
    return gemm(layout, bf, bf, M, N, K, 1, Mat{A, lda, 0}, Mat{B, ldb, 0}, C, ldc, 0, s, 1.f, nullptr, 0, nullptr,
                0, 0, nullptr, true);
}

// Square b x b block products over nblk blocks stored back to back.
struct BlkMat {
    const void* p;
};
inline Mat sq(const void* p, int64_t b) { return Mat{p, b, b * b}; }

// --------------------------------------------------- Cayley-Neumann planning
// Buffers of one Cayley-Neumann call ([nblk, b, b] each).  "32" buffers are
// float32; "c" buffers hold the operand copy in the compute dtype (bf16 on the
// bf16 path; on the float32 path a c buffer is its own float32 buffer or an
// alias of the matching 32 buffer).
struct CnpBufs {
    float* Q32 = nullptr; void* Qc = nullptr;
    // k = 3: U32 = 2Q + 2S, Sc = S, Tc = 2Q + S (one fused epilogue)
    float* U32 = nullptr; void* Sc = nullptr; void* Tc = nullptr;
    // k = 4: S, P1 = Q + S (bf16 path: only its compute copy), E = P1 + P1 S, W (backward scratch)
    float* S32 = nullptr; float* P32 = nullptr; void* Pc = nullptr; float* E32 = nullptr; void* Ec = nullptr;
    float* W32 = nullptr;
    // Horner (other k): D_1..D_k
    float* D32[9] = {}; void* Dc[9] = {};
    // backward scratch
    void* dGc = nullptr;
    float* a32 = nullptr; float* b32 = nullptr; void* c_c = nullptr; void* d_c = nullptr;
    float* e32 = nullptr; float* f32 = nullptr; float* g32 = nullptr;
};

// The compute-dtype copy of a float32 buffer: its own buffer for bf16, the
// float32 buffer itself otherwise.
void* ctake(Carver& cv, bool cbf16, int64_t elems, float* alias32) {
    return cbf16 ? cv.take(2 * (size_t)elems) : static_cast<void*>(alias32);
}
// A compute-dtype buffer of its own.
void* cown(Carver& cv, bool cbf16, int64_t elems) { return cv.take((cbf16 ? 2 : 4) * (size_t)elems); }

// The prologue's outputs (Q, the square and its companions) come from `sv`,
// everything else from `cv`; `sv` is the caller's saved buffer when the
// forward keeps them for the backward, else the workspace itself.
void plan_cnp(Carver& cv, Carver& sv, int64_t nblk, int64_t b, int k, bool cbf16, bool backward, CnpBufs& B) {
    const int64_t e = nblk * b * b;
    B.Q32 = sv.take_n<float>(e);
    B.Qc = ctake(sv, cbf16, e, B.Q32);
    if (k == 3) {
        B.U32 = sv.take_n<float>(e);
        B.Sc = cown(sv, cbf16, e);
        B.Tc = cown(sv, cbf16, e);
    } else if (k == 4) {
        B.S32 = sv.take_n<float>(e);
        B.Sc = ctake(sv, cbf16, e, B.S32);
        // bf16: P1 comes out of the square's epilogue and is kept with it;
        // float32: P1 is formed in its own pass
        if (cbf16) {
            B.Pc = sv.take(2 * (size_t)e);
        } else {
            B.P32 = cv.take_n<float>(e);
            B.Pc = B.P32;
        }
        B.E32 = cv.take_n<float>(e);
        B.Ec = ctake(cv, cbf16, e, B.E32);
        B.W32 = cv.take_n<float>(e);
    } else {
        B.D32[1] = B.Q32;
        B.Dc[1] = B.Qc;
        const int keep = backward ? k : std::min(k, 3);
        for (int i = 2; i <= keep; ++i) {
            B.D32[i] = cv.take_n<float>(e);
            B.Dc[i] = ctake(cv, cbf16, e, B.D32[i]);
        }
    }
    if (backward) {
        B.a32 = cv.take_n<float>(e);
        B.b32 = cv.take_n<float>(e);
        B.c_c = cown(cv, cbf16, e);
        B.d_c = cown(cv, cbf16, e);
        B.e32 = cv.take_n<float>(e);
        B.f32 = cv.take_n<float>(e);
        B.g32 = cv.take_n<float>(e);
        B.dGc = cbf16 ? cv.take(2 * (size_t)e) : nullptr;
    }
}

// Shared front part: Q in float32 and in the compute dtype (one pass), and the
// square S = Q Q = -Q Q^T.  For k = 3 the square's epilogue also emits
// Tc = 2Q + S and U = 2Q + 2S; for k = 4 it emits S (float32 and compute) and,
// on the bf16 path, P1 = Q + S in bf16 (float32: a separate pass).
int cnp_prologue(const float* q, int64_t nblk, int64_t b, int k, bool cbf16, CnpBufs& B, hipStream_t s) {
    HIP_TRY(skew_unpack(q, B.Q32, false, nblk, (int)b, s, cbf16 ? B.Qc : nullptr));
    if (k == 3) {
        GemmArgs g;
        g.A = B.Qc; g.lda = b; g.strideA = b * b;
        g.B = B.Qc; g.ldb = b; g.strideB = b * b;
        g.C = B.U32; g.ldc = b; g.strideC = b * b;
        g.C2 = B.Sc; g.ldc2 = b; g.strideC2 = b * b;
        g.C3 = B.Tc;
        g.Cin1 = B.Q32; g.ldcin1 = b; g.strideCin1 = b * b;
        g.alpha = -1.f;
        g.mode = 1;
        g.M = g.N = g.K = (int)b;
        g.batch = (int)nblk;
        g.k_per_split = (int)b;
        HIP_TRY(small_gemm(g, GemmLayout::NT, cbf16, false, s));
    } else if (k == 4) {
        if (cbf16) {
            GemmArgs g;
            g.A = B.Qc; g.lda = b; g.strideA = b * b;
            g.B = B.Qc; g.ldb = b; g.strideB = b * b;
            g.C = B.S32; g.ldc = b; g.strideC = b * b;
            g.C2 = B.Sc; g.ldc2 = b; g.strideC2 = b * b;
            g.C3 = B.Pc;
            g.Cin1 = B.Q32; g.ldcin1 = b; g.strideCin1 = b * b;
            g.alpha = -1.f;
            g.mode = 3;
            g.M = g.N = g.K = (int)b;
            g.batch = (int)nblk;
            g.k_per_split = (int)b;
            HIP_TRY(small_gemm(g, GemmLayout::NT, cbf16, false, s));
        } else {
            HIP_TRY(gemm(GemmLayout::NT, cbf16, false, b, b, b, nblk, sq(B.Qc, b), sq(B.Qc, b), B.S32, b, b * b, s,
                         -1.f));
            HIP_TRY(combine(nblk, (int)b, B.Q32, 1.f, B.S32, 1.f, nullptr, 0, 0, B.P32, nullptr, false, s));
        }
    }
    return POETX_OK;
}

// Batches from which the k = 3, b = 256 forward (bf16) takes one block per
// workgroup instead of one 32- or 64-row panel per workgroup: one workgroup
// takes about 24 us on its block, the panels spread a few blocks over more CUs
// (64 blocks: 17 us against 27); from about a hundred blocks on the two are even
// (96 to 128: 28 to 31 us both) and building each block's Q image once then
// pulls ahead (160: 34 against 40 us; 15280: 2.5 against 4.2 ms).
constexpr int64_t kBlockFwdMinBlocks = 96;

// Forward Cayley-Neumann schedules.  k = 3: G = I + 2Q + 2S + (2Q + S) S.
// k = 4: E = (Q + S) + (Q + S) S, G = I + Q + E + Q E.  Other k: Horner,
// D_1 = Q, D_{i+1} = Q + Q D_i, G = I + Q + D_k + Q D_k.  Every product is a
// correction term; the leading terms are added in float32 by the epilogue.
int cnp_forward(const float* q, int64_t nblk, int64_t b, int k, bool cbf16, void* G, bool gbf16, CnpBufs& B,
                bool save, hipStream_t s) {
    if (cbf16 && gbf16 && k == 3 && b == 256 && nblk >= kBlockFwdMinBlocks && all_al16(G, B.Sc, B.Tc, B.Qc)) {
        // one block per workgroup: Q built once per block, S and T through memory
        // (the saving forward keeps them; otherwise the workspace holds them)
        HIP_TRY(cnp_fwd_block(q, G, save ? B.Qc : nullptr, B.Sc, B.Tc, nblk, (int)b, s));
        return POETX_OK;
    }
    if (cbf16 && gbf16 && cnp_fused_supported(b, k) && (!save || k == 3) && (reinterpret_cast<uintptr_t>(G) & 15) == 0) {
        // bf16 blocks of 128 or 256: one kernel from the packed parameters to G,
        // every power of Q formed per panel on chip (the saving forward also
        // keeps Q, S and 2Q + S in bf16 for the backward)
        HIP_TRY(cnp_fused_fwd(q, G, save ? B.Qc : nullptr, save ? B.Sc : nullptr, save ? B.Tc : nullptr, nblk, b, k,
                              s));
        return POETX_OK;
    }
    POETX_TRY(cnp_prologue(q, nblk, b, k, cbf16, B, s));
    const int ib = (int)b;
    const int64_t bb = b * b;
    if (k == 3) {
        HIP_TRY(gemm(GemmLayout::NT, cbf16, gbf16, b, b, b, nblk, sq(B.Tc, b), sq(B.Sc, b), G, b, bb, s, 1.f,
                     B.U32, 1.f, nullptr, 0, 1.f));
    } else if (k == 4) {
        // E = P1 + P1 S with P1 = Q + S taken as two addends; G = I + Q + E + Q E
        HIP_TRY(gemm(GemmLayout::NT, cbf16, false, b, b, b, nblk, sq(B.Pc, b), sq(B.Sc, b), B.E32, b, bb, s, 1.f,
                     B.Q32, 1.f, B.S32, 1.f, 0, cbf16 ? B.Ec : nullptr));
        HIP_TRY(gemm(GemmLayout::NN, cbf16, gbf16, b, b, b, nblk, sq(B.Qc, b), sq(B.Ec, b), G, b, bb, s, 1.f,
                     B.Q32, 1.f, B.E32, 1.f, 1.f));
    } else {
        // rolling D buffers: slots 1 (= Q), 2, 3
        int cur = 1;
        for (int i = 1; i < k; ++i) {
            const int nxt = (cur == 2) ? 3 : 2;
            HIP_TRY(gemm(GemmLayout::NN, cbf16, false, b, b, b, nblk, sq(B.Qc, b), sq(B.Dc[cur], b), B.D32[nxt], b,
                         bb, s, 1.f, B.Q32, 1.f, nullptr, 0, 0, cbf16 ? B.Dc[nxt] : nullptr));
            cur = nxt;
        }
        HIP_TRY(gemm(GemmLayout::NN, cbf16, gbf16, b, b, b, nblk, sq(B.Qc, b), sq(B.Dc[cur], b), G, b, bb, s, 1.f,
                     B.Q32, 1.f, B.D32[cur], 1.f, 1.f));
    }
    return POETX_OK;
}

// Batches from which the k = 3, b = 256 backward takes one block per workgroup
// instead of the two passes over tile units.  A lone workgroup takes about
// 54 us on its block, the passes spread a few blocks over the whole chip
// (32 blocks: 23 us; 128: 61 against 63 us); from about 150 blocks on, the
// per-block kernel moves fewer bytes and is ahead (160: 67 against 74 us; 256:
// 84 against 108 us; 15280: 4.8 against 7.7 ms).
constexpr int64_t kBlockBwdMinBlocks = 144;

// Adjoint schedules (reverse of the forward ones), ending with the skew pack.
int cnp_backward(const float* q, const float* dG, int64_t nblk, int64_t b, int k, bool cbf16, float* dq,
                 CnpBufs& B, bool saved, hipStream_t s) {
    if (!saved) POETX_TRY(cnp_prologue(q, nblk, b, k, cbf16, B, s));
    const int ib = (int)b;
    const int64_t bb = b * b;
    if (cbf16 && k == 3 && b == 256 && nblk >= kBlockBwdMinBlocks && all_al16(dG, B.Sc, B.Tc, B.Qc, B.dGc)) {
        // one block per workgroup: every intermediate on chip, dG read as float32
        // and kept as bf16 in the scratch of its compute copy
        HIP_TRY(cnp_bwd_block(dG, B.Sc, B.Tc, B.Qc, B.dGc, dq, nblk, ib, s));
        return POETX_OK;
    }
    const bool dual = cbf16 && b % 64 == 0 && pipe_gemm_supported(false, false, b, b, b, b, b, bb, bb) &&
                      pipe_gemm_supported(true, true, b, b, b, b, b, bb, bb);
    if (k == 3 && dual && al16(dG)) {
        // Only the skew part of dQ reaches dq: with X1 = dG S, X2 = T^T dG,
        // dS = 2 dG + X1 + X2 and Sigma = dS + dS^T (symmetric),
        // dQ - dQ^T = 2 (dA - dA^T) - (P - P^T) with dA = dG + X1, P = Sigma Q,
        // since Q Sigma = -(Sigma Q)^T.  Pass 1 (which rounds dG to bf16 on
        // chip) writes Sigma and the packed 2 (dA - dA^T); pass 2 adds the
        // packed -(P - P^T).  Three products instead of four; the pack rides on
        // both passes.
        HIP_TRY(cnp_bwd_sym(dG, B.Sc, B.Tc, B.c_c, dq, nblk, ib, s));
        HIP_TRY(cnp_bwd_sigq(B.c_c, B.Qc, dq, nblk, ib, s));
        return POETX_OK;
    }
    const void* dGc = dG;
    if (cbf16) {
        HIP_TRY(combine(nblk, ib, dG, 1.f, nullptr, 0, nullptr, 0, 0, nullptr, B.dGc, true, s));
        dGc = B.dGc;
    }
    float* dQ = B.g32;
    bool packed = false;   // dq already written by the last product pair
    if (k == 3) {
        // G = A B with A = I + T, B = I + S (T = 2Q + S, S symmetric):
        // dA = dG + dG S ;  dS = dA + dB with dB = dG + T^T dG ;  dQ = 2 dA + dS Q^T + Q^T dS
        HIP_TRY(gemm(GemmLayout::NT, cbf16, false, b, b, b, nblk, sq(dGc, b), sq(B.Sc, b), B.a32, b, bb, s, 1.f, dG,
                     1.f));
        HIP_TRY(gemm(GemmLayout::TN, cbf16, false, b, b, b, nblk, sq(B.Tc, b), sq(dGc, b), nullptr, b, bb, s, 1.f,
                     dG, 1.f, B.a32, 1.f, 0.f, B.c_c));
        HIP_TRY(gemm(GemmLayout::NT, cbf16, false, b, b, b, nblk, sq(B.c_c, b), sq(B.Qc, b), B.e32, b, bb, s, 1.f,
                     B.a32, 2.f));
        HIP_TRY(gemm(GemmLayout::TN, cbf16, false, b, b, b, nblk, sq(B.Qc, b), sq(B.c_c, b), dQ, b, bb, s, 1.f,
                     B.e32, 1.f));
    } else if (k == 4) {
        // recompute E = P1 + P1 S (P1 = Q + S came with the square; a float32
        // P1 lives in the workspace, so a saved backward forms it again)
        if (!cbf16 && saved)
            HIP_TRY(combine(nblk, ib, B.Q32, 1.f, B.S32, 1.f, nullptr, 0, 0, B.P32, nullptr, false, s));
        HIP_TRY(gemm(GemmLayout::NT, cbf16, false, b, b, b, nblk, sq(B.Pc, b), sq(B.Sc, b), B.E32, b, bb, s, 1.f,
                     B.Q32, 1.f, B.S32, 1.f, 0, cbf16 ? B.Ec : nullptr));
        // X1 = dG + dG E^T ; dE = dG + Q^T dG
        HIP_TRY(gemm(GemmLayout::NT, cbf16, false, b, b, b, nblk, sq(dGc, b), sq(B.Ec, b), B.a32, b, bb, s, 1.f, dG,
                     1.f));
        HIP_TRY(gemm(GemmLayout::TN, cbf16, false, b, b, b, nblk, sq(B.Qc, b), sq(dGc, b), B.b32, b, bb, s, 1.f, dG,
                     1.f, nullptr, 0, 0, cbf16 ? B.c_c : nullptr));
        const void* dEc = cbf16 ? B.c_c : static_cast<void*>(B.b32);
        if (dual) {
            // the last four products paired per launch, as for k = 3:
            // dP1 = dE + dE S (float32) and dS = dP1 + P1^T dE (bf16) from one,
            // dQ = X1 + dP1 + dS Q^T + Q^T dS from the other
            PipeArgs d;
            d.A = dEc; d.lda = b; d.strideA = bb;
            d.B = B.Sc; d.ldb = b; d.strideB = bb;
            d.A2 = B.Pc; d.lda2 = b; d.strideA2 = bb;
            d.B2 = dEc; d.ldb2 = b; d.strideB2 = bb;
            d.C = B.e32; d.ldc = b; d.strideC = bb;
            d.C2 = B.d_c; d.ldc2 = b; d.strideC2 = bb;
            d.Cin1 = B.b32; d.ldcin1 = b; d.strideCin1 = bb;
            d.beta1 = 1.f; d.beta2 = 1.f;
            d.M = d.N = d.K = ib;
            d.batch = (int)nblk;
            d.k_per_split = ib;
            HIP_TRY(pipe_gemm_dual(true, true, d, s));
            PipeArgs e;
            e.A = B.d_c; e.lda = b; e.strideA = bb;
            e.B = B.Qc; e.ldb = b; e.strideB = bb;
            e.A2 = B.Qc; e.lda2 = b; e.strideA2 = bb;
            e.B2 = B.d_c; e.ldb2 = b; e.strideB2 = bb;
            e.C = dQ; e.ldc = b; e.strideC = bb;
            e.Cin1 = B.a32; e.ldcin1 = b; e.strideCin1 = bb; e.beta1 = 1.f;
            e.Cin2 = B.e32; e.ldcin2 = b; e.strideCin2 = bb; e.beta2 = 1.f;
            e.M = e.N = e.K = ib;
            e.batch = (int)nblk;
            e.k_per_split = ib;
            HIP_TRY(cnp_pack_pair(e, dq, ib, s));
            packed = true;
        } else {
            // dP1 = dE + dE S ; dS = P1^T dE + dP1
            HIP_TRY(gemm(GemmLayout::NT, cbf16, false, b, b, b, nblk, sq(dEc, b), sq(B.Sc, b), B.e32, b, bb, s, 1.f,
                         B.b32, 1.f));
            HIP_TRY(gemm(GemmLayout::TN, cbf16, false, b, b, b, nblk, sq(B.Pc, b), sq(dEc, b), nullptr, b, bb, s,
                         1.f, B.e32, 1.f, nullptr, 0, 0, B.d_c));
            // dQ = X1 + dP1 + dS Q^T + Q^T dS
            HIP_TRY(gemm(GemmLayout::NT, cbf16, false, b, b, b, nblk, sq(B.d_c, b), sq(B.Qc, b), B.W32, b, bb, s,
                         1.f, B.a32, 1.f, B.e32, 1.f));
            HIP_TRY(gemm(GemmLayout::TN, cbf16, false, b, b, b, nblk, sq(B.Qc, b), sq(B.d_c, b), dQ, b, bb, s, 1.f,
                         B.W32, 1.f));
        }
    } else {
        // recompute D_2..D_k (D_1 = Q)
        for (int i = 1; i < k; ++i)
            HIP_TRY(gemm(GemmLayout::NN, cbf16, false, b, b, b, nblk, sq(B.Qc, b), sq(B.Dc[i], b), B.D32[i + 1], b,
                         bb, s, 1.f, B.Q32, 1.f, nullptr, 0, 0, cbf16 ? B.Dc[i + 1] : nullptr));
        // G = I + Q + D_k + Q D_k:  acc = dG + dG D_k^T,  dD_k = dG + Q^T dG
        float* acc = B.e32;
        HIP_TRY(gemm(GemmLayout::NT, cbf16, false, b, b, b, nblk, sq(dGc, b), sq(B.Dc[k], b), acc, b, bb, s, 1.f,
                     dG, 1.f));
        float* dD32[2] = {B.a32, B.b32};
        void* dDc[2] = {B.c_c, B.d_c};
        int cur = 0;
        HIP_TRY(gemm(GemmLayout::TN, cbf16, false, b, b, b, nblk, sq(B.Qc, b), sq(dGc, b), dD32[cur], b, bb, s, 1.f,
                     dG, 1.f, nullptr, 0, 0, cbf16 ? dDc[cur] : nullptr));
        for (int i = k - 1; i >= 1; --i) {
            const void* cur_c = cbf16 ? dDc[cur] : static_cast<void*>(dD32[cur]);
            // D_{i+1} = Q + Q D_i:  acc += dD_{i+1} + dD_{i+1} D_i^T ;  dD_i = Q^T dD_{i+1}
            HIP_TRY(gemm(GemmLayout::NT, cbf16, false, b, b, b, nblk, sq(cur_c, b), sq(B.Dc[i], b), B.f32, b, bb, s,
                         1.f, acc, 1.f, dD32[cur], 1.f));
            std::swap(acc, B.f32);
            const int nxt = cur ^ 1;
            HIP_TRY(gemm(GemmLayout::TN, cbf16, false, b, b, b, nblk, sq(B.Qc, b), sq(cur_c, b), dD32[nxt], b, bb, s,
                         1.f, nullptr, 0, nullptr, 0, 0, cbf16 ? dDc[nxt] : nullptr));
            cur = nxt;
        }
        // D_1 = Q: acc += dD_1
        HIP_TRY(combine(nblk, ib, acc, 1.f, dD32[cur], 1.f, nullptr, 0, 0, dQ, nullptr, false, s));
    }
    if (!packed) HIP_TRY(skew_pack(dQ, dq, nblk, ib, s));
    return POETX_OK;
}

// Workspace of one Cayley-Neumann call (with_saved: the prologue outputs live
// in a separate saved buffer) and the size of that saved buffer.
size_t cnp_ws(int64_t nblk, int64_t b, int k, bool cbf16, bool backward, bool with_saved = false) {
    Carver cv(nullptr), sv(nullptr);
    CnpBufs B;
    plan_cnp(cv, with_saved ? sv : cv, nblk, b, k, cbf16, backward, B);
    return cv.off;
}

size_t cnp_saved(int64_t nblk, int64_t b, int k, bool cbf16) {
    Carver cv(nullptr), sv(nullptr);
    CnpBufs B;
    plan_cnp(cv, sv, nblk, b, k, cbf16, true, B);
    return sv.off;
}

// -------------------------------------------------------------- the layer
struct LinearBufs {
    void* buf[3] = {};
    float* part = nullptr;
    int splits_R = 1, splits_P = 1;
    int64_t kps_R = 0, kps_P = 0;
};

// Split-K plan for dG = A^T B with K = T: enough workgroups to cover the chip.
// Tile of the block-gradient products (M = N = b, K = tokens, split along K).
GemmTile grad_tile(bool bf16, int64_t b) {
    if (bf16 && b >= 256) return GemmTile::Large;
    if (b >= 128) return GemmTile::Medium;
    return GemmTile::Small;
}

// Block gradients of bf16 blocks of b >= 64 run on the pipelined kernel
// (64 x 64 tiles, transposed LDS reads for both operands).
bool grad_pipe(bool bf16, int64_t b) { return bf16 && b >= 64 && b % 8 == 0; }

void plan_splits(int64_t T, int64_t b, int64_t nblk, bool bf16, int& splits, int64_t& kps) {
    const GemmTile tile = grad_tile(bf16, b);
    const bool pipe = grad_pipe(bf16, b);
    const int64_t tr = pipe ? pipe_tile_rows(PipeTile::Small) : gemm_tile_rows(tile, bf16);
    const int64_t tc = pipe ? pipe_tile_cols(PipeTile::Small) : gemm_tile_cols(tile, bf16);
    const int64_t tiles = ((b + tr - 1) / tr) * ((b + tc - 1) / tc) * nblk;
    // pipelined 64 x 64 tiles: split the token axis only until about one
    // workgroup per CU, keeping at least 512 tokens per split; register-staged
    // tiles: about four workgroups per CU
    const int64_t target = pipe ? 256 : 1024;
    int64_t want = std::max<int64_t>(1, (target + tiles - 1) / tiles);
    want = std::min<int64_t>(want, std::max<int64_t>(1, T / (pipe ? 512 : 256)));
    int64_t k = (T + want - 1) / want;
    k = std::max<int64_t>(64, (k + 63) / 64 * 64);
    kps = k;
    splits = (int)std::max<int64_t>(1, (T + k - 1) / k);
}

void plan_linear(Carver& cv, const poetx_linear_desc* d, bool backward, LinearBufs& L) {
    const int64_t wide = std::max(d->m, d->n);
    const size_t es = esize(d->dtype);
    const int nb = backward ? 3 : 2;
    for (int i = 0; i < nb; ++i) L.buf[i] = cv.take(es * (size_t)(d->T * wide));
    if (backward) {
        const bool bf = d->dtype == POETX_BF16;
        plan_splits(d->T, d->b, d->m / d->b, bf, L.splits_R, L.kps_R);
        plan_splits(d->T, d->b, d->n / d->b, bf, L.splits_P, L.kps_P);
        const int64_t pr = L.splits_R > 1 ? L.splits_R * d->m * d->b : 0;
        const int64_t pp = L.splits_P > 1 ? L.splits_P * d->n * d->b : 0;
        L.part = cv.take_n<float>(std::max(pr, pp));
    }
}

// Batched block product over the feature axis of a [T, d] activation:
// out[:, jb:(j+1)b] = in[:, jb:(j+1)b] . G_j^T (NT) or . G_j (NN).
hipError_t block_apply(GemmLayout layout, bool bf16, int64_t T, int64_t d, int64_t b, const void* in,
                       const void* G, void* out, hipStream_t s, const float* colscale = nullptr) {
    const bool nn = layout == GemmLayout::NN;
    if (colscale && !(bf16 && nn && pipe_gemm_supported(false, nn, T, b, b, d, b, b, b * b)))
        return hipErrorInvalidValue;
    if (bf16 && pipe_gemm_supported(false, nn, T, b, b, d, b, b, b * b)) {
        PipeArgs p;
        p.A = in; p.lda = d; p.strideA = b;
        p.B = G; p.ldb = b; p.strideB = b * b;
        p.C = out; p.ldc = d; p.strideC = b;
        p.M = (int)T; p.N = (int)b; p.K = (int)b;
        p.batch = (int)(d / b);
        p.k_per_split = (int)b;
        // b >= 256: the largest of 256 x 256, 128 x 256 and 64 x 128 whose grid
        // still gives every CU a workgroup (as for the dense products; measured
        // on 1024- to 14336-wide activations at 2048 to 8192 tokens)
        auto tiles = [&](int64_t bm, int64_t bn) { return ((T + bm - 1) / bm) * ((b + bn - 1) / bn) * (d / b); };
        PipeTile t = PipeTile::Tall;
        if (b >= 256)
            t = tiles(256, 256) >= 256 ? PipeTile::Big : tiles(128, 256) >= 256 ? PipeTile::Wide : PipeTile::Slim;
        if (colscale) {
            // out[:, c] *= colscale[c]: block j's columns start at j b
            p.colscale = colscale;
            p.strideScale = b;
            return pipe_gemm_colscale(p, s, t);
        }
        return pipe_gemm(false, nn, false, p, s, t);
    }
    return gemm(layout, bf16, bf16, T, b, b, d / b, Mat{in, d, b}, Mat{G, b, b * b}, out, d, b, s);
}

// dG_j = A_j^T B_j over the T rows, split along T; partials reduced in order.
int block_grad(bool bf16, int64_t T, int64_t d, int64_t b, const void* A, const void* B, float* dG, int splits,
               int64_t kps, float* part, hipStream_t s) {
    if (grad_pipe(bf16, b)) {
        PipeArgs p;
        p.A = A; p.lda = d; p.strideA = b;
        p.B = B; p.ldb = d; p.strideB = b;
        p.C = splits > 1 ? static_cast<void*>(part) : static_cast<void*>(dG);
        p.ldc = b; p.strideC = b * b;
        p.strideSplit = d * b;  // nblk * b * b
        p.M = (int)b; p.N = (int)b; p.K = (int)T;
        p.batch = (int)(d / b);
        p.splits = splits;
        p.k_per_split = (int)kps;
        HIP_TRY(pipe_gemm(true, true, true, p, s, PipeTile::Small));
        if (splits > 1) HIP_TRY(splitk_reduce(part, dG, d * b, splits, s));
        return POETX_OK;
    }
    GemmArgs g;
    g.A = A; g.lda = d; g.strideA = b;
    g.B = B; g.ldb = d; g.strideB = b;
    g.ldc = b; g.strideC = b * b;
    g.M = (int)b; g.N = (int)b; g.K = (int)T;
    g.batch = (int)(d / b);
    g.splits = splits;
    g.k_per_split = (int)kps;
    if (splits > 1) {
        g.C = part;
        g.strideSplit = d * b;  // nblk * b * b
    } else {
        g.C = dG;
    }
    HIP_TRY(gemm_launch(g, GemmLayout::TN, grad_tile(bf16, b), bf16, false, s));
    if (splits > 1) HIP_TRY(splitk_reduce(part, dG, d * b, splits, s));
    return POETX_OK;
}

// FAST keeps h2 [T, m] and a = x gathered by pi_P [T, n] in `saved`, a at this
// 256-byte aligned offset.
size_t fast_saved_a_offset(const poetx_linear_desc* d) {
    return (esize(d->dtype) * (size_t)(d->T * d->m) + 255) & ~size_t(255);
}

// ------------------------------------------------- four-permutation chain
// The chain over W0 itself, all four permutations applied to the activations:
// y_t = Pi_R^T D_R Pi_R W0 Pi_P^T D_P Pi_P x_t.
int four_perm_forward(const poetx_linear_desc* d, const void* x, const void* W0, const void* G_R, const void* G_P,
                      const int32_t* pi_R, const int32_t* pi_P, void* y, void* h2g, void* a, void* buf0, void* buf1,
                      hipStream_t s) {
    const bool bf = d->dtype == POETX_BF16;
    const int64_t T = d->T, m = d->m, n = d->n, b = d->b;
    // a = Pi_P x;  h1 = D_P a;  Pi_P^T h1
    HIP_TRY(permute_2d(x, a, bf, T, n, nullptr, pi_P, false, s));
    HIP_TRY(block_apply(GemmLayout::NT, bf, T, n, b, a, G_P, buf1, s));
    HIP_TRY(permute_2d(buf1, buf0, bf, T, n, nullptr, pi_P, true, s));
    // h2 = W0 (Pi_P^T h1);  Pi_R h2 (saved)
    HIP_TRY(dense_gemm(GemmLayout::NT, bf, T, m, n, buf0, n, W0, n, buf1, m, s));
    HIP_TRY(permute_2d(buf1, h2g, bf, T, m, nullptr, pi_R, false, s));
    // z = D_R Pi_R h2;  y = Pi_R^T z
    HIP_TRY(block_apply(GemmLayout::NT, bf, T, m, b, h2g, G_R, buf0, s));
    HIP_TRY(permute_2d(buf0, y, bf, T, m, nullptr, pi_R, true, s));
    return POETX_OK;
}

int four_perm_backward(const poetx_linear_desc* d, const void* dy, const void* W0, const void* G_R, const void* G_P,
                       const int32_t* pi_R, const int32_t* pi_P, const void* h2g, const void* a, void* dx,
                       float* dG_R, float* dG_P, const LinearBufs& L, hipStream_t s) {
    const bool bf = d->dtype == POETX_BF16;
    const int64_t T = d->T, m = d->m, n = d->n, b = d->b;
    void* b1 = L.buf[1];
    void* b2 = L.buf[2];
    // dz = Pi_R dy;  dG_R[j] = dz_j^T (Pi_R h2)_j;  Pi_R^T (dz D_R)
    HIP_TRY(permute_2d(dy, b1, bf, T, m, nullptr, pi_R, false, s));
    POETX_TRY(block_grad(bf, T, m, b, b1, h2g, dG_R, L.splits_R, L.kps_R, L.part, s));
    HIP_TRY(block_apply(GemmLayout::NN, bf, T, m, b, b1, G_R, b2, s));
    HIP_TRY(permute_2d(b2, b1, bf, T, m, nullptr, pi_R, true, s));
    // dh1 = Pi_P (dh2 W0);  dG_P[j] = dh1_j^T a_j;  dx = Pi_P^T (dh1 D_P)
    HIP_TRY(dense_gemm(GemmLayout::NN, bf, T, n, m, b1, m, W0, n, b2, n, s));
    HIP_TRY(permute_2d(b2, b1, bf, T, n, nullptr, pi_P, false, s));
    POETX_TRY(block_grad(bf, T, n, b, b1, a, dG_P, L.splits_P, L.kps_P, L.part, s));
    HIP_TRY(block_apply(GemmLayout::NN, bf, T, n, b, b1, G_P, b2, s));
    HIP_TRY(permute_2d(b2, dx, bf, T, n, nullptr, pi_P, true, s));
    return POETX_OK;
}

// --------------------------------------------------- weight-centric POET
// The saved buffer: dense R [m, m], W0 P [m, n] and W_RP [m, n], each at a
// 256-byte boundary.
struct WcSaved {
    void* R = nullptr;
    void* WP = nullptr;
    void* W = nullptr;
};

void plan_wc_saved(Carver& cv, const poetx_linear_desc* d, WcSaved& S) {
    const size_t es = esize(d->dtype);
    S.R = cv.take(es * (size_t)(d->m * d->m));
    S.WP = cv.take(es * (size_t)(d->m * d->n));
    S.W = cv.take(es * (size_t)(d->m * d->n));
}

// One dense product of the weight-centric path, of any layout and output type:
// bf16 on the pipelined kernel where its operand rules allow (the largest tile
// whose grid still gives every CU a workgroup), else the register-staged one.
hipError_t wc_gemm(GemmLayout layout, bool bf, bool out_f32, int64_t M, int64_t N, int64_t K, const void* A,
                   int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, hipStream_t s) {
    const bool a_mn = layout == GemmLayout::TN, b_mn = layout != GemmLayout::NT;
    if (bf && pipe_gemm_supported(a_mn, b_mn, M, N, K, lda, ldb, 0, 0)) {
        if (!a_mn && !out_f32 && dense_gemm_supported(M, N, K, lda, ldb))
            return dense_gemm_bf16(b_mn, A, lda, B, ldb, C, ldc, (int)M, (int)N, (int)K, s);
        PipeArgs p;
        p.A = A; p.lda = lda;
        p.B = B; p.ldb = ldb;
        p.C = C; p.ldc = ldc;
        p.M = (int)M; p.N = (int)N; p.K = (int)K;
        p.k_per_split = (int)K;
        const int64_t tall = ((M + 255) / 256) * ((N + 127) / 128);
        return pipe_gemm(a_mn, b_mn, out_f32, p, s, tall >= 256 ? PipeTile::Tall : PipeTile::Square);
    }
    return gemm(layout, bf, bf && !out_f32, M, N, K, 1, Mat{A, lda, 0}, Mat{B, ldb, 0}, C, ldc, 0, s, 1.f, nullptr,
                0, nullptr, 0, 0, nullptr, true);
}

// R = Pi_R^T diag(G_R) Pi_R and P likewise as dense matrices;  W_RP = R (W0 P);
// y = x W_RP^T.
int wc_forward(const poetx_linear_desc* d, const void* x, const void* W0, const void* G_R, const void* G_P,
               const int32_t* pi_R, const int32_t* pi_P, void* y, const WcSaved& S, void* Pd, int32_t* inv_R,
               int32_t* inv_P, hipStream_t s) {
    const bool bf = d->dtype == POETX_BF16;
    const int64_t T = d->T, m = d->m, n = d->n;
    const int b = (int)d->b;
    HIP_TRY(invert_perm(pi_R, inv_R, m, s));
    HIP_TRY(invert_perm(pi_P, inv_P, n, s));
    HIP_TRY(blockdiag_dense(G_R, inv_R, S.R, bf, m, b, s));
    HIP_TRY(blockdiag_dense(G_P, inv_P, Pd, bf, n, b, s));
    HIP_TRY(wc_gemm(GemmLayout::NN, bf, false, m, n, n, W0, n, Pd, n, S.WP, n, s));
    HIP_TRY(wc_gemm(GemmLayout::NN, bf, false, m, n, m, S.R, m, S.WP, n, S.W, n, s));
    HIP_TRY(wc_gemm(GemmLayout::NT, bf, false, T, m, n, x, n, S.W, n, y, m, s));
    return POETX_OK;
}

// Backward buffers: dW_RP and R^T dW_RP (dtype [m, n]), dR (float32 [m, m]),
// dP (float32 [n, n]).
struct WcBufs {
    void* dW = nullptr;
    void* E = nullptr;
    float* dR = nullptr;
    float* dP = nullptr;
};

void plan_wc_bwd(Carver& cv, const poetx_linear_desc* d, WcBufs& B) {
    const size_t es = esize(d->dtype);
    B.dW = cv.take(es * (size_t)(d->m * d->n));
    B.E = cv.take(es * (size_t)(d->m * d->n));
    B.dR = cv.take_n<float>(d->m * d->m);
    B.dP = cv.take_n<float>(d->n * d->n);
}

// dx = dy W_RP;  dW_RP = dy^T x;  dR = dW_RP (W0 P)^T;  dP = W0^T (R^T dW_RP);
// dG = the diagonal blocks of Pi dR Pi^T and Pi_P dP Pi_P^T.
int wc_backward(const poetx_linear_desc* d, const void* dy, const void* x, const void* W0, const int32_t* pi_R,
                const int32_t* pi_P, const WcSaved& S, void* dx, float* dG_R, float* dG_P, const WcBufs& B,
                hipStream_t s) {
    const bool bf = d->dtype == POETX_BF16;
    const int64_t T = d->T, m = d->m, n = d->n;
    const int b = (int)d->b;
    HIP_TRY(wc_gemm(GemmLayout::NN, bf, false, T, n, m, dy, m, S.W, n, dx, n, s));
    HIP_TRY(wc_gemm(GemmLayout::TN, bf, false, m, n, T, dy, m, x, n, B.dW, n, s));
    HIP_TRY(wc_gemm(GemmLayout::NT, bf, true, m, m, n, B.dW, n, S.WP, n, B.dR, m, s));
    HIP_TRY(wc_gemm(GemmLayout::TN, bf, false, m, n, m, S.R, m, B.dW, n, B.E, n, s));
    HIP_TRY(wc_gemm(GemmLayout::TN, bf, true, n, n, m, W0, n, B.E, n, B.dP, n, s));
    HIP_TRY(blockdiag_gather(B.dR, pi_R, dG_R, m, b, s));
    HIP_TRY(blockdiag_gather(B.dP, pi_P, dG_P, n, b, s));
    return POETX_OK;
}

// The mem chain (MEM, and MEM_Q8 on its dequantized weight) recomputes h1 and h2.
inline bool mem_chain(const poetx_linear_desc* d) { return d->variant == POETX_MEM || d->variant == POETX_MEM_Q8; }

// Quantized weight buffer: int8 codes [m, n], then float32 row scales [m] at the
// next 256-byte boundary.
inline size_t qscale_offset(int64_t m, int64_t n) { return ((size_t)(m * n) + 255) & ~size_t(255); }
inline const int8_t* qcodes(const void* Wq) { return static_cast<const int8_t*>(Wq); }
inline const float* qscales(const void* Wq, int64_t m, int64_t n) {
    return reinterpret_cast<const float*>(static_cast<const char*>(Wq) + qscale_offset(m, n));
}

// The dense products of the chain on the stored weight: Wt itself, or for
// MEM_Q8 its int8 codes with the row scales applied in float32 (forward: per
// output column of h2 in the product's epilogue; backward: on dh2's columns by
// the block product that makes dh2, see poetx_linear_bwd).
hipError_t dense_fwd(const poetx_linear_desc* d, const void* h1, const void* Wt, void* h2, hipStream_t s) {
    const int64_t T = d->T, m = d->m, n = d->n;
    if (d->variant == POETX_MEM_Q8)
        return dense_gemm_q8(false, h1, n, qcodes(Wt), n, qscales(Wt, m, n), h2, m, (int)T, (int)m, (int)n, s);
    return dense_gemm(GemmLayout::NT, d->dtype == POETX_BF16, T, m, n, h1, n, Wt, n, h2, m, s);
}
hipError_t dense_bwd(const poetx_linear_desc* d, const void* dh2, const void* Wt, void* dh1, hipStream_t s) {
    const int64_t T = d->T, m = d->m, n = d->n;
    if (d->variant == POETX_MEM_Q8)
        return dense_gemm_q8(true, dh2, m, qcodes(Wt), n, nullptr, dh1, n, (int)T, (int)n, (int)m, s);
    return dense_gemm(GemmLayout::NN, d->dtype == POETX_BF16, T, n, m, dh2, m, Wt, n, dh1, n, s);
}

// The dense product and the R-side block product of the forward as one launch
// (dense_fold_r): bf16 chains with b = 256, whose 128 x 256 dense tiles are
// whole R blocks, when that tile grid runs in whole waves over the 256 CUs or in
// at least four (same-process timings of fold against dense + block product:
// 2048 x 4096 x 4096 69.0 / 67.6 against 69.3 us with / without h2 kept,
// 8192 x 5120 x 5120 405.7 / 392.2 against 442.1 us; a grid of 3.5 waves,
// 2048 x 14336 x 4096, lost 1-5%, and 64 tiles, 2048 x 1024 x 4096, 48.5
// against 28.1 us).
bool fold_r(const poetx_linear_desc* d) {
    const int64_t T = d->T, m = d->m, n = d->n;
    const int64_t tiles = ((T + 127) / 128) * (m / 256);
    return d->dtype == POETX_BF16 && d->b == 256 &&
           (d->variant == POETX_FAST || d->variant == POETX_MEM || d->variant == POETX_MEM_Q8) &&
           (tiles % 256 == 0 || tiles >= 1024) && dense_fold_r_supported(T, m, n, n, n, m, m, 256);
}

// h2_out receives h2 when the chain keeps it (FAST); z_buf ([T, m], not aliasing
// h1 or a) receives z on the folded path.
int linear_forward(const poetx_linear_desc* d, const void* x, const void* Wt, const void* G_R, const void* G_P,
                   const int32_t* pi_R, const int32_t* pi_P, void* y, void* h2_out, void* buf_a, void* buf_b,
                   void* z_buf, hipStream_t s) {
    const bool bf = d->dtype == POETX_BF16;
    const int64_t T = d->T, m = d->m, n = d->n, b = d->b;
    // a = x gathered by pi_P;  h1 = a . blockdiag(G_P)^T
    HIP_TRY(permute_2d(x, buf_a, bf, T, n, nullptr, pi_P, false, s));
    HIP_TRY(block_apply(GemmLayout::NT, bf, T, n, b, buf_a, G_P, buf_b, s));
    if (fold_r(d)) {
        // z = (h1 . Wt^T) . blockdiag(G_R)^T in one launch; h2 leaves the chip for FAST only
        const bool q8 = d->variant == POETX_MEM_Q8;
        HIP_TRY(dense_fold_r(q8, buf_b, n, q8 ? static_cast<const void*>(qcodes(Wt)) : Wt, n,
                             q8 ? qscales(Wt, m, n) : nullptr, G_R, mem_chain(d) ? nullptr : h2_out, m, z_buf, m,
                             (int)T, (int)m, (int)n, (int)b, s));
        HIP_TRY(permute_2d(z_buf, y, bf, T, m, nullptr, pi_R, true, s));
        return POETX_OK;
    }
    // h2 = h1 . Wt^T (the int8 weight: h1 . codes^T, output column i scaled by scale_i)
    HIP_TRY(dense_fwd(d, buf_b, Wt, h2_out, s));
    // z = h2 . blockdiag(G_R)^T ; y = z scattered by pi_R
    HIP_TRY(block_apply(GemmLayout::NT, bf, T, m, b, h2_out, G_R, buf_b, s));
    HIP_TRY(permute_2d(buf_b, y, bf, T, m, nullptr, pi_R, true, s));
    return POETX_OK;
}

// ------------------------------------------------------ groups of linears
// A group of `count` linears reading the same input x [T, n] runs as one chain
// of width m = sum m_g (outputs concatenated) and n' = count n (one gathered
// copy of x per linear), so every stage is one launch: see poetx.h.
struct GroupPlan {
    poetx_linear_desc lin{};   // the chain: m = sum m_g, n = count n
    int count = 0;
    int64_t n = 0;             // width of the shared input
    PermSegments seg;
};

int check_group(const poetx_group_desc* g, GroupPlan& P) {
    if (!g) return POETX_ERR_INVALID_ARG;
    if (g->count < 1 || g->count > POETX_MAX_GROUP) return POETX_ERR_SHAPE;
    if (g->variant != POETX_FAST && g->variant != POETX_MEM) return POETX_ERR_INVALID_ARG;
    if (g->n <= 0 || g->n > kMaxExtent / g->count) return POETX_ERR_SHAPE;
    int64_t M = 0;
    P.seg.count = g->count;
    P.seg.n = g->n;
    for (int i = 0; i < g->count; ++i) {
        if (g->m[i] <= 0 || g->m[i] > kMaxExtent - M) return POETX_ERR_SHAPE;
        P.seg.off[i] = M;
        M += g->m[i];
    }
    P.seg.off[g->count] = M;
    P.count = g->count;
    P.n = g->n;
    P.lin = poetx_linear_desc{g->T, M, g->count * g->n, g->b, g->k, g->dtype, g->variant, g->reserved};
    POETX_TRY(check_desc(&P.lin));
    for (int i = 0; i < g->count; ++i)
        if (g->m[i] % g->b) return POETX_ERR_SHAPE;
    if (g->n % g->b) return POETX_ERR_SHAPE;
    return POETX_OK;
}

inline const char* byte_off(const void* p, int64_t elems, size_t es) {
    return static_cast<const char*>(p) + (size_t)elems * es;
}
inline char* byte_off(void* p, int64_t elems, size_t es) { return static_cast<char*>(p) + (size_t)elems * es; }

// The dense products of a group.  Forward (nn = false): H2[:, seg g] = H1[:, g n
// .. (g+1) n) . Wt_g^T.  Backward (nn = true): dH1[:, g n .. (g+1) n) =
// dH2[:, seg g] . Wt_g.  Wt is the row-stacked [sum m_g, n] weight.  bf16 with
// 128-column-aligned segments runs as grouped launches of the pipelined
// kernel: the forward products all have k = n and form one launch; backward
// products share a launch only with neighbours of the same k = m_g, so that a
// launch's tiles take equal time (q, k and v: q alone, k with v).  Otherwise
// one dense product per linear.
hipError_t group_dense(const GroupPlan& P, bool nn, const void* A, const void* Wt, void* C, hipStream_t s) {
    const bool bf = P.lin.dtype == POETX_BF16;
    const size_t es = esize(P.lin.dtype);
    const int64_t T = P.lin.T, M = P.lin.m, n = P.n, G = P.count;
    const int64_t lda = nn ? M : G * n, ldc = nn ? G * n : M;
    bool grouped = bf && G > 1 && n % 128 == 0;
    for (int g = 0; g < G && grouped; ++g) {
        const int64_t m_g = P.seg.off[g + 1] - P.seg.off[g];
        grouped = m_g % 128 == 0 && pipe_gemm_supported(false, nn, T, nn ? n : m_g, nn ? m_g : n, lda, n, 0, 0);
    }
    if (grouped) {
        auto m_of = [&](int g) { return P.seg.off[g + 1] - P.seg.off[g]; };
        for (int g0 = 0; g0 < G;) {
            // one launch for the whole group; in the backward the linears may
            // differ in k (q/k/v: m_g = 4096, 1024, 1024), whose tiles the
            // launch deals longest k first and evenly over the XCDs
            const int g1 = (int)G;
            // linears [g0, g1): output columns from c0, relative group table
            const int64_t c0 = nn ? g0 * n : P.seg.off[g0];
            PipeArgs p;
            p.A = A; p.lda = lda;
            p.B = Wt; p.ldb = n;
            p.C = byte_off(C, c0, es); p.ldc = ldc;
            p.M = (int)T;
            p.N = (int)(nn ? (g1 - g0) * n : P.seg.off[g1] - P.seg.off[g0]);
            p.ngroups = g1 - g0;
            int kmax = 0;
            for (int g = g0; g < g1; ++g) {
                const int64_t off = P.seg.off[g];
                PipeGroup& e = p.grp[g - g0];
                if (!nn) {
                    e.n_begin = (int)(off - c0); e.k = (int)n; e.a_off = g * n; e.b_off = off * n - (off - c0) * n;
                } else {
                    e.n_begin = (int)((g - g0) * n); e.k = (int)m_of(g); e.a_off = off; e.b_off = off * n - (g - g0) * n;
                }
                kmax = std::max(kmax, e.k);
            }
            p.K = kmax;
            p.k_per_split = kmax;
            auto tiles = [&](int bm) { return ((T + bm - 1) / bm) * ((p.N + 127) / 128); };
            const PipeTile t = tiles(256) >= 256   ? PipeTile::Tall
                               : tiles(128) >= 256 ? PipeTile::Square
                                                   : PipeTile::Slim;
            const hipError_t e = pipe_gemm(false, nn, false, p, s, t);
            if (e != hipSuccess) return e;
            g0 = g1;
        }
        return hipSuccess;
    }
    for (int g = 0; g < G; ++g) {
        const int64_t off = P.seg.off[g], m_g = P.seg.off[g + 1] - off;
        const void* Wg = byte_off(Wt, off * n, es);
        hipError_t e;
        if (!nn)
            e = dense_gemm(GemmLayout::NT, bf, T, m_g, n, byte_off(A, g * n, es), lda, Wg, n, byte_off(C, off, es),
                           ldc, s);
        else
            e = dense_gemm(GemmLayout::NN, bf, T, n, m_g, byte_off(A, off, es), lda, Wg, n, byte_off(C, g * n, es),
                           ldc, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Index tables in the workspace: pi_R with each linear's output offset added,
// and each P permutation inverted in place of its slice (for the dx sum).
struct GroupIdx {
    int32_t* pi_R = nullptr;
    int32_t* inv_P = nullptr;
};

void plan_group_idx(Carver& cv, const GroupPlan& P, GroupIdx& I) {
    I.pi_R = cv.take_n<int32_t>(P.lin.m);
    I.inv_P = cv.take_n<int32_t>(P.lin.n);
}

int group_forward(const GroupPlan& P, const void* x, const void* Wt, const void* G_R, const void* G_P,
                  const int32_t* pi_P, const int32_t* pi_R_cat, void* y, void* h2, void* a, void* buf,
                  hipStream_t s) {
    const poetx_linear_desc* d = &P.lin;
    const bool bf = d->dtype == POETX_BF16;
    const int64_t T = d->T, M = d->m, nn = d->n, b = d->b;
    // a = [x gathered by pi_P,g for every g];  h1 = a . blockdiag(G_P)^T
    HIP_TRY(gather_sum(x, a, bf, T, P.n, nn, pi_P, 1, s));
    HIP_TRY(block_apply(GemmLayout::NT, bf, T, nn, b, a, G_P, buf, s));
    // h2[:, seg g] = h1_g . Wt_g^T
    HIP_TRY(group_dense(P, false, buf, Wt, h2, s));
    // z = h2 . blockdiag(G_R)^T ; y = z scattered by the offset pi_R
    HIP_TRY(block_apply(GemmLayout::NT, bf, T, M, b, h2, G_R, buf, s));
    HIP_TRY(permute_2d(buf, y, bf, T, M, nullptr, pi_R_cat, true, s));
    return POETX_OK;
}

}  // namespace

// ----------------------------------------------- no-allocation forward scratch
// The workspace of poetx_linear_fwd_noalloc: a file-scope device array, one
// copy on every GPU the library runs on, held until the process ends.  Host
// code never uses the name itself (on the host it is only a stand-in): each
// device's address comes from hipGetSymbolAddress, once per device, and is
// kept below.
static __device__ __align__(256) unsigned char scratch[POETX_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The current device's scratch address (looked up on that device's first call).
int scratch_address(void** out) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxScratchDevices) return POETX_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p) return POETX_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return POETX_OK;
}

}  // namespace

// ======================================================================= ABI
extern "C" {

const char* poetx_version(void) { return "libpoetx 0.1.0 gfx950"; }

const char* poetx_status_string(int status) {
    switch (status) {
        case POETX_OK: return "ok";
        case POETX_ERR_INVALID_ARG: return "invalid argument";
        case POETX_ERR_SHAPE: return "invalid shape";
        case POETX_ERR_UNSUPPORTED: return "unsupported block size, order or dtype";
        case POETX_ERR_WORKSPACE: return "workspace too small";
        case POETX_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

const char* poetx_last_hip_error(void) { return g_last_hip_error.c_str(); }

int poetx_skew_unpack(const float* q, void* Q, int dtype, int64_t nblk, int64_t b, void* stream) {
    if (!dtype_ok(dtype)) return POETX_ERR_INVALID_ARG;
    if (b <= 1 || b > 1024) return b <= 0 ? POETX_ERR_SHAPE : POETX_ERR_UNSUPPORTED;
    POETX_TRY(check_nblk(nblk, b));
    if (nblk == 0) return POETX_OK;
    if (!q || !Q) return POETX_ERR_INVALID_ARG;
    HIP_TRY(skew_unpack(q, Q, dtype == POETX_BF16, nblk, (int)b, as_stream(stream)));
    return POETX_OK;
}

int poetx_skew_pack(const float* dQ, float* dq, int64_t nblk, int64_t b, void* stream) {
    if (b <= 1 || b > 1024) return b <= 0 ? POETX_ERR_SHAPE : POETX_ERR_UNSUPPORTED;
    POETX_TRY(check_nblk(nblk, b));
    if (nblk == 0) return POETX_OK;
    if (!dQ || !dq) return POETX_ERR_INVALID_ARG;
    HIP_TRY(skew_pack(dQ, dq, nblk, (int)b, as_stream(stream)));
    return POETX_OK;
}

size_t poetx_cnp_fwd_workspace_bytes(int64_t nblk, int64_t b, int k, int G_dtype) {
    if (check_block(b) != POETX_OK || check_k(k) != POETX_OK || check_nblk(nblk, b) != POETX_OK ||
        !dtype_ok(G_dtype))
        return 0;
    return cnp_ws(nblk, b, k, G_dtype == POETX_BF16, false);
}

int poetx_cnp_fwd(const float* q, int64_t nblk, int64_t b, int k, void* G, int G_dtype, void* ws, size_t ws_bytes,
                  void* stream) {
    if (!dtype_ok(G_dtype)) return POETX_ERR_INVALID_ARG;
    POETX_TRY(check_block(b));
    POETX_TRY(check_k(k));
    POETX_TRY(check_nblk(nblk, b));
    if (nblk == 0) return POETX_OK;
    if (!q || !G) return POETX_ERR_INVALID_ARG;
    const bool cbf = G_dtype == POETX_BF16;
    const size_t need = cnp_ws(nblk, b, k, cbf, false);
    if (ws_bytes < need) return POETX_ERR_WORKSPACE;
    if (need && !ws) return POETX_ERR_INVALID_ARG;
    Carver cv(ws);
    CnpBufs B;
    plan_cnp(cv, cv, nblk, b, k, cbf, false, B);
    return cnp_forward(q, nblk, b, k, cbf, G, cbf, B, false, as_stream(stream));
}

size_t poetx_cnp_saved_bytes(int64_t nblk, int64_t b, int k, int dtype) {
    if (check_block(b) != POETX_OK || check_k(k) != POETX_OK || check_nblk(nblk, b) != POETX_OK ||
        !dtype_ok(dtype))
        return 0;
    return cnp_saved(nblk, b, k, dtype == POETX_BF16);
}

int poetx_cnp_fwd_save(const float* q, int64_t nblk, int64_t b, int k, void* G, int G_dtype, void* saved,
                       size_t saved_bytes, void* ws, size_t ws_bytes, void* stream) {
    if (!dtype_ok(G_dtype)) return POETX_ERR_INVALID_ARG;
    POETX_TRY(check_block(b));
    POETX_TRY(check_k(k));
    POETX_TRY(check_nblk(nblk, b));
    if (nblk == 0) return POETX_OK;
    if (!q || !G || !saved) return POETX_ERR_INVALID_ARG;
    const bool cbf = G_dtype == POETX_BF16;
    if (saved_bytes < cnp_saved(nblk, b, k, cbf)) return POETX_ERR_WORKSPACE;
    const size_t need = cnp_ws(nblk, b, k, cbf, false, true);
    if (ws_bytes < need) return POETX_ERR_WORKSPACE;
    if (need && !ws) return POETX_ERR_INVALID_ARG;
    Carver cv(ws), sv(saved);
    CnpBufs B;
    plan_cnp(cv, sv, nblk, b, k, cbf, false, B);
    return cnp_forward(q, nblk, b, k, cbf, G, cbf, B, true, as_stream(stream));
}

size_t poetx_cnp_bwd_workspace_bytes(int64_t nblk, int64_t b, int k, int dtype) {
    if (check_block(b) != POETX_OK || check_k(k) != POETX_OK || check_nblk(nblk, b) != POETX_OK ||
        !dtype_ok(dtype))
        return 0;
    return cnp_ws(nblk, b, k, dtype == POETX_BF16, true);
}

int poetx_cnp_bwd(const float* q, const float* dG, int64_t nblk, int64_t b, int k, float* dq, int dtype, void* ws,
                  size_t ws_bytes, void* stream) {
    if (!dtype_ok(dtype)) return POETX_ERR_INVALID_ARG;
    POETX_TRY(check_block(b));
    POETX_TRY(check_k(k));
    POETX_TRY(check_nblk(nblk, b));
    if (nblk == 0) return POETX_OK;
    if (!q || !dG || !dq) return POETX_ERR_INVALID_ARG;
    const bool cbf = dtype == POETX_BF16;
    const size_t need = cnp_ws(nblk, b, k, cbf, true);
    if (ws_bytes < need) return POETX_ERR_WORKSPACE;
    if (need && !ws) return POETX_ERR_INVALID_ARG;
    Carver cv(ws);
    CnpBufs B;
    plan_cnp(cv, cv, nblk, b, k, cbf, true, B);
    return cnp_backward(q, dG, nblk, b, k, cbf, dq, B, false, as_stream(stream));
}

int poetx_cnp_bwd_saved(const float* q, const float* dG, int64_t nblk, int64_t b, int k, float* dq, int dtype,
                        const void* saved, size_t saved_bytes, void* ws, size_t ws_bytes, void* stream) {
    if (!dtype_ok(dtype)) return POETX_ERR_INVALID_ARG;
    POETX_TRY(check_block(b));
    POETX_TRY(check_k(k));
    POETX_TRY(check_nblk(nblk, b));
    if (nblk == 0) return POETX_OK;
    if (!q || !dG || !dq || !saved) return POETX_ERR_INVALID_ARG;
    const bool cbf = dtype == POETX_BF16;
    if (saved_bytes < cnp_saved(nblk, b, k, cbf)) return POETX_ERR_WORKSPACE;
    const size_t need = cnp_ws(nblk, b, k, cbf, true, true);
    if (ws_bytes < need) return POETX_ERR_WORKSPACE;
    if (need && !ws) return POETX_ERR_INVALID_ARG;
    Carver cv(ws), sv(const_cast<void*>(saved));
    CnpBufs B;
    plan_cnp(cv, sv, nblk, b, k, cbf, true, B);
    return cnp_backward(q, dG, nblk, b, k, cbf, dq, B, true, as_stream(stream));
}

int poetx_permute(const void* src, void* dst, int dtype, int64_t rows, int64_t cols, const int32_t* row_idx,
                  const int32_t* col_idx, int scatter_cols, void* stream) {
    if (!dtype_ok(dtype)) return POETX_ERR_INVALID_ARG;
    if (rows < 0 || cols < 0 || rows > kMaxExtent || cols > kMaxExtent) return POETX_ERR_SHAPE;
    if (rows == 0 || cols == 0) return POETX_OK;
    if (!src || !dst) return POETX_ERR_INVALID_ARG;
    if (cols % (16 / (int64_t)esize(dtype)) != 0) return POETX_ERR_SHAPE;
    HIP_TRY(permute_2d(src, dst, dtype == POETX_BF16, rows, cols, row_idx, col_idx, scatter_cols != 0,
                       as_stream(stream)));
    return POETX_OK;
}

int poetx_prepermute(const void* W0, void* Wt, int dtype, int64_t m, int64_t n, const int32_t* pi_R,
                     const int32_t* pi_P, void* stream) {
    if (!dtype_ok(dtype)) return POETX_ERR_INVALID_ARG;
    if (m <= 0 || n <= 0 || m > kMaxExtent || n > kMaxExtent) return POETX_ERR_SHAPE;
    if (!W0 || !Wt || !pi_R || !pi_P) return POETX_ERR_INVALID_ARG;
    if (n % (16 / (int64_t)esize(dtype)) != 0) return POETX_ERR_SHAPE;
    HIP_TRY(permute_2d(W0, Wt, dtype == POETX_BF16, m, n, pi_R, pi_P, false, as_stream(stream)));
    return POETX_OK;
}

size_t poetx_check_perm_workspace_bytes(int64_t len) {
    if (len < 0 || len > kMaxExtent) return 0;
    return (size_t)(len + 1) * sizeof(int32_t);
}

int poetx_check_perm(const int32_t* pi, int64_t len, int32_t* ok, void* ws, size_t ws_bytes, void* stream) {
    if (len < 0 || len > kMaxExtent) return POETX_ERR_SHAPE;
    if (!ok || (len > 0 && !pi)) return POETX_ERR_INVALID_ARG;
    if (ws_bytes < poetx_check_perm_workspace_bytes(len)) return POETX_ERR_WORKSPACE;
    if (!ws) return POETX_ERR_INVALID_ARG;
    int* counts = static_cast<int*>(ws);
    HIP_TRY(check_perm(pi, len, ok, counts, counts + len, as_stream(stream)));
    return POETX_OK;
}

size_t poetx_linear_saved_bytes(const poetx_linear_desc* d) {
    if (check_desc(d) != POETX_OK || mem_chain(d)) return 0;
    if (d->variant == POETX_WEIGHT_CENTRIC) {
        Carver cv(nullptr);
        WcSaved S;
        plan_wc_saved(cv, d, S);
        return cv.off;
    }
    return fast_saved_a_offset(d) + esize(d->dtype) * (size_t)(d->T * d->n);
}

size_t poetx_linear_fwd_workspace_bytes(const poetx_linear_desc* d) {
    if (check_desc(d) != POETX_OK) return 0;
    Carver cv(nullptr);
    if (d->variant == POETX_WEIGHT_CENTRIC) {
        cv.take(esize(d->dtype) * (size_t)(d->n * d->n));  // dense P
        cv.take_n<int32_t>(d->m);                          // pi_R^-1
        cv.take_n<int32_t>(d->n);                          // pi_P^-1
        return cv.off;
    }
    LinearBufs L;
    plan_linear(cv, d, false, L);
    if (mem_chain(d)) cv.take(esize(d->dtype) * (size_t)(d->T * d->m));
    return cv.off;
}

}  // extern "C"

namespace {

// Argument checks of the layer forward that need no workspace (both entry points).
int check_linear_fwd_args(const poetx_linear_desc* d, const void* x, const void* Wt, const void* G_R,
                          const void* G_P, const int32_t* pi_R, const int32_t* pi_P, const void* y,
                          const void* saved) {
    if (!x || !Wt || !G_R || !G_P || !pi_R || !pi_P || !y) return POETX_ERR_INVALID_ARG;
    if (!mem_chain(d) && !saved) return POETX_ERR_INVALID_ARG;
    if (!all_al16(x, Wt, G_R, G_P, pi_R, pi_P, y, saved)) return POETX_ERR_INVALID_ARG;
    return POETX_OK;
}

// The layer forward after validation, on a workspace of at least
// poetx_linear_fwd_workspace_bytes(d) bytes at ws.
int linear_fwd_run(const poetx_linear_desc* d, const void* x, const void* Wt, const void* G_R, const void* G_P,
                   const int32_t* pi_R, const int32_t* pi_P, void* y, void* saved, void* ws, void* stream) {
    Carver cv(ws);
    if (d->variant == POETX_WEIGHT_CENTRIC) {
        Carver sv(saved);
        WcSaved S;
        plan_wc_saved(sv, d, S);
        void* Pd = cv.take(esize(d->dtype) * (size_t)(d->n * d->n));
        int32_t* inv_R = cv.take_n<int32_t>(d->m);
        int32_t* inv_P = cv.take_n<int32_t>(d->n);
        return wc_forward(d, x, Wt, G_R, G_P, pi_R, pi_P, y, S, Pd, inv_R, inv_P, as_stream(stream));
    }
    LinearBufs L;
    plan_linear(cv, d, false, L);
    if (d->variant == POETX_FOUR_PERM)
        return four_perm_forward(d, x, Wt, G_R, G_P, pi_R, pi_P, y, saved,
                                 static_cast<char*>(saved) + fast_saved_a_offset(d), L.buf[0], L.buf[1],
                                 as_stream(stream));
    void* h2 = saved;
    void* a = L.buf[0];
    void* z = L.buf[0];   // FAST: free (a is kept in saved); MEM: h2's buffer, which the folded path skips
    if (mem_chain(d)) {
        h2 = cv.take(esize(d->dtype) * (size_t)(d->T * d->m));
        z = h2;
    } else {
        a = static_cast<char*>(saved) + fast_saved_a_offset(d);
    }
    return linear_forward(d, x, Wt, G_R, G_P, pi_R, pi_P, y, h2, a, L.buf[1], z, as_stream(stream));
}

}  // namespace

extern "C" {

int poetx_linear_fwd(const poetx_linear_desc* d, const void* x, const void* Wt, const void* G_R, const void* G_P,
                     const int32_t* pi_R, const int32_t* pi_P, void* y, void* saved, void* ws, size_t ws_bytes,
                     void* stream) {
    POETX_TRY(check_desc(d));
    if (d->T == 0) return POETX_OK;
    POETX_TRY(check_linear_fwd_args(d, x, Wt, G_R, G_P, pi_R, pi_P, y, saved));
    if (!al16(ws)) return POETX_ERR_INVALID_ARG;
    const size_t need = poetx_linear_fwd_workspace_bytes(d);
    if (ws_bytes < need) return POETX_ERR_WORKSPACE;
    if (!ws) return POETX_ERR_INVALID_ARG;
    return linear_fwd_run(d, x, Wt, G_R, G_P, pi_R, pi_P, y, saved, ws, stream);
}

int poetx_linear_fwd_noalloc(const poetx_linear_desc* d, const void* x, const void* Wt, const void* G_R,
                             const void* G_P, const int32_t* pi_R, const int32_t* pi_P, void* y, void* saved,
                             void* stream) {
    POETX_TRY(check_desc(d));
    if (d->T == 0) return POETX_OK;
    POETX_TRY(check_linear_fwd_args(d, x, Wt, G_R, G_P, pi_R, pi_P, y, saved));
    if (poetx_linear_fwd_workspace_bytes(d) > (size_t)POETX_NOALLOC_SCRATCH_BYTES) return POETX_ERR_WORKSPACE;
    void* ws = nullptr;
    POETX_TRY(scratch_address(&ws));
    return linear_fwd_run(d, x, Wt, G_R, G_P, pi_R, pi_P, y, saved, ws, stream);
}

size_t poetx_linear_bwd_workspace_bytes(const poetx_linear_desc* d) {
    if (check_desc(d) != POETX_OK) return 0;
    Carver cv(nullptr);
    if (d->variant == POETX_WEIGHT_CENTRIC) {
        WcBufs B;
        plan_wc_bwd(cv, d, B);
        return cv.off;
    }
    LinearBufs L;
    plan_linear(cv, d, true, L);
    return cv.off;
}

int poetx_linear_bwd(const poetx_linear_desc* d, const void* dy, const void* x, const void* Wt, const void* G_R,
                     const void* G_P, const int32_t* pi_R, const int32_t* pi_P, const void* saved, void* dx,
                     float* dG_R, float* dG_P, void* ws, size_t ws_bytes, void* stream) {
    POETX_TRY(check_desc(d));
    if (!dG_R || !dG_P) return POETX_ERR_INVALID_ARG;
    const hipStream_t s = as_stream(stream);
    const int64_t T = d->T, m = d->m, n = d->n, b = d->b;
    if (T == 0) {
        HIP_TRY(fill_zero(dG_R, sizeof(float) * (size_t)(m * b), s));
        HIP_TRY(fill_zero(dG_P, sizeof(float) * (size_t)(n * b), s));
        return POETX_OK;
    }
    if (!dy || !x || !Wt || !G_R || !G_P || !pi_R || !pi_P || !dx) return POETX_ERR_INVALID_ARG;
    if (!mem_chain(d) && !saved) return POETX_ERR_INVALID_ARG;
    if (!all_al16(dy, x, Wt, G_R, G_P, pi_R, pi_P, saved, dx, dG_R, dG_P, ws)) return POETX_ERR_INVALID_ARG;
    const size_t need = poetx_linear_bwd_workspace_bytes(d);
    if (ws_bytes < need) return POETX_ERR_WORKSPACE;
    if (!ws) return POETX_ERR_INVALID_ARG;
    Carver cv(ws);
    if (d->variant == POETX_WEIGHT_CENTRIC) {
        Carver sv(const_cast<void*>(saved));
        WcSaved S;
        plan_wc_saved(sv, d, S);
        WcBufs B;
        plan_wc_bwd(cv, d, B);
        return wc_backward(d, dy, x, Wt, pi_R, pi_P, S, dx, dG_R, dG_P, B, s);
    }
    LinearBufs L;
    plan_linear(cv, d, true, L);
    if (d->variant == POETX_FOUR_PERM)
        return four_perm_backward(d, dy, Wt, G_R, G_P, pi_R, pi_P, saved,
                                  static_cast<const char*>(saved) + fast_saved_a_offset(d), dx, dG_R, dG_P, L, s);
    const bool bf = d->dtype == POETX_BF16;
    const void* bufA = L.buf[0];
    void* bufB = L.buf[1];
    void* bufC = L.buf[2];
    const void* h2 = saved;
    if (d->variant == POETX_FAST) {
        // a = x gathered by pi_P, kept by the forward
        bufA = static_cast<const char*>(saved) + fast_saved_a_offset(d);
    } else {
        // a = x gathered by pi_P again (kept for dG_P)
        HIP_TRY(permute_2d(x, L.buf[0], bf, T, n, nullptr, pi_P, false, s));
    }
    if (mem_chain(d)) {
        // recompute h1 and h2 from x
        HIP_TRY(block_apply(GemmLayout::NT, bf, T, n, b, bufA, G_P, bufB, s));
        HIP_TRY(dense_fwd(d, bufB, Wt, bufC, s));
        h2 = bufC;
    }
    // dz = dy gathered by pi_R
    HIP_TRY(permute_2d(dy, bufB, bf, T, m, nullptr, pi_R, false, s));
    // dG_R[j] = dz_j^T h2_j
    POETX_TRY(block_grad(bf, T, m, b, bufB, h2, dG_R, L.splits_R, L.kps_R, L.part, s));
    // dh2 = dz . blockdiag(G_R) (MEM_Q8: column i scaled by the weight's row
    // scale_i, so that the next product can take the int8 codes as they are)
    HIP_TRY(block_apply(GemmLayout::NN, bf, T, m, b, bufB, G_R, bufC, s,
                        d->variant == POETX_MEM_Q8 ? qscales(Wt, m, n) : nullptr));
    // dh1 = dh2 . Wt
    HIP_TRY(dense_bwd(d, bufC, Wt, bufB, s));
    // dG_P[j] = dh1_j^T a_j
    POETX_TRY(block_grad(bf, T, n, b, bufB, bufA, dG_P, L.splits_P, L.kps_P, L.part, s));
    // da = dh1 . blockdiag(G_P) ; dx = da scattered by pi_P
    HIP_TRY(block_apply(GemmLayout::NN, bf, T, n, b, bufB, G_P, bufC, s));
    HIP_TRY(permute_2d(bufC, dx, bf, T, n, nullptr, pi_P, true, s));
    return POETX_OK;
}

size_t poetx_group_saved_bytes(const poetx_group_desc* g) {
    GroupPlan P;
    if (check_group(g, P) != POETX_OK) return 0;
    return poetx_linear_saved_bytes(&P.lin);
}

size_t poetx_group_fwd_workspace_bytes(const poetx_group_desc* g) {
    GroupPlan P;
    if (check_group(g, P) != POETX_OK) return 0;
    Carver cv(nullptr);
    LinearBufs L;
    plan_linear(cv, &P.lin, false, L);
    if (P.lin.variant == POETX_MEM) cv.take(esize(P.lin.dtype) * (size_t)(P.lin.T * P.lin.m));
    GroupIdx I;
    plan_group_idx(cv, P, I);
    return cv.off;
}

int poetx_group_fwd(const poetx_group_desc* g, const void* x, const void* Wt, const void* G_R, const void* G_P,
                    const int32_t* pi_R, const int32_t* pi_P, void* y, void* saved, void* ws, size_t ws_bytes,
                    void* stream) {
    GroupPlan P;
    POETX_TRY(check_group(g, P));
    if (P.lin.T == 0) return POETX_OK;
    if (!x || !Wt || !G_R || !G_P || !pi_R || !pi_P || !y) return POETX_ERR_INVALID_ARG;
    if (P.lin.variant == POETX_FAST && !saved) return POETX_ERR_INVALID_ARG;
    if (!all_al16(x, Wt, G_R, G_P, pi_R, pi_P, y, saved, ws)) return POETX_ERR_INVALID_ARG;
    if (ws_bytes < poetx_group_fwd_workspace_bytes(g)) return POETX_ERR_WORKSPACE;
    if (!ws) return POETX_ERR_INVALID_ARG;
    const hipStream_t s = as_stream(stream);
    Carver cv(ws);
    LinearBufs L;
    plan_linear(cv, &P.lin, false, L);
    void* h2 = saved;
    void* a = L.buf[0];
    if (P.lin.variant == POETX_MEM) h2 = cv.take(esize(P.lin.dtype) * (size_t)(P.lin.T * P.lin.m));
    else a = static_cast<char*>(saved) + fast_saved_a_offset(&P.lin);
    GroupIdx I;
    plan_group_idx(cv, P, I);
    HIP_TRY(group_perms(pi_R, pi_P, I.pi_R, I.inv_P, P.seg, s));
    return group_forward(P, x, Wt, G_R, G_P, pi_P, I.pi_R, y, h2, a, L.buf[1], s);
}

size_t poetx_group_bwd_workspace_bytes(const poetx_group_desc* g) {
    GroupPlan P;
    if (check_group(g, P) != POETX_OK) return 0;
    Carver cv(nullptr);
    LinearBufs L;
    plan_linear(cv, &P.lin, true, L);
    GroupIdx I;
    plan_group_idx(cv, P, I);
    return cv.off;
}

int poetx_group_bwd(const poetx_group_desc* g, const void* dy, const void* x, const void* Wt, const void* G_R,
                    const void* G_P, const int32_t* pi_R, const int32_t* pi_P, const void* saved, void* dx,
                    float* dG_R, float* dG_P, void* ws, size_t ws_bytes, void* stream) {
    GroupPlan P;
    POETX_TRY(check_group(g, P));
    if (!dG_R || !dG_P) return POETX_ERR_INVALID_ARG;
    const hipStream_t s = as_stream(stream);
    const poetx_linear_desc* d = &P.lin;
    const int64_t T = d->T, M = d->m, nn = d->n, b = d->b;
    if (T == 0) {
        HIP_TRY(fill_zero(dG_R, sizeof(float) * (size_t)(M * b), s));
        HIP_TRY(fill_zero(dG_P, sizeof(float) * (size_t)(nn * b), s));
        return POETX_OK;
    }
    if (!dy || !x || !Wt || !G_R || !G_P || !pi_R || !pi_P || !dx) return POETX_ERR_INVALID_ARG;
    if (d->variant == POETX_FAST && !saved) return POETX_ERR_INVALID_ARG;
    if (!all_al16(dy, x, Wt, G_R, G_P, pi_R, pi_P, saved, dx, dG_R, dG_P, ws)) return POETX_ERR_INVALID_ARG;
    if (ws_bytes < poetx_group_bwd_workspace_bytes(g)) return POETX_ERR_WORKSPACE;
    if (!ws) return POETX_ERR_INVALID_ARG;
    Carver cv(ws);
    LinearBufs L;
    plan_linear(cv, d, true, L);
    GroupIdx I;
    plan_group_idx(cv, P, I);
    HIP_TRY(group_perms(pi_R, pi_P, I.pi_R, I.inv_P, P.seg, s));
    const bool bf = d->dtype == POETX_BF16;
    const void* bufA = L.buf[0];
    void* bufB = L.buf[1];
    void* bufC = L.buf[2];
    const void* h2 = saved;
    if (d->variant == POETX_FAST) {
        bufA = static_cast<const char*>(saved) + fast_saved_a_offset(d);
    } else {
        // recompute a, h1 and h2 from x
        HIP_TRY(gather_sum(x, L.buf[0], bf, T, P.n, nn, pi_P, 1, s));
        HIP_TRY(block_apply(GemmLayout::NT, bf, T, nn, b, bufA, G_P, bufB, s));
        HIP_TRY(group_dense(P, false, bufB, Wt, bufC, s));
        h2 = bufC;
    }
    // dz = dy gathered by the offset pi_R;  dG_R = dz_j^T h2_j;  dh2 = dz . blockdiag(G_R)
    HIP_TRY(permute_2d(dy, bufB, bf, T, M, nullptr, I.pi_R, false, s));
    POETX_TRY(block_grad(bf, T, M, b, bufB, h2, dG_R, L.splits_R, L.kps_R, L.part, s));
    HIP_TRY(block_apply(GemmLayout::NN, bf, T, M, b, bufB, G_R, bufC, s));
    // dh1[:, g n .. (g+1) n) = dh2[:, seg g] . Wt_g;  dG_P = dh1_j^T a_j;  da = dh1 . blockdiag(G_P)
    HIP_TRY(group_dense(P, true, bufC, Wt, bufB, s));
    POETX_TRY(block_grad(bf, T, nn, b, bufB, bufA, dG_P, L.splits_P, L.kps_P, L.part, s));
    HIP_TRY(block_apply(GemmLayout::NN, bf, T, nn, b, bufB, G_P, bufC, s));
    // dx = sum over the linears of da_g scattered by pi_P,g
    HIP_TRY(gather_sum(bufC, dx, bf, T, nn, P.n, I.inv_P, P.count, s));
    return POETX_OK;
}

size_t poetx_merge_workspace_bytes(const poetx_linear_desc* d) {
    if (check_desc(d) != POETX_OK || d->variant == POETX_FOUR_PERM || d->variant == POETX_WEIGHT_CENTRIC) return 0;
    const bool bf = d->dtype == POETX_BF16;
    Carver cv(nullptr);
    const size_t es = esize(d->dtype);
    if (d->variant == POETX_MEM_Q8) cv.take(2 * (size_t)(d->m * d->n));  // the dequantized weight
    cv.take(es * (size_t)(d->m * d->b));  // G_R
    cv.take(es * (size_t)(d->n * d->b));  // G_P
    cv.take(es * (size_t)(d->m * d->n));  // D_R Wt
    cv.take(es * (size_t)(d->m * d->n));  // D_R Wt D_P
    cv.take_n<int32_t>(d->m);             // sigma_R
    cv.take_n<int32_t>(d->n);             // sigma_P
    cv.take_n<int32_t>(std::max(d->m, d->n));  // inverse scratch
    cv.take(std::max(cnp_ws(d->m / d->b, d->b, d->k, bf, false), cnp_ws(d->n / d->b, d->b, d->k, bf, false)));
    return cv.off;
}

int poetx_merge(const poetx_linear_desc* d, void* Wt, float* q_R, float* q_P, const int32_t* pi_R_old,
                const int32_t* pi_P_old, const int32_t* pi_R_new, const int32_t* pi_P_new, void* ws,
                size_t ws_bytes, void* stream) {
    POETX_TRY(check_desc(d));
    if (d->variant == POETX_FOUR_PERM || d->variant == POETX_WEIGHT_CENTRIC) return POETX_ERR_UNSUPPORTED;
    if (!Wt || !q_R || !q_P || !pi_R_old || !pi_P_old || !pi_R_new || !pi_P_new) return POETX_ERR_INVALID_ARG;
    const size_t need = poetx_merge_workspace_bytes(d);
    if (ws_bytes < need) return POETX_ERR_WORKSPACE;
    if (!ws) return POETX_ERR_INVALID_ARG;
    const hipStream_t s = as_stream(stream);
    const bool bf = d->dtype == POETX_BF16;
    const int64_t m = d->m, n = d->n, b = d->b;
    const size_t es = esize(d->dtype);
    Carver cv(ws);
    void* Wq = nullptr;
    if (d->variant == POETX_MEM_Q8) {
        // merge in bf16 on the expanded weight, then store it quantized again
        Wq = Wt;
        Wt = cv.take(2 * (size_t)(m * n));
        HIP_TRY(dequantize_rows(qcodes(Wq), qscales(Wq, m, n), Wt, m, n, s));
    }
    void* G_R = cv.take(es * (size_t)(m * b));
    void* G_P = cv.take(es * (size_t)(n * b));
    void* W1 = cv.take(es * (size_t)(m * n));
    void* W2 = cv.take(es * (size_t)(m * n));
    int32_t* sig_R = cv.take_n<int32_t>(m);
    int32_t* sig_P = cv.take_n<int32_t>(n);
    int32_t* inv = cv.take_n<int32_t>(std::max(m, n));
    char* cnp_base = static_cast<char*>(cv.take(0));
    {
        Carver c1(cnp_base);
        CnpBufs B;
        plan_cnp(c1, c1, m / b, b, d->k, bf, false, B);
        POETX_TRY(cnp_forward(q_R, m / b, b, d->k, bf, G_R, bf, B, false, s));
    }
    {
        Carver c2(cnp_base);
        CnpBufs B;
        plan_cnp(c2, c2, n / b, b, d->k, bf, false, B);
        POETX_TRY(cnp_forward(q_P, n / b, b, d->k, bf, G_P, bf, B, false, s));
    }
    // W1 = diag(G_R) . Wt  (row blocks);  W2 = W1 . diag(G_P)  (column blocks)
    HIP_TRY(gemm(GemmLayout::NN, bf, bf, b, n, b, m / b, Mat{G_R, b, b * b}, Mat{Wt, n, b * n}, W1, n, b * n, s));
    HIP_TRY(gemm(GemmLayout::NN, bf, bf, m, b, b, n / b, Mat{W1, n, b}, Mat{G_P, b, b * b}, W2, n, b, s));
    // Wt'[i][j] = W2[sigma_R[i]][sigma_P[j]], sigma = pi_old^-1 o pi_new
    HIP_TRY(compose_perm(pi_R_old, pi_R_new, inv, sig_R, m, s));
    HIP_TRY(compose_perm(pi_P_old, pi_P_new, inv, sig_P, n, s));
    HIP_TRY(permute_2d(W2, Wt, bf, m, n, sig_R, sig_P, false, s));
    if (Wq)
        HIP_TRY(quantize_rows(Wt, true, m, n, static_cast<int8_t*>(Wq),
                              const_cast<float*>(qscales(Wq, m, n)), s));
    HIP_TRY(fill_zero(q_R, sizeof(float) * (size_t)(m / b) * (size_t)(b * (b - 1) / 2), s));
    HIP_TRY(fill_zero(q_P, sizeof(float) * (size_t)(n / b) * (size_t)(b * (b - 1) / 2), s));
    return POETX_OK;
}

size_t poetx_qweight_bytes(int64_t m, int64_t n) {
    if (m <= 0 || n <= 0 || m > kMaxExtent || n > kMaxExtent) return 0;
    return qscale_offset(m, n) + sizeof(float) * (size_t)m;
}

int poetx_quantize_weight(const void* W, int dtype, int64_t m, int64_t n, void* Wq, void* stream) {
    if (!dtype_ok(dtype)) return POETX_ERR_INVALID_ARG;
    if (m <= 0 || n <= 0 || m > kMaxExtent || n > kMaxExtent || n % 16) return POETX_ERR_SHAPE;
    if (!W || !Wq || ((uintptr_t)Wq & 15)) return POETX_ERR_INVALID_ARG;
    HIP_TRY(quantize_rows(W, dtype == POETX_BF16, m, n, static_cast<int8_t*>(Wq),
                          const_cast<float*>(qscales(Wq, m, n)), as_stream(stream)));
    return POETX_OK;
}

int poetx_dequantize_weight(const void* Wq, int64_t m, int64_t n, void* W, void* stream) {
    if (m <= 0 || n <= 0 || m > kMaxExtent || n > kMaxExtent || n % 16) return POETX_ERR_SHAPE;
    if (!Wq || !W || ((uintptr_t)Wq & 15) || ((uintptr_t)W & 15)) return POETX_ERR_INVALID_ARG;
    HIP_TRY(dequantize_rows(qcodes(Wq), qscales(Wq, m, n), W, m, n, as_stream(stream)));
    return POETX_OK;
}

int poetx_gemm(int layout, int dtype, int dense, int64_t M, int64_t N, int64_t K, int64_t batch, const void* A,
               int64_t lda, int64_t strideA, const void* B, int64_t ldb, int64_t strideB, void* C, int64_t ldc,
               int64_t strideC, void* stream) {
    if (!dtype_ok(dtype) || layout < POETX_GEMM_NT || layout > POETX_GEMM_TN) return POETX_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K < 0 || batch < 0 || M > kMaxExtent || N > kMaxExtent || K > kMaxExtent ||
        batch > kMaxExtent)
        return POETX_ERR_SHAPE;
    if (dense && batch > 1) return POETX_ERR_SHAPE;
    if (M == 0 || N == 0 || batch == 0) return POETX_OK;
    if (!A || !B || !C) return POETX_ERR_INVALID_ARG;
    const int64_t vec = 16 / (int64_t)esize(dtype);
    const bool a_kmajor = layout != POETX_GEMM_TN;
    const bool b_kmajor = layout == POETX_GEMM_NT;
    const int64_t a_contig = a_kmajor ? K : M, b_contig = b_kmajor ? K : N;
    if (a_contig % vec || b_contig % vec || lda % vec || ldb % vec || strideA % vec || strideB % vec)
        return POETX_ERR_SHAPE;
    if (lda < a_contig || ldb < b_contig || ldc < N) return POETX_ERR_SHAPE;
    if (((uintptr_t)A | (uintptr_t)B) & 15) return POETX_ERR_INVALID_ARG;
    const GemmLayout L = layout == POETX_GEMM_NT ? GemmLayout::NT : layout == POETX_GEMM_NN ? GemmLayout::NN
                                                                                          : GemmLayout::TN;
    const bool bf = dtype == POETX_BF16;
    if (dense) {
        HIP_TRY(dense_gemm(L, bf, M, N, K, A, lda, B, ldb, C, ldc, as_stream(stream)));
    } else {
        HIP_TRY(gemm(L, bf, bf, M, N, K, batch, Mat{A, lda, strideA}, Mat{B, ldb, strideB}, C, ldc, strideC,
                     as_stream(stream)));
    }
    return POETX_OK;
}

int poetx_block_apply(int dtype, int transpose_G, int64_t T, int64_t d, int64_t b, const void* in, const void* G,
                      void* out, void* stream) {
    if (!dtype_ok(dtype)) return POETX_ERR_INVALID_ARG;
    POETX_TRY(check_block(b));
    if (T < 0 || d <= 0 || d % b || T > kMaxExtent || d > kMaxExtent) return POETX_ERR_SHAPE;
    if (T == 0) return POETX_OK;
    if (!in || !G || !out) return POETX_ERR_INVALID_ARG;
    HIP_TRY(block_apply(transpose_G ? GemmLayout::NT : GemmLayout::NN, dtype == POETX_BF16, T, d, b, in, G, out,
                        as_stream(stream)));
    return POETX_OK;
}

int poetx_dense_fold_r(int dtype, int64_t T, int64_t m, int64_t n, int64_t b, const void* h1, const void* Wt,
                       const void* G_R, void* h2, void* z, void* stream) {
    if (!dtype_ok(dtype)) return POETX_ERR_INVALID_ARG;
    POETX_TRY(check_block(b));
    if (T < 0 || m <= 0 || n <= 0 || m % b || n % b || T > kMaxExtent || m > kMaxExtent || n > kMaxExtent)
        return POETX_ERR_SHAPE;
    if (dtype != POETX_BF16 || b != 256 || !dense_fold_r_supported(std::max<int64_t>(T, 1), m, n, n, n, m, m, 256))
        return POETX_ERR_UNSUPPORTED;
    if (T == 0) return POETX_OK;
    if (!h1 || !Wt || !G_R || !z) return POETX_ERR_INVALID_ARG;
    if (!all_al16(h1, Wt, G_R, z, h2)) return POETX_ERR_INVALID_ARG;
    HIP_TRY(dense_fold_r(false, h1, n, Wt, n, nullptr, G_R, h2, m, z, m, (int)T, (int)m, (int)n, (int)b,
                         as_stream(stream)));
    return POETX_OK;
}

size_t poetx_block_grad_workspace_bytes(int64_t T, int64_t d, int64_t b, int dtype) {
    if (!dtype_ok(dtype) || check_block(b) != POETX_OK || T < 0 || d <= 0 || d % b || T > kMaxExtent ||
        d > kMaxExtent)
        return 0;
    int splits;
    int64_t kps;
    plan_splits(T, b, d / b, dtype == POETX_BF16, splits, kps);
    return splits > 1 ? sizeof(float) * (size_t)(splits * d * b) : 0;
}

int poetx_block_grad(int dtype, int64_t T, int64_t d, int64_t b, const void* A, const void* B, float* dG, void* ws,
                     size_t ws_bytes, void* stream) {
    if (!dtype_ok(dtype)) return POETX_ERR_INVALID_ARG;
    POETX_TRY(check_block(b));
    if (T < 0 || d <= 0 || d % b || T > kMaxExtent || d > kMaxExtent) return POETX_ERR_SHAPE;
    if (!dG) return POETX_ERR_INVALID_ARG;
    const hipStream_t s = as_stream(stream);
    if (T == 0) {
        HIP_TRY(fill_zero(dG, sizeof(float) * (size_t)(d * b), s));
        return POETX_OK;
    }
    if (!A || !B) return POETX_ERR_INVALID_ARG;
    const size_t need = poetx_block_grad_workspace_bytes(T, d, b, dtype);
    if (ws_bytes < need) return POETX_ERR_WORKSPACE;
    if (need && !ws) return POETX_ERR_INVALID_ARG;
    int splits;
    int64_t kps;
    plan_splits(T, b, d / b, dtype == POETX_BF16, splits, kps);
    return block_grad(dtype == POETX_BF16, T, d, b, A, B, dG, splits, kps, static_cast<float*>(ws), s);
}

int poetx_adamw_step(float* q, const float* dq, float* m, float* v, int64_t count, int64_t step,
                     const poetx_adamw_params* p, void* stream) {
    if (!p) return POETX_ERR_INVALID_ARG;
    if (count < 0 || count > kMaxExtent) return POETX_ERR_SHAPE;
    const double lr = p->lr, gamma = p->gamma, b1 = p->beta1, b2 = p->beta2, eps = p->eps, wd = p->weight_decay;
    if (step < 1 || !std::isfinite(lr) || !std::isfinite(gamma) || !(b1 >= 0.0 && b1 < 1.0) ||
        !(b2 >= 0.0 && b2 < 1.0) || !(eps >= 0.0 && std::isfinite(eps)) || !(wd >= 0.0 && std::isfinite(wd)))
        return POETX_ERR_INVALID_ARG;
    if (count == 0) return POETX_OK;
    if (!q || !dq || !m || !v) return POETX_ERR_INVALID_ARG;
    const double eta = lr * gamma;
    const double t = (double)step;
    AdamwCoef c;
    c.beta1 = (float)b1;
    c.one_minus_beta1 = (float)(1.0 - b1);
    c.beta2 = (float)b2;
    c.one_minus_beta2 = (float)(1.0 - b2);
    c.eps = (float)eps;
    c.decay = (float)(1.0 - eta * wd);
    c.step = (float)(eta / (1.0 - std::pow(b1, t)));
    c.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(1.0 - std::pow(b2, t)));
    HIP_TRY(adamw_step(q, dq, m, v, count, c, as_stream(stream)));
    return POETX_OK;
}

int poetx_adamw_reset(float* m, float* v, int64_t count, void* stream) {
    if (count < 0 || count > kMaxExtent) return POETX_ERR_SHAPE;
    if (count == 0) return POETX_OK;
    if (!m || !v) return POETX_ERR_INVALID_ARG;
    HIP_TRY(zero_pair(m, v, count, as_stream(stream)));
    return POETX_OK;
}

}  // extern "C"
