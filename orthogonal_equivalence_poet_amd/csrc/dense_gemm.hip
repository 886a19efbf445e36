// Dense Wt products of the POET-X chain on MFMA (bf16 operands, float32
// accumulation, bf16 output):
//   forward   h2  = h1 . Wt^T   (B = Wt is [N][K], k contiguous)      "NT"
//   backward  dh1 = dh2 . Wt    (B = Wt is [K][N], n contiguous)      "NN"
// These two products carry most of the layer's arithmetic (the input-centric
// chain of the review's Summary keeps W0 frozen and never materialises R W0 P).
//
// Workgroup tile 256 x 128 x 64, four waves in a 2 x 2 grid, each wave owning a
// 128 x 64 sub-tile as 4 x 2 tiles of v_mfma_f32_32x32x16_bf16 (128 float32
// accumulators per lane, in AGPRs).
//
// Operand tiles travel global -> LDS by direct-to-LDS loads
// (global_load_lds_dwordx4: each lane's 16 bytes land at M0 + 16 * lane), so no
// VGPRs stage them and no ds_write is issued.  Three LDS stages of 48 KB form a
// ring: while the MFMAs consume stage kt % 3, the loads of tiles kt+1 and kt+2
// are in flight.  The loads are issued from inline asm so that the compiler does
// not add a conservative vmcnt(0) before every LDS read; the kernel itself waits
// (s_waitcnt vmcnt) for exactly the tile it is about to read, then barriers.
//
// LDS layouts (XOR-swizzled instead of padded, because a DMA writes whole
// 1 KB runs):
//   k-major tile [rows][64 k], 128-byte rows of eight 16-byte chunks: chunk c
//     of row r sits in slot c ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1), which
//     keeps the ds_read_b128 fragment reads free of bank conflicts for 32- and
//     64-bank LDS alike;
//   n-major tile (the NN operand) [64 k][128 n], 256-byte rows of sixteen
//     chunks: chunk c of row k sits in slot c ^ (2 (k & 7)); fragments are read
//     with ds_read_b64_tr_b16, which transposes 16-lane groups so that lane i
//     receives four consecutive k of column i.
//
// Rows past M (tokens) or N are read from the last valid row / column chunk and
// never stored; K must be a multiple of 64 (the host falls back otherwise).
#include "dense_gemm.h"
#include "device_common.h"

namespace poetx {

namespace {

constexpr int BM = 256, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int kStages = 3;
constexpr int kABytes = BM * BK * 2;                 // 32 KB
constexpr int kBBytes = BN * BK * 2;                 // 16 KB
constexpr int kStageBytes = kABytes + kBBytes;       // 48 KB
constexpr int WTM = 128, WTN = 64, MI = 4, NJ = 2;
constexpr int kLoadsPerTile = kABytes / (kThreads * 16) + kBBytes / (kThreads * 16);   // 12

typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)(lds_void_t*)p;
}

// One direct-to-LDS load: 16 bytes from gptr to M0 + 16 * lane.  m0 must be
// wave-uniform.  The instruction writes no VGPR.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(gptr)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ int swz_k(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Issue the loads of one k-tile (A and B) into the LDS stage at byte offset
// `stage`.  Wave w handles the 1 KB runs g = w, w + 4, ...
template <bool B_NN>
__device__ __forceinline__ void dma_tile(uint32_t stage, const uint16_t* __restrict__ A, int64_t lda,
                                         const uint16_t* __restrict__ B, int64_t ldb, int m0, int n0, int M,
                                         int N, int k0, int wave, int lane) {
    // A: 32 runs of 8 rows; lane -> row 8g + lane/8, slot lane % 8
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int g = j * 4 + wave;
        const int r = 8 * g + (lane >> 3);
        const int c = (lane & 7) ^ swz_k(r);
        const int row = min(m0 + r, M - 1);
        dma16(A + (int64_t)row * lda + k0 + c * 8, __builtin_amdgcn_readfirstlane(stage + g * 1024));
    }
    const uint32_t bst = stage + kABytes;
    if constexpr (!B_NN) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int g = j * 4 + wave;
            const int r = 8 * g + (lane >> 3);
            const int c = (lane & 7) ^ swz_k(r);
            const int row = min(n0 + r, N - 1);
            dma16(B + (int64_t)row * ldb + k0 + c * 8, __builtin_amdgcn_readfirstlane(bst + g * 1024));
        }
    } else {
        // B [K][N]: 16 runs of 4 k-rows; lane -> k-row 4g + lane/16, slot lane % 16
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int g = j * 4 + wave;
            const int kr = 4 * g + (lane >> 4);
            const int c = (lane & 15) ^ (2 * (kr & 7));
            const int col = min(n0 + c * 8, N - 8);
            dma16(B + (int64_t)(k0 + kr) * ldb + col, __builtin_amdgcn_readfirstlane(bst + g * 1024));
        }
    }
}

template <bool B_NN>
__device__ __forceinline__ void compute_tile(const unsigned char* __restrict__ st, int wm, int wn, int lane,
                                             f32x16_t (&acc)[MI][NJ]) {
    const unsigned char* as = st;
    const unsigned char* bs = st + kABytes;
    const int fA = (lane & 7) ^ ((lane >> 3) & 1);    // swz_k(row) for every fragment row of this lane
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
        const int slot = (2 * ks + (lane >> 5)) ^ fA;
        uint4 af[MI], bfr[NJ];
#pragma unroll
        for (int i = 0; i < MI; ++i)
            af[i] = *reinterpret_cast<const uint4*>(as + (wm * WTM + i * 32 + (lane & 31)) * 128 + slot * 16);
        if constexpr (!B_NN) {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                bfr[j] = *reinterpret_cast<const uint4*>(bs + (wn * WTN + j * 32 + (lane & 31)) * 128 + slot * 16);
        } else {
            // Two transposed reads per fragment: k = ks*16 + 8*(lane/32) + 4h + e, e = 0..3,
            // column wn*64 + 32j + lane%32.  Lane 4e + q of each 16-lane group
            // addresses k-row (kbase + e) and columns nb + 4q .. nb + 4q + 3.
            const int i16 = lane & 15;
            const int e = i16 >> 2, q = i16 & 3;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int nb = wn * WTN + 32 * j + 16 * ((lane >> 4) & 1) + 4 * q;
                s16x4_t h[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int kr = ks * 16 + 8 * (lane >> 5) + 4 * hh + e;
                    const int sl = (nb >> 3) ^ (2 * (kr & 7));
                    const unsigned char* p = bs + kr * 256 + sl * 16 + (nb & 7) * 2;
                    h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4_t*)((lds_void_t*)p));
                }
                bfr[j] = make_uint4((uint32_t)(uint16_t)h[0][0] | ((uint32_t)(uint16_t)h[0][1] << 16),
                                    (uint32_t)(uint16_t)h[0][2] | ((uint32_t)(uint16_t)h[0][3] << 16),
                                    (uint32_t)(uint16_t)h[1][0] | ((uint32_t)(uint16_t)h[1][1] << 16),
                                    (uint32_t)(uint16_t)h[1][2] | ((uint32_t)(uint16_t)h[1][3] << 16));
            }
        }
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) Mfma32<bf16_t>::run(af[i], bfr[j], acc[i][j]);
    }
}

// XCD-aware tile order: workgroups are dealt round-robin to the 8 XCDs, so
// launch slot id is regrouped to give each XCD a contiguous run of tiles in
// four-M-panel-deep order; the A and B panels an XCD shares stay in its L2.
__device__ __forceinline__ void dense_tile_coords(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int total = tiles_m * tiles_n;
    if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);
    constexpr int G = 4;
    const int group = id / (G * tiles_n);
    const int first = group * G;
    const int gm = min(G, tiles_m - first);
    const int r = id - group * G * tiles_n;
    tm = first + r % gm;
    tn = r / gm;
}

template <bool B_NN>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
dense_gemm_kernel(const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
                  uint16_t* __restrict__ C, int64_t ldc, int M, int N, int K) {
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kStages * kStageBytes];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    int tm, tn;
    dense_tile_coords(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int nk = K / BK;
    const uint32_t base = lds_offset(lds);

    f32x16_t acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    dma_tile<B_NN>(base, A, lda, B, ldb, m0, n0, M, N, 0, wave, lane);
    if (nk > 1) dma_tile<B_NN>(base + kStageBytes, A, lda, B, ldb, m0, n0, M, N, BK, wave, lane);
    int st = 0;   // stage of tile kt
    for (int kt = 0; kt < nk; ++kt) {
        // this thread's loads of tile kt are done when at most those of tile kt+1 remain
        if (kt + 1 < nk) wait_vmcnt<kLoadsPerTile>();
        else wait_vmcnt<0>();
        block_barrier();   // everyone's tile kt has landed; stage (kt+2)%3 is no longer read
        if (kt + 2 < nk) {
            const int st2 = st >= 1 ? st - 1 : 2;   // (kt + 2) % 3
            dma_tile<B_NN>(base + st2 * kStageBytes, A, lda, B, ldb, m0, n0, M, N, (kt + 2) * BK, wave, lane);
        }
        compute_tile<B_NN>(lds + st * kStageBytes, wm, wn, lane, acc);
        st = st == 2 ? 0 : st + 1;
    }

    // epilogue: lane holds rows 8 (r/4) + 4 (lane/32) + r%4 of column lane%32 per tile
    const int col0 = n0 + wn * WTN + (lane & 31);
    const int row0 = m0 + wm * WTM + (lane >> 5) * 4;
    if (m0 + BM <= M && n0 + BN <= N) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    C[(int64_t)(row0 + i * 32 + (r >> 2) * 8 + (r & 3)) * ldc + col0 + j * 32] =
                        f32_to_bf16(acc[i][j][r]);
    } else {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int col = col0 + j * 32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = row0 + i * 32 + (r >> 2) * 8 + (r & 3);
                    if (row < M && col < N) C[(int64_t)row * ldc + col] = f32_to_bf16(acc[i][j][r]);
                }
            }
    }
}

}  // namespace

bool dense_gemm_supported(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb) {
    return M > 0 && N >= 8 && K >= BK && K % BK == 0 && N % 8 == 0 && lda % 8 == 0 && ldb % 8 == 0;
}

hipError_t dense_gemm_bf16(bool b_nn, const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                           int M, int N, int K, hipStream_t stream) {
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    if (b_nn)
        hipLaunchKernelGGL(dense_gemm_kernel<true>, dim3(tiles), dim3(kThreads), 0, stream, (const uint16_t*)A, lda,
                           (const uint16_t*)B, ldb, (uint16_t*)C, ldc, M, N, K);
    else
        hipLaunchKernelGGL(dense_gemm_kernel<false>, dim3(tiles), dim3(kThreads), 0, stream, (const uint16_t*)A,
                           lda, (const uint16_t*)B, ldb, (uint16_t*)C, ldc, M, N, K);
    return hipGetLastError();
}

}  // namespace poetx
