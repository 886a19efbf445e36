// Dense Wt products of the POET-X chain on MFMA (bf16 operands, float32
// accumulation, bf16 output):
//   forward   h2  = h1 . Wt^T   (B = Wt is [N][K], k contiguous)      "NT"
//   backward  dh1 = dh2 . Wt    (B = Wt is [K][N], n contiguous)      "NN"
// These two products carry most of the layer's arithmetic (the input-centric
// chain of the review's Summary keeps W0 frozen and never materialises R W0 P).
//
// Workgroup tile 256 x 128 x 64, four waves in a 2 x 2 grid, each wave owning a
// 128 x 64 sub-tile as 4 x 2 tiles of v_mfma_f32_32x32x16_bf16 (128 float32
// accumulators per lane).  Operand tiles are staged in LDS with k contiguous
// and a 16-byte row pad (conflict-free ds_read_b128 fragments); the NN operand
// is transposed in registers (8 k x 4 n per thread) on its way to LDS.
// Global loads run one k-tile ahead of the MFMAs (one register stage, two LDS
// stages), so a load has a full k-tile of MFMA work to land.  One workgroup per
// CU (110.6 KB of LDS), so the kernel is compiled for one wave per SIMD and may
// use the whole register file.
//
// Rows past M (tokens) or N are read from the last valid row and never
// stored; K must be a multiple of 64 (the host falls back otherwise).
#include "dense_gemm.h"
#include "device_common.h"

namespace poetx {

namespace {

constexpr int BM = 256, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int kRow = BK + 8;                 // LDS row stride in bf16 elements (144 bytes)
constexpr int kStage = (BM + BN) * kRow;     // elements per LDS stage
constexpr int WTM = 128, WTN = 64, MI = 4, NJ = 2;

struct Regs {
    uint4 a[8];   // A: 8 chunks of 16 bytes per thread
    uint4 b[4];   // B (NT): 4 chunks; (NN): 8 x 8-byte loads packed two per uint4
};

template <bool B_NN>
__device__ __forceinline__ void load_tile(Regs& R, const uint16_t* __restrict__ A, int64_t lda,
                                          const uint16_t* __restrict__ B, int64_t ldb, int m0, int n0, int M,
                                          int N, int k0, int tid) {
    // A: 256 rows x 8 chunks; thread -> rows tid/8 + 32 i, chunk tid % 8
    const int kc = tid & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = min(m0 + (tid >> 3) + 32 * i, M - 1);
        R.a[i] = *reinterpret_cast<const uint4*>(A + (int64_t)row * lda + k0 + kc * 8);
    }
    if constexpr (!B_NN) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = min(n0 + (tid >> 3) + 32 * i, N - 1);
            R.b[i] = *reinterpret_cast<const uint4*>(B + (int64_t)row * ldb + k0 + kc * 8);
        }
    } else {
        // B [K][N]: thread owns k = 8 * (tid % 8) .. +7 and n = 4 * (tid / 8) .. +3
        const int n = min(n0 + 4 * (tid >> 3), N - 4);
        const int kb = k0 + 8 * (tid & 7);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint2 v = *reinterpret_cast<const uint2*>(B + (int64_t)(kb + e) * ldb + n);
            if (e & 1) {
                R.b[e >> 1].z = v.x;
                R.b[e >> 1].w = v.y;
            } else {
                R.b[e >> 1].x = v.x;
                R.b[e >> 1].y = v.y;
            }
        }
    }
}

template <bool B_NN>
__device__ __forceinline__ void store_tile(const Regs& R, uint16_t* __restrict__ lds, int tid) {
    uint16_t* la = lds;
    uint16_t* lb = lds + BM * kRow;
    const int kc = tid & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        *reinterpret_cast<uint4*>(la + ((tid >> 3) + 32 * i) * kRow + kc * 8) = R.a[i];
    if constexpr (!B_NN) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint4*>(lb + ((tid >> 3) + 32 * i) * kRow + kc * 8) = R.b[i];
    } else {
        // R.b[e/2] holds k = e (e = 0..7) for the 4 columns: words (x,y) even e, (z,w) odd e.
        // Column j of the 4: bf16 j of the 8-byte group.
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t o[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {  // k pair (2p, 2p+1) -> R.b[p] even/odd halves
                const uint32_t ev = (j < 2) ? R.b[p].x : R.b[p].y;
                const uint32_t od = (j < 2) ? R.b[p].z : R.b[p].w;
                const uint32_t lo = (j & 1) ? (ev >> 16) : (ev & 0xffffu);
                const uint32_t hi = (j & 1) ? (od & 0xffff0000u) : (od << 16);
                o[p] = lo | hi;
            }
            *reinterpret_cast<uint4*>(lb + (4 * (tid >> 3) + j) * kRow + kc * 8) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
}

__device__ __forceinline__ void compute_tile(const uint16_t* __restrict__ lds, int wm, int wn, int lane,
                                             f32x16_t (&acc)[MI][NJ]) {
    const uint16_t* as = lds + (wm * WTM + (lane & 31)) * kRow + (lane >> 5) * 8;
    const uint16_t* bs = lds + BM * kRow + (wn * WTN + (lane & 31)) * kRow + (lane >> 5) * 8;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
        uint4 af[MI], bfr[NJ];
#pragma unroll
        for (int i = 0; i < MI; ++i) af[i] = *reinterpret_cast<const uint4*>(as + i * 32 * kRow + ks * 16);
#pragma unroll
        for (int j = 0; j < NJ; ++j) bfr[j] = *reinterpret_cast<const uint4*>(bs + j * 32 * kRow + ks * 16);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) Mfma32<bf16_t>::run(af[i], bfr[j], acc[i][j]);
    }
}

// XCD-aware tile order (see gemm.hip): each XCD works through a contiguous run
// of tiles grouped four M-panels deep, sharing A and B panels in its L2.
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
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kStage];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    int tm, tn;
    dense_tile_coords(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int nk = K / BK;

    f32x16_t acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // One register stage, two LDS stages: tile kt+1 is written to LDS right
    // after the MFMAs of tile kt and the loads of tile kt+2 are issued at once,
    // so every load has the MFMA work of a whole k-tile to land.
    Regs R;
    load_tile<B_NN>(R, A, lda, B, ldb, m0, n0, M, N, 0, tid);
    store_tile<B_NN>(R, lds, tid);
    if (nk > 1) load_tile<B_NN>(R, A, lda, B, ldb, m0, n0, M, N, BK, tid);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        compute_tile(lds + (kt & 1) * kStage, wm, wn, lane, acc);
        if (kt + 1 < nk) {
            store_tile<B_NN>(R, lds + ((kt + 1) & 1) * kStage, tid);
            if (kt + 2 < nk) load_tile<B_NN>(R, A, lda, B, ldb, m0, n0, M, N, (kt + 2) * BK, tid);
        }
        __syncthreads();
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
    return M > 0 && N >= 4 && K >= BK && K % BK == 0 && N % 8 == 0 && lda % 8 == 0 && ldb % 8 == 0;
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
