// Batched, split-K capable GEMM on MFMA for every product of the POET-X layer:
// the dense Wt products, the batched b x b block products (tokens x b x b per
// block, review Summary "batch-wise block-diagonal matmul"), the block
// gradients (K = tokens) and the Cayley-Neumann products.
//
//   C[z] (M x N) = alpha * op(A[z]) op(B[z]) + beta1 * Cin1[z] + beta2 * Cin2[z] + gamma * I
//
// Layouts (row-major, leading dimensions in elements):
//   A_KMAJOR:  A is [M][K] (lda >= K)  else A is [K][M] (lda >= M)
//   B_KMAJOR:  B is [N][K] (ldb >= K)  else B is [K][N] (ldb >= N)
// so (A_KMAJOR, B_KMAJOR) = (1,1) is A B^T, (1,0) is A B and (0,0) is A^T B.
//
// Each workgroup stages a BM x BK tile of A and a BN x BK tile of B in LDS
// with k contiguous (operands that arrive with M or N contiguous are
// transposed in registers, 8 x 8 for bf16 and 4 x 4 for fp32, on the way in),
// double-buffers the tiles, and every wave multiplies its (BM/WM) x (BN/WN)
// sub-tile with 32x32 MFMAs from 16-byte LDS fragments.
#include "device_common.h"
#include "gemm.h"

namespace poetx {

namespace {

constexpr int kTileBytesK = 128;  // bytes of k per LDS row
constexpr int kPadBytes = 16;     // LDS row padding against bank conflicts
constexpr int kRowBytes = kTileBytesK + kPadBytes;

template <typename CT, int BM, int BN, int WM, int WN>
struct TileCfg {
    static constexpr int kVec = ElemTraits<CT>::kVec;
    static constexpr int BK = kTileBytesK / sizeof(CT);        // k elements per tile
    static constexpr int kRowElems = kRowBytes / sizeof(CT);   // LDS row stride
    static constexpr int kThreads = WM * WN * 64;
    static constexpr int WTM = BM / WM;
    static constexpr int WTN = BN / WN;
    static constexpr int MI = WTM / 32;
    static constexpr int NJ = WTN / 32;
    static constexpr int kStepK = Mfma32<CT>::kStepK;
    static constexpr int kSteps = BK / kStepK;
    static constexpr int kLdsElems = 2 * (BM + BN) * kRowElems;  // double buffered
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
};

// ------------------------------------------------------------ tile staging
// Registers that hold one operand tile in flight between global and LDS.
template <typename CT, int ROWS, int THREADS, bool KMAJOR>
struct Stager {
    static constexpr int kVec = ElemTraits<CT>::kVec;
    static constexpr int BK = kTileBytesK / sizeof(CT);
    static constexpr int kRowElems = kRowBytes / sizeof(CT);
    // K-major: ROWS x (BK / kVec) 16-byte chunks.
    // MN-major: (BK / kVec) x (ROWS / kVec) micro-tiles of kVec x kVec.
    static constexpr int kUnits = KMAJOR ? ROWS * (BK / kVec) : (BK / kVec) * (ROWS / kVec);
    static constexpr int kPerThread = (kUnits + THREADS - 1) / THREADS;
    static constexpr int kRegs = KMAJOR ? kPerThread : kPerThread * kVec;
    uint4 r[kRegs];

    // src points at the operand of this batch entry; row0 = first M/N row of
    // the tile; k0 = first k; rows_total / K bound the valid region.
    __device__ __forceinline__ void load(const CT* __restrict__ src, int64_t ld, int row0,
                                         int rows_total, int k0, int K, int tid) {
        // Rows past rows_total read the last valid row (their results are never
        // stored); k past K must contribute zero, so only a ragged k-tile is
        // predicated (a uniform branch).
        if (k0 + BK <= K) load_impl<false>(src, ld, row0, rows_total, k0, K, tid);
        else load_impl<true>(src, ld, row0, rows_total, k0, K, tid);
    }

    template <bool RAGGED_K>
    __device__ __forceinline__ void load_impl(const CT* __restrict__ src, int64_t ld, int row0,
                                              int rows_total, int k0, int K, int tid) {
#pragma unroll
        for (int u = 0; u < kPerThread; ++u) {
            const int unit = tid + u * THREADS;
            const bool live = (kUnits % THREADS == 0) || unit < kUnits;
            if (KMAJOR) {
                const int row = unit / (BK / kVec);
                const int kc = unit % (BK / kVec);
                const int gr = min(row0 + row, rows_total - 1);
                const int gk = k0 + kc * kVec;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (live && (!RAGGED_K || gk < K))
                    v = *reinterpret_cast<const uint4*>(src + (int64_t)gr * ld + gk);
                r[u] = v;
            } else {
                const int mg = unit % (ROWS / kVec);
                const int kg = unit / (ROWS / kVec);
                const int gm = min(row0 + mg * kVec, rows_total - kVec);
#pragma unroll
                for (int e = 0; e < kVec; ++e) {
                    const int gk = k0 + kg * kVec + e;
                    uint4 v = make_uint4(0, 0, 0, 0);
                    if (live && (!RAGGED_K || gk < K))
                        v = *reinterpret_cast<const uint4*>(src + (int64_t)gk * ld + gm);
                    r[u * kVec + e] = v;
                }
            }
        }
    }

    __device__ __forceinline__ void store(CT* lds, int tid) const {
#pragma unroll
        for (int u = 0; u < kPerThread; ++u) {
            const int unit = tid + u * THREADS;
            if (!(kUnits % THREADS == 0 || unit < kUnits)) continue;
            if (KMAJOR) {
                const int row = unit / (BK / kVec);
                const int kc = unit % (BK / kVec);
                *reinterpret_cast<uint4*>(lds + row * kRowElems + kc * kVec) = r[u];
            } else {
                const int mg = unit % (ROWS / kVec);
                const int kg = unit / (ROWS / kVec);
                uint4 t[kVec];
                transpose(&r[u * kVec], t);
#pragma unroll
                for (int j = 0; j < kVec; ++j)
                    *reinterpret_cast<uint4*>(lds + (mg * kVec + j) * kRowElems + kg * kVec) = t[j];
            }
        }
    }

    // in[e] holds kVec elements (mn = 0..kVec-1) at k = e; out[j] holds the kVec
    // k values of column mn = j.
    __device__ __forceinline__ static void transpose(const uint4* in, uint4* out) {
        if constexpr (sizeof(CT) == 4) {
            const uint32_t* w[4] = {&in[0].x, &in[1].x, &in[2].x, &in[3].x};
#pragma unroll
            for (int j = 0; j < 4; ++j) out[j] = make_uint4(w[0][j], w[1][j], w[2][j], w[3][j]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                uint32_t o[4];
#pragma unroll
                for (int wd = 0; wd < 4; ++wd) {
                    const uint32_t lo_word = (&in[2 * wd].x)[j >> 1];
                    const uint32_t hi_word = (&in[2 * wd + 1].x)[j >> 1];
                    const uint32_t lo = (j & 1) ? (lo_word >> 16) : (lo_word & 0xffffu);
                    const uint32_t hi = (j & 1) ? (hi_word & 0xffff0000u) : (hi_word << 16);
                    o[wd] = lo | hi;
                }
                out[j] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    }
};

// Tile index -> (tile_m, tile_n).  Workgroups are dealt round-robin to the 8
// XCDs; consecutive launch slots are first regrouped so that each XCD owns a
// contiguous run of tiles in GROUP_M-grouped order, which keeps the A and B
// panels that an XCD shares inside its own L2.
__device__ __forceinline__ void tile_coords(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int total = tiles_m * tiles_n;
    if ((total & 7) == 0) {
        const int per_xcd = total >> 3;
        id = (id & 7) * per_xcd + (id >> 3);
    }
    constexpr int GROUP_M = 4;
    const int group_size = GROUP_M * tiles_n;
    const int group = id / group_size;
    const int first_m = group * GROUP_M;
    const int gm = min(GROUP_M, tiles_m - first_m);
    const int in_group = id - group * group_size;
    tm = first_m + in_group % gm;
    tn = in_group / gm;
}

// Register budget: the Large tile's 110.6 KB of LDS allows one workgroup (one
// wave per SIMD) per CU, so it may use the whole register file; the others run
// two or more workgroups per CU.
template <int BM, int BN> struct WavesPerEu {
    static constexpr int lo = (BM * BN >= 256 * 128) ? 1 : 2;
    static constexpr int hi = (BM * BN >= 256 * 128) ? 1 : 4;
};

template <typename CT, typename OutT, bool A_KMAJOR, bool B_KMAJOR, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(WM* WN * 64) __attribute__((amdgpu_waves_per_eu(WavesPerEu<BM, BN>::lo, WavesPerEu<BM, BN>::hi)))
gemm_kernel(const GemmArgs p) {
    using Cfg = TileCfg<CT, BM, BN, WM, WN>;
    constexpr int BK = Cfg::BK;
    constexpr int RE = Cfg::kRowElems;
    constexpr int NT = Cfg::kThreads;
    __shared__ __attribute__((aligned(16))) CT lds[Cfg::kLdsElems];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN;
    const int wn = wave % WN;

    const int tiles_m = (p.M + BM - 1) / BM;
    const int tiles_n = (p.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int split = blockIdx.y;
    const int z = blockIdx.z;

    const CT* A = reinterpret_cast<const CT*>(p.A) + (int64_t)z * p.strideA;
    const CT* B = reinterpret_cast<const CT*>(p.B) + (int64_t)z * p.strideB;

    const int k_begin = split * p.k_per_split;
    const int k_end = min(p.K, k_begin + p.k_per_split);
    const int ntiles_k = k_end > k_begin ? (k_end - k_begin + BK - 1) / BK : 0;

    Stager<CT, BM, NT, A_KMAJOR> sa;
    Stager<CT, BN, NT, B_KMAJOR> sb;

    f32x16_t acc[Cfg::MI][Cfg::NJ];
#pragma unroll
    for (int i = 0; i < Cfg::MI; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    constexpr int kBufElems = (BM + BN) * RE;   // one stage: A tile then B tile

    // One register stage, two LDS stages: after the MFMAs of k-tile kt the
    // registers holding tile kt+1 go to LDS and the loads of tile kt+2 are
    // issued at once, so every load has a whole k-tile of MFMA work to land.
    if (ntiles_k > 0) {
        sa.load(A, p.lda, tm * BM, p.M, k_begin, k_end, tid);
        sb.load(B, p.ldb, tn * BN, p.N, k_begin, k_end, tid);
        sa.store(lds, tid);
        sb.store(lds + BM * RE, tid);
        if (ntiles_k > 1) {
            sa.load(A, p.lda, tm * BM, p.M, k_begin + BK, k_end, tid);
            sb.load(B, p.ldb, tn * BN, p.N, k_begin + BK, k_end, tid);
        }
    }
    __syncthreads();

    const int frag_row = lane & 31;
    const int frag_k = (lane >> 5) * Cfg::kVec;
    for (int kt = 0; kt < ntiles_k; ++kt) {
        const int cur = kt & 1;
        const CT* as = lds + cur * kBufElems + (wm * Cfg::WTM + frag_row) * RE + frag_k;
        const CT* bs = lds + cur * kBufElems + BM * RE + (wn * Cfg::WTN + frag_row) * RE + frag_k;
#pragma unroll
        for (int ks = 0; ks < Cfg::kSteps; ++ks) {
            uint4 af[Cfg::MI], bfr[Cfg::NJ];
#pragma unroll
            for (int i = 0; i < Cfg::MI; ++i)
                af[i] = *reinterpret_cast<const uint4*>(as + i * 32 * RE + ks * Cfg::kStepK);
#pragma unroll
            for (int j = 0; j < Cfg::NJ; ++j)
                bfr[j] = *reinterpret_cast<const uint4*>(bs + j * 32 * RE + ks * Cfg::kStepK);
#pragma unroll
            for (int i = 0; i < Cfg::MI; ++i)
#pragma unroll
                for (int j = 0; j < Cfg::NJ; ++j) Mfma32<CT>::run(af[i], bfr[j], acc[i][j]);
        }
        if (kt + 1 < ntiles_k) {
            sa.store(lds + (cur ^ 1) * kBufElems, tid);
            sb.store(lds + (cur ^ 1) * kBufElems + BM * RE, tid);
            if (kt + 2 < ntiles_k) {
                const int k0 = k_begin + (kt + 2) * BK;
                sa.load(A, p.lda, tm * BM, p.M, k0, k_end, tid);
                sb.load(B, p.ldb, tn * BN, p.N, k0, k_end, tid);
            }
        }
        __syncthreads();
    }

    // ------------------------------------------------------------ epilogue
    OutT* C = reinterpret_cast<OutT*>(p.C);
    CT* C2 = reinterpret_cast<CT*>(p.C2);
    const int64_t zc = (int64_t)z * p.strideC + (int64_t)split * p.strideSplit;
    const int64_t zc2 = (int64_t)z * p.strideC2;
    const int64_t zi1 = (int64_t)z * p.strideCin1;
    const int64_t zi2 = (int64_t)z * p.strideCin2;
    const int col_base = tn * BN + wn * Cfg::WTN + (lane & 31);
    const int row_base = tm * BM + wm * Cfg::WTM + (lane >> 5) * 4;
    const bool plain = !p.Cin1 && !p.Cin2 && !C2 && p.gamma == 0.f && p.alpha == 1.f && p.mode == 0;
    if (plain) {
        OutT* Cz = C + zc;
#pragma clang loop unroll(full)
        for (int i = 0; i < Cfg::MI; ++i)
#pragma clang loop unroll(full)
            for (int j = 0; j < Cfg::NJ; ++j) {
                const int col = col_base + j * 32;
#pragma clang loop unroll(full)
                for (int r = 0; r < 16; ++r) {
                    const int row = row_base + i * 32 + (r >> 2) * 8 + (r & 3);
                    if (row < p.M && col < p.N) store_f32(Cz + (int64_t)row * p.ldc + col, acc[i][j][r]);
                }
            }
    } else {
        // General epilogue: the float32 addends of a 32 x 32 tile are fetched
        // first (16 independent loads per lane), then combined and stored.
        const float* __restrict__ cin1 = p.Cin1 ? p.Cin1 + zi1 : nullptr;
        const float* __restrict__ cin2 = p.Cin2 ? p.Cin2 + zi2 : nullptr;
        OutT* __restrict__ c1 = C ? C + zc : nullptr;
        CT* __restrict__ c2 = C2 ? C2 + zc2 : nullptr;
        CT* __restrict__ c3 = p.C3 ? reinterpret_cast<CT*>(p.C3) + zc2 : nullptr;
#pragma clang loop unroll(full)
        for (int i = 0; i < Cfg::MI; ++i)
#pragma clang loop unroll(full)
            for (int j = 0; j < Cfg::NJ; ++j) {
                const int col = col_base + j * 32;
                float a1[16], a2[16];
#pragma clang loop unroll(full)
                for (int r = 0; r < 16; ++r) {
                    const int row = min(row_base + i * 32 + (r >> 2) * 8 + (r & 3), p.M - 1);
                    const int cc = min(col, p.N - 1);
                    a1[r] = cin1 ? cin1[(int64_t)row * p.ldcin1 + cc] : 0.f;
                    a2[r] = cin2 ? cin2[(int64_t)row * p.ldcin2 + cc] : 0.f;
                }
#pragma clang loop unroll(full)
                for (int r = 0; r < 16; ++r) {
                    const int row = row_base + i * 32 + (r >> 2) * 8 + (r & 3);
                    if (row >= p.M || col >= p.N) continue;
                    const float v = p.alpha * acc[i][j][r];
                    if (p.mode == 1) {
                        const float q2 = 2.f * a1[r];
                        c1[(int64_t)row * p.ldc + col] = ElemTraits<OutT>::from_f32(q2 + 2.f * v);
                        store_f32(c2 + (int64_t)row * p.ldc2 + col, v);
                        store_f32(c3 + (int64_t)row * p.ldc2 + col, q2 + v);
                        continue;
                    }
                    float o = v + p.beta1 * a1[r] + p.beta2 * a2[r];
                    if (row == col) o += p.gamma;
                    if (c1) store_f32(c1 + (int64_t)row * p.ldc + col, o);
                    if (c2) store_f32(c2 + (int64_t)row * p.ldc2 + col, o);
                }
            }
    }
}

template <typename CT, typename OutT, bool AK, bool BKM, int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const GemmArgs& p, hipStream_t stream) {
    const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    constexpr int kMaxZ = 65535;
    for (int z0 = 0; z0 < p.batch; z0 += kMaxZ) {
        GemmArgs q = p;
        q.batch = p.batch - z0 < kMaxZ ? p.batch - z0 : kMaxZ;
        q.A = reinterpret_cast<const CT*>(p.A) + (int64_t)z0 * p.strideA;
        q.B = reinterpret_cast<const CT*>(p.B) + (int64_t)z0 * p.strideB;
        if (p.C) q.C = reinterpret_cast<OutT*>(p.C) + (int64_t)z0 * p.strideC;
        if (p.C2) q.C2 = reinterpret_cast<CT*>(p.C2) + (int64_t)z0 * p.strideC2;
        if (p.C3) q.C3 = reinterpret_cast<CT*>(p.C3) + (int64_t)z0 * p.strideC2;
        if (p.Cin1) q.Cin1 = p.Cin1 + (int64_t)z0 * p.strideCin1;
        if (p.Cin2) q.Cin2 = p.Cin2 + (int64_t)z0 * p.strideCin2;
        dim3 grid(tiles, p.splits, q.batch);
        hipLaunchKernelGGL((gemm_kernel<CT, OutT, AK, BKM, BM, BN, WM, WN>), grid, dim3(WM * WN * 64), 0,
                           stream, q);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename CT, typename OutT, bool AK, bool BKM>
hipError_t launch_layout(const GemmArgs& p, GemmTile tile, hipStream_t stream) {
    if constexpr (sizeof(CT) == 2) {
        switch (tile) {
            case GemmTile::Large: return launch_cfg<CT, OutT, AK, BKM, 256, 128, 2, 2>(p, stream);
            case GemmTile::Medium: return launch_cfg<CT, OutT, AK, BKM, 128, 128, 2, 2>(p, stream);
            default: return launch_cfg<CT, OutT, AK, BKM, 64, 64, 2, 2>(p, stream);
        }
    } else {
        switch (tile) {
            case GemmTile::Small: return launch_cfg<CT, OutT, AK, BKM, 64, 64, 2, 2>(p, stream);
            default: return launch_cfg<CT, OutT, AK, BKM, 128, 128, 2, 2>(p, stream);
        }
    }
}

template <typename CT, typename OutT>
hipError_t launch_types(const GemmArgs& p, GemmLayout layout, GemmTile tile, hipStream_t stream) {
    switch (layout) {
        case GemmLayout::NT: return launch_layout<CT, OutT, true, true>(p, tile, stream);
        case GemmLayout::NN: return launch_layout<CT, OutT, true, false>(p, tile, stream);
        default: return launch_layout<CT, OutT, false, false>(p, tile, stream);
    }
}

}  // namespace

int gemm_tile_rows(GemmTile tile, bool bf16) {
    if (bf16) return tile == GemmTile::Large ? 256 : tile == GemmTile::Medium ? 128 : 64;
    return tile == GemmTile::Small ? 64 : 128;
}

int gemm_tile_cols(GemmTile tile, bool bf16) {
    if (bf16) return tile == GemmTile::Small ? 64 : 128;
    return tile == GemmTile::Small ? 64 : 128;
}

int gemm_tile_k(bool bf16) { return bf16 ? 64 : 32; }

hipError_t gemm_launch(const GemmArgs& p, GemmLayout layout, GemmTile tile, bool compute_bf16,
                       bool out_bf16, hipStream_t stream) {
    if (p.M <= 0 || p.N <= 0 || p.batch <= 0 || p.splits <= 0) return hipSuccess;
    if (compute_bf16) {
        if (out_bf16) return launch_types<bf16_t, bf16_t>(p, layout, tile, stream);
        return launch_types<bf16_t, float>(p, layout, tile, stream);
    }
    return launch_types<float, float>(p, layout, tile, stream);
}

}  // namespace poetx
