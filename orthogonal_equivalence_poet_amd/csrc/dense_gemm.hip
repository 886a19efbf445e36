// Pipelined bf16 MFMA GEMM (float32 accumulation) for the large products of the
// POET-X chain (the input-centric, matrix-free reformulation of the review's
// Summary keeps W0 frozen and never materialises R W0 P):
//   dense   h2  = h1 . Wt^T  (A k-major, B k-major)   dh1 = dh2 . Wt (B n-major)
//   blocks  h1_j = a_j . G_j^T, dh2_j = dz_j . G_j     (batched over blocks j)
//   grads   dG_j = dz_j^T h2_j                          (A and B m/n-major, K = tokens,
//                                                        split along K, float32 out)
//
//   small   the Cayley-Neumann b x b products (batched over blocks, general
//           epilogue with float32 addends and several outputs)
//
// Workgroup tile BM x BN x 64 (256 x 128 for the dense products, 256 x 256 once
// there are enough of those to fill the chip, 128 x 256 for
// the block products, 128 x 128 for the block gradients, 64 x 64 or 128 x 128
// for the small products), four waves in a 2 x 2 grid, each wave owning a
// (BM/2) x (BN/2) sub-tile of v_mfma_f32_32x32x16_bf16 tiles (float32
// accumulators in AGPRs).
//
// Operand tiles travel global -> LDS by direct-to-LDS loads
// (global_load_lds_dwordx4: each lane's 16 bytes land at M0 + 16 * lane), so no
// VGPRs stage them and no ds_write is issued.  S LDS stages form a ring (S = 3
// for the large tiles, 4 for the 128 x 128 and 64 x 64 ones): while the MFMAs
// consume stage kt % S, the loads of tiles kt+1 .. kt+S-1 are in flight, so a
// short product (K = 256) waits for memory once.  The loads are issued from inline asm so that the compiler does not
// add a conservative vmcnt(0) before every LDS read; the kernel itself waits
// (s_waitcnt vmcnt) for exactly the tile it is about to read, then barriers.
//
// LDS layouts (XOR-swizzled instead of padded, because a DMA writes whole
// 1 KB runs):
//   k-major tile [rows][64 k], 128-byte rows of eight 16-byte chunks: chunk c
//     of row r sits in slot c ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1), which
//     keeps the ds_read_b128 fragment reads free of bank conflicts;
//   m/n-major tile [64 k][rows], 256- or 512-byte rows: chunk c of k-row k sits
//     in slot c ^ 4 (k & 3) (128-byte rows: c ^ 4 ((k >> 1) & 1)); fragments are read with ds_read_b64_tr_b16, which
//     transposes 16-lane groups so that lane i receives four consecutive k of
//     column i; the swizzle spreads the four k-rows x four chunks that 32 lanes
//     touch over all 64 banks.
//
// Rows past M or N are read from the last valid row / column chunk and never
// stored.  K-contiguous operands need K % 64 == 0; for m/n-major operands a
// ragged last k-tile is loaded from clamped rows and its rows past K are zeroed
// in LDS before use.
#include <type_traits>

#include "dense_gemm.h"
#include "device_common.h"

namespace poetx {

namespace {

constexpr int BK = 64;

// Workgroup tile BM x BN (x 64 k), NWM x NWN waves, each owning a WTM x WTN
// sub-tile of MI x NJ 32 x 32 MFMA tiles.
template <int BM_, int BN_, int NWM_ = 2, int NWN_ = 2>
struct Geo {
    static constexpr int BM = BM_, BN = BN_, NWM = NWM_, NWN = NWN_;
    static constexpr int NW = NWM * NWN;
    static constexpr int kThreads = 64 * NW;
    static constexpr int kABytes = BM * BK * 2;
    static constexpr int kBBytes = BN * BK * 2;
    static constexpr int kStageBytes = kABytes + kBBytes;
    static constexpr int WTM = BM / NWM, WTN = BN / NWN, MI = WTM / 32, NJ = WTN / 32;
    static constexpr int kLoadsPerTile = (kABytes + kBBytes) / (kThreads * 16);
    static_assert(MI >= 1 && NJ >= 1 && (kABytes + kBBytes) % (kThreads * 16) == 0, "tile geometry");
};

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
// m/n-major k-rows of 16 or more chunks rotate by 4 chunks per k; 64-column
// tiles (8 chunks, two k-rows per 256 bytes of banks) flip by 4 every other k.
template <int ROWS>
__device__ __forceinline__ int swz_mn(int k) {
    if constexpr (ROWS >= 128) return 4 * (k & 3);
    else return 4 * ((k >> 1) & 1);
}

// Loads of one operand tile into LDS at byte offset `dst`.
//   k-major: ROWS rows x 64 k from src[row][k] (ld = row stride), rows clamped to rows_total.
//   m/n-major: 64 k-rows x ROWS from src[k][col] (ld = k-row stride), k clamped to k_end,
//   columns clamped to rows_total.
// With NW waves each thread issues OperandLoads<ROWS, MN, NW>::n loads;
// dma_one issues the j-th.
template <int ROWS, bool MN, int NW>
struct OperandLoads {
    static constexpr int runs = ROWS * BK * 2 / 1024;   // 1 KB runs per operand tile
    static constexpr int n = runs / NW;
    static_assert(runs % NW == 0, "runs per wave");
};

template <int ROWS, bool MN, int NW>
__device__ __forceinline__ void dma_one(int j, uint32_t dst, const uint16_t* __restrict__ src, int64_t ld, int r0,
                                        int rows_total, int k0, int k_end, int wave, int lane) {
    const int g = j * NW + wave;   // 1 KB run of this wave
    if constexpr (!MN) {
        const int r = 8 * g + (lane >> 3);           // 8 rows of 128 bytes per run
        const int c = (lane & 7) ^ swz_k(r);
        const int row = min(r0 + r, rows_total - 1);
        dma16(src + (int64_t)row * ld + k0 + c * 8, __builtin_amdgcn_readfirstlane(dst + g * 1024));
    } else {
        constexpr int kRowBytes = ROWS * 2;          // one k-row
        constexpr int kRowsPerRun = 1024 / kRowBytes;
        constexpr int kSlots = kRowBytes / 16;
        const int kr = kRowsPerRun * g + lane / kSlots;
        const int c = (lane % kSlots) ^ swz_mn<ROWS>(kr);
        const int col = min(r0 + c * 8, rows_total - 8);
        const int k = min(k0 + kr, k_end - 1);
        dma16(src + (int64_t)k * ld + col, __builtin_amdgcn_readfirstlane(dst + g * 1024));
    }
}

// Everything needed to issue the loads of one k-tile into one LDS stage.
struct DmaJob {
    uint32_t stage;
    const uint16_t* A;
    int64_t lda;
    const uint16_t* B;
    int64_t ldb;
    int m0, n0, M, N, k0, k_end, wave, lane;
};

// Part PART of NPARTS of a k-tile's loads (A's loads first, then B's), so the
// loads can be spread over the MFMA work of the tile being computed.
template <class G, bool A_MN, bool B_MN, int PART, int NPARTS>
__device__ __forceinline__ void dma_part(const DmaJob& d) {
    constexpr int NA = OperandLoads<G::BM, A_MN, G::NW>::n, NB = OperandLoads<G::BN, B_MN, G::NW>::n;
    constexpr int L = NA + NB;
    constexpr int lo = PART * L / NPARTS, hi = (PART + 1) * L / NPARTS;
#pragma unroll
    for (int idx = lo; idx < hi; ++idx) {
        if (idx < NA)
            dma_one<G::BM, A_MN, G::NW>(idx, d.stage, d.A, d.lda, d.m0, d.M, d.k0, d.k_end, d.wave, d.lane);
        else
            dma_one<G::BN, B_MN, G::NW>(idx - NA, d.stage + G::kABytes, d.B, d.ldb, d.n0, d.N, d.k0, d.k_end,
                                        d.wave, d.lane);
    }
}

template <class G, bool A_MN, bool B_MN>
__device__ __forceinline__ void dma_tile(const DmaJob& d) {
    dma_part<G, A_MN, B_MN, 0, 1>(d);
}

// Fragment of 32 rows (k-major) or 32 columns (m/n-major) starting at `row0`
// for k-step ks: lane l gets row/column row0 + l%32 and k = 16 ks + 8 (l/32) + 0..7.
template <bool MN, int ROWS>
__device__ __forceinline__ uint4 load_frag(const unsigned char* __restrict__ base, int row0, int ks, int lane) {
    if constexpr (!MN) {
        const int slot = (2 * ks + (lane >> 5)) ^ ((lane & 7) ^ ((lane >> 3) & 1));
        return *reinterpret_cast<const uint4*>(base + (row0 + (lane & 31)) * 128 + slot * 16);
    } else {
        // Two transposed reads: lane 4e + q of each 16-lane group addresses k-row
        // (kbase + e) and columns cb + 4q .. cb + 4q + 3.
        const int i16 = lane & 15;
        const int e = i16 >> 2, q = i16 & 3;
        const int cb = row0 + 16 * ((lane >> 4) & 1) + 4 * q;
        s16x4_t h[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int kr = ks * 16 + 8 * (lane >> 5) + 4 * hh + e;
            const int sl = (cb >> 3) ^ swz_mn<ROWS>(kr);
            const unsigned char* p = base + kr * (ROWS * 2) + sl * 16 + (cb & 7) * 2;
            h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4_t*)((lds_void_t*)p));
        }
        return make_uint4((uint32_t)(uint16_t)h[0][0] | ((uint32_t)(uint16_t)h[0][1] << 16),
                          (uint32_t)(uint16_t)h[0][2] | ((uint32_t)(uint16_t)h[0][3] << 16),
                          (uint32_t)(uint16_t)h[1][0] | ((uint32_t)(uint16_t)h[1][1] << 16),
                          (uint32_t)(uint16_t)h[1][2] | ((uint32_t)(uint16_t)h[1][3] << 16));
    }
}

// One k-tile (four k-steps of 16).  Fragments are double-buffered in
// registers: the LDS reads of step ks+1 are issued before the MFMAs of step
// ks, and scheduling barriers keep the compiler from sinking them, so each
// wave (one per SIMD) waits for LDS once per k-tile instead of once per
// fragment.
template <class G, bool A_MN, bool B_MN>
__device__ __forceinline__ void load_frags(const unsigned char* __restrict__ st, int wm, int wn, int ks, int lane,
                                           uint4 (&af)[G::MI], uint4 (&bfr)[G::NJ]) {
#pragma unroll
    for (int i = 0; i < G::MI; ++i) af[i] = load_frag<A_MN, G::BM>(st, wm * G::WTM + i * 32, ks, lane);
#pragma unroll
    for (int j = 0; j < G::NJ; ++j) bfr[j] = load_frag<B_MN, G::BN>(st + G::kABytes, wn * G::WTN + j * 32, ks, lane);
}

template <class G, bool A_MN, bool B_MN>
__device__ __forceinline__ void compute_tile(const unsigned char* __restrict__ st, int wm, int wn, int lane,
                                             f32x16_t (&acc)[G::MI][G::NJ], const DmaJob& next, bool load_next) {
    uint4 af[2][G::MI], bfr[2][G::NJ];
    load_frags<G, A_MN, B_MN>(st, wm, wn, 0, lane, af[0], bfr[0]);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
        const int cur = ks & 1;
        if (ks + 1 < BK / 16) load_frags<G, A_MN, B_MN>(st, wm, wn, ks + 1, lane, af[cur ^ 1], bfr[cur ^ 1]);
        // a quarter of the next tile's loads per k-step
        if (load_next) {
            switch (ks) {
                case 0: dma_part<G, A_MN, B_MN, 0, 4>(next); break;
                case 1: dma_part<G, A_MN, B_MN, 1, 4>(next); break;
                case 2: dma_part<G, A_MN, B_MN, 2, 4>(next); break;
                default: dma_part<G, A_MN, B_MN, 3, 4>(next); break;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < G::MI; ++i)
#pragma unroll
            for (int j = 0; j < G::NJ; ++j) Mfma32<bf16_t>::run(af[cur][i], bfr[cur][j], acc[i][j]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Zero the k-rows >= valid of an m/n-major tile (ragged last k-tile).
template <int ROWS, int kThreads>
__device__ __forceinline__ void zero_rows_mn(unsigned char* __restrict__ base, int valid, int tid) {
    constexpr int kChunks = ROWS * 2 / 16;   // 16-byte chunks per k-row
    for (int u = tid; u < (64 - valid) * kChunks; u += kThreads) {
        const int r = valid + u / kChunks;
        *reinterpret_cast<uint4*>(base + r * ROWS * 2 + (u % kChunks) * 16) = make_uint4(0, 0, 0, 0);
    }
}

// XCD-aware tile order: workgroups are dealt round-robin to the 8 XCDs, so
// launch slot id is regrouped to give each XCD a contiguous run of tiles in
// four-M-panel-deep order; the A and B panels an XCD shares stay in its L2.
__device__ __forceinline__ void tile_coords(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
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

// Batched launches (grid.y = batch entries): the launch slots an XCD receives
// are regrouped so that each XCD owns whole batch entries, and every operand
// panel of an entry is fetched into one L2 only.  Within an entry tiles run
// down the M direction first.  A single product keeps the grouped order above.
__device__ __forceinline__ void batch_tile_coords(int tiles_m, int tiles_n, int& z, int& tm, int& tn) {
    if (gridDim.y == 1) {
        z = 0;
        tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
        return;
    }
    const int tiles = tiles_m * tiles_n;
    const int total = tiles * (int)gridDim.y;
    int id = blockIdx.x + tiles * blockIdx.y;
    if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);
    z = id / tiles;
    const int t = id - z * tiles;
    tm = t % tiles_m;
    tn = t / tiles_m;
}

// Register budget: the 256 x 128 and 128 x 256 tiles hold 128 accumulators per
// lane and their LDS ring allows one workgroup per CU, so they take the whole
// register file; smaller tiles leave room for several workgroups per CU.
template <int BM, int BN, int NW> struct PipeWaves {
    static constexpr int lo = 1;
    static constexpr int hi = (BM * BN >= 256 * 128) ? NW / 4 : 4;
};

// General epilogue (see PipeArgs), staged through LDS: the waves write their
// accumulators into a BM x BN float32 tile (rows padded by 8 floats so that
// the two row groups of a 32 x 32 MFMA tile land in different banks), then
// every thread combines and stores row-contiguous 4-column chunks: 16-byte
// float32 loads and stores, 8-byte bf16 stores, whole 256- or 512-byte rows
// per wave instruction.  Chunks are taken element-wise when the host found
// the addresses unsuited to vectors or the tile is clipped.
template <int BM, int BN>
struct EpiTile {
    static constexpr int kLd = BN + 8;                       // floats per LDS row
    static constexpr int kBytes = BM * kLd * 4;
};

__device__ __forceinline__ float4 load4(const float* __restrict__ p, bool vec, bool full, int valid) {
    if (vec && full) return *reinterpret_cast<const float4*>(p);
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid > 0) v.x = p[0];
    if (valid > 1) v.y = p[1];
    if (valid > 2) v.z = p[2];
    if (valid > 3) v.w = p[3];
    return v;
}

template <typename T>
__device__ __forceinline__ void store4(T* __restrict__ p, float4 v, bool vec, bool full, int valid) {
    if constexpr (sizeof(T) == 4) {
        if (vec && full) { *reinterpret_cast<float4*>(p) = v; return; }
    } else {
        if (vec && full) {
            const uint32_t lo = (uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16);
            *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
            return;
        }
    }
    if (valid > 0) store_f32(p, v.x);
    if (valid > 1) store_f32(p + 1, v.y);
    if (valid > 2) store_f32(p + 2, v.z);
    if (valid > 3) store_f32(p + 3, v.w);
}

template <class G, typename OutT, bool TWO = false>
__device__ __forceinline__ void general_epilogue(const PipeArgs& p, const f32x16_t (&acc)[G::MI][G::NJ],
                                                 const f32x16_t (&acc2)[G::MI][G::NJ], float* tile, int m0, int n0,
                                                 int wm, int wn, int z, int tid) {
    constexpr int BM = G::BM, BN = G::BN, MI = G::MI, NJ = G::NJ, WTM = G::WTM, WTN = G::WTN;
    constexpr int kThreads = G::kThreads;
    using E = EpiTile<BM, BN>;
    float* tile2 = tile + BM * E::kLd;   // second accumulator (mode 2)
    const int lane = tid & 63;
    block_barrier();   // every wave is done reading the operand stages
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * WTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                const int col = wn * WTN + j * 32 + (lane & 31);
                tile[row * E::kLd + col] = acc[i][j][r];
                if constexpr (TWO) tile2[row * E::kLd + col] = acc2[i][j][r];
            }
    __syncthreads();
    const float* __restrict__ cin1 = p.Cin1 ? p.Cin1 + (int64_t)z * p.strideCin1 : nullptr;
    const float* __restrict__ cin2 = p.Cin2 ? p.Cin2 + (int64_t)z * p.strideCin2 : nullptr;
    OutT* __restrict__ c1 = p.C ? reinterpret_cast<OutT*>(p.C) + (int64_t)z * p.strideC : nullptr;
    bf16_t* __restrict__ c2 = p.C2 ? reinterpret_cast<bf16_t*>(p.C2) + (int64_t)z * p.strideC2 : nullptr;
    bf16_t* __restrict__ c3 = p.C3 ? reinterpret_cast<bf16_t*>(p.C3) + (int64_t)z * p.strideC2 : nullptr;
    const bool vec = p.epi_vec != 0;
    constexpr int kChunks = BM * BN / 4;
#pragma unroll
    for (int u0 = 0; u0 < kChunks; u0 += kThreads) {
        const int u = u0 + tid;
        const int row = u / (BN / 4);
        const int c = (u % (BN / 4)) * 4;
        const int gr = m0 + row, gc = n0 + c;
        if (gr >= p.M || gc >= p.N) continue;
        const int valid = min(4, p.N - gc);
        const bool full = valid == 4;
        float4 v = *reinterpret_cast<const float4*>(tile + row * E::kLd + c);
        v.x *= p.alpha; v.y *= p.alpha; v.z *= p.alpha; v.w *= p.alpha;
        const float4 a1 = cin1 ? load4(cin1 + (int64_t)gr * p.ldcin1 + gc, vec, full, valid) : make_float4(0.f, 0.f, 0.f, 0.f);
        if constexpr (TWO) {   // mode 2: C = v + beta1 Cin1, C2 = v + w + beta2 Cin1
            float4 w = *reinterpret_cast<const float4*>(tile2 + row * E::kLd + c);
            w.x *= p.alpha; w.y *= p.alpha; w.z *= p.alpha; w.w *= p.alpha;
            store4(c1 + (int64_t)gr * p.ldc + gc,
                   make_float4(v.x + p.beta1 * a1.x, v.y + p.beta1 * a1.y, v.z + p.beta1 * a1.z, v.w + p.beta1 * a1.w),
                   vec, full, valid);
            store4(c2 + (int64_t)gr * p.ldc2 + gc,
                   make_float4(v.x + w.x + p.beta2 * a1.x, v.y + w.y + p.beta2 * a1.y, v.z + w.z + p.beta2 * a1.z,
                               v.w + w.w + p.beta2 * a1.w),
                   vec, full, valid);
            continue;
        }
        if (p.mode == 1) {
            const float4 q2 = make_float4(2.f * a1.x, 2.f * a1.y, 2.f * a1.z, 2.f * a1.w);
            store4(c1 + (int64_t)gr * p.ldc + gc,
                   make_float4(q2.x + 2.f * v.x, q2.y + 2.f * v.y, q2.z + 2.f * v.z, q2.w + 2.f * v.w), vec, full, valid);
            store4(c2 + (int64_t)gr * p.ldc2 + gc, v, vec, full, valid);
            store4(c3 + (int64_t)gr * p.ldc2 + gc, make_float4(q2.x + v.x, q2.y + v.y, q2.z + v.z, q2.w + v.w), vec,
                   full, valid);
            continue;
        }
        const float4 a2 = cin2 ? load4(cin2 + (int64_t)gr * p.ldcin2 + gc, vec, full, valid) : make_float4(0.f, 0.f, 0.f, 0.f);
        float4 o = make_float4(v.x + p.beta1 * a1.x + p.beta2 * a2.x, v.y + p.beta1 * a1.y + p.beta2 * a2.y,
                               v.z + p.beta1 * a1.z + p.beta2 * a2.z, v.w + p.beta1 * a1.w + p.beta2 * a2.w);
        if (p.gamma != 0.f) {
            if (gr == gc) o.x += p.gamma;
            if (gr == gc + 1) o.y += p.gamma;
            if (gr == gc + 2) o.z += p.gamma;
            if (gr == gc + 3) o.w += p.gamma;
        }
        if (c1) store4(c1 + (int64_t)gr * p.ldc + gc, o, vec, full, valid);
        if (c2) store4(c2 + (int64_t)gr * p.ldc2 + gc, o, vec, full, valid);
    }
}

// Wait until at most `tiles` k-tiles of this thread's loads are still in flight
// (tiles is wave-uniform and at most S - 2).
template <int LPT, int S>
__device__ __forceinline__ void wait_tiles(int tiles) {
    static_assert(S >= 2 && S <= 8 && LPT * (S - 2) < 64, "vmcnt range");
    switch (tiles) {
        case 0: wait_vmcnt<0>(); break;
        case 1: if constexpr (S > 2) wait_vmcnt<LPT>(); break;
        case 2: if constexpr (S > 3) wait_vmcnt<2 * LPT>(); break;
        case 3: if constexpr (S > 4) wait_vmcnt<3 * LPT>(); break;
        case 4: if constexpr (S > 5) wait_vmcnt<4 * LPT>(); break;
        case 5: if constexpr (S > 6) wait_vmcnt<5 * LPT>(); break;
        default: if constexpr (S > 7) wait_vmcnt<6 * LPT>(); break;
    }
}

// S-stage LDS ring: S - 1 k-tiles are requested before the first one is used,
// so a product with K <= 64 (S - 1) waits for memory once.
// Epilogue kinds: plain store, general (see PipeArgs).
constexpr int kEpiPlain = 0, kEpiGeneral = 1;

// The k loop of one output tile at (m0, n0) into acc (zeroed here).
template <class G, bool A_MN, bool B_MN, int S>
__device__ __forceinline__ void main_loop(unsigned char* lds, const uint16_t* __restrict__ A, int64_t lda,
                                          const uint16_t* __restrict__ B, int64_t ldb, int m0, int n0, int M, int N,
                                          int kb, int ke, int tid, f32x16_t (&acc)[G::MI][G::NJ],
                                          bool zero = true) {
    constexpr int BM = G::BM, BN = G::BN;
    constexpr int kABytes = G::kABytes, kStageBytes = G::kStageBytes;
    constexpr int kLoadsPerTile = G::kLoadsPerTile;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / G::NWN, wn = wave % G::NWN;
    const int nk = ke > kb ? (ke - kb + BK - 1) / BK : 0;
    const uint32_t base = lds_offset(lds);
    if (zero) {
#pragma unroll
        for (int i = 0; i < G::MI; ++i)
#pragma unroll
            for (int j = 0; j < G::NJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    }

    DmaJob job{base, A, lda, B, ldb, m0, n0, M, N, kb, ke, wave, lane};
#pragma unroll
    for (int t = 0; t < S - 1; ++t) {
        if (t < nk) {
            job.stage = base + t * kStageBytes;
            job.k0 = kb + t * BK;
            dma_tile<G, A_MN, B_MN>(job);
        }
    }
    int st = 0;        // stage of tile kt
    int st_load = S - 1;   // stage that receives tile kt + S - 1
    for (int kt = 0; kt < nk; ++kt) {
        // this thread's loads of tile kt are done when at most those of the
        // tiles after it (up to kt + S - 2) remain
        wait_tiles<kLoadsPerTile, S>(min(nk, kt + S - 1) - kt - 1);
        block_barrier();   // everyone's tile kt has landed; stage st_load (tile kt-1) is no longer read
        if constexpr (A_MN || B_MN) {
            const int valid = ke - (kb + kt * BK);
            if (valid < BK) {   // ragged last tile: rows past K were loaded from clamped rows
                if constexpr (A_MN) zero_rows_mn<BM, G::kThreads>(lds + st * kStageBytes, valid, tid);
                if constexpr (B_MN) zero_rows_mn<BN, G::kThreads>(lds + st * kStageBytes + kABytes, valid, tid);
                __syncthreads();
            }
        }
        job.stage = base + st_load * kStageBytes;
        job.k0 = kb + (kt + S - 1) * BK;
        compute_tile<G, A_MN, B_MN>(lds + st * kStageBytes, wm, wn, lane, acc, job, kt + S - 1 < nk);
        st = st == S - 1 ? 0 : st + 1;
        st_load = st_load == S - 1 ? 0 : st_load + 1;
    }
}

// DUAL = 1: acc = op(A) op(B) + A2^T B2 (second product with m/n-major A2, B2);
// DUAL = 2: the second product goes to its own accumulator (general epilogue mode 2).
template <int BM, int BN, bool A_MN, bool B_MN, bool OUT_F32, int EPI, int S, int NWM = 2, int NWN = 2, int DUAL = 0>
__global__ void __launch_bounds__(64 * NWM * NWN)
__attribute__((amdgpu_waves_per_eu(PipeWaves<BM, BN, NWM * NWN>::lo, PipeWaves<BM, BN, NWM * NWN>::hi)))
pipe_gemm_kernel(const PipeArgs p) {
    using G = Geo<BM, BN, NWM, NWN>;
    constexpr int kStageBytes = G::kStageBytes;
    constexpr int MI = G::MI, NJ = G::NJ, WTM = G::WTM, WTN = G::WTN;
    static_assert(S * kStageBytes <= 160 * 1024, "LDS ring exceeds 160 KB");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[S * kStageBytes];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / NWN, wn = wave % NWN;
    const int M = p.M, N = p.N;
    const int kb = blockIdx.z * p.k_per_split;
    const int ke = min(p.K, kb + p.k_per_split);
    int tm, tn;
    int z;
    batch_tile_coords((M + BM - 1) / BM, (N + BN - 1) / BN, z, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const uint16_t* A = reinterpret_cast<const uint16_t*>(p.A) + (int64_t)z * p.strideA;
    const uint16_t* B = reinterpret_cast<const uint16_t*>(p.B) + (int64_t)z * p.strideB;
    f32x16_t acc[MI][NJ], acc2[MI][NJ];
    main_loop<G, A_MN, B_MN, S>(lds, A, p.lda, B, p.ldb, m0, n0, M, N, kb, ke, tid, acc);
    if constexpr (DUAL != 0) {
        const uint16_t* A2 = reinterpret_cast<const uint16_t*>(p.A2) + (int64_t)z * p.strideA2;
        const uint16_t* B2 = reinterpret_cast<const uint16_t*>(p.B2) + (int64_t)z * p.strideB2;
        block_barrier();   // the second product reuses the LDS ring
        if constexpr (DUAL == 1)
            main_loop<G, true, true, S>(lds, A2, p.lda2, B2, p.ldb2, m0, n0, M, N, kb, ke, tid, acc, false);
        else
            main_loop<G, true, true, S>(lds, A2, p.lda2, B2, p.ldb2, m0, n0, M, N, kb, ke, tid, acc2, true);
    }

    // epilogue: lane holds rows 8 (r/4) + 4 (lane/32) + r%4 of column lane%32 per tile
    using OutT = typename std::conditional<OUT_F32, float, bf16_t>::type;
    const int col0 = n0 + wn * WTN + (lane & 31);
    const int row0 = m0 + wm * WTM + (lane >> 5) * 4;
    if constexpr (EPI == kEpiGeneral) {
        static_assert((DUAL == 2 ? 2 : 1) * EpiTile<BM, BN>::kBytes <= S * kStageBytes,
                      "epilogue tile exceeds the LDS ring");
        general_epilogue<G, OutT, DUAL == 2>(p, acc, acc2, reinterpret_cast<float*>(lds), m0, n0, wm, wn, z, tid);
        return;
    }
    OutT* C = reinterpret_cast<OutT*>(p.C) + (int64_t)z * p.strideC + (int64_t)blockIdx.z * p.strideSplit;
    if (m0 + BM <= M && n0 + BN <= N) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    store_f32(C + (int64_t)(row0 + i * 32 + (r >> 2) * 8 + (r & 3)) * p.ldc + col0 + j * 32,
                              acc[i][j][r]);
    } else {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int col = col0 + j * 32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = row0 + i * 32 + (r >> 2) * 8 + (r & 3);
                    if (row < M && col < N) store_f32(C + (int64_t)row * p.ldc + col, acc[i][j][r]);
                }
            }
    }
}

template <int BM, int BN, bool A_MN, bool B_MN, bool OUT_F32, int EPI = kEpiPlain, int S = 3, int NWM = 2, int NWN = 2,
          int DUAL = 0>
hipError_t launch(const PipeArgs& p, hipStream_t stream) {
    const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    constexpr int kMaxY = 65535;
    for (int y0 = 0; y0 < p.batch; y0 += kMaxY) {
        PipeArgs q = p;
        q.batch = min(kMaxY, p.batch - y0);
        q.A = reinterpret_cast<const uint16_t*>(p.A) + (int64_t)y0 * p.strideA;
        q.B = reinterpret_cast<const uint16_t*>(p.B) + (int64_t)y0 * p.strideB;
        if (p.C) q.C = reinterpret_cast<char*>(p.C) + (int64_t)y0 * p.strideC * (OUT_F32 ? 4 : 2);
        if (p.C2) q.C2 = reinterpret_cast<bf16_t*>(p.C2) + (int64_t)y0 * p.strideC2;
        if (p.C3) q.C3 = reinterpret_cast<bf16_t*>(p.C3) + (int64_t)y0 * p.strideC2;
        if (p.Cin1) q.Cin1 = p.Cin1 + (int64_t)y0 * p.strideCin1;
        if (p.Cin2) q.Cin2 = p.Cin2 + (int64_t)y0 * p.strideCin2;
        if (p.A2) q.A2 = reinterpret_cast<const uint16_t*>(p.A2) + (int64_t)y0 * p.strideA2;
        if (p.B2) q.B2 = reinterpret_cast<const uint16_t*>(p.B2) + (int64_t)y0 * p.strideB2;
        hipLaunchKernelGGL((pipe_gemm_kernel<BM, BN, A_MN, B_MN, OUT_F32, EPI, S, NWM, NWN, DUAL>),
                           dim3(tiles, q.batch, p.splits), dim3(64 * NWM * NWN), 0, stream, q);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// A zero the compiler cannot see through: offsets built on it are recomputed
// where they are used instead of being hoisted and kept live in registers.
__device__ __forceinline__ int opaque_zero() {
    int z;
    asm volatile("s_mov_b32 %0, 0" : "=s"(z));
    return z;
}

// ------------------------------------------------ fused Cayley-Neumann forward
// One workgroup per (block, 64-row panel p) for bf16 blocks of b = 128 or 256:
// the block's whole bf16 Q sits in LDS as the B operand ([b/64] k-tiles of
// [b rows][64 k], swizzled as above) and the panel X (64 x b) as the A
// operand.  Horner on the panel rows,
//   X_1 = Q_p,  X_{i+1} = X_i Q = -(X_i Q^T)  (i = 1..k),
//   G_p = I_p + 2 (X_1 + ... + X_k) + X_{k+1}  =  rows p of (I + Q) sum_{i<=k} Q^i,
// keeps the sum in float32 registers and rounds each X_{i+1} to bf16 into LDS
// for the next product; every power of Q is formed once per panel and nothing
// but Q and G crosses HBM.  With S / T given (k >= 2) the kernel also writes
// S_p = X_2 and T_p = 2 Q_p + S_p (what the saving forward keeps for k = 3).
template <int B>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
cnp_fused_kernel(const uint16_t* __restrict__ Qc, uint16_t* __restrict__ G, uint16_t* __restrict__ Sv,
                 uint16_t* __restrict__ Tv, int k, int total) {
    constexpr int KT = B / 64;          // k-tiles of one product
    constexpr int NP = B / 64;          // panels per block
    constexpr int QB = B * 128;         // bytes of one Q k-tile
    constexpr int XB = 64 * 128;        // bytes of one X k-tile
    constexpr int MI = 2, NJ = B / 128; // each wave: 64 rows x B/4 columns
    static_assert(KT * (QB + XB) <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[KT * (QB + XB)];
    unsigned char* qs = lds;
    unsigned char* xs = lds + KT * QB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int id = blockIdx.x;
    if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);   // each XCD gets whole blocks
    const int z = id / NP, p = id - z * NP;
    const int64_t zoff = (int64_t)z * B * B;
    const uint16_t* Qz = Qc + zoff;

    const uint32_t qb = lds_offset(qs), xb = lds_offset(xs);
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int j = 0; j < OperandLoads<B, false, 4>::n; ++j)
            dma_one<B, false, 4>(j, qb + kt * QB, Qz, B, 0, B, kt * 64, B, wave, lane);
#pragma unroll
        for (int j = 0; j < OperandLoads<64, false, 4>::n; ++j)
            dma_one<64, false, 4>(j, xb + kt * XB, Qz, B, 64 * p, B, kt * 64, B, wave, lane);
    }
    wait_vmcnt<0>();
    block_barrier();

    f32x16_t sum[MI][NJ], acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) sum[i][j][r] = 0.f;
    const int n_base = wave * (B / 4);
    for (int it = 1; it <= k; ++it) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
#pragma unroll 1
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                uint4 af[MI], bfr[NJ];
#pragma unroll
                for (int i = 0; i < MI; ++i) af[i] = load_frag<false, 64>(xs + kt * XB, i * 32, ks, lane);
#pragma unroll
                for (int j = 0; j < NJ; ++j) bfr[j] = load_frag<false, B>(qs + kt * QB, n_base + j * 32, ks, lane);
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int j = 0; j < NJ; ++j) Mfma32<bf16_t>::run(af[i], bfr[j], acc[i][j]);
            }
        }
        // X_{it+1} = -acc; weight 2 for it + 1 <= k, 1 for the last power
        const float w = it < k ? -2.f : -1.f;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) sum[i][j][r] += w * acc[i][j][r];
        if (it == 1 && Sv) {   // S_p = X_2, T_p = 2 Q_p + S_p
            const int oz = opaque_zero();
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3) + oz;
                        const int n = n_base + j * 32 + (lane & 31);
                        const int row = 64 * p + m;
                        const uint16_t qv = *reinterpret_cast<const uint16_t*>(
                            qs + (n >> 6) * QB + row * 128 + ((((n & 63) >> 3) ^ swz_k(row)) << 4) + (n & 7) * 2);
                        const float sv = -acc[i][j][r];
                        Sv[zoff + (int64_t)row * B + n] = f32_to_bf16(sv);
                        Tv[zoff + (int64_t)row * B + n] = f32_to_bf16(2.f * bf16_to_f32(qv) + sv);
                    }
        }
        if (it < k) {
            block_barrier();   // every wave is done reading X_it
            const int oz = opaque_zero();
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3) + oz;
                        const int n = n_base + j * 32 + (lane & 31);
                        *reinterpret_cast<uint16_t*>(xs + (n >> 6) * XB + m * 128 +
                                                     ((((n & 63) >> 3) ^ swz_k(m)) << 4) + (n & 7) * 2) =
                            f32_to_bf16(-acc[i][j][r]);
                    }
            __syncthreads();
        }
    }
    // G_p = I_p + 2 Q_p + sum
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                const int n = n_base + j * 32 + (lane & 31);
                const int row = 64 * p + m;
                const uint16_t qv = *reinterpret_cast<const uint16_t*>(
                    qs + (n >> 6) * QB + row * 128 + ((((n & 63) >> 3) ^ swz_k(row)) << 4) + (n & 7) * 2);
                const float g = (row == n ? 1.f : 0.f) + 2.f * bf16_to_f32(qv) + sum[i][j][r];
                G[zoff + (int64_t)row * B + n] = f32_to_bf16(g);
            }
}

}  // namespace

bool pipe_gemm_supported(bool a_mn, bool b_mn, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                         int64_t strideA, int64_t strideB) {
    if (M <= 0 || N <= 0 || K <= 0) return false;
    if (a_mn && !b_mn) return false;
    if (lda % 8 || ldb % 8 || strideA % 8 || strideB % 8) return false;
    if (!a_mn && K % BK) return false;
    if (!b_mn && K % BK) return false;
    if (a_mn && (M % 8 || M < 8)) return false;
    if (b_mn && (N % 8 || N < 8)) return false;
    return true;
}

hipError_t pipe_gemm(bool a_mn, bool b_mn, bool out_f32, const PipeArgs& p, hipStream_t stream, PipeTile tile) {
    if (p.M <= 0 || p.N <= 0 || p.batch <= 0 || p.splits <= 0) return hipSuccess;
    // instantiated combinations: dense / block products (k-major A, bf16 out) and
    // block gradients (m/n-major A and B, float32 out)
    if (!a_mn && !out_f32) {
        if (tile == PipeTile::Big)
            return b_mn ? launch<256, 256, false, true, false, kEpiPlain, 2, 2, 4>(p, stream)
                        : launch<256, 256, false, false, false, kEpiPlain, 2, 2, 4>(p, stream);
        if (tile == PipeTile::Wide)
            return b_mn ? launch<128, 256, false, true, false, kEpiPlain, 3, 2, 4>(p, stream)
                        : launch<128, 256, false, false, false, kEpiPlain, 3, 2, 4>(p, stream);
        return b_mn ? launch<256, 128, false, true, false, kEpiPlain, 3, 4, 2>(p, stream)
                    : launch<256, 128, false, false, false, kEpiPlain, 3, 4, 2>(p, stream);
    }
    if (a_mn && b_mn && out_f32) {
        if (tile == PipeTile::Square) return launch<128, 128, true, true, true, kEpiPlain, 4>(p, stream);
        if (tile == PipeTile::Small) return launch<64, 64, true, true, true, kEpiPlain, 4>(p, stream);
        return launch<256, 128, true, true, true, kEpiPlain, 3, 4, 2>(p, stream);
    }
    return hipErrorInvalidValue;
}

template <int T, bool OUT_F32>
hipError_t launch_general(bool a_mn, bool b_mn, const PipeArgs& p, hipStream_t stream) {
    if (!a_mn && !b_mn) return launch<T, T, false, false, OUT_F32, kEpiGeneral, 4>(p, stream);
    if (!a_mn && b_mn) return launch<T, T, false, true, OUT_F32, kEpiGeneral, 4>(p, stream);
    return launch<T, T, true, true, OUT_F32, kEpiGeneral, 4>(p, stream);
}

hipError_t pipe_gemm_general(bool a_mn, bool b_mn, bool out_f32, const PipeArgs& p_in, hipStream_t stream) {
    if (p_in.M <= 0 || p_in.N <= 0 || p_in.batch <= 0) return hipSuccess;
    PipeArgs p = p_in;
    // 16-byte float32 / 8-byte bf16 epilogue accesses need every row start and
    // every batch stride of every epilogue operand aligned to 4 elements
    auto al = [](const void* ptr, int64_t ld, int64_t stride) {
        return ptr == nullptr || (((uintptr_t)ptr % 16) == 0 && ld % 4 == 0 && stride % 4 == 0);
    };
    p.epi_vec = al(p.C, p.ldc, p.strideC) && al(p.C2, p.ldc2, p.strideC2) && al(p.C3, p.ldc2, p.strideC2) &&
                al(p.Cin1, p.ldcin1, p.strideCin1) && al(p.Cin2, p.ldcin2, p.strideCin2);
    if (a_mn && !b_mn) return hipErrorInvalidValue;
    if (p.splits != 1) return hipErrorInvalidValue;
    // 128 x 128 tiles only when they alone give about four workgroups per CU
    const int64_t big = (int64_t)((p.M + 127) / 128) * ((p.N + 127) / 128) * p.batch;
    if (big >= 1024) {
        return out_f32 ? launch_general<128, true>(a_mn, b_mn, p, stream)
                       : launch_general<128, false>(a_mn, b_mn, p, stream);
    }
    return out_f32 ? launch_general<64, true>(a_mn, b_mn, p, stream) : launch_general<64, false>(a_mn, b_mn, p, stream);
}

hipError_t pipe_gemm_dual(bool separate, bool out_f32, const PipeArgs& p_in, hipStream_t stream) {
    if (p_in.M <= 0 || p_in.N <= 0 || p_in.batch <= 0) return hipSuccess;
    if (p_in.splits != 1 || !p_in.A2 || !p_in.B2) return hipErrorInvalidValue;
    PipeArgs p = p_in;
    auto al = [](const void* ptr, int64_t ld, int64_t stride) {
        return ptr == nullptr || (((uintptr_t)ptr % 16) == 0 && ld % 4 == 0 && stride % 4 == 0);
    };
    p.epi_vec = al(p.C, p.ldc, p.strideC) && al(p.C2, p.ldc2, p.strideC2) && al(p.Cin1, p.ldcin1, p.strideCin1) &&
                al(p.Cin2, p.ldcin2, p.strideCin2);
    if (separate) {
        return out_f32 ? launch<64, 64, false, false, true, kEpiGeneral, 4, 2, 2, 2>(p, stream)
                       : launch<64, 64, false, false, false, kEpiGeneral, 4, 2, 2, 2>(p, stream);
    }
    return out_f32 ? launch<64, 64, false, false, true, kEpiGeneral, 4, 2, 2, 1>(p, stream)
                   : launch<64, 64, false, false, false, kEpiGeneral, 4, 2, 2, 1>(p, stream);
}

int pipe_tile_rows(PipeTile t) {
    return (t == PipeTile::Tall || t == PipeTile::Big) ? 256 : t == PipeTile::Small ? 64 : 128;
}
int pipe_tile_cols(PipeTile t) {
    return (t == PipeTile::Wide || t == PipeTile::Big) ? 256 : t == PipeTile::Small ? 64 : 128;
}

bool dense_gemm_supported(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb) {
    return M > 0 && N >= 8 && K >= BK && K % BK == 0 && N % 8 == 0 && lda % 8 == 0 && ldb % 8 == 0;
}

hipError_t dense_gemm_bf16(bool b_nn, const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                           int M, int N, int K, hipStream_t stream) {
    PipeArgs p;
    p.A = A; p.lda = lda;
    p.B = B; p.ldb = ldb;
    p.C = C; p.ldc = ldc;
    p.M = M; p.N = N; p.K = K;
    p.k_per_split = K;
    // 256 x 256 tiles (two-stage ring, two waves per SIMD) once they alone fill the chip
    const int64_t big_tiles = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
    return pipe_gemm(false, b_nn, false, p, stream, big_tiles >= 256 ? PipeTile::Big : PipeTile::Tall);
}

bool cnp_fused_supported(int64_t b, int k) { return (b == 128 || b == 256) && k >= 1; }

hipError_t cnp_fused_fwd(const void* Qc, void* G, void* S, void* T, int64_t nblk, int64_t b, int k,
                         hipStream_t stream) {
    if (nblk <= 0) return hipSuccess;
    if (!cnp_fused_supported(b, k) || ((S == nullptr) != (T == nullptr)) || (S && k < 2)) return hipErrorInvalidValue;
    const int64_t panels = nblk * (b / 64);
    if (panels > 0x7fffffff) return hipErrorInvalidValue;
    const auto q = static_cast<const uint16_t*>(Qc);
    const auto g = static_cast<uint16_t*>(G);
    const auto sv = static_cast<uint16_t*>(S);
    const auto tv = static_cast<uint16_t*>(T);
    if (b == 256)
        hipLaunchKernelGGL(cnp_fused_kernel<256>, dim3((unsigned)panels), dim3(256), 0, stream, q, g, sv, tv, k,
                           (int)panels);
    else
        hipLaunchKernelGGL(cnp_fused_kernel<128>, dim3((unsigned)panels), dim3(256), 0, stream, q, g, sv, tv, k,
                           (int)panels);
    return hipGetLastError();
}

}  // namespace poetx
