// Pipelined bf16 MFMA GEMM (float32 accumulation) for the products of the
// POET-X chain (the input-centric, matrix-free reformulation of the review's
// Summary keeps W0 frozen and never materialises R W0 P):
//   dense   h2  = h1 . Wt^T  (A k-major, B k-major)   dh1 = dh2 . Wt (B n-major)
//   blocks  h1_j = a_j . G_j^T, dh2_j = dz_j . G_j     (batched over blocks j)
//   grads   dG_j = dz_j^T h2_j                          (A and B m/n-major, K = tokens,
//                                                        float32 out)
//   small   the Cayley-Neumann b x b products (batched over blocks, general
//           epilogue with float32 addends and several outputs; paired products)
// plus the fused Cayley-Neumann forward and the split-K block-gradient kernel.
//
// Workgroup tiles BM x BN x 64 with v_mfma_f32_32x32x16_bf16 (float32
// accumulators): dense products take the largest of 256 x 256, 256 x 128,
// 128 x 128 and 64 x 128 whose grid still gives every CU a workgroup (the
// large ones with eight waves of 64 x 64 or 128 x 64); block products 128 x 256
// (64 x 128 for a few blocks); the small products 64 x 64 with four waves.
//
// Operand tiles travel global -> LDS by direct-to-LDS loads
// (global_load_lds_dwordx4: each lane's 16 bytes land at M0 + 16 * lane), so no
// VGPRs stage them and no ds_write is issued.  S LDS stages form a ring (S = 3
// for 256 x 128 and 128 x 256, 2 for 256 x 256, 4 for the smaller tiles, 2 or 3
// for the b x b products, whose epilogues need more workgroups per CU):
// while the MFMAs consume stage kt % S, the loads of tiles kt+1 .. kt+S-1 are
// in flight, so a short product (K = 256) waits for memory once.  The loads
// are issued from inline asm so that the compiler does not add a conservative
// vmcnt(0) before every LDS read; the kernel itself waits (s_waitcnt vmcnt)
// for exactly the tile it is about to read, then barriers.
//
// LDS layouts (XOR-swizzled instead of padded, because a DMA writes whole
// 1 KB runs):
//   k-major tile [rows][64 k], 128-byte rows of eight 16-byte chunks: chunk c
//     of row r sits in slot c ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1), which
//     keeps the ds_read_b128 fragment reads free of bank conflicts;
//   m/n-major tile [64 k][rows], 256- or 512-byte rows: chunk c of k-row k sits
//     in slot c ^ 4 (k & 3) (128-byte rows: c ^ 4 ((k >> 1) & 1)); fragments
//     are read with ds_read_b64_tr_b16, which
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

// Fragments of k-step ks for one wave (MI A fragments, NJ B fragments).
template <class G, bool A_MN, bool B_MN>
__device__ __forceinline__ void load_frags(const unsigned char* __restrict__ st, int wm, int wn, int ks, int lane,
                                           uint4 (&af)[G::MI], uint4 (&bfr)[G::NJ]) {
#pragma unroll
    for (int i = 0; i < G::MI; ++i) af[i] = load_frag<A_MN, G::BM>(st, wm * G::WTM + i * 32, ks, lane);
#pragma unroll
    for (int j = 0; j < G::NJ; ++j) bfr[j] = load_frag<B_MN, G::BN>(st + G::kABytes, wn * G::WTN + j * 32, ks, lane);
}

// One k-tile (four k-steps of 16) with register double-buffered fragments:
// the LDS reads of step ks+1 are issued before the MFMAs of step ks, and
// scheduling barriers keep the compiler from sinking them; a quarter of the
// next tile's loads goes out with each k-step.
template <class G, bool A_MN, bool B_MN>
__device__ __forceinline__ void compute_tile(const unsigned char* __restrict__ st, int wm, int wn, int lane,
                                             f32x16_t (&acc)[G::MI][G::NJ], const DmaJob& next, bool load_next) {
    uint4 af[2][G::MI], bfr[2][G::NJ];
    load_frags<G, A_MN, B_MN>(st, wm, wn, 0, lane, af[0], bfr[0]);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
        const int cur = ks & 1;
        if (ks + 1 < BK / 16) load_frags<G, A_MN, B_MN>(st, wm, wn, ks + 1, lane, af[cur ^ 1], bfr[cur ^ 1]);
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

// The float32 addends Cin1 / Cin2 of the chunks a thread writes in the general
// epilogue, loaded before the main loop so that their latency hides behind it
// (tiles with at most four chunks per thread; the b x b products are bound by
// this traffic).  Rows or columns outside the product read as zero.
template <int BM, int BN, int kThreads>
struct EpiAddends {
    static constexpr int kChunks = BM * BN / 4;
    static constexpr int kPer = kChunks / kThreads;
    static constexpr bool kOn = kChunks % kThreads == 0 && kPer <= 4;
    float4 a1[kOn ? kPer : 1], a2[kOn ? kPer : 1];
};

template <int BM, int BN, int kThreads>
__device__ __forceinline__ void load_addends(const PipeArgs& p, int m0, int n0, int z, int tid,
                                             EpiAddends<BM, BN, kThreads>& e) {
    using E = EpiAddends<BM, BN, kThreads>;
    const float* __restrict__ cin1 = p.Cin1 ? p.Cin1 + (int64_t)z * p.strideCin1 : nullptr;
    const float* __restrict__ cin2 = p.Cin2 ? p.Cin2 + (int64_t)z * p.strideCin2 : nullptr;
    const bool vec = p.epi_vec != 0;
#pragma unroll
    for (int k = 0; k < E::kPer; ++k) {
        const int u = k * kThreads + tid;
        const int row = u / (BN / 4);
        const int c = (u % (BN / 4)) * 4;
        const int gr = m0 + row, gc = n0 + c;
        const bool in = gr < p.M && gc < p.N;
        const int valid = in ? min(4, p.N - gc) : 0;
        const bool full = valid == 4;
        e.a1[k] = cin1 && in ? load4(cin1 + (int64_t)gr * p.ldcin1 + gc, vec, full, valid) : make_float4(0.f, 0.f, 0.f, 0.f);
        e.a2[k] = cin2 && in ? load4(cin2 + (int64_t)gr * p.ldcin2 + gc, vec, full, valid) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

template <class G, typename OutT, bool TWO = false>
__device__ __forceinline__ void general_epilogue(const PipeArgs& p, const f32x16_t (&acc)[G::MI][G::NJ],
                                                 const f32x16_t (&acc2)[G::MI][G::NJ], float* tile, int m0, int n0,
                                                 int wm, int wn, int z, int tid,
                                                 const EpiAddends<G::BM, G::BN, G::kThreads>& pre) {
    using Pre = EpiAddends<G::BM, G::BN, G::kThreads>;
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
        float4 a1, a2;
        if constexpr (Pre::kOn) {
            a1 = pre.a1[u0 / kThreads];
            a2 = pre.a2[u0 / kThreads];
        } else {
            a1 = cin1 ? load4(cin1 + (int64_t)gr * p.ldcin1 + gc, vec, full, valid) : make_float4(0.f, 0.f, 0.f, 0.f);
            a2 = cin2 ? load4(cin2 + (int64_t)gr * p.ldcin2 + gc, vec, full, valid) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
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
        if (p.mode == 3) {   // k = 4 square: C = v, C2 = v, C3 = Cin1 + v
            store4(c1 + (int64_t)gr * p.ldc + gc, v, vec, full, valid);
            store4(c2 + (int64_t)gr * p.ldc2 + gc, v, vec, full, valid);
            store4(c3 + (int64_t)gr * p.ldc2 + gc, make_float4(a1.x + v.x, a1.y + v.y, a1.z + v.z, a1.w + v.w), vec,
                   full, valid);
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

    if (nk == 0) return;

    DmaJob job{base, A, lda, B, ldb, m0, n0, M, N, kb, ke, wave, lane};
#pragma unroll
    for (int t = 0; t < S - 1; ++t) {
        if (t < nk) {
            job.stage = base + t * kStageBytes;
            job.k0 = kb + t * BK;
            dma_tile<G, A_MN, B_MN>(job);
        }
    }
    // Tile kt becomes readable once this thread's loads of it are done (at most
    // those of the tiles after it, up to kt + S - 2, remain) and every wave has
    // passed the barrier; a ragged last m/n-major tile then gets its rows past K
    // zeroed (they were loaded from clamped rows).
    auto enter = [&](int kt, int stage) {
        wait_tiles<kLoadsPerTile, S>(min(nk, kt + S - 1) - kt - 1);
        block_barrier();
        if constexpr (A_MN || B_MN) {
            const int valid = ke - (kb + kt * BK);
            if (valid < BK) {
                if constexpr (A_MN) zero_rows_mn<BM, G::kThreads>(lds + stage * kStageBytes, valid, tid);
                if constexpr (B_MN) zero_rows_mn<BN, G::kThreads>(lds + stage * kStageBytes + kABytes, valid, tid);
                __syncthreads();
            }
        }
    };
    int st = 0;            // stage of tile kt
    int st_load = S - 1;   // stage that receives tile kt + S - 1
    // 256 x 128 tiles (three stages: tile kt + 1 was requested a whole tile
    // ago) hand over to tile kt + 1 (wait, barrier, its first fragments) before
    // the last k-step's MFMAs of tile kt, which then cover the barrier and the
    // first LDS reads of the next tile; the same barrier frees tile kt's stage,
    // as every wave holds tile kt's last fragments in registers by then.  Other
    // tiles hand over at the top of each tile.
    if constexpr (!(S >= 3 && BM == 256 && BN == 128)) {
        for (int kt = 0; kt < nk; ++kt) {
            enter(kt, st);
            job.stage = base + st_load * kStageBytes;
            job.k0 = kb + (kt + S - 1) * BK;
            compute_tile<G, A_MN, B_MN>(lds + st * kStageBytes, wm, wn, lane, acc, job, kt + S - 1 < nk);
            st = st == S - 1 ? 0 : st + 1;
            st_load = st_load == S - 1 ? 0 : st_load + 1;
        }
        return;
    }
    uint4 af[2][G::MI], bfr[2][G::NJ];
    enter(0, 0);
    load_frags<G, A_MN, B_MN>(lds, wm, wn, 0, lane, af[0], bfr[0]);
    for (int kt = 0; kt < nk; ++kt) {
        job.stage = base + st_load * kStageBytes;
        job.k0 = kb + (kt + S - 1) * BK;
        const bool load_next = kt + S - 1 < nk;
        const unsigned char* cur_st = lds + st * kStageBytes;
        const int st_next = st == S - 1 ? 0 : st + 1;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int cur = ks & 1;
            if (ks + 1 < BK / 16) load_frags<G, A_MN, B_MN>(cur_st, wm, wn, ks + 1, lane, af[cur ^ 1], bfr[cur ^ 1]);
            if (load_next) {
                switch (ks) {
                    case 0: dma_part<G, A_MN, B_MN, 0, 4>(job); break;
                    case 1: dma_part<G, A_MN, B_MN, 1, 4>(job); break;
                    case 2: dma_part<G, A_MN, B_MN, 2, 4>(job); break;
                    default: dma_part<G, A_MN, B_MN, 3, 4>(job); break;
                }
            }
            if (ks == BK / 16 - 1 && kt + 1 < nk) {
                enter(kt + 1, st_next);
                load_frags<G, A_MN, B_MN>(lds + st_next * kStageBytes, wm, wn, 0, lane, af[cur ^ 1], bfr[cur ^ 1]);
            }
            // The MFMAs run at raised wave priority, so the arbiter favours the
            // waves that keep the matrix cores busy over those issuing loads.
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int i = 0; i < G::MI; ++i)
#pragma unroll
                for (int j = 0; j < G::NJ; ++j) Mfma32<bf16_t>::run(af[cur][i], bfr[cur][j], acc[i][j]);
            __builtin_amdgcn_s_setprio(0);
            __builtin_amdgcn_sched_barrier(0);
        }
        st = st_next;
        st_load = st_load == S - 1 ? 0 : st_load + 1;
    }
}

// DUAL = 1: acc = op(A) op(B) + A2^T B2 (second product with m/n-major A2, B2);
// DUAL = 2: the second product goes to its own accumulator (general epilogue mode 2).
// GRP: a grouped product (PipeArgs::grp), a separate instantiation so that the
// plain kernels carry no group lookup.
template <int BM, int BN, bool A_MN, bool B_MN, bool OUT_F32, int EPI, int S, int NWM = 2, int NWN = 2, int DUAL = 0,
          bool GRP = false>
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
    int ke = min(p.K, kb + p.k_per_split);
    int tm, tn;
    int z;
    batch_tile_coords((M + BM - 1) / BM, (N + BN - 1) / BN, z, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const uint16_t* A = reinterpret_cast<const uint16_t*>(p.A) + (int64_t)z * p.strideA;
    const uint16_t* B = reinterpret_cast<const uint16_t*>(p.B) + (int64_t)z * p.strideB;
    if constexpr (GRP) {
        {
            // grouped product: the group whose column range holds n0 (ranges
            // start at multiples of BN, so a tile never spans two groups)
            int64_t a_off = p.grp[0].a_off, b_off = p.grp[0].b_off;
            int gk = p.grp[0].k;
#pragma unroll
            for (int i = 1; i < kMaxPipeGroups; ++i)
                if (i < p.ngroups && n0 >= p.grp[i].n_begin) {
                    a_off = p.grp[i].a_off;
                    b_off = p.grp[i].b_off;
                    gk = p.grp[i].k;
                }
            A += a_off;
            B += b_off;
            ke = min(gk, kb + p.k_per_split);
        }
    }
    f32x16_t acc[MI][NJ], acc2[MI][NJ];
    EpiAddends<BM, BN, G::kThreads> pre;
    if constexpr (EPI == kEpiGeneral && EpiAddends<BM, BN, G::kThreads>::kOn) load_addends(p, m0, n0, z, tid, pre);
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
        general_epilogue<G, OutT, DUAL == 2>(p, acc, acc2, reinterpret_cast<float*>(lds), m0, n0, wm, wn, z, tid,
                                             pre);
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

// The last product pair of the Cayley-Neumann backward with the skew pack
// folded in: dQ = A B^T + A2^T B2 + beta1 Cin1 + beta2 Cin2 over b x b blocks,
// and dq[idx(r, c)] = dQ[r][c] - dQ[c][r] (r < c) written straight from the
// workgroup.  A workgroup owns a mirrored pair of 64 x 64 tiles (I, J) and
// (J, I), I <= J, one per group of four waves (a diagonal pair computes its
// tile twice, so that both groups pass the same barriers); the two dQ tiles
// meet in LDS and only the packed upper triangle leaves the chip.  dQ values
// are formed exactly as the general epilogue forms them, so dq matches the
// unfused product + pack bit for bit.
__device__ __forceinline__ int64_t upper_index(int r, int c, int b) {
    return (int64_t)r * b - (int64_t)r * (r + 1) / 2 + (c - r - 1);
}

template <int S>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(1, 4)))
cnp_pack_pair_kernel(const PipeArgs p, float* __restrict__ dq, int b) {
    using G = Geo<64, 64, 2, 2>;
    constexpr int kRing = S * G::kStageBytes;
    constexpr int kLd = 68;                      // floats per staged row
    static_assert(64 * kLd * 4 <= kRing, "staged tile exceeds a group's ring");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * kRing];
    const int tid = threadIdx.x, grp = tid >> 8, gtid = tid & 255;
    const int lane = tid & 63, w4 = (tid >> 6) & 3;
    const int wm = w4 >> 1, wn = w4 & 1;
    const int nt = b / 64;
    int ti = 0, t = blockIdx.x;
    while (t >= nt - ti) {
        t -= nt - ti;
        ++ti;
    }
    const int tj = ti + t;
    const int z = blockIdx.y;
    // group 0: tile (ti, tj); group 1: tile (tj, ti)
    const int m0 = 64 * (grp ? tj : ti), n0 = 64 * (grp ? ti : tj);
    const uint16_t* A = reinterpret_cast<const uint16_t*>(p.A) + (int64_t)z * p.strideA;
    const uint16_t* B = reinterpret_cast<const uint16_t*>(p.B) + (int64_t)z * p.strideB;
    const uint16_t* A2 = reinterpret_cast<const uint16_t*>(p.A2) + (int64_t)z * p.strideA2;
    const uint16_t* B2 = reinterpret_cast<const uint16_t*>(p.B2) + (int64_t)z * p.strideB2;
    unsigned char* ring = lds + grp * kRing;
    EpiAddends<64, 64, 256> pre;
    load_addends(p, m0, n0, z, gtid, pre);
    f32x16_t acc[1][1];
    main_loop<G, false, false, S>(ring, A, p.lda, B, p.ldb, m0, n0, b, b, 0, b, gtid, acc);
    block_barrier();   // the second product reuses the LDS ring
    main_loop<G, true, true, S>(ring, A2, p.lda2, B2, p.ldb2, m0, n0, b, b, 0, b, gtid, acc, false);
    block_barrier();   // every wave is done reading the operand stages
    float* tile = reinterpret_cast<float*>(ring);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = wm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int col = wn * 32 + (lane & 31);
        tile[row * kLd + col] = acc[0][0][r];
    }
    __syncthreads();
    // dQ = alpha acc + beta1 Cin1 + beta2 Cin2, in place, as the general epilogue forms it
#pragma unroll
    for (int k = 0; k < EpiAddends<64, 64, 256>::kPer; ++k) {
        const int u = k * 256 + gtid;
        const int row = u / 16, c = (u % 16) * 4;
        float4 v = *reinterpret_cast<const float4*>(tile + row * kLd + c);
        v.x *= p.alpha; v.y *= p.alpha; v.z *= p.alpha; v.w *= p.alpha;
        const float4 a1 = pre.a1[k], a2 = pre.a2[k];
        const float4 o = make_float4(v.x + p.beta1 * a1.x + p.beta2 * a2.x, v.y + p.beta1 * a1.y + p.beta2 * a2.y,
                                     v.z + p.beta1 * a1.z + p.beta2 * a2.z, v.w + p.beta1 * a1.w + p.beta2 * a2.w);
        *reinterpret_cast<float4*>(tile + row * kLd + c) = o;
    }
    __syncthreads();
    const float* t0 = reinterpret_cast<const float*>(lds);
    const float* t1 = ti == tj ? t0 : reinterpret_cast<const float*>(lds + kRing);
    float* out = dq + (int64_t)z * ((int64_t)b * (b - 1) / 2);
#pragma unroll
    for (int k = 0; k < 64 * 64 / 512; ++k) {
        const int u = k * 512 + tid;
        const int rl = u >> 6, cl = u & 63;
        const int r = 64 * ti + rl, c = 64 * tj + cl;
        if (r < c) out[upper_index(r, c, b)] = t0[rl * kLd + cl] - t1[cl * kLd + rl];
    }
}

template <int BM, int BN, bool A_MN, bool B_MN, bool OUT_F32, int EPI = kEpiPlain, int S = 3, int NWM = 2, int NWN = 2,
          int DUAL = 0, bool GRP = false>
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
        hipLaunchKernelGGL((pipe_gemm_kernel<BM, BN, A_MN, B_MN, OUT_F32, EPI, S, NWM, NWN, DUAL, GRP>),
                           dim3(tiles, q.batch, p.splits), dim3(64 * NWM * NWN), 0, stream, q);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// ------------------------------------------------ block gradients, split K
// C (64 x 64 tile, float32) = A^T B with A [K][M] and B [K][N] m/n-major (the
// token axis is K).  A stage holds KSW consecutive 64-k tiles; the waves form
// KSW groups of WG waves, group g multiplies tile g of every stage into
// accumulators of its own (WG = 4: a 2 x 2 grid of 32 x 32 wave tiles; WG = 1:
// one wave owns the whole 64 x 64 tile), and the KSW partial tiles are summed
// through LDS in group order at the end, so the result does not depend on
// timing.  k-tiles past K (a ragged last stage) are still loaded, from clamped
// rows, so every stage costs every thread the same number of loads, and skipped.
template <int KSW, int WG, int S>
__global__ void __launch_bounds__(64 * KSW * WG) __attribute__((amdgpu_waves_per_eu(1, 2)))
grad_ks_kernel(const PipeArgs p) {
    constexpr int NWT = KSW * WG;                 // waves
    constexpr int kThreads = 64 * NWT;
    using G = Geo<64, 64, WG == 4 ? 2 : 1, WG == 4 ? 2 : 1>;
    constexpr int kTile = G::kStageBytes;        // A (64 k x 64 m) + B (64 k x 64 n)
    constexpr int kStage = KSW * kTile;
    constexpr int kRuns = OperandLoads<64, true, NWT>::n;   // per operand per k-tile per thread
    constexpr int kLoads = KSW * 2 * kRuns;                 // per thread per stage
    static_assert(S >= 2 && S * kStage <= 160 * 1024 && kLoads * (S - 1) < 64, "grad_ks geometry");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[S * kStage];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = wave / WG, wig = wave % WG;
    const int wm = WG == 4 ? wig >> 1 : 0, wn = WG == 4 ? wig & 1 : 0;
    const int M = p.M, N = p.N;
    const int kb = blockIdx.z * p.k_per_split;
    const int ke = min(p.K, kb + p.k_per_split);
    int z, tm, tn;
    batch_tile_coords((M + 63) / 64, (N + 63) / 64, z, tm, tn);
    const int m0 = tm * 64, n0 = tn * 64;
    const uint16_t* A = reinterpret_cast<const uint16_t*>(p.A) + (int64_t)z * p.strideA;
    const uint16_t* B = reinterpret_cast<const uint16_t*>(p.B) + (int64_t)z * p.strideB;
    const uint32_t base = lds_offset(lds);
    const int nk = ke > kb ? (ke - kb + 63) / 64 : 0;
    const int ng = (nk + KSW - 1) / KSW;
    f32x16_t acc[G::MI][G::NJ];
#pragma unroll
    for (int i = 0; i < G::MI; ++i)
#pragma unroll
        for (int j = 0; j < G::NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    auto issue = [&](int g, int stage) {
#pragma unroll
        for (int t = 0; t < KSW; ++t) {
            const uint32_t dst = base + stage * kStage + t * kTile;
            const int k0 = kb + (KSW * g + t) * 64;
#pragma unroll
            for (int j = 0; j < kRuns; ++j) {
                dma_one<64, true, NWT>(j, dst, A, p.lda, m0, M, k0, ke, wave, lane);
                dma_one<64, true, NWT>(j, dst + G::kABytes, B, p.ldb, n0, N, k0, ke, wave, lane);
            }
        }
    };
#pragma unroll
    for (int g = 0; g < S - 1; ++g)
        if (g < ng) issue(g, g);
    int st = 0, st_load = S - 1;
    for (int g = 0; g < ng; ++g) {
        wait_tiles<kLoads, S>(min(ng, g + S - 1) - g - 1);
        block_barrier();   // stage g landed everywhere; stage g - 1 is no longer read
        if (g + S - 1 < ng) issue(g + S - 1, st_load);
        const int kt = KSW * g + grp;
        if (kt < nk) {
            unsigned char* tile = lds + st * kStage + grp * kTile;
            const int valid = ke - (kb + kt * 64);
            if (valid < 64) {
                // rows past K came from clamped rows: every wave of the group
                // zeroes all of them itself (identical writes) before its own
                // reads, so the group needs no barrier of its own
                zero_rows_mn<64, 64>(tile, valid, lane);
                zero_rows_mn<64, 64>(tile + G::kABytes, valid, lane);
            }
            uint4 af[2][G::MI], bfr[2][G::NJ];
            load_frags<G, true, true>(tile, wm, wn, 0, lane, af[0], bfr[0]);
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) {
                const int cur = ks & 1;
                if (ks + 1 < BK / 16) load_frags<G, true, true>(tile, wm, wn, ks + 1, lane, af[cur ^ 1], bfr[cur ^ 1]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < G::MI; ++i)
#pragma unroll
                    for (int j = 0; j < G::NJ; ++j) Mfma32<bf16_t>::run(af[cur][i], bfr[cur][j], acc[i][j]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        st = st == S - 1 ? 0 : st + 1;
        st_load = st_load == S - 1 ? 0 : st_load + 1;
    }
    // sum of the KSW partial tiles, then rows of 64 floats to C
    block_barrier();   // every wave is done reading the operand stages
    float* part = reinterpret_cast<float*>(lds);   // [KSW][64 rows][64 + 4]
    constexpr int kLd = 68;
    static_assert(KSW * 64 * kLd * 4 <= S * kStage, "partial tiles exceed the LDS ring");
#pragma unroll
    for (int i = 0; i < G::MI; ++i)
#pragma unroll
        for (int j = 0; j < G::NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * G::WTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                const int col = wn * G::WTN + j * 32 + (lane & 31);
                part[(grp * 64 + row) * kLd + col] = acc[i][j][r];
            }
    __syncthreads();
    float* C = reinterpret_cast<float*>(p.C) + (int64_t)z * p.strideC + (int64_t)blockIdx.z * p.strideSplit;
#pragma unroll
    for (int u0 = 0; u0 < 64 * 16; u0 += kThreads) {
        const int u = u0 + tid;
        if (u >= 64 * 16) break;
        const int row = u >> 4, c4 = (u & 15) * 4;
        float4 v = *reinterpret_cast<const float4*>(part + row * kLd + c4);
#pragma unroll
        for (int w = 1; w < KSW; ++w) {
            const float4 x = *reinterpret_cast<const float4*>(part + (w * 64 + row) * kLd + c4);
            v.x += x.x; v.y += x.y; v.z += x.z; v.w += x.w;
        }
        const int gr = m0 + row, gc = n0 + c4;
        if (gr >= M) continue;
        float* dst = C + (int64_t)gr * p.ldc + gc;
        if (gc + 3 < N && (p.ldc & 3) == 0) {
            *reinterpret_cast<float4*>(dst) = v;
        } else {
            if (gc < N) dst[0] = v.x;
            if (gc + 1 < N) dst[1] = v.y;
            if (gc + 2 < N) dst[2] = v.z;
            if (gc + 3 < N) dst[3] = v.w;
        }
    }
}

template <int KSW, int WG, int S>
hipError_t launch_grad_ks(const PipeArgs& p, hipStream_t stream) {
    const int tiles = ((p.M + 63) / 64) * ((p.N + 63) / 64);
    constexpr int kMaxY = 65535;
    for (int y0 = 0; y0 < p.batch; y0 += kMaxY) {
        PipeArgs q = p;
        q.batch = min(kMaxY, p.batch - y0);
        q.A = reinterpret_cast<const uint16_t*>(p.A) + (int64_t)y0 * p.strideA;
        q.B = reinterpret_cast<const uint16_t*>(p.B) + (int64_t)y0 * p.strideB;
        q.C = reinterpret_cast<float*>(p.C) + (int64_t)y0 * p.strideC;
        hipLaunchKernelGGL((grad_ks_kernel<KSW, WG, S>), dim3(tiles, q.batch, p.splits), dim3(64 * KSW * WG), 0,
                           stream, q);
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
// One workgroup per (block z, panel p of PH rows) for bf16 blocks of b = 128 or
// 256, straight from the packed parameters:
//  1. Q = U - U^T is built in LDS in bf16 from the block's strict upper
//     triangle U (row-major packed): each thread takes 8 x 8 sub-blocks of U
//     (16-byte loads of their row segments) and writes their rows, and the
//     negated rows of their transpose, as 16-byte chunks (a diagonal sub-block
//     holds both halves and a zero diagonal).  The image is [b/64] k-tiles of
//     [b rows][64 k], 128-byte rows of eight 16-byte chunks, chunk c of row r in
//     slot c ^ (r & 7) ^ ((r >> 3) & 7): the MFMA fragment reads (16 consecutive
//     rows, one chunk), the row writes (one row, consecutive chunks) and the
//     transposed writes (rows 8 apart, one chunk) all meet at most two lanes
//     per bank group.
//  2. Horner on the panel rows, X_1 = Q_p, X_{i+1} = X_i Q, each product taken
//     transposed, C = Q X_i^T = -X_{i+1}^T, so that a lane holds four
//     consecutive columns of a row of X_{i+1} (one 8-byte LDS write).  X_1 is
//     read from the Q image itself.
//  3. G_p = I_p + 2 (X_1 + ... + X_k) + X_{k+1}, the rows p of
//     (I + Q) sum_{i<=k} Q^i: the sum stays in float32 registers, each X_{i+1}
//     is rounded to bf16 into LDS for the next product, and G_p is staged in the
//     X buffer and stored as whole rows.
// With Qc given the panel rows of Q are stored as well; with S / T (k >= 2)
// S_p = X_2 and T_p = 2 Q_p + S_p (what the saving forward keeps for k = 3).
template <int B, int PH>
struct FusedCnp {
    static constexpr int KT = B / 64;         // k-tiles of one product
    static constexpr int NP = B / PH;         // panels per block
    static constexpr int QB = B * 128;        // bytes of one Q k-tile ([B rows][64 k])
    static constexpr int XB = PH * 128;       // bytes of one X k-tile ([PH rows][64 k])
    static constexpr int LDS = KT * (QB + XB);
    static constexpr int MI = B / 128;        // wave w: rows n in [w B/4, (w+1) B/4) of C
    static constexpr int NJ = PH / 32;        //         and all PH columns m
    static constexpr int NPAR = B * (B - 1) / 2;
    static constexpr int NB8 = B / 8;         // 8 x 8 sub-blocks per side
    static constexpr int OFFDIAG = NB8 * (NB8 - 1) / 2;
    static constexpr int TASKS = NB8 + OFFDIAG;
};

__device__ __forceinline__ int cnp_swz(int row) { return (row & 7) ^ ((row >> 3) & 7); }

// Byte offset of element (row, k) in a k-tiled image with k-tile size TILE.
template <int TILE>
__device__ __forceinline__ int img_off(int row, int kk) {
    return (kk >> 6) * TILE + row * 128 + ((((kk & 63) >> 3) ^ cnp_swz(row)) << 4) + (kk & 7) * 2;
}

// k-major fragment of rows row0 .. row0 + 31 (lane l: row row0 + l % 32,
// k = 16 ks + 8 (l / 32) + 0..7) from a k-tile of such an image.
__device__ __forceinline__ uint4 img_frag(const unsigned char* __restrict__ tile, int row0, int ks, int lane) {
    const int row = row0 + (lane & 31);
    const int slot = (2 * ks + (lane >> 5)) ^ cnp_swz(row);
    return *reinterpret_cast<const uint4*>(tile + row * 128 + slot * 16);
}

typedef float f32x4u_t __attribute__((ext_vector_type(4), aligned(4)));

template <int B, int PH>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, B == 256 ? 1 : 2)))
cnp_fused_kernel(const float* __restrict__ q, uint16_t* __restrict__ G, uint16_t* __restrict__ Qc,
                 uint16_t* __restrict__ Sv, uint16_t* __restrict__ Tv, int k, int total) {
    using F = FusedCnp<B, PH>;
    constexpr int KT = F::KT, QB = F::QB, XB = F::XB, MI = F::MI, NJ = F::NJ, NB8 = F::NB8;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[F::LDS];
    unsigned char* qs = lds;
    unsigned char* xs = lds + KT * QB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int id = blockIdx.x;
    if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);   // each XCD gets whole blocks
    const int z = id / F::NP, p = id - z * F::NP;
    const int64_t zoff = (int64_t)z * B * B;
    const float* __restrict__ qz = q + (int64_t)z * F::NPAR;
    const int r0 = PH * p;   // first row of the panel

    // 1. the Q image.  Tasks: the strict upper sub-blocks (sub-rows R' and
    // NB8 - 2 - R' sharing a run of NB8 tasks), then the diagonal ones; every
    // thread issues the loads of all its tasks before it writes any.
    constexpr int NTASK = (F::TASKS + 255) / 256;
    float u[NTASK][8][8];
#pragma unroll
    for (int s = 0; s < NTASK; ++s) {
        const int t = tid + 256 * s;
        if (t < F::OFFDIAG) {
            const int Rp = t / NB8, cp = t - Rp * NB8;
            const bool first = cp < NB8 - 1 - Rp;
            const int R = first ? Rp : NB8 - 2 - Rp;
            const int C = first ? Rp + 1 + cp : R + 1 + cp - (NB8 - 1 - Rp);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 8 * R + i;
                const float* src = qz + (r * B - r * (r + 1) / 2 - r - 1 + 8 * C);   // U[r][8C]
                const f32x4u_t lo = *reinterpret_cast<const f32x4u_t*>(src);
                const f32x4u_t hi = *reinterpret_cast<const f32x4u_t*>(src + 4);
                u[s][i][0] = lo.x; u[s][i][1] = lo.y; u[s][i][2] = lo.z; u[s][i][3] = lo.w;
                u[s][i][4] = hi.x; u[s][i][5] = hi.y; u[s][i][6] = hi.z; u[s][i][7] = hi.w;
            }
        } else if (t < F::TASKS) {   // diagonal sub-block: scalar loads, clamped below the diagonal
            const int R = t - F::OFFDIAG;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 8 * R + i;
                const int base = r * B - r * (r + 1) / 2 - r - 1;   // U[r][c] at base + c
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int c = 8 * R + j;
                    const float v = qz[max(base + c, 0)];   // base + c >= -1 below the diagonal
                    u[s][i][j] = c > r ? v : 0.f;
                }
            }
        }
    }
#pragma unroll
    for (int s = 0; s < NTASK; ++s) {
        const int t = tid + 256 * s;
        if (t < F::OFFDIAG) {
            const int Rp = t / NB8, cp = t - Rp * NB8;
            const bool first = cp < NB8 - 1 - Rp;
            const int R = first ? Rp : NB8 - 2 - Rp;
            const int C = first ? Rp + 1 + cp : R + 1 + cp - (NB8 - 1 - Rp);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                *reinterpret_cast<uint4*>(qs + img_off<QB>(8 * R + i, 8 * C)) =
                    make_uint4(pack_bf16x2(u[s][i][0], u[s][i][1]), pack_bf16x2(u[s][i][2], u[s][i][3]),
                               pack_bf16x2(u[s][i][4], u[s][i][5]), pack_bf16x2(u[s][i][6], u[s][i][7]));
#pragma unroll
            for (int j = 0; j < 8; ++j)
                *reinterpret_cast<uint4*>(qs + img_off<QB>(8 * C + j, 8 * R)) =
                    make_uint4(pack_bf16x2(-u[s][0][j], -u[s][1][j]), pack_bf16x2(-u[s][2][j], -u[s][3][j]),
                               pack_bf16x2(-u[s][4][j], -u[s][5][j]), pack_bf16x2(-u[s][6][j], -u[s][7][j]));
        } else if (t < F::TASKS) {
            // rows of the diagonal sub-block: U above the diagonal, -U^T below
            const int R = t - F::OFFDIAG;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = j > i ? u[s][i][j] : (j < i ? -u[s][j][i] : 0.f);
                *reinterpret_cast<uint4*>(qs + img_off<QB>(8 * R + i, 8 * R)) =
                    make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                               pack_bf16x2(v[6], v[7]));
            }
        }
    }
    __syncthreads();

    // rows of an image as 16-byte chunks: PH rows x B/8 chunks over the workgroup
    auto copy_rows = [&](uint16_t* __restrict__ dst, auto chunk_value) {
        for (int u = tid; u < PH * (B / 8); u += 256) {
            const int m = u / (B / 8), c8 = u - m * (B / 8);
            *reinterpret_cast<uint4*>(dst + zoff + (int64_t)(r0 + m) * B + 8 * c8) = chunk_value(m, 8 * c8);
        }
    };
    if (Qc)
        copy_rows(Qc, [&](int m, int c) { return *reinterpret_cast<const uint4*>(qs + img_off<QB>(r0 + m, c)); });

    // 2. Horner: acc = Q X_it^T, X_{it+1} = -acc^T
    f32x16_t sum[MI][NJ], acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) sum[i][j][r] = 0.f;
    const int n_base = wave * (B / 4);
    for (int it = 1; it <= k; ++it) {
        // B operand: X_1 = rows r0.. of the Q image, later X_it in the X buffer
        const unsigned char* xb = it == 1 ? qs : xs;
        const int xtile = it == 1 ? QB : XB;
        const int xrow = it == 1 ? r0 : 0;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
        uint4 af[2][MI], bfr[2][NJ];
        auto load = [&](int ks, uint4 (&a)[MI], uint4 (&b)[NJ]) {
            const int kt = ks >> 2, kk = ks & 3;
#pragma unroll
            for (int i = 0; i < MI; ++i) a[i] = img_frag(qs + kt * QB, n_base + i * 32, kk, lane);
#pragma unroll
            for (int j = 0; j < NJ; ++j) b[j] = img_frag(xb + kt * xtile, xrow + j * 32, kk, lane);
        };
        load(0, af[0], bfr[0]);
#pragma unroll
        for (int ks = 0; ks < 4 * KT; ++ks) {
            const int cur = ks & 1;
            if (ks + 1 < 4 * KT) load(ks + 1, af[cur ^ 1], bfr[cur ^ 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) Mfma32<bf16_t>::run(af[cur][i], bfr[cur][j], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // X_{it+1} enters the sum with weight 2 up to X_k, 1 for X_{k+1}
        const float w = it < k ? -2.f : -1.f;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) sum[i][j][r] += w * acc[i][j][r];
        if (it < k) {
            block_barrier();   // every wave is done reading X_it
            // lane: column m = 32 j + lane % 32 of C, rows n = n0 .. n0 + 3 per (i, r / 4)
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int m = j * 32 + (lane & 31);
                        const int n0 = n_base + i * 32 + r4 * 8 + (lane >> 5) * 4;
                        *reinterpret_cast<uint2*>(xs + img_off<XB>(m, n0)) =
                            make_uint2(pack_bf16x2(-acc[i][j][4 * r4], -acc[i][j][4 * r4 + 1]),
                                       pack_bf16x2(-acc[i][j][4 * r4 + 2], -acc[i][j][4 * r4 + 3]));
                    }
            __syncthreads();
            if (it == 1 && Sv) {   // S_p = X_2, T_p = 2 Q_p + S_p
                copy_rows(Sv, [&](int m, int c) { return *reinterpret_cast<const uint4*>(xs + img_off<XB>(m, c)); });
                copy_rows(Tv, [&](int m, int c) {
                    const uint4 sv = *reinterpret_cast<const uint4*>(xs + img_off<XB>(m, c));
                    const uint4 qv = *reinterpret_cast<const uint4*>(qs + img_off<QB>(r0 + m, c));
                    const uint32_t s4[4] = {sv.x, sv.y, sv.z, sv.w}, q4[4] = {qv.x, qv.y, qv.z, qv.w};
                    uint32_t t4[4];
#pragma unroll
                    for (int h = 0; h < 4; ++h)
                        t4[h] = pack_bf16x2(2.f * bf16_to_f32((uint16_t)q4[h]) + bf16_to_f32((uint16_t)s4[h]),
                                            2.f * bf16_to_f32((uint16_t)(q4[h] >> 16)) +
                                                bf16_to_f32((uint16_t)(s4[h] >> 16)));
                    return make_uint4(t4[0], t4[1], t4[2], t4[3]);
                });
            }
        }
    }

    // 3. G_p = I_p + 2 Q_p + sum, staged in the X buffer, then stored by rows
    block_barrier();   // every wave is done reading the X buffer
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int m = j * 32 + (lane & 31);
                const int n0 = n_base + i * 32 + r4 * 8 + (lane >> 5) * 4;
                const uint2 qv = *reinterpret_cast<const uint2*>(qs + img_off<QB>(r0 + m, n0));
                float g[4];
                const uint32_t q2[2] = {qv.x, qv.y};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint16_t qh = (uint16_t)(q2[e >> 1] >> (16 * (e & 1)));
                    g[e] = (r0 + m == n0 + e ? 1.f : 0.f) + 2.f * bf16_to_f32(qh) + sum[i][j][4 * r4 + e];
                }
                *reinterpret_cast<uint2*>(xs + img_off<XB>(m, n0)) =
                    make_uint2(pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]));
            }
    __syncthreads();
    copy_rows(G, [&](int m, int c) { return *reinterpret_cast<const uint4*>(xs + img_off<XB>(m, c)); });
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
    // instantiated combinations: dense / block products (k-major A, bf16 out),
    // block gradients (m/n-major A and B, float32 out) and the two below
    if (p.ngroups > 0) {
        // grouped dense products (k-major A, bf16 out, 128-column tiles)
        if (a_mn || out_f32 || p.batch != 1 || p.splits != 1 || p.ngroups > kMaxPipeGroups) return hipErrorInvalidValue;
        if (tile == PipeTile::Square)
            return b_mn ? launch<128, 128, false, true, false, kEpiPlain, 4, 2, 2, 0, true>(p, stream)
                        : launch<128, 128, false, false, false, kEpiPlain, 4, 2, 2, 0, true>(p, stream);
        if (tile == PipeTile::Slim)
            return b_mn ? launch<64, 128, false, true, false, kEpiPlain, 4, 2, 2, 0, true>(p, stream)
                        : launch<64, 128, false, false, false, kEpiPlain, 4, 2, 2, 0, true>(p, stream);
        if (tile != PipeTile::Tall) return hipErrorInvalidValue;
        return b_mn ? launch<256, 128, false, true, false, kEpiPlain, 3, 4, 2, 0, true>(p, stream)
                    : launch<256, 128, false, false, false, kEpiPlain, 3, 4, 2, 0, true>(p, stream);
    }
    if (!a_mn && !out_f32) {
        if (tile == PipeTile::Square)
            return b_mn ? launch<128, 128, false, true, false, kEpiPlain, 4>(p, stream)
                        : launch<128, 128, false, false, false, kEpiPlain, 4>(p, stream);
        if (tile == PipeTile::Slim)
            return b_mn ? launch<64, 128, false, true, false, kEpiPlain, 4>(p, stream)
                        : launch<64, 128, false, false, false, kEpiPlain, 4>(p, stream);
        if (tile == PipeTile::Big)
            return b_mn ? launch<256, 256, false, true, false, kEpiPlain, 2, 2, 4>(p, stream)
                        : launch<256, 256, false, false, false, kEpiPlain, 2, 2, 4>(p, stream);
        if (tile == PipeTile::Wide)
            return b_mn ? launch<128, 256, false, true, false, kEpiPlain, 3, 2, 4>(p, stream)
                        : launch<128, 256, false, false, false, kEpiPlain, 3, 2, 4>(p, stream);
        return b_mn ? launch<256, 128, false, true, false, kEpiPlain, 3, 4, 2>(p, stream)
                    : launch<256, 128, false, false, false, kEpiPlain, 3, 4, 2>(p, stream);
    }
    // dense products of the weight-centric variant: float32 output with k-major
    // A (NT, NN), bf16 output with m/n-major A and B (TN)
    if (!a_mn && out_f32) {
        if (tile == PipeTile::Square)
            return b_mn ? launch<128, 128, false, true, true, kEpiPlain, 4>(p, stream)
                        : launch<128, 128, false, false, true, kEpiPlain, 4>(p, stream);
        return b_mn ? launch<256, 128, false, true, true, kEpiPlain, 3, 4, 2>(p, stream)
                    : launch<256, 128, false, false, true, kEpiPlain, 3, 4, 2>(p, stream);
    }
    if (a_mn && b_mn && !out_f32) {
        if (tile == PipeTile::Square) return launch<128, 128, true, true, false, kEpiPlain, 4>(p, stream);
        return launch<256, 128, true, true, false, kEpiPlain, 3, 4, 2>(p, stream);
    }
    if (a_mn && b_mn && out_f32) {
        if (tile == PipeTile::Square) return launch<128, 128, true, true, true, kEpiPlain, 4>(p, stream);
        // 64 x 64 block-gradient tiles: two k-tiles per stage, one per group of
        // four waves, for token runs up to 4096; longer runs stream better with
        // one k-tile per stage and a four-stage ring
        if (tile == PipeTile::Small)
            return p.k_per_split <= 4096 ? launch_grad_ks<2, 4, 2>(p, stream)
                                         : launch<64, 64, true, true, true, kEpiPlain, 4>(p, stream);
        return launch<256, 128, true, true, true, kEpiPlain, 3, 4, 2>(p, stream);
    }
    return hipErrorInvalidValue;
}

template <int T, bool OUT_F32, int S>
hipError_t launch_general(bool a_mn, bool b_mn, const PipeArgs& p, hipStream_t stream) {
    if (!a_mn && !b_mn) return launch<T, T, false, false, OUT_F32, kEpiGeneral, S>(p, stream);
    if (!a_mn && b_mn) return launch<T, T, false, true, OUT_F32, kEpiGeneral, S>(p, stream);
    return launch<T, T, true, true, OUT_F32, kEpiGeneral, S>(p, stream);
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
    // 64 x 64 tiles: measured ahead of 128 x 128 ones for b = 256 and 512 from
    // 32 to 4000 blocks (the K = b products are short and bound by their
    // epilogue traffic; more workgroups per CU overlap it).  For the same reason
    // the ring is shallow: two stages (five workgroups per CU) for K <= 256,
    // three for longer K (same-process sweep: 320 blocks of 256 101 -> 76 us,
    // 36 blocks of 512 40 -> 32 us, against four stages).
    if (p.k_per_split <= 256)
        return out_f32 ? launch_general<64, true, 2>(a_mn, b_mn, p, stream)
                       : launch_general<64, false, 2>(a_mn, b_mn, p, stream);
    return out_f32 ? launch_general<64, true, 3>(a_mn, b_mn, p, stream)
                   : launch_general<64, false, 3>(a_mn, b_mn, p, stream);
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
    // shallow rings as for pipe_gemm_general (mode 2 keeps two epilogue tiles,
    // so at least three stages): 320 blocks of 256 119 -> 98 us and 109 -> 96 us
    if (separate) {
        return out_f32 ? launch<64, 64, false, false, true, kEpiGeneral, 3, 2, 2, 2>(p, stream)
                       : launch<64, 64, false, false, false, kEpiGeneral, 3, 2, 2, 2>(p, stream);
    }
    if (p.k_per_split <= 256)
        return out_f32 ? launch<64, 64, false, false, true, kEpiGeneral, 2, 2, 2, 1>(p, stream)
                       : launch<64, 64, false, false, false, kEpiGeneral, 2, 2, 2, 1>(p, stream);
    return out_f32 ? launch<64, 64, false, false, true, kEpiGeneral, 3, 2, 2, 1>(p, stream)
                   : launch<64, 64, false, false, false, kEpiGeneral, 3, 2, 2, 1>(p, stream);
}

hipError_t cnp_pack_pair(const PipeArgs& p_in, float* dq, int b, hipStream_t stream) {
    if (p_in.batch <= 0) return hipSuccess;
    if (b % 64 != 0 || !p_in.A2 || !p_in.B2 || p_in.M != b || p_in.N != b || p_in.K != b)
        return hipErrorInvalidValue;
    PipeArgs p = p_in;
    auto al = [](const void* ptr, int64_t ld, int64_t stride) {
        return ptr == nullptr || (((uintptr_t)ptr % 16) == 0 && ld % 4 == 0 && stride % 4 == 0);
    };
    p.epi_vec = al(p.Cin1, p.ldcin1, p.strideCin1) && al(p.Cin2, p.ldcin2, p.strideCin2);
    const int nt = b / 64;
    const int64_t ntri = (int64_t)b * (b - 1) / 2;
    constexpr int kMaxY = 65535;
    for (int y0 = 0; y0 < p_in.batch; y0 += kMaxY) {
        PipeArgs q = p;
        q.batch = min(kMaxY, p_in.batch - y0);
        q.A = reinterpret_cast<const uint16_t*>(p.A) + (int64_t)y0 * p.strideA;
        q.B = reinterpret_cast<const uint16_t*>(p.B) + (int64_t)y0 * p.strideB;
        q.A2 = reinterpret_cast<const uint16_t*>(p.A2) + (int64_t)y0 * p.strideA2;
        q.B2 = reinterpret_cast<const uint16_t*>(p.B2) + (int64_t)y0 * p.strideB2;
        if (p.Cin1) q.Cin1 = p.Cin1 + (int64_t)y0 * p.strideCin1;
        if (p.Cin2) q.Cin2 = p.Cin2 + (int64_t)y0 * p.strideCin2;
        const dim3 grid(nt * (nt + 1) / 2, q.batch);
        if (b <= 256)
            hipLaunchKernelGGL(cnp_pack_pair_kernel<2>, grid, dim3(512), 0, stream, q, dq + (int64_t)y0 * ntri, b);
        else
            hipLaunchKernelGGL(cnp_pack_pair_kernel<3>, grid, dim3(512), 0, stream, q, dq + (int64_t)y0 * ntri, b);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

int pipe_tile_rows(PipeTile t) {
    return (t == PipeTile::Tall || t == PipeTile::Big) ? 256 : (t == PipeTile::Small || t == PipeTile::Slim) ? 64 : 128;
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
    // the largest tile whose grid still gives every CU a workgroup: 256 x 256
    // (two-stage ring, two waves per SIMD), 256 x 128, 128 x 128, else 64 x 128
    auto tiles = [&](int bm, int bn) { return (int64_t)((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    const PipeTile t = tiles(256, 256) >= 256   ? PipeTile::Big
                       : tiles(256, 128) >= 256 ? PipeTile::Tall
                       : tiles(128, 128) >= 256 ? PipeTile::Square
                                                : PipeTile::Slim;
    return pipe_gemm(false, b_nn, false, p, stream, t);
}

bool cnp_fused_supported(int64_t b, int k) { return (b == 128 || b == 256) && k >= 1; }

hipError_t cnp_fused_fwd(const float* q, void* G, void* Qc, void* S, void* T, int64_t nblk, int64_t b, int k,
                         hipStream_t stream) {
    if (nblk <= 0) return hipSuccess;
    if (!cnp_fused_supported(b, k) || ((S == nullptr) != (T == nullptr)) || (S && k < 2)) return hipErrorInvalidValue;
    // 64-row panels, or 32-row ones while 64-row panels would not give every CU one
    const bool tall = nblk * (b / 64) >= 256;
    const int64_t panels = nblk * (b / (tall ? 64 : 32));
    if (panels > 0x7fffffff) return hipErrorInvalidValue;
    const auto g = static_cast<uint16_t*>(G);
    const auto qc = static_cast<uint16_t*>(Qc);
    const auto sv = static_cast<uint16_t*>(S);
    const auto tv = static_cast<uint16_t*>(T);
    const dim3 grid((unsigned)panels);
    if (b == 256 && tall)
        hipLaunchKernelGGL((cnp_fused_kernel<256, 64>), grid, dim3(256), 0, stream, q, g, qc, sv, tv, k, (int)panels);
    else if (b == 256)
        hipLaunchKernelGGL((cnp_fused_kernel<256, 32>), grid, dim3(256), 0, stream, q, g, qc, sv, tv, k, (int)panels);
    else if (tall)
        hipLaunchKernelGGL((cnp_fused_kernel<128, 64>), grid, dim3(256), 0, stream, q, g, qc, sv, tv, k, (int)panels);
    else
        hipLaunchKernelGGL((cnp_fused_kernel<128, 32>), grid, dim3(256), 0, stream, q, g, qc, sv, tv, k, (int)panels);
    return hipGetLastError();
}

}  // namespace poetx
