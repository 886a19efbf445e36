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
#include <algorithm>
#include <type_traits>

#include "dense_gemm.h"
#include "device_common.h"

namespace poetx {

namespace {

constexpr int BK = 64;

// Workgroup tile BM x BN (x 64 k), NWM x NWN waves, each owning a WTM x WTN
// sub-tile of MI x NJ 32 x 32 MFMA tiles.
// Q8: B is an int8 operand.  A stage then holds A and the int8 B tile (BN x 64
// bytes); the bf16 B tile the fragments read lives in a double buffer after the
// ring, widened from the int8 tile one k-tile ahead.
template <int BM_, int BN_, int NWM_ = 2, int NWN_ = 2, bool Q8_ = false>
struct Geo {
    static constexpr int BM = BM_, BN = BN_, NWM = NWM_, NWN = NWN_;
    static constexpr bool Q8 = Q8_;
    static constexpr int NW = NWM * NWN;
    static constexpr int kThreads = 64 * NW;
    static constexpr int kABytes = BM * BK * 2;
    static constexpr int kBBytes = BN * BK * 2;    // bf16 B tile
    static constexpr int kB8Bytes = BN * BK;       // int8 B tile
    static constexpr int kStageBytes = kABytes + (Q8 ? kB8Bytes : kBBytes);
    static constexpr int kExtraBytes = Q8 ? 2 * kBBytes : 0;   // the widened double buffer
    static constexpr int WTM = BM / NWM, WTN = BN / NWN, MI = WTM / 32, NJ = WTN / 32;
    static constexpr int kLoadsPerTile = kStageBytes / (kThreads * 16);
    static_assert(MI >= 1 && NJ >= 1 && kStageBytes % (kThreads * 16) == 0, "tile geometry");
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

// The same load with a wave-uniform 64-bit base (SGPR pair) and a 32-bit
// per-lane byte offset: the base moves with the k-tile, the offsets stay
// fixed, so the loop issues no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0): this wave's LDS reads and writes are done.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4)); }

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

// Loads of an int8 operand tile (unswizzled in LDS: it is only read by the
// widening pass, one 16-byte chunk per thread).
//   k-major: ROWS rows x 64 k bytes from src[row][k], rows clamped to rows_total;
//   n-major: 64 k-rows x ROWS bytes from src[k][col], k clamped to k_end,
//   columns clamped to rows_total (a multiple of 16).
template <int ROWS, int NW>
struct OperandLoads8 {
    static constexpr int runs = ROWS * BK / 1024;
    static constexpr int n = runs / NW;
    static_assert(runs % NW == 0, "int8 runs per wave");
};

template <int ROWS, bool MN, int NW>
__device__ __forceinline__ void dma_one8(int j, uint32_t dst, const int8_t* __restrict__ src, int64_t ld, int r0,
                                         int rows_total, int k0, int k_end, int wave, int lane) {
    const int g = j * NW + wave;
    if constexpr (!MN) {
        const int r = 16 * g + (lane >> 2);             // 16 rows of 64 bytes per run
        const int row = min(r0 + r, rows_total - 1);
        dma16(src + (int64_t)row * ld + k0 + (lane & 3) * 16, __builtin_amdgcn_readfirstlane(dst + g * 1024));
    } else {
        constexpr int kSlots = ROWS / 16;               // 16-byte chunks per k-row
        constexpr int kRowsPerRun = 1024 / ROWS;
        const int kr = kRowsPerRun * g + lane / kSlots;
        const int col = min(r0 + (lane % kSlots) * 16, rows_total - 16);
        const int k = min(k0 + kr, k_end - 1);
        dma16(src + (int64_t)k * ld + col, __builtin_amdgcn_readfirstlane(dst + g * 1024));
    }
}

// Byte offset of the j-th 1 KB run's 16 bytes for this lane, relative to the
// operand's k-tile base (k-major: src + k0; m/n-major: src + k0 ld), with the
// row / column clamps of dma_one; k needs no clamp (whole k-tiles only).
template <int ROWS, bool MN, int NW>
__device__ __forceinline__ uint32_t dma_voff(int j, int64_t ld, int r0, int rows_total, int wave, int lane) {
    const int g = j * NW + wave;
    if constexpr (!MN) {
        const int r = 8 * g + (lane >> 3);
        const int c = (lane & 7) ^ swz_k(r);
        const int row = min(r0 + r, rows_total - 1);
        return (uint32_t)(2 * ((int64_t)row * ld + c * 8));
    } else {
        constexpr int kRowBytes = ROWS * 2;
        constexpr int kRowsPerRun = 1024 / kRowBytes;
        constexpr int kSlots = kRowBytes / 16;
        const int kr = kRowsPerRun * g + lane / kSlots;
        const int c = (lane % kSlots) ^ swz_mn<ROWS>(kr);
        const int col = min(r0 + c * 8, rows_total - 8);
        return (uint32_t)(2 * ((int64_t)kr * ld + col));
    }
}

// The same for an int8 operand tile (dma_one8's addressing), in bytes.
template <int ROWS, bool MN, int NW>
__device__ __forceinline__ uint32_t dma_voff8(int j, int64_t ld, int r0, int rows_total, int wave, int lane) {
    const int g = j * NW + wave;
    if constexpr (!MN) {
        const int r = 16 * g + (lane >> 2);
        const int row = min(r0 + r, rows_total - 1);
        return (uint32_t)((int64_t)row * ld + (lane & 3) * 16);
    } else {
        constexpr int kSlots = ROWS / 16;
        constexpr int kRowsPerRun = 1024 / ROWS;
        const int kr = kRowsPerRun * g + lane / kSlots;
        const int col = min(r0 + (lane % kSlots) * 16, rows_total - 16);
        return (uint32_t)((int64_t)kr * ld + col);
    }
}

// Everything needed to issue the loads of one k-tile into one LDS stage.
// Q8 jobs load the int8 B tile of the NEXT k-tile (k0_b) into stage_b, so that
// it can be widened while the current tile computes.  Products with a k-major
// A (SADDR) carry fixed per-lane offsets and move only the two uniform bases.
struct DmaJob {
    uint32_t stage;
    const uint16_t* A;
    int64_t lda;
    const uint16_t* B;
    int64_t ldb;
    int m0, n0, M, N, k0, k_end, wave, lane;
    uint32_t stage_b = 0;
    int k0_b = 0;
    const char* a_k = nullptr;   // SADDR: A + k0 (bytes), B + k0 or B + k0 ldb
    const char* b_k = nullptr;
    uint32_t voff[16] = {};      // SADDR: per-lane offsets of the tile's loads (A's, then B's)
};

// Part PART of NPARTS of a k-tile's loads (A's loads first, then B's), so the
// loads can be spread over the MFMA work of the tile being computed.
template <class G, bool A_MN>
constexpr bool kSaddr = !A_MN;

template <class G, bool A_MN, bool B_MN, int PART, int NPARTS>
__device__ __forceinline__ void dma_part(const DmaJob& d) {
    constexpr int NA = OperandLoads<G::BM, A_MN, G::NW>::n;
    constexpr int NB = G::Q8 ? OperandLoads8<G::BN, G::NW>::n : OperandLoads<G::BN, B_MN, G::NW>::n;
    constexpr int L = NA + NB;
    constexpr int lo = PART * L / NPARTS, hi = (PART + 1) * L / NPARTS;
    static_assert(!kSaddr<G, A_MN> || L <= 16, "per-lane offsets");
#pragma unroll
    for (int idx = lo; idx < hi; ++idx) {
        if constexpr (kSaddr<G, A_MN>) {
            const bool is_a = idx < NA;
            const int g = (is_a ? idx : idx - NA) * G::NW + d.wave;
            const uint32_t m0 = (is_a ? d.stage : G::Q8 ? d.stage_b : d.stage + (uint32_t)G::kABytes) + g * 1024;
            dma16s(is_a ? d.a_k : d.b_k, d.voff[idx], __builtin_amdgcn_readfirstlane(m0));
            continue;
        }
        if (idx < NA)
            dma_one<G::BM, A_MN, G::NW>(idx, d.stage, d.A, d.lda, d.m0, d.M, d.k0, d.k_end, d.wave, d.lane);
        else if constexpr (G::Q8)
            dma_one8<G::BN, B_MN, G::NW>(idx - NA, d.stage_b, reinterpret_cast<const int8_t*>(d.B), d.ldb, d.n0, d.N,
                                         d.k0_b, d.k_end, d.wave, d.lane);
        else
            dma_one<G::BN, B_MN, G::NW>(idx - NA, d.stage + G::kABytes, d.B, d.ldb, d.n0, d.N, d.k0, d.k_end,
                                        d.wave, d.lane);
    }
}

// Widening of an int8 B tile into the bf16 B layout the fragment reads use
// (k-major: rows of 64 k, chunk c of row r at slot c ^ swz_k(r); n-major:
// k-rows of BN, chunk c of k-row k at slot c ^ swz_mn(k)).  A thread owns
// kPer 16-byte int8 chunks (16 values); widen_load reads them into registers,
// widen_part<P> turns the P-th quarter of their dwords (4 values each) into
// 8-byte bf16 runs, so that the work can ride between a tile's four MFMA
// groups.  n-major k-rows at or past `valid` become zero (a ragged last k-tile
// was loaded from clamped rows).
template <class G>
struct Widen8 {
    static constexpr int kPer = G::BN * BK / 16 / G::kThreads;
    static_assert(kPer >= 1 && (G::BN * BK / 16) % G::kThreads == 0, "widening chunks per thread");
    uint4 w[kPer];
};

template <class G>
__device__ __forceinline__ void widen_load(const unsigned char* __restrict__ src8, int tid, Widen8<G>& r) {
#pragma unroll
    for (int c = 0; c < Widen8<G>::kPer; ++c)
        r.w[c] = *reinterpret_cast<const uint4*>(src8 + (c * G::kThreads + tid) * 16);
}

// 4 int8 values -> 4 bf16 (exact for |v| <= 128), element 0 in the low half.
__device__ __forceinline__ uint2 widen4(uint32_t d) {
    const uint32_t x = d ^ 0x80808080u;
    const float f0 = (float)(x & 0xffu) - 128.f;
    const float f1 = (float)((x >> 8) & 0xffu) - 128.f;
    const float f2 = (float)((x >> 16) & 0xffu) - 128.f;
    const float f3 = (float)(x >> 24) - 128.f;
    return make_uint2(pack_bf16x2(f0, f1), pack_bf16x2(f2, f3));
}

template <class G, bool B_MN, int PART>
__device__ __forceinline__ void widen_part(unsigned char* __restrict__ dst, int valid, int tid, const Widen8<G>& r) {
    constexpr int BN = G::BN;
    constexpr int D = Widen8<G>::kPer * 4;   // dwords per thread
    static_assert(D % 4 == 0, "quarters");
#pragma unroll
    for (int q = PART * D / 4; q < (PART + 1) * D / 4; ++q) {
        const int c = q >> 2, dw = q & 3;
        const int u = c * G::kThreads + tid;
        const uint4& w = r.w[c];
        uint32_t word = dw == 0 ? w.x : dw == 1 ? w.y : dw == 2 ? w.z : w.w;
        // an ordered no-op on the input: the conversion cannot be hoisted
        // above the scheduling barrier of the k-step it belongs to
        asm volatile("" : "+v"(word));
        uint2 v = widen4(word);
        int off;
        if constexpr (!B_MN) {
            const int row = u >> 2, ch = 2 * (u & 3) + (dw >> 1);
            off = row * 128 + ((ch ^ swz_k(row)) << 4) + (dw & 1) * 8;
        } else {
            constexpr int kPerRow = BN / 16;
            const int k = u / kPerRow, ch = 2 * (u % kPerRow) + (dw >> 1);
            if (k >= valid) v = make_uint2(0, 0);
            off = k * (BN * 2) + ((ch ^ swz_mn<BN>(k)) << 4) + (dw & 1) * 8;
        }
        *reinterpret_cast<uint2*>(dst + off) = v;
    }
}

template <class G, bool B_MN>
__device__ __forceinline__ void widen_all(const unsigned char* __restrict__ src8, unsigned char* __restrict__ dst,
                                          int valid, int tid) {
    Widen8<G> r;
    widen_load<G>(src8, tid, r);
    widen_part<G, B_MN, 0>(dst, valid, tid, r);
    widen_part<G, B_MN, 1>(dst, valid, tid, r);
    widen_part<G, B_MN, 2>(dst, valid, tid, r);
    widen_part<G, B_MN, 3>(dst, valid, tid, r);
}

// The k-step ks share of a tile's widening (Q8), after that step's MFMAs.
template <class G, bool B_MN>
__device__ __forceinline__ void widen_step(int ks, unsigned char* __restrict__ dst, int valid, int tid,
                                           const Widen8<G>& r) {
    switch (ks) {
        case 0: widen_part<G, B_MN, 0>(dst, valid, tid, r); break;
        case 1: widen_part<G, B_MN, 1>(dst, valid, tid, r); break;
        case 2: widen_part<G, B_MN, 2>(dst, valid, tid, r); break;
        default: widen_part<G, B_MN, 3>(dst, valid, tid, r); break;
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
// A from stage st, B from bst (the stage's B tile, or the widened buffer for Q8).
template <class G, bool A_MN, bool B_MN>
__device__ __forceinline__ void load_frags(const unsigned char* __restrict__ st, const unsigned char* __restrict__ bst,
                                           int wm, int wn, int ks, int lane, uint4 (&af)[G::MI],
                                           uint4 (&bfr)[G::NJ]) {
#pragma unroll
    for (int i = 0; i < G::MI; ++i) af[i] = load_frag<A_MN, G::BM>(st, wm * G::WTM + i * 32, ks, lane);
#pragma unroll
    for (int j = 0; j < G::NJ; ++j) bfr[j] = load_frag<B_MN, G::BN>(bst, wn * G::WTN + j * 32, ks, lane);
}
template <class G, bool A_MN, bool B_MN>
__device__ __forceinline__ void load_frags(const unsigned char* __restrict__ st, int wm, int wn, int ks, int lane,
                                           uint4 (&af)[G::MI], uint4 (&bfr)[G::NJ]) {
    load_frags<G, A_MN, B_MN>(st, st + G::kABytes, wm, wn, ks, lane, af, bfr);
}

// One k-tile (four k-steps of 16) with register double-buffered fragments:
// the LDS reads of step ks+1 are issued before the MFMAs of step ks, and
// scheduling barriers keep the compiler from sinking them; a quarter of the
// next tile's loads goes out with each k-step.
// The widening of the next k-tile's int8 B operand (Q8), spread over a tile's
// four k-steps (a quarter after each step's MFMAs are issued).
struct WidenJob {
    const unsigned char* src = nullptr;
    unsigned char* dst = nullptr;
    int valid = 0;
    bool on = false;
};

template <class G, bool A_MN, bool B_MN>
__device__ __forceinline__ void compute_tile(const unsigned char* __restrict__ st, const unsigned char* __restrict__ bst,
                                             int wm, int wn, int lane, f32x16_t (&acc)[G::MI][G::NJ],
                                             const DmaJob& next, bool load_next, const WidenJob& wj, int tid) {
    uint4 af[2][G::MI], bfr[2][G::NJ];
    Widen8<G> w8;
    if constexpr (G::Q8)
        if (wj.on) widen_load<G>(wj.src, tid, w8);
    load_frags<G, A_MN, B_MN>(st, bst, wm, wn, 0, lane, af[0], bfr[0]);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
        const int cur = ks & 1;
        if (ks + 1 < BK / 16) load_frags<G, A_MN, B_MN>(st, bst, wm, wn, ks + 1, lane, af[cur ^ 1], bfr[cur ^ 1]);
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
        if constexpr (G::Q8) {
            if (wj.on) widen_step<G, B_MN>(ks, wj.dst, wj.valid, tid, w8);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

template <class G, bool A_MN, bool B_MN>
__device__ __forceinline__ void compute_tile(const unsigned char* __restrict__ st, int wm, int wn, int lane,
                                             f32x16_t (&acc)[G::MI][G::NJ], const DmaJob& next, bool load_next) {
    compute_tile<G, A_MN, B_MN>(st, st + G::kABytes, wm, wn, lane, acc, next, load_next, WidenJob{}, 0);
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

// Grouped launches (PipeArgs::grp) whose groups differ in k: the groups' tiles
// are taken longest k first (ties in table order) and dealt to the XCDs the way
// the hardware deals launch slots, round-robin, so every XCD gets an equal share
// of every group and starts its long tiles first; within an XCD a group's share
// is one contiguous run in the four-M-panel-deep order of single products, so
// the panels it reads stay in that XCD's L2.  With one k for every group the
// whole grid takes the order of a single product (tile_coords).
__device__ __forceinline__ void grp_tile_coords(const PipeArgs& p, int bn, int tiles_m, int tiles_n, int& tm,
                                                int& tn) {
    constexpr int NG = kMaxPipeGroups;
    const int ng = p.ngroups;
    int k[NG], c0[NG], cols[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        k[i] = i < ng ? p.grp[i].k : -1;
        c0[i] = p.grp[i].n_begin / bn;
        int c1 = tiles_n;
        if (i + 1 < NG && i + 1 < ng) c1 = p.grp[i + 1].n_begin / bn;
        cols[i] = i < ng ? c1 - c0[i] : 0;
    }
    bool mixed = false;
#pragma unroll
    for (int i = 1; i < NG; ++i) mixed = mixed || (i < ng && k[i] != k[0]);
    if (!mixed) {
        tile_coords((int)blockIdx.x, tiles_m, tiles_n, tm, tn);
        return;
    }
    const int x = (int)blockIdx.x & 7;   // the XCD this slot is dealt to
    const int u = (int)blockIdx.x;       // position in the longest-k-first deal
    tm = tiles_m;                         // past every group: no tile
    tn = tiles_n;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const int cnt = tiles_m * cols[i];
        int off = 0;   // tiles of the groups dealt before group i
#pragma unroll
        for (int j = 0; j < NG; ++j)
            if (j != i && (k[j] > k[i] || (k[j] == k[i] && j < i))) off += tiles_m * cols[j];
        if (i < ng && u >= off && u < off + cnt) {
            // group i's tiles go to the XCDs in rotated order starting at XCD off % 8
            const int rho = (x - off % 8 + 8) & 7;
            const int u0 = off + rho;                     // first tile of group i dealt to XCD x
            const int start = rho * (cnt >> 3) + min(rho, cnt & 7);
            const int id = start + (u - u0) / 8;          // contiguous per XCD
            constexpr int D = 4;                          // M panels deep
            const int grp = id / (D * cols[i]);
            const int first = grp * D;
            const int gm = min(D, tiles_m - first);
            const int r = id - grp * D * cols[i];
            tm = first + r % gm;
            tn = c0[i] + r / gm;
        }
    }
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

// Wait until at most `jobs` k-tiles of this thread's loads are in flight
// (0 <= jobs <= S - 1): everything issued before them has landed.
template <int LPT, int S>
__device__ __forceinline__ void wait_jobs(int jobs) {
    static_assert(S >= 2 && S <= 8 && LPT * (S - 1) < 64, "vmcnt range");
    switch (jobs) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<LPT>(); break;
        case 2: if constexpr (S > 2) wait_vmcnt<2 * LPT>(); break;
        case 3: if constexpr (S > 3) wait_vmcnt<3 * LPT>(); break;
        case 4: if constexpr (S > 4) wait_vmcnt<4 * LPT>(); break;
        case 5: if constexpr (S > 5) wait_vmcnt<5 * LPT>(); break;
        default: if constexpr (S > 6) wait_vmcnt<6 * LPT>(); break;
    }
}

// S-stage LDS ring: S - 1 k-tiles are requested before the first one is used,
// so a product with K <= 64 (S - 1) waits for memory once.
// Epilogue kinds: plain store, general (see PipeArgs), plain store with the
// output columns scaled by PipeArgs::colscale.
// kEpiFoldR: the R-side block product of the layer forward applied to the tile
// (fold_r_epilogue).
constexpr int kEpiPlain = 0, kEpiGeneral = 1, kEpiColScale = 2, kEpiFoldR = 3;

// The k loop of one output tile at (m0, n0) into acc (zeroed here).
// Q8 (G::Q8): B is int8.  Job t loads A(t) into stage t % S and the int8 B of
// tile t + 1 into the int8 area of stage (t + 1) % S (that area's previous
// tile was widened before tile t began); tile t widens the int8 B of tile t + 1
// into the bf16 buffer (t + 1) & 1 while it computes from buffer t & 1, and the
// barrier that opens tile t + 1 publishes it.  The int8 B of tile 0 is loaded
// and widened before the loop.  Past the last tile, job nk - 1 loads a clamped,
// unused int8 tile, so that every job issues the same loads and the vmcnt
// arithmetic stays exact.
template <class G, bool A_MN, bool B_MN, int S>
__device__ __forceinline__ void main_loop(unsigned char* lds, const uint16_t* __restrict__ A, int64_t lda,
                                          const uint16_t* __restrict__ B, int64_t ldb, int m0, int n0, int M, int N,
                                          int kb, int ke, int tid, f32x16_t (&acc)[G::MI][G::NJ],
                                          bool zero = true) {
    constexpr int BM = G::BM, BN = G::BN;
    constexpr int kABytes = G::kABytes, kStageBytes = G::kStageBytes;
    constexpr int kLoadsPerTile = G::kLoadsPerTile;
    const int lane = tid & 63;
    // the wave index is uniform: held in a scalar register, the LDS destinations
    // of the loads (M0) are formed without per-lane arithmetic
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / G::NWN, wn = wave % G::NWN;
    const int nk = ke > kb ? (ke - kb + BK - 1) / BK : 0;
    const uint32_t base = lds_offset(lds);
    unsigned char* const bbf = lds + S * kStageBytes;   // Q8: widened B, two tiles
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
    if constexpr (kSaddr<G, A_MN>) {
        constexpr int NA = OperandLoads<BM, A_MN, G::NW>::n;
        constexpr int NB = G::Q8 ? OperandLoads8<BN, G::NW>::n : OperandLoads<BN, B_MN, G::NW>::n;
#pragma unroll
        for (int j = 0; j < NA; ++j) job.voff[j] = dma_voff<BM, false, G::NW>(j, lda, m0, M, wave, lane);
#pragma unroll
        for (int j = 0; j < NB; ++j)
            job.voff[NA + j] = G::Q8 ? dma_voff8<BN, B_MN, G::NW>(j, ldb, n0, N, wave, lane)
                                     : dma_voff<BN, B_MN, G::NW>(j, ldb, n0, N, wave, lane);
    }
    // the uniform bases of job k0 (SADDR)
    auto set_bases = [&]() {
        if constexpr (kSaddr<G, A_MN>) {
            job.a_k = reinterpret_cast<const char*>(A) + 2 * (int64_t)job.k0;
            if constexpr (G::Q8)   // int8 B of tile k0_b
                job.b_k = reinterpret_cast<const char*>(B) + (B_MN ? (int64_t)job.k0_b * ldb : (int64_t)job.k0_b);
            else
                job.b_k = reinterpret_cast<const char*>(B) + 2 * (B_MN ? (int64_t)job.k0 * ldb : (int64_t)job.k0);
        }
    };
    // Q8: where job t puts the int8 B of tile t + 1, and its k (a tile past K
    // is clamped to the last one; K is whole 64-k tiles)
    auto set_b8 = [&](int t, int stage_of_t) {
        if constexpr (G::Q8) {
            const int sb = stage_of_t == S - 1 ? 0 : stage_of_t + 1;
            job.stage_b = base + sb * kStageBytes + kABytes;
            job.k0_b = min(kb + (t + 1) * BK, ke - BK);
        }
    };
    if constexpr (G::Q8) {
        // the int8 B of tile 0, ahead of every job
        DmaJob j0 = job;
        j0.stage_b = base + kABytes;
        j0.k0_b = kb;
        constexpr int NA = OperandLoads<BM, A_MN, G::NW>::n, NB = OperandLoads8<BN, G::NW>::n;
#pragma unroll
        for (int j = 0; j < NB; ++j)
            dma_one8<BN, B_MN, G::NW>(j, j0.stage_b, reinterpret_cast<const int8_t*>(B), ldb, n0, N, kb, ke, wave,
                                      lane);
        (void)NA;
    }
#pragma unroll
    for (int t = 0; t < S - 1; ++t) {
        if (t < nk) {
            job.stage = base + t * kStageBytes;
            job.k0 = kb + t * BK;
            set_b8(t, t);
            set_bases();
            dma_tile<G, A_MN, B_MN>(job);
        }
    }
    if constexpr (G::Q8) {
        // tile 0's int8 B landed (only the jobs may still be in flight) for every
        // thread: widen it into buffer 0
        wait_jobs<kLoadsPerTile, S>(min(S - 1, nk));
        block_barrier();
        widen_all<G, B_MN>(lds + kABytes, bbf, ke - kb, tid);
    }
    // Tile kt becomes readable once this thread's loads of it are done (at most
    // those of the tiles after it, up to kt + S - 2, remain) and every wave has
    // passed the barrier; a ragged last m/n-major tile then gets its rows past K
    // zeroed (they were loaded from clamped rows; Q8 B tiles are zeroed when widened).
    // pending: this thread's k-tiles of loads that may stay in flight, S - 2 in
    // the steady part of the loop (a constant the wait folds to one s_waitcnt)
    auto enter = [&](int kt, int stage, int pending) {
        wait_tiles<kLoadsPerTile, S>(pending);
        // Q8: the widening's LDS writes (read by other waves past the barrier)
        // and this wave's reads of the widened buffer the next tile rewrites
        // must be done: a barrier does not wait for LDS operations
        if constexpr (G::Q8) wait_lgkm0();
        block_barrier();
        // a k-major A means whole 64-k tiles (no ragged tile); Q8 B tiles are
        // zeroed when widened
        constexpr bool zb = B_MN && A_MN;
        if constexpr (A_MN || zb) {
            const int valid = ke - (kb + kt * BK);
            if (valid < BK) {
                if constexpr (A_MN) zero_rows_mn<BM, G::kThreads>(lds + stage * kStageBytes, valid, tid);
                if constexpr (zb) zero_rows_mn<BN, G::kThreads>(lds + stage * kStageBytes + kABytes, valid, tid);
                __syncthreads();
            }
        }
    };
    // the B tile that tile kt reads, and the widening tile kt does for tile kt + 1
    auto b_tile = [&](int kt, int stage) -> const unsigned char* {
        if constexpr (G::Q8) return bbf + (kt & 1) * G::kBBytes;
        else return lds + stage * kStageBytes + kABytes;
    };
    auto widen_job = [&](int kt, int stage) {
        WidenJob w;
        if constexpr (G::Q8) {
            const int sn = stage == S - 1 ? 0 : stage + 1;
            w.src = lds + sn * kStageBytes + kABytes;
            w.dst = bbf + ((kt + 1) & 1) * G::kBBytes;
            w.valid = ke - (kb + (kt + 1) * BK);
            w.on = kt + 1 < nk;
        }
        return w;
    };
    int st = 0;            // stage of tile kt
    int st_load = S - 1;   // stage that receives tile kt + S - 1
    // 256 x 128 tiles (three stages: tile kt + 1 was requested a whole tile
    // ago) hand over to tile kt + 1 (wait, barrier, its first fragments) before
    // the last k-step's MFMAs of tile kt, which then cover the barrier and the
    // first LDS reads of the next tile; the same barrier frees tile kt's stage,
    // as every wave holds tile kt's last fragments in registers by then.  Other
    // tiles hand over at the top of each tile.
    // The loop runs in two parts: a steady one, where every tile issues the
    // loads of tile kt + S - 1 and waits with a fixed count, and the last
    // S - 1 tiles, which issue none and wait for what is left.
    if constexpr (!(S >= 3 && BM == 256 && BN == 128)) {
        auto tile = [&](int kt, auto steady_c) {
            constexpr bool STEADY = decltype(steady_c)::value;
            enter(kt, st, STEADY ? S - 2 : min(nk, kt + S - 1) - kt - 1);
            job.stage = base + st_load * kStageBytes;
            job.k0 = kb + (kt + S - 1) * BK;
            set_b8(kt + S - 1, st_load);
            set_bases();
            WidenJob wj = widen_job(kt, st);
            if constexpr (STEADY && G::Q8) wj.on = true;
            compute_tile<G, A_MN, B_MN>(lds + st * kStageBytes, b_tile(kt, st), wm, wn, lane, acc, job,
                                        STEADY || kt + S - 1 < nk, wj, tid);
            st = st == S - 1 ? 0 : st + 1;
            st_load = st_load == S - 1 ? 0 : st_load + 1;
        };
        int kt = 0;
        for (; kt + S - 1 < nk; ++kt) tile(kt, std::true_type{});
        for (; kt < nk; ++kt) tile(kt, std::false_type{});
        return;
    }
    uint4 af[2][G::MI], bfr[2][G::NJ];
    enter(0, 0, min(nk, S - 1) - 1);
    load_frags<G, A_MN, B_MN>(lds, b_tile(0, 0), wm, wn, 0, lane, af[0], bfr[0]);
    // steady: tile kt + S - 1 exists (so does tile kt + 1, and kt + S <= nk)
    auto tile = [&](int kt, auto steady_c) {
        constexpr bool STEADY = decltype(steady_c)::value;
        job.stage = base + st_load * kStageBytes;
        job.k0 = kb + (kt + S - 1) * BK;
        set_b8(kt + S - 1, st_load);
        set_bases();
        const bool load_next = STEADY || kt + S - 1 < nk;
        const bool has_next = STEADY || kt + 1 < nk;
        const unsigned char* cur_st = lds + st * kStageBytes;
        const unsigned char* cur_b = b_tile(kt, st);
        const int st_next = st == S - 1 ? 0 : st + 1;
        WidenJob wj = widen_job(kt, st);
        if constexpr (STEADY && G::Q8) wj.on = true;
        Widen8<G> w8;
        if constexpr (G::Q8)
            if (wj.on) widen_load<G>(wj.src, tid, w8);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int cur = ks & 1;
            if (ks + 1 < BK / 16)
                load_frags<G, A_MN, B_MN>(cur_st, cur_b, wm, wn, ks + 1, lane, af[cur ^ 1], bfr[cur ^ 1]);
            if (load_next) {
                switch (ks) {
                    case 0: dma_part<G, A_MN, B_MN, 0, 4>(job); break;
                    case 1: dma_part<G, A_MN, B_MN, 1, 4>(job); break;
                    case 2: dma_part<G, A_MN, B_MN, 2, 4>(job); break;
                    default: dma_part<G, A_MN, B_MN, 3, 4>(job); break;
                }
            }
            if (ks == BK / 16 - 1 && has_next) {
                enter(kt + 1, st_next, STEADY ? S - 2 : min(nk, kt + S) - kt - 2);
                load_frags<G, A_MN, B_MN>(lds + st_next * kStageBytes, b_tile(kt + 1, st_next), wm, wn, 0, lane,
                                          af[cur ^ 1], bfr[cur ^ 1]);
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
            if constexpr (G::Q8) {
                // every quarter must land before the barrier that opens tile
                // kt + 1 (taken at the last k-step, before its MFMAs): the
                // third k-step does the last two quarters
                if (wj.on && ks < BK / 16 - 1) widen_step<G, B_MN>(ks, wj.dst, wj.valid, tid, w8);
                if (wj.on && ks == BK / 16 - 2) widen_step<G, B_MN>(ks + 1, wj.dst, wj.valid, tid, w8);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        st = st_next;
        st_load = st_load == S - 1 ? 0 : st_load + 1;
    };
    int kt = 0;
    for (; kt + S - 1 < nk; ++kt) tile(kt, std::true_type{});
    for (; kt < nk; ++kt) tile(kt, std::false_type{});
}

// The R-side block product of the layer forward, folded into the dense
// product's epilogue: a 128 x 256 tile of h2 = h1 Wt^T is one token tile of one
// R block (b = 256), so z = h2 G_j^T for that tile needs only G_j (b x b,
// k-major rows).  h2 is rounded to bf16 as the unfused chain stores it (for an
// int8 weight after its column scale), stored when the caller keeps it (C2),
// and kept in LDS as four k-major 128 x 64 A tiles; G_j streams through a
// three-stage ring of 256 x 64 tiles behind it.  The second product runs the
// tiles, k-steps and MFMAs of the 128 x 256 block product in the same order,
// so z equals the unfused chain's bit for bit.
template <class G>
__device__ __forceinline__ void fold_r_epilogue(const PipeArgs& p, f32x16_t (&acc)[G::MI][G::NJ],
                                                unsigned char* lds, int m0, int n0, int tid, const float (&csc)[G::NJ]) {
    static_assert(G::BM == 128 && G::BN == 256 && G::NWM == 2 && G::NWN == 4, "fold tile");
    constexpr int MI = G::MI, NJ = G::NJ, WTM = G::WTM, WTN = G::WTN;
    constexpr int kATile = 128 * BK * 2;        // 16 KB: h2 columns [64 kt, 64 kt + 64)
    constexpr int kPanel = 4 * kATile;          // the tile's h2, 64 KB
    constexpr int kBTile = 256 * BK * 2;        // 32 KB: one k-tile of G_j
    constexpr int kRing = 3;
    static_assert(kPanel + kRing * kBTile <= 160 * 1024, "fold LDS");
    constexpr int NB = OperandLoads<256, false, G::NW>::n;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / G::NWN, wn = wave % G::NWN;
    const uint32_t base = lds_offset(lds);
    const uint16_t* Gj = reinterpret_cast<const uint16_t*>(p.Gfold) + (int64_t)(n0 / 256) * (256 * 256);
    auto load_g = [&](int kt, int stage) {
#pragma unroll
        for (int j = 0; j < NB; ++j)
            dma_one<256, false, G::NW>(j, base + kPanel + stage * kBTile, Gj, 256, 0, 256, kt * BK, 256, wave, lane);
    };
    block_barrier();   // every wave is done reading the operand stages
#pragma unroll
    for (int kt = 0; kt < kRing; ++kt) load_g(kt, kt);
    // h2 in bf16: stored (C2) and staged; element (row, col) of the tile goes to
    // A tile col / 64, row `row`, k = col % 64 (the k-major swizzle of the ring)
    bf16_t* C2 = reinterpret_cast<bf16_t*>(p.C2);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * WTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                const int col = wn * WTN + j * 32 + (lane & 31);
                const bf16_t h = ElemTraits<bf16_t>::from_f32(G::Q8 ? acc[i][j][r] * csc[j] : acc[i][j][r]);
                if (C2 && m0 + row < p.M) C2[(int64_t)(m0 + row) * p.ldc2 + n0 + col] = h;
                const int kk = col & 63;
                *reinterpret_cast<bf16_t*>(lds + (col >> 6) * kATile + row * 128 +
                                           (((kk >> 3) ^ swz_k(row)) << 4) + (kk & 7) * 2) = h;
            }
    f32x16_t z[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) z[i][j][r] = 0.f;
    wait_vmcnt<0>();
    __syncthreads();   // the h2 panel and G's first three k-tiles are in LDS
    auto compute = [&](int kt, int stage) {
        const unsigned char* at = lds + kt * kATile;
        const unsigned char* bt = lds + kPanel + stage * kBTile;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            uint4 af[MI], bfr[NJ];
            load_frags<G, false, false>(at, bt, wm, wn, ks, lane, af, bfr);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) Mfma32<bf16_t>::run(af[i], bfr[j], z[i][j]);
        }
    };
    compute(0, 0);
    __syncthreads();   // stage 0 is free
    load_g(3, 0);
    compute(1, 1);
    compute(2, 2);
    wait_vmcnt<0>();
    __syncthreads();
    compute(3, 0);
    bf16_t* C = reinterpret_cast<bf16_t*>(p.C);
    const int col0 = n0 + wn * WTN + (lane & 31);
    const int row0 = m0 + wm * WTM + (lane >> 5) * 4;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = row0 + i * 32 + (r >> 2) * 8 + (r & 3);
                if (row < p.M) store_f32(C + (int64_t)row * p.ldc + col0 + j * 32, z[i][j][r]);
            }
}

// DUAL = 1: acc = op(A) op(B) + A2^T B2 (second product with m/n-major A2, B2);
// DUAL = 2: the second product goes to its own accumulator (general epilogue mode 2).
// GRP: a grouped product (PipeArgs::grp), a separate instantiation so that the
// plain kernels carry no group lookup.
// Q8: B is int8 (the quantized weight), see main_loop.
template <int BM, int BN, bool A_MN, bool B_MN, bool OUT_F32, int EPI, int S, int NWM = 2, int NWN = 2, int DUAL = 0,
          bool GRP = false, bool Q8 = false>
__global__ void __launch_bounds__(64 * NWM * NWN)
__attribute__((amdgpu_waves_per_eu(PipeWaves<BM, BN, NWM * NWN>::lo, PipeWaves<BM, BN, NWM * NWN>::hi)))
pipe_gemm_kernel(const PipeArgs p) {
    using G = Geo<BM, BN, NWM, NWN, Q8>;
    constexpr int kStageBytes = G::kStageBytes;
    constexpr int MI = G::MI, NJ = G::NJ, WTM = G::WTM, WTN = G::WTN;
    static_assert(S * kStageBytes + G::kExtraBytes <= 160 * 1024, "LDS ring exceeds 160 KB");
    static_assert(!Q8 || (!A_MN && DUAL == 0 && EPI != kEpiGeneral), "int8 B: k-major A, single product");
    static_assert(EPI != kEpiFoldR || (!A_MN && !B_MN && !OUT_F32 && DUAL == 0 && !GRP), "fold: the NT forward");
    constexpr int kLds = EPI == kEpiFoldR ? 160 * 1024 : S * kStageBytes + G::kExtraBytes;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kLds];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / NWN, wn = wave % NWN;
    const int M = p.M, N = p.N;
    const int kb = blockIdx.z * p.k_per_split;
    int ke = min(p.K, kb + p.k_per_split);
    int tm, tn;
    int z;
    if constexpr (GRP) {
        z = 0;
        grp_tile_coords(p, BN, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
        if (tm * BM >= M || tn * BN >= N) return;
    } else {
        batch_tile_coords((M + BM - 1) / BM, (N + BN - 1) / BN, z, tm, tn);
    }
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
    // column scales of this lane's NJ columns (kEpiColScale, or the fold on an
    // int8 weight), 1 otherwise
    float csc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        if constexpr (EPI == kEpiColScale || (EPI == kEpiFoldR && Q8)) {
            const float* sc = p.colscale + (int64_t)z * p.strideScale;
            csc[j] = col0 + j * 32 < N ? sc[col0 + j * 32] : 0.f;
        } else {
            csc[j] = 1.f;
        }
    }
    if constexpr (EPI == kEpiFoldR) {
        fold_r_epilogue<G>(p, acc, lds, m0, n0, tid, csc);
        return;
    }
    if (m0 + BM <= M && n0 + BN <= N) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float v = EPI == kEpiColScale ? acc[i][j][r] * csc[j] : acc[i][j][r];
                    store_f32(C + (int64_t)(row0 + i * 32 + (r >> 2) * 8 + (r & 3)) * p.ldc + col0 + j * 32, v);
                }
    } else {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int col = col0 + j * 32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = row0 + i * 32 + (r >> 2) * 8 + (r & 3);
                    const float v = EPI == kEpiColScale ? acc[i][j][r] * csc[j] : acc[i][j][r];
                    if (row < M && col < N) store_f32(C + (int64_t)row * p.ldc + col, v);
                }
            }
    }
}

// Tile pair (ti, tj), ti <= tj, of nt x nt tiles and batch entry z of this
// workgroup (grid: pairs of a block along x, blocks along y).  Launch slots are
// dealt round-robin to the 8 XCDs, so slot ids are regrouped to give each XCD
// a contiguous run of work: whole blocks, whose operands are then fetched into
// one L2 only (dealt as they come, the pairs of one block spread over several
// XCDs and each of their L2s fetched the block again).
__device__ __forceinline__ void pair_of(int nt, int& ti, int& tj, int& z) {
    const int pairs = (int)gridDim.x;
    const int total = pairs * (int)gridDim.y;
    int id = (int)blockIdx.x + pairs * (int)blockIdx.y;
    if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);
    z = id / pairs;
    int i = 0, t = id - z * pairs;
    while (t >= nt - i) {
        t -= nt - i;
        ++i;
    }
    ti = i;
    tj = i + t;
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

// The work units of one block of nt x nt 64 x 64 tiles for the k = 3 passes:
// the nt (nt - 1) / 2 mirrored pairs (I, J), I < J, one tile per group of four
// waves, then the diagonal tiles two at a time, one per group (diag; a lone
// last one when nt is odd is computed by both groups and kept by group 0), so
// that every unit carries two tiles of work.
__host__ __device__ constexpr int units_per_block(int nt) { return nt * (nt - 1) / 2 + (nt + 1) / 2; }

__device__ __forceinline__ void unit_of(int nt, int& ti, int& tj, int& z, bool& diag) {
    const int units = (int)gridDim.x;
    const int total = units * (int)gridDim.y;
    int id = (int)blockIdx.x + units * (int)blockIdx.y;
    if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);   // each XCD gets whole blocks
    z = id / units;
    int t = id - z * units;
    const int npairs = nt * (nt - 1) / 2;
    diag = t >= npairs;
    if (diag) {
        ti = 2 * (t - npairs);
        tj = min(ti + 1, nt - 1);
        return;
    }
    int i = 0;
    while (t >= nt - 1 - i) {
        t -= nt - 1 - i;
        ++i;
    }
    ti = i;
    tj = i + 1 + t;
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
    int ti, tj, z;
    pair_of(b / 64, ti, tj, z);
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

// ------------------------------------------- Cayley-Neumann backward, k = 3
// G = (I + T)(I + S) with S = Q Q (symmetric) and T = 2Q + S.  The pack keeps
// only the skew part of dQ, dq[idx(r, c)] = dQ[r][c] - dQ[c][r], and with
//   X1 = dG S,  X2 = T^T dG,  dA = dG + X1,  dS = 2 dG + X1 + X2,
//   Sigma = dS + dS^T (symmetric),  P = Sigma Q
// that part is 2 (dA - dA^T) - (P - P^T): Q Sigma = -(Sigma Q)^T for a skew Q
// and a symmetric Sigma, so the two products dS Q^T and Q^T dS of the full dQ
// become the one product P.  Two passes over units of two 64 x 64 tiles, one
// per group of four waves (unit_of): a mirrored pair (I, J) and (J, I), I < J,
// or two diagonal tiles, each its own mirror:
//   pass 1 (cnp_bwd_sym_kernel): X1 and X2 of both tiles; writes Sigma (bf16,
//     both tiles) and dq[idx(r, c)] = 2 (dA[r][c] - dA[c][r]) for the unit's
//     upper-triangle entries;
//   pass 2 (cnp_bwd_sigq_kernel): -P = Sigma Q^T of both tiles (Q^T = -Q);
//     dq[idx(r, c)] += P[c][r] - P[r][c], in place (each entry has one owner).

// A 64 x 64 float32 tile in LDS, element (r, c) at r * 64 + (c ^ 4 ((r >> 2) & 15)):
// four consecutive columns of a row stay one 16-byte access, and a column read
// by 64 lanes (16 groups of four columns x four rows) meets 64 different banks.
__device__ __forceinline__ int t64(int r, int c) { return r * 64 + (c ^ (((r >> 2) & 15) << 2)); }

// Accumulator of a 2 x 2-wave 64 x 64 tile into a t64 tile (lane holds rows
// 8 (r/4) + 4 (lane/32) + r%4 of column lane%32 of its 32 x 32 wave tile).
__device__ __forceinline__ void stage_acc(float* __restrict__ tile, const f32x16_t& acc, int wm, int wn, int lane) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = wm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int col = wn * 32 + (lane & 31);
        tile[t64(row, col)] = acc[r];
    }
}

template <int S>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(1, 4)))
cnp_bwd_sym_kernel(const PipeArgs p, float* __restrict__ dq, uint16_t* __restrict__ sig, int b) {
    using G = Geo<64, 64, 2, 2>;
    constexpr int kRing = S * G::kStageBytes;
    static_assert(2 * 64 * 64 * 4 <= kRing, "two staged tiles exceed a group's ring");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * kRing];
    const int tid = threadIdx.x, grp = tid >> 8, gtid = tid & 255;
    const int lane = tid & 63, w4 = (tid >> 6) & 3;
    const int wm = w4 >> 1, wn = w4 & 1;
    int ti, tj, z;
    bool diag;
    unit_of(b / 64, ti, tj, z, diag);
    // pair: group 0 tile (ti, tj), group 1 tile (tj, ti); diagonal unit: group 0
    // tile (ti, ti), group 1 tile (tj, tj)
    const int m0 = 64 * (grp ? tj : ti), n0 = diag ? m0 : 64 * (grp ? ti : tj);
    const bool keep = !(diag && ti == tj && grp == 1);   // a lone diagonal tile: group 0's
    const int64_t bb = (int64_t)b * b;
    // X1 = dG S: A = dG rows (k-major), B = S rows (S = S^T); X2 = T^T dG:
    // A2 = T ([K][M], m-major), B2 = dG ([K][N], n-major).  S and T come by DMA;
    // dG's tiles come from its float32 copy (Cin1) through registers, rounded to
    // bf16 into the stage (the rounding the bf16 copy of dG would get).
    const uint16_t* B = reinterpret_cast<const uint16_t*>(p.B) + z * bb;
    const uint16_t* A2 = reinterpret_cast<const uint16_t*>(p.A2) + z * bb;
    const float* dGz = p.Cin1 + z * p.strideCin1;
    unsigned char* ring = lds + grp * kRing;
    const uint32_t rbase = lds_offset(ring);
    const int gw = __builtin_amdgcn_readfirstlane(w4);   // wave within the group
    constexpr int NB = OperandLoads<64, false, G::NW>::n;   // DMA loads of a 64 x 64 tile per thread
    static_assert(NB == OperandLoads<64, true, G::NW>::n, "tile loads");
    const int nk = b / 64;
    // 16 consecutive floats of dG row `row` at column `col` (this thread's part
    // of a 64 x 64 tile: row gtid / 4, columns 16 (gtid % 4) ..)
    float4 st[4];
    auto load_dg = [&](int row, int col) __attribute__((always_inline)) {
        const float4* src = reinterpret_cast<const float4*>(dGz + (int64_t)row * b + col);
#pragma unroll
        for (int i = 0; i < 4; ++i) st[i] = src[i];
    };
    // ... as two 16-byte chunks of row gtid / 4 of a 128-byte-row image whose
    // chunk c sits in slot c ^ swz(row)
    auto put_dg = [&](unsigned char* img, int swz) __attribute__((always_inline)) {
        const int r = gtid >> 2, sg = gtid & 3;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float4 u = st[2 * h], v = st[2 * h + 1];
            *reinterpret_cast<uint4*>(img + r * 128 + (((2 * sg + h) ^ swz) << 4)) =
                make_uint4(pack_bf16x2(u.x, u.y), pack_bf16x2(u.z, u.w), pack_bf16x2(v.x, v.y),
                           pack_bf16x2(v.z, v.w));
        }
    };
    auto compute = [&](auto amn_c, auto bmn_c, const unsigned char* stage, f32x16_t& acc)
                       __attribute__((always_inline)) {
        constexpr bool AMN = decltype(amn_c)::value, BMN = decltype(bmn_c)::value;
        uint4 af[2][1], bfr[2][1];
        load_frags<G, AMN, BMN>(stage, wm, wn, 0, lane, af[0], bfr[0]);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int cur = ks & 1;
            if (ks + 1 < BK / 16) load_frags<G, AMN, BMN>(stage, wm, wn, ks + 1, lane, af[cur ^ 1], bfr[cur ^ 1]);
            asm volatile("" ::: "memory");
            Mfma32<bf16_t>::run(af[cur][0], bfr[cur][0], acc);
        }
    };
    // One product over the nk k-tiles in a two-stage ring: the dG tile through
    // registers (its loads issued before the DMA of the other operand, so a wait
    // for them leaves the DMA in flight), tile kt + 1 into the stage tile kt - 1
    // used once every wave has passed the barrier that opens tile kt.
    // X1: dG rows m0.. as the k-major A, S rows n0.. as the k-major B
    // X2: T rows (columns m0..) as the m-major A, dG rows (columns n0..) as the n-major B
    // Both products start from dG's float32 values of the group's tile (the lane's
    // accumulator entries, loaded straight into the accumulators): X1's gives
    // dA = dG + X1, and the two together dS = 2 dG + X1 + X2.
    auto product = [&](auto x2_c, f32x16_t& acc) __attribute__((always_inline)) {
        constexpr bool X2 = decltype(x2_c)::value;
        {
            const float* t0 = dGz + (int64_t)(m0 + wm * 32 + 4 * (lane >> 5)) * b + n0 + wn * 32 + (lane & 31);
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[q] = t0[(8 * (q >> 2) + (q & 3)) * b];
        }
        const int r = gtid >> 2, c16 = 16 * (gtid & 3);
        auto issue = [&](int kt) __attribute__((always_inline)) {
            const uint32_t dst = rbase + (kt & 1) * G::kStageBytes;
            if constexpr (!X2) {
                load_dg(m0 + r, 64 * kt + c16);
#pragma unroll
                for (int j = 0; j < NB; ++j) dma_one<64, false, G::NW>(j, dst + G::kABytes, B, b, n0, b, 64 * kt, b, gw, lane);
            } else {
                load_dg(64 * kt + r, n0 + c16);
#pragma unroll
                for (int j = 0; j < NB; ++j) dma_one<64, true, G::NW>(j, dst, A2, b, m0, b, 64 * kt, b, gw, lane);
            }
        };
        auto put = [&](int kt) __attribute__((always_inline)) {
            unsigned char* stage = ring + (kt & 1) * G::kStageBytes;
            if constexpr (!X2) put_dg(stage, swz_k(r));
            else put_dg(stage + G::kABytes, swz_mn<64>(r));
        };
        issue(0);
        wait_vmcnt<NB>();
        put(0);
#pragma unroll 1
        for (int kt = 0; kt < nk; ++kt) {
            wait_vmcnt<0>();
            wait_lgkm0();
            block_barrier();   // tile kt complete in every wave
            if (kt + 1 < nk) issue(kt + 1);
            compute(std::integral_constant<bool, X2>{}, std::integral_constant<bool, X2>{},
                    ring + (kt & 1) * G::kStageBytes, acc);
            if (kt + 1 < nk) {
                wait_vmcnt<NB>();
                put(kt + 1);
            }
        }
    };
    f32x16_t x1[1][1], x2[1][1];
    product(std::false_type{}, x1[0][0]);
    block_barrier();   // the second product reuses the LDS ring
    product(std::true_type{}, x2[0][0]);
    block_barrier();   // every wave is done reading the operand stages
    float* E = reinterpret_cast<float*>(ring);   // 2 dG + X1 + X2 (= dS)
    float* F = E + 64 * 64;                      // dG + X1 (= dA)
    {
        f32x16_t e = x1[0][0] + x2[0][0];
        stage_acc(E, e, wm, wn, lane);
        stage_acc(F, x1[0][0], wm, wn, lane);
    }
    __syncthreads();
    const float* E0 = reinterpret_cast<const float*>(lds);
    const float* F0 = E0 + 64 * 64;
    const float* E1 = reinterpret_cast<const float*>(lds + kRing);
    const float* F1 = E1 + 64 * 64;
    // Sigma of this group's tile: Sigma[r][c] = dS[r][c] + dS[c][r], the
    // transposed entries from the mirrored tile (the own tile on the diagonal)
    if (keep) {
        const float* Eo = grp ? E1 : E0;
        const float* Ex = diag ? Eo : (grp ? E0 : E1);
        uint16_t* sz = sig + z * bb;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int u = k * 256 + gtid;
            const int row = u >> 4, c = (u & 15) * 4;
            const float4 v = *reinterpret_cast<const float4*>(Eo + t64(row, c));
            const float s0 = v.x + Ex[t64(c, row)], s1 = v.y + Ex[t64(c + 1, row)];
            const float s2 = v.z + Ex[t64(c + 2, row)], s3 = v.w + Ex[t64(c + 3, row)];
            *reinterpret_cast<uint2*>(sz + (int64_t)(m0 + row) * b + n0 + c) =
                make_uint2(pack_bf16x2(s0, s1), pack_bf16x2(s2, s3));
        }
    }
    // dq = 2 (dA - dA^T) on the unit's upper-triangle entries
    float* out = dq + (int64_t)z * ((int64_t)b * (b - 1) / 2);
    if (!diag) {
#pragma unroll
        for (int k = 0; k < 64 * 64 / 512; ++k) {
            const int u = k * 512 + tid;
            const int rl = u >> 6, cl = u & 63;
            out[upper_index(64 * ti + rl, 64 * tj + cl, b)] = 2.f * (F0[t64(rl, cl)] - F1[t64(cl, rl)]);
        }
    } else if (keep) {
        const float* Fo = grp ? F1 : F0;
#pragma unroll
        for (int k = 0; k < 64 * 64 / 256; ++k) {
            const int u = k * 256 + gtid;
            const int rl = u >> 6, cl = u & 63;
            if (rl < cl) out[upper_index(m0 + rl, m0 + cl, b)] = 2.f * (Fo[t64(rl, cl)] - Fo[t64(cl, rl)]);
        }
    }
}

template <int S>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(1, 4)))
cnp_bwd_sigq_kernel(const PipeArgs p, float* __restrict__ dq, int b) {
    using G = Geo<64, 64, 2, 2>;
    constexpr int kRing = S * G::kStageBytes;
    static_assert(64 * 64 * 4 <= kRing, "staged tile exceeds a group's ring");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * kRing];
    const int tid = threadIdx.x, grp = tid >> 8, gtid = tid & 255;
    const int lane = tid & 63, w4 = (tid >> 6) & 3;
    const int wm = w4 >> 1, wn = w4 & 1;
    int ti, tj, z;
    bool diag;
    unit_of(b / 64, ti, tj, z, diag);
    const int m0 = 64 * (grp ? tj : ti), n0 = diag ? m0 : 64 * (grp ? ti : tj);
    const bool keep = !(diag && ti == tj && grp == 1);
    const int64_t bb = (int64_t)b * b;
    // A = Sigma (bf16, symmetric), B = Q (rows of Q as [N][K]): acc = Sigma Q^T = -P
    const uint16_t* A = reinterpret_cast<const uint16_t*>(p.A) + z * bb;
    const uint16_t* B = reinterpret_cast<const uint16_t*>(p.B) + z * bb;
    unsigned char* ring = lds + grp * kRing;
    // the partial dq this pass adds to, read before the main loop (its latency
    // hides behind the products); every thread owns fixed entries: the whole
    // workgroup a pair's tile (ti, tj), each group its own diagonal tile
    float* out = dq + (int64_t)z * ((int64_t)b * (b - 1) / 2);
    constexpr int kPer = 64 * 64 / 256;
    auto entry = [&](int k, int& rl, int& cl) -> bool {
        if (!diag) {
            const int u = k * 512 + tid;
            rl = u >> 6, cl = u & 63;
            return k < 64 * 64 / 512;
        }
        const int u = k * 256 + gtid;
        rl = u >> 6, cl = u & 63;
        return keep && rl < cl;
    };
    const int r0 = diag ? m0 : 64 * ti, c0 = diag ? m0 : 64 * tj;
    float part[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        int rl, cl;
        part[k] = entry(k, rl, cl) ? out[upper_index(r0 + rl, c0 + cl, b)] : 0.f;
    }
    f32x16_t acc[1][1];
    main_loop<G, false, false, S>(ring, A, b, B, b, m0, n0, b, b, 0, b, gtid, acc);
    block_barrier();   // every wave is done reading the operand stages
    stage_acc(reinterpret_cast<float*>(ring), acc[0][0], wm, wn, lane);
    __syncthreads();
    // -P[r][c] + P[c][r] = acc(I, J)[rl][cl] - acc(J, I)[cl][rl] (a diagonal
    // tile: its own transposed entries)
    const float* N0 = reinterpret_cast<const float*>(diag ? ring : lds);
    const float* N1 = reinterpret_cast<const float*>(diag ? ring : lds + kRing);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        int rl, cl;
        if (entry(k, rl, cl)) out[upper_index(r0 + rl, c0 + cl, b)] = part[k] + (N0[t64(rl, cl)] - N1[t64(cl, rl)]);
    }
}

// The k = 3 backward of one b = 256 block per workgroup (large batches): the
// same algebra as the two pair passes, with every intermediate kept on chip.
// With X1 = dG S, X2 = T^T dG, dS = 2 dG + X1 + X2, Sigma = dS + dS^T, P = Sigma Q
// and dA = dG + X1, the packed dq is E - E^T on the upper triangle for
// E = 2 dA - P = 2 dG + 2 X1 - P.  Eight waves, wave (wm, wn) owning rows
// [64 wm, 64 wm + 64) and columns [128 wn, 128 wn + 128) of the block, share one
// set of accumulators (two waves per SIMD leave 256 registers a lane, room for
// one 64 x 128 float32 set and the operands).  The float32 leading terms enter
// as the accumulators' starting value, loaded straight from dG, and the
// products carry halved operands, so that no phase adds dG element by element
// (halving is exact in bf16 and float32):
//   A. acc = dG + (dG / 2) S + T^T (dG / 2) = dS / 2, doubled: dS;
//   B. dS to LDS in bf16, each lane adds the transposed entries of its own:
//      Sigma (the transposed half rounded to bf16 twice, there and in Sigma);
//      Sigma / 2, symmetric, goes back as the m-major A image of phase C;
//   C. acc = dG + (Sigma / 2) Q^T = dG - P / 2, Q's rows by DMA;
//   D. acc / 2 + (dG / 2) S = E / 4 for E = 2 dG + 2 X1 - P, times 4: E;
//   E. dq[idx(r, c)] = E[r][c] - E[c][r] (r < c), the transposed entries through
//      LDS in float32, one column half of the block at a time.
// dG enters the products rounded to bf16 (as the pair passes' bf16 copy) and
// the leading 2 dG terms in float32.  The products run two-stage rings (the next
// tile's loads in flight over the current tile's MFMAs).  dG is read as float32
// twice (the starting values of A and C) and once more for A's first product,
// whose 64-column panels pass through registers: converted to bf16 (dG / 2)
// there, they also go to a row-major scratch copy, from which the later
// products take dG's rows (A's n-major B) and columns (D's k-major A) by DMA,
// as they take S, T and Q.
constexpr int kBlkB = 256;

// LDS images read transposed: dS (bf16, 256 x 256) holds entry (r, c) at
// element r * 256 + (c ^ 4 (r & 31)), a column half of E (float32, 256 x 128)
// holds (r, cc) at element r * 128 + (cc ^ 4 (r & 15)).  The XOR moves whole
// groups of four columns, so four consecutive columns of a row stay one aligned
// 8- or 16-byte access, and 32 lanes reading one column of 32 consecutive rows
// meet every bank.

__global__ void __launch_bounds__(512, 1)
cnp_bwd_block_kernel(const float* __restrict__ dG, const uint16_t* __restrict__ Sg, const uint16_t* __restrict__ Tg,
                     const uint16_t* __restrict__ Qg, uint16_t* __restrict__ dGh, float* __restrict__ dq) {
    using G = Geo<256, 256, 4, 2>;
    constexpr int MI = G::MI, NJ = G::NJ;        // 2 x 4 tiles of 32 x 32 per wave
    constexpr int kStage = 64 * 1024;            // A (32 KB) + B (32 KB)
    constexpr int kQBuf = 128 * 1024;            // phase C's B tile
    constexpr int NB = OperandLoads<256, false, G::NW>::n;   // DMA loads of a 256 x 64 tile per thread
    static_assert(NB == OperandLoads<256, true, G::NW>::n && NB == 4, "tile loads");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[160 * 1024];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / G::NWN, wn = wave % G::NWN;
    const int64_t z = blockIdx.x;
    const float* __restrict__ g = dG + z * (kBlkB * kBlkB);
    const uint16_t* __restrict__ S = Sg + z * (kBlkB * kBlkB);
    const uint16_t* __restrict__ T = Tg + z * (kBlkB * kBlkB);
    const uint16_t* __restrict__ Q = Qg + z * (kBlkB * kBlkB);
    uint16_t* __restrict__ H = dGh + z * (kBlkB * kBlkB);   // dG / 2 in bf16, row-major
    const uint32_t base = lds_offset(lds);

    f32x16_t acc[MI][NJ];
    // f(tile, first row, first column) for each 32 x 32 accumulator tile; the
    // bounds are uniform over the wave.  A lane holds rows r0 + 8 q + u (q, u < 4,
    // r0 = first row + 4 L) of column first column + l31 of its tile, the element
    // in accumulator 4 q + u.
    const int L = lane >> 5, l31 = lane & 31;
    auto for_tiles = [&](auto&& f) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) f(acc[i][j], wm * 64 + 32 * i, wn * 128 + 32 * j);
    };
    // acc = dG, loaded straight into the accumulators (no arithmetic on the
    // loaded values, so the loads stay in flight until the first MFMA needs them)
    // The wave's 64 x 128 region from a uniform base and 32-bit per-lane byte
    // offsets; the lane index passes through an ordered no-op first, so that no
    // part of the offsets is kept (or spilled) from one call to the next.
    auto init_dg = [&]() __attribute__((always_inline)) {
        const char* gw = reinterpret_cast<const char*>(g + wm * 64 * kBlkB + wn * 128);
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const uint32_t o = 4 * ((ln >> 5) * 4 * kBlkB + (ln & 31));
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const uint32_t c = 4 * ((i * 32 + (rr >> 2) * 8 + (rr & 3)) * kBlkB + j * 32);
                    acc[i][j][rr] = *reinterpret_cast<const float*>(gw + (o + c));
                }
    };
    auto scale_acc = [&](float f) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) acc[i][j][rr] *= f;
    };

    float4 st[8];   // this thread's 32 floats of the next dG panel
    // dG[:, 64 kt + 32 h .. + 32) of row r = tid / 2, h = tid % 2, times `scale` (k-major A)
    auto load_cols = [&](int kt) __attribute__((always_inline)) {
        const float4* src = reinterpret_cast<const float4*>(g + (tid >> 1) * kBlkB + kt * 64 + (tid & 1) * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) st[i] = src[i];
    };
    // the panel as bf16 (dG / 2) into the A stage and into its row-major copy H
    auto put_cols = [&](int stage, int kt) __attribute__((always_inline)) {
        const int r = tid >> 1, h = tid & 1;
        unsigned char* dst = lds + stage * kStage + r * 128;
        uint4* hrow = reinterpret_cast<uint4*>(H + r * kBlkB + kt * 64);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = 4 * h + i;
            const float4 u = st[2 * i], v = st[2 * i + 1];
            const uint4 w = make_uint4(pack_bf16x2(0.5f * u.x, 0.5f * u.y), pack_bf16x2(0.5f * u.z, 0.5f * u.w),
                                       pack_bf16x2(0.5f * v.x, 0.5f * v.y), pack_bf16x2(0.5f * v.z, 0.5f * v.w));
            *reinterpret_cast<uint4*>(dst + ((c ^ swz_k(r)) << 4)) = w;
            hrow[c] = w;
        }
    };
    // S rows (k-major B), T rows (m-major A), H rows (n-major B) and columns
    // (k-major A), Q rows (k-major B of phase C)
    auto dma_rows = [&](auto mn_c, const uint16_t* src, int kt, uint32_t dst) __attribute__((always_inline)) {
        constexpr bool MN = decltype(mn_c)::value;
#pragma unroll
        for (int j = 0; j < NB; ++j) dma_one<256, MN, G::NW>(j, dst, src, kBlkB, 0, kBlkB, kt * 64, kBlkB, wave, lane);
    };
    // One k-tile: the fragments of step ks + 1 are read before the MFMAs of step
    // ks (two sets live), and the fence keeps later reads from moving up.
    auto compute = [&](auto amn_c, auto bmn_c, const unsigned char* at, const unsigned char* bt)
                       __attribute__((always_inline)) {
        constexpr bool AMN = decltype(amn_c)::value, BMN = decltype(bmn_c)::value;
        uint4 af[2][MI], bfr[2][NJ];
        load_frags<G, AMN, BMN>(at, bt, wm, wn, 0, lane, af[0], bfr[0]);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int cur = ks & 1;
            if (ks + 1 < BK / 16) load_frags<G, AMN, BMN>(at, bt, wm, wn, ks + 1, lane, af[cur ^ 1], bfr[cur ^ 1]);
            asm volatile("" ::: "memory");
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) Mfma32<bf16_t>::run(af[cur][i], bfr[cur][j], acc[i][j]);
        }
    };
    // acc += (dG / 2) S over the four k-tiles, dG's panels through registers
    // (converted to bf16 into the A stage and into H).  Issue order per tile:
    // the register loads (8), then the DMA (4), so a wait for the registers
    // leaves the DMA in flight (vmcnt 4); the four stores of H follow, and a wait
    // for the DMA leaves them in flight (memory operations report completion in
    // issue order).  Tile kt + 1 goes to the stage tile kt - 1 used, once every
    // wave has passed the barrier that opens tile kt.
    // The first tile (stage 0), issued ahead.
    auto x1_first = [&]() __attribute__((always_inline)) {
        load_cols(0);
        dma_rows(std::false_type{}, S, 0, base + G::kABytes);
    };
    // next_first(): the next phase's first loads, issued over this phase's last
    // tile (stage 0 is free then: tile 2 is done everywhere) once every wave's
    // stores of H have completed.
    auto x1_loop = [&](auto&& next_first) __attribute__((always_inline)) {
        wait_vmcnt<4>();
        put_cols(0, 0);
#pragma unroll 1
        for (int kt = 0; kt < 4; ++kt) {
            if (kt + 1 < 4) wait_vmcnt<4>();
            else wait_vmcnt<0>();
            wait_lgkm0();
            block_barrier();
            if (kt + 1 < 4) {
                load_cols(kt + 1);
                dma_rows(std::false_type{}, S, kt + 1, base + ((kt + 1) & 1) * kStage + G::kABytes);
            } else {
                next_first();
            }
            compute(std::false_type{}, std::false_type{}, lds + (kt & 1) * kStage, lds + (kt & 1) * kStage + G::kABytes);
            if (kt + 1 < 4) {
                wait_vmcnt<4>();
                put_cols((kt + 1) & 1, kt + 1);
            }
        }
    };
    // acc += A B over the four k-tiles, both operands by DMA, in the same
    // two-stage ring; the first tile is issued by the phase before.
    auto dma_loop = [&](auto amn_c, auto bmn_c, const uint16_t* a_src, const uint16_t* b_src)
                        __attribute__((always_inline)) {
#pragma unroll 1
        for (int kt = 0; kt < 4; ++kt) {
            wait_vmcnt<0>();
            wait_lgkm0();
            block_barrier();
            if (kt + 1 < 4) {
                dma_rows(amn_c, a_src, kt + 1, base + ((kt + 1) & 1) * kStage);
                dma_rows(bmn_c, b_src, kt + 1, base + ((kt + 1) & 1) * kStage + G::kABytes);
            }
            compute(amn_c, bmn_c, lds + (kt & 1) * kStage, lds + (kt & 1) * kStage + G::kABytes);
        }
    };

    // ---- A. acc = dG + (dG / 2) S + T^T (dG / 2) = dS / 2 (halving is exact in
    // bf16 and float32, so 2 acc is dS as 2 dG + X1 + X2); the first product
    // leaves dG / 2 in bf16 in H, whose rows the second takes by DMA
    init_dg();
    x1_first();
    x1_loop([&]() {   // T^T (dG / 2)'s first tile, over (dG / 2) S's last
        dma_rows(std::true_type{}, T, 0, base);
        dma_rows(std::true_type{}, H, 0, base + G::kABytes);
    });
    dma_loop(std::true_type{}, std::true_type{}, T, H);
    scale_acc(2.f);    // dS
    block_barrier();   // every wave is done reading the stages
    dma_rows(std::false_type{}, Q, 0, base + kQBuf);   // Q's first k-tile, past the dS image

    // ---- B. Sigma = dS + dS^T through LDS.  A lane holds four consecutive rows
    // r..r+3 of a column c in each group of four accumulators, so it reads the
    // transposed entries dS[c][r..r+3] as one 8-byte access, and writes Sigma,
    // symmetric, as Sigma[c][r..r+3]: row c of the m-major A image of phase C
    // (k-row c, m = r..r+3), again one 8-byte access.  Each tile's LDS addresses
    // come from one per-lane base: the swizzle terms that vary with the
    // accumulator index occupy bits of their own, so they enter as a constant
    // XOR and a constant offset.
    for_tiles([&](f32x16_t& t, int row_lo, int col_lo) {
        const int r0 = row_lo + 4 * L, c = col_lo + l31;
        uint32_t a = 512 * r0 + 2 * (c ^ (16 * L));     // dS (r0, c)
        asm volatile("" : "+v"(a)::"memory");
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                *reinterpret_cast<uint16_t*>(lds + ((a ^ (64 * q + 8 * u)) + 512 * (8 * q + u))) =
                    ElemTraits<bf16_t>::from_f32(t[4 * q + u]).bits;
    });
    wait_lgkm0();
    block_barrier();
    for_tiles([&](f32x16_t& t, int row_lo, int col_lo) {
        const int r0 = row_lo + 4 * L, c = col_lo + l31;
        uint32_t a = 512 * c + 2 * (r0 ^ (4 * l31));    // dS (c, r0..r0+3)
        asm volatile("" : "+v"(a)::"memory");
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint2 v = *reinterpret_cast<const uint2*>(lds + (a ^ (16 * q)));
            t[4 * q + 0] += bf16_to_f32((uint16_t)(v.x & 0xffff));
            t[4 * q + 1] += bf16_to_f32((uint16_t)(v.x >> 16));
            t[4 * q + 2] += bf16_to_f32((uint16_t)(v.y & 0xffff));
            t[4 * q + 3] += bf16_to_f32((uint16_t)(v.y >> 16));
        }
    });
    wait_lgkm0();
    block_barrier();   // dS no longer read
    for_tiles([&](f32x16_t& t, int row_lo, int col_lo) {
        const int c = col_lo + l31;
        // k-row c, m = r0 + 8 q .. + 3 of the m-major image (swz_mn<256> of k-row c)
        uint32_t a = 512 * c + ((((row_lo >> 3)) ^ (4 * (c & 3))) << 4) + 8 * L;
        asm volatile("" : "+v"(a)::"memory");
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<uint2*>(lds + a + 16 * q) =
                make_uint2(pack_bf16x2(0.5f * t[4 * q], 0.5f * t[4 * q + 1]),
                           pack_bf16x2(0.5f * t[4 * q + 2], 0.5f * t[4 * q + 3]));
    });
    init_dg();   // phase C's starting value

    // ---- C. acc += (Sigma / 2) Q^T = -P / 2 (one Q buffer)
#pragma unroll 1
    for (int kt = 0; kt < 4; ++kt) {
        wait_vmcnt<0>();
        wait_lgkm0();
        block_barrier();   // Sigma complete; Q tile kt landed everywhere
        if (kt == 3) {   // phase D's first tile: Sigma's tiles 0 and 1 (stage 0) are done
            dma_rows(std::false_type{}, H, 0, base);
            dma_rows(std::false_type{}, S, 0, base + G::kABytes);
        }
        compute(std::true_type{}, std::false_type{}, lds + kt * G::kABytes, lds + kQBuf);
        if (kt + 1 < 4) {
            block_barrier();   // every wave is done reading Q tile kt
            dma_rows(std::false_type{}, Q, kt + 1, base + kQBuf);
        }
    }

    // ---- D. acc / 2 + (dG / 2) S = E / 4, H's columns by DMA (its loop's
    // barriers keep stage 1, Sigma's last tiles, untouched until every wave is
    // done with them)
    scale_acc(0.5f);
    dma_loop(std::false_type{}, std::false_type{}, H, S);
    scale_acc(4.f);    // E

    // ---- E. dq = E - E^T on the upper triangle, by column halves: E[c][r..r+3]
    // for a lane's rows r..r+3 of column c is one 16-byte read.  Only the part of
    // E below the diagonal is read from LDS, so tiles wholly above it are not
    // written, and tiles wholly below it store nothing.  The packed index of
    // (r, c) steps by b - r - 2 from row r to row r + 1; the stores go through a
    // buffer resource spanning the block's dq, where an entry on or below the
    // diagonal takes an offset past its end and the store is dropped (no branch).
    // (stride 0: a raw byte range of num_records bytes; the last word selects the
    // 32-bit data format, the one the untyped buffer accesses of gfx9 parts use)
    constexpr int kFmt32 = 0x00020000;
    const __amdgpu_buffer_rsrc_t out =
        __builtin_amdgcn_make_buffer_rsrc(dq + z * (kBlkB * (kBlkB - 1) / 2), 0, kBlkB * (kBlkB - 1) / 2 * 4, kFmt32);
    constexpr uint32_t kDrop = 0x80000000u;   // past the resource's end
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
        wait_lgkm0();
        block_barrier();   // the LDS is free (the ring, or the previous half, no longer read)
        if (wn == h)
            for_tiles([&](f32x16_t& t, int row_lo, int col_lo) {
                if (row_lo < col_lo) return;   // wholly above the diagonal: never read
                const int r0 = row_lo + 4 * L, cc = col_lo - 128 * h + l31;
                uint32_t a = 512 * r0 + 4 * (cc ^ (16 * L));    // E (r0, cc)
                asm volatile("" : "+v"(a)::"memory");
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        *reinterpret_cast<float*>(lds + ((a ^ (128 * (q & 1) + 16 * u)) + 512 * (8 * q + u))) =
                            t[4 * q + u];
            });
        wait_lgkm0();
        block_barrier();
        // owners of (r, c), r < c, with r in this column half read E[c][r]
        if ((wm >> 1) == h)
            for_tiles([&](f32x16_t& t, int row_lo, int col_lo) {
                if (row_lo > col_lo) return;   // wholly below the diagonal: nothing to store
                const int r0 = row_lo + 4 * L, c = col_lo + l31;
                uint32_t a = 512 * c + 4 * ((r0 - 128 * h) ^ (4 * (l31 & 15)));   // E[c][r0..r0+3]
                // byte offset of dq[idx(r0, c)], its step to the next row, and the
                // number of rows r0 + d above the diagonal (d < lim)
                uint32_t j = 2 * r0 * (511 - r0) + 4 * (c - r0 - 1);
                const uint32_t k4 = 4 * (254 - r0);
                const int lim = c - r0;
                asm volatile("" : "+v"(a), "+v"(j)::"memory");
                // the four reads first (the buffer stores would otherwise order them)
                float4 e[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) e[q] = *reinterpret_cast<const float4*>(lds + (a ^ (32 * q)));
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float ev[4] = {e[q].x, e[q].y, e[q].z, e[q].w};
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int d = 8 * q + u;
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(t[4 * q + u] - ev[u]), out,
                                                              d < lim ? j : kDrop, 0, 0);
                        // to row r0 + d + 1, or from the quad's last row to the next quad's first
                        j += u < 3 ? k4 - 4 * d : 5 * k4 - 4 * (5 * d + 10);
                    }
                }
            });
    }
}

template <int BM, int BN, bool A_MN, bool B_MN, bool OUT_F32, int EPI = kEpiPlain, int S = 3, int NWM = 2, int NWN = 2,
          int DUAL = 0, bool GRP = false, bool Q8 = false>
hipError_t launch(const PipeArgs& p, hipStream_t stream) {
    if constexpr (!A_MN) {
        // the loads address each operand k-tile by 32-bit per-lane byte offsets
        const int64_t span_a = (int64_t)p.M * p.lda * 2,
                      span_b = (int64_t)(B_MN ? p.K : p.N) * p.ldb * (Q8 ? 1 : 2);
        if (span_a >= (int64_t(1) << 32) || span_b >= (int64_t(1) << 32)) return hipErrorInvalidValue;
    }
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
        if (p.colscale) q.colscale = p.colscale + (int64_t)y0 * p.strideScale;
        hipLaunchKernelGGL((pipe_gemm_kernel<BM, BN, A_MN, B_MN, OUT_F32, EPI, S, NWM, NWN, DUAL, GRP, Q8>),
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
// b = 256 runs eight waves (NT = 512): the image build, the same work for
// every panel of a block, is then split over twice the lanes (32 blocks:
// 11 us against 13 with four waves), and each wave's share of C is 32 rows.
template <int B, int PH, int NW = 4>
struct FusedCnp {
    static constexpr int KT = B / 64;         // k-tiles of one product
    static constexpr int NP = B / PH;         // panels per block
    static constexpr int QB = B * 128;        // bytes of one Q k-tile ([B rows][64 k])
    static constexpr int XB = PH * 128;       // bytes of one X k-tile ([PH rows][64 k])
    static constexpr int LDS = KT * (QB + XB);
    static constexpr int MI = B / (32 * NW);  // wave w of NW: rows n in [w B/NW, (w+1) B/NW) of C
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

// Step 1 of the fused forward for one block: Q = U - U^T in LDS (bf16, the
// k-tiled image described above) from the block's packed triangle qz, by NT
// threads.  Tasks: the strict upper 8 x 8 sub-blocks (sub-rows R' and
// NB8 - 2 - R' sharing a run of NB8 tasks), then the diagonal ones; every
// thread issues the loads of all its tasks before it writes any.
template <int B, int NT>
__device__ __forceinline__ void build_q_image(const float* __restrict__ qz, unsigned char* __restrict__ qs, int tid) {
    using F = FusedCnp<B, 64>;
    constexpr int QB = F::QB, NB8 = F::NB8;
    constexpr int NTASK = (F::TASKS + NT - 1) / NT;
    float u[NTASK][8][8];
#pragma unroll
    for (int s = 0; s < NTASK; ++s) {
        const int t = tid + NT * s;
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
        const int t = tid + NT * s;
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
}

template <int B, int PH, int NT = 256>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(NT / 256, B == 256 ? NT / 256 : 2)))
cnp_fused_kernel(const float* __restrict__ q, uint16_t* __restrict__ G, uint16_t* __restrict__ Qc,
                 uint16_t* __restrict__ Sv, uint16_t* __restrict__ Tv, int k, int total) {
    using F = FusedCnp<B, PH, NT / 64>;
    static_assert(F::MI >= 1, "a wave owns at least 32 rows");
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

    // 1. the Q image
    build_q_image<B, NT>(qz, qs, tid);
    __syncthreads();

    // rows of an image as 16-byte chunks: PH rows x B/8 chunks over the workgroup
    auto copy_rows = [&](uint16_t* __restrict__ dst, auto chunk_value) {
        for (int u = tid; u < PH * (B / 8); u += NT) {
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
    const int n_base = wave * (B / (NT / 64));
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

// The k = 3 Cayley-Neumann forward of one b = 256 block per workgroup (large
// batches), keeping Q, S and T for the backward.  G = I + 2Q + 2S + T S with
// S = Q Q and T = 2Q + S (the same factorization as the unfused products):
//   1. the Q image in LDS from the packed triangle (the per-panel kernel's
//      step 1, over the whole workgroup); Q's rows to Qc;
//   2. acc = Q Q^T = -S from the image (both operands k-major rows of Q);
//   3. S and T = 2Q + S to memory in bf16 (T from the bf16 Q and S, as the
//      per-panel kernel forms it);
//   4. acc = I + 2Q + 2S in float32 (2S from the accumulators, 2Q from the image);
//   5. acc += S T^T, S's and T's rows back by DMA;
//   6. G to memory in bf16.
// S is symmetric, so the accumulator a lane holds for rows r..r+3 of column c,
// (Q Q^T)(r.., c), is also S's row c at columns r..r+3, and the product of
// step 5, (S T^T)(r.., c) = (T S)(c, r..), lands on G's row c at columns
// r..r+3.  Eight waves, wave (wm, wn) owning rows [64 wm, 64 wm + 64) and
// columns [128 wn, 128 wn + 128) of the accumulators, i.e. columns
// [64 wm, 64 wm + 64) of rows [128 wn, 128 wn + 128) of S, T and G.  Each wave
// passes its share through 4 KB of LDS of its own, 32 rows x 64 columns at a
// time, so that the stores go out as whole 128-byte row segments.
__global__ void __launch_bounds__(512, 1)
cnp_fwd_block_kernel(const float* __restrict__ q, uint16_t* __restrict__ Gout, uint16_t* __restrict__ Qc,
                     uint16_t* __restrict__ Sv, uint16_t* __restrict__ Tv) {
    using F = FusedCnp<kBlkB, 64>;
    using GE = Geo<256, 256, 4, 2>;
    constexpr int MI = GE::MI, NJ = GE::NJ;     // 2 x 4 tiles of 32 x 32 per wave
    constexpr int QB = F::QB;                   // one k-tile of the Q image, 32 KB
    constexpr int kStage = 64 * 1024;           // step 5's A (32 KB) + B (32 KB)
    constexpr int NB = OperandLoads<256, false, GE::NW>::n;
    static_assert(4 * QB == 2 * kStage, "the ring takes the image's place");
    constexpr int kStageOut = 4 * QB;           // the waves' 4 KB output stages
    __shared__ __attribute__((aligned(1024))) unsigned char lds[4 * QB + 8 * 4096];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / GE::NWN, wn = wave % GE::NWN;
    const int64_t z = blockIdx.x, zoff = z * (kBlkB * kBlkB);
    const uint32_t base = lds_offset(lds);
    const int L = lane >> 5, l31 = lane & 31;

    // 1. the Q image, and Q's rows as 16-byte chunks
    build_q_image<kBlkB, 512>(q + z * F::NPAR, lds, tid);
    __syncthreads();
    if (Qc)
        for (int u = tid; u < kBlkB * (kBlkB / 8); u += 512) {
            const int m = u / (kBlkB / 8), c = 8 * (u % (kBlkB / 8));
            *reinterpret_cast<uint4*>(Qc + zoff + m * kBlkB + c) =
                *reinterpret_cast<const uint4*>(lds + img_off<QB>(m, c));
        }

    // a lane holds rows r0 + 8 q + u (q, u < 4, r0 = first row + 4 L) of column
    // first column + l31 of each 32 x 32 accumulator tile, in accumulator 4 q + u
    f32x16_t acc[MI][NJ];

    // 2. acc = Q Q^T, fragments straight from the image (two sets in flight)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    {
        uint4 af[2][MI], bfr[2][NJ];
        auto frags = [&](int ks, uint4 (&a)[MI], uint4 (&b)[NJ]) __attribute__((always_inline)) {
            const unsigned char* t = lds + (ks >> 2) * QB;
#pragma unroll
            for (int i = 0; i < MI; ++i) a[i] = img_frag(t, wm * 64 + 32 * i, ks & 3, lane);
#pragma unroll
            for (int j = 0; j < NJ; ++j) b[j] = img_frag(t, wn * 128 + 32 * j, ks & 3, lane);
        };
        frags(0, af[0], bfr[0]);
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            const int cur = ks & 1;
            if (ks + 1 < 16) frags(ks + 1, af[cur ^ 1], bfr[cur ^ 1]);
            asm volatile("" ::: "memory");
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) Mfma32<bf16_t>::run(af[cur][i], bfr[cur][j], acc[i][j]);
        }
    }

    // Rows [128 wn + 32 j, + 32) x columns [64 wm, + 64) of an output through the
    // wave's stage: put(i, qd, half) gives the 8-byte run of row 128 wn + 32 j + l31
    // at columns 64 wm + 32 i + 8 qd + 4 half; the stage holds (row, column) at
    // row * 128 + 16 ((column / 8) ^ ((row / 2) & 7)) + 8 ((column / 4 & 1) ^ (row / 16 & 1))
    // (32 lanes writing one column of 32 rows meet distinct banks), and each
    // lane then stores 16-byte chunks, eight lanes to a row.
    unsigned char* ostage = lds + kStageOut + wave * 4096;
    auto out_rows = [&](uint16_t* __restrict__ dst, int j, auto&& put) __attribute__((always_inline)) {
        const int rw = l31;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int ch = 4 * i + qd;
                *reinterpret_cast<uint2*>(ostage + rw * 128 + 16 * (ch ^ ((rw >> 1) & 7)) + 8 * (L ^ ((rw >> 4) & 1))) =
                    put(i, qd);
            }
        wait_lgkm0();
#pragma unroll
        for (int ps = 0; ps < 4; ++ps) {
            const int row = 8 * ps + (lane >> 3), ch = lane & 7;
            uint4 v = *reinterpret_cast<const uint4*>(ostage + row * 128 + 16 * (ch ^ ((row >> 1) & 7)));
            if ((row >> 4) & 1) v = make_uint4(v.z, v.w, v.x, v.y);
            *reinterpret_cast<uint4*>(dst + zoff + (wn * 128 + 32 * j + row) * kBlkB + wm * 64 + 8 * ch) = v;
        }
        wait_lgkm0();
    };

    // 3. S = -acc and T = 2Q + S, row c = 128 wn + 32 j + l31, columns
    // r = 64 wm + 32 i + 4 L + 8 q + u; 4. acc = I + 2Q + 2S at the same entries
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int c = wn * 128 + 32 * j + l31;
        uint2 sv[MI][4], tv[MI][4];
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            f32x16_t& t = acc[i][j];
            const int r0 = wm * 64 + 32 * i + 4 * L;
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const uint2 qv = *reinterpret_cast<const uint2*>(lds + img_off<QB>(c, r0 + 8 * qd));
                const float qf[4] = {bf16_to_f32((uint16_t)(qv.x & 0xffff)), bf16_to_f32((uint16_t)(qv.x >> 16)),
                                     bf16_to_f32((uint16_t)(qv.y & 0xffff)), bf16_to_f32((uint16_t)(qv.y >> 16))};
                float sf[4], tf[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float sx = -t[4 * qd + u];
                    sf[u] = bf16_to_f32(ElemTraits<bf16_t>::from_f32(sx).bits);
                    tf[u] = 2.f * qf[u] + sf[u];
                    t[4 * qd + u] = (c == r0 + 8 * qd + u ? 1.f : 0.f) + 2.f * qf[u] + 2.f * sx;
                }
                sv[i][qd] = make_uint2(pack_bf16x2(sf[0], sf[1]), pack_bf16x2(sf[2], sf[3]));
                tv[i][qd] = make_uint2(pack_bf16x2(tf[0], tf[1]), pack_bf16x2(tf[2], tf[3]));
            }
        }
        out_rows(Sv, j, [&](int i, int qd) { return sv[i][qd]; });
        out_rows(Tv, j, [&](int i, int qd) { return tv[i][qd]; });
    }

    // 5. acc += S T^T over four k-tiles of 64, S's rows (A) and T's rows (B) by
    // DMA into a two-stage ring over the image's place, tile kt + 1 issued
    // over tile kt's products
    const uint16_t* Sz = Sv + zoff;
    const uint16_t* Tz = Tv + zoff;
    auto dma_tile = [&](int kt) __attribute__((always_inline)) {
        const uint32_t dst = base + (kt & 1) * kStage;
#pragma unroll
        for (int j = 0; j < NB; ++j) dma_one<256, false, GE::NW>(j, dst, Sz, kBlkB, 0, kBlkB, kt * 64, kBlkB, wave, lane);
#pragma unroll
        for (int j = 0; j < NB; ++j)
            dma_one<256, false, GE::NW>(j, dst + GE::kABytes, Tz, kBlkB, 0, kBlkB, kt * 64, kBlkB, wave, lane);
    };
    wait_vmcnt<0>();   // this thread's S and T stores have completed
    wait_lgkm0();
    block_barrier();   // everyone's have, and the image is no longer read
    dma_tile(0);
#pragma unroll 1
    for (int kt = 0; kt < 4; ++kt) {
        wait_vmcnt<0>();
        block_barrier();   // tile kt landed everywhere; tile kt - 1's stage is free
        if (kt + 1 < 4) dma_tile(kt + 1);
        const unsigned char* at = lds + (kt & 1) * kStage;
        uint4 af[2][MI], bfr[2][NJ];
        load_frags<GE, false, false>(at, at + GE::kABytes, wm, wn, 0, lane, af[0], bfr[0]);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int cur = ks & 1;
            if (ks + 1 < BK / 16)
                load_frags<GE, false, false>(at, at + GE::kABytes, wm, wn, ks + 1, lane, af[cur ^ 1], bfr[cur ^ 1]);
            asm volatile("" ::: "memory");
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) Mfma32<bf16_t>::run(af[cur][i], bfr[cur][j], acc[i][j]);
        }
    }

    // 6. G's rows through the stages
#pragma unroll
    for (int j = 0; j < NJ; ++j)
        out_rows(Gout, j, [&](int i, int qd) {
            const f32x16_t& t = acc[i][j];
            return make_uint2(pack_bf16x2(t[4 * qd], t[4 * qd + 1]), pack_bf16x2(t[4 * qd + 2], t[4 * qd + 3]));
        });
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

// Launch helper of the two k = 3 backward passes: pairs of 64 x 64 tiles of
// every block, batch entries in chunks of at most 65535 (grid.y).
template <class Fn>
hipError_t launch_pairs(int64_t nblk, int b, Fn&& fn, bool units = false) {
    const int nt = b / 64;
    constexpr int kMaxY = 65535;
    for (int64_t y0 = 0; y0 < nblk; y0 += kMaxY) {
        const int ny = (int)std::min<int64_t>(kMaxY, nblk - y0);
        fn(y0, dim3(units ? units_per_block(nt) : nt * (nt + 1) / 2, ny));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t cnp_bwd_sym(const float* dG, const void* S, const void* T, void* sigma, float* dq, int64_t nblk, int b,
                       hipStream_t stream) {
    if (nblk <= 0) return hipSuccess;
    if (b % 64 != 0 || b > 1024) return hipErrorInvalidValue;
    if (reinterpret_cast<uintptr_t>(dG) & 15) return hipErrorInvalidValue;   // 16-byte loads of dG
    const int64_t bb = (int64_t)b * b, ntri = (int64_t)b * (b - 1) / 2;
    return launch_pairs(nblk, b, [&](int64_t y0, dim3 grid) {
        PipeArgs p;
        p.B = static_cast<const uint16_t*>(S) + y0 * bb;
        p.A2 = static_cast<const uint16_t*>(T) + y0 * bb;
        p.Cin1 = dG + y0 * bb; p.ldcin1 = b; p.strideCin1 = bb;
        p.M = p.N = p.K = b;
        uint16_t* sg = static_cast<uint16_t*>(sigma) + y0 * bb;
        if (b <= 256)
            hipLaunchKernelGGL(cnp_bwd_sym_kernel<2>, grid, dim3(512), 0, stream, p, dq + y0 * ntri, sg, b);
        else
            hipLaunchKernelGGL(cnp_bwd_sym_kernel<3>, grid, dim3(512), 0, stream, p, dq + y0 * ntri, sg, b);
    }, true);
}

hipError_t cnp_bwd_sigq(const void* sigma, const void* Q, float* dq, int64_t nblk, int b, hipStream_t stream) {
    if (nblk <= 0) return hipSuccess;
    if (b % 64 != 0 || b > 1024) return hipErrorInvalidValue;
    const int64_t bb = (int64_t)b * b, ntri = (int64_t)b * (b - 1) / 2;
    return launch_pairs(nblk, b, [&](int64_t y0, dim3 grid) {
        PipeArgs p;
        p.A = static_cast<const uint16_t*>(sigma) + y0 * bb;
        p.B = static_cast<const uint16_t*>(Q) + y0 * bb;
        p.M = p.N = p.K = b;
        if (b <= 256)
            hipLaunchKernelGGL(cnp_bwd_sigq_kernel<2>, grid, dim3(512), 0, stream, p, dq + y0 * ntri, b);
        else
            hipLaunchKernelGGL(cnp_bwd_sigq_kernel<3>, grid, dim3(512), 0, stream, p, dq + y0 * ntri, b);
    }, true);
}

hipError_t cnp_bwd_block(const float* dG, const void* S, const void* T, const void* Q, void* dGh, float* dq,
                         int64_t nblk, int b, hipStream_t stream) {
    if (nblk <= 0) return hipSuccess;
    if (b != kBlkB) return hipErrorInvalidValue;
    const int64_t bb = (int64_t)b * b, ntri = (int64_t)b * (b - 1) / 2;
    constexpr int64_t kMaxGrid = 0x7fffffff;
    for (int64_t z0 = 0; z0 < nblk; z0 += kMaxGrid) {
        const int64_t nz = std::min<int64_t>(kMaxGrid, nblk - z0);
        hipLaunchKernelGGL(cnp_bwd_block_kernel, dim3((unsigned)nz), dim3(512), 0, stream, dG + z0 * bb,
                           static_cast<const uint16_t*>(S) + z0 * bb, static_cast<const uint16_t*>(T) + z0 * bb,
                           static_cast<const uint16_t*>(Q) + z0 * bb, static_cast<uint16_t*>(dGh) + z0 * bb,
                           dq + z0 * ntri);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

bool dense_fold_r_supported(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int64_t ldc2,
                            int b) {
    return b == 256 && M > 0 && N > 0 && N % 256 == 0 && K >= BK && K % BK == 0 && lda % 8 == 0 && ldb % 8 == 0 &&
           ldc % 8 == 0 && ldc2 % 8 == 0 && ldc >= N && ldc2 >= N && M <= 0x7fffffff && N <= 0x7fffffff &&
           K <= 0x7fffffff;
}

hipError_t dense_fold_r(bool q8, const void* A, int64_t lda, const void* B, int64_t ldb, const float* colscale,
                        const void* G, void* h2, int64_t ldh2, void* z, int64_t ldz, int M, int N, int K, int b,
                        hipStream_t stream) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (!dense_fold_r_supported(M, N, K, lda, ldb, ldz, h2 ? ldh2 : ldz, b) || !G || !z || (q8 && !colscale))
        return hipErrorInvalidValue;
    if (q8 && ldb % 16 != 0) return hipErrorInvalidValue;
    PipeArgs p;
    p.A = A; p.lda = lda;
    p.B = B; p.ldb = ldb;
    p.C = z; p.ldc = ldz;
    p.C2 = h2; p.ldc2 = ldh2;
    p.Gfold = G;
    p.colscale = colscale;
    p.M = M; p.N = N; p.K = K;
    p.k_per_split = K;
    if (q8) return launch<128, 256, false, false, false, kEpiFoldR, 3, 2, 4, 0, false, true>(p, stream);
    return launch<128, 256, false, false, false, kEpiFoldR, 3, 2, 4>(p, stream);
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

bool dense_gemm_q8_supported(bool b_nn, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb) {
    (void)b_nn;
    // A is k-major bf16 (whole 64-k tiles); int8 B chunks are 16 bytes
    return M > 0 && N >= 16 && N % 16 == 0 && K >= BK && K % BK == 0 && lda % 8 == 0 && ldb % 16 == 0;
}

hipError_t dense_gemm_q8(bool b_nn, const void* A, int64_t lda, const int8_t* B, int64_t ldb, const float* colscale,
                         void* C, int64_t ldc, int M, int N, int K, hipStream_t stream) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (!dense_gemm_q8_supported(b_nn, M, N, K, lda, ldb) || (!b_nn && !colscale)) return hipErrorInvalidValue;
    PipeArgs p;
    p.A = A; p.lda = lda;
    p.B = B; p.ldb = ldb;
    p.C = C; p.ldc = ldc;
    p.M = M; p.N = N; p.K = K;
    p.k_per_split = K;
    p.colscale = b_nn ? nullptr : colscale;
    // tiles as for the bf16 dense products
    auto tiles = [&](int bm, int bn) { return (int64_t)((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    if (!b_nn) {
        if (tiles(256, 256) >= 256)
            return launch<256, 256, false, false, false, kEpiColScale, 2, 2, 4, 0, false, true>(p, stream);
        if (tiles(256, 128) >= 256)
            return launch<256, 128, false, false, false, kEpiColScale, 3, 4, 2, 0, false, true>(p, stream);
        if (tiles(128, 128) >= 256)
            return launch<128, 128, false, false, false, kEpiColScale, 4, 2, 2, 0, false, true>(p, stream);
        return launch<64, 128, false, false, false, kEpiColScale, 4, 2, 2, 0, false, true>(p, stream);
    }
    if (tiles(256, 256) >= 256) return launch<256, 256, false, true, false, kEpiPlain, 2, 2, 4, 0, false, true>(p, stream);
    if (tiles(256, 128) >= 256) return launch<256, 128, false, true, false, kEpiPlain, 3, 4, 2, 0, false, true>(p, stream);
    if (tiles(128, 128) >= 256) return launch<128, 128, false, true, false, kEpiPlain, 4, 2, 2, 0, false, true>(p, stream);
    return launch<64, 128, false, true, false, kEpiPlain, 4, 2, 2, 0, false, true>(p, stream);
}

hipError_t pipe_gemm_colscale(const PipeArgs& p, hipStream_t stream, PipeTile tile) {
    if (p.M <= 0 || p.N <= 0 || p.batch <= 0) return hipSuccess;
    if (!p.colscale || p.splits != 1) return hipErrorInvalidValue;
    switch (tile) {
        case PipeTile::Big: return launch<256, 256, false, true, false, kEpiColScale, 2, 2, 4>(p, stream);
        case PipeTile::Wide: return launch<128, 256, false, true, false, kEpiColScale, 3, 2, 4>(p, stream);
        case PipeTile::Slim: return launch<64, 128, false, true, false, kEpiColScale, 4>(p, stream);
        case PipeTile::Tall: return launch<256, 128, false, true, false, kEpiColScale, 3, 4, 2>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t cnp_fwd_block(const float* q, void* G, void* Qc, void* S, void* T, int64_t nblk, int b,
                         hipStream_t stream) {
    if (nblk <= 0) return hipSuccess;
    if (b != kBlkB || !G || !S || !T) return hipErrorInvalidValue;
    const int64_t bb = (int64_t)b * b, npar = (int64_t)b * (b - 1) / 2;
    constexpr int64_t kMaxGrid = 0x7fffffff;
    for (int64_t z0 = 0; z0 < nblk; z0 += kMaxGrid) {
        const int64_t nz = std::min<int64_t>(kMaxGrid, nblk - z0);
        hipLaunchKernelGGL(cnp_fwd_block_kernel, dim3((unsigned)nz), dim3(512), 0, stream, q + z0 * npar,
                           static_cast<uint16_t*>(G) + z0 * bb, Qc ? static_cast<uint16_t*>(Qc) + z0 * bb : nullptr,
                           static_cast<uint16_t*>(S) + z0 * bb, static_cast<uint16_t*>(T) + z0 * bb);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
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
        hipLaunchKernelGGL((cnp_fused_kernel<256, 64, 512>), grid, dim3(512), 0, stream, q, g, qc, sv, tv, k, (int)panels);
    else if (b == 256)
        hipLaunchKernelGGL((cnp_fused_kernel<256, 32, 512>), grid, dim3(512), 0, stream, q, g, qc, sv, tv, k, (int)panels);
    else if (tall)
        hipLaunchKernelGGL((cnp_fused_kernel<128, 64>), grid, dim3(256), 0, stream, q, g, qc, sv, tv, k, (int)panels);
    else
        hipLaunchKernelGGL((cnp_fused_kernel<128, 32>), grid, dim3(256), 0, stream, q, g, qc, sv, tv, k, (int)panels);
    return hipGetLastError();
}

}  // namespace poetx
