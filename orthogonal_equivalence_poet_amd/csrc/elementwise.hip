// Memory-bound kernels of libpoetx: compact skew unpack / pack, the 2-D
// permutation (gather or scatter of columns, optional row gather), the
// split-K reduction, the float32 combine used between Cayley-Neumann
// products, fills, permutation helpers and the dense block-diagonal transforms
// of the weight-centric variant.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "elementwise.h"

namespace poetx {

namespace {

// Storage position of Q[r][c], r < c, in the row-major strict upper triangle.
__device__ __forceinline__ int64_t tri_index(int64_t r, int64_t c, int64_t b) {
    return r * b - (r * (r + 1)) / 2 + (c - r - 1);
}

constexpr int kSkewTile = 32;

// Q[j] = unpack(q[j]).  One workgroup per (block, 32 x 32 output tile).  Tiles
// below the diagonal are produced from the mirrored upper tile staged in LDS,
// so global reads are contiguous row segments of the triangle and writes are
// contiguous row segments of Q.
template <typename T>
__global__ void __launch_bounds__(256) skew_unpack_kernel(const float* __restrict__ q, T* __restrict__ Q,
                                                          int b, bf16_t* __restrict__ Q2) {
    __shared__ float tile[kSkewTile][kSkewTile + 1];
    const int tiles = b / kSkewTile;
    const int ti = blockIdx.x / tiles;
    const int tj = blockIdx.x % tiles;
    const int64_t blk = blockIdx.y;
    const int64_t ntri = (int64_t)b * (b - 1) / 2;
    const float* qb = q + blk * ntri;
    T* Qb = Q + blk * (int64_t)b * b;
    const int tx = threadIdx.x & 31;
    const int ty = threadIdx.x >> 5;  // 0..7
    // the upper tile (min(ti,tj), max(ti,tj)) staged as tile[row][col]
    const int ui = min(ti, tj), uj = max(ti, tj);
    for (int rr = ty; rr < kSkewTile; rr += 8) {
        const int r = ui * kSkewTile + rr;
        const int c = uj * kSkewTile + tx;
        tile[rr][tx] = (r < c) ? qb[tri_index(r, c, b)] : 0.f;
    }
    __syncthreads();
    for (int rr = ty; rr < kSkewTile; rr += 8) {
        const int r = ti * kSkewTile + rr;
        const int c = tj * kSkewTile + tx;
        float v;
        if (ti < tj) v = tile[rr][tx];
        else if (ti > tj) v = -tile[tx][rr];
        else v = (rr < tx) ? tile[rr][tx] : (rr > tx ? -tile[tx][rr] : 0.f);
        store_f32(Qb + (int64_t)r * b + c, v);
        if (Q2) Q2[blk * (int64_t)b * b + (int64_t)r * b + c] = ElemTraits<bf16_t>::from_f32(v);
    }
}

// dq[j][idx(r,c)] = dQ[j][r][c] - dQ[j][c][r] for r < c.  One workgroup per
// (block, 32 x 32 tile on or above the diagonal; the grid holds only those);
// the mirrored tile is staged in LDS.
__global__ void __launch_bounds__(256) skew_pack_kernel(const float* __restrict__ dQ, float* __restrict__ dq,
                                                        int b) {
    __shared__ float up[kSkewTile][kSkewTile + 1];
    __shared__ float lo[kSkewTile][kSkewTile + 1];
    const int tiles = b / kSkewTile;
    // tile row ti holds the tiles - ti pairs (ti, ti .. tiles - 1)
    int ti = 0, t = blockIdx.x;
    while (t >= tiles - ti) {
        t -= tiles - ti;
        ++ti;
    }
    const int tj = ti + t;
    const int64_t blk = blockIdx.y;
    const int64_t ntri = (int64_t)b * (b - 1) / 2;
    const float* G = dQ + blk * (int64_t)b * b;
    float* out = dq + blk * ntri;
    const int tx = threadIdx.x & 31;
    const int ty = threadIdx.x >> 5;
    for (int rr = ty; rr < kSkewTile; rr += 8) {
        up[rr][tx] = G[(int64_t)(ti * kSkewTile + rr) * b + tj * kSkewTile + tx];
        lo[rr][tx] = G[(int64_t)(tj * kSkewTile + rr) * b + ti * kSkewTile + tx];
    }
    __syncthreads();
    for (int rr = ty; rr < kSkewTile; rr += 8) {
        const int r = ti * kSkewTile + rr;
        const int c = tj * kSkewTile + tx;
        if (r < c) out[tri_index(r, c, b)] = up[rr][tx] - lo[tx][rr];
    }
}

// Small-block variants (b not a multiple of 32): one thread per element.
template <typename T>
__global__ void skew_unpack_simple(const float* __restrict__ q, T* __restrict__ Q, int b, int64_t total,
                                   bf16_t* __restrict__ Q2) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int64_t bb = (int64_t)b * b;
    const int64_t blk = i / bb;
    const int r = (int)((i % bb) / b);
    const int c = (int)(i % b);
    const float* qb = q + blk * ((int64_t)b * (b - 1) / 2);
    float v = 0.f;
    if (r < c) v = qb[tri_index(r, c, b)];
    else if (r > c) v = -qb[tri_index(c, r, b)];
    store_f32(Q + i, v);
    if (Q2) Q2[i] = ElemTraits<bf16_t>::from_f32(v);
}

__global__ void skew_pack_simple(const float* __restrict__ dQ, float* __restrict__ dq, int b, int64_t nblk) {
    const int64_t ntri = (int64_t)b * (b - 1) / 2;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nblk * ntri) return;
    const int64_t blk = i / ntri;
    int64_t t = i % ntri;
    // invert idx(r, c): row r holds b - 1 - r entries
    int r = 0;
    while (t >= b - 1 - r) { t -= b - 1 - r; ++r; }
    const int c = r + 1 + (int)t;
    const float* G = dQ + blk * (int64_t)b * b;
    dq[i] = G[(int64_t)r * b + c] - G[(int64_t)c * b + r];
}

// ------------------------------------------------------------- permutation
// A workgroup owns `rows_per_wg` full rows, staged in LDS: gathers read the
// row contiguously and pick from LDS; scatters place into LDS and write the
// row contiguously.  Both global streams are 16-byte vectors.  Every thread
// issues NB loads (data and indices) before it uses any of them, so a
// workgroup waits for memory a few times, not once per vector.  NB is the
// thread's share of the workgroup's vectors, up to 8: registers beyond it would
// cost resident workgroups (at 2 vectors a thread, 46 registers keep eight
// workgroups of 256 threads on a CU, 120 kept four).  When the share fits one
// batch of at most 4, a gather loads its column indices together with the row,
// so that the two latencies overlap (for 8 the indices would stay live across
// the barrier, at a cost in resident workgroups).
template <typename T, int NB>
__global__ void __launch_bounds__(256) permute_rows_lds(const T* __restrict__ src, T* __restrict__ dst,
                                                        int64_t rows, int cols, const int* __restrict__ row_idx,
                                                        const int* __restrict__ col_idx, int scatter,
                                                        int rows_per_wg) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    T* buf = reinterpret_cast<T*>(smem_raw);
    constexpr int V = ElemTraits<T>::kVec;
    const int chunks = cols / V;
    const int64_t row0 = (int64_t)blockIdx.x * rows_per_wg;
    const int nrows = (int)min<int64_t>(rows_per_wg, rows - row0);
    const int total = nrows * chunks;
    const bool scat = scatter && col_idx;
    const bool gath = !scatter && col_idx;
    const bool one = NB <= 4 && total <= 256 * NB;   // one batch: a gather's indices load with the row
    int ci[NB][V];
    for (int u0 = threadIdx.x; u0 < total; u0 += 256 * NB) {
        uint4 v[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int u = u0 + k * 256;
            if (u < total) {
                const int r = u / chunks;
                const int c = (u % chunks) * V;
                const int64_t gr = row0 + r;
                const int64_t sr = row_idx ? row_idx[gr] : gr;
                v[k] = *reinterpret_cast<const uint4*>(src + sr * cols + c);
                if (scat || (gath && one)) {
#pragma unroll
                    for (int i = 0; i < V; ++i) ci[k][i] = col_idx[c + i];
                }
            }
        }
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int u = u0 + k * 256;
            if (u < total) {
                const int r = u / chunks;
                const int c = (u % chunks) * V;
                if (scat) {
                    const T* e = reinterpret_cast<const T*>(&v[k]);
#pragma unroll
                    for (int i = 0; i < V; ++i) buf[r * cols + ci[k][i]] = e[i];
                } else {
                    *reinterpret_cast<uint4*>(buf + r * cols + c) = v[k];
                }
            }
        }
    }
    __syncthreads();
    for (int u0 = threadIdx.x; u0 < total; u0 += 256 * NB) {
        if (gath && !one) {
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const int u = u0 + k * 256;
                if (u < total) {
                    const int c = (u % chunks) * V;
#pragma unroll
                    for (int i = 0; i < V; ++i) ci[k][i] = col_idx[c + i];
                }
            }
        }
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int u = u0 + k * 256;
            if (u < total) {
                const int r = u / chunks;
                const int c = (u % chunks) * V;
                uint4 v;
                if (!gath) {
                    v = *reinterpret_cast<const uint4*>(buf + r * cols + c);
                } else {
                    T* e = reinterpret_cast<T*>(&v);
#pragma unroll
                    for (int i = 0; i < V; ++i) e[i] = buf[r * cols + ci[k][i]];
                }
                *reinterpret_cast<uint4*>(dst + (row0 + r) * cols + c) = v;
            }
        }
    }
}

// Rows too long for LDS: element-wise gather / scatter straight from memory.
template <typename T>
__global__ void permute_direct(const T* __restrict__ src, T* __restrict__ dst, int64_t rows, int64_t cols,
                               const int* __restrict__ row_idx, const int* __restrict__ col_idx, int scatter) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= rows * cols) return;
    const int64_t r = i / cols;
    const int64_t c = i % cols;
    const int64_t sr = row_idx ? row_idx[r] : r;
    if (!col_idx) {
        dst[i] = src[sr * cols + c];
    } else if (scatter) {
        dst[r * cols + col_idx[c]] = src[sr * cols + c];
    } else {
        dst[i] = src[sr * cols + col_idx[c]];
    }
}

// -------------------------------------------------------------- reductions
__global__ void splitk_reduce_kernel(const float* __restrict__ part, float* __restrict__ out, int64_t count,
                                     int splits) {
    const int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i4 >= count) return;
    if (i4 + 4 <= count && (count & 3) == 0) {
        float4 s = *reinterpret_cast<const float4*>(part + i4);
        for (int k = 1; k < splits; ++k) {
            const float4 v = *reinterpret_cast<const float4*>(part + (int64_t)k * count + i4);
            s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
        }
        *reinterpret_cast<float4*>(out + i4) = s;
    } else {
        for (int64_t i = i4; i < min(count, i4 + 4); ++i) {
            float s = part[i];
            for (int k = 1; k < splits; ++k) s += part[(int64_t)k * count + i];
            out[i] = s;
        }
    }
}

// out = c0*in0 + c1*in1 + c2*in2 + gamma*I over nblk b x b blocks (absent
// inputs are skipped); written as float32 and/or in the compute dtype.
template <typename CT>
__global__ void combine_kernel(int64_t total, int b, const float* __restrict__ in0, float c0,
                               const float* __restrict__ in1, float c1, const float* __restrict__ in2, float c2,
                               float gamma, float* __restrict__ out32, CT* __restrict__ outc) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    float v = 0.f;
    if (in0) v += c0 * in0[i];
    if (in1) v += c1 * in1[i];
    if (in2) v += c2 * in2[i];
    if (gamma != 0.f) {
        const int64_t e = i % ((int64_t)b * b);
        if (e / b == e % b) v += gamma;
    }
    if (out32) out32[i] = v;
    if (outc) store_f32(outc + i, v);
}

// The same on four consecutive elements of one row (b % 4 == 0, 16-byte
// aligned arrays): float4 loads and stores.
template <typename CT>
__global__ void combine4_kernel(int64_t total4, int b, const float* __restrict__ in0, float c0,
                                const float* __restrict__ in1, float c1, const float* __restrict__ in2, float c2,
                                float gamma, float* __restrict__ out32, CT* __restrict__ outc) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total4) return;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    auto add = [&](const float* in, float c) {
        const float4 a = reinterpret_cast<const float4*>(in)[i];
        v.x += c * a.x;
        v.y += c * a.y;
        v.z += c * a.z;
        v.w += c * a.w;
    };
    if (in0) add(in0, c0);
    if (in1) add(in1, c1);
    if (in2) add(in2, c2);
    if (gamma != 0.f) {
        const int64_t e = (4 * i) % ((int64_t)b * b);
        const int d = (int)(e / b) - (int)(e % b);   // the diagonal sits at offset d in this group of four
        if (d == 0) v.x += gamma;
        if (d == 1) v.y += gamma;
        if (d == 2) v.z += gamma;
        if (d == 3) v.w += gamma;
    }
    if (out32) reinterpret_cast<float4*>(out32)[i] = v;
    if (outc) {
        if constexpr (sizeof(CT) == 4) {
            reinterpret_cast<float4*>(outc)[i] = v;
        } else {
            reinterpret_cast<uint2*>(outc)[i] = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
        }
    }
}

__global__ void fill_zero_kernel(uint32_t* __restrict__ p, int64_t words) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < words) p[i] = 0u;
}

// sigma[i] = inv_old[pi_new[i]] with inv_old the inverse of pi_old.
__global__ void invert_perm_kernel(const int* __restrict__ pi, int* __restrict__ inv, int64_t len) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < len) inv[pi[i]] = (int)i;
}

__global__ void compose_perm_kernel(const int* __restrict__ inv_old, const int* __restrict__ pi_new,
                                    int* __restrict__ sigma, int64_t len) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < len) sigma[i] = inv_old[pi_new[i]];
}

__global__ void count_perm_kernel(const int* __restrict__ pi, int* __restrict__ counts, int64_t len,
                                  int* __restrict__ bad) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= len) return;
    const int v = pi[i];
    if (v < 0 || v >= len) { atomicOr(bad, 1); return; }
    atomicAdd(&counts[v], 1);
}

__global__ void check_counts_kernel(const int* __restrict__ counts, int64_t len, int* __restrict__ bad) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < len && counts[i] != 1) atomicOr(bad, 1);
}

__global__ void finish_check_kernel(const int* __restrict__ bad, int* __restrict__ ok) {
    if (threadIdx.x == 0 && blockIdx.x == 0) ok[0] = bad[0] ? 0 : 1;
}

// ------------------------------------------------- grouped column gathers
// dst[r][c] = sum_{g < nsum} src[r][idx[g * dst_cols + c]] (float32 sum, one
// rounding), src [rows, src_cols], dst [rows, dst_cols].  With nsum = 1 this
// is a gather between rows of different widths (one input into the gathered
// copies of several linears); with nsum > 1 it adds several gathered slices
// (the input gradient of linears that share that input).  A workgroup stages
// rows_per_wg source rows in LDS, as the permutation kernel does.
template <typename T>
__global__ void __launch_bounds__(256) gather_sum_lds(const T* __restrict__ src, T* __restrict__ dst, int64_t rows,
                                                      int src_cols, int dst_cols, const int* __restrict__ idx,
                                                      int nsum, int rows_per_wg) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    T* buf = reinterpret_cast<T*>(smem_raw);
    constexpr int V = ElemTraits<T>::kVec;
    const int64_t row0 = (int64_t)blockIdx.x * rows_per_wg;
    const int nrows = (int)min<int64_t>(rows_per_wg, rows - row0);
    const int src_chunks = src_cols / V;
    for (int u = threadIdx.x; u < nrows * src_chunks; u += 256) {
        const int r = u / src_chunks;
        const int c = (u % src_chunks) * V;
        *reinterpret_cast<uint4*>(buf + r * src_cols + c) =
            *reinterpret_cast<const uint4*>(src + (row0 + r) * src_cols + c);
    }
    __syncthreads();
    const int dst_chunks = dst_cols / V;
    for (int u = threadIdx.x; u < nrows * dst_chunks; u += 256) {
        const int r = u / dst_chunks;
        const int c = (u % dst_chunks) * V;
        float acc[V];
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = 0.f;
        for (int g = 0; g < nsum; ++g) {
#pragma unroll
            for (int i = 0; i < V; ++i) acc[i] += load_f32(buf + r * src_cols + idx[g * dst_cols + c + i]);
        }
        T v[V];
#pragma unroll
        for (int i = 0; i < V; ++i) store_f32(&v[i], acc[i]);
        uint4 w;
        __builtin_memcpy(&w, v, sizeof(w));
        *reinterpret_cast<uint4*>(dst + (row0 + r) * dst_cols + c) = w;
    }
}

// Rows too long for LDS: the same from global memory, one output per thread.
template <typename T>
__global__ void gather_sum_direct(const T* __restrict__ src, T* __restrict__ dst, int64_t rows, int src_cols,
                                  int dst_cols, const int* __restrict__ idx, int nsum) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= rows * dst_cols) return;
    const int64_t r = i / dst_cols;
    const int c = (int)(i % dst_cols);
    float acc = 0.f;
    for (int g = 0; g < nsum; ++g) acc += load_f32(src + r * src_cols + idx[g * dst_cols + c]);
    store_f32(dst + i, acc);
}

// Offsets for a group of linears: out_R[i] = pi_R[i] + off[g] for i in segment
// g of [0, off[count]); inv_P[g n + pi_P[j]] = j for j in [g n, (g + 1) n).
__global__ void group_perms_kernel(const int* __restrict__ pi_R, const int* __restrict__ pi_P,
                                   int* __restrict__ out_R, int* __restrict__ inv_P, PermSegments seg) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nR = seg.off[seg.count];
    if (i < nR) {
        int64_t o = 0;
        for (int g = 1; g < seg.count; ++g)
            if (i >= seg.off[g]) o = seg.off[g];
        out_R[i] = pi_R[i] + (int)o;
    }
    const int64_t nP = seg.count * seg.n;
    if (i < nP) {
        const int64_t g = i / seg.n;
        inv_P[g * seg.n + pi_P[i]] = (int)i;
    }
}

// ------------------------------------------------------ int8 weight storage
// One workgroup per row: scale = max |w| / 127, q = the integer nearest w /
// scale (ties to even) in [-127, 127], all in float32 with correctly rounded
// divisions; a row of zeros gets scale 0 and codes 0.
template <typename T>
__global__ void __launch_bounds__(256) quantize_rows_kernel(const T* __restrict__ W, int64_t n,
                                                            int8_t* __restrict__ q, float* __restrict__ scale) {
    __shared__ float red[256];
    const int64_t row = blockIdx.x;
    const T* __restrict__ w = W + row * n;
    float amax = 0.f;
    for (int64_t j = threadIdx.x; j < n; j += 256) amax = fmaxf(amax, fabsf(load_f32(w + j)));
    red[threadIdx.x] = amax;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + h]);
        __syncthreads();
    }
    const float sc = red[0] / 127.0f;
    if (threadIdx.x == 0) scale[row] = sc;
    for (int64_t j = threadIdx.x; j < n; j += 256) {
        float v = 0.f;
        if (sc > 0.f) v = fminf(fmaxf(rintf(load_f32(w + j) / sc), -127.f), 127.f);
        q[row * n + j] = static_cast<int8_t>(v);
    }
}

// out[i][j] = bf16(q[i][j] * scale[i]); one thread per 16 codes (n % 16 == 0).
__global__ void __launch_bounds__(256) dequantize_rows_kernel(const int8_t* __restrict__ q,
                                                              const float* __restrict__ scale,
                                                              bf16_t* __restrict__ out, int64_t m, int64_t n) {
    const int64_t chunks = n / 16;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= m * chunks) return;
    const int64_t row = idx / chunks;
    const int64_t c0 = (idx % chunks) * 16;
    const uint4 v = *reinterpret_cast<const uint4*>(q + row * n + c0);
    const float sc = scale[row];
    int8_t e[16];
    __builtin_memcpy(e, &v, sizeof(e));
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = pack_bf16x2((float)e[2 * i] * sc, (float)e[2 * i + 1] * sc);
    uint4* dst = reinterpret_cast<uint4*>(out + row * n + c0);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

// ------------------------------------------- dense block-diagonal transforms
// out (d x d) = Pi^T diag(G_0, G_1, ...) Pi as a dense matrix, inv the inverse
// of pi: out[a][c] = G[i / b][i % b][j % b] with i = inv[a], j = inv[c] when i
// and j fall in the same block, else 0.  One thread writes V consecutive
// outputs of a row (one 16-byte store).
template <typename T>
__global__ void __launch_bounds__(256) blockdiag_dense_kernel(const T* __restrict__ G, const int* __restrict__ inv,
                                                              T* __restrict__ out, int64_t d, int b) {
    constexpr int V = ElemTraits<T>::kVec;
    const int64_t chunks = d / V;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= d * chunks) return;
    const int64_t a = idx / chunks;
    const int64_t c0 = (idx % chunks) * V;
    const int64_t i = inv[a];
    const int64_t blk = i / b;
    const T* __restrict__ grow = G + i * b;  // row i % b of block blk
    T v[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        const int64_t j = inv[c0 + e];
        store_f32(&v[e], j / b == blk ? load_f32(grow + (j - blk * b)) : 0.f);
    }
    uint4 w;
    __builtin_memcpy(&w, v, sizeof(w));
    *reinterpret_cast<uint4*>(out + a * d + c0) = w;
}

// dG[j][r][c] = D[pi[j b + r]][pi[j b + c]]: the diagonal b x b blocks of
// Pi D Pi^T for a dense float32 d x d matrix D.
__global__ void __launch_bounds__(256) blockdiag_gather_kernel(const float* __restrict__ D, const int* __restrict__ pi,
                                                               float* __restrict__ dG, int64_t d, int b) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= d * b) return;
    const int64_t row = idx / b;
    const int64_t col = (row / b) * b + idx % b;
    dG[idx] = D[(int64_t)pi[row] * d + pi[col]];
}

constexpr int64_t kMaxGridY = 65535;

inline unsigned blocks_for(int64_t n, int threads) { return (unsigned)((n + threads - 1) / threads); }

}  // namespace

hipError_t skew_unpack(const float* q, void* Q, bool bf16, int64_t nblk, int b, hipStream_t s, void* Q2_bf16) {
    if (nblk <= 0) return hipSuccess;
    bf16_t* Q2 = static_cast<bf16_t*>(Q2_bf16);
    if (b % kSkewTile == 0) {
        const int64_t ntri = (int64_t)b * (b - 1) / 2, bb = (int64_t)b * b;
        for (int64_t z0 = 0; z0 < nblk; z0 += kMaxGridY) {
            const unsigned nz = (unsigned)std::min<int64_t>(kMaxGridY, nblk - z0);
            dim3 grid((b / kSkewTile) * (b / kSkewTile), nz);
            bf16_t* q2 = Q2 ? Q2 + z0 * bb : nullptr;
            if (bf16)
                hipLaunchKernelGGL(skew_unpack_kernel<bf16_t>, grid, dim3(256), 0, s, q + z0 * ntri,
                                   (bf16_t*)Q + z0 * bb, b, q2);
            else
                hipLaunchKernelGGL(skew_unpack_kernel<float>, grid, dim3(256), 0, s, q + z0 * ntri,
                                   (float*)Q + z0 * bb, b, q2);
        }
    } else {
        const int64_t total = nblk * (int64_t)b * b;
        if (bf16) hipLaunchKernelGGL(skew_unpack_simple<bf16_t>, dim3(blocks_for(total, 256)), dim3(256), 0, s, q,
                                     (bf16_t*)Q, b, total, Q2);
        else hipLaunchKernelGGL(skew_unpack_simple<float>, dim3(blocks_for(total, 256)), dim3(256), 0, s, q,
                                (float*)Q, b, total, Q2);
    }
    return hipGetLastError();
}

hipError_t skew_pack(const float* dQ, float* dq, int64_t nblk, int b, hipStream_t s) {
    if (nblk <= 0) return hipSuccess;
    if (b % kSkewTile == 0) {
        const int64_t ntri = (int64_t)b * (b - 1) / 2, bb = (int64_t)b * b;
        for (int64_t z0 = 0; z0 < nblk; z0 += kMaxGridY) {
            const unsigned nz = (unsigned)std::min<int64_t>(kMaxGridY, nblk - z0);
            const int tiles = b / kSkewTile;
            dim3 grid(tiles * (tiles + 1) / 2, nz);
            hipLaunchKernelGGL(skew_pack_kernel, grid, dim3(256), 0, s, dQ + z0 * bb, dq + z0 * ntri, b);
        }
    } else {
        const int64_t total = nblk * ((int64_t)b * (b - 1) / 2);
        hipLaunchKernelGGL(skew_pack_simple, dim3(blocks_for(total, 256)), dim3(256), 0, s, dQ, dq, b, nblk);
    }
    return hipGetLastError();
}

size_t permute_lds_row_limit_bytes() { return 64 * 1024; }

hipError_t permute_2d(const void* src, void* dst, bool bf16, int64_t rows, int64_t cols, const int* row_idx,
                      const int* col_idx, bool scatter, hipStream_t s) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    const int esz = bf16 ? 2 : 4;
    const int64_t row_bytes = cols * esz;
    if (row_bytes <= (int64_t)permute_lds_row_limit_bytes() && (cols % (16 / esz)) == 0) {
        // The fewest rows that make at least 4 KB per workgroup: many small
        // workgroups keep more loads in flight per CU than a few large ones
        // (measured on 1024- to 14336-column bf16 rows at 2048 to 8192 rows).
        int rpw = (int)std::max<int64_t>(1, (4 * 1024 + row_bytes - 1) / row_bytes);
        rpw = (int)std::min<int64_t>(rpw, rows);
        const size_t smem = (size_t)rpw * row_bytes;
        const unsigned grid = (unsigned)((rows + rpw - 1) / rpw);
        // 16-byte vectors per thread of one workgroup
        const int64_t per = (rpw * row_bytes / 16 + 255) / 256;
        auto go = [&](auto nb_c) {
            constexpr int NB = decltype(nb_c)::value;
            if (bf16)
                hipLaunchKernelGGL((permute_rows_lds<bf16_t, NB>), dim3(grid), dim3(256), smem, s, (const bf16_t*)src,
                                   (bf16_t*)dst, rows, (int)cols, row_idx, col_idx, scatter ? 1 : 0, rpw);
            else
                hipLaunchKernelGGL((permute_rows_lds<float, NB>), dim3(grid), dim3(256), smem, s, (const float*)src,
                                   (float*)dst, rows, (int)cols, row_idx, col_idx, scatter ? 1 : 0, rpw);
        };
        if (per <= 2) go(std::integral_constant<int, 2>{});
        else if (per <= 4) go(std::integral_constant<int, 4>{});
        else go(std::integral_constant<int, 8>{});
    } else {
        const int64_t total = rows * cols;
        if (bf16)
            hipLaunchKernelGGL(permute_direct<bf16_t>, dim3(blocks_for(total, 256)), dim3(256), 0, s,
                               (const bf16_t*)src, (bf16_t*)dst, rows, cols, row_idx, col_idx, scatter ? 1 : 0);
        else
            hipLaunchKernelGGL(permute_direct<float>, dim3(blocks_for(total, 256)), dim3(256), 0, s,
                               (const float*)src, (float*)dst, rows, cols, row_idx, col_idx, scatter ? 1 : 0);
    }
    return hipGetLastError();
}

hipError_t splitk_reduce(const float* part, float* out, int64_t count, int splits, hipStream_t s) {
    if (count <= 0) return hipSuccess;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks_for((count + 3) / 4, 256)), dim3(256), 0, s, part, out,
                       count, splits);
    return hipGetLastError();
}

hipError_t combine(int64_t nblk, int b, const float* in0, float c0, const float* in1, float c1, const float* in2,
                   float c2, float gamma, float* out32, void* outc, bool outc_bf16, hipStream_t s) {
    const int64_t total = nblk * (int64_t)b * b;
    if (total <= 0) return hipSuccess;
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    if (b % 4 == 0 && al16(in0) && al16(in1) && al16(in2) && al16(out32) && al16(outc)) {
        const int64_t total4 = total / 4;
        if (outc_bf16)
            hipLaunchKernelGGL(combine4_kernel<bf16_t>, dim3(blocks_for(total4, 256)), dim3(256), 0, s, total4, b,
                               in0, c0, in1, c1, in2, c2, gamma, out32, (bf16_t*)outc);
        else
            hipLaunchKernelGGL(combine4_kernel<float>, dim3(blocks_for(total4, 256)), dim3(256), 0, s, total4, b,
                               in0, c0, in1, c1, in2, c2, gamma, out32, (float*)outc);
        return hipGetLastError();
    }
    if (outc_bf16)
        hipLaunchKernelGGL(combine_kernel<bf16_t>, dim3(blocks_for(total, 256)), dim3(256), 0, s, total, b, in0, c0,
                           in1, c1, in2, c2, gamma, out32, (bf16_t*)outc);
    else
        hipLaunchKernelGGL(combine_kernel<float>, dim3(blocks_for(total, 256)), dim3(256), 0, s, total, b, in0, c0,
                           in1, c1, in2, c2, gamma, out32, (float*)outc);
    return hipGetLastError();
}

hipError_t fill_zero(void* p, size_t bytes, hipStream_t s) {
    const int64_t words = (int64_t)(bytes / 4);
    if (words <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks_for(words, 256)), dim3(256), 0, s, (uint32_t*)p, words);
    return hipGetLastError();
}

hipError_t compose_perm(const int* pi_old, const int* pi_new, int* inv_tmp, int* sigma, int64_t len,
                        hipStream_t s) {
    if (len <= 0) return hipSuccess;
    hipLaunchKernelGGL(invert_perm_kernel, dim3(blocks_for(len, 256)), dim3(256), 0, s, pi_old, inv_tmp, len);
    hipLaunchKernelGGL(compose_perm_kernel, dim3(blocks_for(len, 256)), dim3(256), 0, s, inv_tmp, pi_new, sigma,
                       len);
    return hipGetLastError();
}

hipError_t gather_sum(const void* src, void* dst, bool bf16, int64_t rows, int64_t src_cols, int64_t dst_cols,
                      const int* idx, int nsum, hipStream_t s) {
    if (rows <= 0 || dst_cols <= 0) return hipSuccess;
    const int esz = bf16 ? 2 : 4;
    const int V = 16 / esz;
    const int64_t row_bytes = src_cols * esz;
    if (row_bytes <= (int64_t)permute_lds_row_limit_bytes() && src_cols % V == 0 && dst_cols % V == 0) {
        int rpw = (int)std::max<int64_t>(1, (4 * 1024 + row_bytes - 1) / row_bytes);
        rpw = (int)std::min<int64_t>({rpw, rows, (int64_t)permute_lds_row_limit_bytes() / row_bytes});
        const size_t smem = (size_t)rpw * row_bytes;
        const unsigned grid = (unsigned)((rows + rpw - 1) / rpw);
        if (bf16)
            hipLaunchKernelGGL(gather_sum_lds<bf16_t>, dim3(grid), dim3(256), smem, s, (const bf16_t*)src,
                               (bf16_t*)dst, rows, (int)src_cols, (int)dst_cols, idx, nsum, rpw);
        else
            hipLaunchKernelGGL(gather_sum_lds<float>, dim3(grid), dim3(256), smem, s, (const float*)src,
                               (float*)dst, rows, (int)src_cols, (int)dst_cols, idx, nsum, rpw);
    } else {
        const int64_t total = rows * dst_cols;
        if (bf16)
            hipLaunchKernelGGL(gather_sum_direct<bf16_t>, dim3(blocks_for(total, 256)), dim3(256), 0, s,
                               (const bf16_t*)src, (bf16_t*)dst, rows, (int)src_cols, (int)dst_cols, idx, nsum);
        else
            hipLaunchKernelGGL(gather_sum_direct<float>, dim3(blocks_for(total, 256)), dim3(256), 0, s,
                               (const float*)src, (float*)dst, rows, (int)src_cols, (int)dst_cols, idx, nsum);
    }
    return hipGetLastError();
}

hipError_t group_perms(const int* pi_R, const int* pi_P, int* out_R, int* inv_P, const PermSegments& seg,
                       hipStream_t s) {
    const int64_t len = std::max<int64_t>(seg.off[seg.count], (int64_t)seg.count * seg.n);
    if (len <= 0) return hipSuccess;
    hipLaunchKernelGGL(group_perms_kernel, dim3(blocks_for(len, 256)), dim3(256), 0, s, pi_R, pi_P, out_R, inv_P,
                       seg);
    return hipGetLastError();
}

hipError_t quantize_rows(const void* W, bool bf16, int64_t m, int64_t n, int8_t* q, float* scale, hipStream_t s) {
    if (m <= 0 || n <= 0) return hipSuccess;
    if (m > 0x7fffffff) return hipErrorInvalidValue;
    if (bf16)
        hipLaunchKernelGGL(quantize_rows_kernel<bf16_t>, dim3((unsigned)m), dim3(256), 0, s, (const bf16_t*)W, n, q,
                           scale);
    else
        hipLaunchKernelGGL(quantize_rows_kernel<float>, dim3((unsigned)m), dim3(256), 0, s, (const float*)W, n, q,
                           scale);
    return hipGetLastError();
}

hipError_t dequantize_rows(const int8_t* q, const float* scale, void* out, int64_t m, int64_t n, hipStream_t s) {
    if (m <= 0 || n <= 0) return hipSuccess;
    if (n % 16 || ((uintptr_t)q & 15) || ((uintptr_t)out & 15)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(dequantize_rows_kernel, dim3(blocks_for(m * (n / 16), 256)), dim3(256), 0, s, q, scale,
                       (bf16_t*)out, m, n);
    return hipGetLastError();
}

hipError_t invert_perm(const int* pi, int* inv, int64_t len, hipStream_t s) {
    if (len <= 0) return hipSuccess;
    hipLaunchKernelGGL(invert_perm_kernel, dim3(blocks_for(len, 256)), dim3(256), 0, s, pi, inv, len);
    return hipGetLastError();
}

hipError_t blockdiag_dense(const void* G, const int* inv, void* out, bool bf16, int64_t d, int b, hipStream_t s) {
    if (d <= 0) return hipSuccess;
    const int V = bf16 ? 8 : 4;
    if (d % b || d % V || ((uintptr_t)out & 15)) return hipErrorInvalidValue;
    const int64_t threads = d * (d / V);
    if (bf16)
        hipLaunchKernelGGL(blockdiag_dense_kernel<bf16_t>, dim3(blocks_for(threads, 256)), dim3(256), 0, s,
                           (const bf16_t*)G, inv, (bf16_t*)out, d, b);
    else
        hipLaunchKernelGGL(blockdiag_dense_kernel<float>, dim3(blocks_for(threads, 256)), dim3(256), 0, s,
                           (const float*)G, inv, (float*)out, d, b);
    return hipGetLastError();
}

hipError_t blockdiag_gather(const float* D, const int* pi, float* dG, int64_t d, int b, hipStream_t s) {
    if (d <= 0) return hipSuccess;
    if (d % b) return hipErrorInvalidValue;
    hipLaunchKernelGGL(blockdiag_gather_kernel, dim3(blocks_for(d * b, 256)), dim3(256), 0, s, D, pi, dG, d, b);
    return hipGetLastError();
}

hipError_t check_perm(const int* pi, int64_t len, int* ok, int* counts, int* bad, hipStream_t s) {
    hipError_t e = fill_zero(counts, (size_t)(len + 1) * sizeof(int), s);
    if (e != hipSuccess) return e;
    if (len > 0) {
        hipLaunchKernelGGL(count_perm_kernel, dim3(blocks_for(len, 256)), dim3(256), 0, s, pi, counts, len, bad);
        hipLaunchKernelGGL(check_counts_kernel, dim3(blocks_for(len, 256)), dim3(256), 0, s, counts, len, bad);
    }
    hipLaunchKernelGGL(finish_check_kernel, dim3(1), dim3(64), 0, s, bad, ok);
    return hipGetLastError();
}

}  // namespace poetx
