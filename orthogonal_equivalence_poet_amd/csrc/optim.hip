// AdamW on the compact skew parameters q and the reset of its moments.
//
// The optimizer only ever sees the b(b-1)/2 upper-triangle values per block, so
// its state is the same size as q (the SAI replication review's point that
// POET-X keeps optimizer state on the compact parameters only).  The update is
// decoupled-decay AdamW (Loshchilov and Hutter, 2019) with Adam's bias-corrected
// moments (Kingma and Ba, 2015), run at the POET-scaled rate lr * gamma (gamma =
// 0.5 on the pages: R - I is about 2Q, so a step in q moves R twice as far).
//
// The kernel is a pure stream: per element it reads q, dq, m, v (16 bytes) and
// writes q, m, v (12 bytes), in float4 when all four pointers are 16-byte
// aligned.  Each thread owns kUnroll float4 slots a workgroup-width apart, loads
// all of them before the arithmetic, and the grid covers the array once (no
// grid-stride loop: the arrays are large, one wave of work per slot).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "elementwise.h"

namespace poetx {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 2;

__device__ __forceinline__ void adamw_one(float& q, float g, float& m, float& v, const AdamwCoef& c) {
    m = c.beta1 * m + c.one_minus_beta1 * g;
    v = c.beta2 * v + c.one_minus_beta2 * (g * g);
    const float den = sqrtf(v) * c.inv_sqrt_bc2 + c.eps;
    q = q * c.decay - c.step * (m / den);
}

__global__ __launch_bounds__(kThreads) void adamw_vec_kernel(float* __restrict__ q, const float* __restrict__ g,
                                                             float* __restrict__ m, float* __restrict__ v,
                                                             int64_t n4, int64_t count, AdamwCoef c) {
    const int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
    float4 qv[kUnroll], gv[kUnroll], mv[kUnroll], vv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kThreads;
        if (i < n4) {
            qv[u] = reinterpret_cast<const float4*>(q)[i];
            gv[u] = reinterpret_cast<const float4*>(g)[i];
            mv[u] = reinterpret_cast<const float4*>(m)[i];
            vv[u] = reinterpret_cast<const float4*>(v)[i];
        }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kThreads;
        if (i < n4) {
            adamw_one(qv[u].x, gv[u].x, mv[u].x, vv[u].x, c);
            adamw_one(qv[u].y, gv[u].y, mv[u].y, vv[u].y, c);
            adamw_one(qv[u].z, gv[u].z, mv[u].z, vv[u].z, c);
            adamw_one(qv[u].w, gv[u].w, mv[u].w, vv[u].w, c);
            reinterpret_cast<float4*>(q)[i] = qv[u];
            reinterpret_cast<float4*>(m)[i] = mv[u];
            reinterpret_cast<float4*>(v)[i] = vv[u];
        }
    }
    // The count % 4 trailing elements go to the first threads of the grid.
    const int64_t t = 4 * n4 + (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t < count) {
        float qs = q[t], ms = m[t], vs = v[t];
        adamw_one(qs, g[t], ms, vs, c);
        q[t] = qs;
        m[t] = ms;
        v[t] = vs;
    }
}

__global__ __launch_bounds__(kThreads) void adamw_scalar_kernel(float* __restrict__ q, const float* __restrict__ g,
                                                                float* __restrict__ m, float* __restrict__ v,
                                                                int64_t count, AdamwCoef c) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= count) return;
    float qs = q[i], ms = m[i], vs = v[i];
    adamw_one(qs, g[i], ms, vs, c);
    q[i] = qs;
    m[i] = ms;
    v[i] = vs;
}

__global__ __launch_bounds__(kThreads) void zero2_kernel(float* __restrict__ a, float* __restrict__ b, int64_t count) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < count) {
        a[i] = 0.f;
        b[i] = 0.f;
    }
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t adamw_step(float* q, const float* g, float* m, float* v, int64_t count, const AdamwCoef& c, hipStream_t s) {
    if (count <= 0) return hipSuccess;
    if (aligned16(q) && aligned16(g) && aligned16(m) && aligned16(v)) {
        const int64_t n4 = count / 4;
        const int64_t per_block = (int64_t)kThreads * kUnroll;
        // At least one workgroup so that a count below 4 still reaches the tail.
        const int64_t blocks = n4 > 0 ? (n4 + per_block - 1) / per_block : 1;
        hipLaunchKernelGGL(adamw_vec_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, q, g, m, v, n4, count, c);
    } else {
        const int64_t blocks = (count + kThreads - 1) / kThreads;
        hipLaunchKernelGGL(adamw_scalar_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, q, g, m, v, count, c);
    }
    return hipGetLastError();
}

hipError_t zero_pair(float* a, float* b, int64_t count, hipStream_t s) {
    if (count <= 0) return hipSuccess;
    const int64_t blocks = (count + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(zero2_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, a, b, count);
    return hipGetLastError();
}

}  // namespace poetx
