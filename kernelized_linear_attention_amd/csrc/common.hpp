// common.hpp -- device-side helpers shared by the kernels of liblinattn.so:
// element loads/stores for float32 and bfloat16, and the per-feature maps.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace linattn {

constexpr int D = 64;     // query/key width handled by the kernels
constexpr int DV = 64;    // value width handled by the kernels
constexpr int RMAX = 512; // largest feature width of the forward and decode kernels
constexpr int RMAX_BWD = 256; // largest feature width of the backward and projected calls
constexpr float LOG2E = 1.4426950408889634f;

enum : int { PHI_IDENTITY = 0, PHI_ELU1 = 1, PHI_FAVOR = 2, PHI_DPFP = 3 };
enum : int { NORM_ATTN = 0, NORM_NONE = 1 };

// Method parameters as the kernels see them.
struct Cfg {
    int phi;
    int r;
    int nu;
    int sum_norm;
    int norm;
    float scale;
    float eps;
    float favor_log2_bias; // log2(1/sqrt(r)): the 1/sqrt(m) factor folded into exp2
};

// bfloat16 is carried as its raw 16 bits.
using bf16_raw = uint16_t;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float32 -> bfloat16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ bf16_raw f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_raw)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16_raw)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float* p, long i) { return p[i]; }
    static __device__ __forceinline__ float4 load4(const float* p, long i) {
        return *reinterpret_cast<const float4*>(p + i);
    }
    static __device__ __forceinline__ void store(float* p, long i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_raw> {
    static __device__ __forceinline__ float load(const bf16_raw* p, long i) { return bf16_to_f32(p[i]); }
    static __device__ __forceinline__ float4 load4(const bf16_raw* p, long i) {
        uint2 w = *reinterpret_cast<const uint2*>(p + i);
        return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                           __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
    }
    static __device__ __forceinline__ void store(bf16_raw* p, long i, float v) { p[i] = f32_to_bf16(v); }
};

// ELU with alpha = 1, plus one (Kernel Zoo running example): x + 1 for x > 0,
// exp(x) for x <= 0 (there elu(x) + 1 = exp(x) - 1 + 1).
__device__ __forceinline__ float elu1(float x) { return x > 0.f ? x + 1.f : expf(x); }

// DPFP input doubling (Kernel Zoo sec. 6.3): kt_j = relu([u, -u])_j, j < 2d.
__device__ __forceinline__ float dpfp_kt(const float* u, int j) {
    return j < D ? fmaxf(u[j], 0.f) : fmaxf(-u[j - D], 0.f);
}

// DPFP-nu feature f (Kernel Zoo sec. 6.3): block s = f / 2d + 1 holds
// kt_i * kt_{(i + s) mod 2d} with i = f mod 2d.
__device__ __forceinline__ float dpfp_feature(const float* u, int f) {
    const int i = f & (2 * D - 1);
    const int s = f / (2 * D) + 1;
    return dpfp_kt(u, i) * dpfp_kt(u, (i + s) & (2 * D - 1));
}

// FAVOR+ feature from the projection dot = omega_f . u and nrm = |u|^2
// (Kernel Zoo sec. 4.2): exp(dot - nrm/2) / sqrt(r), evaluated as one exp2.
__device__ __forceinline__ float favor_feature(const Cfg& c, float dot, float nrm) {
    return exp2f(fmaf(dot - 0.5f * nrm, LOG2E, c.favor_log2_bias));
}

// phi_f(u) for one feature of one already-scaled input vector u[D] in LDS.
template <typename T>
__device__ __forceinline__ float phi_feature(const Cfg& c, const float* u, float nrm, int f,
                                             const T* __restrict__ omega) {
    switch (c.phi) {
    case PHI_IDENTITY:
        return u[f];
    case PHI_ELU1:
        return elu1(u[f]);
    case PHI_DPFP:
        return dpfp_feature(u, f);
    default: {
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < D; i += 4) {
            float4 w = Elem<T>::load4(omega, (long)f * D + i);
            dot = fmaf(w.x, u[i], dot);
            dot = fmaf(w.y, u[i + 1], dot);
            dot = fmaf(w.z, u[i + 2], dot);
            dot = fmaf(w.w, u[i + 3], dot);
        }
        return favor_feature(c, dot, nrm);
    }
    }
}

// Workgroup barrier for LDS traffic only.  __syncthreads() also waits for
// every outstanding global load (its fence covers global memory), which
// drains the prefetches a loop keeps in flight; use this where the waves
// communicate through LDS alone.
__device__ __forceinline__ void sync_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt vmcnt(0) as a builtin (expcnt and lgkmcnt at their maxima), so
// the compiler's load counting sees it, unlike the same instruction in
// inline asm.  Placed before a loop that uses registers loaded ahead of it:
// the counting merges the loop entry with the back edge and would otherwise
// wait for every load in flight, the loop's own prefetches included, at the
// first use of such a register in every iteration.
__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

} // namespace linattn
