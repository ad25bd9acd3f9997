// tiles.hpp -- LDS tile helpers of the vector kernels (generic.hip,
// backward.hip): row loads, row norms and the feature map of a token tile.
#pragma once

#include "common.hpp"

namespace linattn {

constexpr int VNT = 256; // threads per workgroup of the vector kernels

// Copies `rows` rows of a [*, 64] matrix (zero rows after `rows`, up to L)
// into dst[L][64] as scale * x.
template <typename T, int L>
__device__ void load_rows(const T* __restrict__ src, int rows, float scale, float* dst) {
    for (int g = threadIdx.x; g < L * (D / 4); g += VNT) {
        const int row = g / (D / 4), c4 = (g % (D / 4)) * 4;
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row < rows) x = Elem<T>::load4(src, (long)row * D + c4);
        float* o = dst + row * D + c4;
        o[0] = scale * x.x;
        o[1] = scale * x.y;
        o[2] = scale * x.z;
        o[3] = scale * x.w;
    }
}

// nrm[t] = |u_t|^2 for the L rows of u[L][64] (one wave per row).
template <int L>
__device__ void row_norms(const float* u, float* nrm) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int t = w; t < L; t += VNT / 64) {
        float a = u[t * D + lane];
        float s = wave_sum(a * a);
        if (lane == 0) nrm[t] = s;
    }
}

// Optional sum normalisation of a feature tile out[L][r] (row stride ol):
// rs[t] = 1 / max(sum_f, eps) and, when `live` is given, live[t] = 1 where
// the sum exceeds eps (the clamp does not hold); rows are scaled by rs.
// The tile must be complete (caller synchronised).  Ends with a barrier.
template <int L>
__device__ void sum_normalize(const Cfg& c, float* out, int ol, float* rs, float* live) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    for (int t = w; t < L; t += VNT / 64) {
        float s = 0.f;
        for (int f = lane; f < c.r; f += 64) s += out[t * ol + f];
        s = wave_sum(s);
        if (lane == 0) {
            rs[t] = 1.f / fmaxf(s, c.eps);
            if (live) live[t] = s > c.eps ? 1.f : 0.f;
        }
    }
    __syncthreads();
    for (int idx = tid; idx < L * c.r; idx += VNT) {
        const int t = idx / c.r, f = idx - t * c.r;
        out[t * ol + f] *= rs[t];
    }
    __syncthreads();
}

// out[t][f] = phi_f(u_t) for t < L, f < r (rows >= `rows` are zero), then the
// optional sum normalisation (sum_normalize).  u, nrm must be complete
// (caller synchronised).  Ends with a barrier.
template <typename T, int L>
__device__ void phi_tile(const Cfg& c, const float* u, const float* nrm,
                         const T* __restrict__ omega, int rows, float* out, int ol, float* rs,
                         float* live = nullptr) {
    const int tid = threadIdx.x;
    if (c.phi == PHI_FAVOR) {
        for (int f = tid; f < c.r; f += VNT) {
            float w[D];
#pragma unroll
            for (int i = 0; i < D; i += 4) {
                float4 x = Elem<T>::load4(omega, (long)f * D + i);
                w[i] = x.x;
                w[i + 1] = x.y;
                w[i + 2] = x.z;
                w[i + 3] = x.w;
            }
            for (int t = 0; t < L; ++t) {
                float dot = 0.f;
#pragma unroll
                for (int i = 0; i < D; ++i) dot = fmaf(w[i], u[t * D + i], dot);
                out[t * ol + f] = t < rows ? favor_feature(c, dot, nrm[t]) : 0.f;
            }
        }
    } else {
        for (int idx = tid; idx < L * c.r; idx += VNT) {
            const int t = idx / c.r, f = idx - t * c.r;
            float y = 0.f;
            if (t < rows) y = phi_feature<T>(c, u + t * D, 0.f, f, omega);
            out[t * ol + f] = y;
        }
    }
    __syncthreads();
    if (c.sum_norm) sum_normalize<L>(c, out, ol, rs, live);
}

} // namespace linattn
