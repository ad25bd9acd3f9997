// orf.hip -- orthogonal random features built on the device (Performer page
// sec. 2 step 4; Kernel Zoo sec. 5.1-5.3): every block of d rows of omega is
// Gram-Schmidt of the rows of a d x d Gaussian matrix, each row then scaled
// to the length of an independent Gaussian vector (or to sqrt(d)).  The
// Gaussian draws are inputs: the caller's generator makes them.
//
// One wave per (matrix, block), d <= 64.  The block is orthogonalised in
// float64 in LDS, row by row in order; each row has its projections on the
// earlier rows removed twice (classical Gram-Schmidt with one
// reorthogonalisation pass: the pages' procedure in exact arithmetic, and
// orthogonal to float64 precision in floating point).  Lane j forms the dot
// product with earlier row j by a loop over the columns and lane k updates
// column k, so no step needs a cross-lane reduction except the row norm;
// a single wave needs no barrier (its LDS accesses complete in order).
#include "launch.hpp"

namespace linattn {
namespace {

constexpr int NT = 64;
constexpr int DMAX = 64;
constexpr int LD = DMAX + 1; // LDS row stride (doubles)

__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// DC: the row length as a constant (64: every loop unrolls, so the LDS reads
// of a dot product are issued together), or 0 for any d <= 64.
template <typename T, int DC>
__global__ __launch_bounds__(NT) void k_orf(const float* __restrict__ gauss,
                                            const float* __restrict__ len_gauss, int64_t r, int d_,
                                            int64_t nblk, T* __restrict__ omega) {
    const int d = DC ? DC : d_;
    constexpr int DCU = DC ? DC : 1; // the unroll count of the dot products
    __shared__ double e_s[DMAX * LD];
    __shared__ double c_s[DMAX];
    const int lane = threadIdx.x;
    const int64_t m = blockIdx.x / nblk, b = blockIdx.x % nblk;
    const float* g = gauss + (m * nblk + b) * d * d;

    for (int x = lane; x < d * d; x += NT) e_s[(x / d) * LD + x % d] = (double)g[x];

    for (int i = 0; i < d; ++i) {
        double* ei = e_s + i * LD;
        for (int pass = 0; pass < 2; ++pass) {
            if (lane < i) { // c_j = e_j . e_i
                const double* ej = e_s + lane * LD;
                double c[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll DCU
                for (int k = 0; k < d; ++k) c[k & 3] = fma(ej[k], ei[k], c[k & 3]);
                c_s[lane] = (c[0] + c[1]) + (c[2] + c[3]);
            }
            if (lane < d) { // e_i -= sum_j c_j e_j
                double x = ei[lane];
                for (int j = 0; j < i; ++j) x = fma(-c_s[j], e_s[j * LD + lane], x);
                ei[lane] = x;
            }
        }
        const double x = lane < d ? ei[lane] : 0.0;
        const double n2 = wave_sum_d(x * x);
        if (lane < d) ei[lane] = x / sqrt(n2);
    }

    // rows of this block that exist (the last block may be cut at r)
    const int rows = (int)min<int64_t>(d, r - b * d);
    for (int i = 0; i < rows; ++i) {
        const int64_t f = b * d + i;
        double len = sqrt((double)d);
        if (len_gauss) {
            const float* lg = len_gauss + (m * nblk * d + f) * d;
            len = sqrt(wave_sum_d(lane < d ? (double)lg[lane] * (double)lg[lane] : 0.0));
        }
        if (lane < d) Elem<T>::store(omega, (m * r + f) * d + lane, (float)(e_s[i * LD + lane] * len));
    }
}

} // namespace

hipError_t launch_orf(const float* gauss, const float* len_gauss, int64_t n_mat, int64_t r, int d,
                      int dtype, void* omega, hipStream_t st) {
    const int64_t nblk = (r + d - 1) / d;
    const dim3 grid((unsigned)(n_mat * nblk)), block(NT);
    if (dtype == 0) {
        if (d == DMAX)
            hipLaunchKernelGGL((k_orf<float, DMAX>), grid, block, 0, st, gauss, len_gauss, r, d,
                               nblk, (float*)omega);
        else
            hipLaunchKernelGGL((k_orf<float, 0>), grid, block, 0, st, gauss, len_gauss, r, d, nblk,
                               (float*)omega);
    } else {
        if (d == DMAX)
            hipLaunchKernelGGL((k_orf<bf16_raw, DMAX>), grid, block, 0, st, gauss, len_gauss, r, d,
                               nblk, (bf16_raw*)omega);
        else
            hipLaunchKernelGGL((k_orf<bf16_raw, 0>), grid, block, 0, st, gauss, len_gauss, r, d,
                               nblk, (bf16_raw*)omega);
    }
    return hipGetLastError();
}

} // namespace linattn
