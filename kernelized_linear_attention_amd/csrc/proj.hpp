// proj.hpp -- the q/k/v input projection of a chunk of tokens, fused into
// the loads of the vector kernels (Kernel Zoo sec. 1.2 step 1:
// k, v, q = W_k x, W_v x, W_q x for every token x).
//
// One wave computes one 32 x 32 tile of u = x W^T with 32x32x16 bfloat16
// matrix-core products and float32 accumulation.  Both operands come
// straight from global memory: a lane reads 8 consecutive bfloat16 of one
// row of x (the A operand) and of one row of W (the B operand, W^T's
// column), 16 bytes each.  The head's 64 rows of each W stay in L2 and are
// re-read by every chunk: they do not fit in LDS beside the attention
// tiles (3 x 64 x dm bfloat16 is 192 KB at dm = 512).  The result goes to
// a float tile in LDS, scaled, so q, k and v never exist in HBM.
#pragma once

#include "tiles.hpp"

namespace linattn {

enum : int { PROJ_Q = 0, PROJ_K = 1, PROJ_V = 2 };

struct Proj {
    const bf16_raw* x;    // [B, N, dm] tokens
    const bf16_raw* w[3]; // W_q, W_k, W_v: [H * 64, dm]; row h*64 + i is output i of head h
    int64_t dm;           // model width, a multiple of 16
    int64_t H;            // heads (the kernels' bh = b * H + h)
};

typedef __bf16 pj_bf16x8 __attribute__((ext_vector_type(8)));
typedef float pj_f32x16 __attribute__((ext_vector_type(16)));

// One 32 x 32 tile: dst[rb*32 + t][ct*32 + n] = scale * sum_c x[t0 + rb*32 + t][c] W[h*64 + ct*32 + n][c]
// for t < 32 (rows at or past `rows` are zero); dst row stride 64.
__device__ __forceinline__ void project_tile(const Proj& P, const bf16_raw* __restrict__ w,
                                             int64_t b, int64_t h, int64_t N, int64_t t0, int rows,
                                             int rb, int ct, float scale, float* dst) {
    const int lane = threadIdx.x & 63;
    const int r = rb * 32 + (lane & 31);
    const int kq = 8 * (lane >> 5);
    const bool valid = r < rows;
    const bf16_raw* xa = P.x + (b * N + t0 + (valid ? r : 0)) * P.dm + kq;
    const bf16_raw* wb = w + (h * 64 + ct * 32 + (lane & 31)) * P.dm + kq;
    pj_f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll 4
    for (int64_t c = 0; c < P.dm; c += 16) {
        uint4 av = make_uint4(0u, 0u, 0u, 0u);
        if (valid) av = *reinterpret_cast<const uint4*>(xa + c);
        const uint4 bv = *reinterpret_cast<const uint4*>(wb + c);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(pj_bf16x8, av),
                                                      __builtin_bit_cast(pj_bf16x8, bv), acc, 0, 0,
                                                      0);
    }
    // accumulator i of lane l holds row 8(i/4) + 4(l/32) + i%4, column l%32
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int row = rb * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        dst[row * 64 + ct * 32 + (lane & 31)] = scale * acc[i];
    }
}

// Projects the L-row chunk starting at token t0 of head bh through up to two
// matrices: m0 -> dst0 (scaled by s0) and, when m1 >= 0, m1 -> dst1 (s1).
// The 32 x 32 tiles are dealt to the workgroup's waves in turn.  The caller
// synchronises before the tiles are read.
template <int L>
__device__ void project_chunk(const Proj& P, int64_t bh, int64_t N, int64_t t0, int rows, int m0,
                              float* dst0, float s0, int m1, float* dst1, float s1) {
    static_assert(L % 32 == 0 && L >= 32, "the projection deals whole 32-row tiles");
    constexpr int RB = L / 32;
    const int64_t b = bh / P.H, h = bh % P.H;
    const int nt = (m1 >= 0 ? 2 : 1) * RB * 2;
    for (int tile = threadIdx.x >> 6; tile < nt; tile += VNT / 64) {
        const int which = tile / (RB * 2), rb = (tile >> 1) % RB, ct = tile & 1;
        if (which == 0)
            project_tile(P, P.w[m0], b, h, N, t0, rows, rb, ct, s0, dst0);
        else
            project_tile(P, P.w[m1], b, h, N, t0, rows, rb, ct, s1, dst1);
    }
}

} // namespace linattn
