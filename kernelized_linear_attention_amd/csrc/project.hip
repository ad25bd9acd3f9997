// project.hip -- the q/k/v input projection as one matrix-core GEMM whose
// epilogue writes the attention kernels' head-major layout (Kernel Zoo sec.
// 1.2 step 1: k, v, q = W_k x, W_v x, W_q x for every token x).
//
// The three weight matrices are taken as one [3*H*d, dm] matrix (rows of
// W_q, then W_k, then W_v), so one launch computes all of y = x W^T for the
// M = B*N tokens.  Tiles of 128 tokens x 128 output columns, K in steps of
// 32; four waves, each a 64 x 64 block of 2 x 2 32x32x16 bf16 MFMA tiles
// with float32 accumulation.  A and B tiles are double-buffered in LDS
// (rows padded to 40 elements, so the 16-byte fragment reads of 16 lanes
// hit distinct banks), the next K tiles are fetched into registers while the
// current one is multiplied (two steps in flight), one barrier per K step.  The epilogue rounds to
// bf16, stages the 128 x 128 tile through LDS and writes each 64-column
// half as rows of one head of q, k or v: [B, H, N, d] for each, d = 64.
#include "launch.hpp"

namespace linattn {
namespace {

typedef __bf16 gm_bf16x8 __attribute__((ext_vector_type(8)));
typedef float gm_f32x16 __attribute__((ext_vector_type(16)));

constexpr int GT = 256;   // threads: 4 waves, 2 x 2 blocks of 64 x 64
constexpr int BM = 128;   // tokens per tile
constexpr int BN = 128;   // output columns per tile
constexpr int BK = 32;    // reduction step
constexpr int LDK = 40;   // LDS row length (elements) of the A and B tiles
constexpr int LDO = 136;  // LDS row length of the output tile
constexpr int AP = BM * BK / 8 / GT; // 16-byte pieces per thread per A tile (2)
constexpr int BP = BN * BK / 8 / GT; // per B tile (2)
constexpr int STAGE = (BM + BN) * LDK; // elements of one LDS stage

struct ProjArgs {
    const bf16_raw* x;    // [M, dm]
    const bf16_raw* w[3]; // [H*d, dm] each
    bf16_raw* out[3];     // [B, H, N, d] each
    int64_t M, N, dm, H, cols; // cols = 3*H*d
};

__device__ __forceinline__ const bf16_raw* w_row(const ProjArgs& a, int64_t c) {
    const int64_t hd = a.H * 64;
    const int which = (int)(c / hd);
    return a.w[which] + (c - which * hd) * a.dm;
}

// Global -> registers: 16-byte piece p of a tile row holds K elements
// 8p .. 8p+7 of the step; thread t takes pieces t, t + GT, ... of the A tile
// (row = piece / 8) and of the B tile.  pa / pb: this thread's row starts,
// fixed for the block; rows past the matrix are clamped to its last row (their
// products are never stored).  Every load is unconditional, so the compiler
// can count the loads in flight and wait for one K step's alone.
struct Rows {
    const bf16_raw* pa[AP];
    const bf16_raw* pb[BP];
};

__device__ __forceinline__ Rows tile_rows(const ProjArgs& a, int64_t m0, int64_t n0) {
    Rows r;
#pragma unroll
    for (int j = 0; j < AP; ++j) {
        const int64_t m = min<int64_t>(m0 + (threadIdx.x + j * GT) / (BK / 8), a.M - 1);
        r.pa[j] = a.x + m * a.dm + 8 * (threadIdx.x % (BK / 8));
    }
#pragma unroll
    for (int j = 0; j < BP; ++j) {
        const int64_t n = min<int64_t>(n0 + (threadIdx.x + j * GT) / (BK / 8), a.cols - 1);
        r.pb[j] = w_row(a, n) + 8 * (threadIdx.x % (BK / 8));
    }
    return r;
}

// Whether this thread's pieces of K step s lie inside the rows (dm is a
// multiple of 16, so only the last step can end early); GT is a multiple of
// BK / 8, so every piece of a thread has the same K.
__device__ __forceinline__ bool k_inside(const ProjArgs& a, int64_t s) {
    return s * BK + 8 * (threadIdx.x % (BK / 8)) < a.dm;
}

// Loads of K step s; pieces past dm read the row start instead (in bounds)
// and are zeroed before they are stashed.
__device__ __forceinline__ void fetch(const ProjArgs& a, const Rows& r, int64_t s,
                                      uint4 (&ra)[AP], uint4 (&rb)[BP]) {
    const int64_t k0 = k_inside(a, s) ? s * BK : 0;
#pragma unroll
    for (int j = 0; j < AP; ++j) ra[j] = *reinterpret_cast<const uint4*>(r.pa[j] + k0);
#pragma unroll
    for (int j = 0; j < BP; ++j) rb[j] = *reinterpret_cast<const uint4*>(r.pb[j] + k0);
}

__device__ __forceinline__ void stash(bf16_raw* st, const uint4 (&ra)[AP], const uint4 (&rb)[BP]) {
    bf16_raw* As = st;
    bf16_raw* Bs = st + BM * LDK;
#pragma unroll
    for (int j = 0; j < AP; ++j) {
        const int piece = threadIdx.x + j * GT;
        *reinterpret_cast<uint4*>(As + (piece / (BK / 8)) * LDK + 8 * (piece % (BK / 8))) = ra[j];
    }
#pragma unroll
    for (int j = 0; j < BP; ++j) {
        const int piece = threadIdx.x + j * GT;
        *reinterpret_cast<uint4*>(Bs + (piece / (BK / 8)) * LDK + 8 * (piece % (BK / 8))) = rb[j];
    }
}

// Stash of K step s: a last step that ends inside the tile (dm % BK = 16)
// has its pieces past dm zeroed first (a uniform branch: the masking runs
// only there).
__device__ __forceinline__ void stash_step(const ProjArgs& a, int64_t s, int64_t KT, bf16_raw* st,
                                           uint4 (&ra)[AP], uint4 (&rb)[BP]) {
    if (s + 1 == KT && a.dm % BK != 0 && !k_inside(a, s)) {
#pragma unroll
        for (int j = 0; j < AP; ++j) ra[j] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int j = 0; j < BP; ++j) rb[j] = make_uint4(0u, 0u, 0u, 0u);
    }
    stash(st, ra, rb);
}

__global__ __launch_bounds__(GT) void k_qkv_project(ProjArgs a) {
    __shared__ __align__(16) bf16_raw smem[2 * STAGE]; // [stage][A 128 rows | B 128 rows][40]
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    // Workgroups are dealt to the 8 XCDs in turn (block b to XCD b % 8), each
    // with its own L2: all column tiles of one token tile go to the same XCD,
    // back to back, so the token tile is fetched into that L2 once.
    const int64_t tiles_n = (a.cols + BN - 1) / BN, tiles_m = (a.M + BM - 1) / BM;
    int64_t tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
    if (tiles_m % 8 == 0) {
        const int64_t xcd = blockIdx.x % 8, idx = blockIdx.x / 8;
        tm = (idx / tiles_n) * 8 + xcd;
        tn = idx % tiles_n;
    }
    const int64_t m0 = tm * BM, n0 = tn * BN;
    const int wm = (wv >> 1) * 64, wn = (wv & 1) * 64;

    gm_f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int64_t KT = (a.dm + BK - 1) / BK;
    const Rows rows = tile_rows(a, m0, n0);
    // K step s sits in register set (s + 1) % 2 until it is stashed: two steps
    // are in flight while one is multiplied
    // (steps past the last fetch the last one again: the loads stay the same
    // in every iteration)
    auto last = [&](int64_t s) { return s < KT ? s : KT - 1; };
    uint4 ra0[AP], rb0[BP], ra1[AP], rb1[BP];
    fetch(a, rows, 0, ra0, rb0);
    stash_step(a, 0, KT, smem, ra0, rb0);
    fetch(a, rows, last(1), ra0, rb0);
    fetch(a, rows, last(2), ra1, rb1);
    sync_lds();
    auto mma_step = [&](int64_t kt) {
        const bf16_raw* As = smem + (kt & 1) * STAGE;
        const bf16_raw* Bs = As + BM * LDK;
#pragma unroll
        for (int ks = 0; ks < BK; ks += 16) {
            // A lane l: row l%32 of the 32-row block, K elements 8(l/32) .. +7
            gm_bf16x8 fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint4 va = *reinterpret_cast<const uint4*>(
                    As + (wm + 32 * i + (lane & 31)) * LDK + ks + 8 * (lane >> 5));
                const uint4 vb = *reinterpret_cast<const uint4*>(
                    Bs + (wn + 32 * i + (lane & 31)) * LDK + ks + 8 * (lane >> 5));
                fa[i] = __builtin_bit_cast(gm_bf16x8, va);
                fb[i] = __builtin_bit_cast(gm_bf16x8, vb);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j],
                                                                        0, 0, 0);
        }
    };
    // pairs of steps (no exit between the two halves: the accumulators then
    // stay in one set of registers), then the last step when KT is odd
    int64_t kt = 0;
    for (; kt + 1 < KT; kt += 2) {
        // even step: the next step is in set 0
        mma_step(kt);
        stash_step(a, kt + 1, KT, smem + STAGE, ra0, rb0);
        fetch(a, rows, last(kt + 3), ra0, rb0);
        sync_lds();
        // odd step: the next step is in set 1
        mma_step(kt + 1);
        if (kt + 2 < KT) stash_step(a, kt + 2, KT, smem, ra1, rb1);
        fetch(a, rows, last(kt + 4), ra1, rb1);
        sync_lds();
    }
    if (kt < KT) {
        mma_step(kt);
        sync_lds(); // the epilogue reuses the stages
    }

    // epilogue: bf16 tile [128][128] through LDS (the A/B buffers are free
    // after the last barrier), then rows of 64 columns to the head-major outputs
    bf16_raw* Os = smem;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                const int col = wn + 32 * j + (lane & 31);
                // the hardware conversion (round to nearest even)
                Os[row * LDO + col] = __builtin_bit_cast(bf16_raw, (__bf16)acc[i][j][e]);
            }
    sync_lds();
    // 128 rows x 2 halves of 64 columns = 256 row pieces of 128 bytes; each
    // thread writes one piece as eight 16-byte stores
    {
        const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
        const int64_t m = m0 + row, c = n0 + 64 * half;
        if (m < a.M && c < a.cols) {
            const int64_t hd = a.H * 64;
            const int which = (int)(c / hd);
            const int64_t h = (c - which * hd) / 64;
            const int64_t b = m / a.N, tok = m - b * a.N;
            bf16_raw* dst = a.out[which] + ((b * a.H + h) * a.N + tok) * 64;
            const bf16_raw* src = Os + row * LDO + 64 * half;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                *reinterpret_cast<uint4*>(dst + 8 * j) = *reinterpret_cast<const uint4*>(src + 8 * j);
        }
    }
}

} // namespace

hipError_t launch_qkv_project(const void* x, const void* w_q, const void* w_k, const void* w_v,
                              int64_t B, int64_t N, int64_t dm, int64_t H, void* q, void* k,
                              void* v, hipStream_t st) {
    ProjArgs a;
    a.x = (const bf16_raw*)x;
    a.w[0] = (const bf16_raw*)w_q;
    a.w[1] = (const bf16_raw*)w_k;
    a.w[2] = (const bf16_raw*)w_v;
    a.out[0] = (bf16_raw*)q;
    a.out[1] = (bf16_raw*)k;
    a.out[2] = (bf16_raw*)v;
    a.M = B * N;
    a.N = N;
    a.dm = dm;
    a.H = H;
    a.cols = 3 * H * 64;
    const int64_t blocks = ((a.M + BM - 1) / BM) * ((a.cols + BN - 1) / BN);
    hipLaunchKernelGGL(k_qkv_project, dim3((unsigned)blocks), dim3(GT), 0, st, a);
    return hipGetLastError();
}

} // namespace linattn
