// mfma_f32.hip -- the chunked causal scan, its segment increments and the
// bidirectional readout on the float32 matrix cores, for the feature maps
// with a closed form: identity, ELU+1 and DPFP-nu (Kernel Zoo sec. 1.2-1.3
// for the recurrence, sec. 6.3 for DPFP, sec. 7 for the sum normalisation).
//
// Every product is a v_mfma_f32_16x16x4_f32 (float32 operands, float32
// accumulation): the same arithmetic as the vector kernels in generic.hip,
// in another summation order.  These maps need no projection, so a chunk's
// work is four contractions -- the readout phi(Q_c) S_{c-1}, the intra-chunk
// block phi(Q_c) phi(K_c)^T, that block times V_c, and the update
// S += phi(K_c)^T V_c -- which is what the matrix cores do, at twice the
// float32 rate of the vector ALU without packed instructions.
//
// One workgroup of four waves per (head, segment).  Wave w keeps value
// columns [16w, 16w + 16) of the state S, for all r features, in
// accumulator registers, so each output column is finished by one wave and
// no partial outputs cross waves; only the denominators do.  Per chunk of
// 32 tokens:
//   phase 1  q, k, v are staged (v transposed) and phi(q), phi(k) computed
//            once per workgroup into LDS -- lane (token t, block b) computes
//            r/8 features of token t -- with the sum normalisation and the
//            inter-chunk denominator phi(q_t) . z_{c-1};
//   phase 2  (after a barrier) the readout against S_{c-1}; the block, as
//            the three 16 x 16 tiles on and below the diagonal, one per wave
//            0-2, masked and written to LDS; the update of S (registers) and
//            of z (LDS, double-buffered);
//   phase 3  (after a barrier) the block's masked row sums complete the
//            denominators, and the block times V joins the readout.
// Chunk c's outputs are normalised and stored after the next chunk's first
// barrier, when all of its normalisers are in LDS.
#include <type_traits>

#include "launch.hpp"

namespace linattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CL = 32;        // tokens per chunk
constexpr int FNT = 256;      // threads per workgroup (four waves)
constexpr int VL = CL;        // row stride of V^T (floats)
constexpr int AL = CL + 4;    // row stride of the intra-chunk block (floats)

enum : int { M_SUMS = 0, M_CAUSAL = 1, M_READOUT = 2 };

// D += A B over one 4-wide slice of the contraction: lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16]; D is four registers, lane l
// register i holding D[4 (l / 16) + i][l % 16].
__device__ __forceinline__ f32x4 mma(float a, float b, f32x4 d) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, d, 0, 0, 0);
}

// Sixteen contraction indices in four slices: in slice i, lane group
// g = l / 16 supplies index 4g + i, so a lane's four operands are four
// consecutive indices (one 16-byte LDS read when they are contiguous).
__device__ __forceinline__ f32x4 mma16(f32x4 a, f32x4 b, f32x4 d) {
    d = mma(a[0], b[0], d);
    d = mma(a[1], b[1], d);
    d = mma(a[2], b[2], d);
    d = mma(a[3], b[3], d);
    return d;
}

__device__ __forceinline__ f32x4 lds4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; }

// One output element through a buffer resource (byte offset; dropped past
// the resource's range).
template <typename T> __device__ __forceinline__ void store_out(__amdgpu_buffer_rsrc_t rs, int off, float y);
template <> __device__ __forceinline__ void store_out<float>(__amdgpu_buffer_rsrc_t rs, int off, float y) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), rs, off, 0, 0);
}
template <> __device__ __forceinline__ void store_out<bf16_raw>(__amdgpu_buffer_rsrc_t rs, int off, float y) {
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(y), rs, off, 0, 0);
}

// Columns 4b .. 4b + 3 and 32 + 4b .. 32 + 4b + 3 of one input row, raw
// (loaded one chunk ahead).  The eight lanes of a token (b = 0 .. 7) thus
// cover the row in 16-byte blocks that are adjacent across lanes.
template <typename T> struct Row8;
template <> struct Row8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float* row, int blk) {
        a = reinterpret_cast<const float4*>(row + 4 * blk)[0];
        b = reinterpret_cast<const float4*>(row + 32 + 4 * blk)[0];
    }
    __device__ __forceinline__ f32x4 lo() const { return f32x4{a.x, a.y, a.z, a.w}; }
    __device__ __forceinline__ f32x4 hi() const { return f32x4{b.x, b.y, b.z, b.w}; }
};
template <> struct Row8<bf16_raw> {
    uint2 a, b;
    __device__ __forceinline__ void load(const bf16_raw* row, int blk) {
        a = *reinterpret_cast<const uint2*>(row + 4 * blk);
        b = *reinterpret_cast<const uint2*>(row + 32 + 4 * blk);
    }
    static __device__ __forceinline__ f32x4 unpack(uint2 x) {
        return f32x4{__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
                     __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u)};
    }
    __device__ __forceinline__ f32x4 lo() const { return unpack(a); }
    __device__ __forceinline__ f32x4 hi() const { return unpack(b); }
};

// LDS.  Feature tiles are [32 tokens][r + 4] (the padding keeps the 16-byte
// row reads of the operand loads and the strided column reads of phi(K)^T
// free of bank conflicts).  Each token's inputs are staged in the first 64
// floats of its own feature row: the token's eight lanes are in one wave,
// which reads the staged row completely before it writes the features.
//   M_CAUSAL   pq, pk, v^T, the block, z (double-buffered), denominators:
//              81,792 bytes at r = 256, two workgroups per CU
//   M_READOUT  pq (double-buffered), z, denominators
//   M_SUMS     pk, v^T
template <int R, int MODE> struct SmemF32 {
    static constexpr int NPQ = MODE == M_SUMS ? 0 : (MODE == M_READOUT ? 2 : 1);
    float pq[NPQ ? NPQ : 1][NPQ ? CL * (R + 4) : 4];
    float pk[MODE == M_READOUT ? 4 : CL * (R + 4)];
    float vt[MODE == M_READOUT ? 4 : DV * VL];
    float as[MODE == M_CAUSAL ? CL * AL : 4];
    float z[MODE == M_SUMS ? 1 : 2][MODE == M_SUMS ? 4 : R];
    float den[3][MODE == M_SUMS ? 4 : CL]; // per token: 1 / max(den, eps), or 1
};

// Float offset of column `col` of token row t in a feature tile of width R.
template <int R>
__device__ __forceinline__ int fidx(int t, int col) {
    return t * (R + 4) + col;
}

// Float offset of token t in row `col` of V^T ([64][32]): 4-token blocks are
// rotated by ((col / 4) mod 8), so that the eight lanes of a token, which
// write rows 4b + j and 32 + 4b + j, hit distinct banks.
__device__ __forceinline__ int vidx(int col, int t) {
    return col * VL + (t ^ (((col >> 2) & 7) << 2));
}

// phi of token t for features 32 m + 4 b + e (m < r / 32, e < 4) into
// f[4 m + e], from its staged (scaled) input in the first 64 floats of row t
// of tile.  PHI is identity or ELU+1 (r = 64) or DPFP-nu (r = 2 d nu):
// feature f = i + 2d (s - 1) is kt_i kt_{(i + s) mod 2d}, kt = relu([u, -u])
// (Kernel Zoo sec. 6.3).
template <int PHI, int R>
__device__ __forceinline__ void token_features(const float* tile, int t, int b, float (&f)[R / 8]) {
    if constexpr (PHI == PHI_DPFP) {
        constexpr int NU = R / (2 * D);
        // kt_{32 mu + 4 b .. 32 mu + 4 b + 7} (mod 2d) for mu = 0 .. 3: two
        // blocks of four inputs, each of one sign
        float kt[4][8];
#pragma unroll
        for (int mu = 0; mu < 4; ++mu) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int i = (32 * mu + 4 * b + 4 * h) & (2 * D - 1);
                const f32x4 x = lds4(tile + fidx<R>(t, i & (D - 1)));
                const bool neg = (i & D) != 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) kt[mu][4 * h + e] = fmaxf(neg ? -x[e] : x[e], 0.f);
            }
        }
        // feature 32 m + 4 b + e: block s = m / 4 + 1, i = 32 (m % 4) + 4 b + e
#pragma unroll
        for (int m = 0; m < 4 * NU; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                f[4 * m + e] = kt[m & 3][e] * kt[m & 3][e + (m >> 2) + 1];
    } else {
#pragma unroll
        for (int m = 0; m < R / 32; ++m) {
            const f32x4 x = lds4(tile + fidx<R>(t, 32 * m + 4 * b));
#pragma unroll
            for (int e = 0; e < 4; ++e) f[4 * m + e] = PHI == PHI_ELU1 ? elu1(x[e]) : x[e];
        }
    }
}

// The factor a token's numerator is multiplied by: 1 / max(den, eps) for
// attention normalisation, 1 for none.
__device__ __forceinline__ float normaliser(const Cfg& c, float den) {
    return c.norm == NORM_ATTN ? 1.f / fmaxf(den, c.eps) : 1.f;
}

// Sum over the eight lanes of one token (lanes 8a .. 8a + 7).
__device__ __forceinline__ float sum8(float x) {
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    return x;
}

// Features of token t, lane b, for a staged tile: zero past the chunk's
// rows, optionally sum-normalised, written over the staged row; returns
// them in f.  Every read of the staged row precedes every write (the whole
// wave's, in program order).
template <int PHI, int R>
__device__ __forceinline__ void tile_features(const Cfg& c, float* tile, int t, int b, bool live,
                                              float (&f)[R / 8]) {
    constexpr int FB = R / 8;
    token_features<PHI, R>(tile, t, b, f);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < FB; ++j) {
        f[j] = live ? f[j] : 0.f;
        s += f[j];
    }
    if (c.sum_norm) {
        const float rs = 1.f / fmaxf(sum8(s), c.eps);
#pragma unroll
        for (int j = 0; j < FB; ++j) f[j] *= rs;
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int m = 0; m < FB / 4; ++m)
        st4(tile + fidx<R>(t, 32 * m + 4 * b), f32x4{f[4 * m], f[4 * m + 1], f[4 * m + 2], f[4 * m + 3]});
}

// One workgroup per (head, segment).  MODE:
//   M_SUMS     the segment's increment (sum phi(k) v^T, sum phi(k)) -> ws
//   M_CAUSAL   outputs of the chunked recurrence from the carried-in state
//   M_READOUT  outputs against a fixed summary (bidirectional form)
template <typename T, int PHI, int R, int MODE>
__global__ __launch_bounds__(FNT, 2) void k_f32mm(Cfg c, const T* __restrict__ q,
                                              const T* __restrict__ k, const T* __restrict__ v,
                                              int64_t N, int64_t G, int64_t seg_len,
                                              const int64_t* __restrict__ tab, int64_t sub,
                                              const float* __restrict__ state, int64_t st_bh,
                                              int64_t st_g, T* __restrict__ out,
                                              float* __restrict__ ws) {
    constexpr int NT16 = R / 16; // 16-feature tiles of the state
    constexpr int FB = R / 8;    // features per lane in phase 1
    constexpr int ZF = R / 4;    // features of z each wave updates
    constexpr bool HAS_Q = MODE != M_SUMS;
    constexpr bool HAS_K = MODE != M_READOUT;
    __shared__ __align__(16) SmemF32<R, MODE> sm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g4 = lane >> 4; // MFMA lane coordinates
    const int ft = tid >> 3, fb = tid & 7;     // phase-1 token and feature block
    const int64_t bh = blockIdx.x / G, g = blockIdx.x % G;
    int64_t t0, t1;
    seg_range(tab, MODE == M_SUMS ? 1 : sub, g, seg_len, N, t0, t1);
    const int64_t nck = t1 > t0 ? (t1 - t0 + CL - 1) / CL : 0;

    // S[16 tt + 4 g4 + i][16w + n16] in S[tt][i]
    f32x4 S[NT16];
    float zacc = 0.f; // M_SUMS: z of feature ZF w + lane
    if constexpr (MODE == M_SUMS) {
#pragma unroll
        for (int tt = 0; tt < NT16; ++tt) S[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
        const float* sin = state + bh * st_bh + g * st_g;
#pragma unroll
        for (int tt = 0; tt < NT16; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[tt][i] = sin[(16 * tt + 4 * g4 + i) * DV + 16 * w + n16];
        for (int f = tid; f < R; f += FNT) sm.z[0][f] = sin[R * DV + f];
        sync_lds();
    }

    // chunk inputs, one chunk ahead: lane (ft, fb) loads columns 4 fb .. 4 fb + 3
    // and 32 + 4 fb .. 32 + 4 fb + 3 of token ft (rows clamped into the
    // segment: every load is issued)
    Row8<T> xq, xk, xv;
    auto load_chunk = [&](int64_t ci) {
        const int64_t c0 = t0 + ci * CL;
        const int64_t row = min<int64_t>(c0 + ft, t1 - 1);
        const int64_t off = (bh * N + row) * D;
        if (HAS_Q) xq.load(q + off, fb);
        if (HAS_K) {
            xk.load(k + off, fb);
            xv.load(v + (bh * N + row) * DV, fb);
        }
    };
    if (nck > 0) load_chunk(0);

    f32x4 num0 = {0.f, 0.f, 0.f, 0.f}, num1 = {0.f, 0.f, 0.f, 0.f};
    int64_t prev_c0 = 0;
    int prev_rows = 0;
    // normalise and store the outputs of a finished chunk: wave w, lane
    // (n16, g4), register i of num_ta is token 16 ta + 4 g4 + i, column
    // 16w + n16.  Stores go through a buffer resource covering the chunk's
    // rows, whose range check drops the rows past the end.
    auto finish = [&](int64_t pc, int64_t c0, int rows) {
        const float* inv = sm.den[pc % 3];
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            out + (bh * N + c0) * DV, 0, rows * DV * (int)sizeof(T), 0x00020000);
#pragma unroll
        for (int ta = 0; ta < 2; ++ta) {
            const f32x4 nm = ta ? num1 : num0;
            const f32x4 iv = lds4(inv + 16 * ta + 4 * g4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * ta + 4 * g4 + i;
                store_out<T>(rs, (t * DV + 16 * w + n16) * (int)sizeof(T), nm[i] * iv[i]);
            }
        }
    };

    for (int64_t ci = 0; ci < nck; ++ci) {
        const int p = (int)(ci & 1);
        const int64_t c0 = t0 + ci * CL;
        const int rows = (int)min<int64_t>(CL, t1 - c0);
        const bool live = ft < rows;
        float* pq = sm.pq[MODE == M_READOUT ? p : 0];
        float* pk = sm.pk;

        // ---- phase 1: stage, prefetch, features
        const float sc = live ? c.scale : 0.f;
        if (HAS_Q) {
            st4(pq + fidx<R>(ft, 4 * fb), sc * xq.lo());
            st4(pq + fidx<R>(ft, 32 + 4 * fb), sc * xq.hi());
        }
        if (HAS_K) {
            st4(pk + fidx<R>(ft, 4 * fb), sc * xk.lo());
            st4(pk + fidx<R>(ft, 32 + 4 * fb), sc * xk.hi());
            const f32x4 va = live ? xv.lo() : f32x4{0.f, 0.f, 0.f, 0.f};
            const f32x4 vb = live ? xv.hi() : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sm.vt[vidx(4 * fb + j, ft)] = va[j];
                sm.vt[vidx(32 + 4 * fb + j, ft)] = vb[j];
            }
        }
        load_chunk(ci + 1 < nck ? ci + 1 : ci);
        // a token's eight lanes are in one wave: its staged row is complete
        // once the wave's LDS writes are (they execute in order)
        __builtin_amdgcn_wave_barrier();

        float den_q = 0.f;
        if (HAS_Q) {
            float f[FB];
            tile_features<PHI, R>(c, pq, ft, fb, live, f);
            const float* zc = sm.z[MODE == M_READOUT ? 0 : p] + 4 * fb;
#pragma unroll
            for (int m = 0; m < FB / 4; ++m) {
                const f32x4 zz = lds4(zc + 32 * m);
#pragma unroll
                for (int e = 0; e < 4; ++e) den_q = fmaf(f[4 * m + e], zz[e], den_q);
            }
            den_q = sum8(den_q);
            if (MODE == M_READOUT && fb == 0) sm.den[ci % 3][ft] = normaliser(c, den_q);
        }
        if (HAS_K) {
            float f[FB];
            tile_features<PHI, R>(c, pk, ft, fb, live, f);
        }
        sync_lds();

        if (HAS_Q && ci > 0) finish(ci - 1, prev_c0, prev_rows);

        // ---- phase 2: readout, intra-chunk block, update
        f32x4 vb0 = {0.f, 0.f, 0.f, 0.f}, vb1 = vb0;
        if (HAS_K) {
            // V[token 16 tq + 4 g4 + i][column 16w + n16] (B operand)
            vb0 = lds4(sm.vt + vidx(16 * w + n16, 4 * g4));
            vb1 = lds4(sm.vt + vidx(16 * w + n16, 16 + 4 * g4));
        }
        // the block tile of waves 0-2: rows 16 ta, columns 16 tb
        const int ta = w == 0 ? 0 : 1, tb = w == 2 ? 1 : 0;
        f32x4 blk = {0.f, 0.f, 0.f, 0.f};
        num0 = f32x4{0.f, 0.f, 0.f, 0.f};
        num1 = num0;
        // One loop per role, chosen once per wave: ROLE 0 has no block tile,
        // ROLE 1 a tile of rows 0-15, ROLE 2 of rows 16-31.  The operands of
        // feature tile tt + 1 are read while tile tt is multiplied; the
        // scheduling barrier keeps each tile's reads in its own step, which
        // bounds the registers in flight.
        struct Ops {
            f32x4 a0, a1, bk;
        };
        auto contract = [&](auto role) {
            constexpr int ROLE = decltype(role)::value;
            auto load = [&](int tt) {
                Ops o;
                if constexpr (HAS_Q) {
                    o.a0 = lds4(pq + fidx<R>(n16, 16 * tt + 4 * g4));
                    o.a1 = lds4(pq + fidx<R>(16 + n16, 16 * tt + 4 * g4));
                    if constexpr (ROLE != 0)
                        o.bk = lds4(pk + fidx<R>(16 * tb + n16, 16 * tt + 4 * g4));
                }
                return o;
            };
            Ops cur = load(0);
#pragma unroll
            for (int tt = 0; tt < NT16; ++tt) {
                // phi(K)^T[feature 16 tt + n16][token 16 tq + 4 g4 + i], read
                // at the start of the step and used after the readout
                f32x4 k0, k1;
                if constexpr (HAS_K) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        k0[i] = pk[fidx<R>(4 * g4 + i, 16 * tt + n16)];
                        k1[i] = pk[fidx<R>(16 + 4 * g4 + i, 16 * tt + n16)];
                    }
                }
                Ops nxt = cur;
                if (tt + 1 < NT16) nxt = load(tt + 1);
                if constexpr (HAS_Q) {
                    num0 = mma16(cur.a0, S[tt], num0);
                    num1 = mma16(cur.a1, S[tt], num1);
                    if constexpr (ROLE == 1) blk = mma16(cur.a0, cur.bk, blk);
                    if constexpr (ROLE == 2) blk = mma16(cur.a1, cur.bk, blk);
                }
                if constexpr (HAS_K) {
                    S[tt] = mma16(k0, vb0, S[tt]);
                    S[tt] = mma16(k1, vb1, S[tt]);
                }
                cur = nxt;
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        if (MODE == M_CAUSAL && w < 3) {
            if (w == 0)
                contract(std::integral_constant<int, 1>{});
            else
                contract(std::integral_constant<int, 2>{});
        } else {
            contract(std::integral_constant<int, 0>{});
        }
        if constexpr (HAS_K) {
            if (lane < ZF) {
                const int f = ZF * w + lane;
                float zs = 0.f;
#pragma unroll 8
                for (int t = 0; t < CL; ++t) zs += pk[fidx<R>(t, f)];
                if (MODE == M_SUMS)
                    zacc += zs;
                else
                    sm.z[p ^ 1][f] = sm.z[p][f] + zs;
            }
        }
        if constexpr (MODE == M_SUMS) sync_lds(); // pk and v^T are restaged next
        if constexpr (MODE == M_CAUSAL) {
            if (w < 3) {
                // lane (n16, g4), register i: token 16 ta + 4 g4 + i, key 16 tb + n16
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * ta + 4 * g4 + i, j = 16 * tb + n16;
                    sm.as[t * AL + j] = j <= t ? blk[i] : 0.f;
                }
            }
            sync_lds();

            // ---- phase 3: denominators, block times V
            {
                // keys 4 fb .. 4 fb + 3 of token ft (the tile above the
                // diagonal is never written: keys >= 16 of tokens < 16)
                float a = 0.f;
                if (4 * fb < 16 * (ft / 16 + 1)) {
                    const f32x4 x = lds4(sm.as + ft * AL + 4 * fb);
                    a = (x[0] + x[1]) + (x[2] + x[3]);
                }
                a = sum8(a);
                if (fb == 0) sm.den[ci % 3][ft] = normaliser(c, den_q + a);
            }
            num0 = mma16(lds4(sm.as + n16 * AL + 4 * g4), vb0, num0);
            num1 = mma16(lds4(sm.as + (16 + n16) * AL + 4 * g4), vb0, num1);
            num1 = mma16(lds4(sm.as + (16 + n16) * AL + 16 + 4 * g4), vb1, num1);
        }
        prev_c0 = c0;
        prev_rows = rows;
    }

    if constexpr (HAS_Q) {
        if (nck > 0) {
            sync_lds();
            finish(nck - 1, prev_c0, prev_rows);
        }
    } else {
        float* dst = ws + (bh * G + g) * state_elems(R);
#pragma unroll
        for (int tt = 0; tt < NT16; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(16 * tt + 4 * g4 + i) * DV + 16 * w + n16] = S[tt][i];
        if (lane < ZF) dst[R * DV + ZF * w + lane] = zacc;
    }
}

template <typename T, int PHI, int R, int MODE>
void launch_f32(const Cfg& c, const void* q, const void* k, const void* v, Shape s,
                const SegPlan& sp, const float* state, int64_t sbh, int64_t sg, void* out,
                float* ws, hipStream_t st) {
    hipLaunchKernelGGL((k_f32mm<T, PHI, R, MODE>), dim3((unsigned)(sp.G * s.BH)), dim3(FNT), 0, st,
                       c, (const T*)q, (const T*)k, (const T*)v, s.N, sp.G, sp.seg_len, sp.tab,
                       sp.sub, state, sbh, sg, (T*)out, ws);
}

template <typename T, int MODE>
hipError_t dispatch_f32(const Cfg& c, const void* q, const void* k, const void* v, Shape s,
                        const SegPlan& sp, const float* state, int64_t sbh, int64_t sg, void* out,
                        float* ws, hipStream_t st) {
    if (c.phi == PHI_IDENTITY && c.r == 64)
        launch_f32<T, PHI_IDENTITY, 64, MODE>(c, q, k, v, s, sp, state, sbh, sg, out, ws, st);
    else if (c.phi == PHI_ELU1 && c.r == 64)
        launch_f32<T, PHI_ELU1, 64, MODE>(c, q, k, v, s, sp, state, sbh, sg, out, ws, st);
    else if (c.phi == PHI_DPFP && c.r == 128)
        launch_f32<T, PHI_DPFP, 128, MODE>(c, q, k, v, s, sp, state, sbh, sg, out, ws, st);
    else if (c.phi == PHI_DPFP && c.r == 256)
        launch_f32<T, PHI_DPFP, 256, MODE>(c, q, k, v, s, sp, state, sbh, sg, out, ws, st);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

} // namespace

bool f32mm_supported(const Cfg& c) {
    return ((c.phi == PHI_IDENTITY || c.phi == PHI_ELU1) && c.r == 64) ||
           (c.phi == PHI_DPFP && (c.r == 128 || c.r == 256));
}

hipError_t launch_f32mm_sums(const Cfg& c, int dtype, const void* k, const void* v, Shape s,
                             SegPlan sp, float* ws, hipStream_t st) {
    return dtype == 0
               ? dispatch_f32<float, M_SUMS>(c, nullptr, k, v, s, sp, nullptr, 0, 0, nullptr, ws, st)
               : dispatch_f32<bf16_raw, M_SUMS>(c, nullptr, k, v, s, sp, nullptr, 0, 0, nullptr, ws,
                                                st);
}

hipError_t launch_f32mm_outputs(const Cfg& c, int dtype, int causal, const void* q, const void* k,
                                const void* v, Shape s, SegPlan sp, const float* state,
                                int64_t sbh, int64_t sg, void* out, hipStream_t st) {
    if (dtype == 0)
        return causal ? dispatch_f32<float, M_CAUSAL>(c, q, k, v, s, sp, state, sbh, sg, out,
                                                      nullptr, st)
                      : dispatch_f32<float, M_READOUT>(c, q, k, v, s, sp, state, sbh, sg, out,
                                                       nullptr, st);
    return causal ? dispatch_f32<bf16_raw, M_CAUSAL>(c, q, k, v, s, sp, state, sbh, sg, out,
                                                     nullptr, st)
                  : dispatch_f32<bf16_raw, M_READOUT>(c, q, k, v, s, sp, state, sbh, sg, out,
                                                      nullptr, st);
}

} // namespace linattn
