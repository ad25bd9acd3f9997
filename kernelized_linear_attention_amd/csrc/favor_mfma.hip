// favor_mfma.hip -- FAVOR+ attention on the matrix cores (bfloat16 inputs,
// r = 256 features, d = dv = 64, float32 accumulation and state).
//
// One workgroup of four waves handles one sequence segment of one head, in
// chunks of 32 tokens (one MFMA tile: the intra-chunk block is a single
// masked 32 x 32 tile).
// Wave w owns the features F_w = [64w, 64w + 64): the rows of omega for F_w
// stay in its registers for the whole segment, and so does its slice
// S[F_w, :] of the state (float32 MFMA accumulators).  Per chunk (Kernel Zoo sec. 4.2 / 5.4 map; causal recurrence of sec. 1.3 in
// chunked form, see generic.hip):
//   P_Q^T = omega_w Q_c^T           -> phi(Q_c)[:, F_w]  (tokens on lanes)
//   P_K   = K_c omega_w^T           -> phi(K_c)[:, F_w]  (features on lanes)
//   phi   = exp2(P * s*log2(e) + per-token bias), the bias holding
//           -s^2 |x|^2 / 2 and -log2(sqrt(r)) (x unscaled, s = scale)
//   num_w = phi(Q_c) S_{c-1}[F_w]                         (inter-chunk readout)
//         + ((phi(Q_c) phi(K_c)^T)|_{F_w} o causal mask) V_c (intra-chunk block)
//   den_w = phi(Q_c) z_{c-1}[F_w] + row sums of the masked block
//   S[F_w] += phi(K_c)[:, F_w]^T V_c,  z[F_w] += column sums of phi(K_c)
// and the partial num_w, den_w of the four waves are summed through LDS.
// Every contraction is a v_mfma_f32_32x32x16_bf16; the MFMA accumulator
// layout of one product is reused as an operand of the next where the
// contraction index allows it (a k-slot permutation applied to both
// operands), so only phi(K) (for the intra block) and V (transposed) pass
// through LDS.
//
// Modes: SUMS     -- per-segment state increments (no outputs);
//        CAUSAL   -- chunked recurrence from the carried-in state;
//        READOUT  -- bidirectional readout against the full summary.
#include "launch.hpp"

namespace linattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;       // four waves
constexpr int NW = 4;
constexpr int R = 256;        // features: 64 per wave
constexpr int L = 32;         // chunk length: one 32-token MFMA tile
constexpr int LDK = 72;       // LDS row stride (bf16) of a wave's phi(K) tile [32 t][64 f]: 144 B
constexpr int LDV = 40;       // LDS row stride (bf16) of the V^T tile [64 n][32 t]: 80 B

enum { MODE_SUMS = 0, MODE_CAUSAL = 1, MODE_READOUT = 2 };

// Register budget.  omega's fragments stay in registers (re-reading them per
// projection doubles the L1 traffic of a chunk) and each chunk's inputs are
// loaded one chunk ahead; that takes more than the 256 registers per lane of
// two workgroups per CU, so the kernel runs one workgroup per CU and hides
// latency with the prefetch.
constexpr bool OMEGA_IN_REGS = true;
constexpr bool PREFETCH = true;
constexpr int MIN_WG_PER_CU = 1;

struct FavorArgs {
    const u16* q;
    const u16* k;
    const u16* v;
    const u16* omega;
    int64_t N;
    int64_t G;
    int64_t seg_len;
    float a_scale;  // scale * log2(e)
    float b_norm;   // -scale^2 * log2(e) / 2
    float b_const;  // log2(1 / sqrt(r))
    float eps;
    int norm;
    float* state;   // SUMS: increments out; CAUSAL: carried-in states; READOUT: summaries
    int64_t st_bh;
    int64_t st_g;
    u16* out;
};

// Workgroup barrier for LDS traffic only.  __syncthreads() also waits for
// every outstanding global load, which would stall on the next chunk's
// prefetch; here all communication between waves goes through LDS.
__device__ __forceinline__ void sync_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 pack8(const f32x16& c, int base) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)c[base + e];
    return r;
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 r;
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = 0.f;
    return r;
}

// Raw bits of element e of a bfloat16 vector (through 32-bit words: a bit
// cast of a single __bf16 vector element does not lower reliably).
__device__ __forceinline__ u16 bf16_bits(const bf16x8& v, int e) {
    const u32x4 u = __builtin_bit_cast(u32x4, v);
    const uint32_t word = u[e >> 1];
    return (e & 1) ? (u16)(word >> 16) : (u16)(word & 0xffffu);
}

// Column order of the LDS tiles that feed MFMA operands.  An accumulator
// element i of lane half h belongs to index 8(i/4) + 4h + i%4 within a
// 16-block; the operand built from it holds, in k-slot e, index
// 8(e/4) + 4h + e%4.  Storing index x at column swap23(x) (bits 2 and 3
// exchanged) makes those eight indices the contiguous columns 8h .. 8h + 7,
// so each operand is one 16-byte LDS read.
__device__ __forceinline__ int swap23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// One MFMA operand: 8 contiguous bf16 of an LDS row.
__device__ __forceinline__ bf16x8 lds8(const u16* p) { return *reinterpret_cast<const bf16x8*>(p); }

// f[ks] = X[lo][16 ks + 8 h .. +7] of the chunk at X: the A operand
// (tokens as M) and the B operand (tokens as N) of a contraction over d.
// Rows past `rows` repeat row rows-1: every load stays in bounds without
// per-lane branches (which would make the compiler wait for the loads right
// away); the kernel zeroes phi(K) of those rows and never stores their
// outputs.
__device__ __forceinline__ void load_x(const u16* __restrict__ X, int rows, int lo, int h,
                                       bf16x8 (&f)[4]) {
    const int t = min(lo, rows - 1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        f[ks] = *reinterpret_cast<const bf16x8*>(X + (int64_t)t * D + 16 * ks + 8 * h);
}

// |x_t|^2 for t = lo from its fragments (the two lane halves hold
// complementary halves of the row); bf16 products are exact in float32.
__device__ __forceinline__ float sq_norm(const bf16x8 (&f)[4]) {
    float s = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const bf16x2 x = {f[ks][e], f[ks][e + 1]};
            s = __builtin_amdgcn_fdot2_f32_bf16(x, x, s, false);
        }
    return s + __shfl_xor(s, 32, 64);
}

// Raw V rows of the chunk for the transposed LDS copy: thread th holds
// V[th/8][8 (th%8) .. +7] (rows past `rows` repeat row rows-1; they only
// ever meet zero weights).
__device__ __forceinline__ bf16x8 load_v(const u16* __restrict__ V, int rows, int tid) {
    const int t = min(tid >> 3, rows - 1), n0 = (tid & 7) * 8;
    return *reinterpret_cast<const bf16x8*>(V + (int64_t)t * DV + n0);
}

// V^T in LDS: row n holds V[t][n] at column vt_col(n, swap23(t)); the
// 16-byte chunks of a row are rotated by (n / 8) % 4 so that the transposing
// stores (eight rows 8 apart at a time) fall on different banks.
__device__ __forceinline__ int vt_col(int n, int c) { return (((c >> 3) ^ ((n >> 3) & 3)) << 3) | (c & 7); }

__device__ __forceinline__ void store_vt(u16* vt, int tid, const bf16x8& vr) {
    const int t = swap23(tid >> 3), n0 = (tid & 7) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) vt[(n0 + e) * LDV + vt_col(n0 + e, t)] = bf16_bits(vr, e);
}

// omega[f0 + 32 t + lo][16 ks + 8 h ..]: A operand of omega X^T (t = feature
// tile as M) and B operand of X omega^T (t = feature tile as N) at once.
__device__ __forceinline__ bf16x8 omega_frag(const u16* __restrict__ omega, int f0, int t, int ks,
                                             int lo, int h) {
    return *reinterpret_cast<const bf16x8*>(omega + (int64_t)(f0 + 32 * t + lo) * D + 16 * ks + 8 * h);
}

template <int MODE>
__global__ __launch_bounds__(NT, MIN_WG_PER_CU) void k_favor_mfma(FavorArgs a) {
    __shared__ __attribute__((aligned(16))) u16 vt_s[2][DV * LDV];        // V^T, double buffered
    __shared__ __attribute__((aligned(16))) u16 pk_s[NW][L * LDK];        // phi(K)[:, F_w], bf16
    __shared__ __attribute__((aligned(16))) float red_s[2][2][NW][2][64][4]; // partial num blocks
    __shared__ __attribute__((aligned(16))) float z_s[R];
    __shared__ __attribute__((aligned(16))) float den_s[NW][L];
    __shared__ __attribute__((aligned(16))) float kb_s[NW][L];            // key biases by token

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6); // wave index, uniform
    const int lo = lane & 31, h = lane >> 5;
    const int f0 = 64 * w;
    const int64_t bh = blockIdx.x / a.G, g = blockIdx.x % a.G;
    const int64_t t0 = g * a.seg_len;
    const int64_t t1 = min<int64_t>(a.N, t0 + a.seg_len);
    constexpr bool HAS_K = MODE != MODE_READOUT;
    constexpr bool HAS_Q = MODE != MODE_SUMS;
    // this wave finishes rows [16 oq, 16 oq + 16) of output tile on (columns 32 on + ..)
    const int on = w & 1, oq = w >> 1;

    bf16x8 om[2][4]; // omega rows of F_w, when they stay in registers
    if (OMEGA_IN_REGS) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) om[mt][ks] = omega_frag(a.omega, f0, mt, ks, lo, h);
    }

    // State slice S[F_w, :] in accumulator layout: element i of S[mt][nt]
    // is S[f0 + 32 mt + 8 (i/4) + 4 h + i%4][32 nt + lo].
    f32x16 S[2][2];
    float zreg[2] = {0.f, 0.f}; // z[f0 + 32 nt + lo]
    const float* st = a.state + bh * a.st_bh + g * a.st_g;
    if (MODE == MODE_SUMS) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) S[mt][nt] = zero16();
    } else {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int f = f0 + 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
                    S[mt][nt][i] = st[(int64_t)f * DV + 32 * nt + lo];
                }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) zreg[nt] = st[(int64_t)R * DV + f0 + 32 * nt + lo];
        if (h == 0) {
            z_s[f0 + lo] = zreg[0];
            z_s[f0 + 32 + lo] = zreg[1];
        }
    }

    const u16* qb = a.q + bh * a.N * D;
    const u16* kb = a.k + bh * a.N * D;
    const u16* vb = a.v + bh * a.N * DV;

    bf16x8 qf[4], kf[4], vr;
    int rows = (int)min<int64_t>(L, t1 - t0);
    if (PREFETCH && HAS_Q && rows > 0) load_x(qb + t0 * D, rows, lo, h, qf);
    if (PREFETCH && HAS_K && rows > 0) load_x(kb + t0 * D, rows, lo, h, kf);
    if (HAS_K && rows > 0) {
        vr = load_v(vb + t0 * DV, rows, tid);
        store_vt(vt_s[0], tid, vr);
    }

    // causal mask of the diagonal tile: element i of lane (lo, h) pairs query
    // lo with key 8(i/4) + 4h + i%4, kept when 8(i/4) + i%4 <= lo - 4h
    const int keep_thr = lo - 4 * h;

    int buf = 0;
    for (int64_t c0 = t0; c0 < t1; c0 += L, buf ^= 1) {
        rows = (int)min<int64_t>(L, t1 - c0);
        const int64_t cn = c0 + L;
        const int rows_next = cn < t1 ? (int)min<int64_t>(L, t1 - cn) : 0;
        sync_lds(); // (A) vt_s[buf] complete; last chunk's red_s / den_s reads done

        // ---- phi(K) = exp(K omega_w^T ...), features on lanes -------------------
        bf16x8 fk[2][2]; // [nt][kk]: A operand of the update
        float zpart[2] = {0.f, 0.f};
        if (HAS_K) {
            if (!PREFETCH) load_x(kb + c0 * D, rows, lo, h, kf);
            // keys past the end of the segment get bias -inf: exp2 gives exactly 0,
            // so they add nothing to S, z or the intra-chunk block
            const float bk = lo < rows ? fmaf(a.b_norm, sq_norm(kf), a.b_const) : -INFINITY;
            kb_s[w][lo] = bk; // both lane halves write the same value
            f32x16 PK[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                f32x16 c = zero16();
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    c = mfma(kf[ks], OMEGA_IN_REGS ? om[nt][ks] : omega_frag(a.omega, f0, nt, ks, lo, h), c);
                PK[nt] = c; // token 8(i/4) + 4h + i%4, feature f0 + 32 nt + lo
            }
            // the next chunk's keys and values load while this one is computed
            if (PREFETCH && rows_next > 0) {
                load_x(kb + cn * D, rows_next, lo, h, kf);
                vr = load_v(vb + cn * DV, rows_next, tid);
            }
            f32x4 kbias[4]; // biases of the tokens 8 j + 4 h + (0..3)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                kbias[j] = *reinterpret_cast<const f32x4*>(&kb_s[w][8 * j + 4 * h]);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                f32x16& c = PK[nt];
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    c[i] = __builtin_amdgcn_exp2f(fmaf(c[i], a.a_scale, kbias[i >> 2][i & 3]));
#pragma unroll
                for (int i = 0; i < 16; ++i) zpart[nt] += c[i];
                fk[nt][0] = pack8(c, 0);
                fk[nt][1] = pack8(c, 8);
            }
            if (MODE == MODE_CAUSAL) {
                // phi(K) rows to LDS for the intra-chunk block: row t, column swap23(f)
                u16* pk = pk_s[w] + swap23(lo);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int t = 8 * (i >> 2) + 4 * h + (i & 3);
                        pk[t * LDK + 32 * nt] = bf16_bits(fk[nt][i >> 3], i & 7);
                    }
            }
        }

        // keep the query side's loads (omega, q) from being hoisted into the key
        // side: that would hold both phases' operands at once
        asm volatile("" ::: "memory");

        // V fragment (kk, nt): k-slot e <-> token 16 kk + 8 (e/4) + 4 h + e%4,
        // lane <-> column 32 nt + lo (re-read from LDS where needed: cheaper
        // than keeping it in registers)
        const u16* vt = vt_s[buf];
        auto vfrag = [&](int kk, int nt) {
            return lds8(vt + (32 * nt + lo) * LDV + vt_col(32 * nt + lo, 16 * kk + 8 * h));
        };

        // ---- queries: phi(Q), readout against S_{c-1}, intra-chunk block ---------
        f32x16 own = zero16(); // rows 16 oq .. of output tile on, in regs 8 oq .. 8 oq + 7
        if (HAS_Q) {
            if (!PREFETCH) load_x(qb + c0 * D, rows, lo, h, qf);
            const float bq = fmaf(a.b_norm, sq_norm(qf), a.b_const);
            bf16x8 fq[2][2]; // [mt][kk]
            float den = 0.f;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                // P_Q^T tile mt: feature f0 + 32 mt + 8(i/4) + 4h + i%4, token lo
                f32x16 c = zero16();
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    c = mfma(OMEGA_IN_REGS ? om[mt][ks] : omega_frag(a.omega, f0, mt, ks, lo, h), qf[ks], c);
                f32x4 zq[4]; // z_{c-1} of the features f0 + 32 mt + 8 j + 4 h + (0..3)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    zq[j] = *reinterpret_cast<const f32x4*>(&z_s[f0 + 32 * mt + 8 * j + 4 * h]);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float y = __builtin_amdgcn_exp2f(fmaf(c[i], a.a_scale, bq));
                    c[i] = y;
                    den = fmaf(y, zq[i >> 2][i & 3], den);
                }
                fq[mt][0] = pack8(c, 0);
                fq[mt][1] = pack8(c, 8);
            }
            // this chunk's queries are consumed: load the next chunk's
            if (PREFETCH && rows_next > 0) load_x(qb + cn * D, rows_next, lo, h, qf);
            bf16x8 at[2]; // masked intra-chunk block A[lo][j] as the A operand of A V
            if (MODE == MODE_CAUSAL) {
                // masked block, transposed: c[i] = A[lo][j], j = 8(i/4) + 4h + i%4, over F_w
                const u16* pk = pk_s[w] + lo * LDK + 8 * h;
                f32x16 c = zero16();
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) c = mfma(lds8(pk + 32 * mt + 16 * kk), fq[mt][kk], c);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    c[i] = 8 * (i >> 2) + (i & 3) <= keep_thr ? c[i] : 0.f;
                    den += c[i];
                }
                at[0] = pack8(c, 0);
                at[1] = pack8(c, 8);
            }
            den += __shfl_xor(den, 32, 64);
            den_s[w][lo] = den; // both lane halves hold the full sum
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                // num tile nt: row 8(i/4) + 4h + i%4, column 32 nt + lo
                f32x16 c = zero16();
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) c = mfma(fq[mt][kk], pack8(S[mt][nt], 8 * kk), c);
                if (MODE == MODE_CAUSAL) {
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) c = mfma(at[kk], vfrag(kk, nt), c);
                }
                // blocks (nt, q) of the other waves go to LDS; this wave keeps (on, oq)
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    if (nt == on && q == oq) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) own[i] = c[8 * q + i];
                    } else {
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            const f32x4 x = {c[8 * q + 4 * j], c[8 * q + 4 * j + 1], c[8 * q + 4 * j + 2],
                                             c[8 * q + 4 * j + 3]};
                            *reinterpret_cast<f32x4*>(&red_s[nt][q][w][j][lane][0]) = x;
                        }
                    }
                }
            }
        }

        asm volatile("" ::: "memory");

        // ---- state update: S[F_w] += phi(K)^T V, z[F_w] += column sums ---------------
        if (HAS_K) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) S[mt][nt] = mfma(fk[mt][kk], vfrag(kk, nt), S[mt][nt]);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                zreg[nt] += zpart[nt] + __shfl_xor(zpart[nt], 32, 64);
                if (MODE == MODE_CAUSAL) z_s[f0 + 32 * nt + lo] = zreg[nt];
            }
        }

        if (HAS_Q) {
            sync_lds(); // (B) partial blocks and denominators of all waves in LDS
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) {
                if (w2 == w) continue;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const f32x4 x = *reinterpret_cast<const f32x4*>(&red_s[on][oq][w2][j][lane][0]);
                    own[4 * j] += x[0];
                    own[4 * j + 1] += x[1];
                    own[4 * j + 2] += x[2];
                    own[4 * j + 3] += x[3];
                }
            }
            u16* ob = a.out + (bh * a.N + c0) * DV + 32 * on + lo;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int tb = 16 * oq + 8 * j + 4 * h; // rows of regs 8 oq + 4 j .. + 3
                f32x4 dsum = *reinterpret_cast<const f32x4*>(&den_s[0][tb]);
#pragma unroll
                for (int w2 = 1; w2 < NW; ++w2) {
                    const f32x4 x = *reinterpret_cast<const f32x4*>(&den_s[w2][tb]);
                    dsum[0] += x[0];
                    dsum[1] += x[1];
                    dsum[2] += x[2];
                    dsum[3] += x[3];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float y = own[4 * j + e];
                    if (a.norm == NORM_ATTN) y *= __builtin_amdgcn_rcpf(fmaxf(dsum[e], a.eps));
                    own[4 * j + e] = y;
                }
            }
            if (rows == L) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int t = 16 * oq + 8 * (i >> 2) + 4 * h + (i & 3);
                    ob[(int64_t)t * DV] = __builtin_bit_cast(u16, (__bf16)own[i]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int t = 16 * oq + 8 * (i >> 2) + 4 * h + (i & 3);
                    if (t < rows) ob[(int64_t)t * DV] = __builtin_bit_cast(u16, (__bf16)own[i]);
                }
            }
        }

        // next chunk's V^T (its loads were issued above)
        if (HAS_K && rows_next > 0) {
            if (!PREFETCH) vr = load_v(vb + cn * DV, rows_next, tid);
            store_vt(vt_s[buf ^ 1], tid, vr);
        }
    }

    if (MODE == MODE_SUMS) {
        float* dst = a.state + bh * a.st_bh + g * a.st_g;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int f = f0 + 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
                    dst[(int64_t)f * DV + 32 * nt + lo] = S[mt][nt][i];
                }
        if (h == 0) {
            dst[(int64_t)R * DV + f0 + lo] = zreg[0];
            dst[(int64_t)R * DV + f0 + 32 + lo] = zreg[1];
        }
    }
}

FavorArgs make_args(const Cfg& c, const void* q, const void* k, const void* v, const void* omega,
                    Shape s, SegPlan sp, float* state, int64_t sbh, int64_t sg, void* out) {
    FavorArgs a;
    a.q = (const u16*)q;
    a.k = (const u16*)k;
    a.v = (const u16*)v;
    a.omega = (const u16*)omega;
    a.N = s.N;
    a.G = sp.G;
    a.seg_len = sp.seg_len;
    a.a_scale = c.scale * LOG2E;
    a.b_norm = -0.5f * c.scale * c.scale * LOG2E;
    a.b_const = c.favor_log2_bias;
    a.eps = c.eps;
    a.norm = c.norm;
    a.state = state;
    a.st_bh = sbh;
    a.st_g = sg;
    a.out = (u16*)out;
    return a;
}

} // namespace

bool favor_mfma_supported(const Cfg& c, int dtype) {
    return c.phi == PHI_FAVOR && dtype == 1 && c.r == R && c.sum_norm == 0;
}

hipError_t launch_favor_sums(const Cfg& c, const void* k, const void* v, const void* omega,
                             Shape s, SegPlan sp, float* ws, hipStream_t st) {
    const FavorArgs a = make_args(c, nullptr, k, v, omega, s, sp, ws, sp.G * state_elems(R),
                                  state_elems(R), nullptr);
    hipLaunchKernelGGL(k_favor_mfma<MODE_SUMS>, dim3((unsigned)(sp.G * s.BH)), dim3(NT), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_favor_outputs(const Cfg& c, int causal, const void* q, const void* k,
                                const void* v, const void* omega, Shape s, SegPlan sp,
                                const float* state, int64_t sbh, int64_t sg, void* out,
                                hipStream_t st) {
    const FavorArgs a = make_args(c, q, k, v, omega, s, sp, const_cast<float*>(state), sbh, sg, out);
    if (causal)
        hipLaunchKernelGGL(k_favor_mfma<MODE_CAUSAL>, dim3((unsigned)(sp.G * s.BH)), dim3(NT), 0, st, a);
    else
        hipLaunchKernelGGL(k_favor_mfma<MODE_READOUT>, dim3((unsigned)(sp.G * s.BH)), dim3(NT), 0, st, a);
    return hipGetLastError();
}

} // namespace linattn
