// favor_mfma.hip -- FAVOR+ attention on the matrix cores (bfloat16 inputs,
// r = 256 features, d = dv = 64, float32 accumulation and state).
//
// Forward outputs (k_favor_fused): one workgroup of four waves handles one
// sequence segment of one head, in chunks of 32 tokens (one MFMA tile: the
// intra-chunk block is a single masked 32 x 32 tile), two workgroups per CU.
// Wave w owns the 64 features F_w = [64w, 64w + 64) and does all of their
// work: projections and exponentials of the chunk's keys and queries
// (Kernel Zoo sec. 4.2 / 5.4 map), its share of the masked intra-chunk
// block, its partial readout against S_{c-1}[F_w] and the update
// S[F_w] += phi(K_c)^T V_c (sec. 1.3 recurrence in chunked form).  The four
// partial numerators and denominators are summed through LDS; each wave
// finishes a quarter of the chunk's output.
// Segment increments (k_favor_sums8): eight waves of 32 features each.
// Bidirectional readout (k_favor_readout): the summaries are fixed, so they
// sit in LDS as operand tables and every wave takes whole chunks on its own.
// Every contraction is a v_mfma_f32_32x32x16_bf16; the MFMA accumulator
// layout of one product is reused as an operand of the next where the
// contraction index allows it (a k-slot permutation applied to both
// operands).  The backward pass of both forms has matrix-core kernels here
// too: the bidirectional one with every wave on its own chunks against the
// totals, the causal one with each workgroup walking its segment and the
// state split over its waves by feature (see the comments at those kernels).
#include <atomic>

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

constexpr int NW = 4;         // feature groups of 64, one wave each
constexpr int R = 256;
constexpr int L = 32;         // chunk length: one 32-token MFMA tile
constexpr int LDV = 40;       // LDS row stride (bf16) of the V^T tile [64 n][32 t]: 80 B


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
    float* state;   // increments out (k_favor_sums8); carried-in states (causal); summaries (readout)
    int64_t st_bh;
    int64_t st_g;
    u16* out;
    const int64_t* tab; // segment table (packed sequences) or NULL
    int64_t tsub;       // parts per segment in the table
    const int64_t* order; // segment-major dispatch order or NULL (see SegPlan)
    int64_t osub;
    int64_t BH;
    const float* zw;      // k_favor_sums8: per-token weights of the z sum [BH, N], or NULL (weight 1)
    int64_t cus;          // compute units of the device (workgroups per dispatch round)
};

// The (head, segment) this workgroup runs; false when it runs nothing.
__device__ __forceinline__ bool block_segment(const FavorArgs& a, int64_t& bh, int64_t& g) {
    if (!a.order) {
        bh = blockIdx.x / a.G;
        g = blockIdx.x % a.G;
        return true;
    }
    const int64_t s = blockIdx.x / a.BH;
    bh = blockIdx.x % a.BH;
    const int64_t seg = a.order[s / a.osub];
    g = seg * a.osub + s % a.osub;
    return seg >= 0 && g < a.G;
}

// Two workgroups share each CU in the causal outputs kernel, and the
// hardware issues from the older one's waves first: left alone, the
// workgroup dispatched second trails by about a third (82 against 109 us at
// B=1, H=8, N=65536) and ends alone on its CU.  The two dispatch rounds
// instead take priority in turn, in slots of 1024 ticks (about 10 us) of the
// constant-rate clock, which keeps them level.  `now` is read before a
// barrier whose wait also covers it.
__device__ __forceinline__ void take_turns(uint64_t now, int round) {
    if ((((now >> 10) + (uint64_t)round) & 1) != 0)
        __builtin_amdgcn_s_setprio(1);
    else
        __builtin_amdgcn_s_setprio(0);
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

// Sum of the eight bfloat16 elements, two per v_dot2 against (1, 1).  The
// pairs are built from the elements: a bit cast of the vector to 32-bit
// words was lowered to the same register for different words.
__device__ __forceinline__ float sum8(const bf16x8& v) {
    const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
    float s0 = 0.f, s1 = 0.f;
    s0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[0], v[1]}, one, s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[2], v[3]}, one, s1, false);
    s0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[4], v[5]}, one, s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[6], v[7]}, one, s1, false);
    return s0 + s1;
}

// phi . z over the 16 features of a projection tile held as (p0, p1): word m
// of p0 / p1 (elements 2m, 2m + 1) holds the features 8 (m / 2) + 4 h +
// 2 (m % 2) + (0, 1) of the tile (+16 for p1), and zq[j] the bf16 z of the
// features 8 j + 4 h + (0..3); two dot2 chains.
__device__ __forceinline__ void dot_z(const bf16x8& p0, const bf16x8& p1, const uint2 (&zq)[4],
                                      float& d0, float& d1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const bf16x8& p = j < 2 ? p0 : p1;
        const int e = 4 * (j & 1);
        d0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p[e], p[e + 1]}, __builtin_bit_cast(bf16x2, zq[j].x), d0, false);
        d1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p[e + 2], p[e + 3]}, __builtin_bit_cast(bf16x2, zq[j].y), d1, false);
    }
}

// x[lane] + x[lane ^ 32]: the two lane halves exchanged by one
// v_permlane32_swap (no LDS round trip).
__device__ __forceinline__ float half_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over the eight consecutive lanes 8q .. 8q + 7 (every lane of the group
// gets the same bits): lane ^ 1 and lane ^ 2 within each quad, then the
// other quad of the group through the half-row mirror (lane i <-> 7 - i).
__device__ __forceinline__ float row8_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));
    return x;
}

// |x_t|^2 for t = lo from its fragments (the two lane halves hold
// complementary halves of the row); bf16 products are exact in float32.
__device__ __forceinline__ float sq_norm(const bf16x8 (&f)[4]) {
    float s[2] = {0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const bf16x2 x = {f[ks][e], f[ks][e + 1]};
            s[(e >> 1) & 1] = __builtin_amdgcn_fdot2_f32_bf16(x, x, s[(e >> 1) & 1], false);
        }
    return half_sum(s[0] + s[1]);
}

// A 4 x 4 block of bf16 held by the four lanes of a quad (lane e: row e,
// columns 0 .. 3 as two words of pairs) transposed within the quad: lane e
// gets column e, rows 0 .. 3.  Lanes e and e ^ 2 first swap the column pairs
// they do not keep, then lanes e and e ^ 1 swap halves (two DPP exchanges).
// Every lane of the quad must be active.
__device__ __forceinline__ uint2 quad_transpose4(uint2 x) {
    const int e = threadIdx.x & 3;
    // afterwards P holds row e % 2 and Q row 2 + e % 2, columns 2 (e / 2), +1
    const uint32_t send = e < 2 ? x.y : x.x;
    const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0x4E, 0xF, 0xF, true);
    const uint32_t mine = e < 2 ? x.x : x.y;
    const uint32_t P = e < 2 ? mine : recv, Q = e < 2 ? recv : mine;
    // the even lane keeps the first column of its pair, the odd lane the second
    const uint32_t pP = (uint32_t)__builtin_amdgcn_mov_dpp((int)P, 0xB1, 0xF, 0xF, true);
    const uint32_t pQ = (uint32_t)__builtin_amdgcn_mov_dpp((int)Q, 0xB1, 0xF, 0xF, true);
    if ((e & 1) == 0) return make_uint2((P & 0xffffu) | (pP << 16), (Q & 0xffffu) | (pQ << 16));
    return make_uint2((pP >> 16) | (P & 0xffff0000u), (pQ >> 16) | (Q & 0xffff0000u));
}

// Row length (bf16) of a row-major [token][64] table read by tr_operand:
// 192 bytes, so the four rows one 32-lane read touches (rows r .. r+3 at
// 48-dword steps) tile the 64 banks.
constexpr int LDR = 96;

typedef short i16x4 __attribute__((ext_vector_type(4)));

// The operand of a product over 16 tokens with the 32 lanes of each half on
// columns n0 .. n0+31 of a row-major [token][n] bf16 table (row length LDR),
// k-slot e holding token 16 kk + 8(e/4) + 4h + e%4 (the order of the
// operands made from accumulator tiles): two transposing LDS reads.  Within
// each group of 16 lanes, ds_read_b64_tr_b16 gives lane 4a + b the b-th
// 16-bit value of what lanes a, a+4, a+8, a+12 address, in that order; so
// lane r of the group addresses token 16 kk + 4h + r/4 (8 further for the
// second read) at columns n0 + 16 (group % 2) + 4 (r % 4).
__device__ __forceinline__ bf16x8 tr_operand(const u16* tab, int n0, int kk, int lane) {
    const int r = lane & 15, h = lane >> 5;
    const u16* p = tab + (16 * kk + 4 * h + (r >> 2)) * LDR + n0 + 16 * ((lane >> 4) & 1) + 4 * (r & 3);
    typedef i16x4 __attribute__((address_space(3))) * lds_i16x4;
    const i16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(p));
    const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(p + 8 * LDR));
    const u32x4 w = {(uint32_t)(uint16_t)x0[0] | ((uint32_t)(uint16_t)x0[1] << 16),
                     (uint32_t)(uint16_t)x0[2] | ((uint32_t)(uint16_t)x0[3] << 16),
                     (uint32_t)(uint16_t)x1[0] | ((uint32_t)(uint16_t)x1[1] << 16),
                     (uint32_t)(uint16_t)x1[2] | ((uint32_t)(uint16_t)x1[3] << 16)};
    return __builtin_bit_cast(bf16x8, w);
}

// V of the chunk for a row-major LDS copy: thread th (of 256) holds row
// th / 8, columns 8 (th % 8) .. +7 (rows past `rows` repeat row rows-1).
__device__ __forceinline__ bf16x8 load_vrow(const u16* __restrict__ V, int rows, int tid) {
    return *reinterpret_cast<const bf16x8*>(V + (int64_t)min(tid >> 3, rows - 1) * DV + 8 * (tid & 7));
}

// Raw V rows of the chunk for the transposed LDS copy: thread th (of 256)
// holds row 4 (th / 32) + th % 4, columns 8 ((th / 4) % 8) .. +7, so the four
// lanes of a quad hold four consecutive rows of the same columns (rows past
// `rows` repeat row rows-1; they only ever meet zero weights).
__device__ __forceinline__ int v_row(int tid) { return 4 * (tid >> 5) + (tid & 3); }
__device__ __forceinline__ int v_col(int tid) { return 8 * ((tid >> 2) & 7); }
__device__ __forceinline__ bf16x8 load_v(const u16* __restrict__ V, int rows, int tid) {
    return *reinterpret_cast<const bf16x8*>(V + (int64_t)min(v_row(tid), rows - 1) * DV + v_col(tid));
}

// V^T in LDS: row n holds V[t][n] at column vt_col(n, swap23(t)); the
// 16-byte chunks of a row are rotated by (n / 8) % 4 so that the transposing
// stores fall on different banks.
__device__ __forceinline__ int vt_col(int n, int c) { return (((c >> 3) ^ ((n >> 3) & 3)) << 3) | (c & 7); }

// The quad's 4 rows x 8 columns, transposed within the quad as two 4 x 4
// blocks: lane e writes columns n0 + e and n0 + 4 + e, four rows each, as
// 8-byte pieces (four consecutive rows from a multiple of 4 keep their order
// under swap23 and vt_col).  Called by all four lanes of every quad.
__device__ __forceinline__ void store_vt(u16* vt, int tid, const bf16x8& vr) {
    const int t = swap23(v_row(tid) & ~3), n0 = v_col(tid), e = tid & 3;
    const u32x4 w = __builtin_bit_cast(u32x4, vr);
    const uint2 lo = quad_transpose4(make_uint2(w[0], w[1]));
    const uint2 hi = quad_transpose4(make_uint2(w[2], w[3]));
    *reinterpret_cast<uint2*>(vt + (n0 + e) * LDV + vt_col(n0 + e, t)) = lo;
    *reinterpret_cast<uint2*>(vt + (n0 + 4 + e) * LDV + vt_col(n0 + 4 + e, t)) = hi;
}

// omega[f0 + 32 t + lo][16 ks + 8 h ..]: A operand of omega X^T (t = feature
// tile as M) and B operand of X omega^T (t = feature tile as N) at once.
__device__ __forceinline__ bf16x8 omega_frag(const u16* __restrict__ omega, int f0, int t, int ks,
                                             int lo, int h) {
    return *reinterpret_cast<const bf16x8*>(omega + (int64_t)(f0 + 32 * t + lo) * D + 16 * ks + 8 * h);
}

// Swizzled LDS copy of one chunk of 32 rows x 64 bfloat16 (4 KB): row t,
// 16-byte column block j is stored at block index 8t + (j ^ (t & 7)), so that
// the MFMA operand reads (row = lane, one block per lane) hit all banks.
__device__ __forceinline__ int xs_index(int t, int j) { return 8 * t + (j ^ (t & 7)); }

// Thread th (of 256) loads block th of the chunk: row th / 8, block
// (th % 8) ^ (row % 8), i.e. the block it will store at index th.  Rows past
// `rows` repeat row rows-1.
__device__ __forceinline__ bf16x8 load_block(const u16* __restrict__ X, int rows, int th) {
    const int t = th >> 3, j = (th & 7) ^ (t & 7);
    return *reinterpret_cast<const bf16x8*>(X + (int64_t)min(t, rows - 1) * D + 8 * j);
}

// f[ks] = X[lo][16 ks + 8 h .. +7] from the swizzled copy (as load_x).
__device__ __forceinline__ void lds_x(const bf16x8* xs, int lo, int h, bf16x8 (&f)[4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) f[ks] = xs[xs_index(lo, 2 * ks + h)];
}

// B operand of a transposition through the matrix core: k-slot e of lane
// (n, h) is 1 where token 16 kk + 8(e/4) + 4h + e%4 equals n.  With an
// operand X whose lanes are features and whose k-slots are those tokens,
// sum_kk mfma(X_kk, eye_kk) is X transposed (tokens on lanes), exactly:
// every output is one bfloat16 product by 1 plus zeros.
__device__ __forceinline__ bf16x8 eye_frag(int kk, int lo, int h) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)(16 * kk + 8 * (e >> 2) + 4 * h + (e & 3) == lo ? 1.f : 0.f);
    return r;
}

// ---------------------------------------------------------------------------
// Causal outputs with symmetric waves: k_favor_fused<NORM>.
//
// One workgroup of four waves per (head, segment), two workgroups per CU, so
// that each SIMD runs two independent waves (of different segments).  Wave w
// owns the 64 features F_w = [64w, 64w + 64) and does all of their work for
// every 32-token chunk c: the projections P_K = K_c omega_w^T and
// P_Q^T = omega_w Q_c^T, both exponentials, the partial denominators
// phi(Q_c) z_{c-1}[F_w], the masked intra-chunk block over F_w, the partial
// numerator phi(Q_c) S_{c-1}[F_w] + (block) V_c, and the update
// S[F_w] += phi(K_c)^T V_c (Kernel Zoo sec. 1.3 recurrence in chunked form,
// the maps of sec. 4.2 / 5.4).  The four partial numerators and
// denominators meet in LDS; each wave then finishes a quarter of the chunk's
// output.  q, k and V^T are staged once per workgroup (one 16-byte block of
// each per thread), one chunk ahead; the partial buffers are double-buffered
// by chunk, so one workgroup barrier per chunk suffices.
// Layouts: S[mt][nt] element i is
// S[f0 + 32 mt + 8 (i/4) + 4 h + i%4][32 nt + lo]; phi(K) leaves the
// projection with features on lanes (the A operand of the update) and is
// transposed through the matrix core for the intra-chunk block; phi(Q) leaves
// it with tokens on lanes (the A operand of the readout).
// ---------------------------------------------------------------------------
constexpr int NTF = 64 * NW;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Raw buffer resource over rows [row0, row0 + rows) of an output [*, DV] in
// bfloat16: word 3 selects 32-bit raw accesses with range checking, so
// stores at byte offsets past rows * 2 DV are discarded by the hardware.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rows(u16* out, int64_t row0, int rows) {
    return __builtin_amdgcn_make_buffer_rsrc(out + row0 * DV, 0, rows * DV * 2, 0x00020000);
}

struct SmemF {
    bf16x8 xq[2][256];                  // swizzled q chunk [chunk parity]
    bf16x8 xk[2][256];                  // swizzled k chunk
    u16 vt[2][DV * LDV];                // V^T of the chunk
    float red[2][NW][NW - 1][2][64][4]; // partial numerator blocks [parity][owner][sender][j][lane]
    float dpart[2][L][NW];              // partial denominators [parity][token][group]
    float qb[2][L];                     // query biases by token
    float kb[2][L];                     // key biases by token (-inf past the segment end)
    u16 zb[R];                          // z_{c-1} by feature in bf16 (wave w reads and writes F_w only)
    bf16x8 eye[2][64];                  // identity operands of the transposition, by lane
};

// Columns [32 (W%2) + 16 (W/2), +16) of the chunk's output, all 32 tokens,
// finished by wave W: its own partial (accumulator elements 8 (W/2) .. +7 of
// tile W%2: token lo, columns 4h + {0..3} and 8 + 4h + {0..3} of the block)
// plus the three others from LDS, times the reciprocal of token lo's
// denominator, stored as two 8-byte pieces per lane.
template <int W, int NORM>
__device__ __forceinline__ void finish_fused(const FavorArgs& a, SmemF& sm, const f32x16 (&acc)[2],
                                             int lane, int slot, int64_t bh, int64_t c0, int rows) {
    constexpr int ON = W & 1, OQ = W >> 1;
    const int lo = lane & 31, h = lane >> 5;
    f32x4 part[NW - 1][2];
#pragma unroll
    for (int s = 0; s < NW - 1; ++s)
#pragma unroll
        for (int j = 0; j < 2; ++j) part[s][j] = *reinterpret_cast<const f32x4*>(&sm.red[slot][W][s][j][lane][0]);
    f32x4 dg;
    if (NORM == NORM_ATTN) dg = *reinterpret_cast<const f32x4*>(&sm.dpart[slot][lo][0]);
    float own[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        own[i] = acc[ON][8 * OQ + i];
#pragma unroll
        for (int s = 0; s < NW - 1; ++s) own[i] += part[s][i >> 2][i & 3];
    }
    if (NORM == NORM_ATTN) {
        const float rd = __builtin_amdgcn_rcpf(fmaxf((dg[0] + dg[1]) + (dg[2] + dg[3]), a.eps));
#pragma unroll
        for (int i = 0; i < 8; ++i) own[i] *= rd;
    }
    // unconditional stores through a buffer resource that covers exactly the
    // chunk's rows: the hardware drops the rows past the segment end, so no
    // lane branches around the store and the count of memory operations in
    // flight stays the same on every path (a branch here makes the next
    // chunk's wait for its prefetched loads also wait for these stores)
    const __amdgpu_buffer_rsrc_t orsrc = out_rows(a.out, bh * a.N + c0, rows);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const bf16x2 p0 = {(__bf16)own[4 * j], (__bf16)own[4 * j + 1]};
        const bf16x2 p1 = {(__bf16)own[4 * j + 2], (__bf16)own[4 * j + 3]};
        const u32x2 v2 = {__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
        __builtin_amdgcn_raw_buffer_store_b64(v2, orsrc, lo * (DV * 2) + 2 * (32 * ON + 16 * OQ + 4 * h + 8 * j), 0, 0);
    }
}

// The whole segment for wave W (features F_W); every wave-dependent index is
// a compile-time constant.
template <int NORM, int W>
__device__ __forceinline__ void fused_wave(const FavorArgs& a, SmemF& sm, int tid, int64_t bh,
                                           int64_t g, int64_t t0, int64_t t1, int nck) {
    constexpr int f0 = 64 * W;
    const int lane = tid & 63, lo = lane & 31, h = lane >> 5;
    auto rows_of = [&](int c) { return (int)min<int64_t>(L, t1 - t0 - (int64_t)L * c); };

    bf16x8 om[2][4]; // omega[f0 + 32 t + lo][16 ks + 8 h ..]
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) om[t][ks] = omega_frag(a.omega, f0, t, ks, lo, h);

    // carried-in state
    const float* st = a.state + bh * a.st_bh + g * a.st_g;
    f32x16 S[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int f = f0 + 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
                S[mt][nt][i] = st[(int64_t)f * DV + 32 * nt + lo];
            }
    float zreg[2]; // z[f0 + 32 nt + lo]
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) zreg[nt] = st[(int64_t)R * DV + f0 + 32 * nt + lo];
    // both lane halves store the same value at the same address
    sm.zb[f0 + lo] = __builtin_bit_cast(u16, (__bf16)zreg[0]);
    sm.zb[f0 + 32 + lo] = __builtin_bit_cast(u16, (__bf16)zreg[1]);
    // identity operands of the transposition (read back once per chunk: kept
    // in LDS rather than in eight registers)
    if (W < 2) sm.eye[W][lane] = eye_frag(W, lo, h);
    // causal mask of the diagonal tile: element i of lane (lo, h) pairs query
    // lo with key 8(i/4) + 4h + i%4, kept when 8(i/4) + i%4 <= lo - 4h
    const int keep_thr = lo - 4 * h;

    const u16* qg = a.q + bh * a.N * D;
    const u16* kg = a.k + bh * a.N * D;
    const u16* vg = a.v + bh * a.N * DV;
    auto chunk_ptr = [&](const u16* base, int c, int width) { return base + (t0 + (int64_t)L * c) * width; };
    // staging: thread tid holds one 16-byte block of the chunk's q, k and v
    bf16x8 qr, kr, vr;
    auto stage_load = [&](int c) {
        qr = load_block(chunk_ptr(qg, c, D), rows_of(c), tid);
        kr = load_block(chunk_ptr(kg, c, D), rows_of(c), tid);
        vr = load_v(chunk_ptr(vg, c, DV), rows_of(c), tid);
    };
    // the per-token biases of a chunk, once per workgroup: the eight threads
    // of a row sum their squares; keys past the segment end get -inf (exp2
    // gives 0, so they add nothing to S, z or the intra-chunk block)
    auto row_sq = [&](const bf16x8& blk) {
        float sq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const bf16x2 x = {blk[e], blk[e + 1]};
            sq = __builtin_amdgcn_fdot2_f32_bf16(x, x, sq, false);
        }
        return row8_sum(sq);
    };
    auto stage_store = [&](int c) {
        const int s = c & 1, t = tid >> 3;
        sm.xq[s][tid] = qr;
        // (all eight threads of the row hold the sum and write the same value:
        // a write by one of them only would become a branch)
        const float sq = row_sq(qr);
        sm.qb[s][t] = fmaf(a.b_norm, sq, a.b_const);
        sm.xk[s][tid] = kr;
        const float sk = row_sq(kr);
        sm.kb[s][t] = t < rows_of(c) ? fmaf(a.b_norm, sk, a.b_const) : -INFINITY;
        store_vt(sm.vt[s], tid, vr);
    };

    // projections of one 32 x 32 tile from the chunk's fragments
    bf16x8 qf[4], kf[4];
    auto project_k = [&](int t) {
        f32x16 c = zero16();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) c = mfma(kf[ks], om[t][ks], c);
        return c;
    };
    auto project_q = [&](int t) {
        f32x16 c = zero16();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) c = mfma(om[t][ks], qf[ks], c);
        return c;
    };
    // P0, P1: the first two (key) projection tiles of the chunk about to be
    // processed, issued one iteration early
    f32x16 P0, P1;
    auto first_tiles = [&](int s) {
        lds_x(sm.xq[s], lo, h, qf);
        lds_x(sm.xk[s], lo, h, kf);
        P0 = project_k(0);
        P1 = project_k(1);
    };

    if (nck > 0) {
        stage_load(0);
        stage_store(0);
        stage_load(min(1, nck - 1));
    }
    sync_lds(); // chunk 0 staged, z in LDS

    f32x16 acc[2]; // partial numerator of the chunk, transposed (see below)
    for (int ci = 0; ci < nck; ++ci) {
        const int slot = ci & 1;
        first_tiles(slot);
        // the next chunk into the other slot (its readers finished at the last
        // barrier), then the loads of the one after it (the last chunk again
        // past the end, so every iteration issues the same loads)
        if (ci + 1 < nck) stage_store(ci + 1);
        stage_load(min(ci + 2, nck - 1));
        // the previous chunk's output, stored here rather than at the end of
        // its iteration: the loads waited for at the top of the next iteration
        // then never have a store issued just before their wait (loads and
        // stores share one in-order counter, and with both in flight every
        // wait becomes a wait for all of them)
        if (ci > 0) finish_fused<W, NORM>(a, sm, acc, lane, slot ^ 1, bh, t0 + (int64_t)L * (ci - 1), rows_of(ci - 1));

        // ---- exponentials, one 32 x 32 tile at a time: the query tiles are
        // projected on the matrix core while the key tiles are exponentiated
        bf16x8 fk[2][2], fq[2][2];
        float zpart[2] = {0.f, 0.f};
        float dacc[2] = {0.f, 0.f};
        const float bq = sm.qb[slot][lo];
        // phi(K) tile nt: exponentials, bf16 operands, column sums (z sums the
        // bfloat16 features that also enter S)
        auto key_tile = [&](f32x16& c, int nt) {
            f32x4 kbias[4]; // biases of the tokens 8 j + 4 h + (0..3)
#pragma unroll
            for (int j = 0; j < 4; ++j) kbias[j] = *reinterpret_cast<const f32x4*>(&sm.kb[slot][8 * j + 4 * h]);
#pragma unroll
            for (int i = 0; i < 16; ++i) c[i] = __builtin_amdgcn_exp2f(fmaf(c[i], a.a_scale, kbias[i >> 2][i & 3]));
            fk[nt][0] = pack8(c, 0);
            fk[nt][1] = pack8(c, 8);
            zpart[nt] = sum8(fk[nt][0]) + sum8(fk[nt][1]);
        };
        // phi(Q) tile mt and its denominators against z_{c-1}: phi . z in the
        // bf16 roundings the numerator's products use (phi and S are bf16
        // there); word m of fq[mt][0] / [1] holds the features
        // f0 + 32 mt + 8 (m / 2) + 4 h + 2 (m % 2) + (0, 1) (+16 for [1]), as
        // does the bf16 z word read at the same features
        auto query_tile = [&](f32x16& c, int mt) {
            // z_{c-1} of the features f0 + 32 mt + 8 j + 4 h + (0..3); read by
            // memcpy, as the writes are 16-bit: a typed 8-byte load would be
            // assumed not to alias them and could move past the update below
            uint2 zq[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) __builtin_memcpy(&zq[j], &sm.zb[f0 + 32 * mt + 8 * j + 4 * h], sizeof(uint2));
#pragma unroll
            for (int i = 0; i < 16; ++i) c[i] = __builtin_amdgcn_exp2f(fmaf(c[i], a.a_scale, bq));
            fq[mt][0] = pack8(c, 0);
            fq[mt][1] = pack8(c, 8);
            if (NORM == NORM_ATTN) dot_z(fq[mt][0], fq[mt][1], zq, dacc[0], dacc[1]);
        };
        key_tile(P0, 0);
        P0 = project_q(0);
        key_tile(P1, 1);
        P1 = project_q(1);
        query_tile(P0, 0);
        query_tile(P1, 1);
        float den = NORM == NORM_ATTN ? half_sum(dacc[0] + dacc[1]) : 0.f; // token lo, both halves
        // (no scheduling barriers between the phases below: letting the
        // compiler interleave them took 116 -> 113 us at 256 registers)

        // ---- z[F_W] += column sums of phi(K_c), after the queries read z_{c-1} ----
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            zreg[nt] += half_sum(zpart[nt]);
            sm.zb[f0 + 32 * nt + lo] = __builtin_bit_cast(u16, (__bf16)zreg[nt]); // both halves: same value
        }

        const u16* vt = sm.vt[slot];
        // V^T fragment (kk, nt): lane <-> column 32 nt + lo, k-slot e <-> token
        // 16 kk + 8 (e/4) + 4 h + e%4
        auto vfrag = [&](int kk, int nt) {
            return lds8(vt + (32 * nt + lo) * LDV + vt_col(32 * nt + lo, 16 * kk + 8 * h));
        };

        // ---- masked intra-chunk block over F_W --------------------------------------
        bf16x8 at[2];
        {
            // phi(K) with tokens on lanes: lane (j, h), k-slot e <-> feature
            // f0 + 32 mt + 16 kk + 8(e/4) + 4h + e%4, as in fq
            bf16x8 kt[2][2];
            const bf16x8 eye[2] = {sm.eye[0][lane], sm.eye[1][lane]};
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                f32x16 t = zero16();
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) t = mfma(fk[mt][kk], eye[kk], t);
                kt[mt][0] = pack8(t, 0);
                kt[mt][1] = pack8(t, 8);
            }
            // m[i] = A[lo][j] over F_W, j = 8(i/4) + 4h + i%4
            f32x16 m = zero16();
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) m = mfma(kt[mt][kk], fq[mt][kk], m);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                m[i] = 8 * (i >> 2) + (i & 3) <= keep_thr ? m[i] : 0.f;
                // kept as a float32 select (otherwise the compiler converts
                // each element alone and masks and repacks the halves)
                asm volatile("" : "+v"(m[i]));
            }
            at[0] = pack8(m, 0);
            at[1] = pack8(m, 8);
            // the block's row sums from the bf16 values its product with V uses
            if (NORM == NORM_ATTN) den += half_sum(sum8(at[0]) + sum8(at[1]));
        }

        // ---- partial numerator, transposed (columns as rows, tokens on lanes):
        //   acc^T = S_{c-1}[F_W]^T phi(Q)^T + V^T (block)^T
        // S's accumulator tile packed to bf16 is the A operand of S^T as is.
        // acc[nt] element i: column 32 nt + 8(i/4) + 4h + i%4, token lo
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            acc[nt] = zero16();
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    acc[nt] = mfma(pack8(S[mt][nt], 8 * kk), fq[mt][kk], acc[nt]);
        }
        {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) acc[nt] = mfma(vfrag(kk, nt), at[kk], acc[nt]);
            // ---- state update: S[F_W] += phi(K)^T V ---------------------------------
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) S[mt][nt] = mfma(fk[mt][kk], vfrag(kk, nt), S[mt][nt]);
        }

        // ---- exchange: columns [32 nt + 16 q, +16) belong to wave nt + 2 q ---------
        if (NORM == NORM_ATTN) sm.dpart[slot][lo][W] = den; // both halves: same value
        {
            float(&red)[NW][NW - 1][2][64][4] = sm.red[slot];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int owner = nt + 2 * q;
                    if (owner == W) continue;
                    const int sl = W < owner ? W : W - 1;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const f32x4 x = {acc[nt][8 * q + 4 * j], acc[nt][8 * q + 4 * j + 1],
                                         acc[nt][8 * q + 4 * j + 2], acc[nt][8 * q + 4 * j + 3]};
                        *reinterpret_cast<f32x4*>(&red[owner][sl][j][lane][0]) = x;
                    }
                }
        }
        const uint64_t now = __builtin_amdgcn_s_memrealtime();
        sync_lds(); // partials of chunk ci in LDS; chunk ci + 1 staged
        take_turns(now, (int)(blockIdx.x / a.cus));

        // the next chunk's first projections run on the matrix core while this
        // chunk's output is finished
    }
    if (nck > 0) finish_fused<W, NORM>(a, sm, acc, lane, (nck - 1) & 1, bh, t0 + (int64_t)L * (nck - 1), rows_of(nck - 1));
}

template <int NORM>
__global__ __launch_bounds__(NTF, 2) void k_favor_fused(FavorArgs a) {
    __shared__ SmemF sm;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6); // wave index, uniform
    int64_t bh, g;
    if (!block_segment(a, bh, g)) return; // uniform over the workgroup
    int64_t t0, t1;
    seg_range(a.tab, a.tsub, g, a.seg_len, a.N, t0, t1);
    const int nck = t1 > t0 ? (int)((t1 - t0 + L - 1) / L) : 0;
    switch (w) {
    case 0: fused_wave<NORM, 0>(a, sm, tid, bh, g, t0, t1, nck); break;
    case 1: fused_wave<NORM, 1>(a, sm, tid, bh, g, t0, t1, nck); break;
    case 2: fused_wave<NORM, 2>(a, sm, tid, bh, g, t0, t1, nck); break;
    default: fused_wave<NORM, 3>(a, sm, tid, bh, g, t0, t1, nck); break;
    }
}

// Segment sums (increments of S and z) with eight symmetric waves: wave w
// owns the 32 features F_w = [32w, 32w + 32) and, per chunk, projects the
// keys on its rows of omega, takes the exponentials and adds
// phi(K)[:, F_w]^T V to its slice of S in MFMA accumulators.  Nothing is
// reduced across waves; the chunk's keys, their per-token biases and V^T
// are loaded (computed) once per workgroup by waves 0..3 and staged in LDS
// (one barrier per chunk), and every wave has the same mix of matrix-core
// and vector work.
constexpr int NT8 = 512;
// ZW: the z sum weighted per token by a.zw (a separate instantiation, so the
// plain one keeps its registers).
template <bool ZW>
__global__ __launch_bounds__(NT8, 2) void k_favor_sums8(FavorArgs a) {
    __shared__ __attribute__((aligned(16))) u16 vr_s[2][L * LDR]; // V, row-major [token][n]
    __shared__ bf16x8 ks_s[2][256];
    __shared__ __attribute__((aligned(16))) float kb_s[2][L]; // key biases by chunk parity
    __shared__ __attribute__((aligned(16))) float zw_s[ZW ? 2 : 1][L]; // z weights by chunk parity
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lo = lane & 31, h = lane >> 5;
    const int f0 = 32 * w;
    int64_t bh, g;
    if (!block_segment(a, bh, g)) return; // uniform over the workgroup
    int64_t t0, t1;
    seg_range(a.tab, a.tsub, g, a.seg_len, a.N, t0, t1);
    const int nck = t1 > t0 ? (int)((t1 - t0 + L - 1) / L) : 0;
    auto rows_of = [&](int c) { return (int)min<int64_t>(L, t1 - t0 - (int64_t)L * c); };
    const bool stager = w < 4; // waves 0..3 (threads 0..255) stage K and V^T

    bf16x8 om[4]; // omega[f0 + lo][16 ks + 8 h ..]
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) om[ks] = omega_frag(a.omega, f0, 0, ks, lo, h);
    f32x16 S[2] = {zero16(), zero16()}; // S[f0 + 8(i/4) + 4h + i%4][32 nt + lo]
    float zacc = 0.f;                   // z[f0 + lo]

    const u16* kb = a.k + bh * a.N * D;
    const u16* vb = a.v + bh * a.N * DV;
    auto kchunk = [&](int c) { return kb + (t0 + (int64_t)L * c) * D; };
    auto vchunk = [&](int c) { return vb + (t0 + (int64_t)L * c) * DV; };
    // stagers hold the keys (and z weights) of chunk c + 1 and the values of
    // chunk c in registers at the top of iteration c
    bf16x8 kr, vr;
    float zr = 0.f; // ZW: the weight of token tid / 8 (the eight threads of a row alike)
    const float* zwb = ZW ? a.zw + bh * a.N + t0 : nullptr;
    auto load_zw = [&](int c) {
        if (ZW) zr = zwb[(int64_t)L * c + min(tid >> 3, rows_of(c) - 1)];
    };
    auto stage_zw = [&](int c) {
        if (ZW) zw_s[c & 1][tid >> 3] = (tid >> 3) < rows_of(c) ? zr : 0.f;
    };
    // the key bias of a chunk is computed once, by the stagers, from the
    // blocks they hold: the eight threads of a row sum their squares (keys
    // past the end of the segment get bias -inf, so exp2 gives 0) and all
    // eight write it (a write by one of them only would become a branch)
    auto stage_bias = [&](const bf16x8& blk, int c) {
        float sq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const bf16x2 x = {blk[e], blk[e + 1]};
            sq = __builtin_amdgcn_fdot2_f32_bf16(x, x, sq, false);
        }
        sq = row8_sum(sq);
        const int t = tid >> 3;
        kb_s[c & 1][t] = t < rows_of(c) ? fmaf(a.b_norm, sq, a.b_const) : -INFINITY;
    };
    if (nck > 0 && stager) {
        const bf16x8 k0 = load_block(kchunk(0), rows_of(0), tid);
        load_zw(0);
        ks_s[0][tid] = k0;
        stage_bias(k0, 0);
        stage_zw(0);
        const int c1 = min(1, nck - 1);
        kr = load_block(kchunk(c1), rows_of(c1), tid);
        load_zw(c1);
        vr = load_vrow(vchunk(0), rows_of(0), tid);
    }
    sync_lds(); // keys of chunk 0 staged
    wait_all_loads(); // omega's fragments, once, not in every iteration

    for (int ci = 0; ci < nck; ++ci) {
        if (stager) {
            // past the end: the last chunk again, so every iteration has the same loads
            const int c1 = min(ci + 1, nck - 1), c2 = min(ci + 2, nck - 1);
            ks_s[(ci + 1) & 1][tid] = kr;
            if (ci + 1 < nck) {
                stage_bias(kr, ci + 1);
                stage_zw(ci + 1);
            }
            // V of this chunk, row-major (rows past the end repeat the last
            // row; they meet zero features)
            *reinterpret_cast<bf16x8*>(&vr_s[ci & 1][(tid >> 3) * LDR + 8 * (tid & 7)]) = vr;
            kr = load_block(kchunk(c2), rows_of(c2), tid);
            load_zw(c2);
            vr = load_vrow(vchunk(c1), rows_of(c1), tid);
        }
        bf16x8 kf[4];
        lds_x(ks_s[ci & 1], lo, h, kf);
        f32x16 c = zero16();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) c = mfma(kf[ks], om[ks], c); // token 8(i/4)+4h+i%4, feature f0+lo
        f32x4 kbias[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) kbias[j] = *reinterpret_cast<const f32x4*>(&kb_s[ci & 1][8 * j + 4 * h]);
#pragma unroll
        for (int i = 0; i < 16; ++i) c[i] = __builtin_amdgcn_exp2f(fmaf(c[i], a.a_scale, kbias[i >> 2][i & 3]));
        const bf16x8 fk0 = pack8(c, 0), fk1 = pack8(c, 8);
        if (!ZW) {
            zacc += sum8(fk0) + sum8(fk1); // the bfloat16 features that also enter S
        } else {
            // weighted: element i is token 8(i/4) + 4h + i%4 of the chunk (the
            // staged weights are zero past the end)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 wz = *reinterpret_cast<const f32x4*>(&zw_s[ci & 1][8 * j + 4 * h]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * j + e;
                    zacc = fmaf((float)(i < 8 ? fk0[i] : fk1[i - 8]), wz[e], zacc);
                }
            }
        }
        sync_lds(); // V^T of this chunk and the keys of the next staged
        const u16* vr = vr_s[ci & 1];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            S[nt] = mfma(fk0, tr_operand(vr, 32 * nt, 0, lane), S[nt]);
            S[nt] = mfma(fk1, tr_operand(vr, 32 * nt, 1, lane), S[nt]);
        }
    }
    float* dst = a.state + bh * a.st_bh + g * a.st_g;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int f = f0 + 8 * (i >> 2) + 4 * h + (i & 3);
            dst[(int64_t)f * DV + 32 * nt + lo] = S[nt][i];
        }
    const float zt = half_sum(zacc);
    if (h == 0) dst[(int64_t)R * DV + f0 + lo] = zt;
}

// ---------------------------------------------------------------------------
// Backward of the bidirectional form on the matrix cores (see backward.hip
// for the derivatives).  The state is one total per head, so every wave
// takes its own 32-token chunks and nothing is exchanged between waves:
// the workgroup first builds bf16 operand tables of the state and of
// omega^T in LDS, then each wave walks its chunks over the 8 feature tiles.
//   query pass:  phi(Q)^T per tile (omega Q^T, exp), num^T += S^T phi(Q)^T,
//                den; then dnum, dden; then per tile
//                dphi(Q)^T = S dnum^T + z dden^T, w = dphi o phi,
//                du^T += omega^T w^T; dq = scale (du - (sum_f w) u).
//                dnum (bf16) and dden go to memory for the backward state.
//   key pass:    per tile phi(K)^T, dphi(K)^T = G V^T + g, dv^T += G^T phi(K)^T,
//                w, du^T; dk = scale (du - (sum_f w) u).
// Tables store the 16-blocks of their contraction index in swap23 order, so
// an accumulator tile of the previous product is the other operand as is.
// ---------------------------------------------------------------------------
constexpr int NTB = 512;          // 8 waves, one chunk each at a time
constexpr int64_t BWD_BIDIR_BLOCKS = 256; // workgroups of a bidirectional backward pass
constexpr int LDF = R + 8;        // row length of the [64][R] tables (bank spread)
constexpr int LDN = DV + 8;       // row length of the [R][64] table

struct BwdArgs {
    const u16* x;      // q (query pass) or k (key pass) [BH, N, D]
    const u16* y;      // dout (query pass) or v (key pass) [BH, N, DV]
    const u16* omega;  // [R, D]
    const float* st;   // per head: (S | z) total (query pass) or (G | g) total (key pass)
    int64_t N, G, seg_len;
    float a_scale, b_norm, b_const, scale, eps;
    int norm;
    u16* dx;           // dq or dk [BH, N, D]
    u16* dy;           // key pass: dv [BH, N, DV]; query pass: dnum (bf16) [BH, N, DV]
    float* dden;       // query pass: dden [BH, N]
};

struct BwdTables {
    u16 mt[DV * LDF];   // M^T [n][f']: M[16b + swap23(j)][n] at column 16b + j
    u16 mn[R * LDN];    // query pass: S [f][n'] (n in swap23 order); key pass: G [f][n] natural
    u16 wt[D * LDF];    // omega^T [d][f']: omega[16b + swap23(j)][d] at column 16b + j
    bf16x8 om[R * 8];   // omega rows, 16-byte block j of row f at xs_index(f, j)
    float m1[R];        // z or g
};

__device__ __forceinline__ u16 f2bf(float x) { return __builtin_bit_cast(u16, (__bf16)x); }

// Build the tables from the head's state total (float32 [R][DV] then [R])
// and omega; `swap_n`: store the n index of mn in swap23 order.  Every
// global load is issued before the first LDS write (one round trip), and
// each thread writes whole 16-byte words where the layout allows.
__device__ void build_tables(BwdTables& tb, const float* __restrict__ st,
                             const u16* __restrict__ omega, bool swap_n) {
    const int tid = threadIdx.x;
    // M^T: thread (n, q) forms the words at positions 8 q' .. 8 q' + 7 of
    // row n, q' = q + 8 u: features 16 (q' / 2) + swap23(8 (q' % 2) + e)
    constexpr int NU = R / 8 / (NTB / DV);
    const int n = tid & (DV - 1), q = tid / DV;
    float sv[NU][8];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int qq = q + (NTB / DV) * u;
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[u][e] = st[(16 * (qq >> 1) + swap23(8 * (qq & 1) + e)) * DV + n];
    }
    // M: thread (f, half) holds 32 consecutive n of row f (8 float4) for
    // f = tid / 2 (R rows, two threads each)
    const int fr = tid >> 1, nh = 32 * (tid & 1);
    f32x4 mv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) mv[u] = *reinterpret_cast<const f32x4*>(st + (int64_t)fr * DV + nh + 4 * u);
    // omega: four 16-byte blocks per thread (as 32-bit words: single bf16
    // elements are taken by shifts, not vector-element casts)
    constexpr int NO = R * 8 / NTB;
    u32x4 ov[NO];
#pragma unroll
    for (int u = 0; u < NO; ++u) {
        const int b = tid + NTB * u;
        ov[u] = *reinterpret_cast<const u32x4*>(omega + (int64_t)(b >> 3) * D + 8 * (b & 7));
    }
    const float m1v = st[R * DV + (tid & (R - 1))];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        bf16x8 w;
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = (__bf16)sv[u][e];
        *reinterpret_cast<bf16x8*>(&tb.mt[n * LDF + 8 * (q + (NTB / DV) * u)]) = w;
    }
    // row fr of mn: positions p hold n = swap23 within each 16-block (or n)
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            bf16x8 w;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = swap_n ? swap23(8 * half + e) : 8 * half + e; // n within the 16-block
                w[e] = (__bf16)mv[4 * blk + (j >> 2)][j & 3];
            }
            *reinterpret_cast<bf16x8*>(&tb.mn[fr * LDN + nh + 16 * blk + 8 * half]) = w;
        }
#pragma unroll
    for (int u = 0; u < NO; ++u) {
        const int b = tid + NTB * u, f = b >> 3, d0 = 8 * (b & 7);
        *reinterpret_cast<u32x4*>(&tb.om[xs_index(f, b & 7)]) = ov[u];
        const int fc = (f & ~15) + swap23(f & 15);
#pragma unroll
        for (int e = 0; e < 8; ++e) tb.wt[(d0 + e) * LDF + fc] = (u16)(ov[u][e >> 1] >> (16 * (e & 1)));
    }
    if (tid < R) tb.m1[tid] = m1v;
}

// Loads 4 consecutive bf16 of row `row` of X at column c0 as floats (0 past `rows`).
__device__ __forceinline__ void load4(const u16* __restrict__ X, int ld, int row, int rows, int c0,
                                      float (&o)[4]) {
    uint2 w = make_uint2(0u, 0u);
    if (row < rows) w = *reinterpret_cast<const uint2*>(X + (int64_t)row * ld + c0);
    o[0] = __uint_as_float(w.x << 16);
    o[1] = __uint_as_float(w.x & 0xffff0000u);
    o[2] = __uint_as_float(w.y << 16);
    o[3] = __uint_as_float(w.y & 0xffff0000u);
}

__device__ __forceinline__ void store4(u16* __restrict__ X, int ld, int row, int c0, const float* v) {
    uint2 w;
    w.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
    w.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
    *reinterpret_cast<uint2*>(X + (int64_t)row * ld + c0) = w;
}

// phi(X)^T for feature tile b of the chunk: C[f][t] = omega_f . x_t, then
// exp2(C a_scale + bias_t); tokens past `rows` are zero.
__device__ __forceinline__ f32x16 feature_tile(const BwdArgs& a, const BwdTables& tb,
                                               const bf16x8 (&xf)[4], int b, float bias, bool live,
                                               int lo, int h) {
    f32x16 c = zero16();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) c = mfma(tb.om[xs_index(32 * b + lo, 2 * ks + h)], xf[ks], c);
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = live ? __builtin_amdgcn_exp2f(fmaf(c[i], a.a_scale, bias)) : 0.f;
    return c;
}

// dx[t][d] = scale (du[d][t] - wsum_t u[t][d]), u = scale x, for the lane's
// token; du in accumulator layout (d = 32 dt + 8(i/4) + 4h + i%4).
__device__ __forceinline__ void store_dx(const BwdArgs& a, const u16* xrow0, u16* dxrow0,
                                         const f32x16 (&du)[2], float wsum, int lo, int h,
                                         int rows) {
    if (lo >= rows) return;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int c0 = 32 * dt + 8 * m + 4 * h;
            float xv[4], o[4];
            load4(xrow0, D, lo, rows, c0, xv);
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = a.scale * (du[dt][4 * m + j] - wsum * a.scale * xv[j]);
            store4(dxrow0, D, lo, c0, o);
        }
}

__global__ __launch_bounds__(NTB) void k_bwd_query_favor(BwdArgs a) {
    __shared__ BwdTables tb;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); // wave index, uniform
    const int lo = lane & 31, h = lane >> 5;
    const int64_t bh = blockIdx.x / a.G, g = blockIdx.x % a.G;
    build_tables(tb, a.st + bh * state_elems(R), a.omega, true);
    __syncthreads();
    const int64_t t0 = g * a.seg_len, t1 = min<int64_t>(t0 + a.seg_len, a.N);
    const int nck = t1 > t0 ? (int)((t1 - t0 + L - 1) / L) : 0;
    const bool attn = a.norm == NORM_ATTN;
    for (int ci = wv; ci < nck; ci += NTB / 64) {
        const int64_t c0 = t0 + (int64_t)L * ci;
        const int rows = (int)min<int64_t>(L, t1 - c0);
        const bool live = lo < rows;
        const u16* xr = a.x + (bh * a.N + c0) * D;
        const u16* yr = a.y + (bh * a.N + c0) * DV;
        bf16x8 xf[4];
        load_x(xr, rows, lo, h, xf);
        const float bias = fmaf(a.b_norm, sq_norm(xf), a.b_const);

        // pass 1: features and the readout against the total
        bf16x8 ph[8][2];
        f32x16 num[2] = {zero16(), zero16()};
        float den = 0.f;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const f32x16 c = feature_tile(a, tb, xf, b, bias, live, lo, h);
            ph[b][0] = pack8(c, 0);
            ph[b][1] = pack8(c, 8);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                den = fmaf((float)ph[b][i >> 3][i & 7], tb.m1[32 * b + 8 * (i >> 2) + 4 * h + (i & 3)], den);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
                    num[nt] = mfma(lds8(tb.mt + (32 * nt + lo) * LDF + 32 * b + 16 * s2 + 8 * h),
                                   ph[b][s2], num[nt]);
            // one tile at a time: keeps the scheduler from hoisting every
            // tile's operand loads (which spills)
            __builtin_amdgcn_sched_barrier(0);
        }
        den = half_sum(den);

        // dnum, dden of the lane's token (num in accumulator layout: n = 32 nt + 8(i/4) + 4h + i%4)
        const float inv = attn ? 1.f / fmaxf(den, a.eps) : 1.f;
        float dn[2][16], dot = 0.f;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                float o[4];
                load4(yr, DV, lo, rows, 32 * nt + 8 * m + 4 * h, o);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    dot = fmaf(o[j], num[nt][4 * m + j], dot);
                    dn[nt][4 * m + j] = o[j] * inv;
                }
            }
        dot = half_sum(dot);
        const float dden = (attn && den > a.eps) ? -dot * inv * inv : 0.f;
        if (live) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    store4(a.dy + (bh * a.N + c0) * DV, DV, lo, 32 * nt + 8 * m + 4 * h, &dn[nt][4 * m]);
            if (h == 0) a.dden[bh * a.N + c0 + lo] = dden;
        }
        bf16x8 dnf[2][2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                bf16x8 r;
#pragma unroll
                for (int e = 0; e < 8; ++e) r[e] = (__bf16)dn[nt][8 * s2 + e];
                dnf[nt][s2] = r;
            }

        // pass 2: dphi(Q) = S dnum + z dden per tile, w, du
        f32x16 du[2] = {zero16(), zero16()};
        float wsum = 0.f;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            f32x16 gq = zero16();
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
                    gq = mfma(lds8(tb.mn + (32 * b + lo) * LDN + 32 * nt + 16 * s2 + 8 * h),
                              dnf[nt][s2], gq);
            f32x16 w;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float gi = fmaf(tb.m1[32 * b + 8 * (i >> 2) + 4 * h + (i & 3)], dden, gq[i]);
                w[i] = gi * (float)ph[b][i >> 3][i & 7];
                wsum += w[i];
            }
            const bf16x8 w0 = pack8(w, 0), w1 = pack8(w, 8);
#pragma unroll
            for (int dt = 0; dt < 2; ++dt) {
                du[dt] = mfma(lds8(tb.wt + (32 * dt + lo) * LDF + 32 * b + 8 * h), w0, du[dt]);
                du[dt] = mfma(lds8(tb.wt + (32 * dt + lo) * LDF + 32 * b + 16 + 8 * h), w1, du[dt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        wsum = half_sum(wsum);
        store_dx(a, xr, a.dx + (bh * a.N + c0) * D, du, wsum, lo, h, rows);
    }
}

__global__ __launch_bounds__(NTB) void k_bwd_key_favor(BwdArgs a) {
    __shared__ BwdTables tb;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); // wave index, uniform
    const int lo = lane & 31, h = lane >> 5;
    const int64_t bh = blockIdx.x / a.G, g = blockIdx.x % a.G;
    build_tables(tb, a.st + bh * state_elems(R), a.omega, false);
    __syncthreads();
    const int64_t t0 = g * a.seg_len, t1 = min<int64_t>(t0 + a.seg_len, a.N);
    const int nck = t1 > t0 ? (int)((t1 - t0 + L - 1) / L) : 0;
    for (int ci = wv; ci < nck; ci += NTB / 64) {
        const int64_t c0 = t0 + (int64_t)L * ci;
        const int rows = (int)min<int64_t>(L, t1 - c0);
        const bool live = lo < rows;
        const u16* xr = a.x + (bh * a.N + c0) * D;
        const u16* yr = a.y + (bh * a.N + c0) * DV;
        bf16x8 xf[4], vf[4];
        load_x(xr, rows, lo, h, xf);
        load_x(yr, rows, lo, h, vf); // V^T as the B operand (n natural: 16 ks + 8h + e)
        const float bias = fmaf(a.b_norm, sq_norm(xf), a.b_const);
        f32x16 dv[2] = {zero16(), zero16()}, du[2] = {zero16(), zero16()};
        float wsum = 0.f;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const f32x16 c = feature_tile(a, tb, xf, b, bias, live, lo, h);
            const bf16x8 p0 = pack8(c, 0), p1 = pack8(c, 8);
            // dphi(K)^T = G V^T + g
            f32x16 gk = zero16();
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                gk = mfma(lds8(tb.mn + (32 * b + lo) * LDN + 16 * ks + 8 * h), vf[ks], gk);
            // dv^T += G^T phi(K)^T
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                dv[nt] = mfma(lds8(tb.mt + (32 * nt + lo) * LDF + 32 * b + 8 * h), p0, dv[nt]);
                dv[nt] = mfma(lds8(tb.mt + (32 * nt + lo) * LDF + 32 * b + 16 + 8 * h), p1, dv[nt]);
            }
            f32x16 w;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float gi = gk[i] + tb.m1[32 * b + 8 * (i >> 2) + 4 * h + (i & 3)];
                w[i] = live ? gi * c[i] : 0.f;
                wsum += w[i];
            }
            const bf16x8 w0 = pack8(w, 0), w1 = pack8(w, 8);
#pragma unroll
            for (int dt = 0; dt < 2; ++dt) {
                du[dt] = mfma(lds8(tb.wt + (32 * dt + lo) * LDF + 32 * b + 8 * h), w0, du[dt]);
                du[dt] = mfma(lds8(tb.wt + (32 * dt + lo) * LDF + 32 * b + 16 + 8 * h), w1, du[dt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        wsum = half_sum(wsum);
        if (live) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int m = 0; m < 4; ++m)
                {
                    const float o[4] = {dv[nt][4 * m], dv[nt][4 * m + 1], dv[nt][4 * m + 2],
                                        dv[nt][4 * m + 3]};
                    store4(a.dy + (bh * a.N + c0) * DV, DV, lo, 32 * nt + 8 * m + 4 * h, o);
                }
        }
        store_dx(a, xr, a.dx + (bh * a.N + c0) * D, du, wsum, lo, h, rows);
    }
}

// ---------------------------------------------------------------------------
// Bidirectional readout with every wave on its own chunks: k_favor_readout.
// The summaries S, z do not change along the sequence ("Reassociate a
// feature-map kernel...", par. 1 and 3: form them once, then read them for
// every query), so a workgroup of eight waves (one head, one block of its
// tokens) first puts them in LDS: S^T as a bf16 operand table (the rounding
// every bf16 product here uses) and z in float32, with omega in the swizzled
// row layout of the staged chunks.  Then each wave takes whole 32-token
// chunks of the block, and per 32-feature tile forms phi(Q)^T = exp2(omega
// Q^T a + b_t) (Kernel Zoo sec. 4.2 / 5.4 map; the token's bias b_t is per
// lane, as tokens are), adds the tile's part of the denominator phi(q).z and
// num^T += S^T phi(Q)^T on the matrix core; then out = num / max(den, eps).
// Nothing crosses waves inside the loop, so it has no barrier, and each
// chunk's loads are issued one chunk ahead.
// ---------------------------------------------------------------------------
constexpr int NTR = 512;
constexpr int NWR = NTR / 64;
constexpr int64_t READOUT_BLOCKS = 256;

struct ReadoutArgs {
    const u16* q;
    const u16* omega;
    const float* total;  // (S | z) per head: float32 [R][DV] then [R]
    int64_t st_bh;       // floats between heads' totals
    int64_t N;
    int64_t BH;
    int64_t blk_len;     // tokens per workgroup (a multiple of 32)
    float a_scale, b_norm, b_const, eps;
    int norm;
    u16* out;
};

struct ReadoutSmem {
    u16 mt[DV * LDF];   // S^T [n][f'], f in swap23 order within each 16-block
    bf16x8 om[R * 8];   // omega rows, 16-byte block j of row f at xs_index(f, j)
    u16 zb[R];          // z in bf16, by feature
};

template <int NORM>
__global__ __launch_bounds__(NTR, 2) void k_favor_readout(ReadoutArgs a) {
    __shared__ ReadoutSmem sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6); // wave index, uniform
    const int lo = lane & 31, h = lane >> 5;
    // the workgroups of one head are BH apart in the grid: with BH a
    // multiple of 8 they run on one XCD and share its L2 copy of the total
    const int64_t bh = blockIdx.x % a.BH, blk = blockIdx.x / a.BH;
    const float* tot = a.total + bh * a.st_bh;
    const int64_t t0 = blk * a.blk_len;
    const int64_t t1 = min<int64_t>(t0 + a.blk_len, a.N);
    const int nck = t1 > t0 ? (int)((t1 - t0 + L - 1) / L) : 0;
    auto rows_of = [&](int ci) { return (int)min<int64_t>(L, t1 - t0 - (int64_t)L * ci); };
    auto qrow = [&](int ci) { return a.q + (bh * a.N + t0 + (int64_t)L * ci) * D; };
    // the wave's first queries, then every load of the tables (one round
    // trip for all of them), then the LDS writes
    bf16x8 xn[4];
    if (wv < nck) load_x(qrow(wv), rows_of(wv), lo, h, xn);
    // S^T: thread (n, q) forms the 16-byte words of row n at positions
    // 8 q' .. 8 q' + 7 of the swap23-ordered features, q' = q + 8 u: the
    // features 16 (q' / 2) + swap23(8 (q' % 2) + e); each load instruction
    // reads 64 consecutive floats of one row of S
    constexpr int NU = R / 8 / (NTR / DV);
    const int n = tid & (DV - 1), q = tid / DV;
    float sv[NU][8];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int qq = q + (NTR / DV) * u;
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[u][e] = tot[(16 * (qq >> 1) + swap23(8 * (qq & 1) + e)) * DV + n];
    }
    constexpr int NO = R * 8 / NTR;
    bf16x8 ov[NO];
#pragma unroll
    for (int u = 0; u < NO; ++u) {
        const int b = tid + NTR * u;
        ov[u] = *reinterpret_cast<const bf16x8*>(a.omega + (int64_t)(b >> 3) * D + 8 * (b & 7));
    }
    const f32x4 zv = *reinterpret_cast<const f32x4*>(tot + R * DV + 4 * (tid & (R / 4 - 1)));
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        bf16x8 w;
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = (__bf16)sv[u][e];
        *reinterpret_cast<bf16x8*>(&sm.mt[n * LDF + 8 * (q + (NTR / DV) * u)]) = w;
    }
#pragma unroll
    for (int u = 0; u < NO; ++u) {
        const int b = tid + NTR * u;
        sm.om[xs_index(b >> 3, b & 7)] = ov[u];
    }
    if (NORM == NORM_ATTN && tid < R / 4) {
        const bf16x2 z01 = {(__bf16)zv[0], (__bf16)zv[1]}, z23 = {(__bf16)zv[2], (__bf16)zv[3]};
        *reinterpret_cast<uint2*>(&sm.zb[4 * tid]) =
            make_uint2(__builtin_bit_cast(uint32_t, z01), __builtin_bit_cast(uint32_t, z23));
    }
    __syncthreads();

    for (int ci = wv; ci < nck; ci += NWR) {
        const int rows = rows_of(ci);
        bf16x8 xf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) xf[ks] = xn[ks];
        // the next chunk's queries (this chunk again past the end, so every
        // iteration issues the same loads)
        const int cnx = ci + NWR < nck ? ci + NWR : ci;
        load_x(qrow(cnx), rows_of(cnx), lo, h, xn);
        const float bias = fmaf(a.b_norm, sq_norm(xf), a.b_const);
        f32x16 num[2] = {zero16(), zero16()};
        float den = 0.f, den2 = 0.f;
        // LDS operands, read one feature tile ahead of their use: omega rows
        // 32 b .. +31 (A operand of the projection), S^T for the tile (A
        // operand of num^T, columns 32 nt + lo) and z (bf16 pairs)
        auto read_om = [&](int b, bf16x8 (&o)[4]) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) o[ks] = sm.om[xs_index(32 * b + lo, 2 * ks + h)];
        };
        auto read_mt = [&](int b, bf16x8 (&o)[4]) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) o[2 * nt + s2] = lds8(sm.mt + (32 * nt + lo) * LDF + 32 * b + 16 * s2 + 8 * h);
        };
        auto read_z = [&](int b, uint2 (&o)[4]) {
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = *reinterpret_cast<const uint2*>(&sm.zb[32 * b + 8 * j + 4 * h]);
        };
        auto project = [&](const bf16x8 (&o)[4]) {
            f32x16 c = zero16();
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) c = mfma(o[ks], xf[ks], c);
            return c;
        };
        // software pipeline over the 8 feature tiles: region b exponentiates
        // tile b, projects tile b + 1 on the matrix core and adds tile b to
        // num; the LDS reads for the next region are issued at the end of
        // this one (a scheduling barrier ends each region, so they are not
        // moved next to their uses)
        bf16x8 om_n[4], mt_n[4];
        uint2 zb_n[4];
        read_om(0, om_n);
        f32x16 cn = project(om_n);
        read_om(1, om_n);
        read_mt(0, mt_n);
        if (NORM == NORM_ATTN) read_z(0, zb_n);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < R / 32; ++b) {
            f32x16 c = cn;
            bf16x8 mt_c[4];
            uint2 zb_c[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                mt_c[j] = mt_n[j];
                zb_c[j] = zb_n[j];
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) c[i] = __builtin_amdgcn_exp2f(fmaf(c[i], a.a_scale, bias));
            if (b + 1 < R / 32) cn = project(om_n);
            const bf16x8 p0 = pack8(c, 0), p1 = pack8(c, 8);
            // phi . z over the tile's features, in the bf16 roundings the
            // numerator's products use (S^T and phi are bf16 there)
            if (NORM == NORM_ATTN) dot_z(p0, p1, zb_c, den, den2);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                num[nt] = mfma(mt_c[2 * nt], p0, num[nt]);
                num[nt] = mfma(mt_c[2 * nt + 1], p1, num[nt]);
            }
            if (b + 2 < R / 32) read_om(b + 2, om_n);
            if (b + 1 < R / 32) {
                read_mt(b + 1, mt_n);
                if (NORM == NORM_ATTN) read_z(b + 1, zb_n);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        float inv = 1.f;
        if (NORM == NORM_ATTN) inv = __builtin_amdgcn_rcpf(fmaxf(half_sum(den + den2), a.eps));
        // token lo, columns 32 nt + 8 m + 4 h + (0..3); rows past the block's
        // end are dropped by the buffer resource's range
        const __amdgpu_buffer_rsrc_t orsrc = out_rows(a.out, bh * a.N + t0 + (int64_t)L * ci, rows);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const bf16x2 p0 = {(__bf16)(num[nt][4 * m] * inv), (__bf16)(num[nt][4 * m + 1] * inv)};
                const bf16x2 p1 = {(__bf16)(num[nt][4 * m + 2] * inv), (__bf16)(num[nt][4 * m + 3] * inv)};
                const u32x2 v2 = {__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
                __builtin_amdgcn_raw_buffer_store_b64(v2, orsrc, lo * (DV * 2) + 2 * (32 * nt + 8 * m + 4 * h), 0, 0);
            }
    }
}

// Compute units of the current device (cached per device; 256 if unknown).
int64_t device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
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
    a.tab = sp.tab;
    a.tsub = sp.sub;
    a.order = sp.order;
    a.osub = sp.osub;
    a.BH = s.BH;
    a.zw = nullptr;
    a.cus = device_cus();
    return a;
}

} // namespace

bool favor_mfma_supported(const Cfg& c, int dtype) {
    return c.phi == PHI_FAVOR && dtype == 1 && c.r == R && c.sum_norm == 0;
}

hipError_t launch_favor_sums(const Cfg& c, const void* k, const void* v, const void* omega,
                             Shape s, SegPlan sp, float* ws, hipStream_t st, const float* zw) {
    FavorArgs a = make_args(c, nullptr, k, v, omega, s, sp, ws, sp.G * state_elems(R),
                            state_elems(R), nullptr);
    a.zw = zw;
    if (zw)
        hipLaunchKernelGGL(k_favor_sums8<true>, dim3((unsigned)(sp.G * s.BH)), dim3(NT8), 0, st, a);
    else
        hipLaunchKernelGGL(k_favor_sums8<false>, dim3((unsigned)(sp.G * s.BH)), dim3(NT8), 0, st,
                           a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Causal backward on the matrix cores (FAVOR+, bf16, r = 256).  One workgroup
// of eight waves per (head, segment) walks its chunks in order (query pass)
// or in reverse (key pass); wave w keeps the 32 features F_w = [32w, 32w + 32)
// of the evolving state in float32 accumulators (the query pass S^T, the key
// pass the backward state G).  Two waves share each SIMD.  Each chunk's q, k,
// V, dout (or dnum), the per-token feature biases and dden are staged once
// per workgroup in LDS, one chunk ahead.  Products over all features reach
// the other waves in one of three forms:
// - the readout enters the query gradient only through two scalars per token,
//   the denominator and dot_t = dout_t . num_t, and dot_t is
//   sum_f phi(q_t)_f (S dout_t)_f + sum_j A1[j][t] (v_j . dout_t): both are
//   linear in the waves' parts over F_w, so only those scalars cross waves;
// - w = dphi o phi leaves each wave as bfloat16 rows of a [token][feature]
//   table; waves 0..3 then contract the table with omega over all r features,
//   two 16 x 16 tiles of du^T each (16x16x32 products), so no partial du
//   crosses;
// - the key pass sums the eight waves' parts of dv^T through LDS.
// The query pass writes dnum_t = dout_t / D_t (in bfloat16, the operand the
// products take) and dden_t; the segments' backward increments
// sum_t phi(q_t) (dnum_t, dden_t) come from the increment kernel.
// Two workgroup barriers per chunk.  32 x 32 tiles are accumulator tiles;
// T as an operand is pack8(T, 8 kk) (k-slots in swap23 order): the B operand
// of a product over T's rows, or the A operand of T^T.  transpose32 turns a
// tile into its transpose with the identity operand (exact: one bf16
// product by 1 each).
// ---------------------------------------------------------------------------
constexpr int NWC = 8;         // waves, 32 features each
constexpr int NTC = 64 * NWC;
constexpr int LDT = 40;        // row length of the per-chunk transposed tables (bank spread)
constexpr int LDW = R + 8;     // row length of the [d][f] omega^T and [t][f] w tables

__device__ __forceinline__ f32x16 transpose32(const f32x16& t, const bf16x8 (&eye)[2]) {
    return mfma(pack8(t, 8), eye[1], mfma(pack8(t, 0), eye[0], zero16()));
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct CausalArgs {
    const u16* q;
    const u16* k;
    const u16* v;
    const u16* dout;    // query pass
    const u16* omega;
    int64_t N, G, seg_len;
    float a_scale, b_norm, b_const, scale, eps;
    int norm;
    const float* state; // query: forward prefix per segment; key: backward suffix per segment
    int64_t st_bh, st_g;
    u16* dnum;          // dnum_t = dout_t / D_t in bfloat16 [BH, N, DV]: written by the query
                        // pass, read by the key pass
    float* dden;        // dden_t [BH, N]: likewise
    u16* dx;            // dq or dk
    u16* dv;            // key pass: dv
};

// A 32 x 32 accumulator tile in LDS, lane by lane: lane l's 16 elements at
// floats [16 l, 16 l + 16), as four 16-byte pieces in the order
// m ^ tile_swz(l), so that the lanes of each piece's access fall on distinct
// banks.
__device__ __forceinline__ int tile_swz(int l) { return ((l >> 1) ^ (l >> 3)) & 3; }
__device__ __forceinline__ void put_tile(float* base, int lane, const f32x16& t) {
    float* p = base + 16 * lane;
    const int sw = tile_swz(lane);
#pragma unroll
    for (int m = 0; m < 4; ++m)
        *reinterpret_cast<f32x4*>(p + 4 * (m ^ sw)) = f32x4{t[4 * m], t[4 * m + 1], t[4 * m + 2], t[4 * m + 3]};
}

// A 32 x 32 tile as the two bf16 operands it feeds (k-slots 0..7 and 8..15
// of each lane's 16 elements): what is kept of a tile that only ever enters
// matrix products.
struct Tile2 {
    bf16x8 k[2];
};
__device__ __forceinline__ Tile2 packt(const f32x16& t) { return Tile2{{pack8(t, 0), pack8(t, 8)}}; }
__device__ __forceinline__ f32x16 transpose_p(const Tile2& t, const bf16x8 (&eye)[2]) {
    return mfma(t.k[1], eye[1], mfma(t.k[0], eye[0], zero16()));
}

constexpr int LDD = DV + 4; // row length (bf16) of the per-chunk dout / dnum table (bank spread)

struct CausalSmem {
    u16 wt[D * LDW];               // omega^T [d][f]
    u16 wq[L * LDW];               // w of the chunk in bfloat16, [token][f]
    u16 vt[2][DV * LDT];           // V^T [n][j'] of the chunk (j in swap23 order)
    u16 vs[2][L * LDN];            // V [j][n'] of the chunk (n in swap23 order)
    bf16x8 xs[2][256];             // q and k of the chunk (swizzled, xs_index)
    u16 ds[L * LDD];               // dout (query pass) or dnum (key pass) of the chunk, [token][n]
    float xb[2][L];                // per token of the chunk: the feature map's bias for q and k
                                   // (-inf past the chunk's end)
    float wsum[NWC][L];            // per wave, per token: sum_f w over F_w
    float z[R];                    // z (query pass) or g (key pass)
};

struct CausalQuerySmem {
    CausalSmem c;
    float red[NWC][2][L];          // per wave, per token: partial denominator and dout . num
    bf16x8 om[R * 8];              // omega rows, 16-byte block j of row f at xs_index(f, j)
};

struct CausalKeySmem {
    CausalSmem c;
    u16 dnt[DV * LDT];             // dnum^T [n][i'] of the chunk (i in swap23 order)
    float dden[2][L] __attribute__((aligned(16))); // dden of the chunk's queries (by chunk parity)
    float part[NWC][2][64 * 16];   // per wave: partial dv^T tiles (put_tile)
};

// A chunk's global loads, held in registers until they are staged: thread th
// fetches 16-byte block th%256 of q (th < 256) or k; row vrow(th), columns
// vcol(th) .. +3 of V and of dout (query pass) or dnum (key pass) (the four
// lanes of a quad hold four consecutive rows of the same columns); and (key
// pass, th < 32) dden of token th; at rows clamped into the chunk.
struct ChunkLoads {
    bf16x8 xb;
    uint2 vx, dx;
    float dd;
};

__device__ __forceinline__ int vrow(int th) { return 4 * (th >> 6) + (th & 3); }
__device__ __forceinline__ int vcol(int th) { return 4 * ((th >> 2) & 15); }

template <bool KEY>
__device__ __forceinline__ void fetch_chunk(const CausalArgs& a, int64_t row0, int rows,
                                            ChunkLoads& ld) {
    const int th = threadIdx.x;
    ld.xb = load_block((th < 256 ? a.q : a.k) + row0 * D, rows, th & 255);
    const int64_t j = row0 + min(vrow(th), rows - 1);
    ld.vx = *reinterpret_cast<const uint2*>(a.v + j * DV + vcol(th));
    ld.dx = *reinterpret_cast<const uint2*>((KEY ? a.dnum : a.dout) + j * DV + vcol(th));
    if (KEY) ld.dd = a.dden[row0 + min(th & (L - 1), rows - 1)];
}

// A quad's 4 x 4 block (lane e: row j0 + e, columns n0 .. n0+3) into a
// transposed table [n][j'] (j in swap23 order): lane e writes column n0 + e
// of the four rows as one 8-byte piece (four consecutive j from a multiple
// of 4 keep their order under swap23).  Called by all four lanes of a quad.
__device__ __forceinline__ void put_transposed_quad(u16* tt, int j0, int n0, uint2 x) {
    const int e = threadIdx.x & 3;
    *reinterpret_cast<uint2*>(tt + (n0 + e) * LDT + (j0 & ~15) + swap23(j0 & 15)) = quad_transpose4(x);
}

// ... and their LDS copies (V, dout / dnum zero past `rows`), with the
// per-token biases of the feature map: the eight threads of a q or k row sum
// their squares; tokens past the end get -inf (exp2 gives 0).  The key pass
// also writes the transposed dnum table dnt.  Per-token values are written
// by every lane that holds them (the same value to the same address), so
// that no store needs a branch.
template <bool KEY>
__device__ __forceinline__ void stash_chunk(const CausalArgs& a, CausalSmem& sm, int buf,
                                            const ChunkLoads& ld, int rows, u16* dnt) {
    const int th = threadIdx.x;
    sm.xs[th >> 8][th & 255] = ld.xb;
    {
        float sq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const bf16x2 x = {ld.xb[e], ld.xb[e + 1]};
            sq = __builtin_amdgcn_fdot2_f32_bf16(x, x, sq, false);
        }
        sq = row8_sum(sq);
        const int t = (th & 255) >> 3;
        sm.xb[th >> 8][t] = t < rows ? fmaf(a.b_norm, sq, a.b_const) : -INFINITY;
    }
    const int j = vrow(th), n0 = vcol(th);
    const bool in = j < rows;
    const uint2 x = in ? ld.vx : make_uint2(0u, 0u);
    put_transposed_quad(sm.vt[buf], j & ~3, n0, x);
    // four consecutive n keep their order under swap23 (bits 0, 1 untouched)
    *reinterpret_cast<uint2*>(sm.vs[buf] + j * LDN + (n0 & ~15) + swap23(n0 & 15)) = x;
    const uint2 dx = in ? ld.dx : make_uint2(0u, 0u);
    *reinterpret_cast<uint2*>(sm.ds + j * LDD + n0) = dx;
    if (KEY) put_transposed_quad(dnt, j & ~3, n0, dx);
}

// Row lo of the chunk's dout / dnum table as the lane's pieces
// [32 nt + 8 m + 4h, +4) (accumulator layout of a [n x t] tile pair).
__device__ __forceinline__ void read_ds(const CausalSmem& sm, int lo, int h, uint2 (&r)[2][4]) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int m = 0; m < 4; ++m)
            r[nt][m] = *reinterpret_cast<const uint2*>(sm.ds + lo * LDD + 32 * nt + 8 * m + 4 * h);
}

// q or k (xs[x]) at the lane's du_tile position: row t, columns c .. c+3.
__device__ __forceinline__ uint2 read_xs4(const CausalSmem& sm, int x, int t, int c) {
    const u16* blk = reinterpret_cast<const u16*>(&sm.xs[x][xs_index(t, c >> 3)]);
    return *reinterpret_cast<const uint2*>(blk + (c & 7));
}

__device__ __forceinline__ void unpack4(uint2 w, float (&o)[4]) {
    o[0] = __uint_as_float(w.x << 16);
    o[1] = __uint_as_float(w.x & 0xffff0000u);
    o[2] = __uint_as_float(w.y << 16);
    o[3] = __uint_as_float(w.y & 0xffff0000u);
}

__device__ __forceinline__ uint32_t bf16pair(float a, float b) {
    return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

// phi(X)^T tile of this wave's features: C[f][t], f in F_w, token t = lo,
// from the token's staged bias (zero past the chunk's end).
// phi^T of the wave's 32 features, c[f][t] = exp2(omega_f . x_t a + bias_t),
// with omega's rows read from LDS (xs_index layout; OM_LDS) or from memory
// (the key pass has no LDS left for them: a copy from omega^T by
// transposing reads pushed it to 16 spilled registers, 248 -> 319 us)
template <bool OM_LDS>
__device__ __forceinline__ f32x16 features1(const CausalArgs& a, const bf16x8* om, const bf16x8 (&xf)[4],
                                            int w, float bias, int lo, int h) {
    f32x16 c = zero16();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        c = mfma(OM_LDS ? om[xs_index(32 * w + lo, 2 * ks + h)] : omega_frag(a.omega, 32 * w, 0, ks, lo, h),
                 xf[ks], c);
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = __builtin_amdgcn_exp2f(fmaf(c[i], a.a_scale, bias));
    return c;
}

// p[8 (i/4) + 4h + i%4] for the lane's 16 rows i of an accumulator tile, as
// four 16-byte reads (p 16-byte aligned).
__device__ __forceinline__ void read_rows(const float* p, int h, float (&r)[16]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(p + 8 * m + 4 * h);
#pragma unroll
        for (int j = 0; j < 4; ++j) r[4 * m + j] = x[j];
    }
}

// z (or g) at the lane's 16 rows f = fw + 8 (i/4) + 4h + i%4 of a [f x t] tile.
__device__ __forceinline__ void read_z(const CausalSmem& sm, int fw, int h, float (&zr)[16]) {
    read_rows(sm.z + fw, h, zr);
}

// This wave's rows of w (tile [f x t], f in F_w) into the bfloat16 table.
__device__ __forceinline__ void put_w(u16* wq, int w, int lo, int h, const f32x16& x) {
    u16* p = wq + lo * LDW + 32 * w + 4 * h;
#pragma unroll
    for (int m = 0; m < 4; ++m)
        *reinterpret_cast<uint2*>(p + 8 * m) =
            make_uint2(bf16pair(x[4 * m], x[4 * m + 1]), bf16pair(x[4 * m + 2], x[4 * m + 3]));
}

// du^T = omega^T w^T over all r features, by waves 0..3: wave w < 4 forms the
// two 16 x 16 tiles of rows d = 16 w + 4 (lane/16) + i and columns
// t = 16 k + lane%16 (k = 0, 1) with 16x16x32 products, one omega^T operand
// serving both.  (Waves 4..7, on the same SIMDs, have none: each SIMD still
// runs sixteen of these products per chunk, from three quarters of the LDS
// reads that one tile per wave would need.)
__device__ __forceinline__ void du_tiles(const CausalSmem& sm, int w, int lane, f32x4 (&acc)[2]) {
    const int c = lane & 15, g = lane >> 4;
    const u16* pa = sm.wt + (16 * w + c) * LDW + 8 * g;
    const u16* pb = sm.wq + c * LDW + 8 * g;
    acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc[1] = acc[0];
#pragma unroll
    for (int s = 0; s < R / 32; ++s) {
        const bf16x8 af = lds8(pa + 32 * s);
        acc[0] = mfma16(af, lds8(pb + 32 * s), acc[0]);
        acc[1] = mfma16(af, lds8(pb + 16 * LDW + 32 * s), acc[1]);
    }
}

// The lane's output positions in the chunk (wave w < 4, tile k).
__device__ __forceinline__ int du_token(int k, int lane) { return 16 * k + (lane & 15); }
__device__ __forceinline__ int du_col(int w, int lane) { return 16 * (w & 3) + 4 * (lane >> 4); }

// Raw buffer resource over the first `rows` rows of width `width` (bf16)
// at p: stores at byte offsets past the end are dropped by the hardware, so
// the chunk's stores need no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(void* p, int rows, int width) {
    return __builtin_amdgcn_make_buffer_rsrc(p, 0, rows * width * 2, 0x00020000);
}
__device__ __forceinline__ void store_b64(__amdgpu_buffer_rsrc_t rs, int byte_off, uint2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{v.x, v.y}, rs, byte_off, 0, 0);
}
__device__ __forceinline__ uint2 bf16x4_bits(const float (&o)[4]) {
    return make_uint2(bf16pair(o[0], o[1]), bf16pair(o[2], o[3]));
}

// dx[t][d .. d+3] = scale (du - wsum_t u), u = scale x, at token t and
// columns d .. d+3 (dropped past the chunk's rows).
__device__ __forceinline__ void store_dx(const CausalArgs& a, const CausalSmem& sm, u16* dxc,
                                         int t, int d, int rows, const f32x4& du, uint2 xe) {
    float ws = 0.f;
#pragma unroll
    for (int u = 0; u < NWC; ++u) ws += sm.wsum[u][t];
    float xv[4], o[4];
    unpack4(xe, xv);
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = a.scale * (du[j] - ws * a.scale * xv[j]);
    store_b64(chunk_rsrc(dxc, rows, D), 2 * (t * D + d), bf16x4_bits(o));
}

// dq or dk of the chunk from waves 0..3's du tiles (xe: q or k at the lane's
// two positions).
__device__ __forceinline__ void store_du(const CausalArgs& a, const CausalSmem& sm, u16* dxc,
                                         int w, int lane, int rows, const uint2 (&xe)[2]) {
    if (w >= 4) return; // uniform over the wave
    f32x4 acc[2];
    du_tiles(sm, w, lane, acc);
#pragma unroll
    for (int k = 0; k < 2; ++k) store_dx(a, sm, dxc, du_token(k, lane), du_col(w, lane), rows, acc[k], xe[k]);
}

// omega^T in LDS, natural f order.
// omega^T [d][f] (row length LDW) and omega's rows in the swizzled layout of
// the staged chunks: every global load is issued first (one round trip),
// single bf16 values are taken from 32-bit words by shifts.
__device__ __forceinline__ void stage_omega_t(u16* wt, bf16x8* rows, const u16* __restrict__ omega) {
    constexpr int NO = R * 8 / NTC;
    u32x4 ov[NO];
#pragma unroll
    for (int u = 0; u < NO; ++u) {
        const int b = threadIdx.x + NTC * u;
        ov[u] = *reinterpret_cast<const u32x4*>(omega + (int64_t)(b >> 3) * D + 8 * (b & 7));
    }
#pragma unroll
    for (int u = 0; u < NO; ++u) {
        const int b = threadIdx.x + NTC * u, f = b >> 3, d0 = 8 * (b & 7);
        *reinterpret_cast<u32x4*>(&rows[xs_index(f, b & 7)]) = ov[u];
#pragma unroll
        for (int e = 0; e < 8; ++e) wt[(d0 + e) * LDW + f] = (u16)(ov[u][e >> 1] >> (16 * (e & 1)));
    }
}

__global__ __launch_bounds__(NTC) void k_bwd_causal_query_favor(CausalArgs a) {
    __shared__ CausalQuerySmem smq;
    CausalSmem& sm = smq.c;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); // wave index, uniform
    const int lo = lane & 31, h = lane >> 5;
    const int64_t bh = blockIdx.x / a.G, g = blockIdx.x % a.G;
    const int64_t t0 = g * a.seg_len, t1 = min<int64_t>(t0 + a.seg_len, a.N);
    const int nck = t1 > t0 ? (int)((t1 - t0 + L - 1) / L) : 0;
    if (nck == 0) return; // uniform over the workgroup
    const bool attn = a.norm == NORM_ATTN;
    const bf16x8 eye[2] = {eye_frag(0, lo, h), eye_frag(1, lo, h)};
    // element i of a [row x token] tile pairs token lo with row 8(i/4) + 4h + i%4
    const int keep_thr = lo - 4 * h; // row <= token  <=>  8(i/4) + i%4 <= keep_thr
    const int fw = 32 * w;           // first feature of this wave
    const int pn = 32 * (w >> 2) + 8 * (w & 3) + 4 * h; // the dnum piece this wave stores

    stage_omega_t(sm.wt, smq.om, a.omega);
    // the forward state carried into the segment, transposed: S^T[n][F_w] in
    // accumulators (tile nt: rows n = 32 nt + 8(i/4) + 4h + i%4, column
    // f = fw + lo), z in LDS
    const float* st = a.state + bh * a.st_bh + g * a.st_g;
    f32x16 S[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            S[nt][i] = st[(int64_t)(fw + lo) * DV + 32 * nt + 8 * (i >> 2) + 4 * h + (i & 3)];
    for (int f = threadIdx.x; f < R; f += NTC) sm.z[f] = st[(int64_t)R * DV + f];

    auto chunk_at = [&](int ci, int64_t& c0, int& rows) {
        c0 = t0 + (int64_t)L * ci;
        rows = (int)min<int64_t>(L, t1 - c0);
    };
    // Global loads run two chunks ahead: chunk c + 2's are issued at the top
    // of chunk c into one register set, chunk c + 1's (issued a chunk
    // earlier, into the other set) are staged between chunk c's barriers.
    ChunkLoads LA, LB;
    {
        ChunkLoads first;
        fetch_chunk<false>(a, bh * a.N + t0, (int)min<int64_t>(L, t1 - t0), first);
        stash_chunk<false>(a, sm, 0, first, (int)min<int64_t>(L, t1 - t0), nullptr);
        int64_t c1;
        int rows1;
        chunk_at(min(1, nck - 1), c1, rows1);
        fetch_chunk<false>(a, bh * a.N + c1, rows1, LA);
    }
    __syncthreads(); // omega^T table, z and chunk 0's tables

    auto body = [&](int ci, const ChunkLoads& sl, ChunkLoads& il) {
        int64_t c0;
        int rows;
        chunk_at(ci, c0, rows);
        const bool live = lo < rows;
        const int buf = ci & 1;
        bf16x8 qf[4], kf[4];
        lds_x(sm.xs[0], lo, h, qf);
        lds_x(sm.xs[1], lo, h, kf);
        const uint2 xe[2] = {read_xs4(sm, 0, du_token(0, lane), du_col(w, lane)),
                             read_xs4(sm, 0, du_token(1, lane), du_col(w, lane))};
        // dout of token lo as the B operand of products over n (its raw
        // bf16 pieces), and this wave's piece of it for the dnum store
        Tile2 dt[2];
        {
            uint2 dr[2][4];
            read_ds(sm, lo, h, dr);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                dt[nt].k[0] = __builtin_bit_cast(bf16x8, u32x4{dr[nt][0].x, dr[nt][0].y, dr[nt][1].x, dr[nt][1].y});
                dt[nt].k[1] = __builtin_bit_cast(bf16x8, u32x4{dr[nt][2].x, dr[nt][2].y, dr[nt][3].x, dr[nt][3].y});
            }
        }
        const uint2 dpiece = *reinterpret_cast<const uint2*>(sm.ds + lo * LDD + pn);
        // chunk c + 2's loads (the last chunk's again past the end)
        int64_t c0n;
        int rowsn;
        chunk_at(min(ci + 2, nck - 1), c0n, rowsn);
        fetch_chunk<false>(a, bh * a.N + c0n, rowsn, il);
        chunk_at(min(ci + 1, nck - 1), c0n, rowsn);

        const f32x16 PQ = features1<true>(a, smq.om, qf, w, sm.xb[0][lo], lo, h);
        const Tile2 pk = packt(features1<true>(a, smq.om, kf, w, sm.xb[1][lo], lo, h));

        // Over F_w: the masked intra-chunk block A1^T [j x t] = phi(K) phi(Q)^T
        // (keys j <= query t), SD [f x t] = S dout^T and VD [j x t] = V dout^T.
        // The readout num_t enters the gradient only through the denominator
        // and dot_t = dout_t . num_t = sum_f phi(Q)[f][t] SD[f][t] +
        // sum_j A1^T[j][t] VD[j][t]: each wave folds its features' part of
        // both into the token's two scalars, and only those cross waves.
        f32x16 a1 = zero16(), SD = zero16(), VD = zero16();
        {
            const Tile2 pq = packt(PQ);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) a1 = mfma(pk.k[kk], pq.k[kk], a1);
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) SD = mfma(pack8(S[nt], 8 * kk), dt[nt].k[kk], SD);
        const u16* vs = sm.vs[buf];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                VD = mfma(lds8(vs + lo * LDN + 32 * nt + 16 * kk + 8 * h), dt[nt].k[kk], VD);
        float den = 0.f, dot = 0.f;
        {
            float zr[16];
            read_z(sm, fw, h, zr);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                den = fmaf(PQ[i], zr[i], den);
                dot = fmaf(PQ[i], SD[i], dot);
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            a1[i] = (8 * (i >> 2) + (i & 3) <= keep_thr) ? a1[i] : 0.f;
            den += a1[i];
            dot = fmaf(a1[i], VD[i], dot);
        }
        den = half_sum(den);
        dot = half_sum(dot);
        smq.red[w][0][lo] = den; // both halves: the same value
        smq.red[w][1][lo] = dot;
        sync_lds(); // B1: the waves' scalars; every wave is done with this chunk's q, k, dout

        // the next chunk's tables (V into the other pair: its last reader,
        // the chunk before this one, finished before B1); B2 publishes them
        stash_chunk<false>(a, sm, buf ^ 1, sl, rowsn, nullptr);

        den = 0.f;
        dot = 0.f;
#pragma unroll
        for (int u = 0; u < NWC; ++u) {
            den += smq.red[u][0][lo];
            dot += smq.red[u][1][lo];
        }
        // dnum_t = dout_t / D_t, dden_t (zero past the chunk's end); the key
        // pass and the increments take dnum in bfloat16
        // (both are formed in every lane and then selected: work under a
        // lane condition would become a branch)
        float rden = 1.f / fmaxf(den, a.eps);
        asm volatile("" : "+v"(rden), "+v"(dot));
        const float inv = live ? (attn ? rden : 1.f) : 0.f;
        const float dd_all = -dot * inv * inv;
        const float dden = (attn && den > a.eps) ? dd_all : 0.f;
        {
            float o[4];
            unpack4(dpiece, o);
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] *= inv;
            store_b64(chunk_rsrc(a.dnum + (bh * a.N + c0) * DV, rows, DV), 2 * (lo * DV + pn),
                      bf16x4_bits(o));
            // dden from wave 0's first half (every other lane's offset is past the end)
            const __amdgpu_buffer_rsrc_t rs =
                __builtin_amdgcn_make_buffer_rsrc(a.dden + bh * a.N + c0, 0, rows * 4, 0x00020000);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dden), rs,
                                                  (w == 0 && h == 0) ? 4 * lo : 4 * L, 0, 0);
        }

        // A2^T [j x t] = V dnum^T + dden_t = VD / D_t + dden_t, masked
        f32x16 a2;
#pragma unroll
        for (int i = 0; i < 16; ++i) a2[i] = (8 * (i >> 2) + (i & 3) <= keep_thr) ? fmaf(VD[i], inv, dden) : 0.f;

        // dphi(Q)^T [f x t] = SD / D_t + z dden + phi(K)^T A2^T, w = dphi o phi
        // (phi(K)^T is exact in bf16: a transposition of bf16 values)
        float zs = 0.f;
        Tile2 pkt;
        {
            const f32x16 t = transpose_p(pk, eye);
#pragma unroll
            for (int i = 0; i < 16; ++i) zs += t[i];
            pkt = packt(t);
        }
        {
            float zr[16];
            read_z(sm, fw, h, zr);
#pragma unroll
            for (int i = 0; i < 16; ++i) SD[i] = fmaf(zr[i], dden, SD[i] * inv);
        }
        {
            const Tile2 a2p = packt(a2);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) SD = mfma(pkt.k[kk], a2p.k[kk], SD);
        }
        float wsum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            SD[i] *= PQ[i];
            wsum += SD[i];
        }
        put_w(sm.wq, w, lo, h, SD);
        wsum = half_sum(wsum);
        sm.wsum[w][lo] = wsum; // both halves: the same value
        sync_lds(); // B2: the w table, the sums of w and the next chunk's tables
        store_du(a, sm, a.dx + (bh * a.N + c0) * D, w, lane, rows, xe);

        // state update: S^T[:, F_w] += V^T phi(K), z[F_w] += phi(K)^T 1
        const u16* vt = sm.vt[buf];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                S[nt] = mfma(lds8(vt + (32 * nt + lo) * LDT + 16 * kk + 8 * h), pkt.k[kk], S[nt]);
        zs = half_sum(zs);
        sm.z[fw + lo] += zs; // both halves: the same value
    };
    for (int ci = 0; ci < nck; ci += 2) {
        body(ci, LA, LB);
        if (ci + 1 < nck) body(ci + 1, LB, LA);
    }
}

__global__ __launch_bounds__(NTC) void k_bwd_causal_key_favor(CausalArgs a) {
    __shared__ CausalKeySmem smk;
    CausalSmem& sm = smk.c;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); // wave index, uniform
    const int lo = lane & 31, h = lane >> 5;
    const int64_t bh = blockIdx.x / a.G, g = blockIdx.x % a.G;
    const int64_t t0 = g * a.seg_len, t1 = min<int64_t>(t0 + a.seg_len, a.N);
    const int nck = t1 > t0 ? (int)((t1 - t0 + L - 1) / L) : 0;
    if (nck == 0) return; // uniform over the workgroup
    const bf16x8 eye[2] = {eye_frag(0, lo, h), eye_frag(1, lo, h)};
    // element i of a [row x key] tile pairs key lo with row (query) 8(i/4) + 4h + i%4
    const int keep_thr = lo - 4 * h; // query >= key  <=>  8(i/4) + i%4 >= keep_thr
    const int fw = 32 * w;

    // (the key pass keeps the element loop: with the batched loads its main
    // loop ran ~3 % slower at its 256-register limit)
    for (int e = threadIdx.x; e < R * D; e += NTC) sm.wt[(e % D) * LDW + e / D] = a.omega[e];
    // the backward state after the segment (suffix): G[F_w] in accumulators, g in LDS
    const float* st = a.state + bh * a.st_bh + g * a.st_g;
    f32x16 Gs[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            Gs[nt][i] = st[(int64_t)(fw + 8 * (i >> 2) + 4 * h + (i & 3)) * DV + 32 * nt + lo];
    for (int f = threadIdx.x; f < R; f += NTC) sm.z[f] = st[(int64_t)R * DV + f];

    auto chunk_at = [&](int cr, int64_t& c0, int& rows) {
        const int ci = nck - 1 - cr; // chunks last to first
        c0 = t0 + (int64_t)L * ci;
        rows = (int)min<int64_t>(L, t1 - c0);
    };
    // Global loads run two chunks ahead (as in the query pass).
    ChunkLoads LA, LB;
    {
        int64_t c0;
        int rows;
        chunk_at(0, c0, rows);
        ChunkLoads first;
        fetch_chunk<true>(a, bh * a.N + c0, rows, first);
        stash_chunk<true>(a, sm, 0, first, rows, smk.dnt);
        // every thread holds dden of token th % 32
        smk.dden[0][threadIdx.x & (L - 1)] = (int)(threadIdx.x & (L - 1)) < rows ? first.dd : 0.f;
        chunk_at(min(1, nck - 1), c0, rows);
        fetch_chunk<true>(a, bh * a.N + c0, rows, LA);
    }
    __syncthreads(); // omega^T table, g and the first chunk's tables

    auto body = [&](int cr, const ChunkLoads& sl, ChunkLoads& il) {
        int64_t c0;
        int rows;
        chunk_at(cr, c0, rows);
        const int buf = cr & 1;
        bf16x8 qf[4], kf[4];
        lds_x(sm.xs[0], lo, h, qf);
        lds_x(sm.xs[1], lo, h, kf);
        const uint2 xe[2] = {read_xs4(sm, 1, du_token(0, lane), du_col(w, lane)),
                             read_xs4(sm, 1, du_token(1, lane), du_col(w, lane))};
        // dnum^T [n x i] of the lane's query i = lo: its bfloat16 pieces are the
        // operands; and its transpose [i x n] as operands from the transposed table
        Tile2 dn[2], dnr[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) dnr[nt].k[kk] = lds8(smk.dnt + (32 * nt + lo) * LDT + 16 * kk + 8 * h);
        {
            uint2 dr[2][4];
            read_ds(sm, lo, h, dr);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                dn[nt].k[0] = __builtin_bit_cast(bf16x8, u32x4{dr[nt][0].x, dr[nt][0].y, dr[nt][1].x, dr[nt][1].y});
                dn[nt].k[1] = __builtin_bit_cast(bf16x8, u32x4{dr[nt][2].x, dr[nt][2].y, dr[nt][3].x, dr[nt][3].y});
            }
        }
        int64_t c0n;
        int rowsn;
        chunk_at(min(cr + 2, nck - 1), c0n, rowsn);
        fetch_chunk<true>(a, bh * a.N + c0n, rowsn, il);
        chunk_at(min(cr + 1, nck - 1), c0n, rowsn);

        const Tile2 pq = packt(features1<false>(a, nullptr, qf, w, sm.xb[0][lo], lo, h));
        const f32x16 PK = features1<false>(a, nullptr, kf, w, sm.xb[1][lo], lo, h);
        const Tile2 pk = packt(PK);

        // partials over F_w: dv^T [n x j] = G^T phi(K)^T, B1 [i x j] = phi(Q) phi(K)^T
        f32x16 dvp[2] = {zero16(), zero16()}, b1 = zero16();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) dvp[nt] = mfma(pack8(Gs[nt], 8 * kk), pk.k[kk], dvp[nt]);
            b1 = mfma(pq.k[kk], pk.k[kk], b1);
        }
        // dv^T = G^T phi(K)^T + dnum^T (B1 masked: query i >= key j) is linear
        // in the parts over F_w, so each wave adds its own masked block's
        // term before its part crosses waves
#pragma unroll
        for (int i = 0; i < 16; ++i) b1[i] = (8 * (i >> 2) + (i & 3) >= keep_thr) ? b1[i] : 0.f;
        {
            const Tile2 b1p = packt(b1);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) dvp[nt] = mfma(dnr[nt].k[kk], b1p.k[kk], dvp[nt]);
        }
        put_tile(smk.part[w][0], lane, dvp[0]);
        put_tile(smk.part[w][1], lane, dvp[1]);
        sync_lds(); // B1: partials; every wave is done with this chunk's q, k, dnum

        // the next chunk's tables (V and dden into the other pair: their last
        // reader, the chunk before this one, finished before B1); B2
        // publishes them
        stash_chunk<true>(a, sm, buf ^ 1, sl, rowsn, smk.dnt);
        smk.dden[buf ^ 1][threadIdx.x & (L - 1)] = (int)(threadIdx.x & (L - 1)) < rowsn ? sl.dd : 0.f;

        // dv: wave w sums elements 4 (w%4) .. +3 of tile w/4 over the eight
        // parts: rows n = 32 (w/4) + 8 (w%4) + 4h + e, column j = lo
        {
            const int nt = w >> 2, qq = w & 3;
            const int off = 16 * lane + 4 * (qq ^ tile_swz(lane));
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < NWC; ++u) s += *reinterpret_cast<const f32x4*>(smk.part[u][nt] + off);
            const float o[4] = {s[0], s[1], s[2], s[3]};
            store_b64(chunk_rsrc(a.dv + (bh * a.N + c0) * DV, rows, DV),
                      2 * (lo * DV + 32 * nt + 8 * qq + 4 * h), bf16x4_bits(o));
        }
        // A3 [i x j] = dnum_i . v_j + dden_i, masked (i >= j)
        const u16* vs = sm.vs[buf];
        float ddn[16]; // dden of the lane's 16 query rows
        read_rows(smk.dden[buf], h, ddn);
        f32x16 a3 = zero16();
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                a3 = mfma(dn[nt].k[kk], lds8(vs + lo * LDN + 32 * nt + 16 * kk + 8 * h), a3);
#pragma unroll
        for (int i = 0; i < 16; ++i) a3[i] = (8 * (i >> 2) + (i & 3) >= keep_thr) ? a3[i] + ddn[i] : 0.f;
        // dphi(K)^T [f x j] = G V^T + g + phi(Q)^T A3, w = dphi o phi
        // (phi(Q)^T is exact in bf16: a transposition of bf16 values)
        float gsum = 0.f;
        Tile2 pqt;
        {
            const f32x16 t = transpose_p(pq, eye); // [i x f]
#pragma unroll
            for (int i = 0; i < 16; ++i) gsum = fmaf(t[i], ddn[i], gsum);
            pqt = packt(t);
        }
        f32x16 gk = zero16();
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const Tile2 gt = packt(transpose32(Gs[nt], eye)); // [n x f]
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                gk = mfma(gt.k[kk], lds8(vs + lo * LDN + 32 * nt + 16 * kk + 8 * h), gk);
        }
        {
            const Tile2 a3p = packt(a3);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) gk = mfma(pqt.k[kk], a3p.k[kk], gk);
        }
        float wsum = 0.f;
        {
            float zr[16];
            read_z(sm, fw, h, zr);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                gk[i] = (gk[i] + zr[i]) * PK[i];
                wsum += gk[i];
            }
        }
        put_w(sm.wq, w, lo, h, gk);
        wsum = half_sum(wsum);
        sm.wsum[w][lo] = wsum; // both halves: the same value
        sync_lds(); // B2: the w table, the sums of w and the next chunk's tables
        store_du(a, sm, a.dx + (bh * a.N + c0) * D, w, lane, rows, xe);

        // suffix update for the earlier chunks: G[F_w] += phi(Q)^T dnum, g += phi(Q)^T dden
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) Gs[nt] = mfma(pqt.k[kk], dnr[nt].k[kk], Gs[nt]);
        gsum = half_sum(gsum);
        sm.z[fw + lo] += gsum; // both halves: the same value
    };
    for (int cr = 0; cr < nck; cr += 2) {
        body(cr, LA, LB);
        if (cr + 1 < nck) body(cr + 1, LB, LA);
    }
}

static BwdArgs bwd_args(const Cfg& c, const void* x, const void* y, const void* omega, Shape s,
                        SegPlan sp, const float* st, void* dx, void* dy, float* dden) {
    BwdArgs a;
    a.x = (const u16*)x;
    a.y = (const u16*)y;
    a.omega = (const u16*)omega;
    a.st = st;
    a.N = s.N;
    a.G = sp.G;
    a.seg_len = sp.seg_len;
    a.a_scale = c.scale * LOG2E;
    a.b_norm = -0.5f * c.scale * c.scale * LOG2E;
    a.b_const = c.favor_log2_bias;
    a.scale = c.scale;
    a.eps = c.eps;
    a.norm = c.norm;
    a.dx = (u16*)dx;
    a.dy = (u16*)dy;
    a.dden = dden;
    return a;
}

hipError_t launch_favor_bwd_query(const Cfg& c, const void* q, const void* dout, const void* omega,
                                  Shape s, SegPlan sp, const float* total, void* dq, void* dnum,
                                  float* dden, hipStream_t st) {
    // every token's gradient reads only the totals, so the passes take their
    // own blocks of tokens: about one workgroup (eight waves) per CU
    const SegPlan wp = plan_segments(s.BH, s.N, 0, BWD_BIDIR_BLOCKS);
    (void)sp;
    const BwdArgs a = bwd_args(c, q, dout, omega, s, wp, total, dq, dnum, dden);
    hipLaunchKernelGGL(k_bwd_query_favor, dim3((unsigned)(wp.G * s.BH)), dim3(NTB), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_favor_bwd_key(const Cfg& c, const void* k, const void* v, const void* omega,
                                Shape s, SegPlan sp, const float* total, void* dk, void* dv,
                                hipStream_t st) {
    const SegPlan wp = plan_segments(s.BH, s.N, 0, BWD_BIDIR_BLOCKS);
    (void)sp;
    const BwdArgs a = bwd_args(c, k, v, omega, s, wp, total, dk, dv, nullptr);
    hipLaunchKernelGGL(k_bwd_key_favor, dim3((unsigned)(wp.G * s.BH)), dim3(NTB), 0, st, a);
    return hipGetLastError();
}

static CausalArgs causal_args(const Cfg& c, const void* q, const void* k, const void* v,
                              const void* dout, const void* omega, Shape s, SegPlan sp,
                              const float* state, int64_t sbh, int64_t sg, void* dnum, float* dden,
                              void* dx, void* dv) {
    CausalArgs a;
    a.q = (const u16*)q;
    a.k = (const u16*)k;
    a.v = (const u16*)v;
    a.dout = (const u16*)dout;
    a.omega = (const u16*)omega;
    a.N = s.N;
    a.G = sp.G;
    a.seg_len = sp.seg_len;
    a.a_scale = c.scale * LOG2E;
    a.b_norm = -0.5f * c.scale * c.scale * LOG2E;
    a.b_const = c.favor_log2_bias;
    a.scale = c.scale;
    a.eps = c.eps;
    a.norm = c.norm;
    a.state = state;
    a.st_bh = sbh;
    a.st_g = sg;
    a.dnum = (u16*)dnum;
    a.dden = dden;
    a.dx = (u16*)dx;
    a.dv = (u16*)dv;
    return a;
}

hipError_t launch_favor_causal_bwd_query(const Cfg& c, const void* q, const void* k, const void* v,
                                         const void* dout, const void* omega, Shape s, SegPlan sp,
                                         const float* prefix, int64_t sbh, int64_t sg, void* dnum,
                                         float* dden, void* dq, hipStream_t st) {
    const CausalArgs a =
        causal_args(c, q, k, v, dout, omega, s, sp, prefix, sbh, sg, dnum, dden, dq, nullptr);
    hipLaunchKernelGGL(k_bwd_causal_query_favor, dim3((unsigned)(sp.G * s.BH)), dim3(NTC), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_favor_causal_bwd_key(const Cfg& c, const void* q, const void* k, const void* v,
                                       const void* omega, Shape s, SegPlan sp, const float* suffix,
                                       int64_t sbh, int64_t sg, const void* dnum, const float* dden,
                                       void* dk, void* dv, hipStream_t st) {
    const CausalArgs a = causal_args(c, q, k, v, nullptr, omega, s, sp, suffix, sbh, sg,
                                     const_cast<void*>(dnum), const_cast<float*>(dden), dk, dv);
    hipLaunchKernelGGL(k_bwd_causal_key_favor, dim3((unsigned)(sp.G * s.BH)), dim3(NTC), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_favor_readout(const Cfg& c, const void* q, const void* omega, Shape s,
                                const float* total, int64_t st_bh, void* out, hipStream_t st) {
    ReadoutArgs a;
    a.q = (const u16*)q;
    a.omega = (const u16*)omega;
    a.total = total;
    a.st_bh = st_bh;
    a.N = s.N;
    a.BH = s.BH;
    a.a_scale = c.scale * LOG2E;
    a.b_norm = -0.5f * c.scale * c.scale * LOG2E;
    a.b_const = c.favor_log2_bias;
    a.eps = c.eps;
    a.norm = c.norm;
    a.out = (u16*)out;
    // blocks of whole chunks, about one workgroup per CU (two do not fit
    // beside each other's registers)
    const int64_t nblk0 = (READOUT_BLOCKS + s.BH - 1) / s.BH;
    const int64_t chunks = (s.N + L - 1) / L;
    a.blk_len = L * ((chunks + nblk0 - 1) / nblk0);
    const int64_t nblk = (s.N + a.blk_len - 1) / a.blk_len;
    const dim3 grid((unsigned)(nblk * s.BH));
    if (c.norm == NORM_ATTN)
        hipLaunchKernelGGL(k_favor_readout<NORM_ATTN>, grid, dim3(NTR), 0, st, a);
    else
        hipLaunchKernelGGL(k_favor_readout<NORM_NONE>, grid, dim3(NTR), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_favor_outputs(const Cfg& c, const void* q, const void* k, const void* v,
                                const void* omega, Shape s, SegPlan sp, const float* state,
                                int64_t sbh, int64_t sg, void* out, hipStream_t st) {
    const FavorArgs a = make_args(c, q, k, v, omega, s, sp, const_cast<float*>(state), sbh, sg, out);
    const dim3 grid((unsigned)(sp.G * s.BH));
    if (c.norm == NORM_ATTN)
        hipLaunchKernelGGL(k_favor_fused<NORM_ATTN>, grid, dim3(NTF), 0, st, a);
    else
        hipLaunchKernelGGL(k_favor_fused<NORM_NONE>, grid, dim3(NTF), 0, st, a);
    return hipGetLastError();
}

} // namespace linattn
