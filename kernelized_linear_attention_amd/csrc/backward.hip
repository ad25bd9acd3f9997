// backward.hip -- gradients of the bidirectional form and of the causal
// recurrence (from zero state) with respect to q, k and v: the chain rule
// through the readout, the summaries and the feature map (Kernel Zoo sec.
// 1.3 and 5.4 for the forward definitions; "Reassociate a feature-map
// kernel..." par. 6 asks for the gradients to be evaluated).  Vector kernels,
// float32 arithmetic, every feature map, float32 and bfloat16 inputs.
//
// With D_i = max(den_i, eps), query i read against the state (S_i, z_i) it
// sees, and dout_i = dL/dout_i:
//   dnum_i = dout_i / D_i,  dden_i = -(dout_i . out_i) / D_i where den_i > eps
//   (0 where the clamp holds D_i fixed); NORM_NONE: dnum_i = dout_i, dden_i = 0
//   dphi(q_i) = S_i dnum_i + z_i dden_i
//   dphi(k_j) = G_j v_j + g_j,   dv_j = G_j^T phi(k_j)
// where (G_j, g_j) sums (phi(q_i) dnum_i^T, phi(q_i) dden_i) over the queries
// i that see key j: all of them in the bidirectional form, i >= j in the
// causal one.  The causal G_j is a suffix sum and is evaluated like the
// forward prefix, mirrored: segments -> chunks walked last to first ->
// tokens, with an exclusive suffix over per-segment increments.  Through the
// map, dx = scale * J_phi(u)^T dphi at u = scale * x.
//
// With bfloat16 inputs and FAVOR+, the two contractions with omega run on
// the matrix cores (32x32x16 bf16, float32 accumulation): the projections
// omega . x of the feature map (exact bf16 products, as in the forward
// kernels) and du = sum_f w_f omega_f of the map's backward (w rounded to
// bf16, against omega^T prepared once per call).
//
// Launch order (abi.hip): forward increments, forward scan, omega^T (bf16
// FAVOR+ only), query pass (dq, backward increments, per-token (1/D, dden)
// for the causal form), backward scan (suffix for causal), key pass (dk, dv).
#include "launch.hpp"
#include "tiles.hpp"

namespace linattn {
namespace {

constexpr int NT = VNT;
constexpr int L = 16;       // tokens per chunk
constexpr int SL = DV + 4;  // LDS row stride of a state matrix [R][DV]

typedef __bf16 bw_bf16x8 __attribute__((ext_vector_type(8)));
typedef float bw_f32x16 __attribute__((ext_vector_type(16)));

template <typename T> constexpr bool is_bf16() { return false; }
template <> constexpr bool is_bf16<bf16_raw>() { return true; }

__device__ __forceinline__ bw_f32x16 mfma32(uint4 a, uint4 b, bw_f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bw_bf16x8, a),
                                                   __builtin_bit_cast(bw_bf16x8, b), c, 0, 0, 0);
}

// FAVOR+ features of the chunk's rows x (bfloat16, [rows][D] in global
// memory) with the projections on the matrix cores: C[f][t] = omega_f . x_t
// for 32-feature blocks, the waves taking blocks in turn.  Lane l holds token
// t = l % 32 (rows at or past `rows` are zero, t < 32 covers L = 16), and
// accumulator i feature 8(i/4) + 4(l/32) + i%4 of the block.  Then
// out[t][f] = exp(scale (omega_f . x_t) - |u_t|^2 / 2) / sqrt(r) (u = scale x,
// nrm[t] = |u_t|^2).  Ends without a barrier.
template <int FPT>
__device__ void favor_tile_mfma(const Cfg& c, const bf16_raw* __restrict__ x, int rows,
                                const bf16_raw* __restrict__ omega, const float* nrm, float* out,
                                int ol) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int tok = lane & 31, kq = 8 * (lane >> 5);
    uint4 bx[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        bx[ks] = make_uint4(0u, 0u, 0u, 0u);
        if (tok < rows) bx[ks] = *reinterpret_cast<const uint4*>(x + tok * D + 16 * ks + kq);
    }
    for (int fb = wv; fb < FPT; fb += NT / 64) {
        bw_f32x16 acc;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = 0.f;
        const bf16_raw* wa = omega + (int64_t)(fb * 32 + (lane & 31)) * D + kq;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            acc = mfma32(*reinterpret_cast<const uint4*>(wa + 16 * ks), bx[ks], acc);
        if (tok < L) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int f = fb * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                out[tok * ol + f] = tok < rows ? favor_feature(c, c.scale * acc[i], nrm[tok]) : 0.f;
            }
        }
    }
}

// The feature tile of the chunk: matrix-core projections for bfloat16
// FAVOR+, else phi_tile.  x: the chunk's raw rows; u, nrm as phi_tile.
// Ends with a barrier.
template <typename T, int FPT>
__device__ void bwd_phi_tile(const Cfg& c, const float* u, const float* nrm,
                             const T* __restrict__ omega, const T* __restrict__ x, int rows,
                             float* out, int ol, float* rs, float* live = nullptr) {
    if constexpr (is_bf16<T>()) {
        if (c.phi == PHI_FAVOR) {
            favor_tile_mfma<FPT>(c, x, rows, omega, nrm, out, ol);
            __syncthreads();
            if (c.sum_norm) sum_normalize<L>(c, out, ol, rs, live);
            return;
        }
    }
    phi_tile<T, L>(c, u, nrm, omega, rows, out, ol, rs, live);
}

// omega^T [D][r] (bfloat16) for the matrix-core du contraction.
__global__ __launch_bounds__(NT) void k_transpose_omega(const bf16_raw* __restrict__ omega, int r,
                                                        bf16_raw* __restrict__ omega_t) {
    const int64_t idx = (int64_t)blockIdx.x * NT + threadIdx.x;
    if (idx >= (int64_t)r * D) return;
    const int d = (int)(idx / r), f = (int)(idx % r);
    omega_t[idx] = omega[(int64_t)f * D + d];
}

// Loads state block src = (M [R][DV], m [R]) into M_s (row stride SL), m_s.
template <int R>
__device__ void load_state(const float* __restrict__ src, float* M_s, float* m_s) {
    for (int e = threadIdx.x; e < R * (DV / 4); e += NT) {
        const int f = e / (DV / 4), n4 = (e % (DV / 4)) * 4;
        *reinterpret_cast<float4*>(M_s + f * SL + n4) =
            *reinterpret_cast<const float4*>(src + (long)f * DV + n4);
    }
    for (int f = threadIdx.x; f < R; f += NT) m_s[f] = src[(long)R * DV + f];
}

// First of the 2*FPT contiguous features a thread owns in the state updates.
template <int FPT>
__device__ __forceinline__ int feat0() { return (threadIdx.x / 16) * 2 * FPT; }

// Outer-product sums over the rows of a chunk, for the items of this thread:
// features f = feat0() + it, value columns n4 = 4*(tid % 16) .. n4+3:
//   acc[it][j] += sum_t x[t][f] y[t][n4+j],   macc[it] += sum_t x[t][f] s[t]
// (s == NULL: s[t] = 1).  x has row stride ol, y row stride DV.
template <int FPT>
__device__ void outer_accum(const float* x, int ol, const float* y, const float* s, int rows,
                            float (&acc)[2 * FPT][4], float (&macc)[2 * FPT]) {
    const int f0 = feat0<FPT>(), n4 = (threadIdx.x % 16) * 4;
    for (int t = 0; t < rows; ++t) {
        const float4 yv = *reinterpret_cast<const float4*>(y + t * DV + n4);
        const float st = s ? s[t] : 1.f;
        float xf[2 * FPT];
#pragma unroll
        for (int it = 0; it < 2 * FPT; it += 2) {
            const float2 x2 = *reinterpret_cast<const float2*>(x + t * ol + f0 + it);
            xf[it] = x2.x;
            xf[it + 1] = x2.y;
        }
#pragma unroll
        for (int it = 0; it < 2 * FPT; ++it) {
            acc[it][0] = fmaf(xf[it], yv.x, acc[it][0]);
            acc[it][1] = fmaf(xf[it], yv.y, acc[it][1]);
            acc[it][2] = fmaf(xf[it], yv.z, acc[it][2]);
            acc[it][3] = fmaf(xf[it], yv.w, acc[it][3]);
            macc[it] = fmaf(xf[it], st, macc[it]);
        }
    }
}

// In-LDS state update M += x^T y, m += x^T s over the rows of a chunk.
// Caller synchronises before (readers of M done) and after.
template <int FPT>
__device__ void state_update(float* M_s, float* m_s, const float* x, int ol, const float* y,
                             const float* s, int rows) {
    const int f0 = feat0<FPT>(), n4 = (threadIdx.x % 16) * 4;
    float acc[2 * FPT][4], macc[2 * FPT];
#pragma unroll
    for (int it = 0; it < 2 * FPT; ++it) {
        const float4 a = *reinterpret_cast<const float4*>(M_s + (f0 + it) * SL + n4);
        acc[it][0] = a.x;
        acc[it][1] = a.y;
        acc[it][2] = a.z;
        acc[it][3] = a.w;
        macc[it] = 0.f;
    }
    outer_accum<FPT>(x, ol, y, s, rows, acc, macc);
#pragma unroll
    for (int it = 0; it < 2 * FPT; ++it) {
        *reinterpret_cast<float4*>(M_s + (f0 + it) * SL + n4) =
            make_float4(acc[it][0], acc[it][1], acc[it][2], acc[it][3]);
        if (n4 == 0) m_s[f0 + it] += macc[it];
    }
}

// dp[t][f] = sum_n M[f][n] y[t][n] + m[f] s[t] + sum_j cm[t][j] x[j][f] for
// the L rows of a chunk (s == NULL: s[t] = 1; cm == NULL: no third term; cm
// row stride L+1, already zero outside the mask).  Item (feature f, token
// group of 8 rows).
template <int FPT>
__device__ void dphi_rows(const float* M_s, const float* m_s, const float* y, const float* s,
                          const float* cm, const float* x, int ol, float* dp) {
    constexpr int R = 32 * FPT;
    for (int p = threadIdx.x; p < 2 * R; p += NT) {
        const int f = p % R, t0 = (p / R) * 8;
        float acc[8];
        const float mf = m_s[f];
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[t] = s ? mf * s[t0 + t] : mf;
        for (int n = 0; n < DV; n += 4) {
            const float4 w = *reinterpret_cast<const float4*>(M_s + f * SL + n);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float4 yv = *reinterpret_cast<const float4*>(y + (t0 + t) * DV + n);
                acc[t] = fmaf(w.x, yv.x, acc[t]);
                acc[t] = fmaf(w.y, yv.y, acc[t]);
                acc[t] = fmaf(w.z, yv.z, acc[t]);
                acc[t] = fmaf(w.w, yv.w, acc[t]);
            }
        }
        if (cm) {
            for (int j = 0; j < L; ++j) {
                const float xv = x[j * ol + f];
#pragma unroll
                for (int t = 0; t < 8; ++t) acc[t] = fmaf(cm[(t0 + t) * (L + 1) + j], xv, acc[t]);
            }
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) dp[(t0 + t) * ol + f] = acc[t];
    }
}

// cm[t][j] = (j <= t) ? a[t] . b[j] : 0 (LOWER) or (j >= t) ? ... (upper),
// plus add[t] (may be NULL) inside the mask; a, b row stride `ld`, length n.
template <bool LOWER>
__device__ void masked_products(const float* a, const float* b, int ld, int n, const float* add,
                                float* cm) {
    for (int p = threadIdx.x; p < L * L; p += NT) {
        const int t = p / L, j = p % L;
        float acc = 0.f;
        if (LOWER ? j <= t : j >= t) {
            const float* x = a + t * ld;
            const float* y = b + j * ld;
            for (int e = 0; e < n; e += 4) {
                const float4 a4 = *reinterpret_cast<const float4*>(x + e);
                const float4 b4 = *reinterpret_cast<const float4*>(y + e);
                acc = fmaf(a4.x, b4.x, acc);
                acc = fmaf(a4.y, b4.y, acc);
                acc = fmaf(a4.z, b4.z, acc);
                acc = fmaf(a4.w, b4.w, acc);
            }
            if (add) acc += add[j];
        }
        cm[t * (L + 1) + j] = acc;
    }
}

// out[t] = scale * J_phi(u_t)^T dp_t for the rows t < rows of a chunk.
// phi: the map's output tile (after sum normalisation), rs / live from
// phi_tile; dp (dphi, row stride ol) is overwritten.  Starts after a barrier
// (dp, phi, u complete); ends without one.
template <typename T, int FPT>
__device__ void phi_backward_tile(const Cfg& c, const float* u, const float* phi, int ol,
                                  const float* rs, const float* live, float* dp, float* cc,
                                  const T* __restrict__ omega,
                                  const bf16_raw* __restrict__ omega_t, int rows,
                                  T* __restrict__ out) {
    constexpr int R = 32 * FPT;
    const int tid = threadIdx.x;
    if (c.sum_norm) {
        // through phi = p / max(sum p, eps): dp = (dphi - [sum > eps] dphi . phi) / max(sum, eps)
        const int lane = tid & 63, w = tid >> 6;
        for (int t = w; t < L; t += NT / 64) {
            float s = 0.f;
            for (int f = lane; f < R; f += 64) s = fmaf(dp[t * ol + f], phi[t * ol + f], s);
            s = wave_sum(s);
            if (lane == 0) cc[t] = live[t] != 0.f ? s : 0.f;
        }
        __syncthreads();
    }
    if (c.sum_norm || c.phi == PHI_FAVOR) {
        // FAVOR+ keeps dp_f * p_f = (dphi_f - c) * phi_f (d p_f / d u = p_f (omega_f - u))
        for (int idx = tid; idx < L * R; idx += NT) {
            const int t = idx / R, f = idx - t * R;
            float g = dp[t * ol + f];
            if (c.sum_norm) g -= cc[t];
            if (c.phi == PHI_FAVOR) g *= phi[t * ol + f];
            else g *= rs[t];
            dp[t * ol + f] = g;
        }
        __syncthreads();
    }
    if constexpr (is_bf16<T>()) {
        if (c.phi == PHI_FAVOR && omega_t) {
            // cc[t] = sum_f w[t][f] (cc is free after the transform above)
            const int lane = tid & 63, w = tid >> 6;
            for (int t = w; t < L; t += NT / 64) {
                float sacc = 0.f;
                for (int f = lane; f < R; f += 64) sacc += dp[t * ol + f];
                sacc = wave_sum(sacc);
                if (lane == 0) cc[t] = sacc;
            }
            __syncthreads();
            // du as C[t][d] = sum_f w[t][f] omega[f][d]: waves 0 and 1 take
            // the two 32-column halves of d; A = w rows (bf16), B = omega^T rows
            if (w < 2) {
                const int tok = lane & 31, kq = 8 * (lane >> 5);
                const int dcol = 32 * w + (lane & 31);
                bw_f32x16 acc;
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[e] = 0.f;
                const bf16_raw* wb = omega_t + (int64_t)dcol * R + kq;
#pragma unroll 4
                for (int f0 = 0; f0 < R; f0 += 16) {
                    uint4 a = make_uint4(0u, 0u, 0u, 0u);
                    if (tok < L) {
                        const float4 x0 = *reinterpret_cast<const float4*>(dp + tok * ol + f0 + kq);
                        const float4 x1 = *reinterpret_cast<const float4*>(dp + tok * ol + f0 + kq + 4);
                        bw_bf16x8 h;
                        h[0] = (__bf16)x0.x; h[1] = (__bf16)x0.y; h[2] = (__bf16)x0.z; h[3] = (__bf16)x0.w;
                        h[4] = (__bf16)x1.x; h[5] = (__bf16)x1.y; h[6] = (__bf16)x1.z; h[7] = (__bf16)x1.w;
                        a = __builtin_bit_cast(uint4, h);
                    }
                    acc = mfma32(a, *reinterpret_cast<const uint4*>(wb + f0), acc);
                }
                // accumulator e: token 8(e/4) + 4(l/32) + e%4, column dcol
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int t = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                    if (t < rows)
                        Elem<T>::store(out, (long)t * D + dcol,
                                       c.scale * (acc[e] - cc[t] * u[t * D + dcol]));
                }
            }
            return;
        }
    }
    const int i = tid & 63, t0 = (tid >> 6) * (L / 4);
    float du[L / 4];
    if (c.phi == PHI_FAVOR) {
        float a[L / 4], wsum[L / 4];
#pragma unroll
        for (int m = 0; m < L / 4; ++m) a[m] = wsum[m] = 0.f;
        // omega column i, 4 rows at a time; the dp rows as 16-byte reads
        for (int f = 0; f < R; f += 4) {
            float om[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) om[j] = Elem<T>::load(omega, (long)(f + j) * D + i);
#pragma unroll
            for (int m = 0; m < L / 4; ++m) {
                const float4 wv = *reinterpret_cast<const float4*>(dp + (t0 + m) * ol + f);
                a[m] = fmaf(wv.x, om[0], a[m]);
                a[m] = fmaf(wv.y, om[1], a[m]);
                a[m] = fmaf(wv.z, om[2], a[m]);
                a[m] = fmaf(wv.w, om[3], a[m]);
                wsum[m] += (wv.x + wv.y) + (wv.z + wv.w);
            }
        }
#pragma unroll
        for (int m = 0; m < L / 4; ++m) du[m] = a[m] - wsum[m] * u[(t0 + m) * D + i];
    } else if (c.phi == PHI_ELU1) {
#pragma unroll
        for (int m = 0; m < L / 4; ++m) {
            const float x = u[(t0 + m) * D + i];
            du[m] = dp[(t0 + m) * ol + i] * (x > 0.f ? 1.f : expf(x));
        }
    } else if (c.phi == PHI_IDENTITY) {
#pragma unroll
        for (int m = 0; m < L / 4; ++m) du[m] = dp[(t0 + m) * ol + i];
    } else {
        // DPFP: feature (s-1)*2D + j = kt_j * kt_{(j+s) mod 2D}; kt = relu([u, -u])
        constexpr int M2 = 2 * D - 1;
#pragma unroll
        for (int m = 0; m < L / 4; ++m) {
            const float* ut = u + (t0 + m) * D;
            const float* g = dp + (t0 + m) * ol;
            float dpos = 0.f, dneg = 0.f; // d/d kt_i, d/d kt_{D+i}
            for (int s = 1; s <= c.nu; ++s) {
                const float* gs = g + (s - 1) * 2 * D;
                dpos = fmaf(gs[i], dpfp_kt(ut, (i + s) & M2), dpos);
                dpos = fmaf(gs[(i - s) & M2], dpfp_kt(ut, (i - s) & M2), dpos);
                dneg = fmaf(gs[D + i], dpfp_kt(ut, (D + i + s) & M2), dneg);
                dneg = fmaf(gs[(D + i - s) & M2], dpfp_kt(ut, (D + i - s) & M2), dneg);
            }
            const float x = ut[i];
            du[m] = (x > 0.f ? dpos : 0.f) - (x < 0.f ? dneg : 0.f);
        }
    }
#pragma unroll
    for (int m = 0; m < L / 4; ++m)
        if (t0 + m < rows) Elem<T>::store(out, (long)(t0 + m) * D + i, c.scale * du[m]);
}

// ---------------------------------------------------------------------------
// Query pass.  One workgroup per (head, segment).
// ---------------------------------------------------------------------------
template <typename T, int FPT, bool CAUSAL>
__global__ __launch_bounds__(NT) void k_bwd_query(Cfg c, const T* __restrict__ q,
                                                  const T* __restrict__ k, const T* __restrict__ v,
                                                  const T* __restrict__ dout,
                                                  const T* __restrict__ omega, int64_t N, int64_t G,
                                                  int64_t seg_len, const float* __restrict__ state,
                                                  int64_t st_bh, int64_t st_g,
                                                  const bf16_raw* __restrict__ omega_t,
                                                  float* __restrict__ inc, float* __restrict__ tok,
                                                  T* __restrict__ dq) {
    constexpr int R = 32 * FPT;
    constexpr int OL = R + 4;
    constexpr int LC = CAUSAL ? L : 1;
    __shared__ __align__(16) float S_s[R * SL];
    __shared__ __align__(16) float z_s[R];
    __shared__ __align__(16) float u_s[L * D];
    __shared__ __align__(16) float pq_s[L * OL];
    __shared__ __align__(16) float pk_s[LC * OL];
    __shared__ __align__(16) float dp_s[L * OL];
    __shared__ __align__(16) float v_s[LC * DV];
    __shared__ __align__(16) float dn_s[L * DV];
    __shared__ float dd_s[L], a_s[LC * (L + 1)];
    __shared__ float nrm_s[L], rs_s[L], live_s[L], cc_s[L];
    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x / G, g = blockIdx.x % G;
    const int64_t t0 = g * seg_len, t1 = t0 + seg_len < N ? t0 + seg_len : N;

    load_state<R>(state + bh * st_bh + g * st_g, S_s, z_s);
    float acc[2 * FPT][4], macc[2 * FPT];
#pragma unroll
    for (int it = 0; it < 2 * FPT; ++it) {
        macc[it] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[it][j] = 0.f;
    }
    const int rt = tid / 16, cb = (tid % 16) * 4; // readout: token, 4 value columns

    for (int64_t c0 = t0; c0 < t1; c0 += L) {
        const int rows = (int)min<int64_t>(L, t1 - c0);
        if (CAUSAL) {
            load_rows<T, L>(k + (bh * N + c0) * D, rows, c.scale, u_s);
            load_rows<T, L>(v + (bh * N + c0) * DV, rows, 1.f, v_s);
            __syncthreads();
            row_norms<L>(u_s, nrm_s);
            __syncthreads();
            bwd_phi_tile<T, FPT>(c, u_s, nrm_s, omega, k + (bh * N + c0) * D, rows, pk_s, OL,
                                 rs_s);
        }
        load_rows<T, L>(q + (bh * N + c0) * D, rows, c.scale, u_s);
        __syncthreads();
        row_norms<L>(u_s, nrm_s);
        __syncthreads();
        bwd_phi_tile<T, FPT>(c, u_s, nrm_s, omega, q + (bh * N + c0) * D, rows, pq_s, OL, rs_s,
                             live_s);
        if (CAUSAL) {
            masked_products<true>(pq_s, pk_s, OL, R, nullptr, a_s);
            __syncthreads();
        }

        // forward readout of token rt, then dnum, dden
        {
            float num[4] = {0.f, 0.f, 0.f, 0.f};
            float den = 0.f;
            const float* x = pq_s + rt * OL;
            for (int f = 0; f < R; f += 4) {
                const float4 p4 = *reinterpret_cast<const float4*>(x + f);
                const float4 z4 = *reinterpret_cast<const float4*>(z_s + f);
                const float pf[4] = {p4.x, p4.y, p4.z, p4.w};
                den = fmaf(p4.x, z4.x, den);
                den = fmaf(p4.y, z4.y, den);
                den = fmaf(p4.z, z4.z, den);
                den = fmaf(p4.w, z4.w, den);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float4 sv = *reinterpret_cast<const float4*>(S_s + (f + j) * SL + cb);
                    num[0] = fmaf(pf[j], sv.x, num[0]);
                    num[1] = fmaf(pf[j], sv.y, num[1]);
                    num[2] = fmaf(pf[j], sv.z, num[2]);
                    num[3] = fmaf(pf[j], sv.w, num[3]);
                }
            }
            if (CAUSAL) {
                for (int j = 0; j <= rt; ++j) {
                    const float a = a_s[rt * (L + 1) + j];
                    den += a;
                    const float4 vv = *reinterpret_cast<const float4*>(v_s + j * DV + cb);
                    num[0] = fmaf(a, vv.x, num[0]);
                    num[1] = fmaf(a, vv.y, num[1]);
                    num[2] = fmaf(a, vv.z, num[2]);
                    num[3] = fmaf(a, vv.w, num[3]);
                }
            }
            const bool attn = c.norm == NORM_ATTN;
            const float inv = attn ? 1.f / fmaxf(den, c.eps) : 1.f;
            float4 go = make_float4(0.f, 0.f, 0.f, 0.f);
            if (rt < rows) go = Elem<T>::load4(dout, (bh * N + c0 + rt) * DV + cb);
            // dout . out over the 16 lanes of this token
            float dot = go.x * num[0] + go.y * num[1] + go.z * num[2] + go.w * num[3];
#pragma unroll
            for (int off = 8; off > 0; off >>= 1) dot += __shfl_xor(dot, off, 64);
            const float dden = (attn && den > c.eps) ? -dot * inv * inv : 0.f;
            *reinterpret_cast<float4*>(dn_s + rt * DV + cb) =
                make_float4(go.x * inv, go.y * inv, go.z * inv, go.w * inv);
            if (cb == 0) {
                dd_s[rt] = dden;
                if (CAUSAL && rt < rows) {
                    tok[2 * (bh * N + c0 + rt)] = inv;
                    tok[2 * (bh * N + c0 + rt) + 1] = dden;
                }
            }
        }
        __syncthreads();
        if (CAUSAL) {
            // coefficient of phi(k_j) in dphi(q_t): v_j . dnum_t + dden_t, j <= t
            masked_products<true>(dn_s, v_s, DV, DV, nullptr, a_s);
            __syncthreads();
            for (int p = tid; p < L * L; p += NT) {
                const int t = p / L, j = p % L;
                if (j <= t) a_s[t * (L + 1) + j] += dd_s[t];
            }
            __syncthreads();
        }
        dphi_rows<FPT>(S_s, z_s, dn_s, dd_s, CAUSAL ? a_s : nullptr, pk_s, OL, dp_s);
        outer_accum<FPT>(pq_s, OL, dn_s, dd_s, rows, acc, macc);
        __syncthreads();
        phi_backward_tile<T, FPT>(c, u_s, pq_s, OL, rs_s, live_s, dp_s, cc_s, omega, omega_t, rows,
                                  dq + (bh * N + c0) * D);
        if (CAUSAL) state_update<FPT>(S_s, z_s, pk_s, OL, v_s, nullptr, rows);
        __syncthreads();
    }

    float* dst = inc + (bh * G + g) * state_elems(R);
    const int f0 = feat0<FPT>();
#pragma unroll
    for (int it = 0; it < 2 * FPT; ++it) {
        const int f = f0 + it;
        *reinterpret_cast<float4*>(dst + (long)f * DV + cb) =
            make_float4(acc[it][0], acc[it][1], acc[it][2], acc[it][3]);
        if (cb == 0) dst[(long)R * DV + f] = macc[it];
    }
}

// ---------------------------------------------------------------------------
// Key pass.  One workgroup per (head, segment); causal chunks last to first.
// ---------------------------------------------------------------------------
template <typename T, int FPT, bool CAUSAL>
__global__ __launch_bounds__(NT) void k_bwd_key(Cfg c, const T* __restrict__ q,
                                                const T* __restrict__ k, const T* __restrict__ v,
                                                const T* __restrict__ dout,
                                                const T* __restrict__ omega, int64_t N, int64_t G,
                                                int64_t seg_len, const float* __restrict__ state,
                                                int64_t st_bh, int64_t st_g,
                                                const bf16_raw* __restrict__ omega_t,
                                                const float* __restrict__ tok, T* __restrict__ dk,
                                                T* __restrict__ dv) {
    constexpr int R = 32 * FPT;
    constexpr int OL = R + 4;
    constexpr int LC = CAUSAL ? L : 1;
    __shared__ __align__(16) float G_s[R * SL];
    __shared__ __align__(16) float g_s[R];
    __shared__ __align__(16) float uk_s[L * D];
    __shared__ __align__(16) float uq_s[LC * D];
    __shared__ __align__(16) float pk_s[L * OL];
    __shared__ __align__(16) float pq_s[LC * OL];
    __shared__ __align__(16) float dp_s[L * OL];
    __shared__ __align__(16) float v_s[L * DV];
    __shared__ __align__(16) float dn_s[LC * DV];
    __shared__ float dd_s[LC], a_s[LC * (L + 1)], b_s[LC * (L + 1)];
    __shared__ float nrm_s[L], rs_s[L], live_s[L], cc_s[L], rsq_s[L];
    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x / G, g = blockIdx.x % G;
    const int64_t t0 = g * seg_len, t1 = t0 + seg_len < N ? t0 + seg_len : N;
    const int64_t nch = (t1 - t0 + L - 1) / L;

    load_state<R>(state + bh * st_bh + g * st_g, G_s, g_s);
    const int rt = tid / 16, cb = (tid % 16) * 4; // dv: key, 4 value columns

    for (int64_t ci = 0; ci < nch; ++ci) {
        const int64_t c0 = t0 + (CAUSAL ? nch - 1 - ci : ci) * L;
        const int rows = (int)min<int64_t>(L, t1 - c0);
        if (CAUSAL) {
            // the chunk's queries: phi(q_i), dnum_i = dout_i / D_i, dden_i
            load_rows<T, L>(q + (bh * N + c0) * D, rows, c.scale, uq_s);
            for (int e = tid; e < L * (DV / 4); e += NT) {
                const int t = e / (DV / 4), n4 = (e % (DV / 4)) * 4;
                float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
                float inv = 0.f;
                if (t < rows) {
                    x = Elem<T>::load4(dout, (bh * N + c0 + t) * DV + n4);
                    inv = tok[2 * (bh * N + c0 + t)];
                }
                *reinterpret_cast<float4*>(dn_s + t * DV + n4) =
                    make_float4(x.x * inv, x.y * inv, x.z * inv, x.w * inv);
            }
            for (int t = tid; t < L; t += NT) dd_s[t] = t < rows ? tok[2 * (bh * N + c0 + t) + 1] : 0.f;
            __syncthreads();
            row_norms<L>(uq_s, nrm_s);
            __syncthreads();
            bwd_phi_tile<T, FPT>(c, uq_s, nrm_s, omega, q + (bh * N + c0) * D, rows, pq_s, OL,
                                 rsq_s);
        }
        load_rows<T, L>(k + (bh * N + c0) * D, rows, c.scale, uk_s);
        load_rows<T, L>(v + (bh * N + c0) * DV, rows, 1.f, v_s);
        __syncthreads();
        row_norms<L>(uk_s, nrm_s);
        __syncthreads();
        bwd_phi_tile<T, FPT>(c, uk_s, nrm_s, omega, k + (bh * N + c0) * D, rows, pk_s, OL, rs_s,
                             live_s);
        if (CAUSAL) {
            // b[j][i] = phi(k_j) . phi(q_i); a[j][i] = v_j . dnum_i + dden_i; i >= j
            masked_products<false>(pk_s, pq_s, OL, R, nullptr, b_s);
            masked_products<false>(v_s, dn_s, DV, DV, dd_s, a_s);
            __syncthreads();
        }
        dphi_rows<FPT>(G_s, g_s, v_s, nullptr, CAUSAL ? a_s : nullptr, pq_s, OL, dp_s);
        {
            // dv_j = G^T phi(k_j) + sum_{i >= j} b[j][i] dnum_i
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
            const float* x = pk_s + rt * OL;
            for (int f = 0; f < R; f += 4) {
                const float4 p4 = *reinterpret_cast<const float4*>(x + f);
                const float pf[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float4 gv = *reinterpret_cast<const float4*>(G_s + (f + j) * SL + cb);
                    acc[0] = fmaf(pf[j], gv.x, acc[0]);
                    acc[1] = fmaf(pf[j], gv.y, acc[1]);
                    acc[2] = fmaf(pf[j], gv.z, acc[2]);
                    acc[3] = fmaf(pf[j], gv.w, acc[3]);
                }
            }
            if (CAUSAL) {
                for (int i = rt; i < L; ++i) {
                    const float b = b_s[rt * (L + 1) + i];
                    const float4 dn = *reinterpret_cast<const float4*>(dn_s + i * DV + cb);
                    acc[0] = fmaf(b, dn.x, acc[0]);
                    acc[1] = fmaf(b, dn.y, acc[1]);
                    acc[2] = fmaf(b, dn.z, acc[2]);
                    acc[3] = fmaf(b, dn.w, acc[3]);
                }
            }
            if (rt < rows) {
                T* o = dv + (bh * N + c0 + rt) * DV + cb;
#pragma unroll
                for (int j = 0; j < 4; ++j) Elem<T>::store(o, j, acc[j]);
            }
        }
        __syncthreads();
        phi_backward_tile<T, FPT>(c, uk_s, pk_s, OL, rs_s, live_s, dp_s, cc_s, omega, omega_t, rows,
                                  dk + (bh * N + c0) * D);
        if (CAUSAL) state_update<FPT>(G_s, g_s, pq_s, OL, dn_s, dd_s, rows);
        __syncthreads();
    }
}

template <typename T, int FPT>
void query_fpt(const Cfg& c, int causal, const void* q, const void* k, const void* v,
               const void* dout, const void* omega, Shape s, SegPlan sp, const float* state,
               int64_t sbh, int64_t sg, const bf16_raw* omega_t, float* inc, float* tok, void* dq,
               hipStream_t st) {
    const dim3 grid((unsigned)(sp.G * s.BH)), block(NT);
    if (causal)
        hipLaunchKernelGGL((k_bwd_query<T, FPT, true>), grid, block, 0, st, c, (const T*)q,
                           (const T*)k, (const T*)v, (const T*)dout, (const T*)omega, s.N, sp.G,
                           sp.seg_len, state, sbh, sg, omega_t, inc, tok, (T*)dq);
    else
        hipLaunchKernelGGL((k_bwd_query<T, FPT, false>), grid, block, 0, st, c, (const T*)q,
                           (const T*)k, (const T*)v, (const T*)dout, (const T*)omega, s.N, sp.G,
                           sp.seg_len, state, sbh, sg, omega_t, inc, tok, (T*)dq);
}

template <typename T, int FPT>
void key_fpt(const Cfg& c, int causal, const void* q, const void* k, const void* v,
             const void* dout, const void* omega, Shape s, SegPlan sp, const float* state,
             int64_t sbh, int64_t sg, const bf16_raw* omega_t, const float* tok, void* dk,
             void* dv, hipStream_t st) {
    const dim3 grid((unsigned)(sp.G * s.BH)), block(NT);
    if (causal)
        hipLaunchKernelGGL((k_bwd_key<T, FPT, true>), grid, block, 0, st, c, (const T*)q,
                           (const T*)k, (const T*)v, (const T*)dout, (const T*)omega, s.N, sp.G,
                           sp.seg_len, state, sbh, sg, omega_t, tok, (T*)dk, (T*)dv);
    else
        hipLaunchKernelGGL((k_bwd_key<T, FPT, false>), grid, block, 0, st, c, (const T*)q,
                           (const T*)k, (const T*)v, (const T*)dout, (const T*)omega, s.N, sp.G,
                           sp.seg_len, state, sbh, sg, omega_t, tok, (T*)dk, (T*)dv);
}

template <typename T>
hipError_t query_t(const Cfg& c, int causal, const void* q, const void* k, const void* v,
                   const void* dout, const void* omega, Shape s, SegPlan sp, const float* state,
                   int64_t sbh, int64_t sg, const bf16_raw* omega_t, float* inc, float* tok,
                   void* dq, hipStream_t st) {
#define LINATTN_QUERY(F)                                                                         \
    case F: query_fpt<T, F>(c, causal, q, k, v, dout, omega, s, sp, state, sbh, sg, omega_t, inc,  \
                            tok, dq, st);                                                        \
        break;
    switch (c.r / 32) {
        LINATTN_QUERY(1) LINATTN_QUERY(2) LINATTN_QUERY(3) LINATTN_QUERY(4)
        LINATTN_QUERY(5) LINATTN_QUERY(6) LINATTN_QUERY(7) LINATTN_QUERY(8)
    default: return hipErrorInvalidValue;
    }
#undef LINATTN_QUERY
    return hipGetLastError();
}

template <typename T>
hipError_t key_t(const Cfg& c, int causal, const void* q, const void* k, const void* v,
                 const void* dout, const void* omega, Shape s, SegPlan sp, const float* state,
                 int64_t sbh, int64_t sg, const bf16_raw* omega_t, const float* tok, void* dk,
                 void* dv, hipStream_t st) {
#define LINATTN_KEY(F)                                                                            \
    case F: key_fpt<T, F>(c, causal, q, k, v, dout, omega, s, sp, state, sbh, sg, omega_t, tok, dk, \
                          dv, st);                                                               \
        break;
    switch (c.r / 32) {
        LINATTN_KEY(1) LINATTN_KEY(2) LINATTN_KEY(3) LINATTN_KEY(4)
        LINATTN_KEY(5) LINATTN_KEY(6) LINATTN_KEY(7) LINATTN_KEY(8)
    default: return hipErrorInvalidValue;
    }
#undef LINATTN_KEY
    return hipGetLastError();
}

} // namespace

hipError_t launch_transpose_omega(const void* omega, int r, void* omega_t, hipStream_t st) {
    const int64_t n = (int64_t)r * D;
    hipLaunchKernelGGL(k_transpose_omega, dim3((unsigned)((n + NT - 1) / NT)), dim3(NT), 0, st,
                       (const bf16_raw*)omega, r, (bf16_raw*)omega_t);
    return hipGetLastError();
}

hipError_t launch_backward_query(const Cfg& c, int dtype, int causal, const void* q,
                                 const void* k, const void* v, const void* dout, const void* omega,
                                 Shape s, SegPlan sp, const float* state, int64_t sbh, int64_t sg,
                                 const void* omega_t, float* inc, float* tok, void* dq,
                                 hipStream_t st) {
    const bf16_raw* ot = (const bf16_raw*)omega_t;
    return dtype == 0 ? query_t<float>(c, causal, q, k, v, dout, omega, s, sp, state, sbh, sg, ot,
                                       inc, tok, dq, st)
                      : query_t<bf16_raw>(c, causal, q, k, v, dout, omega, s, sp, state, sbh, sg,
                                          ot, inc, tok, dq, st);
}

hipError_t launch_backward_key(const Cfg& c, int dtype, int causal, const void* q, const void* k,
                               const void* v, const void* dout, const void* omega, Shape s,
                               SegPlan sp, const float* state, int64_t sbh, int64_t sg,
                               const void* omega_t, const float* tok, void* dk, void* dv,
                               hipStream_t st) {
    const bf16_raw* ot = (const bf16_raw*)omega_t;
    return dtype == 0 ? key_t<float>(c, causal, q, k, v, dout, omega, s, sp, state, sbh, sg, ot,
                                     tok, dk, dv, st)
                      : key_t<bf16_raw>(c, causal, q, k, v, dout, omega, s, sp, state, sbh, sg, ot,
                                        tok, dk, dv, st);
}

} // namespace linattn
