// decode.hip -- one decode step for B*H independent heads (Kernel Zoo sec. 1.2
// steps 2-3, "update, then read"):
//   S <- S + phi(k) v^T,  z <- z + phi(k),
//   out = phi(q)^T S / max(phi(q) . z, eps)     (or phi(q)^T S, NORM_NONE)
//
// The step is a streaming read-modify-write of the float32 state: per head
// r*dv*4 bytes of S (64 KiB at r = 256) are read and written once, against
// ~2 flops per byte, so the kernel is bound by HBM bandwidth.  One workgroup
// per head (512 or 1024 threads): every thread issues all of its S loads
// (16-byte, non-temporal) before its share of phi(q), phi(k) is computed, so
// the feature map runs under the load latency; the new S goes straight back
// with non-temporal stores and the readout is accumulated from registers.
#include "launch.hpp"

namespace linattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Row f of omega, raw (bfloat16 pairs or float32), loaded early and
// unpacked only when the feature is computed.
template <typename T> struct OmegaRow;
template <> struct OmegaRow<bf16_raw> {
    uint4 w[D / 8];
    __device__ __forceinline__ void load(const bf16_raw* om, int f) {
#pragma unroll
        for (int i = 0; i < D / 8; ++i) w[i] = reinterpret_cast<const uint4*>(om + (int64_t)f * D)[i];
    }
    // omega_f . a and omega_f . b in one pass: each element is unpacked and
    // used at once, so the unpacked row is never live as a whole (that would
    // cost 64 registers on top of the state's 64 and halve the occupancy)
    __device__ __forceinline__ void dot2(const float* a, const float* b, float& da,
                                         float& db) const {
        float sa = 0.f, sb = 0.f;
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
            const uint32_t x[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float lo = __uint_as_float(x[j] << 16), hi = __uint_as_float(x[j] & 0xffff0000u);
                sa = fmaf(lo, a[8 * i + 2 * j], sa);
                sb = fmaf(lo, b[8 * i + 2 * j], sb);
                sa = fmaf(hi, a[8 * i + 2 * j + 1], sa);
                sb = fmaf(hi, b[8 * i + 2 * j + 1], sb);
            }
        }
        da = sa;
        db = sb;
    }
};
template <> struct OmegaRow<float> {
    float4 w[D / 4];
    __device__ __forceinline__ void load(const float* om, int f) {
#pragma unroll
        for (int i = 0; i < D / 4; ++i) w[i] = reinterpret_cast<const float4*>(om + (int64_t)f * D)[i];
    }
    __device__ __forceinline__ void dot2(const float* a, const float* b, float& da,
                                         float& db) const {
        float sa = 0.f, sb = 0.f;
#pragma unroll
        for (int i = 0; i < D / 4; ++i) {
            const float e[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sa = fmaf(e[j], a[4 * i + j], sa);
                sb = fmaf(e[j], b[4 * i + j], sb);
            }
        }
        da = sa;
        db = sb;
    }
};

// NT threads per head (512 or 1024, NT dividing 16 r): the state is split
// NT ways, 16 r / NT float4 per thread, so few registers hold it and many
// waves stream it; threads tid < r also compute feature tid.  RM: the
// largest r of the instance (256, or RMAX): the register array of the
// state is sized for it.
template <typename T, int NT, int RM>
__global__ __launch_bounds__(NT) void k_decode(Cfg c, const T* __restrict__ q,
                                               const T* __restrict__ k,
                                               const T* __restrict__ v,
                                               const T* __restrict__ omega,
                                               float* __restrict__ S, float* __restrict__ z,
                                               T* __restrict__ out) {
    __shared__ float uq_s[D], uk_s[D], v_s[DV];
    __shared__ float pq_s[RM], pk_s[RM];
    __shared__ float red_s[NT / 64][DV];
    constexpr int MAXM = RM * DV / 4 / NT; // float4 of S per thread at r = RM
    __shared__ float scal_s[2 + NT / 64]; // |u_q|^2, |u_k|^2, then den per wave
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t bh = blockIdx.x;
    const int r = c.r;
    const int m_count = r * DV / 4 / NT; // float4 of S per thread
    const bool favor = c.phi == PHI_FAVOR;

    // 1. the feature map's inputs first: vector-memory counters retire in
    //    order, so anything issued after the S stream would wait for all of it
    float xq = 0.f, xk = 0.f, xv = 0.f;
    if (tid < D) {
        xq = Elem<T>::load(q, bh * D + tid);
        xk = Elem<T>::load(k, bh * D + tid);
        xv = Elem<T>::load(v, bh * DV + tid);
    }
    OmegaRow<T> om;
    if (favor && tid < r) om.load(omega, tid);

    // 2. the state stream: float4 e = tid + NT*m is row e/16, columns
    //    4*(tid%16) .. +3.  Every load is issued unconditionally (past m_count
    //    the last block of rows is read again): with a data-dependent load
    //    count the compiler cannot count the loads still in flight and waits
    //    for the whole stream before the feature map.
    f32x4* S4 = reinterpret_cast<f32x4*>(S + bh * (int64_t)r * DV);
    f32x4 s[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m)
        s[m] = __builtin_nontemporal_load(S4 + tid + NT * (m < m_count ? m : m_count - 1));
    const float zold = __builtin_nontemporal_load(z + bh * r + (tid < r ? tid : r - 1));

    if (tid < D) {
        uq_s[tid] = c.scale * xq;
        uk_s[tid] = c.scale * xk;
        v_s[tid] = xv;
        if (favor) {
            // |scale x|^2 of q (wave 0 holds all 64 components)
            const float nq = wave_sum(uq_s[tid] * uq_s[tid]);
            const float nk = wave_sum(uk_s[tid] * uk_s[tid]);
            if (lane == 0) {
                scal_s[0] = nq;
                scal_s[1] = nk;
            }
        }
    }
    sync_lds();

    // 3. one feature of phi(q) and phi(k) per thread
    float pq = 0.f, pk = 0.f;
    if (tid < r) {
        if (favor) {
            // omega . (scale x), from the unscaled row and the scaled input
            float dq, dk;
            om.dot2(uq_s, uk_s, dq, dk);
            pq = favor_feature(c, dq, scal_s[0]);
            pk = favor_feature(c, dk, scal_s[1]);
        } else {
            pq = phi_feature<T>(c, uq_s, 0.f, tid, omega);
            pk = phi_feature<T>(c, uk_s, 0.f, tid, omega);
        }
    }
    if (c.sum_norm) {
        const float a = wave_sum(pq), b = wave_sum(pk);
        if (lane == 0) {
            red_s[w][0] = a;
            red_s[w][1] = b;
        }
        sync_lds();
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int i = 0; i < NT / 64; ++i) {
            sq += red_s[i][0];
            sk += red_s[i][1];
        }
        pq *= 1.f / fmaxf(sq, c.eps);
        pk *= 1.f / fmaxf(sk, c.eps);
        sync_lds(); // red_s is reused below
    }
    if (tid < r) {
        pq_s[tid] = pq;
        pk_s[tid] = pk;
    }

    // 4. z <- z + phi(k); den = phi(q) . z
    float den_part = 0.f;
    if (tid < r) {
        const float zn = zold + pk;
        __builtin_nontemporal_store(zn, z + bh * r + tid);
        den_part = pq * zn;
    }
    den_part = wave_sum(den_part);
    if (lane == 0) scal_s[2 + w] = den_part;
    sync_lds();

    // 5. S rows: S <- S + phi(k)_row v^T, o += phi(q)_row S_row
    const int c4 = (tid % 16) * 4;
    const float4 vv = make_float4(v_s[c4], v_s[c4 + 1], v_s[c4 + 2], v_s[c4 + 3]);
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
        if (m < m_count) {
            const int row = tid / 16 + (NT / 16) * m;
            const float a = pk_s[row], b = pq_s[row];
            f32x4 x = s[m];
            x.x = fmaf(a, vv.x, x.x);
            x.y = fmaf(a, vv.y, x.y);
            x.z = fmaf(a, vv.z, x.z);
            x.w = fmaf(a, vv.w, x.w);
            __builtin_nontemporal_store(x, S4 + tid + NT * m);
            o.x = fmaf(b, x.x, o.x);
            o.y = fmaf(b, x.y, o.y);
            o.z = fmaf(b, x.z, o.z);
            o.w = fmaf(b, x.w, o.w);
        }
    }
    // 6. reduce o over the threads sharing columns c4..c4+3: lanes l^16,
    //    l^32 within the wave, then the NT/64 waves through LDS.
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
        o.x += __shfl_xor(o.x, off, 64);
        o.y += __shfl_xor(o.y, off, 64);
        o.z += __shfl_xor(o.z, off, 64);
        o.w += __shfl_xor(o.w, off, 64);
    }
    if (lane < 16) {
        red_s[w][c4] = o.x;
        red_s[w][c4 + 1] = o.y;
        red_s[w][c4 + 2] = o.z;
        red_s[w][c4 + 3] = o.w;
    }
    sync_lds();
    if (tid < DV) {
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int i = 0; i < NT / 64; ++i) {
            num += red_s[i][tid];
            den += scal_s[2 + i];
        }
        const float y = c.norm == NORM_ATTN ? num / fmaxf(den, c.eps) : num;
        Elem<T>::store(out, bh * DV + tid, y);
    }
}

template <int NT, int RM>
hipError_t launch_decode_nt(const Cfg& c, int dtype, const void* q, const void* k, const void* v,
                            const void* omega, int64_t BH, float* S, float* z, void* out,
                            hipStream_t st) {
    if (dtype == 0)
        hipLaunchKernelGGL((k_decode<float, NT, RM>), dim3((unsigned)BH), dim3(NT), 0, st, c,
                           (const float*)q, (const float*)k, (const float*)v,
                           (const float*)omega, S, z, (float*)out);
    else
        hipLaunchKernelGGL((k_decode<bf16_raw, NT, RM>), dim3((unsigned)BH), dim3(NT), 0, st, c,
                           (const bf16_raw*)q, (const bf16_raw*)k, (const bf16_raw*)v,
                           (const bf16_raw*)omega, S, z, (bf16_raw*)out);
    return hipGetLastError();
}

} // namespace

// 1024 threads per head where they split the state evenly (r a multiple of
// 64), else 512 (r is a multiple of 32).  Measured at r = 256: 1024 threads
// stream the state ~10 % faster than 256 (more waves, fewer registers each).
hipError_t launch_decode(const Cfg& c, int dtype, const void* q, const void* k, const void* v,
                         const void* omega, int64_t BH, float* S, float* z, void* out,
                         hipStream_t st) {
    // widths past 256 get their own instances, so that the r <= 256 ones keep
    // their register count (a state array sized for r = 512 would issue
    // twice the loads at r = 256)
    if (c.r <= 256) {
        if (c.r % 64 == 0)
            return launch_decode_nt<1024, 256>(c, dtype, q, k, v, omega, BH, S, z, out, st);
        return launch_decode_nt<512, 256>(c, dtype, q, k, v, omega, BH, S, z, out, st);
    }
    if (c.r % 64 == 0)
        return launch_decode_nt<1024, RMAX>(c, dtype, q, k, v, omega, BH, S, z, out, st);
    return launch_decode_nt<512, RMAX>(c, dtype, q, k, v, omega, BH, S, z, out, st);
}

} // namespace linattn
