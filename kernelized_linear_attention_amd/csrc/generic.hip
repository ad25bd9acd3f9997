// generic.hip -- LDS-tiled kernels with float32 vector arithmetic, for every
// feature map, float32 and bfloat16 inputs, r a multiple of 32 up to 256.
//
// The chunked scan follows the causal recurrence of the Kernel Zoo (sec. 1.3,
// sec. 5.4): S_t = S_{t-1} + phi(k_t) v_t^T, z_t = z_{t-1} + phi(k_t),
// out_t = phi(q_t)^T S_t / max(phi(q_t) . z_t, eps).  It is evaluated as
//   segments (workgroups) -> chunks of L tokens -> tokens,
// where for a chunk c with carried-in state (S_{c-1}, z_{c-1})
//   num_t = phi(q_t)^T S_{c-1} + sum_{j<=t in c} (phi(q_t) . phi(k_j)) v_j
//   den_t = phi(q_t) . z_{c-1} + sum_{j<=t in c}  phi(q_t) . phi(k_j)
// and S_c = S_{c-1} + phi(K_c)^T V_c, z_c = z_{c-1} + phi(K_c)^T 1: the same
// sums, re-associated.  Segment starting states come from an exclusive prefix
// sum of per-segment increments (launch_segment_scan), summed in a fixed
// order, so results are bitwise reproducible.
#include <algorithm>

#include "launch.hpp"
#include "proj.hpp"
#include "tiles.hpp"

namespace linattn {
namespace {

constexpr int NT = VNT; // threads per workgroup in this file

// ---------------------------------------------------------------------------
// Feature map alone: phi [BH, N, r] float32.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(NT) void k_featuremap(Cfg c, const T* __restrict__ x,
                                                   const T* __restrict__ omega, int64_t N,
                                                   int64_t tiles, float* __restrict__ phi) {
    constexpr int L = 32;
    __shared__ float u_s[L * D];
    __shared__ float p_s[L * (RMAX + 4)];
    __shared__ float nrm_s[L], rs_s[L];
    const int64_t bh = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    const int64_t t0 = tile * L;
    const int rows = (int)min<int64_t>(L, N - t0);
    const int ol = c.r + 4;
    load_rows<T, L>(x + (bh * N + t0) * D, rows, c.scale, u_s);
    __syncthreads();
    row_norms<L>(u_s, nrm_s);
    __syncthreads();
    phi_tile<T, L>(c, u_s, nrm_s, omega, rows, p_s, ol, rs_s);
    float* dst = phi + (bh * N + t0) * c.r;
    for (int idx = threadIdx.x; idx < rows * c.r; idx += NT) {
        const int t = idx / c.r, f = idx - t * c.r;
        dst[(long)t * c.r + f] = p_s[t * ol + f];
    }
}

// ---------------------------------------------------------------------------
// Segment state increments: ws[bh][g] = (sum phi(k_j) v_j^T, sum phi(k_j)).
// Thread (fb = tid/8, nb = tid%8) owns S[fb*FPT + i][nb*8 + j], i < FPT, j < 8.
// ---------------------------------------------------------------------------
// PROJ: k and v are projected from the tokens x (proj.hpp) instead of read.
template <typename T, int FPT, bool PROJ>
__global__ __launch_bounds__(NT) void k_segment_sums(Cfg c, const T* __restrict__ k,
                                                     const T* __restrict__ v,
                                                     const T* __restrict__ omega, int64_t N,
                                                     int64_t G, int64_t seg_len,
                                                     const int64_t* __restrict__ tab,
                                                     float* __restrict__ ws, Proj P) {
    // 64-token chunks up to r = 256; 16 above, so that the feature tile
    // (L x (r + 4) floats) stays within LDS
    constexpr int L = FPT <= 8 ? 64 : 16;
    constexpr int R = 32 * FPT;
    constexpr int OL = R + 4;
    __shared__ float u_s[L * D];
    __shared__ float v_s[L * DV];
    __shared__ float p_s[L * OL];
    __shared__ float nrm_s[L], rs_s[L];
    const int tid = threadIdx.x;
    const int fb = tid / 8, nb = tid % 8;
    const int64_t bh = blockIdx.x / G, g = blockIdx.x % G;
    int64_t t0, t1;
    seg_range(tab, 1, g, seg_len, N, t0, t1);

    float acc[FPT][8];
    float zacc[FPT];
#pragma unroll
    for (int i = 0; i < FPT; ++i) {
        zacc[i] = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
    }
    for (int64_t c0 = t0; c0 < t1; c0 += L) {
        const int rows = (int)min<int64_t>(L, t1 - c0);
        if constexpr (PROJ) {
            project_chunk<L>(P, bh, N, c0, rows, PROJ_K, u_s, c.scale, PROJ_V, v_s, 1.f);
        } else {
            load_rows<T, L>(k + (bh * N + c0) * D, rows, c.scale, u_s);
            load_rows<T, L>(v + (bh * N + c0) * DV, rows, 1.f, v_s);
        }
        __syncthreads();
        row_norms<L>(u_s, nrm_s);
        __syncthreads();
        phi_tile<T, L>(c, u_s, nrm_s, omega, rows, p_s, OL, rs_s);
        for (int t = 0; t < rows; ++t) {
            float vv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) vv[j] = v_s[t * DV + nb * 8 + j];
#pragma unroll
            for (int i = 0; i < FPT; ++i) {
                const float p = p_s[t * OL + fb * FPT + i];
                zacc[i] += p;
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(p, vv[j], acc[i][j]);
            }
        }
        __syncthreads();
    }
    float* dst = ws + (bh * G + g) * state_elems(R);
#pragma unroll
    for (int i = 0; i < FPT; ++i) {
        const int f = fb * FPT + i;
#pragma unroll
        for (int j = 0; j < 8; ++j) dst[(long)f * DV + nb * 8 + j] = acc[i][j];
        if (nb == 0) dst[(long)R * DV + f] = zacc[i];
    }
}

// ---------------------------------------------------------------------------
// Prefix over segments, fixed order.  REV: the same over the segments in
// reverse order (exclusive suffix sums).  The walk is latency-bound (one
// float per state element and segment, strided by a whole state), so each
// element's segments are split into P consecutive ranges (P = 1, 2 or 4, by
// the segment count), one per wave group of the workgroup (NT / P elements
// per workgroup): every thread loads its range's increments at once and sums
// them, the ranges' totals are exchanged through LDS, and each thread then
// writes its range's prefixes from its offset (the totals added in range
// order: a fixed order).
// ---------------------------------------------------------------------------
constexpr int SCAN_BATCH = 16; // increments held in registers per thread

template <bool REV, int P>
__global__ __launch_bounds__(NT) void k_segment_scan(int r, int64_t G, const float* __restrict__ S0,
                                                     const float* __restrict__ z0,
                                                     float* __restrict__ ws, int prefix_stride,
                                                     float* __restrict__ S_fin,
                                                     float* __restrict__ z_fin,
                                                     float* __restrict__ fin) {
    constexpr int EPB = NT / P; // elements per workgroup
    __shared__ float tot_s[P][EPB];
    const int64_t E = state_elems(r);
    const int64_t blocks_per_head = (E + EPB - 1) / EPB;
    const int64_t bh = blockIdx.x / blocks_per_head;
    const int el = threadIdx.x % EPB, part = threadIdx.x / EPB;
    const int64_t e = (blockIdx.x % blocks_per_head) * EPB + el;
    const bool live = e < E;
    const int64_t ec = live ? e : E - 1; // in-bounds element for the loads
    const int64_t rdv = (int64_t)r * DV;
    // this wave's segments [g0, g1) (step i of the walk is segment G-1-i for REV)
    const int64_t per = (G + P - 1) / P;
    const int64_t g0 = min<int64_t>(G, part * per), g1 = min<int64_t>(G, g0 + per);
    auto at = [&](int64_t i) {
        return REV ? ws + (bh * G + G - 1 - i) * E + ec : ws + (bh * G + i) * E + ec;
    };
    // the starting state (any in-bounds value when there is none), then the
    // first SCAN_BATCH increments of the range, every load unconditional
    // (clamped to the range's first segment when the range is shorter or
    // empty; those values are not used)
    const float* init = S0 ? (ec < rdv ? S0 + bh * rdv + ec : z0 + bh * r + (ec - rdv))
                           : at(min<int64_t>(g0, G - 1));
    const float run0 = *init;
    const int n0 = (int)min<int64_t>(SCAN_BATCH, g1 - g0);
    float a[SCAN_BATCH];
#pragma unroll
    for (int i = 0; i < SCAN_BATCH; ++i) a[i] = *at(min<int64_t>(g0 + (i < n0 ? i : 0), G - 1));
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < SCAN_BATCH; ++i)
        if (i < n0) tot += a[i];
    for (int64_t i = g0 + SCAN_BATCH; i < g1; ++i) tot += *at(i);
    // every load above has landed: the prefix stores below then wait for
    // nothing (the compiler's counting cannot see that through the
    // conditional uses, and would wait for each store to complete)
    wait_all_loads();
    if (P > 1) {
        tot_s[part][el] = tot;
        __syncthreads();
    }
    float run = S0 ? run0 : 0.f;
    for (int u = 0; u < part; ++u) run += tot_s[u][el];
    // the exclusive prefix is written back only for the segments that read it
    // (every prefix_stride-th; the stride is a power of two)
    const int64_t pmask = prefix_stride - 1;
    if (live) {
#pragma unroll
        for (int i = 0; i < SCAN_BATCH; ++i) {
            if (i < n0) {
                if (prefix_stride > 0 && ((g0 + i) & pmask) == 0) *at(g0 + i) = run;
                run += a[i];
            }
        }
        for (int64_t i = g0 + SCAN_BATCH; i < g1; ++i) {
            const float x = *at(i);
            if (prefix_stride > 0 && (i & pmask) == 0) *at(i) = run;
            run += x;
        }
    }
    // the last range ends with the total
    if (live && part == P - 1) {
        if (e < rdv) {
            if (S_fin) S_fin[bh * rdv + e] = run;
        } else {
            if (z_fin) z_fin[bh * r + (e - rdv)] = run;
        }
        if (fin) fin[bh * E + e] = run;
    }
}

// ---------------------------------------------------------------------------
// Packed sequences: the segment table and the per-sequence prefix.
// ---------------------------------------------------------------------------
// One workgroup walks the sequences NT at a time: each thread counts its
// sequence's parts, a workgroup scan turns the counts into offsets, and the
// thread writes its parts.  Every range is clamped to [0, total] and every
// index to cap, whatever cu_seqlens holds.  A second walk writes the
// dispatch order: all full segments (seg_len tokens) first, then each
// sequence's partial last segment, in buckets of 64 tokens from the longest
// down (list scheduling, longest first, as the hardware dispatches
// workgroups in order).
__device__ __forceinline__ void seq_bounds(const int32_t* cu, int64_t i, int64_t total, int64_t& s0,
                                           int64_t& s1) {
    s0 = min<int64_t>(max<int64_t>(cu[i], 0), total);
    s1 = min<int64_t>(max<int64_t>(cu[i + 1], s0), total);
}

// Exclusive scan of one value per thread over the workgroup (all threads
// call it); returns this thread's offset and sets *sum to the total.  Each
// wave scans its 64 values with lane shuffles; the waves' totals meet in
// buf[0 .. NT/64) (two barriers per call).
__device__ int64_t block_exclusive_scan(int64_t x, int64_t* buf, int64_t* sum) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int64_t incl = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
    }
    if (lane == 63) buf[w] = incl;
    __syncthreads();
    int64_t before = 0, total = 0;
#pragma unroll
    for (int u = 0; u < NT / 64; ++u) {
        const int64_t t = buf[u];
        if (u < w) before += t;
        total += t;
    }
    *sum = total;
    __syncthreads(); // buf is written again by the next call
    return before + incl - x;
}

__global__ __launch_bounds__(NT) void k_varlen_plan(const int32_t* __restrict__ cu, int64_t num_seqs,
                                                    int64_t total, int64_t seg_len, int64_t sub,
                                                    int64_t cap, int64_t* __restrict__ tab,
                                                    int64_t* __restrict__ first,
                                                    int64_t* __restrict__ order) {
    constexpr int NB = 128; // partial-segment buckets of 64 tokens (seg_len <= 8192)
    __shared__ int64_t buf[NT];
    __shared__ int bucket_n[NB], bucket_at[NB];
    const int tid = threadIdx.x;
    const int64_t part_len = seg_len / sub;
    const int64_t seg_cap = cap / sub;
    const int nb = (int)min<int64_t>(NB, (seg_len + 63) / 64);
    for (int j = tid; j < NB; j += NT) bucket_n[j] = 0;
    for (int64_t e = tid; e < seg_cap; e += NT) order[e] = -1; // every entry defined
    __syncthreads();
    int64_t base = 0, full_base = 0;
    for (int64_t i0 = 0; i0 < num_seqs; i0 += NT) {
        const int64_t i = i0 + tid;
        int64_t s0 = 0, s1 = 0, n = 0, nf = 0;
        if (i < num_seqs) {
            seq_bounds(cu, i, total, s0, s1);
            n = (s1 - s0 + seg_len - 1) / seg_len * sub;
            nf = (s1 - s0) / seg_len;
        }
        int64_t sum, fsum;
        const int64_t e0 = base + block_exclusive_scan(n, buf, &sum);
        block_exclusive_scan(nf, buf, &fsum);
        if (i < num_seqs) {
            first[i] = min<int64_t>(e0, cap);
            for (int64_t j = 0; j < n && e0 + j < cap; ++j) {
                const int64_t x = s0 + j * part_len;
                tab[2 * (e0 + j)] = min<int64_t>(x, s1);
                tab[2 * (e0 + j) + 1] = min<int64_t>(x + part_len, s1);
            }
            const int64_t rem = (s1 - s0) % seg_len;
            if (rem > 0) atomicAdd(&bucket_n[min<int64_t>(nb - 1, (rem - 1) / 64)], 1);
        }
        base += sum;
        full_base += fsum;
    }
    const int64_t used = min<int64_t>(base, cap);
    if (tid == 0) first[num_seqs] = used;
    for (int64_t e = used + tid; e < cap; e += NT) {
        tab[2 * e] = 0;
        tab[2 * e + 1] = 0;
    }
    // bucket offsets, longest partials first (nb <= NB <= NT: one thread each)
    __syncthreads();
    {
        const int j = nb - 1 - tid; // descending bucket index
        int64_t c = (tid < nb) ? bucket_n[j] : 0, sum;
        const int64_t off = block_exclusive_scan(c, buf, &sum);
        if (tid < nb) bucket_at[j] = (int)min<int64_t>(full_base + off, seg_cap);
    }
    __syncthreads();
    // second walk: full segments in sequence order, partials into their bucket
    // (the parts' offsets scanned again rather than read back from first[])
    int64_t fbase = 0, pbase = 0;
    for (int64_t i0 = 0; i0 < num_seqs; i0 += NT) {
        const int64_t i = i0 + tid;
        int64_t s0 = 0, s1 = 0, n = 0, nf = 0;
        if (i < num_seqs) {
            seq_bounds(cu, i, total, s0, s1);
            n = (s1 - s0 + seg_len - 1) / seg_len * sub;
            nf = (s1 - s0) / seg_len;
        }
        int64_t sum, fsum;
        const int64_t e0 = pbase + block_exclusive_scan(n, buf, &sum);
        const int64_t f0 = fbase + block_exclusive_scan(nf, buf, &fsum);
        if (i < num_seqs) {
            const int64_t g0 = min<int64_t>(e0, cap) / sub; // the sequence's first segment
            for (int64_t j = 0; j < nf && f0 + j < seg_cap && g0 + j < seg_cap; ++j)
                order[f0 + j] = g0 + j;
            const int64_t rem = (s1 - s0) % seg_len;
            if (rem > 0) {
                const int pos = atomicAdd(&bucket_at[min<int64_t>(nb - 1, (rem - 1) / 64)], 1);
                if (pos < seg_cap) order[pos] = g0 + nf < seg_cap ? g0 + nf : -1;
            }
        }
        fbase += fsum;
        pbase += sum;
    }
}

// Like k_segment_scan, over the parts of one sequence of one head: a
// sequence starts from its own state, so the carry resets at every sequence
// boundary.  Block (element block, h, i).
__global__ __launch_bounds__(NT) void k_segment_scan_varlen(int r, int64_t H, int64_t parts,
                                                            const int64_t* __restrict__ first,
                                                            const float* __restrict__ S0,
                                                            const float* __restrict__ z0,
                                                            float* __restrict__ ws, int prefix_stride,
                                                            float* __restrict__ S_fin,
                                                            float* __restrict__ z_fin) {
    constexpr int BATCH = 16;
    const int64_t E = state_elems(r);
    const int64_t bpe = (E + NT - 1) / NT;
    const int64_t rest = blockIdx.x / bpe;
    const int64_t h = rest % H, i = rest / H;
    const int64_t e = (blockIdx.x % bpe) * NT + threadIdx.x;
    if (e >= E) return;
    const int64_t rdv = (int64_t)r * DV;
    const int64_t sh = i * H + h;
    float run = 0.f;
    if (S0) run = e < rdv ? S0[sh * rdv + e] : z0[sh * r + (e - rdv)];
    const int64_t g0 = first[i], g1 = first[i + 1];
    float* p = ws + h * parts * E + e;
    const int64_t pmask = prefix_stride - 1;
    for (int64_t gb = g0; gb < g1; gb += BATCH) {
        const int n = (int)min<int64_t>(BATCH, g1 - gb);
        float a[BATCH];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) a[j] = j < n ? p[(gb + j) * E] : 0.f;
        wait_all_loads(); // else each prefix store below waits for the ones before it
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            if (j < n) {
                if (prefix_stride > 0 && ((gb + j - g0) & pmask) == 0) p[(gb + j) * E] = run;
                run += a[j];
            }
        }
    }
    if (e < rdv)
        S_fin[sh * rdv + e] = run;
    else
        z_fin[sh * r + (e - rdv)] = run;
}

// The same scan with one block per (64 elements, head) instead of per
// (element block, head, sequence), for batches of at most MAXS_LDS
// sequences: the sequence starts first[] are staged in LDS once, and the
// head's parts are split into P consecutive ranges, one per wave (64
// elements each, so every branch on the parts is uniform over the wave), so
// that no thread walks more than a few batches of loads.  A sequence that
// spans ranges is carried across them as a segmented scan: each range first
// sums its last sequence's parts within the range (from that sequence's
// starting state when it starts in the range), the ranges' carries are formed
// in range order through LDS (a range whose last sequence starts inside it
// restarts the carry), and each range then writes its prefixes from its
// carry.  Every sum is taken in a fixed order.
constexpr int MAXS_LDS = 1024;
constexpr int VSCAN_BATCH = 16; // parts held in registers per thread
constexpr int VSCAN_RANGE = 32; // parts per range the launcher aims at

template <int P>
__global__ __launch_bounds__(64 * P) void k_segment_scan_varlen_heads(
    int r, int64_t H, int64_t num_seqs, int64_t parts, const int64_t* __restrict__ first,
    const float* __restrict__ S0, const float* __restrict__ z0, float* __restrict__ ws,
    int prefix_stride, float* __restrict__ S_fin, float* __restrict__ z_fin) {
    __shared__ int first_s[MAXS_LDS + 1]; // part indices (the host keeps parts below 2^31)
    __shared__ float tail_s[P][64];
    __shared__ int restart_s[P];
    for (int i = threadIdx.x; i <= num_seqs; i += 64 * P) first_s[i] = (int)first[i];
    __syncthreads();
    const int ns = (int)num_seqs;
    const int64_t E = state_elems(r);
    const int64_t bpe = (E + 63) / 64;
    const int64_t h = blockIdx.x / bpe;
    const int el = threadIdx.x & 63;
    const int part = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t e = (blockIdx.x % bpe) * 64 + el;
    const bool live = e < E;
    const int64_t ec = live ? e : E - 1; // in-bounds element for the loads
    const int64_t rdv = (int64_t)r * DV;
    auto start = [&](int i) -> float {
        if (!S0) return 0.f;
        const int64_t sh = (int64_t)i * H + h;
        return ec < rdv ? S0[sh * rdv + ec] : z0[sh * r + (ec - rdv)];
    };
    auto finish = [&](int i, float v) {
        if (!live) return;
        const int64_t sh = (int64_t)i * H + h;
        if (e < rdv)
            S_fin[sh * rdv + e] = v;
        else
            z_fin[sh * r + (e - rdv)] = v;
    };
    // the sequence whose parts hold part g (the last i with first[i] <= g:
    // sequences without parts end where they start)
    auto seq_of = [&](int g) {
        int lo = 0, hi = ns - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (first_s[mid] <= g) lo = mid; else hi = mid - 1;
        }
        return lo;
    };
    const int Pn = (int)min<int64_t>(first_s[ns], parts); // parts in use
    const int per = (Pn + P - 1) / P;
    const int g0 = min(Pn, part * per), g1 = min(Pn, g0 + per);
    const float* base = ws + h * parts * E + ec;
    auto at = [&](int g) { return base + (int64_t)g * E; };
    const int n0 = min(VSCAN_BATCH, g1 - g0);
    // every load unconditional: clamped to the range's first part (part 0
    // for an empty range); the values past n0 are not used
    const int gl = g1 > g0 ? g0 : 0;
    float a[VSCAN_BATCH];
#pragma unroll
    for (int j = 0; j < VSCAN_BATCH; ++j) a[j] = *at(gl + (j < n0 ? j : 0));
    // the range's last sequence: its parts within the range, from its
    // starting state when it starts here
    float tail = 0.f, start_last = 0.f;
    int restart = 0, il = -1;
    if (g1 > g0) {
        il = seq_of(g1 - 1);
        const int fl = first_s[il];
        restart = fl >= g0;
        start_last = restart ? start(il) : 0.f;
        tail = start_last;
#pragma unroll
        for (int j = 0; j < VSCAN_BATCH; ++j)
            if (j < n0 && g0 + j >= fl) tail += a[j];
        for (int g = max(g0 + VSCAN_BATCH, fl); g < g1; ++g) tail += *at(g);
    }
    wait_all_loads(); // else each prefix store below waits for the ones before it
    if (P > 1) {
        tail_s[part][el] = tail;
        if (el == 0) restart_s[part] = restart;
        __syncthreads();
    }
    // the carry into this range, ranges in order
    float carry = 0.f;
    for (int u = 0; u < part; ++u) carry = restart_s[u] ? tail_s[u][el] : carry + tail_s[u][el];
    // sequences without parts end with their starting state (a share of them
    // per range)
    for (int i = part; i < ns; i += P)
        if (first_s[i + 1] <= first_s[i]) finish(i, start(i));
    if (g1 <= g0) return;
    // S0 and S_fin may be one buffer (the state updated in place), and a
    // document's final state is written by the range holding its last part:
    // so a range takes the starting state of its last document (the only one
    // that can end in another range) from the read before the barrier; any
    // other document it starts also ends in it, read before written by this
    // thread
    auto start_of = [&](int i) { return i == il ? start_last : start(i); };
    int i = seq_of(g0), seq_first = first_s[i], seq_end = first_s[i + 1];
    float run = seq_first == g0 ? start_of(i) : carry;
    const int pmask = prefix_stride - 1;
    auto visit = [&](int g, float x) {
        if (live && prefix_stride > 0 && ((g - seq_first) & pmask) == 0)
            *const_cast<float*>(at(g)) = run;
        run += x;
        if (g + 1 >= seq_end) { // last part of sequence i
            finish(i, run);
            if (g + 1 < g1) { // the next sequence with parts starts at g + 1
                i = seq_of(g + 1);
                seq_first = first_s[i];
                seq_end = first_s[i + 1];
                run = start_of(i);
            }
        }
    };
#pragma unroll
    for (int j = 0; j < VSCAN_BATCH; ++j)
        if (j < n0) visit(g0 + j, a[j]);
    for (int g = g0 + VSCAN_BATCH; g < g1; ++g) visit(g, *at(g));
}

// ---------------------------------------------------------------------------
// Segment outputs.  CAUSAL: chunked recurrence from the carried-in state;
// otherwise: readout of every token against the full summary.
// ---------------------------------------------------------------------------
// PROJ: q, k and v are projected from the tokens x (proj.hpp) instead of read.
template <typename T, int FPT, bool CAUSAL, bool PROJ>
__global__ __launch_bounds__(NT) void k_segment_outputs(Cfg c, const T* __restrict__ q,
                                                        const T* __restrict__ k,
                                                        const T* __restrict__ v,
                                                        const T* __restrict__ omega, int64_t N,
                                                        int64_t G, int64_t seg_len,
                                                        const int64_t* __restrict__ tab, int64_t sub,
                                                        const float* __restrict__ state,
                                                        int64_t st_bh, int64_t st_g,
                                                        T* __restrict__ out, Proj P) {
    // The state S (r x 64 floats) lives in LDS: 32-token chunks up to
    // r = 256, 16 up to r = 384 and 4 up to r = 512 keep the state, the two
    // feature tiles and the chunk within the CU's 160 KB.  The result does
    // not depend on the chunk length beyond rounding.
    constexpr int L = FPT <= 8 ? 32 : (FPT <= 12 ? 16 : 4);
    constexpr int R = 32 * FPT;
    constexpr int OL = R + 4;
    constexpr int LC = CAUSAL ? L : 1;
    __shared__ float S_s[R * DV];
    __shared__ float z_s[R];
    __shared__ float pq_s[L * OL];
    __shared__ float pk_s[LC * OL];
    __shared__ float v_s[LC * DV];
    __shared__ float a_s[LC * (L + 1)];
    __shared__ float u_s[L * D];
    __shared__ float nrm_s[L], rs_s[L];
    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x / G, g = blockIdx.x % G;
    int64_t t0, t1;
    seg_range(tab, sub, g, seg_len, N, t0, t1);

    const float* sin = state + bh * st_bh + g * st_g;
    for (int e = tid; e < R * DV; e += NT) S_s[e] = sin[e];
    for (int f = tid; f < R; f += NT) z_s[f] = sin[R * DV + f];

    // readout thread mapping: token t = tid / 8, value columns nb*8 .. nb*8+7
    const int rt = tid / 8, nb = tid % 8;
    // update thread mapping: features fb*FPT + i, value columns nb*8 + j
    const int fb = tid / 8;

    for (int64_t c0 = t0; c0 < t1; c0 += L) {
        const int rows = (int)min<int64_t>(L, t1 - c0);
        if (CAUSAL) {
            if constexpr (PROJ) {
                project_chunk<L>(P, bh, N, c0, rows, PROJ_K, u_s, c.scale, PROJ_V, v_s, 1.f);
            } else {
                load_rows<T, L>(k + (bh * N + c0) * D, rows, c.scale, u_s);
                load_rows<T, L>(v + (bh * N + c0) * DV, rows, 1.f, v_s);
            }
            __syncthreads();
            row_norms<L>(u_s, nrm_s);
            __syncthreads();
            phi_tile<T, L>(c, u_s, nrm_s, omega, rows, pk_s, OL, rs_s);
        }
        if constexpr (PROJ)
            project_chunk<L>(P, bh, N, c0, rows, PROJ_Q, u_s, c.scale, -1, nullptr, 0.f);
        else
            load_rows<T, L>(q + (bh * N + c0) * D, rows, c.scale, u_s);
        __syncthreads();
        row_norms<L>(u_s, nrm_s);
        __syncthreads();
        phi_tile<T, L>(c, u_s, nrm_s, omega, rows, pq_s, OL, rs_s);

        if (CAUSAL) {
            // masked intra-chunk block a[t][j] = phi(q_t) . phi(k_j), j <= t
            for (int p = tid; p < L * L; p += NT) {
                const int t = p % L, j = p / L;
                float a = 0.f;
                if (j <= t) {
                    const float* x = pq_s + t * OL;
                    const float* y = pk_s + j * OL;
                    for (int f = 0; f < R; f += 4) {
                        a = fmaf(x[f], y[f], a);
                        a = fmaf(x[f + 1], y[f + 1], a);
                        a = fmaf(x[f + 2], y[f + 2], a);
                        a = fmaf(x[f + 3], y[f + 3], a);
                    }
                }
                a_s[t * (L + 1) + j] = a;
            }
            __syncthreads();
        }

        // readout against the carried-in state, plus the intra-chunk block
        // (threads of tokens rt >= L, when L < 32, have no row)
        if (rt < L) {
            float num[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) num[j] = 0.f;
            float den = 0.f;
            const float* x = pq_s + rt * OL;
            for (int f = 0; f < R; ++f) {
                const float pf = x[f];
                den = fmaf(pf, z_s[f], den);
                const float* srow = S_s + f * DV + nb * 8;
#pragma unroll
                for (int j = 0; j < 8; ++j) num[j] = fmaf(pf, srow[j], num[j]);
            }
            if (CAUSAL) {
                for (int jj = 0; jj <= rt; ++jj) {
                    const float a = a_s[rt * (L + 1) + jj];
                    den += a;
                    const float* vrow = v_s + jj * DV + nb * 8;
#pragma unroll
                    for (int j = 0; j < 8; ++j) num[j] = fmaf(a, vrow[j], num[j]);
                }
            }
            if (rt < rows) {
                T* o = out + (bh * N + c0 + rt) * DV + nb * 8;
                const float inv = c.norm == NORM_ATTN ? 1.f / fmaxf(den, c.eps) : 1.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float y = c.norm == NORM_ATTN ? num[j] * inv : num[j];
                    Elem<T>::store(o, j, y);
                }
            }
        }

        if (CAUSAL) {
            __syncthreads(); // every read of S_s / z_s for this chunk is done
#pragma unroll
            for (int i = 0; i < FPT; ++i) {
                const int f = fb * FPT + i;
                float s[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) s[j] = S_s[f * DV + nb * 8 + j];
                float zf = 0.f;
                for (int t = 0; t < rows; ++t) {
                    const float p = pk_s[t * OL + f];
                    zf += p;
                    const float* vrow = v_s + t * DV + nb * 8;
#pragma unroll
                    for (int j = 0; j < 8; ++j) s[j] = fmaf(p, vrow[j], s[j]);
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) S_s[f * DV + nb * 8 + j] = s[j];
                if (nb == 0) z_s[f] += zf;
            }
        }
        __syncthreads();
    }
}

template <typename T>
hipError_t featuremap_t(const Cfg& c, const void* x, const void* omega, Shape s, float* phi,
                        hipStream_t st) {
    const int64_t tiles = (s.N + 31) / 32;
    hipLaunchKernelGGL(k_featuremap<T>, dim3((unsigned)(tiles * s.BH)), dim3(NT), 0, st, c,
                       (const T*)x, (const T*)omega, s.N, tiles, phi);
    return hipGetLastError();
}

template <typename T, int FPT, bool PROJ>
void sums_fpt(const Cfg& c, const void* k, const void* v, const void* omega, Shape s, SegPlan sp,
              float* ws, const Proj& P, hipStream_t st) {
    hipLaunchKernelGGL((k_segment_sums<T, FPT, PROJ>), dim3((unsigned)(sp.G * s.BH)), dim3(NT), 0,
                       st, c, (const T*)k, (const T*)v, (const T*)omega, s.N, sp.G, sp.seg_len,
                       sp.tab, ws, P);
}

// The instance for r = 32 f (f = 1 .. 16; the projected kernels stop at 8).
template <typename T, bool PROJ, int F = 1>
hipError_t segment_sums_t(const Cfg& c, const void* k, const void* v, const void* omega, Shape s,
                          SegPlan sp, float* ws, const Proj& P, hipStream_t st) {
    if constexpr (F > (PROJ ? RMAX_BWD : RMAX) / 32) {
        return hipErrorInvalidValue;
    } else {
        if (c.r != 32 * F) return segment_sums_t<T, PROJ, F + 1>(c, k, v, omega, s, sp, ws, P, st);
        sums_fpt<T, F, PROJ>(c, k, v, omega, s, sp, ws, P, st);
        return hipGetLastError();
    }
}

template <typename T, int FPT, bool PROJ>
void outputs_fpt(const Cfg& c, int causal, const void* q, const void* k, const void* v,
                 const void* omega, Shape s, SegPlan sp, const float* state, int64_t sbh,
                 int64_t sg, void* out, const Proj& P, hipStream_t st) {
    const dim3 grid((unsigned)(sp.G * s.BH)), block(NT);
    if (causal)
        hipLaunchKernelGGL((k_segment_outputs<T, FPT, true, PROJ>), grid, block, 0, st, c,
                           (const T*)q, (const T*)k, (const T*)v, (const T*)omega, s.N, sp.G,
                           sp.seg_len, sp.tab, sp.sub, state, sbh, sg, (T*)out, P);
    else
        hipLaunchKernelGGL((k_segment_outputs<T, FPT, false, PROJ>), grid, block, 0, st, c,
                           (const T*)q, (const T*)k, (const T*)v, (const T*)omega, s.N, sp.G,
                           sp.seg_len, sp.tab, sp.sub, state, sbh, sg, (T*)out, P);
}

template <typename T, bool PROJ, int F = 1>
hipError_t segment_outputs_t(const Cfg& c, int causal, const void* q, const void* k,
                             const void* v, const void* omega, Shape s, SegPlan sp,
                             const float* state, int64_t sbh, int64_t sg, void* out,
                             const Proj& P, hipStream_t st) {
    if constexpr (F > (PROJ ? RMAX_BWD : RMAX) / 32) {
        return hipErrorInvalidValue;
    } else {
        if (c.r != 32 * F)
            return segment_outputs_t<T, PROJ, F + 1>(c, causal, q, k, v, omega, s, sp, state, sbh,
                                                     sg, out, P, st);
        outputs_fpt<T, F, PROJ>(c, causal, q, k, v, omega, s, sp, state, sbh, sg, out, P, st);
        return hipGetLastError();
    }
}

__global__ __launch_bounds__(NT) void k_fill_zero(float* __restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT)
        p[i] = 0.f;
}

} // namespace

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + NT - 1) / NT, 4096);
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(NT), 0, st, p, n);
    return hipGetLastError();
}

hipError_t launch_featuremap(const Cfg& c, int dtype, const void* x, const void* omega, Shape s,
                             float* phi, hipStream_t st) {
    return dtype == 0 ? featuremap_t<float>(c, x, omega, s, phi, st)
                      : featuremap_t<bf16_raw>(c, x, omega, s, phi, st);
}

hipError_t launch_segment_sums(const Cfg& c, int dtype, const void* k, const void* v,
                               const void* omega, Shape s, SegPlan sp, float* ws, hipStream_t st) {
    const Proj none{};
    return dtype == 0 ? segment_sums_t<float, false>(c, k, v, omega, s, sp, ws, none, st)
                      : segment_sums_t<bf16_raw, false>(c, k, v, omega, s, sp, ws, none, st);
}

hipError_t launch_segment_sums_proj(const Cfg& c, const Proj& P, const void* omega, Shape s,
                                    SegPlan sp, float* ws, hipStream_t st) {
    return segment_sums_t<bf16_raw, true>(c, nullptr, nullptr, omega, s, sp, ws, P, st);
}

template <bool REV, int P>
void segment_scan_p(int r, Shape s, int64_t G, const float* S0, const float* z0, float* ws,
                    int prefix_stride, float* S_fin, float* z_fin, float* fin, hipStream_t st) {
    const int64_t epb = NT / P;
    const dim3 grid((unsigned)(((state_elems(r) + epb - 1) / epb) * s.BH));
    hipLaunchKernelGGL((k_segment_scan<REV, P>), grid, dim3(NT), 0, st, r, G, S0, z0, ws,
                       prefix_stride, S_fin, z_fin, fin);
}

// ranges of at most SCAN_BATCH segments where that takes at most 4 of them
template <bool REV>
hipError_t segment_scan(int r, Shape s, int64_t G, const float* S0, const float* z0, float* ws,
                        int prefix_stride, float* S_fin, float* z_fin, float* fin,
                        hipStream_t st) {
    if (G > 2 * SCAN_BATCH)
        segment_scan_p<REV, 4>(r, s, G, S0, z0, ws, prefix_stride, S_fin, z_fin, fin, st);
    else if (G > SCAN_BATCH)
        segment_scan_p<REV, 2>(r, s, G, S0, z0, ws, prefix_stride, S_fin, z_fin, fin, st);
    else
        segment_scan_p<REV, 1>(r, s, G, S0, z0, ws, prefix_stride, S_fin, z_fin, fin, st);
    return hipGetLastError();
}

hipError_t launch_segment_scan(int r, Shape s, SegPlan sp, const float* S0, const float* z0,
                               float* ws, int prefix_stride, float* S_fin, float* z_fin,
                               float* fin, hipStream_t st) {
    return segment_scan<false>(r, s, sp.G, S0, z0, ws, prefix_stride, S_fin, z_fin, fin, st);
}

hipError_t launch_segment_suffix_scan(int r, Shape s, SegPlan sp, float* ws, hipStream_t st) {
    return segment_scan<true>(r, s, sp.G, nullptr, nullptr, ws, 1, nullptr, nullptr, nullptr, st);
}

hipError_t launch_varlen_plan(const int32_t* cu_seqlens, int64_t num_seqs, int64_t total,
                              int64_t seg_len, int64_t sub, int64_t cap, int64_t* tab,
                              int64_t* first, int64_t* order, hipStream_t st) {
    hipLaunchKernelGGL(k_varlen_plan, dim3(1), dim3(NT), 0, st, cu_seqlens, num_seqs, total,
                       seg_len, sub, cap, tab, first, order);
    return hipGetLastError();
}

hipError_t launch_segment_scan_varlen(int r, int64_t H, int64_t num_seqs, int64_t parts,
                                      const int64_t* first, const float* S0, const float* z0,
                                      float* ws, int prefix_stride, float* S_fin, float* z_fin,
                                      hipStream_t st) {
    const int64_t E = state_elems(r);
    if (num_seqs <= MAXS_LDS && parts < ((int64_t)1 << 30)) {
        // ranges of at most VSCAN_RANGE parts where that takes at most 16 of them
        // (shorter ranges measured slower: more waves, each with the same
        // fixed work)
        auto go = [&](auto kernel, int p) {
            const dim3 grid((unsigned)(((E + 63) / 64) * H));
            hipLaunchKernelGGL(kernel, grid, dim3(64 * p), 0, st, r, H, num_seqs, parts, first, S0,
                               z0, ws, prefix_stride, S_fin, z_fin);
        };
        if (parts > 8 * VSCAN_RANGE)
            go(k_segment_scan_varlen_heads<16>, 16);
        else if (parts > 4 * VSCAN_RANGE)
            go(k_segment_scan_varlen_heads<8>, 8);
        else if (parts > 2 * VSCAN_RANGE)
            go(k_segment_scan_varlen_heads<4>, 4);
        else if (parts > VSCAN_RANGE)
            go(k_segment_scan_varlen_heads<2>, 2);
        else
            go(k_segment_scan_varlen_heads<1>, 1);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)(((E + NT - 1) / NT) * H * num_seqs));
    hipLaunchKernelGGL(k_segment_scan_varlen, grid, dim3(NT), 0, st, r, H, parts, first, S0, z0, ws,
                       prefix_stride, S_fin, z_fin);
    return hipGetLastError();
}

hipError_t launch_segment_outputs(const Cfg& c, int dtype, int causal, const void* q,
                                  const void* k, const void* v, const void* omega, Shape s,
                                  SegPlan sp, const float* state, int64_t sbh, int64_t sg,
                                  void* out, hipStream_t st) {
    const Proj none{};
    return dtype == 0 ? segment_outputs_t<float, false>(c, causal, q, k, v, omega, s, sp, state,
                                                        sbh, sg, out, none, st)
                      : segment_outputs_t<bf16_raw, false>(c, causal, q, k, v, omega, s, sp,
                                                           state, sbh, sg, out, none, st);
}

hipError_t launch_segment_outputs_proj(const Cfg& c, int causal, const Proj& P, const void* omega,
                                       Shape s, SegPlan sp, const float* state, int64_t sbh,
                                       int64_t sg, void* out, hipStream_t st) {
    return segment_outputs_t<bf16_raw, true>(c, causal, nullptr, nullptr, nullptr, omega, s, sp,
                                             state, sbh, sg, out, P, st);
}

} // namespace linattn
