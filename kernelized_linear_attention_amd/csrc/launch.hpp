// launch.hpp -- host-side launchers of the kernels, called by the C ABI layer
// after it has validated every argument.  All sizes are already known to be
// in range; each launcher only enqueues work on `st` and reports the launch
// status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "proj.hpp"

namespace linattn {

// Sequence segmentation used by the parallel scan: G segments of seg_len
// tokens per head (the last may be shorter); every segment boundary is a
// multiple of SEG_UNIT tokens.
constexpr int64_t SEG_UNIT = 64;
constexpr int64_t TARGET_BLOCKS_VALU = 512; // vector kernels: about two workgroups per CU
constexpr int64_t TARGET_BLOCKS_MFMA = 512; // matrix-core kernels: two workgroups per CU
constexpr int64_t TARGET_BLOCKS_BWD_CAUSAL_MFMA = 256; // causal backward passes: one per CU

struct SegPlan {
    int64_t G;       // segments per head (one workgroup each for the outputs)
    int64_t seg_len; // tokens per segment
    int64_t sub;     // the state increments are summed over seg_len / sub tokens
    // Segment table (device), or NULL for uniform segments: part e covers
    // tokens [tab[2e], tab[2e+1]) of every head and segment g is parts
    // g*sub .. g*sub + sub - 1 (packed sequences, see launch_varlen_plan).
    const int64_t* tab = nullptr;
    // Dispatch order of the segments (matrix-core kernels, packed sequences):
    // workgroup b runs segment order[b / heads] of head b % heads (-1: none),
    // longest segments first.  NULL: head-major, segment g = b % G.
    const int64_t* order = nullptr;
    int64_t osub = 1; // parts per entry of `order` (the increment kernels run parts)
};

// The plan of the increment and prefix kernels: sub-segments as segments.
inline SegPlan sums_plan(SegPlan p) {
    return SegPlan{p.G * p.sub, p.seg_len / p.sub, 1, p.tab, p.order, p.sub};
}

inline SegPlan plan_segments(int64_t BH, int64_t N, int32_t n_seg_req, int64_t target_blocks) {
    SegPlan p{1, N, 1};
    if (N <= 0 || BH <= 0) return p;
    const int64_t units = (N + SEG_UNIT - 1) / SEG_UNIT;
    int64_t G = n_seg_req > 0 ? n_seg_req : (target_blocks + BH - 1) / BH;
    if (G < 1) G = 1;
    if (G > units) G = units;
    const int64_t per = (units + G - 1) / G;
    p.G = (units + per - 1) / per;
    p.seg_len = per * SEG_UNIT;
    return p;
}

// Elements of one (S | z) state block: r*dv floats of S followed by r of z.
__host__ __device__ inline int64_t state_elems(int r) { return (int64_t)r * DV + r; }

// Token range [t0, t1) of segment g of a head with N tokens (see SegPlan).
__device__ __forceinline__ void seg_range(const int64_t* tab, int64_t sub, int64_t g,
                                          int64_t seg_len, int64_t N, int64_t& t0, int64_t& t1) {
    if (tab) {
        t0 = tab[2 * g * sub];
        t1 = tab[2 * (g * sub + sub - 1) + 1];
    } else {
        t0 = g * seg_len;
        t1 = t0 + seg_len < N ? t0 + seg_len : N;
    }
}

struct Shape {
    int64_t BH; // batch * heads
    int64_t N;  // tokens per head
};

// dtype-erased launchers (T is float or bf16_raw inside)
hipError_t launch_featuremap(const Cfg& c, int dtype, const void* x, const void* omega, Shape s,
                             float* phi, hipStream_t st);

// State increments of every segment: ws[bh][g] = sum over the segment of
// phi(k_j) v_j^T (then z).
hipError_t launch_segment_sums(const Cfg& c, int dtype, const void* k, const void* v,
                               const void* omega, Shape s, SegPlan sp, float* ws, hipStream_t st);

// Prefix over segments.  Reads S0/z0 (may be NULL = zero), overwrites
// ws[bh][g] with the exclusive prefix for every g that is a multiple of
// prefix_stride (a power of two; none when 0), and writes the total to
// S_fin / z_fin / fin (each may be NULL).
hipError_t launch_segment_scan(int r, Shape s, SegPlan sp, const float* S0, const float* z0,
                               float* ws, int prefix_stride, float* S_fin, float* z_fin,
                               float* fin, hipStream_t st);

// Exclusive suffix over segments: overwrites ws[bh][g] with the sum of
// ws[bh][g+1 ..] (zero for the last segment), in a fixed order.
hipError_t launch_segment_suffix_scan(int r, Shape s, SegPlan sp, float* ws, hipStream_t st);

// Outputs of every segment.  causal: chunked recurrence from the segment's
// carried-in state ws[bh][g]; bidirectional: readout against the full
// summary fin[bh].
hipError_t launch_segment_outputs(const Cfg& c, int dtype, int causal, const void* q,
                                  const void* k, const void* v, const void* omega, Shape s,
                                  SegPlan sp, const float* state, int64_t state_bh_stride,
                                  int64_t state_g_stride, void* out, hipStream_t st);

// The same two kernels with q, k, v projected from the tokens P.x through
// P.w (proj.hpp) inside their loads; bfloat16 only.
hipError_t launch_segment_sums_proj(const Cfg& c, const Proj& P, const void* omega, Shape s,
                                    SegPlan sp, float* ws, hipStream_t st);
hipError_t launch_segment_outputs_proj(const Cfg& c, int causal, const Proj& P, const void* omega,
                                       Shape s, SegPlan sp, const float* state, int64_t sbh,
                                       int64_t sg, void* out, hipStream_t st);

// q, k, v [B, H, N, 64] (bf16) = the tokens x [B, N, dm] times W_q, W_k, W_v
// [H*64, dm] transposed: one matrix-core GEMM (project.hip).
hipError_t launch_qkv_project(const void* x, const void* w_q, const void* w_k, const void* w_v,
                              int64_t B, int64_t N, int64_t dm, int64_t H, void* q, void* k,
                              void* v, hipStream_t st);

// Segment table of a packed batch: sequence i covers tokens
// [cu_seqlens[i], cu_seqlens[i+1]) of every head and is cut into
// ceil(len / seg_len) segments of `sub` parts of seg_len / sub tokens (tail
// parts may be empty).  Writes tab[2e], tab[2e+1] for the cap parts (unused
// ones empty), first[i] = first part of sequence i (first[num_seqs] = parts
// used) and the dispatch order of the cap / sub segments (see SegPlan).
// Ranges are clamped to [0, total] and the count to cap, so malformed
// boundaries cannot send a later kernel out of bounds.  One workgroup.
hipError_t launch_varlen_plan(const int32_t* cu_seqlens, int64_t num_seqs, int64_t total,
                              int64_t seg_len, int64_t sub, int64_t cap, int64_t* tab,
                              int64_t* first, int64_t* order, hipStream_t st);

// Prefix over the parts of every (sequence, head): parts first[i] ..
// first[i+1]-1 of head h in ws[h][.], starting from S0/z0[(i*H + h)] (or
// zero), exclusive prefix written at every prefix_stride-th part of the
// sequence, final state to S_fin/z_fin[(i*H + h)].
hipError_t launch_segment_scan_varlen(int r, int64_t H, int64_t num_seqs, int64_t parts,
                                      const int64_t* first, const float* S0, const float* z0,
                                      float* ws, int prefix_stride, float* S_fin, float* z_fin,
                                      hipStream_t st);

// Backward pass (backward.hip), vector kernels, every feature map.
// Query pass: from the forward state of each segment (causal: carried-in
// prefix ws_f[bh][g]; bidirectional: total fin_f[bh]) it writes dq and the
// segment increments ws_b[bh][g] = (sum phi(q_i) dnum_i^T, sum phi(q_i) dden_i);
// causal also writes tok[bh][t] = (1 / max(den_t, eps) or 1, dden_t).
// Key pass: from the backward state of each segment (causal: exclusive
// suffix ws_b[bh][g], chunks walked last to first; bidirectional: total
// fin_b[bh]) it writes dk and dv.
// omega_t: omega^T [64][r] in bfloat16 (launch_transpose_omega) for bfloat16
// FAVOR+ inputs, which then use the matrix-core contractions; else NULL.
hipError_t launch_transpose_omega(const void* omega, int r, void* omega_t, hipStream_t st);
hipError_t launch_backward_query(const Cfg& c, int dtype, int causal, const void* q,
                                 const void* k, const void* v, const void* dout, const void* omega,
                                 Shape s, SegPlan sp, const float* state, int64_t sbh, int64_t sg,
                                 const void* omega_t, float* inc, float* tok, void* dq,
                                 hipStream_t st);
hipError_t launch_backward_key(const Cfg& c, int dtype, int causal, const void* q, const void* k,
                               const void* v, const void* dout, const void* omega, Shape s,
                               SegPlan sp, const float* state, int64_t sbh, int64_t sg,
                               const void* omega_t, const float* tok, void* dk, void* dv,
                               hipStream_t st);

// p[0, n) = 0 with a plain kernel (capturable into a graph).
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st);

// Matrix-core path for FAVOR+ with bfloat16 inputs and r = 256 (favor_mfma.hip);
// same workspace layout and segment scan as the vector path.
bool favor_mfma_supported(const Cfg& c, int dtype);
// zw: optional per-token weights [BH, N] of the z sum (z = sum_t w_t phi(k_t));
// NULL gives the plain sum.
// float32 matrix-core kernels (mfma_f32.hip): identity and ELU+1 at r = 64,
// DPFP at r = 128 and 256, float32 or bfloat16 inputs
bool f32mm_supported(const Cfg& c);
hipError_t launch_f32mm_sums(const Cfg& c, int dtype, const void* k, const void* v, Shape s,
                             SegPlan sp, float* ws, hipStream_t st);
hipError_t launch_f32mm_outputs(const Cfg& c, int dtype, int causal, const void* q, const void* k,
                                const void* v, Shape s, SegPlan sp, const float* state,
                                int64_t sbh, int64_t sg, void* out, hipStream_t st);
hipError_t launch_favor_sums(const Cfg& c, const void* k, const void* v, const void* omega,
                             Shape s, SegPlan sp, float* ws, hipStream_t st,
                             const float* zw = nullptr);
// Bidirectional readout from the per-head totals (S | z) at total + bh * st_bh.
hipError_t launch_favor_readout(const Cfg& c, const void* q, const void* omega, Shape s,
                                const float* total, int64_t st_bh, void* out, hipStream_t st);
// Causal outputs of every segment from its carried-in state.
hipError_t launch_favor_outputs(const Cfg& c, const void* q, const void* k, const void* v,
                                const void* omega, Shape s, SegPlan sp, const float* state,
                                int64_t sbh, int64_t sg, void* out, hipStream_t st);

// Backward of the bidirectional form on the matrix cores (FAVOR+, bfloat16,
// r = 256): total = the head's (S | z) for the query pass, (G | g) for the key
// pass.  The query pass also writes dnum (bf16 [BH, N, DV]) and dden
// (float [BH, N]), from which the increment kernel (with z weights dden)
// forms (G | g).
hipError_t launch_favor_bwd_query(const Cfg& c, const void* q, const void* dout, const void* omega,
                                  Shape s, SegPlan sp, const float* total, void* dq, void* dnum,
                                  float* dden, hipStream_t st);
hipError_t launch_favor_bwd_key(const Cfg& c, const void* k, const void* v, const void* omega,
                                Shape s, SegPlan sp, const float* total, void* dk, void* dv,
                                hipStream_t st);

// Causal backward on the matrix cores (same configuration): the query pass
// from each segment's forward prefix writes dq, dnum (bf16 [BH, N, DV]) and
// dden (float [BH, N]), from which the increment kernel (with z weights dden)
// forms the segments' backward increments; the key pass from each segment's
// backward suffix writes dk and dv.
hipError_t launch_favor_causal_bwd_query(const Cfg& c, const void* q, const void* k, const void* v,
                                         const void* dout, const void* omega, Shape s, SegPlan sp,
                                         const float* prefix, int64_t sbh, int64_t sg, void* dnum,
                                         float* dden, void* dq, hipStream_t st);
hipError_t launch_favor_causal_bwd_key(const Cfg& c, const void* q, const void* k, const void* v,
                                       const void* omega, Shape s, SegPlan sp, const float* suffix,
                                       int64_t sbh, int64_t sg, const void* dnum, const float* dden,
                                       void* dk, void* dv, hipStream_t st);

// Orthogonal random features (orf.hip): n_mat matrices [r, d], d <= 64.
hipError_t launch_orf(const float* gauss, const float* len_gauss, int64_t n_mat, int64_t r, int d,
                      int dtype, void* omega, hipStream_t st);

hipError_t launch_decode(const Cfg& c, int dtype, const void* q, const void* k, const void* v,
                         const void* omega, int64_t BH, float* S, float* z, void* out,
                         hipStream_t st);

} // namespace linattn
