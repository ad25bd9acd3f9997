// abi.hip -- the extern "C" entry points of liblinattn.so (include/lin_attn.h):
// argument validation, segmentation plan, workspace layout and dispatch.
// Validation happens entirely on the host, before anything is enqueued.
#include <math.h>

#include <atomic>

#include "../../include/lin_attn.h"
#include "launch.hpp"

using namespace linattn;

namespace {

bool ptr_ok(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool opt_ptr_ok(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// INVALID checks, then GPU-coverage checks (UNSUPPORTED).
int check_params(const lin_attn_params* p, int64_t d, int64_t dv, const void* omega) {
    if (!p) return LIN_ATTN_ERR_INVALID;
    if (p->reserved != 0) return LIN_ATTN_ERR_INVALID;
    if (p->phi < LIN_ATTN_PHI_IDENTITY || p->phi > LIN_ATTN_PHI_DPFP) return LIN_ATTN_ERR_INVALID;
    if (p->norm != LIN_ATTN_NORM_ATTN && p->norm != LIN_ATTN_NORM_NONE) return LIN_ATTN_ERR_INVALID;
    if (p->dtype != LIN_ATTN_F32 && p->dtype != LIN_ATTN_BF16) return LIN_ATTN_ERR_INVALID;
    if (p->sum_norm != 0 && p->sum_norm != 1) return LIN_ATTN_ERR_INVALID;
    if (!(p->eps > 0.f) || !isfinite(p->eps) || !isfinite(p->scale)) return LIN_ATTN_ERR_INVALID;
    if (p->n_seg < 0) return LIN_ATTN_ERR_INVALID;
    if (d <= 0 || dv <= 0 || p->r <= 0) return LIN_ATTN_ERR_INVALID;
    switch (p->phi) {
    case LIN_ATTN_PHI_IDENTITY:
    case LIN_ATTN_PHI_ELU1:
        if (p->r != d) return LIN_ATTN_ERR_INVALID;
        break;
    case LIN_ATTN_PHI_DPFP:
        if (p->nu < 1 || p->nu > 2 * d - 1) return LIN_ATTN_ERR_INVALID;
        if ((int64_t)p->r != 2 * d * p->nu) return LIN_ATTN_ERR_INVALID;
        break;
    case LIN_ATTN_PHI_FAVOR:
        if (!ptr_ok(omega)) return LIN_ATTN_ERR_INVALID;
        break;
    }
    if (d != D || dv != DV) return LIN_ATTN_ERR_UNSUPPORTED;
    if (p->r % 32 != 0 || p->r > RMAX) return LIN_ATTN_ERR_UNSUPPORTED;
    return LIN_ATTN_OK;
}

Cfg make_cfg(const lin_attn_params* p) {
    Cfg c;
    c.phi = p->phi;
    c.r = p->r;
    c.nu = p->nu;
    c.sum_norm = p->sum_norm;
    c.norm = p->norm;
    c.scale = p->scale;
    c.eps = p->eps;
    c.favor_log2_bias = -0.5f * log2f((float)p->r);
    return c;
}

int check_sizes(int64_t B, int64_t H, int64_t N) {
    if (B < 0 || H < 0 || N < 0) return LIN_ATTN_ERR_INVALID;
    // grid sizes are unsigned 32-bit; keep every flattened grid in range
    if (B > 0 && H > (((int64_t)1 << 31) / B)) return LIN_ATTN_ERR_UNSUPPORTED;
    if (B * H > ((int64_t)1 << 24) || N > ((int64_t)1 << 40)) return LIN_ATTN_ERR_UNSUPPORTED;
    return LIN_ATTN_OK;
}

// Workspace layout (float32):
//   [0, BH*G*E)            per-segment state increments, then carried-in states
//   [BH*G*E, +BH*E)        bidirectional only: the full summary per head
size_t ws_floats(int32_t op, int64_t BH, SegPlan sp, int r) {
    const int64_t E = state_elems(r);
    size_t n = (size_t)(BH * sp.G * sp.sub * E);
    if (op == LIN_ATTN_OP_BIDIR) n += (size_t)(BH * E);
    return n;
}

int launch_status(hipError_t e) { return e == hipSuccess ? LIN_ATTN_OK : LIN_ATTN_ERR_HIP; }

// The kernel family a validated call runs on, and its segmentation.
bool use_mfma(const lin_attn_params* p) { return favor_mfma_supported(make_cfg(p), p->dtype); }

// Both matrix-core kernels (increments and outputs) fit two workgroups per
// CU: the increments are summed over whole segments.
SegPlan plan_for(const lin_attn_params* p, int64_t BH, int64_t N) {
    return plan_segments(BH, N, p->n_seg, use_mfma(p) ? TARGET_BLOCKS_MFMA : TARGET_BLOCKS_VALU);
}

hipError_t segment_sums(const lin_attn_params* p, const Cfg& c, const void* k, const void* v,
                        const void* omega, Shape s, SegPlan sp, float* ws, hipStream_t st) {
    if (use_mfma(p)) return launch_favor_sums(c, k, v, omega, s, sp, ws, st);
    if (f32mm_supported(c)) return launch_f32mm_sums(c, p->dtype, k, v, s, sp, ws, st);
    return launch_segment_sums(c, p->dtype, k, v, omega, s, sp, ws, st);
}

hipError_t segment_outputs(const lin_attn_params* p, const Cfg& c, int causal, const void* q,
                           const void* k, const void* v, const void* omega, Shape s, SegPlan sp,
                           const float* state, int64_t sbh, int64_t sg, void* out,
                           hipStream_t st) {
    if (use_mfma(p) && causal)
        return launch_favor_outputs(c, q, k, v, omega, s, sp, state, sbh, sg, out, st);
    if (use_mfma(p)) return launch_favor_readout(c, q, omega, s, state, sbh, out, st);
    if (f32mm_supported(c))
        return launch_f32mm_outputs(c, p->dtype, causal, q, k, v, s, sp, state, sbh, sg, out, st);
    return launch_segment_outputs(c, p->dtype, causal, q, k, v, omega, s, sp, state, sbh, sg, out,
                                  st);
}

// Packed batch (lin_attn_causal_varlen): the uniform planner over all tokens
// of a head fixes the segment length; every sequence adds at most one
// partial segment, which bounds the segment table.  Workspace: increments
// (float32) [H][parts][E], then the table int64 [parts][2], the first part of
// every sequence int64 [num_seqs + 1] and the dispatch order of the segments
// int64 [segments].
struct VarlenLayout {
    SegPlan sp;        // G = segment capacity per head, seg_len, sub
    int64_t parts;     // table capacity (segments x sub)
    size_t tab_off, first_off, order_off, bytes;
};

VarlenLayout varlen_layout(const lin_attn_params* p, int64_t num_seqs, int64_t H, int64_t total) {
    VarlenLayout L;
    L.sp = plan_for(p, H, total);
    L.sp.G = (total + L.sp.seg_len - 1) / L.sp.seg_len + num_seqs;
    L.parts = L.sp.G * L.sp.sub;
    size_t off = (size_t)(H * L.parts * state_elems(p->r)) * sizeof(float);
    off = (off + 255) & ~(size_t)255;
    L.tab_off = off;
    off += (size_t)L.parts * 2 * sizeof(int64_t);
    L.first_off = off;
    off += (size_t)(num_seqs + 1) * sizeof(int64_t);
    L.order_off = off;
    off += (size_t)L.sp.G * sizeof(int64_t);
    L.bytes = off;
    return L;
}

// Backward pass (no increment halving).  Workspace (float32):
//   [0, BH*G*E)          forward increments, then prefixes (causal)
//   [BH*G*E, 2*BH*G*E)   backward increments, then suffixes (causal)
//   bidirectional: the forward and the backward totals, BH*E each, then
//     dnum (bf16, BH*N*DV) and dden (BH*N) for the matrix-core route;
//   causal: (1/D_t, dden_t) per token, BH*N*2;
//   then, 256-byte aligned, r*64 floats holding omega^T in bfloat16
//   (bfloat16 FAVOR+ on the vector kernels only).
struct BackwardLayout {
    SegPlan sp;
    size_t inc_b, extra, omega_t, floats;
};

BackwardLayout backward_layout(const lin_attn_params* p, bool causal, int64_t BH, int64_t N) {
    BackwardLayout L;
    // the causal matrix-core passes run one workgroup per CU: about one
    // segment per CU (at B=1, H=8, N=65536 this beat two per CU, 611 against
    // 632 us a call: the two scans move half the state)
    L.sp = plan_segments(BH, N, p->n_seg,
                         causal && use_mfma(p) ? TARGET_BLOCKS_BWD_CAUSAL_MFMA : TARGET_BLOCKS_VALU);
    const size_t inc = (size_t)(BH * L.sp.G * state_elems(p->r));
    L.inc_b = inc;
    L.extra = 2 * inc;
    // causal: per token dnum (bf16) and dden on the matrix-core route, two
    // floats on the vector route; bidirectional: the two totals, then dnum
    // and dden
    L.omega_t = L.extra + (causal ? (size_t)(BH * N) * (DV / 2 + 1)
                                  : (size_t)(2 * BH * state_elems(p->r)) +
                                        (size_t)(BH * N) * (DV / 2 + 1));
    L.omega_t = (L.omega_t + 63) & ~(size_t)63; // 256-byte aligned (read as 16-byte pieces)
    L.floats = L.omega_t + (size_t)p->r * D;
    return L;
}

int backward_call(bool causal, const lin_attn_params* p, const void* q, const void* k,
                  const void* v, const void* dout, int64_t B, int64_t H, int64_t N, int64_t d,
                  int64_t dv, const void* omega, void* dq, void* dk, void* dvv, void* ws,
                  size_t ws_bytes, void* stream) {
    int rc = check_params(p, d, dv, omega);
    if (rc == LIN_ATTN_ERR_INVALID) return rc;
    const int rs = check_sizes(B, H, N);
    if (rs == LIN_ATTN_ERR_INVALID) return rs;
    if (!opt_ptr_ok(ws)) return LIN_ATTN_ERR_INVALID;
    if (B * H > 0 && N > 0 &&
        (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(dout) || !ptr_ok(dq) || !ptr_ok(dk) ||
         !ptr_ok(dvv)))
        return LIN_ATTN_ERR_INVALID;
    if (rc != LIN_ATTN_OK) return rc;
    if (rs != LIN_ATTN_OK) return rs;
    if (p->r > RMAX_BWD) return LIN_ATTN_ERR_UNSUPPORTED;
    if (B * H == 0 || N == 0) return LIN_ATTN_OK; // no element to write
    const int64_t BH = B * H;
    const BackwardLayout L = backward_layout(p, causal, BH, N);
    if (ws_bytes < L.floats * sizeof(float) || !ws) return LIN_ATTN_ERR_WORKSPACE;

    const Cfg c = make_cfg(p);
    const Shape s{BH, N};
    const SegPlan sp = L.sp;
    hipStream_t st = (hipStream_t)stream;
    const int64_t E = state_elems(p->r);
    float* inc_f = (float*)ws;
    float* inc_b = inc_f + L.inc_b;
    float* extra = inc_f + L.extra;
    void* omega_t = nullptr;
    hipError_t e = segment_sums(p, c, k, v, omega, s, sp, inc_f, st);
    if (e == hipSuccess && p->phi == LIN_ATTN_PHI_FAVOR && p->dtype == LIN_ATTN_BF16 &&
        !use_mfma(p)) {
        omega_t = inc_f + L.omega_t;
        e = launch_transpose_omega(omega, p->r, omega_t, st);
    }
    if (causal && use_mfma(p)) {
        // matrix-core route: each workgroup walks its segment's chunks with the
        // evolving state in accumulators (forward order, then reverse); the
        // backward increments sum_t phi(q_t) (dnum_t, dden_t) per segment come
        // from the increment kernel on (q, dnum) with z weights dden
        void* dnum = extra;                                  // bf16 [BH, N, DV]
        float* dden = extra + (size_t)BH * N * (DV / 2);     // [BH, N]
        if (e == hipSuccess)
            e = launch_segment_scan(p->r, s, sp, nullptr, nullptr, inc_f, 1, nullptr, nullptr,
                                    nullptr, st);
        if (e == hipSuccess)
            e = launch_favor_causal_bwd_query(c, q, k, v, dout, omega, s, sp, inc_f, sp.G * E, E,
                                              dnum, dden, dq, st);
        if (e == hipSuccess) e = launch_favor_sums(c, q, dnum, omega, s, sp, inc_b, st, dden);
        if (e == hipSuccess) e = launch_segment_suffix_scan(p->r, s, sp, inc_b, st);
        if (e == hipSuccess)
            e = launch_favor_causal_bwd_key(c, q, k, v, omega, s, sp, inc_b, sp.G * E, E, dnum,
                                            dden, dk, dvv, st);
    } else if (causal) {
        if (e == hipSuccess)
            e = launch_segment_scan(p->r, s, sp, nullptr, nullptr, inc_f, 1, nullptr, nullptr,
                                    nullptr, st);
        if (e == hipSuccess)
            e = launch_backward_query(c, p->dtype, 1, q, k, v, dout, omega, s, sp, inc_f, sp.G * E,
                                      E, omega_t, inc_b, extra, dq, st);
        if (e == hipSuccess) e = launch_segment_suffix_scan(p->r, s, sp, inc_b, st);
        if (e == hipSuccess)
            e = launch_backward_key(c, p->dtype, 1, q, k, v, dout, omega, s, sp, inc_b, sp.G * E, E,
                                    omega_t, extra, dk, dvv, st);
    } else if (use_mfma(p)) {
        // matrix-core route: every wave its own chunks against the totals
        float* fin_f = extra;
        float* fin_b = extra + BH * E;
        void* dnum = fin_b + BH * E;                        // bf16 [BH, N, DV]
        float* dden = (float*)dnum + (size_t)BH * N * (DV / 2); // [BH, N]
        if (e == hipSuccess)
            e = launch_segment_scan(p->r, s, sp, nullptr, nullptr, inc_f, 0, nullptr, nullptr,
                                    fin_f, st);
        if (e == hipSuccess)
            e = launch_favor_bwd_query(c, q, dout, omega, s, sp, fin_f, dq, dnum, dden, st);
        // (G | g) = sum_t phi(q_t) (dnum_t, dden_t): the increment kernel on (q, dnum), z weighted
        if (e == hipSuccess) e = launch_favor_sums(c, q, dnum, omega, s, sp, inc_b, st, dden);
        if (e == hipSuccess)
            e = launch_segment_scan(p->r, s, sp, nullptr, nullptr, inc_b, 0, nullptr, nullptr,
                                    fin_b, st);
        if (e == hipSuccess) e = launch_favor_bwd_key(c, k, v, omega, s, sp, fin_b, dk, dvv, st);
    } else {
        float* fin_f = extra;
        float* fin_b = extra + BH * E;
        if (e == hipSuccess)
            e = launch_segment_scan(p->r, s, sp, nullptr, nullptr, inc_f, 0, nullptr, nullptr,
                                    fin_f, st);
        if (e == hipSuccess)
            e = launch_backward_query(c, p->dtype, 0, q, k, v, dout, omega, s, sp, fin_f, E, 0,
                                      omega_t, inc_b, nullptr, dq, st);
        if (e == hipSuccess)
            e = launch_segment_scan(p->r, s, sp, nullptr, nullptr, inc_b, 0, nullptr, nullptr,
                                    fin_b, st);
        if (e == hipSuccess)
            e = launch_backward_key(c, p->dtype, 0, q, k, v, dout, omega, s, sp, fin_b, E, 0,
                                    omega_t, nullptr, dk, dvv, st);
    }
    return launch_status(e);
}

// Input projection from the tokens.  On the matrix-core configuration
// (bfloat16 FAVOR+, r = 256) the projection is one GEMM writing q, k, v
// (bfloat16, head-major) to the front of the workspace, followed by the
// matrix-core kernels, whose workspace follows (256-byte aligned).  Every
// other map runs the vector kernels with q, k, v projected in their loads
// (workspace as lin_attn_causal_chunked / lin_attn_bidir on the vector plan).
SegPlan proj_plan(const lin_attn_params* p, int64_t BH, int64_t N) {
    return plan_segments(BH, N, p->n_seg, TARGET_BLOCKS_VALU);
}

size_t proj_qkv_bytes(int64_t BH, int64_t N) {
    return ((size_t)(3 * BH * N * D) * sizeof(bf16_raw) + 255) & ~(size_t)255;
}

size_t proj_ws_bytes(bool causal, const lin_attn_params* p, int64_t BH, int64_t N) {
    if (use_mfma(p))
        return proj_qkv_bytes(BH, N) +
               ws_floats(causal ? LIN_ATTN_OP_CAUSAL : LIN_ATTN_OP_BIDIR, BH, plan_for(p, BH, N),
                         p->r) * sizeof(float);
    const SegPlan sp = proj_plan(p, BH, N);
    const int64_t E = state_elems(p->r);
    return ((size_t)(BH * sp.G * E) + (causal ? 0 : (size_t)(BH * E))) * sizeof(float);
}

// Checks shared by the two projected calls (beyond check_params / check_sizes).
int proj_checks(const lin_attn_params* p, const void* x, const void* w_q, const void* w_k,
                const void* w_v, int64_t B, int64_t H, int64_t N, int64_t d_model, bool any) {
    if (d_model <= 0) return LIN_ATTN_ERR_INVALID;
    if (any && B * N > 0 && !ptr_ok(x)) return LIN_ATTN_ERR_INVALID;
    if (any && (!ptr_ok(w_q) || !ptr_ok(w_k) || !ptr_ok(w_v))) return LIN_ATTN_ERR_INVALID;
    if (p->dtype != LIN_ATTN_BF16 || p->r > RMAX_BWD) return LIN_ATTN_ERR_UNSUPPORTED;
    if (d_model % 16 != 0 || d_model > 65536) return LIN_ATTN_ERR_UNSUPPORTED;
    // the projection GEMM's grid (one block per 128 tokens x 128 columns) in range
    if (B > 0 && N > ((int64_t)1 << 40) / B) return LIN_ATTN_ERR_UNSUPPORTED;
    const int64_t tiles = ((B * N + 127) / 128) * ((3 * H * D + 127) / 128);
    if (tiles > ((int64_t)1 << 31)) return LIN_ATTN_ERR_UNSUPPORTED;
    return LIN_ATTN_OK;
}

// The kernels of lin_attn_bidir on validated arguments: segment increments,
// their fixed-order total (written to S_out / z_out when given), readout.
hipError_t bidir_run(const lin_attn_params* p, const void* q, const void* k, const void* v,
                     int64_t BH, int64_t N, const void* omega, void* out, float* S_out,
                     float* z_out, float* ws, hipStream_t st) {
    const Cfg c = make_cfg(p);
    const Shape s{BH, N};
    const SegPlan sp = plan_for(p, BH, N);
    const SegPlan ss = sums_plan(sp);
    float* inc = ws;
    float* fin = inc + BH * ss.G * state_elems(p->r);
    hipError_t e = segment_sums(p, c, k, v, omega, s, ss, inc, st);
    if (e == hipSuccess)
        e = launch_segment_scan(p->r, s, ss, nullptr, nullptr, inc, 0, S_out, z_out, fin, st);
    if (e == hipSuccess)
        e = segment_outputs(p, c, 0, q, k, v, omega, s, sp, fin, state_elems(p->r), 0, out, st);
    return e;
}

// The kernels of lin_attn_causal_chunked on validated arguments: segment
// increments, their prefix from the starting state (the final state to S,
// z), the chunked recurrence of every segment from its prefix.
hipError_t causal_run(const lin_attn_params* p, const void* q, const void* k, const void* v,
                      int64_t BH, int64_t N, const void* omega, float* S, float* z,
                      int32_t state_in, void* out, float* ws, hipStream_t st) {
    const Cfg c = make_cfg(p);
    const Shape s{BH, N};
    const SegPlan sp = plan_for(p, BH, N);
    const SegPlan ss = sums_plan(sp);
    float* inc = ws;
    const int64_t E = state_elems(p->r);
    hipError_t e = segment_sums(p, c, k, v, omega, s, ss, inc, st);
    if (e == hipSuccess)
        e = launch_segment_scan(p->r, s, ss, state_in ? S : nullptr, state_in ? z : nullptr, inc,
                                (int)sp.sub, S, z, nullptr, st);
    // segment g starts at sub-segment g * sub: its carried-in state is that prefix
    if (e == hipSuccess)
        e = segment_outputs(p, c, 1, q, k, v, omega, s, sp, inc, ss.G * E, sp.sub * E, out, st);
    return e;
}

// The intra-chunk block length both kernel families run: one 32 x 32 MFMA
// tile on the matrix-core path, and the same length on the float32 path so
// that both round alike.  0 selects it; 64 and 128 are valid lengths of the
// method that no kernel here runs.
// The intra-chunk block length.  0 selects the kernel's own; 32 is the
// length every kernel runs up to r = 256 (one 32 x 32 MFMA tile; the vector
// kernels match it), so it is accepted there.  Past r = 256 the vector
// kernels run 16 (r <= 384) or 4 tokens (the state and tiles must fit LDS),
// and 64 and 128 no kernel runs: valid lengths, refused as unsupported.
int check_chunk(int32_t chunk, int32_t r) {
    if (chunk != 0 && chunk != 32 && chunk != 64 && chunk != 128) return LIN_ATTN_ERR_INVALID;
    if (chunk == 64 || chunk == 128) return LIN_ATTN_ERR_UNSUPPORTED;
    return chunk == 32 && r > 256 ? LIN_ATTN_ERR_UNSUPPORTED : LIN_ATTN_OK;
}

// Static scratch of lin_attn_causal_chunked_noalloc: one copy per GPU, held
// until the process ends.  Host code never uses the array's name as an
// address (on the host it is only a stand-in for the symbol): each device's
// copy is located once with hipGetSymbolAddress, with that device current.
__device__ __align__(256) unsigned char scratch[LIN_ATTN_NOALLOC_SCRATCH_BYTES];
constexpr int SCRATCH_MAX_DEVICES = 64;
std::atomic<void*> scratch_addr[SCRATCH_MAX_DEVICES];

// This device's copy of `scratch`, or NULL when it cannot be located.
void* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_MAX_DEVICES) return nullptr;
    void* ptr = scratch_addr[dev].load(std::memory_order_acquire);
    if (ptr) return ptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    scratch_addr[dev].store(ptr, std::memory_order_release); // same value if two threads race
    return ptr;
}

// lin_attn_causal_chunked, with the workspace either passed in or (noalloc)
// taken from the current device's static scratch.
int causal_call(const lin_attn_params* p, const void* q, const void* k, const void* v, int64_t B,
                int64_t H, int64_t N, int64_t d, int64_t dv, const void* omega, int32_t chunk,
                float* S, float* z, int32_t state_in, void* out, void* ws, size_t ws_bytes,
                void* stream, bool noalloc) {
    int rc = check_params(p, d, dv, omega);
    if (rc == LIN_ATTN_ERR_INVALID) return rc;
    const int rs = check_sizes(B, H, N);
    if (rs == LIN_ATTN_ERR_INVALID) return rs;
    const int rk = check_chunk(chunk, p->r);
    if (rk == LIN_ATTN_ERR_INVALID) return rk;
    if (state_in != 0 && state_in != 1) return LIN_ATTN_ERR_INVALID;
    if (!noalloc && !opt_ptr_ok(ws)) return LIN_ATTN_ERR_INVALID;
    if (B * H > 0 && (!ptr_ok(S) || !ptr_ok(z))) return LIN_ATTN_ERR_INVALID;
    if (B * H > 0 && N > 0 && (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(out)))
        return LIN_ATTN_ERR_INVALID;
    if (rc != LIN_ATTN_OK) return rc;
    if (rs != LIN_ATTN_OK) return rs;
    if (rk != LIN_ATTN_OK) return rk;
    if (B * H == 0) return LIN_ATTN_OK;
    if (N == 0) {
        // no token: the state after token N is the starting state
        if (state_in) return LIN_ATTN_OK;
        hipStream_t st = (hipStream_t)stream;
        hipError_t e = launch_fill_zero(S, B * H * (int64_t)p->r * DV, st);
        if (e == hipSuccess) e = launch_fill_zero(z, B * H * (int64_t)p->r, st);
        return launch_status(e);
    }
    const int64_t BH = B * H;
    const SegPlan sp = plan_for(p, BH, N);
    const size_t need = ws_floats(LIN_ATTN_OP_CAUSAL, BH, sp, p->r) * sizeof(float);
    if (noalloc) {
        if (need > LIN_ATTN_NOALLOC_SCRATCH_BYTES) return LIN_ATTN_ERR_WORKSPACE;
        ws = device_scratch();
        if (!ws) return LIN_ATTN_ERR_HIP;
        ws_bytes = LIN_ATTN_NOALLOC_SCRATCH_BYTES;
    }
    if (ws_bytes < need || !ws) return LIN_ATTN_ERR_WORKSPACE;

    return launch_status(causal_run(p, q, k, v, BH, N, omega, S, z, state_in, out, (float*)ws,
                                    (hipStream_t)stream));
}

} // namespace

extern "C" {

int32_t lin_attn_abi_version(void) { return LIN_ATTN_ABI_VERSION; }

const char* lin_attn_strerror(int32_t code) {
    switch (code) {
    case LIN_ATTN_OK: return "success";
    case LIN_ATTN_ERR_INVALID: return "invalid argument";
    case LIN_ATTN_ERR_UNSUPPORTED: return "valid but unsupported on this GPU path";
    case LIN_ATTN_ERR_WORKSPACE: return "workspace too small";
    case LIN_ATTN_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown error code";
    }
}

size_t lin_attn_workspace_bytes(int32_t op, const lin_attn_params* p, int64_t B, int64_t H,
                                int64_t N, int64_t d, int64_t dv, int32_t chunk) {
    if (op < LIN_ATTN_OP_BIDIR || op > LIN_ATTN_OP_BIDIR_PROJ) return 0;
    if (!p || check_sizes(B, H, N) != LIN_ATTN_OK) return 0;
    if (op == LIN_ATTN_OP_CAUSAL && check_chunk(chunk, p->r) != LIN_ATTN_OK) return 0;
    // omega is not needed to size the workspace: check the rest with a dummy
    const int rc = check_params(p, d, dv, reinterpret_cast<const void*>(uintptr_t(16)));
    if (rc != LIN_ATTN_OK) return 0;
    const int64_t BH = B * H;
    if (BH == 0 || N == 0) return 0;
    if (op == LIN_ATTN_OP_CAUSAL_VARLEN) return varlen_layout(p, B, H, N).bytes;
    const bool proj = op == LIN_ATTN_OP_CAUSAL_PROJ || op == LIN_ATTN_OP_BIDIR_PROJ;
    const bool bwd = op == LIN_ATTN_OP_BIDIR_BACKWARD || op == LIN_ATTN_OP_CAUSAL_BACKWARD;
    if ((proj || bwd) && p->r > RMAX_BWD) return 0; // unsupported there
    if (proj) return proj_ws_bytes(op == LIN_ATTN_OP_CAUSAL_PROJ, p, BH, N);
    if (bwd)
        return backward_layout(p, op == LIN_ATTN_OP_CAUSAL_BACKWARD, BH, N).floats * sizeof(float);
    return ws_floats(op, BH, plan_for(p, BH, N), p->r) * sizeof(float);
}

int lin_attn_featuremap(const lin_attn_params* p, const void* x, int64_t B, int64_t H, int64_t N,
                        int64_t d, const void* omega, float* phi, void* stream) {
    int rc = check_params(p, d, DV, omega);
    if (rc == LIN_ATTN_ERR_INVALID) return rc;
    const int rs = check_sizes(B, H, N);
    if (rs == LIN_ATTN_ERR_INVALID) return rs;
    const bool empty = B * H == 0 || N == 0;
    if (!empty && (!ptr_ok(x) || !ptr_ok(phi))) return LIN_ATTN_ERR_INVALID;
    if (rc != LIN_ATTN_OK) return rc;
    if (rs != LIN_ATTN_OK) return rs;
    if (empty) return LIN_ATTN_OK;
    return launch_status(launch_featuremap(make_cfg(p), p->dtype, x, omega, Shape{B * H, N}, phi,
                                           (hipStream_t)stream));
}

int lin_attn_bidir(const lin_attn_params* p, const void* q, const void* k, const void* v,
                   int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv, const void* omega,
                   void* out, float* S_out, float* z_out, void* ws, size_t ws_bytes,
                   void* stream) {
    int rc = check_params(p, d, dv, omega);
    if (rc == LIN_ATTN_ERR_INVALID) return rc;
    const int rs = check_sizes(B, H, N);
    if (rs == LIN_ATTN_ERR_INVALID) return rs;
    if (!opt_ptr_ok(S_out) || !opt_ptr_ok(z_out) || !opt_ptr_ok(ws)) return LIN_ATTN_ERR_INVALID;
    const bool empty = B * H == 0 || N == 0;
    if (!empty && (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(out)))
        return LIN_ATTN_ERR_INVALID;
    if (rc != LIN_ATTN_OK) return rc;
    if (rs != LIN_ATTN_OK) return rs;
    if (empty) {
        // no key: the summaries are zero
        hipError_t e = hipSuccess;
        if (S_out) e = launch_fill_zero(S_out, B * H * (int64_t)p->r * DV, (hipStream_t)stream);
        if (e == hipSuccess && z_out) e = launch_fill_zero(z_out, B * H * (int64_t)p->r, (hipStream_t)stream);
        return launch_status(e);
    }
    const int64_t BH = B * H;
    const SegPlan sp = plan_for(p, BH, N);
    const size_t need = ws_floats(LIN_ATTN_OP_BIDIR, BH, sp, p->r) * sizeof(float);
    if (ws_bytes < need || !ws) return LIN_ATTN_ERR_WORKSPACE;

    return launch_status(bidir_run(p, q, k, v, BH, N, omega, out, S_out, z_out, (float*)ws,
                                   (hipStream_t)stream));
}

int lin_attn_causal_chunked(const lin_attn_params* p, const void* q, const void* k,
                            const void* v, int64_t B, int64_t H, int64_t N, int64_t d,
                            int64_t dv, const void* omega, int32_t chunk, float* S, float* z,
                            int32_t state_in, void* out, void* ws, size_t ws_bytes,
                            void* stream) {
    return causal_call(p, q, k, v, B, H, N, d, dv, omega, chunk, S, z, state_in, out, ws, ws_bytes,
                       stream, false);
}

int lin_attn_causal_chunked_noalloc(const lin_attn_params* p, const void* q, const void* k,
                                    const void* v, int64_t B, int64_t H, int64_t N, int64_t d,
                                    int64_t dv, const void* omega, int32_t chunk, float* S,
                                    float* z, int32_t state_in, void* out, void* stream) {
    return causal_call(p, q, k, v, B, H, N, d, dv, omega, chunk, S, z, state_in, out, nullptr, 0,
                       stream, true);
}

int lin_attn_causal_varlen(const lin_attn_params* p, const void* q, const void* k,
                           const void* v, const int32_t* cu_seqlens, int64_t num_seqs,
                           int64_t H, int64_t total, int64_t d, int64_t dv, const void* omega,
                           float* S, float* z, int32_t state_in, void* out, void* ws,
                           size_t ws_bytes, void* stream) {
    int rc = check_params(p, d, dv, omega);
    if (rc == LIN_ATTN_ERR_INVALID) return rc;
    const int rs = check_sizes(num_seqs, H, total);
    if (rs == LIN_ATTN_ERR_INVALID) return rs;
    if (state_in != 0 && state_in != 1) return LIN_ATTN_ERR_INVALID;
    if (num_seqs == 0 && total > 0) return LIN_ATTN_ERR_INVALID; // tokens of no sequence
    if (!opt_ptr_ok(ws)) return LIN_ATTN_ERR_INVALID;
    if (num_seqs * H > 0 && (!ptr_ok(S) || !ptr_ok(z))) return LIN_ATTN_ERR_INVALID;
    if (num_seqs > 0 && (!cu_seqlens || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3)))
        return LIN_ATTN_ERR_INVALID;
    if (H > 0 && total > 0 && (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(out)))
        return LIN_ATTN_ERR_INVALID;
    if (rc != LIN_ATTN_OK) return rc;
    if (rs != LIN_ATTN_OK) return rs;
    if (num_seqs * H == 0) return LIN_ATTN_OK;
    hipStream_t st = (hipStream_t)stream;
    if (total == 0) {
        // no token in any sequence: every final state is the starting state
        if (state_in) return LIN_ATTN_OK;
        hipError_t e = launch_fill_zero(S, num_seqs * H * (int64_t)p->r * DV, st);
        if (e == hipSuccess) e = launch_fill_zero(z, num_seqs * H * (int64_t)p->r, st);
        return launch_status(e);
    }
    const VarlenLayout L = varlen_layout(p, num_seqs, H, total);
    if (ws_bytes < L.bytes || !ws) return LIN_ATTN_ERR_WORKSPACE;

    const Cfg c = make_cfg(p);
    const Shape s{H, total};
    float* inc = (float*)ws;
    int64_t* tab = reinterpret_cast<int64_t*>(static_cast<char*>(ws) + L.tab_off);
    int64_t* first = reinterpret_cast<int64_t*>(static_cast<char*>(ws) + L.first_off);
    int64_t* order = reinterpret_cast<int64_t*>(static_cast<char*>(ws) + L.order_off);
    SegPlan sp = L.sp;
    sp.tab = tab;
    // the matrix-core kernels run the segments longest first; the vector
    // kernels keep head-major order
    if (use_mfma(p)) sp.order = order;
    const SegPlan ss = sums_plan(sp);
    const int64_t E = state_elems(p->r);
    hipError_t e = launch_varlen_plan(cu_seqlens, num_seqs, total, sp.seg_len, sp.sub, L.parts, tab,
                                      first, order, st);
    if (e == hipSuccess) e = segment_sums(p, c, k, v, omega, s, ss, inc, st);
    if (e == hipSuccess)
        e = launch_segment_scan_varlen(p->r, H, num_seqs, L.parts, first, state_in ? S : nullptr,
                                       state_in ? z : nullptr, inc, (int)sp.sub, S, z, st);
    // segment g starts at part g * sub: its carried-in state is that prefix
    if (e == hipSuccess)
        e = segment_outputs(p, c, 1, q, k, v, omega, s, sp, inc, ss.G * E, sp.sub * E, out, st);
    return launch_status(e);
}

int lin_attn_orf_omega(const float* gauss, const float* len_gauss, int64_t n_mat, int64_t r,
                       int64_t d, int32_t dtype, void* omega, void* stream) {
    if (n_mat < 0 || r < 0 || d < 1) return LIN_ATTN_ERR_INVALID;
    if (dtype != LIN_ATTN_F32 && dtype != LIN_ATTN_BF16) return LIN_ATTN_ERR_INVALID;
    if (n_mat > 0 && r > 0 && (!ptr_ok(gauss) || !ptr_ok(omega) || !opt_ptr_ok(len_gauss)))
        return LIN_ATTN_ERR_INVALID;
    if (d > 64) return LIN_ATTN_ERR_UNSUPPORTED;
    if (n_mat == 0 || r == 0) return LIN_ATTN_OK;
    const int64_t nblk = (r + d - 1) / d;
    if (n_mat > ((int64_t)1 << 24) || nblk > ((int64_t)1 << 24) / n_mat) return LIN_ATTN_ERR_UNSUPPORTED;
    return launch_status(launch_orf(gauss, len_gauss, n_mat, r, (int)d, dtype, omega,
                                    (hipStream_t)stream));
}

int lin_attn_bidir_backward(const lin_attn_params* p, const void* q, const void* k,
                            const void* v, const void* dout, int64_t B, int64_t H, int64_t N,
                            int64_t d, int64_t dv, const void* omega, void* dq, void* dk,
                            void* dv_out, void* ws, size_t ws_bytes, void* stream) {
    return backward_call(false, p, q, k, v, dout, B, H, N, d, dv, omega, dq, dk, dv_out, ws,
                         ws_bytes, stream);
}

int lin_attn_causal_backward(const lin_attn_params* p, const void* q, const void* k,
                             const void* v, const void* dout, int64_t B, int64_t H, int64_t N,
                             int64_t d, int64_t dv, const void* omega, void* dq, void* dk,
                             void* dv_out, void* ws, size_t ws_bytes, void* stream) {
    return backward_call(true, p, q, k, v, dout, B, H, N, d, dv, omega, dq, dk, dv_out, ws,
                         ws_bytes, stream);
}

int lin_attn_causal_proj(const lin_attn_params* p, const void* x, const void* w_q,
                         const void* w_k, const void* w_v, int64_t B, int64_t H, int64_t N,
                         int64_t d_model, int64_t d, int64_t dv, const void* omega, float* S,
                         float* z, int32_t state_in, void* out, void* ws, size_t ws_bytes,
                         void* stream) {
    int rc = check_params(p, d, dv, omega);
    if (rc == LIN_ATTN_ERR_INVALID) return rc;
    const int rs = check_sizes(B, H, N);
    if (rs == LIN_ATTN_ERR_INVALID) return rs;
    if (state_in != 0 && state_in != 1) return LIN_ATTN_ERR_INVALID;
    if (!opt_ptr_ok(ws)) return LIN_ATTN_ERR_INVALID;
    if (B * H > 0 && (!ptr_ok(S) || !ptr_ok(z))) return LIN_ATTN_ERR_INVALID;
    if (B * H > 0 && N > 0 && !ptr_ok(out)) return LIN_ATTN_ERR_INVALID;
    const int pc = proj_checks(p, x, w_q, w_k, w_v, B, H, N, d_model, B * H > 0 && N > 0);
    if (pc == LIN_ATTN_ERR_INVALID) return pc;
    if (rc != LIN_ATTN_OK) return rc;
    if (rs != LIN_ATTN_OK) return rs;
    if (pc != LIN_ATTN_OK) return pc;
    if (B * H == 0) return LIN_ATTN_OK;
    hipStream_t st = (hipStream_t)stream;
    if (N == 0) {
        // no token: the state after token N is the starting state
        if (state_in) return LIN_ATTN_OK;
        hipError_t e = launch_fill_zero(S, B * H * (int64_t)p->r * DV, st);
        if (e == hipSuccess) e = launch_fill_zero(z, B * H * (int64_t)p->r, st);
        return launch_status(e);
    }
    const int64_t BH = B * H;
    if (ws_bytes < proj_ws_bytes(true, p, BH, N) || !ws) return LIN_ATTN_ERR_WORKSPACE;
    if (use_mfma(p)) {
        bf16_raw* qkv = static_cast<bf16_raw*>(ws);
        const int64_t n = BH * N * D;
        hipError_t e = launch_qkv_project(x, w_q, w_k, w_v, B, N, d_model, H, qkv, qkv + n,
                                          qkv + 2 * n, st);
        if (e == hipSuccess)
            e = causal_run(p, qkv, qkv + n, qkv + 2 * n, BH, N, omega, S, z, state_in, out,
                           reinterpret_cast<float*>(static_cast<char*>(ws) + proj_qkv_bytes(BH, N)),
                           st);
        return launch_status(e);
    }
    const Cfg c = make_cfg(p);
    const Shape s{BH, N};
    const SegPlan sp = proj_plan(p, BH, N);
    const Proj P{(const bf16_raw*)x,
                 {(const bf16_raw*)w_q, (const bf16_raw*)w_k, (const bf16_raw*)w_v},
                 d_model,
                 H};
    float* inc = (float*)ws;
    const int64_t E = state_elems(p->r);
    hipError_t e = launch_segment_sums_proj(c, P, omega, s, sp, inc, st);
    if (e == hipSuccess)
        e = launch_segment_scan(p->r, s, sp, state_in ? S : nullptr, state_in ? z : nullptr, inc,
                                1, S, z, nullptr, st);
    if (e == hipSuccess)
        e = launch_segment_outputs_proj(c, 1, P, omega, s, sp, inc, sp.G * E, E, out, st);
    return launch_status(e);
}

int lin_attn_bidir_proj(const lin_attn_params* p, const void* x, const void* w_q,
                        const void* w_k, const void* w_v, int64_t B, int64_t H, int64_t N,
                        int64_t d_model, int64_t d, int64_t dv, const void* omega, void* out,
                        float* S_out, float* z_out, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_params(p, d, dv, omega);
    if (rc == LIN_ATTN_ERR_INVALID) return rc;
    const int rs = check_sizes(B, H, N);
    if (rs == LIN_ATTN_ERR_INVALID) return rs;
    if (!opt_ptr_ok(S_out) || !opt_ptr_ok(z_out) || !opt_ptr_ok(ws)) return LIN_ATTN_ERR_INVALID;
    const bool empty = B * H == 0 || N == 0;
    if (!empty && !ptr_ok(out)) return LIN_ATTN_ERR_INVALID;
    const int pc = proj_checks(p, x, w_q, w_k, w_v, B, H, N, d_model, !empty);
    if (pc == LIN_ATTN_ERR_INVALID) return pc;
    if (rc != LIN_ATTN_OK) return rc;
    if (rs != LIN_ATTN_OK) return rs;
    if (pc != LIN_ATTN_OK) return pc;
    hipStream_t st = (hipStream_t)stream;
    if (empty) {
        hipError_t e = hipSuccess;
        if (S_out) e = launch_fill_zero(S_out, B * H * (int64_t)p->r * DV, st);
        if (e == hipSuccess && z_out) e = launch_fill_zero(z_out, B * H * (int64_t)p->r, st);
        return launch_status(e);
    }
    const int64_t BH = B * H;
    if (ws_bytes < proj_ws_bytes(false, p, BH, N) || !ws) return LIN_ATTN_ERR_WORKSPACE;
    if (use_mfma(p)) {
        bf16_raw* qkv = static_cast<bf16_raw*>(ws);
        const int64_t n = BH * N * D;
        hipError_t e = launch_qkv_project(x, w_q, w_k, w_v, B, N, d_model, H, qkv, qkv + n,
                                          qkv + 2 * n, st);
        if (e == hipSuccess)
            e = bidir_run(p, qkv, qkv + n, qkv + 2 * n, BH, N, omega, out, S_out, z_out,
                          reinterpret_cast<float*>(static_cast<char*>(ws) + proj_qkv_bytes(BH, N)),
                          st);
        return launch_status(e);
    }
    const Cfg c = make_cfg(p);
    const Shape s{BH, N};
    const SegPlan sp = proj_plan(p, BH, N);
    const Proj P{(const bf16_raw*)x,
                 {(const bf16_raw*)w_q, (const bf16_raw*)w_k, (const bf16_raw*)w_v},
                 d_model,
                 H};
    const int64_t E = state_elems(p->r);
    float* inc = (float*)ws;
    float* fin = inc + BH * sp.G * E;
    hipError_t e = launch_segment_sums_proj(c, P, omega, s, sp, inc, st);
    if (e == hipSuccess)
        e = launch_segment_scan(p->r, s, sp, nullptr, nullptr, inc, 0, S_out, z_out, fin, st);
    if (e == hipSuccess) e = launch_segment_outputs_proj(c, 0, P, omega, s, sp, fin, E, 0, out, st);
    return launch_status(e);
}

int lin_attn_qkv_project(const void* x, const void* w_q, const void* w_k, const void* w_v,
                         int64_t B, int64_t N, int64_t d_model, int64_t H, int64_t d, void* q,
                         void* k, void* v, void* stream) {
    if (B < 0 || N < 0 || H < 0 || d <= 0 || d_model <= 0) return LIN_ATTN_ERR_INVALID;
    const bool empty = B * N == 0 || H == 0;
    if (!empty && (!ptr_ok(x) || !ptr_ok(w_q) || !ptr_ok(w_k) || !ptr_ok(w_v) || !ptr_ok(q) ||
                   !ptr_ok(k) || !ptr_ok(v)))
        return LIN_ATTN_ERR_INVALID;
    if (d != D || d_model % 16 != 0 || d_model > 65536) return LIN_ATTN_ERR_UNSUPPORTED;
    if (check_sizes(B, H, N) != LIN_ATTN_OK) return LIN_ATTN_ERR_UNSUPPORTED;
    if (empty) return LIN_ATTN_OK;
    // grid: one block per 128 tokens x 128 output columns
    const int64_t tiles = ((B * N + 127) / 128) * ((3 * H * D + 127) / 128);
    if (tiles > ((int64_t)1 << 31)) return LIN_ATTN_ERR_UNSUPPORTED;
    return launch_status(
        launch_qkv_project(x, w_q, w_k, w_v, B, N, d_model, H, q, k, v, (hipStream_t)stream));
}

int lin_attn_decode_step(const lin_attn_params* p, const void* q, const void* k, const void* v,
                         int64_t B, int64_t H, int64_t d, int64_t dv, const void* omega, float* S,
                         float* z, void* out, void* stream) {
    int rc = check_params(p, d, dv, omega);
    if (rc == LIN_ATTN_ERR_INVALID) return rc;
    const int rs = check_sizes(B, H, 1);
    if (rs == LIN_ATTN_ERR_INVALID) return rs;
    if (B * H > 0 &&
        (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(out) || !ptr_ok(S) || !ptr_ok(z)))
        return LIN_ATTN_ERR_INVALID;
    if (rc != LIN_ATTN_OK) return rc;
    if (rs != LIN_ATTN_OK) return rs;
    if (B * H == 0) return LIN_ATTN_OK;
    return launch_status(
        launch_decode(make_cfg(p), p->dtype, q, k, v, omega, B * H, S, z, out, (hipStream_t)stream));
}

} // extern "C"
