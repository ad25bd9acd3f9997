/*
 * lin_attn.h -- C ABI of liblinattn.so: kernelized linear attention on
 * AMD MI355X (gfx950): forward pass (also from the tokens, with the q/k/v
 * projection fused in), decode, orthogonal random features and the backward
 * pass.
 *
 * Sources of the operations (the pages the method is taken from):
 *   [KZ] "The Kernel Zoo: Performers, Fast Weight Programmers, and the
 *        Capacity-Approximation Tradeoff in Linear Attention" (prathamp.com)
 *   [RF] "Reassociate a feature-map kernel without claiming exact softmax"
 *        (study.greatitself.com)
 *   [LA] "Linear attention & kernelized approximations" (interactive chapter)
 *   [PF] "Performer -- Random Feature Softmax Approximation" (lizeman.github.io)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Buffers.  Every tensor argument is a DEVICE pointer to contiguous,
 *   row-major memory, 16-byte aligned.  Shapes use B (batch), H (heads),
 *   N (tokens), d (query/key width), dv (value width), r (feature width):
 *     q, k, x    [B, H, N, d]        v, out   [B, H, N, dv]
 *     omega      [r, d]              phi      [B, H, N, r]   (float32)
 *     S          [B, H, r, dv]       z        [B, H, r]      (float32)
 *   q, k, v, omega and out share the element type lin_attn_params.dtype
 *   (float32 or bfloat16).  S and z are always float32.  Heads are
 *   independent; one omega is shared by all heads of a call ([PF] sec. 2,
 *   "sampled once and frozen").
 * Ownership.  The caller allocates and owns every buffer, including the
 *   workspace (size from lin_attn_workspace_bytes).  The library never
 *   allocates, frees or keeps a pointer after returning and is reentrant.
 *   Its only global state is the static scratch array of
 *   lin_attn_causal_chunked_noalloc (one per GPU, see there).
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the null
 *   stream).  All work is enqueued asynchronously on it; nothing
 *   synchronises.  Buffers must stay valid until that work completes.
 *   Device faults surface at the caller's next synchronisation.
 * Errors.  Every int-returning entry point returns LIN_ATTN_OK (0) or a
 *   negative code, checks its arguments before enqueueing anything, and on
 *   error enqueues nothing and leaves every buffer untouched.  It never
 *   prints, throws or aborts.  N == 0 or B*H == 0 is a successful no-op.
 * GPU coverage.  d == dv == 64; r a multiple of 32 in [32, 512] (the
 *   backward and the projected calls: [32, 256]); feature maps identity,
 *   ELU+1, FAVOR+, DPFP; float32 and bfloat16.  Other combinations return
 *   LIN_ATTN_ERR_UNSUPPORTED.  r = 256 is the Performer's choice for
 *   d = 64 ([PF] sec. 2) and 384 = d log2 d one reading of its cost
 *   statement; the pages put the useful range up to r ~ 1024 ([PF] sec. 4).
 */
#ifndef LIN_ATTN_H
#define LIN_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LIN_ATTN_ABI_VERSION 1

/* Feature maps phi: R^d -> R^r. */
#define LIN_ATTN_PHI_IDENTITY 0 /* phi(x) = x, r = d ([KZ] sec. 1.3; [LA])         */
#define LIN_ATTN_PHI_ELU1 1     /* elu(x) + 1 (alpha = 1), r = d ([KZ] running     */
                                /* example; [PF] sec. 1)                           */
#define LIN_ATTN_PHI_FAVOR 2    /* exp(omega_i . x - |x|^2 / 2) / sqrt(r), r rows  */
                                /* of omega ([KZ] sec. 4.2, 5.4; [PF] sec. 2-3)    */
#define LIN_ATTN_PHI_DPFP 3     /* relu([x,-x]) products with rolled copies,      */
                                /* r = 2 d nu ([KZ] sec. 6.3)                      */

/* Readout. */
#define LIN_ATTN_NORM_ATTN 0 /* out = num / max(den, eps) ([RF] par. 1-2; [PF] sketch) */
#define LIN_ATTN_NORM_NONE 1 /* out = num (unnormalised fast-weight read, [KZ] 1.2)   */

/* Element types of q, k, v, omega, out. */
#define LIN_ATTN_F32 0
#define LIN_ATTN_BF16 1 /* bfloat16; float32 accumulation everywhere */

/* Return codes. */
#define LIN_ATTN_OK 0
#define LIN_ATTN_ERR_INVALID (-1)     /* null required pointer, negative size, bad enum,  */
                                      /* eps <= 0, r inconsistent with phi / nu / omega    */
#define LIN_ATTN_ERR_UNSUPPORTED (-2) /* valid, but outside the GPU coverage above         */
#define LIN_ATTN_ERR_WORKSPACE (-3)   /* ws_bytes smaller than lin_attn_workspace_bytes   */
#define LIN_ATTN_ERR_HIP (-4)         /* a kernel launch failed (hipGetLastError)          */

/* Operation ids for lin_attn_workspace_bytes. */
#define LIN_ATTN_OP_BIDIR 1
#define LIN_ATTN_OP_CAUSAL 2
#define LIN_ATTN_OP_CAUSAL_VARLEN 3
#define LIN_ATTN_OP_BIDIR_BACKWARD 4
#define LIN_ATTN_OP_CAUSAL_BACKWARD 5
#define LIN_ATTN_OP_CAUSAL_PROJ 6
#define LIN_ATTN_OP_BIDIR_PROJ 7

/*
 * Method parameters, shared by every call.
 *   phi       LIN_ATTN_PHI_*.
 *   r         feature width: must equal d for IDENTITY and ELU1, the number of
 *             rows of omega for FAVOR, 2*d*nu for DPFP ([KZ] sec. 6.3).
 *   nu        DPFP shift count, 1 <= nu <= 2d-1 ([KZ] sec. 6.3); ignored otherwise.
 *   sum_norm  0 or 1: replace phi(x) by phi(x) / max(sum_i phi(x)_i, eps), for
 *             queries and keys ([KZ] sec. 7.2).
 *   norm      LIN_ATTN_NORM_ATTN or LIN_ATTN_NORM_NONE.
 *   dtype     LIN_ATTN_F32 or LIN_ATTN_BF16.
 *   scale     x <- scale * x for q and k before phi.  d^-1/4 places the
 *             softmax temperature 1/sqrt(d) inside FAVOR+ ([KZ] sec. 3.3: it
 *             can be absorbed into the inputs); 1 reproduces the pages'
 *             worked examples.
 *   eps       > 0.  Lower clamp of the attention denominator
 *             (max(den, eps), the [PF] sketch's clamp) and of the sum in sum
 *             normalisation.  [RF] par. 2 asks that it be stated, not hidden.
 *   n_seg     sequence segments per head for the parallel scan; 0 = choose
 *             automatically.  Changes rounding only, never the result.
 *   reserved  must be 0.
 */
typedef struct lin_attn_params {
    int32_t phi;
    int32_t r;
    int32_t nu;
    int32_t sum_norm;
    int32_t norm;
    int32_t dtype;
    float scale;
    float eps;
    int32_t n_seg;
    int32_t reserved;
} lin_attn_params;

/*
 * Feature map alone: phi = phi(scale * x) for every token, float32 output
 * [B, H, N, r].  omega [r, d] is required for FAVOR and ignored otherwise
 * (may be NULL).  Definitions: [KZ] running example (ELU+1), sec. 4.2 boxed
 * map and sec. 5.4 (FAVOR+), sec. 6.3 (DPFP), sec. 7.2 (sum normalisation).
 */
int lin_attn_featuremap(const lin_attn_params* p, const void* x, int64_t B, int64_t H,
                        int64_t N, int64_t d, const void* omega, float* phi, void* stream);

/*
 * Bidirectional (encoder) attention in the reassociated form
 * ([RF] par. 1; [PF] sec. 2 step 5 and sec. 3 sketch; [LA]):
 *   S = sum_j phi(k_j) v_j^T,  z = sum_j phi(k_j),
 *   out_i = phi(q_i)^T S / max(phi(q_i) . z, eps)   (NORM_ATTN)
 *         = phi(q_i)^T S                            (NORM_NONE)
 * out [B, H, N, dv] has the input dtype.  S_out [B, H, r, dv] and
 * z_out [B, H, r] (float32) receive the summaries when non-NULL.
 * ws: device workspace of at least
 * lin_attn_workspace_bytes(LIN_ATTN_OP_BIDIR, ...) bytes (may be NULL when
 * that is 0); its contents on entry do not matter.
 */
int lin_attn_bidir(const lin_attn_params* p, const void* q, const void* k, const void* v,
                   int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv, const void* omega,
                   void* out, float* S_out, float* z_out, void* ws, size_t ws_bytes,
                   void* stream);

/*
 * Causal prefill by the prefix-sum recurrence ([KZ] sec. 1.3 and sec. 5.4;
 * [RF] par. 4; [PF] sec. 2 step 5 and the sketch's last line):
 *   (S, z) <- (0, 0) when state_in == 0, else the caller's (S, z);
 *   for t = 1..N:  S += phi(k_t) v_t^T;  z += phi(k_t);      (write first)
 *                  out_t = readout of phi(q_t) against (S, z) (then read)
 * so query t sees keys up to and including t.  Computed as a chunked scan:
 * each chunk of `chunk` tokens combines its masked intra-chunk block with
 * the state carried in from earlier chunks, and sequence segments are
 * combined by a prefix sum of their state increments; all of these are
 * exact re-associations of the recurrence.
 *   chunk     intra-chunk block length.  0: the kernel's own, which is 32
 *             (one 32 x 32 MFMA tile) for r <= 256 on every kernel family,
 *             and 16 (r <= 384) or 4 (r <= 512) on the vector kernels that
 *             run the wider maps.  32: accepted for r <= 256.  Every block
 *             length re-associates the [KZ] sec. 1.3 recurrence exactly, so
 *             the result changes only by rounding; 64 and 128 (and 32 past
 *             r = 256) are valid lengths that no kernel here runs:
 *             LIN_ATTN_ERR_UNSUPPORTED.  Other values: LIN_ATTN_ERR_INVALID.
 *   S, z      float32 [B, H, r, dv] / [B, H, r], required, in/out: read
 *             when state_in == 1, always overwritten with the state after
 *             token N (the carried fast-weight memory of [KZ] sec. 9.3; a
 *             packing boundary is a call with state_in == 0, [RF] par. 4).
 *   out       [B, H, N, dv], input dtype.
 *   ws        at least lin_attn_workspace_bytes(LIN_ATTN_OP_CAUSAL, ...) bytes.
 */
int lin_attn_causal_chunked(const lin_attn_params* p, const void* q, const void* k,
                            const void* v, int64_t B, int64_t H, int64_t N, int64_t d,
                            int64_t dv, const void* omega, int32_t chunk, float* S, float* z,
                            int32_t state_in, void* out, void* ws, size_t ws_bytes,
                            void* stream);

/* Size of the static scratch of lin_attn_causal_chunked_noalloc (64 MiB). */
#define LIN_ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * lin_attn_causal_chunked for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, kernels and results as lin_attn_causal_chunked
 * without ws / ws_bytes: the workspace is a static array of
 * LIN_ATTN_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU,
 * located on the call's first use of a device and held until the process
 * ends.  The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).
 *   The scratch of the current device is used: `stream` must belong to it.
 *   Calls that overlap in time on one GPU share its scratch and race; the
 *   caller serialises them (one stream, or events between streams).  Every
 *   scratch byte a call reads was written earlier in the same call, so
 *   nothing left by a previous call needs clearing.
 * Errors as lin_attn_causal_chunked, plus LIN_ATTN_ERR_WORKSPACE when
 * lin_attn_workspace_bytes(LIN_ATTN_OP_CAUSAL, ...) exceeds the scratch
 * (B = 1, H = 8, N = 65536, r = 256 needs 34 MB) and LIN_ATTN_ERR_HIP when
 * the device's copy cannot be located.
 */
int lin_attn_causal_chunked_noalloc(const lin_attn_params* p, const void* q, const void* k,
                                    const void* v, int64_t B, int64_t H, int64_t N, int64_t d,
                                    int64_t dv, const void* omega, int32_t chunk, float* S,
                                    float* z, int32_t state_in, void* out, void* stream);

/*
 * Causal prefill of a packed batch: num_seqs independent sequences laid end
 * to end along the token axis, the state reset at every sequence boundary
 * ([RF] par. 4: packing must reset the state at the logical boundary).
 * Sequence i is tokens [cu_seqlens[i], cu_seqlens[i+1]) of every head and
 * runs the recurrence of lin_attn_causal_chunked from its own state.
 *   q, k        [H, total, d]; v, out [H, total, dv] (head-major, tokens of
 *               all sequences packed), input dtype.
 *   cu_seqlens  device int32 [num_seqs + 1]: nondecreasing, cu_seqlens[0] = 0,
 *               cu_seqlens[num_seqs] = total (4-byte aligned).  It is read on
 *               the device only, so the call stays asynchronous and is not
 *               checked on the host: values are clamped to [0, total] there,
 *               and malformed boundaries give unspecified results but no
 *               access out of bounds.  Empty sequences are allowed.
 *   S, z        float32 [num_seqs, H, r, dv] / [num_seqs, H, r], required,
 *               in/out: each sequence's initial state when state_in == 1
 *               (else zero), its final state after the call (the carry into
 *               a following call).
 *   ws          at least lin_attn_workspace_bytes(LIN_ATTN_OP_CAUSAL_VARLEN,
 *               p, num_seqs, H, total, d, dv, 0) bytes; the library plans the
 *               segments into it on the device.
 * Errors as lin_attn_causal_chunked; tokens with num_seqs == 0 are invalid.
 */
int lin_attn_causal_varlen(const lin_attn_params* p, const void* q, const void* k,
                           const void* v, const int32_t* cu_seqlens, int64_t num_seqs,
                           int64_t H, int64_t total, int64_t d, int64_t dv, const void* omega,
                           float* S, float* z, int32_t state_in, void* out, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * One decode step for B*H single tokens ([KZ] sec. 1.2 steps 2-3; [RF]
 * par. 3 "streaming causal calculation"):
 *   S += phi(k) v^T;  z += phi(k);  out = readout of phi(q) against (S, z).
 * q, k [B, H, d], v [B, H, dv], out [B, H, dv] (input dtype); S, z are
 * updated in place (float32).  Needs no workspace.
 */
int lin_attn_decode_step(const lin_attn_params* p, const void* q, const void* k,
                         const void* v, int64_t B, int64_t H, int64_t d, int64_t dv,
                         const void* omega, float* S, float* z, void* out, void* stream);

/*
 * Orthogonal random features built on the device ([PF] sec. 2 step 4;
 * [KZ] sec. 5.1-5.3): n_mat independent omega matrices [r, d], each from
 * ceil(r/d) blocks; block b is Gram-Schmidt of the rows of the d x d
 * Gaussian matrix gauss[m][b] taken in order, and row f is then scaled to the
 * norm of len_gauss[m][f] (a chi(d)-distributed length), or to sqrt(d) when
 * len_gauss is NULL.  The last block is cut at r rows.  The random draws are
 * the caller's (any generator); this call only does the arithmetic, in
 * float64 (classical Gram-Schmidt with one reorthogonalisation pass, equal
 * to the pages' procedure in exact arithmetic), then rounds to the output
 * dtype through float32 (nearest-even at each step).
 *   gauss      float32 [n_mat, ceil(r/d), d, d]
 *   len_gauss  float32 [n_mat, ceil(r/d) * d, d] or NULL
 *   omega      [n_mat, r, d], dtype LIN_ATTN_F32 or LIN_ATTN_BF16
 * Returns -1 for a null or misaligned pointer, a negative size or a bad
 * dtype, -2 for d > 64; r = 0 or n_mat = 0 is a no-op.  No workspace.
 */
int lin_attn_orf_omega(const float* gauss, const float* len_gauss, int64_t n_mat, int64_t r,
                       int64_t d, int32_t dtype, void* omega, void* stream);

/*
 * Causal prefill and bidirectional attention from the tokens ([KZ] sec.
 * 1.2 step 1: k, v, q = W_k x, W_v x, W_q x for every token x), then exactly
 * lin_attn_causal_chunked (state_in, S, z as there) or lin_attn_bidir
 * (S_out, z_out as there).  Two routes, by configuration:
 *   FAVOR+ with r = 256 and no sum normalisation (the matrix-core
 *   configuration): one projection GEMM writes q, k, v (rounded to
 *   bfloat16, as lin_attn_qkv_project does) into the workspace, then the
 *   matrix-core kernels run on them;
 *   every other map: the vector kernels compute q, k and v in float32 from
 *   x and W inside their loads, chunk by chunk, never writing them out.
 *   x              [B, N, d_model] bfloat16 tokens.
 *   w_q, w_k, w_v  [H * d, d_model] bfloat16 each (out = W x, the layout of a
 *                  linear layer's weight): row h*d + i gives feature i of
 *                  head h.
 *   out            [B, H, N, dv] bfloat16.
 *   d_model        a multiple of 16, at most 65536 (else -2).
 * lin_attn_params.dtype must be LIN_ATTN_BF16 (float32 returns -2).
 *   ws   at least lin_attn_workspace_bytes(LIN_ATTN_OP_CAUSAL_PROJ or
 *        LIN_ATTN_OP_BIDIR_PROJ, p, B, H, N, d, dv, 0) bytes (on the
 *        matrix-core route this includes 3 B H N d bfloat16 for q, k, v).
 * Errors as lin_attn_causal_chunked / lin_attn_bidir; x, w_q, w_k, w_v must
 * be 16-byte aligned.
 */
int lin_attn_causal_proj(const lin_attn_params* p, const void* x, const void* w_q,
                         const void* w_k, const void* w_v, int64_t B, int64_t H, int64_t N,
                         int64_t d_model, int64_t d, int64_t dv, const void* omega, float* S,
                         float* z, int32_t state_in, void* out, void* ws, size_t ws_bytes,
                         void* stream);
int lin_attn_bidir_proj(const lin_attn_params* p, const void* x, const void* w_q,
                        const void* w_k, const void* w_v, int64_t B, int64_t H, int64_t N,
                        int64_t d_model, int64_t d, int64_t dv, const void* omega, void* out,
                        float* S_out, float* z_out, void* ws, size_t ws_bytes, void* stream);

/*
 * The q/k/v input projection alone ([KZ] sec. 1.2 step 1), written in the
 * head-major layout the other calls read: for every token x of x
 * [B, N, d_model] (bfloat16),
 *   q[b, h, t, :] = W_q[h*d : h*d + d, :] x[b, t, :]   (likewise k with w_k, v with w_v),
 * one matrix-core GEMM with float32 accumulation, results rounded to
 * bfloat16 (nearest-even).  w_q, w_k, w_v [H * d, d_model] bfloat16; q, k, v
 * [B, H, N, d] bfloat16, overwritten.  Followed by lin_attn_causal_chunked or
 * lin_attn_bidir this is the unfused route from tokens: q, k, v make one
 * round trip through memory, in the layout the attention kernels read, with
 * no transpose between.  d must be 64 and d_model a multiple of 16 (at most
 * 65536), else -2; -1 for a null or misaligned pointer or a negative size.
 * No workspace.
 */
int lin_attn_qkv_project(const void* x, const void* w_q, const void* w_k, const void* w_v,
                         int64_t B, int64_t N, int64_t d_model, int64_t H, int64_t d, void* q,
                         void* k, void* v, void* stream);

/*
 * Backward pass: the gradients dq, dk, dv of a loss L given dout = dL/dout
 * for the outputs of lin_attn_bidir (lin_attn_bidir_backward) or of
 * lin_attn_causal_chunked from zero state (lin_attn_causal_backward), same
 * parameters and inputs.  [RF] par. 6 asks for gradient error to be
 * evaluated; the derivatives are the chain rule through the definitions of
 * those calls.  With D_i = max(den_i, eps):
 *   dnum_i = dout_i / D_i, dden_i = -(dout_i . out_i) / D_i where den_i > eps,
 *   0 where the clamp holds (NORM_NONE: dnum_i = dout_i, dden_i = 0);
 *   dphi(q_i) = S_i dnum_i + z_i dden_i, with (S_i, z_i) the state query i reads;
 *   dphi(k_j) = G_j v_j + g_j and dv_j = G_j^T phi(k_j), with (G_j, g_j) the
 *   sum of (phi(q_i) dnum_i^T, phi(q_i) dden_i) over the queries that see
 *   key j (every query; causal: i >= j);
 *   dx = scale * J_phi(scale * x)^T dphi(x) for x = q_i, k_j, through the
 *   sum normalisation when it is on.
 * omega is a constant ([PF] sec. 2: sampled once and frozen): no gradient.
 *   q, k, dq, dk [B, H, N, d]; v, dout, dv [B, H, N, dv]; all of the input
 *   dtype.  States and sums are float32; bfloat16 FAVOR+ at r = 256 takes its
 *   products on the matrix cores with bfloat16 operands (the feature maps,
 *   dnum, w = dphi o phi, the states rounded once per product), every other
 *   configuration computes in float32.  dq, dk, dv are overwritten.
 *   ws  at least lin_attn_workspace_bytes(LIN_ATTN_OP_BIDIR_BACKWARD or
 *       LIN_ATTN_OP_CAUSAL_BACKWARD, ...) bytes; contents on entry ignored.
 * Errors as lin_attn_bidir.
 */
int lin_attn_bidir_backward(const lin_attn_params* p, const void* q, const void* k,
                            const void* v, const void* dout, int64_t B, int64_t H, int64_t N,
                            int64_t d, int64_t dv, const void* omega, void* dq, void* dk,
                            void* dv_out, void* ws, size_t ws_bytes, void* stream);
int lin_attn_causal_backward(const lin_attn_params* p, const void* q, const void* k,
                             const void* v, const void* dout, int64_t B, int64_t H, int64_t N,
                             int64_t d, int64_t dv, const void* omega, void* dq, void* dk,
                             void* dv_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Workspace bytes needed by lin_attn_bidir (op = LIN_ATTN_OP_BIDIR),
 * lin_attn_causal_chunked (op = LIN_ATTN_OP_CAUSAL) or, with B = num_seqs and
 * N = total, lin_attn_causal_varlen (op = LIN_ATTN_OP_CAUSAL_VARLEN), and
 * the backward calls (LIN_ATTN_OP_BIDIR_BACKWARD, LIN_ATTN_OP_CAUSAL_BACKWARD) and
 * the projected calls (LIN_ATTN_OP_CAUSAL_PROJ, LIN_ATTN_OP_BIDIR_PROJ).
 * `chunk` is checked for LIN_ATTN_OP_CAUSAL as lin_attn_causal_chunked
 * checks it and ignored for the other operations.
 * Host-only, deterministic in its arguments (independent of the device).
 * Returns 0 for invalid or unsupported arguments.
 */
size_t lin_attn_workspace_bytes(int32_t op, const lin_attn_params* p, int64_t B, int64_t H,
                                int64_t N, int64_t d, int64_t dv, int32_t chunk);

/* Static, NUL-terminated description of a return code. */
const char* lin_attn_strerror(int32_t code);

/* LIN_ATTN_ABI_VERSION of the built library. */
int32_t lin_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIN_ATTN_H */
