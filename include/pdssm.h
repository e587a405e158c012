/*
 * pdssm.h -- C ABI of the Flash PD-SSM forward recurrence scan on MI355X (gfx950).
 *
 * The operation (source: "Flash PD-SSM: Memory-Optimized Structured Sparse
 * State-Space Models", gist.science explainer, Technical Summary):
 *
 *   Methodology, "1. Novel Selection Mechanism (Hard Selection)": a dictionary
 *   of K sparse matrices is fixed in advance; at each step the K scores pick
 *   one of them by argmax and it is used directly.  The picked matrix is a
 *   one-hot column selector P (column j has its single 1 in row pi[j]) times a
 *   diagonal D, so a step costs O(N) and no N x N matrix is ever formed.
 *
 *   Methodology, "3. Hardware-Aware Implementation": the sequence is cut into
 *   chunks; recurrences run independently inside chunks, a prefix scan over
 *   chunk aggregates gives the carry states, and the carries correct the
 *   chunk states.  "Sequential-Parallel Duality in Prefix Scannable Models"
 *   (fugumt.com listing, abstract) frames such models as a parallel prefix
 *   scan with a custom associative operator; here that operator composes two
 *   P D operators by a gather and a multiply.
 *
 *   For every sequence (b,h), with x_{-1} = x0[b,h] (zero when x0 is NULL):
 *       k_t = sel[b,h,t]                      (index modes), or
 *       k_t = argmax_k logits[b,h,t,k]        (logit modes; first maximum wins,
 *                                               -0 == +0, NaN above all numbers,
 *                                               first NaN wins)
 *       pi  = dict_idx[h, k_t, :]
 *       x_t[i] = sum_{j : pi[j] = i} diag[b,h,t,j] * x_{t-1}[j]  +  b[b,h,t,i]
 *       y[b,h,t] = Re( sum_i c[b,h,t,i] * x_t[i] )     (no conjugation)
 *   and x_final[b,h] = x_{L-1}.
 *
 * Arithmetic: fp32 (complex fp32 when PDSSM_COMPLEX), any summation order;
 * y is rounded once to its storage type (round to nearest even).
 *
 * Layouts: contiguous, row-major, DEVICE pointers, each 16-byte aligned.
 *   sel      int32 or int16          [B,H,L]
 *   logits   fp32 or bf16            [B,H,L,K]
 *   dict_idx int32                   [H,K,N], entries in [0,N)
 *   diag     fp32                    [B,H,L,N], or [B,H,L,N,2] complex (re,im interleaved)
 *   b, c     fp32 or bf16            same shape as diag
 *   y        fp32 or bf16            [B,H,L]
 *   x0, x_final fp32                 [B,H,N], or [B,H,N,2] complex
 * A dictionary shared by all heads is passed replicated over H.
 *
 * Ownership: the caller owns every buffer, including the workspace, whose
 * size comes from pdssm_scan_workspace_bytes and grows as O(B*H*L*N / 128),
 * never with N*N*L.  The library allocates nothing and keeps no per-call
 * state; the workspace may hold anything on entry (the library recognises
 * its own header and clears the rest on first use).  Two calls in flight at
 * once need two workspaces.
 *
 * Execution: asynchronous on `stream`; no host synchronisation.  Outputs are
 * valid once the stream has reached the end of the call; inputs must stay
 * unchanged until then.
 *
 * Errors: 0 on success, else a negative PDSSM_ERR_* code; every check except
 * PDSSM_ERR_HIP runs on the host before any HIP call.  Element values are
 * preconditions: a selection outside [0,K) or a map entry outside [0,N) is
 * clamped into range on the device (no fault, result unspecified).
 *
 * Empty shapes: B, H and L may be 0 (N and K may not).  Sizes and flags are
 * still checked.  With no sequences (B*H = 0) every buffer is empty: the
 * call returns 0 and reads none of its pointers, which may be NULL.  With
 * sequences of no steps (L = 0) the state after no steps is the initial one,
 * so x_final = x0 (zero without x0) is written when x_final is given; every
 * per-step buffer and the workspace are empty and not read.  Every entry
 * point below follows the same rule for its own sizes.
 */
#ifndef PDSSM_H
#define PDSSM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* flags: selection storage (2 bits) */
#define PDSSM_SEL_I32 0x0u     /* sel int32 [B,H,L] */
#define PDSSM_SEL_I16 0x1u     /* sel int16 [B,H,L] */
#define PDSSM_LOGITS_F32 0x2u  /* logits fp32 [B,H,L,K] */
#define PDSSM_LOGITS_BF16 0x3u /* logits bf16 [B,H,L,K] */
#define PDSSM_SEL_MASK 0x3u
/* flags: value storage */
#define PDSSM_COMPLEX 0x4u /* diag, b, c, x0, x_final complex (re,im pairs) */
#define PDSSM_BC_BF16 0x8u /* b and c stored as bf16 (else fp32) */
#define PDSSM_Y_BF16 0x10u /* y stored as bf16 (else fp32) */
/* Bitwise reproducible results (pdssm_scan_fwd and its variants, and
 * pdssm_scan_bwd): the carry into every tile of steps is taken from the
 * tile just before it (just after it, in the backward), once that tile's own
 * carry is known, so the same operations run in the same order on every
 * call.  Without the flag the library takes the carry the same way when the
 * batch holds enough sequences to keep the device busy (at most 12 resident
 * workgroups per sequence in the forward, 4 in the backward), which is also
 * the faster way there.  With fewer sequences a tile may compose its carry
 * from the records of several earlier tiles, whichever are ready first,
 * which changes the fp32 rounding order from call to call; there the flag
 * is slower, as the carry advances along a sequence by about one tile per
 * microsecond. */
#define PDSSM_DETERMINISTIC 0x20u
#define PDSSM_FLAGS_ALL 0x3Fu

/* pdssm_router_select only: w is in the packed layout that
 * pdssm_router_pack_weights writes. */
#define PDSSM_ROUTER_W_PACKED 0x1u

/* status codes */
#define PDSSM_OK 0
#define PDSSM_ERR_NULL -1      /* a required pointer is NULL */
#define PDSSM_ERR_DIM -2       /* B,H,L < 0, L > 2^30, N not in [1,64], K not in [1,32767], or too large */
#define PDSSM_ERR_FLAGS -3     /* unknown flag bits, or a mode the call does not take */
#define PDSSM_ERR_ALIGN -4     /* a pointer is not 16-byte aligned */
#define PDSSM_ERR_WORKSPACE -5 /* workspace smaller than the size function returns */
#define PDSSM_ERR_HIP -6       /* a HIP launch failed; pdssm_strerror gives the HIP text */
#define PDSSM_ERR_SCRATCH -7   /* pdssm_scan_fwd_noalloc: the sizes need more than its scratch holds */

/*
 * The forward scan (all five steps of the path: selection, per-step P D
 * update, in-chunk composition, chunk carry, fused readout).
 *   sel_or_logits  selection input, storage given by flags & PDSSM_SEL_MASK
 *   dict_idx       dictionary index maps
 *   diag, b, c     per-step diagonal, input and readout vectors
 *   y              output readout
 *   x_final        output final state, or NULL
 *   x0             initial state, or NULL for zero
 *   workspace      device buffer of workspace_bytes bytes (see above)
 */
int pdssm_scan_fwd(const void *sel_or_logits, const int32_t *dict_idx, const void *diag,
                   const void *b, const void *c, void *y, void *x_final, int64_t B, int64_t H,
                   int64_t L, int32_t N, int32_t K, uint32_t flags, const void *x0,
                   void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes pdssm_scan_fwd and pdssm_compose need for these sizes and
 * flags; 0 when the arguments are invalid. */
size_t pdssm_scan_workspace_bytes(int64_t B, int64_t H, int64_t L, int32_t N, int32_t K,
                                  uint32_t flags);

/*
 * pdssm_scan_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same operation, arguments and errors, without the workspace.  Its
 * workspace is a 64 MiB array of device memory held by the library on every
 * GPU it runs on until the process ends (enough for B*H*L*N up to about
 * 10^8 complex steps at N = 64; pdssm_scan_workspace_bytes gives the need).
 * Sizes whose workspace would not fit return PDSSM_ERR_SCRATCH before any HIP
 * call.  The call allocates nothing (no hipMalloc or allocating library
 * routine); it finds the array's device address once per device.  Every
 * call on one GPU shares that GPU's array: calls that overlap in time on the
 * same GPU (on different streams, or from different host threads) race and
 * give undefined results; calls in sequence on one stream are safe.
 */
int pdssm_scan_fwd_noalloc(const void *sel_or_logits, const int32_t *dict_idx, const void *diag,
                           const void *b, const void *c, void *y, void *x_final, int64_t B,
                           int64_t H, int64_t L, int32_t N, int32_t K, uint32_t flags,
                           const void *x0, hipStream_t stream);

/*
 * pdssm_scan_fwd that also keeps what pdssm_scan_bwd needs: the state just
 * before every chunk of 16 steps, and optionally every step's selection.
 *   x_chunks  fp32 [B,H,ceil(L/16),N], or [B,H,ceil(L/16),N,2] with
 *             PDSSM_COMPLEX:  x_chunks[b,h,c] = x_{16c-1}  (x0, or zero, for
 *             c = 0); caller-owned, 16-byte aligned, not NULL
 *   sel_out   int16 [B,H,L]: the dictionary entry each step selected (the
 *             argmax of its scores in the logits modes), or NULL.  Passed to
 *             pdssm_scan_bwd with PDSSM_SEL_I16 in place of the scores, it
 *             spares the backward the K scores per step.
 * Every other argument, the workspace size and the errors as pdssm_scan_fwd.
 */
int pdssm_scan_fwd_save(const void *sel_or_logits, const int32_t *dict_idx, const void *diag,
                        const void *b, const void *c, void *y, void *x_final, void *x_chunks,
                        int16_t *sel_out, int64_t B, int64_t H, int64_t L, int32_t N, int32_t K,
                        uint32_t flags, const void *x0, void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * Gradients of the forward scan (reverse mode), the pass training needs.
 * Methodology, "1. Novel Selection Mechanism (Hard Selection)": training
 * goes through the hard selection; the pages name a straight-through
 * estimator for the scores but print no formula, so the selection (and the
 * dictionary) get no gradient here.  For a real loss with dL/dy[b,h,t] = gy
 * and dL/dx_final = gx_final, complex gradients written dL/dRe + i dL/dIm,
 * and A_t = P_t D_t as in pdssm_scan_fwd:
 *     lambda_{L-1} = gy_{L-1} conj(c_{L-1}) + gx_final
 *     lambda_t     = gy_t conj(c_t) + A_{t+1}^H lambda_{t+1},
 *                    (A^H l)[j] = conj(d[j]) l[pi[j]]
 *     gb[t] = lambda_t
 *     gc[t] = gy_t conj(x_t)
 *     gd[t][j] = conj(x_{t-1}[j]) lambda_t[pi_t[j]]
 *     gx0 = A_0^H lambda_0
 * Inputs: the forward's sel_or_logits, dict_idx, diag, b, c and flags (or
 *   the forward's saved int16 selections with the selection bits of flags
 *   set to PDSSM_SEL_I16); x_chunks from pdssm_scan_fwd_save on the same
 *   inputs (and x0);
 *   gy [B,H,L] in the storage of y (bf16 with PDSSM_Y_BF16, else fp32);
 *   gx_final fp32 [B,H,N(,2)], or NULL for zero.
 * Outputs (caller-owned, 16-byte aligned): gb and gc in the storage of b and
 *   c (bf16, rounded to nearest even, with PDSSM_BC_BF16, else fp32), gd in
 *   the storage of diag, gx0 fp32 [B,H,N(,2)] or NULL when not wanted.
 * Arithmetic fp32 (complex fp32), any summation order: the adjoint carried
 * between chunks of 16 steps is composed in an order that depends on timing,
 * so repeated calls may differ in the last bits (and a bf16 output by one
 * rounding step).  The adjoint carried between tiles is waited for without
 * a time bound, as the forward's carry is: a workgroup takes its tile ticket
 * when it starts and only waits for tiles of earlier tickets, so the call
 * always completes and never uses a partial carry.  Workspace sized by
 * pdssm_scan_bwd_workspace_bytes; as for pdssm_scan_fwd it may hold anything
 * on entry, and two calls in flight at once need two workspaces.  Errors and
 * empty shapes as pdssm_scan_fwd; with L = 0, gx0 = gx_final (zero without
 * it) is written when gx0 is given.
 */
int pdssm_scan_bwd(const void *sel_or_logits, const int32_t *dict_idx, const void *diag,
                   const void *b, const void *c, const void *x_chunks, const void *gy,
                   const void *gx_final, void *gb, void *gc, void *gd, void *gx0, int64_t B,
                   int64_t H, int64_t L, int32_t N, int32_t K, uint32_t flags, void *workspace,
                   size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes pdssm_scan_bwd needs: 3.5 KB (2 KB real) per 64 steps
 * of every sequence (one carry record per 64 steps, O(B*H*L), never N*N*L),
 * plus the dictionary's entry table; 0 when the arguments are invalid (a
 * positive size for valid empty shapes). */
size_t pdssm_scan_bwd_workspace_bytes(int64_t B, int64_t H, int64_t L, int32_t N, int32_t K,
                                      uint32_t flags);

/*
 * Dictionary pre-compute: the index maps from dense matrices.  Flash PD-SSM
 * summary, Methodology, "1. Novel Selection Mechanism (Hard Selection)": a
 * column-wise hardmax of each dense N x N dictionary matrix leaves a single
 * non-zero per column, a one-hot column selector.  For every entry (h,k) and
 * column j:
 *     dict_idx[h,k,j] = argmax_i m[h,k,i,j]
 * with the selection's rule (the first maximum wins, -0 equals +0, a NaN
 * counts above every number and the first NaN wins).
 *   m         dense matrices [H,K,N,N], row-major (row i, column j); fp32 with
 *             flags = PDSSM_LOGITS_F32, bf16 with PDSSM_LOGITS_BF16 (no other
 *             bits); device pointer, 16-byte aligned
 *   dict_idx  int32 [H,K,N] output, device pointer, 16-byte aligned
 * Errors: PDSSM_ERR_NULL, PDSSM_ERR_DIM (H < 0, N not in [1,64], K not in
 * [1,32767]), PDSSM_ERR_FLAGS, PDSSM_ERR_ALIGN, PDSSM_ERR_HIP; H = 0 writes
 * nothing.  Asynchronous on stream; allocates nothing.
 */
int pdssm_dict_hardmax(const void *m, int32_t *dict_idx, int64_t H, int32_t K, int32_t N,
                       uint32_t flags, hipStream_t stream);

/*
 * One recurrent decode step for every sequence (b,h): the scan with L = 1,
 * the state carried by the caller between calls (the recurrent inference
 * mode the Flash PD-SSM summary names for state-space models, Problem
 * Statement).  With k the step's selection and pi = dict_idx[h,k,:]:
 *     x[b,h] <- P (d * x[b,h]) + b,   y[b,h] = Re(sum_i c[i] x[b,h,i])
 * (x on the right is the state before the call).
 *   sel_or_logits  sel int32/int16 [B,H] or logits fp32/bf16 [B,H,K]
 *   diag, b, c     [B,H,N] or [B,H,N,2] (complex), storages as in
 *                  pdssm_scan_fwd
 *   y              [B,H] output (bf16 with PDSSM_Y_BF16, else fp32)
 *   x              fp32 [B,H,N(,2)] state, read and overwritten in place
 *   flags          as pdssm_scan_fwd
 * Arithmetic fp32; collisions of pi sum in any order.  All pointers are
 * device pointers, 16-byte aligned, not NULL (unless B*H = 0, which writes
 * nothing).  Errors as pdssm_scan_fwd (no workspace).  Asynchronous on
 * stream; allocates nothing.
 */
int pdssm_decode_step(const void *sel_or_logits, const int32_t *dict_idx, const void *diag,
                      const void *b, const void *c, void *y, void *x, int64_t B, int64_t H,
                      int32_t N, int32_t K, uint32_t flags, hipStream_t stream);

/*
 * Router selection fused with its matrix product: the scores never reach
 * memory, only the selected entries do.  Flash PD-SSM summary, Methodology,
 * "1. Novel Selection Mechanism (Hard Selection)": at every step the input
 * u_t produces the K scores by a linear transformation and the largest picks
 * the dictionary entry.  With one K-wide block of weights per head and no
 * bias:
 *     scores[b,h,t,k] = sum_d u[b,t,d] * w[h,k,d]      (fp32 accumulation)
 *     sel_out[b,h,t]  = argmax_k scores[b,h,t,k]       (first maximum wins)
 * The result feeds pdssm_scan_fwd with PDSSM_SEL_I16.
 *   u        bf16 [B,L,D] step inputs
 *   w        bf16 router weights: [H,K,D] (flags 0), or, with
 *            PDSSM_ROUTER_W_PACKED, the packed layout [H][D/8][P][8] of
 *            pdssm_router_pack_weights (P = 64 for K <= 64, else 128), which
 *            the faster of the two kernels reads
 *   sel_out  int16 [B,H,L] output
 *   K in [1,128]; D a positive multiple of 32; flags 0 or
 *   PDSSM_ROUTER_W_PACKED (then H*P*D*2 bytes must stay below 4 GB).  B, L
 *   or H may be 0: nothing is read or written then.
 * The scores are fp32 sums in an unspecified order: where two scores are
 * within their rounding error of each other, either index may be returned
 * (the two layouts may differ there).
 * All pointers are device pointers, 16-byte aligned.  Errors:
 * PDSSM_ERR_NULL, PDSSM_ERR_DIM, PDSSM_ERR_FLAGS, PDSSM_ERR_ALIGN,
 * PDSSM_ERR_HIP.  Asynchronous on stream; allocates nothing.
 */
int pdssm_router_select(const void *u, const void *w, int16_t *sel_out, int64_t B, int64_t L,
                        int64_t H, int32_t K, int32_t D, uint32_t flags, hipStream_t stream);

/*
 * The router weights in the packed layout of pdssm_router_select with
 * PDSSM_ROUTER_W_PACKED: w_packed[h][d/8][k][d%8] = w[h][k][d] for k < K and
 * 0 for K <= k < P (P = 64 for K <= 64, else 128), so the 32 score columns
 * of an 8-feature block are 512 contiguous bytes.  It depends on the
 * weights only: pack once per weight update.
 *   w         bf16 [H,K,D]
 *   w_packed  bf16 [H, D/8, P, 8] output (H*P*D*2 bytes, below 4 GB)
 *   K in [1,128]; D a positive multiple of 32; H = 0 writes nothing.
 * Device pointers, 16-byte aligned.  Errors: PDSSM_ERR_NULL, PDSSM_ERR_DIM,
 * PDSSM_ERR_ALIGN, PDSSM_ERR_HIP.  Asynchronous on stream; allocates nothing.
 */
int pdssm_router_pack_weights(const void *w, void *w_packed, int64_t H, int32_t K, int32_t D,
                              hipStream_t stream);

/*
 * The selection step alone: sel_out[b,h,t] = the dictionary entry step t
 * picks (Methodology, "1. Novel Selection Mechanism": argmax of the K
 * scores; index modes copy the index).  flags: selection bits only.
 */
int pdssm_select(const void *sel_or_logits, int32_t *sel_out, int64_t B, int64_t H, int64_t L,
                 int32_t K, uint32_t flags, hipStream_t stream);

/*
 * The total operator A_{L-1} ... A_0 of every sequence, which is again a
 * one-hot column selector times a diagonal (Methodology, "1. Novel Selection
 * Mechanism": the matrices stay sparse; the composition is the chunk
 * aggregate of "3. Hardware-Aware Implementation", Phase B, over the whole
 * sequence).  Column j of the product has d_out[b,h,j] in row pi_out[b,h,j].
 *   pi_out  int32 [B,H,N]
 *   d_out   fp32  [B,H,N], or [B,H,N,2] with PDSSM_COMPLEX
 * flags: selection bits and PDSSM_COMPLEX.  The workspace is sized by
 * pdssm_scan_workspace_bytes with the same arguments.  With L = 0 the
 * product is the identity (pi_out[j] = j, d_out[j] = 1), written without
 * reading the inputs or the workspace.
 */
int pdssm_compose(const void *sel_or_logits, const int32_t *dict_idx, const void *diag,
                  int32_t *pi_out, void *d_out, int64_t B, int64_t H, int64_t L, int32_t N,
                  int32_t K, uint32_t flags, void *workspace, size_t workspace_bytes,
                  hipStream_t stream);

/* Text for a status code; for PDSSM_ERR_HIP, the HIP error of the failing
 * call on this thread.  The string stays valid until the next call on this
 * thread. */
const char *pdssm_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* PDSSM_H */
