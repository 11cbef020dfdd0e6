/*
 * attn_bwd.h - attention backward for AMD Instinct MI355X (gfx950).
 *
 * The operation: the gradients of the forward in attn_fwd.h with respect to q, k and v,
 * given the gradient dout of its output o. The pages list the attention backward among
 * the kernels written with the ThunderKittens tile library (the paper summary on
 * groovesquid.com) without giving its formulas; this is the chain rule applied to the
 * forward's definition. For every batch b, head h (indices dropped) and rows i, j:
 *
 *   P_ij    = exp(scale * q_i . k_j - lse_i)   for j in J_i (see attn_fwd.h), else 0
 *   dv_j    = sum_i P_ij dout_i
 *   dP_ij   = dout_i . v_j
 *   Delta_i = sum_d dout_id o_id                (= sum_j P_ij dP_ij)
 *   dS_ij   = P_ij (dP_ij - Delta_i)
 *   dq_i    = scale * sum_j dS_ij k_j
 *   dk_j    = scale * sum_i dS_ij q_i
 *
 * lse and o are the forward's outputs for the same q, k, v, causal and scale. The
 * probabilities are recomputed tile by tile (no N x N matrix reaches memory); dS and P
 * enter the matrix products rounded to bf16, with fp32 accumulation; dq, dk, dv are
 * rounded to bf16 (round to nearest even) after the fp32 scaling.
 */
#ifndef ATTN_BWD_H
#define ATTN_BWD_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define ATTN_BWD_OK            0   /* success: the kernels were enqueued on the stream       */
#define ATTN_BWD_EINVAL       -1   /* NULL pointer; B, H or N < 1; causal not 0/1; scale not
                                      finite or <= 0; sizes that overflow the kernels'
                                      indexing (N*D >= 2^31, B*H*ceil(N/64) >= 2^31
                                      workgroups, or B*H*N*D/8 >= 2^31)                     */
#define ATTN_BWD_EUNSUPPORTED -2   /* head dimension D other than 64 or 128                  */
#define ATTN_BWD_EALIGN       -3   /* a tensor not 16-byte aligned, lse not 4-byte, or the
                                      workspace not 256-byte aligned                         */
#define ATTN_BWD_ELAUNCH      -4   /* hipGetLastError() was set after the launches (this also
                                      reports, and clears, an error left pending by an
                                      earlier HIP call on the calling thread)                 */
#define ATTN_BWD_EWORKSPACE   -5   /* workspace_bytes < attn_bwd_workspace_bytes(B, H, N)    */

/*
 * attn_bwd_workspace_bytes - device workspace attn_bwd needs for these sizes: two fp32
 * values per row (B*H*N rows), each array rounded up to 256 bytes. 0 if a size is < 1.
 */
size_t attn_bwd_workspace_bytes(int B, int H, int N);

/*
 * attn_bwd - enqueue the attention backward of all B*H heads on one HIP stream.
 *
 *   q, k, v, o, dout  device pointers, bf16, contiguous [B, H, N, D]. Read only.
 *   lse               device pointer, fp32, contiguous [B, H, N] (natural log). Read only.
 *   dq, dk, dv        device pointers, bf16, contiguous [B, H, N, D]. Written in full.
 *                     Must not overlap each other or any input.
 *   workspace         device pointer to workspace_bytes of scratch (256-byte aligned),
 *                     owned by the caller; its contents on entry do not matter and are
 *                     overwritten. Must not overlap any tensor.
 *   B, H, N, D, causal, scale   as in attn_fwd (D is 64 or 128).
 *   stream            a hipStream_t passed as void*; NULL is the default stream.
 *
 * Ownership: the caller owns every buffer, including the workspace. The library allocates
 * no device memory and keeps no state between calls, so calls on different streams may
 * run concurrently as long as they use different workspaces and outputs.
 *
 * Behaviour: arguments are validated on the host before any HIP call; an invalid call
 * returns a negative code and enqueues nothing. A valid call enqueues three kernels (the
 * per-row Delta, then dk/dv, then dq) and returns without synchronising; device errors
 * are reported by the HIP runtime on the stream. Nothing is printed.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, void* workspace,
             size_t workspace_bytes, int B, int H, int N, int D, int causal, float scale,
             void* stream);

/* attn_bwd_strerror - a static, NUL-terminated description of a return code. */
const char* attn_bwd_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_BWD_H */
