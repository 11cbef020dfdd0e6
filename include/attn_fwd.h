/*
 * attn_fwd.h - fused softmax attention forward for AMD Instinct MI355X (gfx950).
 *
 * The operation (the attention forward of the ThunderKittens pages: the warp-level
 * attention inner loop on the alanwu.xyz blog, and the H100 attention listing in the
 * 10100.com review, section on writing attention with TK; causal masking and the
 * logsumexp output are additions those pages do not show):
 *
 *   for every batch b < B, head h < H and query row i < N:
 *     s_ij   = scale * sum_d q[b,h,i,d] * k[b,h,j,d]
 *     J_i    = { 0 .. N-1 }            (causal == 0)
 *            = { 0 .. i }              (causal == 1: lower-triangular mask, diagonal kept)
 *     o[b,h,i,:] = sum_{j in J_i} exp(s_ij) v[b,h,j,:] / sum_{j in J_i} exp(s_ij)
 *     lse[b,h,i] = ln sum_{j in J_i} exp(s_ij)        (natural log, of the scaled scores)
 *
 * computed tile by tile with an online softmax, so the N x N score matrix never reaches
 * memory. Scores and all softmax state are fp32; the probabilities are rounded to bf16
 * (round to nearest even) for the P*V product, whose accumulation is fp32; O is rounded
 * to bf16 (round to nearest even) at the end.
 */
#ifndef ATTN_FWD_H
#define ATTN_FWD_H

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define ATTN_FWD_OK            0   /* success: the kernel was enqueued on the stream        */
#define ATTN_FWD_EINVAL       -1   /* NULL pointer; B, H or N < 1; causal not 0/1; scale not
                                      finite or <= 0; sizes that overflow the kernel's
                                      indexing (N*D >= 2^31, or B*H*ceil(N/128) >= 2^31
                                      workgroups)                                           */
#define ATTN_FWD_EUNSUPPORTED -2   /* head dimension D other than 64 or 128                  */
#define ATTN_FWD_EALIGN       -3   /* q, k, v or o not 16-byte aligned, or lse not 4-byte    */
#define ATTN_FWD_ELAUNCH      -4   /* hipGetLastError() was set after the launch (this also
                                      reports, and clears, an error left pending by an
                                      earlier HIP call on the calling thread)                 */

/*
 * attn_fwd - enqueue the attention forward of all B*H heads on one HIP stream.
 *
 *   q, k, v  device pointers, bf16 (bfloat16 bit patterns), contiguous [B, H, N, D]
 *            (D innermost). Read only. 16-byte aligned.
 *   o        device pointer, bf16, contiguous [B, H, N, D]. Written for every row.
 *            16-byte aligned. Must not overlap q, k, v or lse.
 *   lse      device pointer, fp32, contiguous [B, H, N]. Written for every row.
 *   B, H, N  batch, heads, sequence length (queries == keys), each >= 1. Any N >= 1 is
 *            valid: a ragged last tile is masked, never read out of bounds.
 *   D        head dimension, 64 or 128.
 *   causal   0: every key is visible; 1: key j is visible to query i iff j <= i.
 *   scale    score multiplier, finite and > 0 (the usual value is 1/sqrt(D)).
 *   stream   a hipStream_t passed as void*; NULL is the default stream.
 *
 * Ownership: the caller owns every buffer. The library allocates no device memory, keeps
 * no state between calls, and may be called concurrently from several host threads on
 * different streams. The kernel is chosen by shape: ping-pong for D = 128; for D = 64,
 * ping-pong when causal == 0 and B * H * ceil(N / 512) is at least the compute-unit count
 * of the current device (queried once per device), else four-wave. Both give identical
 * results. The library reads no environment variable.
 *
 * Behaviour: arguments are validated on the host before any HIP call; an invalid call
 * returns a negative code and enqueues nothing. A valid call enqueues one kernel and
 * returns without synchronising (ATTN_FWD_ELAUNCH also covers a failed query of the
 * compute-unit count); errors raised later by the device are reported by the
 * HIP runtime on the stream, not by this function. Nothing is printed.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int N, int D, int causal, float scale, void* stream);

/* Kernel selectors of attn_fwd_ex. */
#define ATTN_FWD_KERNEL_AUTO      0   /* attn_fwd's choice by shape                          */
#define ATTN_FWD_KERNEL_PINGPONG  1   /* 8 waves, 256 queries per workgroup (512 at D = 64
                                         without the mask), two wave groups alternating
                                         matrix and vector phases on each SIMD              */
#define ATTN_FWD_KERNEL_FOURWAVE  2   /* 4 waves, 128 queries per workgroup, each wave
                                         interleaving its MFMAs and exponentials            */

/*
 * attn_fwd_ex - attn_fwd with the kernel chosen by the caller, for tests and tuning. Same
 * operation, arguments, ownership and behaviour as attn_fwd; kernel is one of the
 * ATTN_FWD_KERNEL_* selectors (anything else is ATTN_FWD_EINVAL). Both kernels run every
 * valid shape and perform the same per-row arithmetic in the same order, so they return
 * bit-identical o and lse.
 */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int N, int D, int causal, float scale, int kernel, void* stream);

/* attn_fwd_strerror - a static, NUL-terminated description of a return code. */
const char* attn_fwd_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_H */
