/*
 * based_fwd.h - Based linear attention forward (causal) for AMD Instinct MI355X (gfx950).
 *
 * The operation: "ThunderKittens 2.0: Faster Kernels, Talking Models, and More Adorable
 * Kittens" (thebeat.tech), sections "New Kernels for Enhanced Performance" and
 * "Performance Benchmarks", lists Based linear attention among the library's new
 * kernels without giving its formulas. The reading implemented is the published Based
 * design, causal linear attention with the second-order Taylor feature map of
 * exp(q.k / sqrt(d)) and the linear-attention normaliser. For every batch b, head h
 * (indices dropped) and token i:
 *
 *   s_ij = (q_i . k_j) / sqrt(d)                  (d = 16)
 *   w_ij = 1 + s_ij + s_ij^2 / 2                  for j <= i
 *   o_i  = sum_{j <= i} w_ij v_j / sum_{j <= i} w_ij
 *
 * w_ij >= 1/2, so the normaliser is never zero. The kernel evaluates this in linear time,
 * in chunks of 64 tokens, with running sums of the feature map
 * phi(x) = [1, x / 2, vec(x x^T) / (4 sqrt 2)] (phi(q) . phi(k) = w): bf16 operands,
 * fp32 accumulation, the normaliser's running sums in fp32, output rounded to bf16
 * (round to nearest even).
 */
#ifndef BASED_FWD_H
#define BASED_FWD_H

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define BASED_OK            0   /* success: the kernel was enqueued on the stream          */
#define BASED_EINVAL       -1   /* NULL pointer; B, H or N < 1; N*dv*2 >= 2^31 bytes per
                                   head, or B*H >= 2^24                                      */
#define BASED_EUNSUPPORTED -2   /* d other than 16 or dv other than 64                      */
#define BASED_EALIGN       -3   /* q, k, v or o not 16-byte aligned, or the workspace not
                                   256-byte aligned                                          */
#define BASED_ELAUNCH      -4   /* hipGetLastError() was set after the launch (this also
                                   reports, and clears, an error left pending by an earlier
                                   HIP call on the calling thread)                           */

/*
 * based_fwd - enqueue the Based linear attention forward of all B*H heads on one stream.
 *
 *   q, k    device pointers, bf16, contiguous [B, H, N, d] (d innermost). Read only.
 *   v       device pointer, bf16, contiguous [B, H, N, dv]. Read only.
 *   o       device pointer, bf16, contiguous [B, H, N, dv]. Written for every row. Must
 *           not overlap q, k or v.
 *   B, H, N batch, heads, sequence length, each >= 1 (any N; a ragged last chunk is
 *           handled).
 *   d, dv   feature sizes: 16 and 64.
 *   stream  a hipStream_t passed as void*; NULL is the default stream.
 *
 * Ownership: the caller owns every buffer. The library allocates no device memory, keeps
 * no state between calls, and may be called concurrently on different streams.
 *
 * Behaviour: arguments are validated on the host before any HIP call; an invalid call
 * returns a negative code and enqueues nothing. A valid call enqueues one kernel (one
 * workgroup per (batch, head)) and returns without synchronising; device errors are
 * reported by the HIP runtime on the stream. Nothing is printed.
 */
int based_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d,
              int dv, void* stream);

/*
 * based_fwd_workspace_bytes - device workspace that based_fwd_ws needs to split each head's
 * sequence over several workgroups on the current device: fp32 running states of every
 * segment but the last, 163840 bytes per (batch, head, segment). 0 when no split pays
 * (B*H at least the device's compute-unit count, or sequences under 16 chunks of 64
 * tokens) or the device query fails.
 */
size_t based_fwd_workspace_bytes(int B, int H, int N);

/*
 * based_fwd_ws - based_fwd with an optional caller-owned workspace (256-byte aligned; its
 * contents on entry do not matter). With workspace_bytes >= based_fwd_workspace_bytes(B,
 * H, N) > 0, each head's chunks are cut into segments of at least 8 chunks, enough for
 * B*H*segments workgroups to cover the device's compute units: a first kernel sums each
 * segment's contribution to the running state, and the second runs one workgroup per
 * (batch, head, segment), each starting from the sum of the segments before it. Otherwise
 * (NULL or a smaller workspace) it runs as based_fwd. Same arguments, ownership and
 * behaviour as based_fwd otherwise; the split changes only the order of the fp32 sums
 * of the running state (results agree with based_fwd to rounding, not bit for bit).
 * Concurrent calls must use different workspaces.
 */
int based_fwd_ws(const void* q, const void* k, const void* v, void* o, void* workspace,
                 size_t workspace_bytes, int B, int H, int N, int d, int dv, void* stream);

/* based_fwd_strerror - a static, NUL-terminated description of a return code. */
const char* based_fwd_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* BASED_FWD_H */
