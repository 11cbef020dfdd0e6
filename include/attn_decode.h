/*
 * attn_decode.h - decode-shaped attention forward for AMD Instinct MI355X (gfx950): a few
 * query rows against a long key/value sequence (a KV cache).
 *
 * The operation (attention inference, which the ThunderKittens paper summary on
 * groovesquid.com lists next to the training kernels without a shape): for every batch b,
 * head h and query row i < Nq,
 *
 *   s_ij   = scale * sum_d q[b,h,i,d] * k[b,h,j,d]              for j < Nk
 *   J_i    = { 0 .. Nk-1 }                  (causal == 0)
 *          = { 0 .. Nk-Nq+i }               (causal == 1: the queries are the last Nq
 *                                            positions of the sequence)
 *   o[b,h,i,:] = sum_{j in J_i} exp(s_ij) v[b,h,j,:] / sum_{j in J_i} exp(s_ij)
 *   lse[b,h,i] = ln sum_{j in J_i} exp(s_ij)
 *
 * With Nq == Nk this is attn_fwd. The keys are split into chunks processed by separate
 * workgroups (split-KV); each chunk's normalised partial output and lse go to the
 * workspace and a second kernel merges them: lse = ln sum_c exp(lse_c),
 * o = sum_c exp(lse_c - lse) o_c. Scores, softmax state and partials are fp32; the
 * probabilities enter the P V product in bf16; o is rounded to bf16 (nearest even).
 */
#ifndef ATTN_DECODE_H
#define ATTN_DECODE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_DECODE_OK            0   /* success: the kernels were enqueued                  */
#define ATTN_DECODE_EINVAL       -1   /* NULL pointer; B, H, Nq or Nk < 1; causal not 0/1;
                                         causal with Nq > Nk; scale not finite or <= 0;
                                         Nk*D >= 2^31 or B*H >= 2^24                        */
#define ATTN_DECODE_EUNSUPPORTED -2   /* D other than 64 or 128, or Nq > 32                  */
#define ATTN_DECODE_EALIGN       -3   /* q, k, v or o not 16-byte aligned, lse not 4-byte,
                                         workspace not 256-byte aligned                      */
#define ATTN_DECODE_ELAUNCH      -4   /* hipGetLastError() was set after the launches (also
                                         reports, and clears, an earlier pending error)      */
#define ATTN_DECODE_EWORKSPACE   -5   /* workspace_bytes < attn_decode_workspace_bytes(...);
                                         attn_decode_noalloc: that size exceeds
                                         ATTN_DECODE_NOALLOC_MAX_WORKSPACE                 */

/* Size of the fixed device scratch of attn_decode_noalloc: 33 MiB. */
#define ATTN_DECODE_NOALLOC_MAX_WORKSPACE ((size_t)33 << 20)

/*
 * attn_decode_workspace_bytes - device workspace attn_decode needs: the partial outputs
 * and lse of every key chunk (fp32), each array rounded up to 256 bytes. 0 for invalid
 * sizes.
 */
size_t attn_decode_workspace_bytes(int B, int H, int Nq, int Nk, int D);

/*
 * attn_decode - enqueue the decode-shaped attention of all B*H heads on one HIP stream.
 *
 *   q        device pointer, bf16, contiguous [B, H, Nq, D]; 1 <= Nq <= 32. Read only.
 *   k, v     device pointers, bf16, contiguous [B, H, Nk, D]; Nk >= 1. Read only.
 *   o        device pointer, bf16, contiguous [B, H, Nq, D]. Written in full.
 *   lse      device pointer, fp32, contiguous [B, H, Nq]. Written in full.
 *   workspace, workspace_bytes   caller-owned device scratch (256-byte aligned) of at
 *            least attn_decode_workspace_bytes(B, H, Nq, Nk, D) bytes; overwritten.
 *   D        64 or 128.  causal, scale, stream  as in attn_fwd.
 *
 * Ownership: the caller owns every buffer; the library allocates nothing and keeps no
 * state. Outputs and workspace must not overlap the inputs or each other.
 * Behaviour: arguments are validated on the host before any HIP call; a valid call
 * enqueues two kernels and returns without synchronising. Nothing is printed.
 */
int attn_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                void* workspace, size_t workspace_bytes, int B, int H, int Nq, int Nk, int D,
                int causal, float scale, void* stream);

/*
 * attn_decode_noalloc - attn_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. It computes exactly what attn_decode computes, with the same
 * kernels, and returns bit-identical o and lse.
 *
 *   q, k, v, o, lse, B, H, Nq, Nk, D, causal, scale   as in attn_decode.
 *   stream   a HIP stream (hipStream_t) of the current device, or NULL for its default
 *            stream; a stream of another device is rejected (ATTN_DECODE_EINVAL).
 *
 * Scratch: the per-chunk partials go to a fixed device array of
 * ATTN_DECODE_NOALLOC_MAX_WORKSPACE bytes inside the library (one per GPU it runs on,
 * held until the process ends). A call whose attn_decode_workspace_bytes(B, H, Nq, Nk, D)
 * exceeds it returns ATTN_DECODE_EWORKSPACE before any HIP call; every B*H <= 1024 fits,
 * whatever Nq (<= 32) and Nk. The first call on a device looks the array's address up
 * (hipGetSymbolAddress); no call allocates (no hipMalloc, hipFree or allocating library
 * routine).
 * Concurrency: all calls on one GPU share that array. Calls that may overlap in time on
 * one GPU (different streams, or threads without ordering between their launches) race
 * on it and give wrong results; calls on one stream are ordered and safe.
 * Errors: as attn_decode (ATTN_DECODE_ELAUNCH also covers a failed address lookup).
 */
int attn_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int Nq, int Nk, int D, int causal, float scale,
                        void* stream);

/* attn_decode_strerror - a static, NUL-terminated description of a return code. */
const char* attn_decode_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_DECODE_H */
