/*
 * tile_gemm.h - plain bf16 matrix product on the attention kernels' MFMA/LDS tile layer,
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation (the matrix-multiply building block of the ThunderKittens pages: the
 * warpgroup mm_ABt of the attention listing in the 10100.com review, and GEMM among the
 * kernels named in the paper summary on groovesquid.com):
 *
 *   C[i, j] = sum_k A[i, k] * B[j, k]          (C = A B^T)
 *
 * with A [M, K] and B [N, K] bf16 row-major (K contiguous), fp32 accumulation and C [M, N]
 * bf16 row-major, rounded to nearest even. (A [K, N] B is passed as its transpose.)
 */
#ifndef TILE_GEMM_H
#define TILE_GEMM_H

#ifdef __cplusplus
extern "C" {
#endif

#define GEMM_OK        0   /* success: the kernel was enqueued                              */
#define GEMM_EINVAL   -1   /* NULL pointer; M, N or K < 1; K or N not a multiple of 8;
                              M*K or N*K >= 2^30                                            */
#define GEMM_EALIGN   -3   /* a, b or c not 16-byte aligned                                 */
#define GEMM_ELAUNCH  -4   /* hipGetLastError() was set after the launch (also reports, and
                              clears, an error left pending by an earlier HIP call)         */

/*
 * gemm_bf16_nt - enqueue C = A B^T on a HIP stream.
 *
 *   a  device pointer, bf16, [M, K] row-major. Read only. 16-byte aligned.
 *   b  device pointer, bf16, [N, K] row-major. Read only. 16-byte aligned.
 *   c  device pointer, bf16, [M, N] row-major. Written in full. Must not overlap a or b.
 *   stream  a hipStream_t passed as void*; NULL is the default stream.
 *
 * The caller owns the buffers; nothing is allocated and no state is kept. Arguments are
 * validated before any HIP call; a valid call enqueues one kernel and returns without
 * synchronising. Nothing is printed.
 */
int gemm_bf16_nt(const void* a, const void* b, void* c, int M, int N, int K, void* stream);

/* gemm_strerror - a static, NUL-terminated description of a return code. */
const char* gemm_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* TILE_GEMM_H */
