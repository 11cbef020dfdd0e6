// Device helpers shared by the attention backward kernels on gfx950: MFMA operand types,
// the LDS chunk permutation of a row-major bf16 tile, buffer resources and the
// global -> LDS copy instructions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn_tile {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.44269504088896341f;
constexpr int kWaitVmcnt0 = 0x0F70;  // s_waitcnt vmcnt(0) (expcnt, lgkmcnt unconstrained)

// LDS tile of BC rows x D bf16, row-major and unpadded, whose 16-byte chunks are
// permuted: logical chunk c of row r sits at physical chunk c ^ swz(r). The LDS has 64
// four-byte banks; 16-byte reads are serviced 16 lanes at a time, 8-byte (and
// transposing) reads 32 at a time. swz spreads both the MFMA row reads (16 lanes read one
// chunk of 16 consecutive rows) and the transposing reads (32 lanes read four adjacent
// chunks of four consecutive rows) over all 64 banks: for D = 128 (256-byte rows)
// swz = 4(r & 3) + ((r >> 2) & 3) over r mod 16; for D = 64 (128-byte rows, two per bank
// line) a 3-bit rotation of (r >> 1) & 7.
template <int D>
__device__ inline int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  const int a = (r >> 1) & 7;
  return ((a & 1) << 2) | (a >> 1);
}

// Both halves of the wave receive x[lane] + x[lane ^ 32].
__device__ inline float sum_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Buffer resource over num_bytes from base: 64-bit base, no stride, raw 32-bit format.
// Loads past num_bytes return zero instead of faulting.
__device__ inline i32x4 make_rsrc(const void* base, uint32_t num_bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane((int)num_bytes);
  r[3] = 0x00020000;
  return r;
}

// Global -> LDS copies (buffer_load ... lds): lane l reads rsrc.base + soff + voff[l] and
// writes LDS address lds + 16*l (dwordx4) or lds + 4*l (dword). Asynchronous, counted by
// vmcnt; wait_copies_and_barrier completes them. Issued from inline assembly without a
// memory clobber, so the compiler neither makes unrelated LDS reads wait for them nor
// orders them with those reads: every copy targets a buffer slot that no wave reads
// before the next barrier, and the reads of the slot's previous contents precede the
// barrier before the copy. M0 is used by nothing else in these kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void copy16_to_lds(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds)
      : "m0");
}
__device__ inline void copy4_to_lds(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %0, %1, %2 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds)
      : "m0");
}
#pragma clang diagnostic pop

__device__ inline void wait_copies_and_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

__device__ inline uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// The wave's share of copying rows [row0, row0 + ROWS) of a row-major [rows, D] bf16
// tensor (rsrc) into an LDS tile at lds_tile, chunk-permuted by swz. Rows at or past
// n_rows repeat row n_rows - 1 (finite data that the caller masks). Each 1 KiB copy
// instruction fills 1024 / (2D) whole rows; the waves of the workgroup take turns.
template <int D, int ROWS, int WAVES>
__device__ inline void copy_tile(const i32x4& rsrc, int row0, int n_rows, uint32_t lds_tile,
                                 int wave, int lane) {
  constexpr int kRowBytes = 2 * D;
  constexpr int kChunks = D / 8;
  constexpr int kRowsPerCopy = 1024 / kRowBytes;
  constexpr int kCopies = ROWS * kRowBytes / 1024;
  static_assert(kCopies % WAVES == 0, "copies must split evenly over the waves");
#pragma unroll
  for (int i = 0; i < kCopies / WAVES; ++i) {
    const int cidx = i * WAVES + wave;
    const int r = cidx * kRowsPerCopy + lane / kChunks;  // tile row this lane fills
    const int src_row = min(row0 + r, n_rows - 1);
    const int logical = (lane % kChunks) ^ swz<D>(r);
    const uint32_t voff = (uint32_t)((src_row - row0) * kRowBytes + logical * 16);
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)row0 * kRowBytes);
    copy16_to_lds(rsrc, voff, soff, __builtin_amdgcn_readfirstlane(lds_tile + cidx * 1024));
  }
}

// 64 fp32 values [i0, i0 + 64) of a vector (rsrc) into LDS (one wave); indices at or past
// n repeat element n - 1.
__device__ inline void copy_vec64(const i32x4& rsrc, int i0, int n, uint32_t lds, int lane) {
  const int src = min(i0 + lane, n - 1);
  copy4_to_lds(rsrc, (uint32_t)(src - i0) * 4u, __builtin_amdgcn_readfirstlane((uint32_t)i0 * 4u),
               __builtin_amdgcn_readfirstlane(lds));
}

}  // namespace attn_tile
