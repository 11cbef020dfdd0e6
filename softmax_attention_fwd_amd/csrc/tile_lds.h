// Device helpers shared by the attention backward and decode kernels on gfx950: MFMA types,
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

// Workgroups are dealt round-robin over the 8 XCDs; when the grid is a multiple of 8,
// renumber them so that consecutive tiles of one head land on the same XCD (one L2).
__device__ inline int remap_block(int g, int remap) {
  if (!remap) return g;
  const int per_xcd = gridDim.x >> 3;
  return (g & 7) * per_xcd + (g >> 3);
}

// Row-read address of an MFMA A operand from a swz-permuted [rows, D] tile: lane (m + 32h)
// reads logical chunk 2st + h of row m, at m*2D + 16((2st + h) ^ swz(m)). Since 2st and h
// occupy disjoint bits, that is row_read_base(m, h) ^ 32st: one base register per lane
// and an XOR per read instead of D/16 registers.
template <int D>
__device__ inline int row_read_base(int col, int hi) {
  return col * (2 * D) + 16 * (hi ^ swz<D>(col));
}
__device__ inline int row_read_addr(int base, int st) { return base ^ (32 * st); }
// Transposed-read base (ds_read_b64_tr_b16) of 4x16 blocks from a swz-permuted
// [rows, D] tile, for output column block d and row half u: in each 16-lane group the
// source lane jj supplies 8 bytes of row 8u + 4h + (jj >> 2) at logical column
// 32d + 16(grp & 1) + 4(jj & 3); the instruction hands lane jj column jj of that 4-row
// block. The permutation depends on the row mod 16, so row offsets that are multiples of
// 16 are added as constants, while the two 8-row halves need bases of their own.
template <int D>
__device__ inline int tr_read_addr(int lane, int d, int u) {
  const int jj = lane & 15, grp = lane >> 4, hi = lane >> 5;
  const int row = 8 * u + 4 * hi + (jj >> 2);
  const int chunk = 4 * d + 2 * (grp & 1) + ((jj >> 1) & 1);
  return row * (2 * D) + 16 * (chunk ^ swz<D>(row)) + 8 * (jj & 1);
}
// A operand of MFMA k-step over rows row0..row0+15 (row0 a multiple of 16) for output
// columns 32d.. from the tile at smem + tile: rows row0 + 4h + {0..3} (low four k) and
// row0 + 8 + 4h + {0..3} (high four k), column 32d + lane % 32.
template <int D>
__device__ inline bf16x8 tr_frag(const char* smem, int tile, const int (&addr)[2], int row0) {
  const char* base = smem + tile + row0 * (2 * D);
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + addr[0]));
  const bf16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + addr[1]));
  return __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Store a D x 32 fp32 accumulator (transposed layout: register r of block d holds column
// 32d + 8(r/4) + 4h + r%4 of row `row`) as bf16 row `row` of out, times s.
template <int D>
__device__ inline void store_rows(__bf16* out_row, const f32x16 (&acc)[D / 32], int hi, float s) {
#pragma unroll
  for (int d = 0; d < D / 32; ++d)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      bf16x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = (__bf16)(acc[d][4 * j4 + i] * s);
      *reinterpret_cast<bf16x4*>(out_row + 32 * d + 8 * j4 + 4 * hi) = w;
    }
}

}  // namespace attn_tile
