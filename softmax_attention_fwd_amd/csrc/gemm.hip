// Plain bf16 matrix product on the tile layer of the attention kernels, for gfx950:
// C = A B^T with A [M, K] and B [N, K] row-major (K contiguous; the layout of the
// tile library's mm_ABt in its attention listing), fp32 accumulation, C [M, N] bf16
// (round to nearest even).
//
// Layer reuse: the operand tiles go global -> LDS through buffer_load ... lds into the
// same chunk-permuted layout (64-wide k slices are 128-byte rows, conflict-free for the
// MFMA row reads), and v_mfma_f32_32x32x16_bf16 computes C^T = B A^T so that every lane
// ends up with four consecutive output columns of one row of C (8-byte stores), as the
// attention epilogue does.
//
// Workgroup: 8 waves (two per SIMD) on a 256 (m) x 256 (n) tile of C; wave (wm, wn) of the
// 2 x 4 grid owns 128 m x 64 n, i.e. 2 x 4 accumulators of 32 x 32. K advances in slices
// of 64 through two LDS stages (2 x 64 KiB).
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "tile_gemm.h"
#include "tile_lds.h"

namespace {

using namespace attn_tile;

constexpr int kWaves = 8;
constexpr int kTm = 256, kTn = 256, kTk = 64;
constexpr int kWaveM = 128, kWaveN = 64;
constexpr int kRowBytes = kTk * 2;              // 128-byte rows of a k slice
constexpr int kTileBytes = 256 * kRowBytes;     // 32 KiB per operand per stage
constexpr int kStageBytes = 2 * kTileBytes;
constexpr int kGroupM = 8;                      // tile rows walked together (L2 reuse)

struct GemmParams {
  const __bf16* a;
  const __bf16* b;
  __bf16* c;
  int M, N, K;
  int tiles_m;  // ceil(M / kTm)
  int tiles_n;  // ceil(N / kTn)
  int remap;
};

// The wave's share of copying rows [row0, row0 + 256), columns [k0, k0 + 64) of a
// row-major [rows, K] bf16 matrix into a chunk-permuted LDS tile (8 rows per 1 KiB copy).
// Rows at or past n_rows and columns at or past K are sent out of the buffer's range on
// purpose and read zeros.
__device__ inline void copy_slice(const i32x4& rsrc, int row0, int n_rows, int k0, int K,
                                  uint32_t lds_tile, int wave, int lane, int i0 = 0,
                                  int i1 = kTileBytes / 1024 / kWaves) {
  constexpr int kChunks = kTk / 8;  // 8 chunks of 16 bytes per row
#pragma unroll
  for (int i = i0; i < i1; ++i) {
    const int cidx = i * kWaves + wave;
    const int r = cidx * 8 + lane / kChunks;
    const int logical = (lane % kChunks) ^ swz<64>(r);
    const int kcol = k0 + 8 * logical;
    const bool inside = kcol < K && row0 + r < n_rows;
    const uint32_t voff = inside ? (uint32_t)(((uint64_t)r * K + kcol) * 2u) : 0x80000000u;
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)row0 * (uint32_t)K * 2u);
    copy16_to_lds(rsrc, voff, soff, __builtin_amdgcn_readfirstlane(lds_tile + cidx * 1024));
  }
}

__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_nt_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kStageBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int hi = lane >> 5;
  const int wm = wave & 1;   // 2 waves along m
  const int wn = wave >> 1;  // 4 waves along n

  // Tile order: after the XCD remap each XCD runs consecutive tile ids; those ids go down
  // groups of kGroupM tile rows first, so the 32 workgroups an XCD holds at a time share
  // 8 A panels and 4 B panels in its L2 (one tile row would need 32 B panels).
  const int g = remap_block(blockIdx.x, p.remap);
  const int per_group = kGroupM * p.tiles_n;
  const int group = g / per_group;
  const int first_m = group * kGroupM;
  const int rows_in_group = min(p.tiles_m - first_m, kGroupM);
  const int local = g - group * per_group;
  const int tm = first_m + local % rows_in_group;
  const int tn = local / rows_in_group;
  const int m0 = tm * kTm, n0 = tn * kTn;
  const int K = p.K;
  const int nk = (K + kTk - 1) / kTk;

  const i32x4 arsrc = make_rsrc(p.a, (uint32_t)p.M * (uint32_t)K * 2u);
  const i32x4 brsrc = make_rsrc(p.b, (uint32_t)p.N * (uint32_t)K * 2u);
  const uint32_t smem_lds = lds_address(smem);
  auto load = [&](int kt, int stage) {
    const uint32_t base = smem_lds + stage * kStageBytes;
    copy_slice(arsrc, m0, p.M, kt * kTk, K, base, wave, lane);
    copy_slice(brsrc, n0, p.N, kt * kTk, K, base + kTileBytes, wave, lane);
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = f32x16{};
  const int rbase = row_read_base<64>(col, hi);

  // The copies of the next slice go out a few at a time, one of A and one of B per 16-wide
  // k step of the current slice, among its MFMAs. Issued all at once after the barrier (64
  // KiB per compute unit), they queue at the vector-memory path and hold back the MFMAs
  // behind them in every wave's instruction stream. The last slice is peeled so that the
  // loop body has no branch around the copies.
  constexpr int kPerStep = kTileBytes / 1024 / kWaves / (kTk / 16);
  auto load_part = [&](int kt, int stage, int part) {
    const uint32_t base = smem_lds + stage * kStageBytes;
    copy_slice(arsrc, m0, p.M, kt * kTk, K, base, wave, lane, part * kPerStep, (part + 1) * kPerStep);
    copy_slice(brsrc, n0, p.N, kt * kTk, K, base + kTileBytes, wave, lane, part * kPerStep, (part + 1) * kPerStep);
  };
  auto slice = [&](int kt, bool next) {
    const int stage = kt & 1;
    wait_copies_and_barrier();
    const char* ta = smem + stage * kStageBytes + wm * kWaveM * kRowBytes;
    const char* tb = smem + stage * kStageBytes + kTileBytes + wn * kWaveN * kRowBytes;
#pragma unroll
    for (int k16 = 0; k16 < kTk / 16; ++k16) {
      if (next) load_part(kt + 1, stage ^ 1, k16);
      const int off = row_read_addr(rbase, k16);
      bf16x8 af[4], bf[2];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) af[mb] = *reinterpret_cast<const bf16x8*>(ta + 32 * mb * kRowBytes + off);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) bf[nb] = *reinterpret_cast<const bf16x8*>(tb + 32 * nb * kRowBytes + off);
      // C^T (n rows, m columns) += B A^T
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[nb], af[mb], acc[nb][mb], 0, 0, 0);
    }
  };
  load(0, 0);
  int kt = 0;
  for (; kt + 1 < nk; ++kt) slice(kt, true);
  slice(kt, false);

  // register r of acc[nb][mb] holds C[m][n], m = m0 + 128wm + 32mb + col,
  // n = n0 + 64wn + 32nb + 8(r/4) + 4h + r%4: four consecutive n per (lane, r/4)
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int m = m0 + wm * kWaveM + 32 * mb + col;
    if (m >= p.M) continue;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int n = n0 + wn * kWaveN + 32 * nb + 8 * g4 + 4 * hi;
        if (n >= p.N) continue;
        bf16x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (__bf16)acc[nb][mb][4 * g4 + i];
        *reinterpret_cast<bf16x4*>(p.c + (size_t)m * p.N + n) = w;
      }
  }
}

}  // namespace

extern "C" {

int gemm_bf16_nt(const void* a, const void* b, void* c, int M, int N, int K, void* stream) {
  if (!a || !b || !c) return GEMM_EINVAL;
  if (M < 1 || N < 1 || K < 1 || K % 8 != 0 || N % 8 != 0) return GEMM_EINVAL;
  if ((int64_t)M * K >= ((int64_t)1 << 30) || (int64_t)N * K >= ((int64_t)1 << 30))
    return GEMM_EINVAL;
  const int64_t tiles_m = ((int64_t)M + kTm - 1) / kTm;
  const int64_t tiles_n = ((int64_t)N + kTn - 1) / kTn;
  if (tiles_m * tiles_n >= ((int64_t)1 << 31)) return GEMM_EINVAL;
  if ((((uintptr_t)a | (uintptr_t)b | (uintptr_t)c) & 15u) != 0) return GEMM_EALIGN;
  GemmParams p;
  p.a = static_cast<const __bf16*>(a);
  p.b = static_cast<const __bf16*>(b);
  p.c = static_cast<__bf16*>(c);
  p.M = M;
  p.N = N;
  p.K = K;
  p.tiles_m = (int)tiles_m;
  p.tiles_n = (int)tiles_n;
  const int64_t grid = tiles_m * tiles_n;
  p.remap = (grid % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL(gemm_nt_kernel, dim3((unsigned)grid), dim3(64 * kWaves), 0,
                     static_cast<hipStream_t>(stream), p);
  if (hipGetLastError() != hipSuccess) return GEMM_ELAUNCH;
  return GEMM_OK;
}

const char* gemm_strerror(int code) {
  switch (code) {
    case GEMM_OK: return "success";
    case GEMM_EINVAL: return "invalid argument (NULL pointer, size < 1, K or N not a multiple of 8, or size overflow)";
    case GEMM_EALIGN: return "misaligned pointer (a, b, c need 16 bytes)";
    case GEMM_ELAUNCH: return "kernel launch failed";
    default: return "unknown error code";
  }
}

}  // extern "C"
