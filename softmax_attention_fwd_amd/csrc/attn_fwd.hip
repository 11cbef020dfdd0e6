// Fused softmax attention forward for gfx950 (AMD Instinct MI355X, CDNA4).
//
// What is computed: the attention forward of the ThunderKittens pages -- the warp-level
// inner loop on the alanwu.xyz blog (S = Q K^T per key tile, -inf fill past the last key,
// running row max, exp2, rescale of the running sum and of O, bf16 P, O += P V, and a
// final division of O by the row sum) and the consumer compute/finish steps of the H100
// listing in the 10100.com review (scale applied in fp32 to the score accumulator as
// TEMPERATURE_SCALE = scale * log2 e, epilogue division by the row sum). Causal masking
// (key j visible to query i iff j <= i) and the natural-log logsumexp output are not on
// those pages; they follow the usual FlashAttention conventions.
//
// gfx950 design (not the H100 one):
//   * one workgroup = 4 waves; each wave owns 32 query rows, so a workgroup covers 128.
//   * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: lane l
//     then holds 16 keys of query (l % 32) per 32-key block, so the row max and row sum
//     are in-lane reductions plus one v_permlane32_swap between the two lane halves.
//   * the output is accumulated transposed, O^T = V^T P^T. The score registers of a lane
//     are already the B operand of that MFMA (8 keys of its query), given that the A
//     operand (V^T) pairs its k positions with the same 8 keys; V^T fragments come from
//     LDS through ds_read_b64_tr_b16, which transposes 4x16 bf16 blocks across lanes.
//   * K and V tiles (64 keys each) are staged through registers into a double-buffered
//     LDS ring whose 16-byte chunks are XOR-swizzled by row, so the row-wise K reads and
//     the transposing V reads spread over the LDS banks.
//   * the exp2 argument is fma(s, c, -m*c) with c = scale*log2(e) in fp32, on the fp32
//     accumulator (the scale is never folded into bf16 Q).
//   * blockIdx is remapped so that consecutive query tiles of one head land on the same
//     XCD (workgroups are dealt round-robin over the 8 XCDs), keeping that head's K/V in
//     one L2; causal launches take the longest query tiles first.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "attn_fwd.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQW = 32;              // query rows per wave
constexpr int kBr = kWaves * kQW;    // query rows per workgroup
constexpr int kBc = 64;              // keys per K/V tile
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.44269504088896341f;

struct Params {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  int N;
  int n_qtiles;  // ceil(N / kBr)
  int remap;     // 1: grid size is a multiple of 8, use the XCD-aware order
  float c;       // scale * log2(e)
};

// Both halves of the wave receive max(x[lane], x[lane ^ 32]).
__device__ inline float max_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Both halves of the wave receive x[lane] + x[lane ^ 32].
__device__ inline float sum_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Byte offset of 16-byte chunk `chunk` of tile row `row` (rows are D bf16 wide).
template <int D>
__device__ inline int lds_offset(int row, int chunk) {
  return row * (D * 2) + ((chunk ^ (row & 7)) << 4);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(const Params p) {
  static_assert(D == 64 || D == 128, "head dimension");
  constexpr int kChunks = D / 8;                  // 16-byte chunks per row
  constexpr int kTileBytes = kBc * D * 2;         // one K or V tile
  constexpr int kLoads = kTileBytes / 16 / kThreads;
  static_assert(kLoads * 16 * kThreads == kTileBytes, "tile must split evenly over threads");
  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * kTileBytes];  // [stage][K, V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;  // query within the wave's 32-row block
  const int hi = lane >> 5;   // which half of the wave

  // ---- work unit: (batch*head, query tile)
  int g = blockIdx.x;
  if (p.remap) {
    const int per_xcd = gridDim.x >> 3;
    g = (g & 7) * per_xcd + (g >> 3);
  }
  const int bh = g / p.n_qtiles;
  int qt = g - bh * p.n_qtiles;
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;  // longest tiles first
  const int N = p.N;
  const size_t head = (size_t)bh * (size_t)N * D;
  const __bf16* Qh = p.q + head;
  const __bf16* Kh = p.k + head;
  const __bf16* Vh = p.v + head;

  const int q0 = qt * kBr + wave * kQW;  // first query row of this wave
  const int qrow = q0 + col;
  const bool wave_active = q0 < N;

  // ---- Q as the B operand of S^T = K Q^T: lane holds Q[qrow][16s + 8hi .. +7]
  bf16x8 qf[D / 16];
  if (qrow < N) {
    const bf16x8* src = reinterpret_cast<const bf16x8*>(Qh + (size_t)qrow * D) + hi;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = src[2 * s];
  } else {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = bf16x8{};
  }

  // ---- key range: the workgroup loads tiles up to its last query (causal) or N
  const int wg_kv_end = CAUSAL ? min(N, (qt + 1) * kBr) : N;
  const int ntiles = (wg_kv_end + kBc - 1) / kBc;
  const int wave_kv_end = CAUSAL ? min(N, q0 + kQW) : N;

  u32x4 kst[kLoads], vst[kLoads];
  auto load_tile = [&](int t) {
    const int key0 = t * kBc;
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int ci = tid + u * kThreads;
      const int r = ci / kChunks;
      const int c = ci % kChunks;
      const int key = key0 + r;
      if (key < N) {
        kst[u] = *reinterpret_cast<const u32x4*>(Kh + (size_t)key * D + c * 8);
        vst[u] = *reinterpret_cast<const u32x4*>(Vh + (size_t)key * D + c * 8);
      } else {
        kst[u] = u32x4{0u, 0u, 0u, 0u};  // zero rows: finite, and masked to -inf anyway
        vst[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&](int stage) {
    char* kb = smem + stage * 2 * kTileBytes;
    char* vb = kb + kTileBytes;
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int ci = tid + u * kThreads;
      const int off = lds_offset<D>(ci / kChunks, ci % kChunks);
      *reinterpret_cast<u32x4*>(kb + off) = kst[u];
      *reinterpret_cast<u32x4*>(vb + off) = vst[u];
    }
  };

  // ---- per-lane pieces of the V^T transposing read (see the header comment)
  const int jj = lane & 15;
  const int grp = lane >> 4;
  const int tr_row = 4 * hi + (jj >> 2);                       // + 16*step (+8 for keys 8..15)
  const int tr_chunk = 2 * (grp & 1) + ((jj & 3) >> 1);       // + 4*db
  const int tr_byte = (jj & 1) * 8;

  float m = -INFINITY;  // running max of raw scores for query qrow
  float l = 0.f;        // running sum of exp2(c*s - c*m) over this lane's keys
  f32x16 o[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) o[d] = f32x16{};

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) load_tile(t + 1);
    const int key0 = t * kBc;
    if (wave_active && key0 < wave_kv_end) {
      const char* kb = smem + (t & 1) * 2 * kTileBytes;
      const char* vb = kb + kTileBytes;
      // S^T = K Q^T for two 32-key blocks
      f32x16 s[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        s[j] = f32x16{};
        const int r = 32 * j + col;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb + lds_offset<D>(r, 2 * st + hi));
          s[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[j], 0, 0, 0);
        }
      }
      // mask: keys past N (ragged last tile) and, causal, keys after the query
      const bool need_mask = (key0 + kBc > N) || (CAUSAL && key0 + kBc - 1 > q0);
      if (need_mask) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * j + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (key >= N || (CAUSAL && key > qrow)) s[j][r] = -INFINITY;
          }
        }
      }
      // online softmax: new running max, rescale factor, exponentials
      float mx = m;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[j][r]);
      mx = max_across_halves(mx);
      const float mc = mx * p.c;
      const float alpha = __builtin_amdgcn_exp2f(m * p.c - mc);  // 0 on the first tile
      m = mx;
      float rs = 0.f;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j][r], p.c, -mc));
          s[j][r] = e;
          rs += e;
        }
      l = l * alpha + rs;
#pragma unroll
      for (int d = 0; d < D / 32; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
      // O^T += V^T P^T, 16 keys per MFMA step
#pragma unroll
      for (int st = 0; st < kBc / 16; ++st) {
        const int j = st >> 1;
        const int h8 = (st & 1) * 8;
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[i] = (__bf16)s[j][h8 + i];
        const int row = 16 * st + tr_row;
#pragma unroll
        for (int d = 0; d < D / 32; ++d) {
          const int chunk = 4 * d + tr_chunk;
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4*)(vb + lds_offset<D>(row, chunk) + tr_byte));
          const bf16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4*)(vb + lds_offset<D>(row + 8, chunk) + tr_byte));
          const bf16x8 a = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
          o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o[d], 0, 0, 0);
        }
      }
    }
    if (t + 1 < ntiles) store_tile((t + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O / l in bf16 (round to nearest even), lse = ln 2 * (c*m + log2 l)
  if (wave_active) {
    const float lt = sum_across_halves(l);  // lanes l and l^32 share a query row
    if (qrow < N) {
      const float inv = 1.f / lt;
      __bf16* orow = p.o + head + (size_t)qrow * D;
#pragma unroll
      for (int d = 0; d < D / 32; ++d)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          bf16x4 w;
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = (__bf16)(o[d][4 * j4 + i] * inv);
          *reinterpret_cast<bf16x4*>(orow + 32 * d + 8 * j4 + 4 * hi) = w;
        }
      if (hi == 0) p.lse[(size_t)bh * N + qrow] = (m * p.c + __builtin_log2f(lt)) * kLn2;
    }
  }
}

}  // namespace

extern "C" {

const char* attn_fwd_strerror(int code) {
  switch (code) {
    case ATTN_FWD_OK: return "success";
    case ATTN_FWD_EINVAL: return "invalid argument (NULL pointer, size < 1, causal not 0/1, scale not finite and > 0, or size overflow)";
    case ATTN_FWD_EUNSUPPORTED: return "unsupported head dimension (D must be 64 or 128)";
    case ATTN_FWD_EALIGN: return "misaligned pointer (q, k, v, o need 16 bytes, lse 4 bytes)";
    case ATTN_FWD_ELAUNCH: return "kernel launch failed";
    default: return "unknown error code";
  }
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int N, int D, int causal, float scale, void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_FWD_EINVAL;
  if (B < 1 || H < 1 || N < 1) return ATTN_FWD_EINVAL;
  if (causal != 0 && causal != 1) return ATTN_FWD_EINVAL;
  if (!(scale > 0.f) || !isfinite(scale)) return ATTN_FWD_EINVAL;
  if (D != 64 && D != 128) return ATTN_FWD_EUNSUPPORTED;
  const int64_t n_qtiles = ((int64_t)N + kBr - 1) / kBr;
  const int64_t grid = (int64_t)B * H * n_qtiles;
  if ((int64_t)N * D >= ((int64_t)1 << 31) || grid >= ((int64_t)1 << 31)) return ATTN_FWD_EINVAL;
  const uintptr_t a16 = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o;
  if ((a16 & 15u) != 0 || ((uintptr_t)lse & 3u) != 0) return ATTN_FWD_EALIGN;

  Params p;
  p.q = static_cast<const __bf16*>(q);
  p.k = static_cast<const __bf16*>(k);
  p.v = static_cast<const __bf16*>(v);
  p.o = static_cast<__bf16*>(o);
  p.lse = lse;
  p.N = N;
  p.n_qtiles = (int)n_qtiles;
  p.remap = (grid % 8 == 0) ? 1 : 0;
  p.c = scale * kLog2e;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid_dim((unsigned)grid), block_dim(kThreads);
  if (D == 64) {
    if (causal) hipLaunchKernelGGL((attn_fwd_kernel<64, true>), grid_dim, block_dim, 0, s, p);
    else hipLaunchKernelGGL((attn_fwd_kernel<64, false>), grid_dim, block_dim, 0, s, p);
  } else {
    if (causal) hipLaunchKernelGGL((attn_fwd_kernel<128, true>), grid_dim, block_dim, 0, s, p);
    else hipLaunchKernelGGL((attn_fwd_kernel<128, false>), grid_dim, block_dim, 0, s, p);
  }
  if (hipGetLastError() != hipSuccess) return ATTN_FWD_ELAUNCH;
  return ATTN_FWD_OK;
}

}  // extern "C"
