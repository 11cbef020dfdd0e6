// Decode-shaped attention forward for gfx950 (AMD Instinct MI355X, CDNA4): Nq <= 32
// queries against Nk keys, split over workgroups along the keys and merged through lse.
//
// What is computed is the forward's softmax attention with Nq != Nk (attention inference,
// named beside the training kernels in the ThunderKittens paper summary on groovesquid.com;
// causal queries are the last Nq positions, so query i sees keys j <= Nk - Nq + i).
//
// The work is bound by reading K and V once from HBM (2 * Nk * D bf16 per head against
// 4 * Nq * Nk * D flop), so the design keeps many loads in flight rather than the matrix
// cores busy:
//   * split kernel: one workgroup per (batch*head, key chunk); its 4 waves take 32-key
//     tiles of the chunk in turn, each through its own double-buffered LDS region (K and V
//     copied by buffer_load ... lds, no workgroup barrier in the loop). Per tile the wave
//     forms S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (lane = query, the 32 query columns
//     padded with zero queries), runs the online softmax of the forward (exp2 with
//     c = scale * log2 e, lazy rescaling), and accumulates O^T += V^T P^T with V^T read
//     transposed from LDS. The 4 waves' partial (max, sum, O) are merged in LDS and the
//     chunk's normalised O and lse written to the workspace.
//   * merge kernel: per (batch*head, query), lse = ln sum_c exp(lse_c) and
//     O = sum_c exp(lse_c - lse) O_c over the chunks, written in bf16.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "attn_decode.h"
#include "tile_lds.h"

namespace {

using namespace attn_tile;

constexpr int kWaves = 4;
constexpr int kKeys = 32;                    // keys per wave tile
constexpr int kChunkAlign = kWaves * kKeys;  // key chunks are multiples of this
constexpr int kMaxQ = 32;
constexpr float kRescaleLog2 = 8.0f;         // lazy-rescale threshold (log2 units)
// One workgroup per compute unit of the MI355X (256): the split kernel's 128 KiB of LDS
// admits one workgroup per CU at a time, and a single round has no tail. Measured against
// 1024 (four rounds): 7%, 39% and 1.4% faster on the three decode workloads (1 query x
// 4096 keys x 256 heads, 8 x 16384 x 32, 1 x 131072 x 32).
constexpr int kTargetWorkgroups = 256;

struct DecParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  float* part_o;    // [B*H][S][Nq][D]: each chunk's normalised output
  float* part_lse;  // [B*H][S][Nq]: each chunk's lse (natural log; -inf if no key visible)
  int Nq;
  int Nk;
  int S;            // key chunks per head
  int chunk;        // keys per chunk (multiple of kChunkAlign)
  float c;          // scale * log2(e)
};

template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // s_waitcnt: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8 (the latter two left
  // unconstrained)
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(1, 2)))
void attn_decode_split_kernel(const DecParams p) {
  constexpr int RB = 2 * D;
  constexpr int kTileBytes = kKeys * RB;             // one K or V tile
  constexpr int kWaveBytes = 4 * kTileBytes;         // two stages of K and V
  constexpr int kCopies = 2 * kTileBytes / 1024;     // copy instructions per stage
  static_assert(kMaxQ * D * 4 + 2 * kMaxQ * 4 <= kWaveBytes, "merge staging fits a wave region");
  __shared__ __attribute__((aligned(1024))) char smem[kWaves * kWaveBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;  // query column
  const int hi = lane >> 5;
  const int Nq = p.Nq, Nk = p.Nk;

  const int bh = blockIdx.x / p.S;
  const int sidx = blockIdx.x - bh * p.S;
  const int ks0 = sidx * p.chunk;
  const int ks1 = min(Nk, ks0 + p.chunk);
  const int t_first = ks0 / kKeys + wave;
  const int t_end = (ks1 + kKeys - 1) / kKeys;

  // Q as the B operand of S^T = K Q^T: lane holds Q[col][16st + 8hi .. +7]; padding
  // columns (col >= Nq) are zero queries
  bf16x8 qf[D / 16];
  if (col < Nq) {
    const bf16x8* src = reinterpret_cast<const bf16x8*>(p.q + ((size_t)bh * Nq + col) * D) + hi;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = src[2 * s];
  } else {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = bf16x8{};
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  const size_t kv_head = (size_t)bh * Nk * D;
  const uint32_t kv_bytes = (uint32_t)Nk * RB;
  const i32x4 krsrc = make_rsrc(p.k + kv_head, kv_bytes);
  const i32x4 vrsrc = make_rsrc(p.v + kv_head, kv_bytes);
  const uint32_t region = lds_address(smem) + wave * kWaveBytes;
  const int rbase = row_read_base<D>(col, hi);
  int ta[D / 32][2];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) {
    ta[d][0] = tr_read_addr<D>(lane, d, 0);
    ta[d][1] = tr_read_addr<D>(lane, d, 1);
  }
  // stage st: K tile at st * 2 * kTileBytes, V tile after it
  auto load = [&](int t, int st) {
    const uint32_t base = region + st * 2 * kTileBytes;
    copy_tile<D, kKeys, 1>(krsrc, t * kKeys, Nk, base, 0, lane);
    copy_tile<D, kKeys, 1>(vrsrc, t * kKeys, Nk, base + kTileBytes, 0, lane);
  };

  float m = -INFINITY;  // running max (raw scores) of query col
  float l = 0.f;        // running sum of exp2(c*s - c*m) over this lane's keys
  f32x16 o[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) o[d] = f32x16{};
  // the last query position a key may take: Nk - Nq + col (causal)
  const int key_limit = CAUSAL ? min(Nk, Nk - Nq + col + 1) : Nk;

  if (t_first < t_end) load(t_first, 0);
  if (t_first + kWaves < t_end) load(t_first + kWaves, 1);
  int it = 0;
  for (int t = t_first; t < t_end; t += kWaves, ++it) {
    const int st = it & 1;
    if (t + kWaves < t_end) wait_vmcnt<kCopies>();  // this stage landed, the next may not
    else wait_vmcnt<0>();
    const int kb = wave * kWaveBytes + st * 2 * kTileBytes;  // K tile offset in smem
    const int vb = kb + kTileBytes;
    // S^T (32 keys x 32 queries): register r holds key t*32 + 8(r/4) + 4hi + r%4
    f32x16 s = f32x16{};
#pragma unroll
    for (int k16 = 0; k16 < D / 16; ++k16) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(smem + kb + row_read_addr(rbase, k16));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[k16], s, 0, 0, 0);
    }
    const int key0 = t * kKeys;
    // only the tile holding key Nk - Nq (causal) or key Nk - 1 needs the mask
    if (key0 + kKeys > Nk || (CAUSAL && key0 + kKeys - 1 > Nk - Nq)) {
      const int lim = key_limit - key0 - 4 * hi;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) >= lim) s[r] = -INFINITY;
    }
    float mx = m;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    // lazy rescale; a column with no visible key so far keeps m = -inf (its exponentials
    // below are taken against 0 and are all 0), and its l and O, still 0, take alpha = 0
    // rather than exp2(-inf + inf)
    if (__builtin_amdgcn_ballot_w64((mx - m) * p.c > kRescaleLog2)) {
      const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m - mx) * p.c);
      m = mx;
      l *= alpha;
#pragma unroll
      for (int d = 0; d < D / 32; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
    }
    const float mc = (m == -INFINITY) ? 0.f : m * p.c;
    bf16x8 pb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], p.c, -mc));
      l += e;
      pb[r >> 3][r & 7] = (__bf16)e;
    }
    // O^T += V^T P^T over the tile's two 16-key steps
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int d = 0; d < D / 32; ++d) {
        const bf16x8 a = tr_frag<D>(smem, vb, ta[d], 16 * k2);
        o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[k2], o[d], 0, 0, 0);
      }
    // the stage is free once its reads are done: refill it with tile t + 2 * kWaves
    if (t + 2 * kWaves < t_end) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      load(t + 2 * kWaves, st);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // every copy and LDS read of this wave has completed
  __syncthreads();                // ... and of every wave: the regions can be reused

  // ---- merge the 4 waves: wave w stages M_w = c*m (log2 units), L_w and O_w (unnormalised)
  // of its 32 columns in its own region: O at [col][D], then M[32], L[32]
  const float lt = sum_across_halves(l);
  float* ow = reinterpret_cast<float*>(smem + wave * kWaveBytes);
  float* mw = ow + kMaxQ * D;
  float* lw = mw + kMaxQ;
#pragma unroll
  for (int d = 0; d < D / 32; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) ow[col * D + 32 * d + 8 * (r >> 2) + 4 * hi + (r & 3)] = o[d][r];
  if (hi == 0) {
    mw[col] = m * p.c;  // -inf when the column saw no key
    lw[col] = lt;
  }
  __syncthreads();
  // thread tid handles query q of rows tid / (D / 4) and 4 consecutive outputs
  constexpr int kThreadsPerQ = D / 4;
  for (int idx = tid; idx < Nq * kThreadsPerQ; idx += 64 * kWaves) {
    const int q = idx / kThreadsPerQ;
    const int d0 = (idx % kThreadsPerQ) * 4;
    float mstar = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      mstar = fmaxf(mstar, reinterpret_cast<const float*>(smem + w * kWaveBytes)[kMaxQ * D + q]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    if (mstar != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float* base = reinterpret_cast<const float*>(smem + w * kWaveBytes);
        const float wgt = __builtin_amdgcn_exp2f(base[kMaxQ * D + q] - mstar);
        L += wgt * base[kMaxQ * D + kMaxQ + q];
        const f32x4 ov = *reinterpret_cast<const f32x4*>(base + q * D + d0);
        acc += wgt * ov;
      }
    }
    const size_t row = ((size_t)bh * p.S + sidx) * Nq + q;
    const f32x4 out = (L > 0.f) ? acc / L : f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(p.part_o + row * D + d0) = out;
    if (d0 == 0) p.part_lse[row] = (L > 0.f) ? (mstar + __builtin_log2f(L)) * kLn2 : -INFINITY;
  }
}

// ---- merge: one wave per (batch*head, query); lane handles D/64 outputs.
template <int D>
__global__ __launch_bounds__(64) void attn_decode_merge_kernel(const DecParams p) {
  constexpr int kPer = D / 64;
  const int lane = threadIdx.x;
  const int row = blockIdx.x;  // bh * Nq + q
  const int bh = row / p.Nq;
  const int q = row - bh * p.Nq;
  const size_t base = (size_t)bh * p.S * p.Nq + q;  // chunk c at base + c * Nq
  float mstar = -INFINITY;
  for (int c = 0; c < p.S; ++c) mstar = fmaxf(mstar, p.part_lse[base + (size_t)c * p.Nq]);
  float L = 0.f;
  float acc[kPer] = {};
  for (int c = 0; c < p.S; ++c) {
    const float lc = p.part_lse[base + (size_t)c * p.Nq];
    if (lc == -INFINITY) continue;
    const float w = __expf(lc - mstar);
    L += w;
    const float* oc = p.part_o + (base + (size_t)c * p.Nq) * D;
#pragma unroll
    for (int i = 0; i < kPer; ++i) acc[i] += w * oc[lane + 64 * i];
  }
  __bf16* out = p.o + (size_t)row * D;
#pragma unroll
  for (int i = 0; i < kPer; ++i) out[lane + 64 * i] = (__bf16)(acc[i] / L);
  if (lane == 0) p.lse[row] = mstar + __logf(L);
}

// Key chunks per head: enough workgroups to fill the chip, chunks a multiple of
// kChunkAlign keys.
void split_plan(int BH, int Nk, int* S, int* chunk) {
  const int max_chunks = (Nk + kChunkAlign - 1) / kChunkAlign;
  int s = (kTargetWorkgroups + BH - 1) / BH;
  s = s < 1 ? 1 : (s > max_chunks ? max_chunks : s);
  int c = (Nk + s - 1) / s;
  c = (c + kChunkAlign - 1) / kChunkAlign * kChunkAlign;
  *chunk = c;
  *S = (Nk + c - 1) / c;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool sizes_ok(int B, int H, int Nq, int Nk, int D) {
  return B >= 1 && H >= 1 && Nq >= 1 && Nk >= 1 && (D == 64 || D == 128) &&
         (int64_t)B * H < ((int64_t)1 << 24) && (int64_t)Nk * D < ((int64_t)1 << 31);
}

// Host-side validation shared by both entry points; makes no HIP call.
int check_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
               int B, int H, int Nq, int Nk, int D, int causal, float scale) {
  if (!q || !k || !v || !o || !lse) return ATTN_DECODE_EINVAL;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return ATTN_DECODE_EINVAL;
  if (causal != 0 && causal != 1) return ATTN_DECODE_EINVAL;
  if (causal && Nq > Nk) return ATTN_DECODE_EINVAL;
  if (!(scale > 0.f) || !isfinite(scale)) return ATTN_DECODE_EINVAL;
  if (D != 64 && D != 128) return ATTN_DECODE_EUNSUPPORTED;
  if (Nq > kMaxQ) return ATTN_DECODE_EUNSUPPORTED;
  if (!sizes_ok(B, H, Nq, Nk, D)) return ATTN_DECODE_EINVAL;
  return ATTN_DECODE_OK;
}

bool aligned(const void* q, const void* k, const void* v, const void* o, const float* lse) {
  const uintptr_t a16 = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o;
  return (a16 & 15u) == 0 && ((uintptr_t)lse & 3u) == 0;
}

// Split and merge kernels over validated arguments; the partials go to `workspace`, a
// device address of at least attn_decode_workspace_bytes(...) bytes, 256-byte aligned.
int launch(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
           int B, int H, int Nq, int Nk, int D, int causal, float scale, void* stream) {
  DecParams p;
  p.q = static_cast<const __bf16*>(q);
  p.k = static_cast<const __bf16*>(k);
  p.v = static_cast<const __bf16*>(v);
  p.o = static_cast<__bf16*>(o);
  p.lse = lse;
  p.Nq = Nq;
  p.Nk = Nk;
  split_plan(B * H, Nk, &p.S, &p.chunk);
  const size_t rows = (size_t)B * H * p.S * Nq;
  p.part_o = static_cast<float*>(workspace);
  p.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                        round_up(rows * D * sizeof(float), 256));
  p.c = scale * kLog2e;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid1((unsigned)(B * H * p.S)), block1(64 * kWaves);
  const dim3 grid2((unsigned)(B * H * Nq)), block2(64);
  if (D == 64) {
    if (causal) hipLaunchKernelGGL((attn_decode_split_kernel<64, true>), grid1, block1, 0, s, p);
    else hipLaunchKernelGGL((attn_decode_split_kernel<64, false>), grid1, block1, 0, s, p);
    hipLaunchKernelGGL(attn_decode_merge_kernel<64>, grid2, block2, 0, s, p);
  } else {
    if (causal) hipLaunchKernelGGL((attn_decode_split_kernel<128, true>), grid1, block1, 0, s, p);
    else hipLaunchKernelGGL((attn_decode_split_kernel<128, false>), grid1, block1, 0, s, p);
    hipLaunchKernelGGL(attn_decode_merge_kernel<128>, grid2, block2, 0, s, p);
  }
  if (hipGetLastError() != hipSuccess) return ATTN_DECODE_ELAUNCH;
  return ATTN_DECODE_OK;
}

// ---- fixed scratch of attn_decode_noalloc
//
// The per-chunk partials of attn_decode_noalloc live in this device array instead of a
// caller workspace. Every GPU the library runs on holds its own copy from the module's
// load until the process ends. In host code `scratch` names a host-side stand-in, not
// the device array: its device address is taken once per device with
// hipGetSymbolAddress (with that device current) and only that address is ever passed
// to a kernel. The split kernel writes every partial the merge kernel reads, so nothing
// has to be cleared between calls.
constexpr size_t kNoAllocScratchBytes = ATTN_DECODE_NOALLOC_MAX_WORKSPACE;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

// The device address of `scratch` on the current device (looked up on the first call on
// that device). A non-null stream must belong to the current device.
int noalloc_scratch(void* stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_DECODE_ELAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return ATTN_DECODE_EUNSUPPORTED;
  if (stream) {
    hipDevice_t sdev = 0;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) return ATTN_DECODE_ELAUNCH;
    if ((int)sdev != dev) return ATTN_DECODE_EINVAL;
  }
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    ptr = g_scratch[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return ATTN_DECODE_ELAUNCH;
      if (((uintptr_t)ptr & 255u) != 0) return ATTN_DECODE_EALIGN;
      g_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return ATTN_DECODE_OK;
}

}  // namespace

extern "C" {

size_t attn_decode_workspace_bytes(int B, int H, int Nq, int Nk, int D) {
  if (!sizes_ok(B, H, Nq, Nk, D) || Nq > kMaxQ) return 0;
  int S, chunk;
  split_plan(B * H, Nk, &S, &chunk);
  const size_t rows = (size_t)B * H * S * Nq;
  return round_up(rows * D * sizeof(float), 256) + round_up(rows * sizeof(float), 256);
}

int attn_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                void* workspace, size_t workspace_bytes, int B, int H, int Nq, int Nk, int D,
                int causal, float scale, void* stream) {
  if (!workspace) return ATTN_DECODE_EINVAL;
  const int rc = check_args(q, k, v, o, lse, B, H, Nq, Nk, D, causal, scale);
  if (rc != ATTN_DECODE_OK) return rc;
  if (workspace_bytes < attn_decode_workspace_bytes(B, H, Nq, Nk, D)) return ATTN_DECODE_EWORKSPACE;
  if (!aligned(q, k, v, o, lse) || ((uintptr_t)workspace & 255u) != 0) return ATTN_DECODE_EALIGN;
  return launch(q, k, v, o, lse, workspace, B, H, Nq, Nk, D, causal, scale, stream);
}

int attn_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int Nq, int Nk, int D, int causal, float scale,
                        void* stream) {
  int rc = check_args(q, k, v, o, lse, B, H, Nq, Nk, D, causal, scale);
  if (rc != ATTN_DECODE_OK) return rc;
  if (attn_decode_workspace_bytes(B, H, Nq, Nk, D) > kNoAllocScratchBytes) return ATTN_DECODE_EWORKSPACE;
  if (!aligned(q, k, v, o, lse)) return ATTN_DECODE_EALIGN;
  void* ws = nullptr;
  rc = noalloc_scratch(stream, &ws);
  if (rc != ATTN_DECODE_OK) return rc;
  return launch(q, k, v, o, lse, ws, B, H, Nq, Nk, D, causal, scale, stream);
}

const char* attn_decode_strerror(int code) {
  switch (code) {
    case ATTN_DECODE_OK: return "success";
    case ATTN_DECODE_EINVAL: return "invalid argument (NULL pointer, size < 1, causal not 0/1 or with Nq > Nk, scale not finite and > 0, or size overflow)";
    case ATTN_DECODE_EUNSUPPORTED: return "unsupported shape (D must be 64 or 128, Nq at most 32)";
    case ATTN_DECODE_EALIGN: return "misaligned pointer (tensors need 16 bytes, lse 4, workspace 256)";
    case ATTN_DECODE_ELAUNCH: return "kernel launch failed";
    case ATTN_DECODE_EWORKSPACE: return "workspace smaller than attn_decode_workspace_bytes(...), or (attn_decode_noalloc) larger than its fixed scratch";
    default: return "unknown error code";
  }
}

}  // extern "C"
