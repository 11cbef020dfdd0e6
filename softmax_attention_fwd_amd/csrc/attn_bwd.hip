// Attention backward for gfx950 (AMD Instinct MI355X, CDNA4): dQ, dK, dV of
// O = softmax(scale * Q K^T [+ causal mask]) V from the forward's per-row lse.
//
// The pages list the attention backward among the tile library's kernels (the summary of
// the ThunderKittens paper on groovesquid.com) without formulas. This is the gradient of
// the forward definition by the chain rule, with the probabilities recomputed from the
// scores and lse (so no N x N matrix is stored):
//   P = exp(scale * Q K^T - lse),  dV = P^T dO,  dP = dO V^T,
//   Delta_i = sum_d dO_id O_id (= sum_j P_ij dP_ij),  dS = P o (dP - Delta),
//   dQ = scale * dS K,  dK = scale * dS^T Q.
//
// Three kernels on the caller's stream:
//   * delta: -Delta_i and -lse_i / scale per row, into the caller's workspace; they
//     seed the dP and S accumulators, so the MFMAs produce dP - Delta and
//     s - lse / scale directly (P = exp2(c (s - lse / scale)), c = scale * log2 e).
//   * dkdv (D = 128): one workgroup per 128 keys, 8 waves in pairs of two roles over 32
//     keys each.
//     The P wave holds K and the dS wave V in registers as MFMA operands; Q and dO stream
//     through LDS in tiles of 64 queries. Per 32 queries and 32 keys: S = Q K^T (P wave)
//     and dP = dO V^T (dS wave) (v_mfma_f32_32x32x16_bf16, each lane then holds one key
//     and 16 queries), P (P wave, passed to the dS wave through LDS) and dS in registers,
//     and dV^T += dO^T P (P wave), dK^T += Q^T dS (dS wave) with dO^T / Q^T read
//     transposed from LDS (ds_read_b64_tr_b16) and P / dS straight from the score
//     registers as the B operand (the MFMA's k order only has to agree between its
//     operands). S and dP are formed once here. At D = 64 one wave holds both K and V
//     and does both roles (dkdv1).
//   * dq: one workgroup per 128 queries (32 per wave), the forward's shape. Q and dO stay
//     in registers; K and V stream through LDS in tiles of 64 keys. Per 32 keys:
//     S^T = K Q^T and dP^T = V dO^T (each lane one query, 16 keys), dS^T, and
//     dQ^T += K^T dS^T with K^T read transposed.
// The five N x N x D products run once each plus S and dP again in dq: 14 N^2 D of
// executed MFMA work for the algorithmic 10 N^2 D. No atomics: every output element is
// owned by one wave, so the results are the same on every call. dQ, dK, dV are written
// in bf16 (round to nearest even) after scaling in fp32.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "attn_bwd.h"
#include "tile_lds.h"

namespace {

using namespace attn_tile;

constexpr int kWaves = 4;
constexpr int kBlk = 32;            // keys (dkdv) or queries (dq) per wave
constexpr int kWgRows = kWaves * kBlk;
constexpr int kTile = 64;           // streamed rows per LDS tile
constexpr int kPairs = 4;           // dkdv: wave pairs (two roles over the same keys)

struct BwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;
  const __bf16* dout;
  const float* lse;
  float* ndelta;  // workspace: -Delta per row
  float* nls;     // workspace: -lse / scale per row
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  int N;
  int n_wg_tiles;  // ceil(N / kWgRows)
  int n_kv_tiles;  // ceil(N / (32 kPairs)): dkdv workgroups per head
  int remap_kv;    // dkdv grid is a multiple of 8: XCD-aware order
  int rows;        // B * H * N
  int remap;       // grid is a multiple of 8: XCD-aware order
  float c;         // scale * log2(e)
  float scale;
};

// ---- delta: -Delta_i = -sum_d dO_id O_id and -lse_i / scale, one row per D/8 lanes.
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(const BwdParams p) {
  constexpr int kLanesPerRow = D / 8;
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int row = t / kLanesPerRow;
  const int part = t % kLanesPerRow;
  float acc = 0.f;
  if (row < p.rows) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(p.dout + (size_t)row * D + part * 8);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(p.o + (size_t)row * D + part * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_fmaf((float)a[i], (float)b[i], acc);
  }
#pragma unroll
  for (int off = kLanesPerRow / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, kLanesPerRow);
  if (row < p.rows && part == 0) {
    p.ndelta[row] = -acc;
    p.nls[row] = -p.lse[row] / p.scale;
  }
}

// ---- dkdv: kPairs pairs of waves (128 keys a workgroup), each pair on 32 keys in two
// roles: the P wave (waves 0-3) forms S = Q K^T, P, and dV^T += dO^T P; the dS wave
// (waves 4-7) forms dP - Delta = dO V^T - Delta, takes P from the P wave through LDS, and
// accumulates dK^T += Q^T dS. Query tiles of 64 stream through LDS (two slots). Each role
// holds one of K, V (32 registers at D = 128) and one accumulator (64), so S and dP are
// formed once without the 128 + 128 registers of both in one wave; the two waves of a
// SIMD share its MFMAs. Per tile: phase 1 forms S and P (P waves) and dP (dS waves);
// after a barrier, phase 2 forms dS (dS waves) and adds both products.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(128 * kPairs) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dkdv_kernel(const BwdParams p) {
  static_assert(D == 128, "the two-role kernel serves D = 128");
  constexpr int RB = 2 * D;
  constexpr int kWaves2 = 2 * kPairs;
  constexpr int kKeys = kPairs * kBlk;                   // keys of the workgroup
  constexpr int kTileBytes = kTile * RB;
  constexpr int kSlot = 2 * kTileBytes + 2 * kTile * 4;  // Q, dO, -lse/scale, -Delta
  constexpr int kPBlock = kBlk * kBlk * 2;                // P of one block (bf16)
  constexpr int kPBytes = (kTile / kBlk) * kPBlock;        // of one pair, one tile
  __shared__ __attribute__((aligned(1024))) char smem[2 * kSlot + kPairs * kPBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool pw = wave < kPairs;  // P wave (else dS wave)
  const int pair = wave % kPairs;
  const int col = lane & 31;
  const int hi = lane >> 5;
  const int N = p.N;

  const int g = remap_block(blockIdx.x, p.remap_kv);
  const int bh = g / p.n_kv_tiles;
  const int kt = g - bh * p.n_kv_tiles;
  const size_t head = (size_t)bh * N * D;
  const int k0 = kt * kKeys + pair * kBlk;  // first key of this pair
  const int key = k0 + col;

  // K (P waves) or V (dS waves) as B operands (lane = key, k = D index 16st + 8h .. +7)
  bf16x8 xf[D / 16];
  {
    const int r = min(key, N - 1);
    const bf16x8* src = reinterpret_cast<const bf16x8*>((pw ? p.k : p.v) + head + (size_t)r * D) + hi;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) xf[s] = src[2 * s];
  }
  // xf has landed before any tile copy is issued. Left outstanding, it made the compiler
  // wait for xf inside the loop with vmcnt(0), which also waited for the next tile's copies
  // in the middle of the first product (removing that wait: +2% at B16 H16 N4096).
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  f32x16 acc[D / 32];  // dV^T (P waves) or dK^T (dS waves)
#pragma unroll
  for (int d = 0; d < D / 32; ++d) acc[d] = f32x16{};

  const uint32_t head_bytes = (uint32_t)N * RB;
  const i32x4 qrsrc = make_rsrc(p.q + head, head_bytes);
  const i32x4 orsrc = make_rsrc(p.dout + head, head_bytes);
  const i32x4 lrsrc = make_rsrc(p.nls + (size_t)bh * N, (uint32_t)N * 4u);
  const i32x4 drsrc = make_rsrc(p.ndelta + (size_t)bh * N, (uint32_t)N * 4u);
  const uint32_t smem_lds = lds_address(smem);

  // query tiles: causal workgroups start at their first key
  const int qt_first = CAUSAL ? (kt * kKeys) / kTile : 0;
  const int qt_end = (N + kTile - 1) / kTile;
  auto load = [&](int qt, int slot) {
    const uint32_t base = smem_lds + slot * kSlot;
    copy_tile<D, kTile, kWaves2>(qrsrc, qt * kTile, N, base, wave, lane);
    copy_tile<D, kTile, kWaves2>(orsrc, qt * kTile, N, base + kTileBytes, wave, lane);
    if (wave == 0) copy_vec64(lrsrc, qt * kTile, N, base + 2 * kTileBytes, lane);
    if (wave == 1) copy_vec64(drsrc, qt * kTile, N, base + 2 * kTileBytes + kTile * 4, lane);
  };

  const int rbase = row_read_base<D>(col, hi);
  int ta[D / 32][2];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) {
    ta[d][0] = tr_read_addr<D>(lane, d, 0);
    ta[d][1] = tr_read_addr<D>(lane, d, 1);
  }
  // this pair's P: block b, half u at pbase + b * kPBlock + u * 1024 + 16 * lane
  const int pbase = 2 * kSlot + pair * kPBytes + 16 * lane;

  // The two roles run separate loops (compile-time PW) with the same barriers: two a
  // tile. Every block of a tile is computed; the causal and ragged masks zero P (so dS
  // too) where a key is not visible, which also covers keys >= N and queries >= N (their
  // rows are clamped copies, finite).
  auto role = [&](auto pw_tag) {
    constexpr bool PW = decltype(pw_tag)::value;
    f32x16 x[2];      // S - lse / scale (P waves) or dP - Delta (dS waves), per block
    bf16x8 fr[2][2];  // P (P waves) or dS (dS waves) as B operands, per block and k-step
    // the first product of both blocks from the tile in slot `sl`: rows of Q (P waves) or
    // dO (dS waves) times xf, seeded with -lse / scale or -Delta
    auto first_product = [&](int sl) {
      const int qs = sl * kSlot;
      const int xs = PW ? qs : qs + kTileBytes;
      const int is = qs + 2 * kTileBytes + (PW ? 0 : kTile * 4);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(smem + is + (b * kBlk + 8 * g4 + 4 * hi) * 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) x[b][4 * g4 + i] = a[i];
        }
      bf16x8 ra[D / 16][2];
#pragma unroll
      for (int st = 0; st < D / 16; ++st)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          ra[st][b] = *reinterpret_cast<const bf16x8*>(smem + xs + b * kBlk * RB + row_read_addr(rbase, st));
#pragma unroll
      for (int st = 0; st < D / 16; ++st)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          x[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[st][b], xf[st], x[b], 0, 0, 0);
      // order: the 8 seed reads and 3 operand reads, then each MFMA followed by the read
      // of the operand three MFMAs ahead. Left to itself the compiler put most reads right
      // before their MFMAs, with an LDS wait in front of each (this order and the same one
      // in the second product: +2 to +6% more, bit-identical).
      __builtin_amdgcn_sched_group_barrier(0x100, 8 + 3, 0);
#pragma unroll
      for (int m = 0; m < 2 * (D / 16); ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (m + 3 < 2 * (D / 16)) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // the second product: acc += (dO or Q of slot `sl`, transposed) fr
    auto second_product = [&](int sl) {
      const int ys = sl * kSlot + (PW ? kTileBytes : 0);
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 ya[2][2][D / 32];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int d = 0; d < D / 32; ++d) ya[b][st][d] = tr_frag<D>(smem, ys, ta[d], b * kBlk + 16 * st);
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int d = 0; d < D / 32; ++d)
            acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ya[b][st][d], fr[b][st], acc[d], 0, 0, 0);
      // order: the reads of three fragments (two transposing reads each), then each MFMA
      // followed by the reads of the fragment three MFMAs ahead
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * 3, 0);
#pragma unroll
      for (int m = 0; m < 4 * (D / 32); ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (m + 3 < 4 * (D / 32)) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // P = exp2(c x), masked (MASK) to keys <= query (causal), key < N and query < N; to
    // fr and to LDS
    auto make_p = [&](auto mask_tag, int qt) {
      constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int qb0 = qt * kTile + b * kBlk;
        // query index minus this lane's offset 4h, against the limits
        const int lo_lim = CAUSAL ? key - qb0 - 4 * hi : -1;  // query offset >= lo_lim
        const int hi_lim = key < N ? N - qb0 - 4 * hi : -1;    // query offset < hi_lim
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pr = __builtin_amdgcn_exp2f(x[b][r] * p.c);
          if (MASK) {
            const int qo = 8 * (r >> 2) + (r & 3);
            if (qo < lo_lim || qo >= hi_lim) pr = 0.f;
          }
          fr[b][r >> 3][r & 7] = (__bf16)pr;
        }
        *reinterpret_cast<bf16x8*>(smem + pbase + b * kPBlock) = fr[b][0];
        *reinterpret_cast<bf16x8*>(smem + pbase + b * kPBlock + 1024) = fr[b][1];
      }
    };
    // dS = P (dP - Delta), P from the P wave through LDS
    auto make_ds = [&]() {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const bf16x8 pv = *reinterpret_cast<const bf16x8*>(smem + pbase + b * kPBlock + u * 1024);
#pragma unroll
          for (int i = 0; i < 8; ++i) fr[b][u][i] = (__bf16)((float)pv[i] * x[b][8 * u + i]);
        }
    };

    for (int qt = qt_first; qt < qt_end; ++qt) {
      const int sl = (qt - qt_first) & 1;
      wait_copies_and_barrier();
      if (qt + 1 < qt_end) load(qt + 1, sl ^ 1);
      first_product(sl);
      if constexpr (PW) {
        // every query of the tile sees every key of the pair, all in range
        const bool plain = (!CAUSAL || qt * kTile >= k0 + kBlk - 1) &&
                           qt * kTile + kTile <= N && k0 + kBlk <= N;
        if (plain) make_p(std::false_type{}, qt);
        else make_p(std::true_type{}, qt);
      }
      __syncthreads();
      if constexpr (!PW) make_ds();
      second_product(sl);
    }
  };
  if (qt_first < qt_end) load(qt_first, 0);
  if (pw) role(std::true_type{});
  else role(std::false_type{});
  if (key < N) {
    if (pw) store_rows<D>(p.dv + head + (size_t)key * D, acc, hi, 1.f);
    else store_rows<D>(p.dk + head + (size_t)key * D, acc, hi, p.scale);
  }
}

// ---- dkdv at D = 64: workgroup = 128 keys, wave = 32 keys holding both K and V (16 + 16
// registers) and both accumulators (32 + 32); query tiles of 64 stream through LDS. At
// D = 128 the same layout leaves too few of a wave's 256 registers for two waves per SIMD,
// hence the two-role kernel above; at D = 64 this one is the faster (its 16 MFMAs per
// block need no barrier in the middle of a tile).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dkdv1_kernel(const BwdParams p) {
  static_assert(D == 64, "one wave holds both K and V only at D = 64");
  constexpr bool kDv = true;
  constexpr bool kDk = true;
  constexpr int RB = 2 * D;
  constexpr int kTileBytes = kTile * RB;
  constexpr int kSlot = 2 * kTileBytes + 2 * kTile * 4;  // Q, dO, -lse/scale, -Delta
  __shared__ __attribute__((aligned(1024))) char smem[2 * kSlot];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int hi = lane >> 5;
  const int N = p.N;

  const int g = remap_block(blockIdx.x, p.remap);
  const int bh = g / p.n_wg_tiles;
  const int kt = g - bh * p.n_wg_tiles;
  const size_t head = (size_t)bh * N * D;
  const int k0 = kt * kWgRows + wave * kBlk;  // first key of this wave
  const int key = k0 + col;

  // K and V as B operands (lane = key, k = D index 16st + 8h .. +7)
  bf16x8 kf[D / 16], vf[D / 16];
  {
    const int r = min(key, N - 1);
    const bf16x8* ks = reinterpret_cast<const bf16x8*>(p.k + head + (size_t)r * D) + hi;
    const bf16x8* vs = reinterpret_cast<const bf16x8*>(p.v + head + (size_t)r * D) + hi;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      kf[s] = ks[2 * s];
      if (kDk) vf[s] = vs[2 * s];
    }
  }
  f32x16 dv[D / 32], dk[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) {
    dv[d] = f32x16{};
    dk[d] = f32x16{};
  }

  const uint32_t head_bytes = (uint32_t)N * RB;
  const i32x4 qrsrc = make_rsrc(p.q + head, head_bytes);
  const i32x4 orsrc = make_rsrc(p.dout + head, head_bytes);
  const i32x4 lrsrc = make_rsrc(p.nls + (size_t)bh * N, (uint32_t)N * 4u);
  const i32x4 drsrc = make_rsrc(p.ndelta + (size_t)bh * N, (uint32_t)N * 4u);
  const uint32_t smem_lds = lds_address(smem);

  // query tiles: causal workgroups start at their first key
  const int qt_first = CAUSAL ? (kt * kWgRows) / kTile : 0;
  const int qt_end = (N + kTile - 1) / kTile;
  auto load = [&](int qt, int slot) {
    const uint32_t base = smem_lds + slot * kSlot;
    copy_tile<D, kTile, kWaves>(qrsrc, qt * kTile, N, base, wave, lane);
    copy_tile<D, kTile, kWaves>(orsrc, qt * kTile, N, base + kTileBytes, wave, lane);
    if (wave == 0) copy_vec64(lrsrc, qt * kTile, N, base + 2 * kTileBytes, lane);
    if (kDk && wave == 1) copy_vec64(drsrc, qt * kTile, N, base + 2 * kTileBytes + kTile * 4, lane);
  };

  const int rbase = row_read_base<D>(col, hi);
  int ta[D / 32][2];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) {
    ta[d][0] = tr_read_addr<D>(lane, d, 0);
    ta[d][1] = tr_read_addr<D>(lane, d, 1);
  }

  if (qt_first < qt_end) load(qt_first, 0);
  for (int qt = qt_first; qt < qt_end; ++qt) {
    const int slot = (qt - qt_first) & 1;
    wait_copies_and_barrier();
    if (qt + 1 < qt_end) load(qt + 1, slot ^ 1);
    const int qs = slot * kSlot;                  // Q tile
    const int os = qs + kTileBytes;               // dO tile
    const int ls = qs + 2 * kTileBytes;           // -lse / scale
    const int ds = ls + kTile * 4;                // -Delta
#pragma unroll
    for (int b = 0; b < kTile / kBlk; ++b) {
      const int qb0 = qt * kTile + b * kBlk;  // first query of this block
      if (CAUSAL && qb0 + kBlk - 1 < k0) continue;  // every query precedes every key
      if (k0 >= N) continue;                        // wave past the last key
      // register r holds query qb0 + 8(r/4) + 4h + r%4 of key `key`; the accumulators
      // start at -lse / scale and -Delta of their query
      f32x16 s, dp;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(smem + ls + (b * kBlk + 8 * g4 + 4 * hi) * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) s[4 * g4 + i] = a[i];
        if (kDk) {
          const f32x4 d = *reinterpret_cast<const f32x4*>(smem + ds + (b * kBlk + 8 * g4 + 4 * hi) * 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) dp[4 * g4 + i] = d[i];
        }
      }
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(smem + qs + b * kBlk * RB + row_read_addr(rbase, st));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[st], s, 0, 0, 0);
        if (kDk) {
          const bf16x8 oa = *reinterpret_cast<const bf16x8*>(smem + os + b * kBlk * RB + row_read_addr(rbase, st));
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vf[st], dp, 0, 0, 0);
        }
      }
      const bool need_mask = (CAUSAL && qb0 < k0 + kBlk - 1) || (qb0 + kBlk > N);
      // visible iff query < N and (causal) key <= query: query index minus this lane's
      // offset 4h, against the limits
      const int lo_lim = CAUSAL ? key - qb0 - 4 * hi : -1;  // need query offset >= lo_lim
      const int hi_lim = N - qb0 - 4 * hi;                  // need query offset < hi_lim
      float pr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(s[r] * p.c);
      if (need_mask) {  // wave-uniform: only diagonal and ragged blocks pay for the selects
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qo = 8 * (r >> 2) + (r & 3);
          if (qo < lo_lim || qo >= hi_lim) pr[r] = 0.f;
        }
      }
      bf16x8 pb[2], sb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (kDv) pb[r >> 3][r & 7] = (__bf16)pr[r];
        if (kDk) sb[r >> 3][r & 7] = (__bf16)(pr[r] * dp[r]);
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the block's 32 queries (two k-steps of 16)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int d = 0; d < D / 32; ++d) {
          if (kDv) {
            const bf16x8 oa = tr_frag<D>(smem, os, ta[d], b * kBlk + 16 * st);
            dv[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, pb[st], dv[d], 0, 0, 0);
          }
          if (kDk) {
            const bf16x8 qa = tr_frag<D>(smem, qs, ta[d], b * kBlk + 16 * st);
            dk[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, sb[st], dk[d], 0, 0, 0);
          }
        }
      }
    }
  }
  if (key < N) {
    if (kDv) store_rows<D>(p.dv + head + (size_t)key * D, dv, hi, 1.f);
    if (kDk) store_rows<D>(p.dk + head + (size_t)key * D, dk, hi, p.scale);
  }
}

// ---- dq: workgroup = 128 queries, wave = 32 queries; key tiles of 64 stream through LDS.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dq_kernel(const BwdParams p) {
  constexpr int RB = 2 * D;
  constexpr int kTileBytes = kTile * RB;
  constexpr int kSlot = 2 * kTileBytes;  // K, V
  __shared__ __attribute__((aligned(1024))) char smem[2 * kSlot];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int hi = lane >> 5;
  const int N = p.N;

  const int g = remap_block(blockIdx.x, p.remap);
  const int bh = g / p.n_wg_tiles;
  int qt = g - bh * p.n_wg_tiles;
  if (CAUSAL) qt = p.n_wg_tiles - 1 - qt;  // longest first
  const size_t head = (size_t)bh * N * D;
  const int q0 = qt * kWgRows + wave * kBlk;
  const int qrow = q0 + col;

  // Q and dO as B operands (lane = query, k = D index 16st + 8h .. +7)
  bf16x8 qf[D / 16], of[D / 16];
  float nls = 0.f, ndl = 0.f;
  {
    const int r = min(qrow, N - 1);
    const bf16x8* qs = reinterpret_cast<const bf16x8*>(p.q + head + (size_t)r * D) + hi;
    const bf16x8* os = reinterpret_cast<const bf16x8*>(p.dout + head + (size_t)r * D) + hi;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      qf[s] = qs[2 * s];
      of[s] = os[2 * s];
    }
    nls = p.nls[(size_t)bh * N + r];
    ndl = p.ndelta[(size_t)bh * N + r];
  }
  f32x16 dq[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) dq[d] = f32x16{};

  const uint32_t head_bytes = (uint32_t)N * RB;
  const i32x4 krsrc = make_rsrc(p.k + head, head_bytes);
  const i32x4 vrsrc = make_rsrc(p.v + head, head_bytes);
  const uint32_t smem_lds = lds_address(smem);

  const int wg_kv_end = CAUSAL ? min(N, (qt + 1) * kWgRows) : N;
  const int nt = (wg_kv_end + kTile - 1) / kTile;
  const int wave_kv_end = CAUSAL ? min(N, q0 + kBlk) : N;  // keys this wave needs
  auto load = [&](int t, int slot) {
    const uint32_t base = smem_lds + slot * kSlot;
    copy_tile<D, kTile, kWaves>(krsrc, t * kTile, N, base, wave, lane);
    copy_tile<D, kTile, kWaves>(vrsrc, t * kTile, N, base + kTileBytes, wave, lane);
  };

  const int rbase = row_read_base<D>(col, hi);
  int ta[D / 32][2];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) {
    ta[d][0] = tr_read_addr<D>(lane, d, 0);
    ta[d][1] = tr_read_addr<D>(lane, d, 1);
  }

  load(0, 0);
  for (int t = 0; t < nt; ++t) {
    const int slot = t & 1;
    wait_copies_and_barrier();
    if (t + 1 < nt) load(t + 1, slot ^ 1);
    const int ks = slot * kSlot;
    const int vs = ks + kTileBytes;
#pragma unroll
    for (int j = 0; j < kTile / kBlk; ++j) {
      const int kb0 = t * kTile + j * kBlk;  // first key of this block
      if (q0 >= N || kb0 >= wave_kv_end) continue;
      // the accumulators start at -lse / scale and -Delta of this lane's query
      f32x16 s = f32x16{} + nls, dp = f32x16{} + ndl;
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(smem + ks + j * kBlk * RB + row_read_addr(rbase, st));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[st], s, 0, 0, 0);
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(smem + vs + j * kBlk * RB + row_read_addr(rbase, st));
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, of[st], dp, 0, 0, 0);
      }
      // register r holds key kb0 + 8(r/4) + 4h + r%4 of query qrow
      const bool need_mask = (CAUSAL && kb0 + kBlk - 1 > q0) || (kb0 + kBlk > N);
      const int lim = (CAUSAL ? min(N, qrow + 1) : N) - kb0 - 4 * hi;  // key offset < lim
      float pr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(s[r] * p.c);
      if (need_mask) {  // wave-uniform: only diagonal and ragged blocks pay for the selects
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + (r & 3) >= lim) pr[r] = 0.f;
      }
      bf16x8 sb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) sb[r >> 3][r & 7] = (__bf16)(pr[r] * dp[r]);
      // dQ^T += K^T dS^T over the block's 32 keys
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int d = 0; d < D / 32; ++d) {
          const bf16x8 ka = tr_frag<D>(smem, ks, ta[d], j * kBlk + 16 * st);
          dq[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, sb[st], dq[d], 0, 0, 0);
        }
    }
  }
  if (qrow < N) store_rows<D>(p.dq + head + (size_t)qrow * D, dq, hi, p.scale);
}

template <int D>
void launch_bwd(int causal, int B, int H, hipStream_t s, const BwdParams& p) {
  const dim3 block(64 * kWaves);
  const int rows_per_block = 256 / (D / 8);
  hipLaunchKernelGGL(attn_bwd_delta_kernel<D>, dim3((p.rows + rows_per_block - 1) / rows_per_block),
                     block, 0, s, p);
  const dim3 grid((unsigned)(B * H * p.n_wg_tiles));
  const dim3 grid_kv((unsigned)(B * H * p.n_kv_tiles));
  if constexpr (D == 64) {
    if (causal) hipLaunchKernelGGL((attn_bwd_dkdv1_kernel<D, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_bwd_dkdv1_kernel<D, false>), grid, block, 0, s, p);
  } else {
    if (causal) hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, true>), grid_kv, dim3(128 * kPairs), 0, s, p);
    else hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, false>), grid_kv, dim3(128 * kPairs), 0, s, p);
  }
  if (causal) hipLaunchKernelGGL((attn_bwd_dq_kernel<D, true>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((attn_bwd_dq_kernel<D, false>), grid, block, 0, s, p);
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

extern "C" {

size_t attn_bwd_workspace_bytes(int B, int H, int N) {
  if (B < 1 || H < 1 || N < 1) return 0;
  return 2 * round_up((size_t)B * H * N * sizeof(float), 256);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, void* workspace,
             size_t workspace_bytes, int B, int H, int N, int D, int causal, float scale,
             void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace)
    return ATTN_BWD_EINVAL;
  if (B < 1 || H < 1 || N < 1) return ATTN_BWD_EINVAL;
  if (causal != 0 && causal != 1) return ATTN_BWD_EINVAL;
  if (!(scale > 0.f) || !isfinite(scale)) return ATTN_BWD_EINVAL;
  if (D != 64 && D != 128) return ATTN_BWD_EUNSUPPORTED;
  const int64_t n_tiles = ((int64_t)N + kWgRows - 1) / kWgRows;
  const int64_t grid = (int64_t)B * H * n_tiles;
  const int64_t grid_kv = (int64_t)B * H * (((int64_t)N + 32 * kPairs - 1) / (32 * kPairs));
  const int64_t rows = (int64_t)B * H * N;
  if ((int64_t)N * D >= ((int64_t)1 << 31) || grid_kv >= ((int64_t)1 << 31) ||
      rows * (D / 8) >= ((int64_t)1 << 31))
    return ATTN_BWD_EINVAL;
  if (workspace_bytes < attn_bwd_workspace_bytes(B, H, N)) return ATTN_BWD_EWORKSPACE;
  const uintptr_t a16 = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o |
                        (uintptr_t)dout | (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv;
  if ((a16 & 15u) != 0 || ((uintptr_t)lse & 3u) != 0 || ((uintptr_t)workspace & 255u) != 0)
    return ATTN_BWD_EALIGN;

  BwdParams p;
  p.q = static_cast<const __bf16*>(q);
  p.k = static_cast<const __bf16*>(k);
  p.v = static_cast<const __bf16*>(v);
  p.o = static_cast<const __bf16*>(o);
  p.dout = static_cast<const __bf16*>(dout);
  p.lse = lse;
  p.ndelta = static_cast<float*>(workspace);
  p.nls = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                    round_up((size_t)rows * sizeof(float), 256));
  p.dq = static_cast<__bf16*>(dq);
  p.dk = static_cast<__bf16*>(dk);
  p.dv = static_cast<__bf16*>(dv);
  p.N = N;
  p.n_wg_tiles = (int)n_tiles;
  p.rows = (int)rows;
  p.remap = (grid % 8 == 0) ? 1 : 0;
  p.n_kv_tiles = (N + 32 * kPairs - 1) / (32 * kPairs);
  p.remap_kv = ((int64_t)B * H * p.n_kv_tiles % 8 == 0) ? 1 : 0;
  p.c = scale * kLog2e;
  p.scale = scale;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (D == 64) launch_bwd<64>(causal, B, H, s, p);
  else launch_bwd<128>(causal, B, H, s, p);
  if (hipGetLastError() != hipSuccess) return ATTN_BWD_ELAUNCH;
  return ATTN_BWD_OK;
}

const char* attn_bwd_strerror(int code) {
  switch (code) {
    case ATTN_BWD_OK: return "success";
    case ATTN_BWD_EINVAL: return "invalid argument (NULL pointer, size < 1, causal not 0/1, scale not finite and > 0, or size overflow)";
    case ATTN_BWD_EUNSUPPORTED: return "unsupported head dimension (D must be 64 or 128)";
    case ATTN_BWD_EALIGN: return "misaligned pointer (tensors need 16 bytes, lse 4, workspace 256)";
    case ATTN_BWD_ELAUNCH: return "kernel launch failed";
    case ATTN_BWD_EWORKSPACE: return "workspace smaller than attn_bwd_workspace_bytes(B, H, N)";
    default: return "unknown error code";
  }
}

}  // extern "C"
