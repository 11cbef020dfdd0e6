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
//   * each wave owns 32 query rows (64 in the non-causal D = 64 ping-pong kernel). Two
//     kernels share the per-row arithmetic below and give identical results: the ping-pong
//     kernel (8 waves, 256 queries per workgroup, 512 at non-causal D = 64; one workgroup
//     per compute unit, two wave groups alternating matrix and vector phases on every
//     SIMD), used at D = 128 and for non-causal D = 64 on grids that fill the device;
//     and the four-wave kernel (128 queries per workgroup, two workgroups per compute
//     unit, each wave interleaving its own MFMAs and exponentials), used otherwise.
//   * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: lane l
//     then holds 16 keys of query (l % 32) per 32-key block, so the row max and row sum
//     are in-lane reductions plus one v_permlane32_swap between the two lane halves.
//   * the output is accumulated transposed, O^T = V^T P^T. The score registers of a lane
//     are already the B operand of that MFMA (8 keys of its query), given that the A
//     operand (V^T) pairs its k positions with the same 8 keys; V^T fragments come from
//     LDS through ds_read_b64_tr_b16, which transposes 4x16 bf16 blocks across lanes.
//   * K and V tiles of 64 keys are copied
//     global -> LDS by buffer_load ... lds into double-buffered rings; the K ring runs one
//     tile ahead, so the score MFMAs of tile t+1 overlap the exponentials of tile t. The
//     16-byte chunks of each tile row are permuted so that the K reads and the transposing
//     V reads are free of LDS bank conflicts. In the ping-pong kernel one wave group issues
//     all the copies, spaced out between its exponentials: issued in a burst, they queue
//     at the compute unit's vector-memory path and stall every wave behind them.
//   * the exp2 argument is fma(s, c, -m*c) with c = scale*log2(e) in fp32, on the fp32
//     accumulator (the scale is never folded into bf16 Q). The running max only moves
//     when a row's max grows by more than 2^8 (lazy rescaling), so O is rarely rescaled.
//   * blockIdx is remapped so that consecutive query tiles of one head land on the same
//     XCD (workgroups are dealt round-robin over the 8 XCDs), keeping that head's K/V in
//     one L2; causal launches take the longest query tiles first.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "attn_fwd.h"
#include "tile_lds.h"

namespace {

using namespace attn_tile;

constexpr int kWaves = 4;
constexpr int kQW = 32;              // query rows per wave
constexpr int kBr = kWaves * kQW;    // query rows per workgroup
constexpr int kWavesPP = 8;          // ping-pong kernel: waves per workgroup
constexpr int kBrPP = kWavesPP * kQW;  // ping-pong kernel: query rows per workgroup and block
// 32-query blocks per wave of the ping-pong kernel: two at D = 64 without the mask (each K
// or V fragment read from LDS then feeds two MFMAs, which halves the reads per MFMA that
// bound the D = 64 matrix phase), else one.
constexpr int pp_query_blocks(int D, bool causal) { return (D == 64 && !causal) ? 2 : 1; }
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold, in log2 units of probability

struct Params {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  int N;
  int n_qtiles;  // ceil(N / kBr)
  int n_units;   // ping-pong kernel: B * H * n_qtiles work units (the grid may be smaller)
  int remap;     // 1: grid size (ping-pong: unit count) is a multiple of 8, use the XCD order
  float c;       // scale * log2(e)
  int causal_pairs;  // causal ping-pong: 0, one unit per workgroup; else the number of (long,
                     // short) unit pairs that a persistent grid walks
};

// Both halves of the wave receive max(x[lane], x[lane ^ 32]).
__device__ inline float max_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// LDS tile layout. A K or V tile is BC rows (keys) of D bf16, row-major and unpadded; the
// 16-byte chunks of each row are permuted: logical chunk c of row r sits at physical chunk
// c ^ f(r). The LDS has 64 four-byte banks; a 16-byte-per-lane read is serviced 16 lanes
// at a time and an 8-byte one (including ds_read_b64_tr_b16) 32 lanes at a time, so a
// conflict-free read must spread each such lane group over all 64 banks.
//  * K tile (score MFMA A operand): 16 consecutive lanes read one logical chunk of 16
//    consecutive rows, so f must be a bijection on the rows' bank groups: for D = 128
//    (256-byte rows) f = 4(r & 3) + ((r >> 2) & 3) over r mod 16; for D = 64 (128-byte
//    rows, two per bank line) a 3-bit rotation of (r >> 1) & 7.
//  * V tile (transposing read): 32 lanes read two adjacent chunks (four 8-byte quarters)
//    of four consecutive rows, twice; f only has to separate those four rows in the chunk
//    bits above the two that vary: f = 4(r & 3) for D = 128, 4((r >> 1) & 1) for D = 64.
// With these choices every read address is a per-lane base (one per K step, one per V
// column block) plus a compile-time offset. The K permutation is attn_tile::swz.
template <int D>
__device__ inline int swz_v(int r) {
  if constexpr (D == 128) return (r & 3) << 2;
  return ((r >> 1) & 1) << 2;
}

template <int D, int BC, int W = kWaves>
struct TileLayout {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;                    // 16-byte chunks per row
  static constexpr int kTileBytes = BC * kRowBytes;        // one K or V tile
  static constexpr int kRowsPerCopy = 1024 / kRowBytes;    // rows one wave-wide copy fills
  static constexpr int kCopies = kTileBytes / 1024 / W;    // copies per wave per tile
  static constexpr int kLdsBytes = 4 * kTileBytes;         // K[2], V[2]
  static_assert(kCopies * 1024 * W == kTileBytes, "tile must split into 1 KiB copies per wave");
  static_assert(kChunks >= 8, "the chunk permutations need 8 chunks per row");
  // copies whose lane offsets differ (the permutations repeat every 16 / 4 rows)
  static constexpr int kPeriodK = 16 / kRowsPerCopy < kCopies ? 16 / kRowsPerCopy : kCopies;
  static constexpr int kPeriodV = 4 / kRowsPerCopy < 1 ? 1 : (4 / kRowsPerCopy < kCopies ? 4 / kRowsPerCopy : kCopies);
};

// Instruction order for the steady-state block "scores of tile t+1 || exponentials of
// tile t, then O += P V of tile t": each score MFMA is paired with a share of the
// exponential work, then the P V MFMAs follow. LDS reads run two MFMAs ahead of the MFMA
// that consumes them, so their latency is hidden behind the matrix core.
template <int D, int BC>
__device__ inline void interleave_schedule() {
  constexpr int kQkMfma = (BC / 32) * (D / 16);
  constexpr int kPvMfma = (BC / 16) * (D / 32);
  constexpr int kValu = 56 * (BC / 32);  // exponential work of the tile, roughly
  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // K reads for the first two MFMAs
#pragma unroll
  for (int i = 0; i < kQkMfma; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                // next DS read
    __builtin_amdgcn_sched_group_barrier(0x002, kValu / kQkMfma, 0);  // VALU
  }
#pragma unroll
  for (int i = 0; i < kPvMfma; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // transposing reads, two ahead
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
  }
}

template <int D, int BC, int W, bool CAUSAL>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(const Params p) {
  static_assert(D == 64 || D == 128, "head dimension");
  static_assert(BC == 64, "key tile");
  constexpr int kBc = BC;
  constexpr int NB = BC / 32;  // 32-key score blocks per tile
  using L = TileLayout<D, BC, W>;
  constexpr int RB = L::kRowBytes;
  constexpr int kBrW = W * kQW;  // query rows per workgroup
  __shared__ __attribute__((aligned(1024))) char smem[L::kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;  // query within the wave's 32-row block
  const int hi = lane >> 5;   // which half of the wave

  // ---- work unit: (batch*head, query tile)
  const int g = remap_block(blockIdx.x, p.remap);
  const int bh = g / p.n_qtiles;
  int qt = g - bh * p.n_qtiles;
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;  // longest tiles first
  const int N = p.N;
  const float c = p.c;
  const size_t head = (size_t)bh * (size_t)N * D;
  const __bf16* Qh = p.q + head;

  const int q0 = qt * kBrW + wave * kQW;  // first query row of this wave
  const int qrow = q0 + col;
  const bool wave_active = q0 < N;

  // ---- key range: the workgroup streams tiles up to its last query (causal) or N;
  // each wave computes only the tiles that hold keys visible to its rows.
  const int wg_kv_end = CAUSAL ? min(N, (qt + 1) * kBrW) : N;
  const int ntiles = (wg_kv_end + kBc - 1) / kBc;
  const int wave_tiles = !wave_active ? 0 : CAUSAL ? (min(N, q0 + kQW) + kBc - 1) / kBc : ntiles;

  // ---- K/V copies. Copy i of wave w fills tile rows (w*kCopies + i)*kRowsPerCopy +
  // lane/kChunks (kRowsPerCopy = 4 for D = 128, 8 for D = 64), lane l writing physical chunk l % kChunks, so it
  // fetches the logical chunk stored there. The per-lane source offsets inside a tile are
  // fixed; the tile start is the scalar offset. In a ragged last tile, rows at or past N
  // repeat key N-1 (finite data that receives probability 0), so no read leaves the tensor.
  const uint32_t head_bytes = (uint32_t)N * RB;
  const i32x4 krsrc = make_rsrc(p.k + head, head_bytes);
  const i32x4 vrsrc = make_rsrc(p.v + head, head_bytes);
  // Copy i starts 1 KiB after copy i-1 in both LDS and the source and covers rows
  // kRowsPerCopy further on; the permutations repeat every 16 (K) or 4 (V) rows, so copy
  // i's lane offsets are those of copy i % kPeriod plus (i / kPeriod) * kPeriod KiB.
  uint32_t koff[L::kPeriodK], voff[L::kPeriodV];
#pragma unroll
  for (int i = 0; i < L::kPeriodK; ++i) {
    const int row = (wave * L::kCopies + i) * L::kRowsPerCopy + lane / L::kChunks;
    koff[i] = row * RB + (((lane % L::kChunks) ^ swz<D>(row)) << 4);
  }
#pragma unroll
  for (int i = 0; i < L::kPeriodV; ++i) {
    const int row = (wave * L::kCopies + i) * L::kRowsPerCopy + lane / L::kChunks;
    voff[i] = row * RB + (((lane % L::kChunks) ^ swz_v<D>(row)) << 4);
  }
  const uint32_t smem_lds = lds_address(smem);
  auto copy_tile = [&](const i32x4& rsrc, const uint32_t* coff, int period, int t, uint32_t dst) {
    const int key0 = t * kBc;
    const uint32_t dst_w = dst + wave * L::kCopies * 1024;
    if (key0 + kBc <= N) {
#pragma unroll
      for (int i = 0; i < L::kCopies; ++i) {
        const uint32_t soff = __builtin_amdgcn_readfirstlane(key0 * RB + (i / period) * period * 1024);
        copy16_to_lds(rsrc, coff[i % period], soff, dst_w + i * 1024);
      }
    } else {
      // ragged last tile: rows at or past N - key0 repeat the last key
      const uint32_t last = (uint32_t)(N - key0 - 1);
      const uint32_t soff = __builtin_amdgcn_readfirstlane(key0 * RB);
#pragma unroll
      for (int i = 0; i < L::kCopies; ++i) {
        const uint32_t o = coff[i % period] + (i / period) * period * 1024;
        copy16_to_lds(rsrc, (min(o / RB, last) * RB) | (o % RB), soff, dst_w + i * 1024);
      }
    }
  };
  const uint32_t kbuf_lds[2] = {smem_lds, smem_lds + L::kTileBytes};
  const uint32_t vbuf_lds[2] = {smem_lds + 2 * L::kTileBytes, smem_lds + 3 * L::kTileBytes};

  auto copy_k = [&](int t, uint32_t dst) { copy_tile(krsrc, koff, L::kPeriodK, t, dst); };
  auto copy_v = [&](int t, uint32_t dst) { copy_tile(vrsrc, voff, L::kPeriodV, t, dst); };
  copy_k(0, kbuf_lds[0]);

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
  // Complete the Q loads here, visibly to the compiler (vmcnt(0)): otherwise it keeps them
  // pending into the main loop and waits on vmcnt there, i.e. on the K/V copies in flight.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  // ---- per-lane LDS read bases
  // K (A operand of S^T = K Q^T): lane (m + 32h) reads logical chunk 2st + h of row
  // 32j + m; the permutation depends on m only, so k_addr[st] covers every j and buffer.
  int k_addr[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) k_addr[st] = col * RB + 16 * ((2 * st + hi) ^ swz<D>(col));
  // V^T (A operand of O^T = V^T P^T) through ds_read_b64_tr_b16: in each 16-lane group
  // the source lane jj supplies 8 bytes of row 16st + 8u + 4h + (jj >> 2) at logical column
  // 32d + 16(grp & 1) + 4(jj & 3); the instruction hands lane jj column jj of that 4-row
  // block, so lane l ends up with V[4 consecutive keys][32d + l % 32]. The permutation
  // depends on (jj >> 2) and h only, so v_addr[d] covers every st, u and buffer.
  const int jj = lane & 15;
  const int grp = lane >> 4;
  int v_addr[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) {
    const int row = 4 * hi + (jj >> 2);
    const int chunk = 4 * d + 2 * (grp & 1) + ((jj >> 1) & 1);
    v_addr[d] = row * RB + 16 * (chunk ^ swz_v<D>(row)) + 8 * (jj & 1);
  }

  // S^T (NB blocks of 32 keys x 32 queries) of the K tile at LDS offset kb
  auto qk = [&](int kb, f32x16 (&s)[NB]) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      s[j] = f32x16{};
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        const char* a = smem + kb + k_addr[st] + 32 * j * RB;
        s[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(a), qf[st],
                                                       s[j], 0, 0, 0);
      }
    }
  };

  float m = -INFINITY;  // running max (raw scores) used by the exponentials of query qrow
  float l = 0.f;        // running sum of exp2(c*s - c*m) over this lane's keys
  f32x16 o[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) o[d] = f32x16{};

  // Masking of tile t: keys past N and, causal, keys after the query. Only a wave's last
  // tile can need it: a wave's rows span 32 queries and tiles 32 or 64 keys (aligned), so
  // every earlier tile ends before the wave's first query, and only the last tile can
  // pass N.
  auto mask_tile = [&](f32x16 (&s)[NB], int t) {
    const int key0 = t * kBc;
    if ((key0 + kBc > N) || (CAUSAL && key0 + kBc - 1 > q0)) {
      // register r of block j holds key key0 + 4*hi + (32j + 8(r/4) + r%4); it is visible
      // iff that key is < N and, causal, <= qrow
      const int limit = (CAUSAL ? min(N, qrow + 1) : N) - key0 - 4 * hi;
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * j + 8 * (r >> 2) + (r & 3) >= limit) s[j][r] = -INFINITY;
    }
  };
  // row max and (lazy) rescale of tile t; leaves the scores in s
  auto softmax_head = [&](f32x16 (&s)[NB]) {
    float mx = m;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[j][r]);
    mx = max_across_halves(mx);
    // Lazy rescale: keep the old max unless some row's max grew by more than a factor
    // 2^8 in probability. Exponentials then stay <= 256, and the final O / l uses the
    // same max in numerator and denominator, so the result is unchanged.
    if (__builtin_amdgcn_ballot_w64((mx - m) * c > kRescaleLog2)) {
      const float alpha = __builtin_amdgcn_exp2f((m - mx) * c);  // 0 on the first tile
      m = mx;
      l *= alpha;
#pragma unroll
      for (int d = 0; d < D / 32; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
    }
  };
  // exponentials of tile t (after softmax_head), then O^T += V^T P^T with the V tile at
  // LDS offset vb
  auto exp_pv = [&](const f32x16 (&s)[NB], int vb) {
    const float mc = m * c;
    float rs = 0.f;
    bf16x8 pb[2 * NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j][r], c, -mc));
        rs += e;
        pb[2 * j + (r >> 3)][r & 7] = (__bf16)e;
      }
    l += rs;
    // step st covers keys 16st..16st+15: lane half h holds keys 16st+4h+{0..3} (low four
    // k positions) and 16st+8+4h+{0..3} (high four), matching pb[st]
#pragma unroll
    for (int st = 0; st < kBc / 16; ++st) {
#pragma unroll
      for (int d = 0; d < D / 32; ++d) {
        const char* a0 = smem + vb + v_addr[d] + 16 * st * RB;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)a0);
        const bf16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a0 + 8 * RB));
        const bf16x8 a = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
        o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[st], o[d], 0, 0, 0);
      }
    }
  };

  // ---- pipeline: the K ring runs one tile ahead of the V ring, so the scores of tile
  // t+1 are formed while tile t goes through the exponentials and the P V product.
  constexpr int kK0 = 0, kK1 = L::kTileBytes, kV0 = 2 * L::kTileBytes, kV1 = 3 * L::kTileBytes;
  f32x16 sa[NB], sb[NB];
  wait_copies_and_barrier();
  if (wave_tiles > 0) qk(kK0, sa);
  if (ntiles > 1) copy_k(1, kbuf_lds[1]);
  copy_v(0, vbuf_lds[0]);
  wait_copies_and_barrier();

  // Every iteration t issues the copies of K(t+2) and V(t+1) and ends with one barrier;
  // all waves of the workgroup run ntiles iterations. A wave computes its tiles
  // 0..wave_tiles-1 (a causal wave stops at its diagonal): steady steps while a next tile
  // exists, then a last step, then barrier-only iterations.
  auto copies = [&](int t) {
    if (t + 2 < ntiles) copy_k(t + 2, kbuf_lds[t & 1]);
    if (t + 1 < ntiles) copy_v(t + 1, vbuf_lds[(t + 1) & 1]);
  };
  auto steady = [&](f32x16 (&cur)[NB], f32x16 (&nxt)[NB], int t) {
    copies(t);
    softmax_head(cur);
    qk((t & 1) ? kK0 : kK1, nxt);
    exp_pv(cur, (t & 1) ? kV1 : kV0);
    interleave_schedule<D, BC>();
    wait_copies_and_barrier();
  };
  auto last = [&](f32x16 (&cur)[NB], int t) {
    copies(t);
    mask_tile(cur, t);
    softmax_head(cur);
    exp_pv(cur, (t & 1) ? kV1 : kV0);
    wait_copies_and_barrier();
  };
  // Pairs of steady steps keep the scores of the current tile in sa at every trip of the
  // loop, so the accumulators keep their registers from one trip to the next.
  int t = 0;
  for (; t + 2 < wave_tiles; t += 2) {
    steady(sa, sb, t);
    steady(sb, sa, t + 1);
  }
  if (t + 1 < wave_tiles) {
    steady(sa, sb, t);
    last(sb, t + 1);
    t += 2;
  } else if (t < wave_tiles) {
    last(sa, t);
    t += 1;
  }
  for (; t < ntiles; ++t) {
    copies(t);
    wait_copies_and_barrier();
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
      if (hi == 0) p.lse[(size_t)bh * N + qrow] = (m * c + __builtin_log2f(lt)) * kLn2;
    }
  }
}

// ---- ping-pong kernel (D = 128, and non-causal D = 64 on grids that fill the device): one
// workgroup of 8 waves (two per SIMD, one workgroup per compute unit) covers 256 queries,
// or 512 at non-causal D = 64, where each wave takes two 32-query blocks (QB = 2) so that
// every K and V fragment it reads from LDS feeds two MFMAs.
// The waves form two groups (waves 0-3 are group 1, waves 4-7 group 0; waves w and w + 4
// share a SIMD) that run the same sequence of phases offset by one:
// a matrix phase (P V of tile j - 1, then the scores of tile j: MFMAs and the LDS reads
// feeding them) and a vector phase (mask, row max, lazy rescale and exponentials of tile
// j). A workgroup barrier ends every phase, so on every SIMD one wave's MFMAs run while
// the other wave's exponentials run; the matrix phase raises its wave's issue priority
// (s_setprio) so that its MFMAs are never starved by the other wave's VALU stream. The
// arithmetic per query row is that of attn_fwd_kernel, in the same order, so both kernels
// give bit-identical results.

// Instruction order of a full matrix phase: the LDS reads (two transposing V reads per P V
// MFMA, one K read per score MFMA) run kAhead MFMAs ahead of the MFMA that consumes them.
// reads_through(m) counts the reads that MFMAs 0..m need. Three ahead measured 0.1-1%
// faster than two, four no better.
constexpr int reads_through(int m, int kPv, int qb = 1) {
  return m < kPv ? 2 * (m / qb + 1) : 2 * (kPv / qb) + ((m - kPv) / qb + 1);
}
constexpr int cmin(int a, int b) { return a < b ? a : b; }
template <int kPv, int M, int kAhead, int QB, int m>
__device__ inline void matrix_phase_step() {
  if constexpr (m < M) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA m
    constexpr int n = reads_through(cmin(m + kAhead, M - 1), kPv, QB) -
                      reads_through(cmin(m + kAhead - 1, M - 1), kPv, QB);
    if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x100, n, 0);  // reads of MFMA m + kAhead
    matrix_phase_step<kPv, M, kAhead, QB, m + 1>();
  }
}
// QB query blocks per wave: every LDS read feeds QB consecutive MFMAs.
template <int D, int BC, int QB>
__device__ inline void matrix_phase_schedule() {
  constexpr int kPvMfma = QB * (BC / 16) * (D / 32);
  constexpr int kQkMfma = QB * (BC / 32) * (D / 16);
  constexpr int M = kPvMfma + kQkMfma;
  constexpr int kAhead = 3;
  __builtin_amdgcn_sched_group_barrier(0x100, reads_through(cmin(kAhead - 1, M - 1), kPvMfma, QB), 0);
  matrix_phase_step<kPvMfma, M, kAhead, QB, 0>();
}

template <int D, int BC, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_pp_kernel(const Params p) {
  static_assert(D == 64 || D == 128, "head dimension");
  static_assert(BC == 64, "key tile");
  constexpr int W = kWavesPP;
  constexpr int kBc = BC;
  constexpr int NB = BC / 32;
  constexpr int QB = pp_query_blocks(D, CAUSAL);  // 32-query blocks per wave
  constexpr int kQWave = QB * kQW;                 // query rows per wave
  using L = TileLayout<D, BC, W>;
  constexpr int RB = L::kRowBytes;
  constexpr int kBrW = W * kQWave;
  __shared__ __attribute__((aligned(1024))) char smem[L::kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Waves w and w + 4 share a SIMD, and waves 0-3 are dispatched first: on every SIMD they
  // are the older wave. The younger wave's matrix phase beside the older wave's dense
  // exponentials ran about 20% longer than the reverse pairing (instrumented, 1632 vs 1340
  // cycles), so the older waves form group 1 (vector phase first, with the copies) and the
  // younger ones group 0; both matrix phases then take about 1330 cycles.
  const int grp = (wave >> 2) ^ 1;
  const int col = lane & 31;
  const int hi = lane >> 5;

  // Work units. Non-causal: persistent when the launch has fewer workgroups than units (one
  // per compute unit): workgroup b walks units b, b + gridDim.x, ...; the XCD order is taken
  // over the units, so each XCD runs consecutive units of the same heads. Causal: with
  // causal_pairs = 0, one unit per workgroup (the loop below runs once), dispatched longest
  // first; otherwise a persistent grid in which workgroup b, iteration it, takes the pair
  // (b mod 8) * causal_pairs / 8 + b / 8 + (it / 2) * gridDim.x / 8 of its XCD's share: a
  // head's query tiles n - 1 - j and j, the long unit first. Every pair holds the same number
  // of key tiles, and an XCD's pairs cover consecutive heads.
  //
  // With kPrefetchNext (D = 128), a unit's Q rows and first K and V tiles are loaded while
  // the workgroup's previous unit finishes (see copies), so only its first unit waits for
  // them. At D = 64, where the kernel already uses 235 of its 256 registers, the extra live
  // values spilled and the kernel measured 0-2% slower; D = 128 gained 0.5-1.5% at B16 H16
  // N4096.
  constexpr bool kPrefetchNext = D == 128;
  // the unit's index g: head g / n_qtiles, query tile g mod n_qtiles (causal: counted from
  // the last tile)
  auto unit_index = [&](int gu, int it) {
    if constexpr (CAUSAL) {
      if (p.causal_pairs == 0) return remap_block(blockIdx.x, p.remap);
      const int half = p.n_qtiles >> 1;
      const int pair = (int)(blockIdx.x & 7) * (p.causal_pairs >> 3) + (int)(blockIdx.x >> 3) +
                       (it >> 1) * (int)(gridDim.x >> 3);
      const int bh = pair / half;
      const int j = pair - bh * half;
      return bh * p.n_qtiles + ((it & 1) ? p.n_qtiles - 1 - j : j);
    } else {
      return p.remap ? (gu & 7) * (p.n_units >> 3) + (gu >> 3) : gu;
    }
  };
  // the next unit's Q rows qrow + 32b, as the unit's own are loaded below
  auto load_next_q = [&](bf16x8 (&dst)[QB][D / 16], const __bf16* Qh, int qrow) {
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      if (qrow + kQW * b < p.N) {
        const bf16x8* src = reinterpret_cast<const bf16x8*>(Qh + (size_t)(qrow + kQW * b) * D) + hi;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) dst[b][s] = src[2 * s];
      } else {
#pragma unroll
        for (int s = 0; s < D / 16; ++s) dst[b][s] = bf16x8{};
      }
    }
  };
  bf16x8 qf_carried[QB][D / 16];  // with kPrefetchNext, loaded by the previous unit
  int it = 0;  // causal: this workgroup's unit count so far
  for (int gu = blockIdx.x;; gu += gridDim.x) {
  if (!CAUSAL && gu >= p.n_units) break;
  const int g = unit_index(gu, it);
  const int bh = g / p.n_qtiles;
  int qt = g - bh * p.n_qtiles;
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;
  const int N = p.N;
  const float c = p.c;
  const size_t head = (size_t)bh * (size_t)N * D;
  const __bf16* Qh = p.q + head;
  const int q0 = qt * kBrW + wave * kQWave;
  const int qrow = q0 + col;  // this lane's row of query block 0 (block b: qrow + 32b)
  const bool wave_active = q0 < N;
  const int wg_kv_end = CAUSAL ? min(N, (qt + 1) * kBrW) : N;
  const int ntiles = (wg_kv_end + kBc - 1) / kBc;
  const int T = !wave_active ? 0 : CAUSAL ? (min(N, q0 + kQWave) + kBc - 1) / kBc : ntiles;

  // K/V copies (the layout and ragged-tile rule of attn_fwd_kernel). Only the four waves
  // of group 1 copy, and in the steady state they spread their copies through their
  // vector phase (see softmax): a copy instruction moves 1 KiB, and a burst of them from
  // every wave at once queues at the compute unit's vector-memory path, stalling the
  // issue of each wave behind it.
  using LC = TileLayout<D, BC, kWavesPP / 2>;
  const int cw = wave & 3;  // copy index of a group-1 wave
  const uint32_t head_bytes = (uint32_t)N * RB;
  const i32x4 krsrc = make_rsrc(p.k + head, head_bytes);
  const i32x4 vrsrc = make_rsrc(p.v + head, head_bytes);
  uint32_t koff[LC::kPeriodK], voff[LC::kPeriodV];
#pragma unroll
  for (int i = 0; i < LC::kPeriodK; ++i) {
    const int row = (cw * LC::kCopies + i) * LC::kRowsPerCopy + lane / LC::kChunks;
    koff[i] = row * RB + (((lane % LC::kChunks) ^ swz<D>(row)) << 4);
  }
#pragma unroll
  for (int i = 0; i < LC::kPeriodV; ++i) {
    const int row = (cw * LC::kCopies + i) * LC::kRowsPerCopy + lane / LC::kChunks;
    voff[i] = row * RB + (((lane % LC::kChunks) ^ swz_v<D>(row)) << 4);
  }
  const uint32_t smem_lds = lds_address(smem);
  // copies i0 .. i1-1 of this wave's share of tile t
  auto copy_range = [&](const i32x4& rsrc, const uint32_t* coff, int period, int t, uint32_t dst,
                        int i0, int i1) {
    const int key0 = t * kBc;
    const uint32_t dst_w = dst + cw * LC::kCopies * 1024;
    if (key0 + kBc <= N) {
#pragma unroll
      for (int i = i0; i < i1; ++i) {
        const uint32_t soff = __builtin_amdgcn_readfirstlane(key0 * RB + (i / period) * period * 1024);
        copy16_to_lds(rsrc, coff[i % period], soff, dst_w + i * 1024);
      }
    } else {
      const uint32_t last = (uint32_t)(N - key0 - 1);
      const uint32_t soff = __builtin_amdgcn_readfirstlane(key0 * RB);
#pragma unroll
      for (int i = i0; i < i1; ++i) {
        const uint32_t o = coff[i % period] + (i / period) * period * 1024;
        copy16_to_lds(rsrc, (min(o / RB, last) * RB) | (o % RB), soff, dst_w + i * 1024);
      }
    }
  };
  const uint32_t kbuf_lds[2] = {smem_lds, smem_lds + L::kTileBytes};
  const uint32_t vbuf_lds[2] = {smem_lds + 2 * L::kTileBytes, smem_lds + 3 * L::kTileBytes};
  auto copy_k = [&](int t, int i0, int i1) { copy_range(krsrc, koff, LC::kPeriodK, t, kbuf_lds[t & 1], i0, i1); };
  auto copy_v = [&](int t, int i0, int i1) { copy_range(vrsrc, voff, LC::kPeriodV, t, vbuf_lds[t & 1], i0, i1); };
  // The workgroup's next unit: with kPrefetchNext its K(0), K(1) and Q rows are loaded in
  // this unit's last slot pair, its V(0) after that pair's last barrier. Its offsets are
  // formed where they are used, so that they hold no registers in the loop.
  // more: this workgroup has a next unit (known here only where it is used)
  bool more = false;
  if constexpr (CAUSAL) more = p.causal_pairs > 0 && it + 1 < 2 * p.causal_pairs / (int)gridDim.x;
  else if constexpr (kPrefetchNext) more = gu + (int)gridDim.x < p.n_units;
  const bool has_next = kPrefetchNext && more;
  auto next_unit = [&](size_t& head_n, int& q0_n, int& nt_n) {
    const int g_n = unit_index(gu + (int)gridDim.x, it + 1);
    const int bh_n = g_n / p.n_qtiles;
    int qt_n = g_n - bh_n * p.n_qtiles;
    if (CAUSAL) qt_n = p.n_qtiles - 1 - qt_n;
    head_n = (size_t)bh_n * (size_t)N * D;
    q0_n = qt_n * kBrW + wave * kQWave;
    nt_n = CAUSAL ? (min(N, (qt_n + 1) * kBrW) + kBc - 1) / kBc : ntiles;
  };
  // A unit that the previous one did not prefetch (a workgroup's first unit, every unit
  // where kPrefetchNext is off) loads its K(0) and Q rows here, and K(1) and V(0) in pair 0.
  const bool prefetched = kPrefetchNext && (CAUSAL ? it > 0 : gu != (int)blockIdx.x);
  bf16x8 qf_unit[QB][D / 16];
  bf16x8 (&qf)[QB][D / 16] = kPrefetchNext ? qf_carried : qf_unit;
  if (!prefetched) {
    if (grp == 1) copy_k(0, 0, LC::kCopies);
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      if (qrow + kQW * b < N) {
        const bf16x8* src = reinterpret_cast<const bf16x8*>(Qh + (size_t)(qrow + kQW * b) * D) + hi;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) qf[b][s] = src[2 * s];
      } else {
#pragma unroll
        for (int s = 0; s < D / 16; ++s) qf[b][s] = bf16x8{};
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  int k_addr[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) k_addr[st] = col * RB + 16 * ((2 * st + hi) ^ swz<D>(col));
  const int jj = lane & 15;
  const int gq = lane >> 4;
  int v_addr[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) {
    const int row = 4 * hi + (jj >> 2);
    const int chunk = 4 * d + 2 * (gq & 1) + ((jj >> 1) & 1);
    v_addr[d] = row * RB + 16 * (chunk ^ swz_v<D>(row)) + 8 * (jj & 1);
  }

  // per query block b: running max m, sum l, O^T accumulators, scores and P
  float m[QB], l[QB];
  f32x16 o[QB][D / 32];
  f32x16 s[QB][NB];
  bf16x8 pb[QB][2 * NB];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    m[b] = -INFINITY;
    l[b] = 0.f;
#pragma unroll
    for (int d = 0; d < D / 32; ++d) o[b][d] = f32x16{};
#pragma unroll
    for (int j = 0; j < NB; ++j) s[b][j] = f32x16{};
#pragma unroll
    for (int j = 0; j < 2 * NB; ++j) pb[b][j] = bf16x8{};
  }

  auto qk = [&](int t) {
    const int kb = (t & 1) * L::kTileBytes;
    // the NB x QB accumulation chains alternate, so consecutive MFMAs are independent;
    // each K fragment read serves the QB query blocks
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
      for (int j = 0; j < NB; ++j) s[b][j] = f32x16{};
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const char* a = smem + kb + k_addr[st] + 32 * j * RB;
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(a);
#pragma unroll
        for (int b = 0; b < QB; ++b)
          s[b][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[b][st], s[b][j], 0, 0, 0);
      }
    }
  };
  auto pv = [&](int t) {
    const int vb = 2 * L::kTileBytes + (t & 1) * L::kTileBytes;
#pragma unroll
    for (int st = 0; st < kBc / 16; ++st) {
#pragma unroll
      for (int d = 0; d < D / 32; ++d) {
        const char* a0 = smem + vb + v_addr[d] + 16 * st * RB;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)a0);
        const bf16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a0 + 8 * RB));
        const bf16x8 a = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int b = 0; b < QB; ++b)
          o[b][d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[b][st], o[b][d], 0, 0, 0);
      }
    }
  };
  // The copies of slot pair i (see below), one per part: this wave's share of K(i+1) in
  // parts 0 .. kCopies-1, of V(i) in the rest. Only for pairs whose two tiles exist and
  // are full, so that no branch separates the parts from the exponentials between them.
  constexpr int kParts = 2 * LC::kCopies;
  auto copy_part = [&](int i, int part) {
    const bool isk = part < LC::kCopies;
    const int t = isk ? i + 1 : i;
    const i32x4& rsrc = isk ? krsrc : vrsrc;
    const uint32_t dst = (isk ? kbuf_lds[t & 1] : vbuf_lds[t & 1]) + cw * LC::kCopies * 1024;
    const int ci = isk ? part : part - LC::kCopies;
    const int period = isk ? LC::kPeriodK : LC::kPeriodV;
    const uint32_t off = isk ? koff[ci % LC::kPeriodK] : voff[ci % LC::kPeriodV];
    const uint32_t soff = __builtin_amdgcn_readfirstlane(t * kBc * RB + (ci / period) * period * 1024);
    copy16_to_lds(rsrc, off, soff, dst + ci * 1024);
  };
  // vector phase of tile t: mask (a wave's last tile only), row max, lazy rescale,
  // exponentials into pb and their sum into l. With copy_pair >= 0 the copies of that
  // slot pair go out one at a time, evenly spaced between the exponentials (the
  // scheduling barriers keep them spread: 4 exponentials apart at D = 128).
  auto softmax = [&](int t, bool last, int copy_pair) {
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      if (last) {
        const int key0 = t * kBc;
        if ((key0 + kBc > N) || (CAUSAL && key0 + kBc - 1 > q0 + kQW * b)) {
          const int limit = (CAUSAL ? min(N, qrow + kQW * b + 1) : N) - key0 - 4 * hi;
#pragma unroll
          for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * j + 8 * (r >> 2) + (r & 3) >= limit) s[b][j][r] = -INFINITY;
        }
      }
      float mx = m[b];
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[b][j][r]);
      mx = max_across_halves(mx);
      if (__builtin_amdgcn_ballot_w64((mx - m[b]) * c > kRescaleLog2)) {
        const float alpha = __builtin_amdgcn_exp2f((m[b] - mx) * c);
        m[b] = mx;
        l[b] *= alpha;
#pragma unroll
        for (int d = 0; d < D / 32; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[b][d][r] *= alpha;
      }
      const float mc = m[b] * c;
      float rs = 0.f;
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          constexpr int kEvery = 16 * NB * QB / kParts;
          const int e_idx = 16 * NB * b + 16 * j + r;  // exponential index in the tile
          if (copy_pair >= 0 && e_idx % kEvery == 0) {
            __builtin_amdgcn_sched_barrier(0);
            copy_part(copy_pair, e_idx / kEvery);
            __builtin_amdgcn_sched_barrier(0);
          }
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][j][r], c, -mc));
          rs += e;
          pb[b][2 * j + (r >> 3)][r & 7] = (__bf16)e;
        }
      l[b] += rs;
    }
  };

  // Slot pairs i = 0 .. ntiles (two barriers each). The copies of K(i+1) and V(i) are
  // issued by group 1 in the first slot of pair i (spread through its vector phase in the
  // steady state) and waited for at the end of the pair; K(i+1) goes to the K slot
  // that held K(i-1), last read in pair i-1, and V(i) to the V slot that held V(i-2), last
  // read in pair i-1 too (two-slot rings). The last pair, ntiles, has none of this unit;
  // with kPrefetchNext, both K slots and the Q registers being free there (last read in
  // pair ntiles - 1), it issues the next unit's K(0), K(1) and Q (Q once the wave's last
  // exponentials are done) and ends without waiting for them; the next unit's V(0) goes
  // out after that pair's last barrier, so a prefetched unit has no copies in pair 0.
  // Group 0 runs, in pair i, the matrix phase of step i (P V of tile i-1, scores of tile
  // i) and then the vector phase of tile i; group 1 runs the vector phase of tile i-1 and
  // then the matrix phase of step i.
  // Each group's sequence is straight-line code (first and last steps peeled), so the
  // accumulators keep their registers across the loop.
  auto copies_mid = [&](int i) {  // pairs 1 .. ntiles - 1, where every unit copies
    if (grp == 1) {
      if (i + 1 < ntiles) copy_k(i + 1, 0, LC::kCopies);
      if (i < ntiles) copy_v(i, 0, LC::kCopies);
    }
  };
  auto copies = [&](int i) {
    if constexpr (!kPrefetchNext) {
      copies_mid(i);
    } else if (i == ntiles) {
      if (has_next) {
        if (grp == 1) {
          size_t head_n;
          int q0_n, nt_n;
          next_unit(head_n, q0_n, nt_n);
          const i32x4 krsrc_n = make_rsrc(p.k + head_n, head_bytes);
          copy_range(krsrc_n, koff, LC::kPeriodK, 0, kbuf_lds[0], 0, LC::kCopies);
          if (1 < nt_n) copy_range(krsrc_n, koff, LC::kPeriodK, 1, kbuf_lds[1], 0, LC::kCopies);
        }
      }
    } else if (i > 0 || !prefetched) {
      copies_mid(i);
    }
  };
  // the next unit's Q rows, once this wave's last scores are consumed
  auto prefetch_q = [&]() {
    if (kPrefetchNext && has_next) {
      size_t head_n;
      int q0_n, nt_n;
      next_unit(head_n, q0_n, nt_n);
      load_next_q(qf, p.q + head_n, q0_n + col);
    }
  };
  auto end_pair = [&](int i) {
    if (kPrefetchNext && has_next && i == ntiles) __syncthreads();
    else wait_copies_and_barrier();
  };
  // A full matrix phase: the P V MFMAs of tile i-1 (key step st, output block d, in that
  // order), then the score MFMAs of tile i (step st, key block j), each LDS read feeding
  // its QB MFMAs. In the non-causal kernel, whose persistent loop leaves the compiler
  // fewer registers, it is written software-pipelined in the source: the A operand of
  // read r+3 is read before the MFMAs of read r, into one of four rotating fragments.
  // Where a scheduling region runs short of registers the compiler keeps the source order;
  // written this way that order still hides the LDS latency (a fragment read right before
  // its MFMA would make every MFMA wait for its read). Same MFMAs in the same order as
  // pv + qk, so the same bits.
  auto matrix = [&](int i) {  // P V of tile i-1 and scores of tile i, both present
    __builtin_amdgcn_s_setprio(2);
    if constexpr (CAUSAL) {
      pv(i - 1);
      qk(i);
    } else {
      constexpr int kPvR = (kBc / 16) * (D / 32);
      constexpr int kR = kPvR + (D / 16) * NB;
      const int vb = 2 * L::kTileBytes + ((i - 1) & 1) * L::kTileBytes;
      const int kb = (i & 1) * L::kTileBytes;
      auto operand = [&](int r) {
        if (r < kPvR) {  // V^T fragment of key step r / (D/32), output block r % (D/32)
          const char* a0 = smem + vb + v_addr[r % (D / 32)] + 16 * (r / (D / 32)) * RB;
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)a0);
          const bf16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a0 + 8 * RB));
          return __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
        }
        const int q = r - kPvR;  // K fragment of step q / NB, key block q % NB
        return *reinterpret_cast<const bf16x8*>(smem + kb + k_addr[q / NB] + 32 * (q % NB) * RB);
      };
      bf16x8 fr[4];
      fr[0] = operand(0);
      fr[1] = operand(1);
      fr[2] = operand(2);
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        if (r + 3 < kR) fr[(r + 3) & 3] = operand(r + 3);
#pragma unroll
        for (int b = 0; b < QB; ++b) {
          if (r < kPvR) {
            const int d = r % (D / 32);
            o[b][d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[r & 3], pb[b][r / (D / 32)], o[b][d], 0, 0, 0);
          } else {
            const int q = r - kPvR, j = q % NB;
            s[b][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[r & 3], qf[b][q / NB],
                                                             q < NB ? f32x16{} : s[b][j], 0, 0, 0);
          }
        }
      }
    }
    matrix_phase_schedule<D, BC, QB>();
    __builtin_amdgcn_s_setprio(0);
  };
  wait_copies_and_barrier();
  int i = 0;
  if (T > 0) {
    if (grp == 0) {
      copies(0);
      qk(0);
      __syncthreads();
      if (T == 1) {
        softmax(0, true, -1);
      } else {
        softmax(0, false, -1);
      }
      wait_copies_and_barrier();
      for (i = 1; i + 1 < T; ++i) {
        copies_mid(i);
        matrix(i);
        __syncthreads();
        softmax(i, false, -1);
        wait_copies_and_barrier();
      }
      if (i < T) {  // i == T - 1 >= 1
        copies_mid(i);
        matrix(i);
        __syncthreads();
        softmax(i, true, -1);
        wait_copies_and_barrier();
        ++i;
      }
      copies(i);  // i == T
      prefetch_q();
      pv(T - 1);
      __syncthreads();
      end_pair(i);
      ++i;
    } else {
      copies(0);
      __syncthreads();
      qk(0);
      wait_copies_and_barrier();
      // pairs whose copies are of full tiles (K(i+1) and V(i) end at or before N) spread
      // them through the exponentials; the rest issue them at once
      const int i_spread = min(T, min(ntiles, N / kBc) - 1);
      for (i = 1; i < i_spread; ++i) {
        softmax(i - 1, false, i);
        __syncthreads();
        matrix(i);
        wait_copies_and_barrier();
      }
      for (; i < T; ++i) {
        copies_mid(i);
        softmax(i - 1, false, -1);
        __syncthreads();
        matrix(i);
        wait_copies_and_barrier();
      }
      copies(i);  // i == T
      softmax(T - 1, true, -1);
      __syncthreads();
      prefetch_q();
      pv(T - 1);
      end_pair(i);
      ++i;
    }
  }
  for (; i <= ntiles; ++i) {
    copies(i);
    if (kPrefetchNext && i == ntiles) prefetch_q();
    __syncthreads();
    end_pair(i);
  }
  // every read of this unit's V tiles is behind the last barrier
  if (kPrefetchNext && has_next && grp == 1) {
    size_t head_n;
    int q0_n, nt_n;
    next_unit(head_n, q0_n, nt_n);
    copy_range(make_rsrc(p.v + head_n, head_bytes), voff, LC::kPeriodV, 0, vbuf_lds[0], 0, LC::kCopies);
  }

  if (wave_active) {
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const float lt = sum_across_halves(l[b]);
      const int row = qrow + kQW * b;
      if (row < N) {
        const float inv = 1.f / lt;
        __bf16* orow = p.o + head + (size_t)row * D;
#pragma unroll
        for (int d = 0; d < D / 32; ++d)
#pragma unroll
          for (int j4 = 0; j4 < 4; ++j4) {
            bf16x4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = (__bf16)(o[b][d][4 * j4 + i] * inv);
            *reinterpret_cast<bf16x4*>(orow + 32 * d + 8 * j4 + 4 * hi) = w;
          }
        if (hi == 0) p.lse[(size_t)bh * N + row] = (m[b] * c + __builtin_log2f(lt)) * kLn2;
      }
    }
  }
  if constexpr (CAUSAL) {
    if (!more) break;
    ++it;
  }
  }  // work units
}

// Kernel choice. D = 128 runs the ping-pong kernel. D = 64 runs the ping-pong kernel when
// the mask is off and its grid (one workgroup of 512 queries per compute unit) fills the
// device, else the four-wave kernel. At D = 64 a vector phase costs as much as at D = 128
// while a matrix phase halves; measured on MI355X (interleaved, 200 launches each), the
// ping-pong kernel with one query block per wave was already 3-7% faster non-causal
// (B16 H16 N1024 to B1 H32 N4096), and two blocks per wave add 7-10%; it is 10% slower
// causal, where the waves of a workgroup stop at different diagonal tiles, and slower on
// grids that leave compute units idle (B1 H4 N8192: 570 vs 630 TFLOP/s).
// attn_fwd_ex can force either kernel, for tests and tuning.
bool use_pingpong(int D, int64_t pp_grid, int causal, int cus) {
  if (D == 128) return true;
  return !causal && pp_grid >= cus;
}

// Compute units per device, queried once per device.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];
std::mutex g_cus_mutex;

int device_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_FWD_ELAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return ATTN_FWD_ELAUNCH;
  int n = g_cus[dev].load(std::memory_order_acquire);
  if (n == 0) {
    std::lock_guard<std::mutex> lock(g_cus_mutex);
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return ATTN_FWD_ELAUNCH;
    g_cus[dev].store(n, std::memory_order_release);
  }
  *cus = n;
  return ATTN_FWD_OK;
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

int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int N, int D, int causal, float scale, int kernel, void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_FWD_EINVAL;
  if (B < 1 || H < 1 || N < 1) return ATTN_FWD_EINVAL;
  if (causal != 0 && causal != 1) return ATTN_FWD_EINVAL;
  if (!(scale > 0.f) || !isfinite(scale)) return ATTN_FWD_EINVAL;
  if (kernel != ATTN_FWD_KERNEL_AUTO && kernel != ATTN_FWD_KERNEL_PINGPONG &&
      kernel != ATTN_FWD_KERNEL_FOURWAVE)
    return ATTN_FWD_EINVAL;
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
  p.n_units = 0;
  p.causal_pairs = 0;
  p.c = scale * kLog2e;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t rows_pp = (int64_t)kBrPP * pp_query_blocks(D, causal != 0);
  const int64_t n_qtiles_pp = ((int64_t)N + rows_pp - 1) / rows_pp;
  const int64_t grid_pp = (int64_t)B * H * n_qtiles_pp;
  bool pingpong = kernel == ATTN_FWD_KERNEL_PINGPONG;
  if (kernel == ATTN_FWD_KERNEL_AUTO) {
    int cus = 0;
    if (D == 64 && !causal) {  // the compute units of the current device decide the D = 64 kernel
      const int rc = device_cus(&cus);
      if (rc != ATTN_FWD_OK) return rc;
    }
    pingpong = use_pingpong(D, grid_pp, causal, cus);
  }
  if (pingpong) {
    p.n_qtiles = (int)n_qtiles_pp;
    p.n_units = (int)grid_pp;
    p.remap = (grid_pp % 8 == 0) ? 1 : 0;
    // Launches with more units than compute units: a persistent grid of one workgroup per
    // compute unit (a multiple of 8: the same share of every XCD). Causal D = 128 launches
    // take it when a head's query tiles pair up (an even count) and the pairs split evenly
    // over the grid; otherwise one unit per workgroup, longest first.
    int cus = 0;
    if (!causal || D == 128) {
      const int rc = device_cus(&cus);
      if (rc != ATTN_FWD_OK) return rc;
    }
    const int64_t per_cu = cus >= 8 ? cus / 8 * 8 : 0;
    int64_t persistent = (!causal && per_cu > 0 && grid_pp > per_cu) ? per_cu : 0;
    if (causal && D == 128 && per_cu > 0 && grid_pp > per_cu && n_qtiles_pp % 2 == 0 &&
        (grid_pp / 2) % per_cu == 0) {
      persistent = per_cu;
      p.causal_pairs = (int)(grid_pp / 2);
    }
    const dim3 gpp((unsigned)(persistent > 0 ? persistent : grid_pp)), bpp(64 * kWavesPP);
    if (D == 64) {
      if (causal) hipLaunchKernelGGL((attn_fwd_pp_kernel<64, 64, true>), gpp, bpp, 0, s, p);
      else hipLaunchKernelGGL((attn_fwd_pp_kernel<64, 64, false>), gpp, bpp, 0, s, p);
    } else {
      if (causal) hipLaunchKernelGGL((attn_fwd_pp_kernel<128, 64, true>), gpp, bpp, 0, s, p);
      else hipLaunchKernelGGL((attn_fwd_pp_kernel<128, 64, false>), gpp, bpp, 0, s, p);
    }
  } else {
    const dim3 grid_dim((unsigned)grid), block(64 * kWaves);
    if (D == 64) {
      if (causal) hipLaunchKernelGGL((attn_fwd_kernel<64, 64, kWaves, true>), grid_dim, block, 0, s, p);
      else hipLaunchKernelGGL((attn_fwd_kernel<64, 64, kWaves, false>), grid_dim, block, 0, s, p);
    } else {
      if (causal) hipLaunchKernelGGL((attn_fwd_kernel<128, 64, kWaves, true>), grid_dim, block, 0, s, p);
      else hipLaunchKernelGGL((attn_fwd_kernel<128, 64, kWaves, false>), grid_dim, block, 0, s, p);
    }
  }
  if (hipGetLastError() != hipSuccess) return ATTN_FWD_ELAUNCH;
  return ATTN_FWD_OK;
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int N, int D, int causal, float scale, void* stream) {
  return attn_fwd_ex(q, k, v, o, lse, B, H, N, D, causal, scale, ATTN_FWD_KERNEL_AUTO, stream);
}

}  // extern "C"
