// Based linear attention forward (causal) for gfx950 (AMD Instinct MI355X, CDNA4).
//
// What is computed: for every (batch, head) and token i, with d = 16 query/key features
// and dv = 64 value features,
//   s_ij = q_i . k_j / 4,   w_ij = 1 + s_ij + s_ij^2 / 2  (j <= i),
//   o_i  = sum_j w_ij v_j / sum_j w_ij.
// The pages ("ThunderKittens 2.0: Faster Kernels, Talking Models, and More Adorable
// Kittens", thebeat.tech, sections "New Kernels for Enhanced Performance" and "Performance
// Benchmarks") name Based linear attention without its formulas; this is the published
// Based design: the second-order Taylor feature map of exp(q.k / sqrt(d)),
//   phi(x) = [1, x / 2, vec(x x^T) / (4 sqrt 2)],   phi(q) . phi(k) = w,
// so that o_i = phi(q_i)^T S / phi(q_i)^T z with running sums S = sum phi(k_j) v_j^T
// (273 x 64) and z = sum phi(k_j).
//
// gfx950 design: one workgroup of 8 waves per (batch, head) walks the sequence in chunks
// of 64 tokens, with two wave roles so that every SIMD overlaps one wave of each. The
// state S lives in MFMA accumulators (fp32) of the 4 state waves: state wave u owns the 64
// quadratic features with first index a in [4u, 4u + 4) for all 64 value columns, plus the
// linear and constant features for value columns [16u, 16u + 16). For chunk c the 4
// output waves split the 64 tokens (16 each) and compute
//   * O_inter^T = S^T phi(Q_c)^T from a bf16 copy of S^T in LDS (written after chunk c-1;
//     its linear rows carry the 1/2 of the query's linear features as well, which the
//     query side then omits: both halves are powers of two, so the product is unchanged),
//   * O_intra^T = V_c^T W^T with W the causal Taylor weights inside the chunk,
//   * the normaliser: t0 + q . ksum / 4 + q^T KK q / 32 in fp32, with KK = sum k k^T and
//     ksum = sum k over earlier chunks (KK enters an MFMA as a bf16 hi + lo pair),
//     plus the row sums of W,
// while the state waves add phi(K_c)^T V_c to their part of S and publish the new bf16 S^T
// for the next chunk. The products are v_mfma_f32_16x16x32_bf16, except those whose depth
// is the 16 key features (in-chunk scores, KK q), which use v_mfma_f32_16x16x16_bf16.
// The quadratic features of K are formed in registers: each lane holds k[token][b] for 8
// tokens (transposing LDS reads) and multiplies by k[token][a] taken from lane a of its
// 16-lane row (a DPP row broadcast folded into the multiply).
// Chunk c+1's Q, K, V are copied global -> LDS (buffer_load ... lds) during chunk c;
// rows past N read as zeros, so they add nothing to S, KK and ksum.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "based_fwd.h"
#include "tile_lds.h"

namespace {

using namespace attn_tile;

constexpr int kD = 16;        // query/key features
constexpr int kDv = 64;       // value features
constexpr int kChunk = 64;    // tokens per chunk
constexpr int kWaves = 8;  // 4 output waves + 4 state waves
constexpr int kStRow = 296;   // bf16 per S^T row in LDS: 288 features + 8 (592-byte rows keep
                              // the 16-byte reads of 16 consecutive rows bank-conflict free)
constexpr float kC2 = 0.17677669529663688f;  // 1 / (4 sqrt 2), the quadratic feature scale

// LDS layout (bytes): two stages of {Q, K, V} chunk tiles, two S^T buffers, two
// {KK hi, KK lo} buffers, two ksum buffers.
constexpr int kQBytes = kChunk * kD * 2;
constexpr int kVBytes = kChunk * kDv * 2;
constexpr int kStage = 2 * kQBytes + kVBytes;
constexpr int kStBytes = kDv * kStRow * 2;
constexpr int kKKBytes = 2 * kD * kD * 2;
constexpr int kOffSt = 2 * kStage;
constexpr int kOffKK = kOffSt + 2 * kStBytes;
constexpr int kOffKs = kOffKK + 2 * kKKBytes;
constexpr int kLds = kOffKs + 2 * kD * 4;

struct BasedParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* ws;       // segment states (split launches), else unused
  int N;
  int n_chunks;
  int n_seg;       // segments per head (1: one workgroup per head)
  int seg_chunks;  // chunks per segment (the last segment may be shorter)
};

// Split launches: a head's chunks are cut into n_seg segments of seg_chunks. A state pass
// (based_state_kernel) writes, for every segment but the last, the fp32 sums of its
// chunks in two halves (group 0 took the even chunks, group 1 the odd ones) in the
// register layout of the state waves: for state wave u and lane l, slot j in [0, 80) at
// ((u * kWsSlots + j) * 64 + l): 0-63 the quadratic tiles, 64-67 the linear, 68-71 the
// constant features, 72-75 KK and 76 the lane's share of ksum (wave 0). The output pass
// starts each segment's state waves from the sum of the earlier segments' halves.
constexpr int kWsSlots = 80;
constexpr int kWsGroup = 4 * kWsSlots * 64;  // floats of one half-segment state

// V chunk tiles (128-byte rows) keep their 16-byte chunks permuted: logical chunk j of row r
// at j ^ swz_v(r). A transposing read covers, per 32 lanes, 8 consecutive rows and two
// adjacent chunks; with this permutation those 8 rows land on 8 distinct bank ranges.
__device__ inline int swz_v(int r) { return ((r >> 1) & 3) << 1; }

__device__ inline bf16x8 pack8(const float (&x)[8]) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)x[j];
  return r;
}

// DPP row_newbcast:n: every lane of a 16-lane row receives x from lane n of that row.
template <int n>
__device__ inline uint32_t row_bcast(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x150 + n, 0xf, 0xf, false);
}
template <int W>
__device__ inline uint32_t row_bcast_feature(uint32_t x, int rb) {
  switch (rb) {  // rb is a compile-time constant after unrolling
    case 0: return row_bcast<4 * W + 0>(x);
    case 1: return row_bcast<4 * W + 1>(x);
    case 2: return row_bcast<4 * W + 2>(x);
    default: return row_bcast<4 * W + 3>(x);
  }
}

__device__ inline float sum_across_16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// v_mfma_f32_16x16x16_bf16: the products whose depth is the 16 key features. Lane l holds
// A row l % 16 and B column l % 16 at depth 4 (l / 16) .. + 3; C as in the 32-deep form.
__device__ inline f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                   0, 0, 0);
}

// Transposing read of a 4-row x 16-column bf16 block: in every 16-lane row, lane c supplies
// the address of row (c >> 2), columns 4 (c & 3) .. + 3 and receives column c of the 4 rows.
__device__ inline bf16x4 tr4(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
}

// One wave's share of copying chunk `chunk` (rows past N read zeros: their offsets are
// placed outside the buffer range on purpose). Copies 0-1: Q, 2-3: K (32 rows of 32 bytes
// each), 4-11: V (8 rows of 128 bytes each, chunk-permuted). Output wave w issues copy w
// (Q or K); state wave u issues copies 4 + 2u and 5 + 2u (V).
__device__ inline void copy_one(const i32x4& qr, const i32x4& kr, const i32x4& vr, int i, int t0, int N,
                                uint32_t stage_lds, int lane) {
  if (i < 4) {
    const int row = 32 * (i & 1) + (lane >> 1);
    const uint32_t voff = (t0 + row < N) ? (uint32_t)((t0 + row) * 32 + 16 * (lane & 1)) : 0x80000000u;
    const uint32_t dst = stage_lds + (i < 2 ? 0 : kQBytes) + 1024 * (i & 1);
    copy16_to_lds(i < 2 ? qr : kr, voff, 0, __builtin_amdgcn_readfirstlane(dst));
  } else {
    const int row = 8 * (i - 4) + (lane >> 3);
    const int logical = (lane & 7) ^ swz_v(row);
    const uint32_t voff = (t0 + row < N) ? (uint32_t)((t0 + row) * 128 + 16 * logical) : 0x80000000u;
    const uint32_t dst = stage_lds + 2 * kQBytes + 1024 * (i - 4);
    copy16_to_lds(vr, voff, 0, __builtin_amdgcn_readfirstlane(dst));
  }
}

struct HeadRefs {
  i32x4 qr, kr, vr;
  __bf16* ob;
  uint32_t smem_lds;
};

__device__ inline HeadRefs head_refs(const BasedParams& p, char* smem, size_t bh) {
  const int N = p.N;
  HeadRefs h;
  h.qr = make_rsrc(p.q + bh * N * kD, (uint32_t)N * kD * 2);
  h.kr = make_rsrc(p.k + bh * N * kD, (uint32_t)N * kD * 2);
  h.vr = make_rsrc(p.v + bh * N * kDv, (uint32_t)N * kDv * 2);
  h.ob = p.o + bh * N * kDv;
  h.smem_lds = lds_address(smem);
  return h;
}

// V^T fragment of the chunk in stage Vs for key step m and value columns 16 cb ..: tokens
// 32 m + 4 g + j (j < 4) and 32 m + 16 + 4 g + j - 4, value column 16 cb + c.
__device__ inline bf16x8 v_frag(const char* Vs, int m, int cb, int g, int c) {
  const int r = 32 * m + 4 * g + (c >> 2);
  const int chunk = (2 * cb + ((c & 3) >> 1)) ^ swz_v(r);
  const char* a0 = Vs + r * 128 + 16 * chunk + 8 * (c & 1);
  return __builtin_shufflevector(tr4(a0), tr4(a0 + 16 * 128), 0, 1, 2, 3, 4, 5, 6, 7);
}

// Output wave W (0..3): the 16 query tokens 16W .. 16W + 15 of every chunk. Reads the bf16
// S^T, KK and ksum published after the previous chunk; computes O_inter, O_intra, the
// normaliser and stores o.
template <int W>
__device__ inline void output_wave(const BasedParams& p, char* smem, int lane, size_t bh, int t_begin,
                                   int t_end) {
  const int g = lane >> 4;  // 16-lane row
  const int c = lane & 15;  // lane within the row
  const int N = p.N;
  const HeadRefs hr = head_refs(p, smem, bh);
  copy_one(hr.qr, hr.kr, hr.vr, W, t_begin * kChunk, N, hr.smem_lds, lane);
  wait_copies_and_barrier();
  for (int t = t_begin; t < t_end; ++t) {
    const int cur = (t - t_begin) & 1;
    if (t + 1 < t_end) copy_one(hr.qr, hr.kr, hr.vr, W, (t + 1) * kChunk, N, hr.smem_lds + (cur ^ 1) * kStage, lane);
    const char* Qs = smem + cur * kStage;
    const char* Ks = Qs + kQBytes;
    const char* Vs = Ks + kQBytes;
    const char* St = smem + kOffSt + cur * kStBytes;
    const char* KKs = smem + kOffKK + cur * kKKBytes;
    const float* kss = reinterpret_cast<const float*>(smem + kOffKs) + cur * kD;

    // ---- this lane's query token (16W + c) and its features
    const int tq = 16 * W + c;
    // feature f = 32 ks + 8 g + j = 16 a + b: a = 2 ks + (g >> 1), b = 8 (g & 1) + j. qb holds
    // q[tq][8 (g & 1) + j] (one lane-addressed read); qa[m] = q[tq][2 m + (g >> 1)] is the
    // low or high bf16 of the m-th dword of the row, taken with a per-lane shift (a select
    // here would be turned into per-lane register indexing).
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 qrow = *reinterpret_cast<const u32x4*>(Qs + tq * 32);
    const u32x4 qrow1 = *reinterpret_cast<const u32x4*>(Qs + tq * 32 + 16);
    const bf16x8 qbv = *reinterpret_cast<const bf16x8*>(Qs + tq * 32 + 16 * (g & 1));
    const uint32_t sh = (g >> 1) ? 0u : 16u;
    float qa[8], qb[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      qa[m] = __uint_as_float((qrow[m] << sh) & 0xFFFF0000u);
      qa[4 + m] = __uint_as_float((qrow1[m] << sh) & 0xFFFF0000u);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) qb[j] = (float)qbv[j];
    // q[tq][4g .. 4g + 3]: the B operand of the 16-deep products over the 16 features
    const bf16x4 q4 = *reinterpret_cast<const bf16x4*>(Qs + tq * 32 + 8 * g);

    // ---- O_inter^T = S^T phi(Q)^T over the 288 (padded) features, 9 steps of 32
    f32x4 o[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) o[cb] = f32x4{};
#pragma unroll
    for (int ks = 0; ks < 9; ++ks) {
      float f[8];
      if (ks < 8) {
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = qa[ks] * (qb[j] * kC2);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = g < 2 ? qb[j] : ((g == 2 && j == 0) ? 1.f : 0.f);
      }
      const bf16x8 bfeat = pack8(f);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(St + (16 * cb + c) * (kStRow * 2) + 2 * (32 * ks + 8 * g));
        o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bfeat, o[cb], 0, 0, 0);
      }
    }

    // ---- intra-chunk: W^T for keys 16 kb + 4 g + i (kb <= W) against token tq
    float zpart = 0.f;
    float wv[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      if (kb <= W) {
        const bf16x4 ak = *reinterpret_cast<const bf16x4*>(Ks + (16 * kb + c) * 32 + 8 * g);
        const f32x4 s = mfma16(ak, q4, f32x4{});
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = 0.25f * s[i];
          const float wt = 1.f + x + 0.5f * x * x;
          wv[kb][i] = (kb < W || 4 * g + i <= c) ? wt : 0.f;
          zpart += wv[kb][i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[kb][i] = 0.f;
      }
    }
#pragma unroll
    for (int m = 0; m <= (W >> 1); ++m) {
      bf16x8 bw;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bw[i] = (__bf16)wv[2 * m][i];
        bw[4 + i] = (__bf16)wv[2 * m + 1][i];
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v_frag(Vs, m, cb, g, c), bw, o[cb], 0, 0, 0);
    }

    // ---- normaliser: t0 + q . ksum / 4 + q^T KK q / 32 (earlier chunks) + row sum of W
    {
      const bf16x4 khi = *reinterpret_cast<const bf16x4*>(KKs + c * 32 + 8 * g);
      const bf16x4 klo = *reinterpret_cast<const bf16x4*>(KKs + 512 + c * 32 + 8 * g);
      f32x4 u = mfma16(khi, q4, f32x4{});
      u = mfma16(klo, q4, u);  // u[i] = (KK q)[4g + i]
      const f32x4 ks4 = *reinterpret_cast<const f32x4*>(kss + 4 * g);
      float zq = 0.f, zl = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        zq += (float)q4[i] * u[i];
        zl += (float)q4[i] * ks4[i];
      }
      zpart += zq * (1.f / 32.f) + zl * 0.25f;
    }
    const float z = (float)(t * kChunk) + sum_across_halves(sum_across_16(zpart));

    // ---- output rows: lane holds o^T[16 cb + 4 g + i][tq]
    const int token = t * kChunk + tq;
    if (token < N) {
      const float inv = 1.f / z;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        bf16x4 wo;
#pragma unroll
        for (int i = 0; i < 4; ++i) wo[i] = (__bf16)(o[cb][i] * inv);
        *reinterpret_cast<bf16x4*>(hr.ob + (size_t)token * kDv + 16 * cb + 4 * g) = wo;
      }
    }
    wait_copies_and_barrier();
  }
}

// The running state of state wave U (0..3): the quadratic features with a in [4U, 4U + 4)
// for all value columns, the linear and constant features of value columns 16U .. 16U + 15,
// and (wave 0) KK and this lane's share of ksum.
struct StateRegs {
  f32x4 sq[4][4];  // quadratic features (a = 4U + rb, b = 4g + i) x value columns 16cb + c
  f32x4 slin;      // sum of k[b] v, b = 4g + i, x value columns 16U + c (unscaled; S^T
                   // gets a quarter: the 1/2 of the key and of the query feature)
  f32x4 sconst;    // row 0: sum of v over value columns 16U + c; rows 1-15 stay zero
  f32x4 kk;        // wave 0: KK[a = 4g + i][b = c]
  float ksum_part; // wave 0: sum of k[token][c] over this lane's tokens
};

__device__ inline void state_zero(StateRegs& st) {
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) st.sq[rb][cb] = f32x4{};
  st.slin = f32x4{};
  st.sconst = f32x4{};
  st.kk = f32x4{};
  st.ksum_part = 0.f;
}

// S += phi(K)^T V, KK += K^T K, ksum += sum k for the chunk whose K and V tiles are at Ks, Vs
// (rows past N are zeros and add nothing).
template <int U>
__device__ inline void state_update(StateRegs& st, const char* Ks, const char* Vs, int g, int c) {
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const char* k0 = Ks + (32 * m + 4 * g + (c >> 2)) * 32 + 8 * (c & 3);
    const bf16x8 kc = __builtin_shufflevector(tr4(k0), tr4(k0 + 16 * 32), 0, 1, 2, 3, 4, 5, 6, 7);
    float kf[8], kfs[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      kf[j] = (float)kc[j];  // k[token_j][c]
      kfs[j] = kf[j] * kC2;
    }
    bf16x8 vfm[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) vfm[cb] = v_frag(Vs, m, cb, g, c);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      float f[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)  // k[token_j][4U + rb] from lane 4U + rb of this row
        f[j] = __uint_as_float(row_bcast_feature<U>(__float_as_uint(kf[j]), rb)) * kfs[j];
      const bf16x8 afeat = pack8(f);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        st.sq[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afeat, vfm[cb], st.sq[rb][cb], 0, 0, 0);
    }
    // linear features: the sums of k v, unscaled (their 1/2, and the query side's 1/2,
    // are applied once when the state is published)
    st.slin = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc, vfm[U], st.slin, 0, 0, 0);
    bf16x8 ones;
#pragma unroll
    for (int j = 0; j < 8; ++j) ones[j] = (__bf16)(c == 0 ? 1.f : 0.f);
    st.sconst = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, vfm[U], st.sconst, 0, 0, 0);
    if (U == 0) {
      st.kk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc, kc, st.kk, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 8; ++j) st.ksum_part += kf[j];
    }
  }
}

// Publish the bf16 S^T (and, wave 0, KK as a hi + lo pair and ksum) into buffer `buf`.
template <int U>
__device__ inline void state_publish(const StateRegs& st, char* smem, int buf, int g, int c) {
  char* Stn = smem + kOffSt + buf * kStBytes;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      bf16x4 x;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = (__bf16)st.sq[rb][cb][i];
      *reinterpret_cast<bf16x4*>(Stn + (16 * cb + c) * (kStRow * 2) + 2 * (16 * (4 * U + rb) + 4 * g)) = x;
    }
  {
    bf16x4 xl, xc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xl[i] = (__bf16)(0.25f * st.slin[i]);  // (k / 2) . (q / 2): both halves, exact
      xc[i] = (__bf16)st.sconst[i];
    }
    *reinterpret_cast<bf16x4*>(Stn + (16 * U + c) * (kStRow * 2) + 2 * (256 + 4 * g)) = xl;
    *reinterpret_cast<bf16x4*>(Stn + (16 * U + c) * (kStRow * 2) + 2 * (272 + 4 * g)) = xc;
  }
  if (U == 0) {
    __bf16* KKn = reinterpret_cast<__bf16*>(smem + kOffKK + buf * kKKBytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const __bf16 hi = (__bf16)st.kk[i];
      KKn[(4 * g + i) * kD + c] = hi;
      KKn[256 + (4 * g + i) * kD + c] = (__bf16)(st.kk[i] - (float)hi);
    }
    const float ks = sum_across_halves(sum_across_16(st.ksum_part));
    if (g == 0) reinterpret_cast<float*>(smem + kOffKs)[buf * kD + c] = ks;
  }
}

// Segment-state slots of state wave U: read (add) or write this lane's registers.
template <int U>
__device__ inline void state_add_from(StateRegs& st, const float* w, int lane) {
  const float* b = w + (size_t)U * kWsSlots * 64 + lane;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) st.sq[rb][cb][i] += b[(16 * rb + 4 * cb + i) * 64];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    st.slin[i] += b[(64 + i) * 64];
    st.sconst[i] += b[(68 + i) * 64];
  }
  if (U == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) st.kk[i] += b[(72 + i) * 64];
    st.ksum_part += b[76 * 64];
  }
}
template <int U>
__device__ inline void state_store_to(const StateRegs& st, float* w, int lane) {
  float* b = w + (size_t)U * kWsSlots * 64 + lane;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) b[(16 * rb + 4 * cb + i) * 64] = st.sq[rb][cb][i];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    b[(64 + i) * 64] = st.slin[i];
    b[(68 + i) * 64] = st.sconst[i];
    b[(72 + i) * 64] = U == 0 ? st.kk[i] : 0.f;
  }
  b[76 * 64] = U == 0 ? st.ksum_part : 0.f;
}

// State wave U (0..3) of the output pass: starts from the state of the segments before
// `seg` (zero for the first) and adds each chunk's contribution, publishing the bf16 S^T
// (and KK, ksum) in the other buffer for the next chunk's output waves.
template <int U>
__device__ inline void state_wave(const BasedParams& p, char* smem, int lane, size_t bh, int seg,
                                  int t_begin, int t_end) {
  const int g = lane >> 4;
  const int c = lane & 15;
  const int N = p.N;
  const HeadRefs hr = head_refs(p, smem, bh);
  copy_one(hr.qr, hr.kr, hr.vr, 4 + 2 * U, t_begin * kChunk, N, hr.smem_lds, lane);
  copy_one(hr.qr, hr.kr, hr.vr, 5 + 2 * U, t_begin * kChunk, N, hr.smem_lds, lane);

  StateRegs st;
  state_zero(st);
  if (seg > 0) {
    const float* w = p.ws + bh * (size_t)(p.n_seg - 1) * 2 * kWsGroup;
    for (int h = 0; h < 2 * seg; ++h) state_add_from<U>(st, w + (size_t)h * kWsGroup, lane);
    state_publish<U>(st, smem, 0, g, c);  // buffer 0, read by the first chunk
  }

  wait_copies_and_barrier();
  for (int t = t_begin; t < t_end; ++t) {
    const int cur = (t - t_begin) & 1;
    if (t + 1 < t_end) {
      const uint32_t stage = hr.smem_lds + (cur ^ 1) * kStage;
      copy_one(hr.qr, hr.kr, hr.vr, 4 + 2 * U, (t + 1) * kChunk, N, stage, lane);
      copy_one(hr.qr, hr.kr, hr.vr, 5 + 2 * U, (t + 1) * kChunk, N, stage, lane);
    }
    const char* Ks = smem + cur * kStage + kQBytes;
    const char* Vs = Ks + kQBytes;
    state_update<U>(st, Ks, Vs, g, c);
    state_publish<U>(st, smem, cur ^ 1, g, c);  // the state after this chunk, for the next one
    wait_copies_and_barrier();
  }
}

// 8 waves: output waves 0-3 and state waves 4-7 (waves w and w + 4 share a SIMD, so every
// SIMD runs one wave of each role); one workgroup per (batch, head, segment). Both roles
// run the segment's chunks with one barrier each, after a common start: S^T buffer 0, KK
// buffer 0 and ksum buffer 0 are zeroed by all waves, and after a barrier the state waves
// of a later segment overwrite them with the state of the segments before it.
__global__ __launch_bounds__(512) void based_fwd_kernel(const BasedParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[kLds];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const size_t bh = blockIdx.x / p.n_seg;
  const int seg = (int)(blockIdx.x - bh * p.n_seg);
  const int t_begin = seg * p.seg_chunks;
  const int t_end = min(p.n_chunks, t_begin + p.seg_chunks);
  for (int i = tid; i < kStBytes / 4; i += 64 * kWaves) reinterpret_cast<uint32_t*>(smem + kOffSt)[i] = 0u;
  for (int i = tid; i < kKKBytes / 4; i += 64 * kWaves) reinterpret_cast<uint32_t*>(smem + kOffKK)[i] = 0u;
  if (tid < kD) reinterpret_cast<float*>(smem + kOffKs)[tid] = 0.f;
  __syncthreads();
  switch (__builtin_amdgcn_readfirstlane(tid >> 6)) {
    case 0: output_wave<0>(p, smem, lane, bh, t_begin, t_end); break;
    case 1: output_wave<1>(p, smem, lane, bh, t_begin, t_end); break;
    case 2: output_wave<2>(p, smem, lane, bh, t_begin, t_end); break;
    case 3: output_wave<3>(p, smem, lane, bh, t_begin, t_end); break;
    case 4: state_wave<0>(p, smem, lane, bh, seg, t_begin, t_end); break;
    case 5: state_wave<1>(p, smem, lane, bh, seg, t_begin, t_end); break;
    case 6: state_wave<2>(p, smem, lane, bh, seg, t_begin, t_end); break;
    default: state_wave<3>(p, smem, lane, bh, seg, t_begin, t_end); break;
  }
}

// State pass of a split launch: one workgroup per (batch, head, segment but the last),
// 8 waves in two groups of 4 state waves; group G takes the segment's chunks t_begin + 2i
// + G, each from its own two LDS stages, and writes its sums to the workspace.
template <int U>
__device__ inline void state_pass_wave(const BasedParams& p, char* smem, int lane, int G, size_t bh,
                                       int seg) {
  const int g = lane >> 4;
  const int c = lane & 15;
  const int N = p.N;
  const HeadRefs hr = head_refs(p, smem, bh);
  const int t_begin = seg * p.seg_chunks;
  const int n_pairs = (p.seg_chunks + 1) / 2;
  auto load = [&](int i) {  // chunk t_begin + 2i + G into stage (2G + i % 2)
    const int t = t_begin + 2 * i + G;
    if (t >= t_begin + p.seg_chunks) return;
    const uint32_t stage = hr.smem_lds + (2 * G + (i & 1)) * kStage;
    if (U < 2) copy_one(hr.qr, hr.kr, hr.vr, 2 + U, t * kChunk, N, stage, lane);
    copy_one(hr.qr, hr.kr, hr.vr, 4 + 2 * U, t * kChunk, N, stage, lane);
    copy_one(hr.qr, hr.kr, hr.vr, 5 + 2 * U, t * kChunk, N, stage, lane);
  };
  StateRegs st;
  state_zero(st);
  load(0);
  for (int i = 0; i < n_pairs; ++i) {
    wait_copies_and_barrier();
    if (i + 1 < n_pairs) load(i + 1);
    // (the stage read here is refilled only after the next iteration's barrier)
    if (t_begin + 2 * i + G < t_begin + p.seg_chunks) {
      const char* Ks = smem + (2 * G + (i & 1)) * kStage + kQBytes;
      state_update<U>(st, Ks, Ks + kQBytes, g, c);
    }
  }
  float* w = p.ws + (bh * (size_t)(p.n_seg - 1) + seg) * 2 * kWsGroup + (size_t)G * kWsGroup;
  state_store_to<U>(st, w, lane);
}

__global__ __launch_bounds__(512) void based_state_kernel(const BasedParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[4 * kStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t bh = blockIdx.x / (p.n_seg - 1);
  const int seg = (int)(blockIdx.x - bh * (p.n_seg - 1));
  switch (wave & 3) {
    case 0: state_pass_wave<0>(p, smem, lane, wave >> 2, bh, seg); break;
    case 1: state_pass_wave<1>(p, smem, lane, wave >> 2, bh, seg); break;
    case 2: state_pass_wave<2>(p, smem, lane, wave >> 2, bh, seg); break;
    default: state_pass_wave<3>(p, smem, lane, wave >> 2, bh, seg); break;
  }
}

// Segments per head for a split launch: enough workgroups to cover the device's compute
// units (queried once per device), but segments of at least kMinSegChunks chunks.
constexpr int kMinSegChunks = 8;
std::atomic<int> g_cus[64];
int split_plan(int B, int H, int N, int* n_seg, int* seg_chunks) {
  const int n_chunks = (N + kChunk - 1) / kChunk;
  *n_seg = 1;
  *seg_chunks = n_chunks;
  if (B < 1 || H < 1 || N < 1) return BASED_EINVAL;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return BASED_ELAUNCH;
  int cus = g_cus[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      return BASED_ELAUNCH;
    g_cus[dev].store(cus, std::memory_order_relaxed);
  }
  const int64_t heads = (int64_t)B * H;
  if (heads >= cus) return BASED_OK;
  const int want = (int)((cus + heads - 1) / heads);
  const int cap = n_chunks / kMinSegChunks;
  const int n = want < cap ? want : cap;
  if (n < 2) return BASED_OK;
  *seg_chunks = (n_chunks + n - 1) / n;
  *n_seg = (n_chunks + *seg_chunks - 1) / *seg_chunks;
  return BASED_OK;
}

}  // namespace

extern "C" {

int based_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d,
              int dv, void* stream) {
  return based_fwd_ws(q, k, v, o, nullptr, 0, B, H, N, d, dv, stream);
}

size_t based_fwd_workspace_bytes(int B, int H, int N) {
  int n_seg = 0, seg_chunks = 0;
  if (split_plan(B, H, N, &n_seg, &seg_chunks) != BASED_OK || n_seg < 2) return 0;
  return (size_t)B * H * (n_seg - 1) * 2 * kWsGroup * sizeof(float);
}

int based_fwd_ws(const void* q, const void* k, const void* v, void* o, void* workspace,
                 size_t workspace_bytes, int B, int H, int N, int d, int dv, void* stream) {
  if (!q || !k || !v || !o) return BASED_EINVAL;
  if (B < 1 || H < 1 || N < 1) return BASED_EINVAL;
  if (d != kD || dv != kDv) return BASED_EUNSUPPORTED;
  if ((int64_t)N * kDv * 2 >= ((int64_t)1 << 31) || (int64_t)B * H >= ((int64_t)1 << 24)) return BASED_EINVAL;
  if ((((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) != 0) return BASED_EALIGN;
  if (workspace && ((uintptr_t)workspace & 255u) != 0) return BASED_EALIGN;
  BasedParams p;
  p.q = static_cast<const __bf16*>(q);
  p.k = static_cast<const __bf16*>(k);
  p.v = static_cast<const __bf16*>(v);
  p.o = static_cast<__bf16*>(o);
  p.ws = nullptr;
  p.N = N;
  p.n_chunks = (N + kChunk - 1) / kChunk;
  p.n_seg = 1;
  p.seg_chunks = p.n_chunks;
  if (workspace) {
    int n_seg = 1, seg_chunks = p.n_chunks;
    const int rc = split_plan(B, H, N, &n_seg, &seg_chunks);
    if (rc != BASED_OK) return rc;
    if (n_seg > 1 && workspace_bytes >= (size_t)B * H * (n_seg - 1) * 2 * kWsGroup * sizeof(float)) {
      p.ws = static_cast<float*>(workspace);
      p.n_seg = n_seg;
      p.seg_chunks = seg_chunks;
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.n_seg > 1)
    hipLaunchKernelGGL(based_state_kernel, dim3((unsigned)((size_t)B * H * (p.n_seg - 1))), dim3(64 * kWaves),
                       0, s, p);
  hipLaunchKernelGGL(based_fwd_kernel, dim3((unsigned)((size_t)B * H * p.n_seg)), dim3(64 * kWaves), 0, s, p);
  if (hipGetLastError() != hipSuccess) return BASED_ELAUNCH;
  return BASED_OK;
}

const char* based_fwd_strerror(int code) {
  switch (code) {
    case BASED_OK: return "success";
    case BASED_EINVAL: return "invalid argument (NULL pointer, size < 1, or size overflow)";
    case BASED_EUNSUPPORTED: return "unsupported feature sizes (d must be 16 and dv 64)";
    case BASED_EALIGN: return "misaligned pointer (q, k, v, o need 16 bytes)";
    case BASED_ELAUNCH: return "kernel launch failed";
    default: return "unknown error code";
  }
}

}  // extern "C"
