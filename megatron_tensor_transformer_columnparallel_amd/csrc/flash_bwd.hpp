// Flash-style attention backward for one tensor-parallel shard (head dims
// 64, 128, 256).
//
// The per-head backward of softmax attention O = softmax(Q K^T / sqrt(d)) V
// (page "Megtron张量/模型并行", section Self-Attention层: each head on its own
// shard) needs, per query i and key j,
//   P_ij  = exp(S_ij - lse_i)                     recomputed from the saved lse
//   dP_ij = dO_i . V_j
//   dS_ij = P_ij (dP_ij - Delta_i) / sqrt(d)      Delta_i = sum_j P_ij dP_ij / sum_j P_ij
// and dQ = dS K, dK = dS^T Q, dV = P^T dO.  The kernels round P (dP - Delta)
// to bf16 for the products and apply the 1 / sqrt(d) to dQ and dK once, in
// fp32, where they are written.  Delta is taken from the same
// fp32 P and dP that form dS, so every row of dS sums to zero: a rounding of
// O or dO cannot leak into dQ through the keys' common component.
//
// Three phases, none of which stores a score, a probability or a dS:
//
//   attn_bwd_q_kernel<D, 0>  (Delta partials) per work item (a block of 128
//       queries and a chunk of its keys): S and dP, then the row sums of
//       P dP and of P over the chunk.
//   attn_bwd_q_kernel<D, 1>  (dQ) per work item: Delta of each row from its
//       block's partials, then over the chunk's keys S, dP, dS and dQ += dS K
//       (dS rounded to bf16 as the A operand straight from the accumulators,
//       K read with the transposing LDS read at the same key rows).
//   attn_bwd_kv_kernel<D>    (dK, dV) per work item (a block of keys and a
//       chunk of the queries at or after them): S^T = K Q^T, P^T from the
//       queries' lse, dV += P^T dO, dP^T = V dO^T, dS^T from Delta,
//       dK += dS^T Q.
//
// In each, a wave keeps its rows' fragments (Q and dO, or K and V) and its
// accumulators in registers and walks the other operand 32 rows at a time,
// its tiles brought into LDS by direct DMA in two stages.  The chunk length
// is chosen so that about one round of items fills the CUs; the chunks of a
// split block write fp32 partials that attn_bwd_merge_kernel adds in chunk
// order (results do not depend on timing).
//
// Every tile is read both row-wise (ds_read_b128, 16-byte chunks of 16
// consecutive rows per 16-lane group) and transposed (ds_read_b64_tr_b16,
// 32 bytes of 4 consecutive rows per 16-lane group, two groups per phase).
// Chunk c of tile row r sits at slot c ^ swz(r).  Rows of 16 or more
// chunks: swz = 4 ((r/4 + r) mod 4) + 2 ((r/4) mod 2), even, so chunk pairs
// stay pairs for the transposed read, and over the 16 rows of a row read
// the slots of one chunk fall 4 apart within each group of 4 rows; rows of
// 8 chunks: swz = r mod 8.  A pattern probe timed both reads of these
// layouts at the conflict-free rate, where swz = 2 (r mod 8) + (r/8 mod 2)
// ran its row reads 1.7x slower.
#pragma once

#include <type_traits>

#include "flash_attn.hpp"

namespace tps {
namespace flash {

constexpr int kBT = 32;    // keys (dq kernel) or queries (dkv kernel) per iteration

// RB 16-row blocks per wave (rows: queries of the dq kernel, keys of the
// dkv kernel) and WAVES waves per workgroup, which owns BB = WAVES 16 RB
// rows.  Four waves of 32 rows (one wave per SIMD, up to 512 registers)
// up to head dim 128.  At 256 a wave's 32 rows of two fragment sets and one
// or two accumulators do not fit: waves of 16 rows, eight of them (128
// queries, two waves per SIMD) in the dq kernel, four (64 keys, one per SIMD)
// in the dkv kernel, whose two accumulators need more than 256 registers.
template <int D, bool DKV>
struct BwdShape {
  static constexpr int RB = D >= 256 ? 1 : 2;
  static constexpr int WAVES = (D >= 256 && !DKV) ? 8 : 4;
  static constexpr int BB = WAVES * 16 * RB;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int KS = D / 32;                       // 32-wide k-steps over the head dim
  static constexpr int NB = D / 16;                       // 16-column blocks of an accumulator
  static constexpr int CPR = D / 8;                       // 16-byte chunks per tile row
  static constexpr int TILE = kBT * D;                    // bf16 elements of one tile
  static constexpr int DPW = kBT * CPR / 64 / WAVES;      // 1 KB DMA instructions per wave per tile
  static constexpr bool AGPR_ACC = DKV && D >= 128;
  static __host__ __device__ constexpr int swz(int r) {
    return CPR >= 16 ? (((((r >> 2) + (r & 3)) & 3) << 2) | (((r >> 2) & 1) << 1)) : (r & 7);
  }
  // element offset of logical chunk c of tile row r
  static __device__ __forceinline__ int off(int r, int c) { return r * D + ((c ^ swz(r)) * 8); }
  static_assert(D == 64 || D == 128 || D == 256, "head dim");
  static_assert(DPW >= 1 && DPW * THREADS == kBT * CPR, "DMA split");
};

struct BwdPlan {
  int sq = 0, hs = 0, nz = 0, causal = 0;
  int64_t ld = 0;    // QKV / dQKV row stride (3 hs d)
  int64_t ldo = 0;   // dO row stride (hs d)
  float scale = 0.f;        // 1 / sqrt(d)
  float scale_log2 = 0.f;   // log2(e) / sqrt(d)
  float neg_sqrt_d = 0.f;   // -sqrt(d)
};

inline BwdPlan make_bwd_plan(int64_t b, int64_t sq, int64_t hs, int d, int causal) {
  BwdPlan p;
  p.sq = (int)sq;
  p.hs = (int)hs;
  p.nz = (int)(b * hs);
  p.causal = causal;
  p.ld = 3 * hs * d;
  p.ldo = hs * d;
  p.scale = 1.f / sqrtf((float)d);
  p.scale_log2 = 1.4426950408889634f / sqrtf((float)d);
  p.neg_sqrt_d = -sqrtf((float)d);
  return p;
}

// DMA of one 32-row tile (rows r0 .. r0+31 of a [rows x ld] operand, head
// columns at `head`) into LDS at byte offset `off` from lds0: instruction i
// of this wave fills slots (wave DPW + i) 64 .. +63; slot q is row q / CPR,
// position q % CPR, which holds the row's logical chunk position ^ swz.
// Rows past `rmax` re-read row rmax (their results are masked or dropped).
// DMA of the fp32 values of queries r0 .. r0+31 (lanes 32..63 repeat them)
// into 256 bytes of LDS at byte address m0: lane l's dword lands at m0 + 4 l.
// Queries past `rmax` re-read rmax.
__device__ __forceinline__ void bwd_dma_rowvals(const float* v, int r0, int rmax, uint32_t m0, int lane) {
  const uint64_t sb = uniform_addr(v);
  const uint32_t voff = (uint32_t)min(r0 + (lane & 31), rmax) * 4u;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(voff), "s"(sb), "s"(m0) : "memory", "m0");
}

template <class S>
__device__ __forceinline__ void bwd_dma_tile(const bf16_t* head, int64_t ld, int r0, int rmax, uint32_t lds0,
                                             uint32_t off, int wave, int lane) {
  const uint64_t sb = uniform_addr(head + (int64_t)r0 * ld);
#pragma unroll
  for (int i = 0; i < S::DPW; ++i) {
    const int ins = wave * S::DPW + i;
    const int q = ins * 64 + lane;
    const int r = q / S::CPR, ph = q % S::CPR;
    const int c = ph ^ S::swz(r);
    const uint32_t voff = (uint32_t)((int64_t)min(r, rmax - r0) * ld * 2 + c * 16);
    const uint32_t m0 = lds0 + off + (uint32_t)(ins * 64 * 16);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(sb), "s"(m0) : "memory", "m0");
  }
}

// Row read: the 16x32 fragment of tile rows 16 h .. +15, k-step ks (lane:
// row 16 h + r16, elements 32 ks + 8 g .. +7).
template <class S>
__device__ __forceinline__ bf16x8_t bwd_row_frag(const bf16_t* tile, int ks, int h, int r16, int g) {
  return *reinterpret_cast<const bf16x8_t*>(tile + S::off(16 * h + r16, 4 * ks + g));
}

// Transposed read: the B operand of an MFMA whose k runs over the tile's
// rows in the order of a packed score fragment (k slots 8 g .. 8 g + 7 =
// rows 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3) and whose n is the head
// column block nb (columns 16 nb .. +15).
template <class S>
__device__ __forceinline__ bf16x8_t bwd_tr_frag(const bf16_t* tile, int nb, int r16, int g) {
  constexpr int D = S::CPR * 8;
  const int row = 4 * g + (r16 >> 2);
  const int c = 2 * nb + ((r16 & 3) >> 1);
  const bf16_t* pl = tile + S::off(row, c) + (r16 & 1) * 4;
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)pl);
  const s16x4_t hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(pl + 16 * D));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ bf16x8_t pack_frag(const float v[8]) {
  return __builtin_bit_cast(bf16x8_t, u32x4_t{cvt_bf16x2(v[0], v[1]), cvt_bf16x2(v[2], v[3]),
                                              cvt_bf16x2(v[4], v[5]), cvt_bf16x2(v[6], v[7])});
}

// ---------------------------------------------------------------- work items
// A phase's work: blocks of bb rows (queries in the Delta and dQ phases, keys
// in the dK/dV phase), each walking its range of 32-row tiles of the other
// operand (keys up to the block's causal limit; queries from the block's
// first key on) in one or more chunks of at most `chunk` tiles.  The chunk
// length is chosen on the host so that about one round of items fills the
// CUs whatever the sequence length; a split block's chunks write fp32
// partials that a merge kernel adds up in chunk order.
struct BwdWork {
  int sq = 0, nz = 0, bb = 0, nb = 0, causal = 0, kv = 0;
  int chunk = 1, items_per_z = 0;
};

// Block of item slot s: slots run over the blocks in the order that puts the
// longest ones last (items are launched last slot first).
__host__ __device__ inline int work_block(const BwdWork& w, int s) { return (w.kv && w.causal) ? w.nb - 1 - s : s; }
__host__ __device__ inline int work_first_tile(const BwdWork& w, int i) {
  return (w.kv && w.causal) ? i * w.bb / kBT : 0;
}
__host__ __device__ inline int work_tiles(const BwdWork& w, int i) {
  if (w.kv) return (w.sq - work_first_tile(w, i) * kBT + kBT - 1) / kBT;
  const int end = w.causal ? min(w.sq, (i + 1) * w.bb) : w.sq;
  return (end + kBT - 1) / kBT;
}
__host__ __device__ inline int work_chunks(const BwdWork& w, int i) { return (work_tiles(w, i) + w.chunk - 1) / w.chunk; }

// item -> (z, block i, chunk c of C, absolute tiles [it0, it1), first item of the block)
__device__ inline Item work_item(const BwdWork& w, int item) {
  Item t;
  t.z = item / w.items_per_z;
  const int r = item - t.z * w.items_per_z;
  const Located l = wave_locate(w.nb, r, [&](int s) { return int2{work_chunks(w, work_block(w, s)), 0}; });
  const int base = __builtin_amdgcn_readfirstlane(l.a);
  t.i = work_block(w, __builtin_amdgcn_readfirstlane(l.s));
  t.c = r - base;
  t.C = work_chunks(w, t.i);
  const int n = work_tiles(w, t.i), f = work_first_tile(w, t.i);
  t.it0 = f + (int)((int64_t)t.c * n / t.C);
  t.it1 = f + (int)((int64_t)(t.c + 1) * n / t.C);
  t.first = t.z * w.items_per_z + base;
  return t;
}

inline BwdWork make_bwd_work(int64_t b, int64_t sq, int64_t hs, int bb, int causal, int kv, int cus) {
  BwdWork w;
  w.sq = (int)sq;
  w.nz = (int)(b * hs);
  w.bb = bb;
  w.nb = (int)((sq + bb - 1) / bb);
  w.causal = causal;
  w.kv = kv;
  int64_t total = 0;
  int maxt = 1;
  for (int i = 0; i < w.nb; ++i) {
    total += work_tiles(w, i);
    maxt = std::max(maxt, work_tiles(w, i));
  }
  total *= w.nz;
  const int64_t lo = std::max<int64_t>(1, (total + cus - 1) / cus);
  int64_t best = -1, best_cost = 0;
  for (int64_t L = lo; L <= std::max<int64_t>(lo, std::min<int64_t>(2 * lo + 4, maxt)); ++L) {
    w.chunk = (int)L;
    int64_t items = 0;
    for (int i = 0; i < w.nb; ++i) items += work_chunks(w, i);
    items *= w.nz;
    const int64_t cost = (items + cus - 1) / cus * L;
    if (best < 0 || cost <= best_cost) {
      best = L;
      best_cost = cost;
    }
  }
  w.chunk = (int)best;
  w.items_per_z = 0;
  for (int i = 0; i < w.nb; ++i) w.items_per_z += work_chunks(w, i);
  return w;
}

__host__ __device__ inline int work_total(const BwdWork& w) { return w.items_per_z * w.nz; }
inline int work_merges_per_z(const BwdWork& w) {
  int n = 0;
  for (int i = 0; i < w.nb; ++i) n += work_chunks(w, i) > 1 ? 1 : 0;
  return n;
}

// ---------------------------------------------------------------- Delta, dQ
// PHASE 0: per item, the partial row sums of P dP and of P over its keys
// (rd[item][row][2]).  PHASE 1: Delta of each row from its block's partials
// (in chunk order, so every chunk of a block gets the same bits), then dQ
// over the item's keys: written as bf16 when the block is one chunk, else
// as an fp32 partial (part[item][row][D]) for the merge; the block's first
// chunk also writes -Delta (negated) for the dK/dV phase.
template <int D, int PHASE>
__global__ void __launch_bounds__((BwdShape<D, false>::THREADS), (D <= 128 ? 2 : 1))
attn_bwd_q_kernel(const bf16_t* __restrict__ qkv, const bf16_t* __restrict__ dO, const float* __restrict__ lse,
                  bf16_t* __restrict__ dqkv, float* __restrict__ delta, float* __restrict__ rd,
                  float* __restrict__ part, BwdPlan p, BwdWork wk) {
  using S = BwdShape<D, false>;
  constexpr int QB = S::RB;     // 16-row blocks per wave
  constexpr int WR = 16 * QB;   // query rows per wave
  __shared__ __attribute__((aligned(16))) bf16_t lds[4 * S::TILE];   // K0 K1 V0 V1

  const int total = work_total(wk);
  const int item = total - 1 - (int)blockIdx.x;   // longest blocks first
  const Item it = work_item(wk, item);
  const int z = it.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int zo = z / p.hs, zi = z - zo * p.hs;
  const bf16_t* Qh = qkv + (int64_t)zo * p.sq * p.ld + (int64_t)zi * D;
  const bf16_t* Kh = Qh + (int64_t)p.hs * D;
  const bf16_t* Vh = Kh + (int64_t)p.hs * D;
  const bf16_t* dOh = dO + (int64_t)zo * p.sq * p.ldo + (int64_t)zi * D;
  const int q0 = it.i * S::BB + wave * WR;
  const int niter = it.it1 - it.it0;

  const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16_t*)lds);
  auto issue = [&](int jj) {   // key tile it0 + jj into stage jj & 1
    const int kb = (it.it0 + jj) * kBT;
    const uint32_t st = (uint32_t)(jj & 1);
    bwd_dma_tile<S>(Kh, p.ld, kb, p.sq - 1, lds0, st * S::TILE * 2, wave, lane);
    bwd_dma_tile<S>(Vh, p.ld, kb, p.sq - 1, lds0, (2 + st) * S::TILE * 2, wave, lane);
  };
  issue(0);
  if (niter > 1) issue(1);

  bf16x8_t qf[QB][S::KS], of[QB][S::KS];
  float lse2[QB], dl[QB];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const int row = min(q0 + 16 * b + r16, p.sq - 1);
    const bf16_t* qs = Qh + (int64_t)row * p.ld + 8 * g;
    const bf16_t* os = dOh + (int64_t)row * p.ldo + 8 * g;
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) {
      qf[b][ks] = *reinterpret_cast<const bf16x8_t*>(qs + 32 * ks);
      of[b][ks] = *reinterpret_cast<const bf16x8_t*>(os + 32 * ks);
    }
    lse2[b] = lse[(int64_t)z * p.sq + row] * 1.4426950408889634f;
    dl[b] = 0.f;
    if constexpr (PHASE == 1) {
      const int rl = wave * WR + 16 * b + r16;
      float num = 0.f, den = 0.f;
      for (int c = 0; c < it.C; ++c) {
        const float* r = rd + ((int64_t)(it.first + c) * S::BB + rl) * 2;
        num += r[0];
        den += r[1];
      }
      dl[b] = den > 0.f ? num / den : 0.f;
    }
  }
#pragma unroll
  for (int b = 0; b < QB; ++b)
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) {
      loaded_here(qf[b][ks]);
      loaded_here(of[b][ks]);
    }
  f32x4_t acc[QB][S::NB];
#pragma unroll
  for (int b = 0; b < QB; ++b)
#pragma unroll
    for (int n = 0; n < S::NB; ++n) acc[b][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float num[QB], den[QB];
#pragma unroll
  for (int b = 0; b < QB; ++b) num[b] = den[b] = 0.f;

  wait_vmem_known();
  __syncthreads();

  for (int jj = 0; jj < niter; ++jj) {
    const int kb = (it.it0 + jj) * kBT;
    const bf16_t* Kt = lds + (jj & 1) * S::TILE;
    const bf16_t* Vt = lds + (2 + (jj & 1)) * S::TILE;
    const bool live = !p.causal || kb <= q0 + WR - 1;
    if (live) {
      // S = Q K^T, then dP = dO V^T: lane holds row 16 b + r16, keys
      // 16 h + 4 g + e.  The S chain goes first, so the P arithmetic runs
      // while the dP MFMAs execute.  The next k-step's fragments are read
      // while this one's MFMAs run; the scheduling barriers keep the compiler
      // from hoisting every read of the loop.
      f32x4_t s[QB][2], dp[QB][2];
      auto chain = [&](const bf16_t* tile, const bf16x8_t (&x)[QB][S::KS], f32x4_t (&c)[QB][2]) {
        bf16x8_t f0 = bwd_row_frag<S>(tile, 0, 0, r16, g), f1 = bwd_row_frag<S>(tile, 0, 1, r16, g);
#pragma unroll
        for (int ks = 0; ks < S::KS; ++ks) {
          bf16x8_t n0 = f0, n1 = f1;
          if (ks + 1 < S::KS) {
            n0 = bwd_row_frag<S>(tile, ks + 1, 0, r16, g);
            n1 = bwd_row_frag<S>(tile, ks + 1, 1, r16, g);
          }
#pragma unroll
          for (int b = 0; b < QB; ++b) {
            const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
            c[b][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f0, x[b][ks], ks == 0 ? z : c[b][0], 0, 0, 0);
            c[b][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f1, x[b][ks], ks == 0 ? z : c[b][1], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
          f0 = n0;
          f1 = n1;
        }
      };
      chain(Kt, qf, s);
      chain(Vt, of, dp);
      // P; the mask is tested only on a tile that reaches past the sequence
      // or (causal) past the wave's first row (wave-uniform choice)
      float pr[QB][8];
      auto probs = [&](auto mask) {
#pragma unroll
        for (int b = 0; b < QB; ++b) {
          const int row = q0 + 16 * b + r16;
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int key = kb + 16 * h + 4 * g + e;
              float x = s[b][h][e] * p.scale_log2 - lse2[b];
              // a masked pair's exponent is -inf (2^-inf = 0): a select, not a branch
              if constexpr (decltype(mask)::value) x = (key >= p.sq || (p.causal && key > row)) ? -INFINITY : x;
              pr[b][4 * h + e] = fast_exp2(x);
            }
        }
      };
      if (kb + kBT <= p.sq && (!p.causal || kb + kBT - 1 <= q0)) probs(std::false_type{});
      else probs(std::true_type{});
      if constexpr (PHASE == 0) {
#pragma unroll
        for (int b = 0; b < QB; ++b)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              num[b] += pr[b][4 * h + e] * dp[b][h][e];
              den[b] += pr[b][4 * h + e];
            }
      } else {
        bf16x8_t dsf[QB];
#pragma unroll
        for (int b = 0; b < QB; ++b) {
          float ds[8];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) ds[4 * h + e] = pr[b][4 * h + e] * (dp[b][h][e] - dl[b]);
          dsf[b] = pack_frag(ds);
        }
        // dQ += dS K: K^T fragment of column block n at key rows 4 g.. and 16 + 4 g..
        bf16x8_t kc = bwd_tr_frag<S>(Kt, 0, r16, g);
#pragma unroll
        for (int n = 0; n < S::NB; ++n) {
          bf16x8_t kn = kc;
          if (n + 1 < S::NB) kn = bwd_tr_frag<S>(Kt, n + 1, r16, g);
#pragma unroll
          for (int b = 0; b < QB; ++b) acc[b][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc, dsf[b], acc[b][n], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          kc = kn;
        }
      }
    }
    if (jj + 1 < niter) {
      wait_vmem();        // this wave's DMA of iteration jj+1 landed
      __syncthreads();    // every wave's did, and every wave is done with stage jj & 1
      if (jj + 2 < niter) issue(jj + 2);
    }
  }

#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const int rl = wave * WR + 16 * b + r16;
    const int row = q0 + 16 * b + r16;
    if constexpr (PHASE == 0) {
      num[b] += __shfl_xor(num[b], 16);
      num[b] += __shfl_xor(num[b], 32);
      den[b] += __shfl_xor(den[b], 16);
      den[b] += __shfl_xor(den[b], 32);
      if (g == 0) *reinterpret_cast<float2*>(rd + ((int64_t)item * S::BB + rl) * 2) = float2{num[b], den[b]};
    } else {
      if (it.C == 1) {
        if (row < p.sq) {
          bf16_t* dst = dqkv + ((int64_t)zo * p.sq + row) * p.ld + (int64_t)zi * D + 4 * g;
#pragma unroll
          for (int n = 0; n < S::NB; ++n) {
            const f32x4_t v = acc[b][n] * p.scale;
            *reinterpret_cast<u32x2_t*>(dst + 16 * n) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          }
        }
      } else {
        float* po = part + ((int64_t)item * S::BB + rl) * D + 4 * g;
#pragma unroll
        for (int n = 0; n < S::NB; ++n) *reinterpret_cast<f32x4_t*>(po + 16 * n) = acc[b][n] * p.scale;
      }
      if (it.c == 0 && g == 0 && row < p.sq) delta[(int64_t)z * p.sq + row] = -dl[b];   // stored negated
    }
  }
}

// ---------------------------------------------------------------- dK, dV
// Per item: the keys of its block against the queries of its chunk; dK and
// dV written as bf16 when the block is one chunk, else as one fp32 partial
// (part[item][key][2 D]: dK then dV) for the merge.
template <int D>
__global__ void __launch_bounds__((BwdShape<D, true>::THREADS), (D <= 64 ? 2 : 1))
attn_bwd_kv_kernel(const bf16_t* __restrict__ qkv, const bf16_t* __restrict__ dO, const float* __restrict__ lse,
                   const float* __restrict__ delta, bf16_t* __restrict__ dqkv, float* __restrict__ part, BwdPlan p,
                   BwdWork wk) {
  using S = BwdShape<D, true>;
  constexpr int KB = S::RB;     // 16-key blocks per wave
  constexpr int WR = 16 * KB;   // keys per wave
  __shared__ __attribute__((aligned(16))) bf16_t lds[4 * S::TILE];   // Q0 Q1 dO0 dO1
  __shared__ __attribute__((aligned(16))) float rowv[2][2][64];        // per stage: lse, Delta of the tile's queries

  const int total = work_total(wk);
  const int item = total - 1 - (int)blockIdx.x;   // longest blocks first
  const Item it = work_item(wk, item);
  const int z = it.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int zo = z / p.hs, zi = z - zo * p.hs;
  const bf16_t* Qh = qkv + (int64_t)zo * p.sq * p.ld + (int64_t)zi * D;
  const bf16_t* Kh = Qh + (int64_t)p.hs * D;
  const bf16_t* Vh = Kh + (int64_t)p.hs * D;
  const bf16_t* dOh = dO + (int64_t)zo * p.sq * p.ldo + (int64_t)zi * D;
  const float* lz = lse + (int64_t)z * p.sq;
  const float* dz = delta + (int64_t)z * p.sq;
  const int k0 = it.i * S::BB + wave * WR;   // first key of this wave
  const int niter = it.it1 - it.it0;

  const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16_t*)lds);
  const uint32_t rv0 = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)(uintptr_t)(__attribute__((address_space(3))) float*)&rowv[0][0][0]);
  auto issue = [&](int jj) {   // query tile it0 + jj (and its lse, Delta) into stage jj & 1
    const int qb = (it.it0 + jj) * kBT;
    const uint32_t st = (uint32_t)(jj & 1);
    bwd_dma_tile<S>(Qh, p.ld, qb, p.sq - 1, lds0, st * S::TILE * 2, wave, lane);
    bwd_dma_tile<S>(dOh, p.ldo, qb, p.sq - 1, lds0, (2 + st) * S::TILE * 2, wave, lane);
    if (wave < 2) bwd_dma_rowvals(wave == 0 ? lz : dz, qb, p.sq - 1, rv0 + (2 * st + wave) * 256, lane);
  };
  issue(0);
  if (niter > 1) issue(1);

  bf16x8_t kf[KB][S::KS], vf[KB][S::KS];
#pragma unroll
  for (int b = 0; b < KB; ++b) {
    const int row = min(k0 + 16 * b + r16, p.sq - 1);
    const bf16_t* ks_ = Kh + (int64_t)row * p.ld + 8 * g;
    const bf16_t* vs_ = Vh + (int64_t)row * p.ld + 8 * g;
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) {
      kf[b][ks] = *reinterpret_cast<const bf16x8_t*>(ks_ + 32 * ks);
      vf[b][ks] = *reinterpret_cast<const bf16x8_t*>(vs_ + 32 * ks);
    }
  }
#pragma unroll
  for (int b = 0; b < KB; ++b)
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) {
      loaded_here(kf[b][ks]);
      loaded_here(vf[b][ks]);
    }
  f32x4_t dk[KB][S::NB], dv[KB][S::NB];
#pragma unroll
  for (int b = 0; b < KB; ++b)
#pragma unroll
    for (int n = 0; n < S::NB; ++n) dk[b][n] = dv[b][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  wait_vmem_known();
  __syncthreads();

  for (int jj = 0; jj < niter; ++jj) {
    const int qb = (it.it0 + jj) * kBT;
    const bf16_t* Qt = lds + (jj & 1) * S::TILE;
    const bf16_t* Ot = lds + (2 + (jj & 1)) * S::TILE;
    // queries of this tile all before the wave's first key: nothing to add
    const bool live = !p.causal || qb + kBT - 1 >= k0;
    if (live) {
      // lane holds key 16 b + r16 and the tile's queries 16 h + 4 g + e
      const float* rv = &rowv[jj & 1][0][0];
      // S^T = K Q^T and dP^T - Delta = V dO^T - Delta back to back, so that
      // the P arithmetic runs while the dP^T MFMAs execute and the dS
      // arithmetic while the dV MFMAs do.  The S^T accumulators start at
      // -lse sqrt(d), so that scaling them by log2(e) / sqrt(d) gives the
      // exponent of P directly; the dP^T ones at -Delta.  The next k-step's
      // fragments are read while this one's MFMAs run.
      f32x4_t sc[KB][2], dc[KB][2];
      {
        f32x4_t l4[2];   // the first k-step's MFMAs start from it
#pragma unroll
        for (int h = 0; h < 2; ++h) l4[h] = *reinterpret_cast<const f32x4_t*>(rv + 16 * h + 4 * g) * p.neg_sqrt_d;
        bf16x8_t f0 = bwd_row_frag<S>(Qt, 0, 0, r16, g), f1 = bwd_row_frag<S>(Qt, 0, 1, r16, g);
#pragma unroll
        for (int ks = 0; ks < S::KS; ++ks) {
          bf16x8_t n0 = f0, n1 = f1;
          if (ks + 1 < S::KS) {
            n0 = bwd_row_frag<S>(Qt, ks + 1, 0, r16, g);
            n1 = bwd_row_frag<S>(Qt, ks + 1, 1, r16, g);
          }
#pragma unroll
          for (int b = 0; b < KB; ++b) {
            sc[b][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f0, kf[b][ks], ks == 0 ? l4[0] : sc[b][0], 0, 0, 0);
            sc[b][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f1, kf[b][ks], ks == 0 ? l4[1] : sc[b][1], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
          f0 = n0;
          f1 = n1;
        }
      }
      {
        f32x4_t d4[2];   // -Delta of the tile's queries (stored negated)
#pragma unroll
        for (int h = 0; h < 2; ++h) d4[h] = *reinterpret_cast<const f32x4_t*>(rv + 64 + 16 * h + 4 * g);
        bf16x8_t f0 = bwd_row_frag<S>(Ot, 0, 0, r16, g), f1 = bwd_row_frag<S>(Ot, 0, 1, r16, g);
#pragma unroll
        for (int ks = 0; ks < S::KS; ++ks) {
          bf16x8_t n0 = f0, n1 = f1;
          if (ks + 1 < S::KS) {
            n0 = bwd_row_frag<S>(Ot, ks + 1, 0, r16, g);
            n1 = bwd_row_frag<S>(Ot, ks + 1, 1, r16, g);
          }
#pragma unroll
          for (int b = 0; b < KB; ++b) {
            dc[b][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f0, vf[b][ks], ks == 0 ? d4[0] : dc[b][0], 0, 0, 0);
            dc[b][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f1, vf[b][ks], ks == 0 ? d4[1] : dc[b][1], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
          f0 = n0;
          f1 = n1;
        }
      }
      // P^T (fp32, kept for dS) and its bf16 fragment.  The mask is tested
      // only on a tile that reaches past the sequence or (causal) before the
      // wave's last key (wave-uniform choice).
      float pr[KB][8];
      bf16x8_t pf[KB];
      {
        auto probs = [&](auto mask) {
#pragma unroll
          for (int b = 0; b < KB; ++b) {
            const int key = k0 + 16 * b + r16;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int q = qb + 16 * h + 4 * g + e;
                float x = sc[b][h][e] * p.scale_log2;
                // a masked pair's exponent is -inf (2^-inf = 0): a select, not a branch
                if constexpr (decltype(mask)::value) x = (q >= p.sq || (p.causal && q < key)) ? -INFINITY : x;
                pr[b][4 * h + e] = fast_exp2(x);
              }
            pf[b] = pack_frag(pr[b]);
          }
        };
        if (qb + kBT <= p.sq && (!p.causal || qb >= k0 + WR - 1)) probs(std::false_type{});
        else probs(std::true_type{});
      }
      // dV += P^T dO: dO^T fragment of column block n at query rows 4 g.. and 16 + 4 g..
      {
        bf16x8_t oc = bwd_tr_frag<S>(Ot, 0, r16, g);
#pragma unroll
        for (int n = 0; n < S::NB; ++n) {
          bf16x8_t on = oc;
          if (n + 1 < S::NB) on = bwd_tr_frag<S>(Ot, n + 1, r16, g);
#pragma unroll
          for (int b = 0; b < KB; ++b) dv[b][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oc, pf[b], dv[b][n], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          oc = on;
        }
      }
      // P^T (dP^T - Delta) as a bf16 fragment (dK takes the 1 / sqrt(d) at the end)
      bf16x8_t dsf[KB];
#pragma unroll
      for (int b = 0; b < KB; ++b) {
        float ds[8];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) ds[4 * h + e] = pr[b][4 * h + e] * dc[b][h][e];
        dsf[b] = pack_frag(ds);
      }
      // dK += dS^T Q: Q^T fragment of column block n at query rows 4 g.. and 16 + 4 g..
      {
        bf16x8_t qc = bwd_tr_frag<S>(Qt, 0, r16, g);
#pragma unroll
        for (int n = 0; n < S::NB; ++n) {
          bf16x8_t qn = qc;
          if (n + 1 < S::NB) qn = bwd_tr_frag<S>(Qt, n + 1, r16, g);
#pragma unroll
          for (int b = 0; b < KB; ++b) dk[b][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qc, dsf[b], dk[b][n], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          qc = qn;
        }
      }
    }
    if constexpr (S::AGPR_ACC) {
      // the accumulators stay in the accumulation registers across
      // iterations (the MFMAs read and write them there in place)
#pragma unroll
      for (int b = 0; b < KB; ++b)
#pragma unroll
        for (int n = 0; n < S::NB; ++n) asm volatile("" : "+a"(dk[b][n]), "+a"(dv[b][n]));
    }
    if (jj + 1 < niter) {
      wait_vmem();
      __syncthreads();
      if (jj + 2 < niter) issue(jj + 2);
    }
  }

#pragma unroll
  for (int b = 0; b < KB; ++b) {
    const int rl = wave * WR + 16 * b + r16;
    const int row = k0 + 16 * b + r16;
    if (it.C == 1) {
      if (row < p.sq) {
        bf16_t* dkd = dqkv + ((int64_t)zo * p.sq + row) * p.ld + (int64_t)(p.hs + zi) * D + 4 * g;
        bf16_t* dvd = dkd + (int64_t)p.hs * D;
#pragma unroll
        for (int n = 0; n < S::NB; ++n) {
          const f32x4_t a = dk[b][n] * p.scale, c = dv[b][n];
          *reinterpret_cast<u32x2_t*>(dkd + 16 * n) = u32x2_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
          *reinterpret_cast<u32x2_t*>(dvd + 16 * n) = u32x2_t{pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3])};
        }
      }
    } else {
      float* po = part + ((int64_t)item * S::BB + rl) * (2 * D) + 4 * g;
#pragma unroll
      for (int n = 0; n < S::NB; ++n) {
        *reinterpret_cast<f32x4_t*>(po + 16 * n) = dk[b][n] * p.scale;
        *reinterpret_cast<f32x4_t*>(po + D + 16 * n) = dv[b][n];
      }
    }
  }
}

// ---------------------------------------------------------------- merge
// Rows of one split block that a merge workgroup covers: one thread per
// (row, 4 of the W columns), W = D (dQ) or 2 D (dK then dV).
template <int W>
constexpr int merge_rows() {
  return kMergeThreads / (W / 4) >= 1 ? kMergeThreads / (W / 4) : 1;
}
// Workgroups of a merge: every split block of every (batch, head).
inline int merge_workgroups(const BwdWork& wk, int merges_per_z, int rows) {
  return merges_per_z * wk.nz * (wk.bb / rows);
}

// Sum of a split block's chunk partials in chunk order, rounded once to
// bf16 into dQKV: W = D columns (dQ of head zi) or 2 D (dK then dV).  Merge
// workgroup `wg` covers merge_rows<W>() rows of one split block.
template <int D, bool KV>
__device__ __forceinline__ void bwd_merge_block(const float* __restrict__ part, bf16_t* __restrict__ dqkv,
                                                const BwdPlan& p, const BwdWork& wk, int merges_per_z, int wg) {
  constexpr int W = KV ? 2 * D : D;
  constexpr int CH = W / 4;
  constexpr int ROWS = merge_rows<W>();
  const int groups = wk.bb / ROWS;
  const int blk = wg / groups;
  const int rg = wg - blk * groups;
  const int z = blk / merges_per_z;
  const int k = blk - z * merges_per_z;   // k-th split block of this (batch, head), in slot order
  const Located l = wave_locate(wk.nb, k, [&](int s) {
    const int c = work_chunks(wk, work_block(wk, s));
    return int2{c > 1 ? 1 : 0, c};
  });
  const int i = work_block(wk, __builtin_amdgcn_readfirstlane(l.s));
  const int base = __builtin_amdgcn_readfirstlane(l.b);
  const int C = work_chunks(wk, i);
  const int first = z * wk.items_per_z + base;
  const int zo = z / p.hs, zi = z - zo * p.hs;
  for (int e = threadIdx.x; e < ROWS * CH; e += kMergeThreads) {
    const int rl = rg * ROWS + e / CH, ch = e % CH;
    const int row = i * wk.bb + rl;
    if (row >= p.sq) continue;
    // four chunks' loads in flight at a time, added in chunk order
    const float* src = part + ((int64_t)first * wk.bb + rl) * W + 4 * ch;
    const int64_t cs = (int64_t)wk.bb * W;   // floats between consecutive chunks' partials
    f32x4_t o = {0.f, 0.f, 0.f, 0.f};
    int c = 0;
    for (; c + 4 <= C; c += 4) {
      const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(src + (c + 0) * cs);
      const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(src + (c + 1) * cs);
      const f32x4_t a2 = *reinterpret_cast<const f32x4_t*>(src + (c + 2) * cs);
      const f32x4_t a3 = *reinterpret_cast<const f32x4_t*>(src + (c + 3) * cs);
      o += a0;
      o += a1;
      o += a2;
      o += a3;
    }
    for (; c < C; ++c) o += *reinterpret_cast<const f32x4_t*>(src + c * cs);
    const int col = 4 * ch;
    const int64_t dcol = KV ? (col < D ? (int64_t)(p.hs + zi) * D + col : (int64_t)(2 * p.hs + zi) * D + col - D)
                            : (int64_t)zi * D + col;
    bf16_t* dst = dqkv + ((int64_t)zo * p.sq + row) * p.ld + dcol;
    *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
  }
}

// Both merges in one launch: workgroups [0, nq_wg) merge the dQ partials
// (split query blocks), the rest the dK/dV partials (split key blocks).  The
// two write disjoint columns of dQKV, and each is latency-bound on its own
// (a few 16-byte loads per thread), so one grid lets them overlap.
template <int D>
__global__ void __launch_bounds__(kMergeThreads) attn_bwd_merge_kernel(const float* __restrict__ qpart,
                                                                       const float* __restrict__ kvpart,
                                                                       bf16_t* __restrict__ dqkv, BwdPlan p,
                                                                       BwdWork wq, int mq, BwdWork wk, int mk,
                                                                       int nq_wg) {
  const int wg = (int)blockIdx.x;
  if (wg < nq_wg) bwd_merge_block<D, false>(qpart, dqkv, p, wq, mq, wg);
  else bwd_merge_block<D, true>(kvpart, dqkv, p, wk, mk, wg - nq_wg);
}

}  // namespace flash
}  // namespace tps
