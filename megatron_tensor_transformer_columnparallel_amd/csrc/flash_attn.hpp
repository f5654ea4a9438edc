// Flash-style attention forward for one tensor-parallel shard (head dims
// 256 and 512; head dims 64 and 128 run the two-group kernel of
// flash_fwd_pp.hpp, which shares this file's plan, layouts and merge).
//
// Per (batch, head) the queries are cut into blocks of 128 rows; a work item
// is one query block and a contiguous range of its keys (all of them when the
// range is short enough, otherwise one of several chunks).  A workgroup of
// four waves (one per SIMD, so each wave may hold 512 registers) runs one
// item: wave w owns 32 query rows, keeps their Q fragments in VGPRs (D/2
// registers) and their output accumulator O (32 x D fp32, D/2 x 4 values per
// lane) in the accumulation registers, and walks the keys 32 at a time:
//
//   S = Q K^T      16x16x32 bf16 MFMAs; K tile from LDS (ds_read_b128)
//   online softmax in the log2 domain, in registers: the running row max is
//                  moved only when a new score exceeds it by more than 8
//                  (the accumulators are rescaled then; otherwise the
//                  probabilities stay below 2^8), masked scores give 0
//   O += P V       P rounded to bf16 as the A operand straight from the S
//                  accumulators: the lane holding keys 4g..4g+3 of both
//                  16-key halves uses them as its k slots 8g..8g+7, and the
//                  V fragment is read with the transposing LDS read at the
//                  same key rows (4g.. and 16+4g..), so no data moves
//                  between lanes
//
// K and V tiles (32 keys x D) go global -> LDS with direct DMA
// (global_load_lds_dwordx4), two stages each (128 KB at D = 512): the tiles
// of iteration j+2 are issued right after the barrier that ends iteration j.
// Neither S nor P ever leaves the chip.  An item that covers all keys of its
// block normalises O by the row sum and writes O (bf16) and the log-sum-exp;
// the chunks of a split block write their unnormalised O, running max and
// row sum (fp32) to the workspace and a merge kernel combines them
// (O = sum_c 2^(m_c - m) O_c / sum_c 2^(m_c - m) l_c).  The split makes
// about one item per CU regardless of the sequence length, so the workspace
// is bounded by the CU count times 128 x D, not by the square of the
// sequence.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>

#include "gemm.hpp"

namespace tps {
namespace flash {

constexpr int kBQ = 128;       // query rows per work item
constexpr int kBK = 32;        // keys per iteration
constexpr float kLazy = 8.f;   // log2 headroom before the running max moves

// QB 16-row MFMA blocks of queries per wave: kBQ / (16 QB) waves per item.
template <int D, int QB>
struct Shape {
  static constexpr int WQ = 16 * QB;          // query rows per wave
  static constexpr int WAVES = kBQ / WQ;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int KS = D / 32;      // 32-wide k-steps of Q K^T
  static constexpr int NB = D / 16;      // 16-column blocks of O
  static constexpr int CPR = D / 8;      // 16-byte chunks per K or V row
  // LDS layout of a K or V tile (kBK key rows of CPR 16-byte chunks).
  // Rows of 16 or 32 chunks: XOR swizzle.  K: chunk c of key row r sits at
  // c ^ (r & 15), so the 16 lanes that read one chunk of 16 consecutive keys
  // hit 16 distinct slots; V: at c ^ 2 (r & 7) (chunk pairs stay pairs), so
  // the transposing read of 4 consecutive key rows x 32 bytes by a 16-lane
  // group, and of two such groups, hits distinct slots.  Rows of 8 chunks
  // (head dim 64): both at c ^ (r & 7), which keeps the row read and the
  // transposing read at full LDS rate (a pattern probe timed 2 (r & 3) for V
  // 1.3x slower there).
  // Rows of 64 chunks (head dim 512): each row is padded to ROT_PITCH chunks
  // and rotated instead (chunk c of K row r at c + (r & 15), of V row r at
  // c + 2 (r & 7)): the same bank spread, but a lane's address for every
  // k-step or column block is one base plus a compile-time offset, which
  // keeps the per-lane address registers down to a few.
  static constexpr bool ROT = CPR >= 64;
  static constexpr int PITCH = ROT ? (CPR + 16) * 8 : D;   // bf16 elements per LDS row
  static constexpr int TILE = kBK * PITCH;                // bf16 elements of one K or V tile
  // slot of logical chunk c of K (V) row r (XOR layouts)
  static __host__ __device__ constexpr int kswz(int r) { return CPR >= 16 ? (r & 15) : (r & 7); }
  static __host__ __device__ constexpr int vswz(int r) { return CPR >= 16 ? 2 * (r & 7) : (r & 7); }
  // element offset of logical chunk c of K (V) row r
  static __device__ __forceinline__ int koff(int r, int c) {
    return r * PITCH + (ROT ? c + (r & 15) : c ^ kswz(r)) * 8;
  }
  static __device__ __forceinline__ int voff(int r, int c) {
    return r * PITCH + (ROT ? c + 2 * (r & 7) : c ^ vswz(r)) * 8;
  }
  static constexpr int DPW = kBK * CPR / 64 / WAVES;   // 1 KB DMA instructions per wave per tile
  static_assert(D % 64 == 0 && D >= 64 && D <= 512, "head dim");
  static_assert(QB == 1 || QB == 2, "one or two row blocks per wave");
  static_assert(DPW >= 1 && DPW * 64 * WAVES == kBK * CPR, "DMA split");
};

// Work decomposition shared by the host, the forward kernel and the merge.
struct Plan {
  int sq = 0;           // sequence length
  int hs = 0;           // heads of this shard
  int bq = kBQ;         // query rows per block (128, or 256 for the two-group kernel)
  int nqb = 0;          // query blocks per (batch, head)
  int causal = 0;
  int chunk = 1;        // most iterations (of kBK keys) in one work item
  int items_per_z = 0;  // items of one (batch, head)
  int nz = 0;           // batch * hs
  int64_t ld = 0;       // QKV row stride (3 hs D)
  int64_t ldo = 0;      // O row stride (hs D)
  float scale_log2 = 0.f;   // log2(e) / sqrt(D)
};

__host__ __device__ inline int block_iters(const Plan& p, int i) {
  const int kend = p.causal ? min(p.sq, (i + 1) * p.bq) : p.sq;
  return (kend + kBK - 1) / kBK;
}
__host__ __device__ inline int block_chunks(const Plan& p, int i) {
  return (block_iters(p, i) + p.chunk - 1) / p.chunk;
}

// Search over blocks 0 .. nb-1 with per-block counts (a, b) = cnt(s): the
// first block s at which the running sum of a exceeds r, and the sums of a
// and of b over the blocks before it.  The wave's 64 lanes take 64 blocks
// at a time and form inclusive prefix sums by shuffles, so a search costs
// one count per lane and round instead of one per block.  Called by every
// lane of the wave; all lanes get the same result.  If r is past the total,
// the last block is returned (with its sums before it).
struct Located {
  int s, a, b;
};
template <class F>
__device__ inline Located wave_locate(int nb, int r, F cnt) {
  const int lane = threadIdx.x & 63;
  int a0 = 0, b0 = 0, la = 0, lb = 0;
  for (int s0 = 0; s0 < nb; s0 += 64) {
    const int s = s0 + lane;
    int ca = 0, cb = 0;
    if (s < nb) {
      const int2 c = cnt(s);
      ca = c.x;
      cb = c.y;
    }
    int ia = ca, ib = cb;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int ta = __shfl_up(ia, off), tb = __shfl_up(ib, off);
      if (lane >= off) {
        ia += ta;
        ib += tb;
      }
    }
    const uint64_t hit = __ballot(a0 + ia > r);
    if (hit) {
      const int L = __ffsll((unsigned long long)hit) - 1;
      return Located{s0 + L, a0 + __shfl(ia - ca, L), b0 + __shfl(ib - cb, L)};
    }
    const int last = min(63, nb - 1 - s0);
    la = __shfl(ca, last);
    lb = __shfl(cb, last);
    a0 += __shfl(ia, 63);
    b0 += __shfl(ib, 63);
  }
  return Located{nb - 1, a0 - la, b0 - lb};
}

// item -> (z, query block i, chunk c of C, its iterations [it0, it1), first item of the block)
struct Item {
  int z, i, c, C, it0, it1, first;
};
__device__ inline Item decode_item(const Plan& p, int item) {
  Item t;
  t.z = item / p.items_per_z;
  const int r = item - t.z * p.items_per_z;
  const Located l = wave_locate(p.nqb, r, [&](int i) { return int2{block_chunks(p, i), 0}; });
  const int base = __builtin_amdgcn_readfirstlane(l.a);
  t.i = __builtin_amdgcn_readfirstlane(l.s);
  t.c = r - base;
  t.C = block_chunks(p, t.i);
  const int n = block_iters(p, t.i);
  t.it0 = (int)((int64_t)t.c * n / t.C);
  t.it1 = (int)((int64_t)(t.c + 1) * n / t.C);
  t.first = t.z * p.items_per_z + base;
  return t;
}

// 2^x by the hardware instruction (v_exp_f32, about 1 ulp; results below the
// normal range flush to 0, which a softmax sum never feels, and 2^-inf = 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wait for every vector-memory operation of this wave (vmcnt(0); expcnt and
// lgkmcnt left at their maxima), as the compiler's own instruction: its
// wait-count pass then knows that the loads issued before this point are
// complete.  The inline-assembly wait does not tell it that, so before a
// loop it would place waits for those loads inside the loop body, where they
// also wait for the tile DMA in flight (which the compiler does not count)
// on every iteration.
__device__ __forceinline__ void wait_vmem_known() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Makes the compiler complete a loaded value here (it places its own wait
// before this point), so that the load is neither moved into nor waited
// for inside a loop that follows.
template <class T>
__device__ __forceinline__ void loaded_here(const T& x) { asm volatile("" :: "v"(x)); }

// Reductions of a value over lanes i and i ^ 16 (i ^ 32) by the lane-swap
// instructions: with both operands holding v, the swap leaves lane i with
// v_i in one and v_(i^16) (v_(i^32)) in the other.
__device__ __forceinline__ float lane_max16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float lane_max32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float lane_sum16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float lane_sum32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two fp32 values to a bf16 pair by the hardware conversion (round to nearest
// even, as pack_bf16x2), one instruction instead of the bit arithmetic.
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{lo, hi}, b2));
}

__device__ __forceinline__ uint64_t uniform_addr(const void* ptr) {
  const uint64_t b = (uint64_t)(uintptr_t)ptr;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}

template <int D, int QB>
__global__ void __launch_bounds__((Shape<D, QB>::THREADS), (D <= 128 ? 2 : 1))
attn_fwd_flash_kernel(const bf16_t* __restrict__ qkv, bf16_t* __restrict__ O, float* __restrict__ lse,
                      float* __restrict__ part, Plan p, int total_items) {
  using S = Shape<D, QB>;
  constexpr int kWQ = S::WQ;
  // stages: K0, K1, V0, V1
  __shared__ __attribute__((aligned(16))) bf16_t lds[4 * S::TILE];

  const int item = total_items - 1 - (int)blockIdx.x;   // long chunks first, short blocks last
  const Item it = decode_item(p, item);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int zo = it.z / p.hs, zi = it.z - zo * p.hs;
  const bf16_t* Qh = qkv + (int64_t)zo * p.sq * p.ld + (int64_t)zi * D;
  const bf16_t* Kh = Qh + (int64_t)p.hs * D;
  const bf16_t* Vh = Kh + (int64_t)p.hs * D;
  const int q0 = it.i * kBQ + wave * kWQ;   // first query row of this wave

  const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16_t*)lds);
  // DMA of one K or V tile (keys kb .. kb+31 of this head) into LDS at byte
  // offset `off`: instruction i of this wave fills slots (wave DPW + i) 64 ..
  // +63; slot q is row q / CPR, chunk position q % CPR, which holds the
  // row's logical chunk position ^ swizzle.  Rows past the sequence re-read
  // the last row (their scores are masked).
  auto dma_tile = [&](const bf16_t* head, int kb, uint32_t off, bool isV) {
    const int rmax = p.sq - 1 - kb;
#pragma unroll
    for (int i = 0; i < S::DPW; ++i) {
      const int ins = wave * S::DPW + i;   // instruction index within the tile (uniform)
      uint64_t sb;
      uint32_t voff;
      uint32_t m0;
      if constexpr (S::ROT) {
        // whole rows per instruction: the row offset goes into the scalar
        // base and the LDS base; the lane's chunk is its only per-lane
        // offset, and the rotation shifts the row's destination
        constexpr int IPR = S::CPR / 64;   // instructions per row
        const int r = ins / IPR;
        const int c0 = (ins % IPR) * 64;
        sb = uniform_addr(head + (int64_t)(kb + min(r, rmax)) * p.ld + c0 * 8);
        voff = (uint32_t)(lane * 16);
        m0 = lds0 + off + (uint32_t)((isV ? S::voff(r, c0) : S::koff(r, c0)) * 2);
      } else {
        const int q = ins * 64 + lane;
        const int r = q / S::CPR, ph = q % S::CPR;
        const int c = ph ^ (isV ? S::vswz(r) : S::kswz(r));
        sb = uniform_addr(head + (int64_t)kb * p.ld);
        voff = (uint32_t)((int64_t)min(r, rmax) * p.ld * 2 + c * 16);
        m0 = lds0 + off + (uint32_t)(ins * 64 * 16);
      }
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                   :: "v"(voff), "s"(sb), "s"(m0) : "memory", "m0");
    }
  };
  auto issue = [&](int jj) {   // tiles of local iteration jj into stage jj & 1
    const int kb = (it.it0 + jj) * kBK;
    const uint32_t st = (uint32_t)(jj & 1);
    dma_tile(Kh, kb, st * S::TILE * 2, false);
    dma_tile(Vh, kb, (2 + st) * S::TILE * 2, true);
  };

  const int niter = it.it1 - it.it0;
  issue(0);
  if (niter > 1) issue(1);

  // Q fragments of the wave's two 16-row blocks (rows past the sequence
  // re-read the last row; their results are not stored)
  bf16x8_t qf[QB][S::KS];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const int row = min(q0 + 16 * b + r16, p.sq - 1);
    const bf16_t* src = Qh + (int64_t)row * p.ld + 8 * g;
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) qf[b][ks] = *reinterpret_cast<const bf16x8_t*>(src + 32 * ks);
  }
#pragma unroll
  for (int b = 0; b < QB; ++b)
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) loaded_here(qf[b][ks]);
  f32x4_t acc[QB][S::NB];
#pragma unroll
  for (int b = 0; b < QB; ++b)
#pragma unroll
    for (int n = 0; n < S::NB; ++n) acc[b][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m[QB], l[QB];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    m[b] = -INFINITY;
    l[b] = 0.f;
  }

  wait_vmem_known();
  __syncthreads();

  for (int jj = 0; jj < niter; ++jj) {
    const int kb = (it.it0 + jj) * kBK;
    const bf16_t* Kt = lds + (jj & 1) * S::TILE;
    const bf16_t* Vt = lds + (2 + (jj & 1)) * S::TILE;
    // keys of this tile all after the wave's last row: nothing to add
    const bool live = !p.causal || kb <= q0 + kWQ - 1;
    if (live) {
      // S = Q K^T: lane holds row 16 b + r16, keys 16 h + 4 g + e.  The K
      // fragments of the next k-step are read while the MFMAs of this one
      // run; the scheduling barriers keep the compiler from hoisting every
      // read of the loop (which would need 4 KS more registers).
      f32x4_t s[QB][2];
#pragma unroll
      for (int b = 0; b < QB; ++b) s[b][0] = s[b][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      auto kread = [&](int ks, int h) {
        const int r = 16 * h + r16;
        const int o = S::ROT ? S::koff(r, g) + 32 * ks : S::koff(r, 4 * ks + g);
        return *reinterpret_cast<const bf16x8_t*>(Kt + o);
      };
      bf16x8_t kc0 = kread(0, 0), kc1 = kread(0, 1);
#pragma unroll
      for (int ks = 0; ks < S::KS; ++ks) {
        bf16x8_t kn0 = kc0, kn1 = kc1;
        if (ks + 1 < S::KS) {
          kn0 = kread(ks + 1, 0);
          kn1 = kread(ks + 1, 1);
        }
#pragma unroll
        for (int b = 0; b < QB; ++b) {
          s[b][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc0, qf[b][ks], s[b][0], 0, 0, 0);
          s[b][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc1, qf[b][ks], s[b][1], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        kc0 = kn0;
        kc1 = kn1;
      }
      // online softmax (log2 domain).  The mask is applied only on a tile
      // that reaches past the sequence or (causal) past the wave's first row
      // (wave-uniform choice), by setting the raw score to -inf in place;
      // the running max m is kept in log2 units (raw max x scale).
      if (!(kb + kBK <= p.sq && (!p.causal || kb + kBK - 1 <= q0))) {
#pragma unroll
        for (int b = 0; b < QB; ++b) {
          const int row = q0 + 16 * b + r16;
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int key = kb + 16 * h + 4 * g + e;
              if (key >= p.sq || (p.causal && key > row)) s[b][h][e] = -INFINITY;
            }
        }
      }
      bool move = false;
      float mn[QB];
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        float mx = fmaxf(fmaxf(fmaxf(s[b][0][0], s[b][0][1]), fmaxf(s[b][0][2], s[b][0][3])),
                         fmaxf(fmaxf(s[b][1][0], s[b][1][1]), fmaxf(s[b][1][2], s[b][1][3])));
        mx = lane_max16(mx);
        mx = lane_max32(mx);
        mn[b] = fmaxf(m[b], mx * p.scale_log2);
        // -inf + 8 = -inf: the first finite max moves it too
        move |= mn[b] > m[b] + kLazy;
      }
      if (__ballot(move)) {
        // move every row's max to its block max (alpha = 1 where unchanged)
#pragma unroll
        for (int b = 0; b < QB; ++b) {
          // m = -inf and a finite new max: 0 (nothing accumulated yet);
          // a row still without any score: unchanged
          const float alpha = mn[b] == -INFINITY ? 1.f : fast_exp2(m[b] - mn[b]);
          l[b] *= alpha;
#pragma unroll
          for (int n = 0; n < S::NB; ++n) acc[b][n] *= alpha;
          m[b] = mn[b];
        }
      }
      uint32_t pk[QB][4];
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        // a row without any score so far keeps m = -inf: its masked scores
        // give 2^(-inf - 0) = 0
        const float sub = m[b] == -INFINITY ? 0.f : m[b];
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = fast_exp2(fmaf(s[b][e >> 2][e & 3], p.scale_log2, -sub));
          l[b] += pv[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[b][e] = cvt_bf16x2(pv[2 * e], pv[2 * e + 1]);
      }
      bf16x8_t pf[QB];
#pragma unroll
      for (int b = 0; b < QB; ++b) pf[b] = __builtin_bit_cast(bf16x8_t, u32x4_t{pk[b][0], pk[b][1], pk[b][2], pk[b][3]});
      // O += P V: V fragment of column block n, key rows 4g.. and 16+4g..
      // (read one block ahead of its MFMAs)
      const int vrow = 4 * g + (r16 >> 2);
      const bf16_t* vbase = Vt + (r16 & 1) * 4;
      auto vread = [&](int n) {
        const int c = 2 * n + ((r16 & 3) >> 1);
        const bf16_t* pl = vbase + (S::ROT ? S::voff(vrow, (r16 & 3) >> 1) + 16 * n : S::voff(vrow, c));
        const s16x4_t lo =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)pl);
        const s16x4_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(pl + 16 * S::PITCH));
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8_t vc = vread(0);
#pragma unroll
      for (int n = 0; n < S::NB; ++n) {
        bf16x8_t vn = vc;
        if (n + 1 < S::NB) vn = vread(n + 1);
#pragma unroll
        for (int b = 0; b < QB; ++b) acc[b][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vc, pf[b], acc[b][n], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        vc = vn;
      }
    }
    if (jj + 1 < niter) {
      wait_vmem();        // this wave's DMA of iteration jj+1 landed
      __syncthreads();    // every wave's did, and every wave is done with stage jj & 1
      if (jj + 2 < niter) issue(jj + 2);
    }
  }

  // row sums over the four lanes of each row
#pragma unroll
  for (int b = 0; b < QB; ++b) l[b] = lane_sum32(lane_sum16(l[b]));
  if (it.C == 1) {
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const int row = q0 + 16 * b + r16;
      if (row < p.sq) {
        const float inv = 1.f / l[b];
        bf16_t* dst = O + ((int64_t)zo * p.sq + row) * p.ldo + (int64_t)zi * D + 4 * g;
#pragma unroll
        for (int n = 0; n < S::NB; ++n) {
          const f32x4_t v = acc[b][n] * inv;
          *reinterpret_cast<u32x2_t*>(dst + 16 * n) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
        if (g == 0) lse[(int64_t)it.z * p.sq + row] = (m[b] + log2f(l[b])) * 0.69314718055994531f;
      }
    }
  } else {
    float* po = part + (int64_t)item * kBQ * D;
    float* pml = part + (int64_t)total_items * kBQ * D + (int64_t)item * kBQ * 2;
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const int rl = wave * kWQ + 16 * b + r16;
#pragma unroll
      for (int n = 0; n < S::NB; ++n) *reinterpret_cast<f32x4_t*>(po + rl * D + 16 * n + 4 * g) = acc[b][n];
      if (g == 0) {
        pml[2 * rl] = m[b];
        pml[2 * rl + 1] = l[b];
      }
    }
  }
}

// Merge of a split query block's chunks: O = sum_c 2^(m_c - M) O_c / L with
// L = sum_c 2^(m_c - M) l_c and M = max_c m_c, then lse = (M + log2 L) ln 2.
// Chunks whose keys all lie after a row carry m_c = -inf and weigh nothing.
// One thread per (row, 4 columns): a workgroup covers kMergeRows rows of one
// split block, so the grid has (split blocks) x 128 / kMergeRows workgroups
// and every thread's loads are independent.
constexpr int kMergeThreads = 256;
template <int D>
__global__ void __launch_bounds__(kMergeThreads) attn_fwd_merge_kernel(const float* __restrict__ part,
                                                                       bf16_t* __restrict__ O, float* __restrict__ lse,
                                                                       Plan p, int total_items, int merges_per_z) {
  constexpr int CH = D / 4;                      // float4 chunks per row
  constexpr int ROWS = kMergeThreads / CH >= 1 ? kMergeThreads / CH : 1;   // rows per workgroup
  const int GROUPS = p.bq / ROWS;                // workgroups per split block
  const int blk = blockIdx.x / GROUPS;
  const int rg = blockIdx.x - blk * GROUPS;
  const int z = blk / merges_per_z;
  const int k = blk - z * merges_per_z;   // k-th split block of this (batch, head)
  const Located l = wave_locate(p.nqb, k, [&](int i) {
    const int c = block_chunks(p, i);
    return int2{c > 1 ? 1 : 0, c};
  });
  const int i = __builtin_amdgcn_readfirstlane(l.s);
  const int base = __builtin_amdgcn_readfirstlane(l.b);
  const int C = block_chunks(p, i);
  const int first = z * p.items_per_z + base;
  const int zo = z / p.hs, zi = z - zo * p.hs;
  const int bq = p.bq;
  const float* pml = part + (int64_t)total_items * bq * D;
  for (int e = threadIdx.x; e < ROWS * CH; e += kMergeThreads) {
    const int rl = rg * ROWS + e / CH, ch = e % CH;
    const int row = i * bq + rl;
    if (row >= p.sq) continue;
    // one pass over the chunks, four at a time: the four chunks' (m, l) and
    // partial O are loaded together, then added in chunk order to a running
    // sum kept relative to the running max (rescaled when a batch raises it)
    const float* ml = pml + ((int64_t)first * bq + rl) * 2;   // (m, l) of chunk c at ml + c * 2 bq
    const float* src = part + ((int64_t)first * bq + rl) * D + 4 * ch;
    const int64_t cs = (int64_t)bq * D;   // floats between consecutive chunks' partials
    float M = -INFINITY, L = 0.f;
    f32x4_t o = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < C; c0 += 4) {
      float2 mlc[4];
      f32x4_t oc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = min(c0 + j, C - 1);
        mlc[j] = *reinterpret_cast<const float2*>(ml + (int64_t)c * 2 * bq);
        oc[j] = *reinterpret_cast<const f32x4_t*>(src + c * cs);
      }
      float Mb = M;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (c0 + j < C) Mb = fmaxf(Mb, mlc[j].x);
      if (Mb > M) {   // -inf > -inf is false: nothing accumulated while every max is -inf
        const float r = M == -INFINITY ? 0.f : exp2f(M - Mb);
        L *= r;
        o *= r;
        M = Mb;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (c0 + j >= C) break;
        const float w = mlc[j].x == -INFINITY ? 0.f : exp2f(mlc[j].x - M);
        L += w * mlc[j].y;
        o += w * oc[j];
      }
    }
    const float inv = 1.f / L;
    bf16_t* dst = O + ((int64_t)zo * p.sq + row) * p.ldo + (int64_t)zi * D + 4 * ch;
    *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
    if (ch == 0) lse[(int64_t)z * p.sq + row] = (M + log2f(L)) * 0.69314718055994531f;
  }
}

// merge workgroups per split block of bq rows
template <int D>
constexpr int merge_groups(int bq) {
  return bq / (kMergeThreads / (D / 4) >= 1 ? kMergeThreads / (D / 4) : 1);
}

// Host: the plan for a call.  The chunk length minimises (rounds of
// `cus` items) x (iterations per item), preferring longer chunks on ties.
inline Plan make_plan(int64_t b, int64_t sq, int64_t hs, int d, int causal, int cus, int bq = kBQ) {
  Plan p;
  p.sq = (int)sq;
  p.hs = (int)hs;
  p.bq = bq;
  p.nqb = (int)((sq + bq - 1) / bq);
  p.causal = causal;
  p.nz = (int)(b * hs);
  p.ld = 3 * hs * d;
  p.ldo = hs * d;
  p.scale_log2 = 1.4426950408889634f / sqrtf((float)d);
  int64_t total_iters = 0;
  int maxit = 1;
  p.chunk = 1;
  for (int i = 0; i < p.nqb; ++i) {
    total_iters += block_iters(p, i);
    maxit = std::max(maxit, block_iters(p, i));
  }
  total_iters *= p.nz;
  const int64_t lo = std::max<int64_t>(1, (total_iters + cus - 1) / cus);
  int64_t best = -1, best_cost = 0;
  for (int64_t L = lo; L <= std::max<int64_t>(lo, std::min<int64_t>(2 * lo + 4, maxit)); ++L) {
    p.chunk = (int)L;
    int64_t items = 0;
    for (int i = 0; i < p.nqb; ++i) items += block_chunks(p, i);
    items *= p.nz;
    const int64_t cost = (items + cus - 1) / cus * L;
    if (best < 0 || cost <= best_cost) {
      best = L;
      best_cost = cost;
    }
  }
  p.chunk = (int)best;
  p.items_per_z = 0;
  for (int i = 0; i < p.nqb; ++i) p.items_per_z += block_chunks(p, i);
  return p;
}

inline int plan_merges_per_z(const Plan& p) {
  int n = 0;
  for (int i = 0; i < p.nqb; ++i) n += block_chunks(p, i) > 1 ? 1 : 0;
  return n;
}

inline size_t plan_workspace(const Plan& p, int d) {
  const int64_t items = (int64_t)p.items_per_z * p.nz;
  return (size_t)items * p.bq * (d + 2) * sizeof(float);
}

}  // namespace flash
}  // namespace tps
