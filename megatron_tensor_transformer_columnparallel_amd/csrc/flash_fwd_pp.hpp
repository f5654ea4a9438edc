// Two-group flash attention forward (head dims 64 and 128).
//
// The same method as attn_fwd_flash_kernel (S = Q K^T, online softmax in
// the log2 domain, O += P V with P taken straight from the S accumulators;
// the tiling, the LDS layouts and the fragment reads are that kernel's), but
// a work item is a block of 256 query rows run by one workgroup of eight
// waves in two groups of four: group 0 owns rows 0-127, group 1 rows
// 128-255, and waves w and w + 4 share a SIMD.  A round j of the key loop
// has two halves separated by barriers:
//
//   half 0:  group 0: products  S(j) = Q K(j)^T, O += P(j-1) V(j-1)
//            group 1: softmax   S(j-1) -> P(j-1)
//   half 1:  group 0: softmax   S(j) -> P(j)
//            group 1: products  S(j), O += P(j-1) V(j-1)
//
// so on every SIMD one wave issues MFMAs while the other runs the softmax
// arithmetic.  The matrix pipe executes one wave's MFMAs while the vector
// ALU executes the other wave's instructions (a wave's own arithmetic placed
// between its MFMAs does not overlap them), which a single group with a
// barrier per tile never arranges.  Both groups read the same K and V tiles,
// so one 32-key tile feeds 256 query rows.
//
// LDS holds three stages; stage j mod 3 holds K(j) and V(j-1), the operands
// of round j (used in both halves).  The tiles of round j + 2 are issued at
// the start of round j into the stage round j - 1 used, so a tile has two
// rounds to arrive; each wave issues one or two 1 KB DMA instructions per
// round (waves 0-3 the K tile, waves 4-7 the V tile).
//
// Work items, split blocks, partials and the merge are those of the
// 128-row kernel with 256-row blocks (Plan::bq = 256).
#pragma once

#include <type_traits>

#include "flash_attn.hpp"

namespace tps {
namespace flash {

constexpr int kPPRows = 256;   // query rows per work item
constexpr int kPPStages = 3;   // LDS stages of (K(j), V(j-1))

template <int D>
struct PPShape {
  using L = Shape<D, 2>;                        // tile layout and fragment reads (32-row waves)
  static constexpr int WAVES = 8;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int KS = L::KS, NB = L::NB, CPR = L::CPR;
  static constexpr int TILE = L::TILE;          // bf16 elements of one K or V tile
  static constexpr int TI = kBK * CPR / 64;     // 1 KB DMA instructions per tile
  static constexpr int DPW = 2 * TI / WAVES;    // DMA instructions per wave per round
  static_assert(D == 64 || D == 128, "two-group forward: head dims 64 and 128");
  static_assert(!L::ROT, "XOR layouts only");
  static_assert(DPW >= 1 && DPW * WAVES == 2 * TI && TI % DPW == 0, "DMA split");
};

__device__ __forceinline__ void pp_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Maxima of scores by the plain instructions.  The compiler's fmaxf places a
// canonicalising v_max_f32 x, x before each operand it cannot prove
// canonical (every MFMA result and lane-swap value here); scores are never
// signalling NaNs, so those are pure latency on the softmax's dependent
// chain.
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float lane_vmax16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float lane_vmax32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Head dim 64: two workgroups per CU (four waves per SIMD, 120 registers,
// fragments one step ahead); head dim 128: one (190 registers).
template <int D>
__global__ void __launch_bounds__(PPShape<D>::THREADS, (D <= 64 ? 2 : 1))
attn_fwd_pp_kernel(const bf16_t* __restrict__ qkv, bf16_t* __restrict__ O, float* __restrict__ lse,
                   float* __restrict__ part, Plan p, int total_items) {
  using S = PPShape<D>;
  using L = typename S::L;
  // stage s: K tile at 2 s TILE, V tile at (2 s + 1) TILE
  __shared__ __attribute__((aligned(16))) bf16_t lds[kPPStages * 2 * S::TILE];

  const int item = total_items - 1 - (int)blockIdx.x;   // long chunks first, short blocks last
  const Item it = decode_item(p, item);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2;
  const int g = lane >> 4, r16 = lane & 15;
  const int zo = it.z / p.hs, zi = it.z - zo * p.hs;
  const bf16_t* Qh = qkv + (int64_t)zo * p.sq * p.ld + (int64_t)zi * D;
  const bf16_t* Kh = Qh + (int64_t)p.hs * D;
  const bf16_t* Vh = Kh + (int64_t)p.hs * D;
  const int q0 = it.i * kPPRows + wave * 32;   // first query row of this wave
  const int n = it.it1 - it.it0;                // key tiles of this item (>= 1)
  const int kb0 = it.it0 * kBK;

  const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16_t*)lds);

  // This wave's DMA instructions: tile instruction t fills slots t 64 .. +63
  // of the tile; slot q is row q / CPR, chunk position q % CPR, holding the
  // row's logical chunk position ^ swizzle.  The per-lane offsets are fixed;
  // rows past the sequence (last tile only) re-read the last row.
  const bool dmaV = wave * S::DPW >= S::TI;
  const bf16_t* dhead = dmaV ? Vh : Kh;
  int drow[S::DPW], dcol[S::DPW];
  uint32_t dvo[S::DPW], dlo[S::DPW];
#pragma unroll
  for (int i = 0; i < S::DPW; ++i) {
    const int t = wave * S::DPW + i - (dmaV ? S::TI : 0);
    const int q = t * 64 + lane;
    const int r = q / S::CPR, ph = q % S::CPR;
    drow[i] = r;
    dcol[i] = (ph ^ (dmaV ? L::vswz(r) : L::kswz(r))) * 16;
    dvo[i] = (uint32_t)((int64_t)r * p.ld * 2 + dcol[i]);
    dlo[i] = (uint32_t)((dmaV ? S::TILE * 2 : 0) + t * 64 * 16);
  }
  // round j's tiles: K(min(j, n-1)) and V(max(j-1, 0)) (the clamped ones are
  // never read) into stage `stage`
  auto issue = [&](int j, int stage) {
    const int tile = dmaV ? max(j - 1, 0) : min(j, n - 1);
    const int kb = kb0 + tile * kBK;
    const uint64_t sb = uniform_addr(dhead + (int64_t)kb * p.ld);
    const bool whole = kb + kBK <= p.sq;
    const uint32_t sbase = lds0 + (uint32_t)(stage * 2 * S::TILE * 2);
#pragma unroll
    for (int i = 0; i < S::DPW; ++i) {
      const uint32_t voff = whole ? dvo[i] : (uint32_t)((int64_t)min(drow[i], p.sq - 1 - kb) * p.ld * 2 + dcol[i]);
      const uint32_t m0 = sbase + dlo[i];
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                   :: "v"(voff), "s"(sb), "s"(m0) : "memory", "m0");
    }
  };

  issue(0, 0);
  issue(1, 1);

  // Q fragments of the wave's two 16-row blocks (rows past the sequence
  // re-read the last row; their results are not stored)
  bf16x8_t qf[2][S::KS];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int row = min(q0 + 16 * b + r16, p.sq - 1);
    const bf16_t* src = Qh + (int64_t)row * p.ld + 8 * g;
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) qf[b][ks] = *reinterpret_cast<const bf16x8_t*>(src + 32 * ks);
  }
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) loaded_here(qf[b][ks]);
  f32x4_t acc[2][S::NB];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int c = 0; c < S::NB; ++c) acc[b][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY};
  // row sums of P by the matrix pipe: ones (16 x 32) times P^T gives every
  // lane of query r16 the sum of that row's P over the tile's 32 keys
  f32x4_t lacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  f32x4_t s[2][2];                    // scores of the last S product: row 16 b + r16, keys 16 h + 4 g + e
  bf16x8_t pf[2] = {bf16x8_t{}, bf16x8_t{}};   // P of the last softmax, as the A operand of P V

  wait_vmem_known();
  pp_barrier();

  // keys of tile t all after the wave's last row: nothing to add
  auto live = [&](int t) { return !p.causal || kb0 + t * kBK <= q0 + 31; };

  // products of round j: O += P(j-1) V(j-1) (from round 1 on), then
  // S(j) = Q K(j)^T (up to round n - 1).  The first and last rounds are
  // peeled, so each instance is straight-line code that keeps the
  // accumulators in place; P is zero for a tile whose keys all follow the
  // wave's rows.
  auto products = [&](int stage, auto do_pv, auto do_s) {
    constexpr bool PV = decltype(do_pv)::value, SC = decltype(do_s)::value;
    // the product phase issues at raised priority, so that on its SIMD the
    // other group's softmax fills the issue slots the MFMAs leave free
    __builtin_amdgcn_s_setprio(1);
    const bf16_t* Kt = lds + stage * 2 * S::TILE;
    const bf16_t* Vt = Kt + S::TILE;
    const int vrow = 4 * g + (r16 >> 2);
    const bf16_t* vbase = Vt + (r16 & 1) * 4;
    auto vread = [&](int c) {
      const bf16_t* pl = vbase + L::voff(vrow, 2 * c + ((r16 & 3) >> 1));
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)pl);
      const s16x4_t hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(pl + 16 * L::PITCH));
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // K fragment of k-step x / 2, key half x % 2
    auto kread = [&](int x) {
      return *reinterpret_cast<const bf16x8_t*>(Kt + L::koff(16 * (x & 1) + r16, 4 * (x >> 1) + g));
    };
    // step x: the two P V MFMAs of column block x (if any) and the two S
    // MFMAs of k-step x / 2, key half x % 2, so that consecutive MFMAs on one
    // S accumulator are eight apart; the fragments of step x + 2 are read
    // during step x (x + 1 at head dim 64).  The row sums of P go first (their operands are in
    // registers).
    if constexpr (PV) {
#pragma unroll
      for (int b = 0; b < 2; ++b) lacc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[b], lacc[b], 0, 0, 0);
    }
    constexpr int NX = 2 * S::KS > S::NB ? 2 * S::KS : S::NB;
    constexpr int PF = D <= 64 ? 1 : 2;
    bf16x8_t vq[NX + PF], kq[NX + PF];
#pragma unroll
    for (int x = 0; x < PF; ++x) {
      if (PV && x < S::NB) vq[x] = vread(x);
      if (SC && x < 2 * S::KS) kq[x] = kread(x);
    }
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      if (PV && x + PF < S::NB) vq[x + PF] = vread(x + PF);
      if (SC && x + PF < 2 * S::KS) kq[x + PF] = kread(x + PF);
      if (PV && x < S::NB) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[b][x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vq[x], pf[b], acc[b][x], 0, 0, 0);
      }
      if (SC && x < 2 * S::KS) {
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};   // the first k-step starts the chains
#pragma unroll
        for (int b = 0; b < 2; ++b)
          s[b][x & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kq[x], qf[b][x >> 1], x < 2 ? zero : s[b][x & 1], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // softmax of tile t: S(t) -> P(t), moving the running max (and rescaling
  // O and the row sums) when a score exceeds it by more than kLazy
  auto softmax = [&](int t) {
    if (t < 0 || t >= n) return;
    if (!live(t)) {
      pf[0] = pf[1] = bf16x8_t{};
      return;
    }
    const int kb = kb0 + t * kBK;
    if (!(kb + kBK <= p.sq && (!p.causal || kb + kBK - 1 <= q0))) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
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
    // The row max moves only when a score exceeds it by more than kLazy, and
    // a row's max exceeds that bound exactly when one of its four lanes'
    // maxima does: the lanes compare their own maxima, and only when some
    // lane of the wave is over are the rows' maxima formed across lanes.
    float mx[2];
    bool over = false;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      mx[b] = vmax3(vmax3(s[b][0][0], s[b][0][1], s[b][0][2]), vmax3(s[b][0][3], s[b][1][0], s[b][1][1]),
                    vmax(s[b][1][2], s[b][1][3])) * p.scale_log2;
      over |= mx[b] > m[b] + kLazy;   // -inf + 8 = -inf: the first finite score moves it too
    }
    if (__ballot(over)) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const float mn = vmax(m[b], lane_vmax32(lane_vmax16(mx[b])));
        if (mn > m[b] + kLazy) {
          // m = -inf and a finite new max: alpha 0 (nothing accumulated yet)
          const float alpha = fast_exp2(m[b] - mn);
          lacc[b] *= alpha;
#pragma unroll
          for (int c = 0; c < S::NB; ++c) acc[b][c] *= alpha;
          m[b] = mn;
        }
      }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float sub = m[b] == -INFINITY ? 0.f : m[b];
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(fmaf(s[b][e >> 2][e & 3], p.scale_log2, -sub));
      pf[b] = __builtin_bit_cast(bf16x8_t, u32x4_t{cvt_bf16x2(pv[0], pv[1]), cvt_bf16x2(pv[2], pv[3]),
                                                   cvt_bf16x2(pv[4], pv[5]), cvt_bf16x2(pv[6], pv[7])});
    }
  };

  int stage = 0;         // stage of round j
  int stage2 = 2;        // stage of round j + 2
  // round j + 1's tiles landed (round j + 2's may still be in flight)
  auto round_end = [&](int j) {
    if (j + 2 <= n) wait_vmem_n<S::DPW>();
    else wait_vmem();
    pp_barrier();
  };
  const std::true_type yes{};
  const std::false_type no{};
  auto advance = [&]() {
    stage = stage == kPPStages - 1 ? 0 : stage + 1;
    stage2 = stage2 == kPPStages - 1 ? 0 : stage2 + 1;
  };
  // rounds 0 (S only), 1 .. n - 1, n (P V only); n >= 1
  if (grp == 0) {
    if (2 <= n) issue(2, stage2);
    products(stage, no, yes);
    pp_barrier();
    softmax(0);
    round_end(0);
    advance();
    for (int j = 1; j < n; ++j) {
      if (j + 2 <= n) issue(j + 2, stage2);
      products(stage, yes, yes);
      pp_barrier();
      softmax(j);
      round_end(j);
      advance();
    }
    products(stage, yes, no);
    pp_barrier();
    round_end(n);
  } else {
    if (2 <= n) issue(2, stage2);
    pp_barrier();
    products(stage, no, yes);
    round_end(0);
    advance();
    for (int j = 1; j < n; ++j) {
      if (j + 2 <= n) issue(j + 2, stage2);
      softmax(j - 1);
      pp_barrier();
      products(stage, yes, yes);
      round_end(j);
      advance();
    }
    softmax(n - 1);
    pp_barrier();
    products(stage, yes, no);
    round_end(n);
  }

  // row sums (every lane of a query holds its row's sum)
  float l[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) l[b] = lacc[b][0];
  if (it.C == 1) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int row = q0 + 16 * b + r16;
      if (row < p.sq) {
        const float inv = 1.f / l[b];
        bf16_t* dst = O + ((int64_t)zo * p.sq + row) * p.ldo + (int64_t)zi * D + 4 * g;
#pragma unroll
        for (int c = 0; c < S::NB; ++c) {
          const f32x4_t v = acc[b][c] * inv;
          *reinterpret_cast<u32x2_t*>(dst + 16 * c) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
        if (g == 0) lse[(int64_t)it.z * p.sq + row] = (m[b] + log2f(l[b])) * 0.69314718055994531f;
      }
    }
  } else {
    float* po = part + (int64_t)item * kPPRows * D;
    float* pml = part + (int64_t)total_items * kPPRows * D + (int64_t)item * kPPRows * 2;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int rl = wave * 32 + 16 * b + r16;
#pragma unroll
      for (int c = 0; c < S::NB; ++c) *reinterpret_cast<f32x4_t*>(po + rl * D + 16 * c + 4 * g) = acc[b][c];
      if (g == 0) {
        pml[2 * rl] = m[b];
        pml[2 * rl + 1] = l[b];
      }
    }
  }
}

}  // namespace flash
}  // namespace tps
