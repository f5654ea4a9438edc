// Dense GEMM kernels for gfx950: C(m,n) = sum_k A(m,k) B(k,n), fp32 accumulate,
// result handed to a fused epilogue functor.
//
// bf16 path: LDS-tiled MFMA kernel (v_mfma_f32_16x16x32_bf16), double-buffered
// LDS with register prefetch of the next K tile, XCD-aware tile order.  Both
// operands are staged in LDS "K-contiguous" ([row][k]) so every MFMA fragment
// is one 16-byte LDS read; an operand stored with M (or N) contiguous is
// transposed 8x8 in registers on its way from global memory to LDS.
//
// fp32 path: LDS-tiled SIMT kernel (4x4 outputs per thread), same epilogues.
#pragma once

#include "common.hpp"

namespace tps {

// Problem description shared by both paths.  Operand layout:
//   A K-contiguous: A(m,k) = A[m*lda + k]   else A(m,k) = A[k*lda + m]
//   B K-contiguous: B(k,n) = B[n*ldb + k]   else B(k,n) = B[k*ldb + n]
// Batched problems: z in [0, batch) splits as (z / batch_inner, z % batch_inner)
// and operand offsets are zo*s?_o + zi*s?_i elements.
struct GemmShape {
  int M = 0, N = 0, K = 0;
  int64_t lda = 0, ldb = 0;
  int batch = 1, batch_inner = 1;
  int64_t sa_o = 0, sa_i = 0, sb_o = 0, sb_i = 0;
  // Per-tile K range for triangular operands:
  //   kmode 0: [0, K)
  //   kmode 1: [0, min(K, m0 + BM))   A(m,k) == 0 for k > m
  //   kmode 2: [floor(m0/BK)*BK, K)   A(m,k) == 0 for k < m
  int kmode = 0;
  // skip_upper: tiles whose every column n exceeds every row m get acc = 0
  // (the epilogue still runs; it is expected to mask n > m itself).
  int skip_upper = 0;
  int group_m = 4;  // tile rows per group in the tile order
};

// ------------------------------------------------------------------ epilogues
// Each epilogue is called with (zo, zi, m, n, v[4], nvalid): the fp32 results
// of C(m, n..n+3), nvalid of which are inside the matrix.

template <typename T>
struct EpiStore {  // C = acc
  T* C;
  int64_t ldc, sc_o, sc_i;
  __device__ void operator()(int zo, int zi, int m, int n, float v[4], int nv) const {
    store4<T>(C + zo * sc_o + zi * sc_i + (int64_t)m * ldc + n, v, nv);
  }
};

template <typename T>
struct EpiGelu {  // P = acc, H = gelu(acc)
  T* P;
  T* H;
  int64_t ld;
  __device__ void operator()(int, int, int m, int n, float v[4], int nv) const {
    const int64_t o = (int64_t)m * ld + n;
    float g[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) g[i] = gelu_f(v[i]);
    store4<T>(P + o, v, nv);
    store4<T>(H + o, g, nv);
  }
};

template <typename T>
struct EpiGeluBwd {  // out = acc * gelu'(P)
  const T* P;
  T* out;
  int64_t ld;
  __device__ void operator()(int, int, int m, int n, float v[4], int nv) const {
    const int64_t o = (int64_t)m * ld + n;
    float p[4];
    load4<T>(P + o, p, nv);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] *= gelu_grad_f(p[i]);
    store4<T>(out + o, v, nv);
  }
};

// Attention probabilities recomputed from the saved log-sum-exp:
// P(m,n) = exp(acc*scale - lse[m]), 0 where causal masks n > m.  One batch
// entry per (batch, head); lse is laid out [b][hs][sq].
template <typename T>
struct EpiAttnProb {
  T* P;
  const float* lse;
  int64_t ldp, sp;  // P row stride and per-(b,head) stride
  int sq, hs, causal;
  float scale_log2;  // scale * log2(e)
  __device__ void operator()(int zo, int zi, int m, int n, float v[4], int nv) const {
    const int z = zo * hs + zi;
    const float l2 = lse[(int64_t)z * sq + m] * 1.4426950408889634f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool masked = causal && (n + i > m);
      v[i] = masked ? 0.f : exp2f(v[i] * scale_log2 - l2);
    }
    store4<T>(P + (int64_t)z * sp + (int64_t)m * ldp + n, v, nv);
  }
};

// dS(m,n) = P(m,n) * (acc - delta[m]) * scale, where acc = (dO V^T)(m,n).
template <typename T>
struct EpiAttnDS {
  const T* P;
  T* dS;
  const float* delta;
  int64_t ldp, sp;
  int sq, hs;
  float scale;
  __device__ void operator()(int zo, int zi, int m, int n, float v[4], int nv) const {
    const int z = zo * hs + zi;
    const int64_t o = (int64_t)z * sp + (int64_t)m * ldp + n;
    const float dl = delta[(int64_t)z * sq + m];
    float p[4];
    load4<T>(P + o, p, nv);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = p[i] * (v[i] - dl) * scale;
    store4<T>(dS + o, v, nv);
  }
};

// ------------------------------------------------------------------ tile order

// Maps a linear workgroup id to (problem z, tile row tm, tile col tn).
// Workgroups are dealt to the 8 XCDs round-robin (id % 8), so each XCD is
// given one contiguous run of the tile sequence; the sequence walks groups of
// `group_m` tile rows column by column, so one XCD's run is a compact block of
// tiles that shares A rows and B columns in that XCD's L2.
__device__ __forceinline__ void tile_coords(int wg, int total, int tiles_m, int tiles_n, int group_m,
                                            int& z, int& tm, int& tn) {
  const int xcd = wg & 7, local = wg >> 3;
  const int base = total >> 3, rem = total & 7;
  const int idx = xcd * base + (xcd < rem ? xcd : rem) + local;
  const int tiles = tiles_m * tiles_n;
  z = idx / tiles;
  const int t = idx - z * tiles;
  const int per_group = group_m * tiles_n;
  const int g = t / per_group;
  const int first = g * group_m;
  const int gs = min(tiles_m - first, group_m);
  const int r = t - g * per_group;
  tm = first + r % gs;
  tn = r / gs;
}

__device__ __forceinline__ void k_range(const GemmShape& s, int m0, int BM, int BK, int& kb, int& ke) {
  kb = 0;
  ke = s.K;
  if (s.kmode == 1) ke = min(s.K, m0 + BM);
  else if (s.kmode == 2) kb = min(s.K, (m0 / BK) * BK);
  if (ke < kb) ke = kb;
}

// ------------------------------------------------------------------ bf16 MFMA

__device__ __forceinline__ u32x4_t mask_vec8(u32x4_t v, int nvalid) {
  // zero bf16 elements [nvalid, 8)
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int e0 = 2 * w, e1 = 2 * w + 1;
    uint32_t keep = (e0 < nvalid ? 0x0000ffffu : 0u) | (e1 < nvalid ? 0xffff0000u : 0u);
    v[w] &= keep;
  }
  return v;
}

template <int BM, int BN, int BK, int WM, int WN>
struct MfmaCfg {
  static constexpr int NT = WM * WN * 64;
  static constexpr int PAD = 8;                 // bf16 elements of row padding in LDS
  static constexpr int LDK = BK + PAD;          // LDS row stride (elements)
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 16, FN = WTN / 16;
  static constexpr int KSTEPS = BK / 32;
  static constexpr int A_VECS = BM * BK / 8 / NT;  // 16-byte vectors per thread per tile
  static constexpr int B_VECS = BN * BK / 8 / NT;
  static constexpr int LDS_ELEMS = 2 * (BM + BN) * LDK;
  static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "wave tile");
  static_assert(BK % 32 == 0, "BK");
  static_assert(A_VECS >= 1 && B_VECS >= 1, "tile too small for thread count");
};

// Global -> register loader for one operand tile of R rows (m or n) x BK.
// KC = operand is K-contiguous in global memory.
template <int R, int BK, int NT, bool KC>
struct TileLoader {
  static constexpr int VECS = R * BK / 8 / NT;
  // For the transposed (MN-contiguous) case: blocks of 8 rows x KB k.
  static constexpr int EPT = R * BK / NT;                 // elements per thread
  static constexpr int KB = KC ? 8 : (EPT / 8 >= 8 ? 8 : EPT / 8);
  static constexpr int NBLK = KC ? 0 : EPT / (8 * KB);   // blocks per thread
  static_assert(KC || (KB == 2 || KB == 4 || KB == 8), "KB");
  static_assert(KC || NBLK * 8 * KB == EPT, "EPT");

  u32x4_t v[VECS];

  // p: operand base (already offset for the batch entry); r0/k0 tile origin;
  // R_total rows, K_total k extent, ld leading dimension.
  __device__ __forceinline__ void load(const bf16_t* __restrict__ p, int64_t ld, int r0, int k0,
                                       int R_total, int K_total, int tid) {
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < VECS; ++i) {
        const int c = tid + i * NT;
        const int row = c / (BK / 8), kc = (c % (BK / 8)) * 8;
        const int gr = r0 + row, gk = k0 + kc;
        u32x4_t x = {0u, 0u, 0u, 0u};
        if (gr < R_total && gk < K_total) {
          x = *reinterpret_cast<const u32x4_t*>(p + (int64_t)gr * ld + gk);
          if (gk + 8 > K_total) x = mask_vec8(x, K_total - gk);
        }
        v[i] = x;
      }
    } else {
#pragma unroll
      for (int b = 0; b < NBLK; ++b) {
        const int blk = tid + b * NT;
        const int rb = blk % (R / 8), kb = blk / (R / 8);
        const int gr = r0 + rb * 8;
#pragma unroll
        for (int j = 0; j < KB; ++j) {
          const int gk = k0 + kb * KB + j;
          u32x4_t x = {0u, 0u, 0u, 0u};
          if (gr < R_total && gk < K_total) {
            x = *reinterpret_cast<const u32x4_t*>(p + (int64_t)gk * ld + gr);
            if (gr + 8 > R_total) x = mask_vec8(x, R_total - gr);
          }
          v[b * KB + j] = x;
        }
      }
    }
  }

  // Register -> LDS (layout [row][LDK], K contiguous).
  template <int LDK>
  __device__ __forceinline__ void store(bf16_t* lds, int tid) const {
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < VECS; ++i) {
        const int c = tid + i * NT;
        const int row = c / (BK / 8), kc = (c % (BK / 8)) * 8;
        *reinterpret_cast<u32x4_t*>(lds + row * LDK + kc) = v[i];
      }
    } else {
#pragma unroll
      for (int b = 0; b < NBLK; ++b) {
        const int blk = tid + b * NT;
        const int rb = blk % (R / 8), kb = blk / (R / 8);
        // v[b*KB + j] holds row-elements rb*8..rb*8+7 at k = kb*KB + j.
        // Output row i needs element i of each of the KB vectors.
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int w = i >> 1;
          const bool hi = i & 1;
          uint32_t out[KB / 2];
#pragma unroll
          for (int q = 0; q < KB / 2; ++q) {
            const uint32_t a = v[b * KB + 2 * q][w], c = v[b * KB + 2 * q + 1][w];
            out[q] = hi ? ((a >> 16) | (c & 0xffff0000u)) : ((a & 0xffffu) | (c << 16));
          }
          bf16_t* dst = lds + (rb * 8 + i) * LDK + kb * KB;
          if constexpr (KB == 8) {
            u32x4_t o = {out[0], out[1], out[2], out[3]};
            *reinterpret_cast<u32x4_t*>(dst) = o;
          } else if constexpr (KB == 4) {
            u32x2_t o = {out[0], out[1]};
            *reinterpret_cast<u32x2_t*>(dst) = o;
          } else {
            *reinterpret_cast<uint32_t*>(dst) = out[0];
          }
        }
      }
    }
  }
};

template <int BM, int BN, int BK, int WM, int WN, bool AK, bool BKC, class Epi>
__global__ void __launch_bounds__(WM * WN * 64, 1)
gemm_bf16_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, GemmShape s, Epi epi) {
  using C = MfmaCfg<BM, BN, BK, WM, WN>;
  __shared__ __attribute__((aligned(16))) bf16_t lds[C::LDS_ELEMS];

  const int tiles_m = (s.M + BM - 1) / BM, tiles_n = (s.N + BN - 1) / BN;
  const int total = tiles_m * tiles_n * s.batch;
  if ((int)blockIdx.x >= total) return;
  int z, tm, tn;
  tile_coords(blockIdx.x, total, tiles_m, tiles_n, s.group_m, z, tm, tn);
  const int zo = z / s.batch_inner, zi = z - zo * s.batch_inner;
  const int m0 = tm * BM, n0 = tn * BN;
  const bf16_t* Ab = A + zo * s.sa_o + zi * s.sa_i;
  const bf16_t* Bb = B + zo * s.sb_o + zi * s.sb_i;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;

  int kb, ke;
  k_range(s, m0, BM, BK, kb, ke);
  if (s.skip_upper && n0 > m0 + BM - 1) ke = kb;
  const int nk = (ke - kb + BK - 1) / BK;

  f32x4_t acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  TileLoader<BM, BK, C::NT, AK> la;
  TileLoader<BN, BK, C::NT, BKC> lb;
  // LDS stage st holds A at lds + st*(BM+BN)*LDK and B right after it.
  auto lds_a = [&](int stage) { return lds + stage * (BM + BN) * C::LDK; };
  auto lds_b = [&](int stage) { return lds + stage * (BM + BN) * C::LDK + BM * C::LDK; };

  if (nk > 0) {
    la.load(Ab, s.lda, m0, kb, s.M, s.K, tid);
    lb.load(Bb, s.ldb, n0, kb, s.N, s.K, tid);
    la.template store<C::LDK>(lds_a(0), tid);
    lb.template store<C::LDK>(lds_b(0), tid);
    __syncthreads();
  }

  const int frag_row = lane & 15, frag_k = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int k0 = kb + (kt + 1) * BK;
      la.load(Ab, s.lda, m0, k0, s.M, s.K, tid);
      lb.load(Bb, s.ldb, n0, k0, s.N, s.K, tid);
    }
    const bf16_t* sa = lds_a(cur) + (wm * C::WTM + frag_row) * C::LDK + frag_k;
    const bf16_t* sb = lds_b(cur) + (wn * C::WTN + frag_row) * C::LDK + frag_k;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      bf16x8_t af[C::FM], bfr[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(sa + i * 16 * C::LDK + ks * 32);
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(sb + j * 16 * C::LDK + ks * 32);
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (more) {
      la.template store<C::LDK>(lds_a(cur ^ 1), tid);
      lb.template store<C::LDK>(lds_b(cur ^ 1), tid);
    }
    __syncthreads();
  }

  // acc[i][j] lane layout (operands swapped above): element e of lane l is
  // C(m = .. + (l & 15), n = .. + 4*(l >> 4) + e).
  const int em = lane & 15, en = (lane >> 4) * 4;
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const int m = m0 + wm * C::WTM + i * 16 + em;
    if (m >= s.M) continue;
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int n = n0 + wn * C::WTN + j * 16 + en;
      if (n >= s.N) continue;
      float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      epi(zo, zi, m, n, v, min(4, s.N - n));
    }
  }
}

// ------------------------------------------------------------------ fp32 SIMT

template <bool AK, bool BKC, class Epi>
__global__ void __launch_bounds__(256)
gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ B, GemmShape s, Epi epi) {
  constexpr int BM = 64, BN = 64, BKf = 16;
  __shared__ float as[BKf][BM + 4];
  __shared__ float bs[BKf][BN + 4];
  const int tiles_m = (s.M + BM - 1) / BM, tiles_n = (s.N + BN - 1) / BN;
  const int total = tiles_m * tiles_n * s.batch;
  if ((int)blockIdx.x >= total) return;
  int z, tm, tn;
  tile_coords(blockIdx.x, total, tiles_m, tiles_n, s.group_m, z, tm, tn);
  const int zo = z / s.batch_inner, zi = z - zo * s.batch_inner;
  const int m0 = tm * BM, n0 = tn * BN;
  const float* Ab = A + zo * s.sa_o + zi * s.sa_i;
  const float* Bb = B + zo * s.sb_o + zi * s.sb_i;
  const int tid = threadIdx.x, tr = tid / 16, tc = tid % 16;
  int kb, ke;
  k_range(s, m0, BM, BKf, kb, ke);
  if (s.skip_upper && n0 > m0 + BM - 1) ke = kb;
  float acc[4][4] = {};
  for (int k0 = kb; k0 < ke; k0 += BKf) {
    for (int e = tid; e < BM * BKf; e += 256) {
      const int mm = AK ? e / BKf : e % BM, kk = AK ? e % BKf : e / BM;
      const int gm = m0 + mm, gk = k0 + kk;
      float x = 0.f;
      if (gm < s.M && gk < s.K) x = AK ? Ab[(int64_t)gm * s.lda + gk] : Ab[(int64_t)gk * s.lda + gm];
      as[kk][mm] = x;
    }
    for (int e = tid; e < BN * BKf; e += 256) {
      const int nn = BKC ? e / BKf : e % BN, kk = BKC ? e % BKf : e / BN;
      const int gn = n0 + nn, gk = k0 + kk;
      float x = 0.f;
      if (gn < s.N && gk < s.K) x = BKC ? Bb[(int64_t)gn * s.ldb + gk] : Bb[(int64_t)gk * s.ldb + gn];
      bs[kk][nn] = x;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BKf; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = as[kk][tr * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = bs[kk][tc * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  const int n = n0 + tc * 4;
  if (n >= s.N) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + tr * 4 + i;
    if (m < s.M) epi(zo, zi, m, n, acc[i], min(4, s.N - n));
  }
}

// ------------------------------------------------------------------ dispatch

template <int BM, int BN, int BK, int WM, int WN, bool AK, bool BKC, class Epi>
inline tps_status launch_mfma(const bf16_t* A, const bf16_t* B, const GemmShape& s, const Epi& epi,
                              hipStream_t st) {
  const int64_t tiles = ceil_div(s.M, BM) * ceil_div(s.N, BN) * (int64_t)s.batch;
  if (tiles == 0) return TPS_OK;
  if (tiles > 0x7fffffff) return set_error(TPS_EINVAL, "gemm: too many tiles");
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, WM, WN, AK, BKC, Epi>), dim3((unsigned)tiles),
                     dim3(WM * WN * 64), 0, st, A, B, s, epi);
  return check_launch("gemm_bf16_kernel");
}

// Picks a tile shape for the problem: 256x256 when that fills the chip,
// otherwise a smaller tile so that the launch has enough workgroups.
template <bool AK, bool BKC, class Epi>
inline tps_status gemm_bf16(const bf16_t* A, const bf16_t* B, const GemmShape& s, const Epi& epi,
                            hipStream_t st) {
  const int64_t big = ceil_div(s.M, 256) * ceil_div(s.N, 256) * (int64_t)s.batch;
  if (big >= 240) return launch_mfma<256, 256, 64, 2, 2, AK, BKC>(A, B, s, epi, st);
  const int64_t mid = ceil_div(s.M, 128) * ceil_div(s.N, 128) * (int64_t)s.batch;
  if (mid >= 200) return launch_mfma<128, 128, 64, 2, 2, AK, BKC>(A, B, s, epi, st);
  return launch_mfma<64, 64, 64, 2, 2, AK, BKC>(A, B, s, epi, st);
}

template <bool AK, bool BKC, class Epi>
inline tps_status gemm_f32(const float* A, const float* B, const GemmShape& s, const Epi& epi,
                           hipStream_t st) {
  const int64_t tiles = ceil_div(s.M, 64) * ceil_div(s.N, 64) * (int64_t)s.batch;
  if (tiles == 0) return TPS_OK;
  hipLaunchKernelGGL((gemm_f32_kernel<AK, BKC, Epi>), dim3((unsigned)tiles), dim3(256), 0, st, A, B,
                     s, epi);
  return check_launch("gemm_f32_kernel");
}

}  // namespace tps
