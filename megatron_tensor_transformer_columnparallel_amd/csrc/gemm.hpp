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
// Each epilogue is called with (zo, zi, m, n, v[8], nvalid): the fp32 results
// of C(m, n..n+7), nvalid of which are inside the matrix; n is a multiple of 8.

template <typename T>
struct EpiStore {  // C = acc
  T* C;
  int64_t ldc, sc_o, sc_i;
  __device__ void operator()(int zo, int zi, int m, int n, float v[8], int nv) const {
    store8<T>(C + zo * sc_o + zi * sc_i + (int64_t)m * ldc + n, v, nv);
  }
};

template <typename T>
struct EpiGelu {  // P = acc, H = gelu(acc)
  T* P;
  T* H;
  int64_t ld;
  __device__ void operator()(int, int, int m, int n, float v[8], int nv) const {
    const int64_t o = (int64_t)m * ld + n;
    float g[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) g[i] = gelu_f(v[i]);
    store8<T>(P + o, v, nv);
    store8<T>(H + o, g, nv);
  }
};

template <typename T>
struct EpiGeluBwd {  // out = acc * gelu'(P)
  const T* P;
  T* out;
  int64_t ld;
  __device__ void operator()(int, int, int m, int n, float v[8], int nv) const {
    const int64_t o = (int64_t)m * ld + n;
    float p[8];
    load8<T>(P + o, p, nv);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= gelu_grad_f(p[i]);
    store8<T>(out + o, v, nv);
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
  __device__ void operator()(int zo, int zi, int m, int n, float v[8], int nv) const {
    const int z = zo * hs + zi;
    const float l2 = lse[(int64_t)z * sq + m] * 1.4426950408889634f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool masked = causal && (n + i > m);
      v[i] = masked ? 0.f : exp2f(v[i] * scale_log2 - l2);
    }
    store8<T>(P + (int64_t)z * sp + (int64_t)m * ldp + n, v, nv);
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

// LDS layout: each operand tile is [rows][BK=64] bf16 with no padding; the
// eight 16-byte chunks of row r are stored XOR-swizzled (chunk c at position
// c ^ (r & 7)).  MFMA fragment reads (8 consecutive lanes = 8 consecutive rows,
// same chunk) and the loaders' 16-byte stores then hit 8 distinct bank groups.
__device__ __forceinline__ int lds_swizzle(int row) { return row & 7; }

// Global -> register -> LDS loader for one operand tile of R rows (m or n)
// by BK.  KC: the operand is K-contiguous in global memory (one 16-byte
// vector = 8 consecutive k of one row).  Otherwise it is M/N-contiguous and
// each thread loads an 8-row x KB-k block and transposes it in registers;
// consecutive lanes take consecutive k-blocks so that their LDS stores land
// in distinct banks.  Each thread walks a pointer through K; the unchecked
// load is used for interior tiles, the checked one zero-fills past M/N/K.
template <int R, int BK, int NT, bool KC>
struct TileLoader {
  static constexpr int VECS = R * BK / 8 / NT;
  static constexpr int EPT = R * BK / NT;
  static constexpr int KB = KC ? 8 : (EPT / 8 >= 8 ? 8 : EPT / 8);
  static constexpr int NBLK = KC ? 0 : EPT / (8 * KB);
  static constexpr int KBLKS = BK / KB;
  static constexpr int ROWS_PER_PASS = NT / (BK / 8);  // KC: rows covered by one vector per thread
  static_assert(BK == 64, "the swizzle assumes 8 chunks per row");
  static_assert(KC || (KB == 2 || KB == 4 || KB == 8), "KB");
  static_assert(KC || NBLK * 8 * KB == EPT, "EPT");
  static_assert(VECS >= 1, "tile too small for the thread count");

  u32x4_t v[VECS];
  const bf16_t* ptr;  // this thread's first element of the next tile
  int64_t step, ld;
  int gr0, gk0;       // global row / k of this thread's first vector in tile 0

  __device__ __forceinline__ void init(const bf16_t* p, int64_t ld_, int r0, int k0, int tid) {
    ld = ld_;
    if constexpr (KC) {
      gr0 = r0 + tid / (BK / 8);
      gk0 = k0 + (tid % (BK / 8)) * 8;
      ptr = p + (int64_t)gr0 * ld + gk0;
      step = BK;
    } else {
      gr0 = r0 + (tid / KBLKS) * 8;
      gk0 = k0 + (tid % KBLKS) * KB;
      ptr = p + (int64_t)gk0 * ld + gr0;
      step = (int64_t)BK * ld;
    }
  }

  __device__ __forceinline__ void load_fast() {
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < VECS; ++i)
        v[i] = *reinterpret_cast<const u32x4_t*>(ptr + (int64_t)i * ROWS_PER_PASS * ld);
    } else {
#pragma unroll
      for (int b = 0; b < NBLK; ++b)
#pragma unroll
        for (int j = 0; j < KB; ++j)
          v[b * KB + j] = *reinterpret_cast<const u32x4_t*>(ptr + (int64_t)j * ld + b * (NT / KBLKS) * 8);
    }
    ptr += step;
  }

  // kt: index of the tile being loaded (relative to the first).
  __device__ __forceinline__ void load_checked(int R_total, int K_total, int kt) {
    const int dk = kt * BK;
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < VECS; ++i) {
        const int gr = gr0 + i * ROWS_PER_PASS, gk = gk0 + dk;
        u32x4_t x = {0u, 0u, 0u, 0u};
        if (gr < R_total && gk < K_total) {
          x = *reinterpret_cast<const u32x4_t*>(ptr + (int64_t)i * ROWS_PER_PASS * ld);
          if (gk + 8 > K_total) x = mask_vec8(x, K_total - gk);
        }
        v[i] = x;
      }
    } else {
#pragma unroll
      for (int b = 0; b < NBLK; ++b) {
        const int gr = gr0 + b * (NT / KBLKS) * 8;
#pragma unroll
        for (int j = 0; j < KB; ++j) {
          const int gk = gk0 + dk + j;
          u32x4_t x = {0u, 0u, 0u, 0u};
          if (gr < R_total && gk < K_total) {
            x = *reinterpret_cast<const u32x4_t*>(ptr + (int64_t)j * ld + b * (NT / KBLKS) * 8);
            if (gr + 8 > R_total) x = mask_vec8(x, R_total - gr);
          }
          v[b * KB + j] = x;
        }
      }
    }
    ptr += step;
  }

  __device__ __forceinline__ void store(bf16_t* lds, int tid) const {
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < VECS; ++i) {
        const int row = tid / (BK / 8) + i * ROWS_PER_PASS, kc = tid % (BK / 8);
        *reinterpret_cast<u32x4_t*>(lds + row * BK + ((kc ^ lds_swizzle(row)) * 8)) = v[i];
      }
    } else {
#pragma unroll
      for (int b = 0; b < NBLK; ++b) {
        const int kb = tid % KBLKS, rb = tid / KBLKS + b * (NT / KBLKS);
        // v[b*KB + j] holds rows rb*8..rb*8+7 at k = kb*KB + j; output row i
        // gathers element i of each of the KB vectors.
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
          const int row = rb * 8 + i;
          const int e = kb * KB;
          bf16_t* dst = lds + row * BK + (((e >> 3) ^ lds_swizzle(row)) * 8) + (e & 7);
          if constexpr (KB == 8) *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{out[0], out[1], out[2], out[3]};
          else if constexpr (KB == 4) *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{out[0], out[1]};
          else *reinterpret_cast<uint32_t*>(dst) = out[0];
        }
      }
    }
  }
};

// One workgroup computes a BM x BN tile with WM x WN waves, each wave a
// (BM/WM) x (BN/WN) block of 16x16 MFMA tiles, K in steps of BK = 64 through
// two LDS stages: while the MFMAs consume stage k, the loads of tile k+1 are
// in flight to registers and land in the other stage at the end of the step.
template <int BM, int BN, int BK, int WM, int WN, bool AK, bool BKC, class Epi>
__global__ void __launch_bounds__(WM * WN * 64, 1)
gemm_bf16_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, GemmShape s, Epi epi) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int KS = BK / 32;
  constexpr int STAGE = (BM + BN) * BK;                 // bf16 elements per LDS stage
  constexpr int BAND_BYTES = WTM * (BN + 4) * 4;        // fp32 epilogue band
  constexpr int LDS_BYTES = 4 * STAGE > BAND_BYTES ? 4 * STAGE : BAND_BYTES;
  static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "wave tile");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) bf16_t lds[LDS_BYTES / 2];

  const int tiles_m = (s.M + BM - 1) / BM, tiles_n = (s.N + BN - 1) / BN;
  const int total = tiles_m * tiles_n * s.batch;
  if ((int)blockIdx.x >= total) return;
  int z, tm, tn;
  tile_coords(blockIdx.x, total, tiles_m, tiles_n, s.group_m, z, tm, tn);
  const int zo = z / s.batch_inner, zi = z - zo * s.batch_inner;
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;

  int kb, ke;
  k_range(s, m0, BM, BK, kb, ke);
  if (s.skip_upper && n0 > m0 + BM - 1) ke = kb;
  const int nk = (ke - kb + BK - 1) / BK;
  const bool full = (m0 + BM <= s.M) && (n0 + BN <= s.N) && ((ke - kb) % BK == 0);

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  TileLoader<BM, BK, NT, AK> la;
  TileLoader<BN, BK, NT, BKC> lb;
  la.init(A + zo * s.sa_o + zi * s.sa_i, s.lda, m0, kb, tid);
  lb.init(B + zo * s.sb_o + zi * s.sb_i, s.ldb, n0, kb, tid);

  // Fragment of a 16x16x32 MFMA: lane reads row (lane & 15) of its 16-row
  // block, chunk ks*4 + (lane >> 4) (8 consecutive k).
  const int fr = lane & 15, fg = lane >> 4;
  const int ra = wm * WTM + fr, rb = wn * WTN + fr;
  int offa[KS], offb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    offa[ks] = ra * BK + (((ks * 4 + fg) ^ lds_swizzle(ra)) * 8);
    offb[ks] = BM * BK + rb * BK + (((ks * 4 + fg) ^ lds_swizzle(rb)) * 8);
  }

  auto compute = [&](const bf16_t* st) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const bf16x8_t*>(st + offa[ks] + i * 16 * BK);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = *reinterpret_cast<const bf16x8_t*>(st + offb[ks] + j * 16 * BK);
      // operands swapped: the result's lane layout is C(m = lane & 15, n = 4*(lane >> 4) + e)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
  };

  if (nk > 0) {
    if (full) { la.load_fast(); lb.load_fast(); }
    else { la.load_checked(s.M, s.K, 0); lb.load_checked(s.N, s.K, 0); }
    la.store(lds, tid);
    lb.store(lds + BM * BK, tid);
    __syncthreads();
  }
  if (full) {
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) { la.load_fast(); lb.load_fast(); }
      compute(lds + cur * STAGE);
      if (more) {
        bf16_t* nx = lds + (cur ^ 1) * STAGE;
        la.store(nx, tid);
        lb.store(nx + BM * BK, tid);
      }
      __syncthreads();
    }
  } else {
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) { la.load_checked(s.M, s.K, kt + 1); lb.load_checked(s.N, s.K, kt + 1); }
      compute(lds + cur * STAGE);
      if (more) {
        bf16_t* nx = lds + (cur ^ 1) * STAGE;
        la.store(nx, tid);
        lb.store(nx + BM * BK, tid);
      }
      __syncthreads();
    }
  }

  // Epilogue staged through LDS (free after the K-loop's last barrier): one
  // band of wave-rows at a time writes its accumulators as fp32, then the
  // whole workgroup applies the epilogue to 8 consecutive columns per thread
  // with 16-byte accesses.
  float* band_buf = reinterpret_cast<float*>(lds);
  constexpr int SLD = BN + 4;
  const int em = lane & 15, en = (lane >> 4) * 4;
#pragma unroll
  for (int band = 0; band < WM; ++band) {
    if (wm == band) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          *reinterpret_cast<f32x4_t*>(band_buf + (i * 16 + em) * SLD + wn * WTN + j * 16 + en) = acc[i][j];
    }
    __syncthreads();
    constexpr int CHUNKS = WTM * BN / 8;
    for (int c = tid; c < CHUNKS; c += NT) {
      const int r = c / (BN / 8), cc = (c % (BN / 8)) * 8;
      const int m = m0 + band * WTM + r, n = n0 + cc;
      if (m < s.M && n < s.N) {
        const f32x4_t a = *reinterpret_cast<const f32x4_t*>(band_buf + r * SLD + cc);
        const f32x4_t b = *reinterpret_cast<const f32x4_t*>(band_buf + r * SLD + cc + 4);
        float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        epi(zo, zi, m, n, v, min(8, s.N - n));
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ fp32 SIMT

template <bool AK, bool BKC, class Epi>
__global__ void __launch_bounds__(256)
gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ B, GemmShape s, Epi epi) {
  // 64 x 128 tile, 256 threads, each 4 rows x 8 consecutive columns.
  constexpr int BM = 64, BN = 128, BKf = 16;
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
  float acc[4][8] = {};
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
      float a[4], b[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = as[kk][tr * 4 + i];
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = bs[kk][tc * 8 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  const int n = n0 + tc * 8;
  if (n >= s.N) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + tr * 4 + i;
    if (m < s.M) epi(zo, zi, m, n, acc[i], min(8, s.N - n));
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

// Tile shape by problem size (measured on MI355X): 256x256 with 8 waves
// (2 per SIMD) when it yields at least 3/4 of a wave of workgroups per CU,
// else 128x128 with 4 waves (two workgroups per CU), else 64x64.
template <bool AK, bool BKC, class Epi>
inline tps_status gemm_bf16(const bf16_t* A, const bf16_t* B, const GemmShape& s, const Epi& epi,
                            hipStream_t st) {
  const int64_t big = ceil_div(s.M, 256) * ceil_div(s.N, 256) * (int64_t)s.batch;
  if (big >= 192) return launch_mfma<256, 256, 64, 2, 4, AK, BKC>(A, B, s, epi, st);
  const int64_t mid = ceil_div(s.M, 128) * ceil_div(s.N, 128) * (int64_t)s.batch;
  if (mid >= 192) return launch_mfma<128, 128, 64, 2, 2, AK, BKC>(A, B, s, epi, st);
  return launch_mfma<64, 64, 64, 2, 2, AK, BKC>(A, B, s, epi, st);
}

template <bool AK, bool BKC, class Epi>
inline tps_status gemm_f32(const float* A, const float* B, const GemmShape& s, const Epi& epi,
                           hipStream_t st) {
  const int64_t tiles = ceil_div(s.M, 64) * ceil_div(s.N, 128) * (int64_t)s.batch;
  if (tiles == 0) return TPS_OK;
  hipLaunchKernelGGL((gemm_f32_kernel<AK, BKC, Epi>), dim3((unsigned)tiles), dim3(256), 0, st, A, B,
                     s, epi);
  return check_launch("gemm_f32_kernel");
}

}  // namespace tps
