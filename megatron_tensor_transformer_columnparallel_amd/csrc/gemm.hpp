// Dense GEMM kernels for gfx950: C(m,n) = sum_k A(m,k) B(k,n), fp32 accumulate,
// result handed to a fused epilogue functor.
//
// bf16 path: LDS-tiled MFMA kernel (v_mfma_f32_16x16x32_bf16), multi-stage
// LDS fed by direct global -> LDS loads (registers only for a ragged last K
// tile), XCD-aware tile order.  Each operand keeps its global orientation in LDS;
// fragments of an M/N-contiguous operand come out of the LDS transpose read.
//
// fp32 path: LDS-tiled SIMT kernel (4x4 outputs per thread), same epilogues.
#pragma once

#include <type_traits>

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
  // With skip_upper and skip_pad > 0, a tile whose first column is at or
  // beyond round_up(row + 1, skip_pad) for every one of its rows does nothing
  // at all (no epilogue): an output that only has to be written up to that
  // limit (1: the diagonal; 256: a zero pad to the next multiple of 256).
  int skip_pad = 0;
  // live_tiles: with skip_upper and skip_pad > 0, the tile shape is chosen by
  // the tiles that compute rather than by the whole grid (for an epilogue
  // heavy enough that every CU should share it; see gemm_bf16).
  int live_tiles = 0;
  int group_m = 8;  // tile rows per group in the tile order (8 measured best for M = 2048)
  // groups = 2: a second problem (GemmAlt) with this same shape, layout,
  // batch and K ranges runs in the same launch.
  int groups = 1;
  // lpt: tiles are issued longest K range first (kmode 1: last tile row
  // first; kmode 2: first tile row first), ranks outermost and then group,
  // batch entry and tile column, so every XCD gets the same mix of lengths
  // and short tiles fill the CUs that long tiles leave idle.
  int lpt = 0;
  // Output coordinates of this problem's (0, 0): the epilogue sees
  // (m + m_base, n + n_base), so a problem can be one part of a larger
  // output (the tail split below).
  int m_base = 0, n_base = 0;
};

// The second problem of a grouped launch: its own operands, strides and
// epilogue; everything else comes from the GemmShape.
template <class Epi>
struct GemmAlt {
  const bf16_t* A;
  const bf16_t* B;
  int64_t lda, ldb, sa_o, sa_i, sb_o, sb_i;
  Epi epi;
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

// LDS layout of one operand tile (BK = 64), as a linear array of 16-byte
// chunks ("slots"):
//   K-contiguous operand: [R rows][64 k], 8 chunks per row; chunk c of row r
//     sits at position c ^ (r & 7).  An MFMA fragment (8 consecutive lanes =
//     8 consecutive rows, same chunk) is one 16-byte read per lane spread
//     over 8 distinct bank groups.
//   M/N-contiguous operand: [64 k][R], R/8 chunks per k-row; chunk c of k-row
//     k sits at position c ^ mn_swizzle<R>(k).  A fragment is read with two
//     ds_read_b64_tr_b16 (transposing 4 k-rows x 16 columns per 16-lane
//     group); the swizzle sends the 8 k-rows that a half-wave touches to 8
//     distinct pairs of bank groups.
// Slot q of either layout holds row q / CPR at position q % CPR, so a wave
// fills 64 consecutive slots with one instruction: global_load_lds_dwordx4
// (lane l lands at LDS base + 16 l) for interior tiles, or 16-byte register
// stores after bounds-checked loads at the edges.
// K-contiguous rows of CPR chunks: 8 consecutive rows reading the same chunk
// land in 8 distinct 16-byte slots of a 128-byte bank window.
template <int CPR>
__device__ __forceinline__ int kc_swizzle(int row) {
  if constexpr (CPR == 8) return row & 7;
  else return (row >> 1) & 3;   // two 64-byte rows per window
}

template <int R>
__device__ __forceinline__ int mn_swizzle(int k) {
  // R = 128, 256: 16-chunk windows.  Other widths (64, 192) stay inside
  // aligned groups of 8 chunks, so the XOR never leaves the row.
  if constexpr (R % 128 == 0) return 2 * ((k & 3) | ((k >> 1) & 4));
  else return 2 * (((k >> 1) & 1) | ((k >> 2) & 2));
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem_n() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

// Loader of one operand tile of R rows (m or n) by BK (32 or 64).  Each
// thread owns VECS slots (tid + i*NT); all of them share one global column
// offset, so a single pointer walks through K.
template <int R, int NT, bool KC, int BK>
struct OperandLoader {
  static constexpr int CPR = KC ? BK / 8 : R / 8;   // 16-byte chunks per LDS row
  static constexpr int VECS = R * BK / 8 / NT;      // slots per thread
  static constexpr int PERIOD = KC ? 8 : 16;        // rows after which the swizzle repeats
  // Regular layout: a thread's slots sit RSTEP = NT / CPR rows apart, either
  // all at one swizzled column (RSTEP a multiple of the period) or
  // alternating between two (half of it).  Otherwise (a row of chunks that
  // does not divide the thread count, e.g. 24 for a 192-wide M/N-contiguous
  // tile) each slot keeps its own offset.
  static constexpr bool REG = NT % CPR == 0 && (2 * (NT / CPR)) % PERIOD == 0;
  static constexpr int RSTEP = REG ? NT / CPR : 1;
  static constexpr bool ALT = REG && RSTEP % PERIOD != 0;
  static_assert(VECS >= 1 && VECS * NT * 8 == R * BK, "operand tile vs thread count");
  static_assert(KC || R >= 64, "M/N-contiguous tiles need at least 8 chunks per k-row");
  static_assert(REG || !KC, "K-contiguous tiles always have the regular layout");

  u32x4_t v[VECS];
  const bf16_t* base;    // tile origin (row r0, current K tile) -- the same for every lane
  uint32_t voff;         // regular: bytes from `base` to this thread's first slot
  uint32_t istep;        // regular: bytes between the thread's slots
  uint32_t goff[REG ? 1 : VECS];   // irregular: bytes from `base` to each slot
  uint32_t rowb;         // regular: bytes per source row
  int rv;                // regular, KC: last row inside the operand (same for every lane); later slots re-read it
  int64_t kstep;         // elements between K tiles
  int row0;              // regular, KC: m/n row of the first slot; else its k row
  int col[2];            // regular, KC: k column, else m/n column, of even and odd slots

  static __device__ __forceinline__ int swz(int row) {
    if constexpr (KC) return kc_swizzle<CPR>(row);
    else return mn_swizzle<R>(row);
  }
  // LDS row and (swizzled) column of slot i of this thread
  static __device__ __forceinline__ int slot_row_of(int q) { return q / CPR; }
  static __device__ __forceinline__ int slot_col_of(int q) { return ((q % CPR) ^ swz(q / CPR)) * 8; }
  __device__ __forceinline__ int slot_col(int i) const { return (ALT && (i & 1)) ? col[1] : col[0]; }
  // byte offset of slot i from `base`
  __device__ __forceinline__ uint32_t slot_off(int i) const {
    if constexpr (REG) {
      const uint32_t alt = (ALT && (i & 1)) ? (uint32_t)(col[1] - col[0]) * 2u : 0u;
      if constexpr (KC) return voff + (uint32_t)((min(row0 + i * RSTEP, rv) - row0) * (int)rowb) + alt;
      else return voff + (uint32_t)i * istep + alt;
    } else {
      return goff[i];
    }
  }

  // ld * rows of the tile * 2 bytes must stay below 2^32, and ld a multiple
  // of 8 (checked on the host).  A tile with only r_valid < R of its rows
  // (K-contiguous) or columns (M/N-contiguous) inside the operand still takes
  // the direct path for full K tiles: K-contiguous slots past the end re-read
  // the last row; M/N-contiguous chunks past the end re-read the chunk that
  // holds the last element (a chunk that straddles the end reads at most 7
  // elements beyond it, inside the row since ld is a multiple of 8).  The
  // values read for missing rows or columns only reach outputs the epilogue
  // drops.
  __device__ __forceinline__ void init(const bf16_t* p, int64_t ld, int r0, int k0, int tid, int r_valid = R) {
    if constexpr (KC) {
      base = p + (int64_t)r0 * ld + k0;
      kstep = BK;
    } else {
      base = p + (int64_t)k0 * ld + r0;
      kstep = (int64_t)BK * ld;
    }
    const int cmax = ((min(r_valid, R) - 1) / 8) * 8;   // M/N-contiguous: last chunk with a valid element
    if constexpr (REG) {
      const int row = tid / CPR, pos = tid % CPR;
      row0 = row;
      col[0] = (pos ^ swz(row)) * 8;
      col[1] = (pos ^ swz(row + RSTEP)) * 8;
      if constexpr (!KC) {
        col[0] = min(col[0], cmax);
        col[1] = min(col[1], cmax);
      }
      voff = (uint32_t)(((int64_t)row * ld + col[0]) * 2);
      istep = (uint32_t)(RSTEP * ld * 2);
      rowb = (uint32_t)(ld * 2);
      rv = (r_valid < R ? r_valid : R) - 1;
    } else {
      row0 = 0;
      col[0] = col[1] = 0;
#pragma unroll
      for (int i = 0; i < VECS; ++i) {
        const int q = tid + i * NT;
        goff[i] = (uint32_t)(((int64_t)slot_row_of(q) * ld + min(slot_col_of(q), cmax)) * 2);
      }
    }
  }

  // Whole tile inside the operand: global -> LDS without registers, as
  // global_load_lds_dwordx4 with the wave-uniform base in scalar registers
  // and a 32-bit per-lane offset.  Issued as inline assembly so that the
  // compiler does not treat the in-flight LDS writes as aliasing the LDS
  // reads of the other stages (it would otherwise wait for them before every
  // fragment read); completion is awaited explicitly with a vmcnt wait before
  // the barrier that publishes the stage.
  // Wave-uniform copy of `base` for the scalar operand of the DMA.
  // readfirstlane yields a signed int: each half goes through uint32_t so
  // that the low half is zero-extended, not sign-extended, into 64 bits.
  __device__ __forceinline__ uint64_t sbase() const {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    return ((uint64_t)hi << 32) | (uint64_t)lo;
  }
  // Slot i of every lane of the wave: 64 lanes x 16 bytes into LDS at byte
  // address `m0` (wave-uniform: the region's slots of this wave, i*NT*16
  // bytes further per slot).  M0 is written one wait state ahead of the DMA
  // that reads it.
  __device__ __forceinline__ void issue_one(int i, uint64_t sb, uint32_t m0_wave) const {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(slot_off(i)), "s"(sb), "s"(m0_wave + (uint32_t)(i * NT * 16)) : "memory", "m0");
  }
  __device__ __forceinline__ void advance() { base += kstep; }

  // Ragged last K tile: r_rem rows (m/n) and k_rem k remain from the tile
  // origin; k outside is zero (m/n outside only reaches dropped outputs).
  __device__ __forceinline__ void load_checked(int r_rem, int k_rem, int tid) {
    const char* b = reinterpret_cast<const char*>(base);
#pragma unroll
    for (int i = 0; i < VECS; ++i) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      const int rr = REG ? row0 + i * RSTEP : slot_row_of(tid + i * NT);
      // the (clamped) column this slot reads; its validity is checked below
      const int cc = REG ? slot_col(i) : min(slot_col_of(tid + i * NT), ((min(r_rem, R) - 1) / 8) * 8);
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(b + slot_off(i));
      if constexpr (KC) {
        if (rr < r_rem && cc < k_rem) {
          x = *src;
          if (cc + 8 > k_rem) x = mask_vec8(x, k_rem - cc);
        }
      } else {
        if (rr < k_rem && cc < r_rem) {
          x = *src;
          if (cc + 8 > r_rem) x = mask_vec8(x, r_rem - cc);
        }
      }
      v[i] = x;
    }
    base += kstep;
  }

  __device__ __forceinline__ void store(bf16_t* region, int tid) const {
#pragma unroll
    for (int i = 0; i < VECS; ++i) *reinterpret_cast<u32x4_t*>(region + (tid + i * NT) * 8) = v[i];
  }
};

// MFMA operand fragments of one wave: FR blocks of 16 rows starting at row
// `base` of an R-row tile.  A fragment gives lane l row (l & 15), k = 8*(l >> 4)
// .. +7 of the current 32-wide k-step.
template <int R, int FR, bool KC, int BK>
struct FragReader {
  static constexpr int KS = BK / 32;
  int off[KC ? KS : FR];  // KC: per k-step; else per fragment (element offsets)

  __device__ __forceinline__ void init(int base, int lane) {
    const int fr = lane & 15, fg = lane >> 4;
    if constexpr (KC) {
      const int r = base + fr;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) off[ks] = r * BK + (((ks * 4 + fg) ^ kc_swizzle<BK / 8>(r)) * 8);
    } else {
      // lane j of a 16-lane group supplies k-row (j >> 2) and columns 4*(j & 3)..+3
      // of its group's 4 x 16 block; the hardware returns column j, k-rows 0..3.
      const int trow = 8 * fg + (fr >> 2);
      const int f = mn_swizzle<R>(trow);   // equal for every k-row this lane reads
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        const int chunk = (base + 16 * i) / 8 + ((fr & 3) >> 1);
        off[i] = trow * R + ((chunk ^ f) * 8) + (fr & 1) * 4;
      }
    }
  }

  __device__ __forceinline__ bf16x8_t read(const bf16_t* region, int ks, int i) const {
    if constexpr (KC) {
      return *reinterpret_cast<const bf16x8_t*>(region + off[ks] + i * 16 * BK);
    } else {
      const bf16_t* p = region + off[i] + ks * 32 * R;
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p);
      const s16x4_t hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p + 4 * R));
      const s16x8_t r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      return __builtin_bit_cast(bf16x8_t, r);
    }
  }
};

// One workgroup computes a BM x BN tile with WM x WN waves, each wave a
// (BM/WM) x (BN/WN) block of 16x16 MFMA tiles.  K advances in tiles of BK
// through NS LDS stages: up to NS full K tiles are in flight from global
// memory straight into LDS while the MFMAs consume the current one (tiles
// that stick out of M or N included); a ragged last K tile goes through
// bounds-checked register loads.  The epilogue runs from the accumulators.
template <int BM, int BN, int BK, int WM, int WN, int NS, bool AK, bool BKC, class Epi>
__global__ void __launch_bounds__(WM * WN * 64, 1)
gemm_bf16_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ B, GemmShape s, Epi epi0,
                 GemmAlt<Epi> alt) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int KS = BK / 32;
  constexpr int STAGE = (BM + BN) * BK;                 // bf16 elements per LDS stage
  constexpr int LDS_BYTES = NS * 2 * STAGE;
  static_assert(BK == 32 || BK == 64, "loaders and swizzles support BK = 32 or 64");
  static_assert(NS >= 2, "at least two stages");
  static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "wave tile");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) bf16_t lds[LDS_BYTES / 2];

  const int tiles_m = (s.M + BM - 1) / BM, tiles_n = (s.N + BN - 1) / BN;
  const int total = tiles_m * tiles_n * s.batch * s.groups;
  if ((int)blockIdx.x >= total) return;
  int z, tm, tn, g = 0;
  if (s.lpt) {
    const int per_rank = tiles_n * s.batch * s.groups, per_group = tiles_n * s.batch;
    const int r = (int)blockIdx.x / per_rank, rem = (int)blockIdx.x - r * per_rank;
    g = rem / per_group;
    const int rem2 = rem - g * per_group;
    z = rem2 / tiles_n;
    tn = rem2 - z * tiles_n;
    tm = s.kmode == 1 ? tiles_m - 1 - r : r;
  } else {
    tile_coords(blockIdx.x, total, tiles_m, tiles_n, s.group_m, z, tm, tn);   // groups == 1
  }
  const int zo = z / s.batch_inner, zi = z - zo * s.batch_inner;
  // operands of this tile's problem
  const bf16_t* const Ap = g ? alt.A : A;
  const bf16_t* const Bp = g ? alt.B : B;
  const int64_t lda = g ? alt.lda : s.lda, ldb = g ? alt.ldb : s.ldb;
  const int64_t sa_o = g ? alt.sa_o : s.sa_o, sa_i = g ? alt.sa_i : s.sa_i;
  const int64_t sb_o = g ? alt.sb_o : s.sb_o, sb_i = g ? alt.sb_i : s.sb_i;
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;

  if (s.skip_upper && s.skip_pad > 0) {
    const int mend = min(m0 + BM, s.M);
    if (n0 >= (mend + s.skip_pad - 1) / s.skip_pad * s.skip_pad) return;   // uniform: the whole workgroup leaves
  }
  int kb, ke;
  k_range(s, m0, BM, BK, kb, ke);
  if (s.skip_upper && n0 > m0 + BM - 1) ke = kb;
  const int nk = (ke - kb + BK - 1) / BK;
  // Full K tiles [0, nkd) are loaded directly, also for tiles that stick out
  // of M or N (the loaders re-read valid rows or chunks for the missing ones,
  // whose outputs the epilogue drops); a ragged last K tile goes through
  // bounds-checked register loads.
  const int nkd = (ke - kb) / BK;

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  using LoaderA = OperandLoader<BM, NT, AK, BK>;
  using LoaderB = OperandLoader<BN, NT, BKC, BK>;
  LoaderA la;
  LoaderB lb;
  la.init(Ap + zo * sa_o + zi * sa_i, lda, m0, kb, tid, s.M - m0);
  lb.init(Bp + zo * sb_o + zi * sb_i, ldb, n0, kb, tid, s.N - n0);
  FragReader<BM, FM, AK, BK> fa;
  FragReader<BN, FN, BKC, BK> fb;
  fa.init(wm * WTM, lane);
  fb.init(wn * WTN, lane);

  const int m_rem = s.M - m0, n_rem = s.N - n0;
  auto compute = [&](const bf16_t* st) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (FM * FN <= 32) {
        bf16x8_t af[FM], bfr[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) af[i] = fa.read(st, ks, i);
#pragma unroll
        for (int j = 0; j < FN; ++j) bfr[j] = fb.read(st + BM * BK, ks, j);
        // operands swapped: the result's lane layout is C(m = lane & 15, n = 4*(lane >> 4) + e)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
      } else {
        // Large wave tile: all B fragments, A fragments one block row at a
        // time with the next one in flight (bounded register footprint).
        bf16x8_t bfr[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) bfr[j] = fb.read(st + BM * BK, ks, j);
        bf16x8_t an = fa.read(st, ks, 0);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const bf16x8_t a = an;
          if (i + 1 < FM) an = fa.read(st, ks, i + 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], a, acc[i][j], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };
  // One k-step's operand fragments, read into registers ahead of their MFMAs.
  struct Frags {
    bf16x8_t a[FM], b[FN];
  };
  auto read_frags = [&](const bf16_t* st, int ks, Frags& f) {
#pragma unroll
    for (int j = 0; j < FN; ++j) f.b[j] = fb.read(st + BM * BK, ks, j);
#pragma unroll
    for (int i = 0; i < FM; ++i) f.a[i] = fa.read(st, ks, i);
  };
  auto mfma_frags = [&](const Frags& f) {
    // operands swapped: the result's lane layout is C(m = lane & 15, n = 4*(lane >> 4) + e)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
  };
  auto load_checked = [&](int kt) {
    const int k_rem = s.K - kb - kt * BK;
    la.load_checked(m_rem, k_rem, tid);
    lb.load_checked(n_rem, k_rem, tid);
  };
  auto store_regs = [&](bf16_t* st) {
    la.store(st, tid);
    lb.store(st + BM * BK, tid);
  };

  // LDS byte address of this wave's DMA slots in stage 0 (wave-uniform).
  const uint32_t lds_wave = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)((uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16_t*)lds + (uint32_t)wave * 1024u));
  constexpr int VA = LoaderA::VECS;
  constexpr int VPT = VA + LoaderB::VECS;   // DMA instructions per wave per K tile
  // DMA instruction d of the K tile bound for `stage` (A slots, then B).
  auto dma_one = [&](int d, int stage, uint64_t sa, uint64_t sb) {
    const uint32_t m0 = lds_wave + (uint32_t)(stage * STAGE * 2);
    if (d < VA) la.issue_one(d, sa, m0);
    else lb.issue_one(d - VA, sb, m0 + (uint32_t)(BM * BK * 2));
  };
  auto issue = [&](int stage) {   // K tiles are issued in order
    const uint64_t sa = la.sbase(), sb = lb.sbase();
#pragma unroll
    for (int d = 0; d < VPT; ++d) dma_one(d, stage, sa, sb);
    la.advance();
    lb.advance();
  };
  auto read_one = [&](const bf16_t* st, int ks, Frags& f, int r) {
    if (r < FN) f.b[r] = fb.read(st + BM * BK, ks, r);
    else f.a[r - FN] = fa.read(st, ks, r - FN);
  };
  // The MFMAs of one k-step with the FM + FN fragment reads of the next
  // k-step spread evenly between them and, with `dma`, the DMA instructions
  // of the K tile bound for `dstage` one after each of the first MFMAs: no
  // wave issues a burst of memory instructions while its matrix unit idles,
  // and the LDS command queue sees a steady stream instead of one burst per
  // wave.
  auto mfma_mix = [&](const Frags& f, const bf16_t* nst, int nks, Frags& nf, auto dma, int dstage) {
    constexpr bool DMA = decltype(dma)::value;
    constexpr int NM = FM * FN, NR = FM + FN;
    uint64_t sa = 0, sb = 0;
    if constexpr (DMA) {
      sa = la.sbase();
      sb = lb.sbase();
    }
#pragma unroll
    for (int t = 0; t < NM; ++t) {
      const int i = t / FN, j = t % FN;
      // operands swapped: the result's lane layout is C(m = lane & 15, n = 4*(lane >> 4) + e)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
      if constexpr (DMA) {
        if (t < VPT) dma_one(t, dstage, sa, sb);
      }
#pragma unroll
      for (int r = 0; r < NR; ++r)
        if ((r * NM) / NR == t) read_one(nst, nks, nf, r);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (DMA) {
#pragma unroll
      for (int d = NM; d < VPT; ++d) dma_one(d, dstage, sa, sb);
      la.advance();
      lb.advance();
    }
  };

  {
    // Every full K tile goes global -> LDS directly, up to NS of them in
    // flight.  Fragments are double-buffered by k-step: the LDS reads of the
    // next k-step go out between the MFMAs of the current one, and the
    // barrier that publishes tile kt+1 (and frees tile kt's stage for tile
    // kt+NS) sits before the MFMAs of tile kt's last k-step, so those MFMAs
    // overlap the first reads of tile kt+1 and the DMA of tile kt+NS.  No
    // other vector-memory operation is issued in this loop, so the vmcnt
    // count is exactly the DMA instructions of the tiles after kt+1.  The
    // barrier also waits for every LDS read of the wave, so the fragments of
    // tile kt's last k-step are complete when their MFMAs start.
    static_assert(KS == 2, "the pipelined loop pairs the two k-steps of a 64-wide K tile");
    if (nkd > 0) {
      const int pre = min(NS, nkd);
      for (int p = 0; p < pre; ++p) issue(p);
      if (nkd >= NS) wait_vmem_n<(NS - 1) * VPT>();   // tile 0 landed
      else wait_vmem();
      __syncthreads();
      Frags f0, f1;
      read_frags(lds, 0, f0);
      int cs = 0;   // stage of tile kt (tile j lives in stage j % NS)
      int kt = 0;
      auto step = [&](auto dma) {
        mfma_mix(f0, lds + cs * STAGE, 1, f1, std::false_type{}, 0);
        const int nx = (cs + 1 == NS) ? 0 : cs + 1;
        if (kt + NS <= nkd) wait_vmem_n<(NS - 2) * VPT>();   // tile kt+1 landed
        else wait_vmem();
        __syncthreads();   // tile kt+1 visible; every wave has read all of tile kt
        mfma_mix(f1, lds + nx * STAGE, 0, f0, dma, cs);   // tile kt+NS goes to stage cs
        cs = nx;
      };
      for (; kt + NS < nkd; ++kt) step(std::true_type{});
      for (; kt + 1 < nkd; ++kt) step(std::false_type{});
      mfma_mix(f0, lds + cs * STAGE, 1, f1, std::false_type{}, 0);   // the last tile
      mfma_frags(f1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (nk > nkd) {
      // the stage after the last direct tile: its last reader (tile nkd-NS)
      // finished before a loop barrier, and every DMA has been waited for
      bf16_t* st = lds + (nkd % NS) * STAGE;
      load_checked(nkd);
      store_regs(st);
      __syncthreads();
      compute(st);
    }
  }

  // Epilogue straight from the accumulators.  Fragment j of block row i gives
  // lane l the row m = 16 i + (l & 15) and the columns 16 j + 4 g .. +3,
  // g = l >> 4.  For a pair of fragments (j0, j1) the lanes of groups g and
  // g ^ 1 (lanes l and l ^ 16) trade four values, after which each lane holds
  // 8 consecutive columns: j0's 8 g' .. +7 for even g, j1's for odd g, with
  // g' = g >> 1.  Each lane then applies the epilogue to its 8 columns with
  // 16-byte accesses; no LDS and no barrier are involved, so waves leave
  // the K-loop independently.
  static_assert(FN % 2 == 0, "fragments are paired along n");
  const Epi epi = g ? alt.epi : epi0;
  const int lg = lane >> 4;
  const bool odd = lg & 1;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * WTM + i * 16 + (lane & 15);
#pragma unroll
    for (int jp = 0; jp < FN; jp += 2) {
      const f32x4_t& a0 = acc[i][jp];
      const f32x4_t& a1 = acc[i][jp + 1];
      float v[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float send = odd ? a0[e] : a1[e];
        const float recv = __shfl_xor(send, 16);
        v[e] = odd ? recv : a0[e];
        v[4 + e] = odd ? a1[e] : recv;
      }
      const int n = n0 + wn * WTN + (jp + (odd ? 1 : 0)) * 16 + (lg >> 1) * 8;
      if (m < s.M && n < s.N) epi(zo, zi, m + s.m_base, n + s.n_base, v, min(8, s.N - n));
    }
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
    if (m < s.M) epi(zo, zi, m + s.m_base, n + s.n_base, acc[i], min(8, s.N - n));
  }
}

// ------------------------------------------------------------------ dispatch

#define TPS_GEMM_TRY(expr) \
  do { tps_status _st = (expr); if (_st != TPS_OK) return _st; } while (0)

template <int BM, int BN, int BK, int WM, int WN, int NS, bool AK, bool BKC, class Epi>
inline tps_status launch_mfma(const bf16_t* A, const bf16_t* B, const GemmShape& s, const Epi& epi,
                              const GemmAlt<Epi>& alt, hipStream_t st) {
  const int64_t tiles = ceil_div(s.M, BM) * ceil_div(s.N, BN) * (int64_t)s.batch * s.groups;
  if (tiles == 0) return TPS_OK;
  if (tiles > 0x7fffffff) return set_error(TPS_EINVAL, "gemm: too many tiles");
  if (s.groups != 1 && (s.groups != 2 || !s.lpt)) return set_error(TPS_EINVAL, "gemm: groups must be 1, or 2 with lpt");
  // per-lane operand offsets inside a tile are 32-bit byte offsets
  int64_t lda = s.lda, ldb = s.ldb;
  if (s.groups == 2) {
    lda = lda > alt.lda ? lda : alt.lda;
    ldb = ldb > alt.ldb ? ldb : alt.ldb;
  }
  // 16-byte chunks of every row (and of each partial tile's re-read chunk)
  // stay aligned and inside their row only with leading dims that are
  // multiples of 8
  if (lda % 8 != 0 || ldb % 8 != 0 || (s.groups == 2 && (alt.lda % 8 != 0 || alt.ldb % 8 != 0)))
    return set_error(TPS_EINVAL, "gemm: leading dimensions must be multiples of 8");
  const int64_t span_a = (AK ? BM : BK) * lda * 2, span_b = (BKC ? BN : BK) * ldb * 2;
  if (span_a >= (1LL << 32) || span_b >= (1LL << 32))
    return set_error(TPS_EINVAL, "gemm: leading dimension too large for 32-bit tile offsets");
  TraceScope tr;
  if (g_trace_on) {
    static const std::string inst = template_args(__PRETTY_FUNCTION__);
    const std::string detail = inst + " " + std::to_string(s.M) + "x" + std::to_string(s.N) + "x" +
                               std::to_string(s.K) + " z" + std::to_string(s.batch * s.groups) +
                               (s.kmode || s.skip_upper ? " causal" : "");
    tr.begin(st, "gemm_bf16_kernel", detail.c_str());
  }
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, WM, WN, NS, AK, BKC, Epi>), dim3((unsigned)tiles),
                     dim3(WM * WN * 64), 0, st, A, B, s, epi, alt);
  return check_launch("gemm_bf16_kernel");
}

// The second problem slot of a single-problem launch (never read).
template <class Epi>
inline GemmAlt<Epi> no_alt(const Epi& e) {
  return GemmAlt<Epi>{nullptr, nullptr, 0, 0, 0, 0, 0, 0, e};
}

// Tile shape by problem size, from cold-cache timings of these kernels on
// MI355X (M = 2048 and the layer's N, K):
//   256x256, 8 waves, two stages, when it yields at least 192 tiles, unless
//     the grid would end with a partly filled second round (257..511 tiles
//     that are not a multiple of 256: 4096x6144x2048 TN takes 132 us at
//     256x256, 120 us at 128x128);
//   128x256, 8 waves of 64x64, three stages, when that fills one round of
//     192..256 tiles (2048x4096x8192 NN: 151 -> 135 us against 128x128;
//     2048x4096x6144 NT: 116 -> 108 us);
//   128x128, 8 waves of 64x32: two stages (64 KB, so two workgroups share a
//     CU and cover each other's waits) above 256 tiles, three stages at most
//     256 tiles, where one K tile in flight leaves the DMA latency exposed
//     (2048x2048x4096: 62 -> 47 us);
//   64x128, 8 waves of 32x32, three stages, when 128x128 tiles would fill
//     fewer than half of the CUs (64..127 tiles): twice the tiles (the
//     tied-logits leftover 2048x553x4096 NT: 28.9 -> 22.0 us);
//   64x64 for problems too small for 64 tiles of 128x128.
// Causal problems with live_tiles count only the tiles that compute: the
// attention probabilities P = exp(S - lse) at 4 heads x 2048 (head dim 512)
// have 144 live tiles of 256x256 (112 CUs idle through the exp epilogue) and
// 544 of 128x128, which take 32.0 us against 37.8; a plain fp32 store of the
// same shape (dP) is faster on the 256x256 grid (29.5 against 34.4 us).
// Longest-first (lpt) launches always take 128x128 with three stages: one
// workgroup per CU, so the CUs that finish short tiles pick up the next
// ones (dV and dK together: 57.6 -> 39.2 us against two launches).
// Otherwise, before all of these: 256x192 (8 waves of 64x96, two stages) when the
// 256x256 grid does not fill whole rounds but a 256x192 grid with no edge
// tiles does (2048x6144x4096 NN: 118 -> 107 us; 4096x6144x2048 TN: 120 us at
// 128x128 -> 116 us).
// Tiles of BM x BN that the dispatch counts: the whole grid, or with
// live_tiles (and skip_upper, skip_pad > 0) only the tiles before the causal
// limit rounded up to skip_pad; the others leave at once and occupy no CU.
inline int64_t tile_count(const GemmShape& s, int64_t BM, int64_t BN) {
  const int64_t tm = ceil_div(s.M, BM), tn = ceil_div(s.N, BN);
  if (!(s.live_tiles && s.skip_upper && s.skip_pad > 0)) return tm * tn * (int64_t)s.batch * s.groups;
  int64_t n = 0;
  for (int64_t i = 0; i < tm; ++i) {
    const int64_t mend = std::min<int64_t>((i + 1) * BM, s.M);
    n += std::min<int64_t>(tn, ceil_div(ceil_div(mend, s.skip_pad) * s.skip_pad, BN));
  }
  return n * s.batch * s.groups;
}

template <bool AK, bool BKC, class Epi>
inline tps_status gemm_bf16(const bf16_t* A, const bf16_t* B, const GemmShape& s, const Epi& epi,
                            const GemmAlt<Epi>& alt, hipStream_t st) {
  const int64_t t256 = tile_count(s, 256, 256);
  // Tail split: a single problem whose 256x256 grid ends in a round at most
  // a quarter full runs as whole rounds of 256x256 tiles plus the leftover
  // columns (or rows) as a second launch with smaller tiles.  Each output
  // element is summed in the same K order either way (bit-identical).
  // 2048x25129x4096 NT: 479 -> 416 us; 25129x4096x2048 TN: 513 -> 469 us (cold).
  if (s.batch == 1 && s.groups == 1 && s.kmode == 0 && !s.skip_upper && t256 > 256 && t256 % 256 != 0 &&
      t256 % 256 <= 64) {
    const int64_t tmr = ceil_div(s.M, 256), tnr = ceil_div(s.N, 256), full = t256 / 256 * 256;
    if (256 % tmr == 0 && full / tmr < tnr) {          // split the columns
      const int nm = (int)(full / tmr * 256);
      GemmShape a = s, b = s;
      a.N = nm;
      b.N = s.N - nm;
      b.n_base = s.n_base + nm;
      TPS_GEMM_TRY((gemm_bf16<AK, BKC>(A, B, a, epi, alt, st)));
      return gemm_bf16<AK, BKC>(A, B + (BKC ? (int64_t)nm * s.ldb : (int64_t)nm), b, epi, alt, st);
    }
    if (256 % tnr == 0 && full / tnr < tmr) {          // split the rows
      const int mm = (int)(full / tnr * 256);
      GemmShape a = s, b = s;
      a.M = mm;
      b.M = s.M - mm;
      b.m_base = s.m_base + mm;
      TPS_GEMM_TRY((gemm_bf16<AK, BKC>(A, B, a, epi, alt, st)));
      return gemm_bf16<AK, BKC>(A + (AK ? (int64_t)mm * s.lda : (int64_t)mm), B, b, epi, alt, st);
    }
  }
  const int64_t t128x256 = tile_count(s, 128, 256);
  const int64_t t128 = tile_count(s, 128, 128);
  const int64_t t192 = ceil_div(s.M, 256) * ceil_div(s.N, 192) * (int64_t)s.batch * s.groups;
  const bool full192 = s.M % 256 == 0 && s.N % 192 == 0 && t192 > 0 && t192 % 256 == 0;
  if (s.lpt) return launch_mfma<128, 128, 64, 2, 4, 3, AK, BKC>(A, B, s, epi, alt, st);
  if (full192 && t256 % 256 != 0) return launch_mfma<256, 192, 64, 4, 2, 2, AK, BKC>(A, B, s, epi, alt, st);
  const bool partial_round = t256 > 256 && t256 < 512 && t256 % 256 != 0;
  if (t256 >= 192 && !partial_round) return launch_mfma<256, 256, 64, 2, 4, 2, AK, BKC>(A, B, s, epi, alt, st);
  if (t128x256 >= 192 && t128x256 <= 256) return launch_mfma<128, 256, 64, 2, 4, 3, AK, BKC>(A, B, s, epi, alt, st);
  if (t128 > 256) return launch_mfma<128, 128, 64, 2, 4, 2, AK, BKC>(A, B, s, epi, alt, st);
  if (t128 >= 64 && t128 < 128) return launch_mfma<64, 128, 64, 2, 4, 3, AK, BKC>(A, B, s, epi, alt, st);
  if (t128 >= 64) return launch_mfma<128, 128, 64, 2, 4, 3, AK, BKC>(A, B, s, epi, alt, st);
  return launch_mfma<64, 64, 64, 2, 2, 2, AK, BKC>(A, B, s, epi, alt, st);
}

// A single problem.
template <bool AK, bool BKC, class Epi>
inline tps_status gemm_bf16(const bf16_t* A, const bf16_t* B, const GemmShape& s, const Epi& epi, hipStream_t st) {
  return gemm_bf16<AK, BKC>(A, B, s, epi, no_alt(epi), st);
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
