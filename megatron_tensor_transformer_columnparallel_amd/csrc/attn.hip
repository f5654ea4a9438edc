// Attention shard: QKV column-parallel by heads, per-head softmax attention,
// row-parallel output projection.
//
// Forward core, per (batch, head): the scores S = Q K^T are an MFMA GEMM
// whose epilogue stores S * scale * log2(e) in fp32 (tiles wholly above the
// causal diagonal are neither computed nor stored); a row pass takes each
// row's max and sum of exp2, writes the normalised probabilities P in bf16
// and saves lse = log(sum exp(S * scale)); O = P V is a second GEMM whose
// K-loop stops at the causal limit of its row tile.  With 4 heads of 512 on
// 2048 tokens this keeps all 256 CUs busy, where one workgroup per
// (head, query block) would occupy at most 128 of them, and it reads K and V
// once per 256-wide tile instead of once per 64-query block.  S and P live in
// a caller workspace of O(sq^2) per head (96 MB for 4 heads at sq = 2048).
//
// Backward core: the probabilities are recomputed from lse tile by tile by
// the GEMM kernel (epilogue exp(S*scale - lse)) and written to the workspace
// in bf16; dP = dO V^T is a GEMM into fp32 and a row pass forms
// dS = P * (dP - delta) * scale with delta taken from the same P and dP;
// dV = P^T dO, dQ = dS K and dK = dS^T Q are then MFMA GEMMs whose K-loops
// skip the causally-zero blocks.
#include <string>

#include "flash_attn.hpp"
#include "flash_bwd.hpp"
#include "flash_fwd_pp.hpp"
#include "gemm.hpp"

namespace tps {

// Scores of one (batch, head) problem, stored in the log2 domain:
// S2(m, n) = acc * scale * log2(e).  With `causal`, 8-column chunks that lie
// entirely after the query (n > m) are not stored: no pass reads them.
struct EpiScore {
  float* S;
  int64_t ld, sp;  // row stride and per-(b,head) stride of S
  int hs, causal;
  float scale_log2;
  __device__ void operator()(int zo, int zi, int m, int n, float v[8], int nv) const {
    if (causal && n > m) return;
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = v[i] * scale_log2;
    store8<float>(S + (int64_t)(zo * hs + zi) * sp + (int64_t)m * ld + n, t, nv);
  }
};

// Rows of S2, P, dP and dS are ldp elements apart with ldp a multiple of 8,
// so every 8-element chunk that starts inside a row lies inside it: the row
// passes below always move whole 16- or 32-byte vectors and mask columns
// past the row's limit arithmetically (values beyond it are never used).
__device__ __forceinline__ void ld_f32x8(const float* p, float v[8]) {
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
  const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3]; v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
}
__device__ __forceinline__ void ld_bf16x8(const bf16_t* p, float v[8]) {
  const u32x4_t x = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
  for (int w = 0; w < 4; ++w) { v[2 * w] = bf16lo(x[w]); v[2 * w + 1] = bf16hi(x[w]); }
}
__device__ __forceinline__ void st_bf16x8(bf16_t* p, const float v[8]) {
  *reinterpret_cast<u32x4_t*>(p) =
      u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
}

// Causal zero padding of P and dS: a row i is written up to this column so
// that the GEMMs that read them (row tiles of at most 256; K-loops ending at
// the tile's last row, or starting at its first) only ever read written
// values.
constexpr int kProbPad = 256;
constexpr int kRowUnroll = 4;   // 8-element chunks in flight per lane

// One wavefront per row of one (batch, head): online max / sum of exp2 over
// the row's unmasked scores (8 per lane per chunk, merged across lanes),
// then P = exp2(S2 - max) / sum in bf16 for the unmasked columns and zeros
// up to the padding limit; lse = (max + log2(sum)) * ln 2.  Rows of at most
// 64 x 8 x kRowUnroll written columns take one pass (S read once).
__global__ void __launch_bounds__(256) attn_softmax_kernel(const float* __restrict__ S2, bf16_t* __restrict__ P,
                                                           float* __restrict__ lse, int64_t rows, int sq,
                                                           int64_t ldp, int causal) {
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= rows) return;
  const int lane = threadIdx.x & 63;
  const int i = (int)(w % sq);
  const int ncol = causal ? i + 1 : sq;
  const int zend = causal ? (int)min(ldp, (int64_t)((i + kProbPad) / kProbPad) * kProbPad) : (int)ldp;
  const float* sr = S2 + w * ldp;
  bf16_t* pr = P + w * ldp;
  float mx = -INFINITY, sum = 0.f;
  if (zend <= 64 * 8 * kRowUnroll) {
    // the whole row is one pass of kRowUnroll chunks per lane: S is read
    // once; row max, then exp2 once per score, row sum, scaled store
    float x[kRowUnroll][8];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int c = lane * 8 + u * 64 * 8;
      if (c < ncol) ld_f32x8(sr + c, x[u]);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c + e >= ncol) x[u][e] = -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, x[u][e]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[u][e] = exp2f(x[u][e] - mx);   // masked: exp2(-inf) = 0
        sum += x[u][e];
      }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
    const float inv = 1.f / sum;
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int c = lane * 8 + u * 64 * 8;
      if (c < zend) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = x[u][e] * inv;
        st_bf16x8(pr + c, p);
      }
    }
    if (lane == 0) lse[w] = (mx + log2f(sum)) * 0.69314718055994531f;
    return;
  }
  for (int c0 = lane * 8; c0 < ncol; c0 += 64 * 8 * kRowUnroll) {
    float x[kRowUnroll][8];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int c = c0 + u * 64 * 8;
      if (c < ncol) ld_f32x8(sr + c, x[u]);
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int c = c0 + u * 64 * 8;
      if (c < ncol) {
        float bm = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) bm = fmaxf(bm, c + e < ncol ? x[u][e] : -INFINITY);
        const float nm = fmaxf(mx, bm);
        float bs = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) bs += c + e < ncol ? exp2f(x[u][e] - nm) : 0.f;
        sum = sum * exp2f(mx - nm) + bs;   // exp2(-inf) = 0 on the first chunk
        mx = nm;
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float om = __shfl_xor(mx, o), os = __shfl_xor(sum, o);
    const float nm = fmaxf(mx, om);
    sum = (nm == -INFINITY) ? 0.f : sum * exp2f(mx - nm) + os * exp2f(om - nm);
    mx = nm;
  }
  const float inv = 1.f / sum;
  for (int c0 = lane * 8; c0 < zend; c0 += 64 * 8 * kRowUnroll) {
    float x[kRowUnroll][8];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int c = c0 + u * 64 * 8;
      if (c < ncol) ld_f32x8(sr + c, x[u]);
      else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int c = c0 + u * 64 * 8;
      if (c < zend) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = (c + e < ncol) ? exp2f(x[u][e] - mx) * inv : 0.f;
        st_bf16x8(pr + c, p);
      }
    }
  }
  if (lane == 0) lse[w] = (mx + log2f(sum)) * 0.69314718055994531f;
}

// One wavefront per row of one (batch, head): with P the stored (bf16)
// probabilities and dP = dO V^T (fp32), delta = sum_j P_j dP_j / sum_j P_j and
// dS_j = P_j (dP_j - delta) * scale.  Taking delta from the same P and dP
// makes every row of dS sum to zero (the softmax gradient of the stored P),
// so the rounding of O and dO does not leak into dQ as a per-row bias.
// Columns at or beyond the causal limit are written as 0 up to the padding
// limit (the whole row without the causal mask).  Rows of at most
// 64 x 8 x kRowUnroll written columns take one pass (P and dP read once).
__global__ void __launch_bounds__(256) attn_ds_kernel(const bf16_t* __restrict__ P, const float* __restrict__ dP,
                                                      bf16_t* __restrict__ dS, int64_t rows, int sq, int64_t ldp,
                                                      int causal, float scale) {
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= rows) return;
  const int lane = threadIdx.x & 63;
  const int i = (int)(w % sq);                    // query index within its head
  const int ncol = causal ? i + 1 : sq;
  const int zend = causal ? (int)min(ldp, (int64_t)((i + kProbPad) / kProbPad) * kProbPad) : (int)ldp;
  const bf16_t* pr = P + w * ldp;
  const float* dpr = dP + w * ldp;
  bf16_t* dsr = dS + w * ldp;
  float num = 0.f, den = 0.f;
  if (zend <= 64 * 8 * kRowUnroll) {
    // the whole row is one pass of kRowUnroll chunks per lane: P and dP are
    // read once and kept in registers
    float p[kRowUnroll][8], d[kRowUnroll][8];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int c = lane * 8 + u * 64 * 8;
      if (c < ncol) { ld_bf16x8(pr + c, p[u]); ld_f32x8(dpr + c, d[u]); }
      else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { p[u][e] = 0.f; d[u][e] = 0.f; }
      }
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int c = lane * 8 + u * 64 * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c + e < ncol) { num += p[u][e] * d[u][e]; den += p[u][e]; }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) { num += __shfl_xor(num, o); den += __shfl_xor(den, o); }
    const float delta = den > 0.f ? num / den : 0.f;
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int c = lane * 8 + u * 64 * 8;
      if (c < zend) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (c + e < ncol) ? p[u][e] * (d[u][e] - delta) * scale : 0.f;
        st_bf16x8(dsr + c, o);
      }
    }
    return;
  }
  for (int c0 = lane * 8; c0 < ncol; c0 += 64 * 8 * kRowUnroll) {
    float p[kRowUnroll][8], d[kRowUnroll][8];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int c = c0 + u * 64 * 8;
      if (c < ncol) { ld_bf16x8(pr + c, p[u]); ld_f32x8(dpr + c, d[u]); }
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int c = c0 + u * 64 * 8;
      if (c < ncol) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c + e < ncol) { num += p[u][e] * d[u][e]; den += p[u][e]; }
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) { num += __shfl_xor(num, o); den += __shfl_xor(den, o); }
  const float delta = den > 0.f ? num / den : 0.f;
  for (int c0 = lane * 8; c0 < zend; c0 += 64 * 8 * kRowUnroll) {
    float p[kRowUnroll][8], d[kRowUnroll][8];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int c = c0 + u * 64 * 8;
      if (c < ncol) { ld_bf16x8(pr + c, p[u]); ld_f32x8(dpr + c, d[u]); }
      else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { p[u][e] = 0.f; d[u][e] = 0.f; }
      }
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int c = c0 + u * 64 * 8;
      if (c < zend) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (c + e < ncol) ? p[u][e] * (d[u][e] - delta) * scale : 0.f;
        st_bf16x8(dsr + c, o);
      }
    }
  }
}

static GemmShape shape(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb) {
  GemmShape s;
  s.M = (int)M; s.N = (int)N; s.K = (int)K; s.lda = lda; s.ldb = ldb;
  return s;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// P and dS are [b][hs][sq][ldp] with the row stride ldp padded to a multiple
// of 8 elements so that every 16-byte vector access stays aligned; the
// padding columns are never read unmasked.
struct AttnWs {
  size_t dO, P, dP, dS, dQKV, total;
  int64_t ldp;
};
static AttnWs attn_ws_layout(int64_t b, int64_t sq, int64_t hs, int64_t d) {
  AttnWs w;
  const size_t M = (size_t)(b * sq);
  w.ldp = (sq + 7) / 8 * 8;
  w.dO = 0;
  w.P = align256(w.dO + M * hs * d * 2);
  w.dP = align256(w.P + (size_t)b * hs * sq * w.ldp * 2);
  w.dS = align256(w.dP + (size_t)b * hs * sq * w.ldp * 4);
  w.dQKV = align256(w.dS + (size_t)b * hs * sq * w.ldp * 2);
  w.total = align256(w.dQKV + M * 3 * hs * d * 2);
  return w;
}

// Flash backward workspace: dO and dQKV (bf16, row-major like O and QKV),
// Delta (fp32, [b][hs][sq]), the per-item row sums of the Delta phase
// (fp32 pairs), and the fp32 partials of split blocks: dQ ([item][128][d])
// and dK, dV ([item][rows][2 d]).  The item counts come from the work plans,
// about one item per CU, so the partials are bounded by the CU count times a
// block, not by the sequence length.
struct AttnFlashBwdWs {
  size_t dO, dQKV, delta, rd, qpart, kvpart, total;
};
static AttnFlashBwdWs attn_flash_bwd_ws_layout(int64_t b, int64_t sq, int64_t hs, int64_t d,
                                               const flash::BwdWork& wq, const flash::BwdWork& wk) {
  AttnFlashBwdWs w;
  const size_t M = (size_t)(b * sq);
  const size_t iq = (size_t)flash::work_total(wq), ik = (size_t)flash::work_total(wk);
  w.dO = 0;
  w.dQKV = align256(w.dO + M * hs * d * 2);
  w.delta = align256(w.dQKV + M * 3 * hs * d * 2);
  w.rd = align256(w.delta + (size_t)b * hs * sq * 4);
  w.qpart = align256(w.rd + iq * wq.bb * 2 * 4);
  w.kvpart = align256(w.qpart + iq * wq.bb * d * 4);
  w.total = align256(w.kvpart + ik * wk.bb * 2 * d * 4);
  return w;
}

// Forward workspace: the log2-domain scores S2 (fp32) and the probabilities
// P (bf16), both [b][hs][sq][ldp].
struct AttnFwdWs {
  size_t S, P, total;
  int64_t ldp;
};
static AttnFwdWs attn_fwd_ws_layout(int64_t b, int64_t sq, int64_t hs) {
  AttnFwdWs w;
  w.ldp = (sq + 7) / 8 * 8;
  const size_t n = (size_t)b * hs * sq * w.ldp;
  w.S = 0;
  w.P = align256(n * 4);
  w.total = align256(w.P + n * 2);
  return w;
}

#define TPS_REQ(cond, msg) \
  do { if (!(cond)) return set_error(TPS_EINVAL, std::string(fn) + ": " + (msg)); } while (0)
#define TPS_TRY(expr) \
  do { tps_status _s = (expr); if (_s != TPS_OK) return _s; } while (0)

static tps_status attn_checks(const char* fn, tps_dtype dt, int64_t b, int64_t sq, int64_t h, int64_t hs, int64_t d,
                              std::initializer_list<const void*> ptrs) {
  TPS_REQ(dt == TPS_F32 || dt == TPS_BF16, "bad dtype");
  TPS_REQ(b > 0 && sq > 0 && h > 0 && hs > 0 && d > 0, "dims must be > 0");
  TPS_REQ(b * sq < 0x7fffffffLL && 3 * hs * d < 0x7fffffffLL && h < 0x7fffffffLL, "dims must be < 2^31");
  TPS_REQ(h % vec_elems(dt) == 0, "h must be a multiple of 8 (bf16)");
  for (const void* p : ptrs) {
    TPS_REQ(p != nullptr, "null pointer");
    TPS_REQ(aligned16(p), "pointer not 16-byte aligned");
  }
  if (dt != TPS_BF16) return set_error(TPS_EUNSUPPORTED, std::string(fn) + ": attention is implemented for bf16 only");
  TPS_REQ(d % 8 == 0, "head dim must be a multiple of 8");
  return TPS_OK;
}

}  // namespace tps

using namespace tps;

// Which forward core a call takes: the flash kernels for head dims 64, 128,
// 256 and 512 at every sequence length; other head dims (multiples of 8)
// take the score GEMM, row softmax and PV GEMM.  Up to 256 each wave keeps
// 32 query rows (Q fragments and the fp32 output accumulator fit one wave's
// registers), and every K or V fragment read from LDS feeds two MFMAs.  At
// 512 a wave can keep only 16 rows, so each fragment feeds one MFMA and the
// kernel is bound by LDS bandwidth; with the merge's single pass it still
// beats the score path at sq = 2048 with 4 heads (48.2 + 16.1 us against
// 68.0 us) and keeps the workspace O(sq d).
static bool use_flash(int64_t d, int64_t sq) {
  (void)sq;
  return d == 64 || d == 128 || d == 256 || d == 512;
}

// Which backward core: the flash kernels are compiled for head dims 64..256
// (at 512 a wave cannot hold the fragments and both accumulators of 32 keys;
// the score / dS GEMM path keeps O(sq^2) workspace there).
static bool use_flash_bwd(int64_t d) { return d == 64 || d == 128 || d == 256; }

// Compute units of the current device (the flash forward sizes its work
// items so that one round of them fills the chip).
static int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  return n;
}

// Workgroups of a kernel that one CU holds at once (registers and LDS), as
// the runtime reports it; 1 when it cannot tell.  Cached per kernel.
template <class K>
static int blocks_per_cu(K kernel, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return 1;
  }
  return n;
}

// Work items the flash forward plans for.  Head dims 64 and 128 run the
// two-group kernel (256-row items, eight waves): CUs times its workgroups
// per CU (two at head dim 64, whose waves fit 128 registers; one at 128).
// Head dims 256 and 512 run the one-group kernel (128-row items): CUs times
// its workgroups per CU, at most two, where the partials of the extra split
// blocks cost the merge more than a third workgroup gains.
static bool fwd_two_group(int64_t d) { return d == 64 || d == 128; }
template <int D>
static int fwd_slots() {
  if constexpr (D <= 128) {
    static const int per_cu = blocks_per_cu(flash::attn_fwd_pp_kernel<D>, flash::PPShape<D>::THREADS);
    return device_cus() * per_cu;
  } else {
    constexpr int QB = D >= 512 ? 1 : 2;
    static const int per_cu = blocks_per_cu(flash::attn_fwd_flash_kernel<D, QB>, flash::Shape<D, QB>::THREADS);
    return device_cus() * (D >= 256 ? std::min(per_cu, 2) : per_cu);
  }
}
static int fwd_slots_d(int64_t d) {
  if (d == 64) return fwd_slots<64>();
  if (d == 128) return fwd_slots<128>();
  if (d == 256) return fwd_slots<256>();
  return fwd_slots<512>();
}
static flash::Plan fwd_plan(int64_t b, int64_t sq, int64_t hs, int64_t d, int causal) {
  return flash::make_plan(b, sq, hs, (int)d, causal, fwd_slots_d(d), fwd_two_group(d) ? flash::kPPRows : flash::kBQ);
}

extern "C" size_t tp_attn_fwd_workspace(tps_dtype dt, int64_t b, int64_t sq, int64_t h, int64_t hs, int64_t d) {
  (void)dt;
  (void)h;
  if (b <= 0 || sq <= 0 || hs <= 0 || d <= 0) return 0;
  if (use_flash(d, sq)) {
    // the query has no causal argument: cover the larger of the two plans
    // (without the mask every block has all keys, so more chunks)
    return std::max(flash::plan_workspace(fwd_plan(b, sq, hs, d, 1), (int)d),
                    flash::plan_workspace(fwd_plan(b, sq, hs, d, 0), (int)d));
  }
  return attn_fwd_ws_layout(b, sq, hs).total;
}

// Flash forward core: O and lse from QKV (see flash_attn.hpp).
// Row blocks per wave: two (32 rows, four waves of up to 512 registers) up
// to head dim 256; at 512 the 32 x 512 fp32 accumulator plus the Q
// fragments do not fit one wave's registers, so waves take 16 rows (eight
// waves of 256 registers).
template <int D>
static tps_status flash_fwd_core(const bf16_t* qkv, bf16_t* o, float* lse, void* ws, const flash::Plan& p,
                                 hipStream_t st) {
  const int total = p.items_per_z * p.nz;
  float* part = static_cast<float*>(ws);
  if constexpr (D <= 128) {
    TraceScope trace_(st, "attn_fwd_pp_kernel");
    hipLaunchKernelGGL((flash::attn_fwd_pp_kernel<D>), dim3((unsigned)total), dim3(flash::PPShape<D>::THREADS), 0,
                       st, qkv, o, lse, part, p, total);
    TPS_TRY(check_launch("attn_fwd_pp_kernel"));
  } else {
    TraceScope trace_(st, "attn_fwd_flash_kernel");
    constexpr int QB = D >= 512 ? 1 : 2;
    hipLaunchKernelGGL((flash::attn_fwd_flash_kernel<D, QB>), dim3((unsigned)total),
                       dim3(flash::Shape<D, QB>::THREADS), 0, st, qkv, o, lse, part, p, total);
    TPS_TRY(check_launch("attn_fwd_flash_kernel"));
  }
  const int mz = flash::plan_merges_per_z(p);
  if (mz == 0) return TPS_OK;
  TraceScope trace_(st, "attn_fwd_merge_kernel");
  hipLaunchKernelGGL((flash::attn_fwd_merge_kernel<D>), dim3((unsigned)(mz * p.nz * flash::merge_groups<D>(p.bq))),
                     dim3(flash::kMergeThreads), 0, st, part, o, lse, p, total, mz);
  return check_launch("attn_fwd_merge_kernel");
}

extern "C" tps_status tp_attn_fwd(tps_dtype dt, int64_t b, int64_t sq, int64_t h, int64_t hs, int64_t d, int causal,
                                  const void* X, const void* Wqkv_i, const void* Wo_i, void* QKV_i, void* O_i,
                                  float* lse_i, void* Z_i, void* ws, size_t ws_bytes, tps_stream_t stream) {
  ApiScope api_scope_("tp_attn_fwd");
  TPS_TRY(attn_checks("tp_attn_fwd", dt, b, sq, h, hs, d, {X, Wqkv_i, Wo_i, QKV_i, O_i, lse_i, Z_i, ws}));
  if (ws_bytes < tp_attn_fwd_workspace(dt, b, sq, h, hs, d))
    return set_error(TPS_EWORKSPACE, "tp_attn_fwd: workspace too small");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (use_flash(d, sq)) {
    const int64_t M = b * sq, w = hs * d, w3 = 3 * w;
    bf16_t* qkv = (bf16_t*)QKV_i;
    bf16_t* o = (bf16_t*)O_i;
    // QKV_i = X Wqkv_i                       (NN)
    TPS_TRY((gemm_bf16<true, false>((const bf16_t*)X, (const bf16_t*)Wqkv_i, shape(M, w3, h, h, w3),
                                    EpiStore<bf16_t>{qkv, w3, 0, 0}, st)));
    const flash::Plan p = fwd_plan(b, sq, hs, d, causal ? 1 : 0);
    if (ws_bytes < flash::plan_workspace(p, (int)d))
      return set_error(TPS_EWORKSPACE, "tp_attn_fwd: workspace too small");
    if (d == 64) TPS_TRY(flash_fwd_core<64>(qkv, o, lse_i, ws, p, st));
    else if (d == 128) TPS_TRY(flash_fwd_core<128>(qkv, o, lse_i, ws, p, st));
    else if (d == 256) TPS_TRY(flash_fwd_core<256>(qkv, o, lse_i, ws, p, st));
    else TPS_TRY(flash_fwd_core<512>(qkv, o, lse_i, ws, p, st));
    // Z_i = O_i Wo_i                         (NN)
    return gemm_bf16<true, false>(o, (const bf16_t*)Wo_i, shape(M, h, w, w, h),
                                  EpiStore<bf16_t>{(bf16_t*)Z_i, h, 0, 0}, st);
  }
  const AttnFwdWs L = attn_fwd_ws_layout(b, sq, hs);
  const int64_t M = b * sq, w = hs * d, w3 = 3 * w;
  const bf16_t* x = (const bf16_t*)X;
  bf16_t* qkv = (bf16_t*)QKV_i;
  bf16_t* o = (bf16_t*)O_i;
  char* base = static_cast<char*>(ws);
  float* S2 = (float*)(base + L.S);
  bf16_t* P = (bf16_t*)(base + L.P);
  const int64_t ldp = L.ldp, sp = sq * L.ldp;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)d);
  // QKV_i = X Wqkv_i                       (NN)
  TPS_TRY((gemm_bf16<true, false>(x, (const bf16_t*)Wqkv_i, shape(M, w3, h, h, w3),
                                  EpiStore<bf16_t>{qkv, w3, 0, 0}, st)));
  // Per (batch, head) problems: z = bi*hs + j.
  // S2 = Q K^T * scale * log2(e)           (NT)  [sq x sq] per head, fp32
  GemmShape s = shape(sq, sq, d, w3, w3);
  s.batch = (int)(b * hs);
  s.batch_inner = (int)hs;
  s.sa_o = sq * w3; s.sa_i = d; s.sb_o = sq * w3; s.sb_i = d;
  s.skip_upper = causal ? 1 : 0;
  s.skip_pad = 1;   // scores are read only up to the diagonal
  TPS_TRY((gemm_bf16<true, true>(qkv, qkv + w, s, EpiScore{S2, ldp, sp, (int)hs, causal ? 1 : 0, scale_log2}, st)));
  // P = softmax rows of S (bf16), lse
  TPS_TRY(([&]() {
    TraceScope trace_(st, "attn_softmax_kernel");
    hipLaunchKernelGGL(attn_softmax_kernel, dim3((unsigned)ceil_div(b * hs * sq, 4)), dim3(256), 0, st, S2, P, lse_i,
                       b * hs * sq, (int)sq, ldp, causal ? 1 : 0);
    return check_launch("attn_softmax_kernel");
  }()));
  // O = P V                                (NN)  [sq x d] per head, K = keys <= query
  GemmShape s2 = shape(sq, d, sq, ldp, w3);
  s2.batch = (int)(b * hs); s2.batch_inner = (int)hs;
  s2.sa_o = hs * sp; s2.sa_i = sp; s2.sb_o = sq * w3; s2.sb_i = d;
  s2.kmode = causal ? 1 : 0;
  TPS_TRY((gemm_bf16<true, false>(P, qkv + 2 * w, s2, EpiStore<bf16_t>{o, w, sq * w, d}, st)));
  // Z_i = O_i Wo_i                         (NN)
  return gemm_bf16<true, false>(o, (const bf16_t*)Wo_i, shape(M, h, w, w, h), EpiStore<bf16_t>{(bf16_t*)Z_i, h, 0, 0},
                                st);
}

// The two work plans of a flash backward call (query blocks over keys for
// the Delta and dQ phases, key blocks over queries for the dK/dV phase).
// (one round of items per phase: CUs times the phase kernel's workgroups per
// CU; the Delta and dQ phases share a plan sized for the dQ kernel)
template <int D>
static void flash_bwd_works(int64_t b, int64_t sq, int64_t hs, int causal, flash::BwdWork& wq, flash::BwdWork& wk) {
  using SQ = flash::BwdShape<D, false>;
  using SK = flash::BwdShape<D, true>;
  static const int per_cu_q = blocks_per_cu(flash::attn_bwd_q_kernel<D, 1>, SQ::THREADS);
  static const int per_cu_k = blocks_per_cu(flash::attn_bwd_kv_kernel<D>, SK::THREADS);
  const int cus = device_cus();
  wq = flash::make_bwd_work(b, sq, hs, SQ::BB, causal, 0, cus * per_cu_q);
  wk = flash::make_bwd_work(b, sq, hs, SK::BB, causal, 1, cus * per_cu_k);
}
static void flash_bwd_works_d(int64_t d, int64_t b, int64_t sq, int64_t hs, int causal, flash::BwdWork& wq,
                              flash::BwdWork& wk) {
  if (d == 64) flash_bwd_works<64>(b, sq, hs, causal, wq, wk);
  else if (d == 128) flash_bwd_works<128>(b, sq, hs, causal, wq, wk);
  else flash_bwd_works<256>(b, sq, hs, causal, wq, wk);
}

extern "C" size_t tp_attn_bwd_workspace(tps_dtype dt, int64_t b, int64_t sq, int64_t h, int64_t hs, int64_t d) {
  (void)dt;
  (void)h;
  if (b <= 0 || sq <= 0 || hs <= 0 || d <= 0) return 0;
  if (use_flash_bwd(d)) {
    // the query has no causal argument: cover both plans
    size_t need = 0;
    for (int causal = 0; causal < 2; ++causal) {
      flash::BwdWork wq, wk;
      flash_bwd_works_d(d, b, sq, hs, causal, wq, wk);
      need = std::max(need, attn_flash_bwd_ws_layout(b, sq, hs, d, wq, wk).total);
    }
    return need;
  }
  return attn_ws_layout(b, sq, hs, d).total;
}

// Flash backward core: Delta partials, then dQ (and Delta), then dK and dV,
// then the merges of split blocks (see flash_bwd.hpp).
template <int D>
static tps_status flash_bwd_core(const bf16_t* qkv, const bf16_t* dO, const float* lse, bf16_t* dqkv, char* ws,
                                 const AttnFlashBwdWs& L, const flash::BwdPlan& p, const flash::BwdWork& wq,
                                 const flash::BwdWork& wk, hipStream_t st) {
  using SQ = flash::BwdShape<D, false>;
  using SK = flash::BwdShape<D, true>;
  float* delta = (float*)(ws + L.delta);
  float* rd = (float*)(ws + L.rd);
  float* qpart = (float*)(ws + L.qpart);
  float* kvpart = (float*)(ws + L.kvpart);
  const unsigned nq = (unsigned)flash::work_total(wq), nk = (unsigned)flash::work_total(wk);
  {
    TraceScope trace_(st, "attn_bwd_delta_kernel");
    hipLaunchKernelGGL((flash::attn_bwd_q_kernel<D, 0>), dim3(nq), dim3(SQ::THREADS), 0, st, qkv, dO, lse, dqkv,
                       delta, rd, qpart, p, wq);
    TPS_TRY(check_launch("attn_bwd_delta_kernel"));
  }
  {
    TraceScope trace_(st, "attn_bwd_dq_kernel");
    hipLaunchKernelGGL((flash::attn_bwd_q_kernel<D, 1>), dim3(nq), dim3(SQ::THREADS), 0, st, qkv, dO, lse, dqkv,
                       delta, rd, qpart, p, wq);
    TPS_TRY(check_launch("attn_bwd_dq_kernel"));
  }
  {
    TraceScope trace_(st, "attn_bwd_dkv_kernel");
    hipLaunchKernelGGL((flash::attn_bwd_kv_kernel<D>), dim3(nk), dim3(SK::THREADS), 0, st, qkv, dO, lse, delta, dqkv,
                       kvpart, p, wk);
    TPS_TRY(check_launch("attn_bwd_dkv_kernel"));
  }
  const int mq = flash::work_merges_per_z(wq), mk = flash::work_merges_per_z(wk);
  const int nq_wg = mq > 0 ? flash::merge_workgroups(wq, mq, flash::merge_rows<D>()) : 0;
  const int nk_wg = mk > 0 ? flash::merge_workgroups(wk, mk, flash::merge_rows<2 * D>()) : 0;
  if (nq_wg + nk_wg > 0) {
    TraceScope trace_(st, "attn_bwd_merge_kernel");
    hipLaunchKernelGGL((flash::attn_bwd_merge_kernel<D>), dim3((unsigned)(nq_wg + nk_wg)), dim3(flash::kMergeThreads),
                       0, st, qpart, kvpart, dqkv, p, wq, mq, wk, mk, nq_wg);
    TPS_TRY(check_launch("attn_bwd_merge_kernel"));
  }
  return TPS_OK;
}

extern "C" tps_status tp_attn_bwd(tps_dtype dt, int64_t b, int64_t sq, int64_t h, int64_t hs, int64_t d, int causal,
                                  const void* X, const void* Wqkv_i, const void* Wo_i, const void* QKV_i,
                                  const void* O_i, const float* lse_i, const void* dZ, void* dX_i, void* dWqkv_i,
                                  void* dWo_i, void* ws, size_t ws_bytes, tps_stream_t stream) {
  ApiScope api_scope_("tp_attn_bwd");
  TPS_TRY(attn_checks("tp_attn_bwd", dt, b, sq, h, hs, d,
                      {X, Wqkv_i, Wo_i, QKV_i, O_i, lse_i, dZ, dX_i, dWqkv_i, dWo_i, ws}));
  if (use_flash_bwd(d)) {
    const char* fn = "tp_attn_bwd";
    // the kernels' per-lane tile offsets (32 rows of QKV) are 32-bit
    TPS_REQ(3 * hs * d <= (1LL << 25), "3 hs d must be <= 2^25");
    flash::BwdWork wq, wk;
    flash_bwd_works_d(d, b, sq, hs, causal ? 1 : 0, wq, wk);
    const AttnFlashBwdWs L = attn_flash_bwd_ws_layout(b, sq, hs, d, wq, wk);
    if (ws_bytes < L.total) return set_error(TPS_EWORKSPACE, "tp_attn_bwd: workspace too small");
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t M = b * sq, w = hs * d, w3 = 3 * w;
    char* base = static_cast<char*>(ws);
    bf16_t* dO = (bf16_t*)(base + L.dO);
    bf16_t* dQKV = (bf16_t*)(base + L.dQKV);
    const bf16_t* qkv = (const bf16_t*)QKV_i;
    const bf16_t* dz = (const bf16_t*)dZ;
    // dWo_i = O_i^T dZ                     (TN)  [w x h], K = M
    TPS_TRY((gemm_bf16<false, false>((const bf16_t*)O_i, dz, shape(w, h, M, w, h),
                                     EpiStore<bf16_t>{(bf16_t*)dWo_i, h, 0, 0}, st)));
    // dO = dZ Wo_i^T                       (NT)  [M x w], K = h
    TPS_TRY((gemm_bf16<true, true>(dz, (const bf16_t*)Wo_i, shape(M, w, h, h, h), EpiStore<bf16_t>{dO, w, 0, 0}, st)));
    const flash::BwdPlan p = flash::make_bwd_plan(b, sq, hs, (int)d, causal ? 1 : 0);
    if (d == 64) TPS_TRY(flash_bwd_core<64>(qkv, dO, lse_i, dQKV, base, L, p, wq, wk, st));
    else if (d == 128) TPS_TRY(flash_bwd_core<128>(qkv, dO, lse_i, dQKV, base, L, p, wq, wk, st));
    else TPS_TRY(flash_bwd_core<256>(qkv, dO, lse_i, dQKV, base, L, p, wq, wk, st));
    // dWqkv_i = X^T dQKV                   (TN)  [h x 3w], K = M
    TPS_TRY((gemm_bf16<false, false>((const bf16_t*)X, dQKV, shape(h, w3, M, h, w3),
                                     EpiStore<bf16_t>{(bf16_t*)dWqkv_i, w3, 0, 0}, st)));
    // dX_i = dQKV Wqkv_i^T                 (NT)  [M x h], K = 3w
    return gemm_bf16<true, true>(dQKV, (const bf16_t*)Wqkv_i, shape(M, h, w3, w3, w3),
                                 EpiStore<bf16_t>{(bf16_t*)dX_i, h, 0, 0}, st);
  }
  const AttnWs L = attn_ws_layout(b, sq, hs, d);
  if (ws_bytes < L.total) return set_error(TPS_EWORKSPACE, "tp_attn_bwd: workspace too small");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t M = b * sq, w = hs * d, w3 = 3 * w;
  char* base = static_cast<char*>(ws);
  bf16_t* dO = (bf16_t*)(base + L.dO);
  bf16_t* P = (bf16_t*)(base + L.P);
  float* dP = (float*)(base + L.dP);
  bf16_t* dS = (bf16_t*)(base + L.dS);
  bf16_t* dQKV = (bf16_t*)(base + L.dQKV);
  const bf16_t* qkv = (const bf16_t*)QKV_i;
  const bf16_t* o = (const bf16_t*)O_i;
  const bf16_t* dz = (const bf16_t*)dZ;
  const float scale = 1.f / sqrtf((float)d);
  const int64_t ldp = L.ldp, sp = sq * L.ldp;

  // dWo_i = O_i^T dZ                       (TN)  [w x h], K = M
  TPS_TRY((gemm_bf16<false, false>(o, dz, shape(w, h, M, w, h), EpiStore<bf16_t>{(bf16_t*)dWo_i, h, 0, 0}, st)));
  // dO = dZ Wo_i^T                         (NT)  [M x w], K = h
  TPS_TRY((gemm_bf16<true, true>(dz, (const bf16_t*)Wo_i, shape(M, w, h, h, h), EpiStore<bf16_t>{dO, w, 0, 0}, st)));
  // Per (batch, head) problems: z = bi*hs + j.
  GemmShape s = shape(sq, sq, d, w3, w3);
  s.batch = (int)(b * hs);
  s.batch_inner = (int)hs;
  s.sa_o = sq * w3; s.sa_i = d; s.sb_o = sq * w3; s.sb_i = d;
  s.skip_upper = causal ? 1 : 0;
  s.skip_pad = kProbPad;   // P: zeros up to the causal pad, nothing beyond
  s.live_tiles = 1;        // tile shape by the live tiles: every CU shares the exp epilogue
  // P = exp(Q K^T * scale - lse)           (NT)  [sq x sq] per head
  TPS_TRY((gemm_bf16<true, true>(qkv, qkv + w, s,
                                 EpiAttnProb<bf16_t>{P, lse_i, ldp, sp, (int)sq, (int)hs, causal ? 1 : 0,
                                                     scale * 1.4426950408889634f},
                                 st)));
  // dP = dO V^T (fp32)                    (NT)  [sq x sq] per head
  GemmShape s2 = s;
  s2.lda = w; s2.sa_o = sq * w; s2.sa_i = d;
  s2.skip_pad = 1;   // dP is read only up to the diagonal
  s2.live_tiles = 0;
  TPS_TRY((gemm_bf16<true, true>(dO, qkv + 2 * w, s2, EpiStore<float>{dP, ldp, hs * sp, sp}, st)));
  // dS = P * (dP - delta) * scale with delta from the same P and dP
  TPS_TRY(([&]() {
    TraceScope trace_(st, "attn_ds_kernel");
    hipLaunchKernelGGL(attn_ds_kernel, dim3((unsigned)ceil_div(b * hs * sq, 4)), dim3(256), 0, st, P, dP, dS,
                       b * hs * sq, (int)sq, ldp, causal ? 1 : 0, scale);
    return check_launch("attn_ds_kernel");
  }()));
  // dV = P^T dO                            (TN)  [sq x d] per head, K = queries >= key
  // dK = dS^T Q                            (TN)  [sq x d] per head
  // One launch, longest K ranges first: the short tiles of either fill the
  // CUs left idle by the long ones.
  GemmShape s3 = shape(sq, d, sq, ldp, w);
  s3.batch = (int)(b * hs); s3.batch_inner = (int)hs;
  s3.sa_o = hs * sp; s3.sa_i = sp; s3.sb_o = sq * w; s3.sb_i = d;
  s3.kmode = causal ? 2 : 0;
  s3.groups = 2;
  s3.lpt = 1;
  const GemmAlt<EpiStore<bf16_t>> dk{dS, qkv, ldp, w3, hs * sp, sp, sq * w3, d,
                                     EpiStore<bf16_t>{dQKV + w, w3, sq * w3, d}};
  TPS_TRY((gemm_bf16<false, false>(P, dO, s3, EpiStore<bf16_t>{dQKV + 2 * w, w3, sq * w3, d}, dk, st)));
  // dQ = dS K                              (NN)  [sq x d] per head, K = keys <= query
  GemmShape s5 = shape(sq, d, sq, ldp, w3);
  s5.batch = (int)(b * hs); s5.batch_inner = (int)hs;
  s5.sa_o = hs * sp; s5.sa_i = sp; s5.sb_o = sq * w3; s5.sb_i = d;
  s5.kmode = causal ? 1 : 0;
  TPS_TRY((gemm_bf16<true, false>(dS, qkv + w, s5, EpiStore<bf16_t>{dQKV, w3, sq * w3, d}, st)));
  // dWqkv_i = X^T dQKV                     (TN)  [h x 3w], K = M
  TPS_TRY((gemm_bf16<false, false>((const bf16_t*)X, dQKV, shape(h, w3, M, h, w3),
                                   EpiStore<bf16_t>{(bf16_t*)dWqkv_i, w3, 0, 0}, st)));
  // dX_i = dQKV Wqkv_i^T                   (NT)  [M x h], K = 3w
  return gemm_bf16<true, true>(dQKV, (const bf16_t*)Wqkv_i, shape(M, h, w3, w3, w3),
                               EpiStore<bf16_t>{(bf16_t*)dX_i, h, 0, 0}, st);
}
