// Attention shard: QKV column-parallel by heads, per-head softmax attention,
// row-parallel output projection.
//
// Forward core: flash-style kernel, one workgroup per (batch, head, 64-query
// block), four wavefronts of 16 queries.  Each wavefront keeps its queries'
// Q fragments in registers and accumulates O^T (head dim x queries) in
// registers while streaming 32-key blocks of K and V^T through LDS with an
// online softmax.  The transposed formulation S^T = K Q^T makes the MFMA
// result layout (one query per lane column) directly usable as the B operand
// of O^T += V^T P^T, so P never leaves registers and the per-query softmax
// rescale is lane-local.  Saves lse = log(sum exp(S)) per query.
//
// Backward core: the probabilities are recomputed from lse tile by tile by
// the GEMM kernel (epilogue exp(S*scale - lse)) and written to the workspace
// in bf16; dP = dO V^T is a GEMM into fp32 and a row pass forms
// dS = P * (dP - delta) * scale with delta taken from the same P and dP;
// dV = P^T dO, dQ = dS K and dK = dS^T Q are then MFMA GEMMs whose K-loops
// skip the causally-zero blocks.  The workspace holds O(sq^2) per head, which the
// 288 GB of HBM per device affords at these sequence lengths.
#include <string>

#include "gemm.hpp"

namespace tps {

constexpr int kFlashBQ = 64;    // queries per workgroup: 4 query groups of 16
constexpr int kFlashBKey = 32;  // keys per LDS block
constexpr int kFlashThreads = 512;  // 8 waves: (query group, half of the head dim)
// The running max used as the softmax reference is only raised when a row's
// block max exceeds it by more than this many powers of two (log2 domain):
// numerator and denominator share the reference, so the result is exact and
// every exp2 stays below 2^kLazyRescale.
constexpr float kLazyRescale = 8.f;

// LDS stage: one K block (keys x head dim) and one V^T block (head dim x keys).
template <int D>
struct FlashStage {
  static constexpr int KLD = D + 8;           // LDS row stride of K (elements)
  static constexpr int VLD = kFlashBKey + 8;  // LDS row stride of V^T
  static constexpr int K_ELEMS = kFlashBKey * KLD;
  static constexpr int ELEMS = K_ELEMS + D * VLD;
  static constexpr int K_CHUNKS = kFlashBKey * (D / 8);         // 16-byte chunks of K
  static constexpr int V_BLOCKS = (kFlashBKey / 8) * (D / 8);   // 8x8 blocks of V
  // Threads [0, V_THREADS) transpose V blocks, the others copy K chunks.
  static constexpr int V_THREADS = V_BLOCKS < kFlashThreads / 2 ? V_BLOCKS : kFlashThreads / 2;
  static constexpr int VB = (V_BLOCKS + V_THREADS - 1) / V_THREADS;
  static constexpr int K_THREADS = kFlashThreads - V_THREADS;
  static constexpr int KV = (K_CHUNKS + K_THREADS - 1) / K_THREADS;
  static constexpr int REGS = (KV > 8 * VB ? KV : 8 * VB);
};

// Register staging of the next K/V block (global -> registers during the
// current block's MFMAs, registers -> the other LDS stage afterwards).
template <int D>
struct FlashPrefetch {
  using S = FlashStage<D>;
  u32x4_t r[S::REGS];

  __device__ __forceinline__ void load(const bf16_t* Kp, const bf16_t* Vp, int64_t ld, int k0, int sq, int tid) {
    if (tid < S::V_THREADS) {
#pragma unroll
      for (int b = 0; b < S::VB; ++b) {
        const int blk = tid + b * S::V_THREADS;
        const int kq = blk % (kFlashBKey / 8), db = blk / (kFlashBKey / 8);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int key = k0 + kq * 8 + jj;
          u32x4_t x = {0u, 0u, 0u, 0u};
          if (blk < S::V_BLOCKS && key < sq) x = *reinterpret_cast<const u32x4_t*>(Vp + (int64_t)key * ld + db * 8);
          r[b * 8 + jj] = x;
        }
      }
    } else {
      const int t = tid - S::V_THREADS;
#pragma unroll
      for (int i = 0; i < S::KV; ++i) {
        const int c = t + i * S::K_THREADS;
        const int row = c / (D / 8), cc = (c % (D / 8)) * 8;
        const int key = k0 + row;
        u32x4_t x = {0u, 0u, 0u, 0u};
        if (c < S::K_CHUNKS && key < sq) x = *reinterpret_cast<const u32x4_t*>(Kp + (int64_t)key * ld + cc);
        r[i] = x;
      }
    }
  }

  __device__ __forceinline__ void store(bf16_t* st, int tid) const {
    if (tid < S::V_THREADS) {
      bf16_t* vts = st + S::K_ELEMS;
#pragma unroll
      for (int b = 0; b < S::VB; ++b) {
        const int blk = tid + b * S::V_THREADS;
        if (blk >= S::V_BLOCKS) continue;
        const int kq = blk % (kFlashBKey / 8), db = blk / (kFlashBKey / 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int w = i >> 1;
          const bool hi = i & 1;
          u32x4_t o;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t a = r[b * 8 + 2 * q][w], c = r[b * 8 + 2 * q + 1][w];
            o[q] = hi ? ((a >> 16) | (c & 0xffff0000u)) : ((a & 0xffffu) | (c << 16));
          }
          *reinterpret_cast<u32x4_t*>(vts + (db * 8 + i) * S::VLD + kq * 8) = o;
        }
      }
    } else {
      const int t = tid - S::V_THREADS;
#pragma unroll
      for (int i = 0; i < S::KV; ++i) {
        const int c = t + i * S::K_THREADS;
        if (c < S::K_CHUNKS) {
          const int row = c / (D / 8), cc = (c % (D / 8)) * 8;
          *reinterpret_cast<u32x4_t*>(st + row * S::KLD + cc) = r[i];
        }
      }
    }
  }
};

// One workgroup per (batch, head, 64-query block); 8 waves.  Wave w handles
// the 16 queries of group w % 4 and accumulates the head-dim half w / 4 of
// O^T = V^T P^T; both waves of a group compute the same S^T = K Q^T (with the
// group's Q fragments in registers) and the same online-softmax statistics.
// The transposed formulation makes the S^T result layout (one query per lane
// column) directly the B operand of the PV MFMA, so P never leaves registers
// and the per-query rescale is lane-local.  K and V^T blocks are double
// buffered in LDS; the next block is fetched into registers while the current
// one is consumed.  Saves lse = log(sum exp(S)) per query for the backward.
template <int D>
__global__ void __launch_bounds__(kFlashThreads, 1)
flash_fwd_kernel(const bf16_t* __restrict__ qkv, bf16_t* __restrict__ out, float* __restrict__ lse, int sq,
                 int hs, int causal, float scale_log2) {
  using S = FlashStage<D>;
  constexpr int DK = D / 32;             // MFMA k-steps over the head dim
  constexpr int DH = D / 2;              // head-dim half accumulated per wave
  constexpr int DT = DH / 16;            // 16-row tiles of this wave's O^T
  constexpr int NCH = DK >= 2 ? 2 : 1;   // independent partial sums per S tile
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * S::ELEMS];

  const int64_t ld = 3LL * hs * D;       // row stride of QKV
  const int64_t ldo = (int64_t)hs * D;   // row stride of O
  const int nqb = (sq + kFlashBQ - 1) / kFlashBQ;
  const int id = blockIdx.x;
  const int qb = nqb - 1 - (id % nqb);   // heaviest (last) query blocks first
  const int rest = id / nqb;
  const int j = rest % hs, bi = rest / hs;
  const bf16_t* Qp = qkv + (int64_t)bi * sq * ld + (int64_t)j * D;
  const bf16_t* Kp = Qp + (int64_t)hs * D;
  const bf16_t* Vp = Qp + 2LL * hs * D;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qg = wave & 3, dh = wave >> 2;
  const int g = lane >> 4;                       // lane group 0..3
  const int myq = qb * kFlashBQ + qg * 16 + (lane & 15);

  // Q^T fragments (B operand): column = my query, k = head-dim slice.
  bf16x8_t qf[DK];
#pragma unroll
  for (int kk = 0; kk < DK; ++kk) {
    u32x4_t x = {0u, 0u, 0u, 0u};
    if (myq < sq) x = *reinterpret_cast<const u32x4_t*>(Qp + (int64_t)myq * ld + kk * 32 + g * 8);
    qf[kk] = __builtin_bit_cast(bf16x8_t, x);
  }
  f32x4_t oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int kend = causal ? min(sq, (qb + 1) * kFlashBQ) : sq;
  const int nkb = (kend + kFlashBKey - 1) / kFlashBKey;
  FlashPrefetch<D> pf;
  pf.load(Kp, Vp, ld, 0, sq, tid);
  pf.store(lds, tid);
  __syncthreads();

  for (int kb = 0; kb < nkb; ++kb) {
    const int k0 = kb * kFlashBKey;
    const bf16_t* st = lds + (kb & 1) * S::ELEMS;
    const bool more = kb + 1 < nkb;
    if (more) pf.load(Kp, Vp, ld, k0 + kFlashBKey, sq, tid);   // lands during this block's MFMAs

    // S^T tiles: rows = 16 keys, column = this lane's query.
    f32x4_t sp[2][NCH];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int c = 0; c < NCH; ++c) sp[t][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8_t kf =
            *reinterpret_cast<const bf16x8_t*>(st + (t * 16 + (lane & 15)) * S::KLD + g * 8 + kk * 32);
        sp[t][kk % NCH] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[kk], sp[t][kk % NCH], 0, 0, 0);
      }
    // Online softmax in the log2 domain.  Element e of tile t is key
    // k0 + 16t + 4g + e.
    float sv[8];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = 0.f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) x += sp[t][c][e];
        const int key = k0 + t * 16 + g * 4 + e;
        x *= scale_log2;
        if (key >= sq || (causal && key > myq)) x = -INFINITY;
        sv[t * 4 + e] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // Raise the reference (and rescale O) only when a row's max outgrew it;
    // the first block always raises it from -inf (key 0 is never masked).
    const bool grow = mx > m_run + kLazyRescale;
    if (__ballot(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = grow ? exp2f(m_run - m_new) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        oacc[t][0] *= alpha; oacc[t][1] *= alpha; oacc[t][2] *= alpha; oacc[t][3] *= alpha;
      }
      m_run = m_new;
    }
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sv[i] = exp2f(sv[i] - m_run);
      rs += sv[i];
    }
    rs += __shfl_xor(rs, 16);
    rs += __shfl_xor(rs, 32);
    l_run += rs;
    // P^T as the B operand: k-slots 0..3 = keys 4g..4g+3, 4..7 = keys 16+4g..16+4g+3.
    const u32x4_t pw = {pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3]), pack_bf16x2(sv[4], sv[5]),
                        pack_bf16x2(sv[6], sv[7])};
    const bf16x8_t pfrag = __builtin_bit_cast(bf16x8_t, pw);
    // O^T (this wave's head-dim half) += V^T P^T; A fragment in pfrag's key order.
    const bf16_t* vts = st + S::K_ELEMS + dh * DH * S::VLD;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const bf16_t* vrow = vts + (t * 16 + (lane & 15)) * S::VLD + g * 4;
      const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vrow);
      const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vrow + 16);
      const u32x4_t vw = {lo[0], lo[1], hi[0], hi[1]};
      oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vw), pfrag, oacc[t], 0, 0, 0);
    }
    if (more) pf.store(lds + ((kb + 1) & 1) * S::ELEMS, tid);
    __syncthreads();
  }

  if (myq < sq) {
    const float inv = 1.f / l_run;
    bf16_t* orow = out + ((int64_t)bi * sq + myq) * ldo + (int64_t)j * D + dh * DH;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const float v[4] = {oacc[t][0] * inv, oacc[t][1] * inv, oacc[t][2] * inv, oacc[t][3] * inv};
      store4<bf16_t>(orow + t * 16 + g * 4, v, 4);
    }
    if (g == 0 && dh == 0) lse[((int64_t)bi * hs + j) * sq + myq] = (m_run + log2f(l_run)) * 0.69314718055994531f;
  }
}

// One wavefront per row of one (batch, head): with P the stored (bf16)
// probabilities and dP = dO V^T (fp32), delta = sum_j P_j dP_j / sum_j P_j and
// dS_j = P_j (dP_j - delta) * scale.  Taking delta from the same P and dP
// makes every row of dS sum to zero (the softmax gradient of the stored P),
// so the rounding of O and dO does not leak into dQ as a per-row bias.
// Columns at or beyond the causal limit (and beyond sq) are written as 0.
__global__ void __launch_bounds__(256) attn_ds_kernel(const bf16_t* __restrict__ P, const float* __restrict__ dP,
                                                      bf16_t* __restrict__ dS, int64_t rows, int sq, int64_t ldp,
                                                      int causal, float scale) {
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= rows) return;
  const int lane = threadIdx.x & 63;
  const int i = (int)(w % sq);                    // query index within its head
  const int ncol = causal ? i + 1 : sq;
  const bf16_t* pr = P + w * ldp;
  const float* dpr = dP + w * ldp;
  bf16_t* dsr = dS + w * ldp;
  float num = 0.f, den = 0.f;
  for (int c = lane * 8; c < ncol; c += 64 * 8) {
    float p[8], d[8];
    load8<bf16_t>(pr + c, p, min(8, ncol - c));
    load8<float>(dpr + c, d, min(8, ncol - c));
#pragma unroll
    for (int e = 0; e < 8; ++e) { num += p[e] * d[e]; den += p[e]; }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) { num += __shfl_xor(num, o); den += __shfl_xor(den, o); }
  const float delta = den > 0.f ? num / den : 0.f;
  for (int c = lane * 8; c < sq; c += 64 * 8) {
    const int nv = min(8, sq - c);
    float p[8], d[8], o[8];
    load8<bf16_t>(pr + c, p, nv);
    load8<float>(dpr + c, d, nv);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (c + e < ncol) ? p[e] * (d[e] - delta) * scale : 0.f;
    store8<bf16_t>(dsr + c, o, nv);
  }
}

template <int D>
static tps_status launch_flash_fwd(const bf16_t* qkv, bf16_t* out, float* lse, int64_t b, int64_t sq, int64_t hs,
                                   int causal, hipStream_t st) {
  const int64_t grid = ceil_div(sq, kFlashBQ) * hs * b;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  hipLaunchKernelGGL(flash_fwd_kernel<D>, dim3((unsigned)grid), dim3(kFlashThreads), 0, st, qkv, out, lse, (int)sq,
                     (int)hs,
                     causal, scale_log2);
  return check_launch("flash_fwd_kernel");
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
  if (d != 64 && d != 128 && d != 256 && d != 512)
    return set_error(TPS_EUNSUPPORTED, std::string(fn) + ": head dim must be 64, 128, 256 or 512");
  return TPS_OK;
}

}  // namespace tps

using namespace tps;

extern "C" tps_status tp_attn_fwd(tps_dtype dt, int64_t b, int64_t sq, int64_t h, int64_t hs, int64_t d, int causal,
                                  const void* X, const void* Wqkv_i, const void* Wo_i, void* QKV_i, void* O_i,
                                  float* lse_i, void* Z_i, tps_stream_t stream) {
  TPS_TRY(attn_checks("tp_attn_fwd", dt, b, sq, h, hs, d, {X, Wqkv_i, Wo_i, QKV_i, O_i, lse_i, Z_i}));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t M = b * sq, w = hs * d;
  const bf16_t* x = (const bf16_t*)X;
  bf16_t* qkv = (bf16_t*)QKV_i;
  bf16_t* o = (bf16_t*)O_i;
  // QKV_i = X Wqkv_i                       (NN)
  TPS_TRY((gemm_bf16<true, false>(x, (const bf16_t*)Wqkv_i, shape(M, 3 * w, h, h, 3 * w),
                                  EpiStore<bf16_t>{qkv, 3 * w, 0, 0}, st)));
  tps_status s;
  switch (d) {
    case 64: s = launch_flash_fwd<64>(qkv, o, lse_i, b, sq, hs, causal ? 1 : 0, st); break;
    case 128: s = launch_flash_fwd<128>(qkv, o, lse_i, b, sq, hs, causal ? 1 : 0, st); break;
    case 256: s = launch_flash_fwd<256>(qkv, o, lse_i, b, sq, hs, causal ? 1 : 0, st); break;
    default: s = launch_flash_fwd<512>(qkv, o, lse_i, b, sq, hs, causal ? 1 : 0, st); break;
  }
  TPS_TRY(s);
  // Z_i = O_i Wo_i                         (NN)
  return gemm_bf16<true, false>(o, (const bf16_t*)Wo_i, shape(M, h, w, w, h), EpiStore<bf16_t>{(bf16_t*)Z_i, h, 0, 0},
                                st);
}

extern "C" size_t tp_attn_bwd_workspace(tps_dtype dt, int64_t b, int64_t sq, int64_t h, int64_t hs, int64_t d) {
  (void)dt;
  (void)h;
  if (b <= 0 || sq <= 0 || hs <= 0 || d <= 0) return 0;
  return attn_ws_layout(b, sq, hs, d).total;
}

extern "C" tps_status tp_attn_bwd(tps_dtype dt, int64_t b, int64_t sq, int64_t h, int64_t hs, int64_t d, int causal,
                                  const void* X, const void* Wqkv_i, const void* Wo_i, const void* QKV_i,
                                  const void* O_i, const float* lse_i, const void* dZ, void* dX_i, void* dWqkv_i,
                                  void* dWo_i, void* ws, size_t ws_bytes, tps_stream_t stream) {
  TPS_TRY(attn_checks("tp_attn_bwd", dt, b, sq, h, hs, d,
                      {X, Wqkv_i, Wo_i, QKV_i, O_i, lse_i, dZ, dX_i, dWqkv_i, dWo_i, ws}));
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
  // P = exp(Q K^T * scale - lse)           (NT)  [sq x sq] per head
  TPS_TRY((gemm_bf16<true, true>(qkv, qkv + w, s,
                                 EpiAttnProb<bf16_t>{P, lse_i, ldp, sp, (int)sq, (int)hs, causal ? 1 : 0,
                                                     scale * 1.4426950408889634f},
                                 st)));
  // dP = dO V^T (fp32)                    (NT)  [sq x sq] per head
  GemmShape s2 = s;
  s2.lda = w; s2.sa_o = sq * w; s2.sa_i = d;
  TPS_TRY((gemm_bf16<true, true>(dO, qkv + 2 * w, s2, EpiStore<float>{dP, ldp, hs * sp, sp}, st)));
  // dS = P * (dP - delta) * scale with delta from the same P and dP
  hipLaunchKernelGGL(attn_ds_kernel, dim3((unsigned)ceil_div(b * hs * sq, 4)), dim3(256), 0, st, P, dP, dS,
                     b * hs * sq, (int)sq, ldp, causal ? 1 : 0, scale);
  TPS_TRY(check_launch("attn_ds_kernel"));
  // dV = P^T dO                            (TN)  [sq x d] per head, K = queries >= key
  GemmShape s3 = shape(sq, d, sq, ldp, w);
  s3.batch = (int)(b * hs); s3.batch_inner = (int)hs;
  s3.sa_o = hs * sp; s3.sa_i = sp; s3.sb_o = sq * w; s3.sb_i = d;
  s3.kmode = causal ? 2 : 0;
  TPS_TRY((gemm_bf16<false, false>(P, dO, s3, EpiStore<bf16_t>{dQKV + 2 * w, w3, sq * w3, d}, st)));
  // dK = dS^T Q                            (TN)  [sq x d] per head
  GemmShape s4 = s3;
  s4.ldb = w3; s4.sb_o = sq * w3; s4.sb_i = d;
  TPS_TRY((gemm_bf16<false, false>(dS, qkv, s4, EpiStore<bf16_t>{dQKV + w, w3, sq * w3, d}, st)));
  // dQ = dS K                              (NN)  [sq x d] per head, K = keys <= query
  GemmShape s5 = s4;
  s5.lda = ldp;
  s5.kmode = causal ? 1 : 0;
  TPS_TRY((gemm_bf16<true, false>(dS, qkv + w, s5, EpiStore<bf16_t>{dQKV, w3, sq * w3, d}, st)));
  // dWqkv_i = X^T dQKV                     (TN)  [h x 3w], K = M
  TPS_TRY((gemm_bf16<false, false>((const bf16_t*)X, dQKV, shape(h, w3, M, h, w3),
                                   EpiStore<bf16_t>{(bf16_t*)dWqkv_i, w3, 0, 0}, st)));
  // dX_i = dQKV Wqkv_i^T                   (NT)  [M x h], K = 3w
  return gemm_bf16<true, true>(dQKV, (const bf16_t*)Wqkv_i, shape(M, h, w3, w3, w3),
                               EpiStore<bf16_t>{(bf16_t*)dX_i, h, 0, 0}, st);
}
