// The full input embedding (page "5-megatron", section Embedding) and
// dropout.
//
// embedding_fwd: out = dropout(sum_r word_r + PE[pos] (+ TE[tt])).  The word
//   embedding's shard partials (vocab_embed_fwd) are summed in shard order in
//   fp32, the position row and the token-type row are added, and dropout is
//   applied once: the same mask holds on every shard, since it comes after
//   the shard sum (page "5-megatron", section 模型并行).
// dropout_apply: y = keep ? x / (1 - p) : 0.  It is also the backward of
//   both: the mask is regenerated from the seed, so nothing is stored.
//
// The mask comes from the counter-based generator Philox4x32-10 (Salmon,
// Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3",
// SC 2011): element e of a call uses word e % 4 of the generator at counter
// (e / 4 as two 32-bit words, 0, 0) and key (seed as two 32-bit words), and
// is dropped when that word is below floor(p * 2^32).  Both kernels are
// HBM-bound (8 elements per thread, 16-byte vectors); two generator blocks
// per 8 elements.
#include <string>

#include "common.hpp"

namespace tps {

namespace {

// One Philox4x32 evaluation with 10 rounds: per round the words 0 and 2 are
// multiplied by the two round multipliers into 64-bit products, the counter
// becomes (hi(c2 M1) ^ c1 ^ k0, lo(c2 M1), hi(c0 M0) ^ c3 ^ k1, lo(c0 M0)),
// and the key advances by the two Weyl constants.
__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    // one 32x32 -> 64-bit multiply gives both halves
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0], p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

struct DropParams {
  uint32_t thr;     // drop when the word is below this (0: keep everything)
  float scale;      // 1 / (1 - p)
  uint32_t k0, k1;  // the seed's two words
};

// keep flags of the 8 elements starting at e (a multiple of 8): blocks e/4, e/4+1
__device__ __forceinline__ void keep8(int64_t e, const DropParams& d, bool k[8]) {
  const uint64_t b = (uint64_t)e >> 2;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t c[4] = {(uint32_t)(b + h), (uint32_t)((b + h) >> 32), 0u, 0u};
    philox4x32_10(c, d.k0, d.k1);
#pragma unroll
    for (int j = 0; j < 4; ++j) k[4 * h + j] = c[j] >= d.thr;
  }
}

struct WordParts {
  const void* p[8];
};

template <typename T, typename To>
__global__ void __launch_bounds__(256) embedding_fwd_kernel(WordParts parts, int np, const T* __restrict__ PE,
                                                            int64_t pos_rows, const int32_t* __restrict__ pos,
                                                            const T* __restrict__ TE, int64_t tt_rows,
                                                            const int32_t* __restrict__ tt, DropParams d,
                                                            To* __restrict__ out, int64_t T_, int64_t H) {
  const int64_t nvec = T_ * H / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
    const int64_t e = v * 8, t = e / H, col = e - t * H;
    float acc[8], x[8];
    load8<T>(static_cast<const T*>(parts.p[0]) + e, acc, 8);
    for (int r = 1; r < np; ++r) {
      load8<T>(static_cast<const T*>(parts.p[r]) + e, x, 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += x[i];
    }
    const int64_t ps = pos[t];
    if (ps >= 0 && ps < pos_rows) {   // an id outside the table adds a zero row
      load8<T>(PE + ps * H + col, x, 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += x[i];
    }
    if (TE) {
      const int64_t ty = tt[t];
      if (ty >= 0 && ty < tt_rows) {
        load8<T>(TE + ty * H + col, x, 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += x[i];
      }
    }
    if (d.thr) {
      bool k[8];
      keep8(e, d, k);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = k[i] ? acc[i] * d.scale : 0.f;
    }
    store8<To>(out + e, acc, 8);
  }
}

template <typename Ti, typename To>
__global__ void __launch_bounds__(256) dropout_kernel(const Ti* __restrict__ x, To* __restrict__ y, int64_t n,
                                                      DropParams d) {
  const int64_t nvec = (n + 7) / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
    const int64_t e = v * 8;
    const int nv = (int)(n - e < 8 ? n - e : 8);
    float a[8];
    load8<Ti>(x + e, a, nv);
    bool k[8];
    keep8(e, d, k);
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = k[i] ? a[i] * d.scale : 0.f;
    store8<To>(y + e, a, nv);
  }
}

tps_status drop_params(const char* fn, float p, uint64_t seed, DropParams& d) {
  if (!(p >= 0.f && p < 1.f)) return set_error(TPS_EINVAL, std::string(fn) + ": p must be in [0, 1)");
  const double t = (double)p * 4294967296.0;
  d.thr = t >= 4294967295.0 ? 0xFFFFFFFFu : (uint32_t)t;
  d.scale = 1.0f / (1.0f - p);
  d.k0 = (uint32_t)seed;
  d.k1 = (uint32_t)(seed >> 32);
  return TPS_OK;
}

dim3 grid_vec(int64_t n) {
  int64_t blocks = ceil_div((n + 7) / 8, 256);
  if (blocks > 65536) blocks = 65536;
  return dim3((unsigned)(blocks > 0 ? blocks : 1));
}

bool dt_ok(tps_dtype d) { return d == TPS_F32 || d == TPS_BF16; }

}  // namespace

}  // namespace tps

using namespace tps;

extern "C" tps_status embedding_fwd(tps_dtype dt, tps_dtype out_dt, int n_parts, const void* const* word_parts,
                                    const void* PE, int64_t pos_rows, const int32_t* pos, const void* TE,
                                    int64_t tt_rows, const int32_t* tt, float p, uint64_t seed, void* out,
                                    int64_t T, int64_t H, tps_stream_t stream) {
  ApiScope api_scope_("embedding_fwd");
  const char* fn = "embedding_fwd";
  if (!dt_ok(dt) || !dt_ok(out_dt)) return set_error(TPS_EINVAL, "embedding_fwd: bad dtype");
  if (n_parts < 1 || n_parts > 8) return set_error(TPS_EINVAL, "embedding_fwd: n_parts must be 1..8");
  if (T < 0 || H <= 0 || H % 8 || pos_rows <= 0 || (TE && tt_rows <= 0))
    return set_error(TPS_EINVAL, "embedding_fwd: need T >= 0, H a positive multiple of 8, table rows > 0");
  if (!word_parts || !PE || !pos || !out || (TE && !tt))
    return set_error(TPS_EINVAL, "embedding_fwd: null pointer");
  WordParts wp{};
  for (int r = 0; r < n_parts; ++r) {
    if (!word_parts[r] || !aligned16(word_parts[r]))
      return set_error(TPS_EINVAL, "embedding_fwd: word partials must be non-null and 16-byte aligned");
    wp.p[r] = word_parts[r];
  }
  if (!aligned16(PE) || !aligned16(out) || (TE && !aligned16(TE)))
    return set_error(TPS_EINVAL, "embedding_fwd: pointers must be 16-byte aligned");
  DropParams d;
  tps_status s = drop_params(fn, p, seed, d);
  if (s != TPS_OK) return s;
  if (T == 0) return TPS_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid = grid_vec(T * H);
#define TPS_EF(TT, TO)                                                                                       \
  hipLaunchKernelGGL((embedding_fwd_kernel<TT, TO>), grid, dim3(256), 0, st, wp, n_parts,                    \
                     static_cast<const TT*>(PE), pos_rows, pos, static_cast<const TT*>(TE), tt_rows, tt, d, \
                     static_cast<TO*>(out), T, H)
  if (dt == TPS_BF16 && out_dt == TPS_BF16) TPS_EF(bf16_t, bf16_t);
  else if (dt == TPS_BF16) TPS_EF(bf16_t, float);
  else if (out_dt == TPS_BF16) TPS_EF(float, bf16_t);
  else TPS_EF(float, float);
#undef TPS_EF
  return check_launch("embedding_fwd_kernel");
}

extern "C" tps_status dropout_apply(tps_dtype in_dt, tps_dtype out_dt, int64_t n, const void* x, float p,
                                    uint64_t seed, void* y, tps_stream_t stream) {
  ApiScope api_scope_("dropout_apply");
  const char* fn = "dropout_apply";
  if (!dt_ok(in_dt) || !dt_ok(out_dt)) return set_error(TPS_EINVAL, "dropout_apply: bad dtype");
  if (n < 0) return set_error(TPS_EINVAL, "dropout_apply: n < 0");
  if (!x || !y) return set_error(TPS_EINVAL, "dropout_apply: null pointer");
  if (!aligned16(x) || !aligned16(y)) return set_error(TPS_EINVAL, "dropout_apply: pointers must be 16-byte aligned");
  DropParams d;
  tps_status s = drop_params(fn, p, seed, d);
  if (s != TPS_OK) return s;
  if (n == 0) return TPS_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid = grid_vec(n);
#define TPS_DA(TI, TO) \
  hipLaunchKernelGGL((dropout_kernel<TI, TO>), grid, dim3(256), 0, st, static_cast<const TI*>(x), static_cast<TO*>(y), n, d)
  if (in_dt == TPS_BF16 && out_dt == TPS_BF16) TPS_DA(bf16_t, bf16_t);
  else if (in_dt == TPS_BF16) TPS_DA(bf16_t, float);
  else if (out_dt == TPS_BF16) TPS_DA(float, bf16_t);
  else TPS_DA(float, float);
#undef TPS_DA
  return check_launch("dropout_kernel");
}
