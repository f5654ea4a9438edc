// Vocab-parallel word embedding, one shard.
//
// Forward (vocab_embed_fwd): a masked row gather.  One wavefront per token
// copies the table row (16-byte vectors) or writes zeros when the id falls
// outside [v_start, v_start + v_rows).  HBM-bound: reads the in-range rows
// once, writes every output row once.
//
// Backward (vocab_embed_bwd): dE_r[id - v_start] += dY[t] for in-range t.
// Deterministic and free of atomics: the composite keys (local_row << 32 | t)
// are unique, so sorting them (bitonic network) yields one fixed order, with
// each row's tokens contiguous and ascending in t.  One wavefront per segment
// head then sums that row's dY rows in fp32 in that order and adds the sum to
// dE_r with a plain read-modify-write (each row has exactly one owner).
#include "common.hpp"

namespace tps {

template <typename T>
__global__ void __launch_bounds__(256) embed_fwd_kernel(const int32_t* __restrict__ ids,
                                                         const T* __restrict__ E, T* __restrict__ Y,
                                                         int64_t ntok, int64_t H, int64_t v_start,
                                                         int64_t v_rows) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= ntok) return;
  const int lane = threadIdx.x & 63;
  const int64_t local = (int64_t)ids[t] - v_start;
  const bool inr = local >= 0 && local < v_rows;
  const int64_t nch = H * (int64_t)sizeof(T) / 16;  // 16-byte chunks per row
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(Y + t * H);
  if (inr) {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(E + local * H);
    for (int64_t c = lane; c < nch; c += 64) dst[c] = src[c];
  } else {
    const u32x4_t z = {0u, 0u, 0u, 0u};
    for (int64_t c = lane; c < nch; c += 64) dst[c] = z;
  }
}

// --- sort of composite keys ------------------------------------------------

constexpr uint64_t kNoKey = ~0ull;
constexpr int kSortChunk = 8192;  // keys sorted per workgroup in LDS (64 KiB)

__global__ void __launch_bounds__(256) embed_keys_kernel(const int32_t* __restrict__ ids, uint64_t* keys,
                                                         int64_t ntok, int64_t npad, int64_t v_start,
                                                         int64_t v_rows) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= npad) return;
  uint64_t k = kNoKey;
  if (p < ntok) {
    const int64_t local = (int64_t)ids[p] - v_start;
    if (local >= 0 && local < v_rows) k = ((uint64_t)local << 32) | (uint64_t)p;
  }
  keys[p] = k;
}

// Sorts (kouter == 0) or finishes the merge stage kouter (strides < chunk) of
// one chunk of `chunk` keys in LDS.  Direction of each compare-exchange comes
// from the global index so the chunks compose into one ascending network.
__global__ void __launch_bounds__(1024) bitonic_local_kernel(uint64_t* keys, int chunk, int64_t kouter) {
  __shared__ uint64_t s[kSortChunk];
  const int64_t base = (int64_t)blockIdx.x * chunk;
  for (int i = threadIdx.x; i < chunk; i += 1024) s[i] = keys[base + i];
  __syncthreads();
  const int half = chunk / 2;
  int64_t kfirst = kouter ? kouter : 2;
  int64_t klast = kouter ? kouter : chunk;
  for (int64_t k = kfirst; k <= klast; k <<= 1) {
    for (int j = (int)((kouter ? chunk : k) >> 1); j >= 1; j >>= 1) {
      for (int q = threadIdx.x; q < half; q += 1024) {
        const int i = 2 * j * (q / j) + (q % j);
        const int l = i + j;
        const bool asc = ((base + i) & k) == 0;
        const uint64_t a = s[i], b = s[l];
        if ((a > b) == asc) { s[i] = b; s[l] = a; }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < chunk; i += 1024) keys[base + i] = s[i];
}

__global__ void __launch_bounds__(256) bitonic_global_kernel(uint64_t* keys, int64_t n, int64_t k, int64_t j) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= n / 2) return;
  const int64_t i = 2 * j * (q / j) + (q % j);
  const int64_t l = i + j;
  const bool asc = (i & k) == 0;
  const uint64_t a = keys[i], b = keys[l];
  if ((a > b) == asc) { keys[i] = b; keys[l] = a; }
}

// One wavefront per sorted position; positions that start a row's segment sum
// that segment.  Columns are processed in slabs of 64 lanes x VEC elements.
template <typename T>
__global__ void __launch_bounds__(256) embed_bwd_accum_kernel(const uint64_t* __restrict__ keys,
                                                               const T* __restrict__ dY, float* dE,
                                                               int64_t ntok, int64_t H) {
  constexpr int VEC = 16 / sizeof(T);
  const int64_t p = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (p >= ntok) return;
  const uint64_t key = keys[p];
  if (key == kNoKey) return;
  const uint64_t row = key >> 32;
  if (p > 0 && (keys[p - 1] >> 32) == row) return;  // not the head of its segment
  const int lane = threadIdx.x & 63;
  int64_t end = p + 1;
  while (end < ntok && keys[end] != kNoKey && (keys[end] >> 32) == row) ++end;
  float* drow = dE + (int64_t)row * H;
  for (int64_t c0 = 0; c0 < H; c0 += 64 * VEC) {
    const int64_t c = c0 + lane * VEC;
    if (c >= H) continue;
    float acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
    for (int64_t q = p; q < end; ++q) {
      const int64_t t = (int64_t)(keys[q] & 0xffffffffu);
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(dY + t * H + c);
      if constexpr (VEC == 8) {
#pragma unroll
        for (int w = 0; w < 4; ++w) { acc[2 * w] += bf16lo(x[w]); acc[2 * w + 1] += bf16hi(x[w]); }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[w] += __uint_as_float(x[w]);
      }
    }
#pragma unroll
    for (int i = 0; i < VEC; i += 4) {
      f32x4_t* d = reinterpret_cast<f32x4_t*>(drow + c + i);
      f32x4_t o = *d;
      o[0] += acc[i]; o[1] += acc[i + 1]; o[2] += acc[i + 2]; o[3] += acc[i + 3];
      *d = o;
    }
  }
}

static int64_t next_pow2(int64_t x) {
  int64_t p = 1;
  while (p < x) p <<= 1;
  return p;
}

static tps_status sort_keys(uint64_t* keys, int64_t npad, hipStream_t st) {
  const int chunk = (int)(npad < kSortChunk ? npad : kSortChunk);
  const int64_t nchunks = npad / chunk;
  hipLaunchKernelGGL(bitonic_local_kernel, dim3((unsigned)nchunks), dim3(1024), 0, st, keys, chunk, (int64_t)0);
  for (int64_t k = 2 * (int64_t)chunk; k <= npad; k <<= 1) {
    for (int64_t j = k >> 1; j >= chunk; j >>= 1)
      hipLaunchKernelGGL(bitonic_global_kernel, dim3((unsigned)ceil_div(npad / 2, 256)), dim3(256), 0, st,
                         keys, npad, k, j);
    hipLaunchKernelGGL(bitonic_local_kernel, dim3((unsigned)nchunks), dim3(1024), 0, st, keys, chunk, k);
  }
  return check_launch("bitonic sort");
}

}  // namespace tps

using namespace tps;

static tps_status embed_common_checks(const char* fn, tps_dtype dt, int64_t T, int64_t H, int64_t v_start,
                                      int64_t v_rows) {
  if (dt != TPS_F32 && dt != TPS_BF16) return set_error(TPS_EINVAL, std::string(fn) + ": bad dtype");
  if (T < 0 || H <= 0 || v_rows <= 0 || v_start < 0)
    return set_error(TPS_EINVAL, std::string(fn) + ": need T >= 0, H > 0, v_rows > 0, v_start >= 0");
  if (H % vec_elems(dt)) return set_error(TPS_EINVAL, std::string(fn) + ": H must be a multiple of 8 (bf16) / 4 (fp32)");
  if (v_rows > 0x7fffffffLL || v_start > 0x7fffffffLL)
    return set_error(TPS_EINVAL, std::string(fn) + ": v_start and v_rows must fit in int32");
  return TPS_OK;
}

extern "C" tps_status vocab_embed_fwd(tps_dtype dt, int64_t T, int64_t H, int64_t v_start, int64_t v_rows,
                                      const int32_t* ids, const void* E_r, void* Y_r, tps_stream_t stream) {
  tps_status s = embed_common_checks("vocab_embed_fwd", dt, T, H, v_start, v_rows);
  if (s != TPS_OK) return s;
  if (!ids || !E_r || !Y_r) return set_error(TPS_EINVAL, "vocab_embed_fwd: null pointer");
  if (!aligned16(E_r) || !aligned16(Y_r)) return set_error(TPS_EINVAL, "vocab_embed_fwd: pointers must be 16-byte aligned");
  if (T == 0) return TPS_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)ceil_div(T, 4));
  if (dt == TPS_BF16)
    hipLaunchKernelGGL(embed_fwd_kernel<bf16_t>, grid, dim3(256), 0, st, ids, static_cast<const bf16_t*>(E_r),
                       static_cast<bf16_t*>(Y_r), T, H, v_start, v_rows);
  else
    hipLaunchKernelGGL(embed_fwd_kernel<float>, grid, dim3(256), 0, st, ids, static_cast<const float*>(E_r),
                       static_cast<float*>(Y_r), T, H, v_start, v_rows);
  return check_launch("embed_fwd_kernel");
}

extern "C" size_t vocab_embed_bwd_workspace(int64_t T, int64_t v_rows) {
  (void)v_rows;
  if (T <= 0) return 0;
  return (size_t)next_pow2(T) * sizeof(uint64_t);
}

extern "C" tps_status vocab_embed_bwd(tps_dtype dt, int64_t T, int64_t H, int64_t v_start, int64_t v_rows,
                                      const int32_t* ids, const void* dY, float* dE_r, void* ws,
                                      size_t ws_bytes, tps_stream_t stream) {
  tps_status s = embed_common_checks("vocab_embed_bwd", dt, T, H, v_start, v_rows);
  if (s != TPS_OK) return s;
  if (T >= 0x7fffffffLL) return set_error(TPS_EINVAL, "vocab_embed_bwd: T must be < 2^31");
  if (!ids || !dY || !dE_r) return set_error(TPS_EINVAL, "vocab_embed_bwd: null pointer");
  if (!aligned16(dY) || !aligned16(dE_r)) return set_error(TPS_EINVAL, "vocab_embed_bwd: pointers must be 16-byte aligned");
  if (T == 0) return TPS_OK;
  if (!ws) return set_error(TPS_EINVAL, "vocab_embed_bwd: null workspace");
  if (!aligned16(ws)) return set_error(TPS_EINVAL, "vocab_embed_bwd: workspace must be 16-byte aligned");
  if (ws_bytes < vocab_embed_bwd_workspace(T, v_rows))
    return set_error(TPS_EWORKSPACE, "vocab_embed_bwd: workspace too small");
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint64_t* keys = static_cast<uint64_t*>(ws);
  const int64_t npad = next_pow2(T);
  hipLaunchKernelGGL(embed_keys_kernel, dim3((unsigned)ceil_div(npad, 256)), dim3(256), 0, st, ids, keys, T, npad,
                     v_start, v_rows);
  s = check_launch("embed_keys_kernel");
  if (s != TPS_OK) return s;
  s = sort_keys(keys, npad, st);
  if (s != TPS_OK) return s;
  const dim3 grid((unsigned)ceil_div(T, 4));
  if (dt == TPS_BF16)
    hipLaunchKernelGGL(embed_bwd_accum_kernel<bf16_t>, grid, dim3(256), 0, st, keys,
                       static_cast<const bf16_t*>(dY), dE_r, T, H);
  else
    hipLaunchKernelGGL(embed_bwd_accum_kernel<float>, grid, dim3(256), 0, st, keys,
                       static_cast<const float*>(dY), dE_r, T, H);
  return check_launch("embed_bwd_accum_kernel");
}
