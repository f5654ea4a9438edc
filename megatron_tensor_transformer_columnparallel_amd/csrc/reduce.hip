// shard_reduce: out = sum of n_parts shard partials, fp32 accumulation in
// shard order, one rounding to the output type.  HBM-bound: every element is
// read once per part and written once, with 16-byte vector accesses.
#include "common.hpp"

namespace tps {

struct PartPtrs {
  const void* p[8];
};

template <typename T> struct Vec8;  // 8 elements as fp32
template <> struct Vec8<bf16_t> {
  __device__ static void load(const bf16_t* p, float v[8]) {
    u32x4_t x = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int w = 0; w < 4; ++w) { v[2 * w] = bf16lo(x[w]); v[2 * w + 1] = bf16hi(x[w]); }
  }
  __device__ static void store(bf16_t* p, const float v[8]) {
    u32x4_t x;
#pragma unroll
    for (int w = 0; w < 4; ++w) x[w] = pack_bf16x2(v[2 * w], v[2 * w + 1]);
    *reinterpret_cast<u32x4_t*>(p) = x;
  }
};
template <> struct Vec8<float> {
  __device__ static void load(const float* p, float v[8]) {
    f32x4_t a = reinterpret_cast<const f32x4_t*>(p)[0], b = reinterpret_cast<const f32x4_t*>(p)[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
  __device__ static void store(float* p, const float v[8]) {
    reinterpret_cast<f32x4_t*>(p)[0] = f32x4_t{v[0], v[1], v[2], v[3]};
    reinterpret_cast<f32x4_t*>(p)[1] = f32x4_t{v[4], v[5], v[6], v[7]};
  }
};

template <typename Tin, typename Tout>
__global__ void __launch_bounds__(256) shard_reduce_kernel(PartPtrs parts, int np, Tout* out, int64_t n) {
  const int64_t nvec = n / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
    float acc[8], x[8];
    Vec8<Tin>::load(static_cast<const Tin*>(parts.p[0]) + v * 8, acc);
    for (int r = 1; r < np; ++r) {
      Vec8<Tin>::load(static_cast<const Tin*>(parts.p[r]) + v * 8, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += x[i];
    }
    Vec8<Tout>::store(out + v * 8, acc);
  }
  // ragged tail (n % 8 elements): one thread
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    for (int64_t i = nvec * 8; i < n; ++i) {
      float a = Elem<Tin>::load(static_cast<const Tin*>(parts.p[0]) + i);
      for (int r = 1; r < np; ++r) a += Elem<Tin>::load(static_cast<const Tin*>(parts.p[r]) + i);
      out[i] = Elem<Tout>::from_f32(a);
    }
  }
}

}  // namespace tps

using namespace tps;

extern "C" tps_status shard_reduce(tps_dtype in_dt, tps_dtype out_dt, int n_parts,
                                   const void* const* parts, void* out, int64_t n,
                                   tps_stream_t stream) {
  if ((in_dt != TPS_F32 && in_dt != TPS_BF16) || (out_dt != TPS_F32 && out_dt != TPS_BF16))
    return set_error(TPS_EINVAL, "shard_reduce: bad dtype");
  if (n_parts < 1 || n_parts > 8) return set_error(TPS_EINVAL, "shard_reduce: n_parts must be in [1, 8]");
  if (!parts || !out) return set_error(TPS_EINVAL, "shard_reduce: null pointer");
  if (n < 0) return set_error(TPS_EINVAL, "shard_reduce: n < 0");
  PartPtrs pp{};
  for (int r = 0; r < n_parts; ++r) {
    if (!parts[r]) return set_error(TPS_EINVAL, "shard_reduce: null part pointer");
    if (!aligned16(parts[r])) return set_error(TPS_EINVAL, "shard_reduce: part not 16-byte aligned");
    pp.p[r] = parts[r];
  }
  if (!aligned16(out)) return set_error(TPS_EINVAL, "shard_reduce: out not 16-byte aligned");
  if (n == 0) return TPS_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t nvec = n / 8;
  int64_t blocks = ceil_div(nvec > 0 ? nvec : 1, 256);
  if (blocks > 65536) blocks = 65536;
#define TPS_RED(TI, TO) \
  hipLaunchKernelGGL((shard_reduce_kernel<TI, TO>), dim3((unsigned)blocks), dim3(256), 0, st, pp, n_parts, \
                     static_cast<TO*>(out), n)
  if (in_dt == TPS_BF16 && out_dt == TPS_BF16) TPS_RED(bf16_t, bf16_t);
  else if (in_dt == TPS_BF16) TPS_RED(bf16_t, float);
  else if (out_dt == TPS_BF16) TPS_RED(float, bf16_t);
  else TPS_RED(float, float);
#undef TPS_RED
  return check_launch("shard_reduce_kernel");
}
