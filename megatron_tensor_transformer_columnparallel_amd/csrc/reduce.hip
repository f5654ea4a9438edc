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

// out = res + sum(parts) (fp32, in order), optional rounded copy.
template <typename Tr, typename Tp, typename To, typename Tc>
__global__ void __launch_bounds__(256) shard_reduce_add_kernel(const Tr* res, PartPtrs parts, int np, To* out,
                                                               Tc* copy, int64_t n) {
  const int64_t nvec = n / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
    float acc[8], x[8];
    Vec8<Tr>::load(res + v * 8, acc);
    for (int r = 0; r < np; ++r) {
      Vec8<Tp>::load(static_cast<const Tp*>(parts.p[r]) + v * 8, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += x[i];
    }
    Vec8<To>::store(out + v * 8, acc);
    if (copy) Vec8<Tc>::store(copy + v * 8, acc);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    for (int64_t i = nvec * 8; i < n; ++i) {
      float a = Elem<Tr>::load(res + i);
      for (int r = 0; r < np; ++r) a += Elem<Tp>::load(static_cast<const Tp*>(parts.p[r]) + i);
      out[i] = Elem<To>::from_f32(a);
      if (copy) copy[i] = Elem<Tc>::from_f32(a);
    }
  }
}

template <typename Tr, typename Tp, typename To>
static void launch_add(tps_dtype copy_dt, const void* res, const PartPtrs& pp, int np, void* out, void* copy,
                       int64_t n, dim3 grid, hipStream_t st) {
  TraceScope trace_(st, "shard_reduce_add_kernel");
  if (copy_dt == TPS_BF16)
    hipLaunchKernelGGL((shard_reduce_add_kernel<Tr, Tp, To, bf16_t>), grid, dim3(256), 0, st,
                       static_cast<const Tr*>(res), pp, np, static_cast<To*>(out), static_cast<bf16_t*>(copy), n);
  else
    hipLaunchKernelGGL((shard_reduce_add_kernel<Tr, Tp, To, float>), grid, dim3(256), 0, st,
                       static_cast<const Tr*>(res), pp, np, static_cast<To*>(out), static_cast<float*>(copy), n);
}

template <typename Tr, typename Tp>
static void launch_add_o(tps_dtype out_dt, tps_dtype copy_dt, const void* res, const PartPtrs& pp, int np, void* out,
                         void* copy, int64_t n, dim3 grid, hipStream_t st) {
  if (out_dt == TPS_BF16) launch_add<Tr, Tp, bf16_t>(copy_dt, res, pp, np, out, copy, n, grid, st);
  else launch_add<Tr, Tp, float>(copy_dt, res, pp, np, out, copy, n, grid, st);
}

}  // namespace tps

using namespace tps;

static bool ok_dt(tps_dtype d) { return d == TPS_F32 || d == TPS_BF16; }

extern "C" tps_status shard_reduce_add(tps_dtype res_dt, const void* res, tps_dtype part_dt, int n_parts,
                                       const void* const* parts, tps_dtype out_dt, void* out, tps_dtype copy_dt,
                                       void* out_copy, int64_t n, tps_stream_t stream) {
  ApiScope api_scope_("shard_reduce_add");
  if (!ok_dt(res_dt) || !ok_dt(part_dt) || !ok_dt(out_dt) || !ok_dt(copy_dt))
    return set_error(TPS_EINVAL, "shard_reduce_add: bad dtype");
  if (n_parts < 1 || n_parts > 7) return set_error(TPS_EINVAL, "shard_reduce_add: n_parts must be in [1, 7]");
  if (!res || !parts || !out) return set_error(TPS_EINVAL, "shard_reduce_add: null pointer");
  if (n < 0) return set_error(TPS_EINVAL, "shard_reduce_add: n < 0");
  PartPtrs pp{};
  for (int r = 0; r < n_parts; ++r) {
    if (!parts[r]) return set_error(TPS_EINVAL, "shard_reduce_add: null part pointer");
    if (!aligned16(parts[r])) return set_error(TPS_EINVAL, "shard_reduce_add: part not 16-byte aligned");
    pp.p[r] = parts[r];
  }
  if (!aligned16(res) || !aligned16(out) || (out_copy && !aligned16(out_copy)))
    return set_error(TPS_EINVAL, "shard_reduce_add: pointers must be 16-byte aligned");
  if (n == 0) return TPS_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int64_t blocks = ceil_div(n / 8 > 0 ? n / 8 : 1, 256);
  if (blocks > 65536) blocks = 65536;
  const dim3 grid((unsigned)blocks);
  if (res_dt == TPS_F32 && part_dt == TPS_BF16) launch_add_o<float, bf16_t>(out_dt, copy_dt, res, pp, n_parts, out, out_copy, n, grid, st);
  else if (res_dt == TPS_F32) launch_add_o<float, float>(out_dt, copy_dt, res, pp, n_parts, out, out_copy, n, grid, st);
  else if (part_dt == TPS_BF16) launch_add_o<bf16_t, bf16_t>(out_dt, copy_dt, res, pp, n_parts, out, out_copy, n, grid, st);
  else launch_add_o<bf16_t, float>(out_dt, copy_dt, res, pp, n_parts, out, out_copy, n, grid, st);
  return check_launch("shard_reduce_add_kernel");
}

extern "C" tps_status shard_reduce(tps_dtype in_dt, tps_dtype out_dt, int n_parts,
                                   const void* const* parts, void* out, int64_t n,
                                   tps_stream_t stream) {
  ApiScope api_scope_("shard_reduce");
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
  TraceScope trace_(st, "shard_reduce_kernel");
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
