// Sequence-parallel exchanges on one device (page "5-megatron": in sequence
// parallel regions the sequence component of an activation is s/N per
// shard).  The rows of an [M x H] activation are split over the shards as
// tps_partition(M, n, r) does.
//
// shard_reduce_scatter: the reduce-scatter that replaces the g all-reduce
//   after a row-parallel GEMM: shard r receives its rows of the sum of the
//   full-size partials (fp32, shard order, one rounding), optionally added
//   to its rows of the residual stream first.
// shard_all_gather: the all-gather that rebuilds the full sequence before a
//   column-parallel GEMM.
// Both are HBM-bound: 8 consecutive elements of a row per thread, 16-byte
// vectors, grid-stride over the full activation.
#include <string>

#include "common.hpp"

namespace tps {

namespace {

struct SpPtrs {
  const void* p[8];
};
struct SpOut {
  void* p[8];
};

// Shard of a row under the tps_partition split: the first `rem` shards hold
// q + 1 rows, the others q.
struct RowSplit {
  int64_t q, rem;
  __device__ __forceinline__ void locate(int64_t row, int& r, int64_t& start) const {
    const int64_t big = rem * (q + 1);
    if (row < big) {
      r = (int)(row / (q + 1));
      start = (int64_t)r * (q + 1);
    } else {
      r = (int)(rem + (row - big) / q);
      start = big + (int64_t)(r - rem) * q;
    }
  }
};

template <typename Tp, typename To>
__global__ void __launch_bounds__(256) sp_reduce_scatter_kernel(SpPtrs parts, int np, SpPtrs res, SpOut outs,
                                                                RowSplit split, int64_t M, int64_t H) {
  const int64_t nvec = M * H / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
    const int64_t e = v * 8, row = e / H, col = e - row * H;
    int r;
    int64_t start;
    split.locate(row, r, start);
    const int64_t o = (row - start) * H + col;
    float acc[8], x[8];
    if (res.p[r]) {
      load8<To>(static_cast<const To*>(res.p[r]) + o, acc, 8);
      for (int k = 0; k < np; ++k) {
        load8<Tp>(static_cast<const Tp*>(parts.p[k]) + e, x, 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += x[i];
      }
    } else {
      load8<Tp>(static_cast<const Tp*>(parts.p[0]) + e, acc, 8);
      for (int k = 1; k < np; ++k) {
        load8<Tp>(static_cast<const Tp*>(parts.p[k]) + e, x, 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += x[i];
      }
    }
    store8<To>(static_cast<To*>(outs.p[r]) + o, acc, 8);
  }
}

template <typename T>
__global__ void __launch_bounds__(256) sp_all_gather_kernel(SpPtrs parts, RowSplit split, T* __restrict__ out,
                                                            int64_t M, int64_t H) {
  const int64_t nvec = M * H / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
    const int64_t e = v * 8, row = e / H, col = e - row * H;
    int r;
    int64_t start;
    split.locate(row, r, start);
    *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(out) + e * sizeof(T)) =
        *reinterpret_cast<const u32x4_t*>(static_cast<const char*>(parts.p[r]) +
                                          ((row - start) * H + col) * sizeof(T));
    if constexpr (sizeof(T) == 4)
      *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(out) + e * 4 + 16) =
          *reinterpret_cast<const u32x4_t*>(static_cast<const char*>(parts.p[r]) + ((row - start) * H + col) * 4 + 16);
  }
}

bool dt_ok(tps_dtype d) { return d == TPS_F32 || d == TPS_BF16; }

tps_status common(const char* fn, int n, int64_t M, int64_t H) {
  if (n < 1 || n > 8) return set_error(TPS_EINVAL, std::string(fn) + ": n_parts must be 1..8");
  if (M <= 0 || H <= 0 || H % 8) return set_error(TPS_EINVAL, std::string(fn) + ": need M > 0 and H a positive multiple of 8");
  return TPS_OK;
}

tps_status ptr_ok(const char* fn, const void* p) {
  if (!p) return set_error(TPS_EINVAL, std::string(fn) + ": null pointer");
  if (!aligned16(p)) return set_error(TPS_EINVAL, std::string(fn) + ": pointers must be 16-byte aligned");
  return TPS_OK;
}

dim3 grid_for(int64_t M, int64_t H) {
  int64_t blocks = ceil_div(M * H / 8, 256);
  if (blocks > 65536) blocks = 65536;
  return dim3((unsigned)(blocks > 0 ? blocks : 1));
}

}  // namespace

}  // namespace tps

using namespace tps;

extern "C" tps_status shard_reduce_scatter(tps_dtype part_dt, tps_dtype out_dt, int n_parts,
                                           const void* const* parts, const void* const* res, void* const* outs,
                                           int64_t M, int64_t H, tps_stream_t stream) {
  ApiScope api_scope_("shard_reduce_scatter");
  const char* fn = "shard_reduce_scatter";
  if (!dt_ok(part_dt) || !dt_ok(out_dt)) return set_error(TPS_EINVAL, "shard_reduce_scatter: bad dtype");
  tps_status s = common(fn, n_parts, M, H);
  if (s != TPS_OK) return s;
  if (!parts || !outs) return set_error(TPS_EINVAL, "shard_reduce_scatter: null pointer");
  SpPtrs pp{}, rp{};
  SpOut op{};
  const RowSplit split{M / n_parts, M % n_parts};
  for (int r = 0; r < n_parts; ++r) {
    const bool rows = split.q + (r < split.rem ? 1 : 0) > 0;   // a shard without rows may pass NULL
    if ((s = ptr_ok(fn, parts[r])) != TPS_OK) return s;
    if (rows && (s = ptr_ok(fn, outs[r])) != TPS_OK) return s;
    if (res && rows && (s = ptr_ok(fn, res[r])) != TPS_OK) return s;
    pp.p[r] = parts[r];
    op.p[r] = outs[r];
    rp.p[r] = res ? res[r] : nullptr;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid = grid_for(M, H);
#define TPS_RS(TP, TO) \
  hipLaunchKernelGGL((sp_reduce_scatter_kernel<TP, TO>), grid, dim3(256), 0, st, pp, n_parts, rp, op, split, M, H)
  if (part_dt == TPS_BF16 && out_dt == TPS_BF16) TPS_RS(bf16_t, bf16_t);
  else if (part_dt == TPS_BF16) TPS_RS(bf16_t, float);
  else if (out_dt == TPS_BF16) TPS_RS(float, bf16_t);
  else TPS_RS(float, float);
#undef TPS_RS
  return check_launch("sp_reduce_scatter_kernel");
}

extern "C" tps_status shard_all_gather(tps_dtype dt, int n_parts, const void* const* parts, void* out, int64_t M,
                                       int64_t H, tps_stream_t stream) {
  ApiScope api_scope_("shard_all_gather");
  const char* fn = "shard_all_gather";
  if (!dt_ok(dt)) return set_error(TPS_EINVAL, "shard_all_gather: bad dtype");
  tps_status s = common(fn, n_parts, M, H);
  if (s != TPS_OK) return s;
  if (!parts) return set_error(TPS_EINVAL, "shard_all_gather: null pointer");
  SpPtrs pp{};
  const RowSplit split{M / n_parts, M % n_parts};
  for (int r = 0; r < n_parts; ++r) {
    if (split.q + (r < split.rem ? 1 : 0) > 0 && (s = ptr_ok(fn, parts[r])) != TPS_OK) return s;
    pp.p[r] = parts[r];
  }
  if ((s = ptr_ok(fn, out)) != TPS_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid = grid_for(M, H);
  if (dt == TPS_BF16)
    hipLaunchKernelGGL(sp_all_gather_kernel<bf16_t>, grid, dim3(256), 0, st, pp, split, static_cast<bf16_t*>(out), M, H);
  else
    hipLaunchKernelGGL(sp_all_gather_kernel<float>, grid, dim3(256), 0, st, pp, split, static_cast<float*>(out), M, H);
  return check_launch("sp_all_gather_kernel");
}
