// The two tensor-parallel linear layers on their own (page "5-megatron",
// sections ColumnParallelLinear and RowParallelLinear), in math layout
// Y = X A + b, one shard per call:
//
//   column shard r:  Y_r = X A_r (+ b_r)       A_r = columns of A, b_r its bias slice;
//                    gather_output = write Y_r into its column slice of the
//                    gathered Y (a row stride), f's backward sums dX_r.
//   row shard r:     Y_r = X_r B_r (partial)  X_r = columns of X (the scatter)
//                    unless the input is already parallel; the shard sum
//                    then adds the full bias once (shard_reduce_bias).
//
// The GEMMs are the MFMA kernels of gemm.hpp with a bias epilogue; the bias
// gradient is a fixed-order column sum (bias_grad_kernel).
#include <string>

#include "gemm.hpp"

namespace tps {

namespace {

// C = acc + bias[n] (bias of the output's element type, 16-byte aligned).
template <typename T>
struct EpiBias {
  T* C;
  int64_t ldc;
  const T* bias;
  __device__ void operator()(int, int, int m, int n, float v[8], int nv) const {
    float b[8];
    load8<T>(bias + n, b, nv);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] += b[i];
    store8<T>(C + (int64_t)m * ldc + n, v, nv);
  }
};

GemmShape lshape(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb) {
  GemmShape s;
  s.M = (int)M; s.N = (int)N; s.K = (int)K; s.lda = lda; s.ldb = ldb;
  return s;
}

template <typename T, bool AK, bool BKC, class Epi>
tps_status lgemm(const T* A, const T* B, const GemmShape& s, const Epi& e, hipStream_t st) {
  if constexpr (sizeof(T) == 2) return gemm_bf16<AK, BKC>(A, B, s, e, st);
  else return gemm_f32<AK, BKC>(A, B, s, e, st);
}

// db[n] = sum over m of dY[m, n] in fp32, in a fixed order (reproducible,
// and identical wherever the same dY is reduced): a workgroup owns 64
// columns (one 128-byte line of bf16 per row); its 1024 threads are 8 lanes
// of 8 columns by 128 row groups, each group summing rows g, g + 128, ... in
// increasing order with four rows' loads in flight; then, per column, each
// run of 8 consecutive groups is summed in order, and the 16 runs in order.
constexpr int kBgGroups = 128;
template <typename T>
__global__ void __launch_bounds__(1024) bias_grad_kernel(const T* __restrict__ dY, int64_t ld, int64_t M, int64_t N,
                                                         float* __restrict__ db) {
  __shared__ float part[kBgGroups][65];
  __shared__ float run[16][65];
  const int tid = threadIdx.x, cg = tid & 7, rg = tid >> 3;
  const int64_t n = (int64_t)blockIdx.x * 64 + cg * 8;
  const int nv = (int)(N - n < 8 ? (N - n > 0 ? N - n : 0) : 8);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (nv > 0) {
    int64_t m = rg;
    for (; m + 3 * kBgGroups < M; m += 4 * kBgGroups) {
      float v0[8], v1[8], v2[8], v3[8];
      load8<T>(dY + m * ld + n, v0, nv);
      load8<T>(dY + (m + kBgGroups) * ld + n, v1, nv);
      load8<T>(dY + (m + 2 * kBgGroups) * ld + n, v2, nv);
      load8<T>(dY + (m + 3 * kBgGroups) * ld + n, v3, nv);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = ((acc[i] + v0[i]) + v1[i] + v2[i]) + v3[i];
    }
    for (; m < M; m += kBgGroups) {
      float v[8];
      load8<T>(dY + m * ld + n, v, nv);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) part[rg][cg * 8 + i] = acc[i];
  __syncthreads();
  const int col = tid & 63, r = tid >> 6;   // 16 runs of 8 groups
  float sr = 0.f;
#pragma unroll
  for (int g = 0; g < 8; ++g) sr += part[r * 8 + g][col];
  run[r][col] = sr;
  __syncthreads();
  if (tid < 64) {
    float t = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) t += run[q][tid];
    const int64_t c = (int64_t)blockIdx.x * 64 + tid;
    if (c < N) db[c] = t;
  }
}

tps_status bias_grad(tps_dtype dt, const void* dY, int64_t ld, int64_t M, int64_t N, float* db, hipStream_t st) {
  const dim3 grid((unsigned)ceil_div(N, 64));
  if (dt == TPS_BF16)
    hipLaunchKernelGGL(bias_grad_kernel<bf16_t>, grid, dim3(1024), 0, st, static_cast<const bf16_t*>(dY), ld, M, N, db);
  else
    hipLaunchKernelGGL(bias_grad_kernel<float>, grid, dim3(1024), 0, st, static_cast<const float*>(dY), ld, M, N, db);
  return check_launch("bias_grad_kernel");
}

struct Parts {
  const void* p[8];
};

// out[m, n] = sum_r parts[r][m, n] (shard order, fp32) + bias[n], rounded once.
template <typename T>
__global__ void __launch_bounds__(256) reduce_bias_kernel(Parts parts, int np, const T* __restrict__ bias,
                                                          T* __restrict__ out, int64_t M, int64_t N) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= M * N) return;
  const int64_t n = i % N;   // N is a multiple of 8: a vector never crosses a row
  float acc[8], v[8];
  load8<T>(static_cast<const T*>(parts.p[0]) + i, acc, 8);
  for (int r = 1; r < np; ++r) {
    load8<T>(static_cast<const T*>(parts.p[r]) + i, v, 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += v[e];
  }
  load8<T>(bias + n, v, 8);
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] += v[e];
  store8<T>(out + i, acc, 8);
}

tps_status dims_ok(const char* fn, tps_dtype dt, int64_t a, int64_t b, int64_t c) {
  if (dt != TPS_F32 && dt != TPS_BF16) return set_error(TPS_EINVAL, std::string(fn) + ": bad dtype");
  if (a <= 0 || b <= 0 || c <= 0) return set_error(TPS_EINVAL, std::string(fn) + ": dims must be > 0");
  if (a >= 0x7fffffffLL || b >= 0x7fffffffLL || c >= 0x7fffffffLL)
    return set_error(TPS_EINVAL, std::string(fn) + ": dims must be < 2^31");
  return TPS_OK;
}

tps_status ld_ok(const char* fn, tps_dtype dt, int64_t ld, int64_t width, const char* what) {
  if (ld < width || ld % 8 != 0)
    return set_error(TPS_EINVAL, std::string(fn) + ": " + what + " must be >= its row width and a multiple of 8");
  (void)dt;
  return TPS_OK;
}

tps_status ptrs_ok(const char* fn, std::initializer_list<const void*> ps) {
  for (const void* p : ps) {
    if (!p) return set_error(TPS_EINVAL, std::string(fn) + ": null pointer");
    if (!aligned16(p)) return set_error(TPS_EINVAL, std::string(fn) + ": pointers must be 16-byte aligned");
  }
  return TPS_OK;
}

#define TPS_LTRY(expr) \
  do { tps_status _s = (expr); if (_s != TPS_OK) return _s; } while (0)

template <typename T>
tps_status column_fwd_t(int64_t M, int64_t h, int64_t n, const T* X, const T* A, const T* b, T* Y, int64_t ldy,
                        hipStream_t st) {
  const GemmShape s = lshape(M, n, h, h, n);   // NN: X [M x h], A_r [h x n]
  if (b) return lgemm<T, true, false>(X, A, s, EpiBias<T>{Y, ldy, b}, st);
  return lgemm<T, true, false>(X, A, s, EpiStore<T>{Y, ldy, 0, 0}, st);
}

template <typename T>
tps_status column_bwd_t(int64_t M, int64_t h, int64_t n, const T* X, const T* A, const T* dY, int64_t lddy,
                        T* dX, T* dA, hipStream_t st) {
  // dX_r = dY_r A_r^T   (NT: dY [M x n] K-contiguous, A_r [h x n] K-contiguous)
  TPS_LTRY((lgemm<T, true, true>(dY, A, lshape(M, h, n, lddy, n), EpiStore<T>{dX, h, 0, 0}, st)));
  // dA_r = X^T dY_r     (TN: X [M x h] M-contiguous, dY [M x n] N-contiguous)
  return lgemm<T, false, false>(X, dY, lshape(h, n, M, h, lddy), EpiStore<T>{dA, n, 0, 0}, st);
}

template <typename T>
tps_status row_fwd_t(int64_t M, int64_t k, int64_t h, const T* X, int64_t ldx, const T* B, T* Y, hipStream_t st) {
  return lgemm<T, true, false>(X, B, lshape(M, h, k, ldx, h), EpiStore<T>{Y, h, 0, 0}, st);
}

template <typename T>
tps_status row_bwd_t(int64_t M, int64_t k, int64_t h, const T* X, int64_t ldx, const T* B, const T* dY, T* dX,
                     int64_t lddx, T* dB, hipStream_t st) {
  // dX_r = dY B_r^T     (NT: dY [M x h], B_r [k x h]), into a column slice of the gathered dX
  TPS_LTRY((lgemm<T, true, true>(dY, B, lshape(M, k, h, h, h), EpiStore<T>{dX, lddx, 0, 0}, st)));
  // dB_r = X_r^T dY     (TN: X_r [M x k] with row stride ldx, dY [M x h])
  return lgemm<T, false, false>(X, dY, lshape(k, h, M, ldx, h), EpiStore<T>{dB, h, 0, 0}, st);
}

}  // namespace

}  // namespace tps

using namespace tps;

extern "C" tps_status column_linear_fwd(tps_dtype dt, int64_t M, int64_t h_in, int64_t n_r, const void* X,
                                        const void* A_r, const void* b_r, void* Y, int64_t ldy,
                                        tps_stream_t stream) {
  ApiScope api_scope_("column_linear_fwd");
  const char* fn = "column_linear_fwd";
  TPS_LTRY(dims_ok(fn, dt, M, h_in, n_r));
  TPS_LTRY(ptrs_ok(fn, {X, A_r, Y}));
  if (b_r && !aligned16(b_r)) return set_error(TPS_EINVAL, "column_linear_fwd: b_r must be 16-byte aligned");
  TPS_LTRY(ld_ok(fn, dt, ldy, n_r, "ldy"));
  if (h_in % 8 || n_r % 8) return set_error(TPS_EINVAL, "column_linear_fwd: h_in and n_r must be multiples of 8");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dt == TPS_BF16)
    return column_fwd_t<bf16_t>(M, h_in, n_r, static_cast<const bf16_t*>(X), static_cast<const bf16_t*>(A_r),
                                static_cast<const bf16_t*>(b_r), static_cast<bf16_t*>(Y), ldy, st);
  return column_fwd_t<float>(M, h_in, n_r, static_cast<const float*>(X), static_cast<const float*>(A_r),
                             static_cast<const float*>(b_r), static_cast<float*>(Y), ldy, st);
}

extern "C" tps_status column_linear_bwd(tps_dtype dt, int64_t M, int64_t h_in, int64_t n_r, const void* X,
                                        const void* A_r, const void* dY, int64_t lddy, void* dX_r, void* dA_r,
                                        float* db_r, tps_stream_t stream) {
  ApiScope api_scope_("column_linear_bwd");
  const char* fn = "column_linear_bwd";
  TPS_LTRY(dims_ok(fn, dt, M, h_in, n_r));
  TPS_LTRY(ptrs_ok(fn, {X, A_r, dY, dX_r, dA_r}));
  if (db_r && !aligned16(db_r)) return set_error(TPS_EINVAL, "column_linear_bwd: db_r must be 16-byte aligned");
  TPS_LTRY(ld_ok(fn, dt, lddy, n_r, "lddy"));
  if (h_in % 8 || n_r % 8) return set_error(TPS_EINVAL, "column_linear_bwd: h_in and n_r must be multiples of 8");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dt == TPS_BF16)
    TPS_LTRY(column_bwd_t<bf16_t>(M, h_in, n_r, static_cast<const bf16_t*>(X), static_cast<const bf16_t*>(A_r),
                                  static_cast<const bf16_t*>(dY), lddy, static_cast<bf16_t*>(dX_r),
                                  static_cast<bf16_t*>(dA_r), st));
  else
    TPS_LTRY(column_bwd_t<float>(M, h_in, n_r, static_cast<const float*>(X), static_cast<const float*>(A_r),
                                 static_cast<const float*>(dY), lddy, static_cast<float*>(dX_r),
                                 static_cast<float*>(dA_r), st));
  if (db_r) return bias_grad(dt, dY, lddy, M, n_r, db_r, st);
  return TPS_OK;
}

extern "C" tps_status row_linear_fwd(tps_dtype dt, int64_t M, int64_t k_r, int64_t h_out, const void* X_r,
                                     int64_t ldx, const void* B_r, void* Y_r, tps_stream_t stream) {
  ApiScope api_scope_("row_linear_fwd");
  const char* fn = "row_linear_fwd";
  TPS_LTRY(dims_ok(fn, dt, M, k_r, h_out));
  TPS_LTRY(ptrs_ok(fn, {X_r, B_r, Y_r}));
  TPS_LTRY(ld_ok(fn, dt, ldx, k_r, "ldx"));
  if (k_r % 8 || h_out % 8) return set_error(TPS_EINVAL, "row_linear_fwd: k_r and h_out must be multiples of 8");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dt == TPS_BF16)
    return row_fwd_t<bf16_t>(M, k_r, h_out, static_cast<const bf16_t*>(X_r), ldx, static_cast<const bf16_t*>(B_r),
                             static_cast<bf16_t*>(Y_r), st);
  return row_fwd_t<float>(M, k_r, h_out, static_cast<const float*>(X_r), ldx, static_cast<const float*>(B_r),
                          static_cast<float*>(Y_r), st);
}

extern "C" tps_status row_linear_bwd(tps_dtype dt, int64_t M, int64_t k_r, int64_t h_out, const void* X_r,
                                     int64_t ldx, const void* B_r, const void* dY, void* dX_r, int64_t lddx,
                                     void* dB_r, float* db, tps_stream_t stream) {
  ApiScope api_scope_("row_linear_bwd");
  const char* fn = "row_linear_bwd";
  TPS_LTRY(dims_ok(fn, dt, M, k_r, h_out));
  TPS_LTRY(ptrs_ok(fn, {X_r, B_r, dY, dX_r, dB_r}));
  if (db && !aligned16(db)) return set_error(TPS_EINVAL, "row_linear_bwd: db must be 16-byte aligned");
  TPS_LTRY(ld_ok(fn, dt, ldx, k_r, "ldx"));
  TPS_LTRY(ld_ok(fn, dt, lddx, k_r, "lddx"));
  if (k_r % 8 || h_out % 8) return set_error(TPS_EINVAL, "row_linear_bwd: k_r and h_out must be multiples of 8");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dt == TPS_BF16)
    TPS_LTRY(row_bwd_t<bf16_t>(M, k_r, h_out, static_cast<const bf16_t*>(X_r), ldx, static_cast<const bf16_t*>(B_r),
                               static_cast<const bf16_t*>(dY), static_cast<bf16_t*>(dX_r), lddx,
                               static_cast<bf16_t*>(dB_r), st));
  else
    TPS_LTRY(row_bwd_t<float>(M, k_r, h_out, static_cast<const float*>(X_r), ldx, static_cast<const float*>(B_r),
                              static_cast<const float*>(dY), static_cast<float*>(dX_r), lddx,
                              static_cast<float*>(dB_r), st));
  if (db) return bias_grad(dt, dY, h_out, M, h_out, db, st);
  return TPS_OK;
}

extern "C" tps_status shard_reduce_bias(tps_dtype dt, int n_parts, const void* const* parts, const void* bias,
                                        void* out, int64_t M, int64_t N, tps_stream_t stream) {
  ApiScope api_scope_("shard_reduce_bias");
  const char* fn = "shard_reduce_bias";
  if (dt != TPS_F32 && dt != TPS_BF16) return set_error(TPS_EINVAL, "shard_reduce_bias: bad dtype");
  if (n_parts < 1 || n_parts > 8) return set_error(TPS_EINVAL, "shard_reduce_bias: n_parts must be 1..8");
  if (M <= 0 || N <= 0 || N % 8) return set_error(TPS_EINVAL, "shard_reduce_bias: need M > 0 and N a positive multiple of 8");
  if (!parts) return set_error(TPS_EINVAL, "shard_reduce_bias: null pointer");
  Parts pp{};
  for (int r = 0; r < n_parts; ++r) {
    TPS_LTRY(ptrs_ok(fn, {parts[r]}));
    pp.p[r] = parts[r];
  }
  TPS_LTRY(ptrs_ok(fn, {bias, out}));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)ceil_div(M * N / 8, 256));
  if (dt == TPS_BF16)
    hipLaunchKernelGGL(reduce_bias_kernel<bf16_t>, grid, dim3(256), 0, st, pp, n_parts,
                       static_cast<const bf16_t*>(bias), static_cast<bf16_t*>(out), M, N);
  else
    hipLaunchKernelGGL(reduce_bias_kernel<float>, grid, dim3(256), 0, st, pp, n_parts,
                       static_cast<const float*>(bias), static_cast<float*>(out), M, N);
  return check_launch("reduce_bias_kernel");
}
