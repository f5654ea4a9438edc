// LayerNorm forward/backward (replicated on every shard; used between the
// attention and MLP sublayers of a stacked model).  One workgroup per row in
// the forward pass with the row held in registers (H <= 8192); the backward
// pass gives each workgroup 8 rows (prefetching one row ahead when H is 4096)
// and writes per-workgroup partial column sums of dgamma/dbeta to
// the workspace, which a second kernel reduces in a fixed order
// (deterministic, no atomics).
#include <string>

#include "common.hpp"

namespace tps {

constexpr int kLnMaxH = 8192;
constexpr int kLnRowsPerBlock = 8;

// 8 consecutive elements <-> fp32 registers (16 bytes of bf16, 32 of fp32).
template <typename T> struct LnVec;
template <> struct LnVec<bf16_t> {
  __device__ static void load(const bf16_t* p, float* v) {
    const u32x4_t x = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int w = 0; w < 4; ++w) { v[2 * w] = bf16lo(x[w]); v[2 * w + 1] = bf16hi(x[w]); }
  }
  __device__ static void store(bf16_t* p, const float* v) {
    u32x4_t x;
#pragma unroll
    for (int w = 0; w < 4; ++w) x[w] = pack_bf16x2(v[2 * w], v[2 * w + 1]);
    *reinterpret_cast<u32x4_t*>(p) = x;
  }
};
template <> struct LnVec<float> {
  __device__ static void load(const float* p, float* v) {
    const f32x4_t a = reinterpret_cast<const f32x4_t*>(p)[0], b = reinterpret_cast<const f32x4_t*>(p)[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
  __device__ static void store(float* p, const float* v) {
    reinterpret_cast<f32x4_t*>(p)[0] = f32x4_t{v[0], v[1], v[2], v[3]};
    reinterpret_cast<f32x4_t*>(p)[1] = f32x4_t{v[4], v[5], v[6], v[7]};
  }
};
constexpr int kLnV = 8;                          // elements per thread chunk
constexpr int kLnNCH = kLnMaxH / kLnV / 256;     // chunks per thread

// Sum over the 256 threads of a workgroup; `red` is 8 floats of LDS.
__device__ __forceinline__ float block_sum(float x, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = x;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// NC chunks of 8 elements per thread (NC = ceil(H / 2048)).  Every load is
// issued before the first reduction and none sits behind a branch: a chunk
// that starts past the row's end re-reads the row's last 8 elements and is
// masked out of the sums and the store.  gamma and beta come in with x.
template <typename TX, typename TY, int NC>
__global__ void __launch_bounds__(256) ln_fwd_kernel(const TX* __restrict__ x, const float* __restrict__ gamma,
                                                     const float* __restrict__ beta, TY* __restrict__ y,
                                                     float* __restrict__ mean, float* __restrict__ rstd, int64_t H,
                                                     float eps) {
  constexpr int V = kLnV;
  __shared__ float red[8];
  const int64_t row = blockIdx.x;
  const TX* xr = x + row * H;
  float v[NC][V], g[NC][V], b[NC][V];
  bool ok[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int64_t c = ((int64_t)i * 256 + threadIdx.x) * V;
    ok[i] = c < H;
    const int64_t cc = ok[i] ? c : H - V;
    LnVec<TX>::load(xr + cc, v[i]);
    LnVec<float>::load(gamma + cc, g[i]);
    LnVec<float>::load(beta + cc, b[i]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i)
#pragma unroll
    for (int e = 0; e < V; ++e) s += ok[i] ? v[i][e] : 0.f;
  const float mu = block_sum(s, red) / (float)H;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i)
#pragma unroll
    for (int e = 0; e < V; ++e) { const float d = v[i][e] - mu; q += ok[i] ? d * d : 0.f; }
  const float var = block_sum(q, red) / (float)H;
  const float rs = rsqrtf(var + eps);
  TY* yr = y + row * H;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int64_t c = ((int64_t)i * 256 + threadIdx.x) * V;
    float o[V];
#pragma unroll
    for (int e = 0; e < V; ++e) o[e] = (v[i][e] - mu) * rs * g[i][e] + b[i][e];
    if (ok[i]) LnVec<TY>::store(yr + c, o);
  }
  if (threadIdx.x == 0) { mean[row] = mu; rstd[row] = rs; }
}

// RES: dx = res + (the LayerNorm gradient), and a bf16 copy of dx when
// `copy` is not null (the residual connection's gradient, added where the
// row is in registers).
template <bool RES, typename TX, typename TDY, typename TDX>
__global__ void __launch_bounds__(256) ln_bwd_kernel(const TX* __restrict__ x, const float* __restrict__ gamma,
                                                     const float* __restrict__ mean, const float* __restrict__ rstd,
                                                     const TDY* __restrict__ dy, TDX* __restrict__ dx,
                                                     float* __restrict__ part, int64_t M, int64_t H,
                                                     const float* __restrict__ res, bf16_t* __restrict__ copy) {
  constexpr int V = kLnV;
  constexpr int NCH = kLnNCH;
  __shared__ float red[8];
  float pg[NCH][V], pb[NCH][V];
#pragma unroll
  for (int i = 0; i < NCH; ++i)
#pragma unroll
    for (int e = 0; e < V; ++e) { pg[i][e] = 0.f; pb[i][e] = 0.f; }
  const int64_t r0 = (int64_t)blockIdx.x * kLnRowsPerBlock;
  for (int rr = 0; rr < kLnRowsPerBlock; ++rr) {
    const int64_t row = r0 + rr;
    if (row >= M) break;
    const float mu = mean[row], rs = rstd[row];
    float xh[NCH][V], gv[NCH][V];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int64_t c = ((int64_t)i * 256 + threadIdx.x) * V;
      if (c < H) {
        float xv[V], dv[V];
        LnVec<TX>::load(x + row * H + c, xv);
        LnVec<TDY>::load(dy + row * H + c, dv);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          xh[i][e] = (xv[e] - mu) * rs;
          gv[i][e] = dv[e] * gamma[c + e];
          s1 += gv[i][e];
          s2 += gv[i][e] * xh[i][e];
          pg[i][e] += dv[e] * xh[i][e];
          pb[i][e] += dv[e];
        }
      }
    }
    const float m1 = block_sum(s1, red) / (float)H;
    const float m2 = block_sum(s2, red) / (float)H;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int64_t c = ((int64_t)i * 256 + threadIdx.x) * V;
      if (c < H) {
        float o[V];
#pragma unroll
        for (int e = 0; e < V; ++e) o[e] = rs * (gv[i][e] - m1 - xh[i][e] * m2);
        if constexpr (RES) {
          float rv[V];
          LnVec<float>::load(res + row * H + c, rv);
#pragma unroll
          for (int e = 0; e < V; ++e) o[e] += rv[e];
          if (copy) LnVec<bf16_t>::store(copy + row * H + c, o);
        }
        LnVec<TDX>::store(dx + row * H + c, o);
      }
    }
  }
  float* pr = part + (int64_t)blockIdx.x * 2 * H;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int64_t c = ((int64_t)i * 256 + threadIdx.x) * V;
    if (c < H) {
#pragma unroll
      for (int e = 0; e < V; ++e) { pr[c + e] = pg[i][e]; pr[H + c + e] = pb[i][e]; }
    }
  }
}

// Backward for H = NCH * 4096 (launched for H = 4096, the layer width; with
// NCH = 2 the two row buffers no longer fit in registers): 512 threads,
// every thread owns NCH full chunks, so no load or store is conditional and
// the compiler counts them exactly.  The loads of row r+1 are issued before row r is
// processed, into the other of two register buffers, so they stay in flight
// across row r's barrier and stores: the barrier waits only for LDS
// operations, and the wait before row r+1 counts only row r+1's loads.  The two row sums
// travel together through a double-buffered LDS exchange: one barrier per
// row.  Same partial-sum layout as ln_bwd_kernel.
constexpr int kLnBwdThreads = 512;

template <int NCH, bool RES, typename TX, typename TDY, typename TDX>
__global__ void __launch_bounds__(kLnBwdThreads) ln_bwd_rows_kernel(const TX* __restrict__ x,
                                                                    const float* __restrict__ gamma,
                                                                    const float* __restrict__ mean,
                                                                    const float* __restrict__ rstd,
                                                                    const TDY* __restrict__ dy, TDX* __restrict__ dx,
                                                                    float* __restrict__ part, int64_t M,
                                                                    const float* __restrict__ res,
                                                                    bf16_t* __restrict__ copy) {
  constexpr int V = kLnV;
  constexpr int NW = kLnBwdThreads / 64;
  constexpr int64_t H = (int64_t)NCH * kLnBwdThreads * V;
  __shared__ float red[2][NW][2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float pg[NCH][V], pb[NCH][V], gm[NCH][V];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int64_t c = ((int64_t)i * kLnBwdThreads + threadIdx.x) * V;
    LnVec<float>::load(gamma + c, gm[i]);
#pragma unroll
    for (int e = 0; e < V; ++e) { pg[i][e] = 0.f; pb[i][e] = 0.f; }
  }
  const int64_t r0 = (int64_t)blockIdx.x * kLnRowsPerBlock;
  const int nr = (int)min((int64_t)kLnRowsPerBlock, M - r0);
  auto load_row = [&](int64_t row, float (&xv)[NCH][V], float (&dv)[NCH][V]) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int64_t c = ((int64_t)i * kLnBwdThreads + threadIdx.x) * V;
      LnVec<TX>::load(x + row * H + c, xv[i]);
      LnVec<TDY>::load(dy + row * H + c, dv[i]);
    }
  };
  // One row: sums, the shared row means, dx, and the dgamma/dbeta partials.
  auto row_pass = [&](int rr, const float (&xv)[NCH][V], const float (&dv)[NCH][V]) {
    const int64_t row = r0 + rr;
    // the residual gradient's row is loaded first: its latency hides behind the row sums
    float rv[NCH][V];
    if constexpr (RES) {
#pragma unroll
      for (int i = 0; i < NCH; ++i)
        LnVec<float>::load(res + row * H + ((int64_t)i * kLnBwdThreads + threadIdx.x) * V, rv[i]);
    }
    const float mu = mean[row], rs = rstd[row];
    float xh[NCH][V], gv[NCH][V];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        xh[i][e] = (xv[i][e] - mu) * rs;
        gv[i][e] = dv[i][e] * gm[i][e];
        s1 += gv[i][e];
        s2 += gv[i][e] * xh[i][e];
        pg[i][e] += dv[i][e] * xh[i][e];
        pb[i][e] += dv[i][e];
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      s1 += __shfl_xor(s1, o);
      s2 += __shfl_xor(s2, o);
    }
    // buffer rr & 1 was last read in row rr-2, before every wave reached
    // row rr-1's barrier
    if (lane == 0) { red[rr & 1][wave][0] = s1; red[rr & 1][wave][1] = s2; }
    __syncthreads();
    float t1 = 0.f, t2 = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) { t1 += red[rr & 1][w][0]; t2 += red[rr & 1][w][1]; }
    const float m1 = t1 / (float)H, m2 = t2 / (float)H;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int64_t c = ((int64_t)i * kLnBwdThreads + threadIdx.x) * V;
      float o[V];
#pragma unroll
      for (int e = 0; e < V; ++e) o[e] = rs * (gv[i][e] - m1 - xh[i][e] * m2);
      if constexpr (RES) {
#pragma unroll
        for (int e = 0; e < V; ++e) o[e] += rv[i][e];
        if (copy) LnVec<bf16_t>::store(copy + row * H + c, o);
      }
      LnVec<TDX>::store(dx + row * H + c, o);
    }
  };
  if (nr == kLnRowsPerBlock) {
    // full block: unrolled, rows alternate between two register buffers
    float xs[2][NCH][V], ds[2][NCH][V];
    load_row(r0, xs[0], ds[0]);
#pragma unroll
    for (int rr = 0; rr < kLnRowsPerBlock; ++rr) {
      if (rr + 1 < kLnRowsPerBlock) load_row(r0 + rr + 1, xs[(rr + 1) & 1], ds[(rr + 1) & 1]);
      row_pass(rr, xs[rr & 1], ds[rr & 1]);
    }
  } else {
    // last, partial block: one buffer plus a copy per row
    float xa[NCH][V], da[NCH][V];
    load_row(r0, xa, da);
    for (int rr = 0; rr < nr; ++rr) {
      float xb[NCH][V], db[NCH][V];
      load_row(rr + 1 < nr ? r0 + rr + 1 : r0 + rr, xb, db);
      row_pass(rr, xa, da);
#pragma unroll
      for (int i = 0; i < NCH; ++i)
#pragma unroll
        for (int e = 0; e < V; ++e) { xa[i][e] = xb[i][e]; da[i][e] = db[i][e]; }
    }
  }
  float* pr = part + (int64_t)blockIdx.x * 2 * H;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int64_t c = ((int64_t)i * kLnBwdThreads + threadIdx.x) * V;
    LnVec<float>::store(pr + c, pg[i]);
    LnVec<float>::store(pr + H + c, pb[i]);
  }
}

// [dgamma | dbeta][j] = sum over row blocks k of part[k][j], j < 2H, in a
// fixed order.  A workgroup owns 8 quads of columns and splits the blocks
// into 32 contiguous slices, one per thread of a quad; the slice sums are
// then added in slice order through LDS.  Deterministic, no atomics.
__global__ void __launch_bounds__(256) ln_param_reduce_kernel(const float* __restrict__ part, float* __restrict__ dgamma,
                                                              float* __restrict__ dbeta, int64_t nblk, int64_t H) {
  constexpr int CQ = 8, SLICES = 256 / CQ;
  __shared__ f32x4_t red[SLICES][CQ];
  const int cq = threadIdx.x % CQ, sl = threadIdx.x / CQ;
  const int64_t W = 2 * H;
  const int64_t j = ((int64_t)blockIdx.x * CQ + cq) * 4;   // H is a multiple of 8: a quad never straddles H
  f32x4_t a = {0.f, 0.f, 0.f, 0.f};
  if (j < W) {
    const int64_t per = (nblk + SLICES - 1) / SLICES;
    const int64_t k0 = sl * per, k1 = min(nblk, k0 + per);
    for (int64_t k = k0; k < k1; ++k) {
      const f32x4_t x = *reinterpret_cast<const f32x4_t*>(part + k * W + j);
      a[0] += x[0]; a[1] += x[1]; a[2] += x[2]; a[3] += x[3];
    }
  }
  red[sl][cq] = a;
  __syncthreads();
  if (sl == 0 && j < W) {
#pragma unroll 8
    for (int k = 1; k < SLICES; ++k) {
      const f32x4_t x = red[k][cq];
      a[0] += x[0]; a[1] += x[1]; a[2] += x[2]; a[3] += x[3];
    }
    float* dst = j < H ? dgamma + j : dbeta + (j - H);
    *reinterpret_cast<f32x4_t*>(dst) = a;
  }
}

static tps_status ln_checks(const char* fn, std::initializer_list<tps_dtype> dts, int64_t M, int64_t H,
                            std::initializer_list<const void*> ptrs) {
  for (tps_dtype d : dts)
    if (d != TPS_F32 && d != TPS_BF16) return set_error(TPS_EINVAL, std::string(fn) + ": bad dtype");
  if (M <= 0 || H <= 0 || M >= 0x7fffffffLL) return set_error(TPS_EINVAL, std::string(fn) + ": need 0 < M < 2^31, H > 0");
  if (H % kLnV) return set_error(TPS_EINVAL, std::string(fn) + ": H must be a multiple of 8");
  for (const void* p : ptrs) {
    if (!p) return set_error(TPS_EINVAL, std::string(fn) + ": null pointer");
    if (!aligned16(p)) return set_error(TPS_EINVAL, std::string(fn) + ": pointer not 16-byte aligned");
  }
  if (H > kLnMaxH) return set_error(TPS_EUNSUPPORTED, std::string(fn) + ": H > 8192");
  return TPS_OK;
}

template <typename TX, typename TY>
static void launch_ln_fwd(int64_t M, int64_t H, float eps, const void* x, const float* g, const float* b, void* y,
                          float* mean, float* rstd, hipStream_t st) {
  const int nc = (int)ceil_div(H, 256 * kLnV);   // 1..4 (H <= 8192)
  TraceScope trace_(st, "ln_fwd_kernel");
#define TPS_LNF(NC)                                                                                             \
  hipLaunchKernelGGL((ln_fwd_kernel<TX, TY, NC>), dim3((unsigned)M), dim3(256), 0, st, static_cast<const TX*>(x), g, \
                     b, static_cast<TY*>(y), mean, rstd, H, eps)
  if (nc == 1) TPS_LNF(1);
  else if (nc == 2) TPS_LNF(2);
  else if (nc == 3) TPS_LNF(3);
  else TPS_LNF(4);
#undef TPS_LNF
}

template <bool RES, typename TX, typename TDY, typename TDX>
static void launch_ln_bwd(int64_t M, int64_t H, const void* x, const float* g, const float* mean, const float* rstd,
                          const void* dy, void* dx, float* part, const float* res, bf16_t* copy, hipStream_t st) {
  const dim3 grid((unsigned)ceil_div(M, kLnRowsPerBlock));
  const TX* xp = static_cast<const TX*>(x);
  const TDY* dyp = static_cast<const TDY*>(dy);
  TDX* dxp = static_cast<TDX*>(dx);
  constexpr int64_t W1 = (int64_t)kLnBwdThreads * kLnV;   // 4096
  TraceScope trace_(st, H == W1 ? "ln_bwd_rows_kernel" : "ln_bwd_kernel");
  if (H == W1)
    hipLaunchKernelGGL((ln_bwd_rows_kernel<1, RES, TX, TDY, TDX>), grid, dim3(kLnBwdThreads), 0, st, xp, g, mean,
                       rstd, dyp, dxp, part, M, res, copy);
  else
    hipLaunchKernelGGL((ln_bwd_kernel<RES, TX, TDY, TDX>), grid, dim3(256), 0, st, xp, g, mean, rstd, dyp, dxp, part,
                       M, H, res, copy);
}

}  // namespace tps

using namespace tps;

extern "C" tps_status layernorm_fwd(tps_dtype x_dt, tps_dtype y_dt, int64_t M, int64_t H, float eps, const void* x,
                                    const float* gamma, const float* beta, void* y, float* mean, float* rstd,
                                    tps_stream_t stream) {
  ApiScope api_scope_("layernorm_fwd");
  tps_status s = ln_checks("layernorm_fwd", {x_dt, y_dt}, M, H, {x, gamma, beta, y, mean, rstd});
  if (s != TPS_OK) return s;
  if (!(eps >= 0.f)) return set_error(TPS_EINVAL, "layernorm_fwd: eps must be >= 0");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool xb = x_dt == TPS_BF16, yb = y_dt == TPS_BF16;
  if (xb && yb) launch_ln_fwd<bf16_t, bf16_t>(M, H, eps, x, gamma, beta, y, mean, rstd, st);
  else if (xb) launch_ln_fwd<bf16_t, float>(M, H, eps, x, gamma, beta, y, mean, rstd, st);
  else if (yb) launch_ln_fwd<float, bf16_t>(M, H, eps, x, gamma, beta, y, mean, rstd, st);
  else launch_ln_fwd<float, float>(M, H, eps, x, gamma, beta, y, mean, rstd, st);
  return check_launch("ln_fwd_kernel");
}

extern "C" size_t layernorm_bwd_workspace(int64_t M, int64_t H) {
  if (M <= 0 || H <= 0) return 0;
  return (size_t)ceil_div(M, kLnRowsPerBlock) * 2 * (size_t)H * sizeof(float);
}

extern "C" tps_status layernorm_bwd(tps_dtype x_dt, tps_dtype dy_dt, tps_dtype dx_dt, int64_t M, int64_t H,
                                    const void* x, const float* gamma, const float* mean, const float* rstd,
                                    const void* dy, void* dx, float* dgamma, float* dbeta, void* ws, size_t ws_bytes,
                                    tps_stream_t stream) {
  ApiScope api_scope_("layernorm_bwd");
  tps_status s = ln_checks("layernorm_bwd", {x_dt, dy_dt, dx_dt}, M, H, {x, gamma, mean, rstd, dy, dx, dgamma, dbeta, ws});
  if (s != TPS_OK) return s;
  if (ws_bytes < layernorm_bwd_workspace(M, H)) return set_error(TPS_EWORKSPACE, "layernorm_bwd: workspace too small");
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* part = static_cast<float*>(ws);
  const int k = (x_dt == TPS_BF16 ? 4 : 0) | (dy_dt == TPS_BF16 ? 2 : 0) | (dx_dt == TPS_BF16 ? 1 : 0);
  switch (k) {
    case 7: launch_ln_bwd<false, bf16_t, bf16_t, bf16_t>(M, H, x, gamma, mean, rstd, dy, dx, part, nullptr, nullptr, st); break;
    case 6: launch_ln_bwd<false, bf16_t, bf16_t, float>(M, H, x, gamma, mean, rstd, dy, dx, part, nullptr, nullptr, st); break;
    case 5: launch_ln_bwd<false, bf16_t, float, bf16_t>(M, H, x, gamma, mean, rstd, dy, dx, part, nullptr, nullptr, st); break;
    case 4: launch_ln_bwd<false, bf16_t, float, float>(M, H, x, gamma, mean, rstd, dy, dx, part, nullptr, nullptr, st); break;
    case 3: launch_ln_bwd<false, float, bf16_t, bf16_t>(M, H, x, gamma, mean, rstd, dy, dx, part, nullptr, nullptr, st); break;
    case 2: launch_ln_bwd<false, float, bf16_t, float>(M, H, x, gamma, mean, rstd, dy, dx, part, nullptr, nullptr, st); break;
    case 1: launch_ln_bwd<false, float, float, bf16_t>(M, H, x, gamma, mean, rstd, dy, dx, part, nullptr, nullptr, st); break;
    default: launch_ln_bwd<false, float, float, float>(M, H, x, gamma, mean, rstd, dy, dx, part, nullptr, nullptr, st); break;
  }
  s = check_launch("ln_bwd_kernel");
  if (s != TPS_OK) return s;
  const int64_t nblk = ceil_div(M, kLnRowsPerBlock);
  TraceScope trace_(st, "ln_param_reduce_kernel");
  hipLaunchKernelGGL(ln_param_reduce_kernel, dim3((unsigned)ceil_div(2 * H, 32)), dim3(256), 0, st, part, dgamma,
                     dbeta, nblk, H);
  return check_launch("ln_param_reduce_kernel");
}

extern "C" tps_status layernorm_bwd_residual(tps_dtype x_dt, tps_dtype dy_dt, int64_t M, int64_t H, const void* x,
                                             const float* gamma, const float* mean, const float* rstd,
                                             const void* dy, const float* res, float* out, void* out_copy,
                                             float* dgamma, float* dbeta, void* ws, size_t ws_bytes,
                                             tps_stream_t stream) {
  ApiScope api_scope_("layernorm_bwd_residual");
  tps_status s = ln_checks("layernorm_bwd_residual", {x_dt, dy_dt}, M, H,
                           {x, gamma, mean, rstd, dy, res, out, dgamma, dbeta, ws});
  if (s != TPS_OK) return s;
  if (out_copy && !aligned16(out_copy))
    return set_error(TPS_EINVAL, "layernorm_bwd_residual: out_copy not 16-byte aligned");
  if ((const void*)res == (const void*)out) return set_error(TPS_EINVAL, "layernorm_bwd_residual: out must not alias res");
  if (ws_bytes < layernorm_bwd_workspace(M, H))
    return set_error(TPS_EWORKSPACE, "layernorm_bwd_residual: workspace too small");
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* part = static_cast<float*>(ws);
  bf16_t* copy = static_cast<bf16_t*>(out_copy);
  const int k = (x_dt == TPS_BF16 ? 2 : 0) | (dy_dt == TPS_BF16 ? 1 : 0);
  switch (k) {
    case 3: launch_ln_bwd<true, bf16_t, bf16_t, float>(M, H, x, gamma, mean, rstd, dy, out, part, res, copy, st); break;
    case 2: launch_ln_bwd<true, bf16_t, float, float>(M, H, x, gamma, mean, rstd, dy, out, part, res, copy, st); break;
    case 1: launch_ln_bwd<true, float, bf16_t, float>(M, H, x, gamma, mean, rstd, dy, out, part, res, copy, st); break;
    default: launch_ln_bwd<true, float, float, float>(M, H, x, gamma, mean, rstd, dy, out, part, res, copy, st); break;
  }
  s = check_launch("ln_bwd_kernel");
  if (s != TPS_OK) return s;
  const int64_t nblk = ceil_div(M, kLnRowsPerBlock);
  TraceScope trace_(st, "ln_param_reduce_kernel");
  hipLaunchKernelGGL(ln_param_reduce_kernel, dim3((unsigned)ceil_div(2 * H, 32)), dim3(256), 0, st, part, dgamma,
                     dbeta, nblk, H);
  return check_launch("ln_param_reduce_kernel");
}
