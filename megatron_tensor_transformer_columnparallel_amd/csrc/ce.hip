// Vocab-parallel cross entropy over the shards of the tied logits.
//
// The method (page "5-megatron", section _VocabParallelCrossEntropy; page
// "notion 310f8c09", section 交叉熵张量并行) takes, per token, the maximum
// logit over all shards (a MAX all-reduce), subtracts it, picks the shifted
// logit at the target's column on the shard that owns the target (0
// elsewhere; a SUM all-reduce), sums exp of the shifted logits over all
// shards (a SUM all-reduce), and returns loss = log(sum) - pick; the backward
// is softmax - onehot(owned target) times the upstream gradient.
//
// Here each shard's logits are read once (vocab_ce_stats): per token the
// shard's own maximum m_r, the sum s_r of exp(x - m_r) over the shard, the
// raw target logit and whether the shard owns the target.  The exchange
// (vocab_ce_combine) forms the global maximum m = max_r m_r, the sum
// sum_r s_r exp(m_r - m) -- equal to the sum of exp(x - m) over every shard --
// and the pick, then the loss and log-sum-exp lse = m + log(sum).  The
// backward (vocab_ce_bwd) reads each shard's logits once more and writes
// dL = dloss * (exp(x - lse) - [column is the target]).  All three are bound
// by HBM: the statistics take one wavefront per token row, the backward one
// workgroup per row; 16-byte vectors, every load issued unconditionally at a
// clamped chunk so that a whole group is in flight.
#include <math.h>

#include "common.hpp"

namespace tps {

namespace {

struct StatPtrs {
  const float* p[8];
};

// Chunk cc (VEC elements, wholly inside the row's stride) of a row as fp32.
template <typename T>
__device__ __forceinline__ void load_whole_chunk(const T* row, int cc, float* v) {
  if constexpr (sizeof(T) == 2) {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(row + (int64_t)cc * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[2 * i] = bf16lo(w[i]); v[2 * i + 1] = bf16hi(w[i]); }
  } else {
    const f32x4_t w = *reinterpret_cast<const f32x4_t*>(row + (int64_t)cc * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = w[i];
  }
}

// Chunk c of a row, read at chunk min(c, nch - 1): the last chunk holding a
// valid column, inside the row's stride (a multiple of VEC).  Callers mask
// what lies past the row.
template <typename T>
__device__ __forceinline__ void load_chunk(const T* row, int c, int nch, float* v) {
  load_whole_chunk<T>(row, c < nch ? c : nch - 1, v);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

constexpr int kGroup = 8;                        // chunks per lane in flight at once
constexpr float kLog2e = 1.4426950408889634f;
// exp(x - m) as 2^((x - m) log2 e) with the hardware 2^x.  The difference
// comes first (exact when x is near m), so large logits lose nothing there.
__device__ __forceinline__ float exp_shifted(float x, float m) {
  return __builtin_amdgcn_exp2f((x - m) * kLog2e);
}

// One wavefront per token row: (m_r, s_r, target logit, owned) as 4 floats.
// Each lane keeps a running maximum and a sum relative to it over groups of
// kGroup chunks (the sum is rescaled when a group raises the maximum); the
// lanes' pairs are then combined across the wave the same way.  Only a chunk
// that reaches past the row masks its elements (to -inf).
template <typename T>
__global__ void __launch_bounds__(256) ce_stats_kernel(const T* __restrict__ L, int64_t ldl, int64_t ntok,
                                                       int v_rows, int64_t v_start,
                                                       const int32_t* __restrict__ targets,
                                                       float* __restrict__ stats) {
  constexpr int VEC = 16 / sizeof(T);
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= ntok) return;
  const int lane = threadIdx.x & 63;
  const T* row = L + t * ldl;
  const int nch = (v_rows + VEC - 1) / VEC;
  // the target's column, read unconditionally (clamped) and kept only when owned
  const int64_t tl = (int64_t)targets[t] - v_start;
  const bool own = tl >= 0 && tl < v_rows;
  const float xt = Elem<T>::to_f32(row[tl < 0 ? 0 : (tl < v_rows ? tl : v_rows - 1)]);
  float m = -INFINITY, s = 0.f;
  // one group: kGroup chunks per lane (c0, c0 + 64, ...), their maximum,
  // then the sum rescaled to it
  auto group = [&](float (&v)[kGroup][VEC]) {
    float gm = m;
#pragma unroll
    for (int g = 0; g < kGroup; ++g)
#pragma unroll
      for (int e = 0; e < VEC; ++e) gm = fmaxf(gm, v[g][e]);
    // m == -inf only before a lane's first valid column: nothing to rescale then
    float acc = m == -INFINITY ? 0.f : s * exp_shifted(m, gm);
#pragma unroll
    for (int g = 0; g < kGroup; ++g)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc += exp_shifted(v[g][e], gm);
    m = gm;
    s = acc;
  };
  // groups whose chunks lie wholly inside the row for every lane (the
  // same for the whole wave): no clamping, no masking
  const int full = v_rows / VEC / (64 * kGroup);
  int c0 = lane;
  for (int gi = 0; gi < full; ++gi, c0 += 64 * kGroup) {
    float v[kGroup][VEC];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) load_whole_chunk<T>(row, c0 + g * 64, v[g]);
    group(v);
  }
  for (; c0 < nch; c0 += 64 * kGroup) {
    float v[kGroup][VEC];
    // every load of the group first: a branch between two loads makes the
    // second wait for the first
#pragma unroll
    for (int g = 0; g < kGroup; ++g) load_chunk<T>(row, c0 + g * 64, nch, v[g]);
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const int c = c0 + g * 64;
      if (c * VEC + VEC > v_rows) {   // past the row, or its partial last chunk
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          if (c * VEC + e >= v_rows) v[g][e] = -INFINITY;
      }
    }
    group(v);
  }
  const float mw = wave_max(m);
  const float sw = wave_sum(m == -INFINITY ? 0.f : s * exp_shifted(m, mw));
  if (lane == 0) {
    const f32x4_t out = {mw, sw, own ? xt : 0.f, own ? 1.f : 0.f};
    *reinterpret_cast<f32x4_t*>(stats + 4 * t) = out;
  }
}

// One thread per token: the exchange over the shards' statistics, in shard
// order.
__global__ void __launch_bounds__(256) ce_combine_kernel(StatPtrs st, int np, int64_t ntok,
                                                         float* __restrict__ loss, float* __restrict__ lse) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= ntok) return;
  f32x4_t v[8];
#pragma unroll
  for (int r = 0; r < 8; ++r)
    if (r < np) v[r] = *reinterpret_cast<const f32x4_t*>(st.p[r] + 4 * t);
  float m = -INFINITY;
#pragma unroll
  for (int r = 0; r < 8; ++r)
    if (r < np) m = fmaxf(m, v[r][0]);
  float denom = 0.f, pick = 0.f;
#pragma unroll
  for (int r = 0; r < 8; ++r)
    if (r < np) {
      denom += v[r][1] * __expf(v[r][0] - m);
      if (v[r][3] != 0.f) pick += v[r][2] - m;
    }
  const float ld = __logf(denom);
  loss[t] = ld - pick;
  lse[t] = m + ld;
}

// One workgroup per token row (grid-stride over rows; consecutive lanes take
// consecutive 16-byte chunks, so the row streams contiguously):
// dL = dloss * (exp(x - lse) - [column = target]).
// Columns past v_rows (up to the row stride) are neither used nor written.
// The target's column is tested once per chunk; bf16 results are rounded to
// nearest-even by the hardware pair conversion.
template <typename T>
__global__ void __launch_bounds__(256) ce_bwd_kernel(const T* L, int64_t ldl, int64_t ntok, int v_rows,
                                                     int64_t v_start, const int32_t* __restrict__ targets,
                                                     const float* __restrict__ lse,
                                                     const float* __restrict__ dloss, T* dL) {
  constexpr int VEC = 16 / sizeof(T);
  const int lane = threadIdx.x;
  const int nch = (v_rows + VEC - 1) / VEC;
  // one workgroup per row at a time: its 256 lanes stream the row contiguously
  const int full = v_rows / VEC / (256 * kGroup);   // groups wholly inside the row
  for (int64_t t = blockIdx.x; t < ntok; t += gridDim.x) {
    const T* row = L + t * ldl;
    T* drow = dL + t * ldl;
    const int64_t tl64 = (int64_t)targets[t] - v_start;
    const int tl = (tl64 >= 0 && tl64 < v_rows) ? (int)tl64 : -VEC;   // owned column, or none
    const float l = lse[t], g = dloss[t];
    // whole groups: exp only.  An owned target that falls here is rewritten
    // afterwards by the lane that stores its chunk (chunk c belongs to lane
    // c mod 256), which reads the target's logit before any of its stores
    // (dL may be L; no other lane writes that chunk).
    const bool fix = tl >= 0 && tl < full * 256 * kGroup * VEC && lane == (tl / VEC) % 256;
    const float xt = Elem<T>::to_f32(row[tl >= 0 ? tl : 0]);
    int c0 = lane;
    for (int gi = 0; gi < full; ++gi, c0 += 256 * kGroup) {
      float v[kGroup][VEC];
#pragma unroll
      for (int k = 0; k < kGroup; ++k) load_whole_chunk<T>(row, c0 + k * 256, v[k]);
#pragma unroll
      for (int k = 0; k < kGroup; ++k) {
        const int c = c0 + k * 256;
        float o[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = g * exp_shifted(v[k][e], l);
        if constexpr (sizeof(T) == 2) {
          typedef float f2 __attribute__((ext_vector_type(2)));
          typedef __bf16 b2 __attribute__((ext_vector_type(2)));
          u32x4_t w;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{o[2 * i], o[2 * i + 1]}, b2));
          *reinterpret_cast<u32x4_t*>(reinterpret_cast<bf16_t*>(drow) + (int64_t)c * 8) = w;
        } else {
          store4<float>(reinterpret_cast<float*>(drow) + (int64_t)c * 4, o, VEC);
        }
      }
    }
    for (; c0 < nch; c0 += 256 * kGroup) {
      float v[kGroup][VEC];
#pragma unroll
      for (int k = 0; k < kGroup; ++k) load_chunk<T>(row, c0 + k * 256, nch, v[k]);
#pragma unroll
      for (int k = 0; k < kGroup; ++k) {
        const int c = c0 + k * 256;
        if (c >= nch) continue;
        float o[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = g * exp_shifted(v[k][e], l);
        if (tl - c * VEC >= 0 && tl - c * VEC < VEC) {   // the chunk holding the owned target
#pragma unroll
          for (int e = 0; e < VEC; ++e)
            if (c * VEC + e == tl) o[e] -= g;
        }
        if constexpr (sizeof(T) == 2) {
          if (c * VEC + VEC <= v_rows) {
            typedef float f2 __attribute__((ext_vector_type(2)));
            typedef __bf16 b2 __attribute__((ext_vector_type(2)));
            u32x4_t w;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{o[2 * i], o[2 * i + 1]}, b2));
            *reinterpret_cast<u32x4_t*>(reinterpret_cast<bf16_t*>(drow) + (int64_t)c * 8) = w;
          } else {
            store8<bf16_t>(reinterpret_cast<bf16_t*>(drow) + (int64_t)c * 8, o, v_rows - c * VEC);
          }
        } else {
          store4<float>(reinterpret_cast<float*>(drow) + (int64_t)c * 4, o,
                        v_rows - c * VEC < VEC ? v_rows - c * VEC : VEC);
        }
      }
    }
    if (fix) {   // after this lane's own store of the chunk (same address, program order)
      float o = g * exp_shifted(xt, l);
      o -= g;
      if constexpr (sizeof(T) == 2) {
        typedef float f2 __attribute__((ext_vector_type(2)));
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{o, 0.f}, b2));
        reinterpret_cast<bf16_t*>(drow)[tl] = (bf16_t)(w & 0xffffu);
      } else {
        reinterpret_cast<float*>(drow)[tl] = o;
      }
    }
  }
}

tps_status ce_row_checks(const char* fn, tps_dtype dt, int64_t T, int64_t v_rows, int64_t ldl, int64_t v_start) {
  if (dt != TPS_F32 && dt != TPS_BF16) return set_error(TPS_EINVAL, std::string(fn) + ": bad dtype");
  if (T < 0 || v_rows <= 0 || v_start < 0)
    return set_error(TPS_EINVAL, std::string(fn) + ": need T >= 0, v_rows > 0, v_start >= 0");
  if (ldl < v_rows || ldl % vec_elems(dt))
    return set_error(TPS_EINVAL, std::string(fn) + ": ldl must be >= v_rows and a multiple of 8 (bf16) / 4 (fp32)");
  if (T >= 0x7fffffffLL * 4) return set_error(TPS_EINVAL, std::string(fn) + ": T too large");
  if (v_rows > 0x7fffffffLL - 64) return set_error(TPS_EINVAL, std::string(fn) + ": v_rows must fit in int32");
  return TPS_OK;
}

}  // namespace

}  // namespace tps

using namespace tps;

extern "C" tps_status vocab_ce_stats(tps_dtype dt, int64_t T, int64_t v_rows, int64_t ldl, int64_t v_start,
                                     const void* L_r, const int32_t* targets, float* stats_r,
                                     tps_stream_t stream) {
  ApiScope api_scope_("vocab_ce_stats");
  tps_status s = ce_row_checks("vocab_ce_stats", dt, T, v_rows, ldl, v_start);
  if (s != TPS_OK) return s;
  if (!L_r || !targets || !stats_r) return set_error(TPS_EINVAL, "vocab_ce_stats: null pointer");
  if (!aligned16(L_r) || !aligned16(stats_r))
    return set_error(TPS_EINVAL, "vocab_ce_stats: L_r and stats_r must be 16-byte aligned");
  if (T == 0) return TPS_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)ceil_div(T, 4));
  TraceScope trace_(st, "ce_stats_kernel");
  if (dt == TPS_BF16)
    hipLaunchKernelGGL(ce_stats_kernel<bf16_t>, grid, dim3(256), 0, st, static_cast<const bf16_t*>(L_r), ldl, T,
                       (int)v_rows, v_start, targets, stats_r);
  else
    hipLaunchKernelGGL(ce_stats_kernel<float>, grid, dim3(256), 0, st, static_cast<const float*>(L_r), ldl, T,
                       (int)v_rows, v_start, targets, stats_r);
  return check_launch("ce_stats_kernel");
}

extern "C" tps_status vocab_ce_combine(int n_parts, const float* const* stats, int64_t T, float* loss, float* lse,
                                       tps_stream_t stream) {
  ApiScope api_scope_("vocab_ce_combine");
  if (n_parts < 1 || n_parts > 8) return set_error(TPS_EINVAL, "vocab_ce_combine: n_parts must be 1..8");
  if (T < 0) return set_error(TPS_EINVAL, "vocab_ce_combine: T < 0");
  if (!stats || !loss || !lse) return set_error(TPS_EINVAL, "vocab_ce_combine: null pointer");
  StatPtrs sp{};
  for (int r = 0; r < n_parts; ++r) {
    if (!stats[r]) return set_error(TPS_EINVAL, "vocab_ce_combine: null statistics pointer");
    if (!aligned16(stats[r])) return set_error(TPS_EINVAL, "vocab_ce_combine: statistics must be 16-byte aligned");
    sp.p[r] = stats[r];
  }
  if (T == 0) return TPS_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  TraceScope trace_(st, "ce_combine_kernel");
  hipLaunchKernelGGL(ce_combine_kernel, dim3((unsigned)ceil_div(T, 256)), dim3(256), 0, st, sp, n_parts, T, loss,
                     lse);
  return check_launch("ce_combine_kernel");
}

extern "C" tps_status vocab_ce_bwd(tps_dtype dt, int64_t T, int64_t v_rows, int64_t ldl, int64_t v_start,
                                   const void* L_r, const int32_t* targets, const float* lse, const float* dloss,
                                   void* dL_r, tps_stream_t stream) {
  ApiScope api_scope_("vocab_ce_bwd");
  tps_status s = ce_row_checks("vocab_ce_bwd", dt, T, v_rows, ldl, v_start);
  if (s != TPS_OK) return s;
  if (!L_r || !targets || !lse || !dloss || !dL_r) return set_error(TPS_EINVAL, "vocab_ce_bwd: null pointer");
  if (!aligned16(L_r) || !aligned16(dL_r))
    return set_error(TPS_EINVAL, "vocab_ce_bwd: L_r and dL_r must be 16-byte aligned");
  if (T == 0) return TPS_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)(T < 65536 ? T : 65536));
  TraceScope trace_(st, "ce_bwd_kernel");
  if (dt == TPS_BF16)
    hipLaunchKernelGGL(ce_bwd_kernel<bf16_t>, grid, dim3(256), 0, st, static_cast<const bf16_t*>(L_r), ldl, T,
                       (int)v_rows, v_start, targets, lse, dloss, static_cast<bf16_t*>(dL_r));
  else
    hipLaunchKernelGGL(ce_bwd_kernel<float>, grid, dim3(256), 0, st, static_cast<const float*>(L_r), ldl, T,
                       (int)v_rows, v_start, targets, lse, dloss, static_cast<float*>(dL_r));
  return check_launch("ce_bwd_kernel");
}
