// Column/row-parallel MLP shard and the tied output projection, composed from
// the GEMM kernels with fused epilogues (GELU forward, GELU' backward).
//
// Operand layouts used below (math layout, row-major):
//   NN  A K-contiguous, B N-contiguous     e.g. X [M x h] * A_i [h x f]
//   NT  A K-contiguous, B K-contiguous     e.g. dZ [M x h] * B_i^T, B_i [f x h]
//   TN  A M-contiguous, B N-contiguous     e.g. H_i^T dZ, H_i [M x f]
#include <string>

#include "gemm.hpp"

namespace tps {

static GemmShape shape(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb) {
  GemmShape s;
  s.M = (int)M; s.N = (int)N; s.K = (int)K; s.lda = lda; s.ldb = ldb;
  return s;
}

static bool fits_int(int64_t x) { return x >= 0 && x < 0x7fffffffLL; }

#define TPS_REQ(cond, msg) \
  do { if (!(cond)) return set_error(TPS_EINVAL, std::string(__func__) + ": " + (msg)); } while (0)
#define TPS_TRY(expr) \
  do { tps_status _s = (expr); if (_s != TPS_OK) return _s; } while (0)

// C[M x N] (ld = ldc) = A op B, with the layouts above; T = element type.
template <typename T, bool AK, bool BKC, class Epi>
static tps_status run_gemm(const T* A, const T* B, const GemmShape& s, const Epi& e, hipStream_t st) {
  if constexpr (sizeof(T) == 2) return gemm_bf16<AK, BKC>(A, B, s, e, st);
  else return gemm_f32<AK, BKC>(A, B, s, e, st);
}

template <typename T>
static tps_status mlp_fwd_t(int64_t M, int64_t h, int64_t f, const T* X, const T* A, const T* B, T* P, T* H,
                            T* Z, hipStream_t st) {
  // P = X A_i ; H = gelu(P)                (NN, epilogue GELU)
  TPS_TRY((run_gemm<T, true, false>(X, A, shape(M, f, h, h, f), EpiGelu<T>{P, H, f}, st)));
  // Z_i = H_i B_i                          (NN)
  return run_gemm<T, true, false>(H, B, shape(M, h, f, f, h), EpiStore<T>{Z, h, 0, 0}, st);
}

template <typename T>
static tps_status mlp_bwd_t(int64_t M, int64_t h, int64_t f, const T* X, const T* A, const T* B, const T* P,
                            const T* H, const T* dZ, T* dX, T* dA, T* dB, T* dP, hipStream_t st) {
  // dB_i = H_i^T dZ                        (TN)  [f x h], K = M
  TPS_TRY((run_gemm<T, false, false>(H, dZ, shape(f, h, M, f, h), EpiStore<T>{dB, h, 0, 0}, st)));
  // dP = (dZ B_i^T) * gelu'(P)             (NT)  [M x f], K = h
  TPS_TRY((run_gemm<T, true, true>(dZ, B, shape(M, f, h, h, h), EpiGeluBwd<T>{P, dP, f}, st)));
  // dA_i = X^T dP                          (TN)  [h x f], K = M
  TPS_TRY((run_gemm<T, false, false>(X, dP, shape(h, f, M, h, f), EpiStore<T>{dA, f, 0, 0}, st)));
  // dX_i = dP A_i^T                        (NT)  [M x h], K = f
  return run_gemm<T, true, true>(dP, A, shape(M, h, f, f, f), EpiStore<T>{dX, h, 0, 0}, st);
}

static tps_status mlp_checks(const char* fn, tps_dtype dt, int64_t M, int64_t h, int64_t f,
                             std::initializer_list<const void*> ptrs) {
  if (dt != TPS_F32 && dt != TPS_BF16) return set_error(TPS_EINVAL, std::string(fn) + ": bad dtype");
  if (M <= 0 || h <= 0 || f <= 0) return set_error(TPS_EINVAL, std::string(fn) + ": dims must be > 0");
  if (!fits_int(M) || !fits_int(h) || !fits_int(f)) return set_error(TPS_EINVAL, std::string(fn) + ": dims must be < 2^31");
  if (h % vec_elems(dt) || f % vec_elems(dt))
    return set_error(TPS_EINVAL, std::string(fn) + ": h and f_i must be multiples of 8 (bf16) / 4 (fp32)");
  for (const void* p : ptrs) {
    if (!p) return set_error(TPS_EINVAL, std::string(fn) + ": null pointer");
    if (!aligned16(p)) return set_error(TPS_EINVAL, std::string(fn) + ": pointer not 16-byte aligned");
  }
  return TPS_OK;
}

}  // namespace tps

using namespace tps;

extern "C" tps_status tp_mlp_fwd(tps_dtype dt, int64_t M, int64_t h, int64_t f_i, const void* X, const void* A_i,
                                 const void* B_i, void* P_i, void* H_i, void* Z_i, tps_stream_t stream) {
  ApiScope api_scope_("tp_mlp_fwd");
  TPS_TRY(mlp_checks("tp_mlp_fwd", dt, M, h, f_i, {X, A_i, B_i, P_i, H_i, Z_i}));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dt == TPS_BF16)
    return mlp_fwd_t<bf16_t>(M, h, f_i, (const bf16_t*)X, (const bf16_t*)A_i, (const bf16_t*)B_i, (bf16_t*)P_i,
                             (bf16_t*)H_i, (bf16_t*)Z_i, st);
  return mlp_fwd_t<float>(M, h, f_i, (const float*)X, (const float*)A_i, (const float*)B_i, (float*)P_i,
                          (float*)H_i, (float*)Z_i, st);
}

extern "C" size_t tp_mlp_bwd_workspace(tps_dtype dt, int64_t M, int64_t h, int64_t f_i) {
  (void)h;
  if (M <= 0 || f_i <= 0) return 0;
  return (size_t)M * (size_t)f_i * elem_bytes(dt);
}

extern "C" tps_status tp_mlp_bwd(tps_dtype dt, int64_t M, int64_t h, int64_t f_i, const void* X, const void* A_i,
                                 const void* B_i, const void* P_i, const void* H_i, const void* dZ, void* dX_i,
                                 void* dA_i, void* dB_i, void* ws, size_t ws_bytes, tps_stream_t stream) {
  ApiScope api_scope_("tp_mlp_bwd");
  TPS_TRY(mlp_checks("tp_mlp_bwd", dt, M, h, f_i, {X, A_i, B_i, P_i, H_i, dZ, dX_i, dA_i, dB_i, ws}));
  if (ws_bytes < tp_mlp_bwd_workspace(dt, M, h, f_i))
    return set_error(TPS_EWORKSPACE, "tp_mlp_bwd: workspace too small");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dt == TPS_BF16)
    return mlp_bwd_t<bf16_t>(M, h, f_i, (const bf16_t*)X, (const bf16_t*)A_i, (const bf16_t*)B_i,
                             (const bf16_t*)P_i, (const bf16_t*)H_i, (const bf16_t*)dZ, (bf16_t*)dX_i,
                             (bf16_t*)dA_i, (bf16_t*)dB_i, (bf16_t*)ws, st);
  return mlp_bwd_t<float>(M, h, f_i, (const float*)X, (const float*)A_i, (const float*)B_i, (const float*)P_i,
                          (const float*)H_i, (const float*)dZ, (float*)dX_i, (float*)dA_i, (float*)dB_i,
                          (float*)ws, st);
}

// ---------------------------------------------------------------- tied logits

static tps_status logits_checks(const char* fn, tps_dtype dt, int64_t T, int64_t H, int64_t v_rows, int64_t ldl,
                                std::initializer_list<const void*> ptrs) {
  if (dt != TPS_F32 && dt != TPS_BF16) return set_error(TPS_EINVAL, std::string(fn) + ": bad dtype");
  if (T <= 0 || H <= 0 || v_rows <= 0) return set_error(TPS_EINVAL, std::string(fn) + ": dims must be > 0");
  if (!fits_int(T) || !fits_int(H) || !fits_int(v_rows) || !fits_int(ldl))
    return set_error(TPS_EINVAL, std::string(fn) + ": dims must be < 2^31");
  if (ldl < v_rows) return set_error(TPS_EINVAL, std::string(fn) + ": ldl < v_rows");
  if (ldl % vec_elems(dt) || H % vec_elems(dt))
    return set_error(TPS_EINVAL, std::string(fn) + ": ldl and H must be multiples of 8 (bf16) / 4 (fp32)");
  for (const void* p : ptrs) {
    if (!p) return set_error(TPS_EINVAL, std::string(fn) + ": null pointer");
    if (!aligned16(p)) return set_error(TPS_EINVAL, std::string(fn) + ": pointer not 16-byte aligned");
  }
  return TPS_OK;
}

extern "C" tps_status tied_logits(tps_dtype dt, int64_t T, int64_t H, int64_t v_rows, int64_t ldl, const void* X,
                                  const void* E_r, void* L_r, tps_stream_t stream) {
  ApiScope api_scope_("tied_logits");
  TPS_TRY(logits_checks("tied_logits", dt, T, H, v_rows, ldl, {X, E_r, L_r}));
  hipStream_t st = static_cast<hipStream_t>(stream);
  // L_r = X E_r^T                          (NT)  [T x v_rows], K = H
  const GemmShape s = shape(T, v_rows, H, H, H);
  if (dt == TPS_BF16)
    return run_gemm<bf16_t, true, true>((const bf16_t*)X, (const bf16_t*)E_r, s,
                                        EpiStore<bf16_t>{(bf16_t*)L_r, ldl, 0, 0}, st);
  return run_gemm<float, true, true>((const float*)X, (const float*)E_r, s, EpiStore<float>{(float*)L_r, ldl, 0, 0},
                                     st);
}

extern "C" tps_status tied_logits_bwd(tps_dtype dt, int64_t T, int64_t H, int64_t v_rows, int64_t ldl,
                                      const void* X, const void* E_r, const void* dL_r, void* dX_r, float* dE_r,
                                      tps_stream_t stream) {
  ApiScope api_scope_("tied_logits_bwd");
  TPS_TRY(logits_checks("tied_logits_bwd", dt, T, H, v_rows, ldl, {X, E_r, dL_r, dX_r, dE_r}));
  hipStream_t st = static_cast<hipStream_t>(stream);
  // dX_r = dL_r E_r                        (NN)  [T x H], K = v_rows
  const GemmShape s1 = shape(T, H, v_rows, ldl, H);
  // dE_r = dL_r^T X                        (TN)  [v_rows x H] fp32, K = T
  const GemmShape s2 = shape(v_rows, H, T, ldl, H);
  if (dt == TPS_BF16) {
    TPS_TRY((run_gemm<bf16_t, true, false>((const bf16_t*)dL_r, (const bf16_t*)E_r, s1,
                                           EpiStore<bf16_t>{(bf16_t*)dX_r, H, 0, 0}, st)));
    return run_gemm<bf16_t, false, false>((const bf16_t*)dL_r, (const bf16_t*)X, s2,
                                          EpiStore<float>{dE_r, H, 0, 0}, st);
  }
  TPS_TRY((run_gemm<float, true, false>((const float*)dL_r, (const float*)E_r, s1,
                                        EpiStore<float>{(float*)dX_r, H, 0, 0}, st)));
  return run_gemm<float, false, false>((const float*)dL_r, (const float*)X, s2, EpiStore<float>{dE_r, H, 0, 0}, st);
}
