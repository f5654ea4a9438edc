// Vocab-parallel word embedding, one shard.
//
// Forward (vocab_embed_fwd): a masked row gather.  One wavefront per token
// copies the table row (16-byte vectors) or writes zeros when the id falls
// outside [v_start, v_start + v_rows).  HBM-bound: reads the in-range rows
// once, writes every output row once.
//
// Backward (vocab_embed_bwd): dE_r[id - v_start] += dY[t] for in-range t.
// Deterministic and free of atomics: the composite keys (local_row << 32 | t)
// are unique, so sorting them (a radix sort per bucket of rows, or a bitonic
// network past 16384 tokens) yields one fixed order, with each row's tokens
// contiguous and ascending in t.  One wavefront per segment
// head then adds that row's dY rows, in that order, to the row of dE_r in
// fp32 with a plain read-modify-write (each row has exactly one owner).
#include <mutex>

#include "common.hpp"

namespace tps {

// One wavefront per token.  Every lane issues all of its 16-byte loads for
// a slab of 64 x 8 chunks before any store, so a whole 8 KiB bf16 row is in
// flight at once.  The output rows are written with non-temporal stores: they
// are not read again by this kernel, and keeping them out of the caches leaves
// room for the table rows (measured 43 -> 30 us for 16384 tokens of 4096).
template <typename T>
__global__ void __launch_bounds__(256) embed_fwd_kernel(const int32_t* __restrict__ ids,
                                                         const T* __restrict__ E, T* __restrict__ Y,
                                                         int64_t ntok, int64_t H, int64_t v_start,
                                                         int64_t v_rows) {
  constexpr int U = 8;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= ntok) return;
  const int lane = threadIdx.x & 63;
  const int64_t local = (int64_t)ids[t] - v_start;
  const bool inr = local >= 0 && local < v_rows;
  const int64_t nch = H * (int64_t)sizeof(T) / 16;  // 16-byte chunks per row
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(Y + t * H);
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(E + (inr ? local : 0) * H);
  for (int64_t c0 = lane; c0 < nch; c0 += 64 * U) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * 64;
      v[u] = u32x4_t{0u, 0u, 0u, 0u};
      if (inr && c < nch) v[u] = src[c];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * 64;
      if (c < nch) __builtin_nontemporal_store(v[u], dst + c);
    }
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
        const int i = ((q & ~(j - 1)) << 1) | (q & (j - 1));   // j is a power of two
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

// Stable sort by row for T <= kRadixMax tokens, one workgroup per bucket of
// `bucket_rows` consecutive rows (a single workgroup when one bucket holds
// every row).  A bucket's tokens are first compacted, in token order, into
// 32-bit keys ((row - first row of the bucket) << tbits | t) (out-of-range
// tokens carry no gradient and only fill the tail of the output with
// kNoKey), so a stable LSD radix sort on those row bits (8 bits per pass)
// leaves each row's tokens ascending in t.  The bucket's keys go to the
// output after those of all earlier buckets -- the in-range tokens whose row
// lies below the bucket's, counted in the same pass over the ids -- so the
// buckets together give the same order as one sort of every key.  Per pass, each
// of the 16 waves owns a contiguous run of the keys and its own 256 digit
// counters; lanes with equal digits are found with eight ballots, so a
// block's count per digit and a lane's rank among earlier lanes with its
// digit need no atomics.  One exclusive scan over (digit, wave) in
// digit-major order gives every wave its starting position per digit.  The
// result is written as the 64-bit keys (row << 32 | t, or kNoKey) the
// accumulation kernel reads.
constexpr int kRadixMax = 16384;
constexpr int kRadixThreads = 1024;
constexpr int kRadixWaves = kRadixThreads / 64;

// Lanes of the wave holding the same 8-bit digit as this lane (among valid lanes).
__device__ __forceinline__ uint64_t same_digit_lanes(uint32_t d, bool valid) {
  uint64_t same = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const uint64_t bal = __ballot(valid && ((d >> bit) & 1u));
    same &= ((d >> bit) & 1u) ? bal : ~bal;
  }
  return same;
}

__global__ void __launch_bounds__(kRadixThreads) embed_radix_sort_kernel(const int32_t* __restrict__ ids,
                                                                          uint64_t* __restrict__ keys_out,
                                                                          int ntok, int64_t v_start,
                                                                          int v_rows, int tbits, int rbits,
                                                                          int bucket_rows) {
  __shared__ uint32_t kb[2][kRadixMax];
  __shared__ uint32_t off[kRadixWaves * 256];   // [wave][digit]: a wave's counters are contiguous
  __shared__ uint32_t wsum[kRadixWaves];
  __shared__ uint32_t wbelow[kRadixWaves];
  static_assert(256 * kRadixWaves == 4 * kRadixThreads, "scan: four entries per thread");
  __shared__ uint32_t nin_s, out0_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t tmask = (1u << tbits) - 1u;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int g = blockIdx.x;
  const int row_lo = g * bucket_rows;
  const int row_hi = min(v_rows, row_lo + bucket_rows);
  {
    // every wave compacts its own run of 64 * PER consecutive tokens: all id
    // loads in flight at once, the in-range lanes counted per chunk of 64 by
    // ballot, one barrier for the runs' totals, then the keys are written in
    // token order at the earlier runs' total plus the in-range lanes before
    // them
    constexpr int PER = kRadixMax / kRadixThreads;
    const int tb = wave * 64 * PER;
    int32_t idv[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      // unconditional loads (clamped index, validity checked below): a
      // guarded load would be waited for before the next one is issued
      const int t = tb + i * 64 + lane;
      idv[i] = ids[min(t, ntok - 1)];
    }
    uint32_t cnt = 0, below = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int t = tb + i * 64 + lane;
      const int64_t local = (int64_t)idv[i] - v_start;
      cnt += (uint32_t)__popcll(__ballot(t < ntok && local >= row_lo && local < row_hi));
      below += (uint32_t)__popcll(__ballot(t < ntok && local >= 0 && local < row_lo));
    }
    if (lane == 0) {
      wsum[wave] = cnt;
      wbelow[wave] = below;
    }
    __syncthreads();
    uint32_t pos = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kRadixWaves; ++w) {
      const uint32_t c = wsum[w];
      pos += w < wave ? c : 0u;
      all += c;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int t = tb + i * 64 + lane;
      const int64_t local = (int64_t)idv[i] - v_start;
      const bool in = t < ntok && local >= row_lo && local < row_hi;
      const uint64_t bal = __ballot(in);
      if (in) kb[0][pos + (uint32_t)__popcll(bal & lt_mask)] = ((uint32_t)(local - row_lo) << tbits) | (uint32_t)t;
      pos += (uint32_t)__popcll(bal);
    }
    if (tid == 0) {
      uint32_t b0 = 0;
      for (int w = 0; w < kRadixWaves; ++w) b0 += wbelow[w];
      nin_s = all;
      out0_s = b0;   // in-range tokens of the earlier buckets
    }
  }
  __syncthreads();
  const int nin = (int)nin_s;
  const uint32_t out0 = out0_s;
  const int per = (nin + kRadixWaves - 1) / kRadixWaves;   // keys per wave
  const int lo = min(nin, wave * per), hi = min(nin, lo + per);
  uint32_t* my = off + wave * 256;
  int cur = 0;
  for (int shift = 0; shift < rbits; shift += 8) {
    for (int i = lane; i < 256; i += 64) my[i] = 0u;
    // counts per (wave, digit): the first lane of each digit group adds the
    // group's size (only this wave touches its counters)
    for (int b = lo; b < hi; b += 64) {
      const int q = b + lane;
      const bool valid = q < hi;
      const uint32_t d = valid ? (kb[cur][q] >> tbits >> shift) & 255u : 0u;
      const uint64_t same = same_digit_lanes(d, valid);
      if (valid && (same & lt_mask) == 0) my[d] += (uint32_t)__popcll(same);
    }
    __syncthreads();
    // exclusive scan over (digit, wave) in digit-major order: entry e is
    // (digit e / 16, wave e % 16); 4 consecutive entries per thread, a
    // shuffle scan per wave, then the 16 wave totals
    {
      uint32_t c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = tid * 4 + i;
        c[i] = off[(e % kRadixWaves) * 256 + e / kRadixWaves];
      }
      const uint32_t mine = c[0] + c[1] + c[2] + c[3];
      uint32_t x = mine;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
      }
      if (lane == 63) wsum[wave] = x;
      __syncthreads();
      uint32_t run = x - mine;
      for (int w = 0; w < wave; ++w) run += wsum[w];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = tid * 4 + i;
        off[(e % kRadixWaves) * 256 + e / kRadixWaves] = run;
        run += c[i];
      }
    }
    __syncthreads();
    // stable scatter: rank among earlier lanes of the block with the same digit
    for (int b = lo; b < hi; b += 64) {
      const int q = b + lane;
      const bool valid = q < hi;
      const uint32_t key = valid ? kb[cur][q] : 0u;
      const uint32_t d = (key >> tbits >> shift) & 255u;
      const uint64_t same = same_digit_lanes(d, valid);
      const uint32_t rank = (uint32_t)__popcll(same & lt_mask);
      const uint32_t base = valid ? my[d] : 0u;
      if (valid) kb[cur ^ 1][base + rank] = key;
      // every lane of a digit group read the same base; the group's first lane advances it
      if (valid && rank == 0) my[d] = base + (uint32_t)__popcll(same);
    }
    cur ^= 1;
    __syncthreads();
  }
  for (int i = tid; i < nin; i += kRadixThreads) {
    const uint32_t key = kb[cur][i];
    keys_out[out0 + i] = ((uint64_t)((key >> tbits) + (uint32_t)row_lo) << 32) | (uint64_t)(key & tmask);
  }
  // the last bucket ends at the number of in-range tokens; the rest is kNoKey
  if (g == (int)gridDim.x - 1)
    for (int t = (int)out0 + nin + tid; t < ntok; t += kRadixThreads) keys_out[t] = kNoKey;
}

__global__ void __launch_bounds__(256) bitonic_global_kernel(uint64_t* keys, int64_t n, int64_t k, int64_t j) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= n / 2) return;
  const int64_t i = ((q & ~(j - 1)) << 1) | (q & (j - 1));   // j is a power of two
  const int64_t l = i + j;
  const bool asc = (i & k) == 0;
  const uint64_t a = keys[i], b = keys[l];
  if ((a > b) == asc) { keys[i] = b; keys[l] = a; }
}

// One wavefront per sorted position; a position that starts a row's segment
// owns that row.  The row goes in passes of NSL slabs of 256 columns; lane l
// holds columns 4l .. 4l+3 of each slab, so every load and store instruction
// of the wave covers one contiguous span (1 KiB of dE, 512 bytes of bf16 dY).
// A pass starts from the row's current dE (the output-side gradient) and adds
// the segment's dY rows in increasing token order in fp32, with the loads of
// two tokens in flight together.  The segment's tokens come 64 at a time (one
// key per lane; the segment ends at the first key of another row -- kNoKey
// sorts last and matches no row) and are read from the keys' lanes into
// scalar registers.  The finished pass is written back once, with
// non-temporal stores.
// 4 consecutive columns of a dY row as loaded (raw; `off` in bytes from the
// wave-uniform row start) and added into fp32.
template <typename T> struct AccumLoad;
template <> struct AccumLoad<bf16_t> {
  typedef u32x2_t raw;
  __device__ static raw get(const char* row, uint32_t off) { return *reinterpret_cast<const u32x2_t*>(row + off); }
  __device__ static void add(float a[4], raw x) {
    a[0] += bf16lo(x[0]); a[1] += bf16hi(x[0]); a[2] += bf16lo(x[1]); a[3] += bf16hi(x[1]);
  }
};
template <> struct AccumLoad<float> {
  typedef f32x4_t raw;
  __device__ static raw get(const char* row, uint32_t off) { return *reinterpret_cast<const f32x4_t*>(row + off); }
  __device__ static void add(float a[4], raw x) { a[0] += x[0]; a[1] += x[1]; a[2] += x[2]; a[3] += x[3]; }
};

template <typename T>
__global__ void __launch_bounds__(256) embed_bwd_accum_kernel(const uint64_t* __restrict__ keys,
                                                               const T* __restrict__ dY, float* __restrict__ dE,
                                                               int64_t ntok, int64_t H) {
  constexpr int NSL = 16;   // a 4096-column row in one pass
  const int64_t p = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (p >= ntok) return;
  const int lane = threadIdx.x & 63;
  // Keys of positions b .. b+63 (one per lane; kNoKey past the end), loaded
  // unconditionally at a clamped position.
  auto chunk_keys = [&](int64_t b) {
    const uint64_t k = keys[min(b + lane, ntok - 1)];
    return b + lane < ntok ? k : kNoKey;
  };
  // The first 64 keys from position p (kept for every pass) and the key
  // before p, loaded together; p's own key is lane 0's.
  const uint64_t k0 = chunk_keys(p);
  const uint64_t kprev = keys[p > 0 ? p - 1 : 0];
  const uint64_t key = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(k0 >> 32), 0) << 32) |
                       (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)k0, 0);
  const uint64_t row = key >> 32;
  // out of range, or not the head of its segment (one test, so that both
  // loads are issued before the branch)
  const bool skip = (key == kNoKey) | ((p > 0) & ((kprev >> 32) == row));
  if (skip) return;
  char* const drow = reinterpret_cast<char*>(dE + (int64_t)row * H);
  // keys of a chunk -> the number n of its leading positions in the segment
  // (a contiguous prefix) and the lanes' tokens
  auto segment = [&](uint64_t kq, int& n, int& tl) {
    const uint64_t in_seg = __ballot(kq != kNoKey && (kq >> 32) == row);
    n = in_seg == ~0ull ? 64 : (int)__builtin_ctzll(~in_seg);
    tl = (int)(kq & 0xffffffffu);
  };
  int n0, tl0;
  segment(k0, n0, tl0);
  // Every load below is unconditional, at a column clamped into the row
  // (H is a multiple of 4): a guarded load would be waited for before the
  // next one is issued.  Sums for columns past H are dropped at the store.
  // Addresses are a wave-uniform row start plus a 32-bit byte offset per
  // slab, shared by every row the pass touches.  The pass loop is uniform
  // over the wave (the ballots need every lane).
  for (int64_t cb = 0; cb < H; cb += 256 * NSL) {
    uint32_t col[NSL];
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) col[sl] = (uint32_t)min(cb + (int64_t)lane * 4 + sl * 256, H - 4);
    float acc[NSL][4];
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      const f32x4_t d = *reinterpret_cast<const f32x4_t*>(drow + col[sl] * 4u);
      acc[sl][0] = d[0]; acc[sl][1] = d[1]; acc[sl][2] = d[2]; acc[sl][3] = d[3];
    }
    // tokens 0 .. n-1 of a chunk, in order, two rows in flight at a time
    auto add_tokens = [&](int n, int tl) {
      int u = 0;
      for (; u + 2 <= n; u += 2) {
        const char* s0 = reinterpret_cast<const char*>(dY + (int64_t)__builtin_amdgcn_readlane(tl, u) * H);
        const char* s1 = reinterpret_cast<const char*>(dY + (int64_t)__builtin_amdgcn_readlane(tl, u + 1) * H);
        typename AccumLoad<T>::raw x0[NSL], x1[NSL];
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) {
          x0[sl] = AccumLoad<T>::get(s0, col[sl] * (uint32_t)sizeof(T));
          x1[sl] = AccumLoad<T>::get(s1, col[sl] * (uint32_t)sizeof(T));
        }
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) {
          AccumLoad<T>::add(acc[sl], x0[sl]);
          AccumLoad<T>::add(acc[sl], x1[sl]);
        }
      }
      if (u < n) {
        const char* s0 = reinterpret_cast<const char*>(dY + (int64_t)__builtin_amdgcn_readlane(tl, u) * H);
        typename AccumLoad<T>::raw x0[NSL];
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) x0[sl] = AccumLoad<T>::get(s0, col[sl] * (uint32_t)sizeof(T));
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) AccumLoad<T>::add(acc[sl], x0[sl]);
      }
    };
    add_tokens(n0, tl0);
    if (n0 == 64) {
      for (int64_t b = p + 64; b < ntok; b += 64) {
        int n, tl;
        segment(chunk_keys(b), n, tl);
        add_tokens(n, tl);
        if (n < 64) break;
      }
    }
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      if (cb + (int64_t)lane * 4 + sl * 256 < H)
        __builtin_nontemporal_store(f32x4_t{acc[sl][0], acc[sl][1], acc[sl][2], acc[sl][3]},
                                    reinterpret_cast<f32x4_t*>(drow + col[sl] * 4u));
    }
  }
}

static int ceil_log2(int64_t x) {   // smallest b with 2^b >= x (x >= 1)
  int b = 0;
  while ((int64_t{1} << b) < x) ++b;
  return b;
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
  ApiScope api_scope_("vocab_embed_fwd");
  tps_status s = embed_common_checks("vocab_embed_fwd", dt, T, H, v_start, v_rows);
  if (s != TPS_OK) return s;
  if (!ids || !E_r || !Y_r) return set_error(TPS_EINVAL, "vocab_embed_fwd: null pointer");
  if (!aligned16(E_r) || !aligned16(Y_r)) return set_error(TPS_EINVAL, "vocab_embed_fwd: pointers must be 16-byte aligned");
  if (T == 0) return TPS_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)ceil_div(T, 4));
  TraceScope trace_(st, "embed_fwd_kernel");
  if (dt == TPS_BF16)
    hipLaunchKernelGGL(embed_fwd_kernel<bf16_t>, grid, dim3(256), 0, st, ids, static_cast<const bf16_t*>(E_r),
                       static_cast<bf16_t*>(Y_r), T, H, v_start, v_rows);
  else
    hipLaunchKernelGGL(embed_fwd_kernel<float>, grid, dim3(256), 0, st, ids, static_cast<const float*>(E_r),
                       static_cast<float*>(Y_r), T, H, v_start, v_rows);
  return check_launch("embed_fwd_kernel");
}

// Row buckets of the sort: up to kRadixBuckets workgroups of at most 256 rows.
constexpr int kRadixBuckets = 256;

extern "C" size_t vocab_embed_bwd_workspace(int64_t T, int64_t v_rows) {
  (void)v_rows;
  if (T <= 0) return 0;
  return (size_t)next_pow2(T) * sizeof(uint64_t);   // the sort keys
}

// Checks shared by both backward entry points (everything but the workspace).
static tps_status embed_bwd_checks(const char* fn, tps_dtype dt, int64_t T, int64_t H, int64_t v_start,
                                   int64_t v_rows, const int32_t* ids, const void* dY, const float* dE_r) {
  tps_status s = embed_common_checks(fn, dt, T, H, v_start, v_rows);
  if (s != TPS_OK) return s;
  if (T >= 0x7fffffffLL) return set_error(TPS_EINVAL, std::string(fn) + ": T must be < 2^31");
  if (!ids || !dY || !dE_r) return set_error(TPS_EINVAL, std::string(fn) + ": null pointer");
  if (!aligned16(dY) || !aligned16(dE_r))
    return set_error(TPS_EINVAL, std::string(fn) + ": pointers must be 16-byte aligned");
  return TPS_OK;
}

// The sort into `keys` (next_pow2(T) entries, every one of them written
// before it is read) and the accumulation.  T > 0.
static tps_status embed_bwd_run(tps_dtype dt, int64_t T, int64_t H, int64_t v_start, int64_t v_rows,
                                const int32_t* ids, const void* dY, float* dE_r, uint64_t* keys, hipStream_t st) {
  tps_status s;
  const int tbits = ceil_log2(T), rbits = ceil_log2(v_rows + 1);
  if (T <= kRadixMax && tbits + 8 <= 32 && v_rows <= 256LL * kRadixBuckets) {
    // one workgroup per bucket of at most 256 rows: one 8-bit pass each
    const int brows = (int)ceil_div(v_rows, kRadixBuckets);
    const int nb = (int)ceil_div(v_rows, brows);
    TraceScope trace_(st, "embed_radix_sort_kernel");
    hipLaunchKernelGGL(embed_radix_sort_kernel, dim3((unsigned)nb), dim3(kRadixThreads), 0, st, ids, keys,
                       (int)T, v_start, (int)v_rows, tbits, ceil_log2(brows), brows);
    s = check_launch("embed_radix_sort_kernel");
  } else if (T <= kRadixMax && tbits + rbits <= 32) {
    hipLaunchKernelGGL(embed_radix_sort_kernel, dim3(1), dim3(kRadixThreads), 0, st, ids, keys,
                       (int)T, v_start, (int)v_rows, tbits, rbits, (int)v_rows);
    s = check_launch("embed_radix_sort_kernel");
  } else {
    const int64_t npad = next_pow2(T);
    hipLaunchKernelGGL(embed_keys_kernel, dim3((unsigned)ceil_div(npad, 256)), dim3(256), 0, st, ids, keys, T,
                       npad, v_start, v_rows);
    s = check_launch("embed_keys_kernel");
    if (s != TPS_OK) return s;
    s = sort_keys(keys, npad, st);
  }
  if (s != TPS_OK) return s;
  const dim3 grid((unsigned)ceil_div(T, 4));
  TraceScope trace_(st, "embed_bwd_accum_kernel");
  if (dt == TPS_BF16)
    hipLaunchKernelGGL(embed_bwd_accum_kernel<bf16_t>, grid, dim3(256), 0, st, keys,
                       static_cast<const bf16_t*>(dY), dE_r, T, H);
  else
    hipLaunchKernelGGL(embed_bwd_accum_kernel<float>, grid, dim3(256), 0, st, keys,
                       static_cast<const float*>(dY), dE_r, T, H);
  return check_launch("embed_bwd_accum_kernel");
}

extern "C" tps_status vocab_embed_bwd(tps_dtype dt, int64_t T, int64_t H, int64_t v_start, int64_t v_rows,
                                      const int32_t* ids, const void* dY, float* dE_r, void* ws,
                                      size_t ws_bytes, tps_stream_t stream) {
  ApiScope api_scope_("vocab_embed_bwd");
  tps_status s = embed_bwd_checks("vocab_embed_bwd", dt, T, H, v_start, v_rows, ids, dY, dE_r);
  if (s != TPS_OK) return s;
  if (T == 0) return TPS_OK;
  if (!ws) return set_error(TPS_EINVAL, "vocab_embed_bwd: null workspace");
  if (!aligned16(ws)) return set_error(TPS_EINVAL, "vocab_embed_bwd: workspace must be 16-byte aligned");
  if (ws_bytes < vocab_embed_bwd_workspace(T, v_rows))
    return set_error(TPS_EWORKSPACE, "vocab_embed_bwd: workspace too small");
  return embed_bwd_run(dt, T, H, v_start, v_rows, ids, dY, dE_r, static_cast<uint64_t*>(ws),
                       static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------- no-alloc variant
//
// The sort keys of vocab_embed_bwd_noalloc live in this file-scope device
// array instead of a caller workspace: one copy per GPU the library runs on,
// kept until the process ends.  Host code never passes the array's name to
// a kernel (in host code it is only a stand-in for the symbol): its device
// address is looked up once per device with hipGetSymbolAddress and cached.
constexpr int64_t kNoAllocMaxTokens = 65536;   // next_pow2(T) keys of 8 bytes: 512 KiB
static __device__ __align__(256) uint64_t scratch[kNoAllocMaxTokens];

static constexpr int kMaxDevices = 64;
static uint64_t* g_scratch_ptr[kMaxDevices] = {};
static std::mutex g_scratch_mu;

static tps_status noalloc_scratch(uint64_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return set_error(TPS_EHIP, "vocab_embed_bwd_noalloc: no current device");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(TPS_EHIP, std::string("vocab_embed_bwd_noalloc: hipGetSymbolAddress failed: ") +
                                     hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<uint64_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return TPS_OK;
}

extern "C" int64_t vocab_embed_bwd_noalloc_max_tokens(void) { return kNoAllocMaxTokens; }

extern "C" tps_status vocab_embed_bwd_noalloc(tps_dtype dt, int64_t T, int64_t H, int64_t v_start, int64_t v_rows,
                                              const int32_t* ids, const void* dY, float* dE_r,
                                              tps_stream_t stream) {
  ApiScope api_scope_("vocab_embed_bwd_noalloc");
  tps_status s = embed_bwd_checks("vocab_embed_bwd_noalloc", dt, T, H, v_start, v_rows, ids, dY, dE_r);
  if (s != TPS_OK) return s;
  if (T > kNoAllocMaxTokens)
    return set_error(TPS_EINVAL, "vocab_embed_bwd_noalloc: T = " + std::to_string(T) +
                                     " exceeds the static scratch's limit of " + std::to_string(kNoAllocMaxTokens) +
                                     " tokens (use vocab_embed_bwd with a workspace)");
  if (T == 0) return TPS_OK;
  uint64_t* keys = nullptr;
  s = noalloc_scratch(&keys);
  if (s != TPS_OK) return s;
  return embed_bwd_run(dt, T, H, v_start, v_rows, ids, dY, dE_r, keys, static_cast<hipStream_t>(stream));
}
