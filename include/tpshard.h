/*
 * tpshard.h -- C ABI of the tensor-parallel transformer-shard library for
 * AMD Instinct MI355X (gfx950).
 *
 * One call executes ONE tensor-parallel shard of one operation at that
 * shard's real per-shard shape; the shard-partial sum that a multi-GPU run
 * would obtain from an all-reduce is the separate call shard_reduce().
 * Sources for what each call computes (pages cited by title and section):
 *   "5-megatron"  formulaic.cloudchewie.com .../distributed-training/5-megatron
 *   "Megtron张量/模型并行"  amentiraz.github.io .../Megtron张量/模型并行/
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Matrices are dense and row-major in the mathematical layout (a linear
 *   layer is Y = X W with W of shape in x out), i.e. the layout of page
 *   "Megtron张量/模型并行", section 切分权重; the leading dimension of every
 *   matrix equals its column count unless an explicit ld argument exists.
 * - Element type: TPS_BF16 (bfloat16 storage, fp32 accumulation, every store
 *   rounded to nearest even) or TPS_F32 (fp32 throughout).  Accumulators that
 *   the caller keeps (dE_r, LayerNorm statistics and parameter gradients) are
 *   always fp32.
 * - Token rows are batch-major: row = batch * seq_len + position.
 * - Pointers are device pointers (caller-owned, e.g. from PyTorch), 16-byte
 *   aligned.  Column counts of matrices read with vector loads (h, f_i, H,
 *   hs*d, ldl) must be multiples of 8 elements (bf16) or 4 (fp32).  Row
 *   counts (M, T, v_rows, sq) are arbitrary.
 * - All calls are asynchronous on `stream` (a hipStream_t; 0 = the default
 *   stream).  Inputs must stay alive until the stream reaches the work.
 * - The library never allocates device memory.  Scratch memory is passed in
 *   as `ws` of at least the size returned by the matching *_workspace() query.
 * - Outputs must not alias inputs (exception: shard_reduce's out may equal
 *   parts[0]).
 * - Errors: arguments are validated on the host before anything is enqueued;
 *   on failure the call returns TPS_EINVAL (or TPS_EUNSUPPORTED /
 *   TPS_EWORKSPACE), enqueues nothing and leaves outputs untouched.  A failed
 *   launch returns TPS_EHIP.  tps_last_error() gives a thread-local message.
 * - Results are deterministic: no floating-point atomics are used, so two runs
 *   on the same inputs give identical bits.
 */
#ifndef TPSHARD_H
#define TPSHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* tps_stream_t;

typedef enum {
  TPS_OK = 0,
  TPS_EINVAL = 1,        /* bad argument (null pointer, size, alignment, ld) */
  TPS_EUNSUPPORTED = 2,  /* valid request this build does not implement      */
  TPS_EWORKSPACE = 3,    /* ws_bytes smaller than the workspace query        */
  TPS_EHIP = 4           /* a HIP launch or runtime call failed              */
} tps_status;

typedef enum { TPS_F32 = 0, TPS_BF16 = 1 } tps_dtype;

const char* tps_status_string(tps_status s);
/* Thread-local description of the last non-OK status returned on this thread. */
const char* tps_last_error(void);
/* Library version string. */
const char* tps_version(void);

/*
 * Split `total` rows into `n` contiguous shards; shard r starts at *start and
 * holds *count rows.  The first (total mod n) shards hold one extra row.
 * Page "5-megatron", section VocabParallelEmbedding (each rank keeps a
 * contiguous vocabulary range [start, end), example [0,5) and [5,10) for 10
 * words); page "Megtron张量/模型并行", section 输入层Embedding (300 words split
 * at 150).  Host-only.  EINVAL if n < 1, r outside [0, n), total < 0 or a
 * null output pointer.
 */
tps_status tps_partition(int64_t total, int n, int r, int64_t* start, int64_t* count);

/* ------------------------------------------------------------------------
 * (1) MLP shard: Z = GELU(X A) B with A column-parallel and B row-parallel.
 * Page "Megtron张量/模型并行", section MLP层 (A split by columns so GELU needs
 * no communication, B split by rows); page "5-megatron", sections
 * ColumnParallelLinear and RowParallelLinear (f = copy, g = all-reduce).
 *
 * tp_mlp_fwd:  P_i = X A_i,  H_i = gelu(P_i) (exact erf),  Z_i = H_i B_i.
 *   X   [M x h]     activations (replicated on every shard)
 *   A_i [h x f_i]   column shard of A
 *   B_i [f_i x h]   row shard of B
 *   P_i, H_i [M x f_i]  outputs, kept for the backward pass
 *   Z_i [M x h]     output: this shard's partial (sum over shards = Z)
 * ------------------------------------------------------------------------ */
tps_status tp_mlp_fwd(tps_dtype dt, int64_t M, int64_t h, int64_t f_i,
                      const void* X, const void* A_i, const void* B_i,
                      void* P_i, void* H_i, void* Z_i, tps_stream_t stream);

/* Bytes of scratch tp_mlp_bwd needs (holds dP_i, M x f_i elements). */
size_t tp_mlp_bwd_workspace(tps_dtype dt, int64_t M, int64_t h, int64_t f_i);

/*
 * tp_mlp_bwd: with dZ the full upstream gradient (g's backward is identity):
 *   dB_i = H_i^T dZ                      [f_i x h]
 *   dP_i = (dZ B_i^T) * gelu'(P_i)       (scratch)
 *   dA_i = X^T dP_i                      [h x f_i]
 *   dX_i = dP_i A_i^T                    [M x h]  partial; f's backward sums them
 */
tps_status tp_mlp_bwd(tps_dtype dt, int64_t M, int64_t h, int64_t f_i,
                      const void* X, const void* A_i, const void* B_i,
                      const void* P_i, const void* H_i, const void* dZ,
                      void* dX_i, void* dA_i, void* dB_i,
                      void* ws, size_t ws_bytes, tps_stream_t stream);

/* ------------------------------------------------------------------------
 * (2) Attention shard: Q/K/V column-parallel by heads, per-head softmax
 * attention, output projection row-parallel.  Page "Megtron张量/模型并行",
 * section Self-Attention层 (each head computed independently, several heads
 * may share a GPU, output linear split by rows); page "5-megatron", section
 * ParallelSelfAttention.  Per head: S = Q K^T / sqrt(d), keys after the query
 * masked when `causal` != 0, P = softmax(S), O = P V.
 *
 *   X      [b*sq x h]
 *   Wqkv_i [h x 3*hs*d]   = [W_Q | W_K | W_V] of this shard's hs heads; head j
 *                           occupies columns j*d..(j+1)*d inside each block
 *   Wo_i   [hs*d x h]     row shard of the output projection
 *   QKV_i  [b*sq x 3*hs*d] output (kept for backward)
 *   O_i    [b*sq x hs*d]  output (kept), head j at columns j*d..(j+1)*d
 *   lse_i  [b x hs x sq]  fp32 output (kept): log of each softmax row's sum
 *                           of exp(S), i.e. P = exp(S - lse) row by row
 *   Z_i    [b*sq x h]     output: this shard's partial
 *   ws     caller scratch of at least tp_attn_fwd_workspace(...) bytes
 *          (16-byte aligned), free again when the stream has passed the
 *          call.  Head dims 64, 128, 256 and 512 take the flash kernels:
 *          fp32 partial outputs of split query blocks, about one block of
 *          128 or 256 rows x d per compute unit (O(sq d), covering the
 *          causal and the non-causal plan).  Other head dims keep the scores
 *          and probabilities of every (batch, head), b*hs*sq*round_up(sq, 8)*6
 *          bytes.
 * Supported: dt = TPS_BF16, d a multiple of 8; TPS_EUNSUPPORTED for fp32.
 * TPS_EWORKSPACE if ws_bytes is too small (nothing is enqueued).
 * ------------------------------------------------------------------------ */
size_t tp_attn_fwd_workspace(tps_dtype dt, int64_t b, int64_t sq, int64_t h, int64_t hs, int64_t d);
tps_status tp_attn_fwd(tps_dtype dt, int64_t b, int64_t sq, int64_t h, int64_t hs, int64_t d,
                       int causal, const void* X, const void* Wqkv_i, const void* Wo_i,
                       void* QKV_i, void* O_i, float* lse_i, void* Z_i,
                       void* ws, size_t ws_bytes, tps_stream_t stream);

size_t tp_attn_bwd_workspace(tps_dtype dt, int64_t b, int64_t sq, int64_t h, int64_t hs, int64_t d);

/*
 * tp_attn_bwd: dWo_i = O_i^T dZ; dO = dZ Wo_i^T; per head dQ, dK, dV of the
 * softmax attention; dWqkv_i = X^T dQKV; dX_i = dQKV Wqkv_i^T (partial).
 * dZ [b*sq x h] is the full upstream gradient.  Outputs dX_i [b*sq x h],
 * dWqkv_i [h x 3*hs*d], dWo_i [hs*d x h].  The probabilities are recomputed
 * from QKV_i and lse_i; each row's softmax term sum_j P dP is taken from the
 * same P and dP that form dS (page "Megtron张量/模型并行", section
 * Self-Attention层, for the per-head computation).
 * ws: caller scratch of at least tp_attn_bwd_workspace(...) bytes (16-byte
 * aligned; the query covers both masks).  Head dims 64, 128, 256 take the
 * flash kernels: dO, dQKV (bf16), one fp32 row term per query and head and
 * fp32 partials of split blocks for about one work item per compute unit,
 * O(sq d).  Other head dims store P (bf16), dP (fp32) and dS (bf16) per
 * (query, key) and head, O(sq^2).
 * TPS_EWORKSPACE if ws_bytes is below this call's need (nothing is enqueued);
 * TPS_EINVAL for 3*hs*d > 2^25 on the flash path.
 */
tps_status tp_attn_bwd(tps_dtype dt, int64_t b, int64_t sq, int64_t h, int64_t hs, int64_t d,
                       int causal, const void* X, const void* Wqkv_i, const void* Wo_i,
                       const void* QKV_i, const void* O_i, const float* lse_i, const void* dZ,
                       void* dX_i, void* dWqkv_i, void* dWo_i,
                       void* ws, size_t ws_bytes, tps_stream_t stream);

/* ------------------------------------------------------------------------
 * (3) 'g' forward / 'f' backward: the shard-partial sum.
 * Page "5-megatron", sections ColumnParallelLinear (_CopyToModelParallelRegion
 * all-reduces the gradient) and RowParallelLinear
 * (_ReduceFromModelParallelRegion all-reduces the output).
 *   out[i] = round(sum_{r=0}^{n_parts-1} parts[r][i]) for i < n, summed in
 *   fp32 in shard order 0..n_parts-1 and rounded once to out_dt.
 *   parts: HOST array of n_parts device pointers (1 <= n_parts <= 8), each of
 *   in_dt.  out may equal parts[0].
 * ------------------------------------------------------------------------ */
tps_status shard_reduce(tps_dtype in_dt, tps_dtype out_dt, int n_parts,
                        const void* const* parts, void* out, int64_t n, tps_stream_t stream);

/*
 * shard_reduce_add: the shard-partial sum fused with a residual add, for a
 * residual stream kept in a wider type than the partials:
 *   s      = res[i] + sum_{r=0}^{n_parts-1} parts[r][i]   (fp32, in that order)
 *   out[i] = round_out_dt(s);  out_copy[i] = round_copy_dt(s) if out_copy != NULL
 * res of res_dt, parts of part_dt (1 <= n_parts <= 7), out of out_dt (may equal
 * res), optional out_copy of copy_dt (e.g. a bf16 copy that feeds the next
 * GEMM).  The pages' layer sums the 'g' all-reduce into the residual
 * (page "5-megatron", section RowParallelLinear: the reduce's result is the
 * layer output the residual connection adds).
 */
tps_status shard_reduce_add(tps_dtype res_dt, const void* res, tps_dtype part_dt, int n_parts,
                            const void* const* parts, tps_dtype out_dt, void* out,
                            tps_dtype copy_dt, void* out_copy, int64_t n, tps_stream_t stream);

/* ------------------------------------------------------------------------
 * (4) Vocab-parallel word embedding and the tied output projection.
 * Page "5-megatron", section VocabParallelEmbedding: ids outside this shard's
 * range [v_start, v_start + v_rows) are masked, the rest index row
 * id - v_start, and masked rows of the result are set to 0 before the sum.
 * Page "Megtron张量/模型并行", sections 输入层Embedding and 输出层Embedding:
 * the output layer reuses the same table, and the table's update must use the
 * sum of the output-side and input-side gradients.
 *
 * vocab_embed_fwd: Y_r[t] = E_r[ids[t] - v_start] if in range, else +0.
 *   ids [T] int32 (any value; out-of-vocabulary ids simply give zero rows),
 *   E_r [v_rows x H], Y_r [T x H] (every row written).  Bit-exact copy.
 * ------------------------------------------------------------------------ */
tps_status vocab_embed_fwd(tps_dtype dt, int64_t T, int64_t H, int64_t v_start, int64_t v_rows,
                           const int32_t* ids, const void* E_r, void* Y_r, tps_stream_t stream);

/* Workspace of vocab_embed_bwd: the sort keys (8 bytes per token, T rounded
 * up to a power of two). */
size_t vocab_embed_bwd_workspace(int64_t T, int64_t v_rows);

/*
 * vocab_embed_bwd (input side): dE_r[j] += sum over t with ids[t] = v_start + j
 * of dY[t], added in increasing t order in fp32 (deterministic, no atomics).
 *   dY [T x H] of dt; dE_r [v_rows x H] fp32, accumulated into (rows no
 *   token hits are not touched).  Requires T < 2^31.
 * Tied-gradient order: call tied_logits_bwd (which overwrites dE_r with the
 * output-side gradient) first, then vocab_embed_bwd.
 */
tps_status vocab_embed_bwd(tps_dtype dt, int64_t T, int64_t H, int64_t v_start, int64_t v_rows,
                           const int32_t* ids, const void* dY, float* dE_r,
                           void* ws, size_t ws_bytes, tps_stream_t stream);

/*
 * vocab_embed_bwd_noalloc: vocab_embed_bwd without a workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments (minus the
 * workspace), same kernels and the same result bit for bit.  The sort keys
 * live in a static device array inside the library (512 KiB on every GPU the
 * library runs on, held until the process ends), so the call allocates
 * nothing; the array's device address is looked up once per device on the
 * first call.  Limit: T <= vocab_embed_bwd_noalloc_max_tokens() (65536);
 * larger T returns TPS_EINVAL with nothing enqueued.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one device (different
 * streams, or host threads) race and must be serialised by the caller.
 * Errors as vocab_embed_bwd, plus TPS_EHIP when the array's address cannot be
 * obtained.
 */
int64_t vocab_embed_bwd_noalloc_max_tokens(void);
tps_status vocab_embed_bwd_noalloc(tps_dtype dt, int64_t T, int64_t H, int64_t v_start, int64_t v_rows,
                                   const int32_t* ids, const void* dY, float* dE_r, tps_stream_t stream);

/*
 * tied_logits: L_r = X E_r^T.
 *   X [T x H], E_r [v_rows x H], L_r [T x v_rows] with row stride ldl
 *   (ldl >= v_rows, multiple of 8 for bf16 / 4 for fp32; columns v_rows..ldl-1
 *   are not written).
 */
tps_status tied_logits(tps_dtype dt, int64_t T, int64_t H, int64_t v_rows, int64_t ldl,
                       const void* X, const void* E_r, void* L_r, tps_stream_t stream);

/*
 * tied_logits_bwd: dX_r = dL_r E_r (partial, [T x H]) and
 * dE_r = dL_r^T X ([v_rows x H] fp32, OVERWRITTEN with the output-side gradient).
 * dL_r [T x v_rows] with row stride ldl; padding columns are ignored.
 */
tps_status tied_logits_bwd(tps_dtype dt, int64_t T, int64_t H, int64_t v_rows, int64_t ldl,
                           const void* X, const void* E_r, const void* dL_r,
                           void* dX_r, float* dE_r, tps_stream_t stream);

/* ------------------------------------------------------------------------
 * The full input embedding (page "5-megatron", section Embedding) and
 * dropout.  Dropout uses the counter-based generator Philox4x32-10 (Salmon,
 * Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC
 * 2011): element e of a call (flat index) takes word e % 4 of Philox4x32-10
 * at counter (low and high words of e / 4, 0, 0) with key (low and high
 * words of seed), and is dropped when that word is below floor(p * 2^32);
 * kept elements are scaled by 1 / (1 - p) (fp32).  The same (seed, element)
 * always gives the same decision, so a backward regenerates the mask.  Per
 * the pages, callers use one seed for every shard after a shard sum (the
 * mask must agree) and a different seed per shard inside a tensor-parallel
 * region.
 *
 * embedding_fwd: out[t] = dropout(sum over shards of word_parts[r][t]
 *   + PE[pos[t]] + TE[tt[t]]), the sum in fp32 in shard order.
 *   word_parts: host array of n_parts (1..8) device pointers to the shards'
 *   vocab_embed_fwd outputs [T x H] of dt; PE [pos_rows x H] of dt; pos [T]
 *   int32; TE [tt_rows x H] of dt with tt [T] int32, or TE = NULL (no
 *   token types); an id outside its table adds a zero row.  out [T x H] of
 *   out_dt.  p in [0, 1) (0: no dropout, no generator).
 * dropout_apply: y[e] = keep(e) ? x[e] / (1 - p) : 0 over n elements of
 *   in_dt -> out_dt (y may be x when the dtypes match).  With the forward's
 *   p and seed applied to the output gradient it is the dropout backward;
 *   the result is then the gradient of the summed embedding, i.e. the dY of
 *   vocab_embed_bwd for every shard's word table, and, with pos (tt) as the
 *   ids, v_start 0 and pos_rows (tt_rows) rows, the position (token-type)
 *   table's gradient through vocab_embed_bwd.
 * Dimensions: T >= 0, H a positive multiple of 8; pointers 16-byte aligned.
 * Errors: TPS_EINVAL (bad dtype, p outside [0, 1), null or misaligned
 * pointers, bad sizes) before anything is enqueued.
 * ------------------------------------------------------------------------ */
tps_status embedding_fwd(tps_dtype dt, tps_dtype out_dt, int n_parts, const void* const* word_parts,
                         const void* PE, int64_t pos_rows, const int32_t* pos, const void* TE, int64_t tt_rows,
                         const int32_t* tt, float p, uint64_t seed, void* out, int64_t T, int64_t H,
                         tps_stream_t stream);
tps_status dropout_apply(tps_dtype in_dt, tps_dtype out_dt, int64_t n, const void* x, float p, uint64_t seed,
                         void* y, tps_stream_t stream);

/* ------------------------------------------------------------------------
 * Sequence parallelism on one device (page "5-megatron": in sequence
 * parallel regions the sequence component of an activation becomes s/N per
 * shard; page "zwxr 246059", section 4.3: those regions' LayerNorm
 * gradients are summed over the tensor-parallel group, which is
 * shard_reduce over the shards' [H] fp32 dgamma / dbeta).  The M rows of an
 * [M x H] activation are split as tps_partition(M, n_parts, r): shard r holds
 * rows [start_r, start_r + count_r) in its own [count_r x H] buffer.
 *
 * shard_reduce_scatter: the reduce-scatter replacing the g all-reduce after a
 *   row-parallel GEMM: outs[r] = res[r] + (sum over k of parts[k]) restricted
 *   to shard r's rows (fp32, the residual first, then the parts in shard
 *   order; one rounding to out_dt).  parts: n_parts full [M x H] partials of
 *   part_dt; res: NULL, or n_parts residual slices of out_dt (res[r] may be
 *   outs[r]); outs: n_parts slices of out_dt.
 * shard_all_gather: out [M x H] = the shards' slices parts[r] stacked in shard
 *   order (the all-gather before a column-parallel GEMM).
 * Both: host arrays of n_parts (1..8) device pointers, 16-byte aligned;
 * M > 0, H a positive multiple of 8; a shard with no rows (M < n_parts) is
 * never touched and may pass NULL for its slice (and residual).
 * Errors: TPS_EINVAL before anything is enqueued.
 * ------------------------------------------------------------------------ */
tps_status shard_reduce_scatter(tps_dtype part_dt, tps_dtype out_dt, int n_parts, const void* const* parts,
                                const void* const* res, void* const* outs, int64_t M, int64_t H,
                                tps_stream_t stream);
tps_status shard_all_gather(tps_dtype dt, int n_parts, const void* const* parts, void* out, int64_t M, int64_t H,
                            tps_stream_t stream);

/* ------------------------------------------------------------------------
 * The two linear layers on their own (page "5-megatron", sections
 * ColumnParallelLinear and RowParallelLinear), math layout Y = X A + b, one
 * shard per call; dt is TPS_BF16 or TPS_F32 for every matrix and bias.
 *
 * column_linear_fwd: Y_r = X A_r (+ b_r).  X [M x h_in] (the f operator's
 *   copy: the same X on every shard), A_r [h_in x n_r] (columns of A), b_r
 *   [n_r] (its slice of the bias; NULL for no bias, also for skip_bias_add,
 *   where the caller keeps the bias).  Y_r [M x n_r] with row stride ldy
 *   (>= n_r, multiple of 8): with gather_output, Y_r is the shard's column
 *   slice of the gathered [M x sum n_r] output (the all-gather is the
 *   layout).
 * column_linear_bwd: for dY_r [M x n_r] with row stride lddy (the split of a
 *   gathered gradient is a column slice): dX_r = dY_r A_r^T [M x h_in], a
 *   partial that the f backward sums over shards (shard_reduce);
 *   dA_r = X^T dY_r [h_in x n_r]; db_r [n_r] fp32 = column sums of dY_r
 *   (NULL: not computed).
 * row_linear_fwd: Y_r = X_r B_r [M x h_out], a partial.  X_r [M x k_r] with
 *   row stride ldx: the shard's column slice of the full input X when the
 *   input is not parallel (the scatter is the layout), or its own [M x k_r]
 *   input; B_r [k_r x h_out] (rows of B).  The sum over shards, plus the
 *   bias once, is shard_reduce_bias (or shard_reduce without bias).
 * row_linear_bwd: for the full dY [M x h_out] (the all-reduce's backward is
 *   the identity): dX_r = dY B_r^T written with row stride lddx (a column
 *   slice of the gathered dX when the input was scattered); dB_r = X_r^T dY
 *   [k_r x h_out]; db [h_out] fp32 = column sums of dY (the replicated
 *   bias's gradient; NULL: not computed).
 * shard_reduce_bias: out[m,n] = sum over parts (shard order, fp32) + bias[n],
 *   one rounding; parts: host array of n_parts (1..8) device pointers to
 *   [M x N] of dt; bias [N] of dt; N a multiple of 8.  out may be parts[0].
 * Dimensions: all > 0 and < 2^31; h_in, n_r, k_r, h_out multiples of 8; every
 * pointer 16-byte aligned.  Outputs must not alias inputs (except as noted).
 * Errors: TPS_EINVAL before anything is enqueued.  db_r/db are written by a
 * fixed-order reduction (reproducible).
 * ------------------------------------------------------------------------ */
tps_status column_linear_fwd(tps_dtype dt, int64_t M, int64_t h_in, int64_t n_r, const void* X,
                             const void* A_r, const void* b_r, void* Y, int64_t ldy, tps_stream_t stream);
tps_status column_linear_bwd(tps_dtype dt, int64_t M, int64_t h_in, int64_t n_r, const void* X,
                             const void* A_r, const void* dY, int64_t lddy, void* dX_r, void* dA_r,
                             float* db_r, tps_stream_t stream);
tps_status row_linear_fwd(tps_dtype dt, int64_t M, int64_t k_r, int64_t h_out, const void* X_r, int64_t ldx,
                          const void* B_r, void* Y_r, tps_stream_t stream);
tps_status row_linear_bwd(tps_dtype dt, int64_t M, int64_t k_r, int64_t h_out, const void* X_r, int64_t ldx,
                          const void* B_r, const void* dY, void* dX_r, int64_t lddx, void* dB_r, float* db,
                          tps_stream_t stream);
tps_status shard_reduce_bias(tps_dtype dt, int n_parts, const void* const* parts, const void* bias, void* out,
                             int64_t M, int64_t N, tps_stream_t stream);

/* ------------------------------------------------------------------------
 * Vocab-parallel cross entropy on the tied logits (page "5-megatron",
 * section _VocabParallelCrossEntropy; page "notion 310f8c09", section
 * 交叉熵张量并行).  Per token t with target id y_t and logits split by vocab
 * rows over the shards: loss_t = log(sum_j exp(x_tj - m_t)) - (x_{t,y_t} - m_t)
 * with m_t the maximum over every shard, i.e. logsumexp - target logit; a
 * target that no shard owns contributes 0 as its shifted logit (the pages'
 * mask), so its loss is logsumexp - m_t.  The shards exchange per-token
 * statistics only (the pages' MAX and SUM all-reduces of b*s values); on one
 * device vocab_ce_combine takes every shard's statistics at once.
 *
 * vocab_ce_stats: one shard's statistics, one pass over its logits.
 *   L_r [T x v_rows] of dt with row stride ldl (ldl >= v_rows, multiple of 8
 *   for bf16 / 4 for fp32; padding columns are not read for use); targets [T]
 *   int32 (any value); stats_r [T x 4] fp32 OUTPUT, 16-byte aligned:
 *   {m_r = max_j L_r[t,j], s_r = sum_j exp(L_r[t,j] - m_r),
 *    x_r = L_r[t, y_t - v_start] if v_start <= y_t < v_start + v_rows else 0,
 *    own_r = 1 if so else 0}.  Logits must be finite.
 * vocab_ce_combine: stats is a host array of n_parts (1..8) device pointers
 *   to the shards' statistics (every shard of the vocabulary, any order of
 *   shards); loss [T] and lse [T] fp32 OUTPUTS:
 *   m = max_r m_r, den = sum_r s_r exp(m_r - m) (shard order),
 *   pick = sum_r own_r (x_r - m), loss = log(den) - pick, lse = m + log(den).
 * vocab_ce_bwd: dL_r[t,j] = dloss[t] * (exp(L_r[t,j] - lse[t]) - [j = y_t - v_start])
 *   for j < v_rows, as dt with row stride ldl (padding columns not written);
 *   dloss [T] fp32 is the upstream gradient of each token's loss.  dL_r may
 *   be L_r itself (in place, as the pages' code does); otherwise the two must
 *   not overlap.  The result is what tied_logits_bwd takes as dL_r.
 * Errors: TPS_EINVAL for a bad dtype, T < 0, v_rows <= 0, v_start < 0, a bad
 * ldl, null or misaligned pointers, n_parts outside 1..8; nothing is
 * enqueued then.  T = 0 is a no-op.
 * ------------------------------------------------------------------------ */
tps_status vocab_ce_stats(tps_dtype dt, int64_t T, int64_t v_rows, int64_t ldl, int64_t v_start,
                          const void* L_r, const int32_t* targets, float* stats_r, tps_stream_t stream);
tps_status vocab_ce_combine(int n_parts, const float* const* stats, int64_t T, float* loss, float* lse,
                            tps_stream_t stream);
tps_status vocab_ce_bwd(tps_dtype dt, int64_t T, int64_t v_rows, int64_t ldl, int64_t v_start,
                        const void* L_r, const int32_t* targets, const float* lse, const float* dloss,
                        void* dL_r, tps_stream_t stream);

/* ------------------------------------------------------------------------
 * LayerNorm (replicated on every shard), for stacking layers.  Page
 * "5-megatron", section 训练一般流程 counts two LayerNorms of 2H parameters
 * per layer; the formula is the standard one with biased variance:
 *   y = (x - mean) / sqrt(var + eps) * gamma + beta   (per row of H, fp32 math)
 * layernorm_fwd: x [M x H] of x_dt, y [M x H] of y_dt (e.g. an fp32 residual
 * stream in, bf16 GEMM input out); gamma, beta [H] fp32; mean, rstd [M] fp32
 * outputs kept for the backward pass.  H <= 8192 (TPS_EUNSUPPORTED above).
 * layernorm_bwd: dy of dy_dt, dx of dx_dt; dgamma, dbeta [H] fp32 OVERWRITTEN
 * (reduced over rows in a fixed order through the workspace).
 * ------------------------------------------------------------------------ */
tps_status layernorm_fwd(tps_dtype x_dt, tps_dtype y_dt, int64_t M, int64_t H, float eps, const void* x,
                         const float* gamma, const float* beta, void* y, float* mean,
                         float* rstd, tps_stream_t stream);

size_t layernorm_bwd_workspace(int64_t M, int64_t H);

tps_status layernorm_bwd(tps_dtype x_dt, tps_dtype dy_dt, tps_dtype dx_dt, int64_t M, int64_t H,
                         const void* x, const float* gamma, const float* mean, const float* rstd,
                         const void* dy, void* dx, float* dgamma, float* dbeta, void* ws,
                         size_t ws_bytes, tps_stream_t stream);

/*
 * layernorm_bwd_residual: the same backward pass for a pre-LN sublayer whose
 * residual connection also carries gradient: out = res + dL/dx, res and out
 * fp32 [M x H] (out must not alias res); out_copy (bf16 [M x H], may be
 * null) receives out rounded once, for the next GEMMs.  dgamma, dbeta and
 * the workspace as for layernorm_bwd.  Equivalent to layernorm_bwd into a
 * temporary followed by the elementwise add, without the temporary.
 */
tps_status layernorm_bwd_residual(tps_dtype x_dt, tps_dtype dy_dt, int64_t M, int64_t H,
                                  const void* x, const float* gamma, const float* mean,
                                  const float* rstd, const void* dy, const float* res, float* out,
                                  void* out_copy, float* dgamma, float* dbeta, void* ws,
                                  size_t ws_bytes, tps_stream_t stream);

/* ------------------------------------------------------------------------
 * Launch tracing (measurement support, not part of the method).
 * While tracing is on, every kernel launch the library makes whose name
 * contains `filter` (an empty string or NULL: every launch) is bracketed by
 * a pair of timing events recorded on the launch's own stream, for at most
 * `max_records` launches.  A launch's name is "<entry point>:<kernel>" plus,
 * for the GEMM kernel, its template arguments and "MxNxK z<problems>".
 * tps_trace_start creates the events (host-side objects, no device memory)
 * and discards earlier records; tps_trace_stop stops recording and keeps the
 * records; tps_trace_get(i) returns record i's name (truncated to name_cap
 * bytes including the terminating 0) and its duration in milliseconds,
 * waiting for the launch to finish; tps_trace_clear releases the events.
 * Tracing is process-wide and not meant for concurrent use from several
 * threads.  Errors: TPS_EINVAL for max_records outside [1, 2^20] or a bad
 * record index, TPS_EHIP when an event call fails.
 * ------------------------------------------------------------------------ */
tps_status tps_trace_start(const char* filter, int max_records);
tps_status tps_trace_stop(void);
int tps_trace_count(void);
tps_status tps_trace_get(int i, char* name, int name_cap, float* ms);
tps_status tps_trace_clear(void);

#ifdef __cplusplus
}
#endif

#endif /* TPSHARD_H */
