/*
 * tpshard -- one rank of a Megatron-style tensor-parallel transformer block,
 * as HIP kernels for MI355X (gfx950) behind a plain C ABI.
 *
 * The operations follow the "Tensor parallelism" page of itwiki (텐서 병렬화):
 *
 *   section "Matmul split"  a column-parallel linear holds a block of columns
 *                           A_i of A and computes Y_i = X A_i from the full X;
 *                           a row-parallel linear holds a block of rows B_i and
 *                           yields a partial sum; the sum over ranks is the
 *                           layer output.  A column split feeds a row split
 *                           with no exchange in between.
 *   section "MLP"           Z = GeLU(X A) B with A by columns and B by rows:
 *                           GeLU is applied per rank and Z = sum_i GeLU(X A_i) B_i.
 *                           The SwiGLU form W2 (SiLU(X W1) * X W3) splits the
 *                           same way (W1, W3 by columns, W2 by rows).
 *   section "Self-attention" heads are split across ranks: the Q/K/V
 *                           projections by columns (a/t heads per rank, a
 *                           divisible by t), attention per head with no
 *                           exchange, o_proj by rows.  With grouped-query
 *                           attention a KV head is replicated on several ranks
 *                           when there are fewer KV heads than ranks.
 *   section "f and g"       the forward exchange is one all-reduce after each
 *                           sublayer; norms and residuals are replicated.
 *
 * On one GPU the all-reduce is stood in for by tp_shard_sum, which adds the
 * ranks' partials inside one device (no collective).
 *
 * Conventions for every call
 * --------------------------
 *  - Device pointers, row-major, contiguous, 16-byte aligned.  The caller owns
 *    every buffer; the library never allocates, frees or synchronises.  Work is
 *    enqueued on `stream` (a hipStream_t; NULL is the null stream) and the
 *    call returns at once; buffers must stay valid until the stream passes.
 *  - Weights are in nn.Linear layout [out_features, in_features], so both
 *    operands of every product are contiguous along the reduction dimension.
 *    (The pages write A as [in, out]; a rank's weight here is A_i transposed.)
 *  - bf16 tensors hold bfloat16 values; arithmetic accumulates in float32.
 *    Every float32 -> bf16 conversion rounds to nearest-even.
 *  - Reduction and feature dimensions (k, n, h, f_shard) must be multiples of
 *    8; m (tokens) may be any value >= 0 (m == 0 enqueues nothing).
 *  - Errors are returned before anything is enqueued, never replaced by a
 *    fallback: TP_ERR_INVALID_ARG (null/misaligned pointer, unknown enum),
 *    TP_ERR_SHAPE (a size or divisibility rule), TP_ERR_WORKSPACE (too small),
 *    TP_ERR_UNSUPPORTED (dtype/option not built, or the device is not gfx950),
 *    TP_ERR_HIP (a HIP launch error).  tp_last_error() gives a message for the
 *    calling thread's last failure.
 *  - Results are deterministic: no atomics, fixed summation order.
 */
#ifndef TPSHARD_H
#define TPSHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tp_status {
  TP_OK = 0,
  TP_ERR_INVALID_ARG = 1,
  TP_ERR_SHAPE = 2,
  TP_ERR_WORKSPACE = 3,
  TP_ERR_UNSUPPORTED = 4,
  TP_ERR_HIP = 5
} tp_status;

typedef enum tp_dtype { TP_F32 = 0, TP_BF16 = 1 } tp_dtype;

/* Nonlinearity applied by the column-parallel GEMM, per rank ("MLP" section). */
typedef enum tp_act {
  TP_ACT_NONE = 0,   /* plain colwise projection, Y_i = X A_i                    */
  TP_ACT_GELU = 1,   /* Y_i = GeLU(X A_i), exact erf form x/2 (1 + erf(x/sqrt2))  */
  TP_ACT_SWIGLU = 2  /* Y_i = SiLU(X W1_i) * (X W3_i), SiLU(x) = x / (1 + e^-x)  */
} tp_act;

/* Maximum number of partials one tp_shard_sum call adds. */
#define TP_MAX_SHARDS 16

/* --------------------------------------------------------------------------
 * Column-parallel linear with a fused nonlinearity ("Matmul split", "MLP").
 *
 *   x  [m, k]      the replicated input (dt)
 *   w  [n, k]      rank i's weight A_i^T                     (act NONE, GELU)
 *      [2n, k]     [W1_i^T ; W3_i^T]: the rank's gate rows then its up rows,
 *                  each block sliced from its own tensor   (act SWIGLU)
 *   bias [n] float32, or [2n] (the gate biases then the up biases, SWIGLU),
 *                  or NULL: rank i's slice of the layer's bias, added before
 *                  the nonlinearity (a column-parallel layer shards its bias
 *                  with its output features: transformers "Tensor
 *                  parallelism" page, partitioning table and DTensor example)
 *   y  [m, n]      rank i's output slice Y_i = act(x A_i + b_i) (dt)
 *
 * dt is TP_BF16 (bf16 in and out, float32 accumulate) or TP_F32 (float32 in,
 * out and arithmetic; meant for small checks).
 * ------------------------------------------------------------------------ */
tp_status tp_colwise(tp_act act, tp_dtype dt, int64_t m, int64_t k, int64_t n,
                     const void* x, const void* w, const float* bias, void* y, void* stream);

/* --------------------------------------------------------------------------
 * Row-parallel linear to a float32 partial sum ("Matmul split").
 *
 *   y        [m, k]  the rank's column slice of the activations (dt)
 *   w        [n, k]  the rank's weight rows B_i, transposed
 *   partial  [m, n]  float32, overwritten with Y_i B_i (the rank's share of
 *                    the sum; no reduction across ranks here)
 * ------------------------------------------------------------------------ */
tp_status tp_rowwise(tp_dtype dt, int64_t m, int64_t k, int64_t n,
                     const void* y, const void* w, float* partial, void* stream);

/* --------------------------------------------------------------------------
 * Row-parallel linear over a replicated input ("rowwise_split_input" of the
 * diffusers tensor-parallel guide, style table: the weight is split along
 * its input features and each rank computes its partial sum from its own
 * slice of the replicated input; the sum over ranks is the layer output).
 *
 *   x        [m, k]      the replicated input (dt); rank r reads its columns
 *                        [r k/t, (r+1) k/t) in place (no copy)
 *   w        [n, k/t]    the rank's weight columns (nn.Linear dim 1 sliced)
 *   partial  [m, n]      float32, overwritten with the rank's share
 * k / t must be a multiple of 8.
 * ------------------------------------------------------------------------ */
tp_status tp_rowwise_split_input(tp_dtype dt, int64_t m, int64_t k, int64_t n, int32_t t, int32_t rank,
                                 const void* x, const void* w, float* partial, void* stream);

/* --------------------------------------------------------------------------
 * One rank's MLP: tp_colwise(act) then tp_rowwise ("MLP" section).
 *
 *   x        [m, h]                      replicated input
 *   w_in     [f_shard, h] or [2 f_shard, h]   as tp_colwise's w
 *   w_out    [h, f_shard]                B_i^T (or W2_i^T)
 *   act_ws   [m, f_shard]  dt            workspace receiving Y_i
 *   partial  [m, h]  float32             overwritten with the rank's partial
 * act must be GELU or SWIGLU.
 * ------------------------------------------------------------------------ */
tp_status tp_shard_mlp(tp_act act, tp_dtype dt, int64_t m, int64_t h, int64_t f_shard,
                       const void* x, const void* w_in, const void* w_out,
                       void* act_ws, float* partial, void* stream);

/* --------------------------------------------------------------------------
 * All t ranks' MLP shards of one layer in one pair of launches (the rank is
 * the second grid dimension), for shapes whose per-rank GEMMs are too small
 * to fill the device.  A one-device helper: on a real tensor-parallel group
 * every rank calls tp_shard_mlp on its own GPU.  Results are bitwise equal
 * to t calls of tp_shard_mlp with the same operands.
 *
 *   t                  1 .. 16
 *   x                  [m, h], shared by every rank
 *   w_in, w_out,       HOST arrays of t device pointers, each as in
 *   act_ws, partial    tp_shard_mlp for rank i
 * ------------------------------------------------------------------------ */
tp_status tp_shard_mlp_group(tp_act act, tp_dtype dt, int32_t t, int64_t m, int64_t h,
                             int64_t f_shard, const void* x, const void* const* w_in,
                             const void* const* w_out, void* const* act_ws,
                             float* const* partial, void* stream);

/* --------------------------------------------------------------------------
 * Column-parallel Q/K/V projection of one rank with rotary embedding
 * ("Self-attention" section), bf16 only.
 *
 *   x      [batch*seq, h]   replicated input; token row r is position r % seq
 *                           of sequence r / seq
 *   w_qkv  [(hq + 2 hkv) * d, h]  the rank's rows: its hq query heads, then
 *                           its hkv key heads, then its hkv value heads, each
 *                           head d consecutive rows
 *   q      [batch*seq, hq*d]    RoPE(x Wq_i), head j in columns [j d, (j+1) d)
 *   k      [batch*seq, hkv*d]   RoPE(x Wk_i)
 *   vt     [batch, hkv, d, seq_pad]  (x Wv_i) transposed per sequence and
 *                           head, seq_pad = seq rounded up to 64; columns
 *                           >= seq are written as zero
 *   bias   [(hq + 2 hkv) * d] float32 or NULL: the rank's q, k, v biases in
 *                           the order of w_qkv's rows, added before RoPE
 * RoPE rotates the pair (c, c + d/2) of every head by the angle
 * pos * rope_base^(-2c/d) (rotate-half form).  d must be 128.
 * ------------------------------------------------------------------------ */
tp_status tp_qkv_rope(int64_t batch, int64_t seq, int64_t h, int32_t hq, int32_t hkv,
                      int32_t head_dim, float rope_base, const void* x, const void* w_qkv,
                      const float* bias, void* q, void* k, void* vt, void* stream);

/* --------------------------------------------------------------------------
 * Attention of one rank's heads ("Self-attention" section), bf16 only.
 *
 *   q, k, vt  as written by tp_qkv_rope
 *   o         [batch*seq, hq*d]  softmax(q k^T / sqrt(d)) v per query head,
 *             query head j of the rank reading KV head j / (hq / hkv);
 *             causal != 0 lets position p see positions <= p of its own
 *             sequence, causal == 0 all positions of its sequence.
 * hq must be a multiple of hkv; d must be 128.  When the launch cuts query
 * blocks over workgroups (tp_flash_attn_plan), their float32 partials pass
 * through a workspace of the library, one per (device, stream), allocated
 * (about 34 MB) at the first such launch on a stream and kept until the
 * process ends; if that allocation fails the launch runs uncut.  This also
 * holds for tp_flash_attn_lse and tp_shard_attn.
 * ------------------------------------------------------------------------ */
tp_status tp_flash_attn(int64_t batch, int64_t seq, int32_t hq, int32_t hkv, int32_t head_dim,
                        int32_t causal, const void* q, const void* k, const void* vt, void* o,
                        void* stream);

/* Bytes of workspace tp_shard_attn needs (q, k, vt and o, each 256-byte aligned). */
size_t tp_shard_attn_workspace_bytes(int64_t batch, int64_t seq, int32_t hq, int32_t hkv,
                                     int32_t head_dim);

/* --------------------------------------------------------------------------
 * One rank's attention sublayer: tp_qkv_rope, tp_flash_attn, then the
 * row-parallel o_proj to a float32 partial ("Self-attention" section).
 *
 *   dt       TP_BF16 (the only attention built; TP_F32 returns
 *            TP_ERR_UNSUPPORTED before anything is enqueued)
 *   w_o      [h, hq*d]   rows of Wo for this rank's heads, transposed
 *   ws       workspace of at least tp_shard_attn_workspace_bytes(...) bytes
 *   partial  [batch*seq, h] float32, overwritten
 * ------------------------------------------------------------------------ */
tp_status tp_shard_attn(tp_dtype dt, int64_t batch, int64_t seq, int64_t h, int32_t hq, int32_t hkv,
                        int32_t head_dim, float rope_base, int32_t causal, const void* x,
                        const void* w_qkv, const void* w_o, void* ws, size_t ws_bytes,
                        float* partial, void* stream);

/* --------------------------------------------------------------------------
 * tp_shard_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, kernels and results as
 * tp_shard_attn; the q, k, vt and o workspace, and the attention's cut-block
 * partials and their flags, are instead a static device array of the
 * library holding 64 MiB (TP_STATIC_SCRATCH_BYTES) on every device it runs
 * on, from the first call on that device until the process ends.  Nothing
 * is allocated or freed by the call.
 *
 *   - A shape whose tp_shard_attn_workspace_bytes(...), plus its cut-block
 *     partials ((pieces - 1) x ceil(ceil(seq/128)/2) x batch x hq slots of
 *     66560 bytes, pieces from tp_flash_attn_plan) and 2 KiB of flags,
 *     exceeds 64 MiB returns TP_ERR_WORKSPACE before anything is enqueued
 *     (every configuration of this library's workloads fits: 36 + 16.3 MiB
 *     at batch 4 x seq 2048 with 8 query heads and 1 KV head).
 *   - Every call on one device shares that device's array, which keeps the
 *     last call's contents; each call writes every byte it later reads (the
 *     transposed-V padding is zeroed by a kernel of the call), except the
 *     flags, which only ever hold the epoch of the call that raised them
 *     (a per-device count, so a flag left by an earlier call never matches
 *     a later one).  Calls that overlap on one device (e.g. on two streams,
 *     or from two threads before the first has drained) race on the array:
 *     the caller must order them.
 *   - The first call on a device looks up the array's device address
 *     (TP_ERR_HIP if that fails).
 * ------------------------------------------------------------------------ */
#define TP_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
tp_status tp_shard_attn_noalloc(tp_dtype dt, int64_t batch, int64_t seq, int64_t h, int32_t hq, int32_t hkv,
                                int32_t head_dim, float rope_base, int32_t causal, const void* x,
                                const void* w_qkv, const void* w_o, float* partial, void* stream);

/* --------------------------------------------------------------------------
 * Sum of the ranks' partials -- the forward all-reduce ("f and g" section),
 * computed inside one device:
 *
 *   out[e] = (((partials[0][e] + partials[1][e]) + ...) + partials[t-1][e])
 *            + residual[e]
 *
 * in float32, ascending rank order, residual (optional, NULL for none) added
 * last.  partials is a HOST array of t device pointers (1 <= t <= 16), each
 * [n] float32; residual is [n] of residual_dt; out [n] float32 may alias
 * residual when residual_dt is TP_F32, but no partial.
 * ------------------------------------------------------------------------ */
tp_status tp_shard_sum(int32_t t, int64_t n, const float* const* partials, const void* residual,
                       tp_dtype residual_dt, float* out, void* stream);

/* --------------------------------------------------------------------------
 * Replicated RMSNorm ("f and g" section: norms run on every rank):
 *   y[r, c] = bf16( x[r, c] / sqrt(mean_c x[r, c]^2 + eps) * gain[c] )
 *   x [m, h] of in_dt, gain [h] float32 or NULL (all ones), y [m, h] bf16.
 * ------------------------------------------------------------------------ */
tp_status tp_rmsnorm(tp_dtype in_dt, int64_t m, int64_t h, const void* x, const float* gain,
                     float eps, void* y, void* stream);

/* --------------------------------------------------------------------------
 * The sum that ends a sublayer and the norm that opens the next one, in one
 * pass over rows of h:
 *   x   = (((partials[0] + partials[1]) + ... + partials[t-1]) + bias) + residual
 *         (t = 0: the residual alone; bias, when given, is the row-parallel
 *         layer's bias, added once after the sum: transformers "Tensor
 *         parallelism" page, RowwiseParallel replicates the bias and adds it
 *         after the reduction)
 *   out = x                                                 (float32, if out)
 *   y   = bf16( x / sqrt(mean_c x^2 + eps) * gain )  per row   (if y)
 * with tp_shard_sum's and tp_rmsnorm's arithmetic exactly (with no bias the
 * results are bitwise those of those calls), and without reading out back.
 *
 * The rows are nrun runs of run_rows consecutive rows, the first rows of
 * consecutive runs run_stride rows apart (run_stride is ignored for one
 * run); every pointer addresses the first row of the first run.  This is
 * the sequence-parallel form ("Tensor parallelism" page, section "Sequence
 * parallelism": a norm acts on every token alone, so each rank normalises
 * only its slice of the sequence, and the sum after a row-parallel layer is
 * a reduce-scatter that leaves each rank the sum over its slice; section
 * "Writing it in PyTorch": the slice is Shard(1), the sequence dimension of
 * (batch, sequence, hidden)).  Rank r of t, with batch sequences of S tokens
 * stored token-major, passes its positions [r S/t, (r+1) S/t) of every
 * sequence as nrun = batch runs of run_rows = S/t, run_stride = S, pointers
 * offset by r S/t rows:
 *   its norm of X:                  t = 0, residual = X, out = NULL, y
 *   reduce-scatter + X, then norm:  t partials, residual = X, out = h1, y
 *   reduce-scatter + h1:            t partials, residual = h1, out = Z, y = NULL
 * (on one device, or over peer pointers).  One run of all rows gives the
 * replicated form.
 *
 *   t          0 .. 16
 *   partials   HOST array of t device pointers, float32 rows
 *   bias       [h] float32 or NULL (t >= 1)
 *   residual   rows of residual_dt (TP_F32 or TP_BF16), or NULL (t >= 1)
 *   out        float32 rows or NULL; may alias a float32 residual, not a partial
 *   gain       [h] float32 or NULL (all ones); y bf16 rows or NULL
 *   out and y may not both be NULL.
 * ------------------------------------------------------------------------ */
tp_status tp_shard_sum_rmsnorm(int32_t t, int64_t nrun, int64_t run_rows, int64_t run_stride, int64_t h,
                               const float* const* partials, const float* bias, const void* residual,
                               tp_dtype residual_dt, float* out, const float* gain, float eps, void* y,
                               void* stream);

/* --------------------------------------------------------------------------
 * Vocabulary-parallel embedding and cross-entropy ("Tensor parallelism"
 * page, section "Embedding and output layer": the embedding matrix is split
 * along the vocabulary; rather than gathering the b x s x v output logits,
 * each rank computes from its own slice the maximum and the sum the
 * cross-entropy needs, and only b x s values cross between ranks;
 * transformers "Tensor parallelism" page, EmbeddingParallel).
 *
 * tp_embedding: out[i, 0:w] = table[ids[i] - v_start, 0:w] for ids in
 * [v_start, v_start + v_rows), zeros otherwise (float32 out, rows ld apart).
 *   vocabulary-sharded lookup (embedding_rowwise): rank r passes its rows
 *     [r v/t, (r+1) v/t) of the [v, h] table, w = ld = h, and out is its
 *     partial: the sum over ranks (tp_shard_sum) is the lookup, exactly;
 *   hidden-sharded lookup (embedding_colwise): rank r passes its columns
 *     [v, h/t] of the table, v_start = 0, v_rows = v, w = h/t, ld = h, out at
 *     column r h/t of the gathered [m, h] buffer.
 *   ids      [m] int32; table [v_rows, w] bf16; out float32
 *
 * tp_vocab_logits: logits[m, v_shard] = x [m, h] . w[v_shard, h]^T, float32
 * (bf16 operands): the rank's slice of the output layer (its vocabulary rows).
 *
 * tp_ce_stats: for each token i, stats[i] = { max_j x_j, sum_j exp(x_j - max),
 * x at the label if the label is in [v_start, v_start + v_shard) else 0,
 * 1 if it is else 0 } over the rank's logits x = logits[i, 0:v_shard).
 *   labels [m] int32 (a label outside [0, v) marks an ignored token);
 *   stats [m, 4] float32.
 *
 * tp_ce_combine: the exchange's result: for each token, with M = max_r max_r
 * and S = sum_r sum_r exp(max_r - M) (ranks in ascending order),
 *   loss[i] = log S + M - x_label    (0 for an ignored token)
 * and, if mean is not NULL, mean[0] = the average over non-ignored tokens.
 *   stats  HOST array of t device pointers [m, 4] (rank r's statistics; on
 *          one device, rows of one [t, m, 4] buffer)
 * ------------------------------------------------------------------------ */
tp_status tp_embedding(int64_t m, int64_t w, int64_t v_start, int64_t v_rows, const int32_t* ids,
                       const void* table, float* out, int64_t ld, void* stream);
tp_status tp_vocab_logits(int64_t m, int64_t h, int64_t v_shard, const void* x, const void* w, float* logits,
                          void* stream);
tp_status tp_ce_stats(int64_t m, int64_t v_shard, int64_t v_start, const float* logits, const int32_t* labels,
                      float* stats, void* stream);
tp_status tp_ce_combine(int32_t t, int64_t m, int64_t v, const float* const* stats, const int32_t* labels,
                        float* loss, float* mean, void* stream);

/* --------------------------------------------------------------------------
 * tp_colwise (bf16, GELU or SWIGLU) that also stores the pre-activation the
 * backward pass needs ("f and g": the rank's backward differentiates its own
 * nonlinearity), so it need not be recomputed:
 *   pre  [m, n] bf16 (GELU: x w^T + bias) or [m, 2n] bf16 (SWIGLU: the n gate
 *        columns x W1_i + b1, then the n up columns x W3_i + b3)
 * ------------------------------------------------------------------------ */
tp_status tp_colwise_save(tp_act act, int64_t m, int64_t k, int64_t n, const void* x, const void* w,
                          const float* bias, void* y, void* pre, void* stream);

/* --------------------------------------------------------------------------
 * Backward pass of one rank's MLP ("Tensor parallelism" page, section "f and
 * g": g's backward is the identity, so every rank receives the whole output
 * gradient dZ; f's backward sums the ranks' input-gradient partials, one
 * all-reduce; a block's backward has two).  bf16 operands, float32
 * accumulation; weights as in tp_shard_mlp.
 *
 *   pre  = x w_in^T                          (recomputed pre-activation, [m, F])
 *   dY   = dZ w_out                          [m, f]
 *   dPre = dY * act'(pre)                    (GeLU; or [dY u SiLU'(g) | dY SiLU(g)]
 *                                             for pre = [g | u], SwiGLU)
 *   dx_partial = dPre w_in                   [m, h] float32 (the rank's share of dX)
 *   dw_out = dZ^T act(pre)                   [h, f] float32
 *   dw_in  = dPre^T x                        [F, h] float32
 * with F = f (GeLU) or 2 f (SwiGLU, rows [W1_i^T ; W3_i^T] as in the forward).
 *
 *   x, dz       [m, h] bf16; m must be a multiple of 8
 *   xt, dzt     [h, m] bf16 transposes of x and dz, or NULL (then the call
 *               makes them in ws; on one device the ranks may share them)
 *   pre         [m, F] bf16 pre-activation saved by tp_colwise_save in the
 *               forward, or NULL: then it is recomputed (x w_in^T)
 *   ws          workspace of tp_shard_mlp_backward_workspace_bytes bytes
 *
 * tp_transpose: dst [cols, rows] = src [rows, cols]^T (bf16).
 * tp_mlp_act_backward: the dPre step alone (and Y if y is not NULL).
 * ------------------------------------------------------------------------ */
/* --------------------------------------------------------------------------
 * tp_gemm_kmajor: the product the backward calls use for a transposed
 * operand ("MLP" and "Self-attention" sections: dX = dPre W_in,
 * dW = dZ^T Y and the like), read where it lies instead of transposed first.
 *   out[i, j] = sum_l x'[i, l] w'[l, j]       [m, n] float32 or bf16 (out_dt)
 *   w  [k, n] bf16, row stride ldw >= n (k-major: w' = w)
 *   x  x_kmajor = 0: [m, k] bf16, row stride ldx >= k (x' = x);
 *      x_kmajor = 1: [k, m] bf16, row stride ldx >= m (x' = x^T)
 * m, n, k, ldx, ldw multiples of 8; each operand under 2 GiB of offsets.
 * bf16 operands, float32 accumulation, device pointers, async on stream.
 * TP_ERR_SHAPE / TP_ERR_INVALID_ARG for bad sizes, strides or pointers.
 * ------------------------------------------------------------------------ */
tp_status tp_gemm_kmajor(tp_dtype out_dt, int32_t x_kmajor, int64_t m, int64_t n, int64_t k, const void* x,
                         int64_t ldx, const void* w, int64_t ldw, void* out, void* stream);

size_t tp_shard_mlp_backward_workspace_bytes(tp_act act, int64_t m, int64_t h, int64_t f_shard);
tp_status tp_shard_mlp_backward(tp_act act, int64_t m, int64_t h, int64_t f_shard, const void* x,
                                const void* w_in, const void* w_out, const void* dz, const void* xt,
                                const void* dzt, const void* pre, void* ws, size_t ws_bytes, float* dx_partial,
                                float* dw_in, float* dw_out, void* stream);
tp_status tp_transpose(int64_t rows, int64_t cols, const void* src, void* dst, void* stream);
tp_status tp_mlp_act_backward(tp_act act, int64_t m, int64_t n, const void* pre, const void* dy, void* dpre,
                              void* y, void* stream);

/* --------------------------------------------------------------------------
 * Backward pass of one rank's attention ("Tensor parallelism" page, sections
 * "Self-attention" and "f and g": the rank differentiates its own heads with
 * no exchange; a KV head read by several of its query heads gets the sum of
 * their gradients; the dX partials are summed over ranks by f's backward).
 * bf16 operands, float32 accumulation; d must be 128.
 *
 * tp_flash_attn_lse: tp_flash_attn that also writes
 *   lse   [batch, hq, seq_pad] float32 (seq_pad = seq rounded up to 64;
 *         entries past seq are left as they are): the log-sum-exp of each
 *         query row's scores in log2 units, so P = exp2(s log2(e)/sqrt(d) - lse).
 *
 * tp_flash_attn_backward: from the forward's q, k, vt, o, lse and the output
 * gradient dout [batch*seq, hq*d], with P the probabilities and
 * D = rowsum(dO * O):
 *   dV = P^T dO,  dS = P * (dO V^T - D),  dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d)
 * (dK, dV summed over the query heads sharing a KV head, in ascending order).
 * Writes bf16 rows of dqkv (row stride ld >= (hq + 2 hkv) d, a multiple of
 * 8): dQ in columns [0, hq d), dK in [hq d, (hq + hkv) d), dV after them, the
 * layout of tp_qkv_rope's projection output.  rope_base > 1 rotates dQ and dK
 * back through RoPE (the transpose of the forward rotation), giving the
 * gradient of the projection before RoPE; rope_base = 0 leaves them as the
 * gradients of the rotated q and k.  ws: at least
 * tp_flash_attn_backward_workspace_bytes bytes.  batch * hq <= 65535.
 *
 * tp_shard_attn_backward: the whole sublayer for the output gradient dZ
 * (weights as in tp_shard_attn):
 *   recompute q, k, vt (tp_qkv_rope), o and lse (tp_flash_attn_lse);
 *   dO = dZ w_o;  dQKV = tp_flash_attn_backward(...) before RoPE;
 *   dx_partial = dQKV w_qkv       [batch*seq, h] float32 (the rank's share of dX)
 *   dw_qkv     = dQKV^T x         [(hq + 2 hkv) d, h] float32
 *   dw_o       = dZ^T O           [h, hq d] float32
 *   x, dz      [batch*seq, h] bf16; batch*seq must be a multiple of 8
 *   xt, dzt    ignored (pass NULL; kept so the signature stays): dW_qkv
 *              and dW_o read x, dz, O and dQKV where they lie, as k-major
 *              operands of tp_gemm_kmajor's product, so no transposed copies
 *              are made (nor for w_o and w_qkv in dO and dX)
 *   saved_q, saved_k, saved_vt, saved_o, saved_lse: the forward's, as written
 *              by tp_shard_attn_save, all five or none (then recomputed)
 *   ws         at least tp_shard_attn_backward_workspace_bytes bytes
 * Biases are not differentiated here.
 *
 * tp_shard_attn_save: tp_shard_attn that keeps what the backward needs in
 * caller buffers instead of a workspace: q, k, vt (as tp_qkv_rope), o
 * [batch*seq, hq d] and lse (as tp_flash_attn_lse).
 * ------------------------------------------------------------------------ */
/* --------------------------------------------------------------------------
 * Backward of the fused shard-sum + RMSNorm (tp_shard_sum_rmsnorm): f's
 * backward sums the ranks' dX partials of the sublayer the norm feeds
 * ("Tensor parallelism" page, "f and g"), then the replicated norm's gradient
 * is taken, per row, and the gradient arriving through the residual added:
 *   dy = ((partials[0] + partials[1]) + ...)        (ascending rank order)
 *   r  = 1 / sqrt(mean(x^2) + eps),  g = gain * dy
 *   dx = r g - x r^3 sum(g x) / h  (+ residual_grad)
 *   dgain = sum over the m rows of dy x r          (partials summed in a fixed order)
 *   partials      t (1..16) float32 [m, h] device pointers (host array)
 *   x             [m, h] the norm's input (x_dt float32 or bf16)
 *   gain          [h] float32 or NULL (gain 1)
 *   residual_grad [m, h] (residual_dt) or NULL; dx may overwrite it if float32
 *   dx            [m, h] float32 or NULL;  dx_bf16 [m, h] bf16 or NULL (not both)
 *   dgain         [h] float32 or NULL; then ws needs
 *                 tp_shard_sum_rmsnorm_backward_workspace_bytes(m, h) bytes
 * The m = nrun * run_rows rows come in runs of run_rows rows, run_stride rows
 * apart (row k of run j is row j * run_stride + k of every [., h] operand), as
 * in tp_shard_sum_rmsnorm: a rank's slice of every sequence in the
 * sequence-parallel form ("Sequence parallelism": the backward of the
 * all-gather before the colwise GEMMs is a reduce-scatter onto the slices);
 * then dgain covers those rows only.  nrun = 1, run_rows = m: all rows.
 * h must be a multiple of 8 and at most 8192.
 * ------------------------------------------------------------------------ */
size_t tp_shard_sum_rmsnorm_backward_workspace_bytes(int64_t m, int64_t h);
tp_status tp_shard_sum_rmsnorm_backward(int32_t t, int64_t nrun, int64_t run_rows, int64_t run_stride, int64_t h,
                                        const float* const* partials, const void* x, tp_dtype x_dt, const float* gain,
                                        float eps, const void* residual_grad, tp_dtype residual_dt, float* dx,
                                        void* dx_bf16, float* dgain, void* ws, size_t ws_bytes, void* stream);

tp_status tp_flash_attn_lse(int64_t batch, int64_t seq, int32_t hq, int32_t hkv, int32_t head_dim,
                            int32_t causal, const void* q, const void* k, const void* vt, void* o, float* lse,
                            void* stream);
size_t tp_flash_attn_backward_workspace_bytes(int64_t batch, int64_t seq, int32_t hq, int32_t hkv,
                                              int32_t head_dim);
tp_status tp_flash_attn_backward(int64_t batch, int64_t seq, int32_t hq, int32_t hkv, int32_t head_dim,
                                 float rope_base, int32_t causal, const void* q, const void* k, const void* vt,
                                 const void* o, const float* lse, const void* dout, void* ws, size_t ws_bytes,
                                 void* dqkv, int64_t ld, void* stream);
size_t tp_shard_attn_backward_workspace_bytes(int64_t batch, int64_t seq, int64_t h, int32_t hq, int32_t hkv,
                                              int32_t head_dim);
tp_status tp_shard_attn_save(int64_t batch, int64_t seq, int64_t h, int32_t hq, int32_t hkv, int32_t head_dim,
                             float rope_base, int32_t causal, const void* x, const void* w_qkv, const void* w_o,
                             void* q, void* k, void* vt, void* o, float* lse, float* partial, void* stream);
tp_status tp_shard_attn_backward(int64_t batch, int64_t seq, int64_t h, int32_t hq, int32_t hkv, int32_t head_dim,
                                 float rope_base, int32_t causal, const void* x, const void* w_qkv, const void* w_o,
                                 const void* dz, const void* xt, const void* dzt, const void* saved_q,
                                 const void* saved_k, const void* saved_vt, const void* saved_o,
                                 const float* saved_lse, void* ws, size_t ws_bytes, float* dx_partial, float* dw_qkv,
                                 float* dw_o, void* stream);

/* --------------------------------------------------------------------------
 * Introspection: how the bf16 GEMM behind tp_colwise / tp_rowwise /
 * tp_qkv_rope tiles an m x n output over depth k (n = output columns; the
 * SwiGLU colwise GEMM's tiles cover 128 output columns instead of 256).
 * Tile columns [0, split) run at tile height bm_main and the remaining ones at
 * bm_tail (heights 256, 192 or 128 rows); with *split_k = 2 the remaining
 * columns run as 256-row tiles each summed by two workgroups over half of k
 * (single bf16-output launches of depth k >= 4096, when that shortens the
 * last round).  bm_main = bm_tail = 64 reports small tiles (64 rows x 128
 * columns, 64 output columns for SwiGLU; split = their tile columns), used
 * when large tiles would leave most of the chip idle (not for Q/K/V).  kind: TP_PLAN_ROWWISE (float32 partial), TP_PLAN_COLWISE
 * (bf16, plain or GeLU), TP_PLAN_SWIGLU, TP_PLAN_QKV.  Host-only; launches
 * nothing.  TP_ERR_SHAPE for non-positive sizes, TP_ERR_INVALID_ARG for an
 * unknown kind or a NULL output.
 * ------------------------------------------------------------------------ */
enum { TP_PLAN_ROWWISE = 0, TP_PLAN_COLWISE = 1, TP_PLAN_SWIGLU = 2, TP_PLAN_QKV = 3 };
tp_status tp_gemm_plan(int64_t m, int64_t n, int64_t k, int32_t kind, int32_t* bm_main, int32_t* split,
                       int32_t* bm_tail, int32_t* split_k);

/* --------------------------------------------------------------------------
 * Introspection: how tp_flash_attn, tp_flash_attn_lse and the attention
 * sublayer calls share the attention of batch x hq heads over seq tokens
 * among workgroups ("Self-attention" section: each head independent).
 * Query blocks of 128 rows are taken in pairs (p, last - p), so every pair
 * holds about the same causal work, and each pair's key tiles (64 keys) are
 * cut into *pieces equal ranges, one workgroup each (1: every query block
 * in one workgroup).  A block whose keys span pieces is completed by the
 * piece holding its last key tile, which merges the float32 partials of
 * the others (running max, sum and unnormalised output) in piece order.
 * Host-only; launches nothing.  TP_ERR_SHAPE for a negative batch or seq or
 * hq < 1, TP_ERR_INVALID_ARG for a NULL output.
 * ------------------------------------------------------------------------ */
tp_status tp_flash_attn_plan(int64_t batch, int64_t seq, int32_t hq, int32_t causal, int32_t* pieces);

/* Message for the calling thread's last error ("" if none). */
const char* tp_last_error(void);

/* TP_OK if the current HIP device is gfx950, else TP_ERR_UNSUPPORTED. */
tp_status tp_device_check(void);

#ifdef __cplusplus
}
#endif

#endif /* TPSHARD_H */
