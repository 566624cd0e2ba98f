// Launch functions of the gfx950 kernels (host side).  Each returns the
// hipError_t of its launch; argument checks happen in the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpk {

enum Epi : int {
  EPI_F32 = 0,     // float32 output (row-parallel partial)
  EPI_BF16 = 1,    // bf16 output, no nonlinearity
  EPI_GELU = 2,    // bf16 GeLU(acc)
  EPI_SWIGLU = 3,  // bf16 SiLU(gate) * up, weight rows [gate block ; up block]
  EPI_QKV = 4,     // Q/K with RoPE, V transposed per sequence
  EPI_GELU_SAVE = 5,    // EPI_GELU that also stores the bf16 pre-activation
  EPI_SWIGLU_SAVE = 6   // EPI_SWIGLU that also stores the bf16 gate and up pre-activations
};

struct QkvOut {
  void* q;
  void* k;
  void* vt;
  int64_t seq;
  int64_t seq_pad;
  int hq;
  int hkv;
  float log2_base;
};

// The _SAVE epilogues also store the bf16 pre-activation to pre: [M, N]
// (GeLU) or [M, 2N] (SwiGLU: the N gate columns, then the N up columns),
// with the bias added, exactly the values the nonlinearity reads.
// out[m, n] = epi( sum_k x[m, k] * w[row(n), k] + bias[n] ), bf16 operands,
// float32 accumulate.  bias (float32, or NULL) is added before the
// nonlinearity (SwiGLU: N gate biases then N up biases; QKV: before RoPE;
// not for EPI_F32).  x rows are lda elements apart (lda = 0: K), of which
// the first K are read.
hipError_t launch_gemm_bf16(int epi, int64_t M, int64_t N, int64_t K, const void* x, const void* w,
                            void* out, const QkvOut* qkv, hipStream_t s, const float* bias = nullptr,
                            int64_t lda = 0, void* pre = nullptr);

// Tile heights the bf16 GEMM launches for an M x N x K GEMM of a kind
// (N = output columns): columns [0, split) at height bm_main, the rest at
// bm_tail, or, with split_k = 2, as pairs of workgroups that each sum half of
// K over 256-row tiles.  groups: independent GEMMs of the same shape launched
// together.
enum { GEMM_PLAN_ROWWISE = 0, GEMM_PLAN_COLWISE = 1, GEMM_PLAN_SWIGLU = 2, GEMM_PLAN_QKV = 3 };
void gemm_plan(int64_t M, int64_t N, int64_t K, int kind, int groups, int* bm_main, int* split, int* bm_tail,
               int* split_k);

// out = epi(x' w') with w' = w stored k-major ([K, N], row stride ldw >= N)
// and x' = x either k-contiguous ([M, K], row stride ldx >= K) or, with
// x_kmajor, k-major too ([K, M], row stride ldx >= M): the backward's
// products of a transposed operand without a transpose pass.  epi: EPI_F32
// or EPI_BF16.  M, N, K multiples of 8; K * ldx * 2 and K * ldw * 2 bytes
// below 2 GiB.
hipError_t launch_gemm_bf16_km(int epi, bool x_kmajor, int64_t M, int64_t N, int64_t K, const void* x, int64_t ldx,
                               const void* w, int64_t ldw, void* out, hipStream_t s);
// G (<= 16) GEMMs of the same shape in one launch: out[g] = epi(x[g] . w[g]^T).
hipError_t launch_gemm_bf16_group(int epi, int groups, int64_t M, int64_t N, int64_t K,
                                  const void* const* x, const void* const* w, void* const* out,
                                  const QkvOut* qkv, hipStream_t s, const float* bias = nullptr,
                                  int64_t lda = 0, void* const* pre = nullptr);

// Same contraction in float32 throughout (EPI_F32 / EPI_BF16 meaning "no
// nonlinearity, float32 out", EPI_GELU, EPI_SWIGLU).
hipError_t launch_gemm_f32(int epi, int64_t M, int64_t N, int64_t K, const float* x, const float* w,
                           float* out, hipStream_t s, const float* bias = nullptr, int64_t lda = 0);

// Flash attention forward.  Query blocks of 128 rows are taken in pairs
// (p, last - p) and each pair's key tiles are cut into equal pieces, one per
// workgroup; a block whose keys are split over pieces is merged by the
// piece holding its last key tile from the float32 partials of the others,
// handed over through a split workspace:
//   part  FA_MAX_SLOTS slots of FA_SLOT_FLOATS floats
//   flag  FA_MAX_SLOTS words that only ever hold launch epochs (zero at first)
//   epoch this launch's epoch, distinct from every earlier one on these flags
// Calls that share a split workspace must not overlap.  ws = NULL: the
// per-(device, stream) workspace of the library, allocated at the first
// split launch on a stream (without it the launch runs unsplit).
// lse (optional): [batch, hq, seq_pad] float32 (entries past seq untouched),
// the log-sum-exp of the scores scaled to log2 units:
// P = exp2(s * log2(e) / sqrt(d) - lse).
constexpr int FA_MAX_SLOTS = 512;
constexpr int FA_SLOT_FLOATS = 128 * 128 + 2 * 256;  // O^T partial of 128 queries, then max and sum per thread
constexpr size_t FA_SLOT_BYTES = (size_t)FA_SLOT_FLOATS * 4;
struct FaSplitWs {
  float* part;
  unsigned* flag;
  unsigned epoch;
};
// Pieces per pair of query blocks the launch uses (1: unsplit); the split
// workspace holds (pieces - 1) x pairs x batch x hq slots.
int flash_attn_pieces(int64_t batch, int64_t seq, int hq, int causal);
size_t flash_attn_split_bytes(int64_t batch, int64_t seq, int hq, int causal);
hipError_t launch_flash_attn(int64_t batch, int64_t seq, int64_t seq_pad, int hq, int hkv,
                             int causal, const void* q, const void* k, const void* vt, void* o,
                             hipStream_t s, float* lse = nullptr, const FaSplitWs* ws = nullptr);

// Backward of launch_flash_attn for head_dim 128.  Inputs as the forward's
// (q, k token-major, vt per head transposed, seq_pad columns) plus kt
// [batch, hkv, 128, seq_pad] and vtok [batch, hkv, seq_pad, 128] (K
// transposed, V token-major, zero past seq), qt, dot [batch, hq, 128, seq_pad]
// (Q and dO transposed), dout [batch*seq, hq*128], lse and dvec
// [batch, hq, seq_pad] (dvec = rowsum(dO * O)).  Writes dQ into columns
// [0, hq*128) of dqkv rows (row stride ld), and dK, dV after it; with
// log2_base != 0 dQ and dK are rotated back through RoPE (base 2^log2_base).
// part: float32 scratch [batch, hkv, nsplit, 2, seq_pad, 128]; nsplit divides
// hq / hkv.
struct AttnBwdIn {
  const void* q;
  const void* k;
  const void* vtok;
  const void* kt;
  const void* qt;
  const void* dout;
  const void* dot;
  const float* lse;
  const float* dvec;
};
hipError_t launch_flash_attn_bwd(int64_t batch, int64_t seq, int64_t seq_pad, int hq, int hkv, int causal,
                                 double log2_base, const AttnBwdIn& in, float* part, int nsplit, void* dqkv,
                                 int64_t ld, hipStream_t s);
// dvec[b, j, p] = sum_c dout[b*seq + p, j*128 + c] * o[...] (rows past seq untouched).
hipError_t launch_attn_dvec(int64_t batch, int64_t seq, int64_t seq_pad, int hq, const void* o, const void* dout,
                            float* dvec, hipStream_t s);

hipError_t launch_shard_sum(int t, int64_t n, const float* const* partials, const void* residual,
                            int residual_bf16, float* out, hipStream_t s);

hipError_t launch_rmsnorm(int in_bf16, int64_t m, int64_t h, const void* x, const float* gain,
                          float eps, void* y, hipStream_t s);

// x = shard-sum of t (0..16) partials (+ bias[h]) (+ residual) over nrun runs of run_rows
// rows of h (runs run_stride rows apart); out = x if out, y = RMSNorm(x)
// (bf16) if y; one pass.
hipError_t launch_sum_rmsnorm(int t, int64_t nrun, int64_t run_rows, int64_t run_stride, int64_t h,
                              const float* const* partials, const float* bias, const void* residual,
                              int residual_bf16, float* out, const float* gain, float eps, void* y,
                              hipStream_t s);

// out[i, 0:w] (rows ld apart, float32) = table[ids[i] - v_start] (bf16) for
// ids in [v_start, v_start + v_rows), else zeros.
hipError_t launch_embedding(int64_t m, int64_t w, int64_t v_start, int64_t v_rows, const int32_t* ids,
                            const void* table, float* out, int64_t ld, hipStream_t s);

// stats[i] = {max, sum of exp(x - max), x_label or 0, 1 if the label is the
// rank's} over logits[i, 0:n) (float32), the rank's vocabulary [v_start, v_start + n).
hipError_t launch_ce_stats(int64_t m, int64_t n, int64_t v_start, const float* logits, const int32_t* labels,
                           float* stats, hipStream_t s);

// Per-token loss from the t ranks' statistics, and (if mean) the mean over
// tokens whose label is in [0, v).
hipError_t launch_ce_combine(int t, int64_t m, const float* const* stats, float* loss, const int32_t* labels,
                             int64_t v, float* mean, hipStream_t s);

// dst [cols, rows] = src [rows, cols]^T, bf16.
hipError_t launch_transpose(int64_t rows, int64_t cols, const void* src, void* dst, hipStream_t s);

// Per batch z = z1 * n2 + z2 (z1 < n1): with src and dst advanced by
// z1 * bs1 + z2 * bs2 of their own, dst[c * ldd + r] = r < rows_in ?
// src[r * lds + c] : 0 for r < rows_out (a multiple of 8), c < cols; reads up
// to 7 elements past cols in each source row (the caller keeps them in bounds).
hipError_t launch_transpose_batched(int64_t n1, int64_t n2, int64_t rows_in, int64_t rows_out, int64_t cols,
                                    int64_t lds, int64_t ldd, int64_t src_bs1, int64_t src_bs2, int64_t dst_bs1,
                                    int64_t dst_bs2, const void* src, void* dst, hipStream_t s);

// Backward of the fused sum + RMSNorm: dy = sum of the t partials (ascending),
// dx = r gain dy - x r^3 sum(gain dy x) / h (+ res), per row; dgain = sum over
// rows of dy x r (ws: norm_bwd_blocks(m) * h float32 partials).  h <= 8192.
// m = nrun * run_rows rows, in runs of run_rows run_stride apart.
int64_t norm_bwd_blocks(int64_t m);
hipError_t launch_sum_rmsnorm_bwd(int t, int64_t nrun, int64_t run_rows, int64_t run_stride, int64_t h,
                                  const float* const* partials, const void* x, int x_bf16, const float* gain,
                                  float eps, const void* res, int res_bf16, float* dx, void* dx_bf16, float* dgain,
                                  float* ws, hipStream_t s);

// From the pre-activation and dY (n columns): dPre and, if y, the activation
// Y.  GeLU: pre [m, n]; SwiGLU: pre [m, 2n] = [gate | up], dPre likewise.
// Size of the static device array tp_shard_attn_noalloc uses as its
// workspace, and the lookup of its address on the current device (once per
// device, then cached; no allocation).
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
hipError_t static_scratch(void** ptr);
// The first kStaticFlagBytes of that array hold the flags of the attention's
// split workspace (only ever written with launch epochs); epoch receives the
// next epoch of this device.
constexpr size_t kStaticFlagBytes = (size_t)FA_MAX_SLOTS * sizeof(unsigned);
hipError_t static_scratch_epoch(unsigned* epoch);

hipError_t launch_act_backward(int swiglu, int64_t m, int64_t n, const void* pre, const void* dy, void* dpre,
                               void* y, hipStream_t s);

}  // namespace tpk
