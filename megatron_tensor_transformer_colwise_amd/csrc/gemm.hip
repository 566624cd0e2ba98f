// bf16 MFMA GEMM for gfx950:  out[m, n] = epi( sum_k X[m, k] * W[row(n), k] ).
//
// This is the contraction of both tensor-parallel linears of the "Tensor
// parallelism" page ("Matmul split"): the column-parallel one, whose output
// slice goes straight through the per-rank nonlinearity ("MLP": GeLU, or
// SwiGLU) or through RoPE ("Self-attention": the Q/K/V projection), and the
// row-parallel one, whose output is the rank's float32 partial sum.
//
// Both operands are contiguous along k (X row-major, W in nn.Linear layout), so
// every MFMA operand of a lane is 16 contiguous bytes of one row.
//
// Tiling: BMT x 256 output tiles, BMT in {256, 192, 128}, always 8 waves (two
// per SIMD, so one issues MFMAs while the other waits on memory or the
// barrier).  A wave owns MI x NJ blocks of v_mfma_f32_32x32x16_bf16: 64 x 128
// at BMT 256 (128 float32 accumulators per lane), 96 x 64 at 192, 64 x 64 at
// 128.  At 192 rows, 4 waves of 96 x 128 read less from LDS but leave each
// SIMD one wave and nothing to cover its waits (13% slower on a QKV
// projection); at 128 rows, 32 x 128 waves would read 5 fragments per 4
// MFMAs instead of 4.  k advances 64 at a time through a
// two-stage LDS ring; tiles are fetched with 16-byte buffer loads that write
// LDS directly (no register staging), all of a stage's loads issued
// together.  The one barrier of a k-step sits halfway through its last
// 16-deep substep: it makes the next stage visible and frees the current
// one, whose refill (two stages ahead) goes out at once while the step's
// remaining MFMAs cover the next stage's first fragment reads; within a
// substep one fragment read follows each MFMA.  Out-of-range rows and the k tail are fetched as zeros by the
// buffer's range check.  Each LDS row holds 64 bf16; its eight 16-byte chunks
// are XOR-permuted by swz(row) so the 32 rows one fragment read touches hit
// distinct banks (measured: no bank conflicts).
//
// The inner loop carries almost no address arithmetic: LDS holds the two A
// stages, then the two B stages, so a fragment's address is a fixed per-lane
// register plus an immediate that selects the stage (the k loop is unrolled
// by the two stages), and a global load's k advance is a scalar offset on a
// fixed per-lane offset.  Only a partial last k-step takes the per-lane
// k-range checks.
//
// The host picks the tile height per launch, and may split the tile columns
// into a main range and a tail range of lower height, to minimise
// rounds-of-256-workgroups x (BMT + 256): the loads of a tile scale with
// BMT + 256 and the kernel is close to its load bound, while a partly filled
// last round costs a whole round.
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "common.h"
#include "kernels.h"

namespace tpk {
namespace {

constexpr int BN = 256;                         // tile columns (weight rows)
constexpr int BK = 64;                          // k per stage
constexpr int NSTAGE = 2;                       // LDS ring depth
constexpr int CH = BK / 8;                      // 16-byte chunks per tile row
constexpr int ROWB = BK * 2;                    // bytes per tile row
constexpr int KSUB = BK / 16;                   // MFMA k-steps per stage
constexpr int B_TILE = BN * ROWB;               // one stage of weight rows
constexpr int B_INSTR = BN * CH / 64;           // wave-instructions per B stage

// 32-row MFMA blocks per wave for a tile height.  The waves split the tile
// rows and columns evenly into 8 waves, so every SIMD carries the same MFMA
// work (rows x columns of waves): 256 -> 4 x 2 waves of 64 x 128, 192 -> 2 x 4
// of 96 x 64, 128 -> 2 x 4 of 64 x 64 (no spills at any height).
constexpr int wave_blocks(int bmt) { return bmt == 256 ? 2 : bmt == 192 ? 3 : 2; }
// 32-column MFMA blocks per wave: 4 (a 128-column half of the tile) or 2.
constexpr int wave_cols(int bmt) { return bmt == 256 ? 4 : 2; }

// Tile column block (0..7, 32 columns each) of a wave's block jj.  A wave
// always holds blocks jj and jj + NJ / 2 exactly 64 columns apart, so the
// SwiGLU gate/up pair and the RoPE pair (c, c + 64) meet in one lane.
template <int NJ>
__device__ __forceinline__ int col_block(int wn, int jj) {
  return NJ == 4 ? 4 * wn + jj : 4 * (wn >> 1) + (wn & 1) + 2 * jj;
}

// W4: the tile worked by four waves (one per SIMD) in a 2 x 2 grid of
// (BMT / 2) x 128 each.
template <int BMT, bool W4 = false>
struct Cfg {
  static constexpr int MI = W4 ? BMT / 64 : wave_blocks(BMT);  // 32-row MFMA blocks per wave
  static constexpr int NJ = W4 ? 4 : wave_cols(BMT);          // 32-column MFMA blocks per wave
  static constexpr int WROWS = 32 * MI;                       // rows per wave
  static constexpr int WC = 8 / NJ;                           // wave columns
  static constexpr int NW = BMT / WROWS * WC;                 // waves
  static_assert(NW % 4 == 0 && BMT % WROWS == 0, "waves must cover the tile and the SIMDs");
  static constexpr int A_TILE = BMT * ROWB;
  static constexpr int SMEM = NSTAGE * (A_TILE + B_TILE);  // A stages, then B stages
  static constexpr int B_BASE = NSTAGE * A_TILE;
  static constexpr int A_INSTR = BMT * CH / 64;               // wave-instructions per A stage
  static constexpr int LA = (A_INSTR + NW - 1) / NW;          // per wave, A
  static constexpr int LB = (B_INSTR + NW - 1) / NW;          // per wave, B
  static_assert(SMEM <= 160 * 1024, "LDS");
};

constexpr int MAX_GROUP = 16;

// Operands of one launch.  A launch may carry G independent GEMMs of equal
// shape (one per tensor-parallel rank): blockIdx.y selects x[g], w[g], out[g].
struct Args {
  const bf16_t* x[MAX_GROUP];
  const bf16_t* w[MAX_GROUP];
  void* out[MAX_GROUP];
  int64_t M, N, K;
  int64_t lda;        // row stride of x in elements (>= K; a column slice when > K); k-major x: of its k rows
  int64_t ldb;        // k-major w (the 16x16 kernel's KM >= 1): row stride of its k rows (>= N)
  const float* bias;  // per output column, added before the epilogue's nonlinearity, or NULL
  void* pre[MAX_GROUP];  // _SAVE epilogues: bf16 pre-activation rows (GeLU N, SwiGLU 2 N wide)
  int num_bm;  // tile rows of this launch (height BMT)
  int num_bn;  // tile columns of this launch
  int bn0;     // first tile column of this launch
  QkvOut qkv;
  // Split-k launches of the 16x16 kernel (NULL sk_ws: none).  Two workgroups
  // share each tile p: the producer sums k-steps [sk_half, nk) into sk_ws
  // tile p and then raises sk_flag[p] to sk_epoch; the consumer sums k-steps
  // [0, sk_half), waits for the flag, adds the partial and runs the epilogue.
  float* sk_ws;
  unsigned* sk_flag;
  unsigned sk_epoch;
  int sk_half;
};

// Chunk permutation of tile row r.  Reads of one fragment touch 32 consecutive
// rows at one logical chunk; the permutation makes every 8-row group (128-byte
// bank window) and every 16-row group (256-byte window) hit distinct banks.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Launch index -> output tile.  Workgroups are dealt to the 8 XCDs round-robin;
// first undo that so each XCD owns a contiguous range of logical tiles, then
// walk tiles in groups of 8 tile-rows so a range is a compact patch whose X
// rows and W rows stay in that XCD's L2.
__device__ __forceinline__ void tile_coords(int id, int nb, int num_bm, int num_bn, int& bm,
                                            int& bn) {
  const int xcd = id & 7, local = id >> 3;
  const int per = nb >> 3, rem = nb & 7;
  const int L = (xcd < rem) ? xcd * (per + 1) + local
                            : rem * (per + 1) + (xcd - rem) * per + local;
  constexpr int G = 8;
  const int span = G * num_bn;
  const int g = L / span;
  const int first = g * G;
  const int gs = min(num_bm - first, G);
  const int inner = L - g * span;
  bm = first + inner % gs;
  bn = inner / gs;
}

// GeLU for bf16 outputs: 0.5 x erfc(-x / sqrt 2) with erfc from the
// Chebyshev fit of Numerical Recipes (Press et al., 2nd ed., section 6.2,
// "erfcc": fractional error below 1.2e-7 for every argument): one exp2, one
// reciprocal and a degree-9 polynomial, without branches, so a wave's
// elements interleave (the library erff branches on the argument's range).
// Its error stays far below a bf16 rounding step.
__device__ __forceinline__ float gelu_bf16out(float x) {
  const float u = -0.70710678118654752440f * x;
  const float z = fabsf(u);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, z, 1.0f));
  float p = 0.17087277f;
  p = fmaf(t, p, -0.82215223f);
  p = fmaf(t, p, 1.48851587f);
  p = fmaf(t, p, -1.13520398f);
  p = fmaf(t, p, 0.27886807f);
  p = fmaf(t, p, -0.18628806f);
  p = fmaf(t, p, 0.09678418f);
  p = fmaf(t, p, 0.37409196f);
  p = fmaf(t, p, 1.00002368f);
  p = fmaf(t, p, -1.26551223f);
  // t exp(-z^2 + p) with exp(y) = exp2(y log2 e)
  const float e = t * __builtin_amdgcn_exp2f((p - z * z) * 1.44269504088896340736f);
  const float erfc_u = u >= 0.0f ? e : 2.0f - e;
  return 0.5f * x * erfc_u;
}

constexpr bool is_swiglu(int epi) { return epi == EPI_SWIGLU || epi == EPI_SWIGLU_SAVE; }
constexpr bool is_gelu(int epi) { return epi == EPI_GELU || epi == EPI_GELU_SAVE; }
constexpr bool saves_pre(int epi) { return epi == EPI_GELU_SAVE || epi == EPI_SWIGLU_SAVE; }

template <int EPI, int BMT, bool W4>
__global__ __launch_bounds__((Cfg<BMT, W4>::NW * 64), 1) void gemm_bf16_kernel(Args args) {
  using C = Cfg<BMT, W4>;
  constexpr int NW = C::NW;
  constexpr int MI = C::MI;
  constexpr int WROWS = C::WROWS;
  constexpr int NJ = C::NJ;
  constexpr int NP = NJ / 2;  // (first, second) block pairs 64 columns apart
  __shared__ __attribute__((aligned(1024))) char smem[C::SMEM];

  const int lane = lane_id();
  const int wave = wave_id();
  const bf16_t* const xg = args.x[blockIdx.y];
  const bf16_t* const wg = args.w[blockIdx.y];
  void* const outg = args.out[blockIdx.y];
  int bm, bn;
  tile_coords(blockIdx.x, gridDim.x, args.num_bm, args.num_bn, bm, bn);
  // The tile coordinates come out of VALU divisions; marking them uniform
  // keeps the buffer descriptors built from them in scalar registers (the
  // compiler otherwise wrapped every global load of some epilogue variants
  // in a loop over the wave's distinct descriptor values).
  bm = __builtin_amdgcn_readfirstlane(bm);
  bn = __builtin_amdgcn_readfirstlane(bn + args.bn0);

  const int64_t M = args.M, N = args.N, K = args.K, lda = args.lda;
  const int64_t m0 = (int64_t)bm * BMT;
  const uint32_t row_bytes = (uint32_t)(K * 2);     // a weight row
  const uint32_t a_row_bytes = (uint32_t)(lda * 2);  // an x row (its first K columns are read)

  // ---- global -> LDS addressing -------------------------------------------
  const int m_rows = (int)min<int64_t>(BMT, M - m0);
  __amdgpu_buffer_rsrc_t rsrc_a = make_rsrc(xg + m0 * lda, (uint32_t)m_rows * a_row_bytes);

  __amdgpu_buffer_rsrc_t rsrc_b;
  int n_valid;  // valid weight rows (plain) or valid output columns (SwiGLU)
  if (is_swiglu(EPI)) {
    const int64_t o0 = (int64_t)bn * (BN / 2);
    n_valid = (int)min<int64_t>(BN / 2, N - o0);
    rsrc_b = make_rsrc(wg + o0 * K, (uint32_t)((N + n_valid) * K * 2));
  } else {
    const int64_t n0 = (int64_t)bn * BN;
    n_valid = (int)min<int64_t>(BN, N - n0);
    rsrc_b = make_rsrc(wg + n0 * K, (uint32_t)n_valid * row_bytes);
  }

  // Wave-instruction blk of a stage fills slots blk * 64 + lane: tile row
  // slot / CH, physical chunk slot % CH, i.e. logical chunk (slot % CH) ^
  // swz(row).  Wave w issues blocks j * NW + w.
  uint32_t a_off[C::LA], b_off[C::LB];
  int a_k[C::LA], b_k[C::LB];  // element offset of the chunk within the k-block
#pragma unroll
  for (int j = 0; j < C::LA; ++j) {
    const int slot = (j * NW + wave) * 64 + lane;
    const int r = slot / CH;
    const int c = (slot % CH) ^ swz(r);
    a_k[j] = c * 8;
    a_off[j] = (uint32_t)r * a_row_bytes + (uint32_t)c * 16;
  }
#pragma unroll
  for (int j = 0; j < C::LB; ++j) {
    const int slot = (j * NW + wave) * 64 + lane;
    const int r = slot / CH;
    const int c = (slot % CH) ^ swz(r);
    b_k[j] = c * 8;
    if (is_swiglu(EPI)) {
      const int wn = r >> 7, qq = r & 127;
      const int o_rel = wn * 64 + (qq & 63);
      const int64_t rel_row = (qq < 64) ? o_rel : N + o_rel;
      b_off[j] = (o_rel < n_valid) ? (uint32_t)(rel_row * K * 2) + (uint32_t)c * 16 : TP_OOB_OFFSET;
    } else {
      b_off[j] = (uint32_t)r * row_bytes + (uint32_t)c * 16;
    }
  }

  // All loads of stage S for k-step kn (blocks past the tile are skipped
  // wave-uniformly).  FULL: a whole k-step, whose k offset is a scalar added
  // to fixed per-lane offsets.  Otherwise each chunk beyond K is sent out of
  // the buffer, so it reads zeros.
  auto load_stage = [&](auto stage_tag, auto full_tag, int kn) {
    constexpr int S = decltype(stage_tag)::value;
    constexpr bool FULL = decltype(full_tag)::value;
    char* const a_dst = smem + S * C::A_TILE;
    char* const b_dst = smem + C::B_BASE + S * B_TILE;
    const uint32_t kb = (uint32_t)kn * (uint32_t)(BK * 2);
    const int64_t k0 = (int64_t)kn * BK;
#pragma unroll
    for (int j = 0; j < C::LA; ++j) {
      const int blk = j * NW + wave;
      if (C::A_INSTR % NW == 0 || blk < C::A_INSTR) {
        if (FULL) {
          buffer_load_lds16_so(rsrc_a, a_dst + blk * 1024, a_off[j], kb);
        } else {
          const bool kin = (k0 + a_k[j]) < K;
          buffer_load_lds16(rsrc_a, a_dst + blk * 1024, kin ? a_off[j] + kb : TP_OOB_OFFSET);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < C::LB; ++j) {
      const int blk = j * NW + wave;
      if (B_INSTR % NW == 0 || blk < B_INSTR) {
        if (FULL) {
          buffer_load_lds16_so(rsrc_b, b_dst + blk * 1024, b_off[j], kb);
        } else {
          const bool kin = (k0 + b_k[j]) < K && b_off[j] != TP_OOB_OFFSET;
          buffer_load_lds16(rsrc_b, b_dst + blk * 1024, kin ? b_off[j] + kb : TP_OOB_OFFSET);
        }
      }
    }
  };

  // Load j (0 .. LA + LB - 1) of stage S for k-step kn: the A loads, then the B loads.
  auto load_one = [&](auto stage_tag, auto full_tag, int kn, int j) {
    constexpr int S = decltype(stage_tag)::value;
    constexpr bool FULL = decltype(full_tag)::value;
    const uint32_t kb = (uint32_t)kn * (uint32_t)(BK * 2);
    const int64_t k0 = (int64_t)kn * BK;
    if (j < C::LA) {
      char* const a_dst = smem + S * C::A_TILE + (j * NW + wave) * 1024;
      if (FULL) buffer_load_lds16_so(rsrc_a, a_dst, a_off[j], kb);
      else buffer_load_lds16(rsrc_a, a_dst, ((k0 + a_k[j]) < K) ? a_off[j] + kb : TP_OOB_OFFSET);
    } else {
      const int jb = j - C::LA;
      char* const b_dst = smem + C::B_BASE + S * B_TILE + (jb * NW + wave) * 1024;
      if (FULL) buffer_load_lds16_so(rsrc_b, b_dst, b_off[jb], kb);
      else {
        const bool kin = (k0 + b_k[jb]) < K && b_off[jb] != TP_OOB_OFFSET;
        buffer_load_lds16(rsrc_b, b_dst, kin ? b_off[jb] + kb : TP_OOB_OFFSET);
      }
    }
  };

  // ---- LDS -> registers addressing ----------------------------------------
  const int wm = wave / C::WC, wn = wave % C::WC;
  const int l31 = lane & 31, hk = lane >> 5;
  uint32_t ra[MI][KSUB], rb[NJ][KSUB];  // [block][s] byte offsets within a tile
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int r_a = wm * WROWS + i * 32 + l31;
#pragma unroll
    for (int s = 0; s < KSUB; ++s) {
      const int c = 2 * s + hk;
      ra[i][s] = (uint32_t)(r_a * ROWB + ((c ^ swz(r_a)) << 4));
    }
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int r_b = col_block<NJ>(wn, j) * 32 + l31;
#pragma unroll
    for (int s = 0; s < KSUB; ++s) {
      const int c = 2 * s + hk;
      rb[j][s] = (uint32_t)(C::B_BASE + r_b * ROWB + ((c ^ swz(r_b)) << 4));
    }
  }

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};

  // Fragments are double-buffered in registers: while the MFMAs of k-step s
  // run, the fragment reads of step s + 1 are in flight, so LDS latency does
  // not stall the matrix pipe inside a stage.
  u32x4 fa[2][MI], fb[2][NJ];
  const int nk = (int)((K + BK - 1) / BK);
  const int nfull = (int)(K / BK);
  using Full = std::true_type;
  using Partial = std::false_type;
  constexpr std::integral_constant<int, 0> st0{};
  constexpr std::integral_constant<int, 1> st1{};
  constexpr int NQ = MI * NJ > MI + NJ ? MI * NJ : MI + NJ;
  constexpr int MID = MI * NJ / 2;  // the hand-over point inside the last k-substep
  static_assert(C::A_INSTR % NW == 0 && B_INSTR % NW == 0, "every wave issues LA + LB loads per stage");
  // One k-step on stage S (resident, its first fragments already in
  // registers).  Two stages are in flight: halfway through the last substep
  // the barrier retires every read of stage S and makes stage kt + 1
  // visible; stage kt + 2 is then fetched into S while the remaining MFMAs
  // of this step cover the first fragment reads of stage kt + 1.
  // Four waves (one per SIMD, 128 x 128 each): a k-step is 4 substeps of 16
  // MFMAs.  With a single wave per SIMD every non-MFMA instruction delays the
  // matrix pipe, so the schedule spreads them out: the 8 fragment reads of
  // the next substep follow the first 8 MFMAs of a substep (A0, B0..B3,
  // A1..A3, the order the MFMAs consume them), and the 16 loads of the stage
  // after next go out one per second MFMA over the three substeps after the
  // barrier that frees its buffer (4 after it in this step, 6 + 6 in the first
  // two substeps of the next), leaving a substep and a half for the last to
  // land.  The k-step's one barrier sits after the 8th MFMA of its last
  // substep: every read of this stage is done and the next stage has landed,
  // so the remaining 8 MFMAs carry the next stage's first fragment reads.
  // Issuing a stage's loads in one burst instead doubled their average L2
  // latency (counter-measured) and cost 8% of the k loop.
  auto kstep4 = [&](auto stage_tag, auto main_tag, int kt) {
    constexpr int S = decltype(stage_tag)::value;
    constexpr bool MAIN = decltype(main_tag)::value;
    constexpr std::integral_constant<int, 1 - S> other_tag{};
    constexpr int NMF = MI * NJ;            // MFMAs per substep
    constexpr int NRD = MI + NJ;            // fragment reads per substep
    constexpr int BPOS = NMF - NRD;         // the barrier follows this many MFMAs of the last substep
    constexpr int NLD = C::LA + C::LB;      // loads per wave per stage
    constexpr int NST = NRD / 2;            // loads after the barrier, one per second MFMA
    constexpr int NC0 = (NLD - NST + 1) / 2, NC1 = NLD - NST - NC0;  // in substeps 0 and 1
    constexpr int SP0 = NMF / NC0, SP1 = NMF / NC1;                 // their spacing in MFMAs
    static_assert(NJ == 4 && BPOS > 0 && SP0 >= 1 && SP1 >= 1, "four-wave schedule");
    const char* const a_st = smem + S * C::A_TILE;
    const char* const b_st = smem + S * B_TILE;
    const char* const a_nx = smem + (1 - S) * C::A_TILE;
    const char* const b_nx = smem + (1 - S) * B_TILE;
    const bool cont = MAIN || (kt >= 1 && kt + 1 < nk);  // rest of step kt + 1's loads
    const bool cont_full = MAIN || kt + 1 < nfull;
    const bool start = MAIN || kt + 2 < nk;               // first loads of step kt + 2
    const bool start_full = MAIN || kt + 2 < nfull;
    // fragment read r: A0, B0..B3, A1.. (the order the MFMAs use them)
    auto rd = [&](const char* a, const char* b, int sub, int r) {
      const int ia = r == 0 ? 0 : (r >= 5 ? r - 4 : -1);
      if (ia >= 0) fa[(sub & 1)][ia] = lds_read16(a + ra[ia][sub]);
      else fb[(sub & 1)][r - 1] = lds_read16(b + rb[r - 1][sub]);
    };
#pragma unroll
    for (int s = 0; s < KSUB; ++s) {
      const int cur = s & 1;
#pragma unroll
      for (int q = 0; q < NMF; ++q) {
        if (s == KSUB - 1 && q == BPOS) {
          wait_vmcnt0();
          wait_lgkmcnt0();
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
        acc[q / NJ][q % NJ] = mfma32x32x16(fa[cur][q / NJ], fb[cur][q % NJ], acc[q / NJ][q % NJ]);
        if (s + 1 < KSUB) {
          if (q < NRD) rd(a_st, b_st, s + 1, q);
        } else if (q >= BPOS) {
          rd(a_nx, b_nx, 0, q - BPOS);
        }
        if (s < 2 && cont) {
          const int sp = s == 0 ? SP0 : SP1;
          const int i = (q + 1) / sp - 1;
          if ((q + 1) % sp == 0 && i < (s == 0 ? NC0 : NC1)) {
            const int j = NST + (s == 0 ? 0 : NC0) + i;
            if (cont_full) load_one(other_tag, Full{}, kt + 1, j);
            else load_one(other_tag, Partial{}, kt + 1, j);
          }
        }
        if (s == KSUB - 1 && q > BPOS && ((q - BPOS) & 1) && start) {
          const int j = (q - BPOS) >> 1;
          if (start_full) load_one(stage_tag, Full{}, kt + 2, j);
          else load_one(stage_tag, Partial{}, kt + 2, j);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto kstep = [&](auto stage_tag, auto main_tag, int kt) {
    constexpr int S = decltype(stage_tag)::value;
    constexpr bool MAIN = decltype(main_tag)::value;
    const char* const a_st = smem + S * C::A_TILE;
    const char* const b_st = smem + S * B_TILE;  // rb[][] holds the B base
    const char* const a_nx = smem + (1 - S) * C::A_TILE;
    const char* const b_nx = smem + (1 - S) * B_TILE;
#pragma unroll
    for (int s = 0; s < KSUB; ++s) {
      const int cur = s & 1, nxt = cur ^ 1;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if (s == KSUB - 1 && q == MID) {
          wait_vmcnt0();
          __syncthreads();
          if (MAIN) load_stage(stage_tag, Full{}, kt + 2);
          else if (kt + 2 < nfull) load_stage(stage_tag, Full{}, kt + 2);
          else if (kt + 2 < nk) load_stage(stage_tag, Partial{}, kt + 2);
        }
        if (q < MI * NJ)
          acc[q / NJ][q % NJ] = mfma32x32x16(fa[cur][q / NJ], fb[cur][q % NJ], acc[q / NJ][q % NJ]);
        if (s + 1 < KSUB) {
          if (q < MI) fa[nxt][q] = lds_read16(a_st + ra[q][s + 1]);
          else if (q < MI + NJ) fb[nxt][q - MI] = lds_read16(b_st + rb[q - MI][s + 1]);
        } else if (q >= MID) {
          // first fragments of stage kt + 1 (beyond K: zeros or unused data)
          const int r = q - MID;
          if (r < MI) fa[nxt][r] = lds_read16(a_nx + ra[r][0]);
          else if (r < MI + NJ) fb[nxt][r - MI] = lds_read16(b_nx + rb[r - MI][0]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (s == KSUB - 1) {
        // fragment reads that did not fit beside the MFMAs after the barrier
#pragma unroll
        for (int r = NQ - MID; r < MI + NJ; ++r) {
          if (r < MI) fa[nxt][r] = lds_read16(a_nx + ra[r][0]);
          else fb[nxt][r - MI] = lds_read16(b_nx + rb[r - MI][0]);
        }
      }
    }
  };
  if (nfull > 0) load_stage(st0, Full{}, 0);
  else load_stage(st0, Partial{}, 0);
  if (nk > 1) {
    if (nfull > 1) load_stage(st1, Full{}, 1);
    else load_stage(st1, Partial{}, 1);
    wait_vmcnt<C::LA + C::LB>();  // stage 0 landed, stage 1 may still be in flight
  } else {
    wait_vmcnt0();
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < MI; ++i) fa[0][i] = lds_read16(smem + ra[i][0]);
#pragma unroll
  for (int j = 0; j < NJ; ++j) fb[0][j] = lds_read16(smem + rb[j][0]);
  int kt = 0;
  // pairs of steps whose stage-after-next is a whole k-step
  if constexpr (NW == 4) {
    kstep4(st0, Partial{}, 0);
    if (nk > 1) kstep4(st1, Partial{}, 1);
    kt = 2;
    for (; kt + 3 < nfull; kt += 2) {
      kstep4(st0, Full{}, kt);
      kstep4(st1, Full{}, kt + 1);
    }
    for (; kt < nk; kt += 2) {
      kstep4(st0, Partial{}, kt);
      if (kt + 1 < nk) kstep4(st1, Partial{}, kt + 1);
    }
  } else {
  for (; kt + 3 < nfull; kt += 2) {
    kstep(st0, Full{}, kt);
    kstep(st1, Full{}, kt + 1);
  }
  for (; kt < nk; kt += 2) {
    kstep(st0, Partial{}, kt);
    if (kt + 1 < nk) kstep(st1, Partial{}, kt + 1);
  }
  }
  wait_vmcnt0();

  // ---- epilogue -----------------------------------------------------------
  // Accumulator element r of block (i, j) in lane L is output row
  // 32 i + 8 (r / 4) + 4 (L / 32) + r % 4 of the wave's rows and column
  // 32 col_block(wn, j) + L % 32 of the tile.  For bf16 outputs each group of 4
  // consecutive rows is transposed across the 4 lanes of a quad, so a lane
  // ends up with 4 consecutive columns of one row and writes them as one
  // 8-byte store instead of four 2-byte ones.  The transposes run in every
  // lane (they exchange data between lanes); only the stores are masked by
  // the output bounds.  float32 partials are stored as they lie, one 4-byte
  // store per element (measured: no slower than 16-byte stores after a
  // transpose, which costs VALU time the tile holds its CU for).  They are
  // stored non-temporally: a partial is next read by the shard-sum after the
  // other ranks' work, and left in the 256 MiB Infinity Cache it evicts the
  // operands the next GEMM reads (measured on the 70B t = 8 block: step
  // 13.23 -> 12.88 ms, the SwiGLU GEMM 732 -> 704 us, attention 0.398 ->
  // 0.347 ms).
  const int64_t row_base = m0 + wm * WROWS + 4 * hk;
  const int q = l31 & 3;             // row within a group after the transpose
  const int cq = 4 * (l31 >> 2);     // first of the lane's 4 columns after it
  const int hg = NJ == 4 ? wn : wn >> 1;  // the wave's 128-column group of the tile
  // column offset, within the first 64 of its group, of pair jp's first block
  auto pair_col = [&](int jp) { return 32 * (NJ == 4 ? jp : (wn & 1)); };
  if (EPI == EPI_F32 && NW == 4) {
    // four waves: 16-byte stores of 4 consecutive columns after a quad transpose
    const int64_t col_base = (int64_t)bn * BN + cq;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int64_t col = col_base + col_block<NJ>(wn, j) * 32;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e];
          quad_transpose(v, q);
          const int64_t row = row_base + i * 32 + 8 * g + q;
          if (row < M && col < N)
            __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]},
                                        reinterpret_cast<f32x4*>(reinterpret_cast<float*>(outg) + row * N + col));
        }
      }
  } else if (EPI == EPI_F32) {
    const int64_t col_base = (int64_t)bn * BN + l31;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int64_t col = col_base + col_block<NJ>(wn, j) * 32;
        if (col >= N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = row_base + i * 32 + 8 * (r >> 2) + (r & 3);
          if (row < M) __builtin_nontemporal_store(acc[i][j][r], reinterpret_cast<float*>(outg) + row * N + col);
        }
      }
  } else if (EPI == EPI_BF16 || is_gelu(EPI)) {
    const int64_t col_base = (int64_t)bn * BN + cq;
    // the bias of each block's column of this lane (before the transpose);
    // -0 is the identity of the float add, so no bias leaves results as they were
    float bcol[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t c = (int64_t)bn * BN + col_block<NJ>(wn, j) * 32 + l31;
      bcol[j] = (args.bias && c < N) ? args.bias[c] : -0.0f;
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int64_t col = col_base + col_block<NJ>(wn, j) * 32;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v[4], pv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = acc[i][j][4 * g + e] + bcol[j];
            if (saves_pre(EPI)) pv[e] = v[e];
            if (is_gelu(EPI)) v[e] = gelu_bf16out(v[e]);
          }
          quad_transpose(v, q);
          const int64_t row = row_base + i * 32 + 8 * g + q;
          if (row < M && col < N)
            *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(outg) + row * N + col) =
                u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          if (saves_pre(EPI)) {
            quad_transpose(pv, q);
            if (row < M && col < N)
              *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(args.pre[blockIdx.y]) + row * N + col) =
                  u32x2{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])};
          }
        }
      }
  } else if (is_swiglu(EPI)) {
    const int64_t col_base = (int64_t)bn * (BN / 2) + hg * 64 + cq;
    // gate and up biases of this lane's output column of each pair (bias
    // holds the N gate biases, then the N up biases); -0 when there is none
    float bg[NP], bu[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int64_t o = (int64_t)bn * (BN / 2) + hg * 64 + pair_col(j) + l31;
      bg[j] = (args.bias && o < N) ? args.bias[o] : -0.0f;
      bu[j] = (args.bias && o < N) ? args.bias[N + o] : -0.0f;
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const int64_t col = col_base + pair_col(j);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v[4], pg[4], pu[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (saves_pre(EPI)) {
              pg[e] = acc[i][j][4 * g + e] + bg[j];
              pu[e] = acc[i][j + NP][4 * g + e] + bu[j];
            }
            v[e] = silu_fast(acc[i][j][4 * g + e] + bg[j]) * (acc[i][j + NP][4 * g + e] + bu[j]);
          }
          quad_transpose(v, q);
          const int64_t row = row_base + i * 32 + 8 * g + q;
          if (row < M && col < N)
            *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(outg) + row * N + col) =
                u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          if (saves_pre(EPI)) {
            quad_transpose(pg, q);
            quad_transpose(pu, q);
            bf16_t* pr = reinterpret_cast<bf16_t*>(args.pre[blockIdx.y]) + row * 2 * N + col;
            if (row < M && col < N) {
              *reinterpret_cast<u32x2*>(pr) = u32x2{pack_bf16x2(pg[0], pg[1]), pack_bf16x2(pg[2], pg[3])};
              *reinterpret_cast<u32x2*>(pr + N) = u32x2{pack_bf16x2(pu[0], pu[1]), pack_bf16x2(pu[2], pu[3])};
            }
          }
        }
      }
  } else {  // EPI_QKV: each 128-column group of the tile is exactly one head
    const QkvOut o = args.qkv;
    const int hd = bn * 2 + hg;
    const int nheads = o.hq + 2 * o.hkv;
    // V heads are transposed through LDS; every wave of the tile passes this
    // barrier (before any returns) so no wave still reads the k loop's stages
    __syncthreads();
    if (hd >= nheads) return;
    const uint32_t seq = (uint32_t)o.seq;
    // Rows 8 g4 + e, e = 0..3, of block i are 4 consecutive tokens.  One
    // division per lane gives (sequence, position) of the lane's first row;
    // a group's first token is that plus its row offset, wrapped.
    const uint32_t b_base = (uint32_t)(row_base / seq);
    const uint32_t p_base = (uint32_t)(row_base - (int64_t)b_base * seq);
    auto split_pos = [&](int off, uint32_t& b, uint32_t& p) {
      p = p_base + (uint32_t)off;
      b = b_base;
      if (p >= seq) {
        if ((uint32_t)off < seq) {
          p -= seq;
          ++b;
        } else {
          b += p / seq;
          p %= seq;
        }
      }
    };
    if (hd < o.hq + o.hkv) {
      const bool is_q = hd < o.hq;
      bf16_t* dst = reinterpret_cast<bf16_t*>(is_q ? o.q : o.k);
      const int64_t ld = (int64_t)(is_q ? o.hq : o.hkv) * 128;
      dst += (int64_t)(is_q ? hd : hd - o.hq) * 128;
      // angle = pos * base^(-2 c1 / 128) radians for the pair (c1, c1 + 64),
      // taken in turns (1 turn = 2 pi): v_sin/v_cos take turns.  The turns
      // per position are held as an unevaluated float sum f_hi + f_lo
      // (evaluated once per lane in float64), and pos * f_hi is split into
      // its rounded value and exact error by an FMA, so only the fraction of
      // a turn is rounded to float32, as if the product were taken in
      // float64.  The 4 rows of a group are consecutive positions: the
      // first angle is evaluated that way and the next three follow by
      // rotating it by one position's angle (angle addition), unless the
      // group crosses into the next sequence.
      // biases of the pair (c1, c1 + 64) of this lane, added before the rotation
      float hb1[NP], hb2[NP];
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const int64_t c = (int64_t)hd * 128 + pair_col(j) + l31;
        hb1[j] = args.bias ? args.bias[c] : -0.0f;
        hb2[j] = args.bias ? args.bias[c + 64] : -0.0f;
      }
      float f_hi[NP], f_lo[NP];
      float c1p[NP], s1p[NP];  // cos / sin of one position's angle
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const double fd = exp2(-(double)(2 * (pair_col(j) + l31)) * (1.0 / 128.0) * (double)o.log2_base) *
                          0.15915494309189533577;
        f_hi[j] = (float)fd;
        f_lo[j] = (float)(fd - (double)f_hi[j]);
        c1p[j] = __builtin_amdgcn_cosf(f_hi[j]);
        s1p[j] = __builtin_amdgcn_sinf(f_hi[j]);
      }
      auto angle = [&](uint32_t pos, int j, float& cs, float& sn) {
        const float pf = (float)pos;  // exact: positions are below 2^24
        const float a = pf * f_hi[j];
        const float err = fmaf(pf, f_hi[j], -a);
        const float frac = (a - floorf(a)) + fmaf(pf, f_lo[j], err);
        sn = __builtin_amdgcn_sinf(frac);
        cs = __builtin_amdgcn_cosf(frac);
      };
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int64_t row0 = row_base + i * 32 + 8 * g4;
          uint32_t b0, p0;
          split_pos(i * 32 + 8 * g4, b0, p0);
          const bool run = p0 + 3 < seq;  // the group stays inside one sequence
#pragma unroll
          for (int j = 0; j < NP; ++j) {
            float cs[4], sn[4];
            angle(p0, j, cs[0], sn[0]);
            if (run) {
#pragma unroll
              for (int e = 1; e < 4; ++e) {
                cs[e] = cs[e - 1] * c1p[j] - sn[e - 1] * s1p[j];
                sn[e] = sn[e - 1] * c1p[j] + cs[e - 1] * s1p[j];
              }
            } else {
#pragma unroll
              for (int e = 1; e < 4; ++e) {
                uint32_t bb, pos;
                split_pos(i * 32 + 8 * g4 + e, bb, pos);
                angle(pos, j, cs[e], sn[e]);
              }
            }
            float y1[4], y2[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x1 = acc[i][j][4 * g4 + e] + hb1[j], x2 = acc[i][j + NP][4 * g4 + e] + hb2[j];
              y1[e] = x1 * cs[e] - x2 * sn[e];
              y2[e] = x2 * cs[e] + x1 * sn[e];
            }
            quad_transpose(y1, q);
            quad_transpose(y2, q);
            const int64_t row = row0 + q;
            if (row < M) {
              bf16_t* line = dst + row * ld + pair_col(j) + cq;
              *reinterpret_cast<u32x2*>(line) = u32x2{pack_bf16x2(y1[0], y1[1]), pack_bf16x2(y1[2], y1[3])};
              *reinterpret_cast<u32x2*>(line + 64) =
                  u32x2{pack_bf16x2(y2[0], y2[1]), pack_bf16x2(y2[2], y2[3])};
            }
          }
        }
    } else if ((seq & 7u) == 0) {
      // V head, stored transposed per sequence: Vt[b][g][c][p].  A lane holds
      // 4-row runs of one channel; written straight out that is one 8-byte
      // store per run, 64 channels apart across the wave.  Instead the wave's
      // block goes through its own LDS region as [channel][row] (rows padded
      // by 8 against bank conflicts), and is read back 8 rows of one channel
      // per lane, so each 16-byte store extends a contiguous run of a channel
      // row of Vt.  With seq a multiple of 8 (and tile rows at multiples of
      // 32) an 8-row chunk never straddles two sequences.  Passes of PI
      // 32-row blocks keep every wave's region inside the tile's LDS.
      constexpr int CH_W = NJ * 32;  // channels of the wave
      constexpr int PI = (NW * CH_W * (MI * 32 + 8) * 2 <= C::SMEM) ? MI
                         : (MI % 2 == 0 && NW * CH_W * (MI * 16 + 8) * 2 <= C::SMEM) ? MI / 2 : 1;
      constexpr int RP = PI * 32 + 8;  // padded row length of a channel in LDS
      static_assert(NW * CH_W * RP * 2 <= C::SMEM, "V staging region");
      constexpr int CPC = PI * 4;      // 8-row chunks per channel per pass
      const int g = hd - o.hq - o.hkv;
      bf16_t* vt = reinterpret_cast<bf16_t*>(o.vt);
      bf16_t* reg = reinterpret_cast<bf16_t*>(smem) + wave * CH_W * RP;
      float vb[NJ];  // bias of this lane's channel of each block
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        vb[j] = args.bias ? args.bias[(int64_t)hd * 128 + (col_block<NJ>(wn, j) & 3) * 32 + l31] : -0.0f;
      const int64_t wrow0 = m0 + wm * WROWS;  // the wave's first row (a multiple of 32)
      const uint32_t vb0 = (uint32_t)(wrow0 / seq), vp0 = (uint32_t)(wrow0 - (int64_t)vb0 * seq);
#pragma unroll
      for (int i0 = 0; i0 < MI; i0 += PI) {
        if (i0 > 0) wait_lgkmcnt0();  // the previous pass's reads are done
#pragma unroll
        for (int ii = 0; ii < PI; ++ii)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const u32x2 pr = {pack_bf16x2(acc[i0 + ii][j][4 * g4 + 0] + vb[j], acc[i0 + ii][j][4 * g4 + 1] + vb[j]),
                                pack_bf16x2(acc[i0 + ii][j][4 * g4 + 2] + vb[j], acc[i0 + ii][j][4 * g4 + 3] + vb[j])};
              *reinterpret_cast<u32x2*>(reg + (j * 32 + l31) * RP + ii * 32 + 8 * g4 + 4 * hk) = pr;
            }
        wait_lgkmcnt0();
#pragma unroll
        for (int it = 0; it < CH_W * CPC / 64; ++it) {
          const int idx = it * 64 + lane;
          const int cl = idx / CPC, k = idx % CPC;
          const u32x4 v = lds_read16(reg + cl * RP + 8 * k);
          const int off = (i0 * 32) + 8 * k;  // row offset within the wave
          if (wrow0 + off < M) {
            uint32_t b = vb0, p = vp0 + (uint32_t)off;
            if (p >= seq) {
              b += p / seq;
              p %= seq;
            }
            const int c = (col_block<NJ>(wn, cl >> 5) & 3) * 32 + (cl & 31);
            *reinterpret_cast<u32x4*>(vt + (((int64_t)b * o.hkv + g) * 128 + c) * o.seq_pad + p) = v;
          }
        }
      }
    } else {
      const int g = hd - o.hq - o.hkv;
      bf16_t* vt = reinterpret_cast<bf16_t*>(o.vt);
      const bool vec = (seq & 3u) == 0;  // groups of 4 never straddle sequences
      float vb[NJ];  // bias of this lane's channel of each block
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        vb[j] = args.bias ? args.bias[(int64_t)hd * 128 + (col_block<NJ>(wn, j) & 3) * 32 + l31] : -0.0f;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int64_t row0 = row_base + i * 32 + 8 * g4;
          if (row0 >= M) continue;
          uint32_t b0, p0;
          split_pos(i * 32 + 8 * g4, b0, p0);
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const int c = (col_block<NJ>(wn, j) & 3) * 32 + l31;
            if (vec && row0 + 3 < M) {
              bf16_t* line = vt + (((int64_t)b0 * o.hkv + g) * 128 + c) * o.seq_pad;
              const u32x2 pr = {pack_bf16x2(acc[i][j][4 * g4 + 0] + vb[j], acc[i][j][4 * g4 + 1] + vb[j]),
                                pack_bf16x2(acc[i][j][4 * g4 + 2] + vb[j], acc[i][j][4 * g4 + 3] + vb[j])};
              *reinterpret_cast<u32x2*>(line + p0) = pr;
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if (row0 + e >= M) continue;
                uint32_t b = b0, pos = p0 + e;
                if (pos >= seq) {
                  pos -= seq;
                  ++b;
                }
                vt[(((int64_t)b * o.hkv + g) * 128 + c) * o.seq_pad + pos] =
                    f32_to_bf16(acc[i][j][4 * g4 + e] + vb[j]);
              }
            }
          }
        }
    }
  }
}

// ---- 16 x 16 x 32 MFMA variant for deep k ---------------------------------
//
// The same 256-column tiles, two-stage LDS ring and four waves (2 x 2, one
// per SIMD, BMT / 2 x 128 each), but the wave's block is built from
// v_mfma_f32_16x16x32_bf16 instead of 32x32x16.  Under sustained load the
// board sits at its power limit and the clock is what the matrix work can
// afford: a long MFMA stream with the GEMM's fragment reads holds 1.66 GHz
// with 32x32x16 and 1.91 GHz with 16x16x32 on the same random bf16 data
// (1.70 vs 1.89 PFLOP/s), since the smaller instruction moves less
// accumulator data per flop.  The 16x16 stream costs a little more issue
// time per flop, which deep k loops amortise: at k = 8192 the SwiGLU GEMM of
// the 70B shard and an 8192^3 GEMM run 5-7% faster this way; at k = 3584 it
// is 1% slower, so shorter k stays on the 32x32 kernel.  Accumulation order
// and results are bitwise those of the 32x32 kernel.  Every epilogue runs
// here, Q/K/V + RoPE included (a wave's 128 columns are one head).
//
// Fragment of a 16-row block for k-step s: lane l reads row l % 16, 16-byte
// chunk 4 s + l / 16 of the 64-deep stage.  The LDS chunk permutation here
// depends on the row within its 16-row group only (swz16), which keeps the 16
// rows one read phase touches on distinct banks and makes block i's address
// the block-0 address plus 2048 i, an immediate offset: two address
// registers per operand instead of one per block.  A fragments are single
// buffered (A_i of the next k-step is read into its registers right after
// its last MFMA), B fragments double buffered.  Output block (i, j): lane l
// holds column l % 16 of rows 4 (l / 16) + e, e = 0..3.
constexpr int64_t MFMA16_MIN_K = 4096;
constexpr int CPOL_SC0_SC1 = 1 | 16;  // cache policy bits of a system-coherent buffer access

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ int swz16(int r) { return (r >> 1) & 7; }

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// LDS-DMA load issued from inline asm, for the kernels that read LDS with
// transposing reads.  The compiler assumes such a read may alias any LDS-DMA
// store it knows to be in flight and waits for all of them (vmcnt(0)) before
// each one, which drains the prefetch; loads issued here are not tracked by
// it, and the kernel's own waits before every barrier cover them.  The load
// writes LDS only (no register result), and M0, its LDS base, is set in the
// same statement.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_lds16_asm(__amdgpu_buffer_rsrc_t rsrc, void* lds_wave_base, uint32_t voffset,
                                              uint32_t soffset) {
  const uint32_t base = (uint32_t)(uintptr_t)LDS_PTR(lds_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(base), "v"(voffset), "s"(rsrc),
               "s"(soffset)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// KM: operand layouts.  0: x [M, K] and w [N, K] (k contiguous); 1: w stored
// k-major, [K, N]; 2: x [K, M] and w [K, N] both k-major.  A k-major tile
// sits in LDS as groups of 8 k rows, each group as the tile's 16-row blocks
// of 8 x 32 bytes: one DMA instruction fills 4 blocks x 8 k rows from 8
// global segments of 128 bytes, and fragments come from pairs of transposing
// reads (ds_read_b64_tr_b16: 16 lanes give 4 k rows x 16 rows, each lane
// gets one row's 4 k values).  The MFMA's k slots run through the 32 k of a
// step in the order 8 g + 4 h + t -> 16 (g >> 1) + 8 h + 4 (g & 1) + t (lane
// group g, read h, t < 4), the same for both operands, so each half wave
// reads 8 consecutive k rows of a block (256 contiguous bytes: no bank
// conflicts) and block, step and read offsets are immediates.  A
// k-contiguous x beside a k-major w takes the same order with 8-byte reads.
template <int EPI, int BMT, int KM = 0>
__global__ __launch_bounds__(256, 1) void gemm16_kernel(Args args) {
  constexpr bool KA = KM == 2, KB = KM >= 1;
  static_assert(!KB || (EPI == EPI_F32 || EPI == EPI_BF16), "k-major operands: plain epilogues");
  constexpr int NW = 4;
  constexpr int WROWS = BMT / 2;  // 2 x 2 waves
  constexpr int MI = WROWS / 16;  // 16-row blocks per wave
  constexpr int NJ = 8;           // 16-column blocks per wave (128 columns)
  constexpr int KS = BK / 32;     // MFMA k-steps per stage
  constexpr int A_TILE = BMT * ROWB;
  constexpr int SMEM = NSTAGE * (A_TILE + B_TILE);
  constexpr int B_BASE = NSTAGE * A_TILE;
  constexpr int A_INSTR = BMT * CH / 64;
  constexpr int LA = A_INSTR / NW, LB = B_INSTR / NW;
  static_assert(A_INSTR % NW == 0 && B_INSTR % NW == 0 && SMEM <= 160 * 1024, "tile");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int lane = lane_id();
  const int wave = wave_id();
  const bf16_t* const xg = args.x[blockIdx.y];
  const bf16_t* const wg = args.w[blockIdx.y];
  void* const outg = args.out[blockIdx.y];
  // Split launches: launch index b works on tile 8 (b / 16) + b % 8, the
  // upper half of k when (b / 8) is even (the producer) and the lower half
  // otherwise, so a tile's two workgroups sit on the same XCD (b and b + 8)
  // and tile_coords sees tile ids in their XCD's order; the grid is 16 per 8
  // tiles and the ids past the last tile have nothing to do.
  const bool split = args.sk_ws != nullptr;
  const bool producer = split && ((blockIdx.x >> 3) & 1) == 0;
  const int ntiles = args.num_bm * args.num_bn;
  const int tile_id = split ? (int)((blockIdx.x >> 4) * 8 + (blockIdx.x & 7)) : (int)blockIdx.x;
  if (tile_id >= ntiles) return;
  int bm, bn;
  tile_coords(tile_id, ntiles, args.num_bm, args.num_bn, bm, bn);
  bm = __builtin_amdgcn_readfirstlane(bm);
  bn = __builtin_amdgcn_readfirstlane(bn + args.bn0);
  const int64_t M = args.M, N = args.N, K = args.K, lda = args.lda;
  const int64_t m0 = (int64_t)bm * BMT;
  const uint32_t row_bytes = (uint32_t)(K * 2);
  const uint32_t a_row_bytes = (uint32_t)(lda * 2);
  const int m_rows = (int)min<int64_t>(BMT, M - m0);
  __amdgpu_buffer_rsrc_t rsrc_a = KA ? make_rsrc(xg, (uint32_t)(K * lda * 2))
                                     : make_rsrc(xg + m0 * lda, (uint32_t)m_rows * a_row_bytes);
  __amdgpu_buffer_rsrc_t rsrc_b;
  int n_valid;  // valid weight rows (plain) or valid output columns (SwiGLU)
  if (is_swiglu(EPI)) {
    const int64_t o0 = (int64_t)bn * (BN / 2);
    n_valid = (int)min<int64_t>(BN / 2, N - o0);
    rsrc_b = make_rsrc(wg + o0 * K, (uint32_t)((N + n_valid) * K * 2));
  } else if (KB) {
    n_valid = (int)min<int64_t>(BN, N - (int64_t)bn * BN);
    rsrc_b = make_rsrc(wg, (uint32_t)(K * args.ldb * 2));
  } else {
    const int64_t n0 = (int64_t)bn * BN;
    n_valid = (int)min<int64_t>(BN, N - n0);
    rsrc_b = make_rsrc(wg + n0 * K, (uint32_t)n_valid * row_bytes);
  }
  // k-major operands: a stage moves 64 k rows of its tile, BK * ld * 2 bytes
  const uint32_t a_step = KA ? (uint32_t)(BK * lda * 2) : (uint32_t)(BK * 2);
  const uint32_t b_step = KB ? (uint32_t)(BK * args.ldb * 2) : (uint32_t)(BK * 2);

  // global -> LDS: wave-instruction blk of a stage fills tile row slot / CH,
  // physical chunk slot % CH, from logical chunk (slot % CH) ^ swz16(row).
  // SwiGLU tiles hold gate rows o .. o + 63, then the matching up rows, for
  // each 64-output half (the same interleave as the 32x32 kernel).
  uint32_t a_off[LA], b_off[LB];
  int a_k[LA], b_k[LB];
  // k-major tile of R rows: instruction q covers k rows 8 (q / (R / 64)) ..
  // + 7 of the 16-row blocks 4 (q % (R / 64)) .. + 3; lane L reads block
  // + L / 16, k row (L % 16) / 2, 8 columns from 8 (L % 2).  The k row is
  // returned in *kk; the offset is TP_OOB_OFFSET past the valid columns.
  auto km_off = [&](int q, int R, int64_t col0, int64_t ncol, int64_t ld, int* kk) -> uint32_t {
    const int kg = q / (R / 64), b4 = q % (R / 64);
    const int blk = 4 * b4 + (lane >> 4), krow = kg * 8 + ((lane & 15) >> 1);
    const int64_t col = 16 * blk + 8 * (lane & 1);
    *kk = krow;
    return col < ncol ? (uint32_t)(krow * ld * 2 + (col0 + col) * 2) : TP_OOB_OFFSET;
  };
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    const int slot = (j * NW + wave) * 64 + lane;
    if (KA) {
      a_off[j] = km_off(j * NW + wave, BMT, m0, m_rows, lda, &a_k[j]);
      continue;
    }
    const int r = slot / CH;
    const int c = (slot % CH) ^ swz16(r);
    a_k[j] = c * 8;
    a_off[j] = (uint32_t)r * a_row_bytes + (uint32_t)c * 16;
  }
#pragma unroll
  for (int j = 0; j < LB; ++j) {
    const int slot = (j * NW + wave) * 64 + lane;
    if (KB) {
      b_off[j] = km_off(j * NW + wave, BN, (int64_t)bn * BN, n_valid, args.ldb, &b_k[j]);
      continue;
    }
    const int r = slot / CH;
    const int c = (slot % CH) ^ swz16(r);
    b_k[j] = c * 8;
    if (is_swiglu(EPI)) {
      const int half = r >> 7, qq = r & 127;
      const int o_rel = half * 64 + (qq & 63);
      const int64_t rel_row = (qq < 64) ? o_rel : N + o_rel;
      b_off[j] = (o_rel < n_valid) ? (uint32_t)(rel_row * K * 2) + (uint32_t)c * 16 : TP_OOB_OFFSET;
    } else {
      b_off[j] = (uint32_t)r * row_bytes + (uint32_t)c * 16;
    }
  }
  // (k-major variants: every load from inline asm, see dma_lds16_asm)
  auto dma = [&](__amdgpu_buffer_rsrc_t r, char* dst, uint32_t voff, uint32_t soff) {
    if constexpr (KM != 0) dma_lds16_asm(r, dst, voff, soff);
    else if (soff) buffer_load_lds16_so(r, dst, voff, soff);
    else buffer_load_lds16(r, dst, voff);
  };
  auto load_a = [&](auto stage_tag, auto full_tag, int kn, int j) {
    constexpr int S = decltype(stage_tag)::value;
    char* const dst = smem + S * A_TILE + (j * NW + wave) * 1024;
    const uint32_t kb = (uint32_t)kn * a_step;
    if (decltype(full_tag)::value) {
      if constexpr (KM != 0) dma_lds16_asm(rsrc_a, dst, a_off[j], kb);
      else buffer_load_lds16_so(rsrc_a, dst, a_off[j], kb);
    } else {
      dma(rsrc_a, dst,
          ((int64_t)kn * BK + a_k[j]) < K && a_off[j] != TP_OOB_OFFSET ? a_off[j] + kb : TP_OOB_OFFSET, 0u);
    }
  };
  auto load_b = [&](auto stage_tag, auto full_tag, int kn, int j) {
    constexpr int S = decltype(stage_tag)::value;
    char* const dst = smem + B_BASE + S * B_TILE + (j * NW + wave) * 1024;
    const uint32_t kb = (uint32_t)kn * b_step;
    if (decltype(full_tag)::value) {
      if constexpr (KM != 0) dma_lds16_asm(rsrc_b, dst, b_off[j], kb);
      else buffer_load_lds16_so(rsrc_b, dst, b_off[j], kb);
    } else {
      dma(rsrc_b, dst,
          ((int64_t)kn * BK + b_k[j]) < K && b_off[j] != TP_OOB_OFFSET ? b_off[j] + kb : TP_OOB_OFFSET, 0u);
    }
  };
  // load j (0 .. LA + LB - 1) of a stage: the A loads, then the B loads
  auto load_one = [&](auto stage_tag, auto full_tag, int kn, int j) {
    if (j < LA) load_a(stage_tag, full_tag, kn, j);
    else load_b(stage_tag, full_tag, kn, j - LA);
  };
  auto load_stage = [&](auto stage_tag, auto full_tag, int kn) {
#pragma unroll
    for (int j = 0; j < LA + LB; ++j) load_one(stage_tag, full_tag, kn, j);
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int l15 = lane & 15, kq = lane >> 4;
  uint32_t ra[KS], rb[KS];  // block 0's fragment address per k-step; block i at + 2048 i
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int c = 4 * s + kq;
    const int r_a = wm * WROWS + l15, r_b = wn * 128 + l15;
    ra[s] = (uint32_t)(r_a * ROWB + ((c ^ swz16(r_a)) << 4));
    rb[s] = (uint32_t)(B_BASE + r_b * ROWB + ((c ^ swz16(r_b)) << 4));
  }
  // k-major fragments: the lane's address in its block's group of 8 k rows
  // (half wave g >> 1 two groups further); + 256 per block, + (4 s + h) x
  // blocks x 256 per step s and read h.  A k-contiguous x beside a k-major w:
  // two 8-byte reads at k chunk 4 s + 2 (g >> 1) + h, bytes 8 (g & 1) on.
  const uint32_t tr_lane = (uint32_t)((4 * (kq & 1) + (l15 >> 2)) * 32 + 8 * (l15 & 3));
  const uint32_t ra_km = (uint32_t)((kq >> 1) * 2 * (BMT / 16) * 256 + wm * (WROWS / 16) * 256) + tr_lane;
  const uint32_t rb_km = (uint32_t)(B_BASE + (kq >> 1) * 2 * (BN / 16) * 256 + wn * 8 * 256) + tr_lane;
  uint32_t ra_pi[KS][2];
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r_a = wm * WROWS + l15;
      const int c = 4 * s + 2 * (kq >> 1) + h;
      ra_pi[s][h] = (uint32_t)(r_a * ROWB + ((c ^ swz16(r_a)) << 4) + 8 * (kq & 1));
    }
  f32x4 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{};
  u32x4 fa[MI], fb[2][NJ];
  auto tr_pair = [](const char* p0, const char* p1) {
    typedef __attribute__((address_space(3))) v4i16_t* lds_v4;
    const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4)(LDS_PTR(p0))));
    const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4)(LDS_PTR(p1))));
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  auto rd_a = [&](const char* a, int s, int i) {
    if constexpr (KA) {
      const char* p = a + ra_km + 256 * i + 4 * s * (BMT / 16) * 256;
      fa[i] = tr_pair(p, p + (BMT / 16) * 256);
    } else if constexpr (KB) {
      const u32x2 lo = lds_read8(a + ra_pi[s][0] + 2048 * i), hi = lds_read8(a + ra_pi[s][1] + 2048 * i);
      fa[i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    } else {
      fa[i] = lds_read16(a + ra[s] + 2048 * i);
    }
  };
  auto rd_b = [&](const char* b, int s, int j) {
    if constexpr (KB) {
      const char* p = b + rb_km + 256 * j + 4 * s * (BN / 16) * 256;
      fb[s & 1][j] = tr_pair(p, p + (BN / 16) * 256);
    } else {
      fb[s & 1][j] = lds_read16(b + rb[s] + 2048 * j);
    }
  };

  const int nfull = (int)(K / BK);  // k-steps without a k tail
  // this workgroup's k-steps [kb, ke)
  const int kb = split && producer ? args.sk_half : 0;
  const int ke = split && !producer ? args.sk_half : (int)((K + BK - 1) / BK);
  using Full = std::true_type;
  using Partial = std::false_type;
  constexpr std::integral_constant<int, 0> st0{};
  constexpr std::integral_constant<int, 1> st1{};
  // Per k-step of 64: KS substeps of MI x NJ MFMAs.  The one barrier sits
  // NRD MFMAs before the end of the last substep: every read of this stage
  // is done and the next stage has landed, so the remaining MFMAs carry the
  // next stage's first fragment reads (A blocks already finished, then the
  // B blocks, then each remaining A block after its last use).  The loads of
  // the stage after next go out after the barrier that frees its buffer: a
  // few spread over the rest of that substep, the others one every few MFMAs
  // over the next step's first substep, leaving its second substep for the
  // last of them to land.
  constexpr int NMF = MI * NJ, NRD = MI + NJ, BPOS = NMF - NRD;
  constexpr int NLD = LA + LB;
  constexpr int NST = MI == 8 ? 4 : NRD / 2;       // loads after the barrier ...
  constexpr int SPB = MI == 8 ? 4 : 2;             // ... one every SPB MFMAs
  constexpr int NC0 = NLD - NST;                    // loads in the first substep ...
  constexpr int SP0 = MI == 8 ? 5 : NMF / NC0;      // ... one every SP0 MFMAs
  constexpr int IB = BPOS / NJ;                     // A blocks finished before the barrier
  static_assert(KS == 2 && BPOS > 0 && NST * SPB <= NRD && NC0 > 0 && NC0 * SP0 <= NMF, "schedule");
  auto kstep = [&](auto stage_tag, auto main_tag, int kt) {
    constexpr int S = decltype(stage_tag)::value;
    constexpr bool MAIN = decltype(main_tag)::value;
    constexpr std::integral_constant<int, 1 - S> other_tag{};
    const char* const a_st = smem + S * A_TILE;
    const char* const b_st = smem + S * B_TILE;  // rb holds the B base
    const char* const a_nx = smem + (1 - S) * A_TILE;
    const char* const b_nx = smem + (1 - S) * B_TILE;
    const bool cont = MAIN || (kt > kb && kt + 1 < ke);  // rest of step kt + 1's loads
    const bool cont_full = MAIN || kt + 1 < nfull;
    const bool start = MAIN || kt + 2 < ke;              // first loads of step kt + 2
    const bool start_full = MAIN || kt + 2 < nfull;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int q = 0; q < NMF; ++q) {
        const int i = q / NJ, j = q % NJ;
        if (s == KS - 1 && q == BPOS) {
          wait_vmcnt0();
          wait_lgkmcnt0();
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
        acc[i][j] = mfma16x16x32(fa[i], fb[s][j], acc[i][j]);
        if (s + 1 < KS) {
          if (q % MI == MI / 2) rd_b(b_st, s + 1, q / MI);
          if (j == NJ - 1) rd_a(a_st, s + 1, i);
        } else if (q >= BPOS) {
          const int r = q - BPOS;
          if (r < IB) rd_a(a_nx, 0, r);
          if (i >= IB && j == NJ - 1) rd_a(a_nx, 0, i);
          if (r >= MI && r - MI < NJ) rd_b(b_nx, 0, r - MI);
        }
        if (s == 0 && cont && (q + 1) % SP0 == 0 && (q + 1) / SP0 - 1 < NC0) {
          const int jj = NST + (q + 1) / SP0 - 1;
          if (cont_full) load_one(other_tag, Full{}, kt + 1, jj);
          else load_one(other_tag, Partial{}, kt + 1, jj);
        }
        if (s == KS - 1 && q >= BPOS && (q - BPOS) % SPB == SPB - 1 && (q - BPOS) / SPB < NST && start) {
          const int jj = (q - BPOS) / SPB;
          if (start_full) load_one(stage_tag, Full{}, kt + 2, jj);
          else load_one(stage_tag, Partial{}, kt + 2, jj);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  if (kb < nfull) load_stage(st0, Full{}, kb);
  else load_stage(st0, Partial{}, kb);
  if (kb + 1 < ke) {
    if (kb + 1 < nfull) load_stage(st1, Full{}, kb + 1);
    else load_stage(st1, Partial{}, kb + 1);
    wait_vmcnt<LA + LB>();  // stage 0 landed, stage 1 may still be in flight
  } else {
    wait_vmcnt0();
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < MI; ++i) rd_a(smem, 0, i);
#pragma unroll
  for (int j = 0; j < NJ; ++j) rd_b(smem, 0, j);
  kstep(st0, Partial{}, kb);
  if (kb + 1 < ke) kstep(st1, Partial{}, kb + 1);
  int kt = kb + 2;
  const int kmain = min(nfull, ke);
  for (; kt + 3 < kmain; kt += 2) {
    kstep(st0, Full{}, kt);
    kstep(st1, Full{}, kt + 1);
  }
  for (; kt < ke; kt += 2) {
    kstep(st0, Partial{}, kt);
    if (kt + 1 < ke) kstep(st1, Partial{}, kt + 1);
  }
  wait_vmcnt0();

  if (split) {
    // The partial of k-steps [sk_half, nk) crosses workgroups (and XCDs):
    // it is written and read with system-coherent accesses (sc0 sc1: past
    // the non-coherent L2s), lane by lane in accumulator order, and the flag
    // goes up only after every wave's stores have completed.
    constexpr int NBLK = MI * NJ;
    __amdgpu_buffer_rsrc_t ws =
        make_rsrc(args.sk_ws + (size_t)tile_id * (BMT * BN), (uint32_t)(BMT * BN * sizeof(float)));
    unsigned* const flag = args.sk_flag + tile_id;
    if (producer) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), ws,
                                                 (uint32_t)(((wave * NBLK + i * NJ + j) * 64 + lane) * 16), 0,
                                                 CPOL_SC0_SC1);
      wait_vmcnt0();
      __syncthreads();
      if (threadIdx.x == 0) __hip_atomic_store(flag, args.sk_epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    if (threadIdx.x == 0) {
      // the producer has the lower launch index (b - 8), so it was dispatched
      // first and never waits: this ends; the bound only guards against a
      // broken launch (the result would then be wrong, not hung)
      for (uint32_t n = 0; n < (1u << 22); ++n) {
        if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == args.sk_epoch) break;
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
    // one row of blocks (NJ loads) in flight at a time: all of them at once
    // would need 4 x MI x NJ more registers than the kernel has
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      u32x4 v[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        v[j] = __builtin_amdgcn_raw_buffer_load_b128(ws, (uint32_t)(((wave * NBLK + i * NJ + j) * 64 + lane) * 16), 0,
                                                     CPOL_SC0_SC1);
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] += __builtin_bit_cast(f32x4, v[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- epilogue: a quad transpose gives each lane 4 consecutive columns of
  // one row (rows 4 kq + q of each block, q = lane & 3)
  const int64_t row_base = m0 + wm * WROWS + 4 * kq;
  const int q = lane & 3;
  const int cq = 4 * (l15 >> 2);
  if constexpr (EPI == EPI_F32) {
    // float32 partials, stored non-temporally (next read by the shard-sum)
    const int64_t col_base = (int64_t)bn * BN + wn * 128 + cq;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
        quad_transpose(v, q);
        const int64_t row = row_base + i * 16 + q;
        const int64_t col = col_base + j * 16;
        if (row < M && col < N)
          __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]},
                                      reinterpret_cast<f32x4*>(reinterpret_cast<float*>(outg) + row * N + col));
      }
  } else if constexpr (EPI == EPI_BF16 || is_gelu(EPI)) {
    const int64_t col_base = (int64_t)bn * BN + wn * 128 + cq;
    float bcol[NJ];  // bias of the lane's column of each block (-0: none)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t c = (int64_t)bn * BN + wn * 128 + 16 * j + l15;
      bcol[j] = (args.bias && c < N) ? args.bias[c] : -0.0f;
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        float v[4], pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = acc[i][j][e] + bcol[j];
          if (saves_pre(EPI)) pv[e] = v[e];
          if (is_gelu(EPI)) v[e] = gelu_bf16out(v[e]);
        }
        quad_transpose(v, q);
        const int64_t row = row_base + i * 16 + q;
        const int64_t col = col_base + j * 16;
        if (row < M && col < N)
          *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(outg) + row * N + col) =
              u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        if (saves_pre(EPI)) {
          quad_transpose(pv, q);
          if (row < M && col < N)
            *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(args.pre[blockIdx.y]) + row * N + col) =
                u32x2{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])};
        }
      }
  } else if constexpr (EPI == EPI_QKV) {
    // One wave's 128 columns are one head (hd): Q and K heads rotated (the
    // pair (c1, c1 + 64) is blocks j and j + 4 of a lane), V heads stored
    // transposed per sequence.  The RoPE angles follow the 32x32 kernel's
    // epilogue (turns as an unevaluated float sum, rows of a lane's 4-row
    // group by angle addition).
    const QkvOut o = args.qkv;
    const int hd = bn * 2 + wn;
    const int nheads = o.hq + 2 * o.hkv;
    // V heads are transposed through LDS; every wave of the tile passes this
    // barrier (before any returns) so no wave still reads the k loop's stages
    __syncthreads();
    if (hd >= nheads) return;
    const uint32_t seq = (uint32_t)o.seq;
    const uint32_t b_base = (uint32_t)(row_base / seq);
    const uint32_t p_base = (uint32_t)(row_base - (int64_t)b_base * seq);
    auto split_pos = [&](int off, uint32_t& b, uint32_t& p) {
      p = p_base + (uint32_t)off;
      b = b_base;
      if (p >= seq) {
        if ((uint32_t)off < seq) {
          p -= seq;
          ++b;
        } else {
          b += p / seq;
          p %= seq;
        }
      }
    };
    if (hd < o.hq + o.hkv) {
      const bool is_q = hd < o.hq;
      bf16_t* dst = reinterpret_cast<bf16_t*>(is_q ? o.q : o.k);
      const int64_t ld = (int64_t)(is_q ? o.hq : o.hkv) * 128;
      dst += (int64_t)(is_q ? hd : hd - o.hq) * 128;
      float hb1[4], hb2[4], f_hi[4], f_lo[4], c1p[4], s1p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c1 = 16 * j + l15;
        hb1[j] = args.bias ? args.bias[(int64_t)hd * 128 + c1] : -0.0f;
        hb2[j] = args.bias ? args.bias[(int64_t)hd * 128 + c1 + 64] : -0.0f;
        const double fd = exp2(-(double)(2 * c1) * (1.0 / 128.0) * (double)o.log2_base) * 0.15915494309189533577;
        f_hi[j] = (float)fd;
        f_lo[j] = (float)(fd - (double)f_hi[j]);
        c1p[j] = __builtin_amdgcn_cosf(f_hi[j]);
        s1p[j] = __builtin_amdgcn_sinf(f_hi[j]);
      }
      auto angle = [&](uint32_t pos, int j, float& cs, float& sn) {
        const float pf = (float)pos;  // exact: positions are below 2^24
        const float a = pf * f_hi[j];
        const float err = fmaf(pf, f_hi[j], -a);
        const float frac = (a - floorf(a)) + fmaf(pf, f_lo[j], err);
        sn = __builtin_amdgcn_sinf(frac);
        cs = __builtin_amdgcn_cosf(frac);
      };
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        uint32_t b0, p0;
        split_pos(i * 16, b0, p0);
        const bool run = p0 + 3 < seq;  // the group stays inside one sequence
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float cs[4], sn[4];
          angle(p0, j, cs[0], sn[0]);
          if (run) {
#pragma unroll
            for (int e = 1; e < 4; ++e) {
              cs[e] = cs[e - 1] * c1p[j] - sn[e - 1] * s1p[j];
              sn[e] = sn[e - 1] * c1p[j] + cs[e - 1] * s1p[j];
            }
          } else {
#pragma unroll
            for (int e = 1; e < 4; ++e) {
              uint32_t bb, pos;
              split_pos(i * 16 + e, bb, pos);
              angle(pos, j, cs[e], sn[e]);
            }
          }
          float y1[4], y2[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x1 = acc[i][j][e] + hb1[j], x2 = acc[i][j + 4][e] + hb2[j];
            y1[e] = x1 * cs[e] - x2 * sn[e];
            y2[e] = x2 * cs[e] + x1 * sn[e];
          }
          quad_transpose(y1, q);
          quad_transpose(y2, q);
          const int64_t row = row_base + i * 16 + q;
          if (row < M) {
            bf16_t* line = dst + row * ld + 16 * j + cq;
            *reinterpret_cast<u32x2*>(line) = u32x2{pack_bf16x2(y1[0], y1[1]), pack_bf16x2(y1[2], y1[3])};
            *reinterpret_cast<u32x2*>(line + 64) = u32x2{pack_bf16x2(y2[0], y2[1]), pack_bf16x2(y2[2], y2[3])};
          }
        }
      }
    } else {
      // V head, stored transposed per sequence: Vt[b][g][c][p].  A lane
      // holds 4-row runs of one channel; through the wave's own LDS region
      // as [channel][row] (rows padded by 8), read back 8 rows of a channel
      // per lane, each 16-byte store extends a run of a channel row of Vt.
      // With seq a multiple of 8 an 8-row chunk never straddles two
      // sequences; passes of PI 16-row blocks keep the regions in the LDS.
      const int g = hd - o.hq - o.hkv;
      bf16_t* vt = reinterpret_cast<bf16_t*>(o.vt);
      float vb[8];  // bias of this lane's channel of each block
#pragma unroll
      for (int j = 0; j < 8; ++j) vb[j] = args.bias ? args.bias[(int64_t)hd * 128 + 16 * j + l15] : -0.0f;
      if ((seq & 7u) == 0) {
        constexpr int PI = (NW * 128 * (MI * 16 + 8) * 2 <= SMEM) ? MI : MI / 2;
        constexpr int RP = PI * 16 + 8;  // padded row length of a channel in LDS
        static_assert(MI % PI == 0 && NW * 128 * RP * 2 <= SMEM, "V staging region");
        constexpr int CPC = PI * 2;      // 8-row chunks per channel per pass
        bf16_t* reg = reinterpret_cast<bf16_t*>(smem) + wave * 128 * RP;
        const int64_t wrow0 = m0 + wm * WROWS;  // the wave's first row (a multiple of 8)
        const uint32_t vb0 = (uint32_t)(wrow0 / seq), vp0 = (uint32_t)(wrow0 - (int64_t)vb0 * seq);
#pragma unroll
        for (int i0 = 0; i0 < MI; i0 += PI) {
          if (i0 > 0) wait_lgkmcnt0();  // the previous pass's reads are done
#pragma unroll
          for (int ii = 0; ii < PI; ++ii)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const u32x2 pr = {pack_bf16x2(acc[i0 + ii][j][0] + vb[j], acc[i0 + ii][j][1] + vb[j]),
                                pack_bf16x2(acc[i0 + ii][j][2] + vb[j], acc[i0 + ii][j][3] + vb[j])};
              *reinterpret_cast<u32x2*>(reg + (16 * j + l15) * RP + ii * 16 + 4 * kq) = pr;
            }
          wait_lgkmcnt0();
#pragma unroll
          for (int it = 0; it < 128 * CPC / 64; ++it) {
            const int idx = it * 64 + lane;
            const int cl = idx / CPC, kk = idx % CPC;
            const u32x4 v = lds_read16(reg + cl * RP + 8 * kk);
            const int off = i0 * 16 + 8 * kk;  // row offset within the wave
            if (wrow0 + off < M) {
              uint32_t b = vb0, p = vp0 + (uint32_t)off;
              if (p >= seq) {
                b += p / seq;
                p %= seq;
              }
              *reinterpret_cast<u32x4*>(vt + (((int64_t)b * o.hkv + g) * 128 + cl) * o.seq_pad + p) = v;
            }
          }
        }
      } else {
        const bool vec = (seq & 3u) == 0;  // groups of 4 never straddle sequences
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const int64_t row0 = row_base + i * 16;
          if (row0 >= M) continue;
          uint32_t b0, p0;
          split_pos(i * 16, b0, p0);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int c = 16 * j + l15;
            if (vec && row0 + 3 < M) {
              bf16_t* line = vt + (((int64_t)b0 * o.hkv + g) * 128 + c) * o.seq_pad;
              const u32x2 pr = {pack_bf16x2(acc[i][j][0] + vb[j], acc[i][j][1] + vb[j]),
                                pack_bf16x2(acc[i][j][2] + vb[j], acc[i][j][3] + vb[j])};
              *reinterpret_cast<u32x2*>(line + p0) = pr;
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if (row0 + e >= M) continue;
                uint32_t b = b0, pos = p0 + e;
                if (pos >= seq) {
                  pos -= seq;
                  ++b;
                }
                vt[(((int64_t)b * o.hkv + g) * 128 + c) * o.seq_pad + pos] = f32_to_bf16(acc[i][j][e] + vb[j]);
              }
            }
          }
        }
      }
    }
  } else {  // SwiGLU: gate block j and up block j + 4 of a wave are the same 16 outputs
    const int64_t ocol0 = (int64_t)bn * (BN / 2) + wn * 64;
    float bg[4], bu[4];  // gate and up biases of the lane's output column (-0: none)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t o = ocol0 + 16 * j + l15;
      bg[j] = (args.bias && o < N) ? args.bias[o] : -0.0f;
      bu[j] = (args.bias && o < N) ? args.bias[N + o] : -0.0f;
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float v[4], pg[4], pu[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (saves_pre(EPI)) {
            pg[e] = acc[i][j][e] + bg[j];
            pu[e] = acc[i][j + 4][e] + bu[j];
          }
          v[e] = silu_fast(acc[i][j][e] + bg[j]) * (acc[i][j + 4][e] + bu[j]);
        }
        quad_transpose(v, q);
        const int64_t row = row_base + i * 16 + q;
        const int64_t col = ocol0 + 16 * j + cq;
        if (row < M && col < N)
          *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(outg) + row * N + col) =
              u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        if (saves_pre(EPI)) {
          quad_transpose(pg, q);
          quad_transpose(pu, q);
          bf16_t* pr = reinterpret_cast<bf16_t*>(args.pre[blockIdx.y]) + row * 2 * N + col;
          if (row < M && col < N) {
            *reinterpret_cast<u32x2*>(pr) = u32x2{pack_bf16x2(pg[0], pg[1]), pack_bf16x2(pg[2], pg[3])};
            *reinterpret_cast<u32x2*>(pr + N) = u32x2{pack_bf16x2(pu[0], pu[1]), pack_bf16x2(pu[2], pu[3])};
          }
        }
      }
  }
}

// ---- small tiles for launches that would leave most of the chip idle -----
//
// A GEMM whose large-tile plan runs in one partly filled round (the GPT-sized
// shard, 2048 x 1024 x 1024: 64 tiles of 128 x 256 on 256 CUs) leaves most
// CUs idle while each busy one streams its whole k range.  Here a tile is 64
// rows x 128 weight rows (SwiGLU: 64 outputs), four times as many tiles,
// worked by four waves in a 2 x 2 grid of 32 x 64 with
// v_mfma_f32_16x16x32_bf16 (two 16-row by four 16-column blocks per wave).
// Stages of 64 k (24 KiB) cycle through a four-slot LDS ring with one barrier
// per stage: after the barrier of stage kt every wave has finished reading
// stage kt - 1, so the loads of stage kt + 3 go out into its slot at once.
// Measured per stage (timestamps): ~1000 cycles against 256 of matrix work,
// the same with 32 or 256 busy CUs and with rings of 3 to 6 slots, while the
// same loads alone stream at ~58 B per cycle per CU (400 cycles a stage): the
// stage's LDS traffic (24 KiB of DMA writes, 48 KiB of fragment reads) and
// its barrier set the pace, not the memory behind it.  Fragment addressing,
// the chunk permutation (swz16) and the output layout are those of the 16x16
// kernel, and each output's sum runs over k in the same order with the same
// instruction, so results are bitwise those of the large tiles.  SwiGLU tiles
// hold, for each 32-output half, the 32 gate rows and then the 32 up rows, so
// gate block j and up block j + 2 of a wave are the same outputs in the same
// lane.
constexpr int SBM = 64;    // small tile rows
constexpr int SBN = 128;   // small tile weight rows
constexpr int SNS = 4;     // LDS ring slots
constexpr int SPD = SNS - 1;  // stages loaded ahead

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int EPI>
__global__ __launch_bounds__(256, 1) void gemm_small_kernel(Args args) {
  static_assert(EPI != EPI_QKV, "the QKV epilogue runs on the large tiles");
  constexpr int A_T = SBM * ROWB;
  constexpr int B_T = SBN * ROWB;
  constexpr int ST = A_T + B_T;
  constexpr int LA = SBM * CH / 64 / 4, LB = SBN * CH / 64 / 4;  // wave-instructions per wave and stage
  static_assert(LA * 256 == SBM * CH && LB * 256 == SBN * CH && SNS * ST <= 160 * 1024, "tile");
  __shared__ __attribute__((aligned(1024))) char smem[SNS * ST];

  const int lane = lane_id();
  const int wave = wave_id();
  const bf16_t* const xg = args.x[blockIdx.y];
  const bf16_t* const wg = args.w[blockIdx.y];
  void* const outg = args.out[blockIdx.y];
  int bm, bn;
  tile_coords((int)blockIdx.x, args.num_bm * args.num_bn, args.num_bm, args.num_bn, bm, bn);
  bm = __builtin_amdgcn_readfirstlane(bm);
  bn = __builtin_amdgcn_readfirstlane(bn);
  const int64_t M = args.M, N = args.N, K = args.K, lda = args.lda;
  const int64_t m0 = (int64_t)bm * SBM;
  const uint32_t row_bytes = (uint32_t)(K * 2);
  const uint32_t a_row_bytes = (uint32_t)(lda * 2);
  const int m_rows = (int)min<int64_t>(SBM, M - m0);
  const __amdgpu_buffer_rsrc_t rsrc_a = make_rsrc(xg + m0 * lda, (uint32_t)m_rows * a_row_bytes);
  __amdgpu_buffer_rsrc_t rsrc_b;
  int n_valid;  // valid weight rows (plain) or valid output columns (SwiGLU)
  if (is_swiglu(EPI)) {
    const int64_t o0 = (int64_t)bn * (SBN / 2);
    n_valid = (int)min<int64_t>(SBN / 2, N - o0);
    rsrc_b = make_rsrc(wg + o0 * K, (uint32_t)((N + n_valid) * K * 2));
  } else {
    const int64_t n0 = (int64_t)bn * SBN;
    n_valid = (int)min<int64_t>(SBN, N - n0);
    rsrc_b = make_rsrc(wg + n0 * K, (uint32_t)n_valid * row_bytes);
  }

  // global -> LDS: wave-instruction j of an operand fills tile row slot / CH,
  // physical chunk slot % CH, from logical chunk (slot % CH) ^ swz16(row)
  uint32_t a_off[LA], b_off[LB];
  int a_k[LA], b_k[LB];
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    const int slot = (j * 4 + wave) * 64 + lane;
    const int r = slot / CH;
    const int c = (slot % CH) ^ swz16(r);
    a_k[j] = c * 8;
    a_off[j] = (uint32_t)r * a_row_bytes + (uint32_t)c * 16;
  }
#pragma unroll
  for (int j = 0; j < LB; ++j) {
    const int slot = (j * 4 + wave) * 64 + lane;
    const int r = slot / CH;
    const int c = (slot % CH) ^ swz16(r);
    b_k[j] = c * 8;
    if (is_swiglu(EPI)) {
      const int qq = r & 63;
      const int o_rel = (r >> 6) * 32 + (qq & 31);
      const int64_t rel_row = qq < 32 ? o_rel : N + o_rel;
      b_off[j] = o_rel < n_valid ? (uint32_t)(rel_row * K * 2) + (uint32_t)c * 16 : TP_OOB_OFFSET;
    } else {
      b_off[j] = (uint32_t)r * row_bytes + (uint32_t)c * 16;
    }
  }
  const int nk = (int)((K + BK - 1) / BK);
  const int nfull = (int)(K / BK);  // k-steps without a k tail
  // load j (0 .. LA + LB - 1) of stage kt: the A loads, then the B loads
  auto load_one = [&](int kt, int j) __attribute__((always_inline)) {
    char* const st = smem + (kt % SNS) * ST;
    const uint32_t kb = (uint32_t)kt * (uint32_t)(BK * 2);
    if (j < LA) {
      char* const dst = st + (j * 4 + wave) * 1024;
      if (kt < nfull) buffer_load_lds16_so(rsrc_a, dst, a_off[j], kb);
      else buffer_load_lds16(rsrc_a, dst, ((int64_t)kt * BK + a_k[j]) < K ? a_off[j] + kb : TP_OOB_OFFSET);
    } else {
      const int jb = j - LA;
      char* const dst = st + A_T + (jb * 4 + wave) * 1024;
      if (kt < nfull) buffer_load_lds16_so(rsrc_b, dst, b_off[jb], kb);
      else
        buffer_load_lds16(rsrc_b, dst,
                          ((int64_t)kt * BK + b_k[jb]) < K && b_off[jb] != TP_OOB_OFFSET ? b_off[jb] + kb
                                                                                          : TP_OOB_OFFSET);
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int l15 = lane & 15, kq = lane >> 4;
  // block 0's fragment address per 32-deep k-step s; block i at + 2048 i
  uint32_t ra[2], rb[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int c = (4 * s + kq) ^ swz16(l15);
    ra[s] = (uint32_t)((wm * 32 + l15) * ROWB + (c << 4));
    rb[s] = (uint32_t)(A_T + (wn * 64 + l15) * ROWB + (c << 4));
  }
  f32x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{};

  for (int kt = 0; kt < SPD && kt < nk; ++kt)
#pragma unroll
    for (int j = 0; j < LA + LB; ++j) load_one(kt, j);
  for (int kt = 0; kt < nk; ++kt) {
    // this wave's loads of stage kt have landed (those of the later stages
    // already issued may not), then every wave's have, and every wave is
    // done reading stage kt - 1
    static_assert(SPD <= 6, "the waits below");
    switch (min(nk - 1 - kt, SPD - 1)) {
      case 5: wait_vmcnt<5 * (LA + LB)>(); break;
      case 4: wait_vmcnt<4 * (LA + LB)>(); break;
      case 3: wait_vmcnt<3 * (LA + LB)>(); break;
      case 2: wait_vmcnt<2 * (LA + LB)>(); break;
      case 1: wait_vmcnt<LA + LB>(); break;
      default: wait_vmcnt0(); break;
    }
    lds_barrier();
    // the loads of stage kt + SPD at once (spread between the MFMAs they
    // were slower), then all 12 fragment reads of the stage and its 16 MFMAs
    const char* const st = smem + (kt % SNS) * ST;
    if (kt + SPD < nk) {
#pragma unroll
      for (int j = 0; j < LA + LB; ++j) load_one(kt + SPD, j);
    }
    u32x4 fa[2][2], fb[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[s][i] = lds_read16(st + ra[s] + 2048 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[s][j] = lds_read16(st + rb[s] + 2048 * j);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int s = q >> 3, i = (q >> 2) & 1, j = q & 3;
      acc[i][j] = mfma16x16x32(fa[s][i], fb[s][j], acc[i][j]);
    }
  }

  // ---- epilogue: after a quad transpose a lane holds 4 consecutive columns
  // of row 4 kq + q of each block
  const int64_t row_base = m0 + wm * 32 + 4 * kq;
  const int q = lane & 3;
  const int cq = 4 * (l15 >> 2);
  if constexpr (EPI == EPI_F32) {
    const int64_t col_base = (int64_t)bn * SBN + wn * 64 + cq;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
        quad_transpose(v, q);
        const int64_t row = row_base + i * 16 + q;
        const int64_t col = col_base + j * 16;
        if (row < M && col < N)
          __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]},
                                      reinterpret_cast<f32x4*>(reinterpret_cast<float*>(outg) + row * N + col));
      }
  } else if constexpr (EPI == EPI_BF16 || is_gelu(EPI)) {
    const int64_t col_base = (int64_t)bn * SBN + wn * 64 + cq;
    float bcol[4];  // bias of the lane's column of each block (-0: none)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t c = (int64_t)bn * SBN + wn * 64 + 16 * j + l15;
      bcol[j] = (args.bias && c < N) ? args.bias[c] : -0.0f;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float v[4], pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = acc[i][j][e] + bcol[j];
          if (saves_pre(EPI)) pv[e] = v[e];
          if (is_gelu(EPI)) v[e] = gelu_bf16out(v[e]);
        }
        quad_transpose(v, q);
        const int64_t row = row_base + i * 16 + q;
        const int64_t col = col_base + j * 16;
        if (row < M && col < N)
          *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(outg) + row * N + col) =
              u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        if (saves_pre(EPI)) {
          quad_transpose(pv, q);
          if (row < M && col < N)
            *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(args.pre[blockIdx.y]) + row * N + col) =
                u32x2{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])};
        }
      }
  } else {  // SwiGLU: gate block j and up block j + 2 of a wave are the same 16 outputs
    const int64_t ocol0 = (int64_t)bn * (SBN / 2) + wn * 32;
    float bg[2], bu[2];  // gate and up biases of the lane's output column (-0: none)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t o = ocol0 + 16 * j + l15;
      bg[j] = (args.bias && o < N) ? args.bias[o] : -0.0f;
      bu[j] = (args.bias && o < N) ? args.bias[N + o] : -0.0f;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float v[4], pg[4], pu[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (saves_pre(EPI)) {
            pg[e] = acc[i][j][e] + bg[j];
            pu[e] = acc[i][j + 2][e] + bu[j];
          }
          v[e] = silu_fast(acc[i][j][e] + bg[j]) * (acc[i][j + 2][e] + bu[j]);
        }
        quad_transpose(v, q);
        const int64_t row = row_base + i * 16 + q;
        const int64_t col = ocol0 + 16 * j + cq;
        if (row < M && col < N)
          *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(outg) + row * N + col) =
              u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        if (saves_pre(EPI)) {
          quad_transpose(pg, q);
          quad_transpose(pu, q);
          bf16_t* pr = reinterpret_cast<bf16_t*>(args.pre[blockIdx.y]) + row * 2 * N + col;
          if (row < M && col < N) {
            *reinterpret_cast<u32x2*>(pr) = u32x2{pack_bf16x2(pg[0], pg[1]), pack_bf16x2(pg[2], pg[3])};
            *reinterpret_cast<u32x2*>(pr + N) = u32x2{pack_bf16x2(pu[0], pu[1]), pack_bf16x2(pu[2], pu[3])};
          }
        }
      }
  }
}

// Zeroes the padding columns [seq, seq_pad) of every row of the transposed V,
// so attention over a partial last key tile reads zeros there.
__global__ void vt_pad_zero_kernel(bf16_t* vt, int64_t rows, int64_t seq, int64_t seq_pad) {
  const int64_t w = seq_pad - seq;
  const int64_t total = rows * w;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x)
    vt[(e / w) * seq_pad + seq + e % w] = 0;
}

}  // namespace

// ---- launch planning --------------------------------------------------------

namespace {

struct Plan {
  int bm_main, split, bm_tail;  // columns [0, split) at bm_main, [split, nbn) at bm_tail
  int split_k;                  // 2: columns [split, nbn) as split-k pairs of 256-row tiles
  int64_t cost;
};

// 256-row tiles switch from eight waves to four (one per SIMD) from this
// depth on: a short k loop leaves the four-wave tile's prologue and epilogue
// exposed (an o_proj of k = 1024 runs 6% slower on four waves, a down
// projection of k = 3584 as fast, k = 8192 5-7% faster).
constexpr int64_t W4_MIN_K = 2048;

int64_t rounds_of(int64_t tiles) { return (tiles + 255) / 256; }

// Cost of a launch ~ rounds of 256 workgroups x (BMT + 256): close to the
// load bound, a tile's time scales with the rows it streams.
int64_t cost(int64_t M, int64_t cols, int bmt, int groups) {
  if (cols <= 0) return 0;
  const int64_t tiles = ((M + bmt - 1) / bmt) * cols * groups;
  return rounds_of(tiles) * (bmt + 256);
}

// max_h: the tallest tile height allowed (256, or 192 for the k-major
// variants, whose 256-row tiles do not fit the register file: the allocator
// then shuffles accumulators through the k loop).
Plan plan_for(int64_t M, int64_t nbn, int groups, int max_h = 256) {
  static const int H[3] = {256, 192, 128};
  Plan best{max_h, (int)nbn, max_h, 0, 0};
  int64_t best_cost = cost(M, nbn, max_h, groups);
  for (int hm : H) {
    if (hm > max_h) continue;
    const int64_t one = cost(M, nbn, hm, groups);
    if (one < best_cost) {
      best_cost = one;
      best = Plan{hm, (int)nbn, hm, 0, 0};
    }
    for (int64_t split = 1; split < nbn; ++split)
      for (int ht : H) {
        if (ht >= hm) continue;  // a tail only at a lower height
        const int64_t c = cost(M, split, hm, groups) + cost(M, nbn - split, ht, groups);
        if (c < best_cost) {
          best_cost = c;
          best = Plan{hm, (int)split, ht, 0, 0};
        }
      }
  }
  best.cost = best_cost;
  return best;
}

// Split-k tail (single 16x16-kernel launches with bf16 outputs): the first
// tile columns on whole rounds of 256-row tiles, the last ones as pairs of
// workgroups that each sum half of k, when that round of half-depth
// 256-row tiles (cost 256 + 256 per pair of halves, i.e. 256 per workgroup
// round) beats the best plain plan.  At the 70B shard's SwiGLU GEMM (32 x 28
// tiles): 768 tiles on 3 rounds, then 128 tiles as 256 half-k workgroups,
// instead of the 4 tile columns as a round of 128-row tiles.
constexpr int SK_MAX_TILES = 128;

// Small tiles (64 rows x 128 weight rows) cost 64 + 128 per round on the
// same scale; they replace a plain plan they beat (bm_main = 64 then, with
// split = the small tile columns).  nbn_small = 0: not available (Q/K/V).
Plan with_small(Plan p, int64_t M, int64_t nbn_small, int groups) {
  if (p.split_k || nbn_small <= 0) return p;
  const int64_t c = rounds_of(((M + SBM - 1) / SBM) * nbn_small * groups) * (SBM + SBN);
  return c < p.cost ? Plan{SBM, (int)nbn_small, SBM, 0, c} : p;
}

Plan plan_with_split(int64_t M, int64_t nbn, int64_t K, int groups, bool bf16_out, int64_t nbn_small) {
  Plan p = plan_for(M, nbn, groups);
  const int64_t nk = (K + BK - 1) / BK;
  if (!bf16_out || groups != 1 || K < MFMA16_MIN_K || nk < 4) return with_small(p, M, nbn_small, groups);
  const int64_t nbm = (M + 255) / 256;
  for (int64_t c = nbn - 1; c >= 0; --c) {
    const int64_t main_t = nbm * c, tail_t = nbm * (nbn - c);
    if (2 * tail_t > 2 * SK_MAX_TILES || 2 * tail_t > 256) break;  // fewer main columns only add tail tiles
    if (main_t % 256 != 0) continue;
    const int64_t c_split = rounds_of(main_t) * (256 + 256) + 256;
    if (c_split < p.cost) p = Plan{256, (int)c, 256, 2, c_split};
    break;
  }
  return with_small(p, M, nbn_small, groups);
}

// Workspace of the split-k pairs: one float32 256 x 256 partial and one flag
// per tile, per (device, stream), allocated at the first split launch on that
// stream and kept until the process ends (calls on one stream are ordered;
// calls on different streams use different workspaces).  A flag holds the
// epoch of the launch that last raised it, so it is never cleared.
struct SkSlot {
  float* ws = nullptr;
  unsigned* flag = nullptr;
  unsigned epoch = 0;
};
std::mutex g_sk_mu;
std::map<std::pair<int, hipStream_t>, SkSlot> g_sk;

// The slot for this stream with its epoch advanced, or NULL when it cannot be
// allocated (the caller then runs the plain plan).
SkSlot* sk_acquire(hipStream_t s, unsigned* epoch) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(g_sk_mu);
  SkSlot& slot = g_sk[{dev, s}];
  if (!slot.ws) {
    constexpr size_t ws_bytes = (size_t)SK_MAX_TILES * 256 * BN * sizeof(float);
    void* p = nullptr;
    if (hipMalloc(&p, ws_bytes + SK_MAX_TILES * sizeof(unsigned)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    slot.ws = static_cast<float*>(p);
    slot.flag = reinterpret_cast<unsigned*>(static_cast<char*>(p) + ws_bytes);
    if (hipMemsetAsync(slot.flag, 0, SK_MAX_TILES * sizeof(unsigned), s) != hipSuccess) return nullptr;
  }
  *epoch = ++slot.epoch;
  if (*epoch == 0) *epoch = ++slot.epoch;  // 0 is the flags' initial value
  return &slot;
}

template <int EPI, int BMT>
void launch_part(Args a, int bn0, int cols, int groups, hipStream_t s) {
  a.bn0 = bn0;
  a.num_bn = cols;
  a.num_bm = (int)((a.M + BMT - 1) / BMT);
  const int nb = a.num_bm * cols;
  if (nb == 0) return;
  if (a.K >= MFMA16_MIN_K) {
    hipLaunchKernelGGL((gemm16_kernel<EPI, BMT>), dim3(a.sk_ws ? 16 * ((nb + 7) / 8) : nb, groups), dim3(256), 0, s,
                       a);
    return;
  }
  if (a.K >= W4_MIN_K) {
    hipLaunchKernelGGL((gemm_bf16_kernel<EPI, BMT, true>), dim3(nb, groups), dim3(Cfg<BMT, true>::NW * 64), 0, s, a);
    return;
  }
  hipLaunchKernelGGL((gemm_bf16_kernel<EPI, BMT, false>), dim3(nb, groups), dim3(Cfg<BMT>::NW * 64), 0, s, a);
}

// Small tile columns of an n-column output (0 for Q/K/V, which has no
// small-tile epilogue).
int64_t small_cols(int epi, int64_t N) {
  if (epi == EPI_QKV) return 0;
  const int64_t w = is_swiglu(epi) ? SBN / 2 : SBN;
  return (N + w - 1) / w;
}

template <int EPI>
void launch_planned(const Args& a, int64_t nbn, int groups, hipStream_t s) {
  constexpr bool BF16_OUT = EPI == EPI_BF16 || is_gelu(EPI) || is_swiglu(EPI);
  const Plan p = plan_with_split(a.M, nbn, a.K, groups, BF16_OUT, small_cols(EPI, a.N));
  if constexpr (EPI != EPI_QKV) {
    if (p.bm_main == SBM) {
      Args b = a;
      b.bn0 = 0;
      b.num_bn = p.split;
      b.num_bm = (int)((a.M + SBM - 1) / SBM);
      hipLaunchKernelGGL((gemm_small_kernel<EPI>), dim3(b.num_bm * b.num_bn, groups), dim3(256), 0, s, b);
      return;
    }
  }
  if constexpr (BF16_OUT) {
    unsigned epoch = 0;
    SkSlot* sk = p.split_k ? sk_acquire(s, &epoch) : nullptr;
    if (sk) {
      if (p.split > 0) launch_part<EPI, 256>(a, 0, p.split, 1, s);
      Args b = a;
      b.sk_ws = sk->ws;
      b.sk_flag = sk->flag;
      b.sk_epoch = epoch;
      b.sk_half = (int)((a.K + BK - 1) / BK / 2);
      launch_part<EPI, 256>(b, p.split, (int)(nbn - p.split), 1, s);
      return;
    }
  }
  auto part = [&](int bmt, int bn0, int cols) {
    switch (bmt) {
      case 256: launch_part<EPI, 256>(a, bn0, cols, groups, s); break;
      case 192: launch_part<EPI, 192>(a, bn0, cols, groups, s); break;
      default: launch_part<EPI, 128>(a, bn0, cols, groups, s); break;
    }
  };
  if (p.split_k) {  // no workspace: the plain plan
    const Plan q = plan_for(a.M, nbn, groups);
    part(q.bm_main, 0, q.split);
    if (q.split < nbn) part(q.bm_tail, q.split, (int)(nbn - q.split));
    return;
  }
  part(p.bm_main, 0, p.split);
  if (p.split < nbn) part(p.bm_tail, p.split, (int)(nbn - p.split));
}

template <int EPI, int KM>
void launch_km(Args a, int64_t nbn, hipStream_t s) {
  const Plan p = plan_for(a.M, nbn, 1, 192);
  auto part = [&](int bmt, int bn0, int cols) {
    a.bn0 = bn0;
    a.num_bn = cols;
    if (cols <= 0) return;
    switch (bmt) {
      case 192:
        a.num_bm = (int)((a.M + 191) / 192);
        hipLaunchKernelGGL((gemm16_kernel<EPI, 192, KM>), dim3(a.num_bm * cols), dim3(256), 0, s, a);
        break;
      default:
        a.num_bm = (int)((a.M + 127) / 128);
        hipLaunchKernelGGL((gemm16_kernel<EPI, 128, KM>), dim3(a.num_bm * cols), dim3(256), 0, s, a);
        break;
    }
  };
  part(p.bm_main, 0, p.split);
  part(p.bm_tail, p.split, (int)(nbn - p.split));
}

}  // namespace

hipError_t launch_gemm_bf16_km(int epi, bool x_kmajor, int64_t M, int64_t N, int64_t K, const void* x, int64_t ldx,
                               const void* w, int64_t ldw, void* out, hipStream_t s) {
  if (epi != EPI_F32 && epi != EPI_BF16) return hipErrorInvalidValue;
  Args a;
  for (int g = 0; g < MAX_GROUP; ++g) {
    a.x[g] = reinterpret_cast<const bf16_t*>(x);
    a.w[g] = reinterpret_cast<const bf16_t*>(w);
    a.out[g] = out;
    a.pre[g] = nullptr;
  }
  a.M = M;
  a.N = N;
  a.K = K;
  a.lda = ldx;
  a.ldb = ldw;
  a.bias = nullptr;
  a.num_bm = a.num_bn = a.bn0 = 0;
  a.sk_ws = nullptr;
  a.sk_flag = nullptr;
  a.sk_epoch = 0;
  a.sk_half = 0;
  a.qkv = QkvOut{};
  const int64_t nbn = (N + BN - 1) / BN;
  if (M == 0 || nbn == 0) return hipSuccess;
  if (epi == EPI_F32) {
    if (x_kmajor) launch_km<EPI_F32, 2>(a, nbn, s);
    else launch_km<EPI_F32, 1>(a, nbn, s);
  } else {
    if (x_kmajor) launch_km<EPI_BF16, 2>(a, nbn, s);
    else launch_km<EPI_BF16, 1>(a, nbn, s);
  }
  return hipGetLastError();
}

void gemm_plan(int64_t M, int64_t N, int64_t K, int kind, int groups, int* bm_main, int* split, int* bm_tail,
               int* split_k) {
  const bool swiglu = kind == GEMM_PLAN_SWIGLU;
  const int64_t nbn = (N + (swiglu ? BN / 2 : BN) - 1) / (swiglu ? BN / 2 : BN);
  const bool bf16_out = kind == GEMM_PLAN_COLWISE || kind == GEMM_PLAN_SWIGLU;
  const int epi = kind == GEMM_PLAN_QKV ? EPI_QKV : swiglu ? EPI_SWIGLU : EPI_BF16;
  const Plan p = plan_with_split(M, nbn, K, groups, bf16_out, small_cols(epi, N));
  *bm_main = p.bm_main;
  *split = p.split;
  *bm_tail = p.bm_tail;
  *split_k = p.split_k;
}

hipError_t launch_gemm_bf16_group(int epi, int groups, int64_t M, int64_t N, int64_t K,
                                  const void* const* x, const void* const* w, void* const* out,
                                  const QkvOut* qkv, hipStream_t s, const float* bias, int64_t lda,
                                  void* const* pre) {
  if (groups < 1 || groups > MAX_GROUP) return hipErrorInvalidValue;
  if ((epi == EPI_GELU_SAVE || epi == EPI_SWIGLU_SAVE) && !pre) return hipErrorInvalidValue;
  Args a;
  for (int g = 0; g < MAX_GROUP; ++g) {
    const int src = g < groups ? g : 0;
    a.x[g] = reinterpret_cast<const bf16_t*>(x[src]);
    a.w[g] = reinterpret_cast<const bf16_t*>(w[src]);
    a.out[g] = out[src];
    a.pre[g] = pre ? pre[src] : nullptr;
  }
  a.M = M;
  a.N = N;
  a.K = K;
  a.lda = lda > 0 ? lda : K;
  a.ldb = 0;
  a.bias = bias;
  a.num_bm = a.num_bn = a.bn0 = 0;
  a.sk_ws = nullptr;
  a.sk_flag = nullptr;
  a.sk_epoch = 0;
  a.sk_half = 0;
  if (qkv) a.qkv = *qkv; else a.qkv = QkvOut{};
  const int64_t bn_cols = is_swiglu(epi) ? BN / 2 : BN;
  const int64_t nbn = (N + bn_cols - 1) / bn_cols;
  if (M == 0 || nbn == 0) return hipSuccess;
  switch (epi) {
    case EPI_F32: launch_planned<EPI_F32>(a, nbn, groups, s); break;
    case EPI_BF16: launch_planned<EPI_BF16>(a, nbn, groups, s); break;
    case EPI_GELU: launch_planned<EPI_GELU>(a, nbn, groups, s); break;
    case EPI_SWIGLU: launch_planned<EPI_SWIGLU>(a, nbn, groups, s); break;
    case EPI_GELU_SAVE: launch_planned<EPI_GELU_SAVE>(a, nbn, groups, s); break;
    case EPI_SWIGLU_SAVE: launch_planned<EPI_SWIGLU_SAVE>(a, nbn, groups, s); break;
    case EPI_QKV: {
      if (groups != 1) return hipErrorInvalidValue;
      if (a.qkv.seq_pad > a.qkv.seq) {
        const int64_t rows = (M / a.qkv.seq) * a.qkv.hkv * 128;
        const int64_t total = rows * (a.qkv.seq_pad - a.qkv.seq);
        const int64_t blocks = total < 256 * 1024 ? (total + 255) / 256 : 1024;
        hipLaunchKernelGGL(vt_pad_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                           reinterpret_cast<bf16_t*>(a.qkv.vt), rows, a.qkv.seq, a.qkv.seq_pad);
      }
      launch_planned<EPI_QKV>(a, nbn, 1, s);
      break;
    }
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(int epi, int64_t M, int64_t N, int64_t K, const void* x, const void* w,
                            void* out, const QkvOut* qkv, hipStream_t s, const float* bias, int64_t lda,
                            void* pre) {
  const void* xs[1] = {x};
  const void* ws[1] = {w};
  void* os[1] = {out};
  void* ps[1] = {pre};
  return launch_gemm_bf16_group(epi, 1, M, N, K, xs, ws, os, qkv, s, bias, lda, pre ? ps : nullptr);
}

}  // namespace tpk
