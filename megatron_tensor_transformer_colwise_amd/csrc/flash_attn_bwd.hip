// Backward of the causal grouped-query flash attention for one rank's heads,
// gfx950, d = 128.
//
// "Tensor parallelism" page, sections "Self-attention" and "f and g": a rank's
// heads are independent in the backward pass too, so it differentiates its
// own a/t heads with no exchange; a KV head read by several of its query
// heads receives the sum of their gradients.
//
// With P = softmax(S) for S = Q K^T / sqrt(d) (causal), O = P V and the output
// gradient dO:
//   dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),   D = rowsum(dO * O),
//   dQ = dS K / sqrt(d),   dK = dS^T Q / sqrt(d).
// P is recomputed tile by tile from the forward's per-row log-sum-exp (log2
// units: P = exp2(s * log2(e) / sqrt(d) - lse)), never stored.
//
// Two kernels, no atomics (every sum has a fixed order):
//   dQ    one workgroup per (sequence, query head, 128 queries), 4 waves of 32
//         queries, the forward's structure: S^T = K Q^T and dP^T = V dO^T put a
//         query in each lane's column, so lse and D are per-lane scalars; then
//         dQ^T += K^T dS^T with dS^T as the B operand (bf16, one permlane32 swap
//         per 16 keys).  K, V (token-major) and K^T tiles of 64 keys stream
//         through LDS in two stages.
//   dK/dV one workgroup per (sequence, KV head, head split, 128 keys), 4 waves
//         of 32 keys: S = Q K^T and dP = dO V^T put a key in each lane's column
//         (K and V rows of the wave's keys stay in registers); then
//         dV^T += dO^T P and dK^T += Q^T dS.  Q, dO (token-major), Q^T, dO^T
//         tiles of 64 queries, with their lse and D values, stream through LDS
//         in two stages; a workgroup walks the query tiles of the query heads
//         of its split of the group one after the other and writes float32
//         partials, which a third kernel sums over the splits in order.
// The inverse RoPE rotation (the transpose of the forward's) is applied to dQ
// in the dQ kernel's epilogue and to dK in the sum kernel, so the outputs are
// the gradients of the projections before RoPE, packed as the QKV
// projection's output columns.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace tpk {
namespace {

constexpr int D = 128;
constexpr int NT = 256;
constexpr int ROW_TILE = 64 * D * 2;  // [64 tokens][128 d], 256-byte rows
constexpr int COL_TILE = D * 64 * 2;  // [128 d][64 tokens], 128-byte rows
constexpr int VEC_TILE = 1024;        // 64 float32 values (+ the zeros of idle lanes)
// LDS layouts, two stages each.  The row tiles of both stages sit in the first
// 64 KiB and the column tiles from 64 KiB on, so that every fragment read is
// a per-lane register (the column-tile offsets carry the 64 KiB) plus an
// immediate below 64 KiB.
//   dQ:    K(s) = 32 KiB s, V(s) = 32 KiB s + 16 KiB, K^T(s) = 64 KiB + 16 KiB s
//   dK/dV: Q(s) = 32 KiB s, dO(s) = 32 KiB s + 16 KiB, Q^T(s) = 64 KiB + 32 KiB s,
//          dO^T(s) = Q^T(s) + 16 KiB, lse(s) = 128 KiB + 2 KiB s, D(s) = lse(s) + 1 KiB
constexpr int COLS = 65536;
constexpr int DQ_LDS = COLS + 2 * COL_TILE;
constexpr int KV_LDS = COLS + 4 * COL_TILE + 4 * VEC_TILE;
static_assert(4 * ROW_TILE == COLS && 2 * ROW_TILE + 2 * COL_TILE == 65536, "layout");

struct BwdArgs {
  const bf16_t* q;     // [batch*seq, hq*D], RoPE applied
  const bf16_t* k;     // [batch*seq, hkv*D], RoPE applied
  const bf16_t* vtok;  // [batch, hkv, seq_pad, D]
  const bf16_t* kt;    // [batch, hkv, D, seq_pad]
  const bf16_t* qt;    // [batch, hq, D, seq_pad]
  const bf16_t* dout;  // [batch*seq, hq*D]
  const bf16_t* dot;   // [batch, hq, D, seq_pad]
  const float* lse;    // [batch, hq, seq_pad]
  const float* dvec;   // [batch, hq, seq_pad]
  bf16_t* dq;          // row r of dQ at dq + r * ld_dq, head j at column j*D
  float* part;         // [batch, hkv, nsplit, 2, seq_pad, D]
  int64_t ld_dq, seq, seq_pad;
  int hq, hkv, batch, nsplit, causal;
  float scale_log2, scale;
  double log2_base;  // 0: no RoPE rotation
};

__device__ __forceinline__ int swz_row(int r) { return r & 15; }             // 16 chunks per 256-byte row
__device__ __forceinline__ int swz_col(int d) { return (d ^ (d >> 3)) & 7; }  // 8 chunks per 128-byte row

// cos and sin of RoPE's angle pos * base^(-2k/128), evaluated in turns: the
// frequency in float64, split into two floats, the product with the position
// taken with its rounding error so the fraction of a turn keeps float
// precision for long sequences.
__device__ __forceinline__ void rope_cs(int pos, int k, double log2_base, float& c, float& s) {
  const double fd = exp2(-(double)(2 * k) * (1.0 / 128.0) * log2_base) * 0.15915494309189533577;
  const float fh = (float)fd, fl = (float)(fd - (double)fh);
  const float pf = (float)pos;  // exact: positions are below 2^24
  const float a = pf * fh;
  const float err = fmaf(pf, fh, -a);
  const float frac = (a - floorf(a)) + fmaf(pf, fl, err);
  s = __builtin_amdgcn_sinf(frac);
  c = __builtin_amdgcn_cosf(frac);
}

// B operand of 16 consecutive tokens (block of 32 chosen by u >> 1, half by
// u & 1) from bf16 pairs packed in the C layout of a 32 x 32 block: register
// r holds token 8 (r / 4) + 4 h + r % 4.  After one swap across the wave's
// halves, lanes 0-31 hold tokens 16u + 0..7 and lanes 32-63 tokens 16u + 8..15.
__device__ __forceinline__ u32x4 c_to_b(const uint32_t (&pk)[2][8], int u) {
  const int blk = u >> 1, r0 = (u & 1) * 4;
  auto s0 = __builtin_amdgcn_permlane32_swap(pk[blk][r0 + 0], pk[blk][r0 + 2], false, false);
  auto s1 = __builtin_amdgcn_permlane32_swap(pk[blk][r0 + 1], pk[blk][r0 + 3], false, false);
  return u32x4{s0[0], s1[0], s0[1], s1[1]};
}

// The same for one 32-token block's packed pairs: half hf (0 or 1) gives
// tokens 16 hf + 0..7 (lanes 0-31) and 16 hf + 8..15 (lanes 32-63).
__device__ __forceinline__ u32x4 c_to_b1(const uint32_t (&pk)[8], int hf) {
  const int r0 = hf * 4;
  auto s0 = __builtin_amdgcn_permlane32_swap(pk[r0 + 0], pk[r0 + 2], false, false);
  auto s1 = __builtin_amdgcn_permlane32_swap(pk[r0 + 1], pk[r0 + 3], false, false);
  return u32x4{s0[0], s1[0], s0[1], s1[1]};
}

// Zeroes [off, off + bytes) of the workgroup's LDS (16 bytes per thread and step).
template <int NTH>
__device__ __forceinline__ void lds_zero(char* smem, int off, int bytes) {
  for (int o = off + (int)threadIdx.x * 16; o < off + bytes; o += NTH * 16)
    *reinterpret_cast<u32x4*>(smem + o) = u32x4{0, 0, 0, 0};
}

// ---------------------------------------------------------------- dQ

// DQW waves of 32 queries per workgroup.  4 is launched: 8 (two waves per
// SIMD, one wave's vector work beside the other's MFMAs) measured slower at
// the 70B t = 8 shape (111 against 104 us), its 256 workgroups of 256
// queries leaving the causal imbalance between query blocks uncovered.
template <int DQW>
__global__ __launch_bounds__(DQW * 64, 1) void attn_bwd_dq_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[DQ_LDS];
  const int lane = lane_id(), wave = wave_id();
  const int l31 = lane & 31, h = lane >> 5;
  constexpr int QB = DQW * 32;     // queries per workgroup
  constexpr int LI = 16 / DQW;     // 16 KiB tile loads per wave

  // heaviest query blocks first
  const int per_qb = a.hq * a.batch;
  const int nqb = (int)((a.seq + QB - 1) / QB);
  const int qb = nqb - 1 - (int)(blockIdx.x / per_qb);
  const int rest = (int)(blockIdx.x % per_qb);
  const int j = rest % a.hq;
  const int b = rest / a.hq;
  const int g = j / (a.hq / a.hkv);
  const int64_t seq = a.seq, sp = a.seq_pad;
  const int64_t ldq = (int64_t)a.hq * D, ldk = (int64_t)a.hkv * D;
  const int q0 = qb * QB;
  const int qpos = q0 + wave * 32 + l31;
  const bool qok = qpos < seq;

  // Q and dO rows of this lane's query: B operands, d = 16 s + 8 h .. +7
  u32x4 qf[8], df[8];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + (int64_t)b * seq * ldq, (uint32_t)(seq * ldq * 2));
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.dout + (int64_t)b * seq * ldq, (uint32_t)(seq * ldq * 2));
    const uint32_t base = (uint32_t)((int64_t)qpos * ldq * 2 + (int64_t)j * D * 2 + h * 16);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qf[s] = buffer_load16(rq, qok ? base + s * 32 : TP_OOB_OFFSET);
      df[s] = buffer_load16(rd, qok ? base + s * 32 : TP_OOB_OFFSET);
    }
  }
  const int64_t vrow = ((int64_t)b * a.hq + j) * sp + qpos;
  const float lse = qok ? a.lse[vrow] : 0.0f;
  const float dd = qok ? a.dvec[vrow] : 0.0f;

  const __amdgpu_buffer_rsrc_t rk =
      make_rsrc(a.k + (int64_t)b * seq * ldk + (int64_t)g * D, (uint32_t)(seq * ldk * 2));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.vtok + ((int64_t)b * a.hkv + g) * sp * D, (uint32_t)(sp * D * 2));
  const __amdgpu_buffer_rsrc_t rkt = make_rsrc(a.kt + ((int64_t)b * a.hkv + g) * D * sp, (uint32_t)(D * sp * 2));
  // load slots: s = (i*DQW + wave)*64 + lane; row tiles: token s/16, physical
  // chunk s%16; column tile: row d = s/8, physical chunk s%8
  uint32_t k_off[LI], v_off[LI], t_off[LI];
  int row_of[LI];
#pragma unroll
  for (int i = 0; i < LI; ++i) {
    const int s = (i * DQW + wave) * 64 + lane;
    const int row = s >> 4, ck = (s & 15) ^ swz_row(row);
    row_of[i] = row;
    k_off[i] = (uint32_t)((int64_t)row * ldk * 2 + ck * 16);
    v_off[i] = (uint32_t)(row * D * 2 + ck * 16);
    const int d = s >> 3, cv = (s & 7) ^ swz_col(d);
    t_off[i] = (uint32_t)((int64_t)d * sp * 2 + cv * 16);
  }
  auto load_tile = [&](auto stage_tag, int t) {
    constexpr int S = decltype(stage_tag)::value;
    char* sk = smem + S * 2 * ROW_TILE;
    char* sv = sk + ROW_TILE;
    char* st = smem + COLS + S * COL_TILE;
    const int kb = t * 64;
#pragma unroll
    for (int i = 0; i < LI; ++i) {
      const bool ok = kb + row_of[i] < seq;
      const int slot = (i * DQW + wave) * 1024;
      buffer_load_lds16(rk, sk + slot, ok ? k_off[i] + (uint32_t)((int64_t)kb * ldk * 2) : TP_OOB_OFFSET);
      buffer_load_lds16(rv, sv + slot, ok ? v_off[i] + (uint32_t)(kb * D * 2) : TP_OOB_OFFSET);
      buffer_load_lds16(rkt, st + slot, t_off[i] + (uint32_t)(kb * 2));
    }
  };

  // LDS read offsets.  Row tiles: token 32 blk + l31 at d step s is
  // rr[s] + blk * 8192 (the swizzle depends on the token mod 16 only).
  // Column tiles: d = 32 db + l31 at token step u is crb[db & 1][u] - COLS +
  // (db >> 1) * 8192 (the swizzle repeats every 64 rows; crb carries the
  // column tiles' base).
  uint32_t rr[8], crb[2][4];
#pragma unroll
  for (int s = 0; s < 8; ++s) rr[s] = (uint32_t)(l31 * 256 + (((2 * s + h) ^ swz_row(l31)) << 4));
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    const int d = db * 32 + l31;
#pragma unroll
    for (int u = 0; u < 4; ++u) crb[db][u] = (uint32_t)(COLS + d * 128 + (((2 * u + h) ^ swz_col(d)) << 4));
  }

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = f32x16{};
  const int64_t last_q = min<int64_t>((int64_t)q0 + QB - 1, seq - 1);
  const int n_kv = a.causal ? (int)(last_q / 64) + 1 : (int)((seq + 63) / 64);
  const int key_lim = a.causal ? min(qpos, (int)seq - 1) : (int)seq - 1;

  constexpr std::integral_constant<int, 0> st0{};
  constexpr std::integral_constant<int, 1> st1{};
  auto kv_tile = [&](auto stage_tag, int t) {
    constexpr int S = decltype(stage_tag)::value;
    wait_vmcnt0();
    __syncthreads();
    if (t + 1 < n_kv) load_tile(std::integral_constant<int, 1 - S>{}, t + 1);
    const char* sk = smem + S * 2 * ROW_TILE;
    const char* sv = sk + ROW_TILE;
    const char* st = smem + S * COL_TILE;  // + COLS, carried by crb

    // per 32-key block: S^T = K Q^T and dP^T = V dO^T (two interleaved MFMA
    // chains, fragments read as they are used), dS^T = P^T (dP^T - D) rounded
    // to bf16 pairs (zero where the key is masked or past the sequence), then
    // dQ^T += K^T dS^T over the block's two 16-key steps
    const int key0 = t * 64;
    const bool live = t < n_kv;  // the odd tail's second tile is computed fully masked
    const bool need_mask = !live || (a.causal && key0 + 63 > q0) || (key0 + 64 > seq);
    const int klim = live ? key_lim : -1;
    uint32_t dsk[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const u32x4 kf = lds_read16(sk + rr[s] + kb * 8192);
        const u32x4 vf = lds_read16(sv + rr[s] + kb * 8192);
        sacc = mfma32x32x16(kf, qf[s], sacc);
        pacc = mfma32x32x16(vf, df[s], pacc);
      }
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[r], a.scale_log2, -lse));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[r + 1], a.scale_log2, -lse));
        float d0 = p0 * (pacc[r] - dd), d1 = p1 * (pacc[r + 1] - dd);
        if (need_mask) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          d0 = key > klim ? 0.0f : d0;
          d1 = key + 1 > klim ? 0.0f : d1;
        }
        dsk[kb][r >> 1] = pack_bf16x2(d0, d1);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 2 * kb; u < 2 * kb + 2; ++u) {
        const u32x4 bs = c_to_b(dsk, u);
#pragma unroll
        for (int db = 0; db < 4; ++db)
          acc[db] = mfma32x32x16(lds_read16(st + crb[db & 1][u] + (db >> 1) * 8192), bs, acc[db]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // tiles in pairs, both always run (see the dK/dV kernel).  Stage 1 starts
  // zeroed: a one-tile walk runs its masked second tile there, and its zero
  // dS must not meet stale non-finite LDS bits (0 x NaN is NaN).
  lds_zero<DQW * 64>(smem, 2 * ROW_TILE, 2 * ROW_TILE);
  lds_zero<DQW * 64>(smem, COLS + COL_TILE, COL_TILE);
  load_tile(st0, 0);
  for (int t = 0; t < n_kv; t += 2) {
    kv_tile(st0, t);
    kv_tile(st1, t + 1);
  }

  // ---- scale, rotate back through RoPE, store: block db, register r ->
  // d = 32 db + 8 (r/4) + 4 h + r%4; the pair (d, d + 64) is (db, db + 2)
  if (!qok) return;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] *= a.scale;
  if (a.log2_base != 0.0) {
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float c, s;
        rope_cs(qpos, db * 32 + 8 * (r >> 2) + 4 * h + (r & 3), a.log2_base, c, s);
        const float x1 = acc[db][r], x2 = acc[db + 2][r];
        acc[db][r] = x1 * c + x2 * s;
        acc[db + 2][r] = x2 * c - x1 * s;
      }
  }
  bf16_t* row = a.dq + ((int64_t)b * seq + qpos) * a.ld_dq + (int64_t)j * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = db * 32 + 8 * r4 + 4 * h;
      *reinterpret_cast<u32x2*>(row + d) = u32x2{pack_bf16x2(acc[db][4 * r4 + 0], acc[db][4 * r4 + 1]),
                                                 pack_bf16x2(acc[db][4 * r4 + 2], acc[db][4 * r4 + 3])};
    }
}

// ---------------------------------------------------------------- dK, dV

__global__ __launch_bounds__(NT, 1) void attn_bwd_dkdv_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[KV_LDS];
  const int lane = lane_id(), wave = wave_id();
  const int l31 = lane & 31, h = lane >> 5;

  // key blocks in ascending order: under the causal mask the first ones see
  // the most queries
  const int per_kb = a.nsplit * a.hkv * a.batch;
  const int kblk = (int)(blockIdx.x / per_kb);
  int rest = (int)(blockIdx.x % per_kb);
  const int spl = rest % a.nsplit;
  rest /= a.nsplit;
  const int g = rest % a.hkv;
  const int b = rest / a.hkv;
  const int gsize = a.hq / a.hkv, hps = gsize / a.nsplit;
  const int j0 = g * gsize + spl * hps;
  const int64_t seq = a.seq, sp = a.seq_pad;
  const int64_t ldq = (int64_t)a.hq * D, ldk = (int64_t)a.hkv * D;
  const int k0 = kblk * 128;
  const int kw = k0 + wave * 32 + l31;  // this lane's key
  const bool kok = kw < seq;

  // K and V rows of this lane's key: B operands, d = 16 s + 8 h .. +7
  u32x4 kf[8], vf[8];
  {
    const __amdgpu_buffer_rsrc_t rk =
        make_rsrc(a.k + (int64_t)b * seq * ldk + (int64_t)g * D, (uint32_t)(seq * ldk * 2));
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(a.vtok + ((int64_t)b * a.hkv + g) * sp * D, (uint32_t)(sp * D * 2));
    const uint32_t kbase = (uint32_t)((int64_t)kw * ldk * 2 + h * 16);
    const uint32_t vbase = (uint32_t)(kw * D * 2 + h * 16);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      kf[s] = buffer_load16(rk, kok ? kbase + s * 32 : TP_OOB_OFFSET);
      vf[s] = buffer_load16(rv, kok ? vbase + s * 32 : TP_OOB_OFFSET);
    }
  }

  uint32_t q_off[4], t_off[4];
  int row_of[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = (i * 4 + wave) * 64 + lane;
    const int row = s >> 4, ck = (s & 15) ^ swz_row(row);
    row_of[i] = row;
    q_off[i] = (uint32_t)((int64_t)row * ldq * 2 + ck * 16);
    const int d = s >> 3, cv = (s & 7) ^ swz_col(d);
    t_off[i] = (uint32_t)((int64_t)d * sp * 2 + cv * 16);
  }
  const int qt0 = a.causal ? k0 / 64 : 0;
  const int nqt = (int)((seq + 63) / 64);
  const int per_head = nqt - qt0;  // >= 1: k0 < seq
  const int n_it = per_head * hps;

  auto load_tile = [&](auto stage_tag, int it) {
    constexpr int S = decltype(stage_tag)::value;
    char* sq = smem + S * 2 * ROW_TILE;
    char* sdo = sq + ROW_TILE;
    char* sqt = smem + COLS + S * 2 * COL_TILE;
    char* sdot = sqt + COL_TILE;
    char* sl = smem + COLS + 4 * COL_TILE + S * 2 * VEC_TILE;
    char* sdv = sl + VEC_TILE;
    const int hi = it / per_head;
    const int jj = j0 + hi;
    const int q0 = (qt0 + it - hi * per_head) * 64;
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(a.q + (int64_t)b * seq * ldq + (int64_t)jj * D, (uint32_t)(seq * ldq * 2));
    const __amdgpu_buffer_rsrc_t rd =
        make_rsrc(a.dout + (int64_t)b * seq * ldq + (int64_t)jj * D, (uint32_t)(seq * ldq * 2));
    const __amdgpu_buffer_rsrc_t rqt =
        make_rsrc(a.qt + ((int64_t)b * a.hq + jj) * D * sp, (uint32_t)(D * sp * 2));
    const __amdgpu_buffer_rsrc_t rdt =
        make_rsrc(a.dot + ((int64_t)b * a.hq + jj) * D * sp, (uint32_t)(D * sp * 2));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = q0 + row_of[i] < seq;
      const uint32_t ro = ok ? q_off[i] + (uint32_t)((int64_t)q0 * ldq * 2) : TP_OOB_OFFSET;
      const int slot = (i * 4 + wave) * 1024;
      buffer_load_lds16(rq, sq + slot, ro);
      buffer_load_lds16(rd, sdo + slot, ro);
      buffer_load_lds16(rqt, sqt + slot, t_off[i] + (uint32_t)(q0 * 2));
      buffer_load_lds16(rdt, sdot + slot, t_off[i] + (uint32_t)(q0 * 2));
    }
    // 64 lse and D values: lanes 0-15 of waves 0 and 1
    const uint32_t vo = lane < 16 ? (uint32_t)(q0 * 4 + lane * 16) : TP_OOB_OFFSET;
    if (wave == 0)
      buffer_load_lds16(make_rsrc(a.lse + ((int64_t)b * a.hq + jj) * sp, (uint32_t)(sp * 4)), sl, vo);
    else if (wave == 1)
      buffer_load_lds16(make_rsrc(a.dvec + ((int64_t)b * a.hq + jj) * sp, (uint32_t)(sp * 4)), sdv, vo);
  };

  // LDS read offsets, as in the dQ kernel
  uint32_t rr[8], crb[2][4];
#pragma unroll
  for (int s = 0; s < 8; ++s) rr[s] = (uint32_t)(l31 * 256 + (((2 * s + h) ^ swz_row(l31)) << 4));
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    const int d = db * 32 + l31;
#pragma unroll
    for (int u = 0; u < 4; ++u) crb[db][u] = (uint32_t)(COLS + d * 128 + (((2 * u + h) ^ swz_col(d)) << 4));
  }

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  constexpr std::integral_constant<int, 0> st0{};
  constexpr std::integral_constant<int, 1> st1{};
  auto q_tile = [&](auto stage_tag, int it) {
    constexpr int S = decltype(stage_tag)::value;
    wait_vmcnt0();
    __syncthreads();
    if (it + 1 < n_it) load_tile(std::integral_constant<int, 1 - S>{}, it + 1);
    const char* sq = smem + S * 2 * ROW_TILE;
    const char* sdo = sq + ROW_TILE;
    const char* sqt = smem + S * 2 * COL_TILE;  // + COLS, carried by crb
    const char* sdot = sqt + COL_TILE;
    const char* sl = smem + COLS + 4 * COL_TILE + S * 2 * VEC_TILE;
    const char* sdv = sl + VEC_TILE;
    const int hi = it / per_head;
    const int q0 = (qt0 + it - hi * per_head) * 64;
    const bool live = it < n_it;  // the odd tail's second tile is computed fully masked

    // per 32-query block: S = Q K^T and dP = dO V^T (two interleaved MFMA
    // chains, fragments read as they are used); P and dS rounded to bf16
    // pairs; then the block's two 16-query steps of dV^T += dO^T P and
    // dK^T += Q^T dS.  Register r of block qb is query
    // q0 + 32 qb + 8 (r/4) + 4 h + r%4.  Kept: queries that exist and (causal)
    // may see this lane's key; only P is masked, since dS = P (dP - D) and D
    // is zero past the sequence.
    const bool need_mask = !live || (a.causal && q0 < k0 + 127) || (q0 + 64 > seq);
    const int q_hi = live ? (int)min<int64_t>(seq, (int64_t)q0 + 64) : 0;
    const int q_lo = a.causal ? kw : 0;
    const uint32_t span = (uint32_t)max(q_hi - q_lo, 0);
    const int qbase = q0 + 4 * h - q_lo;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const u32x4 qa = lds_read16(sq + rr[s] + qb * 8192);
        const u32x4 da = lds_read16(sdo + rr[s] + qb * 8192);
        sacc = mfma32x32x16(qa, kf[s], sacc);
        pacc = mfma32x32x16(da, vf[s], pacc);
      }
      uint32_t pk[8], sk[8];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int qr = qb * 32 + 8 * r4 + 4 * h;
        const f32x4 L = *reinterpret_cast<const f32x4*>(sl + qr * 4);
        const f32x4 Dv = *reinterpret_cast<const f32x4*>(sdv + qr * 4);
        float p[4], ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[e] = __builtin_amdgcn_exp2f(fmaf(sacc[4 * r4 + e], a.scale_log2, -L[e]));
          if (need_mask) p[e] = (uint32_t)(qbase + qb * 32 + 8 * r4 + e) < span ? p[e] : 0.0f;
          ds[e] = p[e] * (pacc[4 * r4 + e] - Dv[e]);
        }
        pk[2 * r4] = pack_bf16x2(p[0], p[1]);
        pk[2 * r4 + 1] = pack_bf16x2(p[2], p[3]);
        sk[2 * r4] = pack_bf16x2(ds[0], ds[1]);
        sk[2 * r4 + 1] = pack_bf16x2(ds[2], ds[3]);
      }
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        const int u = 2 * qb + uu;  // query step within the tile
        const u32x4 pb = c_to_b1(pk, uu);
        const u32x4 sb = c_to_b1(sk, uu);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const uint32_t off = crb[db & 1][u] + (db >> 1) * 8192;
          dv[db] = mfma32x32x16(lds_read16(sdot + off), pb, dv[db]);
          dk[db] = mfma32x32x16(lds_read16(sqt + off), sb, dk[db]);
        }
      }
    }
  };
  // tiles in pairs, both always run: a conditional second tile would make the
  // compiler copy the accumulators between register files at the join.
  // Stage 1 starts zeroed: a one-tile walk runs its masked second tile there,
  // and its zero P and dS must not meet stale non-finite LDS bits (0 x NaN).
  lds_zero<NT>(smem, 2 * ROW_TILE, 2 * ROW_TILE);
  lds_zero<NT>(smem, COLS + 2 * COL_TILE, 2 * COL_TILE);
  lds_zero<NT>(smem, COLS + 4 * COL_TILE + 2 * VEC_TILE, 2 * VEC_TILE);
  load_tile(st0, 0);
  for (int it = 0; it < n_it; it += 2) {
    q_tile(st0, it);
    q_tile(st1, it + 1);
  }

  // ---- partials: lane = key, block db register r -> d = 32 db + 8 (r/4) + 4 h + r%4
  if (!kok) return;
  float* pk_out = a.part + ((((int64_t)b * a.hkv + g) * a.nsplit + spl) * 2 * sp + kw) * D;
  float* pv_out = pk_out + sp * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = db * 32 + 8 * r4 + 4 * h;
      *reinterpret_cast<f32x4*>(pk_out + d) =
          f32x4{dk[db][4 * r4] * a.scale, dk[db][4 * r4 + 1] * a.scale, dk[db][4 * r4 + 2] * a.scale,
                dk[db][4 * r4 + 3] * a.scale};
      *reinterpret_cast<f32x4*>(pv_out + d) =
          f32x4{dv[db][4 * r4], dv[db][4 * r4 + 1], dv[db][4 * r4 + 2], dv[db][4 * r4 + 3]};
    }
}

// dK and dV of KV head g at position p: the sum of the splits' partials in
// ascending order, dK rotated back through RoPE, both stored as bf16.  16
// threads per (sequence, head, position), each owning the pairs
// (k .. k+3, k+64 .. k+67).
__global__ __launch_bounds__(NT) void attn_bwd_kv_sum_kernel(const float* part, bf16_t* dk_out, bf16_t* dv_out,
                                                             int64_t ld, int64_t seq, int64_t sp, int hkv,
                                                             int nsplit, int64_t rows, double log2_base) {
  const int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (e >= rows * 16) return;
  const int64_t row = e >> 4;  // (b * hkv + g) * seq + p
  const int k = (int)(e & 15) * 4;
  const int64_t p = row % seq, bg = row / seq;
  const int g = (int)(bg % hkv);
  const int64_t b = bg / hkv;
  f32x4 k1 = {}, k2 = {}, v1 = {}, v2 = {};
  for (int s = 0; s < nsplit; ++s) {
    const float* src = part + ((bg * nsplit + s) * 2 * sp + p) * D + k;
    k1 += *reinterpret_cast<const f32x4*>(src);
    k2 += *reinterpret_cast<const f32x4*>(src + 64);
    v1 += *reinterpret_cast<const f32x4*>(src + sp * D);
    v2 += *reinterpret_cast<const f32x4*>(src + sp * D + 64);
  }
  if (log2_base != 0.0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float c, s;
      rope_cs((int)p, k + i, log2_base, c, s);
      const float x1 = k1[i], x2 = k2[i];
      k1[i] = x1 * c + x2 * s;
      k2[i] = x2 * c - x1 * s;
    }
  }
  const int64_t o = (b * seq + p) * ld + (int64_t)g * D + k;
  *reinterpret_cast<u32x2*>(dk_out + o) = u32x2{pack_bf16x2(k1[0], k1[1]), pack_bf16x2(k1[2], k1[3])};
  *reinterpret_cast<u32x2*>(dk_out + o + 64) = u32x2{pack_bf16x2(k2[0], k2[1]), pack_bf16x2(k2[2], k2[3])};
  *reinterpret_cast<u32x2*>(dv_out + o) = u32x2{pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3])};
  *reinterpret_cast<u32x2*>(dv_out + o + 64) = u32x2{pack_bf16x2(v2[0], v2[1]), pack_bf16x2(v2[2], v2[3])};
}

// dvec[b, j, p] = sum_c dO[b*seq + p, j*D + c] O[...]: 16 threads per (token,
// head) row of 128 values, 8 each, then a fixed butterfly over the 16.
__global__ __launch_bounds__(NT) void attn_dvec_kernel(const bf16_t* o, const bf16_t* dout, float* dvec,
                                                       int64_t rows, int hq, int64_t seq, int64_t sp) {
  const int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x;
  const int64_t row = e >> 4;  // token * hq + j
  float acc = 0.0f;
  if (row < rows) {
    const int64_t off = row * D + (e & 15) * 8;
    const u32x4 x = *reinterpret_cast<const u32x4*>(o + off);
    const u32x4 y = *reinterpret_cast<const u32x4*>(dout + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(__uint_as_float(x[i] << 16), __uint_as_float(y[i] << 16), acc);
      acc = fmaf(__uint_as_float(x[i] & 0xFFFF0000u), __uint_as_float(y[i] & 0xFFFF0000u), acc);
    }
  }
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && (e & 15) == 0) {
    const int64_t token = row / hq;
    const int j = (int)(row % hq);
    const int64_t b = token / seq, p = token % seq;
    dvec[(b * hq + j) * sp + p] = acc;
    // the row's padding past the sequence is zero (the dK/dV kernel's dS
    // relies on it for rows it masks)
    if (p == seq - 1)
      for (int64_t q = seq; q < sp; ++q) dvec[(b * hq + j) * sp + q] = 0.0f;
  }
}

}  // namespace

hipError_t launch_attn_dvec(int64_t batch, int64_t seq, int64_t seq_pad, int hq, const void* o, const void* dout,
                            float* dvec, hipStream_t s) {
  const int64_t rows = batch * seq * hq;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(attn_dvec_kernel, dim3((unsigned)((rows * 16 + NT - 1) / NT)), dim3(NT), 0, s,
                     reinterpret_cast<const bf16_t*>(o), reinterpret_cast<const bf16_t*>(dout), dvec, rows, hq, seq,
                     seq_pad);
  return hipGetLastError();
}

hipError_t launch_flash_attn_bwd(int64_t batch, int64_t seq, int64_t seq_pad, int hq, int hkv, int causal,
                                 double log2_base, const AttnBwdIn& in, float* part, int nsplit, void* dqkv,
                                 int64_t ld, hipStream_t s) {
  if (batch * seq == 0) return hipSuccess;
  if (hkv <= 0 || hq % hkv != 0 || nsplit <= 0 || (hq / hkv) % nsplit != 0 || seq_pad % 64 != 0 ||
      seq_pad < seq)
    return hipErrorInvalidValue;
  BwdArgs a;
  a.q = reinterpret_cast<const bf16_t*>(in.q);
  a.k = reinterpret_cast<const bf16_t*>(in.k);
  a.vtok = reinterpret_cast<const bf16_t*>(in.vtok);
  a.kt = reinterpret_cast<const bf16_t*>(in.kt);
  a.qt = reinterpret_cast<const bf16_t*>(in.qt);
  a.dout = reinterpret_cast<const bf16_t*>(in.dout);
  a.dot = reinterpret_cast<const bf16_t*>(in.dot);
  a.lse = in.lse;
  a.dvec = in.dvec;
  a.dq = reinterpret_cast<bf16_t*>(dqkv);
  a.part = part;
  a.ld_dq = ld;
  a.seq = seq;
  a.seq_pad = seq_pad;
  a.hq = hq;
  a.hkv = hkv;
  a.batch = (int)batch;
  a.nsplit = nsplit;
  a.causal = causal ? 1 : 0;
  a.scale = 1.0f / sqrtf((float)D);
  a.scale_log2 = 1.4426950408889634f * a.scale;
  a.log2_base = log2_base;
  const int64_t nkb = (seq + 127) / 128;
  constexpr int DQW = 4;
  const int64_t nqb_dq = (seq + DQW * 32 - 1) / (DQW * 32);
  hipLaunchKernelGGL(attn_bwd_dq_kernel<DQW>, dim3((unsigned)(nqb_dq * hq * batch)), dim3(DQW * 64), 0, s, a);
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel, dim3((unsigned)(nkb * nsplit * hkv * batch)), dim3(NT), 0, s, a);
  const int64_t rows = batch * hkv * seq;
  bf16_t* base = reinterpret_cast<bf16_t*>(dqkv);
  hipLaunchKernelGGL(attn_bwd_kv_sum_kernel, dim3((unsigned)((rows * 16 + NT - 1) / NT)), dim3(NT), 0, s, part,
                     base + (int64_t)hq * D, base + (int64_t)(hq + hkv) * D, ld, seq, seq_pad, hkv, nsplit, rows,
                     log2_base);
  return hipGetLastError();
}

}  // namespace tpk
