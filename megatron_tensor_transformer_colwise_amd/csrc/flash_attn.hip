// Causal grouped-query flash attention for one rank's heads, gfx950, d = 128.
//
// "Tensor parallelism" page, section "Self-attention": heads are independent,
// so a rank runs attention over its own a/t query heads with no exchange; with
// grouped-query attention the rank's query heads read the KV heads it holds.
//
// One workgroup = (sequence b, query head j, 128 query rows); 4 waves, 32 query
// rows each.  Keys/values stream through LDS 64 at a time (two stages).
//
// Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
// a lane then owns one query (its column) and 16 keys per 32-key block, so the
// running max and sum of the online softmax are per-lane scalars.  The value
// product is O^T = V^T P^T: P^T is the B operand straight from the score
// registers (after rounding to bf16 and one v_permlane32_swap that makes each
// lane's 8 keys contiguous), and V^T is read from LDS as rows of the
// transposed-V layout the projection writes.  Exponentials are the hardware
// exp2 of one FMA (the 1/sqrt(d) * log2(e) scale folded in; probabilities
// below 2^-126 may flush to zero, far below the bf16 P they feed and the
// float32 sum they join); the running max moves, and
// O is rescaled, only when a score exceeds it by more than 2^8; accumulation
// is float32.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace tpk {
namespace {

constexpr int D = 128;
constexpr int BQ = 128;
constexpr int BKV = 64;
constexpr int NT = 256;
constexpr int K_TILE = BKV * D * 2;            // [64 keys][128 d], 256-byte rows
constexpr int V_TILE = D * BKV * 2;            // [128 d][64 keys], 128-byte rows
constexpr int STAGE = K_TILE + V_TILE;
constexpr float TAU = 8.0f;                    // lazy-rescale threshold, log2 units

struct FaArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* vt;
  bf16_t* o;
  float* lse;  // [batch, hq, seq_pad] log2-domain log-sum-exp of the scaled scores, or NULL
  int64_t seq, seq_pad;
  int hq, hkv, batch, nqb, causal;
  float scale_log2;
};

__device__ __forceinline__ int swz_k(int key) { return key & 15; }          // 16 chunks/row
__device__ __forceinline__ int swz_v(int d) { return (d ^ (d >> 3)) & 7; }  // 8 chunks/row

__device__ __forceinline__ float other_half(float v) {
  // value of the same register in lane L ^ 32
  const uint32_t b = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__global__ __launch_bounds__(NT, 2) void flash_attn_kernel(FaArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int lane = lane_id(), wave = wave_id();
  const int l31 = lane & 31, h = lane >> 5;

  // Query blocks by launch index: the first half of the launch takes the
  // heavier half of the query blocks (heaviest first), the second half the
  // lighter ones (lightest first), so launches i and i + nb/2 -- the two
  // workgroups one CU holds when the launch fills every CU twice -- carry
  // query blocks summing to nqb - 1: equal causal work per CU.
  const int per_qb = a.hq * a.batch;
  int qb, rest;
  const int half = (a.nqb / 2) * per_qb;
  if ((a.nqb & 1) == 0 && (int)blockIdx.x >= half) {
    const int i = (int)blockIdx.x - half;
    qb = i / per_qb;
    rest = i % per_qb;
  } else {
    qb = a.nqb - 1 - (int)(blockIdx.x / per_qb);
    rest = (int)(blockIdx.x % per_qb);
  }
  const int j = rest % a.hq;
  const int b = rest / a.hq;
  const int g = j / (a.hq / a.hkv);

  const int64_t seq = a.seq;
  const int64_t ldq = (int64_t)a.hq * D, ldk = (int64_t)a.hkv * D;
  const int q0 = qb * BQ;

  // ---- Q fragments (B operand of S^T = K Q^T): query q0 + 32 w + l31,
  // head dims 16 s + 8 h .. +7 for s = 0..7
  const int qpos = q0 + wave * 32 + l31;
  u32x4 qf[8];
  {
    __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + (int64_t)b * seq * ldq, (uint32_t)(seq * ldq * 2));
    const uint32_t base = (uint32_t)((int64_t)qpos * ldq * 2 + (int64_t)j * D * 2 + h * 16);
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = buffer_load16(rq, qpos < seq ? base + s * 32 : TP_OOB_OFFSET);
  }

  // ---- K / V^T tile loads straight into LDS
  __amdgpu_buffer_rsrc_t rk =
      make_rsrc(a.k + (int64_t)b * seq * ldk + (int64_t)g * D, (uint32_t)(seq * ldk * 2));
  __amdgpu_buffer_rsrc_t rv =
      make_rsrc(a.vt + ((int64_t)b * a.hkv + g) * D * a.seq_pad, (uint32_t)(D * a.seq_pad * 2));
  // K: slot s = (i*4 + wave)*64 + lane -> key s/16, physical chunk s%16
  // V: slot s -> row d = s/8, physical chunk s%8
  uint32_t k_off[4], v_off[4];
  int k_key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = (i * 4 + wave) * 64 + lane;
    const int key = s >> 4, ck = (s & 15) ^ swz_k(key);
    k_key[i] = key;
    k_off[i] = (uint32_t)((int64_t)key * ldk * 2 + ck * 16);
    const int d = s >> 3, cv = (s & 7) ^ swz_v(d);
    v_off[i] = (uint32_t)((int64_t)d * a.seq_pad * 2 + cv * 16);
  }
  auto load_tile = [&](auto stage_tag, int t) {
    char* sk = smem + decltype(stage_tag)::value * STAGE;
    char* sv = sk + K_TILE;
    const int kb = t * BKV;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = kb + k_key[i] < seq;
      buffer_load_lds16(rk, sk + (i * 4 + wave) * 1024,
                        ok ? k_off[i] + (uint32_t)((int64_t)kb * ldk * 2) : TP_OOB_OFFSET);
      buffer_load_lds16(rv, sv + (i * 4 + wave) * 1024, v_off[i] + (uint32_t)(kb * 2));
    }
  };

  // ---- LDS read offsets
  uint32_t kr[2][8];  // [key block][d step]
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = kb * 32 + l31;
#pragma unroll
    for (int s = 0; s < 8; ++s) kr[kb][s] = (uint32_t)(key * 256 + (((2 * s + h) ^ swz_k(key)) << 4));
  }
  uint32_t vr[4][4];  // [d block][key step]
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int d = db * 32 + l31;
#pragma unroll
    for (int u = 0; u < 4; ++u) vr[db][u] = (uint32_t)(d * 128 + (((2 * u + h) ^ swz_v(d)) << 4));
  }

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
  float m_use = -INFINITY, l_run = 0.0f;

  const int64_t last_q = min<int64_t>((int64_t)q0 + BQ - 1, seq - 1);
  const int n_kv = a.causal ? (int)(last_q / BKV) + 1 : (int)((seq + BKV - 1) / BKV);

  constexpr std::integral_constant<int, 0> st0{};
  constexpr std::integral_constant<int, 1> st1{};
  // One key tile on LDS stage S (a compile-time constant, so fragment
  // addresses are fixed registers plus an immediate).
  auto kv_tile = [&](auto stage_tag, int t) {
    constexpr int S = decltype(stage_tag)::value;
    wait_vmcnt0();
    __syncthreads();
    if (t + 1 < n_kv) load_tile(std::integral_constant<int, 1 - S>{}, t + 1);
    const char* sk = smem + S * STAGE;
    const char* sv = sk + K_TILE;

    // S^T for 64 keys: two 32 x 32 blocks.  All K fragments are read before
    // the first MFMA, and all V^T fragments right after the last one, so LDS
    // latency hides under the score MFMAs and under the softmax.
    u32x4 kf[2][8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) kf[kb][s] = lds_read16(sk + kr[kb][s]);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sacc[kb] = mfma32x32x16(kf[kb][s], qf[s], sacc[kb]);
    }
    u32x4 vf[4][4];  // [key step u][d block]
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int db = 0; db < 4; ++db) vf[u][db] = lds_read16(sv + vr[db][u]);
    __builtin_amdgcn_sched_barrier(0);

    // mask, then the running max in raw score units.  The max used for the
    // exponentials (m_use) only moves when some score exceeds it by more than
    // 2^TAU after scaling; until then probabilities may reach 2^TAU, which
    // float32 sums and bf16 P hold exactly enough, and O / l are rescaled only
    // on the tiles where the max actually moves.
    const int key0 = t * BKV;
    const bool need_mask = (a.causal && key0 + BKV - 1 > q0) || (key0 + BKV > seq);
    if (need_mask) {
      // keys beyond the sequence or after the query (seq < 2^31, checked by the caller)
      const int key_lim = a.causal ? min(qpos, (int)seq - 1) : (int)seq - 1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key > key_lim) sacc[kb][r] = -INFINITY;
        }
    }
    // pairwise (tree) max: depth 5 instead of a 32-long dependency chain
    float mx[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) mx[r] = fmaxf(sacc[0][r], sacc[1][r]);
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
      for (int r = 0; r < w; ++r) mx[r] = fmaxf(mx[r], mx[r + w]);
    const float mt = fmaxf(mx[0], other_half(mx[0]));
    const bool grow = (mt - m_use) * a.scale_log2 > TAU;  // also true on the first tile
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? mt : m_use;
      const float alpha = __builtin_amdgcn_exp2f((m_use - m_new) * a.scale_log2);
      m_use = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    // (a lane whose keys are all masked so far keeps p = 0: exp2(-inf))
    const float mc = m_use == -INFINITY ? 0.0f : -m_use * a.scale_log2;

    // probabilities exp2(s * c - m * c), rounded to bf16 in pairs of keys
    uint32_t pk[2][8];
    float ps[16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], a.scale_log2, mc));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r + 1], a.scale_log2, mc));
        ps[kb * 8 + (r >> 1)] = p0 + p1;
        pk[kb][r >> 1] = pack_bf16x2(p0, p1);
      }
    // pairwise (tree) sum
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
      for (int r = 0; r < w; ++r) ps[r] += ps[r + w];
    l_run += ps[0];

    // O^T += V^T P^T over four 16-key steps
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kb = u >> 1, r0 = (u & 1) * 4;  // packed regs: keys 16u+4h+(0..3) | 16u+8+4h+(0..3)
      uint32_t x0 = pk[kb][r0 + 0], x1 = pk[kb][r0 + 1];  // first run of 4 keys
      uint32_t y0 = pk[kb][r0 + 2], y1 = pk[kb][r0 + 3];  // second run
      auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
      auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
      // lanes 0-31 now hold keys 16u+0..7, lanes 32-63 keys 16u+8..15
      const u32x4 pb = {s0[0], s1[0], s0[1], s1[1]};
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] = mfma32x32x16(vf[u][db], pb, oacc[db]);
    }
  };
  load_tile(st0, 0);
  for (int t = 0; t < n_kv; t += 2) {
    kv_tile(st0, t);
    if (t + 1 < n_kv) kv_tile(st1, t + 1);
  }

  // ---- normalise and store: O^T block db, register r -> d = 32 db + 8 (r/4) + 4 h + r%4
  const float l_tot = l_run + other_half(l_run);
  const float inv = 1.0f / l_tot;
  // for the backward pass: P = exp2(s * scale_log2 - lse), lse = m * scale_log2 + log2(l)
  if (a.lse && h == 0 && qpos < seq)
    a.lse[((int64_t)b * a.hq + j) * a.seq_pad + qpos] = m_use * a.scale_log2 + __builtin_amdgcn_logf(l_tot);
  if (qpos < seq) {
    bf16_t* orow = a.o + ((int64_t)b * seq + qpos) * ldq + (int64_t)j * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = db * 32 + 8 * r4 + 4 * h;
        u32x2 pr = {pack_bf16x2(oacc[db][4 * r4 + 0] * inv, oacc[db][4 * r4 + 1] * inv),
                    pack_bf16x2(oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d) = pr;
      }
  }
}

}  // namespace

hipError_t launch_flash_attn(int64_t batch, int64_t seq, int64_t seq_pad, int hq, int hkv,
                             int causal, const void* q, const void* k, const void* vt, void* o,
                             hipStream_t s, float* lse) {
  FaArgs a;
  a.q = reinterpret_cast<const bf16_t*>(q);
  a.k = reinterpret_cast<const bf16_t*>(k);
  a.vt = reinterpret_cast<const bf16_t*>(vt);
  a.o = reinterpret_cast<bf16_t*>(o);
  a.lse = lse;
  a.seq = seq;
  a.seq_pad = seq_pad;
  a.hq = hq;
  a.hkv = hkv;
  a.batch = (int)batch;
  a.nqb = (int)((seq + BQ - 1) / BQ);
  a.causal = causal ? 1 : 0;
  a.scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  const int64_t nb = (int64_t)a.nqb * hq * batch;
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(flash_attn_kernel, dim3((unsigned)nb), dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace tpk
