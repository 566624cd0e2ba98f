// Causal grouped-query flash attention for one rank's heads, gfx950, d = 128.
//
// "Tensor parallelism" page, section "Self-attention": heads are independent,
// so a rank runs attention over its own a/t query heads with no exchange; with
// grouped-query attention the rank's query heads read the KV heads it holds.
//
// Work: query blocks of 128 rows, taken in pairs (p, last - p) per (sequence
// b, query head j), so that with the causal mask every pair walks about the
// same number of 64-key tiles; each pair's tiles, block p's then block
// last - p's, are cut into equal pieces, one workgroup each (two per CU).  A
// workgroup walks one or two segments (a query block over a range of its key
// tiles); a block whose tiles span pieces is completed by the piece holding
// its last tile from the others' float32 partials.  4 waves of 32 query rows;
// keys/values stream through LDS 64 at a time (two stages).
//
// Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
// a lane then owns one query (its column) and 16 keys per 32-key block, so the
// running max and sum of the online softmax are per-lane scalars.  The value
// product is O^T = V^T P^T: P^T is the B operand straight from the score
// registers (rounded to bf16; the K rows are fed to the score MFMA in an
// order that leaves each lane's 8 keys of a value step in place), and V^T is
// read from LDS as rows of the transposed-V layout the projection writes.
// Exponentials are the hardware
// exp2 of one FMA (the 1/sqrt(d) * log2(e) scale folded in; probabilities
// below 2^-126 may flush to zero, far below the bf16 P they feed and the
// float32 sum they join); the running max moves, and
// O is rescaled, only when a score exceeds it by more than 2^8; accumulation
// is float32.
#include <algorithm>
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

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
  // Work schedule: query blocks are taken in pairs (p, nqb - 1 - p) whose
  // key tiles, concatenated, form one list per (pair, sequence, head); that
  // list is cut into `pieces` equal ranges, one per workgroup.
  int units;   // pairs x batch x hq: workgroups per piece index
  int pieces;
  // Hand-over of split query blocks (pieces > 1): a workgroup that covers a
  // block's keys only up to some tile writes its float32 partial to slot
  // blockIdx.x of part and raises flag[blockIdx.x] to epoch; the workgroup
  // that covers the block's last key tile merges the partials.
  float* part;
  unsigned* flag;
  unsigned epoch;
};

__device__ __forceinline__ int swz_k(int key) { return key & 15; }          // 16 chunks/row
__device__ __forceinline__ int swz_v(int d) { return (d ^ (d >> 3)) & 7; }  // 8 chunks/row

// Key row that lane l31 supplies to the score MFMA: rows 4..7 and 8..11 of
// every 16 trade places, so that score register r of block kb in wave half
// h holds key 32 kb + 16 (r / 8) + 8 h + r % 8.  Each half then holds, per
// 16-key step of the value product, the 8 consecutive keys it supplies as
// that MFMA's B operand, in order: P^T needs no exchange between lanes.
__device__ __forceinline__ int key_row(int l31) { return (l31 & ~12) | ((l31 & 4) << 1) | ((l31 & 8) >> 1); }

__device__ __forceinline__ float other_half(float v) {
  // value of the same register in lane L ^ 32
  const uint32_t b = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

constexpr int CPOL_SC0_SC1 = 1 | 16;  // cache policy bits of a system-coherent buffer access

__global__ __launch_bounds__(NT, 2) void flash_attn_kernel(FaArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int lane = lane_id(), wave = wave_id();
  const int l31 = lane & 31, h = lane >> 5;

  // ---- this workgroup's share of the work
  const int per_qb = a.hq * a.batch;
  const int piece = (int)blockIdx.x / a.units;
  const int rest = (int)blockIdx.x - piece * a.units;
  const int pair = rest / per_qb;
  const int bh = rest - pair * per_qb;
  const int j = bh % a.hq;
  const int b = bh / a.hq;
  const int g = j / (a.hq / a.hkv);
  const int64_t seq = a.seq;
  const int64_t ldq = (int64_t)a.hq * D, ldk = (int64_t)a.hkv * D;

  // key tiles of query block qb: up to its last query (causal) or all keys
  auto n_tiles = [&](int qb) {
    const int64_t last_q = min<int64_t>((int64_t)qb * BQ + BQ - 1, seq - 1);
    return a.causal ? (int)(last_q / BKV) + 1 : (int)((seq + BKV - 1) / BKV);
  };
  const int qx = pair, qy = a.nqb - 1 - pair;
  const int nx = n_tiles(qx), ny = qy != qx ? n_tiles(qy) : 0;
  const uint32_t total = (uint32_t)(nx + ny);
  // start of piece i in the pair's list (uniform; marked so for the compiler)
  auto cut = [&](int i) { return __builtin_amdgcn_readfirstlane((int)(total * (uint32_t)i / (uint32_t)a.pieces)); };
  const int w0 = cut(piece), w1 = cut(piece + 1);
  if (w0 == w1) return;
  // one or two segments, each one query block over a range of its key
  // tiles: block qx's tiles [w0, w1) of the list [0, nx), block qy's the rest
  const bool has_x = w0 < nx, has_y = w1 > nx;
  const int nseg = (int)has_x + (int)has_y;

  // ---- Q fragments (B operand of S^T = K Q^T): query q0 + 32 w + l31,
  // head dims 16 s + 8 h .. +7 for s = 0..7
  __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + (int64_t)b * seq * ldq, (uint32_t)(seq * ldq * 2));
  u32x4 qf[8];
  auto load_q = [&](int qb) {
    const int qp = qb * BQ + wave * 32 + l31;
    const uint32_t base = (uint32_t)((int64_t)qp * ldq * 2 + (int64_t)j * D * 2 + h * 16);
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = buffer_load16(rq, qp < seq ? base + s * 32 : TP_OOB_OFFSET);
  };

  // ---- K / V^T tile loads straight into LDS
  __amdgpu_buffer_rsrc_t rk =
      make_rsrc(a.k + (int64_t)b * seq * ldk + (int64_t)g * D, (uint32_t)(seq * ldk * 2));
  __amdgpu_buffer_rsrc_t rv =
      make_rsrc(a.vt + ((int64_t)b * a.hkv + g) * D * a.seq_pad, (uint32_t)(D * a.seq_pad * 2));
  // K: slot s = (i*4 + wave)*64 + lane -> key s/16, physical chunk s%16
  // V: slot s -> row d = s/8, physical chunk s%8
  uint32_t k_off[4], v_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = (i * 4 + wave) * 64 + lane;
    const int key = s >> 4, ck = (s & 15) ^ swz_k(key);
    k_off[i] = (uint32_t)((int64_t)key * ldk * 2 + ck * 16);
    const int d = s >> 3, cv = (s & 7) ^ swz_v(d);
    v_off[i] = (uint32_t)((int64_t)d * a.seq_pad * 2 + cv * 16);
  }
  auto load_tile = [&](auto stage_tag, int t) {
    char* sk = smem + decltype(stage_tag)::value * STAGE;
    char* sv = sk + K_TILE;
    const int kb = t * BKV;
    const uint32_t ks = (uint32_t)((int64_t)kb * ldk * 2), vs = (uint32_t)(kb * 2);
    if (kb + BKV <= seq) {
      // a whole tile: fixed per-lane offsets plus scalar tile offsets
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        buffer_load_lds16_so(rk, sk + (i * 4 + wave) * 1024, k_off[i], ks);
        buffer_load_lds16_so(rv, sv + (i * 4 + wave) * 1024, v_off[i], vs);
      }
    } else {
      // keys past the sequence read as zeros (their offsets leave the buffer)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = ((i * 4 + wave) * 64 + lane) >> 4;
        buffer_load_lds16(rk, sk + (i * 4 + wave) * 1024, kb + key < seq ? k_off[i] + ks : TP_OOB_OFFSET);
        buffer_load_lds16(rv, sv + (i * 4 + wave) * 1024, v_off[i] + vs);
      }
    }
  };

  // ---- LDS read offsets
  uint32_t kr[2][8];  // [key block][d step]
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = kb * 32 + key_row(l31);
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
  float m_use, l_run;
  int q0 = 0, qpos = 0;

  constexpr std::integral_constant<int, 0> st0{};
  constexpr std::integral_constant<int, 1> st1{};
  // One key tile on LDS stage S (a compile-time constant, so fragment
  // addresses are fixed registers plus an immediate).  t_next: the key tile
  // to fetch into the other stage (-1: none).
  auto kv_tile = [&](auto stage_tag, int t, int t_next) {
    constexpr int S = decltype(stage_tag)::value;
    wait_vmcnt0();
    __syncthreads();
    if (t_next >= 0) load_tile(std::integral_constant<int, 1 - S>{}, t_next);
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
          const int key = key0 + kb * 32 + 16 * (r >> 3) + 8 * h + (r & 7);
          if (key > key_lim) sacc[kb][r] = -INFINITY;
        }
    }
    // max tree of three-input maxima: 16 instructions for the 32 scores
    float m3[11];
#pragma unroll
    for (int i = 0; i < 10; ++i) {
      const int j = 3 * i;
      m3[i] = fmaxf(fmaxf(sacc[j >> 4][j & 15], sacc[(j + 1) >> 4][(j + 1) & 15]), sacc[(j + 2) >> 4][(j + 2) & 15]);
    }
    m3[10] = fmaxf(sacc[1][14], sacc[1][15]);
    const float m9 = fmaxf(fmaxf(m3[0], m3[1]), m3[2]), m10 = fmaxf(fmaxf(m3[3], m3[4]), m3[5]);
    const float m11 = fmaxf(fmaxf(m3[6], m3[7]), m3[8]), m12 = fmaxf(m3[9], m3[10]);
    const float mloc = fmaxf(fmaxf(m9, m10), fmaxf(m11, m12));
    const float mt = fmaxf(mloc, other_half(mloc));
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

    // O^T += V^T P^T over four 16-key steps; packed pairs 4 (u % 2) .. +3 of
    // block u / 2 are this half's keys 16 u + 8 h .. +7
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kb = u >> 1, r0 = (u & 1) * 4;
      const u32x4 pb = {pk[kb][r0], pk[kb][r0 + 1], pk[kb][r0 + 2], pk[kb][r0 + 3]};
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] = mfma32x32x16(vf[u][db], pb, oacc[db]);
    }
  };

  // Key tiles [k0, k1) of one segment, starting on stage S, in pairs of
  // stages; next_k0: the tile to fetch after the last one (-1: none).
  auto walk_tiles = [&](auto stage_tag, int k0, int k1, int next_k0) {
    constexpr int S = decltype(stage_tag)::value;
    constexpr std::integral_constant<int, S> sa{};
    constexpr std::integral_constant<int, 1 - S> sb{};
    for (int t = k0; t < k1; t += 2) {
      kv_tile(sa, t, t + 1 < k1 ? t + 1 : next_k0);
      if (t + 1 < k1) kv_tile(sb, t + 1, t + 2 < k1 ? t + 2 : next_k0);
    }
  };

  // The partial of a split block, in slot `slot`: O^T as this thread holds
  // it (block db, registers 4 r4 .. 4 r4 + 3 at float4 (db * 4 + r4) * NT +
  // thread, so each wave store is one contiguous KiB), then the running max
  // and sum of every thread.  Written and read with system-coherent accesses
  // (sc0 sc1: past the non-coherent L2s of the other XCDs).
  auto slot_rsrc = [&](int slot) {
    return make_rsrc(a.part + (size_t)slot * FA_SLOT_FLOATS, (uint32_t)(FA_SLOT_FLOATS * sizeof(float)));
  };
  const uint32_t t16 = (uint32_t)threadIdx.x * 16;
  const uint32_t m_at = (uint32_t)(D * BQ * 4) + (uint32_t)threadIdx.x * 4;  // byte offsets
  const uint32_t l_at = m_at + NT * 4;

  // ---- the segments; the LDS stages alternate over the workgroup's whole walk
  // segment sg: query block, key tiles [k0, k1) of its n, its first tile's place in the list
  auto seg_q = [&](int sg) { return sg == 0 && has_x ? qx : qy; };
  auto seg_k0 = [&](int sg) { return sg == 0 && has_x ? w0 : max(w0, nx) - nx; };
  auto seg_k1 = [&](int sg) { return sg == 0 && has_x ? min(w1, nx) : w1 - nx; };
  auto seg_n = [&](int sg) { return sg == 0 && has_x ? nx : ny; };
  auto seg_off = [&](int sg) { return sg == 0 && has_x ? 0 : nx; };
  load_q(seg_q(0));
  load_tile(st0, seg_k0(0));
  int walk = 0;
  for (int sg = 0; sg < nseg; ++sg) {
    q0 = seg_q(sg) * BQ;
    qpos = q0 + wave * 32 + l31;
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
    m_use = -INFINITY;
    l_run = 0.0f;
    const int k0 = seg_k0(sg), k1 = seg_k1(sg), n_blk = seg_n(sg);
    const int next_k0 = sg + 1 < nseg ? seg_k0(sg + 1) : -1;
    if (walk & 1) walk_tiles(st1, k0, k1, next_k0);
    else walk_tiles(st0, k0, k1, next_k0);
    walk += k1 - k0;
    // the next segment's Q fragments (their latency overlaps this one's end)
    if (sg + 1 < nseg) load_q(seg_q(sg + 1));

    const bool whole = k0 == 0 && k1 == n_blk;
    if (k1 < n_blk) {
      // keys beyond this range belong to later pieces: hand the partial over
      const int slot = (int)blockIdx.x;
      __amdgpu_buffer_rsrc_t ws = slot_rsrc(slot);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 v = {oacc[db][4 * r4], oacc[db][4 * r4 + 1], oacc[db][4 * r4 + 2], oacc[db][4 * r4 + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ws,
                                                 (uint32_t)((db * 4 + r4) * NT * 16) + t16, 0, CPOL_SC0_SC1);
        }
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m_use), ws, m_at, 0, CPOL_SC0_SC1);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l_run), ws, l_at, 0, CPOL_SC0_SC1);
      wait_vmcnt0();
      __syncthreads();
      if (threadIdx.x == 0) __hip_atomic_store(a.flag + slot, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      continue;
    }
    if (!whole) {
      // this range holds the block's last key tile: merge the partials of the
      // earlier pieces that cover its first tiles, in a fixed order (this
      // piece's own values first, then the others by ascending piece), so the
      // result does not depend on which piece finishes first.  Those pieces
      // have lower launch indices, were dispatched first and never wait on
      // this one, so the wait ends; its bound only guards against a broken
      // launch (the result would then be wrong, not hung).
      const int first = seg_off(sg);  // the block's first tile in the list
      int p_first = 0;
      while (cut(p_first + 1) <= first) ++p_first;
      if (threadIdx.x == 0) {
        for (int p = p_first; p < piece; ++p) {
          if (cut(p) == cut(p + 1)) continue;
          unsigned* fl = a.flag + (p * a.units + rest);
          for (uint32_t n = 0; n < (1u << 22); ++n) {
            if (__hip_atomic_load(fl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.epoch) break;
            __builtin_amdgcn_s_sleep(2);
          }
        }
      }
      __syncthreads();
      float m_fin = m_use;
      for (int p = p_first; p < piece; ++p) {
        if (cut(p) == cut(p + 1)) continue;
        const float mp = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(slot_rsrc(p * a.units + rest), m_at, 0,
                                                                            CPOL_SC0_SC1));
        m_fin = fmaxf(m_fin, mp);
      }
      // every query row has key 0 in range, so m_fin is finite
      const float own = __builtin_amdgcn_exp2f((m_use - m_fin) * a.scale_log2);
      l_run *= own;
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] *= own;
      for (int p = p_first; p < piece; ++p) {
        if (cut(p) == cut(p + 1)) continue;
        __amdgpu_buffer_rsrc_t ws = slot_rsrc(p * a.units + rest);
        const float mp = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ws, m_at, 0, CPOL_SC0_SC1));
        const float lp = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ws, l_at, 0, CPOL_SC0_SC1));
        const float sc = __builtin_amdgcn_exp2f((mp - m_fin) * a.scale_log2);
        l_run += lp * sc;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          f32x4 v[4];
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
            v[r4] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  ws, (uint32_t)((db * 4 + r4) * NT * 16) + t16, 0, CPOL_SC0_SC1));
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
            for (int e = 0; e < 4; ++e) oacc[db][4 * r4 + e] += v[r4][e] * sc;
        }
      }
      m_use = m_fin;
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
}

// The library's split workspace: per (device, stream), allocated at the
// first split launch on that stream and kept until the process ends (calls
// on one stream are ordered; calls on different streams use different
// workspaces).  Flags hold epochs, so they are never cleared.
struct FaSlot {
  float* part = nullptr;
  unsigned* flag = nullptr;
  unsigned epoch = 0;
};
std::mutex g_fa_mu;
std::map<std::pair<int, hipStream_t>, FaSlot> g_fa;

bool fa_acquire(hipStream_t s, FaSplitWs* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  std::lock_guard<std::mutex> lock(g_fa_mu);
  FaSlot& slot = g_fa[{dev, s}];
  if (!slot.part) {
    constexpr size_t part_bytes = (size_t)FA_MAX_SLOTS * FA_SLOT_BYTES;
    void* p = nullptr;
    if (hipMalloc(&p, part_bytes + FA_MAX_SLOTS * sizeof(unsigned)) != hipSuccess) {
      (void)hipGetLastError();
      return false;
    }
    unsigned* flag = reinterpret_cast<unsigned*>(static_cast<char*>(p) + part_bytes);
    if (hipMemsetAsync(flag, 0, FA_MAX_SLOTS * sizeof(unsigned), s) != hipSuccess) {
      (void)hipGetLastError();
      (void)hipFree(p);
      return false;
    }
    slot.part = static_cast<float*>(p);
    slot.flag = flag;
  }
  out->part = slot.part;
  out->flag = slot.flag;
  out->epoch = ++slot.epoch;
  if (out->epoch == 0) out->epoch = ++slot.epoch;  // 0 is the flags' initial value
  return true;
}

}  // namespace

int flash_attn_pieces(int64_t batch, int64_t seq, int hq, int causal) {
  const int64_t nqb = (seq + BQ - 1) / BQ;
  const int64_t units = (nqb + 1) / 2 * hq * batch;
  if (units <= 0) return 1;
  // Measured (forced piece counts, 16 causal shapes on one MI355X): a cut
  // costs more than the chip it fills.  From 512 pair units (two workgroups
  // per CU) one piece is fastest (4 x 4096 tokens, 8 heads: 177 us against
  // 190 with 2 to 8); from 32 to 511 units two pieces are (the Llama-8B and
  // 70B t=16 ranks: 39.6 us against 43 with 4 and 45 with 8; 70B t=8: 49.9
  // against 59 unsplit and 65 with 3 or more; even 32 units, 64 workgroups,
  // beat 256 workgroups of 8 pieces).  Below 32 units the cut fills the chip
  // toward two workgroups per CU.  A piece keeps at least 4 key tiles (the
  // first pair's list is the longest) and the partials fit their slots.
  const int64_t last = std::min<int64_t>(BQ - 1, seq - 1);
  const int64_t nx = causal ? last / BKV + 1 : (seq + BKV - 1) / BKV;
  const int64_t ny = nqb > 1 ? (seq + BKV - 1) / BKV : 0;
  const int64_t list = nx + ny;
  int64_t p = units >= 512 ? 1 : units >= 32 ? 2 : std::min<int64_t>((512 + units / 2) / units, 8);
  while (p > 1 && (list < 4 * p || (p - 1) * units > FA_MAX_SLOTS)) --p;
  return (int)p;
}

size_t flash_attn_split_bytes(int64_t batch, int64_t seq, int hq, int causal) {
  const int p = flash_attn_pieces(batch, seq, hq, causal);
  const int64_t nqb = (seq + BQ - 1) / BQ;
  return (size_t)(p - 1) * (size_t)((nqb + 1) / 2 * hq * batch) * FA_SLOT_BYTES;
}

hipError_t launch_flash_attn(int64_t batch, int64_t seq, int64_t seq_pad, int hq, int hkv,
                             int causal, const void* q, const void* k, const void* vt, void* o,
                             hipStream_t s, float* lse, const FaSplitWs* ws) {
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
  a.units = (int)((int64_t)(a.nqb + 1) / 2 * hq * batch);
  if (a.units == 0) return hipSuccess;
  a.pieces = flash_attn_pieces(batch, seq, hq, causal);
  a.part = nullptr;
  a.flag = nullptr;
  a.epoch = 0;
  FaSplitWs own;
  if (a.pieces > 1 && !ws) {
    if (fa_acquire(s, &own)) ws = &own;
    else a.pieces = 1;
  }
  if (a.pieces > 1) {
    a.part = ws->part;
    a.flag = ws->flag;
    a.epoch = ws->epoch;
  }
  const int64_t nb = (int64_t)a.units * a.pieces;
  hipLaunchKernelGGL(flash_attn_kernel, dim3((unsigned)nb), dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace tpk
