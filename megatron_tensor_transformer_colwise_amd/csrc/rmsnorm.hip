// RMSNorm of the block ("Tensor parallelism" page, section "f and g": norms
// run on every rank; section "Sequence parallelism": or on each rank's slice
// of the sequence, since they act on every token alone):
//   y[r, c] = bf16( x[r, c] / sqrt(mean_c x[r, c]^2 + eps) * gain[c] )
// One workgroup per row; 8 elements per thread per step; float32 math.
// HBM-bound: one read of x, one bf16 write of y.
//
// The fused form takes x itself as a shard-sum, x = ((p_0 + p_1) + ...) +
// residual (the sum that ends the previous sublayer, ascending rank order),
// writes x (float32, the residual stream) and y in the same pass: the sum is
// not read back.  Its arithmetic is that of the shard-sum followed by the
// plain RMSNorm, operation for operation, so the two forms agree bit for bit.
// (At 8192 x 8192 with 8 partials: 521 us against 548 for the two passes;
// with 16, whose loads the registers hold one group at a time, 988 against 930.)
// Rows may come as runs (run_rows rows, run_stride apart), so a rank's
// slice of every sequence of a (batch, sequence, hidden) activation is one
// launch; the residual alone (no partials) and the sum alone (no norm) are
// the same kernel.
#include "common.h"
#include "kernels.h"

namespace tpk {
namespace {

constexpr int NT = 256;
constexpr int MAX_CACHED = 4;  // 8-element groups a thread keeps in registers (h <= 8192)

template <bool IN_BF16>
__device__ __forceinline__ void load8(const void* x, int64_t e, float (&v)[8]) {
  if (IN_BF16) {
    const u32x4 u = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(x) + e);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(x) + e);
    const f32x4 b = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(x) + e + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
}

// Sum of squares of a row across the workgroup: each thread's partial sum,
// then the wave (xor shuffles), then the 4 waves; returns 1 / rms.
__device__ __forceinline__ float row_inv_rms(float ss, int64_t h, float eps, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  return 1.0f / sqrtf(tot / (float)h + eps);
}

// gv = gain[8 gi .. 8 gi + 8), or ones without a gain.
__device__ __forceinline__ void load_gain8(const float* gain, int64_t gi, float (&gv)[8]) {
  if (gain) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(gain + gi * 8);
    const f32x4 b = *reinterpret_cast<const f32x4*>(gain + gi * 8 + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gv[i] = a[i];
      gv[4 + i] = b[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) gv[i] = 1.0f;
  }
}

// y[e .. e + 8) = bf16(v * inv * gv), gv the group's gains.
__device__ __forceinline__ void emit8g(const float (&v)[8], float inv, const float (&gv)[8], bf16_t* y, int64_t e) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = pack_bf16x2(v[2 * i] * inv * gv[2 * i], v[2 * i + 1] * inv * gv[2 * i + 1]);
  *reinterpret_cast<u32x4*>(y + e) = o;
}

__device__ __forceinline__ void emit8(const float (&v)[8], float inv, const float* gain, int64_t gi,
                                      bf16_t* y, int64_t e) {
  float gv[8];
  load_gain8(gain, gi, gv);
  emit8g(v, inv, gv, y, e);
}

template <bool IN_BF16>
__global__ __launch_bounds__(NT) void rmsnorm_kernel(const void* x, const float* gain, float eps,
                                                     bf16_t* y, int64_t h) {
  __shared__ float red[NT / 64];
  const int64_t row = blockIdx.x;
  const int64_t base = row * h;
  const int64_t groups = h >> 3;
  float cache[MAX_CACHED][8];
  // the gains of the cached groups are loaded with the row, so the
  // normalisation after the row's reduction waits on no further load
  float gcache[MAX_CACHED][8];
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < MAX_CACHED; ++i) {
    const int64_t gi = threadIdx.x + (int64_t)i * NT;
    if (gi < groups) {
      load8<IN_BF16>(x, base + gi * 8, cache[i]);
      load_gain8(gain, gi, gcache[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += cache[i][e] * cache[i][e];
    }
  }
  for (int64_t gi = threadIdx.x + (int64_t)MAX_CACHED * NT; gi < groups; gi += NT) {
    float v[8];
    load8<IN_BF16>(x, base + gi * 8, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
  }
  const float inv = row_inv_rms(ss, h, eps, red);
#pragma unroll
  for (int i = 0; i < MAX_CACHED; ++i) {
    const int64_t gi = threadIdx.x + (int64_t)i * NT;
    if (gi < groups) emit8g(cache[i], inv, gcache[i], y, base + gi * 8);
  }
  for (int64_t gi = threadIdx.x + (int64_t)MAX_CACHED * NT; gi < groups; gi += NT) {
    float v[8];
    load8<IN_BF16>(x, base + gi * 8, v);
    emit8(v, inv, gain, gi, y, base + gi * 8);
  }
}

struct SumNormArgs {
  const float* p[16];  // the t partials, at the first row of the first run
  const float* bias;   // [h], added to the sum of the partials, or NULL
  const void* res;     // residual rows (float32 or bf16) or NULL
  float* out;          // sum rows, float32 (may be the float32 residual), or NULL
  const float* gain;
  bf16_t* y;           // normed rows (bf16), or NULL: no norm
  int64_t h;
  int64_t run_rows, run_stride;  // rows are runs of run_rows, run_stride apart
  float eps;
  int res_bf16;
};

__device__ __forceinline__ f32x4 ld_nt4(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}

// For G groups of 8 elements at e[0..G) (columns c[0..G)): x = (((p_0 + p_1)
// + ... + p_{T-1}) + bias) + residual (T = 0: the residual alone; the
// row-parallel bias is added once, after the sum), stored to out when there is one
// (non-temporal: it is next read a sublayer later).  Every load of the G
// groups is issued before the first add and store (the compiler cannot
// reorder loads past a store to a pointer it cannot tell apart).
template <int T, int G>
__device__ __forceinline__ void sum_groups(const SumNormArgs& a, const int64_t (&e)[G], const int64_t (&c)[G],
                                           const bool (&ok)[G], float (&x)[G][8]) {
  constexpr int TL = T > 0 ? T : 1;
  f32x4 lo[G][TL], hi[G][TL], rl[G], rh[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (!ok[g]) continue;
#pragma unroll
    for (int s = 0; s < T; ++s) {
      lo[g][s] = ld_nt4(a.p[s] + e[g]);
      hi[g][s] = ld_nt4(a.p[s] + e[g] + 4);
    }
    rl[g] = rh[g] = f32x4{};
    if (a.res) {
      if (a.res_bf16) {
        const u32x4 u = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(a.res) + e[g]));
        rl[g] = f32x4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xFFFF0000u),
                      __uint_as_float(u[1] << 16), __uint_as_float(u[1] & 0xFFFF0000u)};
        rh[g] = f32x4{__uint_as_float(u[2] << 16), __uint_as_float(u[2] & 0xFFFF0000u),
                      __uint_as_float(u[3] << 16), __uint_as_float(u[3] & 0xFFFF0000u)};
      } else {
        rl[g] = ld_nt4(reinterpret_cast<const float*>(a.res) + e[g]);
        rh[g] = ld_nt4(reinterpret_cast<const float*>(a.res) + e[g] + 4);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (!ok[g]) continue;
    f32x4 sl, sh;
    if constexpr (T == 0) {
      sl = rl[g];
      sh = rh[g];
    } else {
      sl = lo[g][0];
      sh = hi[g][0];
#pragma unroll
      for (int s = 1; s < T; ++s) {
        sl += lo[g][s];
        sh += hi[g][s];
      }
      if (a.bias) {
        sl += *reinterpret_cast<const f32x4*>(a.bias + c[g]);
        sh += *reinterpret_cast<const f32x4*>(a.bias + c[g] + 4);
      }
      if (a.res) {
        sl += rl[g];
        sh += rh[g];
      }
    }
    if (a.out) {
      __builtin_nontemporal_store(sl, reinterpret_cast<f32x4*>(a.out + e[g]));
      __builtin_nontemporal_store(sh, reinterpret_cast<f32x4*>(a.out + e[g] + 4));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[g][i] = sl[i];
      x[g][4 + i] = sh[i];
    }
  }
}

template <int T>
__global__ __launch_bounds__(NT) void sum_rmsnorm_kernel(SumNormArgs a) {
  // one group's loads (every partial's) in flight at a time: fewer registers
  // than two, so more rows share a CU, which measured faster (t = 8, 8192 x
  // 8192: 516 against 525 us per call back to back)
  constexpr int G = 1;
  __shared__ float red[NT / 64];
  const int64_t h = a.h;
  const int64_t r = blockIdx.x;
  const int64_t base = ((r / a.run_rows) * a.run_stride + r % a.run_rows) * h;
  const int64_t groups = h >> 3;
  float cache[MAX_CACHED][8];
  // the gains of the cached groups, loaded before the row so the
  // normalisation after the row's reduction waits on no further load
  float gcache[MAX_CACHED][8];
  if (a.y) {
#pragma unroll
    for (int i = 0; i < MAX_CACHED; ++i) {
      const int64_t gi = threadIdx.x + (int64_t)i * NT;
      if (gi < groups) load_gain8(a.gain, gi, gcache[i]);
    }
  }
  float ss = 0.0f;
#pragma unroll
  for (int i0 = 0; i0 < MAX_CACHED; i0 += G) {
    int64_t e[G], c[G];
    bool ok[G];
    float x[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int64_t gi = threadIdx.x + (int64_t)(i0 + g) * NT;
      ok[g] = gi < groups;
      c[g] = gi * 8;
      e[g] = base + c[g];
    }
    sum_groups<T, G>(a, e, c, ok, x);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (!ok[g]) continue;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        cache[i0 + g][k] = x[g][k];
        ss += x[g][k] * x[g][k];
      }
    }
  }
  for (int64_t gi = threadIdx.x + (int64_t)MAX_CACHED * NT; gi < groups; gi += NT) {
    const int64_t e[1] = {base + gi * 8}, c[1] = {gi * 8};
    const bool ok[1] = {true};
    float x[1][8];
    sum_groups<T, 1>(a, e, c, ok, x);
#pragma unroll
    for (int k = 0; k < 8; ++k) ss += x[0][k] * x[0][k];
  }
  if (!a.y) return;  // a reduce-scatter (+ residual) without a norm
  const float inv = row_inv_rms(ss, h, a.eps, red);
#pragma unroll
  for (int i = 0; i < MAX_CACHED; ++i) {
    const int64_t gi = threadIdx.x + (int64_t)i * NT;
    if (gi < groups) emit8g(cache[i], inv, gcache[i], a.y, base + gi * 8);
  }
  // rows wider than the register cache: the group's sum again (from the
  // sums this thread stored above, ordered by the barrier in row_inv_rms,
  // or recomputed when they are not stored)
  for (int64_t gi = threadIdx.x + (int64_t)MAX_CACHED * NT; gi < groups; gi += NT) {
    float v[8];
    if (a.out) {
      load8<false>(a.out, base + gi * 8, v);
    } else {
      const int64_t e[1] = {base + gi * 8}, c[1] = {gi * 8};
      const bool ok[1] = {true};
      float x[1][8];
      sum_groups<T, 1>(a, e, c, ok, x);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = x[0][k];
    }
    emit8(v, inv, a.gain, gi, a.y, base + gi * 8);
  }
}

}  // namespace

hipError_t launch_rmsnorm(int in_bf16, int64_t m, int64_t h, const void* x, const float* gain,
                          float eps, void* y, hipStream_t s) {
  if (m == 0) return hipSuccess;
  bf16_t* out = reinterpret_cast<bf16_t*>(y);
  if (in_bf16)
    hipLaunchKernelGGL(rmsnorm_kernel<true>, dim3((unsigned)m), dim3(NT), 0, s, x, gain, eps, out, h);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<false>, dim3((unsigned)m), dim3(NT), 0, s, x, gain, eps, out, h);
  return hipGetLastError();
}

hipError_t launch_sum_rmsnorm(int t, int64_t nrun, int64_t run_rows, int64_t run_stride, int64_t h,
                              const float* const* partials, const float* bias, const void* residual,
                              int residual_bf16, float* out, const float* gain, float eps, void* y,
                              hipStream_t s) {
  const int64_t m = nrun * run_rows;
  if (m == 0) return hipSuccess;
  SumNormArgs a;
  for (int i = 0; i < 16; ++i) a.p[i] = i < t ? partials[i] : nullptr;
  a.bias = bias;
  a.res = residual;
  a.out = out;
  a.gain = gain;
  a.y = reinterpret_cast<bf16_t*>(y);
  a.h = h;
  a.run_rows = run_rows;
  a.run_stride = nrun > 1 ? run_stride : run_rows;
  a.eps = eps;
  a.res_bf16 = residual_bf16;
  const dim3 grid((unsigned)m), block(NT);
  switch (t) {
#define TP_SUM_NORM_CASE(T) \
  case T: hipLaunchKernelGGL(sum_rmsnorm_kernel<T>, grid, block, 0, s, a); break;
    TP_SUM_NORM_CASE(0) TP_SUM_NORM_CASE(1) TP_SUM_NORM_CASE(2) TP_SUM_NORM_CASE(3)
    TP_SUM_NORM_CASE(4) TP_SUM_NORM_CASE(5) TP_SUM_NORM_CASE(6) TP_SUM_NORM_CASE(7)
    TP_SUM_NORM_CASE(8) TP_SUM_NORM_CASE(9) TP_SUM_NORM_CASE(10) TP_SUM_NORM_CASE(11)
    TP_SUM_NORM_CASE(12) TP_SUM_NORM_CASE(13) TP_SUM_NORM_CASE(14) TP_SUM_NORM_CASE(15)
    TP_SUM_NORM_CASE(16)
#undef TP_SUM_NORM_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tpk
