// Backward of the fused shard-sum + RMSNorm ("Tensor parallelism" page,
// section "f and g": f's backward is the sum of the ranks' input-gradient
// partials; the norm and the residual are replicated, so their gradients are
// taken after that sum, on every rank).
//
// Per row, with dy = ((p_0 + p_1) + ...) (the t partials in ascending rank
// order), x the norm's input, r = 1 / sqrt(mean x^2 + eps), g = gain * dy:
//   dx = r g - x r^3 (sum_c g x) / h  (+ the gradient arriving through the
//        residual path)
//   dgain = sum over rows of dy * x * r
// Rows may come as runs (run_rows rows, run_stride apart: a rank's slice of
// every sequence in the sequence-parallel form), as in the forward.
// One workgroup walks a run of consecutive rows, keeping each row's dy and x
// in registers between the row's reduction and its output (h <= 8192), and
// accumulating its columns' dgain terms across the run; a second kernel sums
// the runs' dgain partials in a fixed order.  No atomics.
// HBM-bound: t + 1 (+1 residual) float32 reads and one or two writes per element.
#include "common.h"
#include "kernels.h"

namespace tpk {
namespace {

constexpr int NT = 256;
constexpr int MAXC = 4;  // 8-element groups per thread (h <= 8192)

struct NormBwdArgs {
  const float* p[16];  // the t dy partials, [m, h] float32
  const void* x;       // the norm's input rows, float32 or bf16
  const float* gain;   // [h] or NULL (gain 1)
  const void* res;     // gradient through the residual path (float32 or bf16), or NULL
  float* dx;           // float32 rows, or NULL
  bf16_t* dx_bf16;     // bf16 rows, or NULL
  float* dg_part;      // [blocks, h] dgain partials, or NULL
  int64_t m, h, rows_per_block;
  int64_t run_rows, run_stride;  // logical row r is row (r / run_rows) * run_stride + r % run_rows
  float eps;
  int x_bf16, res_bf16;
};

__device__ __forceinline__ void load8f(const void* p, int64_t e, bool bf16, float (&v)[8]) {
  if (bf16) {
    const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(p) + e));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  } else {
    const float* f = reinterpret_cast<const float*>(p) + e;
    const f32x4 lo = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(f));
    const f32x4 hi = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(f + 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = lo[i];
      v[4 + i] = hi[i];
    }
  }
}

template <int T>
__global__ __launch_bounds__(NT) void sum_rmsnorm_bwd_kernel(NormBwdArgs a) {
  __shared__ float red[2][2][NT / 64];  // [row parity][sum][wave]
  __shared__ __attribute__((aligned(16))) float sgain[MAXC * NT * 8];  // the gain, read back per row
  const int64_t h = a.h, groups = h >> 3;
  const int64_t r0 = (int64_t)blockIdx.x * a.rows_per_block;
  const int64_t r1 = min(r0 + a.rows_per_block, a.m);
  float dg[MAXC][8];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int64_t gi = threadIdx.x + (int64_t)i * NT;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      // each thread reads back only the columns it wrote: no barrier needed
      sgain[gi * 8 + k] = (a.gain && gi < groups) ? a.gain[gi * 8 + k] : 1.0f;
      dg[i][k] = 0.0f;
    }
  }
  auto gain8 = [&](int i, float (&g)[8]) {
    const int64_t gi = threadIdx.x + (int64_t)i * NT;
    const f32x4 lo = *reinterpret_cast<const f32x4*>(&sgain[gi * 8]);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(&sgain[gi * 8 + 4]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      g[k] = lo[k];
      g[4 + k] = hi[k];
    }
  };
  for (int64_t r = r0; r < r1; ++r) {
    const int64_t base = ((r / a.run_rows) * a.run_stride + r % a.run_rows) * h;
    float dy[MAXC][8], xv[MAXC][8], rv[MAXC][8];
    float sxx = 0.0f, sgx = 0.0f;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int64_t gi = threadIdx.x + (int64_t)i * NT;
      if (gi >= groups) continue;
      const int64_t e = base + gi * 8;
      f32x4 lo[T], hi[T];
#pragma unroll
      for (int s = 0; s < T; ++s) {
        lo[s] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.p[s] + e));
        hi[s] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.p[s] + e + 4));
      }
      load8f(a.x, e, a.x_bf16 != 0, xv[i]);
      // the residual gradient is loaded with the row's other inputs: one
      // memory round trip per row
#pragma unroll
      for (int k = 0; k < 8; ++k) rv[i][k] = 0.0f;
      if (a.res) load8f(a.res, e, a.res_bf16 != 0, rv[i]);
      f32x4 sl = lo[0], sh = hi[0];
#pragma unroll
      for (int s = 1; s < T; ++s) {
        sl += lo[s];
        sh += hi[s];
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        dy[i][k] = sl[k];
        dy[i][4 + k] = sh[k];
      }
      float gn[8];
      gain8(i, gn);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        sxx += xv[i][k] * xv[i][k];
        sgx += gn[k] * dy[i][k] * xv[i][k];
      }
    }
    // both row sums across the workgroup: the wave's butterfly, then the 4 waves
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      sxx += __shfl_xor(sxx, off);
      sgx += __shfl_xor(sgx, off);
    }
    float(&rb)[2][NT / 64] = red[r & 1];
    if ((threadIdx.x & 63) == 0) {
      rb[0][threadIdx.x >> 6] = sxx;
      rb[1][threadIdx.x >> 6] = sgx;
    }
    __syncthreads();
    const float txx = rb[0][0] + rb[0][1] + rb[0][2] + rb[0][3];
    const float tgx = rb[1][0] + rb[1][1] + rb[1][2] + rb[1][3];
    const float rr = 1.0f / sqrtf(txx / (float)h + a.eps);
    const float coef = rr * rr * rr * tgx / (float)h;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int64_t gi = threadIdx.x + (int64_t)i * NT;
      if (gi >= groups) continue;
      const int64_t e = base + gi * 8;
      float o[8], gn[8];
      gain8(i, gn);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        o[k] = (rr * (gn[k] * dy[i][k]) - xv[i][k] * coef) + rv[i][k];
        dg[i][k] += dy[i][k] * (xv[i][k] * rr);
      }
      if (a.dx) {  // the residual stream's gradient, next read a sublayer later: non-temporal
        __builtin_nontemporal_store(f32x4{o[0], o[1], o[2], o[3]}, reinterpret_cast<f32x4*>(a.dx + e));
        __builtin_nontemporal_store(f32x4{o[4], o[5], o[6], o[7]}, reinterpret_cast<f32x4*>(a.dx + e + 4));
      }
      if (a.dx_bf16)
        *reinterpret_cast<u32x4*>(a.dx_bf16 + e) =
            u32x4{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])};
    }
  }
  if (!a.dg_part) return;
  float* dst = a.dg_part + (int64_t)blockIdx.x * h;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int64_t gi = threadIdx.x + (int64_t)i * NT;
    if (gi >= groups) continue;
    *reinterpret_cast<f32x4*>(dst + gi * 8) = f32x4{dg[i][0], dg[i][1], dg[i][2], dg[i][3]};
    *reinterpret_cast<f32x4*>(dst + gi * 8 + 4) = f32x4{dg[i][4], dg[i][5], dg[i][6], dg[i][7]};
  }
}

// dgain[c] = the blocks' partials summed in a fixed order: 16 interleaved
// slices (slice s takes blocks s, s + 16, ... in ascending order, 8 loads in
// flight), then the 16 slice sums in slice order.  16 columns per workgroup.
__global__ __launch_bounds__(NT) void dgain_sum_kernel(const float* part, int64_t blocks, int64_t h, float* dgain) {
  __shared__ float red[16][17];
  const int cl = threadIdx.x & 15, sl = threadIdx.x >> 4;
  const int64_t c = (int64_t)blockIdx.x * 16 + cl;
  float s = 0.0f;
  if (c < h) {
    int64_t b = sl;
    for (; b + 16 * 7 < blocks; b += 16 * 8) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = part[(b + 16 * i) * h + c];
#pragma unroll
      for (int i = 0; i < 8; ++i) s += v[i];
    }
    for (; b < blocks; b += 16) s += part[b * h + c];
  }
  red[sl][cl] = s;
  __syncthreads();
  if (sl == 0 && c < h) {
    float tot = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) tot += red[k][cl];
    dgain[c] = tot;
  }
}

}  // namespace

// Rows per workgroup: runs of ceil(m / 1024) rows when dgain is wanted (at
// most 1024 dgain partials), else one row per workgroup.
int64_t norm_bwd_rows_per_block(int64_t m, bool dgain) { return dgain ? (m + 1023) / 1024 : 1; }

int64_t norm_bwd_blocks(int64_t m) {
  const int64_t rpb = norm_bwd_rows_per_block(m, true);
  return (m + rpb - 1) / rpb;
}

hipError_t launch_sum_rmsnorm_bwd(int t, int64_t nrun, int64_t run_rows, int64_t run_stride, int64_t h,
                                  const float* const* partials, const void* x, int x_bf16, const float* gain,
                                  float eps, const void* res, int res_bf16, float* dx, void* dx_bf16, float* dgain,
                                  float* ws, hipStream_t s) {
  const int64_t m = nrun * run_rows;
  if (m == 0) return hipSuccess;
  if (t < 1 || t > 16 || h % 8 != 0 || h > (int64_t)MAXC * NT * 8) return hipErrorInvalidValue;
  NormBwdArgs a;
  for (int i = 0; i < 16; ++i) a.p[i] = i < t ? partials[i] : nullptr;
  a.x = x;
  a.gain = gain;
  a.res = res;
  a.dx = dx;
  a.dx_bf16 = reinterpret_cast<bf16_t*>(dx_bf16);
  a.dg_part = dgain ? ws : nullptr;
  a.m = m;
  a.h = h;
  a.rows_per_block = norm_bwd_rows_per_block(m, dgain != nullptr);
  a.run_rows = run_rows;
  a.run_stride = nrun > 1 ? run_stride : run_rows;
  a.eps = eps;
  a.x_bf16 = x_bf16;
  a.res_bf16 = res_bf16;
  const int64_t blocks = (m + a.rows_per_block - 1) / a.rows_per_block;
  const dim3 grid((unsigned)blocks), block(NT);
  switch (t) {
#define TP_NORM_BWD_CASE(T) \
  case T: hipLaunchKernelGGL(sum_rmsnorm_bwd_kernel<T>, grid, block, 0, s, a); break;
    TP_NORM_BWD_CASE(1) TP_NORM_BWD_CASE(2) TP_NORM_BWD_CASE(3) TP_NORM_BWD_CASE(4)
    TP_NORM_BWD_CASE(5) TP_NORM_BWD_CASE(6) TP_NORM_BWD_CASE(7) TP_NORM_BWD_CASE(8)
    TP_NORM_BWD_CASE(9) TP_NORM_BWD_CASE(10) TP_NORM_BWD_CASE(11) TP_NORM_BWD_CASE(12)
    TP_NORM_BWD_CASE(13) TP_NORM_BWD_CASE(14) TP_NORM_BWD_CASE(15) TP_NORM_BWD_CASE(16)
#undef TP_NORM_BWD_CASE
    default: return hipErrorInvalidValue;
  }
  if (dgain)
    hipLaunchKernelGGL(dgain_sum_kernel, dim3((unsigned)((h + 15) / 16)), dim3(NT), 0, s, ws, blocks, h, dgain);
  return hipGetLastError();
}

}  // namespace tpk
