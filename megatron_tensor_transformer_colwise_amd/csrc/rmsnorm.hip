// Replicated RMSNorm (every rank normalises the full activation; "Tensor
// parallelism" page, section "f and g": norms are replicated):
//   y[r, c] = bf16( x[r, c] / sqrt(mean_c x[r, c]^2 + eps) * gain[c] )
// One workgroup per row; 8 elements per thread per step; float32 math.
// HBM-bound: one read of x, one bf16 write of y.
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

template <bool IN_BF16>
__global__ __launch_bounds__(NT) void rmsnorm_kernel(const void* x, const float* gain, float eps,
                                                     bf16_t* y, int64_t h) {
  __shared__ float red[NT / 64];
  const int64_t row = blockIdx.x;
  const int64_t base = row * h;
  const int64_t groups = h >> 3;
  float cache[MAX_CACHED][8];
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < MAX_CACHED; ++i) {
    const int64_t gi = threadIdx.x + (int64_t)i * NT;
    if (gi < groups) {
      load8<IN_BF16>(x, base + gi * 8, cache[i]);
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
  // block reduction: wave (xor shuffles), then across the 4 waves
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float inv = 1.0f / sqrtf(tot / (float)h + eps);

  auto emit = [&](int64_t gi, const float (&v)[8]) {
    float gv[8];
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
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = pack_bf16x2(v[2 * i] * inv * gv[2 * i], v[2 * i + 1] * inv * gv[2 * i + 1]);
    *reinterpret_cast<u32x4*>(y + base + gi * 8) = o;
  };
#pragma unroll
  for (int i = 0; i < MAX_CACHED; ++i) {
    const int64_t gi = threadIdx.x + (int64_t)i * NT;
    if (gi < groups) emit(gi, cache[i]);
  }
  for (int64_t gi = threadIdx.x + (int64_t)MAX_CACHED * NT; gi < groups; gi += NT) {
    float v[8];
    load8<IN_BF16>(x, base + gi * 8, v);
    emit(gi, v);
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

}  // namespace tpk
