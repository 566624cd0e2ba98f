// Shard-sum: the forward all-reduce of the row-parallel output ("Tensor
// parallelism" page, sections "Matmul split" and "f and g"), computed inside
// one device.  out = (((p0 + p1) + ...) + p_{t-1}) + residual, float32,
// ascending rank order, one rounding per add.
//
// HBM-bound: every element is read t (+1) times and written once.  Each
// thread moves 16-byte vectors; the partials are streamed with non-temporal
// loads so they do not evict useful lines, the result with a non-temporal
// store.  The t partial pointers travel in the kernel arguments.
#include "common.h"
#include "kernels.h"

namespace tpk {
namespace {

constexpr int NT = 256;
constexpr int UNROLL = 4;  // float4 vectors per thread per iteration

struct SumArgs {
  const float* p[16];
  const void* res;
  float* out;
  int64_t n;
  int t;
  int res_bf16;
};

__device__ __forceinline__ f32x4 ld_nt(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}

__device__ __forceinline__ f32x4 ld_res(const SumArgs& a, int64_t e) {
  if (a.res_bf16) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(reinterpret_cast<const bf16_t*>(a.res) + e);
    return f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u),
                 __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xFFFF0000u)};
  }
  return *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.res) + e);
}

__global__ __launch_bounds__(NT) void shard_sum_kernel(SumArgs a) {
  const int64_t n4 = a.n >> 2;
  const int64_t stride = (int64_t)gridDim.x * NT;
  int64_t v = (int64_t)blockIdx.x * NT + threadIdx.x;
  // main body: UNROLL independent vectors in flight per thread
  for (; v + (UNROLL - 1) * stride < n4; v += UNROLL * stride) {
    f32x4 acc[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc[u] = ld_nt(a.p[0] + 4 * (v + u * stride));
    for (int s = 1; s < a.t; ++s) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) acc[u] += ld_nt(a.p[s] + 4 * (v + u * stride));
    }
    if (a.res) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) acc[u] += ld_res(a, 4 * (v + u * stride));
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      __builtin_nontemporal_store(acc[u], reinterpret_cast<f32x4*>(a.out + 4 * (v + u * stride)));
  }
  for (; v < n4; v += stride) {
    f32x4 acc = ld_nt(a.p[0] + 4 * v);
    for (int s = 1; s < a.t; ++s) acc += ld_nt(a.p[s] + 4 * v);
    if (a.res) acc += ld_res(a, 4 * v);
    __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(a.out + 4 * v));
  }
  // scalar tail (n % 4 elements)
  if (blockIdx.x == 0 && threadIdx.x < (a.n & 3)) {
    const int64_t e = (n4 << 2) + threadIdx.x;
    float acc = a.p[0][e];
    for (int s = 1; s < a.t; ++s) acc += a.p[s][e];
    if (a.res) {
      acc += a.res_bf16 ? bf16_to_f32(reinterpret_cast<const bf16_t*>(a.res)[e])
                        : reinterpret_cast<const float*>(a.res)[e];
    }
    a.out[e] = acc;
  }
}

}  // namespace

hipError_t launch_shard_sum(int t, int64_t n, const float* const* partials, const void* residual,
                            int residual_bf16, float* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  SumArgs a;
  for (int i = 0; i < 16; ++i) a.p[i] = i < t ? partials[i] : nullptr;
  a.res = residual;
  a.out = out;
  a.n = n;
  a.t = t;
  a.res_bf16 = residual_bf16;
  const int64_t n4 = n >> 2;
  // enough workgroups to cover the device several times, each thread
  // streaming UNROLL vectors per iteration
  int64_t blocks = (n4 + (int64_t)NT * UNROLL - 1) / ((int64_t)NT * UNROLL);
  blocks = blocks < 1 ? 1 : (blocks > 256 * 16 ? 256 * 16 : blocks);
  hipLaunchKernelGGL(shard_sum_kernel, dim3((unsigned)blocks), dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace tpk
