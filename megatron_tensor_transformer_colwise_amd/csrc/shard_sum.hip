// Shard-sum: the forward all-reduce of the row-parallel output ("Tensor
// parallelism" page, sections "Matmul split" and "f and g"), computed inside
// one device.  out = (((p0 + p1) + ...) + p_{t-1}) + residual, float32,
// ascending rank order, one rounding per add.
//
// HBM-bound: every element is read t (+1) times and written once.  Each
// thread moves 16-byte vectors; the inputs are streamed with non-temporal
// loads so they do not evict useful lines, the result with a non-temporal
// store.  The t partial pointers travel in the kernel arguments.
#include "common.h"
#include "kernels.h"

namespace tpk {
namespace {

constexpr int NT = 256;
constexpr int UNROLL = 1;             // float4 vectors per thread per iteration
constexpr int64_t MAX_BLOCKS = 1 << 20;

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
    const u32x2 v = __builtin_nontemporal_load(
        reinterpret_cast<const u32x2*>(reinterpret_cast<const bf16_t*>(a.res) + e));
    return f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u),
                 __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xFFFF0000u)};
  }
  return ld_nt(reinterpret_cast<const float*>(a.res) + e);
}

// T is the number of partials, a compile-time constant so every load of an
// iteration (T x UNROLL vectors, plus the residual) is issued before the first
// add needs one: the sum is bound by how many bytes are in flight.
template <int T>
__global__ __launch_bounds__(NT) void shard_sum_kernel(SumArgs a) {
  const int64_t n4 = a.n >> 2;
  const int64_t stride = (int64_t)gridDim.x * NT;
  int64_t v = (int64_t)blockIdx.x * NT + threadIdx.x;
  for (; v + (UNROLL - 1) * stride < n4; v += UNROLL * stride) {
    f32x4 in[T][UNROLL];
#pragma unroll
    for (int s = 0; s < T; ++s)
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) in[s][u] = ld_nt(a.p[s] + 4 * (v + u * stride));
    f32x4 r[UNROLL];
    if (a.res) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) r[u] = ld_res(a, 4 * (v + u * stride));
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      f32x4 acc = in[0][u];
#pragma unroll
      for (int s = 1; s < T; ++s) acc += in[s][u];
      if (a.res) acc += r[u];
      __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(a.out + 4 * (v + u * stride)));
    }
  }
  for (; v < n4; v += stride) {
    f32x4 acc = ld_nt(a.p[0] + 4 * v);
#pragma unroll
    for (int s = 1; s < T; ++s) acc += ld_nt(a.p[s] + 4 * v);
    if (a.res) acc += ld_res(a, 4 * v);
    __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(a.out + 4 * v));
  }
  // scalar tail (n % 4 elements)
  if (blockIdx.x == 0 && threadIdx.x < (a.n & 3)) {
    const int64_t e = (n4 << 2) + threadIdx.x;
    float acc = a.p[0][e];
#pragma unroll
    for (int s = 1; s < T; ++s) acc += a.p[s][e];
    if (a.res) {
      acc += a.res_bf16 ? bf16_to_f32(reinterpret_cast<const bf16_t*>(a.res)[e])
                        : reinterpret_cast<const float*>(a.res)[e];
    }
    a.out[e] = acc;
  }
}

template <int T>
void launch_t(const SumArgs& a, int64_t blocks, hipStream_t s) {
  hipLaunchKernelGGL(shard_sum_kernel<T>, dim3((unsigned)blocks), dim3(NT), 0, s, a);
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
  // one vector per thread (measured fastest: many short-lived waves keep the
  // most bytes in flight); a grid-stride loop only beyond 2^28 vectors
  int64_t blocks = (n4 + (int64_t)NT * UNROLL - 1) / ((int64_t)NT * UNROLL);
  blocks = blocks < 1 ? 1 : (blocks > MAX_BLOCKS ? MAX_BLOCKS : blocks);
  switch (t) {
    case 1: launch_t<1>(a, blocks, s); break;
    case 2: launch_t<2>(a, blocks, s); break;
    case 3: launch_t<3>(a, blocks, s); break;
    case 4: launch_t<4>(a, blocks, s); break;
    case 5: launch_t<5>(a, blocks, s); break;
    case 6: launch_t<6>(a, blocks, s); break;
    case 7: launch_t<7>(a, blocks, s); break;
    case 8: launch_t<8>(a, blocks, s); break;
    case 9: launch_t<9>(a, blocks, s); break;
    case 10: launch_t<10>(a, blocks, s); break;
    case 11: launch_t<11>(a, blocks, s); break;
    case 12: launch_t<12>(a, blocks, s); break;
    case 13: launch_t<13>(a, blocks, s); break;
    case 14: launch_t<14>(a, blocks, s); break;
    case 15: launch_t<15>(a, blocks, s); break;
    case 16: launch_t<16>(a, blocks, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tpk
