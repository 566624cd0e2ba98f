// Shard-sum: the forward all-reduce of the row-parallel output ("Tensor
// parallelism" page, sections "Matmul split" and "f and g"), computed inside
// one device.  out = (((p0 + p1) + ...) + p_{t-1}) + residual, float32,
// ascending rank order, one rounding per add.
//
// HBM-bound: every element is read t (+1) times and written once.  A
// workgroup owns a 16 KiB stretch of every input (1024 float4), so each of
// the t + 1 streams is read in long contiguous runs; a thread issues the
// loads of all its float4 of every input before the first add, so many bytes
// are in flight.  Inputs are streamed with non-temporal loads so they do not
// evict useful lines, the result with a non-temporal store.  The t partial
// pointers travel in the kernel arguments.  (Measured at 8192 x 8192 x 8
// partials with the Infinity Cache flushed: 75% of 8 TB/s, against 69% for one
// float4 per thread over a flat grid.)
#include "common.h"
#include "kernels.h"

namespace tpk {
namespace {

constexpr int NT = 256;
constexpr int PER_THREAD = 4;                 // float4 per thread per input per chunk
constexpr int CHUNK = NT * PER_THREAD;        // float4 per workgroup chunk
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

// T is the number of partials, a compile-time constant so all loads of a
// pass (T x D float4, plus the residual) are issued before the first add.
// D = float4 per thread and input per pass: the whole chunk at once up to 8
// partials, half of it beyond (register budget).
template <int T>
__global__ __launch_bounds__(NT) void shard_sum_kernel(SumArgs a) {
  constexpr int D = T <= 8 ? PER_THREAD : PER_THREAD / 2;
  const int64_t n4 = a.n >> 2;
  const int64_t nch = (n4 + CHUNK - 1) / CHUNK;
  for (int64_t c = blockIdx.x; c < nch; c += gridDim.x) {
    const int64_t c0 = c * CHUNK + threadIdx.x;
#pragma unroll
    for (int it = 0; it < PER_THREAD; it += D) {
      f32x4 in[T][D], r[D];
#pragma unroll
      for (int u = 0; u < D; ++u) {
        const int64_t v = c0 + (int64_t)(it + u) * NT;
        const bool ok = v < n4;
#pragma unroll
        for (int s = 0; s < T; ++s) in[s][u] = ok ? ld_nt(a.p[s] + 4 * v) : f32x4{};
        r[u] = (ok && a.res) ? ld_res(a, 4 * v) : f32x4{};
      }
#pragma unroll
      for (int u = 0; u < D; ++u) {
        const int64_t v = c0 + (int64_t)(it + u) * NT;
        if (v >= n4) continue;
        f32x4 acc = in[0][u];
#pragma unroll
        for (int s = 1; s < T; ++s) acc += in[s][u];
        if (a.res) acc += r[u];
        __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(a.out + 4 * v));
      }
    }
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
  const int64_t nch = ((n >> 2) + CHUNK - 1) / CHUNK;
  int64_t blocks = nch < 1 ? 1 : (nch > MAX_BLOCKS ? MAX_BLOCKS : nch);
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
