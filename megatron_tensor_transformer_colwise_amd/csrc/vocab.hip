// Vocabulary-parallel embedding and cross-entropy ("Tensor parallelism" page,
// section "Embedding and output layer": the embedding matrix is split along
// the vocabulary, and instead of gathering the output logits (b x s x v
// values) every rank computes, from its own slice of the logits, the maximum
// and the sum the cross-entropy needs, so only b x s values are exchanged;
// transformers "Tensor parallelism" page, EmbeddingParallel: a vocabulary-
// sharded lookup sums the ranks' partial lookups, a hidden-sharded one gathers
// their column slices).
//
// All three kernels are HBM-bound and run one workgroup (or thread) per token:
//   embedding lookup   bytes = m * w * (2 read if the id is the rank's + 4 written)
//   local statistics   bytes = m * v_shard * 4 read (one pass: online max/sum)
//   combination        bytes = m * t * 16 read + m * 4 written
#include "common.h"
#include "kernels.h"

namespace tpk {
namespace {

constexpr int NT = 256;

// out[i, 0:w] = table[ids[i] - v_start, 0:w] (bf16 -> float32) when the id is
// one of the rank's rows [v_start, v_start + v_rows), else zeros.  One
// workgroup per token, 8 values per thread per step.
__global__ __launch_bounds__(NT) void embedding_kernel(const int32_t* ids, const bf16_t* table, int64_t w,
                                                       int64_t v_start, int64_t v_rows, float* out,
                                                       int64_t ld) {
  const int64_t i = blockIdx.x;
  const int64_t id = (int64_t)ids[i] - v_start;
  const bool mine = id >= 0 && id < v_rows;
  float* const o = out + i * ld;
  const bf16_t* const src = table + (mine ? id : 0) * w;
  for (int64_t c = (int64_t)threadIdx.x * 8; c < w; c += NT * 8) {
    f32x4 lo = {}, hi = {};
    if (mine) {
      const u32x4 u = *reinterpret_cast<const u32x4*>(src + c);
      lo = f32x4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xFFFF0000u),
                 __uint_as_float(u[1] << 16), __uint_as_float(u[1] & 0xFFFF0000u)};
      hi = f32x4{__uint_as_float(u[2] << 16), __uint_as_float(u[2] & 0xFFFF0000u),
                 __uint_as_float(u[3] << 16), __uint_as_float(u[3] & 0xFFFF0000u)};
    }
    *reinterpret_cast<f32x4*>(o + c) = lo;
    *reinterpret_cast<f32x4*>(o + c + 4) = hi;
  }
}

// Running maximum and sum of exp(x - max) of a stream of values, merged in a
// fixed order.
struct MaxSum {
  float m, s;
};

__device__ __forceinline__ MaxSum merge(MaxSum a, MaxSum b) {
  if (b.m == -INFINITY) return a;
  if (a.m == -INFINITY) return b;
  const float m = fmaxf(a.m, b.m);
  return MaxSum{m, a.s * __expf(a.m - m) + b.s * __expf(b.m - m)};
}

// stats[i] = {max_j x_j, sum_j exp(x_j - max), x_label (if the rank holds the
// label), 1 if it does else 0} over the rank's logits x = logits[i, 0:n).
// One workgroup per token; each thread folds its float4s into a running
// (max, sum), then the wave and the 4 waves merge in a fixed tree.
__global__ __launch_bounds__(NT) void ce_stats_kernel(const float* logits, int64_t n, int64_t v_start,
                                                      const int32_t* labels, float* stats) {
  __shared__ MaxSum red[NT / 64];
  const int64_t i = blockIdx.x;
  const float* const row = logits + i * n;
  MaxSum acc{-INFINITY, 0.0f};
  for (int64_t c = (int64_t)threadIdx.x * 4; c < n; c += NT * 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(row + c);
    const float m4 = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
    const float s4 = __expf(v[0] - m4) + __expf(v[1] - m4) + __expf(v[2] - m4) + __expf(v[3] - m4);
    acc = merge(acc, MaxSum{m4, s4});
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const MaxSum o{__shfl_xor(acc.m, off), __shfl_xor(acc.s, off)};
    // both lanes of a pair merge in the same (lower lane first) order
    acc = ((threadIdx.x & off) == 0) ? merge(acc, o) : merge(o, acc);
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    MaxSum t = red[0];
#pragma unroll
    for (int k = 1; k < NT / 64; ++k) t = merge(t, red[k]);
    const int64_t lab = (int64_t)labels[i] - v_start;
    const bool mine = lab >= 0 && lab < n;
    *reinterpret_cast<f32x4*>(stats + i * 4) = f32x4{t.m, t.s, mine ? row[lab] : 0.0f, mine ? 1.0f : 0.0f};
  }
}

// mean[0] = sum of loss over the tokens with a label / their count (0 if
// none); labels tell which tokens count.  One workgroup, fixed order: each
// thread sums a strided set, then a tree over the threads.
__global__ __launch_bounds__(1024) void mean_kernel(const float* loss, const int32_t* labels,
                                                    int64_t v, int64_t m, float* mean) {
  __shared__ float s_sum[1024], s_cnt[1024];
  float a = 0.0f, c = 0.0f;
  for (int64_t i = threadIdx.x; i < m; i += 1024) {
    if (labels[i] >= 0 && labels[i] < v) {
      a += loss[i];
      c += 1.0f;
    }
  }
  s_sum[threadIdx.x] = a;
  s_cnt[threadIdx.x] = c;
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) {
      s_sum[threadIdx.x] += s_sum[threadIdx.x + off];
      s_cnt[threadIdx.x] += s_cnt[threadIdx.x + off];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) mean[0] = s_cnt[0] > 0.0f ? s_sum[0] / s_cnt[0] : 0.0f;
}

struct PtrArray {
  const float* p[16];
};

// loss[i] = log(sum_r s_r exp(m_r - M)) + M - x_label, M = max_r m_r, ranks
// taken in ascending order; a token whose label no rank holds (ignored, e.g.
// a negative label) gets loss 0.  One thread per token; the t statistics
// pointers travel in the kernel arguments.
__global__ __launch_bounds__(NT) void ce_combine_kernel(PtrArray st, int t, int64_t m, float* loss) {
  const int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (i >= m) return;
  float mx = -INFINITY, z = 0.0f, owners = 0.0f;
  for (int r = 0; r < t; ++r) {
    const f32x4 s = *reinterpret_cast<const f32x4*>(st.p[r] + i * 4);
    mx = fmaxf(mx, s[0]);
    z += s[2];
    owners += s[3];
  }
  float sum = 0.0f;
  for (int r = 0; r < t; ++r) {
    const f32x4 s = *reinterpret_cast<const f32x4*>(st.p[r] + i * 4);
    sum += s[1] * __expf(s[0] - mx);
  }
  loss[i] = owners == 1.0f ? __logf(sum) + mx - z : 0.0f;
}

}  // namespace

hipError_t launch_embedding(int64_t m, int64_t w, int64_t v_start, int64_t v_rows, const int32_t* ids,
                            const void* table, float* out, int64_t ld, hipStream_t s) {
  if (m == 0) return hipSuccess;
  hipLaunchKernelGGL(embedding_kernel, dim3((unsigned)m), dim3(NT), 0, s, ids,
                     reinterpret_cast<const bf16_t*>(table), w, v_start, v_rows, out, ld);
  return hipGetLastError();
}

hipError_t launch_ce_stats(int64_t m, int64_t n, int64_t v_start, const float* logits, const int32_t* labels,
                           float* stats, hipStream_t s) {
  if (m == 0) return hipSuccess;
  hipLaunchKernelGGL(ce_stats_kernel, dim3((unsigned)m), dim3(NT), 0, s, logits, n, v_start, labels, stats);
  return hipGetLastError();
}

hipError_t launch_ce_combine(int t, int64_t m, const float* const* stats, float* loss, const int32_t* labels,
                             int64_t v, float* mean, hipStream_t s) {
  if (m == 0) return hipSuccess;
  PtrArray a;
  for (int r = 0; r < 16; ++r) a.p[r] = r < t ? stats[r] : nullptr;
  hipLaunchKernelGGL(ce_combine_kernel, dim3((unsigned)((m + NT - 1) / NT)), dim3(NT), 0, s, a, t, m,
                     loss);
  if (mean) hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(1024), 0, s, loss, labels, v, m, mean);
  return hipGetLastError();
}

}  // namespace tpk
