// float32 GEMM with the same epilogues as the bf16 one (no nonlinearity, GeLU,
// SwiGLU), for small float32 checks such as the worked example of the "Tensor
// parallelism" page (section "MLP"), whose tensors are float32.
//
//   out[m, n] = epi( sum_k x[m, k] * w[row(n), k] )
//
// 64 x 64 output tile per workgroup, 4 x 4 outputs per thread, k staged through
// LDS 16 at a time.  Vector float32 FMAs (no matrix cores): these shapes are
// tiny, and the products must stay float32 end to end.
#include "common.h"
#include "kernels.h"

namespace tpk {
namespace {

constexpr int T = 64;
constexpr int TK = 16;
constexpr int NT = 256;

template <int EPI>
__global__ __launch_bounds__(NT) void gemm_f32_kernel(const float* x, const float* w, float* out,
                                                      int64_t M, int64_t N, int64_t K, int64_t lda,
                                                      const float* bias) {
  constexpr bool DUAL = EPI == EPI_SWIGLU;
  __shared__ float xs[TK][T + 1];
  __shared__ float ws[DUAL ? 2 : 1][TK][T + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * T, n0 = (int64_t)blockIdx.x * T;
  float acc[DUAL ? 2 : 1][4][4] = {};
  for (int64_t k0 = 0; k0 < K; k0 += TK) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = threadIdx.x + e * NT;
      const int r = idx >> 4, c = idx & 15;
      const bool kin = k0 + c < K;
      xs[c][r] = (kin && m0 + r < M) ? x[(m0 + r) * lda + k0 + c] : 0.0f;
      ws[0][c][r] = (kin && n0 + r < N) ? w[(n0 + r) * K + k0 + c] : 0.0f;
      if (DUAL) ws[DUAL ? 1 : 0][c][r] = (kin && n0 + r < N) ? w[(N + n0 + r) * K + k0 + c] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b[DUAL ? 2 : 1][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[kk][ty * 4 + i];
#pragma unroll
      for (int q = 0; q < (DUAL ? 2 : 1); ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) b[q][j] = ws[q][kk][tx * 4 + j];
#pragma unroll
      for (int q = 0; q < (DUAL ? 2 : 1); ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[q][i][j] = fmaf(a[i], b[q][j], acc[q][i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = m0 + ty * 4 + i;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + tx * 4 + j;
      if (col >= N) continue;
      float v = acc[0][i][j];
      if (bias) v += bias[col];
      if (EPI == EPI_GELU) v = gelu_erf(v);
      if (EPI == EPI_SWIGLU) v = silu(v) * (acc[DUAL ? 1 : 0][i][j] + (bias ? bias[N + col] : 0.0f));
      out[row * N + col] = v;
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(int epi, int64_t M, int64_t N, int64_t K, const float* x, const float* w,
                           float* out, hipStream_t s, const float* bias, int64_t lda) {
  if (M == 0 || N == 0) return hipSuccess;
  if (lda <= 0) lda = K;
  dim3 grid((unsigned)((N + T - 1) / T), (unsigned)((M + T - 1) / T)), block(NT);
  switch (epi) {
    case EPI_F32:
    case EPI_BF16:
      hipLaunchKernelGGL(gemm_f32_kernel<EPI_F32>, grid, block, 0, s, x, w, out, M, N, K, lda, bias);
      break;
    case EPI_GELU:
      hipLaunchKernelGGL(gemm_f32_kernel<EPI_GELU>, grid, block, 0, s, x, w, out, M, N, K, lda, bias);
      break;
    case EPI_SWIGLU:
      hipLaunchKernelGGL(gemm_f32_kernel<EPI_SWIGLU>, grid, block, 0, s, x, w, out, M, N, K, lda, bias);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tpk
