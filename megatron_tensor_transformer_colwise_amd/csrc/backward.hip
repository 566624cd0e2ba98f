// Pieces of the MLP shard's backward pass ("Tensor parallelism" page,
// section "f and g": g's backward is the identity, so every rank receives the
// whole output gradient dZ; f's backward is an all-reduce of the ranks'
// input-gradient partials).  The GEMMs of the backward pass run on the bf16
// GEMM with both operands contiguous along the contraction; these kernels
// supply what it needs around them:
//
//   transpose           [rows, cols] bf16 -> [cols, rows] bf16 (a token-major
//                       activation or a weight to the layout whose reduction
//                       dimension is contiguous); HBM-bound, bytes = 4 rows cols;
//                       16-byte accesses when both sizes are multiples of 8
//   activation backward from the recomputed pre-activation and dY:
//                       GeLU:   dPre = dY * GeLU'(pre), Y = GeLU(pre)
//                       SwiGLU: pre = [g | u], Y = SiLU(g) u,
//                               dPre = [dY u SiLU'(g) | dY SiLU(g)]
//                       HBM-bound, bytes = (2 or 4 read + 2 or 4 + 2 written) per element
#include "common.h"
#include "kernels.h"

namespace tpk {
namespace {

constexpr int TT = 64;   // transpose tile
constexpr int NT = 256;

// 64 x 64 tiles through LDS (padded rows against bank conflicts); each thread
// moves 16 elements in and 16 out, 2-byte accesses coalesced along rows of
// the source and of the destination.
__global__ __launch_bounds__(NT) void transpose_kernel(const bf16_t* src, bf16_t* dst, int64_t rows,
                                                       int64_t cols) {
  __shared__ bf16_t tile[TT][TT + 2];
  const int64_t r0 = (int64_t)blockIdx.y * TT, c0 = (int64_t)blockIdx.x * TT;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < TT / 4; ++k) {
    const int r = ty + 4 * k;
    if (r0 + r < rows && c0 + tx < cols) tile[r][tx] = src[(r0 + r) * cols + c0 + tx];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < TT / 4; ++k) {
    const int c = ty + 4 * k;
    if (c0 + c < cols && r0 + tx < rows) dst[(c0 + c) * rows + r0 + tx] = tile[tx][c];
  }
}

// The same with 16-byte accesses, generalised for the attention backward's
// layouts.  Per batch z = z1 * n2 + z2 (blockIdx.z; src starts at
// z1 * src_bs1 + z2 * src_bs2, dst at z1 * dst_bs1 + z2 * dst_bs2):
//   dst[c * ldd + r] = r < rows_in ? src[r * lds + c] : 0,  r < rows_out, c < cols
// A thread reads 8 consecutive elements of a source row into LDS and writes 8
// consecutive elements of a destination row, gathered down an LDS column.
// The 16-byte chunk k of tile row r sits at chunk position k ^ ((r / 8) % 8),
// so the rows 8 apart that one column read touches fall in different banks.
// rows_out must be a multiple of 8; a source row is read in chunks of 8 from
// c = 0, so up to 7 elements past cols are read (the caller keeps them in
// bounds: cols a multiple of 8, or padding after each row).
__global__ __launch_bounds__(NT) void transpose16_kernel(const bf16_t* src, bf16_t* dst, int64_t rows_in,
                                                         int64_t rows_out, int64_t cols, int64_t lds, int64_t ldd,
                                                         int n2, int64_t src_bs1, int64_t src_bs2, int64_t dst_bs1,
                                                         int64_t dst_bs2) {
  __shared__ __attribute__((aligned(16))) bf16_t tile[TT][TT];
  const int64_t z1 = blockIdx.z / n2, z2 = blockIdx.z % n2;
  src += z1 * src_bs1 + z2 * src_bs2;
  dst += z1 * dst_bs1 + z2 * dst_bs2;
  const int64_t r0 = (int64_t)blockIdx.y * TT, c0 = (int64_t)blockIdx.x * TT;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int idx = threadIdx.x + k * NT;  // 512 chunks of 8: 64 rows x 8 chunks
    const int r = idx >> 3, ch = (idx & 7) * 8;
    u32x4 v = {0, 0, 0, 0};
    if (r0 + r < rows_in && c0 + ch < cols) v = *reinterpret_cast<const u32x4*>(src + (r0 + r) * lds + c0 + ch);
    *reinterpret_cast<u32x4*>(&tile[r][(((ch >> 3) ^ ((r >> 3) & 7)) << 3)]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int idx = threadIdx.x + k * NT;  // destination: 64 rows (source columns) x 8 chunks
    const int c = idx >> 3, rr = (idx & 7) * 8;
    if (c0 + c < cols && r0 + rr < rows_out) {
      // rows rr .. rr + 7 share rr / 8, so one swizzled column position
      const int cs = ((((c >> 3) ^ ((rr >> 3) & 7)) << 3) | (c & 7));
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = (uint32_t)tile[rr + 2 * e][cs] | ((uint32_t)tile[rr + 2 * e + 1][cs] << 16);
      *reinterpret_cast<u32x4*>(dst + (c0 + c) * ldd + r0 + rr) = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
}

__device__ __forceinline__ float gelu_grad(float x) {
  // d/dx [x Phi(x)] = Phi(x) + x phi(x)
  const float cdf = 0.5f * (1.0f + erff(x * 0.70710678118654752440f));
  const float pdf = 0.39894228040143267794f * __expf(-0.5f * x * x);
  return cdf + x * pdf;
}

// One thread per 8 consecutive elements of a row of dY (n columns).
template <bool SWIGLU>
__global__ __launch_bounds__(NT) void act_backward_kernel(const bf16_t* pre, const bf16_t* dy, bf16_t* dpre,
                                                          bf16_t* y, int64_t m, int64_t n) {
  const int64_t groups = n >> 3;
  const int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (e >= m * groups) return;
  const int64_t row = e / groups, c = (e - row * groups) * 8;
  const int64_t pw = SWIGLU ? 2 * n : n;  // pre-activation row width
  float d[8], g[8], u[8];
  auto ld8 = [](const bf16_t* p, float (&v)[8]) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  };
  auto st8 = [](bf16_t* p, const float (&v)[8]) {
    *reinterpret_cast<u32x4*>(p) =
        u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
  };
  ld8(dy + row * n + c, d);
  ld8(pre + row * pw + c, g);
  float out_y[8], dg[8];
  if (SWIGLU) {
    ld8(pre + row * pw + n + c, u);
    float du[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float sig = 1.0f / (1.0f + __expf(-g[i]));
      const float silu_g = g[i] * sig;
      out_y[i] = silu_g * u[i];
      dg[i] = d[i] * u[i] * (sig * (1.0f + g[i] * (1.0f - sig)));
      du[i] = d[i] * silu_g;
    }
    st8(dpre + row * pw + c, dg);
    st8(dpre + row * pw + n + c, du);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      out_y[i] = gelu_erf(g[i]);
      dg[i] = d[i] * gelu_grad(g[i]);
    }
    st8(dpre + row * pw + c, dg);
  }
  if (y) st8(y + row * n + c, out_y);
}

}  // namespace

hipError_t launch_transpose(int64_t rows, int64_t cols, const void* src, void* dst, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const dim3 grid((unsigned)((cols + TT - 1) / TT), (unsigned)((rows + TT - 1) / TT));
  if (rows % 8 == 0 && cols % 8 == 0)
    hipLaunchKernelGGL(transpose16_kernel, grid, dim3(NT), 0, s, reinterpret_cast<const bf16_t*>(src),
                       reinterpret_cast<bf16_t*>(dst), rows, rows, cols, cols, rows, 1, (int64_t)0, (int64_t)0,
                       (int64_t)0, (int64_t)0);
  else
    hipLaunchKernelGGL(transpose_kernel, grid, dim3(NT), 0, s, reinterpret_cast<const bf16_t*>(src),
                       reinterpret_cast<bf16_t*>(dst), rows, cols);
  return hipGetLastError();
}

hipError_t launch_act_backward(int swiglu, int64_t m, int64_t n, const void* pre, const void* dy, void* dpre,
                               void* y, hipStream_t s) {
  const int64_t total = m * (n >> 3);
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + NT - 1) / NT));
  auto P = [](const void* p) { return reinterpret_cast<const bf16_t*>(p); };
  auto Q = [](void* p) { return reinterpret_cast<bf16_t*>(p); };
  if (swiglu)
    hipLaunchKernelGGL(act_backward_kernel<true>, grid, dim3(NT), 0, s, P(pre), P(dy), Q(dpre), Q(y), m, n);
  else
    hipLaunchKernelGGL(act_backward_kernel<false>, grid, dim3(NT), 0, s, P(pre), P(dy), Q(dpre), Q(y), m, n);
  return hipGetLastError();
}

hipError_t launch_transpose_batched(int64_t n1, int64_t n2, int64_t rows_in, int64_t rows_out, int64_t cols,
                                    int64_t lds, int64_t ldd, int64_t src_bs1, int64_t src_bs2, int64_t dst_bs1,
                                    int64_t dst_bs2, const void* src, void* dst, hipStream_t s) {
  if (n1 == 0 || n2 == 0 || rows_out == 0 || cols == 0) return hipSuccess;
  if (rows_out % 8 != 0 || rows_in > rows_out || n1 * n2 > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((cols + TT - 1) / TT), (unsigned)((rows_out + TT - 1) / TT), (unsigned)(n1 * n2));
  hipLaunchKernelGGL(transpose16_kernel, grid, dim3(NT), 0, s, reinterpret_cast<const bf16_t*>(src),
                     reinterpret_cast<bf16_t*>(dst), rows_in, rows_out, cols, lds, ldd, (int)n2, src_bs1, src_bs2,
                     dst_bs1, dst_bs2);
  return hipGetLastError();
}

}  // namespace tpk
