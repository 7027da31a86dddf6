// Alignment losses: "SSA: Achieving Sparser Attention by Aligning Full and
// Sparse Attention Outputs in Feature Space", section "Bidirectional
// Attention Alignment": L_sparsity = ||a_full - sg[a_sparse]|| and
// L_commitment = ||a_sparse - sg[a_full]||, read as mean squared errors. Both
// forward values are mean((h_full - h_sparse)^2); the stop-gradient only
// decides which output each loss's gradient reaches:
//   dL_sparsity/dh_full = 2 (h_full - h_sparse)/n,
//   dL_commitment/dh_sparse = 2 (h_sparse - h_full)/n.
// The sum is deterministic: a fixed grid of float64 partial sums, each over a
// fixed strided range, reduced in a fixed tree order, then one final
// workgroup sums the partials in a fixed order.
#include "ssa_common.h"
#include "ssa_kernels.h"

namespace ssa {

__device__ __forceinline__ void ld8(const uint16_t* p, double out[8]) {
  const uint4 u = *(const uint4*)p;
  const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = (double)__uint_as_float(w[i] << 16);
    out[2 * i + 1] = (double)__uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void ld8(const float* p, double out[8]) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}
__device__ __forceinline__ void st8(uint16_t* p, const float v[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
  *(uint4*)p = make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ void st8(float* p, const float v[8]) {
  *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
  *(float4*)(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

__device__ __forceinline__ double block_sum(double v, double* sh) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) sh[tid] += sh[tid + s];
    __syncthreads();
  }
  return sh[0];
}

template <typename T>
__global__ __launch_bounds__(256) void loss_partial_kernel(const T* __restrict__ hf,
                                                           const T* __restrict__ hs, long n8,
                                                           T* __restrict__ gf, T* __restrict__ gs,
                                                           double* __restrict__ partials,
                                                           double gscale) {
  __shared__ double sh[256];
  double acc = 0.0;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long)gridDim.x * 256) {
    double a[8], c[8];
    ld8(hf + 8 * i, a);
    ld8(hs + 8 * i, c);
    float g[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double df = a[e] - c[e];
      acc += df * df;
      g[e] = (float)(gscale * df);
    }
    if (gf != nullptr) st8(gf + 8 * i, g);
    if (gs != nullptr) {
#pragma unroll
      for (int e = 0; e < 8; ++e) g[e] = -g[e];
      st8(gs + 8 * i, g);
    }
  }
  const double tot = block_sum(acc, sh);
  if (threadIdx.x == 0) partials[blockIdx.x] = tot;
}

__global__ __launch_bounds__(256) void loss_final_kernel(const double* __restrict__ partials,
                                                         int np, double inv_n,
                                                         float* __restrict__ loss) {
  __shared__ double sh[256];
  double acc = 0.0;
  for (int i = threadIdx.x; i < np; i += 256) acc += partials[i];
  const double tot = block_sum(acc, sh);
  if (threadIdx.x == 0) {
    const float l = (float)(tot * inv_n);
    loss[0] = l;
    loss[1] = l;
  }
}

long align_loss_partials(long n) {
  const long np = (n / 8 + 255) / 256;
  return np < 1 ? 1 : np > kLossPartials ? kLossPartials : np;
}

hipError_t launch_align_loss(const void* hf, const void* hs, bool bf16, long n, float* loss,
                             void* gf, void* gs, double* partials, hipStream_t stream) {
  const long n8 = n / 8;
  const long np = align_loss_partials(n);
  const double gscale = 2.0 / (double)n;
  if (bf16)
    hipLaunchKernelGGL(loss_partial_kernel<uint16_t>, dim3((unsigned)np), dim3(256), 0, stream,
                       (const uint16_t*)hf, (const uint16_t*)hs, n8, (uint16_t*)gf,
                       (uint16_t*)gs, partials, gscale);
  else
    hipLaunchKernelGGL(loss_partial_kernel<float>, dim3((unsigned)np), dim3(256), 0, stream,
                       (const float*)hf, (const float*)hs, n8, (float*)gf, (float*)gs, partials,
                       gscale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(loss_final_kernel, dim3(1), dim3(256), 0, stream, partials, (int)np,
                     1.0 / (double)n, loss);
  return hipGetLastError();
}

}  // namespace ssa
