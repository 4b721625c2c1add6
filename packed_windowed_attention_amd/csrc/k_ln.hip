// LayerNorm with bias (cubic.dev wiki, "Transformer Encoder Layers": the
// encoder uses LayerNorm with bias, not RMSNorm) over fp32 rows, written as
// the next GEMM's operand type.  One wavefront per row; the row stays in
// registers, the statistics are fp32 two-pass (mean, then the mean of squared
// deviations), so the result does not depend on the launch shape.
#include "aut_internal.h"
#include "device_common.h"

namespace aut {

namespace {

constexpr int LN_WAVES = 4;
constexpr int LN_MAXV = 8;  // float4 per lane: d <= 2048

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// four consecutive outputs in one store (8 bytes bf16, 16 bytes fp32)
__device__ __forceinline__ void store_row4(bf16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<u32x2_t*>(p) = u32x2_t{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}
__device__ __forceinline__ void store_row4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

template <typename T>
__global__ __launch_bounds__(64 * LN_WAVES) void ln_kernel(const float* __restrict__ x,
                                                          const float* __restrict__ g,
                                                          const float* __restrict__ b,
                                                          T* __restrict__ y, int rows, int d,
                                                          float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * LN_WAVES + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int nv = d >> 2;
  const float4* xr = reinterpret_cast<const float4*>(x + (size_t)row * d);
  float4 v[LN_MAXV];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) {
    const int c = lane + 64 * i;
    v[i] = c < nv ? xr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  }
  const float mean = wave_sum(s) / (float)d;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) {
    const int c = lane + 64 * i;
    if (c < nv) {
      const float a0 = v[i].x - mean, a1 = v[i].y - mean, a2 = v[i].z - mean, a3 = v[i].w - mean;
      q += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
    }
  }
  const float rstd = rsqrtf(wave_sum(q) / (float)d + eps);
  T* yr = y + (size_t)row * d;
  const float4* g4 = reinterpret_cast<const float4*>(g);
  const float4* b4 = reinterpret_cast<const float4*>(b);
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) {
    const int c = lane + 64 * i;
    if (c < nv) {
      const float4 gg = g4[c], bb = b4[c];
      const float o0 = (v[i].x - mean) * rstd * gg.x + bb.x;
      const float o1 = (v[i].y - mean) * rstd * gg.y + bb.y;
      const float o2 = (v[i].z - mean) * rstd * gg.z + bb.z;
      const float o3 = (v[i].w - mean) * rstd * gg.w + bb.w;
      store_row4(yr + 4 * c, o0, o1, o2, o3);
    }
  }
}

}  // namespace

hipError_t launch_layernorm(const float* x, const float* g, const float* b, void* y, int T, int d,
                            float eps, aut_dtype dt, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (d % 4 || d > 4 * 64 * LN_MAXV) return hipErrorInvalidValue;
  dim3 grid((T + LN_WAVES - 1) / LN_WAVES);
  if (dt == AUT_BF16)
    hipLaunchKernelGGL(ln_kernel<bf16_t>, grid, dim3(64 * LN_WAVES), 0, s, x, g, b, (bf16_t*)y, T,
                       d, eps);
  else
    hipLaunchKernelGGL(ln_kernel<float>, grid, dim3(64 * LN_WAVES), 0, s, x, g, b, (float*)y, T, d,
                       eps);
  return hipGetLastError();
}

}  // namespace aut
