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
constexpr int LN_RPW = 1;   // rows per wave (2 or 4 measured slower)

// butterfly sums over the wavefront of LN_RPW independent values at once
__device__ __forceinline__ void wave_sum_n(float (&v)[LN_RPW]) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
    for (int k = 0; k < LN_RPW; ++k) v[k] += __shfl_xor(v[k], o, 64);
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
  // LN_RPW rows per wave, loaded together so that their loads and their
  // reductions overlap
  const int lane = threadIdx.x & 63;
  const int row0 = (blockIdx.x * LN_WAVES + (threadIdx.x >> 6)) * LN_RPW;
  if (row0 >= rows) return;
  const int nv = d >> 2;
  float4 v[LN_RPW][LN_MAXV];
#pragma unroll
  for (int k = 0; k < LN_RPW; ++k) {
    const float4* xr = reinterpret_cast<const float4*>(x + (size_t)(row0 + k) * d);
    const bool live = row0 + k < rows;
#pragma unroll
    for (int i = 0; i < LN_MAXV; ++i) {
      const int c = lane + 64 * i;
      v[k][i] = (live && c < nv) ? xr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  float mean[LN_RPW], rstd[LN_RPW];
#pragma unroll
  for (int k = 0; k < LN_RPW; ++k) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < LN_MAXV; ++i) s += (v[k][i].x + v[k][i].y) + (v[k][i].z + v[k][i].w);
    mean[k] = s;
  }
  wave_sum_n(mean);
#pragma unroll
  for (int k = 0; k < LN_RPW; ++k) {
    mean[k] /= (float)d;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < LN_MAXV; ++i) {
      const int c = lane + 64 * i;
      if (c < nv) {
        const float a0 = v[k][i].x - mean[k], a1 = v[k][i].y - mean[k];
        const float a2 = v[k][i].z - mean[k], a3 = v[k][i].w - mean[k];
        q += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
      }
    }
    rstd[k] = q;
  }
  wave_sum_n(rstd);
  const float4* g4 = reinterpret_cast<const float4*>(g);
  const float4* b4 = reinterpret_cast<const float4*>(b);
#pragma unroll
  for (int k = 0; k < LN_RPW; ++k) {
    if (row0 + k >= rows) break;
    const float rs = rsqrtf(rstd[k] / (float)d + eps);
    T* yr = y + (size_t)(row0 + k) * d;
#pragma unroll
    for (int i = 0; i < LN_MAXV; ++i) {
      const int c = lane + 64 * i;
      if (c < nv) {
        const float4 gg = g4[c], bb = b4[c];
        const float o0 = (v[k][i].x - mean[k]) * rs * gg.x + bb.x;
        const float o1 = (v[k][i].y - mean[k]) * rs * gg.y + bb.y;
        const float o2 = (v[k][i].z - mean[k]) * rs * gg.z + bb.z;
        const float o3 = (v[k][i].w - mean[k]) * rs * gg.w + bb.w;
        store_row4(yr + 4 * c, o0, o1, o2, o3);
      }
    }
  }
}

}  // namespace

hipError_t launch_layernorm(const float* x, const float* g, const float* b, void* y, int T, int d,
                            float eps, aut_dtype dt, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (d % 4 || d > 4 * 64 * LN_MAXV) return hipErrorInvalidValue;
  dim3 grid((T + LN_WAVES * LN_RPW - 1) / (LN_WAVES * LN_RPW));
  if (dt == AUT_BF16)
    hipLaunchKernelGGL(ln_kernel<bf16_t>, grid, dim3(64 * LN_WAVES), 0, s, x, g, b, (bf16_t*)y, T,
                       d, eps);
  else
    hipLaunchKernelGGL(ln_kernel<float>, grid, dim3(64 * LN_WAVES), 0, s, x, g, b, (float*)y, T, d,
                       eps);
  return hipGetLastError();
}

}  // namespace aut
