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

// four consecutive outputs of an MX-fp8 row: a lane's float4 is an eighth of a
// 32-value block, so the block maximum is a butterfly over the 8 lanes that
// hold it; the first of them writes the scale
__device__ __forceinline__ void store_row4_mx(uint8_t* yr, uint8_t* sc, int row, int c, int d,
                                              float a, float b, float e, float f, bool live) {
  float amax = fmaxf(fmaxf(fabsf(a), fabsf(b)), fmaxf(fabsf(e), fabsf(f)));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
  if (!live) return;
  const int x = mx_exponent(amax);
  *reinterpret_cast<unsigned int*>(yr + 4 * c) =
      pack_fp8x4(mx_scale_down(a, x), mx_scale_down(b, x), mx_scale_down(e, x), mx_scale_down(f, x));
  if ((c & 7) == 0) sc[mx_scale_index(row, c >> 3, d)] = (uint8_t)(x + 127);
}

template <typename T>
__global__ __launch_bounds__(64 * LN_WAVES) void ln_kernel(const float* __restrict__ x,
                                                          const float* __restrict__ g,
                                                          const float* __restrict__ b,
                                                          T* __restrict__ y, int rows, int d,
                                                          float eps, uint8_t* __restrict__ ysc) {
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
      if (64 * i >= nv) break;  // uniform: the row's last float4 lies in an earlier i
      const bool live = c < nv;
      float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
      if (live) {
        const float4 gg = g4[c], bb = b4[c];
        o0 = (v[k][i].x - mean[k]) * rs * gg.x + bb.x;
        o1 = (v[k][i].y - mean[k]) * rs * gg.y + bb.y;
        o2 = (v[k][i].z - mean[k]) * rs * gg.z + bb.z;
        o3 = (v[k][i].w - mean[k]) * rs * gg.w + bb.w;
      }
      if constexpr (sizeof(T) == 1) {
        store_row4_mx(reinterpret_cast<uint8_t*>(yr), ysc, row0 + k, c, d, o0, o1, o2, o3, live);
      } else if (live) {
        store_row4(yr + 4 * c, o0, o1, o2, o3);
      }
    }
  }
}

}  // namespace

hipError_t launch_layernorm(const float* x, const float* g, const float* b, void* y, int T, int d,
                            float eps, aut_dtype dt, hipStream_t s, uint8_t* y_scales) {
  if (T <= 0) return hipSuccess;
  if (d % 4 || d > 4 * 64 * LN_MAXV) return hipErrorInvalidValue;
  dim3 grid((T + LN_WAVES * LN_RPW - 1) / (LN_WAVES * LN_RPW));
  if (dt == AUT_FP8) {
    if (d % 128 || !y_scales) return hipErrorInvalidValue;
    hipLaunchKernelGGL(ln_kernel<uint8_t>, grid, dim3(64 * LN_WAVES), 0, s, x, g, b, (uint8_t*)y,
                       T, d, eps, y_scales);
  } else if (dt == AUT_BF16) {
    hipLaunchKernelGGL(ln_kernel<bf16_t>, grid, dim3(64 * LN_WAVES), 0, s, x, g, b, (bf16_t*)y, T,
                       d, eps, (uint8_t*)nullptr);
  } else {
    hipLaunchKernelGGL(ln_kernel<float>, grid, dim3(64 * LN_WAVES), 0, s, x, g, b, (float*)y, T, d,
                       eps, (uint8_t*)nullptr);
  }
  return hipGetLastError();
}

}  // namespace aut
