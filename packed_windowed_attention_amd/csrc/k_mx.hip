// fp32 rows -> MX-fp8 (OCP Microscaling formats: e4m3 elements, one E8M0
// power-of-two scale per 32 consecutive values of a row).  Used on weights
// when they are packed, and as a plain conversion primitive.  One thread per
// 32-value block: eight 16-byte loads, the block maximum, the exact scale
// exponent, and two 16-byte stores of codes; rows past R up to the next
// multiple of 16 get scale code 0 (2^-127) so that the padded scale rows are
// defined.
#include "aut_internal.h"
#include "device_common.h"

namespace aut {

namespace {

constexpr int MXQ_THREADS = 256;

__global__ __launch_bounds__(MXQ_THREADS) void mx_quantize_kernel(const float* __restrict__ x,
                                                                  long ldx, int R, int K,
                                                                  uint8_t* __restrict__ codes,
                                                                  uint8_t* __restrict__ scales) {
  const int nkb = K / MX_BLOCK;
  const long R16 = ((long)R + 15) / 16 * 16;
  const long idx = (long)blockIdx.x * MXQ_THREADS + threadIdx.x;
  if (idx >= R16 * nkb) return;
  const int r = (int)(idx / nkb);
  const int kb = (int)(idx - (long)r * nkb);
  if (r >= R) {
    scales[mx_scale_index(r, kb, K)] = 0;
    return;
  }
  const float4* src = reinterpret_cast<const float4*>(x + (size_t)r * ldx + (size_t)kb * MX_BLOCK);
  float4 v[8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = src[i];
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
  }
  const int e = mx_exponent(amax);
  unsigned int w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    w[i] = pack_fp8x4(mx_scale_down(v[i].x, e), mx_scale_down(v[i].y, e), mx_scale_down(v[i].z, e),
                      mx_scale_down(v[i].w, e));
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(codes + (size_t)r * K + (size_t)kb * MX_BLOCK);
  dst[0] = u32x4_t{w[0], w[1], w[2], w[3]};
  dst[1] = u32x4_t{w[4], w[5], w[6], w[7]};
  scales[mx_scale_index(r, kb, K)] = (uint8_t)(e + 127);
}

// The same per block, reading a conv-stem weight from its PyTorch layout
// (PACK_CONV / PACK_CONV_OUT, channels padded to cp with zeros).
__global__ __launch_bounds__(MXQ_THREADS) void mx_quantize_gather_kernel(
    const float* __restrict__ src, int mode, int R, int C, int cp, int F,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int per = mode == PACK_CONV ? 9 : F;     // taps or frequency bins
  const int K = per * cp;
  const int nkb = K / MX_BLOCK;
  const long R16 = ((long)R + 15) / 16 * 16;
  const long idx = (long)blockIdx.x * MXQ_THREADS + threadIdx.x;
  if (idx >= R16 * nkb) return;
  const int r = (int)(idx / nkb);
  const int kb = (int)(idx - (long)r * nkb);
  if (r >= R) {
    scales[mx_scale_index(r, kb, K)] = 0;
    return;
  }
  const int outer = (kb * MX_BLOCK) / cp;        // tap or bin (cp is a multiple of 32)
  const int c0 = kb * MX_BLOCK - outer * cp;
  float v[MX_BLOCK];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < MX_BLOCK; ++j) {
    const int c = c0 + j;
    float x = 0.f;
    if (c < C)
      x = mode == PACK_CONV ? src[((size_t)r * C + c) * 9 + outer]
                            : src[(size_t)r * C * F + (size_t)c * F + outer];
    v[j] = x;
    amax = fmaxf(amax, fabsf(x));
  }
  const int e = mx_exponent(amax);
  unsigned int w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    w[i] = pack_fp8x4(mx_scale_down(v[4 * i], e), mx_scale_down(v[4 * i + 1], e),
                      mx_scale_down(v[4 * i + 2], e), mx_scale_down(v[4 * i + 3], e));
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(codes + (size_t)r * K + (size_t)kb * MX_BLOCK);
  dst[0] = u32x4_t{w[0], w[1], w[2], w[3]};
  dst[1] = u32x4_t{w[4], w[5], w[6], w[7]};
  scales[mx_scale_index(r, kb, K)] = (uint8_t)(e + 127);
}

}  // namespace

hipError_t launch_mx_quantize_gather(const float* src, int mode, int rows, int C, int cp, int F,
                                     uint8_t* codes, uint8_t* scales, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if ((mode != PACK_CONV && mode != PACK_CONV_OUT) || cp < C || cp % 128 || F <= 0 ||
      ((size_t)codes & 15))
    return hipErrorInvalidValue;
  const long K = (long)(mode == PACK_CONV ? 9 : F) * cp;
  const long n = ((long)rows + 15) / 16 * 16 * (K / MX_BLOCK);
  hipLaunchKernelGGL(mx_quantize_gather_kernel, dim3((unsigned)((n + MXQ_THREADS - 1) / MXQ_THREADS)),
                     dim3(MXQ_THREADS), 0, s, src, mode, rows, C, cp, F, codes, scales);
  return hipGetLastError();
}

size_t mx_scale_bytes(long rows, int K) { return (size_t)((rows + 15) / 16) * 16 * (size_t)(K / MX_BLOCK); }

hipError_t launch_mx_quantize(const float* x, long ldx, long R, int K, uint8_t* codes,
                              uint8_t* scales, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  if (K <= 0 || K % 128 || ldx % 4 || ((size_t)x & 15) || ((size_t)codes & 15))
    return hipErrorInvalidValue;
  const long R16 = (R + 15) / 16 * 16;
  const long n = R16 * (K / MX_BLOCK);
  hipLaunchKernelGGL(mx_quantize_kernel, dim3((unsigned)((n + MXQ_THREADS - 1) / MXQ_THREADS)),
                     dim3(MXQ_THREADS), 0, s, x, ldx, (int)R, K, codes, scales);
  return hipGetLastError();
}

}  // namespace aut
