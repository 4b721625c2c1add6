// Conv-stem first layer, parameter packing and the sinusoid position table.
//
// conv1 has one input channel and 9 taps per output, far too little depth for
// the matrix cores, so it runs on the vector ALU in fp32: a workgroup makes
// one output row (oy) of one chunk, with the three input mel rows it needs
// staged in LDS and zero-filled past the chunk's valid frames (the m-star
// frontend zero-pads the last piece of a request to a full chunk) and outside
// the image (padding 1).  Output: channels-last [chunk][y][x][c], the operand
// layout of the conv2 implicit GEMM.
#include <math.h>

#include "aut_internal.h"
#include "device_common.h"

namespace aut {

namespace {

constexpr int CONV1_THREADS = 256;
constexpr int MAX_C = 1024;
constexpr int MAX_CF = 256;

template <typename T>
__global__ __launch_bounds__(CONV1_THREADS) void conv1_kernel(
    const float* __restrict__ feat, int T_max, int mel, const int* __restrict__ chunks,
    int chunk_first, const float* __restrict__ w1, const float* __restrict__ b1,
    T* __restrict__ a1, int C, int cf, int h1, int w1out) {
  __shared__ float img[3][MAX_CF + 2];
  __shared__ float ws[MAX_C * 9];
  __shared__ float bs[MAX_C];
  const int oy = blockIdx.x;
  const int cl = blockIdx.y;  // chunk within the batch
  const int* ch = chunks + 5 * (chunk_first + cl);
  const int req = ch[0], frame0 = ch[1], vf = ch[2];
  const int tid = threadIdx.x;

  for (int idx = tid; idx < 3 * (cf + 2); idx += CONV1_THREADS) {
    const int kh = idx / (cf + 2);
    const int ix = idx - kh * (cf + 2) - 1;  // -1 .. cf
    const int iy = 2 * oy + kh - 1;
    float v = 0.f;
    if (iy >= 0 && iy < mel && ix >= 0 && ix < vf)
      v = feat[((size_t)req * mel + iy) * T_max + frame0 + ix];
    img[kh][ix + 1] = v;
  }
  for (int idx = tid; idx < 9 * C; idx += CONV1_THREADS) ws[idx] = w1[idx];
  for (int idx = tid; idx < C; idx += CONV1_THREADS) bs[idx] = b1[idx];
  __syncthreads();

  T* out = a1 + ((size_t)cl * h1 + oy) * w1out * C;
  const int half = C >> 1;
  for (int idx = tid; idx < w1out * half; idx += CONV1_THREADS) {
    const int ox = idx / half;
    const int c = 2 * (idx - ox * half);
    float v0 = bs[c], v1 = bs[c + 1];
#pragma unroll
    for (int kh = 0; kh < 3; ++kh)
#pragma unroll
      for (int kw = 0; kw < 3; ++kw) {
        const float x = img[kh][2 * ox + kw];  // column 2 ox + kw - 1, shifted by the pad
        v0 = fmaf(ws[c * 9 + kh * 3 + kw], x, v0);
        v1 = fmaf(ws[(c + 1) * 9 + kh * 3 + kw], x, v1);
      }
    out[(size_t)ox * C + c] = from_f32<T>(gelu_f(v0));
    out[(size_t)ox * C + c + 1] = from_f32<T>(gelu_f(v1));
  }
}

// Parameter packing: dst[i] = src[gather(i)] converted to T.
//  PACK_CAST     same layout ([rows, cols]).
//  PACK_CONV     [Co, Ci, 3, 3] -> [Co][tap * Ci + ci], tap = 3 kh + kw
//                (the implicit-GEMM k order).
//  PACK_CONV_OUT [d, C * F] with column c * F + f -> [d][f * C + c] (the
//                conv3 output is stored time-major, bins then channels).
template <typename T>
__global__ void pack_kernel(const float* __restrict__ src, T* __restrict__ dst, int mode,
                            int rows, int cols, int C, int F) {
  const size_t total = (size_t)rows * cols;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / cols;
    const int k = (int)(i - r * cols);
    size_t s;
    if (mode == PACK_CONV) {
      const int tap = k / C, ci = k - tap * C;
      s = r * cols + (size_t)ci * 9 + tap;
    } else if (mode == PACK_CONV_OUT) {
      const int f = k / C, c = k - f * C;
      s = r * cols + (size_t)c * F + f;
    } else {
      s = i;
    }
    dst[i] = from_f32<T>(src[s]);
  }
}

// Sinusoid table [rows, d] computed in double and rounded to fp32: column
// i < D is sin(j tau_i), column D + i is cos(j tau_i), tau_i = 10000^(-i/(D-1))
// (Whisper-style table; the pages only say the positions are computed, not
// loaded).
__global__ void pe_kernel(float* pe, int rows, int d) {
  const int D = d / 2;
  const int total = rows * D;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
    const int j = i / D, c = i - j * D;
    const double inc = log(10000.0) / (double)(D - 1);
    const double t = (double)j * exp(-inc * (double)c);
    pe[(size_t)j * d + c] = (float)sin(t);
    pe[(size_t)j * d + D + c] = (float)cos(t);
  }
}

}  // namespace

hipError_t launch_conv1(const float* feat, int T_max, const int* chunks, int chunk_first, int nb,
                        const float* w1, const float* b1, void* a1, aut_dtype dt,
                        const Geometry& g, hipStream_t s) {
  if (nb <= 0) return hipSuccess;
  if (g.C > MAX_C || g.cf > MAX_CF || (g.C & 1)) return hipErrorInvalidValue;
  dim3 grid(g.h1, nb);
  if (dt == AUT_BF16)
    hipLaunchKernelGGL(conv1_kernel<bf16_t>, grid, dim3(CONV1_THREADS), 0, s, feat, T_max, g.mel,
                       chunks, chunk_first, w1, b1, (bf16_t*)a1, g.C, g.cf, g.h1, g.w1);
  else
    hipLaunchKernelGGL(conv1_kernel<float>, grid, dim3(CONV1_THREADS), 0, s, feat, T_max, g.mel,
                       chunks, chunk_first, w1, b1, (float*)a1, g.C, g.cf, g.h1, g.w1);
  return hipGetLastError();
}

hipError_t launch_pack(const float* src, void* dst, aut_dtype dt, int mode, int rows, int cols,
                       int C, int F, hipStream_t s) {
  const size_t total = (size_t)rows * cols;
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const int blocks = (int)((total + threads - 1) / threads < 8192 ? (total + threads - 1) / threads : 8192);
  if (dt == AUT_BF16)
    hipLaunchKernelGGL(pack_kernel<bf16_t>, dim3(blocks), dim3(threads), 0, s, src, (bf16_t*)dst,
                       mode, rows, cols, C, F);
  else
    hipLaunchKernelGGL(pack_kernel<float>, dim3(blocks), dim3(threads), 0, s, src, (float*)dst,
                       mode, rows, cols, C, F);
  return hipGetLastError();
}

hipError_t launch_pe_table(float* pe, int rows, int d, hipStream_t s) {
  const int total = rows * (d / 2);
  const int threads = 256;
  hipLaunchKernelGGL(pe_kernel, dim3((total + threads - 1) / threads), dim3(threads), 0, s, pe,
                     rows, d);
  return hipGetLastError();
}

}  // namespace aut
