// Conv-stem first layer, parameter packing and the sinusoid position table.
//
// conv1 has one input channel and 9 taps per output, far too little depth for
// the matrix cores, so it runs on the vector ALU in fp32.  A workgroup makes
// CONV1_ROWS output rows of one chunk: the 2 CONV1_ROWS + 1 input mel rows it
// needs are staged in LDS, zero past the chunk's valid frames (the m-star
// frontend zero-pads the last piece of a request to a full chunk) and outside
// the image (padding 1).  Each thread owns 8 consecutive output channels, keeps
// their 72 weights and 8 biases in registers, and walks output pixels: per
// pixel 9 broadcast LDS reads, 72 FMAs, 8 GELUs and one 16-byte store of the
// 8 bf16 results.  Output: channels-last [chunk][y][x][c], the operand layout
// of the conv2 implicit GEMM.
#include <math.h>

#include "aut_internal.h"
#include "device_common.h"

namespace aut {

namespace {

constexpr int CONV1_THREADS = 256;
constexpr int CONV1_ROWS = 4;   // output rows per workgroup
constexpr int MAX_CF = 256;

template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&v)[8]);
template <>
__device__ __forceinline__ void store8<bf16_t>(bf16_t* p, const float (&v)[8]) {
  *reinterpret_cast<u32x4_t*>(p) = u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                           pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
}
template <>
__device__ __forceinline__ void store8<float>(float* p, const float (&v)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// MX-fp8 store of a thread's 8 channels: a 32-channel block is 4 consecutive
// lanes (8-channel groups 4b .. 4b + 3), so its maximum is a quad maximum;
// the block's first lane writes the scale.
// Maximum over the 4 lanes of an aligned lane quad: two DPP quad permutes
// (lane i ^ 1, then lane i ^ 2), vector-ALU moves with no LDS round trip.
__device__ __forceinline__ float quad_max(float x) {
  constexpr int XOR1 = 1 | (0 << 2) | (3 << 4) | (2 << 6);  // quad_perm [1, 0, 3, 2]
  constexpr int XOR2 = 2 | (3 << 2) | (0 << 4) | (1 << 6);  // quad_perm [2, 3, 0, 1]
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), XOR1,
                                                                  0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), XOR2,
                                                                  0xF, 0xF, false)));
  return x;
}

__device__ __forceinline__ void store8_mx(uint8_t* p, uint8_t* sc, const float (&v)[8], int cg) {
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
  amax = quad_max(amax);
  const int e = mx_exponent(amax);
  *reinterpret_cast<u32x2_t*>(p) =
      u32x2_t{pack_fp8x4(mx_scale_down(v[0], e), mx_scale_down(v[1], e), mx_scale_down(v[2], e),
                         mx_scale_down(v[3], e)),
              pack_fp8x4(mx_scale_down(v[4], e), mx_scale_down(v[5], e), mx_scale_down(v[6], e),
                         mx_scale_down(v[7], e))};
  if ((cg & 3) == 0) sc[cg >> 2] = (uint8_t)(e + 127);
}

// T = uint8_t: MX-fp8 output, cp channels per pixel (channels past C zero),
// scales row-major cp / 32 bytes per pixel in a1s.
template <typename T>
__global__ __launch_bounds__(CONV1_THREADS) void conv1_kernel(
    const float* __restrict__ feat, int T_max, int mel, const int* __restrict__ chunks,
    int chunk_first, const float* __restrict__ w1, const float* __restrict__ b1,
    T* __restrict__ a1, int C, int cf, int h1, int w1out, uint8_t* __restrict__ a1s, int cp) {
  constexpr bool MX = sizeof(T) == 1;
  __shared__ float img[2 * CONV1_ROWS + 1][MAX_CF + 2];
  const int oy0 = blockIdx.x * CONV1_ROWS;
  const int cl = blockIdx.y;  // chunk within the batch
  const int* ch = chunks + 5 * (chunk_first + cl);
  const int req = ch[0], frame0 = ch[1], vf = ch[2];
  const int tid = threadIdx.x;

  // input rows 2 oy0 - 1 .. 2 (oy0 + CONV1_ROWS) - 1, columns -1 .. cf
  for (int idx = tid; idx < (2 * CONV1_ROWS + 1) * (cf + 2); idx += CONV1_THREADS) {
    const int r = idx / (cf + 2);
    const int ix = idx - r * (cf + 2) - 1;
    const int iy = 2 * oy0 - 1 + r;
    float v = 0.f;
    if (iy >= 0 && iy < mel && ix >= 0 && ix < vf)
      v = feat[((size_t)req * mel + iy) * T_max + frame0 + ix];
    img[r][ix + 1] = v;
  }
  __syncthreads();

  const int cs = MX ? cp : C;                    // channels stored per pixel
  const int groups = cs >> 3;                    // 8-channel groups
  const int xlanes = CONV1_THREADS / groups;     // threads per group
  const int cg = tid % groups;
  const int xl = tid / groups;
  if (xl >= xlanes) return;                      // spare threads (no barrier follows)
  const int c0 = cg * 8;
  float w[8][9], bias[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const bool real = !MX || c0 + k < C;         // padding channels: zero weights and bias
    bias[k] = real ? b1[c0 + k] : 0.f;
#pragma unroll
    for (int t = 0; t < 9; ++t) w[k][t] = real ? w1[(c0 + k) * 9 + t] : 0.f;
  }
  // Output pixels of the workgroup are consecutive in memory (item = ry *
  // w1out + ox), so the store address steps by xlanes pixels per item and only
  // the LDS position needs (ry, ox), advanced without a division.
  const int rows = min(CONV1_ROWS, h1 - oy0);
  const int n_items = rows * w1out;
  const size_t pix_first = ((size_t)cl * h1 + oy0) * w1out + xl;
  int ry = xl / w1out, ox = xl - ry * w1out;   // position of the current item
  const int dry = xlanes / w1out, dox = xlanes - dry * w1out;
  T* out = a1 + pix_first * cs + c0;           // (cs bytes per pixel when T is a byte)
  uint8_t* osc = MX ? a1s + pix_first * (cs >> 5) : nullptr;
  for (int item = xl; item < n_items; item += xlanes) {
    float x[9];
#pragma unroll
    for (int kh = 0; kh < 3; ++kh)
#pragma unroll
      for (int kw = 0; kw < 3; ++kw) x[kh * 3 + kw] = img[2 * ry + kh][2 * ox + kw];
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float a = bias[k];
#pragma unroll
      for (int t = 0; t < 9; ++t) a = fmaf(w[k][t], x[t], a);
      v[k] = sizeof(T) == 4 ? gelu_f(a) : gelu_bf16(a);
    }
    if constexpr (MX) {
      store8_mx(reinterpret_cast<uint8_t*>(out), osc, v, cg);
      osc += (size_t)xlanes * (cs >> 5);
    } else {
      store8<T>(out, v);
    }
    out += (size_t)xlanes * cs;
    ox += dox;
    ry += dry;
    if (ox >= w1out) {
      ox -= w1out;
      ++ry;
    }
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
                        const Geometry& g, hipStream_t s, uint8_t* a1_scales, int cp) {
  if (nb <= 0) return hipSuccess;
  if (g.cf > MAX_CF || (g.C & 7) || (g.C >> 3) > CONV1_THREADS) return hipErrorInvalidValue;
  dim3 grid((g.h1 + CONV1_ROWS - 1) / CONV1_ROWS, nb);
  if (dt == AUT_FP8) {
    // whole 32-channel blocks in aligned lane quads, at least one thread per group
    if (cp < g.C || cp % 128 || (cp >> 3) > CONV1_THREADS || !a1_scales) return hipErrorInvalidValue;
    hipLaunchKernelGGL(conv1_kernel<uint8_t>, grid, dim3(CONV1_THREADS), 0, s, feat, T_max, g.mel,
                       chunks, chunk_first, w1, b1, (uint8_t*)a1, g.C, g.cf, g.h1, g.w1, a1_scales,
                       cp);
  } else if (dt == AUT_BF16) {
    hipLaunchKernelGGL(conv1_kernel<bf16_t>, grid, dim3(CONV1_THREADS), 0, s, feat, T_max, g.mel,
                       chunks, chunk_first, w1, b1, (bf16_t*)a1, g.C, g.cf, g.h1, g.w1,
                       (uint8_t*)nullptr, 0);
  } else {
    hipLaunchKernelGGL(conv1_kernel<float>, grid, dim3(CONV1_THREADS), 0, s, feat, T_max, g.mel,
                       chunks, chunk_first, w1, b1, (float*)a1, g.C, g.cf, g.h1, g.w1,
                       (uint8_t*)nullptr, 0);
  }
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
