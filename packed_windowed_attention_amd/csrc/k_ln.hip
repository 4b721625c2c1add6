// LayerNorm with bias (cubic.dev wiki, "Transformer Encoder Layers": the
// encoder uses LayerNorm with bias, not RMSNorm) over fp32 rows, written as
// the next GEMM's operand type.  A wavefront takes one row at a time (rows
// strided over the grid); the row stays in registers, the statistics are fp32
// two-pass (mean, then the mean of squared deviations), so the result does not
// depend on the launch shape.
#include <algorithm>

#include "aut_internal.h"
#include "device_common.h"

namespace aut {

namespace {

constexpr int LN_WAVES = 4;
constexpr int LN_MAXV = 8;            // float4 per lane: d <= 2048
constexpr int LN_GRID_CAP = 256 * 4;  // workgroups: 16 waves per CU, each over several rows

// Sum over the wavefront, the same value in every lane, without LDS: lane
// pairs and quad pairs by DPP quad permutes, then the 4-lane halves of each
// 8-lane group and the 8-lane halves of each 16-lane row by DPP mirrors (on
// values already uniform over the quads or halves these are the xor-4 and
// xor-8 partners), then row pairs and row halves by v_permlane16_swap and
// v_permlane32_swap.  Each step adds two partners' values, so every lane adds
// the same pairs and ends with the same bits.
__device__ __forceinline__ void wave_sum_n(float (&v)[1]) {
  float x = v[0];
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                          1 | (0 << 2) | (3 << 4) | (2 << 6), 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                          2 | (3 << 2) | (0 << 4) | (1 << 6), 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF,
                                                          false));  // row_half_mirror
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF,
                                                          false));  // row_mirror
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  v[0] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
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
  // the 8 lanes of an aligned group: quad permutes, then the group's half mirror
  amax = fmaxf(amax, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                         __builtin_bit_cast(int, amax), 1 | (0 << 2) | (3 << 4) | (2 << 6), 0xF, 0xF, false)));
  amax = fmaxf(amax, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                         __builtin_bit_cast(int, amax), 2 | (3 << 2) | (0 << 4) | (1 << 6), 0xF, 0xF, false)));
  amax = fmaxf(amax, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                         __builtin_bit_cast(int, amax), 0x141, 0xF, 0xF, false)));  // row_half_mirror
  if (!live) return;
  const int x = mx_exponent(amax);
  *reinterpret_cast<unsigned int*>(yr + 4 * c) =
      pack_fp8x4(mx_scale_down(a, x), mx_scale_down(b, x), mx_scale_down(e, x), mx_scale_down(f, x));
  if ((c & 7) == 0) sc[mx_scale_index(row, c >> 3, d)] = (uint8_t)(x + 127);
}

// V float4 per lane (d <= 256 V).  Rows are strided over the grid's waves; a
// wave loads its next row before it reduces the current one, so that row's
// loads are in flight during the reductions and stores, and the gain and shift
// stay in registers for all its rows.
template <typename T, int V>
__global__ __launch_bounds__(64 * LN_WAVES) void ln_kernel(const float* __restrict__ x,
                                                          const float* __restrict__ g,
                                                          const float* __restrict__ b,
                                                          T* __restrict__ y, int rows, int d,
                                                          float eps, uint8_t* __restrict__ ysc) {
  const int lane = threadIdx.x & 63;
  const int w0 = blockIdx.x * LN_WAVES + (threadIdx.x >> 6);
  const int nw = gridDim.x * LN_WAVES;
  if (w0 >= rows) return;
  const int nv = d >> 2;
  const float4* g4 = reinterpret_cast<const float4*>(g);
  const float4* b4 = reinterpret_cast<const float4*>(b);
  float4 gg[V], bb[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int c = lane + 64 * i;
    gg[i] = c < nv ? g4[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    bb[i] = c < nv ? b4[c] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  auto load_row = [&](float4 (&v)[V], int row) __attribute__((always_inline)) {
    const float4* xr = reinterpret_cast<const float4*>(x + (size_t)row * d);
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int c = lane + 64 * i;
      v[i] = c < nv ? xr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  float4 v[V];
  load_row(v, w0);
  for (int row = w0; row < rows; row += nw) {
    const int nrow = row + nw;
    float4 nx[V];
    if (nrow < rows) load_row(nx, nrow);
    float mean[1], q[1];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    mean[0] = s;
    wave_sum_n(mean);
    const float mu = mean[0] / (float)d;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int c = lane + 64 * i;
      if (c < nv) {
        const float a0 = v[i].x - mu, a1 = v[i].y - mu;
        const float a2 = v[i].z - mu, a3 = v[i].w - mu;
        ss += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
      }
    }
    q[0] = ss;
    wave_sum_n(q);
    const float rs = rsqrtf(q[0] / (float)d + eps);
    T* yr = y + (size_t)row * d;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int c = lane + 64 * i;
      if (64 * i >= nv) break;  // uniform: the row's last float4 lies in an earlier i
      const bool live = c < nv;
      float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
      if (live) {
        o0 = (v[i].x - mu) * rs * gg[i].x + bb[i].x;
        o1 = (v[i].y - mu) * rs * gg[i].y + bb[i].y;
        o2 = (v[i].z - mu) * rs * gg[i].z + bb[i].z;
        o3 = (v[i].w - mu) * rs * gg[i].w + bb[i].w;
      }
      if constexpr (sizeof(T) == 1) {
        store_row4_mx(reinterpret_cast<uint8_t*>(yr), ysc, row, c, d, o0, o1, o2, o3, live);
      } else if (live) {
        store_row4(yr + 4 * c, o0, o1, o2, o3);
      }
    }
    if (nrow < rows) {
#pragma unroll
      for (int i = 0; i < V; ++i) v[i] = nx[i];
    }
  }
}

template <typename T, int V>
hipError_t run_ln(const float* x, const float* g, const float* b, T* y, int T_rows, int d, float eps,
                  uint8_t* ysc, hipStream_t s) {
  const int wgs = std::min((T_rows + LN_WAVES - 1) / LN_WAVES, LN_GRID_CAP);
  hipLaunchKernelGGL((ln_kernel<T, V>), dim3(wgs), dim3(64 * LN_WAVES), 0, s, x, g, b, y, T_rows, d,
                     eps, ysc);
  return hipGetLastError();
}

template <typename T>
hipError_t run_ln_any(const float* x, const float* g, const float* b, T* y, int T_rows, int d,
                      float eps, uint8_t* ysc, hipStream_t s) {
  switch ((d / 4 + 63) / 64) {
    case 1: return run_ln<T, 1>(x, g, b, y, T_rows, d, eps, ysc, s);
    case 2: return run_ln<T, 2>(x, g, b, y, T_rows, d, eps, ysc, s);
    case 3: return run_ln<T, 3>(x, g, b, y, T_rows, d, eps, ysc, s);
    case 4: return run_ln<T, 4>(x, g, b, y, T_rows, d, eps, ysc, s);
    case 5: return run_ln<T, 5>(x, g, b, y, T_rows, d, eps, ysc, s);
    case 6: return run_ln<T, 6>(x, g, b, y, T_rows, d, eps, ysc, s);
    case 7: return run_ln<T, 7>(x, g, b, y, T_rows, d, eps, ysc, s);
    case 8: return run_ln<T, 8>(x, g, b, y, T_rows, d, eps, ysc, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_layernorm(const float* x, const float* g, const float* b, void* y, int T, int d,
                            float eps, aut_dtype dt, hipStream_t s, uint8_t* y_scales) {
  if (T <= 0) return hipSuccess;
  if (d % 4 || d > 4 * 64 * LN_MAXV) return hipErrorInvalidValue;
  if (dt == AUT_FP8) {
    if (d % 128 || !y_scales) return hipErrorInvalidValue;
    return run_ln_any<uint8_t>(x, g, b, (uint8_t*)y, T, d, eps, y_scales, s);
  }
  if (dt == AUT_BF16) return run_ln_any<bf16_t>(x, g, b, (bf16_t*)y, T, d, eps, nullptr, s);
  return run_ln_any<float>(x, g, b, (float*)y, T, d, eps, nullptr, s);
}

}  // namespace aut
