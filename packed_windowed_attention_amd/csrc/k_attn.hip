// Packed window attention for gfx950.
//
// For every window [s, e) of cu_seqlens and every head: O = softmax(Q K^T /
// sqrt(64)) V over the window's own tokens only -- bidirectional, no mask
// inside the window, nothing across windows (m-star API page, module summary
// and AuTAttention: SDPA per window from cu_seqlens; openarchlab "1A",
// section 3: is_causal = False inside each cu_seqlens segment).
//
// One workgroup per (window, head).  The window's K (row-major) and V
// (transposed) live in LDS, zero past the window's end, so padded keys
// contribute exactly nothing and no row of another window is ever read.  Each
// wave takes 16 queries at a time and computes S^T = K Q^T on the matrix
// cores: a lane then holds the scores of one query (its column) for 16 keys
// per tile, which is exactly the B-operand layout of the second product
// O^T = V^T P^T, so P never leaves registers.  The softmax reductions over
// keys run within a lane and across the four lane groups with wavefront
// shuffles.  Windows are visited longest first (the plan's order) so short
// tail windows fill the end of the grid.
#include "aut_internal.h"
#include "device_common.h"

namespace aut {

namespace {

constexpr int ATT_THREADS = 256;
constexpr int LMAX = 128;

template <typename T> struct VtStride;
template <> struct VtStride<bf16_t> { static constexpr int value = LMAX + 8; };
template <> struct VtStride<float> { static constexpr int value = LMAX + 4; };

template <typename T>
__device__ __forceinline__ int kswz(int u, int j) {
  return sizeof(T) == 2 ? (u ^ (j & 7)) : (u ^ ((j & 7) << 1));
}

__device__ __forceinline__ void frag_p(FragBF16& f, const float (&a)[4], const float (&b)[4]) {
  f.v = __builtin_bit_cast(bf16x8_t, u32x4_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                             pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])});
}
__device__ __forceinline__ void frag_p(FragF32& f, const float (&a)[4], const float (&b)[4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    f.v[r] = a[r];
    f.v[4 + r] = b[r];
  }
}

// Four consecutive elements of a transposed-V row: 8 bytes (bf16) or 16 (fp32).
__device__ __forceinline__ void vt_quad(const bf16_t* p, unsigned int (&w)[4], int half) {
  const u32x2_t x = *reinterpret_cast<const u32x2_t*>(p);
  w[2 * half] = x[0];
  w[2 * half + 1] = x[1];
}
__device__ __forceinline__ void frag_v(FragBF16& f, const bf16_t* p0, const bf16_t* p1) {
  unsigned int w[4];
  vt_quad(p0, w, 0);
  vt_quad(p1, w, 1);
  f.v = __builtin_bit_cast(bf16x8_t, u32x4_t{w[0], w[1], w[2], w[3]});
}
__device__ __forceinline__ void frag_v(FragF32& f, const float* p0, const float* p1) {
  const float4 a = *reinterpret_cast<const float4*>(p0);
  const float4 b = *reinterpret_cast<const float4*>(p1);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

template <typename T>
__global__ __launch_bounds__(ATT_THREADS) void attn_kernel(const T* __restrict__ qkv,
                                                          T* __restrict__ o,
                                                          const int* __restrict__ cu,
                                                          const int* __restrict__ worder, int H,
                                                          int d) {
  constexpr int E = UnitElems<T>::value;  // elements per 16-byte unit
  constexpr int UR = 64 / E;              // units per head row
  constexpr int VS = VtStride<T>::value;
  typedef typename FragOf<T>::type Frag;
  __shared__ u32x4_t Ks[LMAX * UR];
  __shared__ T Vt[64 * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, g = lane >> 4;
  const int w = worder[blockIdx.x / H];
  const int h = blockIdx.x - (blockIdx.x / H) * H;
  const int s0 = cu[w];
  const int L = cu[w + 1] - s0;
  const int Lp = (L + 31) & ~31;
  const size_t ld = 3 * (size_t)d;
  const T* qb = qkv + (size_t)s0 * ld + (size_t)h * 64;
  const T* kb = qb + d;
  const T* vb = qb + 2 * (size_t)d;

  for (int idx = tid; idx < Lp * UR; idx += ATT_THREADS) {
    const int j = idx / UR, u = idx - j * UR;
    const u32x4_t kv = j < L ? ldg_unit(kb + (size_t)j * ld + u * E) : zero_unit();
    Ks[j * UR + kswz<T>(u, j)] = kv;
    const u32x4_t vv = j < L ? ldg_unit(vb + (size_t)j * ld + u * E) : zero_unit();
    T tmp[E];
    __builtin_memcpy(tmp, &vv, 16);
#pragma unroll
    for (int e = 0; e < E; ++e) Vt[(u * E + e) * VS + j] = tmp[e];
  }
  __syncthreads();

  const int JT = Lp >> 4;
  // scores in log2 units: softmax(s / 8) = 2^(s log2(e) / 8 - max) / sum
  const float c = 0.125f * 1.44269504088896341f;
  for (int it = wave; it * 16 < L; it += ATT_THREADS / 64) {
    const int i = it * 16 + lrow;
    Frag qf[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const T* qp = qb + (size_t)i * ld + 32 * s + 8 * g;
      if (E == 8) {
        frag_from_units(qf[s], i < L ? ldg_unit(qp) : zero_unit(), zero_unit());
      } else {
        frag_from_units(qf[s], i < L ? ldg_unit(qp) : zero_unit(),
                        i < L ? ldg_unit(qp + 4) : zero_unit());
      }
    }
    float t[8][4];
    float mx = -INFINITY;
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) {
      if (jt < JT) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        const int jr = jt * 16 + lrow;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          Frag kf;
          if (E == 8) {
            frag_from_units(kf, Ks[jr * UR + kswz<T>(4 * s + g, jr)], zero_unit());
          } else {
            const int u = 8 * s + 2 * g;
            frag_from_units(kf, Ks[jr * UR + kswz<T>(u, jr)], Ks[jr * UR + kswz<T>(u + 1, jr)]);
          }
          mma16_k32(acc, kf, qf[s]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = jt * 16 + 4 * g + r;
          t[jt][r] = j < L ? acc[r] * c : -INFINITY;
          mx = fmaxf(mx, t[jt][r]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) t[jt][r] = -INFINITY;
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    float sum = 0.f;
#pragma unroll
    for (int jt = 0; jt < 8; ++jt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        t[jt][r] = jt < JT ? exp2f(t[jt][r] - mx) : 0.f;
        sum += t[jt][r];
      }
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);

    f32x4_t oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      if (2 * tt < JT) {
        Frag pf;
        frag_p(pf, t[2 * tt], t[2 * tt + 1]);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const T* vrow = Vt + (dt * 16 + lrow) * VS + 32 * tt + 4 * g;
          Frag vf;
          frag_v(vf, vrow, vrow + 16);
          mma16_k32(oacc[dt], vf, pf);
        }
      }
    }
    if (i < L) {
      const float inv = 1.0f / sum;
      T* orow = o + (size_t)(s0 + i) * d + (size_t)h * 64;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) orow[dt * 16 + 4 * g + r] = from_f32<T>(oacc[dt][r] * inv);
    }
  }
}

}  // namespace

hipError_t launch_attention(const void* qkv, void* o, const int* cu, const int* worder,
                            int n_windows, int H, int d, aut_dtype dt, hipStream_t s) {
  if (n_windows <= 0) return hipSuccess;
  dim3 grid(n_windows * H);
  if (dt == AUT_BF16)
    hipLaunchKernelGGL(attn_kernel<bf16_t>, grid, dim3(ATT_THREADS), 0, s, (const bf16_t*)qkv,
                       (bf16_t*)o, cu, worder, H, d);
  else
    hipLaunchKernelGGL(attn_kernel<float>, grid, dim3(ATT_THREADS), 0, s, (const float*)qkv,
                       (float*)o, cu, worder, H, d);
  return hipGetLastError();
}

}  // namespace aut
