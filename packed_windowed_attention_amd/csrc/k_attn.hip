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

// Row pitch of the transposed V in LDS.  Fragment reads take 8 bytes (bf16)
// or 16 (fp32) from 16 or 8 consecutive rows per 128-byte LDS cycle: a pitch
// of 8 or 16 bytes past a multiple of 128 puts those rows on distinct banks.
template <typename T> struct VtStride;
template <> struct VtStride<bf16_t> { static constexpr int value = LMAX + 4; };  // 264 bytes
template <> struct VtStride<float> { static constexpr int value = LMAX + 4; };   // 528 bytes

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

// four consecutive outputs in one store (8 bytes bf16, 16 bytes fp32)
__device__ __forceinline__ void store_quad(bf16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<u32x2_t*>(p) = u32x2_t{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}
__device__ __forceinline__ void store_quad(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// MX-fp8 output of a query row's 64 head columns: a lane holds columns
// 16 dt + 4 g + r (dt = 0..3, r = 0..3) of its query, so each 32-column block
// (dt = 0, 1 or dt = 2, 3) is spread over the four lanes of the query's row
// group; its maximum takes two shuffles across them.
__device__ __forceinline__ void store_row_mx(uint8_t* orow, uint8_t* osc, int row, int col0, int d,
                                             int g, const float (&v)[4][4], bool live) {
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    float amax = 0.f;
#pragma unroll
    for (int dt = 2 * blk; dt < 2 * blk + 2; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) amax = fmaxf(amax, fabsf(v[dt][r]));
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    if (!live) continue;
    const int e = mx_exponent(amax);
#pragma unroll
    for (int dt = 2 * blk; dt < 2 * blk + 2; ++dt)
      *reinterpret_cast<unsigned int*>(orow + dt * 16 + 4 * g) =
          pack_fp8x4(mx_scale_down(v[dt][0], e), mx_scale_down(v[dt][1], e),
                     mx_scale_down(v[dt][2], e), mx_scale_down(v[dt][3], e));
    if (g == blk) osc[mx_scale_index(row, (col0 >> 5) + blk, d)] = (uint8_t)(e + 127);
  }
}

template <typename T, bool MX>
__global__ __launch_bounds__(ATT_THREADS) void attn_kernel(const T* __restrict__ qkv,
                                                          void* __restrict__ o_,
                                                          const int* __restrict__ cu,
                                                          const int* __restrict__ worder, int H,
                                                          int d, uint8_t* __restrict__ osc) {
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
  const size_t ld = 3 * (size_t)d;
  const T* qb = qkv + (size_t)s0 * ld + (size_t)h * 64;
  const T* kb = qb + d;
  const T* vb = qb + 2 * (size_t)d;

  // Every global load of the workgroup is issued before any is used: thread t
  // takes unit u = t % UR of the RPT consecutive key rows starting at
  // RPT * (t / UR) (K and V), and each wave the Q fragments of its query tiles
  // wave and wave + 4.  Then K goes to LDS unit by unit and V transposed, RPT
  // rows at a time (one 8- or 32-byte write per element of the unit).
  constexpr int RPT = LMAX * UR / ATT_THREADS;  // key rows per thread: 4 (bf16), 8 (fp32)
  const int ku = tid % UR;
  const int kj0 = RPT * (tid / UR);
  u32x4_t kreg[RPT], vreg[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int j = kj0 + r;
    kreg[r] = j < L ? ldg_unit(kb + (size_t)j * ld + ku * E) : zero_unit();
    vreg[r] = j < L ? ldg_unit(vb + (size_t)j * ld + ku * E) : zero_unit();
  }
  constexpr int QU = E == 8 ? 2 : 4;  // Q units per lane per query tile
  u32x4_t qreg[2][QU];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = (wave + 4 * q) * 16 + lrow;
#pragma unroll
    for (int s = 0; s < QU; ++s) {
      // bf16: units 4 s' + g of k-half s'; fp32: units 8 s' + 2 g (+1)
      const int u = E == 8 ? 4 * s + g : 8 * (s >> 1) + 2 * g + (s & 1);
      qreg[q][s] = i < L ? ldg_unit(qb + (size_t)i * ld + u * E) : zero_unit();
    }
  }
#pragma unroll
  for (int r = 0; r < RPT; ++r) Ks[(kj0 + r) * UR + kswz<T>(ku, kj0 + r)] = kreg[r];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    T col[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      T tmp[E];
      __builtin_memcpy(tmp, &vreg[r], 16);
      col[r] = tmp[e];
    }
    T* dst = &Vt[(ku * E + e) * VS + kj0];
    if (E == 8) {
      u32x2_t w2;
      __builtin_memcpy(&w2, col, 8);
      *reinterpret_cast<u32x2_t*>(dst) = w2;
    } else {
      u32x4_t w4[2];
      __builtin_memcpy(w4, col, 32);
      reinterpret_cast<u32x4_t*>(dst)[0] = w4[0];
      reinterpret_cast<u32x4_t*>(dst)[1] = w4[1];
    }
  }
  __syncthreads();

  // scores in log2 units: softmax(s / 8) = 2^(s log2(e) / 8 - max) / sum
  const float c = 0.125f * 1.44269504088896341f;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int it = wave + 4 * q;
    if (it * 16 >= L) break;
    const int i = it * 16 + lrow;
    Frag qf[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (E == 8) frag_from_units(qf[s], qreg[q][s], zero_unit());
      else frag_from_units(qf[s], qreg[q][2 * s], qreg[q][2 * s + 1]);
    }
    // S^T = K Q^T over all LMAX key rows (rows past the window are zero in LDS
    // and masked below): straight-line code, so every fragment read is issued
    // ahead of the matrix instructions that use it
    Frag kf[8][2];
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) {
      const int jr = jt * 16 + lrow;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (E == 8) {
          frag_from_units(kf[jt][s], Ks[jr * UR + kswz<T>(4 * s + g, jr)], zero_unit());
        } else {
          const int u = 8 * s + 2 * g;
          frag_from_units(kf[jt][s], Ks[jr * UR + kswz<T>(u, jr)], Ks[jr * UR + kswz<T>(u + 1, jr)]);
        }
      }
    }
    float t[8][4];
    float mx = -INFINITY;
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      mma16_k32(acc, kf[jt][0], qf[0]);
      mma16_k32(acc, kf[jt][1], qf[1]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = jt * 16 + 4 * g + r;
        t[jt][r] = j < L ? acc[r] * c : -INFINITY;
        mx = fmaxf(mx, t[jt][r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    float sum = 0.f;
#pragma unroll
    for (int jt = 0; jt < 8; ++jt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        t[jt][r] = __builtin_amdgcn_exp2f(t[jt][r] - mx);  // masked keys: 2^-inf = 0
        sum += t[jt][r];
      }
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);

    // O^T = V^T P^T, V^T fragments read ahead in two batches of 8
    f32x4_t oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      Frag vf[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const T* vrow = Vt + (dt * 16 + lrow) * VS + 32 * (2 * half + u) + 4 * g;
          frag_v(vf[u][dt], vrow, vrow + 16);
        }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int tt = 2 * half + u;
        Frag pf;
        frag_p(pf, t[2 * tt], t[2 * tt + 1]);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) mma16_k32(oacc[dt], vf[u][dt], pf);
      }
    }
    const float inv = __builtin_amdgcn_rcpf(sum);
    if constexpr (MX) {
      float v[4][4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[dt][r] = oacc[dt][r] * inv;
      store_row_mx((uint8_t*)o_ + (size_t)(s0 + i) * d + (size_t)h * 64, osc, s0 + i, h * 64, d, g,
                   v, i < L);
    } else if (i < L) {
      T* orow = (T*)o_ + (size_t)(s0 + i) * d + (size_t)h * 64;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        store_quad(orow + dt * 16 + 4 * g, oacc[dt][0] * inv, oacc[dt][1] * inv,
                   oacc[dt][2] * inv, oacc[dt][3] * inv);
    }
  }
}

}  // namespace

hipError_t launch_attention(const void* qkv, void* o, const int* cu, const int* worder,
                            int n_windows, int H, int d, aut_dtype dt, hipStream_t s,
                            uint8_t* o_scales) {
  if (n_windows <= 0) return hipSuccess;
  dim3 grid(n_windows * H);
  if (dt == AUT_FP8) {
    if (d % 128 || !o_scales) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_kernel<bf16_t, true>), grid, dim3(ATT_THREADS), 0, s,
                       (const bf16_t*)qkv, o, cu, worder, H, d, o_scales);
  } else if (dt == AUT_BF16) {
    hipLaunchKernelGGL((attn_kernel<bf16_t, false>), grid, dim3(ATT_THREADS), 0, s,
                       (const bf16_t*)qkv, o, cu, worder, H, d, (uint8_t*)nullptr);
  } else {
    hipLaunchKernelGGL((attn_kernel<float, false>), grid, dim3(ATT_THREADS), 0, s,
                       (const float*)qkv, o, cu, worder, H, d, (uint8_t*)nullptr);
  }
  return hipGetLastError();
}

}  // namespace aut
