// Packed window attention for gfx950.
//
// For every window [s, e) of cu_seqlens and every head: O = softmax(Q K^T /
// sqrt(64)) V over the window's own tokens only -- bidirectional, no mask
// inside the window, nothing across windows (m-star API page, module summary
// and AuTAttention: SDPA per window from cu_seqlens; openarchlab "1A",
// section 3: is_causal = False inside each cu_seqlens segment).
//
// One workgroup per (window, head).  The window's K (row-major) and V
// (transposed) live in LDS, zero past the window's end (loads go through a
// buffer descriptor that covers the window's rows only, so a load past its end
// reads zero and no row of another window is ever read).  Each wave takes 16
// queries at a time and computes S^T = K Q^T on the matrix cores: a lane then
// holds the scores of one query (its column) for 16 keys per tile, which is
// exactly the B-operand layout of the second product O^T = V^T P^T, so P never
// leaves registers.  Key tiles that hold only padding are skipped and only
// tiles that hold both real and padded keys are masked.  The softmax
// reductions over keys run within a lane and across the four lane groups with
// lane-swap instructions.  Windows are visited longest first (the plan's
// order) so short tail windows fill the end of the grid.
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

// Reductions across the lane groups of a query's scores (lanes l, l ^ 16,
// l ^ 32, l ^ 48): v_permlane16_swap / v_permlane32_swap exchange halves of
// the wavefront in the vector unit, so the pair's two values sit in the two
// results of one instruction, in every lane (no LDS round trip).
__device__ __forceinline__ float pair_max16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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
    amax = pair_max16(amax);
    amax = pair_max32(amax);
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

// One (window, head) item's operands in registers: thread t holds unit
// u = t % UR of the RPT consecutive key rows from RPT * (t / UR) (K and V),
// and each wave the Q fragments of its query tiles wave and wave + 4.
template <typename T>
struct ItemRegs {
  static constexpr int E = UnitElems<T>::value;           // elements per 16-byte unit
  static constexpr int UR = 64 / E;                        // units per head row
  static constexpr int RPT = LMAX * UR / ATT_THREADS;     // key rows per thread: 4 (bf16), 8 (fp32)
  static constexpr int QU = E == 8 ? 2 : 4;                // Q units per lane per query tile
  u32x4_t k[RPT], v[RPT];
  u32x4_t q[2][QU];
};

struct Item {
  int s0, L, h;
  bool ok;
};

// A window order entry outside [0, n_windows), or a window that is not within
// rows [0, T) or holds more than LMAX rows, gives an item that does nothing
// (the planner never makes one; the check keeps a caller's bad table from
// reading or writing outside the buffers).
__device__ __forceinline__ Item item_of(int item, const int* __restrict__ cu,
                                        const int* __restrict__ worder, int H, int n_windows, int T) {
  const int wi = item / H;
  const int w = worder[wi];
  Item it;
  it.h = item - wi * H;
  it.ok = w >= 0 && w < n_windows;
  it.s0 = it.ok ? cu[w] : 0;
  it.L = it.ok ? cu[w + 1] - it.s0 : 0;
  it.ok = it.ok && it.s0 >= 0 && it.L >= 0 && it.L <= LMAX && it.s0 <= T - it.L;
  return it;
}

// The rows of an item's window as a buffer: a load past the window's last row
// returns zero, so the padded keys and queries need no branch (a branch per
// load made the compiler wait for each load before issuing the next).
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t window_rsrc(const T* __restrict__ qkv, const Item& it,
                                                             int d) {
  const size_t ld = 3 * (size_t)d;
  return __builtin_amdgcn_make_buffer_rsrc((void*)(qkv + (size_t)it.s0 * ld), (short)0,
                                           (int)((size_t)it.L * ld * sizeof(T)), 0x00020000);
}

template <typename T>
__device__ __forceinline__ void load_q(ItemRegs<T>& r, const T* __restrict__ qkv, const Item& it,
                                       int d, int tid) {
  constexpr int E = ItemRegs<T>::E, QU = ItemRegs<T>::QU;
  const int lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 15, g = lane >> 4;
  const unsigned ldb = 3u * (unsigned)d * sizeof(T);
  const __amdgpu_buffer_rsrc_t rs = window_rsrc(qkv, it, d);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = (wave + 4 * q) * 16 + lrow;
#pragma unroll
    for (int s = 0; s < QU; ++s) {
      // bf16: units 4 s' + g of k-half s'; fp32: units 8 s' + 2 g (+1)
      const int u = E == 8 ? 4 * s + g : 8 * (s >> 1) + 2 * g + (s & 1);
      const unsigned off = (unsigned)i * ldb + (unsigned)((it.h * 64 + u * E) * sizeof(T));
      r.q[q][s] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    }
  }
}

template <typename T>
__device__ __forceinline__ void load_item(ItemRegs<T>& r, const T* __restrict__ qkv, const Item& it,
                                          int d, int tid) {
  constexpr int E = ItemRegs<T>::E, UR = ItemRegs<T>::UR, RPT = ItemRegs<T>::RPT;
  const unsigned ldb = 3u * (unsigned)d * sizeof(T);
  const __amdgpu_buffer_rsrc_t rs = window_rsrc(qkv, it, d);
  const int ku = tid % UR;
  const int kj0 = RPT * (tid / UR);
  const unsigned koff = (unsigned)((d + it.h * 64 + ku * E) * sizeof(T));
  const unsigned voff = koff + (unsigned)(d * sizeof(T));
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const unsigned row = (unsigned)(kj0 + j) * ldb;
    r.k[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, row + koff, 0, 0));
    r.v[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, row + voff, 0, 0));
  }
  load_q(r, qkv, it, d, tid);
}

// K to LDS unit by unit, V transposed, RPT rows at a time (one 8- or 32-byte
// write per element of the unit).
template <typename T>
__device__ __forceinline__ void stage_item(const ItemRegs<T>& r, u32x4_t* Ks, T* Vt, int tid) {
  constexpr int E = ItemRegs<T>::E, UR = ItemRegs<T>::UR, RPT = ItemRegs<T>::RPT;
  constexpr int VS = VtStride<T>::value;
  const int ku = tid % UR;
  const int kj0 = RPT * (tid / UR);
#pragma unroll
  for (int j = 0; j < RPT; ++j) Ks[(kj0 + j) * UR + kswz<T>(ku, kj0 + j)] = r.k[j];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    T col[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      T tmp[E];
      __builtin_memcpy(tmp, &r.v[j], 16);
      col[j] = tmp[e];
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
}

// One 16-query tile of an item: the scores of NKT key tiles (the rest hold
// only padded keys and are skipped: their probabilities are zero), masked in
// every tile (MASK_ALL, short windows) or in the last one only.  A lane ends
// up with one query's scores (its column of S^T), so the softmax reductions
// are in-lane plus two wavefront shuffles.
template <typename T, typename OT, bool MX, int NKT, bool MASK_ALL>
__device__ __forceinline__ void query_tile(const u32x4_t* Ks, const T* Vt,
                                           const u32x4_t (&qr)[ItemRegs<T>::QU], int qt,
                                           const Item& it, void* __restrict__ o_, int d,
                                           uint8_t* __restrict__ osc, int lane) {
  constexpr int E = ItemRegs<T>::E, UR = ItemRegs<T>::UR;
  constexpr int VS = VtStride<T>::value;
  typedef typename FragOf<T>::type Frag;
  const int lrow = lane & 15, g = lane >> 4;
  const int L = it.L;
  const int i = qt * 16 + lrow;
  Frag qf[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    if (E == 8) frag_from_units(qf[s], qr[s], zero_unit());
    else frag_from_units(qf[s], qr[2 * s], qr[2 * s + 1]);
  }
  // S^T = K Q^T: every fragment read is issued ahead of the matrix
  // instructions that use it.  (The row index is made opaque per query tile:
  // otherwise the compiler keeps one tile's K fragments live for the next and
  // runs out of registers.)
  int krow = lrow;
  asm volatile("" : "+v"(krow));
  Frag kf[NKT][2];
#pragma unroll
  for (int jt = 0; jt < NKT; ++jt) {
    const int jr = jt * 16 + krow;
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
  // raw scores; padded keys -inf
  float t[8][4];
  float mx = -INFINITY;
#pragma unroll
  for (int jt = 0; jt < NKT; ++jt) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    mma16_k32(acc, kf[jt][0], qf[0]);
    mma16_k32(acc, kf[jt][1], qf[1]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = jt * 16 + 4 * g + r;
      t[jt][r] = (MASK_ALL || jt == NKT - 1) && j >= L ? -INFINITY : acc[r];
      mx = fmaxf(mx, t[jt][r]);
    }
  }
  mx = pair_max16(mx);
  mx = pair_max32(mx);
  // softmax(s / 8) = 2^(s c - max c) / sum with c = log2(e) / 8; c > 0, so the
  // scaled maximum is the maximum of the scaled scores
  const float c = 0.125f * 1.44269504088896341f;
  const float mc = mx * c;
  float sum = 0.f;
#pragma unroll
  for (int jt = 0; jt < 8; ++jt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (jt < NKT) {
        t[jt][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(t[jt][r], c, -mc));  // -inf: 0
        sum += t[jt][r];
      } else {
        t[jt][r] = 0.f;
      }
    }
  sum = pair_sum16(sum);
  sum = pair_sum32(sum);

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
  const int s0 = it.s0, h = it.h;
  if constexpr (MX) {
    float v[4][4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) v[dt][r] = oacc[dt][r] * inv;
    store_row_mx((uint8_t*)o_ + (size_t)(s0 + i) * d + (size_t)h * 64, osc, s0 + i, h * 64, d, g, v,
                 i < L);
  } else if (i < L) {
    OT* orow = (OT*)o_ + (size_t)(s0 + i) * d + (size_t)h * 64;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      store_quad(orow + dt * 16 + 4 * g, oacc[dt][0] * inv, oacc[dt][1] * inv, oacc[dt][2] * inv,
                 oacc[dt][3] * inv);
  }
}

// One item's attention from LDS (K, transposed V) and the Q fragments in
// registers: each wave its query tiles wave and wave + 4.  Windows of 97 to
// 112 tokens (the common full window) skip the eighth key tile; windows of
// more than 112 mask the eighth only; shorter ones mask every tile.
template <typename T, typename OT, bool MX>
__device__ __forceinline__ void compute_item(const u32x4_t* Ks, const T* Vt,
                                             const u32x4_t (&qreg)[2][ItemRegs<T>::QU],
                                             const Item& it, void* __restrict__ o_, int d,
                                             uint8_t* __restrict__ osc, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int qt = wave + 4 * q;
    if (qt * 16 >= it.L) break;
    if (it.L > 112)
      query_tile<T, OT, MX, 8, false>(Ks, Vt, qreg[q], qt, it, o_, d, osc, lane);
    else if (it.L > 96)
      query_tile<T, OT, MX, 7, false>(Ks, Vt, qreg[q], qt, it, o_, d, osc, lane);
    else
      query_tile<T, OT, MX, 8, true>(Ks, Vt, qreg[q], qt, it, o_, d, osc, lane);
  }
}

// One workgroup per (window, head) item, items window-major in the plan's
// window order (longest first, so short tail windows fill the end of the
// grid): every load issued at once, K and V to LDS, then the matrix work.
template <typename T, typename OT, bool MX>
__global__ __launch_bounds__(ATT_THREADS)
__attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 4 : 2))) void attn_kernel(
    const T* __restrict__ qkv, void* __restrict__ o_, const int* __restrict__ cu,
    const int* __restrict__ worder, int H, int d, uint8_t* __restrict__ osc, int n_windows, int T_rows) {
  constexpr int UR = ItemRegs<T>::UR;
  constexpr int VS = VtStride<T>::value;
  __shared__ u32x4_t Ks[LMAX * UR];
  __shared__ T Vt[64 * VS];
  const int tid = threadIdx.x;
  ItemRegs<T> r;
  const Item it = item_of((int)blockIdx.x, cu, worder, H, n_windows, T_rows);
  if (!it.ok) return;  // uniform over the workgroup, before any barrier
  load_item(r, qkv, it, d, tid);
  stage_item(r, Ks, Vt, tid);
  __syncthreads();
  compute_item<T, OT, MX>(Ks, Vt, r.q, it, o_, d, osc, tid);
}

}  // namespace

hipError_t launch_attention(const void* qkv, void* o, const int* cu, const int* worder,
                            int n_windows, int H, int d, aut_dtype dt, hipStream_t s,
                            uint8_t* o_scales, int T, bool f32_out) {
  if (n_windows <= 0) return hipSuccess;
  // a window's rows must fit a buffer descriptor's 32-bit byte range; the
  // grid's item count must fit an int
  if (d != 64 * H || (size_t)LMAX * 3 * (size_t)d * (dt == AUT_FP32 ? 4 : 2) >= ((size_t)1 << 31) ||
      (long long)n_windows * H >= ((long long)1 << 31))
    return hipErrorInvalidValue;
  dim3 grid(n_windows * H);
  if (dt == AUT_FP8) {
    if (d % 128 || !o_scales) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_kernel<bf16_t, bf16_t, true>), grid, dim3(ATT_THREADS), 0, s,
                       (const bf16_t*)qkv, o, cu, worder, H, d, o_scales, n_windows, T);
  } else if (dt == AUT_BF16 && f32_out) {
    hipLaunchKernelGGL((attn_kernel<bf16_t, float, false>), grid, dim3(ATT_THREADS), 0, s,
                       (const bf16_t*)qkv, o, cu, worder, H, d, (uint8_t*)nullptr, n_windows, T);
  } else if (dt == AUT_BF16) {
    hipLaunchKernelGGL((attn_kernel<bf16_t, bf16_t, false>), grid, dim3(ATT_THREADS), 0, s,
                       (const bf16_t*)qkv, o, cu, worder, H, d, (uint8_t*)nullptr, n_windows, T);
  } else {
    hipLaunchKernelGGL((attn_kernel<float, float, false>), grid, dim3(ATT_THREADS), 0, s,
                       (const float*)qkv, o, cu, worder, H, d, (uint8_t*)nullptr, n_windows, T);
  }
  return hipGetLastError();
}

}  // namespace aut
