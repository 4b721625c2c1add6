// MFMA GEMM for gfx950, 128 x 128 tiles: C[M, N] = A[M, K] * B[N, K]^T (+ epilogue).
// Used for the fp32 mode (eight fp32 MFMAs per 32-deep step); the bf16 mode
// runs the 256-row kernel in k_gemm256.hip.
//
// Both operands are k-contiguous (B is a PyTorch [out, in] weight), which is
// the natural operand order of the matrix cores: every lane fetches 8
// consecutive k-values of one row for a 32-deep step.
//
// Block tile 128 x 128, 4 waves (2 x 2), each wave 64 x 64 = 4 x 4 tiles of
// 16 x 16.  A k step moves 128 bytes of every tile row (64 bf16 or 32 fp32)
// through LDS; the two LDS buffers are double-buffered with one barrier per
// k step, the next step's global loads in flight during the MFMAs.  LDS rows
// are 8 units of 16 bytes, unit u of row r stored at u ^ (r & 7) so that the
// 16 rows read by one fragment load hit distinct banks.
//
// A-gather modes:
//  A_PLAIN   row-major A with leading dimension lda.
//  A_CONV    implicit GEMM of a 3x3, stride-2, pad-1 convolution over a
//            channels-last [chunk][y][x][c] activation: row m = output pixel,
//            k = tap * C + c with tap = 3 kh + kw (openarchlab "1A", section 3:
//            Conv2d(k=3, s=2, p=1)); taps outside the input grid read zero.
//  A_ROWMAP  row m is row rowmap[m] - rowmap_base of A (conv_out over the
//            valid tokens of a chunk batch).
// Epilogues: +bias, then store (operand type or fp32), GELU then store,
// residual add into fp32, or add a sinusoid position row (EPI_PE).
#include "aut_internal.h"
#include "device_common.h"

namespace aut {

namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int NT = 256;
constexpr int UNITS = 8;  // 16-byte units per tile row per k step

template <typename T, int AMODE, int EPI>
__global__ __launch_bounds__(NT) void gemm_kernel(GemmArgs p) {
  constexpr int E = UnitElems<T>::value;
  constexpr int BK = UNITS * E;
  typedef typename FragOf<T>::type Frag;
  __shared__ u32x4_t As[2][BM * UNITS];
  __shared__ u32x4_t Bs[2][BN * UNITS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int unit = tid & 7;
  const int rbase = tid >> 3;  // 0..31
  const int M = p.M, N = p.N, K = p.K;

  const char* arow[4];
  bool avalid[4];
  int aoy[4], aox[4];
  const char* brow[4];
  bool bvalid[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + rbase + 32 * i;
    avalid[i] = m < M;
    const int mm = avalid[i] ? m : 0;
    aoy[i] = 0;
    aox[i] = 0;
    if (AMODE == A_PLAIN) {
      arow[i] = (const char*)p.A + (size_t)mm * p.lda * sizeof(T);
    } else if (AMODE == A_ROWMAP) {
      const int r = avalid[i] ? (p.rowmap[mm] - p.rowmap_base) : 0;
      arow[i] = (const char*)p.A + (size_t)r * p.lda * sizeof(T);
    } else {
      const int hw = p.hout * p.wout;
      const int chunk = mm / hw;
      const int rem = mm - chunk * hw;
      if (p.xmajor) {
        aox[i] = rem / p.hout;
        aoy[i] = rem - aox[i] * p.hout;
      } else {
        aoy[i] = rem / p.wout;
        aox[i] = rem - aoy[i] * p.wout;
      }
      arow[i] = (const char*)p.A + (size_t)chunk * p.hin * p.win * p.cin * sizeof(T);
    }
    const int n = n0 + rbase + 32 * i;
    bvalid[i] = n < N;
    brow[i] = (const char*)p.B + (size_t)(bvalid[i] ? n : 0) * p.ldb * sizeof(T);
  }

  u32x4_t ra[4], rb[4];
  auto load_tile = [&](int k0) {
    const int k = k0 + unit * E;
    const bool kin = k < K;
    int ci = 0, kh = 0, kw = 0;
    if (AMODE == A_CONV) {
      const int tap = k / p.cin;
      ci = k - tap * p.cin;
      kh = tap / 3;
      kw = tap - 3 * kh;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (AMODE == A_CONV) {
        const int iy = 2 * aoy[i] + kh - 1;
        const int ix = 2 * aox[i] + kw - 1;
        const bool ok = avalid[i] && kin && iy >= 0 && iy < p.hin && ix >= 0 && ix < p.win;
        ra[i] = ok ? ldg_unit(arow[i] + ((size_t)(iy * p.win + ix) * p.cin + ci) * sizeof(T))
                   : zero_unit();
      } else {
        ra[i] = (avalid[i] && kin) ? ldg_unit(arow[i] + (size_t)k * sizeof(T)) : zero_unit();
      }
      rb[i] = (bvalid[i] && kin) ? ldg_unit(brow[i] + (size_t)k * sizeof(T)) : zero_unit();
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rbase + 32 * i;
      As[buf][r * UNITS + (unit ^ (r & 7))] = ra[i];
      Bs[buf][r * UNITS + (unit ^ (r & 7))] = rb[i];
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + BK - 1) / BK;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  const int lrow = lane & 15;
  const int g = lane >> 4;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tile((kt + 1) * BK);
#pragma unroll
    for (int s = 0; s < BK / 32; ++s) {
      Frag af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra_ = wm * 64 + 16 * i + lrow;
        const int rb_ = wn * 64 + 16 * i + lrow;
        if (E == 8) {
          const int u = 4 * s + g;
          frag_from_units(af[i], As[cur][ra_ * UNITS + (u ^ (ra_ & 7))], zero_unit());
          frag_from_units(bf[i], Bs[cur][rb_ * UNITS + (u ^ (rb_ & 7))], zero_unit());
        } else {
          const int u = 2 * g;
          frag_from_units(af[i], As[cur][ra_ * UNITS + (u ^ (ra_ & 7))],
                          As[cur][ra_ * UNITS + ((u + 1) ^ (ra_ & 7))]);
          frag_from_units(bf[i], Bs[cur][rb_ * UNITS + (u ^ (rb_ & 7))],
                          Bs[cur][rb_ * UNITS + ((u + 1) ^ (rb_ & 7))]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mma16_k32(acc[i][j], af[i], bf[j]);
    }
    if (kt + 1 < nk) store_tile(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds C[4 g + r][lrow] of each 16 x 16 tile
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn * 64 + 16 * j + lrow;
    if (n >= N) continue;
    const float bn = p.bias ? p.bias[n] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 64 + 16 * i + 4 * g + r;
        if (m >= M) continue;
        float v = acc[i][j][r] + bn;
        const size_t off = (size_t)m * p.ldo + n;
        if (EPI == EPI_STORE) {
          ((T*)p.out)[off] = from_f32<T>(v);
        } else if (EPI == EPI_STORE_GELU) {
          ((T*)p.out)[off] = from_f32<T>(gelu_f(v));
        } else if (EPI == EPI_RESID) {
          float* o = (float*)p.out + off;
          *o = *o + v;
        } else if (EPI == EPI_PE) {
          const int jpos = p.rowmap[m] % p.tpc;
          ((float*)p.out)[off] = v + p.pe[(size_t)jpos * N + n];
        } else {
          ((float*)p.out)[off] = v;
        }
      }
    }
  }
}

template <typename T, int AMODE, int EPI>
hipError_t run(const GemmArgs& a, hipStream_t s) {
  dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM);
  hipLaunchKernelGGL((gemm_kernel<T, AMODE, EPI>), grid, dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const GemmArgs& a, int amode, int epi, hipStream_t s) {
  if (amode == A_PLAIN) {
    switch (epi) {
      case EPI_STORE: return run<T, A_PLAIN, EPI_STORE>(a, s);
      case EPI_STORE_GELU: return run<T, A_PLAIN, EPI_STORE_GELU>(a, s);
      case EPI_RESID: return run<T, A_PLAIN, EPI_RESID>(a, s);
      case EPI_STORE_F32: return run<T, A_PLAIN, EPI_STORE_F32>(a, s);
      default: break;
    }
  } else if (amode == A_CONV && epi == EPI_STORE_GELU) {
    return run<T, A_CONV, EPI_STORE_GELU>(a, s);
  } else if (amode == A_ROWMAP && epi == EPI_PE) {
    return run<T, A_ROWMAP, EPI_PE>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm128(const GemmArgs& a, int amode, int epi, aut_dtype dt, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (dt == AUT_BF16) return dispatch<bf16_t>(a, amode, epi, s);
  return dispatch<float>(a, amode, epi, s);
}

}  // namespace aut
