// Whisper-style log-mel front end on the GPU: 16 kHz mono audio -> 128-bin
// log-mel at 100 frames/s, the encoder's input ("Audio Encoder Component",
// cubic.dev wiki, Processing Pipeline: 16 kHz mono audio to a 128-bin mel
// spectrogram; m-star module summary: a Whisper-style log-mel input).  The
// recipe beyond what the pages fix is the published Whisper front end: a
// 400-sample periodic Hann window and 400-point DFT every 160 samples on
// reflect-padded centred frames (N / 160 frames), the power spectrum, a
// Slaney mel filterbank over 0..8000 Hz, log10 of max(mel, 1e-10), a floor at
// the request's maximum - 8, then (x + 4) / 4.
//
// Both products are dense and run on the matrix cores in fp32
// (v_mfma_f32_16x16x4_f32): a workgroup takes 64 frames of one request, keeps
// the audio span they cover (reflect-padded at the request's ends) in LDS and
// multiplies it by the window-times-DFT table [400 x 416] (for each 16-bin
// tile, a cosine column tile then a sine one, so a lane holds the real and
// imaginary part of the same bin), streamed through LDS 40 rows at a time.
// The power spectrum goes back to LDS and is multiplied by the filterbank
// [208 bins x 128 mel].  log10 values go straight to the encoder's layout
// [B][128][T_max] with the request's maximum kept by an atomic max; a second
// pass applies the floor and the scaling.
#include <math.h>

#include "aut_internal.h"
#include "device_common.h"

namespace aut {

namespace {

constexpr int LM_FRAMES = 64;                    // frames per workgroup
constexpr int LM_THREADS = 256;                  // 4 waves x 16 frames
constexpr int LM_SPAN = LM_FRAMES * LM_HOP + LM_NFFT - LM_HOP;  // samples covered
constexpr int LM_KC = 40;                        // DFT table rows per LDS chunk
constexpr int LM_TILES = 2 * LM_BIN_TILES;       // cos / sin column tiles
constexpr int LM_COLS = 16 * LM_TILES;           // 416
// LDS layouts, padded so that the reads of a 32-lane cycle (16 frames or rows
// x 2 values of k) fall on distinct banks (32 banks of 4 bytes):
// the audio span with 2 floats after every hop of 160 samples (a frame starts
// 162 floats after the previous one: 2 banks on), the DFT table chunk with a
// row pitch of 432 floats (16 banks on), the power spectrum with 226 (2 on).
constexpr int LM_SPAN_LDS = LM_SPAN + 2 * (LM_SPAN / LM_HOP + 1);
constexpr int LM_COLS_LDS = LM_COLS + 16;        // 432
constexpr int LM_PB_LDS = 16 * LM_BIN_TILES + 18;  // 226
__device__ __forceinline__ int span_slot(int i) { return i + 2 * (i / LM_HOP); }

// Slaney mel scale (linear 3/200 mel per Hz up to 1 kHz = 15 mel, then 27
// mel per factor 6.4) and its inverse
__device__ double slaney_mel(double f) {
  return f >= 1000.0 ? 15.0 + 27.0 * log(f / 1000.0) / log(6.4) : 3.0 * f / 200.0;
}
__device__ double slaney_hz(double m) {
  return m >= 15.0 ? 1000.0 * exp((m - 15.0) * log(6.4) / 27.0) : 200.0 * m / 3.0;
}

// tables: dft [LM_NFFT][LM_COLS], then mel [16 * LM_BIN_TILES][LM_MELS]
__global__ void logmel_tables_kernel(float* dft, float* mel) {
  const int total_dft = LM_NFFT * LM_COLS;
  const int total_mel = 16 * LM_BIN_TILES * LM_MELS;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total_dft + total_mel;
       i += gridDim.x * blockDim.x) {
    if (i < total_dft) {
      const int n = i / LM_COLS, col = i - n * LM_COLS;
      const int tile = col / 16, j = col - tile * 16;
      const int bin = 16 * (tile / 2) + j;
      double v = 0.0;
      if (bin <= LM_NFFT / 2) {
        const double w = 0.5 - 0.5 * cos(2.0 * M_PI * n / LM_NFFT);  // periodic Hann
        const double ph = 2.0 * M_PI * (double)((long)bin * n % LM_NFFT) / LM_NFFT;
        v = w * ((tile & 1) ? -sin(ph) : cos(ph));
      }
      dft[i] = (float)v;
    } else {
      const int k = i - total_dft;
      const int bin = k / LM_MELS, m = k - bin * LM_MELS;
      double v = 0.0;
      if (bin <= LM_NFFT / 2) {
        const double top = slaney_mel(LM_RATE / 2.0);
        const double lo = slaney_hz(top * m / (LM_MELS + 1));
        const double c = slaney_hz(top * (m + 1) / (LM_MELS + 1));
        const double hi = slaney_hz(top * (m + 2) / (LM_MELS + 1));
        const double f = (double)bin * LM_RATE / LM_NFFT;
        const double t = fmin((f - lo) / (c - lo), (hi - f) / (hi - c));
        v = t > 0.0 ? t * 2.0 / (hi - lo) : 0.0;
      }
      mel[k] = (float)v;
    }
  }
}

__global__ void logmel_init_kernel(unsigned* mx, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) mx[b] = 0u;  // below every (log10 value + 16) > 0
}

__device__ __forceinline__ f32x4_t mma4(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(LM_THREADS) void logmel_kernel(
    const float* __restrict__ audio, long s_max, const int* __restrict__ lens, const float* __restrict__ dft,
    const float* __restrict__ melw, float* __restrict__ feat, int T_max, unsigned* __restrict__ mx) {
  __shared__ float span[LM_SPAN_LDS];
  __shared__ float buf[LM_KC * LM_COLS_LDS];  // DFT table chunk, then the power spectrum
  static_assert(LM_FRAMES * LM_PB_LDS <= LM_KC * LM_COLS_LDS, "power tile fits");
  const int b = blockIdx.y;
  const int N = lens[b];
  const int nf = N / LM_HOP;
  const int f0 = blockIdx.x * LM_FRAMES;
  if (f0 >= nf) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, g = lane >> 4;
  const float* x = audio + (long)b * s_max;

  // samples f0 * 160 - 200 .. + LM_SPAN, reflected at the request's ends
  for (int i = tid; i < LM_SPAN; i += LM_THREADS) {
    int s = f0 * LM_HOP - LM_NFFT / 2 + i;
    if (s < 0) s = -s;
    if (s >= N) s = 2 * (N - 1) - s;
    span[span_slot(i)] = (s >= 0 && s < N) ? x[s] : 0.f;
  }

  // DFT: acc[t] = 16 frames (this wave's) x 16 columns of tile t
  f32x4_t acc[LM_TILES];
#pragma unroll
  for (int t = 0; t < LM_TILES; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int frame_off = (16 * wave + lr) * (LM_HOP + 2);  // span_slot of the frame's first sample
  for (int c = 0; c < LM_NFFT / LM_KC; ++c) {
    __syncthreads();  // the previous chunk is consumed (and the span is in place)
    const float4* src = reinterpret_cast<const float4*>(dft + (long)c * LM_KC * LM_COLS);
    for (int i = tid; i < LM_KC * LM_COLS / 4; i += LM_THREADS) {
      const int row = i / (LM_COLS / 4);
      reinterpret_cast<float4*>(buf)[i + row * ((LM_COLS_LDS - LM_COLS) / 4)] = src[i];
    }
    __syncthreads();
#pragma unroll 2
    for (int kk = 0; kk < LM_KC / 4; ++kk) {
      const int k = 4 * kk + g;
      const int q = c * LM_KC + k;  // sample of the frame
      const float a = span[frame_off + q + 2 * (q / LM_HOP)];
      const float* brow = buf + k * LM_COLS_LDS + lr;
#pragma unroll
      for (int t = 0; t < LM_TILES; ++t) acc[t] = mma4(a, brow[16 * t], acc[t]);
    }
  }
  __syncthreads();  // every wave is done with the last table chunk
  // power spectrum -> buf as [frame][bin] (208 bins)
  constexpr int PB = 16 * LM_BIN_TILES;
#pragma unroll
  for (int t = 0; t < LM_BIN_TILES; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float re = acc[2 * t][r], im = acc[2 * t + 1][r];
      buf[(16 * wave + 4 * g + r) * LM_PB_LDS + 16 * t + lr] = re * re + im * im;
    }
  __syncthreads();

  // filterbank: mel[frame][m] = sum_bin power[frame][bin] * melw[bin][m]
  f32x4_t macc[LM_MELS / 16];
#pragma unroll
  for (int t = 0; t < LM_MELS / 16; ++t) macc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const float* prow = buf + (16 * wave + lr) * LM_PB_LDS;
#pragma unroll 4
  for (int kk = 0; kk < PB / 4; ++kk) {
    const int k = 4 * kk + g;
    const float a = prow[k];
    const float* mrow = melw + k * LM_MELS + lr;
#pragma unroll
    for (int t = 0; t < LM_MELS / 16; ++t) macc[t] = mma4(a, mrow[16 * t], macc[t]);
  }

  // log10 into feat[b][m][frame]; lane holds frames 16 wave + 4 g + r of mel 16 t + lr
  float lmax = -1e30f;
  const int fr = f0 + 16 * wave + 4 * g;
#pragma unroll
  for (int t = 0; t < LM_MELS / 16; ++t) {
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      v[r] = log10f(fmaxf(macc[t][r], 1e-10f));
      if (fr + r < nf) lmax = fmaxf(lmax, v[r]);
    }
    float* dst = feat + ((long)b * LM_MELS + 16 * t + lr) * T_max + fr;
    if (fr + 3 < nf && (T_max & 3) == 0) {
      *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (fr + r < nf) dst[r] = v[r];
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, o, 64));
  if (lane == 0 && lmax > -1e29f) atomicMax(mx + b, __float_as_uint(lmax + 16.0f));
}

// floor at the request's maximum - 8 and scale: (max(x, top - 8) + 4) / 4
__global__ void logmel_finish_kernel(float* __restrict__ feat, const int* __restrict__ lens,
                                     const unsigned* __restrict__ mx, int T_max) {
  const int b = blockIdx.y;
  const int nf = lens[b] / LM_HOP;
  const float floor_v = __uint_as_float(mx[b]) - 16.0f - 8.0f;
  const long n = (long)LM_MELS * nf;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
    const int m = (int)(i / nf), f = (int)(i - (long)m * nf);
    float* p = feat + ((long)b * LM_MELS + m) * T_max + f;
    *p = (fmaxf(*p, floor_v) + 4.0f) * 0.25f;
  }
}

}  // namespace

size_t logmel_table_floats() { return (size_t)LM_NFFT * LM_COLS + (size_t)16 * LM_BIN_TILES * LM_MELS; }

hipError_t launch_logmel_tables(float* tables, hipStream_t s) {
  hipLaunchKernelGGL(logmel_tables_kernel, dim3(256), dim3(256), 0, s, tables,
                     tables + (size_t)LM_NFFT * LM_COLS);
  return hipGetLastError();
}

hipError_t launch_logmel(const float* audio, long s_max, const int* lens_dev, int B, int max_frames,
                         const float* tables, float* feat, int T_max, unsigned* mx, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(logmel_init_kernel, dim3((B + 255) / 256), dim3(256), 0, s, mx, B);
  if (max_frames <= 0) return hipGetLastError();
  const dim3 grid((max_frames + LM_FRAMES - 1) / LM_FRAMES, B);
  hipLaunchKernelGGL(logmel_kernel, grid, dim3(LM_THREADS), 0, s, audio, s_max, lens_dev, tables,
                     tables + (size_t)LM_NFFT * LM_COLS, feat, T_max, mx);
  const dim3 grid2((unsigned)((LM_MELS * (long)max_frames + 255) / 256 < 4096 ? (LM_MELS * (long)max_frames + 255) / 256 : 4096), B);
  hipLaunchKernelGGL(logmel_finish_kernel, grid2, dim3(256), 0, s, feat, lens_dev, mx, T_max);
  return hipGetLastError();
}

}  // namespace aut
