// Internal interfaces between the host layer (aut_host.cpp) and the kernel
// launchers (*.hip).  Not part of the public C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/aut.h"

namespace aut {

// Geometry derived from a configuration.
struct Geometry {
  int mel;          // H0 = num_mel_bins
  int cf;           // W0 = chunk frames = 2 * n_window
  int h1, w1;       // conv1 output grid
  int h2, w2;       // conv2 output grid
  int h3, w3;       // conv3 output grid; w3 = tokens per full chunk
  int C;            // conv channels
  int d, H, hd, F, out;
  int layers;
  int window_tokens;
  int chunks_per_window;
};

Geometry geometry(const aut_config& c);

// Whisper-style log-mel front end (16 kHz mono -> 128 bins, 100 frames/s).
constexpr int LM_RATE = 16000;
constexpr int LM_NFFT = 400;
constexpr int LM_HOP = 160;
constexpr int LM_MELS = 128;
constexpr int LM_BIN_TILES = 13;  // 16-bin tiles covering the 201 DFT bins
size_t logmel_table_floats();
hipError_t launch_logmel_tables(float* tables, hipStream_t s);
hipError_t launch_logmel(const float* audio, long s_max, const int* lens_dev, int B, int max_frames,
                         const float* tables, float* feat, int T_max, unsigned* mx, hipStream_t s);

// Audio rows into a decoder embedding sequence: dst[rows[j]] = audio[j].
hipError_t launch_inject(const float* audio, const int* rows, long n, int dim, void* dst,
                         long dst_rows, aut_dtype dt, hipStream_t s);

// The device scratch of aut_encode_noalloc: its size, and this device's
// address of it (looked up on the first call per device, then cached).
size_t scratch_bytes();
hipError_t scratch_ptr(void** ptr);

// Per-launch timing hooks (no-ops unless aut_profile_enable(1)).
void prof_begin(hipStream_t s);
void prof_end(hipStream_t s, aut_kernel_class cls, double flops, double bytes);

// ------------------------------- kernels ---------------------------------

// Weight packing.
enum PackMode { PACK_CAST = 0, PACK_CONV = 1, PACK_CONV_OUT = 2 };
hipError_t launch_pack(const float* src, void* dst, aut_dtype dt, int mode, int rows, int cols,
                       int C, int F, hipStream_t s);
hipError_t launch_pe_table(float* pe, int rows, int d, hipStream_t s);

// conv1 + GELU over `nb` chunks starting at chunk_first of the plan.
// AUT_FP8: MX-fp8 codes [pixel][cp] (channels past C zero) into a1 and their
// scales, row-major cp / 32 bytes per pixel, into a1_scales.
hipError_t launch_conv1(const float* feat, int T_max, const int* chunks, int chunk_first, int nb,
                        const float* w1, const float* b1, void* a1, aut_dtype dt,
                        const Geometry& g, hipStream_t s, uint8_t* a1_scales = nullptr,
                        int cp = 0);

// Generic MFMA GEMM: C[M, N] = A[M, K] * B[N, K]^T with an A-gather mode and
// an epilogue.
enum AMode { A_PLAIN = 0, A_CONV = 1, A_ROWMAP = 2 };
// EPI_GELU_MX: GELU, then MX-fp8 codes into `out` (ldo in bytes) and their
// scales into `out_scale` (mx_scale_index layout over M rows and N columns).
enum Epi { EPI_STORE = 0, EPI_STORE_GELU = 1, EPI_RESID = 2, EPI_PE = 3, EPI_STORE_F32 = 4,
           EPI_GELU_MX = 5 };

struct GemmArgs {
  const void* A; long lda;
  const void* B; long ldb;
  int M, N, K;
  // A_CONV: implicit-GEMM conv with 3x3 kernel, stride 2, pad 1.  Row m of A
  // is output pixel (chunk, oy, ox), decomposed x-major or y-major.
  int hin, win, hout, wout, cin, xmajor;
  // A_ROWMAP: row m of A is A + (rowmap[m] - rowmap_base) * lda.
  const int* rowmap; int rowmap_base; int tpc;
  // A_CONV / A_ROWMAP: bytes of the A buffer (every gathered offset is below;
  // must be < 2^31 for the bf16 kernel's 32-bit buffer offsets)
  size_t a_bytes;
  // epilogue
  const float* bias;   // [N] or null
  void* out; long ldo;
  const float* pe;     // EPI_PE: [tpc, N] position rows, indexed rowmap[m] % tpc
  // MX-fp8 products (launch_gemm_f8): scales of A (over M rows) and B (over N
  // rows) in the mx_scale_index layout; EPI_GELU_MX: the output's scales
  const uint8_t* a_scale;
  const uint8_t* b_scale;
  uint8_t* out_scale;
  // A_CONV / A_ROWMAP under fp8: A's scales are row-major, a_scale_ld bytes
  // per row (per input pixel for A_CONV, per gathered row for A_ROWMAP)
  int a_scale_ld;
  size_t a_scale_bytes;  // bytes of A's scale array (gathered modes)
  // EPI_GELU_MX: columns written (>= N; the ones past N as zero codes), and
  // the output's scale layout: 0 = mx_scale_index over n_store columns,
  // 1 = row-major, n_store / 32 bytes per row
  int n_store;
  int out_scale_rowmajor;
};
// bf16 runs the 256-row kernel (k_gemm256.hip), fp32 the 128 x 128 one
// (k_gemm128.hip).
hipError_t launch_gemm(const GemmArgs& a, int amode, int epi, aut_dtype dt, hipStream_t s);
hipError_t launch_gemm128(const GemmArgs& a, int amode, int epi, aut_dtype dt, hipStream_t s);
hipError_t launch_gemm256(const GemmArgs& a, int amode, int epi, hipStream_t s);

// MX-fp8 products: A [M, K] and B [N, K] as e4m3 codes (lda, ldb in bytes)
// with scales; K a multiple of 128.  A modes: A_PLAIN (scales in the
// mx_scale_index layout), A_CONV (cin a multiple of 128, so a k step stays in
// one tap) and A_ROWMAP (row-major scales).  Epilogues: A_PLAIN with
// EPI_STORE, EPI_STORE_GELU, EPI_RESID, EPI_STORE_F32, EPI_GELU_MX; A_CONV
// with EPI_GELU_MX; A_ROWMAP with EPI_PE.
hipError_t launch_gemm_f8(const GemmArgs& a, int amode, int epi, hipStream_t s);
// relative duration of an implicit-conv GEMM launch (M output pixels, N
// channels) under the tile choice the launchers make (bf16 or MX-fp8 kernel)
double gemm_conv_time_model(int M, int N, bool f8);

// conv-stem weights straight from their PyTorch layout to MX-fp8, channels
// padded to cp with zeros: mode PACK_CONV, [Co, Ci, 3, 3] -> [Co][tap * cp + c];
// PACK_CONV_OUT, [d, C * F] (c * F + f) -> [d][f * cp + c].
hipError_t launch_mx_quantize_gather(const float* src, int mode, int rows, int C, int cp, int F,
                                     uint8_t* codes, uint8_t* scales, hipStream_t s);

// fp32 rows [R, K] (row stride ldx) -> MX-fp8 codes [R, K] and scales
// (mx_scale_bytes(R, K) bytes, rows padded to 16 with scale code 0).
size_t mx_scale_bytes(long rows, int K);
hipError_t launch_mx_quantize(const float* x, long ldx, long R, int K, uint8_t* codes,
                              uint8_t* scales, hipStream_t s);

// LayerNorm rows of fp32 x [T, d] into the GEMM operand type; AUT_FP8: MX-fp8
// codes into y and their scales into y_scales.
hipError_t launch_layernorm(const float* x, const float* g, const float* b, void* y, int T, int d,
                            float eps, aut_dtype dt, hipStream_t s, uint8_t* y_scales = nullptr);

// Window attention: qkv [T, 3d] (q | k | v) -> o [T, d], d = 64 H.  AUT_FP8:
// bf16 qkv, o as MX-fp8 codes with scales in o_scales.  f32_out (AUT_BF16
// only): o in fp32, the values the bf16 and MX outputs round.  Items whose
// window is not within rows [0, T) or holds more than 128 rows do nothing.
hipError_t launch_attention(const void* qkv, void* o, const int* cu, const int* worder,
                            int n_windows, int H, int d, aut_dtype dt, hipStream_t s,
                            uint8_t* o_scales, int T, bool f32_out = false);

}  // namespace aut
