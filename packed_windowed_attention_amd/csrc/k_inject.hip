// Audio rows into the decoder's embedding sequence ("Audio Encoder Component",
// cubic.dev wiki, Data Flow and Integration: the encoder output goes into the
// text sequence at the <|audio_pad|> placeholder positions, not appended):
// dst[rows[j]] = audio[j] for every audio row j, converted to the sequence's
// type; every other row of dst is left as it is (the text embeddings).
// One wavefront per row, 16-byte loads, 16- (fp32) or 8-byte (bf16) stores.
#include "aut_internal.h"
#include "device_common.h"

namespace aut {

namespace {

constexpr int INJ_WAVES = 4;

template <typename T>
__device__ __forceinline__ void put4(T* p, float4 v);
template <>
__device__ __forceinline__ void put4<float>(float* p, float4 v) {
  *reinterpret_cast<float4*>(p) = v;
}
template <>
__device__ __forceinline__ void put4<bf16_t>(bf16_t* p, float4 v) {
  *reinterpret_cast<u32x2_t*>(p) = u32x2_t{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
}

template <typename T>
__global__ __launch_bounds__(64 * INJ_WAVES) void inject_kernel(const float* __restrict__ audio,
                                                               const int* __restrict__ rows,
                                                               long n, int dim, T* __restrict__ dst,
                                                               long dst_rows) {
  const long j = (long)blockIdx.x * INJ_WAVES + (threadIdx.x >> 6);
  if (j >= n) return;
  const long r = rows[j];
  if (r < 0 || r >= dst_rows) return;  // outside the sequence: skipped
  const int lane = threadIdx.x & 63;
  const float4* src = reinterpret_cast<const float4*>(audio + j * (long)dim);
  T* out = dst + r * (long)dim;
  for (int c = lane; c < dim / 4; c += 64) put4<T>(out + 4 * c, src[c]);
}

}  // namespace

hipError_t launch_inject(const float* audio, const int* rows, long n, int dim, void* dst,
                         long dst_rows, aut_dtype dt, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)((n + INJ_WAVES - 1) / INJ_WAVES));
  if (dt == AUT_BF16)
    hipLaunchKernelGGL(inject_kernel<bf16_t>, grid, dim3(64 * INJ_WAVES), 0, s, audio, rows, n, dim,
                       (bf16_t*)dst, dst_rows);
  else
    hipLaunchKernelGGL(inject_kernel<float>, grid, dim3(64 * INJ_WAVES), 0, s, audio, rows, n, dim,
                       (float*)dst, dst_rows);
  return hipGetLastError();
}

}  // namespace aut
