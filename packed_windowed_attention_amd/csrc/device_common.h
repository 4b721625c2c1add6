// Device helpers shared by the gfx950 kernels of the AuT encoder.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;  // one 16-byte unit
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;

typedef __bf16 bf16_t;

// GELU, x * Phi(x) with Phi(x) = erfc(-x / sqrt 2) / 2 ('gelu' activation of
// AuTEncoderConfig: the erf form, not the tanh approximation).
//
// erfc(z), z >= 0, by the rational-exponential fit of Abramowitz & Stegun,
// Handbook of Mathematical Functions, formula 7.1.26:
//   erfc(z) = (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2) + eps,
//   t = 1 / (1 + p z), |eps| <= 1.5e-7,
// evaluated at z = |x| / sqrt 2 with the coefficients halved, which gives the
// upper tail Q = erfc(z) / 2 directly.  Then GELU(x) = max(x, 0) - |x| Q for
// either sign (x >= 0: x - x Q; x < 0: x Q).  Branch-free, one reciprocal and
// one exp2: 13 vector-ALU instructions.  Float32 emulation against the exact
// erf form: max abs error 3.3e-7 over [-12, 12].  Used where the result is
// stored as fp32.
__device__ __forceinline__ float gelu_f(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.23164188f, ax, 1.0f));  // p / sqrt 2
  float q = 0.5307027145f;         // a5 / 2
  q = fmaf(q, t, -0.7265760135f);  // a4 / 2
  q = fmaf(q, t, 0.7107068705f);   // a3 / 2
  q = fmaf(q, t, -0.142248368f);   // a2 / 2
  q = fmaf(q, t, 0.127414796f);    // a1 / 2
  q *= t;
  // exp(-x^2 / 2) = exp2(-x^2 log2(e) / 2)
  const float e = __builtin_amdgcn_exp2f((x * -0.72134752044448170368f) * x);
  return fmaf(-ax, q * e, __builtin_amdgcn_fmed3f(x, 0.0f, __builtin_inff()));
}

// GELU for results stored as bf16 or MX-fp8: accurate to a small fraction of
// their rounding step, for 8 issue slots instead of 13.  The upper tail
// Q(t) = Phi(-t) is taken as 2^P(t) with P a degree-5 polynomial fitted to
// log2 Q on [0, 5] (near-minimax by Lawson's reweighted least squares: at most
// 2.3e-4 off in log2 Q, 1.6e-4 relative in Q).  Past t = 5, where Q < 3e-7,
// P keeps falling (its value stays below -25 from t = 5.5 on and never turns
// upward: the t^5 term dominates before t^4 could), so |x| 2^P(|x|) is far
// below the rounding step there and needs no clamp.  Then GELU(x) =
// max(x, 0) - |x| Q(|x|) as above.  Float32 emulation against the exact erf
// form over [-16, 16]: max abs error 2.25e-5; at most 0.081 of half a bf16
// unit in the last place wherever |GELU| > 1e-3 (an e4m3 code's step is 32
// times coarser still).  Results stored as fp32 keep gelu_f.
__device__ __forceinline__ float gelu_bf16(float x) {
  const float t = fabsf(x);
  float p = fmaf(-2.6991881895810366e-4f, t, 5.29736140742898e-3f);
  p = fmaf(p, t, -4.6319395303726196e-2f);
  p = fmaf(p, t, -4.669073522090912e-1f);
  p = fmaf(p, t, -1.1477890014648438f);
  p = fmaf(p, t, -1.0002282857894897f);
  return fmaf(-t, __builtin_amdgcn_exp2f(p), __builtin_amdgcn_fmed3f(x, 0.0f, __builtin_inff()));
}

typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// Two fp32 -> two bf16 (round to nearest even) in one dword, low half first:
// one v_cvt_pk_bf16_f32.
__device__ __forceinline__ unsigned int pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(unsigned int, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ bf16_t to_bf16(float x) { return (bf16_t)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return to_bf16(x); }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return (float)x; }

// Elements of T in one 16-byte unit.
template <typename T> struct UnitElems { static constexpr int value = 16 / (int)sizeof(T); };

// ---------------------------------------------------------------------------
// 16x16 output tile, 32-deep k step, fp32 accumulate.
//
// Operand fragments: for a k step of 32, lane l (row or column l % 16, group
// g = l / 16) supplies 8 k-values.  The k index each of the 8 slots stands for
// may be any fixed function of (g, slot) as long as the A and B fragments use
// the same one, since the product sums over all 32.  Result: lane l holds
// C[4 g + r][l % 16], r = 0..3.
//
// bf16: one v_mfma_f32_16x16x32_bf16 (slots = the 8 packed bf16).
// fp32: eight v_mfma_f32_16x16x4_f32, instruction s taking slot s of every
//       lane, so that the four groups cover four distinct k per instruction.
// ---------------------------------------------------------------------------
struct FragBF16 { bf16x8_t v; };
struct FragF32 { float v[8]; };

template <typename T> struct FragOf;
template <> struct FragOf<bf16_t> { typedef FragBF16 type; };
template <> struct FragOf<float> { typedef FragF32 type; };

__device__ __forceinline__ void mma16_k32(f32x4_t& acc, const FragBF16& a, const FragBF16& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16_k32(f32x4_t& acc, const FragF32& a, const FragF32& b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], acc, 0, 0, 0);
}

// Fragment from 16-byte units: bf16 needs one unit, fp32 two consecutive ones.
__device__ __forceinline__ void frag_from_units(FragBF16& f, u32x4_t u0, u32x4_t) {
  f.v = __builtin_bit_cast(bf16x8_t, u0);
}
__device__ __forceinline__ void frag_from_units(FragF32& f, u32x4_t u0, u32x4_t u1) {
  f32x4_t a = __builtin_bit_cast(f32x4_t, u0), b = __builtin_bit_cast(f32x4_t, u1);
  f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
  f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
}

__device__ __forceinline__ u32x4_t zero_unit() { return u32x4_t{0u, 0u, 0u, 0u}; }

__device__ __forceinline__ u32x4_t ldg_unit(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// ------------------------------- MX-fp8 ------------------------------------
// OCP Microscaling MX-fp8: e4m3 elements (OCP 8-bit floating point E4M3,
// largest finite 448) in blocks of 32 consecutive values along a product's
// contraction axis, each block with one power-of-two scale stored as E8M0
// (scale = 2^(code - 127)).  The scale of a block is the smallest power of two
// s with max|x| / s <= 448, so no element saturates.
constexpr int MX_BLOCK = 32;

// Byte of the scale of row r, block kb (k = 32 kb .. 32 kb + 31) of an operand
// with K columns (K a multiple of 128): per 16-row group and 128-wide k step,
// 64 bytes in the lane order of one scaled matrix instruction (lane
// 16 (kb % 4) + r % 16).  Rows are padded to a multiple of 16.
__device__ __forceinline__ size_t mx_scale_index(int r, int kb, int K) {
  return ((size_t)(r >> 4) * (size_t)(K >> 7) + (size_t)(kb >> 2)) * 64 + (size_t)((kb & 3) * 16 + (r & 15));
}

// Exponent e of a block's scale 2^e: the smallest e with amax <= 448 * 2^e,
// within [-127, 127] (an all-zero block gives -127).  Exact, from the bits:
// amax = (1 + f) 2^E needs e = E - 8 when 1 + f <= 1.75, else E - 7.
__device__ __forceinline__ int mx_exponent(float amax) {
  const unsigned u = __builtin_bit_cast(unsigned, amax);
  const int E = (int)(u >> 23) - 127;
  const int e = E - 8 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : e;  // zero and tiny blocks
}

// Four fp32 -> four e4m3 codes (round to nearest even; |x| <= 448), first
// value in the lowest byte.
__device__ __forceinline__ unsigned int pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (unsigned int)w;
}

// x * 2^-e, exact
__device__ __forceinline__ float mx_scale_down(float x, int e) { return __builtin_amdgcn_ldexpf(x, -e); }

// The 32 fp8 bytes of a scaled matrix instruction's operand: two 16-byte units.
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
__device__ __forceinline__ i32x8_t units_to_i32x8(u32x4_t lo, u32x4_t hi) {
  return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}
