// bf16 MFMA GEMM for gfx950 with 256-row block tiles:
// C[M, N] = A[M, K] * B[N, K]^T (+ epilogue), fp32 accumulation.
//
// Block tile 256 x BN (BN = 160 or 128), 4 waves in a 2 x 2 grid, each wave
// 128 x BN/2; the accumulators (160 or 128 per lane) live in the accumulation
// registers, one wave per SIMD.  (A 256 x 256 tile needs all 256 accumulation
// registers and the compiler then spills; it is not offered.)
//
// Operands go from memory straight into LDS (buffer_load_dwordx4 ... lds), no
// registers in between, through a ring of three k-steps of 64 bf16 (128 bytes
// per tile row; 156 KiB for BN = 160); loads run two steps ahead of the matrix instructions and each
// step needs one barrier.  A buffer load whose offset lies past the end of its
// buffer returns zero, which gives the zero padding of tile tails (rows past M
// or N, k past K) and of the convolution's border taps for free.  Within a
// 128-byte row the eight 16-byte units are XOR-swizzled by row & 7, which the
// LDS conflict counters show to be conflict-free for the fragment loads (a
// 64-byte-row layout doubled the cycles of every fragment load).
//
// The weight fragment is the matrix instruction's first operand and the
// activation fragment its second, so each lane ends up with four consecutive
// output columns of one row: the epilogue stores 8 (bf16) or 16 (fp32) bytes
// per lane and reads bias, residual and position rows as float4.
//
// Tiles are ordered for the 8 XCDs (each with its own L2): workgroup b runs on
// XCD b % 8, so XCD x is given the contiguous tile range
// [x * per_xcd, (x + 1) * per_xcd), walked 8 M-tiles per N column, so the 32
// tiles an XCD runs at once share 8 A panels and 4 B panels.
//
// A-gather modes: plain; implicit 3x3 stride-2 pad-1 convolution over a
// channels-last activation, k = tap * C + c (openarchlab "1A", section 3:
// Conv2d(k=3, s=2, p=1)); row map (conv_out over the valid tokens).
// Epilogues: bias then store, GELU then store, residual add into fp32,
// position add, fp32 store.
#include "aut_internal.h"
#include "device_common.h"

namespace aut {

namespace {

constexpr int BM = 256;
constexpr int NTHR = 256;
constexpr int KU = 8;       // 16-byte units per row per k step
constexpr int BK = 64;      // bf16 per row per k step
constexpr int GROUP_M = 8;
constexpr unsigned OOB = 0x80000000u;  // an offset past every buffer here: loads zero

// Record count of a tile's A descriptor (based at the tile's first row): the
// rest of the matrix, capped at 2^31 bytes.  A tile reads at most BM rows past
// its base, so the cap never cuts a real access, keeps the count within 32
// bits for any number of rows, and keeps every offset >= OOB out of range.
__device__ __forceinline__ unsigned tile_records(size_t bytes) {
  return bytes < (size_t)OOB ? (unsigned)bytes : OOB;
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int unit, int row) { return unit ^ (row & 7); }

// LDS destination of a direct load, as a wave-uniform address with its origin
// hidden from the compiler: ordering against the fragment reads is kept by the
// explicit vmcnt waits and barriers below, and the compiler then does not add
// a wait for every load in flight before each fragment read.
// The low 32 bits of a flat address inside the LDS aperture are the LDS offset.
__device__ __forceinline__ lds_void* dma_dst(const u32x4_t* p) {
  const unsigned a = (unsigned)(size_t)p;
  return (lds_void*)(size_t)__builtin_amdgcn_readfirstlane(a);
}

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding:
// vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] in bits 15:14).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// a compile-time part index for the phase helpers of the MX-fp8 kernel
template <int P> struct PartC { static constexpr int value = P; };

// s_waitcnt lgkmcnt(0) alone, then a workgroup barrier: orders the LDS traffic
// of the epilogue without waiting for the global stores in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Implicit 3x3 stride-2 pad-1 convolution over a channels-last activation
// (openarchlab "1A", section 3: Conv2d(k=3, s=2, p=1)), k = tap * cin + c.
// Per load row: the byte offset of its window's tap-(0, 0) pixel, channel 0
// (negative when that corner lies in the padding), and a 9-bit mask of the
// taps that fall inside the image (no bit for rows past M).  Per lane: the tap
// and channel of its 16-byte unit at the current k step, advanced one step per
// issue, so a load's offset is a bit test and an add.  Taps past the ninth
// (the k tail) have no bit and load zero.  Kernels declare it full size in
// every A mode: with a one-row instance, the constant out-of-range indices in
// the mode's dead branches made the host compilation pass drop the kernels'
// launch stubs without a diagnostic.
template <int NL, int ES>
struct ConvGather {
  int base[NL];
  unsigned valid[NL];
  int tap, ci;
  __host__ __device__ __forceinline__ void row(const GemmArgs& p, int j, int m) {
    base[j] = 0;
    valid[j] = 0u;
    if (m >= p.M) return;
    const int hw = p.hout * p.wout;
    const int chunk = m / hw;
    const int rem = m - chunk * hw;
    int oy, ox;
    if (p.xmajor) {
      ox = rem / p.hout;
      oy = rem - ox * p.hout;
    } else {
      oy = rem / p.wout;
      ox = rem - oy * p.wout;
    }
    base[j] = (chunk * p.hin * p.win + (2 * oy - 1) * p.win + (2 * ox - 1)) * p.cin * ES;
    unsigned v = 0u;
#pragma unroll
    for (int kh = 0; kh < 3; ++kh)
#pragma unroll
      for (int kw = 0; kw < 3; ++kw) {
        const int iy = 2 * oy + kh - 1, ix = 2 * ox + kw - 1;
        if (iy >= 0 && iy < p.hin && ix >= 0 && ix < p.win) v |= 1u << (3 * kh + kw);
      }
    valid[j] = v;
  }
  __host__ __device__ __forceinline__ void start(int k0, int cin) {
    tap = k0 / cin;
    ci = k0 - tap * cin;
  }
  __host__ __device__ __forceinline__ void advance(int bk, int cin) {
    ci += bk;
    while (ci >= cin) {
      ci -= cin;
      ++tap;
    }
  }
  __host__ __device__ __forceinline__ int tap_offset(const GemmArgs& p) const {
    const int kh = (tap * 11) >> 5;  // tap / 3 for the taps that matter (0..10)
    const int kw = tap - 3 * kh;
    return ((kh * p.win + kw) * p.cin + ci) * ES;
  }
  __host__ __device__ __forceinline__ unsigned offset(int j, int toff) const {
    return ((valid[j] >> tap) & 1u) ? (unsigned)(base[j] + toff) : OOB;
  }
};

// Epilogue through LDS.  A lane's accumulators cover 4 consecutive columns of
// scattered rows, so storing them straight to memory writes 8- or 16-byte
// pieces of many cache lines, which the memory system then writes back as
// partial lines.  Instead the tile goes through LDS (the operand stages are
// free once the k loop is over) in passes of PR rows: the waves write their
// share of the pass (bias and GELU applied), then every thread copies 16-byte
// chunks of whole rows to memory, consecutive threads on consecutive chunks,
// applying the residual or position add on the way.  The staged rows are
// spread over the four largest stage arrays, RB rows each, with a row pitch
// 16 bytes over the row's size so that the 16 rows a wave writes at once fall
// in distinct banks.  Needs N a multiple of the chunk's element count
// (checked on the host).
template <int BN, int WN, int NT, int EPI>
__device__ __forceinline__ void staged_epilogue(const GemmArgs& p, int m0, int n0, int wm, int wn,
                                                int tid, f32x4_t (&acc)[WN / 16][8],
                                                u32x4_t* lds0, u32x4_t* lds1, u32x4_t* lds2,
                                                u32x4_t* lds3) {
  constexpr int NTW = WN / 16;
  constexpr bool MX = EPI == EPI_GELU_MX;
  constexpr bool F32 = EPI == EPI_RESID || EPI == EPI_PE || EPI == EPI_STORE_F32 || MX;
  constexpr int ES = F32 ? 4 : 2;          // output element size
  constexpr int PR = F32 ? 64 : 128;       // rows per pass
  constexpr int RB = PR / 4;               // rows per LDS buffer
  constexpr int PITCH = BN * ES + 16;      // staged row pitch, bytes
  constexpr int CPR = BN * ES / 16;        // 16-byte chunks per row
  constexpr int EPC = 16 / ES;             // elements per chunk
  constexpr int PER_THREAD = PR * CPR / NT;
  static_assert(PR * CPR % NT == 0, "whole chunks per thread");
  // A pass takes HALF rows from each half of the tile (wm = 0: rows 0..127,
  // wm = 1: 128..255), so every wave stages some rows in every pass and
  // frees those accumulators early.
  constexpr int HALF = PR / 2;
  constexpr int IPP = HALF / 16;  // 16-row blocks per wave per pass
  static_assert(HALF % 16 == 0 && RB % 16 == 0, "whole 16-row blocks per buffer");
  const int M = p.M, N = p.N;
  const int lane = tid & 63, lrow = lane & 15, g = lane >> 4;
  float4 bq[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int n = n0 + wn * WN + 16 * j + 4 * g;
    bq[j] = (p.bias && n < N) ? *reinterpret_cast<const float4*>(p.bias + n)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // Have the bias in registers before any store: vector memory operations
  // complete in issue order, so a bias load the compiler sinks into a later
  // pass would wait for every store issued before it.
#pragma unroll
  for (int j = 0; j < NTW; ++j) asm volatile("" ::"v"(bq[j].x), "v"(bq[j].y), "v"(bq[j].z), "v"(bq[j].w));
#pragma unroll
  for (int pass = 0; pass < 256 / PR; ++pass) {
    lds_barrier();  // the k loop, or the previous pass's copy-out, is done with LDS
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i / IPP != pass) continue;  // 16-row blocks i of this pass (compile time)
      // staged row of the block's first row: the wm = 0 half of the pass, then wm = 1
      const int lr0 = wm * HALF + 16 * (i - pass * IPP);
      const int bsel = lr0 / RB;
      char* base = (char*)(bsel == 0 ? lds0 : bsel == 1 ? lds1 : bsel == 2 ? lds2 : lds3) +
                   (lr0 % RB + lrow) * PITCH;
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        f32x4_t av = acc[j][i];
        asm volatile("" : "+v"(av));  // copy out of the accumulators one tile at a time
        float v[4] = {av[0] + bq[j].x, av[1] + bq[j].y, av[2] + bq[j].z, av[3] + bq[j].w};
        if (EPI == EPI_STORE_GELU || MX) {
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = F32 && !MX ? gelu_f(v[r]) : gelu_bf16(v[r]);
        }
        const int col = wn * WN + 16 * j + 4 * g;
        if (F32) {
          *reinterpret_cast<f32x4_t*>(base + col * 4) = f32x4_t{v[0], v[1], v[2], v[3]};
        } else {
          *reinterpret_cast<u32x2_t*>(base + col * 2) =
              u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
      }
    }
    lds_barrier();
    if constexpr (MX) {
      // a thread per 32-value block of a staged row: its maximum, the scale
      // exponent, 32 codes in two 16-byte stores and the scale byte
      constexpr int BPR = BN / MX_BLOCK;
      const int ncols = p.n_store > N ? p.n_store : N;   // columns past N: zero codes
#pragma unroll
      for (int q = tid; q < PR * BPR; q += NT) {
        const int r = q / BPR;
        const int cb = q - r * BPR;
        const int m = m0 + (r / HALF) * 128 + pass * HALF + r % HALF;
        const int n = n0 + cb * MX_BLOCK;
        const int b = r / RB;
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
            (const char*)(b == 0 ? lds0 : b == 1 ? lds1 : b == 2 ? lds2 : lds3) + (r - b * RB) * PITCH +
            cb * MX_BLOCK * 4);
        f32x4_t f[8];
        float amax = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          f[k] = __builtin_bit_cast(f32x4_t, src[k]);
          amax = fmaxf(amax, fmaxf(fmaxf(fabsf(f[k][0]), fabsf(f[k][1])), fmaxf(fabsf(f[k][2]), fabsf(f[k][3]))));
        }
        if (m < M && n < ncols) {
          const int e = mx_exponent(amax);
          unsigned int w[8];
#pragma unroll
          for (int k = 0; k < 8; ++k)
            w[k] = pack_fp8x4(mx_scale_down(f[k][0], e), mx_scale_down(f[k][1], e),
                              mx_scale_down(f[k][2], e), mx_scale_down(f[k][3], e));
          u32x4_t* dst = reinterpret_cast<u32x4_t*>((uint8_t*)p.out + (size_t)m * p.ldo + n);
          dst[0] = u32x4_t{w[0], w[1], w[2], w[3]};
          dst[1] = u32x4_t{w[4], w[5], w[6], w[7]};
          p.out_scale[p.out_scale_rowmajor ? (size_t)m * (ncols / MX_BLOCK) + n / MX_BLOCK
                                           : mx_scale_index(m, n / MX_BLOCK, ncols)] = (uint8_t)(e + 127);
        }
      }
      continue;
    }
    // Copy-out in batches: every load of a batch (staged rows, residual or
    // position rows) is issued before any of its stores, so a batch waits for
    // the earlier stores once rather than once per chunk.
    constexpr int SB = PER_THREAD % 2 == 0 ? PER_THREAD / 2 : PER_THREAD;
#pragma unroll
    for (int s0 = 0; s0 < PER_THREAD; s0 += SB) {
      u32x4_t d[SB];
      float4 add[SB];
      size_t off[SB];
      bool ok[SB];
#pragma unroll
      for (int t = 0; t < SB; ++t) {
        const int q = tid + NT * (s0 + t);
        const int r = q / CPR;
        const int c = q - r * CPR;
        const int m = m0 + (r / HALF) * 128 + pass * HALF + r % HALF;
        const int n = n0 + c * EPC;
        ok[t] = m < M && n < N;
        const int b = r / RB;
        const char* src = (const char*)(b == 0 ? lds0 : b == 1 ? lds1 : b == 2 ? lds2 : lds3) +
                          (r - b * RB) * PITCH + c * 16;
        d[t] = *reinterpret_cast<const u32x4_t*>(src);
        off[t] = (size_t)m * p.ldo + n;
        add[t] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (ok[t]) {
          if (EPI == EPI_RESID) {
            add[t] = *reinterpret_cast<const float4*>((const float*)p.out + off[t]);
          } else if (EPI == EPI_PE) {
            const int jpos = p.rowmap[m] % p.tpc;
            add[t] = *reinterpret_cast<const float4*>(p.pe + (size_t)jpos * N + n);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < SB; ++t) {
        if (!ok[t]) continue;
        if (!F32) {
          *reinterpret_cast<u32x4_t*>((bf16_t*)p.out + off[t]) = d[t];
        } else {
          // (bit-cast the whole vector: a bit cast of one vector element reads element 0)
          const f32x4_t f = __builtin_bit_cast(f32x4_t, d[t]);
          *reinterpret_cast<float4*>((float*)p.out + off[t]) =
              make_float4(f[0] + add[t].x, f[1] + add[t].y, f[2] + add[t].z, f[3] + add[t].w);
        }
      }
    }
  }
}

// Epilogue of a 288-row tile (two groups of nine 16-row blocks): passes of 96
// rows, three blocks from each group, staged in six 16-row slots (slots 0-1 in
// lds0, 2-3 in lds1, 4 in lds2, 5 in lds3: a 32-row fp32 slot pair needs
// 33 KB, a single slot 17 KB), then copied out as in staged_epilogue.
template <int BN, int WN, int NT, int EPI>
__device__ __forceinline__ void staged_epilogue_288(const GemmArgs& p, int m0, int n0, int wm, int wn,
                                                    int tid, f32x4_t (&acc)[WN / 16][9],
                                                    u32x4_t* lds0, u32x4_t* lds1, u32x4_t* lds2,
                                                    u32x4_t* lds3) {
  constexpr int NTW = WN / 16;
  static_assert(EPI == EPI_STORE || EPI == EPI_STORE_GELU || EPI == EPI_RESID || EPI == EPI_STORE_F32,
                "288-row tiles: plain epilogues only");
  constexpr bool F32 = EPI == EPI_RESID || EPI == EPI_STORE_F32;
  constexpr int ES = F32 ? 4 : 2;
  constexpr int RW = 144;                  // rows per group
  constexpr int PR = 96;                   // rows per pass
  constexpr int PITCH = BN * ES + 16;
  constexpr int CPR = BN * ES / 16;
  constexpr int EPC = 16 / ES;
  constexpr int PER_THREAD = PR * CPR / NT;
  static_assert(PR * CPR % NT == 0, "whole chunks per thread");
  static_assert(32 * PITCH <= 256 * KU * 16 * 9 / 8 && 16 * PITCH <= BN * KU * 16, "slots fit the stages");
  const int M = p.M, N = p.N;
  const int lane = tid & 63, lrow = lane & 15, g = lane >> 4;
  auto slot_base = [&](int slot) __attribute__((always_inline)) -> char* {
    return slot < 2 ? (char*)lds0 + slot * 16 * PITCH
         : slot < 4 ? (char*)lds1 + (slot - 2) * 16 * PITCH
         : slot == 4 ? (char*)lds2 : (char*)lds3;
  };
  float4 bq[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int n = n0 + wn * WN + 16 * j + 4 * g;
    bq[j] = (p.bias && n < N) ? *reinterpret_cast<const float4*>(p.bias + n)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // bias in registers before any store (memory operations complete in issue order)
#pragma unroll
  for (int j = 0; j < NTW; ++j) asm volatile("" ::"v"(bq[j].x), "v"(bq[j].y), "v"(bq[j].z), "v"(bq[j].w));
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    lds_barrier();
#pragma unroll
    for (int i = 3 * pass; i < 3 * pass + 3; ++i) {
      char* base = slot_base(wm * 3 + (i - 3 * pass)) + lrow * PITCH;
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        f32x4_t av = acc[j][i];
        asm volatile("" : "+v"(av));
        float v[4] = {av[0] + bq[j].x, av[1] + bq[j].y, av[2] + bq[j].z, av[3] + bq[j].w};
        if (EPI == EPI_STORE_GELU) {
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = gelu_bf16(v[r]);
        }
        const int col = wn * WN + 16 * j + 4 * g;
        if (F32) {
          *reinterpret_cast<f32x4_t*>(base + col * 4) = f32x4_t{v[0], v[1], v[2], v[3]};
        } else {
          *reinterpret_cast<u32x2_t*>(base + col * 2) =
              u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
      }
    }
    lds_barrier();
    constexpr int SB = PER_THREAD % 2 == 0 ? PER_THREAD / 2 : PER_THREAD;
#pragma unroll
    for (int s0 = 0; s0 < PER_THREAD; s0 += SB) {
      u32x4_t d[SB];
      float4 add[SB];
      size_t off[SB];
      bool ok[SB];
#pragma unroll
      for (int t = 0; t < SB; ++t) {
        const int q = tid + NT * (s0 + t);
        const int r = q / CPR;
        const int c = q - r * CPR;
        const int slot = r >> 4;
        const int m = m0 + (slot / 3) * RW + pass * 48 + (slot % 3) * 16 + (r & 15);
        const int n = n0 + c * EPC;
        ok[t] = m < M && n < N;
        d[t] = *reinterpret_cast<const u32x4_t*>(slot_base(slot) + (r & 15) * PITCH + c * 16);
        off[t] = (size_t)m * p.ldo + n;
        add[t] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (EPI == EPI_RESID && ok[t]) add[t] = *reinterpret_cast<const float4*>((const float*)p.out + off[t]);
      }
#pragma unroll
      for (int t = 0; t < SB; ++t) {
        if (!ok[t]) continue;
        if (!F32) {
          *reinterpret_cast<u32x4_t*>((bf16_t*)p.out + off[t]) = d[t];
        } else {
          const f32x4_t f = __builtin_bit_cast(f32x4_t, d[t]);
          *reinterpret_cast<float4*>((float*)p.out + off[t]) =
              make_float4(f[0] + add[t].x, f[1] + add[t].y, f[2] + add[t].z, f[3] + add[t].w);
        }
      }
    }
  }
}

template <int BN> struct Stages { static constexpr int value = BN > 160 ? 2 : 3; };

template <int BN, int AMODE, int EPI>
__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm256_kernel(GemmArgs p, int nM, int nN, int per_xcd) {
  constexpr int STAGES = Stages<BN>::value;
  constexpr int WN = BN / 2;                 // columns per wave
  constexpr int NTW = WN / 16;               // 16-column tiles per wave
  constexpr int A_UNITS = BM * KU;           // 2048 units per stage
  constexpr int B_UNITS = BN * KU;
  constexpr int A_LOADS = A_UNITS / NTHR;    // 8 loads per thread per step
  constexpr int B_LOADS = (B_UNITS + NTHR - 1) / NTHR;
  // loads every wave issues per step (a wave may issue one more B load; the
  // waits below count only the guaranteed ones, which waits a little longer
  // on those waves and never too little)
  constexpr int LOADS = A_LOADS + B_UNITS / NTHR;
  // one LDS object per stage: the compiler gives each its own alias scope, so
  // waiting for one stage's direct loads does not wait for the others
  __shared__ u32x4_t As0[A_UNITS], As1[A_UNITS], As2[STAGES > 2 ? A_UNITS : 1];
  __shared__ u32x4_t Bs0[B_UNITS], Bs1[B_UNITS], Bs2[STAGES > 2 ? B_UNITS : 1];

  const int tile = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (tile >= nM * nN) return;
  const int per_group = GROUP_M * nN;
  const int group = tile / per_group;
  const int first_m = group * GROUP_M;
  const int gsize = min(nM - first_m, GROUP_M);
  const int in_g = tile - group * per_group;
  const int m0 = (first_m + in_g % gsize) * BM;
  const int n0 = (in_g / gsize) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int M = p.M, N = p.N, K = p.K;

  // ---- per-lane source of each direct load -------------------------------
  // Load j of this wave fills LDS units [(j * 4 + wave) * 64, +64) of the
  // stage, i.e. the 8 rows (j * 4 + wave) * 8 + 0..7; LDS unit q holds row
  // q / 8, logical unit swz(q % 8, row).  So lane l always loads row
  // (j * 4 + wave) * 8 + l / 8 and logical unit (l % 8) ^ (l / 8): the unit is
  // the same for every load of a lane and the row advances by 32 per load.
  const int lrow8 = lane >> 3;
  const int lunit = (lane & 7) ^ lrow8;
  const char* a_base;
  unsigned a_bytes;
  if (AMODE == A_PLAIN) {
    a_base = (const char*)p.A + (size_t)m0 * p.lda * 2;
    a_bytes = tile_records((size_t)(M - m0) * p.lda * 2);
  } else {
    a_base = (const char*)p.A;
    a_bytes = (unsigned)p.a_bytes;
  }
  // A_PLAIN: offset of load j = a_off0 + j * a_step + 2 k, k = k0 + 8 * lunit.
  // Rows past M give offsets past a_bytes and load zero.
  const unsigned a_step = (unsigned)(32 * p.lda * 2);
  const unsigned a_off0 = (unsigned)((wave * 8 + lrow8) * p.lda * 2);
  // A_ROWMAP: per-load row offsets; A_CONV: per-load window corners and taps
  unsigned a_rowoff[A_LOADS];
  ConvGather<A_LOADS, 2> cg;  // (full size in every mode: see ConvGather)
  if (AMODE != A_PLAIN) {
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) {
      const int m = m0 + (j * 4 + wave) * 8 + lrow8;
      if (AMODE == A_ROWMAP) {
        a_rowoff[j] = m < M ? (unsigned)((size_t)(p.rowmap[m] - p.rowmap_base) * p.lda * 2) : OOB;
      } else {
        cg.row(p, j, m);
      }
    }
    if (AMODE == A_CONV) cg.start(lunit * 8, p.cin);
  }
  // B: offset of load j = b_off0 + j * b_step + 2 k; rows past N load zero.
  const char* b_base = (const char*)p.B + (size_t)n0 * p.ldb * 2;
  const unsigned b_bytes = (unsigned)((size_t)(N - n0) * p.ldb * 2);
  const unsigned b_step = (unsigned)(32 * p.ldb * 2);
  const unsigned b_off0 = (unsigned)((wave * 8 + lrow8) * p.ldb * 2);
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a_base, (short)0, (int)a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t b_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)b_base, (short)0, (int)b_bytes, 0x00020000);

  auto issue = [&](int kt, u32x4_t* As_s, u32x4_t* Bs_s) {
    const int k = kt * BK + lunit * 8;
    // k past K: an offset that is past every buffer
    const unsigned koff = k < K ? (unsigned)(2 * k) : OOB;
    if (AMODE == A_CONV) {
      const int toff = cg.tap_offset(p);
#pragma unroll
      for (int j = 0; j < A_LOADS; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, dma_dst(&As_s[(j * 4 + wave) * 64]), 16,
                                                 cg.offset(j, toff), 0, 0, 0);
      cg.advance(BK, p.cin);  // steps are issued in increasing order
    } else {
#pragma unroll
      for (int j = 0; j < A_LOADS; ++j) {
        const unsigned off = AMODE == A_PLAIN ? a_off0 + j * a_step + koff
                                              : (a_rowoff[j] == OOB ? OOB : a_rowoff[j] + koff);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, dma_dst(&As_s[(j * 4 + wave) * 64]), 16,
                                                 off, 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) {
      if ((j * 4 + wave) * 64 < B_UNITS) {  // uniform per wave
        __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, dma_dst(&Bs_s[(j * 4 + wave) * 64]), 16,
                                                 b_off0 + j * b_step + koff, 0, 0, 0);
      }
    }
  };

  f32x4_t acc[NTW][8];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[j][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + BK - 1) / BK;
  const int lrow = lane & 15;
  const int g = lane >> 4;
  // one k step from a given stage: wait for this thread's loads of step kt
  // (the steps issued after it, at most STAGES - 2, may stay in flight),
  // barrier so that every wave's loads have landed and step kt - 1 is
  // consumed, refill the stage step kt - 1 used with step kt + STAGES - 1,
  // then the matrix instructions of the two 32-deep halves of the step
  auto step = [&](int kt, const u32x4_t* As_s, const u32x4_t* Bs_s, u32x4_t* As_n, u32x4_t* Bs_n) {
    const int after = min(nk - 1 - kt, STAGES - 2);
    if (after >= 1) wait_vmcnt<LOADS>();
    else wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1, As_n, Bs_n);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      // fragments: all of B and the first two of A up front, then each further
      // A fragment is read while the matrix instructions of an earlier one run
      const int u = 4 * s + g;
      FragBF16 xa[8], wb[NTW];
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int r = wn * WN + 16 * j + lrow;
        frag_from_units(wb[j], Bs_s[r * KU + swz(u, r)], zero_unit());
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = wm * 128 + 16 * i + lrow;
        frag_from_units(xa[i], As_s[r * KU + swz(u, r)], zero_unit());
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) mma16_k32(acc[j][i], wb[j], xa[i]);
      __builtin_amdgcn_sched_group_barrier(0x100, NTW + 2, 0);  // DS reads
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, NTW, 0);     // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);       // DS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * NTW, 0);
      __builtin_amdgcn_sched_barrier(0);  // keep the halves apart: fewer live fragments
    }
  };

  static_assert(STAGES == 2 || STAGES == 3, "two or three LDS stages");
  if (STAGES == 2) {
    issue(0, As0, Bs0);
    for (int kt = 0; kt < nk; kt += 2) {
      step(kt, As0, Bs0, As1, Bs1);
      if (kt + 1 < nk) step(kt + 1, As1, Bs1, As0, Bs0);
    }
  } else {
    issue(0, As0, Bs0);
    if (1 < nk) issue(1, As1, Bs1);
    for (int kt = 0; kt < nk; kt += 3) {
      step(kt, As0, Bs0, As2, Bs2);
      if (kt + 1 < nk) step(kt + 1, As1, Bs1, As0, Bs0);
      if (kt + 2 < nk) step(kt + 2, As2, Bs2, As1, Bs1);
    }
  }
  wait_vmcnt<0>();

  staged_epilogue<BN, WN, NTHR, EPI>(p, m0, n0, wm, wn, tid, acc, As0, As1, Bs0, Bs1);
}

// Eight-wave variant for wide column tiles (BN = 256 or 320): 8 waves (2 per
// SIMD) in a 2 x 4 grid, each wave 128 x BN/4 (128 or 160 accumulators), two
// LDS stages of 64 or 72 KiB.  A 288 x 256 form (each wave 144 x 64, 144
// accumulators, stages of 68 KiB) fits the 256 CUs' rounds better for some
// row counts (14 673 rows: 51 tiles of 288 against 58 of 256).  Fewer operand
// bytes per flop than the four-wave kernel (a 256 x 320 tile needs 7.0 bytes
// per k step per 1000 flops against 10.2 for 256 x 160).  With both waves of a
// SIMD reading, loading and multiplying in step, the matrix cores were busy
// about half the cycles; the ping-pong schedule below offsets the two rows of
// waves.
template <int BN, int AMODE, int EPI, int BMT = BM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm8w_kernel(GemmArgs p, int nM, int nN, int per_xcd) {
  static_assert(BMT == BM || (BMT == 288 && AMODE == A_PLAIN && BN == 256),
                "288-row tiles: plain A operand, 256 columns");
  constexpr int NT8 = 512;
  constexpr int WN = BN / 4;                 // columns per wave
  constexpr int NTW = WN / 16;               // 16-column tiles per wave
  constexpr int RW = BMT / 2;                // rows per wave (128 or 144)
  constexpr int MB = RW / 16;                // 16-row blocks per wave (8 or 9)
  constexpr int A_UNITS = BMT * KU;          // 2048 or 2304 units per stage
  constexpr int B_UNITS = BN * KU;
  constexpr int A_LOADS = (A_UNITS + NT8 - 1) / NT8;  // 4 (or 5 on half the waves)
  // the gathered modes (256-row tiles only) keep their per-load tables at a
  // fixed size: tables sized by the row count made the host compilation pass
  // drop the kernels' launch stubs without a diagnostic
  constexpr int G_LOADS = BM * KU / NT8;
  constexpr int B_LOADS = B_UNITS / NT8;     // 4 or 5
  static_assert(B_UNITS % NT8 == 0, "whole B loads per thread");
  __shared__ u32x4_t As0[A_UNITS], As1[A_UNITS];
  __shared__ u32x4_t Bs0[B_UNITS], Bs1[B_UNITS];

  const int tile = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (tile >= nM * nN) return;
  const int per_group = GROUP_M * nN;
  const int group = tile / per_group;
  const int first_m = group * GROUP_M;
  const int gsize = min(nM - first_m, GROUP_M);
  const int in_g = tile - group * per_group;
  const int m0 = (first_m + in_g % gsize) * BMT;
  const int n0 = (in_g / gsize) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7
  const int wm = wave >> 2, wn = wave & 3;
  const int M = p.M, N = p.N, K = p.K;

  // load j of this wave fills LDS units [(j * 8 + wave) * 64, +64): rows
  // (j * 8 + wave) * 8 + 0..7, unit (l % 8) ^ (l / 8) for lane l
  const int lrow8 = lane >> 3;
  const int lunit = (lane & 7) ^ lrow8;
  const char* a_base;
  unsigned a_bytes;
  if (AMODE == A_PLAIN) {
    a_base = (const char*)p.A + (size_t)m0 * p.lda * 2;
    a_bytes = tile_records((size_t)(M - m0) * p.lda * 2);
  } else {
    a_base = (const char*)p.A;
    a_bytes = (unsigned)p.a_bytes;
  }
  const unsigned a_step = (unsigned)(64 * p.lda * 2);
  const unsigned a_off0 = (unsigned)((wave * 8 + lrow8) * p.lda * 2);
  unsigned a_rowoff[G_LOADS];
  ConvGather<G_LOADS, 2> cg;  // (full size in every mode: see ConvGather)
  if (AMODE != A_PLAIN) {
#pragma unroll
    for (int j = 0; j < G_LOADS; ++j) {
      const int m = m0 + (j * 8 + wave) * 8 + lrow8;
      if (AMODE == A_ROWMAP) {
        a_rowoff[j] = m < M ? (unsigned)((size_t)(p.rowmap[m] - p.rowmap_base) * p.lda * 2) : OOB;
      } else {
        cg.row(p, j, m);
      }
    }
    if (AMODE == A_CONV) cg.start(lunit * 8, p.cin);
  }
  const char* b_base = (const char*)p.B + (size_t)n0 * p.ldb * 2;
  const unsigned b_bytes = (unsigned)((size_t)(N - n0) * p.ldb * 2);
  const unsigned b_step = (unsigned)(64 * p.ldb * 2);
  const unsigned b_off0 = (unsigned)((wave * 8 + lrow8) * p.ldb * 2);
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a_base, (short)0, (int)a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t b_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)b_base, (short)0, (int)b_bytes, 0x00020000);

  auto issue = [&](int kt, u32x4_t* As_s, u32x4_t* Bs_s) __attribute__((always_inline)) {
    const int k = kt * BK + lunit * 8;
    const unsigned koff = k < K ? (unsigned)(2 * k) : OOB;
    if (AMODE == A_CONV) {
      const int toff = cg.tap_offset(p);
#pragma unroll
      for (int j = 0; j < G_LOADS; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, dma_dst(&As_s[(j * 8 + wave) * 64]), 16,
                                                 cg.offset(j, toff), 0, 0, 0);
      cg.advance(BK, p.cin);  // steps are issued in increasing order
    } else if (AMODE == A_PLAIN) {
#pragma unroll
      for (int j = 0; j < A_LOADS; ++j) {
        if (A_UNITS % NT8 != 0 && (j * 8 + wave) * 64 >= A_UNITS) continue;  // uniform per wave
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, dma_dst(&As_s[(j * 8 + wave) * 64]), 16,
                                                 a_off0 + j * a_step + koff, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < G_LOADS; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, dma_dst(&As_s[(j * 8 + wave) * 64]), 16,
                                                 a_rowoff[j] == OOB ? OOB : a_rowoff[j] + koff, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, dma_dst(&Bs_s[(j * 8 + wave) * 64]), 16,
                                               b_off0 + j * b_step + koff, 0, 0, 0);
  };

  f32x4_t acc[NTW][MB];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[j][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + BK - 1) / BK;
  const int lrow = lane & 15;
  const int g = lane >> 4;
  // Ping-pong schedule.  The two rows of waves, G0 (wm = 0) and G1 (wm = 1),
  // one wave of each per SIMD, run one phase apart.  A phase is either the
  // 40 matrix instructions of one 32-deep half step or the fragment reads of
  // the next half step (plus this wave's share of a step's loads), and every
  // phase ends at a barrier.  So while one group's waves issue matrix
  // instructions, at raised priority, the other group's read LDS and issue
  // the loads: a SIMD's two waves no longer compete for the same issue slots
  // at the same moments.  Stage kt % 2 serves step kt; the loads of step
  // kt + 1 fill the other stage, G1's share in phase 0 of step kt and G0's in
  // phase 3 of step kt - 1, after every wave has finished reading step kt - 1
  // there (the readers wait for their reads before the barrier that precedes
  // a refill).  Each output still sums its k steps in increasing order.
  FragBF16 xa[MB], wb[NTW];
  auto rd = [&](const u32x4_t* As_s, const u32x4_t* Bs_s, int h) __attribute__((always_inline)) {
    const int u = 4 * h + g;
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int r = wn * WN + 16 * j + lrow;
      frag_from_units(wb[j], Bs_s[r * KU + swz(u, r)], zero_unit());
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int r = wm * RW + 16 * i + lrow;
      frag_from_units(xa[i], As_s[r * KU + swz(u, r)], zero_unit());
    }
  };
  auto mm = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NTW; ++j) mma16_k32(acc[j][i], wb[j], xa[i]);
    __builtin_amdgcn_s_setprio(0);
  };
  auto bar = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // s_waitcnt lgkmcnt(0) alone: this wave's fragment reads have returned
  auto lgkm0 = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
  };

  issue(0, As0, Bs0);
  wait_vmcnt<0>();
  bar();
  // Both groups pass the same number of barriers: 1 + 4 per step.
  if (wm == 0) {
    rd(As0, Bs0, 0);                          // phase -1: read (0, h0), G0's loads of step 1
    if (1 < nk) issue(1, As1, Bs1);
    lgkm0();
    bar();
    auto g0step = [&](int kt, const u32x4_t* As_s, const u32x4_t* Bs_s, u32x4_t* As_n, u32x4_t* Bs_n)
        __attribute__((always_inline)) {
      mm();                                   // phase 0: (kt, h0)
      bar();
      rd(As_s, Bs_s, 1);                      // phase 1: read (kt, h1)
      lgkm0();
      bar();
      mm();                                   // phase 2: (kt, h1)
      wait_vmcnt<0>();                        // this wave's loads of step kt + 1
      bar();
      if (kt + 1 < nk) rd(As_n, Bs_n, 0);     // phase 3: read (kt + 1, h0), G0's loads of kt + 2
      if (kt + 2 < nk) issue(kt + 2, (u32x4_t*)As_s, (u32x4_t*)Bs_s);
      lgkm0();
      bar();
    };
    for (int kt = 0; kt < nk; kt += 2) {
      g0step(kt, As0, Bs0, As1, Bs1);
      if (kt + 1 < nk) g0step(kt + 1, As1, Bs1, As0, Bs0);
    }
  } else {
    bar();                                    // phase -1
    auto g1step = [&](int kt, const u32x4_t* As_s, const u32x4_t* Bs_s, u32x4_t* As_n, u32x4_t* Bs_n)
        __attribute__((always_inline)) {
      rd(As_s, Bs_s, 0);                      // phase 0: read (kt, h0), G1's loads of kt + 1
      if (kt + 1 < nk) issue(kt + 1, As_n, Bs_n);
      lgkm0();
      bar();
      mm();                                   // phase 1: (kt, h0)
      bar();
      rd(As_s, Bs_s, 1);                      // phase 2: read (kt, h1)
      lgkm0();
      wait_vmcnt<0>();                        // this wave's loads of step kt + 1
      bar();
      mm();                                   // phase 3: (kt, h1)
      bar();
    };
    for (int kt = 0; kt < nk; kt += 2) {
      g1step(kt, As0, Bs0, As1, Bs1);
      if (kt + 1 < nk) g1step(kt + 1, As1, Bs1, As0, Bs0);
    }
  }
  if constexpr (BMT == BM)
    staged_epilogue<BN, WN, NT8, EPI>(p, m0, n0, wm, wn, tid, acc, As0, As1, Bs0, Bs1);
  else
    staged_epilogue_288<BN, WN, NT8, EPI>(p, m0, n0, wm, wn, tid, acc, As0, As1, Bs0, Bs1);
}

// MX-fp8 variant of the eight-wave kernel (OCP Microscaling MX-fp8 operands:
// e4m3 codes, one E8M0 scale per 32 values along k).  A k step is 128 codes
// per row, the same 128 bytes per tile row as a bf16 step, so the LDS ring,
// the swizzle and the direct loads are unchanged; one scaled matrix
// instruction (v_mfma_scale_f32_16x16x128_f8f6f4, twice the bf16 rate)
// consumes a whole step per 16 x 16 tile.  Its operand layout: lane l gives
// row l % 16 and the bytes of k in [16 g, 16 g + 16) and [64 + 16 g, 64 + 16 g
// + 16), g = l / 16 (row units g and g + 4), and the scale byte of row l % 16,
// block g of the step.  The scales of a step are 64 consecutive bytes per
// 16-row group (mx_scale_index); they travel with the step's tiles, straight
// into LDS (one 256-byte load per four groups), and each lane reads its byte
// there: no scale registers live across steps.
//
// A-gather modes as in the bf16 kernels, on codes (one byte per element): the
// implicit 3x3 stride-2 convolution needs cin a multiple of 128 so that a k
// step stays within one tap.  Their scales are row-major (a_scale_ld bytes per
// input pixel or gathered row); a step's four blocks of a row are then four
// consecutive bytes, one 4-byte load per row into an LDS table [row][4].
template <int BN, int AMODE, int EPI>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm8w_f8_kernel(GemmArgs p, int nM, int nN, int per_xcd) {
  constexpr int NT8 = 512;
  constexpr int WN = BN / 4;                 // columns per wave
  constexpr int NTW = WN / 16;               // 16-column tiles per wave
  constexpr int A_UNITS = BM * KU;
  constexpr int B_UNITS = BN * KU;
  constexpr int A_LOADS = A_UNITS / NT8;
  constexpr int B_LOADS = B_UNITS / NT8;
  constexpr int BK8 = 128;                   // codes per row per k step
  constexpr int SA_Q = BM / 64;              // 256-byte scale loads per step: 4 groups / 64 rows each
  constexpr int SB_Q = BN / 64;
  static_assert(B_UNITS % NT8 == 0 && BN % 64 == 0, "whole loads per thread");
  static_assert(SA_Q + SB_Q <= 16, "scale loads: at most two per wave");
  __shared__ u32x4_t As0[A_UNITS], As1[A_UNITS];
  __shared__ u32x4_t Bs0[B_UNITS], Bs1[B_UNITS];
  __shared__ unsigned Sa0[BM], Sa1[BM], Sb0[BN], Sb1[BN];  // 4 scale bytes per row

  const int tile = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (tile >= nM * nN) return;
  const int per_group = GROUP_M * nN;
  const int group = tile / per_group;
  const int first_m = group * GROUP_M;
  const int gsize = min(nM - first_m, GROUP_M);
  const int in_g = tile - group * per_group;
  const int m0 = (first_m + in_g % gsize) * BM;
  const int n0 = (in_g / gsize) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7
  const int wm = wave >> 2, wn = wave & 3;
  const int M = p.M, N = p.N, K = p.K;
  const int KS = K / BK8;                    // k steps (K is a multiple of 128)

  const int lrow8 = lane >> 3;
  const int lunit = (lane & 7) ^ lrow8;
  const char* a_base;
  unsigned a_bytes;
  if (AMODE == A_PLAIN) {
    a_base = (const char*)p.A + (size_t)m0 * p.lda;
    a_bytes = tile_records((size_t)(M - m0) * p.lda);
  } else {
    a_base = (const char*)p.A;
    a_bytes = (unsigned)p.a_bytes;
  }
  const unsigned a_step = (unsigned)(64 * p.lda);
  const unsigned a_off0 = (unsigned)((wave * 8 + lrow8) * p.lda);
  // A_ROWMAP: per-load row offsets; A_CONV: per-load window corners and taps
  unsigned a_rowoff[A_LOADS];
  ConvGather<A_LOADS, 1> cg;  // (full size in every mode: see ConvGather)
  // output pixel of GEMM row m: {chunk, (oy << 16) | ox}
  auto conv_pixel = [&](int m) __attribute__((always_inline)) {
    const int hw = p.hout * p.wout;
    const int chunk = m / hw;
    const int rem = m - chunk * hw;
    int oy, ox;
    if (p.xmajor) {
      ox = rem / p.hout;
      oy = rem - ox * p.hout;
    } else {
      oy = rem / p.wout;
      ox = rem - oy * p.wout;
    }
    return int2{chunk, (oy << 16) | ox};
  };
  if (AMODE != A_PLAIN) {
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) {
      const int m = m0 + (j * 8 + wave) * 8 + lrow8;
      if (AMODE == A_ROWMAP) {
        a_rowoff[j] = m < M ? (unsigned)((size_t)(p.rowmap[m] - p.rowmap_base) * p.lda) : OOB;
      } else {
        cg.row(p, j, m);
      }
    }
    if (AMODE == A_CONV) cg.start(lunit * 16, p.cin);
  }
  // (an MX epilogue that writes zero columns past N may run tiles with n0 >= N:
  // their B rows all load zero)
  const char* b_base = (const char*)p.B + (size_t)(n0 < N ? n0 : 0) * p.ldb;
  const unsigned b_bytes = n0 < N ? (unsigned)((size_t)(N - n0) * p.ldb) : 0u;
  const unsigned b_step = (unsigned)(64 * p.ldb);
  const unsigned b_off0 = (unsigned)((wave * 8 + lrow8) * p.ldb);
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a_base, (short)0, (int)a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t b_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)b_base, (short)0, (int)b_bytes, 0x00020000);
  // Scale loads.  A_PLAIN: wave w < SA_Q takes A groups 4 w .. 4 w + 3 of the
  // tile, lane l bytes 4 (l % 16) .. + 3 of group l / 16.  A_CONV / A_ROWMAP:
  // wave w < SA_Q takes rows 64 w .. 64 w + 63, lane l row 64 w + l.  Waves
  // SA_Q .. SA_Q + SB_Q - 1 (mod 8) take the B groups.  Loads past the scale
  // array read zero.
  const unsigned sa_bytes = AMODE == A_PLAIN ? (unsigned)(((M + 15) >> 4) * KS * 64)
                                             : (unsigned)p.a_scale_bytes;
  const __amdgpu_buffer_rsrc_t sa_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.a_scale, (short)0, (int)sa_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t sb_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.b_scale, (short)0, (int)(((N + 15) >> 4) * KS * 64), 0x00020000);
  const int sq_a = wave;                          // A quad of this wave, if < SA_Q
  const int sq_b0 = (wave - SA_Q) & 7;            // first B quad of this wave
  const int sgrp = lane >> 4, sbyte = 4 * (lane & 15);
  // gathered modes: the scale row of this lane's load
  unsigned s_rowoff = OOB;                        // A_ROWMAP: row * a_scale_ld
  int s_pix = -1, s_chunkpix = 0;                 // A_CONV: (oy << 16) | ox, chunk * hin * win
  if (AMODE != A_PLAIN && sq_a < SA_Q) {
    const int m = m0 + 64 * sq_a + lane;
    if (m < M) {
      if (AMODE == A_ROWMAP) {
        s_rowoff = (unsigned)((size_t)(p.rowmap[m] - p.rowmap_base) * p.a_scale_ld);
      } else {
        const int2 cpx = conv_pixel(m);
        s_pix = cpx.y;
        s_chunkpix = cpx.x * p.hin * p.win;
      }
    }
  }

  auto issue = [&](int kt, u32x4_t* As_s, u32x4_t* Bs_s, unsigned* Sa_s, unsigned* Sb_s)
      __attribute__((always_inline)) {
    if (AMODE == A_CONV) {
      const int toff = cg.tap_offset(p);
#pragma unroll
      for (int j = 0; j < A_LOADS; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, dma_dst(&As_s[(j * 8 + wave) * 64]), 16,
                                                 cg.offset(j, toff), 0, 0, 0);
      cg.advance(BK8, p.cin);  // steps are issued in increasing order
    } else {
      const unsigned koff = (unsigned)(kt * BK8 + lunit * 16);
#pragma unroll
      for (int j = 0; j < A_LOADS; ++j) {
        const unsigned off = AMODE == A_PLAIN ? a_off0 + j * a_step + koff
                                              : (a_rowoff[j] == OOB ? OOB : a_rowoff[j] + koff);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, dma_dst(&As_s[(j * 8 + wave) * 64]), 16,
                                                 off, 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, dma_dst(&Bs_s[(j * 8 + wave) * 64]), 16,
                                               b_off0 + j * b_step + (unsigned)(kt * BK8 + lunit * 16),
                                               0, 0, 0);
    if (sq_a < SA_Q) {
      unsigned off;
      if (AMODE == A_PLAIN) {
        const int grp = (m0 >> 4) + 4 * sq_a + sgrp;
        off = (unsigned)((grp * KS + kt) * 64 + sbyte);
      } else if (AMODE == A_ROWMAP) {
        off = s_rowoff == OOB ? OOB : s_rowoff + 4 * kt;
      } else {
        const int tap = (kt * BK8) / p.cin;
        const int cb = ((kt * BK8) - tap * p.cin) / MX_BLOCK;
        const int kh = tap / 3;
        const int kw = tap - 3 * kh;
        const int iy = 2 * (s_pix >> 16) + kh - 1;
        const int ix = 2 * (s_pix & 0xFFFF) + kw - 1;
        const bool ok = s_pix >= 0 && iy >= 0 && iy < p.hin && ix >= 0 && ix < p.win;
        off = ok ? (unsigned)((s_chunkpix + iy * p.win + ix) * p.a_scale_ld + cb) : OOB;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sa_rsrc, dma_dst((const u32x4_t*)&Sa_s[64 * sq_a]), 4,
                                               off, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int q = sq_b0 + 8 * r;
      if (q < SB_Q) {
        const int grp = (n0 >> 4) + 4 * q + sgrp;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            sb_rsrc, dma_dst((const u32x4_t*)&Sb_s[64 * q]), 4,
            (unsigned)((grp * KS + kt) * 64 + sbyte), 0, 0, 0);
      }
    }
  };

  f32x4_t acc[NTW][8];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[j][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int lrow = lane & 15;
  const int g = lane >> 4;
  // Ping-pong schedule (convolution GEMMs on 256-column tiles; the lockstep
  // loop below serves the rest), as in the bf16 eight-wave kernel: the two rows
  // of waves, G0 (wm = 0) and G1 (wm = 1), run one phase apart, a phase being
  // either the matrix instructions of one half of a step (row blocks 0..3 or
  // 4..7, 20 instructions) or the fragment reads of the next half plus this
  // wave's share of a step's loads, each phase ending at a barrier.  The
  // weight fragments and scales of a step are read with its first half.
  // Stage kt % 2 serves step kt; G1 issues its loads of step kt + 1 in phase 0
  // of step kt and G0 in phase 3 of step kt - 1, after every reader of that
  // stage is past it.  Each output still sums its k steps in increasing order.
  i32x8_t wb[NTW], xa[4];
  int sw[NTW], sx[4];
  auto rd = [&](const u32x4_t* As_s, const u32x4_t* Bs_s, const unsigned* Sa_s, const unsigned* Sb_s,
                auto part_c) __attribute__((always_inline)) {
    constexpr int part = decltype(part_c)::value;
    // A_PLAIN: group wm * 8 + i, byte 64 i + lane; gathered: row wm * 128 + 16 i + lrow, byte g
    const uint8_t* sa = AMODE == A_PLAIN ? (const uint8_t*)Sa_s + wm * 512 + lane
                                         : (const uint8_t*)Sa_s + (wm * 128 + lrow) * 4 + g;
    if constexpr (part == 0) {
      const uint8_t* sb = (const uint8_t*)Sb_s + wn * (WN * 4) + lane;
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int r = wn * WN + 16 * j + lrow;
        wb[j] = units_to_i32x8(Bs_s[r * KU + swz(g, r)], Bs_s[r * KU + swz(g + 4, r)]);
        sw[j] = sb[64 * j];
      }
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = 4 * part + ii;
      const int r = wm * 128 + 16 * i + lrow;
      xa[ii] = units_to_i32x8(As_s[r * KU + swz(g, r)], As_s[r * KU + swz(g + 4, r)]);
      sx[ii] = sa[64 * i];   // 64 bytes per 16 rows in both layouts
    }
  };
  auto mm = [&](auto part_c) __attribute__((always_inline)) {
    constexpr int part = decltype(part_c)::value;
    __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int j = 0; j < NTW; ++j)
        acc[j][4 * part + ii] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            wb[j], xa[ii], acc[j][4 * part + ii], 0, 0, 0, sw[j], 0, sx[ii]);
    // pin the phase's matrix instructions here: they touch no memory, so
    // without a use the compiler sinks them past the barriers that follow
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int j = 0; j < NTW; ++j) asm volatile("" : "+v"(acc[j][4 * part + ii]));
    __builtin_amdgcn_s_setprio(0);
  };
  auto bar = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // s_waitcnt lgkmcnt(0) alone: this wave's fragment reads have returned
  auto lgkm0 = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
  };

  if constexpr (BN > 256 || AMODE != A_CONV) {
    // The lockstep loop, one barrier per step.  256 x 320 tiles have no
    // registers for the ping-pong's fragments next to the 160 accumulators;
    // the ping-pong pays (conv GEMMs 4% faster) only on the convolution's long
    // k loops: on the 256-column layer GEMMs it cost 18%, on conv_out 5%.
    auto step = [&](int kt, const u32x4_t* As_s, const u32x4_t* Bs_s, const unsigned* Sa_s,
                    const unsigned* Sb_s, u32x4_t* As_n, u32x4_t* Bs_n, unsigned* Sa_n, unsigned* Sb_n)
        __attribute__((always_inline)) {
      wait_vmcnt<0>();
      bar();
      if (kt + 1 < KS) issue(kt + 1, As_n, Bs_n, Sa_n, Sb_n);
      const uint8_t* sa = AMODE == A_PLAIN ? (const uint8_t*)Sa_s + wm * 512 + lane
                                           : (const uint8_t*)Sa_s + (wm * 128 + lrow) * 4 + g;
      const uint8_t* sb = (const uint8_t*)Sb_s + wn * (WN * 4) + lane;
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int r = wn * WN + 16 * j + lrow;
        wb[j] = units_to_i32x8(Bs_s[r * KU + swz(g, r)], Bs_s[r * KU + swz(g + 4, r)]);
        sw[j] = sb[64 * j];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = wm * 128 + 16 * i + lrow;
        const i32x8_t x = units_to_i32x8(As_s[r * KU + swz(g, r)], As_s[r * KU + swz(g + 4, r)]);
        const int sxi = sa[64 * i];
#pragma unroll
        for (int j = 0; j < NTW; ++j)
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wb[j], x, acc[j][i], 0, 0, 0,
                                                                       sw[j], 0, sxi);
      }
    };
    issue(0, As0, Bs0, Sa0, Sb0);
    for (int kt = 0; kt < KS; kt += 2) {
      step(kt, As0, Bs0, Sa0, Sb0, As1, Bs1, Sa1, Sb1);
      if (kt + 1 < KS) step(kt + 1, As1, Bs1, Sa1, Sb1, As0, Bs0, Sa0, Sb0);
    }
  } else {
  issue(0, As0, Bs0, Sa0, Sb0);
  wait_vmcnt<0>();
  bar();
  // Both groups pass the same number of barriers: 1 + 4 per step.
  if (wm == 0) {
    rd(As0, Bs0, Sa0, Sb0, PartC<0>{});      // phase -1: read (0, h0), G0's loads of step 1
    if (1 < KS) issue(1, As1, Bs1, Sa1, Sb1);
    lgkm0();
    bar();
    auto g0step = [&](int kt, const u32x4_t* As_s, const u32x4_t* Bs_s, const unsigned* Sa_s,
                      const unsigned* Sb_s, u32x4_t* As_n, u32x4_t* Bs_n, unsigned* Sa_n,
                      unsigned* Sb_n) __attribute__((always_inline)) {
      mm(PartC<0>{});                         // phase 0: (kt, h0)
      bar();
      rd(As_s, Bs_s, Sa_s, Sb_s, PartC<1>{}); // phase 1: read (kt, h1)
      lgkm0();
      bar();
      mm(PartC<1>{});                         // phase 2: (kt, h1)
      wait_vmcnt<0>();                        // this wave's loads of step kt + 1
      bar();
      if (kt + 1 < KS) rd(As_n, Bs_n, Sa_n, Sb_n, PartC<0>{});  // phase 3: read (kt + 1, h0), G0's loads of kt + 2
      if (kt + 2 < KS) issue(kt + 2, (u32x4_t*)As_s, (u32x4_t*)Bs_s, (unsigned*)Sa_s, (unsigned*)Sb_s);
      lgkm0();
      bar();
    };
    for (int kt = 0; kt < KS; kt += 2) {
      g0step(kt, As0, Bs0, Sa0, Sb0, As1, Bs1, Sa1, Sb1);
      if (kt + 1 < KS) g0step(kt + 1, As1, Bs1, Sa1, Sb1, As0, Bs0, Sa0, Sb0);
    }
  } else {
    bar();                                    // phase -1
    auto g1step = [&](int kt, const u32x4_t* As_s, const u32x4_t* Bs_s, const unsigned* Sa_s,
                      const unsigned* Sb_s, u32x4_t* As_n, u32x4_t* Bs_n, unsigned* Sa_n,
                      unsigned* Sb_n) __attribute__((always_inline)) {
      rd(As_s, Bs_s, Sa_s, Sb_s, PartC<0>{}); // phase 0: read (kt, h0), G1's loads of kt + 1
      if (kt + 1 < KS) issue(kt + 1, As_n, Bs_n, Sa_n, Sb_n);
      lgkm0();
      bar();
      mm(PartC<0>{});                         // phase 1: (kt, h0)
      bar();
      rd(As_s, Bs_s, Sa_s, Sb_s, PartC<1>{}); // phase 2: read (kt, h1)
      lgkm0();
      wait_vmcnt<0>();                        // this wave's loads of step kt + 1
      bar();
      mm(PartC<1>{});                         // phase 3: (kt, h1)
      bar();
    };
    for (int kt = 0; kt < KS; kt += 2) {
      g1step(kt, As0, Bs0, Sa0, Sb0, As1, Bs1, Sa1, Sb1);
      if (kt + 1 < KS) g1step(kt + 1, As1, Bs1, Sa1, Sb1, As0, Bs0, Sa0, Sb0);
    }
  }
  }

  staged_epilogue<BN, WN, NT8, EPI>(p, m0, n0, wm, wn, tid, acc, As0, As1, Bs0, Bs1);
}

template <int BN, int AMODE, int EPI>
hipError_t run8_f8(const GemmArgs& a, hipStream_t s) {
  const int nM = (a.M + BM - 1) / BM;
  // an MX epilogue also writes the zero columns up to n_store
  const int ncols = EPI == EPI_GELU_MX && a.n_store > a.N ? a.n_store : a.N;
  const int nN = (ncols + BN - 1) / BN;
  const int tiles = nM * nN;
  const int per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL((gemm8w_f8_kernel<BN, AMODE, EPI>), dim3(8 * per_xcd), dim3(512), 0, s, a, nM,
                     nN, per_xcd);
  return hipGetLastError();
}

template <int BN, int AMODE, int EPI, int BMT = BM>
hipError_t run8(const GemmArgs& a, hipStream_t s) {
  const int nM = (a.M + BMT - 1) / BMT;
  const int nN = (a.N + BN - 1) / BN;
  const int tiles = nM * nN;
  const int per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL((gemm8w_kernel<BN, AMODE, EPI, BMT>), dim3(8 * per_xcd), dim3(512), 0, s, a, nM,
                     nN, per_xcd);
  return hipGetLastError();
}

template <int BN, int AMODE, int EPI>
hipError_t run(const GemmArgs& a, hipStream_t s) {
  const int nM = (a.M + BM - 1) / BM;
  const int nN = (a.N + BN - 1) / BN;
  const int tiles = nM * nN;
  const int per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL((gemm256_kernel<BN, AMODE, EPI>), dim3(8 * per_xcd), dim3(NTHR), 0, s, a, nM,
                     nN, per_xcd);
  return hipGetLastError();
}

template <int BN, int AMODE, int EPI>
hipError_t run_any(const GemmArgs& a, hipStream_t s) {
  if constexpr (BN >= 256) return run8<BN, AMODE, EPI>(a, s);
  else return run<BN, AMODE, EPI>(a, s);
}

template <int BN>
hipError_t dispatch(const GemmArgs& a, int amode, int epi, hipStream_t s) {
  if (amode == A_PLAIN) {
    switch (epi) {
      case EPI_STORE: return run_any<BN, A_PLAIN, EPI_STORE>(a, s);
      case EPI_STORE_GELU: return run_any<BN, A_PLAIN, EPI_STORE_GELU>(a, s);
      case EPI_RESID: return run_any<BN, A_PLAIN, EPI_RESID>(a, s);
      case EPI_STORE_F32: return run_any<BN, A_PLAIN, EPI_STORE_F32>(a, s);
      case EPI_GELU_MX: return run_any<BN, A_PLAIN, EPI_GELU_MX>(a, s);
      default: break;
    }
  } else if (amode == A_CONV && epi == EPI_STORE_GELU) {
    return run_any<BN, A_CONV, EPI_STORE_GELU>(a, s);
  } else if (amode == A_ROWMAP && epi == EPI_PE) {
    return run_any<BN, A_ROWMAP, EPI_PE>(a, s);
  }
  return hipErrorInvalidValue;
}

// 288 x 256 tiles of the eight-wave kernel (plain A operand and the plain
// epilogues only)
hipError_t dispatch288(const GemmArgs& a, int amode, int epi, hipStream_t s) {
  if (amode == A_PLAIN) {
    switch (epi) {
      case EPI_STORE: return run8<256, A_PLAIN, EPI_STORE, 288>(a, s);
      case EPI_STORE_GELU: return run8<256, A_PLAIN, EPI_STORE_GELU, 288>(a, s);
      case EPI_RESID: return run8<256, A_PLAIN, EPI_RESID, 288>(a, s);
      case EPI_STORE_F32: return run8<256, A_PLAIN, EPI_STORE_F32, 288>(a, s);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

// Column tile for an N: the candidate with the best estimated throughput,
// i.e. tile-slot use on 256 CUs (partly empty last round, columns past N)
// times the measured relative speed of the kernel per tile-slot (eight-wave
// 256 x 320 / 256 x 256 tiles run ~1.3x the four-wave 256 x 160 ones on the
// layer GEMMs and the conv3 implicit GEMM; 256 x 128 ~0.87x); ties to the
// first candidate.
int pick_bn(int M, int N) {
  const int cands[4] = {320, 256, 160, 128};
  const double speed[4] = {1.3, 1.3, 1.0, 0.87};
  const int nM = (M + BM - 1) / BM;
  int best = 320;
  double best_eff = -1.0;
  for (int c = 0; c < 4; ++c) {
    const int bn = cands[c];
    const int nN = (N + bn - 1) / bn;
    const long tiles = (long)nM * nN;
    const long slots = ((tiles + 255) / 256) * 256;
    const double eff = speed[c] * (double)tiles / (double)slots * (double)N / (double)(nN * bn);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = bn;
    }
  }
  return best;
}

// Whether a 288 x 256 tile beats the eight-wave column tile pick_bn chose:
// estimated time = rounds of 256 tiles x (k steps x per-step cost + per-tile
// cost), with the costs measured on MI355X on the layer GEMM shapes (us with
// every CU busy: 256 x 320 1.65 per 64-deep step and ~20 per tile, 288 x 256
// 1.69 and ~18.5, 256 x 256 1.49 and ~18).  It wins where the k loop is short
// against the epilogue and the row count fits 288-row tiles better (14 673
// rows at K = 1280: 51 tiles of 288 against 58 of 256), and loses on long k
// loops (K = 5120).
bool use_288(int M, int N, int K, int bn) {
  if (bn != 320 && bn != 256) return false;
  const long nk = (K + BK - 1) / BK;
  auto est = [&](int bm, int bnn, double step, double tile) {
    const long tiles = (long)((M + bm - 1) / bm) * ((N + bnn - 1) / bnn);
    return (double)((tiles + 255) / 256) * ((double)nk * step + tile);
  };
  const double cur = bn == 320 ? est(256, 320, 1.65, 20.0) : est(256, 256, 1.49, 18.0);
  return est(288, 256, 1.69, 18.5) < cur * (1.0 - 1e-9);
}

// the epilogue copies 16-byte chunks (or, for MX output, 32-value blocks) of
// output rows
bool epilogue_fits(const GemmArgs& a, int epi) {
  if ((size_t)a.out & 15) return false;
  if (epi == EPI_GELU_MX) {
    const int ncols = a.n_store > a.N ? a.n_store : a.N;
    return ncols % 128 == 0 && a.ldo % 16 == 0 && a.ldo >= ncols && a.out_scale != nullptr;
  }
  const int epc = (epi == EPI_STORE || epi == EPI_STORE_GELU) ? 8 : 4;
  return a.N % epc == 0 && a.ldo % epc == 0;
}

}  // namespace

int g_gemm256_force_bn = 0;  // tuning hook: 0 = automatic

namespace {

template <int BN>
hipError_t dispatch_f8(const GemmArgs& a, int amode, int epi, hipStream_t s) {
  if (amode == A_PLAIN) {
    switch (epi) {
      case EPI_STORE: return run8_f8<BN, A_PLAIN, EPI_STORE>(a, s);
      case EPI_STORE_GELU: return run8_f8<BN, A_PLAIN, EPI_STORE_GELU>(a, s);
      case EPI_RESID: return run8_f8<BN, A_PLAIN, EPI_RESID>(a, s);
      case EPI_STORE_F32: return run8_f8<BN, A_PLAIN, EPI_STORE_F32>(a, s);
      case EPI_GELU_MX: return run8_f8<BN, A_PLAIN, EPI_GELU_MX>(a, s);
      default: break;
    }
  } else if (amode == A_CONV && epi == EPI_GELU_MX) {
    return run8_f8<BN, A_CONV, EPI_GELU_MX>(a, s);
  } else if (amode == A_ROWMAP && epi == EPI_PE) {
    return run8_f8<BN, A_ROWMAP, EPI_PE>(a, s);
  }
  return hipErrorInvalidValue;
}

// column tile of the fp8 kernel: 320 or 256, whichever fills the 256 CUs'
// tile slots and the columns better (ties to 320, fewer operand bytes per flop)
int pick_bn_f8(int M, int N) {
  const int nM = (M + BM - 1) / BM;
  int best = 320;
  double best_eff = -1.0;
  for (int bn : {320, 256}) {
    const int nN = (N + bn - 1) / bn;
    const long tiles = (long)nM * nN;
    const long slots = ((tiles + 255) / 256) * 256;
    const double eff = (double)tiles / (double)slots * (double)N / (double)(nN * bn);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = bn;
    }
  }
  return best;
}

}  // namespace

int g_gemm_f8_force_bn = 0;  // tuning hook: 0 = automatic

// Relative duration of a gathered-A (conv) launch of M x N in the model the
// column-tile choice uses: rounds of 256 tiles (one tile per CU at a time,
// every tile of a launch equally long) times a tile's width over the kernel's
// relative speed per tile slot.  K drops out (the conv GEMMs share it).
double gemm_conv_time_model(int M, int N, bool f8) {
  if (M <= 0 || N <= 0) return 0.0;
  const int bn = f8 ? (g_gemm_f8_force_bn ? g_gemm_f8_force_bn : pick_bn_f8(M, N))
                    : (g_gemm256_force_bn ? g_gemm256_force_bn : pick_bn(M, N));
  const long tiles = (long)((M + BM - 1) / BM) * ((N + bn - 1) / bn);
  const double speed = f8 ? 1.0 : (bn >= 256 ? 1.3 : bn == 160 ? 1.0 : 0.87);
  return (double)((tiles + 255) / 256) * (double)bn / speed;
}

hipError_t launch_gemm_f8(const GemmArgs& a, int amode, int epi, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.K <= 0 || a.K % 128 || a.lda % 16 || a.ldb % 16 || !a.a_scale || !a.b_scale ||
      ((size_t)a.A & 15) || ((size_t)a.B & 15) || !epilogue_fits(a, epi))
    return hipErrorInvalidValue;
  // gathered A: a k step within one tap, whole 4-byte scale rows, 32-bit offsets
  if (amode == A_CONV && (a.cin % 128 || a.K != 9 * a.cin)) return hipErrorInvalidValue;
  if (amode != A_PLAIN && (a.a_scale_ld % 4 || a.a_scale_bytes >= ((size_t)1 << 31) ||
                           a.a_bytes >= ((size_t)1 << 31)))
    return hipErrorInvalidValue;
  const int bn = g_gemm_f8_force_bn ? g_gemm_f8_force_bn : pick_bn_f8(a.M, a.N);
  if (bn == 320) return dispatch_f8<320>(a, amode, epi, s);
  if (bn == 256) return dispatch_f8<256>(a, amode, epi, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm256(const GemmArgs& a, int amode, int epi, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (!epilogue_fits(a, epi)) return hipErrorInvalidValue;
  // gathered A: one descriptor over the whole buffer, 32-bit offsets below OOB
  if (amode != A_PLAIN && a.a_bytes >= (size_t)OOB) return hipErrorInvalidValue;
  // 288-row tiles: plain A operand, plain epilogues (a tuning value of 288
  // forces them)
  const bool plain = amode == A_PLAIN && (epi == EPI_STORE || epi == EPI_STORE_GELU ||
                                          epi == EPI_RESID || epi == EPI_STORE_F32);
  const int bn = g_gemm256_force_bn ? g_gemm256_force_bn : pick_bn(a.M, a.N);
  if (bn == 288 || (!g_gemm256_force_bn && plain && use_288(a.M, a.N, a.K, bn)))
    return plain ? dispatch288(a, amode, epi, s) : hipErrorInvalidValue;
  switch (bn) {
    case 320: return dispatch<320>(a, amode, epi, s);
    case 256: return dispatch<256>(a, amode, epi, s);
    case 160: return dispatch<160>(a, amode, epi, s);
    case 128: return dispatch<128>(a, amode, epi, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(const GemmArgs& a, int amode, int epi, aut_dtype dt, hipStream_t s) {
  if (dt == AUT_BF16) return launch_gemm256(a, amode, epi, s);
  return launch_gemm128(a, amode, epi, dt, s);
}

}  // namespace aut
