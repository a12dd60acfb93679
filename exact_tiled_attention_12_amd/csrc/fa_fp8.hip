// fp8 (e4m3) path for gfx950: block quantisation with an optional orthogonal
// rotation, and the fused attention forward on fp8 operands.
//
// What it computes ("FlashAttention v1～v4 完整进化史", v3 part 3):
//   * each block of 64 rows (all d columns) of one (batch, head) gets its own
//     scale instead of one scale for the whole tensor: amax / 448, or (the
//     form is not stated; V takes this one) the smallest power of two at or
//     above it, the fp8 matrix cores' block-scale form; Q and K may first be
//     multiplied by one orthogonal matrix, which leaves Q K^T unchanged and
//     spreads outlier channels over all columns;
//   * both attention products run on fp8 matrix cores; the exponentiated
//     scores are themselves rounded to fp8 for the product with V.
// Format: OCP e4m3fn (bias 7, largest finite 448, no infinity); encoding
// saturates to +-448 and then rounds to nearest, ties to even.
//
// Attention schedule (same skeleton as the bf16 forward):
//   * one workgroup = 8 waves = 256 query rows; each wave owns 32 rows, which
//     lie inside one 64-row scale block; key tiles of 64 keys coincide with
//     the scale blocks of K and V;
//   * K and V tiles move from HBM into an 8-stage LDS ring with buffer loads
//     that write LDS directly, up to six tiles ahead of use;
//   * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x64_f8f6f4. K rows are
//     read in a permuted order so that each lane's 32 scores of its query are
//     exactly the 32 bytes of the P^T operand; V stays row-major and is read
//     with ds_read_b64_tr_b8;
//   * the scores are scaled by scale * log2(e) * sQ * sK_j in one FMA that
//     also folds in the factor 448, so P' = 448 P~ comes out of exp2 ready to
//     convert; l sums the float32 P' (the factor 448 cancels in O = acc / l);
//   * each row's reference m is its running maximum rounded up to a whole
//     power of two (the lazy rescaling of "FlashAttention v1～v4 完整进化史",
//     v4 part 3, kept inside e4m3's range: P' <= 448 still), so every factor
//     between references is a power of two. The product of a tile's P with V
//     carries two such factors as the matrix instruction's 8-bit exponent
//     scales: the tile's V block scale on the V operand, and 2^(m - mr) on
//     the P operand, per query row, where mr is the accumulator's own
//     reference. The accumulator is multiplied only when m passes mr by more
//     than 2^8 (in practice once per row, at its first key), and O = acc *
//     2^(mr - m) / l at the end.
#include <algorithm>
#include <cfloat>
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

// ---------------------------------------------------------------- encoder

// e4m3fn code of x: saturate to +-448, round to nearest even, NaN -> 0x7F.
// Works on the float32 bit pattern: for normal results the 3 kept mantissa
// bits are rounded at bit 20 (the exponent carry is the correct result), and
// results below 2^-6 are multiples of 2^-9, rounded with rint.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a > 0x7F800000u) {
    code = 0x7Fu;
  } else if (a >= 0x43E00000u) {            // |x| >= 448
    code = 0x7Eu;
  } else if (a >= 0x3C800000u) {            // |x| >= 2^-6: normal e4m3
    code = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
  } else {
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.f);
  }
  return sign | code;
}

// Buffer resource over [base, base + bytes): loads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// ---------------------------------------------------------------- quantiser

constexpr int kQRows = 64;      // rows per scale block
constexpr int kQThreads = 256;
constexpr int kQWaves = kQThreads / 64;
constexpr int kQGrid = 1024;    // persistent workgroups (four per CU where the registers allow)
constexpr float kMinNormal = 1.17549435e-38f;

enum QuantMode { kBlockScale = 0, kAmaxOnly = 1, kGivenScale = 2 };

// Codes of four values with |q| < 464, packed little-endian. The hardware
// conversion rounds to nearest even and agrees with e4m3_code on that range
// (checked on MI355X over every float32 in [440, 480] and 4M random values
// of the e4m3 range); from 464 up it gives NaN, so callers keep |q| < 464.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Scale of a block whose largest magnitude is am: float32(am / 448) (a
// correctly rounded division; the smallest positive float32 where it
// underflows), or with pow2 the smallest power of two at or above it, at
// least 2^-126 (a valid 8-bit matrix-core exponent); 1 for an all-zero block.
__device__ __forceinline__ float block_scale(float am, bool pow2) {
  if (!(am > 0.f)) return 1.f;
  uint32_t b = __float_as_uint(am / 448.f);
  if (!pow2) return b ? __uint_as_float(b) : __uint_as_float(1u);
  if (b < 0x00800000u) return FLT_MIN;         // at or below 2^-126
  if (b & 0x007FFFFFu) b = (b & 0x7F800000u) + 0x00800000u;
  return __uint_as_float(b);
}

// Divisor of a block in the form the quotients below take: s = bn * 2^-k
// with bn in [1, 2), rn = RN(1 / bn); or, for s a power of two, rs = 1 / s
// (exact).
struct Divisor {
  float bn, rn;
  int k;
  bool p2;
};
__device__ __forceinline__ Divisor make_divisor(float s) {
  const uint32_t sb = __float_as_uint(s);
  Divisor v;
  v.p2 = (sb & 0x007FFFFFu) == 0u;
  v.k = 127 - (int)((sb >> 23) & 0xFFu);
  v.bn = __uint_as_float((sb & 0x007FFFFFu) | 0x3F800000u);
  v.rn = v.p2 ? 1.f / s : 1.f / v.bn;
  return v;
}

// The float32 quotient a / s rounded to nearest (what a division gives), for
// s normal and |a / s| <= 448 (1 + 2^-23). a and s are first scaled by the
// same power of two (exactly) so that the divisor bn lies in [1, 2); then
// from rn = RN(1 / bn) two corrections with the remainder: by Markstein's
// theorem, with rn = RN(1 / bn) and q1 within one unit in the last place of
// the quotient, RN(q1 + (a' - bn q1) rn) is RN(a' / bn), provided the
// remainder does not underflow. Scaled, it underflows only for quotients
// below about 2^-100, whose e4m3 code is 0 whatever their last bit (without
// the scaling, a block of values near 2^-110 gave codes one step off at
// rounding ties). The sign is copied from a so that -0 stays -0.
__device__ __forceinline__ float div_rn(float a, const Divisor& v) {
  const float an = __builtin_amdgcn_ldexpf(a, v.k);
  const float q0 = an * v.rn;
  const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, v.bn, an), v.rn, q0);
  const float q2 = __builtin_fmaf(__builtin_fmaf(-q1, v.bn, an), v.rn, q1);
  return __builtin_copysignf(q2, a);
}

// Four codes of y / s. With s a normal float32 at or above fl(amax / 448),
// |y / s| <= 448 (1 + 2^-23) and the hardware conversion is exact; with s a
// power of two, y / s = y * (1 / s) exactly. A subnormal s (a block of tiny
// values) takes the division and the saturating encoder.
__device__ __forceinline__ uint32_t codes4(const float* y, float s, const Divisor& v, bool fast) {
  if (fast && v.p2) return e4m3x4(y[0] * v.rn, y[1] * v.rn, y[2] * v.rn, y[3] * v.rn);
  if (fast) return e4m3x4(div_rn(y[0], v), div_rn(y[1], v), div_rn(y[2], v), div_rn(y[3], v));
  return e4m3_code(y[0] / s) | e4m3_code(y[1] / s) << 8 | e4m3_code(y[2] / s) << 16 | e4m3_code(y[3] / s) << 24;
}

// Persistent workgroups of 4 waves walk the 64-row blocks of all (batch,
// head) pairs; the next block is loaded into registers while the current one
// is computed.
//
// Without rotation, thread t holds 16-byte chunks t + 256 i of the block
// (row-major), so loads and code stores are contiguous.
//
// With rotation, Y = X R is formed on the bf16 matrix cores as
// Y^T = R^T X^T: X is exact in bf16 and R is split into three bf16 parts
// R = R1 + R2 + R3 + E with |E| <= 2^-24 |R| elementwise, all summed into one
// float32 accumulator. The block goes through LDS (rows swizzled by 16-byte
// chunk) to form the B operand; the R^T fragments of the wave's 32 output
// columns stay in registers for the whole launch. Accumulator slot i of lane
// l then holds row l % 32 of the row tile and columns 8 (i / 4) +
// 4 (l / 32) + i % 4 of the column tile.
template <int D, bool ROT, int MODE>
__global__ __launch_bounds__(kQThreads, 2) void quant_kernel(QuantArgs a, int nb, int total) {
  constexpr int CH = D / 8;                      // 16-byte chunks per row
  constexpr int LPT = kQRows * CH / kQThreads;   // 16-byte loads per thread per block
  constexpr int CT = D / 32;                     // 32-column tiles
  constexpr int WPC = kQWaves / CT;              // waves per column tile
  constexpr int RT = 2 / WPC;                    // 32-row tiles per wave
  constexpr int KC = D / 16;                     // 16-wide k chunks
  constexpr int NV = ROT ? 16 * RT : 8 * LPT;    // values per thread
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int N = a.N;
  const unsigned head_bytes = (unsigned)N * D * 2;

  __shared__ float red[2][kQWaves];
  __shared__ __attribute__((aligned(16))) __bf16 xs[ROT ? kQRows * D : 8];

  auto load_block = [&](int g, u32x4 (&r)[LPT]) {
    const int bh = g / nb, blk = g - bh * nb;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc((const __bf16*)a.x + (size_t)bh * N * D, head_bytes);
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int f = tid + kQThreads * i;
      const unsigned off = ((unsigned)(blk * kQRows + f / CH) * D + 8 * (f % CH)) * 2;
      r[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    }
  };

  const int ct = wave % CT;
  const int rt0 = (wave / CT) * RT;
  bf16x8 r1[ROT ? KC : 1], r2[ROT ? KC : 1], r3[ROT ? KC : 1];
  if constexpr (ROT) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float r = a.rot[(16 * kc + 8 * hh + e) * D + 32 * ct + l32];
        const __bf16 p1 = (__bf16)r;
        const float t1 = r - (float)p1;     // exact
        const __bf16 p2 = (__bf16)t1;
        const float t2 = t1 - (float)p2;    // exact
        r1[kc][e] = p1;
        r2[kc][e] = p2;
        r3[kc][e] = (__bf16)t2;
      }
  }

  u32x4 nx[LPT];
  int g = blockIdx.x;
  if (g < total) load_block(g, nx);
  for (int par = 0; g < total; g += gridDim.x, par ^= 1) {
    float y[NV];
    if constexpr (ROT) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int f = tid + kQThreads * i;
        const int row = f / CH, c = f % CH;
        *(u32x4*)&xs[row * D + 8 * (c ^ (row & (CH - 1)))] = nx[i];
      }
      __syncthreads();
      if (g + (int)gridDim.x < total) load_block(g + gridDim.x, nx);
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int row = 32 * (rt0 + t) + l32;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const bf16x8 b = *(const bf16x8*)&xs[row * D + 8 * ((2 * kc + hh) ^ (row & (CH - 1)))];
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r3[kc], b, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r2[kc], b, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r1[kc], b, acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) y[16 * t + i] = acc[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const bf16x8 v = __builtin_bit_cast(bf16x8, nx[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[8 * i + e] = (float)v[e];
      }
      if (g + (int)gridDim.x < total) load_block(g + gridDim.x, nx);
    }

    const int bh = g / nb, blk = g - bh * nb;
    float* sc = a.scales + g;
    float s;
    if constexpr (MODE == kGivenScale) {
      s = *sc;
    } else {
      float am = 0.f;
#pragma unroll
      for (int i = 0; i < NV; ++i) am = fmaxf(am, fabsf(y[i]));
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) am = fmaxf(am, __shfl_xor(am, o));
      if (lane == 0) red[par][wave] = am;
      __syncthreads();
      am = fmaxf(fmaxf(red[par][0], red[par][1]), fmaxf(red[par][2], red[par][3]));
      if constexpr (MODE == kAmaxOnly) {
        if (tid == 0) *sc = am;
        continue;
      }
      s = block_scale(am, a.pow2 != 0);
      if (tid == 0) *sc = s;
    }
    if constexpr (ROT) {
      // Without a reduction barrier (given scale) the LDS block must still be
      // released before the next iteration overwrites it.
      if constexpr (MODE == kGivenScale) __syncthreads();
    }

    const bool fast = s >= kMinNormal;
    const Divisor dv = make_divisor(s);
    const int rows = min(kQRows, N - blk * kQRows);
    unsigned char* x8 = a.x8 + ((size_t)bh * N + (size_t)blk * kQRows) * D;
    if constexpr (ROT) {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int row = 32 * (rt0 + t) + l32;
        if (row < rows) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *(uint32_t*)(x8 + (size_t)row * D + 32 * ct + 8 * q + 4 * hh) = codes4(&y[16 * t + 4 * q], s, dv, fast);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int f = tid + kQThreads * i;
        const int row = f / CH;
        if (row < rows) {
          u32x2 w;
          w[0] = codes4(&y[8 * i], s, dv, fast);
          w[1] = codes4(&y[8 * i + 4], s, dv, fast);
          *(u32x2*)(x8 + (size_t)row * D + 8 * (f % CH)) = w;
        }
      }
    }
  }
}

// Per-tensor scale: the largest of the per-block amax values written by the
// kAmaxOnly pass, turned into s and broadcast to every block entry.
constexpr int kRedThreads = 1024;
__global__ __launch_bounds__(kRedThreads) void quant_tensor_scale_kernel(float* scales, int n, int pow2) {
  const int tid = threadIdx.x;
  float am = 0.f;
  for (int i = tid; i < n; i += kRedThreads) am = fmaxf(am, scales[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) am = fmaxf(am, __shfl_xor(am, o));
  __shared__ float red[kRedThreads / 64];
  if ((tid & 63) == 0) red[tid >> 6] = am;
  __syncthreads();
  am = red[0];
#pragma unroll
  for (int i = 1; i < kRedThreads / 64; ++i) am = fmaxf(am, red[i]);
  const float s = block_scale(am, pow2 != 0);
  for (int i = tid; i < n; i += kRedThreads) scales[i] = s;
}

template <int D, bool ROT>
hipError_t launch_quant_d(const QuantArgs& a, int B, int H, hipStream_t st) {
  const int nb = (a.N + kQRows - 1) / kQRows;
  const int total = B * H * nb;
  const int grid = min(total, kQGrid);
  if (a.block_rows == 64) {
    hipLaunchKernelGGL((quant_kernel<D, ROT, kBlockScale>), dim3(grid), dim3(kQThreads), 0, st, a, nb, total);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((quant_kernel<D, ROT, kAmaxOnly>), dim3(grid), dim3(kQThreads), 0, st, a, nb, total);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(quant_tensor_scale_kernel, dim3(1), dim3(kRedThreads), 0, st, a.scales, total, a.pow2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((quant_kernel<D, ROT, kGivenScale>), dim3(grid), dim3(kQThreads), 0, st, a, nb, total);
  return hipGetLastError();
}

// ---------------------------------------------------------------- decoding

// out = decode(code) * s of the code's 64-row block, rounded to bf16, 16
// codes per thread. The e4m3 decode and, for a power-of-two s, the product
// are exact; so is the bf16 value while it stays inside bf16's range. A
// block whose scale is not a power of two in [2^-126, 2^127] is written as
// NaN: the backward built on these values requires exact ones.
__global__ __launch_bounds__(256) void dequant_kernel(const unsigned char* x8, const float* scales, __bf16* out,
                                                      int N, int d, int nb64, int bh0) {
  // grid: x covers one (batch, head) in 16-code chunks, y the (batch, head)
  const unsigned per_head16 = (unsigned)N * (unsigned)d / 16u;
  const unsigned i = blockIdx.x * 256u + threadIdx.x;
  if (i >= per_head16) return;
  const size_t bh = (size_t)bh0 + blockIdx.y;
  const unsigned row = i * 16u / (unsigned)d;
  const float s = scales[bh * nb64 + row / 64u];
  const uint32_t sb = __float_as_uint(s), e8 = (sb >> 23) & 0xFFu;
  const bool bad = (sb & 0x807FFFFFu) != 0u || e8 == 0u || e8 == 255u;
  const size_t e0 = bh * N * d + (size_t)i * 16u;
  const u32x4 c = *(const u32x4*)(x8 + e0);
  const float nan = __builtin_nanf("");
  u32x4 w[2];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[k], false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[k], true);
    w[k >> 1][2 * (k & 1)] = pack_bf16x2(bad ? nan : lo[0] * s, bad ? nan : lo[1] * s);
    w[k >> 1][2 * (k & 1) + 1] = pack_bf16x2(bad ? nan : hi[0] * s, bad ? nan : hi[1] * s);
  }
  *(u32x4*)(out + e0) = w[0];
  *(u32x4*)(out + e0 + 8) = w[1];
}

// ---------------------------------------------------------------- attention

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBR = 32 * kWaves;    // query rows per workgroup
constexpr int kBC = 64;             // keys per tile = rows per scale block
constexpr int kStages = 8;
constexpr int kD = 128;
constexpr int kRB = kD;             // bytes per fp8 row
constexpr int kTile = kBC * kRB;    // 8 KiB
constexpr int kStage = 2 * kTile;   // K then V
constexpr float kLog2_448 = 8.807354922057604f;
// The accumulator is re-based when a row's reference m passes the
// accumulator's reference mr by more than this (log2 units): it then holds
// at most 448 * 2^8 times the sum of |P V| in the units of O.
constexpr float kRebase = 8.f;

#define LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// Physical 16-byte chunk of logical chunk c in LDS row r is c ^ swz(r).
// K: the 16 rows one 16-lane group reads together (keys 0-7 and 16-23 of a
// 32-key block, shifted by 4 per group) land on 16 distinct bank groups.
// V: the 8 consecutive rows x 2 chunks of one transposed read do.
__device__ __forceinline__ int k_swz(int r) { return ((r >> 1) & 3) | (((r >> 4) & 1) << 2); }
__device__ __forceinline__ int v_swz(int r) { return r & 6; }

// Transposed 8-byte read at LDS byte address addr.
__device__ __forceinline__ u32x2 tr8_read(unsigned addr) {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS(i32x2, addr)));
}

__device__ __forceinline__ f32x16 mma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // Format 0 (e4m3) for both operands; zero block scales select the plain
  // (unscaled) instruction.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The same product with the A operand's blocks scaled by 2^(ea - 127) (an
// 8-bit exponent, the biased exponent field of a power-of-two float; one
// value for the wave) and the B operand's by 2^(eb - 127), eb taken per
// lane: lane l scales column l % 32 of B for the operand's 32-deep half
// l / 32, so lanes l and l + 32 must pass the same eb to scale a column.
__device__ __forceinline__ f32x16 mma_fp8_scale_ab(i32x8 a, i32x8 b, f32x16 c, int ea, int eb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
}


// Accumulator slot r of lane half h in 32-key block t holds key 32t + 16h + r
// of the tile (the K rows are permuted to make it so). A position p of the A
// operand therefore loads key 32t + 16*((p>>2)&1) + 4*(p>>3) + (p&3).
__device__ __forceinline__ int pos_to_key(int p) { return 16 * ((p >> 2) & 1) + 4 * (p >> 3) + (p & 3); }

// Maximum of three scores (finite or -inf) as one v_maximum3_f32: fmaxf
// would first quiet each matrix-core result against signalling NaNs, one
// extra instruction per score.
__device__ __forceinline__ float max3(float a, float b, float c) {
  return __builtin_elementwise_maximum(a, __builtin_elementwise_maximum(b, c));
}

// The larger of the two lane halves' values (lanes l and l ^ 32), as one
// v_maximum3_f32 after the swap: fmaxf would first quiet both swapped words.
__device__ __forceinline__ float halves_maximum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max3(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1]));
}

// Materialises x at this point of the instruction stream: values produced in
// one pipeline step for the next must not be sunk into the next step, where
// nothing would overlap them.
template <class T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

template <int N_>
using IC = std::integral_constant<int, N_>;
#define INL __attribute__((always_inline)) __device__

// Workgroup barrier for the LDS ring, ordering LDS only: each wave first
// waits (vmcnt) for its own copies of the tile; copies still in flight to
// other stages stay in flight.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The fp8 attention runs the same software pipeline as the bf16 forward:
// step j (one 64-key tile) forms the softmax of tile j while the matrix cores
// run S of tile j+1 and the product of tile j-1 with V; none of the step's 8
// products depends on its vector work, so they are interleaved one product
// at a time. The reference m never falls below the running maximum (a stale
// maximum would push 448 P past the e4m3 range); it is that maximum rounded
// up to a whole power of two. The V block scale of tile j-1 and 2^(m_{j-1} -
// mr) (both powers of two) scale the product of tile j-1 inside the matrix
// instruction, so the accumulator is multiplied only when a row's m moves
// more than 2^8 past mr.
template <bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_fp8_kernel(Fp8FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kStages * kStage];
  auto sp = [&](auto stag) INL -> unsigned char* { return ring + decltype(stag)::value * kStage; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  int wg = blockIdx.x;
  if (a.remap) wg = xcd_remap(wg, gridDim.x);
  const int bh = wg / a.n_qtiles;
  const int t = wg - bh * a.n_qtiles;
  const int qt = CAUSAL ? (a.n_qtiles - 1 - t) : t;
  const int N = a.N;
  const int nb = (N + kBC - 1) / kBC;
  const size_t base = (size_t)bh * (size_t)N * kD;
  const unsigned head_bytes = (unsigned)N * kRB;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q8 + base, head_bytes);
  const i32x4 rk = dma_rsrc(a.k8 + base, head_bytes);
  const i32x4 rv = dma_rsrc(a.v8 + base, head_bytes);
  // Block scales are read through the constant address space so that they
  // come in by scalar loads: a vector load would make the compiler wait for
  // every outstanding copy of the ring before its use.
  typedef __attribute__((address_space(4))) const float cfloat;
  const cfloat* sk = (const cfloat*)(a.sk + (size_t)bh * nb);
  const cfloat* sv = (const cfloat*)(a.sv + (size_t)bh * nb);

  const int q0 = qt * kBR;
  const int wrow0 = q0 + wave * 32;
  const int qrow = wrow0 + l32;
  const float sq = a.sq[(size_t)bh * nb + min(wrow0 / kBC, nb - 1)];
  const float cq = a.c * sq;

  const int kv_end = CAUSAL ? min(nb, (min(q0 + kBR, N) - 1) / kBC + 1) : nb;

  // Tile copies: wave w fills rows 8w .. 8w+7 of K and of V; lane l writes
  // physical chunk l % 8 of row 8w + l / 8 with the logical chunk the
  // swizzle maps there. A tile at or past kv_end reads past the buffer
  // (zeros, no traffic), so every tile has two copies per wave in flight.
  auto issue_tile = [&](int j, auto stag) INL {
    const int row = wave * 8 + (lane >> 3);
    const int p = lane & 7;
    const unsigned grow = j < kv_end ? (unsigned)(j * kBC + row) * kRB : 0x80000000u;
    const unsigned kd = (unsigned)(uintptr_t)LDS(unsigned char, sp(stag)) + wave * 1024;
    dma_load16(rk, kd, grow + 16 * (p ^ k_swz(row)));
    dma_load16(rv, kd + kTile, grow + 16 * (p ^ v_swz(row)));
  };

  // Q rows of this wave as the B operand of S^T = K Q^T: lane (l32, hh)
  // holds bytes 64*ks + 32*hh .. +32 of row qrow for d step ks.
  i32x8 qf[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const unsigned o = (unsigned)qrow * kRB + 64 * ks + 32 * hh;
    const u32x4 lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, o, 0, 0));
    const u32x4 hi = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, o + 16, 0, 0));
    qf[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // K fragment of lane (l32, hh) for 32-key block tb, d step ks, 16-byte half
  // hb: row 32tb + pos_to_key(l32), logical chunk 4ks + 2hh + hb. The swizzle
  // depends on l32 only, and ks / hb flip address bits 6 / 4.
  const int krow = pos_to_key(l32);
  const unsigned k_lane = (unsigned)krow * kRB + 16 * ((2 * hh) ^ k_swz(krow));
  // V fragment for d block mt, read q (keys 32(q/2) + 16h + 8(q%2) + 0..7):
  // source lane j of 16-lane group G points at row 16(G/2) + j/2 (plus the
  // read's offset) and bytes 32mt + 16(G%2) + 8(j%2); the result lane then
  // holds 8 consecutive keys of one d column.
  const int g16 = lane >> 4, j16 = lane & 15;
  const int vrow = 16 * (g16 >> 1) + (j16 >> 1);
  const unsigned v_lane = (unsigned)vrow * kRB + 16 * ((g16 & 1) ^ v_swz(vrow)) + 8 * (j16 & 1);

  float m = -INFINITY;     // the row's reference: an integer >= its running maximum (scaled log2 units)
  float l = 0.f;           // sum of P' = 448 P~ over this lane half's keys, in units of 2^m
  float mr = -INFINITY;    // the accumulator's reference: an integer in [m - 8, m], or -inf before any key
  int ev = 127;            // 8-bit exponent of the V scale of the newest softmax tile
  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = f32x16{};

  // Operands of the step's products. Positions 0..3 are the S products
  // (tb, ks) = (p/2, p%2) of the next tile, positions 4..7 the V products
  // mt = p-4 of the previous tile: S comes first so that its row maximum can
  // be formed inside the step, off the next step's critical path.
  struct Ops {
    i32x8 kf[4];
    i32x8 vf[4];
  };
  // LDS byte addresses of this lane's fragments in stage 0 and in stage 4:
  // the rest of a read's address (stage within its half of the ring, key
  // block, transposed-read group) fits the 16-bit immediate offset of the
  // LDS read, but the lane's swizzled part does not combine with it by an
  // addition, so each variant is formed once here and held in registers
  // (pinned: otherwise the compiler re-forms them in every step, one VALU
  // instruction and one hazard wait per read). K: [stage half][d step ks]
  // [16-byte half]; V: [stage half][d block mt].
  const unsigned ring0 = (unsigned)(uintptr_t)LDS(unsigned char, ring);
  unsigned kadr[2][2][2], vadr[2][4];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        kadr[hi][ks][hb] = ring0 + hi * 4 * kStage + ((k_lane ^ (64u * ks)) ^ (16u * hb));
        pin(kadr[hi][ks][hb]);
      }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      vadr[hi][mt] = ring0 + hi * 4 * kStage + kTile + (v_lane ^ (32u * mt));
      pin(vadr[hi][mt]);
    }
  }
  // Operands of position p from K of stage kst and V of stage vst.
  auto fetch = [&](int p, Ops& o, int kst, int vst) INL {
    if (p < 4) {
      const int tb = p / 2, ks = p % 2;
      const unsigned off = (unsigned)((kst & 3) * kStage + tb * 32 * kRB);
      const u32x4 lo = *LDS(u32x4, kadr[kst >> 2][ks][0] + off);
      const u32x4 hi = *LDS(u32x4, kadr[kst >> 2][ks][1] + off);
      o.kf[p] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    } else {
      const int mt = p - 4;
      u32x2 vr[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        vr[q] = tr8_read(vadr[vst >> 2][mt] + (unsigned)((vst & 3) * kStage + 4096 * (q >> 1) + 1024 * (q & 1)));
      o.vf[mt] = i32x8{(int)vr[0][0], (int)vr[0][1], (int)vr[1][0], (int)vr[1][1],
                       (int)vr[2][0], (int)vr[2][1], (int)vr[3][0], (int)vr[3][1]};
    }
  };
  constexpr int AHEAD = 3;

  // Scores of tile j past N or (causal) above the diagonal -> -inf; needed on
  // ragged and diagonal tiles only.
  auto masked = [&](int j) INL { return j * kBC + kBC > N || (CAUSAL && j * kBC + kBC - 1 > wrow0); };
  auto apply_mask = [&](int j, f32x16 (&sc)[2]) INL {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j * kBC + 32 * tb + 16 * hh + r;
        const bool ok = key < N && (!CAUSAL || key <= qrow);
        sc[tb][r] = ok ? sc[tb][r] : -INFINITY;
      }
  };

  // Raw row maximum over the 64 scores of one tile (both lane halves).
  auto half_max = [&](const f32x16& x) INL -> float {
    const float a0 = max3(max3(x[0], x[1], x[2]), max3(x[3], x[4], x[5]), max3(x[6], x[7], x[8]));
    return max3(a0, max3(x[9], x[10], x[11]), max3(x[12], x[13], x[14]));
  };
  auto row_max = [&](const f32x16 (&x)[2]) INL -> float {
    return halves_maximum(max3(half_max(x[0]), half_max(x[1]), max3(x[0][15], x[1][15], x[1][15])));
  };

  // One pipeline step: softmax of tile j (raw scores sc, fp8 P to pc), S of
  // tile j+1 into sn, and O += V^T P^T of tile j-1 (pp, V operands from the
  // step's fetches, V scaled by its block scale and P by 2^(m - mr) in the
  // instruction). mxr holds the raw row maximum of sc on entry (of the
  // unmasked scores) and that of sn on exit.
  auto step = [&](int j, f32x16 (&sc)[2], f32x16 (&sn)[2], const i32x8& pp, i32x8& pc, Ops& cur, Ops& nxt,
                  int kst, int vst, int nkst, int nvst, float skj, float svj_in, float& mxr) INL {
    if (masked(j)) {
      apply_mask(j, sc);
      mxr = row_max(sc);
    }
    // Tile scales (a drain step past the last tile keeps the V unit; its
    // exponentials are all zero, whatever c_j is). c_j > 0, so the scaled
    // maximum is c_j times the raw one.
    // c_j > 0 keeps masked scores at -inf after scaling (scale 0 or an
    // underflowing product would turn -inf * 0 into NaN).
    const float cj = fmaxf(cq * skj, FLT_MIN);
    // P of tile j-1 enters the accumulator scaled by 2^(m - mr), m and mr as
    // they stand before this step's update (any scale while the row has no
    // key yet: that P is zero). Both lane halves hold the same m and mr.
    const int eb_prev = m == -INFINITY ? 127 : 127 + (int)(m - mr);
    const float cand = __builtin_ceilf(mxr * cj);
    const float m_new = max3(m, cand, cand);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);      // a power of two (0 at the first key)
    // Re-base at the row's first key (mr = -inf: the accumulator is still
    // zero, factor 0) and when m passes mr by more than kRebase; NaN, so
    // no re-base, while both are -inf.
    const bool rebase = m_new - mr > kRebase;
    const float g = rebase ? fast_exp2(mr - m_new) : 1.f;
    mr = rebase ? m_new : mr;
    const int ev_prev = ev;
    m = m_new;
    l *= alpha;
    // P' = 2^(c_j s - m + log2 448) = 448 P~, four per position.
    const float nmo = kLog2_448 - m_use;
    f32x16 acc[2] = {f32x16{}, f32x16{}};
    float part[4];
    float hm0 = 0.f, hm1 = 0.f;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      if (p + AHEAD < 8)
        fetch(p + AHEAD, cur, kst, vst);
      else
        fetch(p + AHEAD - 8, nxt, nkst, nvst);
      // Issue priority (s_setprio) falls through the step: 2 while the
      // S products are issued, 1 for the V products, 0 for the bookkeeping
      // and the ring barrier between steps, so that on a SIMD the wave still
      // inside its step issues before the one already at the barrier (the
      // barrier then waits less for the slowest wave: 3.7% faster, measured).
      if (p == 0) __builtin_amdgcn_s_setprio(2);
      if (p == 4) __builtin_amdgcn_s_setprio(1);
      if (p < 4) {
        const int tb = p / 2, ks = p % 2;
        acc[tb] = mma_fp8(cur.kf[p], qf[ks], acc[tb]);
      } else {
        const int mt = p - 4;
        oacc[mt] = mma_fp8_scale_ab(cur.vf[mt], pp, oacc[mt], ev_prev, eb_prev);
      }
      // Scores 4p .. 4p+3: word p of the fp8 P operand.
      float e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[i] = fast_exp2(__builtin_fmaf(sc[p >> 2][4 * (p & 3) + i], cj, nmo));
        part[i] = p == 0 ? e[i] : part[i] + e[i];
      }
      // The low half is converted into an undefined word (the high half is
      // written next), which spares a register clear per word.
      int word;
      asm volatile("" : "=v"(word));
      word = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], word, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], word, true);
      pin(word);
      pc[p] = word;
      // Uniform bookkeeping, and the next tile's row maximum once its S
      // products (positions 0..3) have completed.
      if (p == 0) {
        // (a drain step past the last tile has no V: its P is all zero)
        ev = j < kv_end ? (int)((__float_as_uint(svj_in) >> 23) & 0xFFu) : 127;
      }
      if (p == 5) hm0 = half_max(acc[0]);
      if (p == 6) hm1 = half_max(acc[1]);
      if (p == 7) mxr = halves_maximum(max3(hm0, hm1, max3(acc[0][15], acc[1][15], acc[1][15])));
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    sn[0] = acc[0];
    sn[1] = acc[1];
    l += (part[0] + part[1]) + (part[2] + part[3]);
    // The re-base, after tile j-1's product and before tile j's (next step).
    if (__builtin_amdgcn_ballot_w64(rebase) != 0) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) oacc[mt] *= g;
    }
  };

  // Ring bookkeeping, once every two steps, before step j (j even, j >= 2):
  // steps j and j+1 read K of tiles j+1 .. j+3 and V of tiles j-1 .. j+1, so
  // tile j+3 must be resident while tile j+4 stays in flight; tiles j-3 and
  // j-2 were last read by step j-1, so their stages take tiles j+5 and j+6.
  auto pair_sync = [&](int j, auto st5, auto st6) INL {
    __builtin_amdgcn_s_waitcnt(wait_vm(2));
    ring_barrier();
    issue_tile(j + 5, st5);
    issue_tile(j + 6, st6);
  };

  // Prologue: tiles 0..6 in flight, tiles 0..3 resident; S of tile 0;
  // step 0 (its product with V is of a zero P against tile 0's V, which is
  // finite).
  issue_tile(0, IC<0>{});
  issue_tile(1, IC<1>{});
  issue_tile(2, IC<2>{});
  issue_tile(3, IC<3>{});
  issue_tile(4, IC<4>{});
  issue_tile(5, IC<5>{});
  issue_tile(6, IC<6>{});
  __builtin_amdgcn_s_waitcnt(wait_vm(6));
  ring_barrier();

  f32x16 sa[2], sb[2];
  i32x8 pa, pb = i32x8{};
  Ops oa, ob;
  {
    const unsigned char* kt = sp(IC<0>{});
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const unsigned a0 = (k_lane ^ (64u * ks)) + tb * 32 * kRB;
        const u32x4 lo = *LDS(u32x4, kt + a0);
        const u32x4 hi = *LDS(u32x4, kt + (a0 ^ 16u));
        const i32x8 kf = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        acc = mma_fp8(kf, qf[ks], acc);
      }
      sa[tb] = acc;
    }
  }
  float mxr = row_max(sa);
#pragma unroll
  for (int p = 0; p < AHEAD; ++p) fetch(p, oa, 1, 0);
  step(0, sa, sb, pb, pa, oa, ob, 1, 0, 2, 0, sk[0], sv[0], mxr);

  // Scales of tiles j0 .. j0+7 (indices clamped to the last block: past
  // kv_end they are not used).
  auto ld_scales = [&](int j0, float (&ks)[kStages], float (&vs)[kStages]) INL {
#pragma unroll
    for (int i = 0; i < kStages; ++i) {
      const int b = min(j0 + i, nb - 1);
      ks[i] = sk[b];
      vs[i] = sv[b];
    }
  };
  float skc[kStages], svc[kStages], skn[kStages], svn[kStages];
  ld_scales(1, skc, svc);

  // Steps 1..kv_end, eight per iteration (ring stages are compile-time). Step
  // j reads K of tile j+1 (stage (j+1) % 8) and V of tile j-1 (stage
  // (j-1) % 8). Step kv_end is a drain: its tile is past the last key or
  // above the diagonal, so the mask zeroes its exponentials, and it completes
  // the product of tile kv_end-1.
  auto one = [&](auto s_tag, int j0) INL -> bool {
    constexpr int S = decltype(s_tag)::value;   // j = j0 + S, j0 = 1 (mod 8)
    const int j = j0 + S;
    if constexpr (S % 2 == 1) pair_sync(j, IC<(S + 6) % kStages>{}, IC<(S + 7) % kStages>{});
    constexpr int kst = (S + 2) % kStages, vst = S % kStages;
    constexpr int nkst = (S + 3) % kStages, nvst = (S + 1) % kStages;
    if constexpr (S % 2 == 0)
      step(j, sb, sa, pa, pb, ob, oa, kst, vst, nkst, nvst, skc[S], svc[S], mxr);
    else
      step(j, sa, sb, pb, pa, oa, ob, kst, vst, nkst, nvst, skc[S], svc[S], mxr);
    return j == kv_end;
  };
  for (int j0 = 1;; j0 += kStages) {
    ld_scales(j0 + kStages, skn, svn);
    if (one(IC<0>{}, j0)) break;
    if (one(IC<1>{}, j0)) break;
    if (one(IC<2>{}, j0)) break;
    if (one(IC<3>{}, j0)) break;
    if (one(IC<4>{}, j0)) break;
    if (one(IC<5>{}, j0)) break;
    if (one(IC<6>{}, j0)) break;
    if (one(IC<7>{}, j0)) break;
#pragma unroll
    for (int i = 0; i < kStages; ++i) {
      skc[i] = skn[i];
      svc[i] = svn[i];
    }
  }
  __builtin_amdgcn_s_waitcnt(wait_vm(0));

  // Only the exponent of a V scale enters the instruction, so the V scales
  // of the visited tiles must be powers of two in [2^-126, 2^127]; any other
  // value turns this workgroup's rows into NaN instead of being rounded
  // down. Checked here, off the loop, one tile per lane.
  bool bad_v = false;
  for (int j0 = 0; j0 < kv_end; j0 += 64) {
    const int jj = j0 + lane;
    const uint32_t vb = jj < kv_end ? __float_as_uint(a.sv[(size_t)bh * nb + jj]) : 0x3F800000u;
    const uint32_t e8 = (vb >> 23) & 0xFFu;
    const bool bad = (vb & 0x807FFFFFu) != 0u || e8 == 0u || e8 == 255u;
    bad_v |= __builtin_amdgcn_ballot_w64(bad) != 0;
  }

  // O = acc * 2^(mr - m) / l' and LSE = (m + log2 l' - log2 448) ln 2 (mr
  // and m are finite whenever l' > 0).
  const float lt = halves_sum(l);
  const float inv = bad_v ? __builtin_nanf("") : lt == 0.f ? 0.f : fast_exp2(mr - m) / lt;
  // The lane half, formed anew from the lane id (kept from the start, it
  // took the register the loop needs most).
  const int hh_e = (int)(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) >> 5);
  if (qrow < N) {
    __bf16* og = (__bf16*)a.o + base + (size_t)qrow * kD;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[mt][4 * g + 0] * inv, oacc[mt][4 * g + 1] * inv);
        w[1] = pack_bf16x2(oacc[mt][4 * g + 2] * inv, oacc[mt][4 * g + 3] * inv);
        *(u32x2*)(og + mt * 32 + 8 * g + 4 * hh_e) = w;
      }
    if (hh_e == 0)
      a.lse[(size_t)bh * N + qrow] = bad_v ? __builtin_nanf("")
                                     : lt == 0.f ? -INFINITY : (m + fast_log2(lt) - kLog2_448) * kLn2;
  }
#endif
}

template <bool CAUSAL>
hipError_t launch_attn(const Fp8FwdArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((fwd_fp8_kernel<CAUSAL>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_fp8(int d, QuantArgs a, int B, int H, hipStream_t s) {
  if (d == 64) return a.rot ? launch_quant_d<64, true>(a, B, H, s) : launch_quant_d<64, false>(a, B, H, s);
  return a.rot ? launch_quant_d<128, true>(a, B, H, s) : launch_quant_d<128, false>(a, B, H, s);
}

hipError_t launch_dequant_fp8(const unsigned char* x8, const float* scales, void* out, int B, int H, int N, int d,
                              hipStream_t s) {
  const unsigned per_head16 = (unsigned)N * (unsigned)d / 16u;
  const unsigned gx = (per_head16 + 255u) / 256u;
  const int nbh = B * H;
  for (int bh0 = 0; bh0 < nbh; bh0 += 65535) {
    const int gy = std::min(65535, nbh - bh0);
    hipLaunchKernelGGL(dequant_kernel, dim3(gx, (unsigned)gy), dim3(256), 0, s, x8, scales, (__bf16*)out, N, d,
                       (N + 63) / 64, bh0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_fwd_fp8(int d, int causal, Fp8FwdArgs a, int B, int H, hipStream_t s) {
  if (d != kD) return hipErrorNotSupported;
  a.n_qtiles = (a.N + kBR - 1) / kBR;
  const long long grid = (long long)B * H * a.n_qtiles;
  a.remap = (grid % 8 == 0) ? 1 : 0;
  return causal ? launch_attn<true>(a, (int)grid, s) : launch_attn<false>(a, (int)grid, s);
}

}  // namespace fa
