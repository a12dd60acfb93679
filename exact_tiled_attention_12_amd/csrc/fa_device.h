// Device helpers shared by the gfx950 attention kernels.
//
// Matrix-core conventions used throughout (CDNA 32x32 MFMA outputs):
//   a 32x32 float accumulator is 16 floats per lane; lane l holds column
//   n = l % 32 and rows 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
//   Operand fragments hold, per lane, one row index (A) or one column index
//   (B) equal to l % 32 and a run of contraction indices chosen by l / 32.
//   Since A and B use the same lane-half -> contraction-index rule, any
//   consistent assignment of contraction indices to (lane half, slot) gives
//   the same product; the kernels rely only on that and on the accumulator
//   layout above.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Values of lanes l and l ^ 32 combined. v_permlane32_swap exchanges the upper
// half of its first operand with the lower half of its second; with both set
// to x, element 0 holds x of lanes 0..31 and element 1 holds x of lanes
// 32..63 on every lane.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row of a 32-row accumulator block -> which of 32 consecutive keys that row
// should hold so that, on every lane, accumulator slots 0..7 are 8
// consecutive keys and slots 8..15 the next-but-one 8 (lane half h holds keys
// 8h..8h+7 and 16+8h..16+8h+7). Used to permute the rows of an A operand.
__device__ __forceinline__ int acc_row_to_key(int i) {
  const int a = i >> 3, h = (i >> 2) & 1, b = i & 3;
  return 16 * (a >> 1) + 8 * h + 4 * (a & 1) + b;
}
// Key held by accumulator slot r on lane half h (inverse view of the above).
__host__ __device__ constexpr int slot_key(int r, int h) { return 16 * (r >> 3) + 8 * h + (r & 7); }

// x *= s with the product written back into the register it was read from.
// When an accumulator is rescaled on one branch only, a plain multiply lets
// the register allocator give the product new registers and then copy the
// untouched accumulator into them on the other branch; tying input and
// output keeps one set of registers on both paths.
__device__ __forceinline__ void scale_in_place(f32x16& x, float s) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float t = x[i];
    asm("v_mul_f32 %0, %1, %0" : "+v"(t) : "v"(s));
    x[i] = t;
  }
}

// bf16 pair packing with round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Element-type traits for the 32x32 MFMA family.
struct TrBF16 {
  using T = __bf16;
  using Frag = bf16x8;                 // 8 contraction values per lane
  static constexpr int KPL = 8;
  __device__ static __forceinline__ f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ Frag load(const T* p) { return *(const Frag*)p; }
  __device__ static __forceinline__ Frag zero() { return Frag{}; }
  __device__ static __forceinline__ Frag pack(const float* x) {
    Frag f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (__bf16)x[i];
    return f;
  }
};

struct TrF32 {
  using T = float;
  using Frag = float;                  // 1 contraction value per lane
  static constexpr int KPL = 1;
  __device__ static __forceinline__ f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ Frag load(const T* p) { return *p; }
  __device__ static __forceinline__ Frag zero() { return 0.f; }
  __device__ static __forceinline__ Frag pack(const float* x) { return x[0]; }
};

// Store NB bytes (4, 8, 16, 32 or 64; destination aligned to min(NB, 16))
// from an array of elements.
template <int NB>
__device__ __forceinline__ void store_bytes(void* dst, const void* src) {
  if constexpr (NB == 4) {
    *(uint32_t*)dst = *(const uint32_t*)src;
  } else if constexpr (NB == 8) {
    *(u32x2*)dst = *(const u32x2*)src;
  } else if constexpr (NB == 16) {
    *(u32x4*)dst = *(const u32x4*)src;
  } else {
    static_assert(NB == 32 || NB == 64, "unsupported store width");
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) ((u32x4*)dst)[i] = ((const u32x4*)src)[i];
  }
}

// ---- HBM -> LDS copies (buffer loads with an LDS destination).

typedef int i32x4 __attribute__((ext_vector_type(4)));

// A raw buffer resource (base, num_records = bytes, no stride) as four scalar
// words. Offsets at or past `bytes` read as zero.
__device__ __forceinline__ i32x4 dma_rsrc(const void* base, unsigned bytes) {
  const unsigned long long b = (unsigned long long)base;
  return i32x4{__builtin_amdgcn_readfirstlane((int)(unsigned)b),
               __builtin_amdgcn_readfirstlane((int)((unsigned)(b >> 32) & 0xFFFFu)),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

// 16 bytes per lane from buffer offset `voffset` to LDS byte address
// lds_addr + 16 * lane; lds_addr is wave-uniform and goes in M0. Written as
// inline assembly so that the compiler does not count the copy as a pending
// writer of the LDS reads that follow (with the builtin it waits for every
// copy in flight before them); the kernels order the copies themselves with
// vmcnt waits and barriers.
__device__ __forceinline__ void dma_load16(i32x4 rsrc, unsigned lds_addr, unsigned voffset) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voffset), "s"(rsrc) : "memory", "m0");
}

// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt <= n (n < 64) only.
constexpr int wait_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Map the hardware workgroup id to a logical id so that consecutive logical
// ids run on the same XCD: workgroups are dealt to the 8 XCDs round-robin,
// so hardware id w runs on XCD w % 8. Requires grid % 8 == 0.
__device__ __forceinline__ int xcd_remap(int w, int grid) {
  return (w & 7) * (grid >> 3) + (w >> 3);
}

}  // namespace fa
