// Host-side declarations of the kernel launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

enum class DType { F32, BF16 };

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int N;
  int n_qtiles;   // filled by the launcher
  float c;        // scale * log2(e)
  int remap;      // filled by the launcher
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* dq_acc;  // [B,H,N,d] float32 workspace
  float* dvec;    // [B,H,N] float32 workspace: D = rowsum(dO * O)
  int N;
  int n_tiles;    // filled by the launcher
  float scale;
  float c;        // scale * log2(e)
  int remap;      // filled by the launcher
};

struct QuantArgs {
  const void* x;       // bf16 [B,H,N,d]
  const float* rot;    // d x d or nullptr
  unsigned char* x8;
  float* scales;       // [B,H,ceil(N/64)]
  int N;
  int block_rows;      // 64 or 0
};

struct Fp8FwdArgs {
  const unsigned char* q8;
  const unsigned char* k8;
  const unsigned char* v8;
  const float* sq;
  const float* sk;
  const float* sv;
  void* o;
  float* lse;
  int N;
  int n_qtiles;   // filled by the launcher
  float c;        // scale * log2(e)
  int remap;      // filled by the launcher
};

hipError_t launch_fwd(DType dt, int d, int causal, FwdArgs a, int B, int H, hipStream_t s);
hipError_t launch_fwd_bf16(int d, int causal, FwdArgs a, int B, int H, hipStream_t s);
// stage_mask: 1 = preprocess (D, zero the dQ accumulator), 2 = main, 4 = dQ finish.
hipError_t launch_bwd(DType dt, int d, int causal, BwdArgs a, int B, int H, int stage_mask, hipStream_t s);
hipError_t launch_bwd_bf16_main(int d, int causal, BwdArgs a, int B, int H, hipStream_t s);
hipError_t launch_quant_fp8(int d, QuantArgs a, int B, int H, hipStream_t s);
hipError_t launch_fwd_fp8(int d, int causal, Fp8FwdArgs a, int B, int H, hipStream_t s);

}  // namespace fa
