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
  int H;          // query heads
  int group;      // query heads per K/V head (1 unless grouped-query, bf16 only)
  // Packed variable-length batch (bf16): cumulative sequence lengths
  // [n_seq + 1], or nullptr. N is then the packed length T (the row stride of
  // a head) and n_qtiles the tiles of the longest sequence.
  const int* cu_seqlens;
  int max_seqlen;
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
  float* dq_acc;  // [B,H,N,d] float32 workspace (nullptr in the fixed-order mode)
  float* dvec;    // [B,H,N] float32 workspace: D = rowsum(dO * O)
  float* dq_part; // fixed-order mode: dQ partial tiles (bwd_det_parts), else nullptr
  int N;
  int n_tiles;    // filled by the launcher
  float scale;
  float c;        // scale * log2(e)
  int remap;      // filled by the launcher
  int H;          // query heads
  int group;      // query heads per K/V head (1 unless grouped-query, bf16 only)
  int B;          // batch
  float* dkv_part;  // grouped K/V heads: float32 dK, dV per query head, [B H_kv][group][N][d] each; else nullptr
  // Packed variable-length batch: cumulative sequence lengths [B + 1], or
  // nullptr. N is then the packed length T (the row stride of a head; B = 1
  // for the streaming passes) and max_seqlen bounds every sequence.
  const int* cu_seqlens;
  int n_seq;
  int max_seqlen;
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

// Fixed-order (deterministic) dQ of the bf16 backward: each 256-key tile
// stores its dQ contribution to every query row it visits (float32, its own
// rows: no atomics), and the finish pass adds them per row in ascending
// key-tile order. Per (batch, head), key tile kt owns a block of
// bwd_visits(N, causal, kt) tiles of kBwdPartFloats floats, after the blocks
// of key tiles 0 .. kt-1: its visited rows (32 per query tile, from its first
// visited tile on) x d, once per key half for d = 64 (the two halves of its
// keys are summed by different waves).
constexpr int kBwdKeyTile = 256;
constexpr int kBwdRowTile = 32;
constexpr int kBwdPartFloats = 4096;   // floats per partial tile (both d)

__host__ __device__ inline int bwd_row_tiles(int N) { return (N + kBwdRowTile - 1) / kBwdRowTile; }
__host__ __device__ inline int bwd_key_tiles(int N) { return (N + kBwdKeyTile - 1) / kBwdKeyTile; }
// Query tiles key tile kt visits: all of them, or (causal) those at or below
// the diagonal, i.e. from tile kt * 256 / 32 on.
__host__ __device__ inline int bwd_visits(int N, int causal, int kt) {
  return bwd_row_tiles(N) - (causal ? kt * (kBwdKeyTile / kBwdRowTile) : 0);
}
// Partial tiles of key tiles 0 .. kt-1 (kt = number of key tiles: all of them).
__host__ __device__ inline long long bwd_part_offset(int N, int causal, int kt) {
  const long long r = bwd_row_tiles(N);
  const long long c = causal ? kBwdKeyTile / kBwdRowTile : 0;
  return (long long)kt * r - c * ((long long)kt * (kt - 1) / 2);
}
__host__ __device__ inline long long bwd_det_parts(int N, int causal) {
  return bwd_part_offset(N, causal, bwd_key_tiles(N));
}

hipError_t launch_fwd(DType dt, int d, int causal, FwdArgs a, int B, int H, hipStream_t s);
hipError_t launch_fwd_bf16(int d, int causal, FwdArgs a, int B, int H, hipStream_t s);
// stage_mask: 1 = preprocess (D, zero the dQ accumulator), 2 = main, 4 = dQ finish.
// With a.dq_part set (bf16 only) the dQ accumulator is not used: the main
// kernel writes partial tiles and the finish pass adds them in a fixed order.
hipError_t launch_bwd(DType dt, int d, int causal, BwdArgs a, int B, int H, int stage_mask, hipStream_t s);
hipError_t launch_bwd_bf16_main(int d, int causal, BwdArgs a, int B, int H, hipStream_t s);
hipError_t launch_quant_fp8(int d, QuantArgs a, int B, int H, hipStream_t s);
hipError_t launch_fwd_fp8(int d, int causal, Fp8FwdArgs a, int B, int H, hipStream_t s);

}  // namespace fa
