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
  int n_items;    // filled by the launcher: work items (batch or sequence, head, query tile)
  int persist;    // filled by the launcher: 1 if workgroups loop over items
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
  float* dq_acc;  // [B,H,N,d] float32 workspace: the dQ accumulator
  float* dvec;    // [B,H,N] float32 workspace: D = rowsum(dO * O)
  // Fixed-order mode (bf16, one K/V head per query head): per (batch, head,
  // 32-row query tile) kBwdSlots counters of the key-tile contributions added
  // to that tile's dQ rows so far, then one error flag; nullptr otherwise.
  int* dq_cnt;
  int* dq_err;
  int n_cnt;      // counters (and the flag) the preprocess pass clears
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
  int pow2;            // 1: power-of-two scales; 0: amax / 448
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

// Fixed-order (deterministic) dQ of the bf16 backward: the key tiles of a
// (batch, head) add their dQ contributions to each 32-row query tile in
// ascending key-tile order (read, add, write back; no float atomics), each
// waiting on a counter of that query tile for its predecessor. For d = 128
// the four waves of a key tile own one 32-column block of dQ each; for
// d = 64 two waves share a column block, key half 0 before key half 1.
constexpr int kBwdKeyTile = 256;
constexpr int kBwdRowTile = 32;
constexpr int kBwdSlots = 4;           // counters per query tile

__host__ __device__ inline int bwd_row_tiles(int N) { return (N + kBwdRowTile - 1) / kBwdRowTile; }

hipError_t launch_fwd(DType dt, int d, int causal, FwdArgs a, int B, int H, hipStream_t s);
hipError_t launch_fwd_bf16(int d, int causal, FwdArgs a, int B, int H, hipStream_t s);
// stage_mask: 1 = preprocess (D, zero the dQ accumulator), 2 = main, 4 = dQ finish.
// With a.dq_cnt set (bf16 only) the main kernel adds to the dQ accumulator in
// a fixed key-tile order and the preprocess pass also clears the counters.
hipError_t launch_bwd(DType dt, int d, int causal, BwdArgs a, int B, int H, int stage_mask, hipStream_t s);
hipError_t launch_bwd_bf16_main(int d, int causal, BwdArgs a, int B, int H, hipStream_t s);
// Compute units of the current device (0 if it cannot be read), looked up
// once per device.
int cu_count();

hipError_t launch_quant_fp8(int d, QuantArgs a, int B, int H, hipStream_t s);
hipError_t launch_fwd_fp8(int d, int causal, Fp8FwdArgs a, int B, int H, hipStream_t s);
hipError_t launch_dequant_fp8(const unsigned char* x8, const float* scales, void* out, int B, int H, int N, int d,
                              hipStream_t s);

}  // namespace fa
